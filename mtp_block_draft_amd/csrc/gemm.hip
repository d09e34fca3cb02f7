// Generic float32-output GEMM for the fusion projections and the drafter's
// layer projections: C = R + A B^T, with a deterministic split over K for the
// small-M, weight-streaming (HBM-bound) shapes of this path.
#include "gemm_core.hpp"
#include "kernels.hpp"

namespace dmtp {

namespace {

struct GemmParams {
  const void* A;
  size_t lda;
  int M;
  const void* B;
  size_t ldb;
  int N;
  int k_per_split;
  float* C;
  size_t ldc;
  const float* R;
  size_t ldr;
  float* part;   // [splits, M, N] when gridDim.z > 1
};

template <class T>
__global__ __launch_bounds__(T::THREADS) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[T::LDS_A + T::LDS_B];
  const int n0 = blockIdx.x * T::BN, m0 = blockIdx.y * T::BM;
  const int z = blockIdx.z;
  Acc<T> acc;
  gemm_mainloop<T>(acc, lds, p.A, p.lda, p.M, p.B, p.ldb, p.N, m0, n0, z * p.k_per_split,
                   (z + 1) * p.k_per_split);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wm0 = (wave / T::WAVES_N) * T::WM, wn0 = (wave % T::WAVES_N) * T::WN;
  const bool split = gridDim.z > 1;
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm0 + 16 * i + 4 * (lane >> 4) + r;
        const int col = n0 + wn0 + 16 * j + (lane & 15);
        if (row >= p.M || col >= p.N) continue;
        const float v = acc.v[i][j][r];
        if (split) {
          p.part[((size_t)z * p.M + row) * p.N + col] = v;
        } else {
          const float base = p.R ? p.R[(size_t)row * p.ldr + col] : 0.f;
          p.C[(size_t)row * p.ldc + col] = base + v;
        }
      }
}

// C = R + sum_z part[z] in a fixed order.
__global__ void splitk_reduce(const float* __restrict__ part, int splits, int M, int N, float* C,
                              size_t ldc, const float* R, size_t ldr) {
  const size_t total = (size_t)M * N;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
       e += (size_t)gridDim.x * blockDim.x) {
    const int row = (int)(e / N), col = (int)(e % N);
    float s = 0.f;
    for (int z = 0; z < splits; ++z) s += part[(size_t)z * total + e];
    const float base = R ? R[(size_t)row * ldr + col] : 0.f;
    C[(size_t)row * ldc + col] = base + s;
  }
}

typedef GemmTile<64, 64, 32, 32, 2, 1> TileF32xBF16;
typedef GemmTile<64, 64, 32, 32, 2, 2> TileF32xF32;
typedef GemmTile<64, 64, 32, 32, 1, 1> TileBF16xBF16;
typedef GemmTile<64, 64, 32, 32, 1, 2> TileBF16xF32;

template <class T>
hipError_t launch(const GemmParams& p, int splits, hipStream_t s) {
  dim3 grid((p.N + T::BN - 1) / T::BN, (p.M + T::BM - 1) / T::BM, splits);
  hipLaunchKernelGGL(gemm_kernel<T>, grid, dim3(T::THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int gemm_splits(int M, int N, int K) {
  const int tiles = ((M + 63) / 64) * ((N + 63) / 64);
  int splits = 1;
  // aim for >= 1024 workgroups on 256 CUs, keep >= 4 K-stages per split
  while (tiles * splits < 1024 && K % (2 * splits * 64) == 0 && K / (2 * splits) >= 256)
    splits *= 2;
  return splits;
}

size_t gemm_ws_bytes(int M, int N, int K) {
  const int sp = gemm_splits(M, N, K);
  return sp > 1 ? (size_t)sp * M * N * sizeof(float) : 0;
}

hipError_t gemm(const GemmArgs& a, float* ws, hipStream_t s) {
  const int splits = gemm_splits(a.M, a.N, a.K);
  GemmParams p{a.A, a.lda, a.M, a.B, a.ldb, a.N, a.K / splits, a.C, a.ldc, a.R, a.ldr, ws};
  hipError_t e;
  if (a.a_f32 && !a.b_f32)
    e = launch<TileF32xBF16>(p, splits, s);
  else if (a.a_f32 && a.b_f32)
    e = launch<TileF32xF32>(p, splits, s);
  else if (!a.a_f32 && !a.b_f32)
    e = launch<TileBF16xBF16>(p, splits, s);
  else
    e = launch<TileBF16xF32>(p, splits, s);
  if (e != hipSuccess || splits == 1) return e;
  const size_t total = (size_t)a.M * a.N;
  const int blocks = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  hipLaunchKernelGGL(splitk_reduce, dim3(blocks), dim3(256), 0, s, ws, splits, a.M, a.N, a.C,
                     a.ldc, a.R, a.ldr);
  return hipGetLastError();
}

}  // namespace dmtp

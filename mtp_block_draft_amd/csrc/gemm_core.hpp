// Tiled bf16 matrix-core GEMM main loop: C[M, N] = A[M, K] * B[N, K]^T.
//
// Both operands are K-contiguous (row-major A, weights stored [out, in]), so a
// lane's eight k values of an MFMA fragment are one 16-byte LDS read for A and
// for B alike.  A float32 operand enters as two bf16 planes (x = hi + lo to
// 2^-18): activations arrive already split by the kernel that produced them,
// float32 weights are split on their way into LDS.  The tile product
// accumulates the plane pairs (hi,hi), (hi,lo), (lo,hi): a float32 activation
// times a bf16 weight costs two MFMAs, float32 x float32 three.  Accumulation
// is float32.
#pragma once

#include "common.hpp"

namespace dmtp {

template <int BM_, int BN_, int WM_, int WN_, int AP_, int BP_>
struct GemmTile {
  static constexpr int BM = BM_, BN = BN_;    // workgroup tile
  static constexpr int WM = WM_, WN = WN_;    // wave tile
  static constexpr int BK = 64;               // K per LDS stage (two MFMA k-steps)
  static constexpr int AP = AP_, BP = BP_;    // bf16 planes of A and B (1 or 2)
  static constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static constexpr int NWAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = NWAVES * kWave;
  static constexpr int TM = WM / 16, TN = WN / 16;   // 16x16 MFMA tiles per wave
  static constexpr int LDK = BK + 8;                 // padded LDS row (bf16 elements)
  static constexpr int LDS_A = AP * BM * LDK;        // uint16 elements
  static constexpr int LDS_B = BP * BN * LDK;
  static constexpr int LDS_BYTES = (LDS_A + LDS_B) * 2;
  static_assert(BM % WM == 0 && BN % WN == 0 && WM % 16 == 0 && WN % 16 == 0, "tile");
};

// Accumulators of one wave: acc[tm][tn] covers rows wm0 + 16 tm + 4 (l / 16) + i,
// columns wn0 + 16 tn + (l % 16).
template <class T>
struct Acc {
  f32x4_t v[T::TM][T::TN];
};

// Stage one BM x BK (or BN x BK) tile of a row-major K-contiguous operand into
// LDS: a float32 operand (SRC == 2) split into its hi and lo bf16 planes, an
// operand already held as two bf16 planes (SRC == 3, lo plane at g + pst), or a
// bf16 operand (SRC == 1) as is.  Rows >= nrows are zero-filled.
template <int ROWS, int BK, int LDK, int THREADS, int SRC>
__device__ __forceinline__ void stage_tile(uint16_t* __restrict__ lds, const void* __restrict__ g,
                                           size_t ld, size_t pst, int row0, int nrows, int k0) {
  if (SRC == 3) {
    const uint16_t* src = (const uint16_t*)g;
    constexpr int V8 = ROWS * BK / 8;
    for (int idx = threadIdx.x; idx < 2 * V8; idx += THREADS) {
      const int p = idx / V8, e = idx % V8;
      const int r = e / (BK / 8), c8 = e % (BK / 8);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row0 + r < nrows) v = *(const uint4*)(src + p * pst + (size_t)(row0 + r) * ld + k0 + 8 * c8);
      *(uint4*)(lds + p * ROWS * LDK + r * LDK + 8 * c8) = v;
    }
  } else if (SRC == 2) {
    const float* src = (const float*)g;
    constexpr int V4 = ROWS * BK / 4;
    for (int idx = threadIdx.x; idx < V4; idx += THREADS) {
      const int r = idx / (BK / 4), c4 = idx % (BK / 4);
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (row0 + r < nrows) v = *(const float4*)(src + (size_t)(row0 + r) * ld + k0 + 4 * c4);
      uint16_t h0, h1, h2, h3, l0, l1, l2, l3;
      split_bf16(v.x, h0, l0);
      split_bf16(v.y, h1, l1);
      split_bf16(v.z, h2, l2);
      split_bf16(v.w, h3, l3);
      *(uint2*)(lds + r * LDK + 4 * c4) = make_uint2(pack2(h0, h1), pack2(h2, h3));
      *(uint2*)(lds + ROWS * LDK + r * LDK + 4 * c4) = make_uint2(pack2(l0, l1), pack2(l2, l3));
    }
  } else {
    const uint16_t* src = (const uint16_t*)g;
    constexpr int V8 = ROWS * BK / 8;
    for (int idx = threadIdx.x; idx < V8; idx += THREADS) {
      const int r = idx / (BK / 8), c8 = idx % (BK / 8);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row0 + r < nrows) v = *(const uint4*)(src + (size_t)(row0 + r) * ld + k0 + 8 * c8);
      *(uint4*)(lds + r * LDK + 8 * c8) = v;
    }
  }
}

// Main loop over k in [k_begin, k_end) (multiples of BK) for the workgroup tile
// at (m0, n0).  A is [M, lda]: bf16 when T::AP == 1; when T::AP == 2 two bf16
// planes (lo at A + a_pst) if A_F32 is false, else float32 split on the way in.
// B is [N, ldb], float32 when T::BP == 2 else bf16.
template <class T, bool A_F32 = false>
__device__ __forceinline__ void gemm_mainloop(Acc<T>& acc, uint16_t* lds, const void* A, size_t lda,
                                              size_t a_pst, int M, const void* B, size_t ldb, int N,
                                              int m0, int n0, int k_begin, int k_end) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int wm0 = (wave / T::WAVES_N) * T::WM;
  const int wn0 = (wave % T::WAVES_N) * T::WN;
  uint16_t* As = lds;
  uint16_t* Bs = lds + T::LDS_A;
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j) acc.v[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, fk = (lane >> 4) * 8;
  for (int k0 = k_begin; k0 < k_end; k0 += T::BK) {
    stage_tile<T::BM, T::BK, T::LDK, T::THREADS, T::AP == 1 ? 1 : (A_F32 ? 2 : 3)>(As, A, lda, a_pst,
                                                                                   m0, M, k0);
    stage_tile<T::BN, T::BK, T::LDK, T::THREADS, T::BP>(Bs, B, ldb, 0, n0, N, k0);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < T::BK; kk += 32) {
      uint4 a[T::AP][T::TM], b[T::BP][T::TN];
#pragma unroll
      for (int p = 0; p < T::AP; ++p)
#pragma unroll
        for (int i = 0; i < T::TM; ++i)
          a[p][i] = *(const uint4*)(As + p * T::BM * T::LDK + (wm0 + 16 * i + fr) * T::LDK + kk + fk);
#pragma unroll
      for (int p = 0; p < T::BP; ++p)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
          b[p][j] = *(const uint4*)(Bs + p * T::BN * T::LDK + (wn0 + 16 * j + fr) * T::LDK + kk + fk);
#pragma unroll
      for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
          acc.v[i][j] = mfma_16x16x32(a[0][i], b[0][j], acc.v[i][j]);
          if (T::BP > 1) acc.v[i][j] = mfma_16x16x32(a[0][i], b[T::BP - 1][j], acc.v[i][j]);
          if (T::AP > 1) acc.v[i][j] = mfma_16x16x32(a[T::AP - 1][i], b[0][j], acc.v[i][j]);
        }
    }
    __syncthreads();
  }
}

}  // namespace dmtp

// Row-wise kernels of the path: RMSNorm (float64 sum of squares), the fusion
// prologue, draft-slot assembly, the rotary embedding, SwiGLU and the drafter's
// final norm.  One workgroup per row; all of them are a few MB of traffic.
#include "common.hpp"
#include "kernels.hpp"

namespace dmtp {

namespace {

constexpr int kRowThreads = 256;

__device__ double block_sum(double v, double* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  if (l == 0) red[w] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < (int)(blockDim.x / kWave); ++i) t += red[i];
  __syncthreads();
  return t;
}

// 1 / sqrt(mean(x^2) + eps) of a row read through `ld` (float64 accumulation).
template <class Load>
__device__ double inv_rms(Load ld, int H, float eps, double* red) {
  double ss = 0.0;
  for (int i = threadIdx.x; i < H; i += blockDim.x) {
    const double v = ld(i);
    ss += v * v;
  }
  ss = block_sum(ss, red);
  return 1.0 / sqrt(ss / H + (double)eps);
}

// y = RMSNorm(x; g) written as bf16 planes [2][rows][H] (plane stride pst).
__global__ __launch_bounds__(kRowThreads) void rmsnorm_rows_kernel(const float* __restrict__ x,
                                                                   const float* __restrict__ g,
                                                                   float eps, uint16_t* __restrict__ y,
                                                                   size_t pst, int H) {
  __shared__ double red[kRowThreads / kWave];
  const float* xr = x + (size_t)blockIdx.x * H;
  const double inv = inv_rms([&](int i) { return (double)xr[i]; }, H, eps, red);
  const size_t r0 = (size_t)blockIdx.x * H;
  for (int i = threadIdx.x; i < H; i += blockDim.x)
    store_planes(y, pst, r0 + i, (float)((double)xr[i] * inv * g[i]));
}

struct RowSrc {
  const void* rows;
  int dtype;
  const int32_t* ids;
  const void* table;
  int n_table;
};

// Element i of row r: the row itself, or table[ids[r]] (zero for an id outside the table).
__device__ __forceinline__ float row_elem(const RowSrc& s, int r, int H, int i) {
  if (s.rows) return load_elem(s.rows, s.dtype, (size_t)r * H + i);
  const int id = s.ids[r];
  if (id < 0 || id >= s.n_table) return 0.f;
  return load_elem(s.table, s.dtype, (size_t)id * H + i);
}

__global__ __launch_bounds__(kRowThreads) void fuse_prep_kernel(RowSrc x1, RowSrc x2, RowSrc res,
                                                                int has_res, const float* g1,
                                                                const float* g2, float eps, int H,
                                                                uint16_t* __restrict__ cat,
                                                                size_t pst,
                                                                float* __restrict__ out) {
  __shared__ double red[kRowThreads / kWave];
  const int r = blockIdx.x;
  const double i1 = inv_rms([&](int i) { return (double)row_elem(x1, r, H, i); }, H, eps, red);
  const double i2 = inv_rms([&](int i) { return (double)row_elem(x2, r, H, i); }, H, eps, red);
  const size_t c0 = (size_t)r * 2 * H;
  for (int i = threadIdx.x; i < H; i += blockDim.x) {
    store_planes(cat, pst, c0 + i, (float)((double)row_elem(x1, r, H, i) * i1 * g1[i]));
    store_planes(cat, pst, c0 + H + i, (float)((double)row_elem(x2, r, H, i) * i2 * g2[i]));
    if (has_res) out[(size_t)r * H + i] = row_elem(res, r, H, i);
  }
}

__global__ void build_slots_kernel(const int32_t* __restrict__ anchor, const float* __restrict__ x_t1,
                                   const void* __restrict__ emb, int dtype, int mask_id, int V, int S,
                                   int n_anchor, int H, float* __restrict__ X) {
  const int b = blockIdx.x / S, s = blockIdx.x % S;
  float* xr = X + (size_t)blockIdx.x * H;
  if (s == n_anchor - 1) {
    const float* src = x_t1 + (size_t)b * H;
    for (int i = threadIdx.x; i < H; i += blockDim.x) xr[i] = src[i];
    return;
  }
  const int tok = (n_anchor == 2 && s == 0) ? anchor[b] : mask_id;
  const bool ok = tok >= 0 && tok < V;
  for (int i = threadIdx.x; i < H; i += blockDim.x)
    xr[i] = ok ? load_elem(emb, dtype, (size_t)tok * H + i) : 0.f;
}

// Rotary embedding, rotate-half form: dims i and i + d/2 turn by pos * base^(-2i/d).
// Angles and their sines in float64 so that positions up to 32K keep full accuracy.
__global__ void rope_split_kernel(const float* __restrict__ qkv, const int32_t* __restrict__ cu_ctx,
                                  int ctx_rows, int S, int Hq, int Hkv, int d, float rope_base,
                                  float* __restrict__ q, float* __restrict__ kb,
                                  float* __restrict__ vb) {
  const int b = blockIdx.x / S, s = blockIdx.x % S;
  const int G = Hq / Hkv, NQ = S * G, half = d / 2;
  const int pos = ctx_len_of(cu_ctx, b, ctx_rows) + s;
  const float* row = qkv + (size_t)blockIdx.x * (Hq + 2 * Hkv) * d;
  const double lnb = log((double)rope_base);
  // rotated heads: Hq query heads then Hkv key heads, pairs (i, i + d/2)
  for (int e = threadIdx.x; e < (Hq + Hkv) * half; e += blockDim.x) {
    const int h = e / half, i = e % half;
    const double ang = (double)pos * exp(-(2.0 * i / d) * lnb);
    double sn, cs;
    sincos(ang, &sn, &cs);
    const double x1 = row[h * d + i], x2 = row[h * d + i + half];
    const float o1 = (float)(x1 * cs - x2 * sn), o2 = (float)(x2 * cs + x1 * sn);
    if (h < Hq) {
      float* dst = q + (((size_t)b * Hkv + h / G) * NQ + s * G + h % G) * d;
      dst[i] = o1;
      dst[i + half] = o2;
    } else {
      float* dst = kb + (((size_t)b * Hkv + (h - Hq)) * S + s) * d;
      dst[i] = o1;
      dst[i + half] = o2;
    }
  }
  for (int e = threadIdx.x; e < Hkv * d; e += blockDim.x) {
    const int h = e / d, i = e % d;
    vb[(((size_t)b * Hkv + h) * S + s) * d + i] = row[(Hq + Hkv) * d + e];
  }
}

// a = silu(g) * u, written as bf16 planes [2][n] (plane stride n).
__global__ void swiglu_kernel(const float* __restrict__ g, const float* __restrict__ u,
                              uint16_t* __restrict__ a, size_t n) {
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (size_t)gridDim.x * blockDim.x) {
    const float x = g[e];
    store_planes(a, n, e, x / (1.0f + expf(-x)) * u[e]);
  }
}

__global__ __launch_bounds__(kRowThreads) void final_norm_kernel(const float* __restrict__ X,
                                                                 const float* __restrict__ g,
                                                                 float eps, int S, int n_anchor,
                                                                 int Km1, int H, int dtype,
                                                                 void* __restrict__ out) {
  __shared__ double red[kRowThreads / kWave];
  const int b = blockIdx.x / Km1, j = blockIdx.x % Km1;
  const float* xr = X + ((size_t)b * S + n_anchor + j) * H;
  const double inv = inv_rms([&](int i) { return (double)xr[i]; }, H, eps, red);
  for (int i = threadIdx.x; i < H; i += blockDim.x)
    store_elem(out, dtype, (size_t)blockIdx.x * H + i, (float)((double)xr[i] * inv * g[i]));
}

RowSrc src_of(const dmtp_rows& r, int w_dtype) {
  RowSrc s;
  s.rows = r.rows;
  s.dtype = r.rows ? r.dtype : w_dtype;
  s.ids = r.ids;
  s.table = r.table;
  s.n_table = r.table_rows;
  return s;
}

}  // namespace

hipError_t rmsnorm_rows(const float* x, const float* g, float eps, uint16_t* y, int rows, int H,
                        hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_rows_kernel, dim3(rows), dim3(kRowThreads), 0, s, x, g, eps, y,
                     (size_t)rows * H, H);
  return hipGetLastError();
}

hipError_t fuse_prep(const dmtp_fuse_desc& d, uint16_t* cat, hipStream_t s) {
  const int has_res = d.res.rows != nullptr || d.res.ids != nullptr;
  hipLaunchKernelGGL(fuse_prep_kernel, dim3(d.rows), dim3(kRowThreads), 0, s,
                     src_of(d.x1, d.w_dtype), src_of(d.x2, d.w_dtype), src_of(d.res, d.w_dtype),
                     has_res, d.g1, d.g2, d.eps, d.H, cat, (size_t)d.rows * 2 * d.H, d.out);
  return hipGetLastError();
}

hipError_t build_slots(const dmtp_draft_desc& d, float* X, hipStream_t s) {
  const int S = d.K - 1 + d.n_anchor;
  hipLaunchKernelGGL(build_slots_kernel, dim3(d.B * S), dim3(256), 0, s, d.anchor_ids, d.x_t1,
                     d.emb, d.dtype, d.mask_id, d.V, S, d.n_anchor, d.H, X);
  return hipGetLastError();
}

hipError_t rope_split(const float* qkv, const int32_t* cu_ctx, int ctx_rows, int B, int S, int Hq,
                      int Hkv, int d, float rope_base, float* q, float* kb, float* vb,
                      hipStream_t s) {
  hipLaunchKernelGGL(rope_split_kernel, dim3(B * S), dim3(256), 0, s, qkv, cu_ctx, ctx_rows, S, Hq,
                     Hkv, d, rope_base, q, kb, vb);
  return hipGetLastError();
}

hipError_t swiglu(const float* g, const float* u, uint16_t* a, size_t n, hipStream_t s) {
  const size_t blocks = (n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192;
  hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)blocks), dim3(256), 0, s, g, u, a, n);
  return hipGetLastError();
}

hipError_t final_norm_mask(const float* X, const float* g, float eps, int B, int S, int n_anchor,
                           int K, int H, int dtype, void* out, hipStream_t s) {
  hipLaunchKernelGGL(final_norm_kernel, dim3(B * (K - 1)), dim3(kRowThreads), 0, s, X, g, eps, S,
                     n_anchor, K - 1, H, dtype, out);
  return hipGetLastError();
}

}  // namespace dmtp

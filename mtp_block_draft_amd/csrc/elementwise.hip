// Row-wise kernels of the path: the fusion prologue, draft-slot assembly,
// RMSNorm (float64 sum of squares), the rotary embedding, SwiGLU and the
// drafter's final norm.  One workgroup per row; each reads its row once into
// registers.  The kernels that follow a drafter GEMM read its result through
// a SplitOut view, which adds the float32 split-K partials (and the residual)
// in a fixed order, so no separate reduction pass is needed.
#include "common.hpp"
#include "kernels.hpp"

namespace dmtp {

namespace {

// Threads per row of the row-wise kernels (one workgroup per row).  512
// measured faster than 256 on rows of 2048 and 5120: fewer float4 per thread
// shorten each thread's chain of loads.
constexpr int kRowThreads = 512;

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

// value(m, n .. n + 3) of a GEMM result: the finished row when it was not split
// over K, else R + (part[0] + part[1] + ...), the order the reduction uses.
// split_issue4 starts the loads of the first Z partials (and of R) without
// waiting for them; split_finish4 adds them in that order, loading any splits
// past Z itself.  Issuing every load of a row before the first sum keeps one
// memory latency per row instead of one per split.
template <int Z>
struct SplitAcc {
  float4 t[Z];
  float4 r;
};

template <int Z>
__device__ __forceinline__ void split_issue4(const SplitOut& o, int m, int n, SplitAcc<Z>& a) {
  if (o.splits == 1) {
    a.t[0] = *(const float4*)(o.C + (size_t)m * o.ldc + n);
    return;
  }
  const size_t mn = (size_t)m * o.N + n, plane = (size_t)o.M * o.N;
#pragma unroll
  for (int z = 0; z < Z; ++z)
    if (z < o.splits) a.t[z] = *(const float4*)(o.part + z * plane + mn);
  if (o.R) a.r = *(const float4*)(o.R + (size_t)m * o.ldr + n);
}

__device__ __forceinline__ void add4(float4& s, const float4& v) {
  s.x += v.x;
  s.y += v.y;
  s.z += v.z;
  s.w += v.w;
}

template <int Z>
__device__ __forceinline__ float4 split_finish4(const SplitOut& o, int m, int n, const SplitAcc<Z>& a) {
  if (o.splits == 1) return a.t[0];
  float4 s = a.t[0];
#pragma unroll
  for (int z = 1; z < Z; ++z)
    if (z < o.splits) add4(s, a.t[z]);
  if (o.splits > Z) {
    const size_t mn = (size_t)m * o.N + n, plane = (size_t)o.M * o.N;
    for (int z = Z; z < o.splits; ++z) add4(s, *(const float4*)(o.part + z * plane + mn));
  }
  if (o.R) s = make_float4(a.r.x + s.x, a.r.y + s.y, a.r.z + s.z, a.r.w + s.w);
  return s;
}

// splits held in flight per float4 for a thread that fetches V4 of them
template <int V4>
constexpr int zb_of() {
  return V4 >= 8 ? 1 : 8 / V4;
}

__device__ __forceinline__ double sumsq4(const float4& v) {
  return (double)v.x * v.x + (double)v.y * v.y + (double)v.z * v.z + (double)v.w * v.w;
}

// Planes of y = x * inv * g for four consecutive elements at index i.
__device__ __forceinline__ void store_norm4(uint16_t* y, size_t pst, size_t i, const float4& x,
                                            double inv, const float4& gg) {
  store_planes(y, pst, i + 0, (float)((double)x.x * inv * gg.x));
  store_planes(y, pst, i + 1, (float)((double)x.y * inv * gg.y));
  store_planes(y, pst, i + 2, (float)((double)x.z * inv * gg.z));
  store_planes(y, pst, i + 3, (float)((double)x.w * inv * gg.w));
}

// X[m] = value(m) (the residual update, when write_x) and y[m] =
// RMSNorm(value(m); g) as bf16 planes [2][rows][H].  V4 float4 per thread.
template <int V4>
__global__ __launch_bounds__(kRowThreads) void residual_rmsnorm_kernel(SplitOut o, float* X, size_t ldx,
                                                                       int write_x, const float* g,
                                                                       float eps, uint16_t* y,
                                                                       size_t pst, int H) {
  __shared__ double red[kRowThreads / kWave];
  const int m = blockIdx.x;
  float4 v[V4], gv[V4];
  SplitAcc<zb_of<V4>()> acc[V4];
#pragma unroll
  for (int k = 0; k < V4; ++k) {
    const int n = 4 * (threadIdx.x + kRowThreads * k);
    if (n < H) {
      split_issue4(o, m, n, acc[k]);
      gv[k] = *(const float4*)(g + n);
    }
  }
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < V4; ++k) {
    const int n = 4 * (threadIdx.x + kRowThreads * k);
    if (n < H) {
      v[k] = split_finish4(o, m, n, acc[k]);
      ss += sumsq4(v[k]);
    }
  }
  ss = block_sum(ss, red);
  const double inv = 1.0 / sqrt(ss / H + (double)eps);
#pragma unroll
  for (int k = 0; k < V4; ++k) {
    const int n = 4 * (threadIdx.x + kRowThreads * k);
    if (n < H) {
      if (write_x) *(float4*)(X + (size_t)m * ldx + n) = v[k];
      store_norm4(y, pst, (size_t)m * H + n, v[k], inv, gv[k]);
    }
  }
}

// out[b, j] = round_dtype(RMSNorm(value(b S + n_anchor + j); g)), j < K - 1.
template <int V4>
__global__ __launch_bounds__(kRowThreads) void final_norm_kernel(SplitOut o, const float* g, float eps,
                                                                 int S, int n_anchor, int Km1, int H,
                                                                 int dtype, void* out) {
  __shared__ double red[kRowThreads / kWave];
  const int b = blockIdx.x / Km1, j = blockIdx.x % Km1;
  const int m = b * S + n_anchor + j;
  float4 v[V4], gv[V4];
  SplitAcc<zb_of<V4>()> acc[V4];
#pragma unroll
  for (int k = 0; k < V4; ++k) {
    const int n = 4 * (threadIdx.x + kRowThreads * k);
    if (n < H) {
      split_issue4(o, m, n, acc[k]);
      gv[k] = *(const float4*)(g + n);
    }
  }
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < V4; ++k) {
    const int n = 4 * (threadIdx.x + kRowThreads * k);
    if (n < H) {
      v[k] = split_finish4(o, m, n, acc[k]);
      ss += sumsq4(v[k]);
    }
  }
  ss = block_sum(ss, red);
  const double inv = 1.0 / sqrt(ss / H + (double)eps);
  const size_t r0 = (size_t)blockIdx.x * H;
#pragma unroll
  for (int k = 0; k < V4; ++k) {
    const int n = 4 * (threadIdx.x + kRowThreads * k);
    if (n < H) {
      const float4 gg = gv[k];
      store_elem(out, dtype, r0 + n + 0, (float)((double)v[k].x * inv * gg.x));
      store_elem(out, dtype, r0 + n + 1, (float)((double)v[k].y * inv * gg.y));
      store_elem(out, dtype, r0 + n + 2, (float)((double)v[k].z * inv * gg.z));
      store_elem(out, dtype, r0 + n + 3, (float)((double)v[k].w * inv * gg.w));
    }
  }
}

// Four consecutive elements (n % 4 == 0) of a row stored in dtype.
__device__ __forceinline__ float4 load4(const void* base, int dtype, size_t off) {
  if (dtype == DMTP_BF16) {
    const uint2 u = *(const uint2*)((const uint16_t*)base + off);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
  }
  return *(const float4*)((const float*)base + off);
}

struct RowSrc {
  const void* rows;
  int dtype;
  const int32_t* ids;
  const void* table;
  int n_table;
};

// Elements n .. n + 3 of row r: the row itself, or table[ids[r]] (zero for an
// id outside the table).
__device__ __forceinline__ float4 row_elem4(const RowSrc& s, int r, int H, int n) {
  if (s.rows) return load4(s.rows, s.dtype, (size_t)r * H + n);
  const int id = s.ids[r];
  if (id < 0 || id >= s.n_table) return make_float4(0.f, 0.f, 0.f, 0.f);
  return load4(s.table, s.dtype, (size_t)id * H + n);
}

// cat[r] = [RMSNorm(x1[r]; g1), RMSNorm(x2[r]; g2)] as bf16 planes, and
// out[r] = res[r] when has_res.
template <int V4>
__global__ __launch_bounds__(kRowThreads) void fuse_prep_kernel(RowSrc x1, RowSrc x2, RowSrc res,
                                                                int has_res, const float* g1,
                                                                const float* g2, float eps, int H,
                                                                uint16_t* __restrict__ cat,
                                                                size_t pst,
                                                                float* __restrict__ out) {
  __shared__ double red[2][kRowThreads / kWave];
  const int r = blockIdx.x;
  // up to 4 float4 per thread, the residual and the gains are loaded with the
  // rows; longer rows load them in the store loop to stay within registers
  constexpr bool PRE = V4 <= 4;
  constexpr int VP = PRE ? V4 : 1;
  float4 a[V4], c[V4], e[VP], ga[VP], gc[VP];
#pragma unroll
  for (int k = 0; k < V4; ++k) {
    const int n = 4 * (threadIdx.x + kRowThreads * k);
    if (n < H) {
      a[k] = row_elem4(x1, r, H, n);
      c[k] = row_elem4(x2, r, H, n);
      if (PRE) {
        if (has_res) e[k % VP] = row_elem4(res, r, H, n);
        ga[k % VP] = *(const float4*)(g1 + n);
        gc[k % VP] = *(const float4*)(g2 + n);
      }
    }
  }
  double s1 = 0.0, s2 = 0.0;
#pragma unroll
  for (int k = 0; k < V4; ++k) {
    const int n = 4 * (threadIdx.x + kRowThreads * k);
    if (n < H) {
      s1 += sumsq4(a[k]);
      s2 += sumsq4(c[k]);
    }
  }
  s1 = wave_sum(s1);
  s2 = wave_sum(s2);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  if (l == 0) {
    red[0][w] = s1;
    red[1][w] = s2;
  }
  __syncthreads();
  s1 = s2 = 0.0;
  for (int i = 0; i < kRowThreads / kWave; ++i) {
    s1 += red[0][i];
    s2 += red[1][i];
  }
  const double i1 = 1.0 / sqrt(s1 / H + (double)eps), i2 = 1.0 / sqrt(s2 / H + (double)eps);
  const size_t c0 = (size_t)r * 2 * H;
#pragma unroll
  for (int k = 0; k < V4; ++k) {
    const int n = 4 * (threadIdx.x + kRowThreads * k);
    if (n < H) {
      if (PRE) {
        store_norm4(cat, pst, c0 + n, a[k], i1, ga[k % VP]);
        store_norm4(cat, pst, c0 + H + n, c[k], i2, gc[k % VP]);
        if (has_res) *(float4*)(out + (size_t)r * H + n) = e[k % VP];
      } else {
        store_norm4(cat, pst, c0 + n, a[k], i1, *(const float4*)(g1 + n));
        store_norm4(cat, pst, c0 + H + n, c[k], i2, *(const float4*)(g2 + n));
        if (has_res) *(float4*)(out + (size_t)r * H + n) = row_elem4(res, r, H, n);
      }
    }
  }
}

// Draft slot rows X [B * S, H] (float32): slot n_anchor - 1 is x_t1[b], slot
// 0 of a dual-anchor block the anchor's embedding, every other slot the MASK
// embedding (zeros for an id outside the table); and, as residual_rmsnorm_kernel
// computes it from X, their RMSNorm with gains g as bf16 planes y [2][rows][H].
template <int V4>
__global__ __launch_bounds__(kRowThreads) void build_slots_kernel(
    const int32_t* __restrict__ anchor, const float* __restrict__ x_t1, const void* __restrict__ emb,
    int dtype, int mask_id, int V, int S, int n_anchor, int H, float* __restrict__ X,
    const float* __restrict__ g, float eps, uint16_t* __restrict__ y, size_t pst) {
  __shared__ double red[kRowThreads / kWave];
  const int m = blockIdx.x, b = m / S, s = m % S;
  const bool from_t1 = s == n_anchor - 1;
  const int tok = (n_anchor == 2 && s == 0) ? anchor[b] : mask_id;
  const bool ok = tok >= 0 && tok < V;
  float4 v[V4], gv[V4];
#pragma unroll
  for (int k = 0; k < V4; ++k) {
    const int n = 4 * (threadIdx.x + kRowThreads * k);
    if (n < H) {
      v[k] = from_t1 ? *(const float4*)(x_t1 + (size_t)b * H + n)
                     : (ok ? load4(emb, dtype, (size_t)tok * H + n) : make_float4(0.f, 0.f, 0.f, 0.f));
      gv[k] = *(const float4*)(g + n);
    }
  }
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < V4; ++k)
    if (4 * (threadIdx.x + kRowThreads * k) < H) ss += sumsq4(v[k]);
  ss = block_sum(ss, red);
  const double inv = 1.0 / sqrt(ss / H + (double)eps);
#pragma unroll
  for (int k = 0; k < V4; ++k) {
    const int n = 4 * (threadIdx.x + kRowThreads * k);
    if (n < H) {
      *(float4*)(X + (size_t)m * H + n) = v[k];
      store_norm4(y, pst, (size_t)m * H + n, v[k], inv, gv[k]);
    }
  }
}

// q/k/v split of the QKV projection with the rotary embedding at the slot's
// position: pair (i, i + d/2) of every query and key head is rotated by
// pos * base^(-2i/d).  The angles depend only on (pos, i), so their cosines and
// sines are computed once per row (float64) into LDS.
__global__ __launch_bounds__(256) void rope_split_kernel(SplitOut o, const int32_t* __restrict__ cu_ctx,
                                                         int ctx_rows, int S, int Hq, int Hkv, int d,
                                                         float rope_base, float* __restrict__ q,
                                                         float* __restrict__ kb,
                                                         float* __restrict__ vb) {
  __shared__ double cs[64], sn[64];
  const int m = blockIdx.x;
  const int b = m / S, s = m % S;
  const int G = Hq / Hkv, NQ = S * G, half = d / 2;
  // rotated heads: Hq query heads then Hkv key heads, four pairs per item;
  // then the value heads, four elements per item
  const int quads = (Hq + Hkv) * half / 4, vquads = Hkv * d / 4;
  // the partial loads of each thread's first items go out before the angles
  // are computed, so that their latency overlaps the float64 sincos
  const int e0 = threadIdx.x;
  SplitAcc<4> p1, p2;
  SplitAcc<8> pv;
  if (e0 < quads) {
    const int h = (4 * e0) / half, i0 = (4 * e0) % half;
    split_issue4(o, m, h * d + i0, p1);
    split_issue4(o, m, h * d + i0 + half, p2);
  }
  if (e0 < vquads) split_issue4(o, m, (Hq + Hkv) * d + 4 * e0, pv);
  const int pos = ctx_len_of(cu_ctx, b, ctx_rows) + s;
  const double lnb = log((double)rope_base);
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double ang = (double)pos * exp(-(2.0 * i / d) * lnb);
    double sv, cv;
    sincos(ang, &sv, &cv);
    sn[i] = sv;
    cs[i] = cv;
  }
  __syncthreads();
  auto rotate = [&](int e, const SplitAcc<4>& a, const SplitAcc<4>& c) __attribute__((always_inline)) {
    const int h = (4 * e) / half, i0 = (4 * e) % half;
    const float4 x1 = split_finish4(o, m, h * d + i0, a), x2 = split_finish4(o, m, h * d + i0 + half, c);
    const float a1[4] = {x1.x, x1.y, x1.z, x1.w}, a2[4] = {x2.x, x2.y, x2.z, x2.w};
    float r1[4], r2[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const double cc = cs[i0 + t], sv = sn[i0 + t];
      r1[t] = (float)((double)a1[t] * cc - (double)a2[t] * sv);
      r2[t] = (float)((double)a2[t] * cc + (double)a1[t] * sv);
    }
    float* dst = h < Hq ? q + (((size_t)b * Hkv + h / G) * NQ + s * G + h % G) * d
                        : kb + (((size_t)b * Hkv + (h - Hq)) * S + s) * d;
    *(float4*)(dst + i0) = make_float4(r1[0], r1[1], r1[2], r1[3]);
    *(float4*)(dst + i0 + half) = make_float4(r2[0], r2[1], r2[2], r2[3]);
  };
  auto value = [&](int e, const SplitAcc<8>& a) __attribute__((always_inline)) {
    const int h = (4 * e) / d, i = (4 * e) % d;
    *(float4*)(vb + (((size_t)b * Hkv + h) * S + s) * d + i) = split_finish4(o, m, (Hq + Hkv) * d + 4 * e, a);
  };
  if (e0 < quads) rotate(e0, p1, p2);
  if (e0 < vquads) value(e0, pv);
  for (int e = e0 + blockDim.x; e < quads; e += blockDim.x) {
    const int h = (4 * e) / half, i0 = (4 * e) % half;
    split_issue4(o, m, h * d + i0, p1);
    split_issue4(o, m, h * d + i0 + half, p2);
    rotate(e, p1, p2);
  }
  for (int e = e0 + blockDim.x; e < vquads; e += blockDim.x) {
    split_issue4(o, m, (Hq + Hkv) * d + 4 * e, pv);
    value(e, pv);
  }
}

// Two bf16 planes of n elements (x = hi + lo to 2^-18; lo = 0 for bf16 input).
__global__ void to_planes_kernel(const void* __restrict__ x, int dtype, size_t n,
                                 uint16_t* __restrict__ planes) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    store_planes(planes, n, i, load_elem(x, dtype, i));
}

// One workgroup per row: keys rotated at the row's position (angles in
// float64, as in rope_split_kernel), keys and values stored in dtype at the
// row's cache slot.  The row is the split GEMM result's value (partials added
// in split order, as the other consumers of a deferred GEMM do).
__global__ __launch_bounds__(256) void rope_scatter_kernel(SplitOut o,
                                                           const int32_t* __restrict__ positions,
                                                           const int32_t* __restrict__ dst_rows,
                                                           int Hkv, int d, float rope_base, int dtype,
                                                           int ctx_rows, void* __restrict__ k_cache,
                                                           void* __restrict__ v_cache) {
  __shared__ double cs[64], sn[64];
  const int r = blockIdx.x;
  const int dst = dst_rows[r];
  if (dst < 0 || dst >= ctx_rows) return;
  const int half = d / 2, pos = positions[r];
  const double lnb = log((double)rope_base);
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double ang = (double)pos * exp(-(2.0 * i / d) * lnb);
    double sv, cv;
    sincos(ang, &sv, &cv);
    sn[i] = sv;
    cs[i] = cv;
  }
  __syncthreads();
  const size_t ob = (size_t)dst * Hkv * d;
  // keys: four rotation pairs (i, i + d/2) per thread
  for (int e = threadIdx.x; e < Hkv * half / 4; e += blockDim.x) {
    const int h = (4 * e) / half, i0 = (4 * e) % half;
    SplitAcc<4> p1, p2;
    split_issue4(o, r, h * d + i0, p1);
    split_issue4(o, r, h * d + i0 + half, p2);
    const float4 x1 = split_finish4(o, r, h * d + i0, p1), x2 = split_finish4(o, r, h * d + i0 + half, p2);
    const float a1[4] = {x1.x, x1.y, x1.z, x1.w}, a2[4] = {x2.x, x2.y, x2.z, x2.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const double c = cs[i0 + t], sv = sn[i0 + t];
      store_elem(k_cache, dtype, ob + h * d + i0 + t, (float)((double)a1[t] * c - (double)a2[t] * sv));
      store_elem(k_cache, dtype, ob + h * d + i0 + half + t,
                 (float)((double)a2[t] * c + (double)a1[t] * sv));
    }
  }
  // values as they are
  for (int e = threadIdx.x; e < Hkv * d / 4; e += blockDim.x) {
    SplitAcc<8> pv;
    split_issue4(o, r, Hkv * d + 4 * e, pv);
    const float4 v = split_finish4(o, r, Hkv * d + 4 * e, pv);
    store_elem(v_cache, dtype, ob + 4 * e + 0, v.x);
    store_elem(v_cache, dtype, ob + 4 * e + 1, v.y);
    store_elem(v_cache, dtype, ob + 4 * e + 2, v.z);
    store_elem(v_cache, dtype, ob + 4 * e + 3, v.w);
  }
}

// out[m] = value(m) in float32: the finished rows of a split GEMM result.
template <int V4>
__global__ __launch_bounds__(kRowThreads) void finish_rows_kernel(SplitOut o, float* __restrict__ out,
                                                                  size_t ldo, int H) {
  const int m = blockIdx.x;
  SplitAcc<zb_of<V4>()> acc[V4];
#pragma unroll
  for (int k = 0; k < V4; ++k) {
    const int n = 4 * (threadIdx.x + kRowThreads * k);
    if (n < H) split_issue4(o, m, n, acc[k]);
  }
#pragma unroll
  for (int k = 0; k < V4; ++k) {
    const int n = 4 * (threadIdx.x + kRowThreads * k);
    if (n < H) *(float4*)(out + (size_t)m * ldo + n) = split_finish4(o, m, n, acc[k]);
  }
}

// Block keys / values [B, Hkv, S, d] (float32) -> rows [B, S, Hkv, d] in dtype:
// the rows a key/value cache appends.  One workgroup per (b, s).
__global__ void export_kv_kernel(const float* __restrict__ kb, const float* __restrict__ vb, int S,
                                 int Hkv, int d, int dtype, void* __restrict__ k_new,
                                 void* __restrict__ v_new) {
  const int b = blockIdx.x / S, sl = blockIdx.x % S;
  const int n = Hkv * d;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const int h = e / d, i = e % d;
    const size_t src = (((size_t)b * Hkv + h) * S + sl) * d + i;
    const size_t dst = (size_t)blockIdx.x * n + e;
    if (k_new) store_elem(k_new, dtype, dst, kb[src]);
    if (v_new) store_elem(v_new, dtype, dst, vb[src]);
  }
}

// a = silu(g) * u over [rows, F], written as bf16 planes [2][rows][F].
__global__ void swiglu_kernel(SplitOut gs, SplitOut us, uint16_t* __restrict__ a, int rows, int F) {
  const size_t n4 = (size_t)rows * F / 4, pst = (size_t)rows * F;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4;
       e += (size_t)gridDim.x * blockDim.x) {
    const int m = (int)(4 * e / F), n = (int)(4 * e % F);
    SplitAcc<4> pg, pu;
    split_issue4(gs, m, n, pg);
    split_issue4(us, m, n, pu);
    const float4 g = split_finish4(gs, m, n, pg), u = split_finish4(us, m, n, pu);
    const size_t i = 4 * e;
    store_planes(a, pst, i + 0, g.x / (1.0f + expf(-g.x)) * u.x);
    store_planes(a, pst, i + 1, g.y / (1.0f + expf(-g.y)) * u.y);
    store_planes(a, pst, i + 2, g.z / (1.0f + expf(-g.z)) * u.z);
    store_planes(a, pst, i + 3, g.w / (1.0f + expf(-g.w)) * u.w);
  }
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

// float4 groups per thread for a row of H elements (H % 4 == 0, H <= 16384,
// so at most 8 with kRowThreads = 512; the callers validate H).
int v4_of(int H) {
  static_assert(16384 / 4 <= 8 * kRowThreads, "row width");
  const int g = (H / 4 + kRowThreads - 1) / kRowThreads;
  return g <= 1 ? 1 : g <= 2 ? 2 : g <= 4 ? 4 : 8;
}

}  // namespace

SplitOut split_out_plain(const float* C, size_t ldc, int M, int N) {
  SplitOut o{};
  o.C = C;
  o.ldc = ldc;
  o.splits = 1;
  o.M = M;
  o.N = N;
  return o;
}

hipError_t residual_rmsnorm(const SplitOut& x, float* X, size_t ldx, int write_x, const float* g,
                            float eps, uint16_t* y, int rows, int H, hipStream_t s) {
  const size_t pst = (size_t)rows * H;
  switch (v4_of(H)) {
#define DMTP_CASE(n)                                                                               \
  case n:                                                                                          \
    hipLaunchKernelGGL(residual_rmsnorm_kernel<n>, dim3(rows), dim3(kRowThreads), 0, s, x, X, ldx,  \
                       write_x, g, eps, y, pst, H);                                                \
    break;
    DMTP_CASE(1) DMTP_CASE(2) DMTP_CASE(4) DMTP_CASE(8)
#undef DMTP_CASE
  }
  return hipGetLastError();
}

hipError_t fuse_prep(const dmtp_fuse_desc& d, uint16_t* cat, hipStream_t s) {
  const int has_res = d.res.rows != nullptr || d.res.ids != nullptr;
  const RowSrc a = src_of(d.x1, d.w_dtype), b = src_of(d.x2, d.w_dtype), r = src_of(d.res, d.w_dtype);
  const size_t pst = (size_t)d.rows * 2 * d.H;
  switch (v4_of(d.H)) {
#define DMTP_CASE(n)                                                                               \
  case n:                                                                                          \
    hipLaunchKernelGGL(fuse_prep_kernel<n>, dim3(d.rows), dim3(kRowThreads), 0, s, a, b, r,         \
                       has_res, d.g1, d.g2, d.eps, d.H, cat, pst, d.out);                          \
    break;
    DMTP_CASE(1) DMTP_CASE(2) DMTP_CASE(4) DMTP_CASE(8)
#undef DMTP_CASE
  }
  return hipGetLastError();
}

hipError_t build_slots(const dmtp_draft_desc& d, float* X, const float* g, uint16_t* y, hipStream_t s) {
  const int S = d.K - 1 + d.n_anchor;
  const int rows = d.B * S;
  const size_t pst = (size_t)rows * d.H;
  switch (v4_of(d.H)) {
#define DMTP_CASE(n)                                                                               \
  case n:                                                                                          \
    hipLaunchKernelGGL(build_slots_kernel<n>, dim3(rows), dim3(kRowThreads), 0, s, d.anchor_ids,    \
                       d.x_t1, d.emb, d.dtype, d.mask_id, d.V, S, d.n_anchor, d.H, X, g, d.eps, y, \
                       pst);                                                                       \
    break;
    DMTP_CASE(1) DMTP_CASE(2) DMTP_CASE(4) DMTP_CASE(8)
#undef DMTP_CASE
  }
  return hipGetLastError();
}

hipError_t rope_split(const SplitOut& qkv, const int32_t* cu_ctx, int ctx_rows, int B, int S, int Hq,
                      int Hkv, int d, float rope_base, float* q, float* kb, float* vb,
                      hipStream_t s) {
  hipLaunchKernelGGL(rope_split_kernel, dim3(B * S), dim3(256), 0, s, qkv, cu_ctx, ctx_rows, S, Hq,
                     Hkv, d, rope_base, q, kb, vb);
  return hipGetLastError();
}

hipError_t swiglu(const SplitOut& g, const SplitOut& u, uint16_t* a, int rows, int F, hipStream_t s) {
  const size_t n4 = (size_t)rows * F / 4;
  const size_t blocks = (n4 + 255) / 256 < 8192 ? (n4 + 255) / 256 : 8192;
  hipLaunchKernelGGL(swiglu_kernel, dim3((unsigned)blocks), dim3(256), 0, s, g, u, a, rows, F);
  return hipGetLastError();
}

hipError_t to_planes(const void* x, int dtype, size_t n, uint16_t* planes, hipStream_t s) {
  const size_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(to_planes_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, dtype, n, planes);
  return hipGetLastError();
}

hipError_t rope_scatter(const SplitOut& kv, const int32_t* positions, const int32_t* dst_rows, int N,
                        int Hkv, int d, float rope_base, int dtype, int ctx_rows, void* k_cache,
                        void* v_cache, hipStream_t s) {
  hipLaunchKernelGGL(rope_scatter_kernel, dim3(N), dim3(256), 0, s, kv, positions, dst_rows, Hkv, d,
                     rope_base, dtype, ctx_rows, k_cache, v_cache);
  return hipGetLastError();
}

hipError_t finish_rows(const SplitOut& x, float* out, size_t ldo, int rows, int H, hipStream_t s) {
  switch (v4_of(H)) {
#define DMTP_CASE(n)                                                                               \
  case n:                                                                                          \
    hipLaunchKernelGGL(finish_rows_kernel<n>, dim3(rows), dim3(kRowThreads), 0, s, x, out, ldo, H);  \
    break;
    DMTP_CASE(1) DMTP_CASE(2) DMTP_CASE(4) DMTP_CASE(8)
#undef DMTP_CASE
  }
  return hipGetLastError();
}

hipError_t export_kv(const float* kb, const float* vb, int B, int S, int Hkv, int d, int dtype,
                     void* k_new, void* v_new, hipStream_t s) {
  if (!k_new && !v_new) return hipSuccess;
  hipLaunchKernelGGL(export_kv_kernel, dim3(B * S), dim3(256), 0, s, kb, vb, S, Hkv, d, dtype, k_new,
                     v_new);
  return hipGetLastError();
}

hipError_t final_norm_mask(const SplitOut& x, const float* g, float eps, int B, int S, int n_anchor,
                           int K, int H, int dtype, void* out, hipStream_t s) {
  switch (v4_of(H)) {
#define DMTP_CASE(n)                                                                               \
  case n:                                                                                          \
    hipLaunchKernelGGL(final_norm_kernel<n>, dim3(B * (K - 1)), dim3(kRowThreads), 0, s, x, g, eps,  \
                       S, n_anchor, K - 1, H, dtype, out);                                         \
    break;
    DMTP_CASE(1) DMTP_CASE(2) DMTP_CASE(4) DMTP_CASE(8)
#undef DMTP_CASE
  }
  return hipGetLastError();
}

}  // namespace dmtp

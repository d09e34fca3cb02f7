// Shared vocabulary LM head: logits = W x on bf16 matrix cores, with the row
// statistics fused into the GEMM epilogue so that the [M, V] logits never go
// to memory unless a sampled row needs them.
//
//   prep      rows of the segments -> [M, H] head input (RMSNorm + rounding
//             for float32 hidden segments)
//   gemm      per (vocab tile, row tile): running max, lowest-index argmax,
//             second-best value and sum of exp((l - max) / t) per row, written
//             as one 16-byte partial per (row, vocab tile); logits rows with a
//             store index are written in float32
//   merge     per row: exact merge of the partials -> max, lse, argmax, gap
//   plan/scan (only when temperatures are given) Gumbel-max draws over the
//             stored logits rows of sampled rows, in vocabulary chunks
//   finalize  token per row: draw, planted row argmax, or argmax
#include <cstdlib>
#include <type_traits>

#include "dma.hpp"
#include "gemm_core.hpp"
#include "kernels.hpp"

namespace dmtp {

namespace {

struct RowStat {
  float m;    // max logit of the tile
  float s;    // sum exp((l - m) / t)
  int idx;    // argmax (lowest index)
  float v2;   // second-best logit
};

__device__ __forceinline__ RowStat stat_merge(const RowStat& a, const RowStat& b, float inv_t) {
  RowStat r;
  Top2 ta{a.m, a.idx, a.v2}, tb{b.m, b.idx, b.v2};
  Top2 t = top2_merge(ta, tb);
  r.m = t.v1;
  r.idx = t.i1;
  r.v2 = t.v2;
  const float sc = inv_t * 1.4426950408889634f;
  const float wa = a.s > 0.f ? a.s * hw_exp2((a.m - r.m) * sc) : 0.f;
  const float wb = b.s > 0.f ? b.s * hw_exp2((b.m - r.m) * sc) : 0.f;
  r.s = wa + wb;
  return r;
}

// v_max / v_min / v_max3 as the hardware executes them.  fmaxf on a value of
// unknown origin (here: accumulators read from AGPRs) is compiled with an
// extra quieting instruction per input; the row statistics never see
// signalling NaNs, so that step is skipped.
__device__ __forceinline__ float hw_max(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float hw_min(float a, float b) {
  float r;
  asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float hw_max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ RowStat stat_empty() { return RowStat{-INFINITY, 0.f, 0x7FFFFFFF, -INFINITY}; }

struct Seg {
  const void* x;
  int n, ld, dtype;
  const float* g;
};

struct HeadParams {
  Seg seg[4];
  int n_seg, M, H, V, dtype;
  float eps;
  const void* W;
  const float* temperature;
  const uint64_t* draw_key;
  uint64_t seed;
  const int32_t* plant_row;
  const int32_t* store_row;
  float* logits;
  int logits_rows;
  void* prepared;        // [M, H] head input
  const void* A;         // rows the GEMM reads: prepared, or the single input segment
  RowStat* part;         // [M, n_vtiles]
  int n_vtiles;
  int32_t* amax;         // [M]
  float* gap_greedy;     // [M]
  int32_t* list;         // [M] sampled rows
  int32_t* list_pos;     // [M] position in list or -1
  int32_t* list_count;   // [1]
  Top2* scan_part;       // [M, n_chunks]
  int n_chunks;
  int32_t* token;
  float* row_max;
  float* lse;
  float* gap;
};

constexpr int kPrepThreads = 256;

__global__ __launch_bounds__(kPrepThreads) void head_prep_kernel(HeadParams p) {
  __shared__ double red[kPrepThreads / kWave];
  int m = blockIdx.x, si = 0;
  while (si < p.n_seg - 1 && m >= p.seg[si].n) {
    m -= p.seg[si].n;
    ++si;
  }
  const Seg sg = p.seg[si];
  const int H = p.H;
  const size_t orow = (size_t)blockIdx.x * H;
  if (sg.g) {
    const float* xr = (const float*)sg.x + (size_t)m * sg.ld;
    double ss = 0.0;
    for (int i = threadIdx.x; i < H; i += blockDim.x) ss += (double)xr[i] * xr[i];
    ss = wave_sum(ss);
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = ss;
    __syncthreads();
    double t = 0.0;
    for (int w = 0; w < kPrepThreads / kWave; ++w) t += red[w];
    const double inv = 1.0 / sqrt(t / H + (double)p.eps);
    for (int i = threadIdx.x; i < H; i += blockDim.x)
      store_elem(p.prepared, p.dtype, orow + i, (float)((double)xr[i] * inv * sg.g[i]));
  } else if (p.dtype == DMTP_BF16) {
    const uint16_t* xr = (const uint16_t*)sg.x + (size_t)m * sg.ld;
    for (int i = threadIdx.x; i < H; i += blockDim.x) ((uint16_t*)p.prepared)[orow + i] = xr[i];
  } else {
    const float* xr = (const float*)sg.x + (size_t)m * sg.ld;
    for (int i = threadIdx.x; i < H; i += blockDim.x) ((float*)p.prepared)[orow + i] = xr[i];
  }
}

__device__ __forceinline__ float inv_temp(const float* temperature, int m) {
  if (!temperature) return 1.f;
  const float t = temperature[m];
  return t > 0.f ? 1.f / t : 1.f;
}

template <class T>
__global__ __launch_bounds__(T::THREADS) void head_gemm_kernel(HeadParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[T::LDS_A + T::LDS_B];
  __shared__ RowStat wstat[T::WAVES_N][T::BM];
  const int n0 = blockIdx.x * T::BN, m0 = blockIdx.y * T::BM;
  Acc<T> acc;
  gemm_mainloop<T, true>(acc, lds, p.A, (size_t)p.H, 0, p.M, p.W, (size_t)p.H, p.V, m0, n0, 0, p.H);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wmi = wave / T::WAVES_N, wni = wave % T::WAVES_N;
  const int wm0 = wmi * T::WM, wn0 = wni * T::WN;
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int lrow = wm0 + 16 * i + 4 * (lane >> 4) + r;
      const int row = m0 + lrow;
      const bool row_ok = row < p.M;
      const float it = row_ok ? inv_temp(p.temperature, row) : 1.f;
      int srow = (row_ok && p.store_row) ? p.store_row[row] : -1;
      if (srow >= p.logits_rows) srow = -1;
      Top2 t = top2_empty();
#pragma unroll
      for (int j = 0; j < T::TN; ++j) {
        const int col = n0 + wn0 + 16 * j + (lane & 15);
        if (col < p.V) {
          const float v = acc.v[i][j][r];
          top2_push(t, v, col);
          if (srow >= 0) p.logits[(size_t)srow * p.V + col] = v;
        }
      }
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < T::TN; ++j) {
        const int col = n0 + wn0 + 16 * j + (lane & 15);
        if (col < p.V) s += expf((acc.v[i][j][r] - t.v1) * it);
      }
      RowStat st{t.v1, s, t.i1, t.v2};
      // reduce over the 16 lanes that share this row
#pragma unroll
      for (int mask = 1; mask < 16; mask <<= 1) {
        RowStat o;
        o.m = shfl_xor(st.m, mask);
        o.s = shfl_xor(st.s, mask);
        o.idx = shfl_xor(st.idx, mask);
        o.v2 = shfl_xor(st.v2, mask);
        st = stat_merge(st, o, it);
      }
      if ((lane & 15) == 0) wstat[wni][lrow] = st;
    }
  __syncthreads();
  for (int lr = threadIdx.x; lr < T::BM; lr += T::THREADS) {
    const int row = m0 + lr;
    if (row >= p.M) continue;
    const float it = inv_temp(p.temperature, row);
    RowStat st = wstat[0][lr];
    for (int w = 1; w < T::WAVES_N; ++w) st = stat_merge(st, wstat[w][lr], it);
    p.part[(size_t)row * p.n_vtiles + blockIdx.x] = st;
  }
}

// ---- bf16 head GEMM: vocabulary rows on the MFMA row side.
//
// Workgroup tile: 128 vocabulary rows x (64 * NBW) head-input rows; wave w owns
// input rows 64 w .. 64 w + 63 against all 128 vocabulary rows (4 x 2 tiles of
// 32 x 32).  With the vocabulary on the row side, a lane's accumulators hold
// 64 logits of each of its two input rows, so the per-row statistics reduce
// inside the lane and across one lane pair only.  All input rows of a chunk
// (up to 448) share one pass over W, which is read from HBM once per chunk.
//
// Data movement per 128-wide K slice: the W slice (128 x 128, shared by every
// wave) goes through registers into one of two LDS buffers, 16-byte chunks
// XOR-swizzled by row, and is fetched two slices ahead; each wave's input-row
// fragments come straight from L2 into registers one slice ahead (no LDS: no
// other wave reads them).  Inside a slice, lane half h supplies k = 64 h + 8 kk
// .. + 7 at step kk, so a lane's eight input-row fragments are 128 contiguous
// bytes; the W fragments read from LDS use the same k assignment.
template <int NBW>
struct HeadBig {
  static constexpr int BV = 128, BK = 128, BB = 64 * NBW, THREADS = 64 * NBW;
  static constexpr int KSTEPS = BK / 16;                    // MFMA k-steps per slice
  static constexpr int W_CH = BV * BK / 8;                  // 16-byte chunks per W slice
  static constexpr int WPT = (W_CH + THREADS - 1) / THREADS;
  static constexpr int STAGE = BV * BK;                     // bf16 elements per W buffer
  static constexpr size_t LDS_BYTES = (size_t)2 * STAGE * 2;
};

__device__ __forceinline__ int swz64(int r, int c) { return r * 64 + ((c ^ (r & 7)) << 3); }
// row r, 16-byte chunk c of a [rows][128] bf16 tile, chunks XOR-swizzled by row
__device__ __forceinline__ int swz128(int r, int c) { return r * 128 + ((c ^ (r & 15)) << 3); }



template <int NBW>
__global__ __launch_bounds__(HeadBig<NBW>::THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void head_gemm_big_kernel(HeadParams p, int n_mchunks) {
  typedef HeadBig<NBW> C;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int total = p.n_vtiles * n_mchunks;
  // Workgroup i runs on XCD i % 8: each XCD gets a contiguous range of
  // (vocabulary tile, row chunk) pairs, so the row chunks of one vocabulary
  // tile meet in the same L2.
  const int per = (total + 7) / 8;
  const int t = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (t >= total) return;
  const int vt = t / n_mchunks, mc = t % n_mchunks;
  const int v0 = vt * C::BV, m0 = mc * C::BB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, lk = lane >> 5;
  const int H = p.H, V = p.V, M = p.M;
  const uint16_t* __restrict__ W = (const uint16_t*)p.W;
  const uint16_t* __restrict__ X = (const uint16_t*)p.A;
  // Loads clamp their row into range instead of branching: rows past V or M
  // only feed accumulators that the epilogue never reads.
  const uint16_t* wsrc[C::WPT];
  int wdst[C::WPT];
#pragma unroll
  for (int s = 0; s < C::WPT; ++s) {
    const int idx = min(tid + s * C::THREADS, C::W_CH - 1);
    const int r = idx >> 4, c = idx & 15;
    wsrc[s] = W + (size_t)min(v0 + r, V - 1) * H + 8 * c;
    wdst[s] = swz128(r, c);
  }
  // lane half lk supplies k = 64 lk + 8 kk .. + 7 at step kk of a slice
  const uint16_t* xp0 = X + (size_t)min(m0 + 64 * wave + lr, M - 1) * H + 64 * lk;
  const uint16_t* xp1 = X + (size_t)min(m0 + 64 * wave + 32 + lr, M - 1) * H + 64 * lk;

  f32x16_t acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  auto gload_w = [&](u32x4* wr, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < C::WPT; ++s) wr[s] = *(const u32x4*)(wsrc[s] + k0);
  };
  auto store_w = [&](const u32x4* wr, uint16_t* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < C::WPT; ++s) *(u32x4*)(buf + wdst[s]) = wr[s];
  };
  auto gload_x = [&](u32x4* x0, u32x4* x1, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      x0[kk] = *(const u32x4*)(xp0 + k0 + 8 * kk);
      x1[kk] = *(const u32x4*)(xp1 + k0 + 8 * kk);
    }
  };
  auto compute = [&](const uint16_t* cur, const u32x4* x0, const u32x4* x1)
                     __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < C::KSTEPS; ++kk) {
      u32x4 a_[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        a_[u] = *(const u32x4*)(cur + swz128(32 * u + lr, C::KSTEPS * lk + kk));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[u][0] = mfma32(a_[u], x0[kk], acc[u][0]);
        acc[u][1] = mfma32(a_[u], x1[kk], acc[u][1]);
      }
    }
  };

  const int nK = H / C::BK;
  const int last = (nK - 1) * C::BK;
  uint16_t* buf0 = smem;
  uint16_t* buf1 = smem + C::STAGE;
  u32x4 wA[C::WPT], wB[C::WPT];
  u32x4 xa0[C::KSTEPS], xa1[C::KSTEPS], xb0[C::KSTEPS], xb1[C::KSTEPS];
  gload_w(wA, 0);
  gload_w(wB, min(C::BK, last));
  gload_x(xa0, xa1, 0);
  store_w(wA, buf0);
  __syncthreads();
  // Two K slices per trip keep every register ring index static.  Slice kt
  // computes from buf0 / xa while W of slice kt + 1 (in wB) and kt + 2 (into
  // wA) are in flight.  Past the end the loads repeat the last slice, which
  // nothing reads.
  int kt = 0;
  for (; kt + 1 < nK; kt += 2) {
    gload_w(wA, min((kt + 2) * C::BK, last));
    gload_x(xb0, xb1, (kt + 1) * C::BK);
    compute(buf0, xa0, xa1);
    store_w(wB, buf1);
    __syncthreads();
    gload_w(wB, min((kt + 3) * C::BK, last));
    gload_x(xa0, xa1, min((kt + 2) * C::BK, last));
    compute(buf1, xb0, xb1);
    store_w(wA, buf0);
    __syncthreads();
  }
  if (kt < nK) compute(buf0, xa0, xa1);   // odd slice count: the last sits in buf0 / xa

  // ---- epilogue: statistics of each of the lane's two input rows
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int m = m0 + 64 * wave + 32 * j + lr;
    const bool m_ok = m < M;
    const float it = m_ok ? inv_temp(p.temperature, m) : 1.f;
    int srow = (m_ok && p.store_row) ? p.store_row[m] : -1;
    if (srow >= p.logits_rows) srow = -1;
    Top2 tp = top2_empty();
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int v = v0 + 32 * u + 8 * (i >> 2) + 4 * lk + (i & 3);
        if (v < V) top2_push(tp, acc[u][j][i], v);
      }
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int v = v0 + 32 * u + 8 * (i >> 2) + 4 * lk + (i & 3);
        if (v < V) sum += expf((acc[u][j][i] - tp.v1) * it);
      }
    if (srow >= 0) {
      float* dst = p.logits + (size_t)srow * V;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int v = v0 + 32 * u + 8 * (i >> 2) + 4 * lk + (i & 3);
          if (v < V) dst[v] = acc[u][j][i];
        }
    }
    RowStat st{tp.v1, sum, tp.i1, tp.v2};
    RowStat o;
    o.m = shfl_xor(st.m, 32);
    o.s = shfl_xor(st.s, 32);
    o.idx = shfl_xor(st.idx, 32);
    o.v2 = shfl_xor(st.v2, 32);
    st = stat_merge(st, o, it);
    if (lk == 0 && m_ok) p.part[(size_t)m * p.n_vtiles + vt] = st;
  }
}

// ---- bf16 head GEMM for at most 64 head-input rows (the MTP candidate rows).
//
// Weight-streaming and HBM-bound: every wave owns 128 vocabulary rows and
// reads them straight from HBM into registers in MFMA fragment order (64
// contiguous bytes per lane and row per half K slice, two in flight); the few input rows are fragments read from L2.  No LDS and no
// barriers, so all ~1200 waves of a 151936-row vocabulary are resident at once
// and keep enough bytes in flight to cover HBM latency.  The epilogue is the
// one of the big kernel (same partial layout).
template <int NB>   // 32-row input tiles: 1 (M <= 32) or 2 (M <= 64)
__global__ __launch_bounds__(256) void head_gemm_skinny_kernel(HeadParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int vt = blockIdx.x * 4 + wave;
  if (vt >= p.n_vtiles) return;
  const int lr = lane & 31, lk = lane >> 5;
  const int H = p.H, V = p.V, M = p.M;
  const int v0 = vt * 128;
  const uint16_t* __restrict__ W = (const uint16_t*)p.W;
  const uint16_t* __restrict__ X = (const uint16_t*)p.A;
  // Same k grouping per MFMA as the big kernel (lane half lk supplies
  // k = 128 s + 64 lk + 8 kk .. + 7 at step kk of slice s), issued in two
  // half-slices of four steps, so every row gets bit-identical logits
  // whichever kernel its launch size selects.
  const uint16_t* wp[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) wp[u] = W + (size_t)min(v0 + 32 * u + lr, V - 1) * H + 64 * lk;
  const uint16_t* xp[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) xp[j] = X + (size_t)min(32 * j + lr, M - 1) * H + 64 * lk;

  f32x16_t acc[4][NB];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[u][j][i] = 0.f;

  auto load = [&](u32x4 (&w)[4][4], u32x4 (&x)[NB][4], int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) w[u][kk] = *(const u32x4*)(wp[u] + k0 + 8 * kk);
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) x[j][kk] = *(const u32x4*)(xp[j] + k0 + 8 * kk);
  };
  auto compute = [&](const u32x4 (&w)[4][4], const u32x4 (&x)[NB][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[u][j] = mfma32(w[u][kk], x[j][kk], acc[u][j]);
  };
  // half-slice hs covers steps 4 (hs & 1) .. + 3 of slice hs / 2
  auto k_of = [](int hs) { return 128 * (hs >> 1) + 32 * (hs & 1); };
  const int nH = H / 64;            // half-slices (H is a multiple of 128)
  u32x4 wa[4][4], wb[4][4], xa[NB][4], xb[NB][4];
  load(wa, xa, 0);
  for (int hs = 0; hs < nH; hs += 2) {
    load(wb, xb, k_of(hs + 1));
    compute(wa, xa);
    load(wa, xa, k_of(min(hs + 2, nH - 1)));
    compute(wb, xb);
  }

#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int m = 32 * j + lr;
    const bool m_ok = m < M;
    const float it = m_ok ? inv_temp(p.temperature, m) : 1.f;
    int srow = (m_ok && p.store_row) ? p.store_row[m] : -1;
    if (srow >= p.logits_rows) srow = -1;
    Top2 tp = top2_empty();
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int v = v0 + 32 * u + 8 * (i >> 2) + 4 * lk + (i & 3);
        if (v < V) top2_push(tp, acc[u][j][i], v);
      }
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int v = v0 + 32 * u + 8 * (i >> 2) + 4 * lk + (i & 3);
        if (v < V) sum += expf((acc[u][j][i] - tp.v1) * it);
      }
    if (srow >= 0) {
      float* dst = p.logits + (size_t)srow * V;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int v = v0 + 32 * u + 8 * (i >> 2) + 4 * lk + (i & 3);
          if (v < V) dst[v] = acc[u][j][i];
        }
    }
    RowStat st{tp.v1, sum, tp.i1, tp.v2};
    RowStat o;
    o.m = shfl_xor(st.m, 32);
    o.s = shfl_xor(st.s, 32);
    o.idx = shfl_xor(st.idx, 32);
    o.v2 = shfl_xor(st.v2, 32);
    st = stat_merge(st, o, it);
    if (lk == 0 && m_ok) p.part[(size_t)m * p.n_vtiles + vt] = st;
  }
}

// ---- bf16 head GEMM, LDS-DMA version.
//
// Workgroup: 4 waves, 128 vocabulary rows x 64 T head-input rows (a row chunk);
// wave w computes the 128 vocabulary rows against its own 16 T input rows with
// 16 x 16 x 32 MFMAs (8 x T accumulator tiles, held in AGPRs).  T = 7 covers
// 448 rows, the draft + target rows of a batch-32 round, without padding.
//
// K runs in 32-wide slices through a ring of four LDS stages filled by
// global_load_lds_dwordx4 (no register staging): each instruction moves 64 x 16
// bytes, and lane i fetches the 16-byte chunk that belongs at LDS position i of
// the XOR-swizzled tile, so every instruction reads whole 64-byte row segments
// from memory.  Slice s + 3 is requested while slice s is computed; a wave waits
// only for its own requests of slice s (s_waitcnt vmcnt) and a barrier makes the
// other waves' parts visible.  Vocabulary rows are on the MFMA row side, so the
// per-row statistics reduce inside a lane (32 logits per input row and lane)
// and across the four lanes that share an input row.
template <int T>
struct HeadLds {
  static constexpr int BV = 128, BK = 32, NBUF = 4, WAVES = 4, THREADS = 256;
  static constexpr int BB = 64 * T;                 // input rows per chunk
  static constexpr int W_INSTR = BV * BK / 8 / 64;  // 16-byte DMA instructions per slice (8)
  static constexpr int X_INSTR = BB * BK / 8 / 64;  // (4 T)
  static constexpr int PER_WAVE = (W_INSTR + X_INSTR) / WAVES;   // 2 + T
  static constexpr int STAGE = (BV + BB) * BK;      // bf16 elements per stage
  static constexpr size_t LDS_BYTES = (size_t)NBUF * STAGE * 2;
};

// position of 16-byte chunk c (0..3) of row r in a [rows][32] bf16 tile
__device__ __forceinline__ int swz32(int r, int c) { return r * 32 + ((c ^ ((r >> 1) & 3)) << 3); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2)))
void head_gemm_lds_kernel(HeadParams p, int n_mchunks) {
  typedef HeadLds<T> C;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int total = p.n_vtiles * n_mchunks;
  const int per = (total + 7) / 8;   // XCD-contiguous ranges (workgroup i runs on XCD i % 8)
  const int tt = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (tt >= total) return;
  const int vt = tt / n_mchunks, mc = tt % n_mchunks;
  const int v0 = vt * C::BV, m0 = mc * C::BB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int H = p.H, V = p.V, M = p.M;
  const uint16_t* __restrict__ W = (const uint16_t*)p.W;
  const uint16_t* __restrict__ X = (const uint16_t*)p.A;

  // DMA sources of this lane (rows clamped into range: their results are unused)
  const uint16_t* wsrc[C::W_INSTR / C::WAVES];
#pragma unroll
  for (int q = 0; q < C::W_INSTR / C::WAVES; ++q) {
    const int instr = wave * (C::W_INSTR / C::WAVES) + q;
    const int idx = instr * 64 + lane, r = idx >> 2, pos = idx & 3;
    const int c = pos ^ ((r >> 1) & 3);
    wsrc[q] = W + (size_t)min(v0 + r, V - 1) * H + 8 * c;
  }
  const uint16_t* xsrc[T];
#pragma unroll
  for (int q = 0; q < T; ++q) {
    const int instr = wave * T + q;
    const int idx = instr * 64 + lane, r = idx >> 2, pos = idx & 3;
    const int c = pos ^ ((r >> 1) & 3);
    xsrc[q] = X + (size_t)min(m0 + r, M - 1) * H + 8 * c;
  }
  auto issue = [&](int slice) __attribute__((always_inline)) {
    uint16_t* st = smem + (slice % C::NBUF) * C::STAGE;
    const int k0 = slice * C::BK;
#pragma unroll
    for (int q = 0; q < C::W_INSTR / C::WAVES; ++q) {
      const int instr = wave * (C::W_INSTR / C::WAVES) + q;
      __builtin_amdgcn_global_load_lds((const void*)(wsrc[q] + k0),
                                       (__attribute__((address_space(3))) void*)(st + instr * 512),
                                       16, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < T; ++q) {
      const int instr = wave * T + q;
      __builtin_amdgcn_global_load_lds((const void*)(xsrc[q] + k0),
                                       (__attribute__((address_space(3))) void*)(st + C::BV * C::BK +
                                                                                  instr * 512),
                                       16, 0, 0);
    }
  };

  f32x4_t acc[8][T];
#pragma unroll
  for (int u = 0; u < 8; ++u)
#pragma unroll
    for (int t = 0; t < T; ++t) acc[u][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, fq = lane >> 4;
  const int nK = H / C::BK;
#pragma unroll
  for (int s0 = 0; s0 < C::NBUF - 1; ++s0)
    if (s0 < nK) issue(s0);
  for (int ks = 0; ks < nK; ++ks) {
    const int newer = nK - 1 - ks;   // slices requested after ks and still possibly in flight
    if (newer >= 2)
      wait_vmcnt<2 * C::PER_WAVE>();
    else if (newer == 1)
      wait_vmcnt<C::PER_WAVE>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (ks + C::NBUF - 1 < nK) issue(ks + C::NBUF - 1);
    const uint16_t* st = smem + (ks % C::NBUF) * C::STAGE;
    u32x4 a[8], b[T];
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] = *(const u32x4*)(st + swz32(16 * u + fr, fq));
#pragma unroll
    for (int t = 0; t < T; ++t)
      b[t] = *(const u32x4*)(st + C::BV * C::BK + swz32(16 * T * wave + 16 * t + fr, fq));
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int t = 0; t < T; ++t)
        acc[u][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[u]),
                                                            __builtin_bit_cast(bf16x8_t, b[t]),
                                                            acc[u][t], 0, 0, 0);
  }

  // ---- epilogue: lane holds, for each of its T input rows, 32 vocabulary logits
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int m = m0 + 16 * T * wave + 16 * t + fr;
    const bool m_ok = m < M;
    const float it = m_ok ? inv_temp(p.temperature, m) : 1.f;
    int srow = (m_ok && p.store_row) ? p.store_row[m] : -1;
    if (srow >= p.logits_rows) srow = -1;
    Top2 tp = top2_empty();
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = v0 + 16 * u + 4 * fq + i;
        if (v < V) top2_push(tp, acc[u][t][i], v);
      }
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = v0 + 16 * u + 4 * fq + i;
        if (v < V) sum += expf((acc[u][t][i] - tp.v1) * it);
      }
    if (srow >= 0) {
      float* dst = p.logits + (size_t)srow * V;
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = v0 + 16 * u + 4 * fq + i;
          if (v < V) dst[v] = acc[u][t][i];
        }
    }
    RowStat st{tp.v1, sum, tp.i1, tp.v2};
#pragma unroll
    for (int mask = 16; mask < 64; mask <<= 1) {
      RowStat o;
      o.m = shfl_xor(st.m, mask);
      o.s = shfl_xor(st.s, mask);
      o.idx = shfl_xor(st.idx, mask);
      o.v2 = shfl_xor(st.v2, mask);
      st = stat_merge(st, o, it);
    }
    if (fq == 0 && m_ok) p.part[(size_t)m * p.n_vtiles + vt] = st;
  }
}

template <int T>
hipError_t launch_head_lds(const HeadParams& p, int n_mchunks, hipStream_t s) {
  typedef HeadLds<T> C;
  static_assert(C::LDS_BYTES <= 160 * 1024, "head LDS");
  hipError_t e = hipFuncSetAttribute((const void*)head_gemm_lds_kernel<T>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int total = p.n_vtiles * n_mchunks;
  hipLaunchKernelGGL(head_gemm_lds_kernel<T>, dim3(8 * ((total + 7) / 8)), dim3(C::THREADS),
                     C::LDS_BYTES, s, p, n_mchunks);
  return hipGetLastError();
}

// ---- bf16 head GEMM, 32 x 32 x 16 MFMA version.
//
// Workgroup: 4 waves on 128 vocabulary rows x 64 TB head-input rows; wave w
// takes vocabulary half (w & 1) (64 rows) against input half (w >> 1) (32 TB
// rows): 2 x TB accumulator tiles of 32 x 32 held in AGPRs (TB = 7: 448 rows,
// the draft + target rows of a batch-32 round, in one pass over W).  K runs in
// BK-wide slices through an LDS ring filled by global_load_lds_dwordx4; each
// wave reads the fragments of the next 16-wide k-step from LDS while the MFMAs
// of the current one drain, so neither the LDS latency nor the barrier sits on
// the matrix-core critical path.  16-byte chunks are XOR-swizzled per row
// (swz_chunk), which keeps the lanes of a read pass on distinct banks.  The two
// vocabulary halves' row statistics meet in LDS.
// Default ring depth: as many stages as fit 144 KB of LDS (at most 12), so that
// the weight-streaming calls with few rows keep enough copies in flight.
constexpr int head_mf32_nbuf(int TB, int BK) {
  return (147456 / ((128 + 64 * TB) * BK * 2)) > 12 ? 12 : (147456 / ((128 + 64 * TB) * BK * 2));
}

template <int TB, int BK_ = 32, int NBUF_ = head_mf32_nbuf(TB, BK_)>
struct HeadMf32 {
  static constexpr int BV = 128, BK = BK_, NBUF = NBUF_, THREADS = 256;
  static constexpr int BB = 64 * TB;
  static constexpr int CPR = BK / 8;                  // 16-byte chunks per row
  static constexpr int KS = BK / 16;                  // MFMA k-steps per slice
  static constexpr int W_INSTR = BV * BK * 2 / 1024;  // 1 KB copies per slice
  static constexpr int X_INSTR = BB * BK * 2 / 1024;
  static constexpr int WPW = W_INSTR / 4, XPW = X_INSTR / 4;   // per wave
  static constexpr int PER_WAVE = WPW + XPW;
  static constexpr int STAGE = (BV + BB) * BK;
  static constexpr size_t LDS_BYTES = (size_t)NBUF * STAGE * 2;
  static_assert(W_INSTR % 4 == 0 && X_INSTR % 4 == 0 && KS % 2 == 0, "tile");
};

template <int TB, int BK, int NBUF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void head_gemm_mf32_kernel(HeadParams p, int n_mchunks) {
  typedef HeadMf32<TB, BK, NBUF> C;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int total = p.n_vtiles * n_mchunks;
  const int per = (total + 7) / 8;   // XCD-contiguous ranges (workgroup i runs on XCD i % 8)
  const int tt = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (tt >= total) return;
  const int vt = tt / n_mchunks, mc = tt % n_mchunks;
  const int v0 = vt * C::BV, m0 = mc * C::BB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int vh = wave & 1, bh = wave >> 1;
  const int lr = lane & 31, lk = lane >> 5;
  const int H = p.H, V = p.V, M = p.M;
  const uint16_t* __restrict__ W = (const uint16_t*)p.W;
  const uint16_t* __restrict__ X = (const uint16_t*)p.A;

  // Raw per-row inputs of the epilogue, loaded ahead of the main loop so that
  // their memory latency is spent under it rather than once per row group at
  // the end (one wave per SIMD leaves nothing else to hide it).
  float t_in[TB];   // temperature of the lane's row in tile t (1 when none given)
  int s_in[TB];     // logits store index of that row (-1: none)
#pragma unroll
  for (int t = 0; t < TB; ++t) {
    const int m = m0 + 32 * TB * bh + 32 * t + lr;
    const bool ok = m < M;
    t_in[t] = (ok && p.temperature) ? p.temperature[m] : 1.f;
    s_in[t] = (ok && p.store_row) ? p.store_row[m] : -1;
  }
  constexpr int NFIN = (C::BB + C::THREADS - 1) / C::THREADS;
  float tf_in[NFIN];   // temperatures of the rows this thread writes partials for
#pragma unroll
  for (int j = 0; j < NFIN; ++j) {
    const int r = threadIdx.x + j * C::THREADS;
    tf_in[j] = (r < C::BB && m0 + r < M && p.temperature) ? p.temperature[m0 + r] : 1.f;
  }

  // Copy q of a slice (q < WPW: W rows, then input rows): lane's source is row
  // idx / CPR of the tile, the chunk that lands at position idx % CPR (rows past
  // the end are clamped; their results are unused); dst its 1 KB block.
  const uint16_t* src[C::PER_WAVE];
  int dst[C::PER_WAVE];
#pragma unroll
  for (int q = 0; q < C::PER_WAVE; ++q) {
    if (q < C::WPW) {
      const int idx = (wave * C::WPW + q) * 64 + lane, r = idx / C::CPR;
      src[q] = W + (size_t)min(v0 + r, V - 1) * H + 8 * swz_chunk<BK>(r, idx % C::CPR);
      dst[q] = (wave * C::WPW + q) * 512;
    } else {
      const int qq = q - C::WPW;
      const int idx = (wave * C::XPW + qq) * 64 + lane, r = idx / C::CPR;
      src[q] = X + (size_t)min(m0 + r, M - 1) * H + 8 * swz_chunk<BK>(r, idx % C::CPR);
      dst[q] = C::BV * C::BK + (wave * C::XPW + qq) * 512;
    }
  }
  auto issue_one = [&](int slice, int q) __attribute__((always_inline)) {
    lds_dma16(src[q] + slice * C::BK, smem + (slice % C::NBUF) * C::STAGE + dst[q]);
  };
  // fragments of one 16-wide k-step
  struct Frag {
    u32x4 a[2];    // vocabulary tiles
    u32x4 b[TB];   // input tiles
  };
  auto read = [&](Frag& f, int slice, int ks) __attribute__((always_inline)) {
    const uint16_t* st = smem + (slice % C::NBUF) * C::STAGE;
#pragma unroll
    for (int u = 0; u < 2; ++u) f.a[u] = *(const u32x4*)(st + swz_row<BK>(64 * vh + 32 * u + lr, 2 * ks + lk));
#pragma unroll
    for (int t = 0; t < TB; ++t)
      f.b[t] = *(const u32x4*)(st + C::BV * C::BK + swz_row<BK>(32 * TB * bh + 32 * t + lr, 2 * ks + lk));
  };
  f32x16_t acc[2][TB];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[u][t][i] = 0.f;
  const int nK = H / C::BK;
  // With three or more stages the copies of slice s + NBUF - 1 are spread over
  // the MFMA pairs of slice s (copy q after pair q * PAIRS / PER_WAVE), so the
  // wave never stalls on a burst of copies while the matrix unit idles.  With
  // two stages every copy of the next slice must be issued before the wait for
  // it, so they go out in one burst after the barrier.
  constexpr bool INTER = C::NBUF >= 3;
  constexpr int PAIRS = C::KS * TB;
  auto compute = [&](const Frag& f, int ks, int s_fill) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < TB; ++t) {
#pragma unroll
      for (int u = 0; u < 2; ++u) acc[u][t] = mfma32(f.a[u], f.b[t], acc[u][t]);
      if constexpr (INTER) {
#pragma unroll
        for (int q = 0; q < C::PER_WAVE; ++q)
          if ((q * PAIRS) / C::PER_WAVE == ks * TB + t && s_fill < nK) issue_one(s_fill, q);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // copies of the slice being filled that go out before the wait at the last k-step
  constexpr int Q_BEFORE = [] {
    int c = 0;
    for (int q = 0; q < C::PER_WAVE; ++q)
      if ((q * PAIRS) / C::PER_WAVE < (C::KS - 1) * TB) ++c;
    return c;
  }();
  // Slice s is in LDS for every wave once this wave's own copies of it have
  // landed -- vmcnt allows exactly the copies issued after them to stay in
  // flight -- and all waves passed the barrier.  lgkmcnt(0) first: the buffer
  // the next copies refill was read into registers just before, by every wave.
  auto wait_slice = [&](int s) __attribute__((always_inline)) {
    if constexpr (!INTER) {
      wait_newer<C::PER_WAVE, C::NBUF - 2>(min(nK - 1 - s, C::NBUF - 2));
    } else {
      // issued after slice s: slices s+1 .. s+NBUF-3 whole (those that exist) and
      // Q_BEFORE copies of slice s+NBUF-2 (the one being filled, if it exists).
      // In the prologue slice NBUF-2 is already whole, so this waits longer than
      // needed there, never shorter.
      constexpr int STEADY = (C::NBUF - 3) * C::PER_WAVE + Q_BEFORE;
      if (s + C::NBUF - 2 < nK) {
        wait_vm_lgkm0<STEADY>();
      } else {
        const int full = nK - 1 - s > C::NBUF - 3 ? C::NBUF - 3 : (nK - 1 - s < 0 ? 0 : nK - 1 - s);
        wait_vm_dyn<STEADY>(full * C::PER_WAVE);
      }
    }
    ring_barrier();
  };

#pragma unroll
  for (int s0 = 0; s0 < C::NBUF - 1; ++s0)
    if (s0 < nK)
#pragma unroll
      for (int q = 0; q < C::PER_WAVE; ++q) issue_one(s0, q);
  Frag f0, f1;
  wait_slice(0);
  if (!INTER && C::NBUF - 1 < nK)
#pragma unroll
    for (int q = 0; q < C::PER_WAVE; ++q) issue_one(C::NBUF - 1, q);
  read(f0, 0, 0);
  // the next k-step's fragments are read from LDS while this one's MFMAs drain;
  // the k-steps run in increasing k whatever BK is, so results do not depend on it
  for (int s = 0; s < nK; ++s) {
    const int s_fill = s + C::NBUF - 1;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      Frag& cur = (ks & 1) ? f1 : f0;
      Frag& nxt = (ks & 1) ? f0 : f1;
      if (ks + 1 < C::KS) {
        read(nxt, s, ks + 1);
      } else if (s + 1 < nK) {
        wait_slice(s + 1);
        if (!INTER && s + C::NBUF < nK)
#pragma unroll
          for (int q = 0; q < C::PER_WAVE; ++q) issue_one(s + C::NBUF, q);
        read(nxt, s + 1, 0);
      }
      compute(cur, ks, s_fill);
    }
  }

  // ---- epilogue: per input row, 32 logits in the lane (element e = 16 u + i
  // sits at vocabulary offset off(e) from the lane's first column, rising with
  // e); merge the lane pair (xor 32), then the two vocabulary halves in LDS.
  __syncthreads();
  RowStat* xch = (RowStat*)smem;   // [2 vocabulary halves][BB rows]
  const int vl = v0 + 64 * vh + 4 * lk;
  auto off = [](int e) { return 32 * (e >> 4) + 8 * ((e & 15) >> 2) + (e & 3); };
  // TAIL: the last vocabulary tile, whose columns past V hold clamped rows and
  // are masked out; every other tile takes the path without the checks.
  auto row_stats = [&](auto TAIL) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      // Pin this tile's accumulators in AGPRs up to here, so that the copies to
      // VGPRs are made one tile at a time rather than all at the loop exit.
      asm volatile("" : "+a"(acc[0][t]), "+a"(acc[1][t])::"memory");
      const int lrow = 32 * TB * bh + 32 * t + lr;
      const float it = t_in[t] > 0.f ? 1.f / t_in[t] : 1.f;
      const int srow = s_in[t] < p.logits_rows ? s_in[t] : -1;
      float x[32];
#pragma unroll
      for (int e = 0; e < 32; ++e)
        x[e] = (!decltype(TAIL)::value || vl + off(e) < V) ? acc[e >> 4][t][e & 15] : -INFINITY;
      // largest and second largest (a repeated maximum counts twice) by a
      // pairwise tree, then the lowest element holding the largest
      float h[16], l[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        h[j] = hw_max(x[2 * j], x[2 * j + 1]);
        l[j] = hw_min(x[2 * j], x[2 * j + 1]);
      }
#pragma unroll
      for (int w = 16; w > 1; w >>= 1)
#pragma unroll
        for (int j = 0; j < w / 2; ++j) {
          const float hh = hw_max(h[2 * j], h[2 * j + 1]);
          l[j] = hw_max3(hw_min(h[2 * j], h[2 * j + 1]), l[2 * j], l[2 * j + 1]);
          h[j] = hh;
        }
      const float v1 = h[0], v2 = l[0];
      int e1 = 31;
#pragma unroll
      for (int e = 30; e >= 0; --e) e1 = x[e] == v1 ? e : e1;
      // exp((x - v1) t^-1) as exp2(x sc - v1 sc)
      const float sc = it * 1.4426950408889634f, bias = -v1 * sc;
      float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 32; ++e) ps[e & 3] += hw_exp2(fmaf(x[e], sc, bias));
      float sum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
      int i1 = vl + off(e1);
      if (decltype(TAIL)::value && !(v1 > -INFINITY)) {   // lane wholly past V
        sum = 0.f;
        i1 = 0x7FFFFFFF;
      }
      if (srow >= 0) {
        float* dst = p.logits + (size_t)srow * V + vl;
#pragma unroll
        for (int e = 0; e < 32; ++e)
          if (!decltype(TAIL)::value || vl + off(e) < V) dst[off(e)] = x[e];
      }
      RowStat st{v1, sum, i1, v2};
      RowStat o;
      o.m = shfl_xor(st.m, 32);
      o.s = shfl_xor(st.s, 32);
      o.idx = shfl_xor(st.idx, 32);
      o.v2 = shfl_xor(st.v2, 32);
      st = stat_merge(st, o, it);
      if (lk == 0) xch[vh * C::BB + lrow] = st;
    }
  };
  if (v0 + C::BV > V)
    row_stats(std::true_type{});
  else
    row_stats(std::false_type{});
  __syncthreads();
#pragma unroll
  for (int j = 0; j < NFIN; ++j) {
    const int r = threadIdx.x + j * C::THREADS, m = m0 + r;
    if (r >= C::BB || m >= M) continue;
    const float it = tf_in[j] > 0.f ? 1.f / tf_in[j] : 1.f;
    p.part[(size_t)m * p.n_vtiles + vt] = stat_merge(xch[r], xch[C::BB + r], it);
  }
}

template <int TB, int BK, int NBUF = head_mf32_nbuf(TB, BK)>
hipError_t launch_head_mf32(const HeadParams& p, int n_mchunks, hipStream_t s) {
  typedef HeadMf32<TB, BK, NBUF> C;
  static_assert(C::LDS_BYTES <= 160 * 1024, "head LDS");
  static_assert(C::NBUF >= 2 && C::PER_WAVE * (C::NBUF - 2) < 64, "vmcnt");
  hipError_t e = hipFuncSetAttribute((const void*)head_gemm_mf32_kernel<TB, BK, NBUF>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int total = p.n_vtiles * n_mchunks;
  hipLaunchKernelGGL((head_gemm_mf32_kernel<TB, BK, NBUF>), dim3(8 * ((total + 7) / 8)),
                     dim3(C::THREADS), C::LDS_BYTES, s, p, n_mchunks);
  return hipGetLastError();
}

int head_tune(const char* name, int dflt) {
  const char* e = getenv(name);
  return e ? atoi(e) : dflt;
}

// Row chunks of at most 448 rows, split evenly; TB = 64-row tiles per
// workgroup.  One or two tiles (weight streaming): 64-wide slices, deep ring.
// More: 32-wide slices, three stages, copies spread over the MFMAs.
hipError_t launch_head_mf32_any(const HeadParams& p, hipStream_t s) {
  const int nc = (p.M + 447) / 448;
  const int rows = (p.M + nc - 1) / nc;
  const int tb = (rows + 63) / 64;
  static const int big = head_tune("DMTP_HEAD_BIG", 0);
  switch (tb) {
    case 1: return launch_head_mf32<1, 64>(p, nc, s);
    case 2: return launch_head_mf32<2, 64>(p, nc, s);
    case 3: return launch_head_mf32<3, 32, 3>(p, nc, s);
    case 4: return launch_head_mf32<4, 32, 3>(p, nc, s);
    case 5: return launch_head_mf32<5, 32, 3>(p, nc, s);
    case 6: return launch_head_mf32<6, 32, 3>(p, nc, s);
    default:
      if (big == 1) return launch_head_mf32<7, 32, 4>(p, nc, s);
      if (big == 2) return launch_head_mf32<7, 64, 2>(p, nc, s);
      return launch_head_mf32<7, 32, 3>(p, nc, s);
  }
}

// Row chunks of at most 448 rows, split evenly; T = 16-row tiles per wave.
hipError_t launch_head_lds_any(const HeadParams& p, hipStream_t s) {
  const int nc = (p.M + 447) / 448;
  const int rows = (p.M + nc - 1) / nc;
  switch ((rows + 63) / 64) {
    case 1: return launch_head_lds<1>(p, nc, s);
    case 2: return launch_head_lds<2>(p, nc, s);
    case 3: return launch_head_lds<3>(p, nc, s);
    case 4: return launch_head_lds<4>(p, nc, s);
    case 5: return launch_head_lds<5>(p, nc, s);
    case 6: return launch_head_lds<6>(p, nc, s);
    default: return launch_head_lds<7>(p, nc, s);
  }
}

template <int NBW>
hipError_t launch_head_big(const HeadParams& p, int n_mchunks, hipStream_t s) {
  typedef HeadBig<NBW> C;
  static_assert(C::LDS_BYTES <= 160 * 1024, "head LDS");
  hipError_t e = hipFuncSetAttribute((const void*)head_gemm_big_kernel<NBW>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int total = p.n_vtiles * n_mchunks;
  const int grid = 8 * ((total + 7) / 8);
  hipLaunchKernelGGL(head_gemm_big_kernel<NBW>, dim3(grid), dim3(C::THREADS), C::LDS_BYTES, s, p,
                     n_mchunks);
  return hipGetLastError();
}

// Row chunks of at most 256 rows (four waves, one per SIMD, so that each wave
// may hold 512 registers), split evenly.
void head_chunks(int M, int& n_mchunks, int& nbw) {
  n_mchunks = (M + 255) / 256;
  const int rows = (M + n_mchunks - 1) / n_mchunks;
  nbw = (rows + 63) / 64;
}

hipError_t launch_head_big_any(const HeadParams& p, hipStream_t s) {
  if (p.M <= 64) {
    const dim3 grid((p.n_vtiles + 3) / 4);
    if (p.M <= 32)
      hipLaunchKernelGGL(head_gemm_skinny_kernel<1>, grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(head_gemm_skinny_kernel<2>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
  }
  int nc, nbw;
  head_chunks(p.M, nc, nbw);
  switch (nbw) {   // rows per chunk > 64 here, so nbw >= 2
    case 2: return launch_head_big<2>(p, nc, s);
    case 3: return launch_head_big<3>(p, nc, s);
    default: return launch_head_big<4>(p, nc, s);
  }
}

constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void head_merge_kernel(HeadParams p, int final_greedy) {
  __shared__ RowStat red[kMergeThreads / kWave];
  const int m = blockIdx.x;
  const float it = inv_temp(p.temperature, m);
  RowStat st = stat_empty();
  for (int t = threadIdx.x; t < p.n_vtiles; t += blockDim.x)
    st = stat_merge(st, p.part[(size_t)m * p.n_vtiles + t], it);
#pragma unroll
  for (int mask = 1; mask < kWave; mask <<= 1) {
    RowStat o;
    o.m = shfl_xor(st.m, mask);
    o.s = shfl_xor(st.s, mask);
    o.idx = shfl_xor(st.idx, mask);
    o.v2 = shfl_xor(st.v2, mask);
    st = stat_merge(st, o, it);
  }
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = st;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kMergeThreads / kWave; ++w) st = stat_merge(st, red[w], it);
    p.amax[m] = st.idx;
    p.gap_greedy[m] = st.m - st.v2;
    if (p.row_max) p.row_max[m] = st.m;
    if (p.lse) p.lse[m] = st.m * it + logf(st.s);
    if (final_greedy) {
      p.token[m] = st.idx;
      if (p.gap) p.gap[m] = st.m - st.v2;
    }
  }
}

// Deterministic list of the rows that are drawn (temperature > 0, logits stored).
__global__ void head_plan_kernel(HeadParams p) {
  __shared__ int32_t base;
  if (threadIdx.x == 0) base = 0;
  __syncthreads();
  for (int c0 = 0; c0 < p.M; c0 += blockDim.x) {
    const int m = c0 + threadIdx.x;
    const int flag = (m < p.M && p.temperature[m] > 0.f && p.draw_key[m] != DMTP_NO_DRAW &&
                      p.store_row && p.store_row[m] >= 0 &&
                      p.store_row[m] < p.logits_rows && !(p.plant_row && p.plant_row[m] >= 0 &&
                                                          p.plant_row[m] < p.M))
                         ? 1
                         : 0;
    // block-wide exclusive scan of flag
    __shared__ int32_t sc[1024];
    sc[threadIdx.x] = flag;
    __syncthreads();
    for (int o = 1; o < (int)blockDim.x; o <<= 1) {
      const int v = threadIdx.x >= (unsigned)o ? sc[threadIdx.x - o] : 0;
      __syncthreads();
      sc[threadIdx.x] += v;
      __syncthreads();
    }
    if (m < p.M) {
      const int pos = base + sc[threadIdx.x] - flag;
      p.list_pos[m] = flag ? pos : -1;
      if (flag) p.list[pos] = m;
    }
    __syncthreads();
    if (threadIdx.x == blockDim.x - 1) base += sc[threadIdx.x];
    __syncthreads();
  }
  if (threadIdx.x == 0) p.list_count[0] = base;
}

constexpr int kScanThreads = 256;
constexpr int kScanChunk = kScanThreads * 8;  // vocabulary entries per work item

// Gumbel-max scan: item = (list index, chunk); score_j = l_j / t + g_j.
__global__ __launch_bounds__(kScanThreads) void head_scan_kernel(HeadParams p) {
  __shared__ Top2 red[kScanThreads / kWave];
  const int count = p.list_count[0];
  const int items = count * p.n_chunks;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int li = item / p.n_chunks, ch = item % p.n_chunks;
    const int m = p.list[li];
    const float it = 1.f / p.temperature[m];
    const float* lr = p.logits + (size_t)p.store_row[m] * p.V;
    const int j0 = ch * kScanChunk + 8 * threadIdx.x;
    Top2 t = top2_empty();
    if (j0 < p.V) {
      uint32_t w[8];
      philox_words8(p.seed, p.draw_key[m], (uint64_t)(j0 >> 3), w);
      float l[8];
      if (j0 + 8 <= p.V && (p.V & 3) == 0) {
        const float4 a = *(const float4*)(lr + j0), b = *(const float4*)(lr + j0 + 4);
        l[0] = a.x; l[1] = a.y; l[2] = a.z; l[3] = a.w; l[4] = b.x; l[5] = b.y; l[6] = b.z; l[7] = b.w;
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) l[k] = j0 + k < p.V ? lr[j0 + k] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = j0 + k;
        if (j < p.V) top2_push(t, l[k] * it + gumbel_fast(w[k]), j);
      }
    }
#pragma unroll
    for (int mask = 1; mask < kWave; mask <<= 1) t = top2_merge(t, top2_shfl_xor(t, mask));
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w2 = 1; w2 < kScanThreads / kWave; ++w2) t = top2_merge(t, red[w2]);
      p.scan_part[(size_t)li * p.n_chunks + ch] = t;
    }
    __syncthreads();
  }
}

// One wave per row: the chunk maxima of a drawn row are merged across lanes.
__global__ __launch_bounds__(256) void head_finalize_kernel(HeadParams p) {
  const int m = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (m >= p.M) return;
  int tok = p.amax[m];
  float g = p.gap_greedy[m];
  if (p.plant_row && p.plant_row[m] >= 0 && p.plant_row[m] < p.M) {
    tok = p.amax[p.plant_row[m]];
    g = p.gap_greedy[p.plant_row[m]];
  } else if (p.temperature && p.temperature[m] > 0.f && p.draw_key[m] != DMTP_NO_DRAW) {
    const int li = p.list_pos ? p.list_pos[m] : -1;
    if (li < 0) {
      tok = -1;  // a sampled row without a stored logits row
      g = 0.f;
    } else {
      Top2 t = top2_empty();
      for (int c = lane; c < p.n_chunks; c += kWave) t = top2_merge(t, p.scan_part[(size_t)li * p.n_chunks + c]);
#pragma unroll
      for (int mask = 1; mask < kWave; mask <<= 1) t = top2_merge(t, top2_shfl_xor(t, mask));
      tok = t.i1;
      g = t.v1 - t.v2;
    }
  }
  if (lane == 0) {
    p.token[m] = tok;
    if (p.gap) p.gap[m] = g;
  }
}

typedef GemmTile<64, 64, 32, 32, 2, 2> HeadTileF32;
typedef GemmTile<128, 64, 64, 32, 1, 1> HeadTileBF16;   // H not a multiple of 128

struct WsLayout {
  size_t prepared, part, amax, gapg, list, list_pos, list_count, scan, total;
  int n_vtiles, n_chunks;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(const dmtp_head_desc& d, int M) {
  WsLayout w;
  w.n_vtiles = (d.dtype == DMTP_BF16 && d.H % 128 == 0) ? (d.V + 127) / 128 : (d.V + 63) / 64;
  w.n_chunks = (d.V + kScanChunk - 1) / kScanChunk;
  const size_t esz = d.dtype == DMTP_BF16 ? 2 : 4;
  size_t o = 0;
  w.prepared = o; o = align256(o + (size_t)M * d.H * esz);
  w.part = o; o = align256(o + (size_t)w.n_vtiles * M * sizeof(RowStat));
  w.amax = o; o = align256(o + (size_t)M * 4);
  w.gapg = o; o = align256(o + (size_t)M * 4);
  w.list = o; o = align256(o + (size_t)M * 4);
  w.list_pos = o; o = align256(o + (size_t)M * 4);
  w.list_count = o; o = align256(o + 4);
  w.scan = o;
  if (d.temperature) o = align256(o + (size_t)M * w.n_chunks * sizeof(Top2));
  w.total = o;
  return w;
}

// Selects the bf16 head kernel variant from DMTP_HEAD_KERNEL, read once:
// 0 (default) the 32 x 32 x 16 LDS-DMA kernel, 1 the register-staged pair,
// 2 the 16 x 16 x 32 LDS-DMA kernel.
int head_kernel_choice() {
  static int v = [] {
    const char* e = getenv("DMTP_HEAD_KERNEL");
    return e ? atoi(e) : 0;
  }();
  return v;
}

}  // namespace

size_t lm_head_ws_bytes(const dmtp_head_desc& d, int M) { return ws_layout(d, M).total; }

hipError_t lm_head_run(const dmtp_head_desc& d, int M, void* ws, hipStream_t s) {
  const WsLayout w = ws_layout(d, M);
  char* base = (char*)ws;
  HeadParams p;
  for (int i = 0; i < 4; ++i) {
    p.seg[i].x = i < d.n_seg ? d.seg[i].x : nullptr;
    p.seg[i].n = i < d.n_seg ? d.seg[i].n : 0;
    p.seg[i].ld = i < d.n_seg ? d.seg[i].ld : 0;
    p.seg[i].dtype = i < d.n_seg ? d.seg[i].dtype : d.dtype;
    p.seg[i].g = i < d.n_seg ? d.seg[i].g_norm : nullptr;
  }
  p.n_seg = d.n_seg;
  p.M = M;
  p.H = d.H;
  p.V = d.V;
  p.dtype = d.dtype;
  p.eps = d.eps;
  p.W = d.W;
  p.temperature = d.temperature;
  p.draw_key = d.draw_key;
  p.seed = d.seed;
  p.plant_row = d.plant_row;
  p.store_row = d.store_row;
  p.logits = d.logits;
  p.logits_rows = d.store_row ? d.logits_rows : 0;
  p.prepared = d.prepared ? d.prepared : (void*)(base + w.prepared);
  p.part = (RowStat*)(base + w.part);
  p.n_vtiles = w.n_vtiles;
  p.amax = (int32_t*)(base + w.amax);
  p.gap_greedy = (float*)(base + w.gapg);
  p.list = (int32_t*)(base + w.list);
  p.list_pos = d.temperature ? (int32_t*)(base + w.list_pos) : nullptr;
  p.list_count = (int32_t*)(base + w.list_count);
  p.scan_part = (Top2*)(base + w.scan);
  p.n_chunks = w.n_chunks;
  p.token = d.token;
  p.row_max = d.row_max;
  p.lse = d.lse;
  p.gap = d.gap;

  // a single segment of ready head-input rows is read in place
  const bool direct = d.n_seg == 1 && !d.seg[0].g_norm && d.seg[0].ld == d.H && !d.prepared;
  p.A = direct ? d.seg[0].x : p.prepared;
  hipError_t e = hipSuccess;
  if (!direct) {
    hipLaunchKernelGGL(head_prep_kernel, dim3(M), dim3(kPrepThreads), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (d.dtype == DMTP_BF16 && d.H % 128 == 0) {
    const int kc = head_kernel_choice();
    e = kc == 1 ? launch_head_big_any(p, s) : kc == 2 ? launch_head_lds_any(p, s)
                                                       : launch_head_mf32_any(p, s);
    if (e != hipSuccess) return e;
  } else if (d.dtype == DMTP_BF16) {
    dim3 grid(w.n_vtiles, (M + HeadTileBF16::BM - 1) / HeadTileBF16::BM);
    hipLaunchKernelGGL(head_gemm_kernel<HeadTileBF16>, grid, dim3(HeadTileBF16::THREADS), 0, s, p);
  } else {
    dim3 grid(w.n_vtiles, (M + HeadTileF32::BM - 1) / HeadTileF32::BM);
    hipLaunchKernelGGL(head_gemm_kernel<HeadTileF32>, grid, dim3(HeadTileF32::THREADS), 0, s, p);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int simple = !d.temperature && !d.plant_row;
  hipLaunchKernelGGL(head_merge_kernel, dim3(M), dim3(kMergeThreads), 0, s, p, simple);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (simple) return hipSuccess;
  if (d.temperature) {
    hipLaunchKernelGGL(head_plan_kernel, dim3(1), dim3(1024), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(head_scan_kernel, dim3(2048), dim3(kScanThreads), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(head_finalize_kernel, dim3((M + 3) / 4), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace dmtp

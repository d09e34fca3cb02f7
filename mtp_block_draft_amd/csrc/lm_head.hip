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
//   plan/mass (only when temperatures are given) the list of drawn rows, and
//             one memory-bound pass over their stored logits rows giving the
//             softmax mass of every block of kDrawBlock entries
//   finalize  token per row: a two-level Gumbel-max draw (block by its mass,
//             then an entry of that block), the planted row's argmax, or the
//             argmax
#include <algorithm>
#include <type_traits>

#include <hip/hip_ext.h>

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
  const void* Wp;        // W in the packed stage layout (dmtp_head_pack), or NULL
  const float* temperature;
  const uint64_t* draw_key;
  uint64_t seed;
  const int32_t* plant_row;
  const int32_t* store_row;
  float* logits;
  int logits_rows;
  void* prepared;        // head input: [M, H], or [H / a_sl][M][a_sl] when a_sl > 0
  int a_sl;              // k-slice width of a slice-major prepared layout (0: row-major)
  int a_frag;            // prepared rows in the fragment layout of the register-input GEMM
  const void* A;         // rows the GEMM reads: prepared, or the single input segment
  RowStat* part;         // [M, n_vtiles]
  int n_vtiles;
  int32_t* amax;         // [M]
  float* gap_greedy;     // [M]
  int32_t* list;         // [M] sampled rows
  int32_t* list_pos;     // [M] position in list or -1
  int32_t* list_count;   // [1]
  float* rmax;           // [M] row max of the logits (the mass pass's reference)
  float* mass;           // [M, n_blocks] block masses of drawn rows (list order)
  int n_blocks;          // blocks of kDrawBlock entries
  int block_stats;       // the GEMM's per-tile statistics are per block: they give the masses
  int n_chunks;          // work items of the mass pass per row
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
  // element i of this row: row-major, or inside k-slice i / a_sl of a
  // slice-major layout (a_sl a multiple of 4, so a group of four stays whole),
  // or in the fragment layout: k-slices of 32 over the rows padded to a
  // multiple of 16, each slice a run of 16-row tiles, each tile its four
  // 8-element chunks in turn, each chunk the tile's 16 rows in turn
  const size_t orow = p.a_sl ? (size_t)blockIdx.x * p.a_sl : (size_t)blockIdx.x * H;
  const size_t mp = ((size_t)p.M + 15) & ~(size_t)15;
  const size_t ftile = (size_t)(blockIdx.x >> 4) * 512 + (blockIdx.x & 15) * 8;
  auto oidx = [&](int i) -> size_t {
    if (p.a_frag) return (size_t)(i >> 5) * mp * 32 + ftile + ((i & 31) >> 3) * 128 + (i & 7);
    return p.a_sl ? (size_t)(i / p.a_sl) * p.M * p.a_sl + orow + (i % p.a_sl) : orow + i;
  };
  if (sg.g && H % 4 == 0 && H <= 8 * 4 * kPrepThreads) {
    // the row and its gains in registers: every load issued before the first use
    const float* xr = (const float*)sg.x + (size_t)m * sg.ld;
    float4 xv[8], gv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = 4 * (threadIdx.x + kPrepThreads * k);
      if (i < H) {
        xv[k] = *(const float4*)(xr + i);
        gv[k] = *(const float4*)(sg.g + i);
      }
    }
    double ss = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (4 * (threadIdx.x + kPrepThreads * k) < H)
        ss += (double)xv[k].x * xv[k].x + (double)xv[k].y * xv[k].y + (double)xv[k].z * xv[k].z +
              (double)xv[k].w * xv[k].w;
    ss = wave_sum(ss);
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = ss;
    __syncthreads();
    double t = 0.0;
    for (int w = 0; w < kPrepThreads / kWave; ++w) t += red[w];
    const double inv = 1.0 / sqrt(t / H + (double)p.eps);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int i = 4 * (threadIdx.x + kPrepThreads * k);
      if (i < H) {
        const size_t o = oidx(i);
        store_elem(p.prepared, p.dtype, o + 0, (float)((double)xv[k].x * inv * gv[k].x));
        store_elem(p.prepared, p.dtype, o + 1, (float)((double)xv[k].y * inv * gv[k].y));
        store_elem(p.prepared, p.dtype, o + 2, (float)((double)xv[k].z * inv * gv[k].z));
        store_elem(p.prepared, p.dtype, o + 3, (float)((double)xv[k].w * inv * gv[k].w));
      }
    }
  } else if (sg.g) {
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
      store_elem(p.prepared, p.dtype, oidx(i), (float)((double)xr[i] * inv * sg.g[i]));
  } else {
    // rows already in the head dtype: 16-byte pieces (8 bf16 or 4 float32
    // elements, which every output layout keeps together; H is a multiple of
    // 64 and rows and strides are 16-byte aligned), all loads of the row
    // issued before the first store
    const int per = p.dtype == DMTP_BF16 ? 8 : 4;
    const char* xr = (const char*)sg.x + (size_t)m * sg.ld * (p.dtype == DMTP_BF16 ? 2 : 4);
    const int np = H / per;
    constexpr int KP = 8;   // pieces per thread per pass: 8 x 256 x 8 = 16384 bf16 elements
    for (int j0 = 0; j0 < np; j0 += KP * kPrepThreads) {
      uint4 v[KP];
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        const int j = j0 + threadIdx.x + kPrepThreads * k;
        if (j < np) v[k] = *(const uint4*)(xr + (size_t)16 * j);
      }
#pragma unroll
      for (int k = 0; k < KP; ++k) {
        const int j = j0 + threadIdx.x + kPrepThreads * k;
        if (j < np) {
          const size_t o = oidx(per * j);
          if (p.dtype == DMTP_BF16) *(uint4*)((uint16_t*)p.prepared + o) = v[k];
          else *(uint4*)((float*)p.prepared + o) = v[k];
        }
      }
    }
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

template <int TB, int BK, int NBUF, bool PK = false>
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
  // input rows: row-major [M, H], or slice-major with k-slices of width BK
  const size_t x_rs = p.a_sl ? (size_t)BK : (size_t)H;
  const size_t x_ss = p.a_sl ? (size_t)M * BK : (size_t)BK;

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
      // PK (64-wide slices): the packed copy holds each slice's weight stage
      // as its LDS image, 16 KB in a row per 128-row tile
      src[q] = PK ? (const uint16_t*)p.Wp + (size_t)v0 * H + 8 * idx
                  : W + (size_t)min(v0 + r, V - 1) * H + 8 * swz_chunk<BK>(r, idx % C::CPR);
      dst[q] = (wave * C::WPW + q) * 512;
    } else {
      const int qq = q - C::WPW;
      const int idx = (wave * C::XPW + qq) * 64 + lane, r = idx / C::CPR;
      src[q] = X + (size_t)min(m0 + r, M - 1) * x_rs + 8 * swz_chunk<BK>(r, idx % C::CPR);
      dst[q] = C::BV * C::BK + (wave * C::XPW + qq) * 512;
    }
  }
  // The weight rows are read once per call and the matrix is larger than the
  // 256 MB last-level cache: their copies are non-temporal, which keeps them
  // from evicting the input rows every workgroup re-reads.
  auto issue_one = [&](int slice, int q) __attribute__((always_inline)) {
    if (q < C::WPW)
      lds_dma16<2>(src[q] + (size_t)slice * (PK ? C::BV * C::BK : C::BK), smem + (slice % C::NBUF) * C::STAGE + dst[q]);
    else
      lds_dma16(src[q] + (size_t)slice * x_ss, smem + (slice % C::NBUF) * C::STAGE + dst[q]);
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

// Buffer descriptor over `bytes` bytes from `base` (raw, dword data format).
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// 16 bytes per lane from descriptor r at byte offset vo (this lane) + so
// (uniform) to LDS at dst + 16 lane; non-temporal (the weights are read once).
__device__ __forceinline__ void buf_dma16(buf_rsrc r, uint32_t vo, uint32_t so, uint16_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, vo, so, 0, 2);
}

// 16 x 16 x 32 bf16 MFMA on fragments held as four words per lane
__device__ __forceinline__ f32x4_t mfma16(const u32x4& a, const u32x4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ---- bf16 head GEMM, 16 x 16 x 32 MFMA, input fragments in registers.
//
// Workgroup: 4 waves on 128 vocabulary rows x 64 TQ input rows; wave w takes
// all 128 vocabulary rows against 16 TQ input rows of its own (8 x TQ
// accumulator tiles of 16 x 16).  Only the weight tile goes through LDS: a
// ring of four 32-wide k-slices (8 KB each) filled by buffer loads with an LDS
// destination and read by all four waves.  Each wave loads its input rows'
// fragments of the next slice straight into registers (with the slice-major
// input layout a 16-row fragment is one contiguous 1 KB read), so no input row
// passes through LDS.  Per slice and workgroup, LDS takes 8 KB of copies and
// 32 KB of fragment reads, against 36 KB and 72 KB for the 32 x 32 x 16
// kernel above, whose waves share their input rows through LDS.
// Input slices loaded ahead: one for 6 or 7 tiles per wave, three for fewer
// (four register sets).  Each input load waits, in vmcnt's issue order, for
// the weight copies issued before it, so the further ahead, the more of the
// weights' HBM latency it covers; with 7 tiles three slices ahead measured
// slower (about three times the input loads in flight on the vector memory
// path beside the weight copies).
constexpr int head_xr_xd(int TQ) { return TQ <= 5 ? 3 : 1; }

template <int TQ, int NW_ = 4>
struct HeadXr {
  static constexpr int BV = 128, BK = 32, THREADS = 256;
  static constexpr int XD = head_xr_xd(TQ);            // input slices loaded ahead
  static constexpr int XS = XD + 1;                    // input register sets
  static constexpr int WK = 64;                        // k-width of a weight stage (whole 128-byte lines)
  static constexpr int NW = NW_;                       // weight stages
  static constexpr int NU = BV / 16;                   // vocabulary tiles of 16 rows
  static constexpr int RW = 16 * TQ;                   // input rows per wave
  static constexpr int BB = 4 * RW;                    // input rows per workgroup
  static constexpr int CPR = WK / 8;                   // 16-byte chunks per weight row of a stage
  static constexpr int W_INSTR = BV * WK * 2 / 1024;   // 1 KB weight copies per stage
  static constexpr int WPW = W_INSTR / 4;              // per wave
  static constexpr int STAGE = BV * WK;                // bf16 elements
  static constexpr size_t LDS_BYTES = (size_t)NW * STAGE * 2;
  // vector-memory instructions after a stage's copies at the wait for them
  static constexpr int WAIT_N = (2 * NW - 2) * TQ + (NW - 2) * WPW;
  static_assert(XS == 2 || XS == 4, "register sets");
  static_assert(W_INSTR % 4 == 0 && NW >= 2 && WAIT_N < 64, "copies");
};

template <int TQ, int NW, bool PK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void head_gemm_xr_kernel(HeadParams p, int n_mchunks) {
  typedef HeadXr<TQ, NW> C;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int total = p.n_vtiles * n_mchunks;
  const int per = (total + 7) / 8;   // XCD-contiguous ranges (workgroup i runs on XCD i % 8)
  const int tt = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (tt >= total) return;
  const int vt = tt / n_mchunks, mc = tt % n_mchunks;
  const int v0 = vt * C::BV;
  // the wave index is uniform across the wave: read from lane 0, so that the
  // offsets derived from it stay in scalar registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int fr = lane & 15, fg = lane >> 4;
  const int H = p.H, V = p.V, M = p.M;
  const int rw0 = mc * C::BB + C::RW * wave;   // first input row of this wave

  // Both operands are read through buffer descriptors, so that every address
  // is a lane offset fixed for the whole kernel plus a scalar offset.
  // A weight stage holds 64 k-values (one whole 128-byte line) of each of the
  // tile's 128 rows.  Weight copy q of this wave: rows 8 (WPW wave + q) .. + 7
  // of the tile, lane idx = 64 (WPW wave + q) + lane supplying row idx / CPR,
  // the chunk that lands at position idx % CPR.  The descriptor ends at row V,
  // so the rows of the last tile past V read as zeros (their columns are
  // masked).  PK: the packed copy holds each stage as exactly that LDS image,
  // 16 KB in a row (rows past V stored as zeros), so lane idx reads 16 idx.
  const buf_rsrc wr = PK ? make_rsrc((const uint16_t*)p.Wp + (size_t)v0 * H, C::BV * H * 2)
                         : make_rsrc((const uint16_t*)p.W + (size_t)v0 * H, min(C::BV, V - v0) * H * 2);
  constexpr uint32_t w_ss = PK ? C::STAGE * 2 : C::WK * 2;   // bytes between stages
  uint32_t woff[C::WPW];
  int wdst[C::WPW];
#pragma unroll
  for (int q = 0; q < C::WPW; ++q) {
    const int idx = (wave * C::WPW + q) * 64 + lane, r = idx / C::CPR;
    woff[q] = PK ? (uint32_t)(16 * idx) : (uint32_t)(r * H * 2 + 16 * swz_chunk<C::WK>(r, idx % C::CPR));
    wdst[q] = (wave * C::WPW + q) * 512;
  }
  // Input fragment t (B operand): row rw0 + 16 t + fr, k chunk fg of the
  // 32-wide slice.  In the fragment layout (the prep pass's, rows padded to
  // Mp, a multiple of 16) lane l's 16 bytes sit at 16 l of the tile's 1 KB, so
  // a load is one run in lane order; tiles past Mp are clamped to the last
  // one.  Row-major [M, H] input (the caller's prepared rows) clamps the row
  // to M - 1.  Results of rows past M are never written.  The host keeps the
  // input's bytes below 2^31.
  const int Mp = (M + 15) & ~15;
  const buf_rsrc xr = make_rsrc(p.A, (p.a_frag ? Mp : M) * H * 2);
  const uint32_t x_ss = p.a_frag ? (uint32_t)Mp * C::BK : C::BK;   // elements between slices
  uint32_t xoff[TQ];
#pragma unroll
  for (int t = 0; t < TQ; ++t)
    xoff[t] = p.a_frag ? ((uint32_t)min((rw0 >> 4) + t, (Mp >> 4) - 1) * 512 + 8 * lane) * 2
                       : ((uint32_t)min(rw0 + 16 * t + fr, M - 1) * H + 8 * fg) * 2;

  constexpr int XD = C::XD, XS = C::XS;
  u32x4 xf[XS][TQ];   // input fragments, set = slice % XS
  auto load_x = [&](int slice, int set) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < TQ; ++t)
      xf[set][t] = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[t], (uint32_t)slice * x_ss * 2, 0);
  };
  auto issue_w = [&](int stage, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < C::WPW; ++q)
      buf_dma16(wr, woff[q], (uint32_t)stage * w_ss, smem + slot * C::STAGE + wdst[q]);
  };
  u32x4 wf[2][C::NU];   // weight fragments (A operand) of a 32-wide slice, double-buffered
  // fragments of slice k: stage k / 2 (in slot (k / 2) % NW), chunks 4 (k % 2) + fg
  auto read_w = [&](int k, int b) __attribute__((always_inline)) {
    const uint16_t* st = smem + ((k >> 1) % C::NW) * C::STAGE;
#pragma unroll
    for (int u = 0; u < C::NU; ++u)
      wf[b][u] = *(const u32x4*)(st + swz_row<C::WK>(16 * u + fr, 4 * (k & 1) + fg));
  };

  f32x4_t acc[C::NU][TQ];

  // Per step k (32-wide slice k) the vector-memory instructions go out in one
  // fixed order: the input loads of slice k + 1, then, at odd k only and after
  // the barrier, the copies of stage (k + 1) / 2 + NW - 1 into the slot of
  // stage (k - 1) / 2, whose last fragments every wave read before that
  // barrier.  Past the last slice and stage the same instructions are issued
  // again for the last ones (into a slot and an input set nobody reads), so
  // the order never changes.  A step's fragments for slice k + 1 come from
  // the stage of slice k at even k (no wait: that stage was waited for and
  // shared at step k - 1) and from a new stage at odd k: there the wave waits
  // until at most WAIT_N newer instructions are in flight -- the input loads
  // of the 2 NW - 2 slices up to k + 1 and the copies of NW - 2 later stages
  // -- so that stage (k + 1) / 2 has landed, then meets the others at the
  // barrier.  The first NW - 1 stages land at the prologue's full wait.  The
  // compiler waits for the input loads of slice k + 1 before the MFMAs that
  // use them.
  const int nK = H / C::BK;    // a multiple of 4 (H % 128 == 0)
  const int nS = nK / 2;       // weight stages
#pragma unroll
  for (int s = 0; s < C::NW - 1; ++s) issue_w(min(s, nS - 1), s);
#pragma unroll
  for (int s = 0; s < XD; ++s) load_x(min(s, nK - 1), s);
  wait_vm_lgkm0<0>();
  ring_barrier();
  read_w(0, 0);
  issue_w(min(C::NW - 1, nS - 1), C::NW - 1);
  // step k with register sets J (= k modulo XS): weight fragments k % 2,
  // input set k % XS; FIRST: slice 0, whose MFMAs start from zero
  // accumulators (an inline zero operand: accumulators that enter the loop as
  // constants make the compiler move them between registers on every MFMA);
  // NEXT: a slice k + 1 exists.  No MFMA sits under a run-time branch, so the
  // accumulators stay in place from step to step.
  auto step = [&](int k, auto J, auto FIRST, auto NEXT) __attribute__((always_inline)) {
    constexpr int pb = decltype(J)::value % 2, xs = decltype(J)::value % XS;
    constexpr bool first = decltype(FIRST)::value, next = decltype(NEXT)::value;
    auto mfmas = [&](int u0, int u1) __attribute__((always_inline)) {
#pragma unroll
      for (int u = u0; u < u1; ++u)
#pragma unroll
        for (int t = 0; t < TQ; ++t)
          acc[u][t] = mfma16(wf[pb][u], xf[xs][t], first ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[u][t]);
    };
    // the scheduling barriers keep this order: left to itself the compiler
    // sinks the input loads below the MFMAs, which undoes the prefetch
    load_x(min(k + XD, nK - 1), (xs + XD) % XS);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(0, C::NU / 2);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (pb == 0) {
      if constexpr (next) read_w(k + 1, 1);
    } else {
      if constexpr (next) {
        wait_vm_lgkm0<C::WAIT_N>();
        ring_barrier();
        read_w(k + 1, 0);
      }
      issue_w(min((k + 1) / 2 + C::NW - 1, nS - 1), ((k - 1) / 2) % C::NW);
    }
    __builtin_amdgcn_sched_barrier(0);
    mfmas(C::NU / 2, C::NU);
    __builtin_amdgcn_sched_barrier(0);
  };
  const std::true_type Y;
  const std::false_type N;
  typedef std::integral_constant<int, 1> J1;
  typedef std::integral_constant<int, 2> J2;
  typedef std::integral_constant<int, 3> J3;
  typedef std::integral_constant<int, 4> J4;
  step(0, std::integral_constant<int, 0>{}, Y, Y);   // nK >= 4
  // steps k0 + 1 .. k0 + XS per iteration (XS register sets; nK is a
  // multiple of 4), then the last XS - 1 steps, the final one without a next
  // slice.  (Two steps per iteration where two sets suffice: four measured
  // slower there.)
  int k0 = 0;
  if constexpr (XS == 4) {
    for (; k0 + 4 < nK; k0 += 4) {
      step(k0 + 1, J1{}, N, Y);
      step(k0 + 2, J2{}, N, Y);
      step(k0 + 3, J3{}, N, Y);
      step(k0 + 4, J4{}, N, Y);
    }
    step(k0 + 1, J1{}, N, Y);
    step(k0 + 2, J2{}, N, Y);
    step(k0 + 3, J3{}, N, N);
  } else {
    for (; k0 + 2 < nK; k0 += 2) {
      step(k0 + 1, J1{}, N, Y);
      step(k0 + 2, J2{}, N, Y);
    }
    step(k0 + 1, J1{}, N, N);
  }
  // the repeated copies of the last steps land before the workgroup ends
  wait_vm_lgkm0<0>();

  // per-row inputs of the epilogue
  float t_in[TQ];   // temperature of the lane's row in tile t (1 when none given)
  int s_in[TQ];     // logits store index of that row (-1: none)
#pragma unroll
  for (int t = 0; t < TQ; ++t) {
    const int m = rw0 + 16 * t + fr;
    const bool ok = m < M;
    t_in[t] = (ok && p.temperature) ? p.temperature[m] : 1.f;
    s_in[t] = (ok && p.store_row) ? p.store_row[m] : -1;
  }

  // ---- epilogue: per input row tile t, the lane holds 32 logits of its row
  // (element e = 4 u + i at vocabulary column v0 + 16 u + 4 fg + i, rising with
  // e); the four lane groups that share the row merge by two exchanges.
  const int vl = v0 + 4 * fg;
  auto off = [](int e) { return 16 * (e >> 2) + (e & 3); };
  auto row_stats = [&](auto TAIL) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < TQ; ++t) {
      const int row = rw0 + 16 * t + fr;
      const float it = t_in[t] > 0.f ? 1.f / t_in[t] : 1.f;
      const int srow = s_in[t] < p.logits_rows ? s_in[t] : -1;
      float x[32];
#pragma unroll
      for (int e = 0; e < 32; ++e)
        x[e] = (!decltype(TAIL)::value || vl + off(e) < V) ? acc[e >> 2][t][e & 3] : -INFINITY;
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
#pragma unroll
      for (int mask = 16; mask < 64; mask <<= 1) {
        RowStat o;
        o.m = shfl_xor(st.m, mask);
        o.s = shfl_xor(st.s, mask);
        o.idx = shfl_xor(st.idx, mask);
        o.v2 = shfl_xor(st.v2, mask);
        st = stat_merge(st, o, it);
      }
      if (fg == 0 && row < M) p.part[(size_t)row * p.n_vtiles + vt] = st;
    }
  };
  if (v0 + C::BV > V)
    row_stats(std::true_type{});
  else
    row_stats(std::false_type{});
}

// Optional start/stop events of the vocabulary GEMM launch (both or neither).
struct GemmEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

template <int TB, int BK, int NBUF = head_mf32_nbuf(TB, BK)>
hipError_t launch_head_mf32(const HeadParams& p, int n_mchunks, const GemmEvents& ev, hipStream_t s) {
  typedef HeadMf32<TB, BK, NBUF> C;
  static_assert(C::LDS_BYTES <= 160 * 1024, "head LDS");
  static_assert(C::NBUF >= 2 && C::PER_WAVE * (C::NBUF - 2) < 64, "vmcnt");
  const int total = p.n_vtiles * n_mchunks;
  const dim3 grid(8 * ((total + 7) / 8));
  auto go = [&](auto kern) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)C::LDS_BYTES);
    if (e != hipSuccess) return e;
    if (ev.start && ev.stop)
      hipExtLaunchKernelGGL(kern, grid, dim3(C::THREADS), (uint32_t)C::LDS_BYTES, s, ev.start, ev.stop, 0u, p,
                            n_mchunks);
    else
      hipLaunchKernelGGL(kern, grid, dim3(C::THREADS), C::LDS_BYTES, s, p, n_mchunks);
    return hipGetLastError();
  };
  // the packed copy's stages are 64 wide
  if constexpr (BK == 64) {
    if (p.Wp) return go(head_gemm_mf32_kernel<TB, BK, NBUF, true>);
  }
  return go(head_gemm_mf32_kernel<TB, BK, NBUF, false>);
}


template <int TQ>
hipError_t launch_head_xr(const HeadParams& p, int n_mchunks, const GemmEvents& ev, hipStream_t s) {
  typedef HeadXr<TQ> C;
  static_assert(C::LDS_BYTES <= 160 * 1024, "head LDS");
  const int total = p.n_vtiles * n_mchunks;
  const dim3 grid(8 * ((total + 7) / 8));
  auto go = [&](auto kern) {
    if (ev.start && ev.stop)
      hipExtLaunchKernelGGL(kern, grid, dim3(C::THREADS), (uint32_t)C::LDS_BYTES, s, ev.start, ev.stop, 0u, p,
                            n_mchunks);
    else
      hipLaunchKernelGGL(kern, grid, dim3(C::THREADS), C::LDS_BYTES, s, p, n_mchunks);
    return hipGetLastError();
  };
  return p.Wp ? go(head_gemm_xr_kernel<TQ, C::NW, true>) : go(head_gemm_xr_kernel<TQ, C::NW, false>);
}

// Row chunks of at most 448 rows, split evenly; TB = 64-row tiles per
// workgroup.  One or two tiles (weight streaming): 64-wide slices, deep ring.
// More: 32-wide slices, three stages, copies spread over the MFMAs.
int head_mf32_tb(int M) {
  const int nc = (M + 447) / 448;
  return ((M + nc - 1) / nc + 63) / 64;
}
// k-slice width of the kernel launch_head_mf32_any picks for M rows
int head_mf32_bk(int M) { return head_mf32_tb(M) <= 2 ? 64 : 32; }
// calls the register-input kernel takes: three or more 64-row tiles, input
// rows (padded to a multiple of 16) addressed through one buffer descriptor
bool head_xr_fits(int M, int H) {
  return head_mf32_tb(M) >= 3 && ((size_t)(M + 15) & ~(size_t)15) * H * 2 < ((size_t)1 << 31);
}

hipError_t launch_head_mf32_any(const HeadParams& p, const GemmEvents& ev, hipStream_t s) {
  const int nc = (p.M + 447) / 448;
  const int tb = head_mf32_tb(p.M);
  if (head_xr_fits(p.M, p.H)) {
    switch (tb) {
      case 3: return launch_head_xr<3>(p, nc, ev, s);
      case 4: return launch_head_xr<4>(p, nc, ev, s);
      case 5: return launch_head_xr<5>(p, nc, ev, s);
      case 6: return launch_head_xr<6>(p, nc, ev, s);
      default: return launch_head_xr<7>(p, nc, ev, s);
    }
  }
  switch (tb) {
    case 1: return launch_head_mf32<1, 64>(p, nc, ev, s);
    case 2: return launch_head_mf32<2, 64>(p, nc, ev, s);
    case 3: return launch_head_mf32<3, 32, 3>(p, nc, ev, s);
    case 4: return launch_head_mf32<4, 32, 3>(p, nc, ev, s);
    case 5: return launch_head_mf32<5, 32, 3>(p, nc, ev, s);
    case 6: return launch_head_mf32<6, 32, 3>(p, nc, ev, s);
    default: return launch_head_mf32<7, 32, 3>(p, nc, ev, s);
  }
}

// ---- bf16 head GEMM for calls of at most 32 input rows (weight streaming).
//
// Such a call is bound by one read of the [V, H] weight matrix, so the design
// serves the read pattern.  Persistent workgroups (one per CU) each take a
// contiguous run of 32-row vocabulary tiles.  Stream wave w (of four) covers k-quarter w of
// every tile through a ring of its own: stages of 32 rows x 128 k, each copy
// instruction reading 256 contiguous bytes of four weight rows, so a tile's
// 128 KB are read as four long runs.  The input rows' k-quarter stays in the
// stream wave's registers for the whole kernel (no input copies at all).  A
// fifth wave adds the four partial 32 x 32 tiles in wave order and folds
// each tile's row statistics into one partial per row and workgroup, in tile
// order, while the stream waves go on to the next tile.  Splitting k changes the float32 summation
// order against the kernels above, which sum over k in one sequence: the two
// agree to rounding, not bit for bit; each is batch invariant on its own.
constexpr int kT1Stream = 4;                       // stream waves
constexpr int kT1Threads = (kT1Stream + 1) * kWave;
constexpr int kT1BK = 128;                         // stage width in k
constexpr int kT1NB = 3;                           // stages per stream wave
constexpr int kT1Stage = 32 * kT1BK;               // elements per stage
constexpr int kT1Copies = kT1Stage * 2 / 1024;     // 1 KB copies per stage
constexpr int kT1Red = kT1Stream * 16 * kWave;     // floats of one partial set
constexpr int kT1Grid = 256;                       // workgroups (at most; one per CU)
constexpr size_t kT1Lds = (size_t)kT1Stream * kT1NB * kT1Stage * 2 + 2 * (size_t)kT1Red * 4;

// Position of 16-byte chunk c of row r in a [32][128] stage (an involution):
// the 16 lanes of one read pass land on the 16 positions of the bank window.
__device__ __forceinline__ int t1_swz(int r, int c) { return c ^ (r & 15); }

// Wait until this wave has at most N vector-memory operations outstanding,
// leaving the LDS counter alone.
template <int N>
__device__ __forceinline__ void wait_vm_only() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int KQ>   // 16-wide k-steps per quarter: H = 64 KQ
__global__ __launch_bounds__(kT1Threads) void head_t1_kernel(HeadParams p, int n_tiles) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  constexpr int KPS = kT1BK / 16;                  // k-steps per stage
  constexpr int SUB = KQ / KPS;                    // stages per tile and stream wave
  static_assert(KQ % KPS == 0, "quarter");
  static_assert(kT1Copies * (kT1NB - 2) < 64, "vmcnt");
  float* red = (float*)(smem + kT1Stream * kT1NB * kT1Stage);   // [2][stream wave][16][64]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, lk = lane >> 5;
  const int H = p.H, V = p.V, M = p.M;
  // tiles t0 .. t0 + my_tiles - 1: n_tiles split into gridDim.x runs whose
  // lengths differ by at most one (gridDim.x <= n_tiles, so none is empty)
  const int G = gridDim.x, b = blockIdx.x;
  const int my_tiles = n_tiles / G + (b < n_tiles % G ? 1 : 0);
  const int t0 = b * (n_tiles / G) + min(b, n_tiles % G);

  if (wave < kT1Stream) {
    const uint16_t* __restrict__ W = (const uint16_t*)p.W;
    const uint16_t* __restrict__ X = (const uint16_t*)p.A;
    const int kq0 = wave * KQ * 16;
    // MFMA B operands of the quarter: input row lr (rows past M repeat row
    // M - 1; their results are never written), k = kq0 + 16 j + 8 lk ..
    u32x4 xf[KQ];
    const uint16_t* xr = X + (size_t)min(lr, M - 1) * H + kq0 + 8 * lk;
#pragma unroll
    for (int j = 0; j < KQ; ++j) xf[j] = *(const u32x4*)(xr + 16 * j);
    // these loads complete before the first copy is issued, so no later wait
    // for them drains the ring
    wait_vm_only<0>();
    uint16_t* ring = smem + wave * kT1NB * kT1Stage;
    const int nseq = my_tiles * SUB;
    // stage q: tile t0 + q / SUB, k from kq0 + 128 (q % SUB); copy i covers
    // rows 4 i .. 4 i + 3 (lane / 16), chunk position lane % 16
    auto issue = [&](int q) __attribute__((always_inline)) {
      const int t = t0 + q / SUB;
      const int k0 = kq0 + kT1BK * (q % SUB);
      uint16_t* st = ring + (q % kT1NB) * kT1Stage;
#pragma unroll
      for (int i = 0; i < kT1Copies; ++i) {
        const int r = 4 * i + (lane >> 4);
        lds_dma16<2>(W + (size_t)min(32 * t + r, V - 1) * H + k0 + 8 * t1_swz(r, lane & 15), st + 512 * i);
      }
    };
    for (int q = 0; q < kT1NB - 1 && q < nseq; ++q) issue(q);
    for (int tile = 0; tile < my_tiles; ++tile) {
      f32x16_t acc;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
      for (int s = 0; s < SUB; ++s) {
        const int q = tile * SUB + s;
        // stage q has landed once only the copies of the stages issued after
        // it may be outstanding; lgkmcnt(0) as well, since the stage refilled
        // below was read just before
        wait_vm_dyn<kT1Copies * (kT1NB - 2)>(kT1Copies * min(nseq - 1 - q, kT1NB - 2));
        const uint16_t* st = ring + (q % kT1NB) * kT1Stage;
        u32x4 wf[KPS];
#pragma unroll
        for (int j = 0; j < KPS; ++j) wf[j] = *(const u32x4*)(st + lr * kT1BK + 8 * t1_swz(lr, 2 * j + lk));
#pragma unroll
        for (int j = 0; j < KPS; ++j) acc = mfma32(wf[j], xf[s * KPS + j], acc);
        if (q + kT1NB - 1 < nseq) issue(q + kT1NB - 1);
      }
      float* rb = red + (size_t)(tile & 1) * kT1Red + wave * 16 * kWave;
#pragma unroll
      for (int i = 0; i < 16; ++i) rb[i * kWave + lane] = acc[i];
      // the partials are in LDS before the barrier; the copies stay in flight
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) only
      ring_barrier();
    }
    return;
  }

  // statistics wave: lane (lr, lk) holds input row lr and the 16 vocabulary
  // rows 32 t + 8 (i / 4) + 4 lk + (i % 4), i = 0 .. 15, of tile t
  const bool ok = lr < M;
  const float tin = (ok && p.temperature) ? p.temperature[lr] : 1.f;
  const int sin = (ok && p.store_row) ? p.store_row[lr] : -1;
  const float it = tin > 0.f ? 1.f / tin : 1.f;
  const int srow = sin < p.logits_rows ? sin : -1;
  const float sc = it * 1.4426950408889634f;
  auto off = [](int i) { return 8 * (i >> 2) + (i & 3); };
  RowStat run = stat_empty();   // the row's statistics over this workgroup's tiles so far
  for (int tile = 0; tile < my_tiles; ++tile) {
    ring_barrier();
    const int t = t0 + tile;
    const int vl = 32 * t + 4 * lk;
    const float* rb = red + (size_t)(tile & 1) * kT1Red + lane;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = rb[i * kWave];
#pragma unroll
      for (int w = 1; w < kT1Stream; ++w) v += rb[(w * 16 + i) * kWave];
      x[i] = vl + off(i) < V ? v : -INFINITY;
    }
    float h[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      h[j] = hw_max(x[2 * j], x[2 * j + 1]);
      l[j] = hw_min(x[2 * j], x[2 * j + 1]);
    }
#pragma unroll
    for (int w = 8; w > 1; w >>= 1)
#pragma unroll
      for (int j = 0; j < w / 2; ++j) {
        const float hh = hw_max(h[2 * j], h[2 * j + 1]);
        l[j] = hw_max3(hw_min(h[2 * j], h[2 * j + 1]), l[2 * j], l[2 * j + 1]);
        h[j] = hh;
      }
    const float v1 = h[0], v2 = l[0];
    int e1 = 15;
#pragma unroll
    for (int e = 14; e >= 0; --e) e1 = x[e] == v1 ? e : e1;
    const float bias = -v1 * sc;
    float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 16; ++e) ps[e & 3] += hw_exp2(fmaf(x[e], sc, bias));
    float sum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
    int i1 = vl + off(e1);
    if (!(v1 > -INFINITY)) {   // lane wholly past V
      sum = 0.f;
      i1 = 0x7FFFFFFF;
    }
    if (srow >= 0) {
      float* dst = p.logits + (size_t)srow * V + vl;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (vl + off(e) < V) dst[off(e)] = x[e];
    }
    RowStat st{v1, sum, i1, v2};
    RowStat o;
    o.m = shfl_xor(st.m, 32);
    o.s = shfl_xor(st.s, 32);
    o.idx = shfl_xor(st.idx, 32);
    o.v2 = shfl_xor(st.v2, 32);
    run = stat_merge(run, stat_merge(st, o, it), it);
  }
  if (lk == 0 && ok) p.part[(size_t)lr * p.n_vtiles + b] = run;
}

// The weight-streaming kernel serves bf16 calls of at most 32 rows whose
// k-quarter fits the stream waves' registers (H = 512 .. 2048, a multiple of 512).
bool head_t1_fits(const dmtp_head_desc& d, int M) {
  return d.dtype == DMTP_BF16 && M <= 32 && d.H % 512 == 0 && d.H <= 2048;
}

template <int KQ>
hipError_t launch_head_t1_kq(const HeadParams& p, int n_tiles, const GemmEvents& ev, hipStream_t s) {
  static_assert(kT1Lds <= 160 * 1024, "head LDS");
  hipError_t e = hipFuncSetAttribute((const void*)head_t1_kernel<KQ>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kT1Lds);
  if (e != hipSuccess) return e;
  // one workgroup per partial (p.n_vtiles of them)
  if (ev.start && ev.stop)
    hipExtLaunchKernelGGL((head_t1_kernel<KQ>), dim3(p.n_vtiles), dim3(kT1Threads), (uint32_t)kT1Lds, s,
                          ev.start, ev.stop, 0u, p, n_tiles);
  else
    hipLaunchKernelGGL((head_t1_kernel<KQ>), dim3(p.n_vtiles), dim3(kT1Threads), kT1Lds, s, p, n_tiles);
  return hipGetLastError();
}

// partials per row of the streaming kernel: one per workgroup
int head_t1_grid(int V) { return std::min((V + 31) / 32, kT1Grid); }

hipError_t launch_head_t1(const HeadParams& p, const GemmEvents& ev, hipStream_t s) {
  const int n_tiles = (p.V + 31) / 32;
  switch (p.H / 64) {
    case 8: return launch_head_t1_kq<8>(p, n_tiles, ev, s);
    case 16: return launch_head_t1_kq<16>(p, n_tiles, ev, s);
    case 24: return launch_head_t1_kq<24>(p, n_tiles, ev, s);
    default: return launch_head_t1_kq<32>(p, n_tiles, ev, s);
  }
}

constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void head_merge_kernel(HeadParams p, int final_greedy) {
  __shared__ RowStat red[kMergeThreads / kWave];
  const int m = blockIdx.x;
  const float it = inv_temp(p.temperature, m);
  RowStat st = stat_empty();
  // tiles t = threadIdx.x + kMergeThreads j, merged in increasing j; eight
  // partials are loaded together before they are merged
  constexpr int PB = 8;
  const RowStat* pr = p.part + (size_t)m * p.n_vtiles;
  for (int t0 = threadIdx.x; t0 < p.n_vtiles; t0 += PB * kMergeThreads) {
    RowStat v[PB];
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const int t = t0 + j * kMergeThreads;
      v[j] = t < p.n_vtiles ? pr[t] : stat_empty();
    }
#pragma unroll
    for (int j = 0; j < PB; ++j)
      if (t0 + j * kMergeThreads < p.n_vtiles) st = stat_merge(st, v[j], it);
  }
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
    p.rmax[m] = st.m;
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

// Block masses of the drawn rows.  A work item is (list index, chunk of
// kMassChunk entries) and belongs to one wave: lane l takes the 8-entry groups
// l, l + 64, ... of the chunk (kMassU of them) and loads them all before any
// arithmetic.  Group u of lanes 16 q .. 16 q + 15 covers one block of
// kDrawBlock entries; its mass sum exp((l_j - max) / t) is added lane by lane
// and then over the 16 lanes in a fixed order.  One exp2 per entry: the pass
// is bound by the read of the logits.
constexpr int kMassWaves = 4;
constexpr int kMassU = 4;
constexpr int kMassGrid = 8192;                  // workgroups of the mass pass (grid-stride over the items)
constexpr int kMassChunk = kWave * 8 * kMassU;   // 2048 vocabulary entries per item
static_assert(kMassChunk % kDrawBlock == 0 && kDrawBlock == 16 * 8, "block layout of a mass item");
static_assert(512 * kMassU == kMassChunk, "group stride");

__device__ __forceinline__ Top2 wave_top2(Top2 t) {
#pragma unroll
  for (int mask = 1; mask < kWave; mask <<= 1) t = top2_merge(t, top2_shfl_xor(t, mask));
  return t;
}

__global__ __launch_bounds__(kMassWaves * kWave) void head_mass_kernel(HeadParams p) {
  const int lane = threadIdx.x % kWave;
  const int nw = gridDim.x * kMassWaves;
  const int items = p.list_count[0] * p.n_chunks;
  const bool vec = (p.V & 3) == 0;
  for (int item = blockIdx.x * kMassWaves + threadIdx.x / kWave; item < items; item += nw) {
    const int li = item / p.n_chunks, ch = item % p.n_chunks;
    const int m = p.list[li];
    const float sc = 1.4426950408889634f / p.temperature[m];   // log2(e) / t
    const float ref = p.rmax[m];
    const float* lr = p.logits + (size_t)p.store_row[m] * p.V;
    const int base = ch * kMassChunk + 8 * lane;
    float s[kMassU];
    if (vec && ch * kMassChunk + kMassChunk <= p.V) {
      float4 a[kMassU], b[kMassU];
#pragma unroll
      for (int u = 0; u < kMassU; ++u) {
        a[u] = *(const float4*)(lr + base + 512 * u);
        b[u] = *(const float4*)(lr + base + 512 * u + 4);
      }
#pragma unroll
      for (int u = 0; u < kMassU; ++u) {
        const float l[8] = {a[u].x, a[u].y, a[u].z, a[u].w, b[u].x, b[u].y, b[u].z, b[u].w};
        float t = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) t += hw_exp2((l[k] - ref) * sc);
        s[u] = t;
      }
    } else {
      // the last chunk (or rows that are not 16-byte aligned): entry by entry
#pragma unroll
      for (int u = 0; u < kMassU; ++u) {
        const int j0 = base + 512 * u;
        float t = 0.f;
        for (int k = 0; k < 8 && j0 + k < p.V; ++k) t += hw_exp2((lr[j0 + k] - ref) * sc);
        s[u] = t;
      }
    }
#pragma unroll
    for (int u = 0; u < kMassU; ++u) {
#pragma unroll
      for (int mask = 1; mask < 16; mask <<= 1) s[u] += shfl_xor(s[u], mask);
      const int blk = ch * (kMassChunk / kDrawBlock) + 4 * u + (lane >> 4);
      if ((lane & 15) == 0 && blk < p.n_blocks) p.mass[(size_t)li * p.n_blocks + blk] = s[u];
    }
  }
}

// Level 1 of a two-level draw over the n_blocks block masses of one row, by
// the kFinThreads threads of one workgroup: thread i takes blocks 8 i .. 8 i + 7
// (+ 8 kFinThreads r), one Philox call per eight blocks; score log Z_b + g1_b,
// zero-mass blocks out of the race.  Each wave's best two go through LDS and
// every thread merges them in wave order, so all threads return the same pick.
constexpr int kFinThreads = 256;

// Z_b comes from the mass pass (mass != NULL), or from the GEMM epilogue's
// statistics of the row's vocabulary tiles, which are the blocks: a tile's
// (max m, sum of exp((l - m) / t)) gives log Z_b = m / t + log s.
__device__ __forceinline__ Top2 draw_block(const float* mass, const RowStat* tiles, float it,
                                           int n_blocks, uint64_t seed, uint64_t key, Top2* red) {
  const float ln2 = 0.6931471805599453f;
  Top2 t = top2_empty();
  for (int b0 = 8 * threadIdx.x; b0 < n_blocks; b0 += 8 * kFinThreads) {
    float lz[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      lz[k] = -INFINITY;
      if (b0 + k < n_blocks) {
        if (mass) {
          const float z = mass[b0 + k];
          if (z > 0.f) lz[k] = hw_log2(z) * ln2;
        } else {
          const RowStat st = tiles[b0 + k];
          if (st.s > 0.f) lz[k] = fmaf(st.m, it, hw_log2(st.s) * ln2);
        }
      }
    }
    uint32_t w[8];
    philox_words8(seed, key, (uint64_t)(b0 >> 3), w, 1);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (lz[k] > -INFINITY) top2_push_inc(t, lz[k] + gumbel_fast(w[k]), b0 + k);
  }
  t = wave_top2(t);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = t;
  __syncthreads();
  Top2 r = red[0];
#pragma unroll
  for (int i = 1; i < kFinThreads / kWave; ++i) r = top2_merge(r, red[i]);
  return r;
}

// One workgroup per row: the token (a two-level draw, the planted row's
// argmax, or the argmax) and its decision margin.
__global__ __launch_bounds__(kFinThreads) void head_finalize_kernel(HeadParams p) {
  __shared__ Top2 red[kFinThreads / kWave];
  const int m = blockIdx.x;
  const int lane = threadIdx.x % kWave;
  int tok = p.amax[m];
  float g = p.gap_greedy[m];
  if (p.plant_row && p.plant_row[m] >= 0 && p.plant_row[m] < p.M) {
    tok = p.amax[p.plant_row[m]];
    g = p.gap_greedy[p.plant_row[m]];
  } else if (p.temperature && p.temperature[m] > 0.f && p.draw_key[m] != DMTP_NO_DRAW) {
    const bool stored = p.store_row && p.store_row[m] >= 0 && p.store_row[m] < p.logits_rows;
    const int li = (stored && !p.block_stats) ? p.list_pos[m] : -1;
    if (!stored) {
      tok = -1;  // a sampled row without a stored logits row
      g = 0.f;
    } else {
      const uint64_t key = p.draw_key[m];
      const float it = 1.f / p.temperature[m];
      const Top2 t1 =
          draw_block(p.block_stats ? nullptr : p.mass + (size_t)li * p.n_blocks,
                     p.part + (size_t)m * p.n_vtiles, it, p.n_blocks, p.seed, key, red);
      if (threadIdx.x >= kWave) return;   // level 2 is wave 0's (no barrier follows)
      // level 2 over the chosen block: lanes 0..15 take 8 entries each
      const float* lr = p.logits + (size_t)p.store_row[m] * p.V;
      Top2 t2 = top2_empty();
      const bool any = t1.v1 > -INFINITY;
      const int j0 = (any ? t1.i1 : 0) * kDrawBlock + 8 * lane;
      if (any && lane < kDrawBlock / 8 && j0 < p.V) {
        float l[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) l[k] = j0 + k < p.V ? lr[j0 + k] : 0.f;
        uint32_t w[8];
        philox_words8(p.seed, key, (uint64_t)(j0 >> 3), w, 0);
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (j0 + k < p.V) top2_push_inc(t2, fmaf(l[k], it, gumbel_fast(w[k])), j0 + k);
      }
      t2 = wave_top2(t2);
      tok = (any && t2.i1 != 0x7FFFFFFF) ? t2.i1 : -1;
      g = tok >= 0 ? fminf(t1.v1 - t1.v2, t2.v1 - t2.v2) : 0.f;
    }
  }
  if (threadIdx.x == 0) {
    p.token[m] = tok;
    if (p.gap) p.gap[m] = g;
  }
}

typedef GemmTile<64, 64, 32, 32, 2, 2> HeadTileF32;
typedef GemmTile<128, 64, 64, 32, 1, 1> HeadTileBF16;   // H not a multiple of 128

struct WsLayout {
  size_t prepared, part, amax, gapg, rmax, list, list_pos, list_count, mass, total;
  int n_vtiles, n_blocks, n_chunks;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(const dmtp_head_desc& d, int M) {
  WsLayout w;
  // partials per row: one per workgroup (streaming kernel), per 128 (MFMA
  // kernel) or per 64 vocabulary rows
  w.n_vtiles = head_t1_fits(d, M)                        ? head_t1_grid(d.V)
               : (d.dtype == DMTP_BF16 && d.H % 128 == 0) ? (d.V + 127) / 128
                                                          : (d.V + 63) / 64;
  w.n_blocks = (d.V + kDrawBlock - 1) / kDrawBlock;
  w.n_chunks = (d.V + kMassChunk - 1) / kMassChunk;
  const size_t esz = d.dtype == DMTP_BF16 ? 2 : 4;
  size_t o = 0;
  w.prepared = o; o = align256(o + (size_t)(M + 15) * d.H * esz);   // rows padded for the fragment layout
  w.part = o; o = align256(o + (size_t)w.n_vtiles * M * sizeof(RowStat));
  w.amax = o; o = align256(o + (size_t)M * 4);
  w.gapg = o; o = align256(o + (size_t)M * 4);
  w.rmax = o; o = align256(o + (size_t)M * 4);
  w.list = o; o = align256(o + (size_t)M * 4);
  w.list_pos = o; o = align256(o + (size_t)M * 4);
  w.list_count = o; o = align256(o + 4);
  w.mass = o;
  if (d.temperature) o = align256(o + (size_t)M * w.n_blocks * sizeof(float));
  w.total = o;
  return w;
}

// The packed copy of W: one thread per 16-byte piece of out.  Piece 8 r + j of
// block s of tile t is columns 64 s + 8 (j ^ ((r >> 1) & 7)) .. + 7 of row
// 128 t + r (zeros past V): the stage image of the register-input GEMM.
constexpr int kPackBV = 128, kPackWK = 64;
__global__ void head_pack_kernel(const uint16_t* __restrict__ W, int V, int H, uint4* __restrict__ out,
                                 size_t pieces) {
  const int per_row = kPackWK / 8, per_block = kPackBV * per_row, blocks = H / kPackWK;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < pieces; i += (size_t)gridDim.x * blockDim.x) {
    const int idx = (int)(i % per_block);
    const size_t tb = i / per_block;
    const int sblk = (int)(tb % blocks);
    const size_t t = tb / blocks;
    const int r = idx / per_row, j = idx % per_row;
    const size_t row = t * kPackBV + r;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < (size_t)V)
      v = *(const uint4*)(W + row * H + kPackWK * sblk + 8 * swz_chunk<kPackWK>(r, j));
    out[i] = v;
  }
}

}  // namespace

size_t head_pack_bytes(int V, int H) { return (size_t)((V + kPackBV - 1) / kPackBV) * kPackBV * H * 2; }

hipError_t head_pack_run(const void* W, int V, int H, void* out, hipStream_t s) {
  static_assert(kPackBV == HeadXr<7>::BV && kPackWK == HeadXr<7>::WK, "stage of the register-input GEMM");
  const size_t pieces = head_pack_bytes(V, H) / 16;
  const int blocks = (int)std::min<size_t>((pieces + 255) / 256, 8192);
  hipLaunchKernelGGL(head_pack_kernel, dim3(blocks), dim3(256), 0, s, (const uint16_t*)W, V, H, (uint4*)out, pieces);
  return hipGetLastError();
}

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
  p.Wp = (d.dtype == DMTP_BF16 && d.H % 128 == 0) ? d.w_packed : nullptr;
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
  p.rmax = (float*)(base + w.rmax);
  p.mass = (float*)(base + w.mass);
  p.n_blocks = w.n_blocks;
  p.n_chunks = w.n_chunks;
  p.token = d.token;
  p.row_max = d.row_max;
  p.lse = d.lse;
  p.gap = d.gap;

  // The 32-wide-slice kernels read their input rows slice-major (each k-slice
  // of all rows one contiguous block) unless the caller asked for the
  // row-major prepared rows; otherwise a single segment of ready head-input
  // rows is read in place.
  const bool mf32 = d.dtype == DMTP_BF16 && d.H % 128 == 0;
  p.block_stats = mf32 && !head_t1_fits(d, M) && w.n_vtiles == w.n_blocks;
  p.a_frag = mf32 && !d.prepared && !head_t1_fits(d, M) && head_xr_fits(M, d.H);
  p.a_sl = (mf32 && !d.prepared && head_mf32_bk(M) == 32) ? 32 : 0;
  const bool direct =
      !p.a_sl && d.n_seg == 1 && !d.seg[0].g_norm && d.seg[0].ld == d.H && !d.prepared;
  p.A = direct ? d.seg[0].x : p.prepared;
  hipError_t e = hipSuccess;
  if (!direct) {
    hipLaunchKernelGGL(head_prep_kernel, dim3(M), dim3(kPrepThreads), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (mf32) {
    GemmEvents ev;
    ev.start = (hipEvent_t)d.gemm_start_event;
    ev.stop = (hipEvent_t)d.gemm_stop_event;
    e = head_t1_fits(d, M) ? launch_head_t1(p, ev, s) : launch_head_mf32_any(p, ev, s);
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
  // The matrix-core GEMM's statistics are per 128-entry vocabulary tile, so
  // they are the draws' block masses; other GEMMs need the mass pass.
  if (d.temperature && !p.block_stats) {
    hipLaunchKernelGGL(head_plan_kernel, dim3(1), dim3(1024), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(head_mass_kernel, dim3(kMassGrid), dim3(kMassWaves * kWave), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(head_finalize_kernel, dim3(M), dim3(kFinThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace dmtp

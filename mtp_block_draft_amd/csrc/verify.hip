// Block verification.
//
//   main   one thread per sequence: greedy prefix compare, or the accept tests
//          u < p_i(d_i) / q_i(d_i) evaluated in log space from two gathered
//          logits and the row lse values; builds a deterministic list of the
//          sequences that need a draw (correction from max(0, p - q), or bonus
//          from p_K)
//   mass   the draws' memory-bound pass over the float32 rows, split into
//          vocabulary chunks: the mass of max(0, p - q) (and of p, for the bonus
//          and for the zero-residual fallback) in every block of kDrawBlock
//          entries
//   final  per drawn sequence, a two-level Gumbel-max draw: a block by its
//          mass, then an entry of that block by its log weight, and writes the
//          correction/bonus token
//   stats  acceptance histogram of a batch of verify rounds, added to a running
//          histogram, and the statistics derived from it
#include <hip/hip_ext.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dmtp {

namespace {

// Mass work items are (sequence in the draw list, vocabulary chunk of kChunk
// entries), one wave each: lane l takes the 8-entry groups l, l + 64, ...
// (kScanU of them) and loads them all before any arithmetic; group u of lanes
// 16 q .. 16 q + 15 is one block of kDrawBlock entries.
// 512 entries of each row per work item and a grid that covers every item of
// a batch-128 draw in one pass: measured faster than longer items (the pass is
// short, so its memory latency chain dominates)
constexpr int kScanWaves = 4;
constexpr int kScanU = 1;
constexpr int kScanGrid = 8192;   // workgroups of the mass pass (grid-stride over the items)

// 16 bytes of a logits row
__device__ __forceinline__ float4 ld_row4(const float* q) { return *(const float4*)q; }
constexpr int kChunk = kWave * 8 * kScanU;
static_assert(kChunk % kDrawBlock == 0 && kDrawBlock == 16 * 8, "block layout of a mass item");

// Row pointers and lse values of a drawn sequence: the residual at row L
// (p: target row K + L, q: candidate row L), or the bonus from target row 2K.
struct DrawRows {
  const float* pr;
  const float* qr;
  float lse_p, lse_q, it;
  bool resid;
};

struct VerifyParams {
  int B, K, V;
  const int32_t* t1;
  const int32_t* drafts;
  const int32_t* target;
  const float* temperature;
  const float* logits;
  const float* t1_lse;
  const float* draft_lse;
  const float* target_lse;
  const float* u_acc;
  uint64_t seed;
  const uint64_t* final_key;
  int32_t* accept_len;
  int32_t* out_tokens;
  int32_t* n_out;
  int target_only;
  // workspace
  int32_t* list;       // [B]
  int32_t* list_pos;   // [B]
  int32_t* count;      // [1]
  int32_t* mode;       // [B]: 0 greedy/done, 1 residual draw at row L, 2 bonus draw
  float* mass_r;       // [B, n_blocks] residual block masses (list order)
  float* mass_p;       // [B, n_blocks] block masses of p
  DrawRows* draws;     // [B] rows and lse values of each listed draw (list order)
  int n_blocks, n_chunks;
};

__device__ __forceinline__ int cand(const VerifyParams& p, int b, int i) {
  return i == 0 ? p.t1[b] : p.drafts[(size_t)b * (p.K - 1) + i - 1];
}

__device__ __forceinline__ DrawRows draw_rows(const VerifyParams& p, int b) {
  const int K = p.K, V = p.V, L = p.accept_len[b];
  const float* rows = p.logits + (size_t)b * (2 * K + 1) * V;
  DrawRows r;
  r.resid = p.mode[b] == 1;
  r.it = 1.f / p.temperature[b];
  r.pr = rows + (size_t)(K + L) * V;
  r.qr = rows + (size_t)L * V;
  r.lse_p = p.target_lse[(size_t)b * (K + 1) + L];
  r.lse_q = r.resid ? (L == 0 ? p.t1_lse[b] : p.draft_lse[(size_t)b * (K - 1) + L - 1]) : 0.f;
  return r;
}

__global__ __launch_bounds__(1024) void verify_main_kernel(VerifyParams p) {
  __shared__ int32_t sc[1024 / kWave];
  __shared__ int32_t base;
  if (threadIdx.x == 0) base = 0;
  __syncthreads();
  const int K = p.K, V = p.V;
  for (int c0 = 0; c0 < p.B; c0 += blockDim.x) {
    const int b = c0 + threadIdx.x;
    int flag = 0;
    if (b < p.B) {
      // target-only verification compares with the target's picks at any temperature
      const float t = (p.temperature && !p.target_only) ? p.temperature[b] : 0.f;
      int L = 0, md = 0;
      // the candidates, their gathered logits and lse values and the uniforms
      // of eight rows at a time are loaded before any test, so a sequence
      // costs one memory latency per eight rows instead of one per row
      constexpr int G = 8;
      if (t > 0.f) {
        const float it = 1.f / t;
        const float* rows = p.logits + (size_t)b * (2 * K + 1) * V;
        L = K;
        for (int i0 = 0; i0 < K && L == K; i0 += G) {
          int d[G];
          float lq[G], lp[G], u[G];
#pragma unroll
          for (int g = 0; g < G; ++g) d[g] = i0 + g < K ? cand(p, b, i0 + g) : -1;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const int i = i0 + g;
            lq[g] = lp[g] = 0.f;
            u[g] = 1.f;
            if (i < K && d[g] >= 0 && d[g] < V) {
              lq[g] = rows[(size_t)i * V + d[g]] * it -
                      (i == 0 ? p.t1_lse[b] : p.draft_lse[(size_t)b * (K - 1) + i - 1]);
              lp[g] = rows[(size_t)(K + i) * V + d[g]] * it - p.target_lse[(size_t)b * (K + 1) + i];
              u[g] = p.u_acc[(size_t)b * K + i];
            }
          }
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const int i = i0 + g;
            if (i >= K || L < K) continue;
            const bool acc = d[g] >= 0 && d[g] < V && ((u[g] <= 0.f) || (logf(u[g]) < lp[g] - lq[g]));
            if (!acc) L = i;
          }
        }
        md = L < K ? 1 : 2;
        flag = 1;
      } else {
        for (int i0 = 0; i0 < K && L == i0; i0 += G) {
          int d[G], y[G];
#pragma unroll
          for (int g = 0; g < G; ++g) {
            d[g] = i0 + g < K ? cand(p, b, i0 + g) : -1;
            y[g] = i0 + g < K ? p.target[(size_t)b * (K + 1) + i0 + g] : -2;
          }
#pragma unroll
          for (int g = 0; g < G; ++g)
            if (L == i0 + g && i0 + g < K && d[g] == y[g]) ++L;
        }
      }
      int32_t* out = p.out_tokens + (size_t)b * (K + 1);
      for (int i = 0; i < L; ++i) out[i] = cand(p, b, i);
      out[L] = md ? -1 : p.target[(size_t)b * (K + 1) + L];
      for (int i = L + 1; i <= K; ++i) out[i] = -1;
      p.accept_len[b] = L;
      p.n_out[b] = L + 1;
      p.mode[b] = md;
    }
    // exclusive prefix of the flags: within a wave by ballot, across waves
    // through LDS (one barrier per pass over the batch)
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
    const uint64_t bal = __ballot(flag);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) sc[wv] = __popcll(bal);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wv; ++w) off += sc[w];
    int total = 0;
    for (int w = 0; w < (int)(blockDim.x / kWave); ++w) total += sc[w];
    if (b < p.B) {
      const int pos = off + before;
      p.list_pos[b] = flag ? pos : -1;
      if (flag) {
        p.list[pos] = b;
        p.draws[pos] = draw_rows(p, b);
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) base += total;
    __syncthreads();
  }
  if (threadIdx.x == 0) p.count[0] = base;
}


// p_j and the residual max(0, p_j - q_j) of one entry from its logits: with
// a = log p_j and c = log q_j, the residual is p_j (1 - e^(c - a)) where a > c,
// the difference taken without cancelling.
__device__ __forceinline__ void entry_mass(float lp, float lq, const DrawRows& r, float& pm,
                                           float& rm) {
  const float log2e = 1.4426950408889634f;
  const float a = fmaf(lp, r.it, -r.lse_p);
  pm = hw_exp2(a * log2e);
  rm = 0.f;
  if (r.resid) {
    const float c = fmaf(lq, r.it, -r.lse_q);
    rm = a > c ? pm * one_minus_exp(c - a) : 0.f;
  }
}

__global__ __launch_bounds__(kScanWaves * kWave) void verify_mass_kernel(VerifyParams p) {
  const int lane = threadIdx.x % kWave;
  const int nw = gridDim.x * kScanWaves;
  const int items = p.count[0] * p.n_chunks;
  const int V = p.V;
  const bool vec = (V & 3) == 0;
  for (int item = blockIdx.x * kScanWaves + threadIdx.x / kWave; item < items; item += nw) {
    const int li = item / p.n_chunks, ch = item % p.n_chunks;
    const DrawRows r = p.draws[li];
    const int base = ch * kChunk + 8 * lane;
    float sp[kScanU], sr[kScanU];
    if (vec && ch * kChunk + kChunk <= V) {
      float4 pa[kScanU], pb[kScanU], qa[kScanU], qb[kScanU];
#pragma unroll
      for (int u = 0; u < kScanU; ++u) {
        pa[u] = ld_row4(r.pr + base + 512 * u);
        pb[u] = ld_row4(r.pr + base + 512 * u + 4);
      }
      if (r.resid) {
#pragma unroll
        for (int u = 0; u < kScanU; ++u) {
          qa[u] = ld_row4(r.qr + base + 512 * u);
          qb[u] = ld_row4(r.qr + base + 512 * u + 4);
        }
      } else {
#pragma unroll
        for (int u = 0; u < kScanU; ++u) qa[u] = qb[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kScanU; ++u) {
        const float lp[8] = {pa[u].x, pa[u].y, pa[u].z, pa[u].w, pb[u].x, pb[u].y, pb[u].z, pb[u].w};
        const float lq[8] = {qa[u].x, qa[u].y, qa[u].z, qa[u].w, qb[u].x, qb[u].y, qb[u].z, qb[u].w};
        float tp = 0.f, tr = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          float pm, rm;
          entry_mass(lp[k], lq[k], r, pm, rm);
          tp += pm;
          tr += rm;
        }
        sp[u] = tp;
        sr[u] = tr;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kScanU; ++u) {
        const int j0 = base + 512 * u;
        float tp = 0.f, tr = 0.f;
        for (int k = 0; k < 8 && j0 + k < V; ++k) {
          float pm, rm;
          entry_mass(r.pr[j0 + k], r.resid ? r.qr[j0 + k] : 0.f, r, pm, rm);
          tp += pm;
          tr += rm;
        }
        sp[u] = tp;
        sr[u] = tr;
      }
    }
#pragma unroll
    for (int u = 0; u < kScanU; ++u) {
#pragma unroll
      for (int mask = 1; mask < 16; mask <<= 1) {
        sp[u] += shfl_xor(sp[u], mask);
        sr[u] += shfl_xor(sr[u], mask);
      }
      const int blk = ch * (kChunk / kDrawBlock) + 4 * u + (lane >> 4);
      if ((lane & 15) == 0 && blk < p.n_blocks) {
        p.mass_p[(size_t)li * p.n_blocks + blk] = sp[u];
        if (r.resid) p.mass_r[(size_t)li * p.n_blocks + blk] = sr[u];
      }
    }
  }
}

__device__ __forceinline__ Top2 wave_top2(Top2 t) {
#pragma unroll
  for (int mask = 1; mask < kWave; mask <<= 1) t = top2_merge(t, top2_shfl_xor(t, mask));
  return t;
}

// One workgroup per drawn sequence: the residual draw (or, when the residual
// has no mass, the fallback draw from p), or the bonus draw from p_K.  Level 1
// picks a block by log Z_b + g1_b -- thread i takes blocks 8 i .. 8 i + 7, one
// Philox call per eight blocks, and the waves' best two are merged through
// LDS in wave order -- and level 2 (wave 0) an entry of that block by its log
// weight plus g0_j, the log residual log p_j + log(1 - e^(c - a)) taken
// without cancelling.
constexpr int kFinThreads = 256;

__global__ __launch_bounds__(kFinThreads) void verify_final_kernel(VerifyParams p) {
  __shared__ Top2 red[kFinThreads / kWave];
  __shared__ int any_resid;
  const float ln2 = 0.6931471805599453f;
  const int b = blockIdx.x;
  const int lane = threadIdx.x % kWave;
  const int li = p.list_pos[b];
  if (li < 0) return;   // the whole workgroup, before any barrier
  DrawRows r = p.draws[li];
  const uint64_t key = p.final_key[b];
  const int nb = p.n_blocks;
  const float* mr = p.mass_r + (size_t)li * nb;
  const float* mp = p.mass_p + (size_t)li * nb;
  // both mass rows are loaded before the choice between them is known
  float zr[8], zp[8];
  Top2 tr = top2_empty(), tp = top2_empty();
  if (threadIdx.x == 0) any_resid = 0;
  __syncthreads();
  for (int b0 = 8 * threadIdx.x; b0 < nb; b0 += 8 * kFinThreads) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      zp[k] = b0 + k < nb ? mp[b0 + k] : 0.f;
      zr[k] = (r.resid && b0 + k < nb) ? mr[b0 + k] : 0.f;
    }
    uint32_t w[8];
    philox_words8(p.seed, key, (uint64_t)(b0 >> 3), w, 1);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float g = gumbel_fast(w[k]);
      if (zp[k] > 0.f) top2_push_inc(tp, fmaf(hw_log2(zp[k]), ln2, g), b0 + k);
      if (zr[k] > 0.f) top2_push_inc(tr, fmaf(hw_log2(zr[k]), ln2, g), b0 + k);
    }
  }
  // no positive residual mass in any block: the draw falls back to p
  if (r.resid && tr.v1 > -INFINITY) any_resid = 1;   // benign race: every writer stores 1
  __syncthreads();
  r.resid = r.resid && any_resid;
  Top2 t1 = wave_top2(r.resid ? tr : tp);
  if (lane == 0) red[threadIdx.x / kWave] = t1;
  __syncthreads();
  if (threadIdx.x >= kWave) return;   // level 2 is wave 0's (no barrier follows)
  t1 = red[0];
#pragma unroll
  for (int i = 1; i < kFinThreads / kWave; ++i) t1 = top2_merge(t1, red[i]);
  const bool found = t1.v1 > -INFINITY;
  Top2 t2 = top2_empty();
  const int j0 = (found ? t1.i1 : 0) * kDrawBlock + 8 * lane;
  if (found && lane < kDrawBlock / 8 && j0 < p.V) {
    float lp[8], lq[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      lp[k] = j0 + k < p.V ? r.pr[j0 + k] : 0.f;
      lq[k] = (r.resid && j0 + k < p.V) ? r.qr[j0 + k] : 0.f;
    }
    uint32_t w[8];
    philox_words8(p.seed, key, (uint64_t)(j0 >> 3), w, 0);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = j0 + k;
      if (j < p.V) {
        const float a = fmaf(lp[k], r.it, -r.lse_p);
        float lw = a;
        if (r.resid) {
          const float c = fmaf(lq[k], r.it, -r.lse_q);
          lw = a > c ? a + log1m_exp(c - a) : -INFINITY;
        }
        if (lw > -INFINITY) top2_push_inc(t2, lw + gumbel_fast(w[k]), j);
      }
    }
  }
  t2 = wave_top2(t2);
  const int y = (found && t2.i1 != 0x7FFFFFFF) ? t2.i1 : -1;
  if (lane == 0) p.out_tokens[(size_t)b * (p.K + 1) + p.accept_len[b]] = y;
}

constexpr int kStatsThreads = 256;
constexpr int kStatsMaxK = 64;

// One workgroup: LDS histogram of the batch, added to the running histogram
// bin by bin (a single writer per bin), then the summary from the result.
__global__ __launch_bounds__(kStatsThreads) void accept_stats_kernel(int B, int K,
                                                                     const int32_t* accept_len,
                                                                     int64_t* hist, double* summary) {
  __shared__ int32_t h[kStatsMaxK + 1];
  __shared__ int64_t tot[kStatsMaxK + 1];
  for (int k = threadIdx.x; k <= K; k += blockDim.x) h[k] = 0;
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const int L = accept_len[b];
    if (L >= 0 && L <= K) atomicAdd(&h[L], 1);
  }
  __syncthreads();
  for (int k = threadIdx.x; k <= K; k += blockDim.x) {
    const int64_t v = hist[k] + h[k];
    hist[k] = v;
    tot[k] = v;
  }
  __syncthreads();
  if (summary == nullptr || threadIdx.x != 0) return;
  int64_t n = 0, wsum = 0;
  for (int k = 0; k <= K; ++k) {
    n += tot[k];
    wsum += (int64_t)k * tot[k];
  }
  const double nan = __longlong_as_double(0x7FF8000000000000ll);
  const double N = (double)n;
  summary[0] = n ? 1.0 + (double)wsum / N : nan;
  summary[1] = n ? 1.0 - (double)tot[0] / N : nan;
  // P(L >= k) from the tail sums; conditional = P(L >= k) / P(L >= k - 1)
  int64_t geq_prev = n;
  int64_t tail = n;
  for (int k = 1; k <= K; ++k) {
    tail -= tot[k - 1];   // rounds with L >= k
    summary[2 + k - 1] = n ? (double)tail / N : nan;
    summary[2 + K + k - 1] = geq_prev ? (double)tail / (double)geq_prev : nan;
    geq_prev = tail;
  }
}

struct WsL {
  size_t list, list_pos, count, mode, mass_r, mass_p, draws, total;
  int n_blocks, n_chunks;
};

size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

WsL layout(const dmtp_verify_desc& d) {
  WsL w;
  w.n_blocks = (d.V + kDrawBlock - 1) / kDrawBlock;
  w.n_chunks = (d.V + kChunk - 1) / kChunk;
  size_t o = 0;
  w.list = o; o = al(o + (size_t)d.B * 4);
  w.list_pos = o; o = al(o + (size_t)d.B * 4);
  w.count = o; o = al(o + 4);
  w.mode = o; o = al(o + (size_t)d.B * 4);
  const bool draws = d.temperature && !d.target_only;
  w.mass_r = o;
  if (draws) o = al(o + (size_t)d.B * w.n_blocks * sizeof(float));
  w.mass_p = o;
  if (draws) o = al(o + (size_t)d.B * w.n_blocks * sizeof(float));
  w.draws = o;
  if (draws) o = al(o + (size_t)d.B * sizeof(DrawRows));
  w.total = o;
  return w;
}

}  // namespace

size_t verify_ws_bytes(const dmtp_verify_desc& d) { return layout(d).total; }

hipError_t verify_run(const dmtp_verify_desc& d, void* ws, hipStream_t s) {
  const WsL w = layout(d);
  char* base = (char*)ws;
  VerifyParams p;
  p.B = d.B;
  p.K = d.K;
  p.V = d.V;
  p.t1 = d.t1;
  p.drafts = d.drafts;
  p.target = d.target;
  p.temperature = d.temperature;
  p.logits = d.logits;
  p.t1_lse = d.t1_lse;
  p.draft_lse = d.draft_lse;
  p.target_lse = d.target_lse;
  p.u_acc = d.u_acc;
  p.seed = d.seed;
  p.final_key = d.final_key;
  p.accept_len = d.accept_len;
  p.out_tokens = d.out_tokens;
  p.n_out = d.n_out;
  p.target_only = d.target_only != 0;
  p.list = (int32_t*)(base + w.list);
  p.list_pos = (int32_t*)(base + w.list_pos);
  p.count = (int32_t*)(base + w.count);
  p.mode = (int32_t*)(base + w.mode);
  p.mass_r = (float*)(base + w.mass_r);
  p.mass_p = (float*)(base + w.mass_p);
  p.draws = (DrawRows*)(base + w.draws);
  p.n_blocks = w.n_blocks;
  p.n_chunks = w.n_chunks;
  // one workgroup; up to 1024 threads, whole waves, as many as the batch needs
  const int vthreads = d.B >= 1024 ? 1024 : ((d.B + kWave - 1) / kWave) * kWave;
  hipLaunchKernelGGL(verify_main_kernel, dim3(1), dim3(vthreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !d.temperature || d.target_only) return e;
  if (d.mass_start_event && d.mass_stop_event)
    hipExtLaunchKernelGGL(verify_mass_kernel, dim3(kScanGrid), dim3(kScanWaves * kWave), 0u, s,
                          (hipEvent_t)d.mass_start_event, (hipEvent_t)d.mass_stop_event, 0u, p);
  else
    hipLaunchKernelGGL(verify_mass_kernel, dim3(kScanGrid), dim3(kScanWaves * kWave), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(verify_final_kernel, dim3(d.B), dim3(kFinThreads), 0, s, p);
  return hipGetLastError();
}

int accept_stats_max_k() { return kStatsMaxK; }

hipError_t accept_stats_run(const dmtp_stats_desc& d, hipStream_t s) {
  hipLaunchKernelGGL(accept_stats_kernel, dim3(1), dim3(kStatsThreads), 0, s, d.B, d.K,
                     d.accept_len, d.hist, d.summary);
  return hipGetLastError();
}

}  // namespace dmtp

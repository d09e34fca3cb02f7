// Block verification.
//
//   main   one thread per sequence: greedy prefix compare, or the accept tests
//          u < p_i(d_i) / q_i(d_i) evaluated in log space from two gathered
//          logits and the row lse values; builds a deterministic list of the
//          sequences that need a draw (correction from max(0, p - q), or bonus
//          from p_K)
//   scan   the draws: HBM-bound pass over the float32 rows, split into
//          vocabulary chunks, Gumbel-max over log(max(0, p - q)) (and over log p
//          for the zero-residual fallback) with the same Philox noise
//   final  merges the chunk maxima and writes the correction/bonus token
//   stats  acceptance histogram of a batch of verify rounds, added to a running
//          histogram, and the statistics derived from it
#include "common.hpp"
#include "kernels.hpp"

namespace dmtp {

namespace {

// Scan work items are (sequence in the draw list, vocabulary chunk of kChunk
// entries), one wave each: lane l takes the 8-entry blocks l, l + 64, ...
// (kScanU of them), loads them all before any arithmetic and keeps running
// top-2s in increasing index; one butterfly merge per item.
constexpr int kScanWaves = 4;
constexpr int kScanU = 4;
constexpr int kChunk = kWave * 8 * kScanU;

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
  Top2* part;          // [B, n_chunks, 2]
  int n_chunks;
};

__device__ __forceinline__ int cand(const VerifyParams& p, int b, int i) {
  return i == 0 ? p.t1[b] : p.drafts[(size_t)b * (p.K - 1) + i - 1];
}

__global__ void verify_main_kernel(VerifyParams p) {
  __shared__ int32_t sc[1024];
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
      if (t > 0.f) {
        const float it = 1.f / t;
        const float* rows = p.logits + (size_t)b * (2 * K + 1) * V;
        L = K;
        for (int i = 0; i < K; ++i) {
          const int d = cand(p, b, i);
          bool acc = false;
          if (d >= 0 && d < V) {
            const float lq = rows[(size_t)i * V + d] * it -
                             (i == 0 ? p.t1_lse[b] : p.draft_lse[(size_t)b * (K - 1) + i - 1]);
            const float lp = rows[(size_t)(K + i) * V + d] * it - p.target_lse[(size_t)b * (K + 1) + i];
            const float u = p.u_acc[(size_t)b * K + i];
            acc = (u <= 0.f) || (logf(u) < lp - lq);
          }
          if (!acc) {
            L = i;
            break;
          }
        }
        md = L < K ? 1 : 2;
        flag = 1;
      } else {
        while (L < K && cand(p, b, L) == p.target[(size_t)b * (K + 1) + L]) ++L;
      }
      int32_t* out = p.out_tokens + (size_t)b * (K + 1);
      for (int i = 0; i < L; ++i) out[i] = cand(p, b, i);
      out[L] = md ? -1 : p.target[(size_t)b * (K + 1) + L];
      for (int i = L + 1; i <= K; ++i) out[i] = -1;
      p.accept_len[b] = L;
      p.n_out[b] = L + 1;
      p.mode[b] = md;
    }
    sc[threadIdx.x] = flag;
    __syncthreads();
    for (int o = 1; o < (int)blockDim.x; o <<= 1) {
      const int v = threadIdx.x >= (unsigned)o ? sc[threadIdx.x - o] : 0;
      __syncthreads();
      sc[threadIdx.x] += v;
      __syncthreads();
    }
    if (b < p.B) {
      const int pos = base + sc[threadIdx.x] - flag;
      p.list_pos[b] = flag ? pos : -1;
      if (flag) p.list[pos] = b;
    }
    __syncthreads();
    if (threadIdx.x == blockDim.x - 1) base += sc[threadIdx.x];
    __syncthreads();
  }
  if (threadIdx.x == 0) p.count[0] = base;
}

// Per entry j of the scanned rows: a = log p_j = lp_j / t - lse_p; the bonus /
// fallback score a + g_j; in residual mode c = log q_j and the residual score
// log(p_j - q_j) + g_j where p_j > q_j (the same Gumbel noise g_j).
__device__ __forceinline__ void verify_entry(float lp, float lq, float it, float lse_p, float lse_q,
                                             bool resid, uint32_t word, int j, Top2& tr, Top2& tp) {
  const float g = gumbel_fast(word);
  const float a = fmaf(lp, it, -lse_p);
  top2_push_inc(tp, a + g, j);
  if (resid) {
    const float c = fmaf(lq, it, -lse_q);
    const float sres = a > c ? a + log1m_exp(c - a) : -INFINITY;
    top2_push_inc(tr, sres + g, j);
  }
}

__global__ __launch_bounds__(kScanWaves * kWave) void verify_scan_kernel(VerifyParams p) {
  const int lane = threadIdx.x % kWave;
  const int nw = gridDim.x * kScanWaves;
  const int items = p.count[0] * p.n_chunks;
  const int K = p.K, V = p.V;
  const bool vec = (V & 3) == 0;
  for (int item = blockIdx.x * kScanWaves + threadIdx.x / kWave; item < items; item += nw) {
    const int li = item / p.n_chunks, ch = item % p.n_chunks;
    const int b = p.list[li];
    const int L = p.accept_len[b];
    const bool resid = p.mode[b] == 1;
    const float it = 1.f / p.temperature[b];
    const float* rows = p.logits + (size_t)b * (2 * K + 1) * V;
    // residual at row L: p row K + L, q row L; bonus: p row 2K
    const float* pr = rows + (size_t)(K + L) * V;
    const float* qr = rows + (size_t)L * V;
    const float lse_p = p.target_lse[(size_t)b * (K + 1) + L];
    const float lse_q = resid ? (L == 0 ? p.t1_lse[b] : p.draft_lse[(size_t)b * (K - 1) + L - 1]) : 0.f;
    const uint64_t key = p.final_key[b];
    const int base = ch * kChunk + 8 * lane;
    Top2 tr = top2_empty(), tp = top2_empty();
    if (vec && ch * kChunk + kChunk <= V) {
      float4 pa[kScanU], pb[kScanU], qa[kScanU], qb[kScanU];
#pragma unroll
      for (int u = 0; u < kScanU; ++u) {
        pa[u] = *(const float4*)(pr + base + 512 * u);
        pb[u] = *(const float4*)(pr + base + 512 * u + 4);
      }
      if (resid) {
#pragma unroll
        for (int u = 0; u < kScanU; ++u) {
          qa[u] = *(const float4*)(qr + base + 512 * u);
          qb[u] = *(const float4*)(qr + base + 512 * u + 4);
        }
      } else {
#pragma unroll
        for (int u = 0; u < kScanU; ++u) qa[u] = qb[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kScanU; ++u) {
        const int j0 = base + 512 * u;
        uint32_t w[8];
        philox_words8(p.seed, key, (uint64_t)(j0 >> 3), w);
        const float lp[8] = {pa[u].x, pa[u].y, pa[u].z, pa[u].w, pb[u].x, pb[u].y, pb[u].z, pb[u].w};
        const float lq[8] = {qa[u].x, qa[u].y, qa[u].z, qa[u].w, qb[u].x, qb[u].y, qb[u].z, qb[u].w};
#pragma unroll
        for (int k = 0; k < 8; ++k) verify_entry(lp[k], lq[k], it, lse_p, lse_q, resid, w[k], j0 + k, tr, tp);
      }
    } else {
      for (int u = 0; u < kScanU; ++u) {
        const int j0 = base + 512 * u;
        if (j0 >= V) break;
        uint32_t w[8];
        philox_words8(p.seed, key, (uint64_t)(j0 >> 3), w);
        for (int k = 0; k < 8 && j0 + k < V; ++k)
          verify_entry(pr[j0 + k], resid ? qr[j0 + k] : 0.f, it, lse_p, lse_q, resid, w[k], j0 + k,
                       tr, tp);
      }
    }
#pragma unroll
    for (int mask = 1; mask < kWave; mask <<= 1) {
      tr = top2_merge(tr, top2_shfl_xor(tr, mask));
      tp = top2_merge(tp, top2_shfl_xor(tp, mask));
    }
    if (lane == 0) {
      p.part[((size_t)li * p.n_chunks + ch) * 2 + 0] = tr;
      p.part[((size_t)li * p.n_chunks + ch) * 2 + 1] = tp;
    }
  }
}

// One wave per row: the chunk maxima of the row's draw are merged across lanes.
__global__ __launch_bounds__(256) void verify_final_kernel(VerifyParams p) {
  const int b = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (b >= p.B) return;
  const int li = p.list_pos[b];
  if (li < 0) return;
  Top2 tr = top2_empty(), tp = top2_empty();
  for (int c = lane; c < p.n_chunks; c += kWave) {
    tr = top2_merge(tr, p.part[((size_t)li * p.n_chunks + c) * 2 + 0]);
    tp = top2_merge(tp, p.part[((size_t)li * p.n_chunks + c) * 2 + 1]);
  }
#pragma unroll
  for (int mask = 1; mask < kWave; mask <<= 1) {
    tr = top2_merge(tr, top2_shfl_xor(tr, mask));
    tp = top2_merge(tp, top2_shfl_xor(tp, mask));
  }
  // residual mode with no positive residual falls back to p
  const int y = (p.mode[b] == 1 && tr.v1 > -INFINITY) ? tr.i1 : tp.i1;
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
  size_t list, list_pos, count, mode, part, total;
  int n_chunks;
};

size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

WsL layout(const dmtp_verify_desc& d) {
  WsL w;
  w.n_chunks = (d.V + kChunk - 1) / kChunk;
  size_t o = 0;
  w.list = o; o = al(o + (size_t)d.B * 4);
  w.list_pos = o; o = al(o + (size_t)d.B * 4);
  w.count = o; o = al(o + 4);
  w.mode = o; o = al(o + (size_t)d.B * 4);
  w.part = o;
  if (d.temperature && !d.target_only) o = al(o + (size_t)d.B * w.n_chunks * 2 * sizeof(Top2));
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
  p.part = (Top2*)(base + w.part);
  p.n_chunks = w.n_chunks;
  hipLaunchKernelGGL(verify_main_kernel, dim3(1), dim3(1024), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !d.temperature || d.target_only) return e;
  hipLaunchKernelGGL(verify_scan_kernel, dim3(2048), dim3(kScanWaves * kWave), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(verify_final_kernel, dim3((d.B + 3) / 4), dim3(256), 0, s, p);
  return hipGetLastError();
}

int accept_stats_max_k() { return kStatsMaxK; }

hipError_t accept_stats_run(const dmtp_stats_desc& d, hipStream_t s) {
  hipLaunchKernelGGL(accept_stats_kernel, dim3(1), dim3(kStatsThreads), 0, s, d.B, d.K,
                     d.accept_len, d.hist, d.summary);
  return hipGetLastError();
}

}  // namespace dmtp

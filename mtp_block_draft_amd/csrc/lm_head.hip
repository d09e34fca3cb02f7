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
  const float wa = a.s > 0.f ? a.s * expf((a.m - r.m) * inv_t) : 0.f;
  const float wb = b.s > 0.f ? b.s * expf((b.m - r.m) * inv_t) : 0.f;
  r.s = wa + wb;
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
  RowStat* part;         // [n_vtiles, M]
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
  gemm_mainloop<T>(acc, lds, p.prepared, (size_t)p.H, p.M, p.W, (size_t)p.H, p.V, m0, n0, 0, p.H);
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
    p.part[(size_t)blockIdx.x * p.M + row] = st;
  }
}

constexpr int kMergeThreads = 256;

__global__ __launch_bounds__(kMergeThreads) void head_merge_kernel(HeadParams p, int final_greedy) {
  __shared__ RowStat red[kMergeThreads / kWave];
  const int m = blockIdx.x;
  const float it = inv_temp(p.temperature, m);
  RowStat st = stat_empty();
  for (int t = threadIdx.x; t < p.n_vtiles; t += blockDim.x)
    st = stat_merge(st, p.part[(size_t)t * p.M + m], it);
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
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int j = j0 + k;
        if (j < p.V) top2_push(t, lr[j] * it + gumbel_of_word(w[k]), j);
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

__global__ void head_finalize_kernel(HeadParams p) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
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
      for (int c = 0; c < p.n_chunks; ++c) t = top2_merge(t, p.scan_part[(size_t)li * p.n_chunks + c]);
      tok = t.i1;
      g = t.v1 - t.v2;
    }
  }
  p.token[m] = tok;
  if (p.gap) p.gap[m] = g;
}

typedef GemmTile<64, 64, 32, 32, 1, 1> HeadTileBF16;
typedef GemmTile<64, 64, 32, 32, 2, 2> HeadTileF32;

struct WsLayout {
  size_t prepared, part, amax, gapg, list, list_pos, list_count, scan, total;
  int n_vtiles, n_chunks;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(const dmtp_head_desc& d, int M) {
  WsLayout w;
  w.n_vtiles = (d.V + 63) / 64;
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

  hipLaunchKernelGGL(head_prep_kernel, dim3(M), dim3(kPrepThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (d.dtype == DMTP_BF16) {
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
  hipLaunchKernelGGL(head_finalize_kernel, dim3((M + 255) / 256), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace dmtp

// Block attention of the drafter: every block slot's query reads all context
// keys of its sequence (or the last `window`) and all S block keys, no mask.
//
// Work split: one workgroup per (context chunk, kv head, sequence).  The query
// rows of a workgroup are the S slots x G query heads that share the kv head,
// so GQA costs one pass over each context tile.  Context K/V tiles of 64 keys
// are staged in LDS (V transposed so that the PV product reads it
// K-contiguously); S = Q K^T and O += P V run on bf16 matrix cores, with the
// float32 queries and probabilities split into hi/lo bf16 planes.  Each chunk
// leaves an unnormalised partial (O, running max m, running sum l); a combine
// kernel merges the chunks exactly and adds the S block keys in float32.
//
// bf16 context K/V (attn_wave_kernel): one wave per (context chunk, kv head,
// 32-row query tile, sequence), no workgroup barriers.  32-key K and V tiles
// stream through a private ring of LDS stages filled by global_load_lds copies;
// S^T = K Q^T is one 32 x 32 MFMA tile with the query planes held in
// registers, so every lane owns one query row and its online softmax needs a
// single exchange with lane l ^ 32; O^T += V^T P^T takes the V^T operand from
// the transposing LDS read (ds_read_b64_tr_b16) and P^T straight from the
// softmax registers.  The float32 K/V path keeps the workgroup kernel.
#include <hip/hip_ext.h>

#include "dma.hpp"
#include "kernels.hpp"

namespace dmtp {

namespace {

constexpr int kAttnThreads = 256;
constexpr int KT = 64;  // keys per LDS tile
constexpr size_t kLdsLimit = 160 * 1024;

template <int RT, int D, int KVP>
struct AttnCfg {
  static constexpr int NQP = 16 * RT;          // padded query rows
  static constexpr int LDQ = D + 8;            // bf16 row stride of Q and K tiles
  static constexpr int LDT = KT + 8;           // bf16 row stride of V^T and P tiles
  static constexpr int Q_ELEMS = 2 * NQP * LDQ;
  static constexpr int K_ELEMS = KVP * KT * LDQ;
  static constexpr int V_ELEMS = KVP * D * LDT;
  static constexpr int P_ELEMS = 2 * NQP * LDT;
  static constexpr int OT = RT * (D / 16);     // 16x16 output tiles
  static constexpr int OT_PER_WAVE = (OT + 3) / 4;
  static constexpr size_t LDS_BYTES =
      (size_t)(Q_ELEMS + K_ELEMS + V_ELEMS + P_ELEMS) * 2 + (size_t)NQP * KT * 4 + (size_t)3 * NQP * 4;
};

template <int RT, int D, int KVP>
__global__ __launch_bounds__(kAttnThreads) void attn_chunk_kernel(
    const float* __restrict__ q, const void* __restrict__ ctx_k, const void* __restrict__ ctx_v,
    const int32_t* __restrict__ cu_ctx, int ctx_rows, int Hkv, int NQ, int chunk, int n_chunks,
    int window, float scale, float* __restrict__ part_o, float* __restrict__ part_ml) {
  typedef AttnCfg<RT, D, KVP> C;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* Qs = smem;                      // [2][NQP][LDQ]
  uint16_t* Ks = Qs + C::Q_ELEMS;           // [KVP][KT][LDQ]
  uint16_t* Vt = Ks + C::K_ELEMS;           // [KVP][D][LDT]
  uint16_t* Ps = Vt + C::V_ELEMS;           // [2][NQP][LDT]
  float* Ss = (float*)(Ps + C::P_ELEMS);    // [NQP][KT]
  float* m_run = Ss + C::NQP * KT;
  float* l_run = m_run + C::NQP;
  float* alpha = l_run + C::NQP;

  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int L = ctx_len_of(cu_ctx, b, ctx_rows);
  const int start = (window > 0 && L > window) ? L - window : 0;
  const int k_lo = start + c * chunk;
  const int k_hi = min(k_lo + chunk, L);
  const size_t pbase = (((size_t)b * Hkv + kvh) * n_chunks + c);
  float* po = part_o + pbase * C::NQP * D;
  float* pml = part_ml + pbase * 2 * C::NQP;
  if (k_lo >= k_hi) {  // empty chunk: neutral partial
    for (int r = threadIdx.x; r < C::NQP; r += blockDim.x) {
      pml[r] = -INFINITY;
      pml[C::NQP + r] = 0.f;
    }
    return;
  }

  // queries -> two bf16 planes
  const float* qg = q + ((size_t)b * Hkv + kvh) * NQ * D;
  for (int e = threadIdx.x; e < C::NQP * D; e += blockDim.x) {
    const int r = e / D, k = e % D;
    const float v = r < NQ ? qg[(size_t)r * D + k] : 0.f;
    uint16_t hi, lo;
    split_bf16(v, hi, lo);
    Qs[r * C::LDQ + k] = hi;
    Qs[C::NQP * C::LDQ + r * C::LDQ + k] = lo;
  }
  for (int r = threadIdx.x; r < C::NQP; r += blockDim.x) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }

  f32x4_t acc[C::OT_PER_WAVE];
#pragma unroll
  for (int t = 0; t < C::OT_PER_WAVE; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const size_t row_stride = (size_t)Hkv * D;      // elements between consecutive keys
  const size_t seq0 = (size_t)cu_ctx[b];
  const int fr = lane & 15, fk = (lane >> 4) * 8;

  for (int kt = k_lo; kt < k_hi; kt += KT) {
    const int nk = min(KT, k_hi - kt);
    // ---- stage K [KT][D] and V^T [D][KT]
    if (KVP == 1) {
      const uint16_t* kg = (const uint16_t*)ctx_k;
      const uint16_t* vg = (const uint16_t*)ctx_v;
      for (int e = threadIdx.x; e < KT * D / 8; e += blockDim.x) {
        const int key = e / (D / 8), c8 = e % (D / 8);
        uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        if (key < nk) {
          const size_t off = (seq0 + kt + key) * row_stride + (size_t)kvh * D + 8 * c8;
          kv = *(const uint4*)(kg + off);
          vv = *(const uint4*)(vg + off);
        }
        *(uint4*)(Ks + key * C::LDQ + 8 * c8) = kv;
        const uint16_t* vh = (const uint16_t*)&vv;
#pragma unroll
        for (int j = 0; j < 8; ++j) Vt[(8 * c8 + j) * C::LDT + key] = vh[j];
      }
    } else {
      const float* kg = (const float*)ctx_k;
      const float* vg = (const float*)ctx_v;
      for (int e = threadIdx.x; e < KT * D / 4; e += blockDim.x) {
        const int key = e / (D / 4), c4 = e % (D / 4);
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
        if (key < nk) {
          const size_t off = (seq0 + kt + key) * row_stride + (size_t)kvh * D + 4 * c4;
          kv = *(const float4*)(kg + off);
          vv = *(const float4*)(vg + off);
        }
        const float kf[4] = {kv.x, kv.y, kv.z, kv.w}, vf[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint16_t hi, lo;
          split_bf16(kf[j], hi, lo);
          Ks[key * C::LDQ + 4 * c4 + j] = hi;
          Ks[KT * C::LDQ + key * C::LDQ + 4 * c4 + j] = lo;
          split_bf16(vf[j], hi, lo);
          Vt[(4 * c4 + j) * C::LDT + key] = hi;
          Vt[D * C::LDT + (4 * c4 + j) * C::LDT + key] = lo;
        }
      }
    }
    __syncthreads();

    // ---- S = Q K^T: wave w owns keys 16w .. 16w + 15 for all row tiles
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < D; k0 += 32) {
        const uint4 qh = *(const uint4*)(Qs + (16 * rt + fr) * C::LDQ + k0 + fk);
        const uint4 ql = *(const uint4*)(Qs + C::NQP * C::LDQ + (16 * rt + fr) * C::LDQ + k0 + fk);
        const uint4 kh = *(const uint4*)(Ks + (16 * wave + fr) * C::LDQ + k0 + fk);
        s = mfma_16x16x32(qh, kh, s);
        s = mfma_16x16x32(ql, kh, s);
        if (KVP == 2) {
          const uint4 kl = *(const uint4*)(Ks + KT * C::LDQ + (16 * wave + fr) * C::LDQ + k0 + fk);
          s = mfma_16x16x32(qh, kl, s);
        }
      }
      const int key = 16 * wave + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * rt + 4 * (lane >> 4) + i;
        Ss[row * KT + key] = key < nk ? s[i] * scale : -INFINITY;
      }
    }
    __syncthreads();

    // ---- online softmax: four threads per row, 16 keys each
    for (int t = threadIdx.x; t < C::NQP * 4; t += blockDim.x) {
      const int row = t >> 2, qd = t & 3;
      const float* sr = Ss + row * KT + 16 * qd;
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sr[j]);
      mx = fmaxf(mx, __shfl_xor(mx, 1, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 2, kWave));
      const float m_old = m_run[row];
      const float m_new = fmaxf(m_old, mx);
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = expf(sr[j] - m_new);
        sum += p;
        uint16_t hi, lo;
        split_bf16(p, hi, lo);
        Ps[row * C::LDT + 16 * qd + j] = hi;
        Ps[C::NQP * C::LDT + row * C::LDT + 16 * qd + j] = lo;
      }
      sum += __shfl_xor(sum, 1, kWave);
      sum += __shfl_xor(sum, 2, kWave);
      if (qd == 0) {
        const float a = expf(m_old - m_new);   // 0 on the first tile (m_old = -inf)
        alpha[row] = a;
        l_run[row] = l_run[row] * a + sum;
        m_run[row] = m_new;
      }
    }
    __syncthreads();

    // ---- O = alpha O + P V
#pragma unroll
    for (int t = 0; t < C::OT_PER_WAVE; ++t) {
      const int tile = wave + 4 * t;
      if (tile >= C::OT) break;
      const int rt = tile / (D / 16), dt = tile % (D / 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] *= alpha[16 * rt + 4 * (lane >> 4) + i];
#pragma unroll
      for (int k0 = 0; k0 < KT; k0 += 32) {
        const uint4 ph = *(const uint4*)(Ps + (16 * rt + fr) * C::LDT + k0 + fk);
        const uint4 pl = *(const uint4*)(Ps + C::NQP * C::LDT + (16 * rt + fr) * C::LDT + k0 + fk);
        const uint4 vh = *(const uint4*)(Vt + (16 * dt + fr) * C::LDT + k0 + fk);
        acc[t] = mfma_16x16x32(ph, vh, acc[t]);
        acc[t] = mfma_16x16x32(pl, vh, acc[t]);
        if (KVP == 2) {
          const uint4 vl = *(const uint4*)(Vt + D * C::LDT + (16 * dt + fr) * C::LDT + k0 + fk);
          acc[t] = mfma_16x16x32(ph, vl, acc[t]);
        }
      }
    }
    __syncthreads();
  }

  // ---- write the unnormalised partial
#pragma unroll
  for (int t = 0; t < C::OT_PER_WAVE; ++t) {
    const int tile = wave + 4 * t;
    if (tile >= C::OT) break;
    const int rt = tile / (D / 16), dt = tile % (D / 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * rt + 4 * (lane >> 4) + i;
      po[(size_t)row * D + 16 * dt + (lane & 15)] = acc[t][i];
    }
  }
  for (int r = threadIdx.x; r < C::NQP; r += blockDim.x) {
    pml[r] = m_run[r];
    pml[C::NQP + r] = l_run[r];
  }
}

// ------------------------------------------------------ bf16 K/V, per wave --
template <int D, int NBUF_>
struct WaveAttn {
  static constexpr int KT = 32;                  // keys per tile
  static constexpr int CPR = D / 8;              // 16-byte chunks per key row
  static constexpr int RPI = 64 / CPR;           // key rows per 1 KB copy
  static constexpr int INSTR = KT / RPI;         // copies per operand per tile
  static constexpr int PER_TILE = 2 * INSTR;
  static constexpr int NBUF = NBUF_;
  static constexpr int STAGE = 2 * KT * D;       // bf16 elements: K tile, then V tile
  static constexpr size_t LDS_BYTES = (size_t)NBUF * STAGE * 2;
  static constexpr int DS = D / 16;              // k-steps of Q K^T
  static constexpr int DT = D / 32;              // 32-row tiles of O^T
};

// XOR swizzles of the 16-byte chunks of key row r.  K is read 16 rows x one
// chunk per pass: distinct chunk positions for any 16 consecutive rows.  V is
// read by the transposing load as 4 consecutive rows x 2 chunks: 2 (r % 4)
// keeps those eight chunks apart.
template <int D>
__device__ __forceinline__ int swz_key(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
__device__ __forceinline__ int swz_val(int r) { return 2 * (r & 3); }

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// bf16 hi/lo planes of the pair (a, b), packed two to a word: the hi floats
// are read back from the packed word by a byte permute (low half to the top,
// zeros below) and a mask, instead of converting each value again.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi2, uint32_t& lo2) {
  const bf16x2_t h = {(__bf16)a, (__bf16)b};
  hi2 = __builtin_bit_cast(uint32_t, h);
  const float ha = __uint_as_float(__builtin_amdgcn_perm(0u, hi2, 0x01000c0cu));
  const float hb = __uint_as_float(hi2 & 0xffff0000u);
  const bf16x2_t l = {(__bf16)(a - ha), (__bf16)(b - hb)};
  lo2 = __builtin_bit_cast(uint32_t, l);
}

// Buffer descriptor over `bytes` bytes from `base` (raw, dword data format):
// the copies below address one K or V tile through it.
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// 16 bytes per lane from descriptor r at byte offset vo (this lane) + so
// (uniform) to LDS at dst + 16 lane; non-temporal (the context is read once).
__device__ __forceinline__ void buf_dma16(buf_rsrc r, uint32_t vo, uint32_t so, uint16_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, vo, so, 0, 2);
}

// Four bf16 of the transposing LDS read; see the V^T operand below.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Workgroup: the waves of up to kAttnQtw 32-row query tiles of one (context
// chunk, kv head, sequence).  They share one LDS ring of K/V tiles, so a chunk
// is read once for all of them: wave 0 issues every copy and waits for it, a
// workgroup barrier per tile hands the tile to the others.  With more query
// tiles than that, blockIdx.y also selects the group of tiles.
constexpr int kAttnQtw = 4;

// At most 256 registers, so that two waves share a SIMD (two multi-wave
// workgroups a CU).
template <int D, int NBUF>
__global__ __launch_bounds__(64 * kAttnQtw) __attribute__((amdgpu_waves_per_eu(2))) void attn_wave_kernel(
    const float* __restrict__ q, const uint16_t* __restrict__ ctx_k,
    const uint16_t* __restrict__ ctx_v, const int32_t* __restrict__ cu_ctx, int ctx_rows, int Hkv,
    int NQ, int NQP, int chunk, int n_chunks, int window, float scale, float* __restrict__ part_o,
    float* __restrict__ part_ml) {
  typedef WaveAttn<D, NBUF> C;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int c = blockIdx.x, kvh = blockIdx.y % Hkv, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
  const int qt = (blockIdx.y / Hkv) * waves + wave;
  const bool live = 32 * qt < NQP;     // a wave past the last query tile only joins the barriers
  const bool issuer = wave == 0;
  const int lane = threadIdx.x & 63, lr = lane & 31, g = lane >> 5;
  const int L = ctx_len_of(cu_ctx, b, ctx_rows);
  const int start = (window > 0 && L > window) ? L - window : 0;
  const int k_lo = start + c * chunk;
  const int k_hi = min(k_lo + chunk, L);
  const size_t slot = ((size_t)b * Hkv + kvh) * n_chunks + c;
  float* po = part_o + slot * NQP * D;
  float* pml = part_ml + slot * 2 * NQP;
  const int qrow = 32 * qt + lr;   // this lane's query row
  if (k_lo >= k_hi) {               // empty chunk: neutral partial
    if (g == 0 && live) {
      pml[qrow] = -INFINITY;
      pml[NQP + qrow] = 0.f;
    }
    return;
  }
  const int nkeys = k_hi - k_lo;
  const int nt = (nkeys + C::KT - 1) / C::KT;

  // copies: instruction i of a tile moves key rows RPI i .. RPI i + RPI - 1;
  // lane supplies row RPI i + lane / CPR, chunk position lane % CPR.  They are
  // buffer copies over one tile's rows: the tile's first row is the
  // descriptor's base, instruction i's first row a scalar offset, and the lane
  // part a vector offset that depends on i only through the key swizzle, which
  // repeats every KPER instructions (RPI KPER = 16 rows); the value swizzle
  // reads r % 4 = lane row % 4 and does not depend on i.
  constexpr int KPER = 16 / C::RPI;
  static_assert(C::RPI % 4 == 0 && C::INSTR % KPER == 0, "copy layout");
  const uint32_t row_bytes = (uint32_t)(Hkv * D * 2);
  const size_t head0 = ((size_t)cu_ctx[b] + k_lo) * row_bytes + (size_t)kvh * D * 2;
  const char* kbase = (const char*)ctx_k + head0;
  const char* vbase = (const char*)ctx_v + head0;
  const int rr = lane / C::CPR, pos = lane % C::CPR;
  uint32_t koff[KPER];
#pragma unroll
  for (int i = 0; i < KPER; ++i) koff[i] = rr * row_bytes + 16 * (pos ^ swz_key<D>(C::RPI * i + rr));
  const uint32_t voff = rr * row_bytes + 16 * (pos ^ swz_val(rr));
  // context K/V is read once per call: non-temporal copies
  auto issue = [&](int t) __attribute__((always_inline)) {
    uint16_t* st = smem + (t % C::NBUF) * C::STAGE;
    const size_t t0 = (size_t)C::KT * t * row_bytes;
    const int tile_bytes = C::KT * (int)row_bytes;
    const buf_rsrc kr = make_rsrc(kbase + t0, tile_bytes), vr = make_rsrc(vbase + t0, tile_bytes);
    if (C::KT * (t + 1) <= nkeys) {
#pragma unroll
      for (int i = 0; i < C::INSTR; ++i) {
        const uint32_t r0 = (uint32_t)(C::RPI * i) * row_bytes;
        buf_dma16(kr, koff[i % KPER], r0, st + i * 512);
        buf_dma16(vr, voff, r0, st + C::KT * D + i * 512);
      }
    } else {   // last tile: rows past the chunk end repeat its last key (masked below)
#pragma unroll
      for (int i = 0; i < C::INSTR; ++i) {
        const int r = C::RPI * i + rr;
        const uint32_t row = (uint32_t)min(r, nkeys - 1 - C::KT * t) * row_bytes;
        buf_dma16(kr, row + 16 * (pos ^ swz_key<D>(r)), 0, st + i * 512);
        buf_dma16(vr, row + 16 * (pos ^ swz_val(r)), 0, st + C::KT * D + i * 512);
      }
    }
  };

  // query fragments (B operand of S^T = K Q^T): column = query row, 8 d values,
  // times scale / ln 2 so that the scores come out in log2 units; loaded
  // before the first copies so that waiting for them leaves those in flight
  const float scale2 = scale * 1.4426950408889634f;
  const float* qg = q + (((size_t)b * Hkv + kvh) * NQ) * D;
  u32x4 qh[C::DS], ql[C::DS];
#pragma unroll
  for (int ds = 0; ds < C::DS; ++ds) {
    float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
    if (qrow < NQ) {
      x0 = *(const float4*)(qg + (size_t)qrow * D + 16 * ds + 8 * g);
      x1 = *(const float4*)(qg + (size_t)qrow * D + 16 * ds + 8 * g + 4);
      x0 = make_float4(x0.x * scale2, x0.y * scale2, x0.z * scale2, x0.w * scale2);
      x1 = make_float4(x1.x * scale2, x1.y * scale2, x1.z * scale2, x1.w * scale2);
    }
    uint32_t h[4], l[4];
    split2(x0.x, x0.y, h[0], l[0]);
    split2(x0.z, x0.w, h[1], l[1]);
    split2(x1.x, x1.y, h[2], l[2]);
    split2(x1.z, x1.w, h[3], l[3]);
    qh[ds] = u32x4{h[0], h[1], h[2], h[3]};
    ql[ds] = u32x4{l[0], l[1], l[2], l[3]};
  }

  if (issuer)
#pragma unroll
    for (int t0 = 0; t0 < C::NBUF - 1; ++t0)
      if (t0 < nt) issue(t0);

  f32x16_t o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
  // reference max of the exponentials, in log2 units, and running sum
  float m_run = -INFINITY, l_run = 0.f;

  // per-lane LDS offsets of the fragments (elements within a stage)
  int k_frag[C::DS];
#pragma unroll
  for (int ds = 0; ds < C::DS; ++ds) k_frag[ds] = lr * D + (((2 * ds + g) ^ swz_key<D>(lr)) << 3);
  // transposing read: in each block of 16 lanes, source lane s points at
  // V[kb + s / 4][dd0 + 4 (s % 4) ..]; lane o of the block receives
  // V[kb + j][dd0 + o], j = 0..3.  Key rows kb = 16 ks + 4 (blk / 2) + s / 4
  // (and kb + 8) only add whole rows, since the value swizzle reads kb % 4; the
  // chunk of column dd0 = 32 dt + .. is 4 dt + (0..3), and the swizzle (bits 1
  // and 2) can flip bit 0 of dt only, so dt = 2, 3 sit 8 chunks after dt = 0, 1.
  const int blk = lane >> 4, sl = lane & 15;
  int v_frag[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int dd = 32 * e + 16 * (blk & 1) + 4 * (sl & 3);
    const int ch = dd >> 3, half = (dd >> 2) & 1;
    const int ka = 4 * (blk >> 1) + (sl >> 2);
    v_frag[e] = C::KT * D + ka * D + ((ch ^ swz_val(ka)) << 3) + 4 * half;
  }

  for (int t = 0; t < nt; ++t) {
    if (issuer) wait_newer<C::PER_TILE, C::NBUF - 2>(min(nt - 1 - t, C::NBUF - 2));
    // tile t is in LDS for every wave; every wave has consumed tile t - 1 (its
    // MFMAs used the fragments read from it), whose buffer is refilled next
    ring_barrier();
    if (issuer && t + C::NBUF - 1 < nt) issue(t + C::NBUF - 1);
    const uint16_t* st = smem + (t % C::NBUF) * C::STAGE;

    // S^T[key][query] in log2 units: element i is key 8 (i / 4) + 4 g + i % 4
    // of this lane's query row; both query planes accumulate in one chain
    f32x16_t s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int ds = 0; ds < C::DS; ++ds) {
      const u32x4 kf = *(const u32x4*)(st + k_frag[ds]);
      s = mfma32(kf, qh[ds], s);
      s = mfma32(kf, ql[ds], s);
    }
    const int valid = nkeys - C::KT * t;   // keys of this tile inside the chunk
    if (valid < C::KT) {                   // the chunk's last tile: mask the repeated keys
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + 4 * g + (i & 3) >= valid) s[i] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    // The exponentials are taken against a reference max m_run, moved (and O
    // and l rescaled) only when some row's max exceeds it by more than 2^8:
    // the (m, l, O) triple stays exact for any reference, and a stale one
    // keeps every weight at most 2^8.  mx is the max of this lane's half of
    // the row's keys; the two halves (lanes l and l ^ 32) share m_run, so the
    // row max is exchanged only when the reference moves.
    if (__ballot(mx > m_run + 8.f) != 0) {
      const float m_new = fmaxf(m_run, fmaxf(mx, shfl_xor(mx, 32)));
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first tile
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
      m_run = m_new;
    }
    float ps = 0.f;
    uint32_t ph[8], pl[8];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float p0 = __builtin_amdgcn_exp2f(s[i] - m_run);
      const float p1 = __builtin_amdgcn_exp2f(s[i + 1] - m_run);
      ps += p0 + p1;
      split_pair(p0, p1, ph[i / 2], pl[i / 2]);
    }
    l_run += ps;   // this lane's half of the row; the halves are added at the end

    // O^T[dd][query] += V^T P^T over the tile's keys in two k-steps; k-step ks
    // takes this lane group's keys 16 ks + 4 g + (0..3) and 16 ks + 8 + 4 g + (0..3),
    // which are the P values it holds (i = 8 ks .. 8 ks + 7)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 pfh = u32x4{ph[4 * ks], ph[4 * ks + 1], ph[4 * ks + 2], ph[4 * ks + 3]};
      const u32x4 pfl = u32x4{pl[4 * ks], pl[4 * ks + 1], pl[4 * ks + 2], pl[4 * ks + 3]};
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const uint16_t* vp = st + v_frag[dt & 1] + 64 * (dt >> 1) + 16 * ks * D;
        const uint2 va = lds_read_tr16(vp);
        const uint2 vb = lds_read_tr16(vp + 8 * D);
        const u32x4 vf = u32x4{va.x, va.y, vb.x, vb.y};
        o[dt] = mfma32(vf, pfh, o[dt]);
        o[dt] = mfma32(vf, pfl, o[dt]);
      }
    }
  }

  l_run += shfl_xor(l_run, 32);
  // partial: O^T element i of tile dt is dd = 32 dt + 8 (i / 4) + 4 g + i % 4 of query qrow
  if (!live) return;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int dd = 32 * dt + 8 * gq + 4 * g;
      *(float4*)(po + (size_t)qrow * D + dd) =
          make_float4(o[dt][4 * gq], o[dt][4 * gq + 1], o[dt][4 * gq + 2], o[dt][4 * gq + 3]);
    }
  if (g == 0) {
    pml[qrow] = m_run * 0.6931471805599453f;   // back to natural units
    pml[NQP + qrow] = l_run;
  }
}

// Merge the chunk partials and the S block keys; o [B * S, Hq * D] as bf16
// planes (hi at o, lo at o + o_pst).  causal != 0: the query of slot s reads
// block keys 0..s only (the context keys in full).
// One wave per query row (rows r = 4 blockIdx.y + wave of kv head blockIdx.x);
// lane l owns dims l (and l + 64 when D = 128).  Every global load that does
// not depend on another one -- the query row, the chunk maxima and sums, the
// first CB chunk partials, and the block keys and values (staged once in LDS
// for the workgroup's four rows) -- is issued up front, so that a row costs
// about one memory latency instead of one per step.  The block-key scores are
// exact float32 dot products; chunk weights exp(m_c - M) are shared through
// the wave's slice of LDS, block weights by lane reads.
template <int D>
__global__ __launch_bounds__(kAttnThreads) void attn_combine_kernel(
    const float* __restrict__ q, const float* __restrict__ kb, const float* __restrict__ vb,
    const float* __restrict__ part_o, const float* __restrict__ part_ml, int Hkv, int G, int S,
    int NQP, int n_chunks, float scale, int causal, uint16_t* __restrict__ o, size_t o_pst) {
  constexpr int DL = D / kWave;   // dims per lane
  constexpr int CB = 16;          // chunk partials in flight per batch
  extern __shared__ __attribute__((aligned(16))) float kvs[];   // [2][S][D] block keys, values
  __shared__ float w_chunk[4][256];
  const int kvh = blockIdx.x % Hkv, b = blockIdx.x / Hkv;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int NQ = S * G;
  const int r = blockIdx.y * 4 + wave;
  const bool live = r < NQ;
  const int rr = live ? r : NQ - 1;   // a wave past the last row loads in range and stores nothing
  const size_t bh = (size_t)b * Hkv + kvh;

  float qv[DL];
#pragma unroll
  for (int i = 0; i < DL; ++i) qv[i] = q[(bh * NQ + rr) * D + lane + kWave * i];
  const float* ml = part_ml + bh * n_chunks * 2 * NQP;
  float mc[4], lc[4];   // chunks lane + 64 i (at most 256)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane + kWave * i;
    mc[i] = c < n_chunks ? ml[(size_t)c * 2 * NQP + rr] : -INFINITY;
    lc[i] = c < n_chunks ? ml[(size_t)c * 2 * NQP + NQP + rr] : 0.f;
  }
  // chunk c of this row at po + c * NQP * D; an empty chunk never wrote its
  // partial, which is read here but weighted out below
  const float* po = part_o + (bh * n_chunks * NQP + rr) * D + lane;
  const size_t cstride = (size_t)NQP * D;
  float pv[CB][DL];
#pragma unroll
  for (int c = 0; c < CB; ++c)
#pragma unroll
    for (int i = 0; i < DL; ++i) pv[c][i] = c < n_chunks ? po[c * cstride + kWave * i] : 0.f;
  {
    const float4* k4 = (const float4*)(kb + bh * S * D);
    const float4* v4 = (const float4*)(vb + bh * S * D);
    float4* s4 = (float4*)kvs;
    const int n4 = S * D / 4;
    for (int e = threadIdx.x; e < n4; e += kAttnThreads) {
      s4[e] = k4[e];
      s4[n4 + e] = v4[e];
    }
  }
  __syncthreads();
  if (!live) return;

  float M = fmaxf(fmaxf(mc[0], mc[1]), fmaxf(mc[2], mc[3]));
  float s_lane = -INFINITY;   // lane j < S: score of block key j (-inf where hidden)
  const int nvis = causal ? r / G + 1 : S;   // block keys this row sees (its own slot included)
  for (int j = 0; j < nvis; ++j) {
    float part = 0.f;
#pragma unroll
    for (int i = 0; i < DL; ++i) part = fmaf(qv[i], kvs[j * D + lane + kWave * i], part);
    const float sj = wave_sum(part) * scale;
    s_lane = lane == j ? sj : s_lane;
  }
  M = wave_max(fmaxf(M, s_lane));
  float Lsum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float w = mc[i] == -INFINITY ? 0.f : expf(mc[i] - M);
    w_chunk[wave][lane + kWave * i] = w;
    Lsum = fmaf(w, lc[i], Lsum);
  }
  const float wb = lane < nvis ? expf(s_lane - M) : 0.f;
  Lsum = wave_sum(Lsum + wb);
  __threadfence_block();
  __builtin_amdgcn_wave_barrier();

  float acc[DL];
#pragma unroll
  for (int i = 0; i < DL; ++i) acc[i] = 0.f;
  for (int c0 = 0; c0 < n_chunks; c0 += CB) {
    if (c0 > 0)
#pragma unroll
      for (int c = 0; c < CB; ++c)
#pragma unroll
        for (int i = 0; i < DL; ++i)
          pv[c][i] = c0 + c < n_chunks ? po[(c0 + c) * cstride + kWave * i] : 0.f;
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const float w = c0 + c < n_chunks ? w_chunk[wave][c0 + c] : 0.f;
#pragma unroll
      for (int i = 0; i < DL; ++i) acc[i] = w != 0.f ? fmaf(w, pv[c][i], acc[i]) : acc[i];
    }
  }
  for (int j = 0; j < nvis; ++j) {
    const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wb), j));
#pragma unroll
    for (int i = 0; i < DL; ++i) acc[i] = fmaf(w, kvs[S * D + j * D + lane + kWave * i], acc[i]);
  }
  const float inv_l = 1.0f / Lsum;
  const int sl = r / G, g = r % G;
  const size_t orow = ((size_t)b * S + sl) * ((size_t)Hkv * G * D) + ((size_t)kvh * G + g) * D;
#pragma unroll
  for (int i = 0; i < DL; ++i) store_planes(o, o_pst, orow + lane + kWave * i, acc[i] * inv_l);
}

template <int RT, int D, int KVP>
hipError_t launch_chunks(const AttnPlan& p, const float* q, const void* ck, const void* cv,
                         const int32_t* cu, int ctx_rows, float* po, float* pml, float scale,
                         hipStream_t s) {
  typedef AttnCfg<RT, D, KVP> C;
  if constexpr (C::LDS_BYTES > kLdsLimit) {
    return hipErrorInvalidConfiguration;   // refused on the host by attn_max_nq()
  }
  hipError_t e = hipFuncSetAttribute((const void*)attn_chunk_kernel<RT, D, KVP>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
  if (e != hipSuccess) return e;
  dim3 grid(p.n_chunks, p.Hkv, p.B);
  hipLaunchKernelGGL((attn_chunk_kernel<RT, D, KVP>), grid, dim3(kAttnThreads), C::LDS_BYTES, s, q,
                     ck, cv, cu, ctx_rows, p.Hkv, p.NQ, p.chunk, p.n_chunks, p.window, scale, po,
                     pml);
  return hipGetLastError();
}

template <int D, int KVP>
hipError_t dispatch_rt(const AttnPlan& p, const float* q, const void* ck, const void* cv,
                       const int32_t* cu, int cr, float* po, float* pml, float scale,
                       hipStream_t s) {
  const int rt = (p.NQ + 15) / 16;
  if (rt <= 1) return launch_chunks<1, D, KVP>(p, q, ck, cv, cu, cr, po, pml, scale, s);
  if (rt <= 2) return launch_chunks<2, D, KVP>(p, q, ck, cv, cu, cr, po, pml, scale, s);
  if (rt <= 4) return launch_chunks<4, D, KVP>(p, q, ck, cv, cu, cr, po, pml, scale, s);
  if (rt <= 6) return launch_chunks<6, D, KVP>(p, q, ck, cv, cu, cr, po, pml, scale, s);
  return launch_chunks<8, D, KVP>(p, q, ck, cv, cu, cr, po, pml, scale, s);
}

template <int D, int KVP>
size_t AttnCfg_bytes(int rt) {
  switch (rt) {
    case 1: return AttnCfg<1, D, KVP>::LDS_BYTES;
    case 2: return AttnCfg<2, D, KVP>::LDS_BYTES;
    case 4: return AttnCfg<4, D, KVP>::LDS_BYTES;
    case 6: return AttnCfg<6, D, KVP>::LDS_BYTES;
    default: return AttnCfg<8, D, KVP>::LDS_BYTES;
  }
}

int nqp_of(int NQ) {
  const int rt = (NQ + 15) / 16;
  return 16 * (rt <= 1 ? 1 : rt <= 2 ? 2 : rt <= 4 ? 4 : rt <= 6 ? 6 : 8);
}

}  // namespace

int attn_max_nq(int d, int kv_f32) {
  if (!kv_f32) return 256;   // per-wave kernel: any number of 32-row query tiles
  auto fits = [&](int rt) -> bool {
    return d == 64 ? AttnCfg_bytes<64, 2>(rt) <= kLdsLimit : AttnCfg_bytes<128, 2>(rt) <= kLdsLimit;
  };
  const int rts[5] = {8, 6, 4, 2, 1};
  for (int rt : rts)
    if (fits(rt)) return 16 * rt;
  return 0;
}

AttnPlan attn_plan(int B, int Hq, int Hkv, int S, int d, int max_ctx, int window, int kv_f32,
                   int ctx_rows) {
  AttnPlan p;
  p.B = B;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.S = S;
  p.d = d;
  p.NQ = S * p.G;
  p.kv_f32 = kv_f32;
  p.window = window;
  p.causal = 0;
  p.nqp = kv_f32 ? nqp_of(p.NQ) : 32 * ((p.NQ + 31) / 32);
  const int eff = (window > 0 && max_ctx > window) ? window : max_ctx;
  if (eff <= 0) {
    p.chunk = KT;
    p.n_chunks = 0;
    return p;
  }
  if (!kv_f32) {
    // per-wave kernel: about 768 query-tile waves over the context rows
    // actually present (ctx_rows / B per sequence on average), at least four
    // 32-key tiles each, at most 256 chunks per sequence for the combine.
    // Measured against 384 .. 3072 with one-wave workgroups (32 query rows
    // per kv head): fewer, longer chunks keep each wave's copy pipeline full
    // for longer.  When a kv head has several query tiles, their waves share
    // one workgroup and its ring, and 1536 waves (two such workgroups per CU,
    // so that one's softmax overlaps the other's matrix products) measured
    // faster than 768 and 3072.
    const long keys = (long)(ctx_rows > 0 ? ctx_rows : (long)B * eff);
    const long tiles = keys * Hkv * (p.nqp / 32);
    const long target = p.nqp > 32 ? 1536 : 768;
    long per = (tiles + target * 32 - 1) / (target * 32);
    if (per < 4) per = 4;
    int chunk = (int)(32 * per);
    const int min_chunk = ((eff + 255) / 256 + 31) / 32 * 32;
    if (chunk < min_chunk) chunk = min_chunk;
    p.chunk = chunk;
    p.n_chunks = (eff + chunk - 1) / chunk;
    return p;
  }
  const int pairs = B * Hkv;
  int want = (1024 + pairs - 1) / pairs;           // chunks per (sequence, kv head)
  int chunk = (eff + want - 1) / want;
  chunk = ((chunk + KT - 1) / KT) * KT;
  if (chunk < 4 * KT && eff > 4 * KT) chunk = 4 * KT;
  if (chunk < KT) chunk = KT;
  // the combine merges at most 256 chunk partials per row
  const int min_chunk = (((eff + 255) / 256 + KT - 1) / KT) * KT;
  if (chunk < min_chunk) chunk = min_chunk;
  p.chunk = chunk;
  p.n_chunks = (eff + chunk - 1) / chunk;
  return p;
}

size_t attn_ws_bytes(const AttnPlan& p) {
  const size_t nqp = p.nqp;
  const size_t slots = (size_t)p.B * p.Hkv * (p.n_chunks > 0 ? p.n_chunks : 1);
  return slots * nqp * p.d * 4 + slots * 2 * nqp * 4 + 256;
}

template <int D, int NBUF>
hipError_t launch_wave_n(const AttnPlan& p, const float* q, const void* ck, const void* cv,
                         const int32_t* cu, int ctx_rows, float* po, float* pml, float scale,
                         hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  typedef WaveAttn<D, NBUF> C;
  hipError_t e = hipFuncSetAttribute((const void*)attn_wave_kernel<D, NBUF>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int qtiles = p.nqp / 32;
  const int qtw = qtiles < kAttnQtw ? qtiles : kAttnQtw;
  dim3 grid(p.n_chunks, p.Hkv * ((qtiles + qtw - 1) / qtw), p.B);
  if (e0 && e1)
    hipExtLaunchKernelGGL((attn_wave_kernel<D, NBUF>), grid, dim3(64 * qtw), (uint32_t)C::LDS_BYTES, s, e0, e1,
                          0u, q, (const uint16_t*)ck, (const uint16_t*)cv, cu, ctx_rows, p.Hkv, p.NQ, p.nqp,
                          p.chunk, p.n_chunks, p.window, scale, po, pml);
  else
    hipLaunchKernelGGL((attn_wave_kernel<D, NBUF>), grid, dim3(64 * qtw), C::LDS_BYTES, s, q,
                       (const uint16_t*)ck, (const uint16_t*)cv, cu, ctx_rows, p.Hkv, p.NQ, p.nqp, p.chunk,
                       p.n_chunks, p.window, scale, po, pml);
  return hipGetLastError();
}

template <int D>
hipError_t launch_wave(const AttnPlan& p, const float* q, const void* ck, const void* cv,
                       const int32_t* cu, int ctx_rows, float* po, float* pml, float scale,
                       hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
  return launch_wave_n<D, 2>(p, q, ck, cv, cu, ctx_rows, po, pml, scale, s, e0, e1);
}

hipError_t attention(const AttnPlan& p, const float* q, const float* kb, const float* vb,
                     const void* ctx_k, const void* ctx_v, const int32_t* cu_ctx, int ctx_rows,
                     float* ws, uint16_t* o, hipStream_t s, hipEvent_t ev_start, hipEvent_t ev_stop) {
  const int nqp = p.nqp;
  const size_t slots = (size_t)p.B * p.Hkv * (p.n_chunks > 0 ? p.n_chunks : 1);
  float* po = ws;
  float* pml = ws + slots * nqp * p.d;
  const float scale = (float)(1.0 / sqrt((double)p.d));
  hipError_t e = hipSuccess;
  if (p.n_chunks > 0 && !p.kv_f32) {
    e = p.d == 64 ? launch_wave<64>(p, q, ctx_k, ctx_v, cu_ctx, ctx_rows, po, pml, scale, s, ev_start, ev_stop)
                  : launch_wave<128>(p, q, ctx_k, ctx_v, cu_ctx, ctx_rows, po, pml, scale, s, ev_start, ev_stop);
    if (e != hipSuccess) return e;
  } else if (p.n_chunks > 0) {
    const int cr = ctx_rows;
    e = p.d == 64 ? dispatch_rt<64, 2>(p, q, ctx_k, ctx_v, cu_ctx, cr, po, pml, scale, s)
                  : dispatch_rt<128, 2>(p, q, ctx_k, ctx_v, cu_ctx, cr, po, pml, scale, s);
    if (e != hipSuccess) return e;
  }
  const dim3 cgrid(p.B * p.Hkv, (p.NQ + 3) / 4);
  const size_t clds = (size_t)2 * p.S * p.d * sizeof(float);
  const size_t o_pst = (size_t)p.B * p.S * p.Hkv * p.G * p.d;
  if (p.d == 64)
    hipLaunchKernelGGL(attn_combine_kernel<64>, cgrid, dim3(kAttnThreads), clds, s, q, kb, vb, po, pml,
                       p.Hkv, p.G, p.S, nqp, p.n_chunks, scale, p.causal, o, o_pst);
  else
    hipLaunchKernelGGL(attn_combine_kernel<128>, cgrid, dim3(kAttnThreads), clds, s, q, kb, vb, po,
                       pml, p.Hkv, p.G, p.S, nqp, p.n_chunks, scale, p.causal, o, o_pst);
  return hipGetLastError();
}

}  // namespace dmtp

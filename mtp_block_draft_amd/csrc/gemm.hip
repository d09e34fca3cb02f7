// Float32-output GEMMs of the fusion projections and the drafter's layer
// projections: C = R + A B^T, where A is a float32 activation held as two bf16
// planes (hi + lo) and B a weight stored [out, in].
//
// These are small-M, weight-streaming shapes (M = the 32 fused rows or the
// B * S draft slots, N and K in the thousands).  A bf16 weight goes through
// gemm_dma_kernel: 32 x 32 x 16 MFMA tiles fed by a ring of LDS stages that
// global_load_lds copies fill several k-slices ahead (spread over the MFMAs of
// the slice before, with three or more stages), with K split into
// contiguous ranges so that about one workgroup per CU is busy; the float32
// partial sums are added in a fixed order by splitk_reduce4, so results are
// deterministic.  A float32 weight (the float32 configurations) goes through
// the plain tiled kernel of gemm_core.hpp.
#include "dma.hpp"
#include "gemm_core.hpp"
#include "kernels.hpp"

namespace dmtp {

namespace {

struct GemmParams {
  const void* A;
  size_t a_pst;
  size_t lda;
  int M;
  const void* B;
  size_t ldb;
  int N;
  int K;
  int splits;
  float* C;
  size_t ldc;
  const float* R;
  size_t ldr;
  float* part;   // [splits, M, N] when splits > 1
  const void* B2;  // rows n >= N1 of the weight come from B2 (NULL: B only)
  int N1;
  // SwiGLU output (LDS-ring kernel, one split): B holds the gate rows and B2
  // the up rows of F = N / 2 columns, taken as the interleaved matrix whose
  // 32-row block b is gate rows 16 b .. 16 b + 15, then up rows 16 b ..
  // 16 b + 15, so that each lane holds matching gate and up columns; act
  // [2][M][F] receives the bf16 planes of silu(gate) * up and C is not
  // written.  NULL: an ordinary product.
  uint16_t* act = nullptr;
};

// ------------------------------------------------- bf16 weight, LDS ring ----
// Workgroup of four waves, WAVES_N along N times 4 / WAVES_N along M; wave tile
// 32 UN (weight rows) x 32 UM (activation rows).  One k-slice of BK is staged
// as W [BN][BK] and the AP activation planes [AP][BM][BK], bf16, 16-byte chunks
// swizzled by swz_row (a 64-wide slice copies whole 128-byte lines).  AP = 2:
// a float32 activation as hi + lo planes; AP = 1: a bf16 activation as is.
template <int UN_, int UM_, int WAVES_N_, int BK_ = 64, int AP_ = 2>
struct DmaTile {
  static constexpr int UN = UN_, UM = UM_, WAVES_N = WAVES_N_, WAVES_M = 4 / WAVES_N_;
  static constexpr int BN = 32 * UN * WAVES_N, BM = 32 * UM * WAVES_M, BK = BK_, AP = AP_;
  static constexpr int CPR = BK / 8, KS = BK / 16;   // 16-byte chunks per row, k-steps per slice
  static constexpr int W_INSTR = BN * BK * 2 / 1024;   // 1 KB copies per slice
  static constexpr int A_INSTR = AP * BM * BK * 2 / 1024;
  static_assert((W_INSTR + A_INSTR) % 4 == 0 && A_INSTR % AP == 0, "copies per wave");
  static constexpr int PER_WAVE = (W_INSTR + A_INSTR) / 4;
  static constexpr int STAGE = (BN + AP * BM) * BK;    // bf16 elements
  static constexpr int NBUF_FIT = 147456 / (STAGE * 2);
  static constexpr int NBUF = NBUF_FIT > 8 ? 8 : NBUF_FIT;
  static_assert(NBUF >= 2 && PER_WAVE * (NBUF - 2) < 64, "ring");
  static constexpr size_t LDS_BYTES = (size_t)NBUF * STAGE * 2;
};

// Rotary cache scatter of a key/value projection, in place of C (the
// 128 x 32 tiles, one split): row m of the product is [keys Hkv d | values
// Hkv d]; its keys are rotated at positions[m] (pair (i, i + d / 2) of each
// head turned by pos * base^(-2 i / d), angles in float64) and keys and values
// stored in dtype at cache row dst_rows[m] ([rows, Hkv, d]; rows out of
// range are skipped).
struct RopeOut {
  const int32_t* positions;
  const int32_t* dst_rows;
  void* k_cache;
  void* v_cache;
  int Hkv, d, dtype, rows;
  float rope_base;
};

template <class T, int ROPE = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_dma_kernel(GemmParams p, int n_tiles_n, int n_tiles_m, RopeOut ro) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  const int total = n_tiles_n * n_tiles_m * p.splits;
  const int per = (total + 7) / 8;   // XCD-contiguous ranges (workgroup i runs on XCD i % 8)
  const int t = (blockIdx.x % 8) * per + blockIdx.x / 8;
  if (t >= total) return;
  // consecutive t: the row tiles that share one weight tile (and split), so
  // that they run together on one XCD and its L2 serves the second read of
  // the weights; then the splits, then the tiles along N
  const int m0 = (t % n_tiles_m) * T::BM;
  const int z = (t / n_tiles_m) % p.splits;
  const int n0 = (t / n_tiles_m / p.splits) * T::BN;
  const int nK = p.K / T::BK;   // K % BK == 0 is checked by the launcher
  const int s_begin = (int)((long)z * nK / p.splits), s_end = (int)((long)(z + 1) * nK / p.splits);
  const int ns = s_end - s_begin;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave % T::WAVES_N, wm = wave / T::WAVES_N;
  const int lr = lane & 31, lk = lane >> 5;
  const uint16_t* __restrict__ W = (const uint16_t*)p.B;
  const uint16_t* __restrict__ W2 = (const uint16_t*)p.B2;
  const uint16_t* __restrict__ A = (const uint16_t*)p.A;

  // sources of this wave's copies: W rows first, then the hi and lo planes of A
  // (rows clamped into range; their results are never stored)
  const uint16_t* src[T::PER_WAVE];
#pragma unroll
  for (int q = 0; q < T::PER_WAVE; ++q) {
    const int instr = wave * T::PER_WAVE + q;
    if (instr < T::W_INSTR) {
      const int idx = instr * 64 + lane, r = idx / T::CPR;
      const int wr = min(n0 + r, p.N - 1);
      const int gi = 16 * (wr >> 5) + (wr & 15);   // SwiGLU: gate / up row of interleaved row wr
      const uint16_t* wrow = p.act ? ((wr & 16) ? W2 : W) + (size_t)gi * p.ldb
                           : (W2 && wr >= p.N1) ? W2 + (size_t)(wr - p.N1) * p.ldb
                                                : W + (size_t)wr * p.ldb;
      src[q] = wrow + 8 * swz_chunk<T::BK>(r, idx % T::CPR);
    } else {
      const int j = instr - T::W_INSTR, pl = j / (T::A_INSTR / T::AP);
      const int idx = (j % (T::A_INSTR / T::AP)) * 64 + lane, r = idx / T::CPR;
      src[q] = A + pl * p.a_pst + (size_t)min(m0 + r, p.M - 1) * p.lda +
               8 * swz_chunk<T::BK>(r, idx % T::CPR);
    }
  }
  auto issue_one = [&](int s, int q) __attribute__((always_inline)) {
    lds_dma16(src[q] + (s_begin + s) * T::BK,
              smem + (s % T::NBUF) * T::STAGE + (wave * T::PER_WAVE + q) * 512);
  };
  auto issue = [&](int s) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < T::PER_WAVE; ++q) issue_one(s, q);
  };
  struct Frag {
    u32x4 w[T::UN];
    u32x4 a[T::AP][T::UM];
  };
  auto read = [&](Frag& f, int s, int ks) __attribute__((always_inline)) {
    const uint16_t* st = smem + (s % T::NBUF) * T::STAGE;
    const int c = 2 * ks + lk;
#pragma unroll
    for (int u = 0; u < T::UN; ++u)
      f.w[u] = *(const u32x4*)(st + swz_row<T::BK>(32 * (T::UN * wn + u) + lr, c));
#pragma unroll
    for (int pl = 0; pl < T::AP; ++pl)
#pragma unroll
      for (int v = 0; v < T::UM; ++v)
        f.a[pl][v] = *(const u32x4*)(st + T::BN * T::BK + pl * T::BM * T::BK +
                                     swz_row<T::BK>(32 * (T::UM * wm + v) + lr, c));
  };
  f32x16_t acc[T::UN][T::UM];
#pragma unroll
  for (int u = 0; u < T::UN; ++u)
#pragma unroll
    for (int v = 0; v < T::UM; ++v)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[u][v][i] = 0.f;
  // With three or more stages the copies of slice s + NBUF - 1 are spread over
  // the MFMA units (pairs of plane products) of slice s, copy q after unit
  // q * UNITS / PER_WAVE; with two stages they go out in one burst after the
  // barrier, since all of them must land before the next wait.
  constexpr bool INTER = T::NBUF >= 3;
  constexpr int UNITS = T::KS * T::UM * T::UN;   // per slice
  auto compute = [&](const Frag& f, int ks, int s_fill) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < T::UM; ++v)
#pragma unroll
      for (int u = 0; u < T::UN; ++u) {
        acc[u][v] = mfma32(f.w[u], f.a[0][v], acc[u][v]);
        if constexpr (T::AP == 2) acc[u][v] = mfma32(f.w[u], f.a[1][v], acc[u][v]);
        if constexpr (INTER) {
          const int unit = (ks * T::UM + v) * T::UN + u;
#pragma unroll
          for (int q = 0; q < T::PER_WAVE; ++q)
            if ((q * UNITS) / T::PER_WAVE == unit && s_fill < ns) issue_one(s_fill, q);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
  };
  // copies of the slice being filled that go out before the wait at the last k-step
  constexpr int Q_BEFORE = [] {
    int c = 0;
    for (int q = 0; q < T::PER_WAVE; ++q)
      if ((q * UNITS) / T::PER_WAVE < (T::KS - 1) * T::UM * T::UN) ++c;
    return c;
  }();
  // Slice s is in LDS once this wave's copies of it have landed -- vmcnt lets
  // exactly the copies issued after them stay in flight -- and every wave has
  // passed the barrier; the buffer the next copies refill was read into
  // registers just before, by every wave.
  auto wait_slice = [&](int s) __attribute__((always_inline)) {
    if constexpr (!INTER) {
      wait_newer<T::PER_WAVE, T::NBUF - 2>(min(ns - 1 - s, T::NBUF - 2));
    } else {
      // issued after slice s: slices s+1 .. s+NBUF-3 whole (those that exist)
      // and Q_BEFORE copies of slice s+NBUF-2 when it exists.  In the prologue
      // that slice is already whole, so the wait there is longer than needed.
      constexpr int STEADY = (T::NBUF - 3) * T::PER_WAVE + Q_BEFORE;
      if (s + T::NBUF - 2 < ns) {
        wait_vm_lgkm0<STEADY>();
      } else {
        const int full = ns - 1 - s > T::NBUF - 3 ? T::NBUF - 3 : (ns - 1 - s < 0 ? 0 : ns - 1 - s);
        wait_vm_dyn<STEADY>(full * T::PER_WAVE);
      }
    }
    ring_barrier();
  };

#pragma unroll
  for (int s0 = 0; s0 < T::NBUF - 1; ++s0)
    if (s0 < ns) issue(s0);
  Frag f0, f1;
  wait_slice(0);
  if (!INTER && T::NBUF - 1 < ns) issue(T::NBUF - 1);
  read(f0, 0, 0);
  for (int s = 0; s < ns; ++s) {
    const int s_fill = s + T::NBUF - 1;
#pragma unroll
    for (int ks = 0; ks < T::KS; ++ks) {
      Frag& cur = (ks & 1) ? f1 : f0;
      Frag& nxt = (ks & 1) ? f0 : f1;
      if (ks + 1 < T::KS) {
        read(nxt, s, ks + 1);
      } else if (s + 1 < ns) {
        wait_slice(s + 1);
        if (!INTER && s + T::NBUF < ns) issue(s + T::NBUF);
        read(nxt, s + 1, 0);
      }
      compute(cur, ks, s_fill);
    }
  }

  // element i of acc[u][v]: weight row n = n0 + 32 (UN wn + u) + 8 (i / 4) + 4 lk + i % 4,
  // activation row m = m0 + 32 (UM wm + v) + lr; four consecutive n per store
  if constexpr (ROPE) {
    // the 32 x 128 tile through LDS (the ring is idle once every wave is past
    // its last fragment reads), so that each rotation pair -- both halves of
    // a head lie in the tile, d dividing 128 -- meets in one thread
    static_assert(T::UN == 1 && T::UM == 1 && T::BN == 128 && T::BM == 32, "rope tile");
    constexpr int LD = T::BN + 4;   // padded row of the exchange tile
    float* xt = (float*)smem;
    ring_barrier();
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *(float4*)(xt + lr * LD + 32 * wn + 8 * g + 4 * lk) =
          make_float4(acc[0][0][4 * g], acc[0][0][4 * g + 1], acc[0][0][4 * g + 2], acc[0][0][4 * g + 3]);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    ring_barrier();
    const int d = ro.d, half = d / 2, hkd = ro.Hkv * d;
    if (n0 < hkd) {
      // keys: items (row, head, i < d / 2)
      const double lnb = log((double)ro.rope_base);
      for (int e = threadIdx.x; e < T::BM * 64; e += 256) {
        const int r = e >> 6, j = e & 63, hl = j / half, i = j % half;
        const int m = m0 + r;
        if (m >= p.M) continue;
        const int dst = ro.dst_rows[m];
        if (dst < 0 || dst >= ro.rows) continue;
        const double ang = (double)ro.positions[m] * exp(-(2.0 * i / d) * lnb);
        double sv, cv;
        sincos(ang, &sv, &cv);
        const int c = hl * d + i;
        const double a1 = xt[r * LD + c], a2 = xt[r * LD + c + half];
        const size_t o = (size_t)dst * hkd + n0 + c;
        store_elem(ro.k_cache, ro.dtype, o, (float)(a1 * cv - a2 * sv));
        store_elem(ro.k_cache, ro.dtype, o + half, (float)(a2 * cv + a1 * sv));
      }
    } else {
      // values as they are
      for (int e = threadIdx.x; e < T::BM * T::BN; e += 256) {
        const int r = e >> 7, c = e & 127;
        const int m = m0 + r;
        if (m >= p.M) continue;
        const int dst = ro.dst_rows[m];
        if (dst < 0 || dst >= ro.rows) continue;
        store_elem(ro.v_cache, ro.dtype, (size_t)dst * hkd + (n0 - hkd) + c, xt[r * LD + c]);
      }
    }
    return;
  }
  if (p.act) {
    // SwiGLU: elements i < 8 are gate columns 16 b + c (b = the 32-row
    // block, c = 8 (i / 4) + 4 lk + i % 4), element i + 8 the up column of
    // the same c; the lane writes four consecutive act columns from i = 0 .. 3
    // and from 4 .. 7 as bf16 planes
    const int F = p.N / 2;
    const size_t pst = (size_t)p.M * F;
#pragma unroll
    for (int v = 0; v < T::UM; ++v) {
      const int m = m0 + 32 * (T::UM * wm + v) + lr;
      if (m >= p.M) continue;
#pragma unroll
      for (int u = 0; u < T::UN; ++u) {
        const int nb = n0 + 32 * (T::UN * wn + u);
        if (nb >= p.N) continue;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float a[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float g = acc[u][v][4 * h + i], up = acc[u][v][4 * h + i + 8];
            a[i] = g / (1.0f + expf(-g)) * up;
          }
          uint32_t hi[2], lo[2];
          split2(a[0], a[1], hi[0], lo[0]);
          split2(a[2], a[3], hi[1], lo[1]);
          const size_t j = (size_t)m * F + (nb >> 1) + 8 * h + 4 * lk;
          *(uint2*)(p.act + j) = make_uint2(hi[0], hi[1]);
          *(uint2*)(p.act + pst + j) = make_uint2(lo[0], lo[1]);
        }
      }
    }
    return;
  }
  const bool split = p.splits > 1;
#pragma unroll
  for (int v = 0; v < T::UM; ++v) {
    const int m = m0 + 32 * (T::UM * wm + v) + lr;
    if (m >= p.M) continue;
#pragma unroll
    for (int u = 0; u < T::UN; ++u)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + 32 * (T::UN * wn + u) + 8 * g + 4 * lk;
        if (n >= p.N) continue;
        float4 r = make_float4(acc[u][v][4 * g], acc[u][v][4 * g + 1], acc[u][v][4 * g + 2],
                               acc[u][v][4 * g + 3]);
        if (split) {
          *(float4*)(p.part + ((size_t)z * p.M + m) * p.N + n) = r;
        } else {
          if (p.R) {
            const float4 b = *(const float4*)(p.R + (size_t)m * p.ldr + n);
            r.x += b.x;
            r.y += b.y;
            r.z += b.z;
            r.w += b.w;
          }
          *(float4*)(p.C + (size_t)m * p.ldc + n) = r;
        }
      }
  }
}

// C = R + sum_z part[z] in the order z = 0, 1, ...; four consecutive columns
// per thread (N % 4 == 0).  The partials are loaded sixteen splits at a time,
// all in flight together, before they are added.
__global__ void splitk_reduce4(const float* __restrict__ part, int splits, int M, int N, float* C,
                               size_t ldc, const float* R, size_t ldr) {
  constexpr int ZB = 16;
  const size_t total4 = (size_t)M * N / 4;
  const size_t zs = (size_t)M * N;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < total4;
       e += (size_t)gridDim.x * blockDim.x) {
    const int row = (int)(4 * e / N), col = (int)(4 * e % N);
    const float4 b = R ? *(const float4*)(R + (size_t)row * ldr + col) : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int z0 = 0; z0 < splits; z0 += ZB) {
      float4 v[ZB];
#pragma unroll
      for (int z = 0; z < ZB; ++z)
        if (z0 + z < splits) v[z] = *(const float4*)(part + (size_t)(z0 + z) * zs + 4 * e);
#pragma unroll
      for (int z = 0; z < ZB; ++z)
        if (z0 + z < splits) {
          if (z0 + z == 0) {
            s = v[0];
          } else {
            s.x += v[z].x;
            s.y += v[z].y;
            s.z += v[z].z;
            s.w += v[z].w;
          }
        }
    }
    if (R) {
      s.x = b.x + s.x;
      s.y = b.y + s.y;
      s.z = b.z + s.z;
      s.w = b.w + s.w;
    }
    *(float4*)(C + (size_t)row * ldc + col) = s;
  }
}

typedef DmaTile<1, 1, 4> DmaM32;    // 128 x 32
typedef DmaTile<2, 2, 2> DmaM128;   // 128 x 128
typedef DmaTile<1, 1, 4, 64, 1> DmaM32Bf16;    // the same tiles for a bf16 activation
typedef DmaTile<2, 2, 2, 64, 1> DmaM128Bf16;
typedef DmaTile<3, 1, 1> DmaM128N96;            // 96 x 128
typedef DmaTile<3, 1, 1, 64, 1> DmaM128N96Bf16;
typedef DmaTile<1, 5, 4, 32> DmaM160;             // 160 x 128, 32-wide slices

struct DmaPlan {
  int cfg;   // 0: DmaM32, 1: DmaM128, 2: DmaM128N96, 3: DmaM160 (two planes only)
  int tn, tm, splits;
};

// Tile and split-K choice.  Measured on the drafter shapes (M = 256 slot rows,
// N and K of 2048 .. 6144): 128 x 128 tiles with about 192 workgroups in total
// beat larger tiles and a full wave of 256 (fewer float32 partials to write
// and re-read).  Where N is a multiple of 96 and 96-wide tiles fit one pass
// over 256 CUs (the QKV and the fused gate/up projections of the batch-32
// drafter), those fill the machine instead: 64 tiles x 4 splits and 256
// tiles, against 192 workgroups.  The 32 fused rows take the 128 x 32 tile.
// 129 .. 160 rows of a two-plane activation (136 slot rows of the long-block
// drafter) take one 160-row tile instead of two 128-row tiles, the second
// nearly empty: 160 x 128 with 32-wide slices and five stages measured faster
// than both that and 160 x 256 tiles.
DmaPlan dma_plan(int M, int N, int K, int a_planes) {
  DmaPlan pl;
  int BM, target;
  if (M <= 32) {
    pl.cfg = 0;
    BM = DmaM32::BM;
    target = 256;
  } else {
    pl.cfg = 1;
    BM = DmaM128::BM;
    target = 192;
  }
  pl.tn = (N + 127) / 128;
  pl.tm = (M + BM - 1) / BM;
  int BK = 64;
  if (M > 128 && M <= 160 && a_planes == 2) {
    pl.cfg = 3;
    pl.tn = (N + DmaM160::BN - 1) / DmaM160::BN;
    pl.tm = 1;
    target = 256;
    BK = 32;
  } else if (M > 32 && N % 96 == 0 && (N / 96) * pl.tm <= 256) {
    pl.cfg = 2;
    pl.tn = N / 96;
    target = 256;
  }
  const int tiles = pl.tn * pl.tm;
  const int nK = K / BK;
  // each split at least four k-slices long; the 160-row tiles stay within one
  // pass over the CUs (56 QKV tiles of the long-block drafter: 4 splits, not 5)
  int sp = pl.cfg == 3 ? target / tiles : (target + tiles / 2) / tiles;
  if (sp > nK / 4) sp = nK / 4;
  pl.splits = sp < 1 ? 1 : sp;
  return pl;
}

bool dma_ok(const GemmArgs& a) {
  return !a.b_f32 && (a.a_planes == 1 || a.a_planes == 2) && (!a.B2 || (a.N1 > 0 && a.N1 < a.N)) && a.K % 64 == 0 && a.N % 4 == 0 && a.ldc % 4 == 0 && (!a.R || a.ldr % 4 == 0) &&
         a.lda % 8 == 0 && a.ldb % 8 == 0 && a.a_pst % 8 == 0;
}

template <class T, int ROPE = 0>
hipError_t launch_dma(const GemmParams& p, const DmaPlan& pl, hipStream_t s, const RopeOut& ro = RopeOut{}) {
  hipError_t e = hipFuncSetAttribute((const void*)gemm_dma_kernel<T, ROPE>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)T::LDS_BYTES);
  if (e != hipSuccess) return e;
  const int total = pl.tn * pl.tm * pl.splits;
  hipLaunchKernelGGL((gemm_dma_kernel<T, ROPE>), dim3(8 * ((total + 7) / 8)), dim3(256), T::LDS_BYTES, s, p,
                     pl.tn, pl.tm, ro);
  return hipGetLastError();
}

hipError_t launch_dma_any(const GemmParams& p, const DmaPlan& pl, int a_planes, hipStream_t s) {
  if (pl.cfg == 3) return launch_dma<DmaM160>(p, pl, s);
  if (pl.cfg == 2) return a_planes == 1 ? launch_dma<DmaM128N96Bf16>(p, pl, s) : launch_dma<DmaM128N96>(p, pl, s);
  if (a_planes == 1) return pl.cfg == 0 ? launch_dma<DmaM32Bf16>(p, pl, s) : launch_dma<DmaM128Bf16>(p, pl, s);
  return pl.cfg == 0 ? launch_dma<DmaM32>(p, pl, s) : launch_dma<DmaM128>(p, pl, s);
}

// ------------------------------------- at most 32 rows: weight streaming ----
// The fusion projections and the MTP block's projections multiply at most 32
// activation rows by a weight matrix that is read once: the call is a weight
// stream.  K is split into 512-wide ranges.  Persistent workgroups (at most
// kSkGrid, about equally many per range) each keep one range of the
// activation planes in registers -- stream wave w of four holds k 128 w ..
// 128 w + 127 of the range -- and take a contiguous run of 32-row weight tiles
// (32 output columns each).  A stream wave copies its 32 x 128 piece of every
// tile through a three-stage LDS ring of its own, four weight rows x 256
// contiguous bytes per copy, and accumulates the planes in turn.  A fifth
// wave adds the four partial tiles in wave order and stores the range's sum
// as split z of the [splits][M][N] partials, which the readers of a split-K
// result add in split order.
constexpr int kSkStream = 4;
constexpr int kSkThreads = (kSkStream + 1) * kWave;
constexpr int kSkBK = 128;                       // k per stream wave and tile
constexpr int kSkRange = kSkStream * kSkBK;      // k per split
constexpr int kSkNB = 3;                         // ring stages per stream wave
constexpr int kSkStage = 32 * kSkBK;             // bf16 elements per stage
constexpr int kSkCopies = kSkStage * 2 / 1024;   // 1 KB copies per stage
constexpr int kSkRed = kSkStream * 16 * kWave;   // floats of one set of partial tiles
constexpr size_t kSkLds = (size_t)kSkStream * kSkNB * kSkStage * 2 + 2 * (size_t)kSkRed * 4;
constexpr int kSkGrid = 256;
constexpr int kSkMaxSplits = 32;                 // fused projection: 2 H <= 16384

__device__ __forceinline__ void add4f(float4& s, const float4& v) {
  s.x += v.x;
  s.y += v.y;
  s.z += v.z;
  s.w += v.w;
}

// Position of 16-byte chunk c of row r in a [32][128] stage (an involution):
// the 16 lanes of one read pass land on the 16 positions of the bank window.
__device__ __forceinline__ int sk_swz(int r, int c) { return c ^ (r & 15); }

// Copy of the stream wave's 32 x 128 piece of weight tile t (rows 32 t .. 32 t
// + 31, k0 .. k0 + 127) into ring stage st: copy i covers rows 4 i .. 4 i + 3
// (lane / 16), chunk position lane % 16.
__device__ __forceinline__ void sk_issue(const GemmParams& p, int k0, int t, int lane, uint16_t* st) {
  const int n0 = 32 * t;
  const uint16_t* __restrict__ W = (const uint16_t*)p.B;
  const uint16_t* __restrict__ W2 = (const uint16_t*)p.B2;
#pragma unroll
  for (int i = 0; i < kSkCopies; ++i) {
    const int r = 4 * i + (lane >> 4);
    const int n = min(n0 + r, p.N - 1);
    const uint16_t* wrow = (W2 && n >= p.N1) ? W2 + (size_t)(n - p.N1) * p.ldb : W + (size_t)n * p.ldb;
    lds_dma16(wrow + k0 + 8 * sk_swz(r, lane & 15), st + 512 * i);
  }
}

// The copies of a stream wave's first tiles (as many as its ring takes before
// the loop), issued right after its activation loads: the loads, older, are
// waited for alone (vmcnt counts in issue order), and the copies' latency
// passes under the work on the loaded rows.  Returns how many were issued.
// The same copies through a buffer descriptor over the weight rows (no second
// matrix), whose offsets the compiler tracks as plain loads.
__device__ __forceinline__ void sk_issue_buf(__amdgpu_buffer_rsrc_t wr, const GemmParams& p, int k0, int t,
                                             int lane, uint16_t* st) {
  const int n0 = 32 * t;
#pragma unroll
  for (int i = 0; i < kSkCopies; ++i) {
    const int r = 4 * i + (lane >> 4);
    const int n = min(n0 + r, p.N - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        wr, (__attribute__((address_space(3))) void*)(st + 512 * i), 16,
        (uint32_t)((size_t)n * p.ldb + k0 + 8 * sk_swz(r, lane & 15)) * 2, 0, 0, 0);
  }
}

// All of them go out whatever my is (past the run's last tile the rows are
// clamped into the matrix and the stage is never read; the ring's waits
// cover them), so that the count of instructions after the loads is known
// where the loads are waited for: past a branch around some of the copies
// the compiler would wait for all of them.
__device__ __forceinline__ int sk_issue_first(const GemmParams& p, int k0, int t0, int lane, int wave,
                                              uint16_t* smem) {
  uint16_t* ring = smem + wave * kSkNB * kSkStage;
#pragma unroll
  for (int q = 0; q < kSkNB - 1; ++q) sk_issue(p, k0, t0 + q, lane, ring + q * kSkStage);
  return kSkNB - 1;
}

// The stream waves' part of a skinny workgroup once their activation
// registers xf hold k0 .. k0 + 127 of the rows and the copies of the first
// `issued` tiles are on their way: copy each tile's 32 x 128 weight piece
// through the wave's own ring, multiply, and hand the partial tile to the sum
// wave through LDS.
template <int AP>
__device__ __forceinline__ void skinny_stream(const GemmParams& p, const u32x4 (&xf)[AP][kSkBK / 16],
                                              int k0, int t0, int my, int issued, int lane, int wave,
                                              uint16_t* smem, float* red) {
  constexpr int KPS = kSkBK / 16;                // k-steps per stage
  const int lr = lane & 31, lk = lane >> 5;
  uint16_t* ring = smem + wave * kSkNB * kSkStage;
  for (int q = issued; q < kSkNB - 1 && q < my; ++q) sk_issue(p, k0, t0 + q, lane, ring + q * kSkStage);
  for (int tile = 0; tile < my; ++tile) {
    // tile has landed once only the copies issued after it may be
    // outstanding; lgkmcnt(0) too, since the stage refilled below was read
    // just before
    wait_vm_dyn<kSkCopies * (kSkNB - 2)>(kSkCopies * min(my - 1 - tile, kSkNB - 2));
    const uint16_t* st = ring + (tile % kSkNB) * kSkStage;
    u32x4 wf[KPS];
#pragma unroll
    for (int jj = 0; jj < KPS; ++jj) wf[jj] = *(const u32x4*)(st + lr * kSkBK + 8 * sk_swz(lr, 2 * jj + lk));
    f32x16_t acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int jj = 0; jj < KPS; ++jj)
#pragma unroll
      for (int pl = 0; pl < AP; ++pl) acc = mfma32(wf[jj], xf[pl][jj], acc);
    if (tile + kSkNB - 1 < my)
      sk_issue(p, k0, t0 + tile + kSkNB - 1, lane, ring + ((tile + kSkNB - 1) % kSkNB) * kSkStage);
    float* rb = red + (size_t)(tile & 1) * kSkRed + wave * 16 * kWave;
#pragma unroll
    for (int i = 0; i < 16; ++i) rb[i * kWave + lane] = acc[i];
    // the partial tile is in LDS before the barrier; the copies stay in flight
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) only
    ring_barrier();
  }
}

// The sum wave: lane (lr, lk) holds activation row lr and output columns
// 32 t + 8 (i / 4) + 4 lk + (i % 4), i = 0 .. 15, of tile t; it adds the four
// partial tiles in wave order and stores split z of the partials.
__device__ __forceinline__ void skinny_sum(const GemmParams& p, int z, int t0, int my, int lane,
                                           float* red) {
  const int lr = lane & 31, lk = lane >> 5;
  const int M = p.M, N = p.N;
  for (int tile = 0; tile < my; ++tile) {
    ring_barrier();
    const int n0 = 32 * (t0 + tile);
    const float* rb = red + (size_t)(tile & 1) * kSkRed + lane;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float a = rb[i * kWave];
#pragma unroll
      for (int w = 1; w < kSkStream; ++w) a += rb[(w * 16 + i) * kWave];
      v[i] = a;
    }
    if (lr < M) {
      float* dst = p.part + ((size_t)z * M + lr) * N;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + 8 * g + 4 * lk;
        if (n < N) *(float4*)(dst + n) = make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
      }
    }
  }
}

// blockIdx.x = z per_split + j: split z, run j of the n_tiles weight tiles.
template <int AP>
__global__ __launch_bounds__(kSkThreads) void gemm_skinny_kernel(GemmParams p, int n_tiles, int per_split) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  static_assert(kSkCopies * (kSkNB - 2) < 64, "vmcnt");
  constexpr int KPS = kSkBK / 16;
  float* red = (float*)(smem + kSkStream * kSkNB * kSkStage);   // [2][stream wave][16][64]
  const int z = blockIdx.x / per_split, j = blockIdx.x % per_split;
  const int my = n_tiles / per_split + (j < n_tiles % per_split ? 1 : 0);
  const int t0 = j * (n_tiles / per_split) + min(j, n_tiles % per_split);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, lk = lane >> 5;
  if (my == 0) return;   // the whole workgroup, before any barrier

  if (wave < kSkStream) {
    const uint16_t* __restrict__ A = (const uint16_t*)p.A;
    const int k0 = z * kSkRange + wave * kSkBK;
    // MFMA B operands of the range: activation row lr (rows past M repeat row
    // M - 1; their results are never stored), k = k0 + 16 j + 8 lk ..
    u32x4 xf[AP][KPS];
    const uint16_t* xr = A + (size_t)min(lr, p.M - 1) * p.lda + k0 + 8 * lk;
#pragma unroll
    for (int pl = 0; pl < AP; ++pl)
#pragma unroll
      for (int jj = 0; jj < KPS; ++jj) xf[pl][jj] = *(const u32x4*)(xr + pl * p.a_pst + 16 * jj);
    __builtin_amdgcn_sched_barrier(0);
    const int issued = sk_issue_first(p, k0, t0, lane, wave, smem);
    __builtin_amdgcn_sched_barrier(0);
    skinny_stream<AP>(p, xf, k0, t0, my, issued, lane, wave, smem, red);
    return;
  }
  skinny_sum(p, z, t0, my, lane, red);
}

// ------------------------------------- fused RMSNorm-concat projection ----
// out[r] = res[r] + W [RMSNorm(x1[r]; g1); RMSNorm(x2[r]; g2)] for at most 32
// rows, in two launches.  A row's RMSNorm is its gain-weighted row divided by
// one scalar, so
//     W [RMSNorm(x1; g1); RMSNorm(x2; g2)]
//         = (W1 (x1 * g1)) / rms(x1) + (W2 (x2 * g2)) / rms(x2),
// W1 / W2 the columns acting on each stream.  fuse_skinny_kernel is the
// weight-streaming GEMM above whose stream waves load their k-range of the
// raw rows (rows or embedding ids), multiply by the gains and split the
// products into the two bf16 planes in registers -- no normalised copy of the
// rows is written -- and also store the range's sum of squares of the raw
// rows.  Each split range lies in one stream (H % 512 == 0).  fuse_finish_kernel
// then adds the partials of each stream in split order, scales each sum by
// that stream's 1 / rms, and adds the residual.
struct FuseSrc {
  const void* rows[2];       // stream rows [M, H] (NULL: gathered by ids)
  int dtype[2];              // of the rows, or of the table they are gathered from
  const int32_t* ids[2];
  const void* table[2];      // [n_table, H]
  int n_table[2];
  const float* g[2];
  int H;
  float* ssp;                // [splits * kSkStream][M] sums of squares per wave range
};

// Elements k .. k + 7 of row r of stream s as float (zero for an id outside
// the table).
__device__ __forceinline__ void fuse_load8(const FuseSrc& f, int s, int r, int k, float (&x)[8]) {
  const void* base;
  int dt;
  size_t off;
  if (f.rows[s]) {
    base = f.rows[s];
    dt = f.dtype[s];
    off = (size_t)r * f.H + k;
  } else {
    const int id = f.ids[s][r];
    if (id < 0 || id >= f.n_table[s]) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
      return;
    }
    base = f.table[s];
    dt = f.dtype[s];
    off = (size_t)id * f.H + k;
  }
  if (dt == DMTP_BF16) {
    const uint4 u = *(const uint4*)((const uint16_t*)base + off);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(w[e] << 16);
      x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *(const float4*)((const float*)base + off);
    const float4 b = *(const float4*)((const float*)base + off + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// Row r of stream s: where it starts, in what dtype, and whether it reads as
// zeros (an id outside the table; base then points at row 0).
// (The stream's fields are picked by selects, not by indexing with s: an
// array indexed at run time would be read from memory, one more latency.)
__device__ __forceinline__ void fuse_row(const FuseSrc& f, int s, int r, const void*& base, int& dt,
                                         bool& zero) {
  const void* rows = s ? f.rows[1] : f.rows[0];
  dt = s ? f.dtype[1] : f.dtype[0];
  zero = false;
  const size_t esz = dt == DMTP_BF16 ? 2 : 4;
  if (rows) {
    base = (const char*)rows + (size_t)r * f.H * esz;
  } else {
    const int id = (s ? f.ids[1] : f.ids[0])[r];
    zero = id < 0 || id >= (s ? f.n_table[1] : f.n_table[0]);
    base = (const char*)(s ? f.table[1] : f.table[0]) + (size_t)(zero ? 0 : id) * f.H * esz;
  }
}

// A stream wave of the fused projection, for rows stored as bf16 (BF) or
// float32: the row's start first (an id lookup), then all of its loads and
// the gains' in flight together, then the first weight copies (waited for
// later, by the ring), then the arithmetic on the rows: two memory latencies,
// the second beside the copies'.  One straight-line body per dtype, so that
// the compiler counts the loads still in flight at each use.
template <bool BF>
__device__ __forceinline__ void fuse_stream(const GemmParams& p, const FuseSrc& f, int z, int j, int t0,
                                            int my, int lane, int wave, uint16_t* smem, float* red,
                                            const void* rb, bool zero) {
  constexpr int KPS = kSkBK / 16;
  const int lr = lane & 31, lk = lane >> 5;
  const int k0 = z * kSkRange + wave * kSkBK;     // in the concatenated [x1 | x2]
  const int s = k0 >= f.H ? 1 : 0;
  const int kk = k0 - s * f.H + 8 * lk;
  const float* gs = s ? f.g[1] : f.g[0];
  float4 raw[KPS][BF ? 1 : 2];   // bf16: 16 bytes; float32: 32 bytes
  float4 g[KPS][2];
#pragma unroll
  for (int jj = 0; jj < KPS; ++jj) {
    if constexpr (BF) {
      raw[jj][0] = *(const float4*)((const uint16_t*)rb + kk + 16 * jj);
    } else {
      raw[jj][0] = *(const float4*)((const float*)rb + kk + 16 * jj);
      raw[jj][1] = *(const float4*)((const float*)rb + kk + 16 * jj + 4);
    }
  }
#pragma unroll
  for (int jj = 0; jj < KPS; ++jj) {
    g[jj][0] = *(const float4*)(gs + kk + 16 * jj);
    g[jj][1] = *(const float4*)(gs + kk + 16 * jj + 4);
  }
  __builtin_amdgcn_sched_barrier(0);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(p.B), (short)0, (int)((size_t)p.N * p.ldb * 2), 0x00020000);
  uint16_t* ring = smem + wave * kSkNB * kSkStage;
#pragma unroll
  for (int q = 0; q < kSkNB - 1; ++q) sk_issue_buf(wr, p, k0, t0 + q, lane, ring + q * kSkStage);
  const int issued = kSkNB - 1;
  __builtin_amdgcn_sched_barrier(0);
  float x[KPS][8];
#pragma unroll
  for (int jj = 0; jj < KPS; ++jj) {
    if constexpr (BF) {
      const uint32_t w[4] = {__float_as_uint(raw[jj][0].x), __float_as_uint(raw[jj][0].y),
                             __float_as_uint(raw[jj][0].z), __float_as_uint(raw[jj][0].w)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[jj][2 * e] = __uint_as_float(w[e] << 16);
        x[jj][2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    } else {
      x[jj][0] = raw[jj][0].x; x[jj][1] = raw[jj][0].y; x[jj][2] = raw[jj][0].z; x[jj][3] = raw[jj][0].w;
      x[jj][4] = raw[jj][1].x; x[jj][5] = raw[jj][1].y; x[jj][6] = raw[jj][1].z; x[jj][7] = raw[jj][1].w;
    }
    // an id outside the table reads zeros (a select: a branch here would
    // make the compiler wait for every load in flight at its join)
#pragma unroll
    for (int e = 0; e < 8; ++e) x[jj][e] = zero ? 0.f : x[jj][e];
  }
  u32x4 xf[2][KPS];
  float ss = 0.f;
#pragma unroll
  for (int jj = 0; jj < KPS; ++jj) {
    const float gg[8] = {g[jj][0].x, g[jj][0].y, g[jj][0].z, g[jj][0].w,
                         g[jj][1].x, g[jj][1].y, g[jj][1].z, g[jj][1].w};
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ss = fmaf(x[jj][2 * e], x[jj][2 * e], ss);
      ss = fmaf(x[jj][2 * e + 1], x[jj][2 * e + 1], ss);
      split2(x[jj][2 * e] * gg[2 * e], x[jj][2 * e + 1] * gg[2 * e + 1], hi[e], lo[e]);
    }
    xf[0][jj] = u32x4{hi[0], hi[1], hi[2], hi[3]};
    xf[1][jj] = u32x4{lo[0], lo[1], lo[2], lo[3]};
  }
  // the row's sum of squares over this wave's 128 k (lanes lk = 0, 1 hold
  // its two halves); one workgroup per split writes it
  ss += shfl_xor(ss, 32);
  if (j == 0 && lk == 0 && lr < p.M) f.ssp[(size_t)(z * kSkStream + wave) * p.M + lr] = ss;
  skinny_stream<2>(p, xf, k0, t0, my, issued, lane, wave, smem, red);
}

__global__ __launch_bounds__(kSkThreads) void fuse_skinny_kernel(GemmParams p, FuseSrc f, int n_tiles,
                                                                 int per_split) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  constexpr int KPS = kSkBK / 16;
  float* red = (float*)(smem + kSkStream * kSkNB * kSkStage);
  const int z = blockIdx.x / per_split, j = blockIdx.x % per_split;
  const int my = n_tiles / per_split + (j < n_tiles % per_split ? 1 : 0);
  const int t0 = j * (n_tiles / per_split) + min(j, n_tiles % per_split);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 31, lk = lane >> 5;
  if (my == 0) return;

  if (wave < kSkStream) {
    const int k0 = z * kSkRange + wave * kSkBK;
    const int s = k0 >= f.H ? 1 : 0;
    const void* rb;
    int dt;
    bool zero;
    fuse_row(f, s, min(lr, p.M - 1), rb, dt, zero);
    if (dt == DMTP_BF16)
      fuse_stream<true>(p, f, z, j, t0, my, lane, wave, smem, red, rb, zero);
    else
      fuse_stream<false>(p, f, z, j, t0, my, lane, wave, smem, red, rb, zero);
    return;
  }
  skinny_sum(p, z, t0, my, lane, red);
}

// out[m, n .. n+3] = res + (sum_{z < z1} part[z]) / rms1 + (sum_{z >= z1} part[z]) / rms2,
// rms_s = sqrt(sum of the stream's squares / H + eps).  One workgroup of 256
// threads per (row, 1024 columns); wave 0 turns the per-wave sums of squares
// into the two scales.
__global__ __launch_bounds__(256) void fuse_finish_kernel(const float* __restrict__ part, int splits,
                                                          int z1, const float* __restrict__ ssp,
                                                          int M, int H, float eps, FuseSrc res,
                                                          int has_res, float* __restrict__ out) {
  __shared__ float scale[2];
  const int m = blockIdx.y;
  const int n = 4 * (blockIdx.x * 256 + threadIdx.x);
  const size_t plane = (size_t)M * H;
  // Loads in dependency order, every one issued before the first sum (vmcnt
  // counts in issue order, so a load waited for early would wait for all
  // those before it): the residual row's start (an id lookup) and this
  // row's sums of squares (wave 0; at most 2 x 64 ranges), then the first
  // eight partials -- unconditional, columns clamped into the row and splits
  // past the last repeating it, so that no sum sits between them -- then the
  // residual row itself.
  const void* rrb = nullptr;
  int rdt = DMTP_F32;
  bool rzero = true;
  if (has_res) fuse_row(res, 0, m, rrb, rdt, rzero);
  const int nw = splits * kSkStream, w1 = z1 * kSkStream;
  float q[2] = {0.f, 0.f};
  if (threadIdx.x < kWave) {
#pragma unroll
    for (int t = 0; t < 2; ++t) q[t] = ssp[(size_t)min((int)threadIdx.x + t * kWave, nw - 1) * M + m];
  }
  const float* pp = part + (size_t)m * H + (n < H ? n : H - 4);
  float4 v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) v[u] = *(const float4*)(pp + (size_t)min(u, splits - 1) * plane);
  float4 rv = make_float4(0.f, 0.f, 0.f, 0.f);
  if (has_res && n < H) {
    if (rdt == DMTP_BF16) {
      const uint2 w = *(const uint2*)((const uint16_t*)rrb + n);
      rv = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
    } else {
      rv = *(const float4*)((const float*)rrb + n);
    }
    if (rzero) rv = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  if (threadIdx.x < kWave) {
    double a = 0.0, b = 0.0;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int i = threadIdx.x + t * kWave;
      if (i < w1) a += q[t];
      else if (i < nw) b += q[t];
    }
    a = wave_sum(a);
    b = wave_sum(b);
    if (threadIdx.x == 0) {
      scale[0] = (float)(1.0 / sqrt(a / H + (double)eps));
      scale[1] = (float)(1.0 / sqrt(b / H + (double)eps));
    }
  }
  // each stream's partials in split order, eight at a time
  float4 s1 = make_float4(0.f, 0.f, 0.f, 0.f), s2 = s1;
  for (int z0 = 0;; z0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (z0 + u < z1) add4f(s1, v[u]);
      else if (z0 + u < splits) add4f(s2, v[u]);
    }
    if (z0 + 8 >= splits) break;
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *(const float4*)(pp + (size_t)min(z0 + 8 + u, splits - 1) * plane);
  }
  __syncthreads();
  if (n >= H) return;
  const float c1 = scale[0], c2 = scale[1];
  float4 y;
  y.x = rv.x + (s1.x * c1 + s2.x * c2);
  y.y = rv.y + (s1.y * c1 + s2.y * c2);
  y.z = rv.z + (s1.z * c1 + s2.z * c2);
  y.w = rv.w + (s1.w * c1 + s2.w * c2);
  *(float4*)(out + (size_t)m * H + n) = y;
}

// Calls of at most 32 rows whose K is a multiple of the split range, with
// at least two ranges (the kernel writes partials only: readers of a result
// of one split read C instead).
bool skinny_fits(int M, int K) { return M <= 32 && K % kSkRange == 0 && K >= 2 * kSkRange; }

hipError_t launch_skinny(const GemmParams& p, int a_planes, hipStream_t s) {
  static_assert(kSkLds <= 160 * 1024, "skinny LDS");
  const int splits = p.K / kSkRange;
  const int n_tiles = (p.N + 31) / 32;
  int per = kSkGrid / splits;
  per = per < 1 ? 1 : (per > n_tiles ? n_tiles : per);
  const void* fn = a_planes == 1 ? (const void*)gemm_skinny_kernel<1> : (const void*)gemm_skinny_kernel<2>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSkLds);
  if (e != hipSuccess) return e;
  if (a_planes == 1)
    hipLaunchKernelGGL(gemm_skinny_kernel<1>, dim3(splits * per), dim3(kSkThreads), kSkLds, s, p, n_tiles, per);
  else
    hipLaunchKernelGGL(gemm_skinny_kernel<2>, dim3(splits * per), dim3(kSkThreads), kSkLds, s, p, n_tiles, per);
  return hipGetLastError();
}

// ---------------------------------------------------- float32 weight path ----
template <class T>
__global__ __launch_bounds__(T::THREADS) void gemm_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[T::LDS_A + T::LDS_B];
  const int n0 = blockIdx.x * T::BN, m0 = blockIdx.y * T::BM;
  Acc<T> acc;
  gemm_mainloop<T>(acc, lds, p.A, p.lda, p.a_pst, p.M, p.B, p.ldb, p.N, m0, n0, 0, p.K);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wm0 = (wave / T::WAVES_N) * T::WM, wn0 = (wave % T::WAVES_N) * T::WN;
#pragma unroll
  for (int i = 0; i < T::TM; ++i)
#pragma unroll
    for (int j = 0; j < T::TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm0 + 16 * i + 4 * (lane >> 4) + r;
        const int col = n0 + wn0 + 16 * j + (lane & 15);
        if (row >= p.M || col >= p.N) continue;
        const float base = p.R ? p.R[(size_t)row * p.ldr + col] : 0.f;
        p.C[(size_t)row * p.ldc + col] = base + acc.v[i][j][r];
      }
}

typedef GemmTile<64, 64, 32, 32, 2, 2> TilePlanesF32;

}  // namespace

size_t gemm_ws_bytes(int M, int N, int K, int b_f32) {
  if (b_f32) return 0;
  if (skinny_fits(M, K)) return (size_t)(K / kSkRange) * M * N * sizeof(float);
  // either activation form: the larger of the two plans
  const int splits = max(dma_plan(M, N, K, 1).splits, dma_plan(M, N, K, 2).splits);
  return splits > 1 ? (size_t)splits * M * N * sizeof(float) : 0;
}

hipError_t gemm_deferred(const GemmArgs& a, float* ws, hipStream_t s, SplitOut* out) {
  GemmParams p{a.A, a.a_pst, a.lda, a.M, a.B, a.ldb, a.N, a.K, 1, a.C, a.ldc, a.R, a.ldr, ws,
               a.B2, a.B2 ? a.N1 : a.N};
  *out = SplitOut{a.C, a.ldc, ws, 1, a.M, a.N, a.R, a.ldr};
  if (!a.b_f32) {
    if (!dma_ok(a)) return hipErrorInvalidValue;
    if (skinny_fits(a.M, a.K)) {
      p.splits = a.K / kSkRange;
      out->splits = p.splits;
      return launch_skinny(p, a.a_planes, s);
    }
    const DmaPlan pl = dma_plan(a.M, a.N, a.K, a.a_planes);
    p.splits = pl.splits;
    out->splits = pl.splits;
    return launch_dma_any(p, pl, a.a_planes, s);
  }
  dim3 grid((a.N + TilePlanesF32::BN - 1) / TilePlanesF32::BN,
            (a.M + TilePlanesF32::BM - 1) / TilePlanesF32::BM);
  hipLaunchKernelGGL(gemm_kernel<TilePlanesF32>, grid, dim3(TilePlanesF32::THREADS), 0, s, p);
  return hipGetLastError();
}

hipError_t gemm_rope_scatter(const GemmArgs& a, const int32_t* positions, const int32_t* dst_rows,
                             int Hkv, int d, float rope_base, int dtype, int ctx_rows, void* k_cache,
                             void* v_cache, hipStream_t s) {
  if (a.b_f32 || a.a_planes != 2 || a.B2 || a.N != 2 * Hkv * d || (Hkv * d) % 128 != 0 || 128 % d != 0 ||
      !dma_ok(a))
    return hipErrorNotSupported;
  DmaPlan pl;
  pl.cfg = 0;
  pl.tn = a.N / DmaM32::BN;
  pl.tm = (a.M + DmaM32::BM - 1) / DmaM32::BM;
  pl.splits = 1;
  GemmParams p{a.A, a.a_pst, a.lda, a.M, a.B, a.ldb, a.N, a.K, 1, nullptr, 0, nullptr, 0, nullptr,
               nullptr, a.N};
  const RopeOut ro{positions, dst_rows, k_cache, v_cache, Hkv, d, dtype, ctx_rows, rope_base};
  return launch_dma<DmaM32, 1>(p, pl, s, ro);
}

hipError_t gemm_swiglu(const GemmArgs& a, uint16_t* act, hipStream_t s) {
  if (a.b_f32 || !a.B2 || a.N != 2 * a.N1 || a.N1 % 16 != 0 || !dma_ok(a) || skinny_fits(a.M, a.K))
    return hipErrorNotSupported;
  const DmaPlan pl = dma_plan(a.M, a.N, a.K, a.a_planes);
  if (pl.splits != 1) return hipErrorNotSupported;
  GemmParams p{a.A, a.a_pst, a.lda, a.M, a.B, a.ldb, a.N, a.K, 1, nullptr, 0, nullptr, 0, nullptr,
               a.B2, a.N1};
  p.act = act;
  return launch_dma_any(p, pl, a.a_planes, s);
}

hipError_t gemm(const GemmArgs& a, float* ws, hipStream_t s) {
  GemmParams p{a.A, a.a_pst, a.lda, a.M, a.B, a.ldb, a.N, a.K, 1, a.C, a.ldc, a.R, a.ldr, ws,
               a.B2, a.B2 ? a.N1 : a.N};
  if (!a.b_f32) {
    if (!dma_ok(a)) return hipErrorInvalidValue;
    hipError_t e;
    if (skinny_fits(a.M, a.K)) {
      p.splits = a.K / kSkRange;
      e = launch_skinny(p, a.a_planes, s);
    } else {
      const DmaPlan pl = dma_plan(a.M, a.N, a.K, a.a_planes);
      p.splits = pl.splits;
      e = launch_dma_any(p, pl, a.a_planes, s);
    }
    if (e != hipSuccess || p.splits == 1) return e;
    const size_t total4 = (size_t)a.M * a.N / 4;
    const int blocks = (int)((total4 + 255) / 256 < 4096 ? (total4 + 255) / 256 : 4096);
    hipLaunchKernelGGL(splitk_reduce4, dim3(blocks), dim3(256), 0, s, ws, p.splits, a.M, a.N, a.C,
                       a.ldc, a.R, a.ldr);
    return hipGetLastError();
  }
  dim3 grid((a.N + TilePlanesF32::BN - 1) / TilePlanesF32::BN,
            (a.M + TilePlanesF32::BM - 1) / TilePlanesF32::BM);
  hipLaunchKernelGGL(gemm_kernel<TilePlanesF32>, grid, dim3(TilePlanesF32::THREADS), 0, s, p);
  return hipGetLastError();
}


bool fuse_fits(const dmtp_fuse_desc& d) {
  const int K = 2 * d.H;
  return d.w_dtype == DMTP_BF16 && d.rows <= 32 && d.H % kSkRange == 0 && skinny_fits(d.rows, K) &&
         K / kSkRange <= kSkMaxSplits;
}

size_t fuse_fused_ws(const dmtp_fuse_desc& d) {
  const int splits = 2 * d.H / kSkRange;
  const size_t part = (size_t)splits * d.rows * d.H * sizeof(float);
  return ((part + 255) & ~(size_t)255) + (size_t)splits * kSkStream * d.rows * sizeof(float);
}

namespace {
FuseSrc fuse_src_of(const dmtp_rows& a, const dmtp_rows& b, int w_dtype) {
  FuseSrc f{};
  const dmtp_rows* r[2] = {&a, &b};
  for (int s = 0; s < 2; ++s) {
    f.rows[s] = r[s]->rows;
    f.dtype[s] = r[s]->rows ? r[s]->dtype : w_dtype;
    f.ids[s] = r[s]->ids;
    f.table[s] = r[s]->table;
    f.n_table[s] = r[s]->table_rows;
  }
  return f;
}
}  // namespace

hipError_t fuse_fused(const dmtp_fuse_desc& d, void* ws, hipStream_t s) {
  const int K = 2 * d.H, splits = K / kSkRange;
  float* part = (float*)ws;
  const size_t part_bytes = (size_t)splits * d.rows * d.H * sizeof(float);
  float* ssp = (float*)((char*)ws + ((part_bytes + 255) & ~(size_t)255));
  FuseSrc f = fuse_src_of(d.x1, d.x2, d.w_dtype);
  f.g[0] = d.g1;
  f.g[1] = d.g2;
  f.H = d.H;
  f.ssp = ssp;
  GemmParams p{nullptr, 0, 0, d.rows, d.W, (size_t)K, d.H, K, splits, nullptr, 0, nullptr, 0, part,
               nullptr, d.H};
  const int n_tiles = (d.H + 31) / 32;
  int per = kSkGrid / splits;
  per = per < 1 ? 1 : (per > n_tiles ? n_tiles : per);
  hipError_t e = hipFuncSetAttribute((const void*)fuse_skinny_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kSkLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fuse_skinny_kernel, dim3(splits * per), dim3(kSkThreads), kSkLds, s, p, f,
                     n_tiles, per);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const bool has_res = d.res.rows || d.res.ids;
  FuseSrc r = fuse_src_of(d.res, d.res, d.w_dtype);
  r.H = d.H;
  hipLaunchKernelGGL(fuse_finish_kernel, dim3((d.H + 1023) / 1024, d.rows), dim3(256), 0, s, part,
                     splits, splits / 2, ssp, d.rows, d.H, d.eps, r, has_res ? 1 : 0, d.out);
  return hipGetLastError();
}

}  // namespace dmtp

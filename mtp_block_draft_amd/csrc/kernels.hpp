// Internal launch interface of the DMTP kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dmtp.h"

namespace dmtp {

// ------------------------------------------------------------------ GEMM ----
// C[M, N] (float32, ldc) = R[M, N] (optional, may alias C) + A[M, K] B[N, K]^T.
// A is a float32 activation held as two bf16 planes (hi at A, lo at A + a_pst,
// row stride lda), or, with a_planes = 1 and a bf16 weight, a bf16 activation;
// B is a weight stored [out, in], bf16 or float32.
struct GemmArgs {
  const uint16_t* A;
  size_t a_pst;
  size_t lda;
  int M;
  const void* B;
  int b_f32;
  size_t ldb;
  int N;
  int K;            // multiple of 64
  float* C;
  size_t ldc;
  const float* R;   // residual or NULL
  size_t ldr;
  // Optional second weight matrix: output columns n >= N1 use row n - N1 of B2
  // (same ldb and dtype), so two projections of one input run as one GEMM.
  const void* B2 = nullptr;
  int N1 = 0;
  int a_planes = 2;
};

// float32 workspace the GEMM launcher needs for its split-K partials.
size_t gemm_ws_bytes(int M, int N, int K, int b_f32);
hipError_t gemm(const GemmArgs& a, float* ws, hipStream_t s);

// A GEMM result that may still be split over K.  splits == 1: the finished C
// [M, ldc] (R already added).  splits > 1: value(m, n) = R[m, n] (if R) +
// sum_z part[z][m][n], summed in z order by the kernel that reads it.
struct SplitOut {
  const float* C;
  size_t ldc;
  const float* part;   // [splits][M][N]
  int splits, M, N;
  const float* R;
  size_t ldr;
};
SplitOut split_out_plain(const float* C, size_t ldc, int M, int N);
// The GEMM without its reduction pass: the reader of *out adds the partials.
hipError_t gemm_deferred(const GemmArgs& a, float* ws, hipStream_t s, SplitOut* out);

// The key/value rows of a layer for the context cache in one launch: the
// product of the two-plane rows A [M, K] with the bf16 key/value weight rows
// B [2 Hkv d, K] (keys, then values), unsplit on 128 x 32 tiles, whose
// epilogue rotates the keys at positions[m] and stores keys and values in
// dtype at cache row dst_rows[m] (skipped when out of [0, ctx_rows)), as
// rope_scatter does with a finished product.  hipErrorNotSupported (nothing
// launched) for other weights or shapes (d must divide 128 and 128 divide
// Hkv d).
hipError_t gemm_rope_scatter(const GemmArgs& a, const int32_t* positions, const int32_t* dst_rows,
                             int Hkv, int d, float rope_base, int dtype, int ctx_rows, void* k_cache,
                             void* v_cache, hipStream_t s);

// act = silu(x Wgᵀ) * (x Wuᵀ) as bf16 planes [2][M][F] in one launch, for
// bf16 weights B = Wg and B2 = Wu (N = 2 F, N1 = F, F % 16 == 0) where the
// LDS-ring kernel takes the product without a K split; hipErrorNotSupported
// (nothing launched) elsewhere.
hipError_t gemm_swiglu(const GemmArgs& a, uint16_t* act, hipStream_t s);

// The fusion projection out = res + W [RMSNorm(x1; g1); RMSNorm(x2; g2)] as
// one weight-streaming GEMM with the norms folded in, plus a pass that adds
// its split-K partials with each stream's 1 / rms and the residual.  For bf16
// weights, at most 32 rows and H a multiple of 512 (up to 8192).
bool fuse_fits(const dmtp_fuse_desc& d);
size_t fuse_fused_ws(const dmtp_fuse_desc& d);
hipError_t fuse_fused(const dmtp_fuse_desc& d, void* ws, hipStream_t s);

// -------------------------------------------------------------- elementwise --
// X[r] = value(r) (when write_x; the residual stream update) and y[r] =
// RMSNorm(value(r); g) as bf16 planes [2][rows][H], for the rows of x.
hipError_t residual_rmsnorm(const SplitOut& x, float* X, size_t ldx, int write_x, const float* g,
                            float eps, uint16_t* y, int rows, int H, hipStream_t s);

// Fusion prologue: cat[r] = [RMSNorm(x1[r]; g1), RMSNorm(x2[r]; g2)] as bf16
// planes [2][rows][2H], and out[r] = res[r] (float32) when res is present.
hipError_t fuse_prep(const dmtp_fuse_desc& d, uint16_t* cat, hipStream_t s);

// Draft slots X [B * S, H] float32 from anchor ids, x_t1 rows and the MASK row,
// and y [2][B * S][H] = their RMSNorm with gains g as bf16 planes.
hipError_t build_slots(const dmtp_draft_desc& d, float* X, const float* g, uint16_t* y, hipStream_t s);

// q/k/v split of the QKV projection with the rotary embedding at slot
// positions: q [B, Hkv, S * G, d], kb and vb [B, Hkv, S, d] (float32).
hipError_t rope_split(const SplitOut& qkv, const int32_t* cu_ctx, int ctx_rows, int B, int S, int Hq,
                      int Hkv, int d, float rope_base, float* q, float* kb, float* vb,
                      hipStream_t s);

// a = silu(g) * u elementwise over [rows, F] (bf16 planes [2][rows][F] out)
hipError_t swiglu(const SplitOut& g, const SplitOut& u, uint16_t* a, int rows, int F, hipStream_t s);

// planes [2][n] (hi at planes, lo at planes + n) of n elements of x in dtype
hipError_t to_planes(const void* x, int dtype, size_t n, uint16_t* planes, hipStream_t s);

// Context cache rows: for row r of kv = value of the split GEMM result [N,
// 2 Hkv d] (keys then values; its partials are added here), rotate the keys at
// positions[r] and write both in dtype to k_cache / v_cache [ctx_rows, Hkv, d]
// at row dst_rows[r] (skipped when out of range).
hipError_t rope_scatter(const SplitOut& kv, const int32_t* positions, const int32_t* dst_rows, int N,
                        int Hkv, int d, float rope_base, int dtype, int ctx_rows, void* k_cache,
                        void* v_cache, hipStream_t s);

// out[m] = value(m) (float32, row stride ldo) for the rows of x
hipError_t finish_rows(const SplitOut& x, float* out, size_t ldo, int rows, int H, hipStream_t s);

// k_new / v_new [B, S, Hkv, d] in dtype from the block keys / values kb, vb
// [B, Hkv, S, d] (float32; rounded to bf16 for DMTP_BF16).  Either may be NULL.
hipError_t export_kv(const float* kb, const float* vb, int B, int S, int Hkv, int d, int dtype,
                     void* k_new, void* v_new, hipStream_t s);

// out[b, j] = round_dtype(RMSNorm(value(b S + n_anchor + j); g)) for j = 0 .. K-2
hipError_t final_norm_mask(const SplitOut& x, const float* g, float eps, int B, int S, int n_anchor,
                           int K, int H, int dtype, void* out, hipStream_t s);

// -------------------------------------------------------------- attention --
struct AttnPlan {
  int B, Hkv, G, S, d, NQ, nqp, chunk, n_chunks, kv_f32, window;
  int causal;   // block keys: slot s sees slots 0..s only (0 from attn_plan)
};
// ctx_rows: total context rows of the batch (sizes the chunks for bf16 K/V).
AttnPlan attn_plan(int B, int Hq, int Hkv, int S, int d, int max_ctx, int window, int kv_f32,
                   int ctx_rows);
// Largest number of query rows per kv head (S * Hq / Hkv) the kernels support.
int attn_max_nq(int d, int kv_f32);
size_t attn_ws_bytes(const AttnPlan& p);
// o [B * S, Hq * d] = attention of the block queries over context + block
// keys, written as bf16 planes [2][B * S][Hq * d].
// ev_start / ev_stop (both or neither): events of the bf16 context kernel's
// own dispatch (hipExtLaunchKernel), for timing it alone.
hipError_t attention(const AttnPlan& p, const float* q, const float* kb, const float* vb,
                     const void* ctx_k, const void* ctx_v, const int32_t* cu_ctx, int ctx_rows,
                     float* ws, uint16_t* o, hipStream_t s, hipEvent_t ev_start = nullptr,
                     hipEvent_t ev_stop = nullptr);

// ---------------------------------------------------------------- LM head --
size_t lm_head_ws_bytes(const dmtp_head_desc& d, int M);
hipError_t lm_head_run(const dmtp_head_desc& d, int M, void* ws, hipStream_t s);
// The packed copy of the head matrix that the register-input LM-head GEMM
// streams (layout in the header, at dmtp_head_pack): its size and the copy.
size_t head_pack_bytes(int V, int H);
hipError_t head_pack_run(const void* W, int V, int H, void* out, hipStream_t s);

// ----------------------------------------------------------------- verify --
size_t verify_ws_bytes(const dmtp_verify_desc& d);
hipError_t verify_run(const dmtp_verify_desc& d, void* ws, hipStream_t s);
// Largest K the acceptance-statistics kernel supports.
int accept_stats_max_k();
hipError_t accept_stats_run(const dmtp_stats_desc& d, hipStream_t s);

}  // namespace dmtp

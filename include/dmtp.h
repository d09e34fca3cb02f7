/*
 * dmtp.h -- C ABI of one DMTP speculative-decoding round on MI355X (gfx950).
 *
 * The round the pages define ("DMTP: A Better First Token for Block Drafting
 * via MTP", sections 2, 3 and 5): the MTP head proposes the first candidate T1
 * from a fused hidden state, a residual built from T1's embedding and the MTP
 * hidden is added to T1's embedding slot, one parallel block-draft forward over
 * [E(A), E(T1)+Delta, E(MASK)...] proposes the remaining candidates, and the
 * target verifies all of them, committing the accepted prefix plus one
 * correction or bonus token.  Four calls cover it; the MTP decoder block and a
 * summary of acceptance over rounds complete the set:
 *
 *   dmtp_fuse         RMSNorm-concat-projection (MTP input fusion; DMTP residual)
 *   dmtp_fuse_noalloc the same without a caller workspace (static scratch)
 *   dmtp_mtp_block    the MTP decoder block (causal, with its own KV cache)
 *   dmtp_ctx_kv       the drafter's context K/V rows from target features
 *   dmtp_block_draft  the block drafter's layers and final norm
 *   dmtp_lm_head      the shared vocabulary head with argmax / sampling
 *   dmtp_verify       greedy, rejection-sampling or target-only block verification
 *   dmtp_accept_stats acceptance histogram and statistics of verify rounds
 *
 * Conventions (all calls)
 *   - Tensor pointers are DEVICE pointers to row-major, contiguous data,
 *     16-byte aligned; sizes are element counts.  Weight matrices are stored
 *     [out, in].  Ids are int32, logits/probabilities/lse are float32.
 *   - `dtype` (DMTP_F32 or DMTP_BF16) is the storage type of weights,
 *     embeddings, context K/V and the rows that enter the LM head.  All other
 *     activations (fused hidden, residual stream) are float32.  bf16 is stored
 *     as its 16-bit pattern.  Gains are float32 [H].
 *   - Ownership: the caller owns every buffer, including the workspace
 *     `ws` of the size the matching *_ws() query returns.  The library never
 *     allocates, frees, synchronises or copies to the host.  Each call only
 *     enqueues kernels on the caller's stream and can be captured in a graph.
 *   - Errors: every call returns an int status.  Negative values are argument
 *     errors found on the host BEFORE anything is enqueued (nothing has run).
 *     DMTP_E_LAUNCH reports a failed kernel launch.  Device-side faults surface
 *     at the caller's next synchronisation.  Shapes the kernels do not support
 *     are refused, never silently degraded.
 *   - The library holds no state across calls and is safe to call from
 *     several host threads on different streams; calls that share output or
 *     workspace buffers must be ordered by the caller.  The one exception is
 *     dmtp_fuse_noalloc, whose scratch is a static array per GPU.
 */
#ifndef DMTP_H
#define DMTP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DMTP_ABI_VERSION 8

enum dmtp_status {
  DMTP_OK = 0,
  DMTP_E_NULL = -1,      /* a required pointer is NULL */
  DMTP_E_SHAPE = -2,     /* a size is out of the supported range */
  DMTP_E_DTYPE = -3,     /* unknown or unsupported dtype */
  DMTP_E_WORKSPACE = -4, /* workspace smaller than the *_ws() query */
  DMTP_E_ALIGN = -5,     /* a pointer is not 16-byte aligned */
  DMTP_E_DEVICE = -6,    /* the current device is not gfx950 */
  DMTP_E_LAUNCH = -7,    /* a kernel launch failed */
  DMTP_E_ARG = -8,       /* an inconsistent combination of arguments */
  DMTP_E_SCRATCH = -9    /* the call needs more than the static scratch buffer holds */
};

enum dmtp_dtype { DMTP_F32 = 0, DMTP_BF16 = 1 };

/* draw_key value of a row that takes the argmax even when its temperature is
 * positive (its lse is still taken at that temperature). */
#define DMTP_NO_DRAW 0xFFFFFFFFFFFFFFFFull

/* Entries per block of the two-level draws of dmtp_lm_head and dmtp_verify. */
#define DMTP_DRAW_BLOCK 128

/* Rows of a fusion input: either `rows` [n, H] in `dtype` (row stride H), or,
 * when rows == NULL, the gather table[ids[r]] with table [V, H] in the call's
 * weight dtype.  A dmtp_rows with rows == NULL and ids == NULL is "absent". */
typedef struct {
  const void* rows;
  int32_t dtype;          /* DMTP_F32 or DMTP_BF16 (rows mode) */
  const int32_t* ids;     /* [n], each in [0, table_rows) */
  const void* table;
  int32_t table_rows;
} dmtp_rows;

/* ---------------------------------------------------------------- fuse ----
 * out[r] = res[r] + W [RMSNorm(x1[r]; g1); RMSNorm(x2[r]; g2)]
 * RMSNorm(x; g) = x / sqrt(mean(x^2) + eps) * g.  W is [H, 2H] in w_dtype:
 * columns [0, H) act on the normalised x1, [H, 2H) on the normalised x2.
 *   MTP input fusion ("DFlash vs MTP", "MTP: Sequential Prediction Heads
 *   Trained With the Model": h' = M[RMSNorm(h); RMSNorm(Emb(t))]):
 *       x1 = target hidden rows, x2 = ids of the pending token A, res absent.
 *   DMTP residual (DMTP blog section 3, the Delta and e~ equations):
 *       x1 = ids T1, x2 = MTP hidden rows, res = ids T1 (E(T1) + Delta).
 * out is float32 [rows, H].  Zero W returns res bit for bit. */
typedef struct {
  int32_t rows;           /* >= 1 */
  int32_t H;              /* multiple of 64, <= 16384 */
  int32_t w_dtype;        /* dtype of W and of id-gathered tables */
  float eps;
  dmtp_rows x1, x2, res;  /* res may be absent */
  const float* g1;        /* [H] */
  const float* g2;        /* [H] */
  const void* W;          /* [H, 2H] */
  float* out;             /* [rows, H] */
} dmtp_fuse_desc;

size_t dmtp_fuse_ws(const dmtp_fuse_desc* d);
int dmtp_fuse(const dmtp_fuse_desc* d, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------ fuse without an allocation ----
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Computes
 * exactly what dmtp_fuse computes, with the same kernels, but takes no
 * workspace: its scratch (the split-K partials and sums of squares, or the
 * normalised rows) lives in a static device array of DMTP_SCRATCH_BYTES inside
 * the library, one per GPU, held until the process ends.  The caller still
 * owns the input and output buffers.
 *   - Returns DMTP_E_SCRATCH, before anything is enqueued, when the call
 *     would need more than DMTP_SCRATCH_BYTES (dmtp_fuse_ws(d) is that need).
 *   - Allocates nothing: no hipMalloc / hipFree on any call.  The first call
 *     on a device looks up that device's copy of the array.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents; nothing in it has to start at zero (every call writes
 *     all the scratch it reads).  Calls that overlap on one GPU -- on
 *     different streams, or from different host threads -- race on it: the
 *     caller must order them.
 * Other errors are those of dmtp_fuse. */
#define DMTP_SCRATCH_BYTES ((size_t)16 << 20)
int dmtp_fuse_noalloc(const dmtp_fuse_desc* d, hipStream_t stream);

/* ---------------------------------------------------------- block draft ----
 * The block drafter ("DFlash vs MTP", "DFlash: Block Diffusion as a Draft
 * Model"; DMTP blog sections 3 and 6.2).  Per sequence b the S = K - 1 +
 * n_anchor slots are
 *     n_anchor = 2:  [E(anchor_ids[b]), x_t1[b], E(mask_id) x (K-1)]
 *     n_anchor = 1:  [x_t1[b], E(mask_id) x (K-1)]
 * at positions ctx_len[b] + j (ctx_len[b] = cu_ctx[b+1] - cu_ctx[b], which must
 * not exceed max_ctx).  Each layer: x^ = RMSNorm(X; g_attn); q, k, v
 * = x^ Wqkv^T (rows of Wqkv: Hq query heads, Hkv key heads, Hkv value heads,
 * d each); rotary embedding (rotate-half, base rope_base) on block q and k;
 * every slot attends, with no mask, to the context keys of its own sequence
 * (the last `window` when window > 0) and to all S block keys; GQA maps
 * query head h to kv head h / (Hq / Hkv); X1 = X + o Wo^T; X = X1 +
 * (silu(x^2 Wg^T) * (x^2 Wu^T)) Wd^T with x^2 = RMSNorm(X1; g_ffn).  After the
 * last layer the MASK slots (slots n_anchor .. S-1) are written as
 * RMSNorm(X; g_final) rounded to dtype: out [B, K-1, H] -- the LM-head input
 * of candidates 1 .. K-1.  Context keys are supplied already rotated. */
typedef struct {
  const float* g_attn;    /* [H] */
  const void* wqkv;       /* [(Hq + 2 Hkv) d, H] */
  const void* wo;         /* [H, Hq d] */
  const float* g_ffn;     /* [H] */
  const void* wg;         /* [F, H] */
  const void* wu;         /* [F, H] */
  const void* wd;         /* [H, F] */
  const void* ctx_k;      /* [sum ctx_len, Hkv, d]  (sequence b at rows cu_ctx[b] ..) */
  const void* ctx_v;      /* [sum ctx_len, Hkv, d] */
} dmtp_layer;

typedef struct {
  int32_t B, H, Hq, Hkv, d, F, n_layers, K, n_anchor, dtype;
  float eps;
  float rope_base;
  int32_t window;         /* 0 = whole context */
  int32_t max_ctx;        /* host-side upper bound of ctx_len[b] (plans the split) */
  int32_t ctx_rows;       /* rows of ctx_k / ctx_v; sequences are clamped to them */
  int32_t V;              /* rows of emb */
  const int32_t* anchor_ids;  /* [B] (unused when n_anchor == 1) */
  const float* x_t1;      /* [B, H] float32 (output of the DMTP residual fusion) */
  int32_t mask_id;
  const void* emb;        /* [V, H] */
  const int32_t* cu_ctx;  /* [B + 1] prefix sums of the context lengths */
  const dmtp_layer* layers;   /* HOST array of n_layers entries */
  const float* g_final;   /* [H] */
  void* out;              /* [B, K - 1, H] in dtype */
  /* Optional profiling hook: when both are set (hipEvent_t handles created
   * with timing enabled), the context-attention kernel of layer 0 (bf16
   * context K/V) is launched with them as its start and stop events, taken
   * from that kernel's own dispatch, so hipEventElapsedTime(start, stop) is
   * its duration and no extra command enters the stream.  Ignored when no
   * context row is read or the context is float32 (then neither is
   * recorded). */
  void* attn_start_event;
  void* attn_stop_event;
} dmtp_draft_desc;

size_t dmtp_block_draft_ws(const dmtp_draft_desc* d);
int dmtp_block_draft(const dmtp_draft_desc* d, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ MTP block ----
 * The MTP decoder block ("DFlash vs MTP", "MTP: Sequential Prediction Heads
 * Trained With the Model": a dedicated Transformer block after the input
 * projection h' = M[RMSNorm(h); RMSNorm(Emb(t))]; DMTP blog section 6.5:
 * full-history causal attention, projections, normalisation and a
 * feed-forward network; colibri: the head keeps its own causal KV cache, to
 * which every completed pair contributes its K/V).  Per sequence b, S new rows
 * x[b, j] (the fused inputs h' produced by dmtp_fuse) at positions
 * ctx_len[b] + j, where ctx_len[b] = cu_ctx[b+1] - cu_ctx[b] is the length of
 * the block's cache.  Each of the n_layers layers is the decoder layer of
 * dmtp_block_draft, except that row j attends to the whole cache (no window)
 * and to new rows 0..j only (causal); layers[l].ctx_k / ctx_v are layer l's
 * cache [sum ctx_len, Hkv, d] in dtype, keys already rotated.
 *   out [B, S, H] float32: h_MTP of each new row, the residual stream after the
 *       last layer (no final norm; the LM head applies its own).
 *   k_new[l] / v_new[l] (HOST array of n_layers device pointers, or NULL):
 *       [B, S, Hkv, d] in dtype, layer l's rotated keys and values of the new
 *       rows -- what the caller appends to the cache once the rows are
 *       committed.  A NULL entry skips that output. */
typedef struct {
  int32_t B, S, H, Hq, Hkv, d, F, n_layers, dtype;
  float eps;
  float rope_base;
  int32_t max_ctx;        /* host-side upper bound of ctx_len[b] */
  int32_t ctx_rows;       /* rows of each layer's cache; sequences are clamped to them */
  const float* x;         /* [B, S, H] float32 */
  const int32_t* cu_ctx;  /* [B + 1] prefix sums of the cache lengths */
  const dmtp_layer* layers;   /* HOST array of n_layers entries */
  float* out;             /* [B, S, H] float32 */
  void* const* k_new;     /* HOST array of n_layers pointers, or NULL */
  void* const* v_new;     /* HOST array of n_layers pointers, or NULL */
} dmtp_mtp_desc;

size_t dmtp_mtp_block_ws(const dmtp_mtp_desc* d);
int dmtp_mtp_block(const dmtp_mtp_desc* d, void* ws, size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------------- context K/V ----
 * The drafter's context key/value rows of newly committed target rows
 * ("DFlash vs MTP", "DFlash: Block Diffusion as a Draft Model": KV injection
 * of hidden features from a few target layers into the cache of every draft
 * layer; DMTP blog section 3, ablation notes: context fusion concatenates
 * five target feature streams and projects them back to the hidden size).
 * Per new row n: c = W_fc [f_1; ...; f_n_feat] (feats[n] holds the streams),
 * then for every drafter layer l, with x^ = RMSNorm(c; layers[l].g_attn) and
 * the key / value rows of layers[l].wqkv:
 *     k = RoPE(x^ Wk^T, positions[n]) (rotate-half, base rope_base),
 *     v = x^ Wv^T,
 * written in dtype to k_cache[l][dst_rows[n]] and v_cache[l][dst_rows[n]]
 * ([ctx_rows, Hkv, d] each) -- the rows dmtp_block_draft then reads as
 * context.  A dst_rows entry outside [0, ctx_rows) writes nothing.  ctx_out,
 * when given, receives c [N, H] float32. */
typedef struct {
  int32_t N;              /* new rows, 1 .. 65536 */
  int32_t n_feat;         /* feature streams per row, 1 .. 8 */
  int32_t H, Hq, Hkv, d, n_layers, dtype;
  float eps;
  float rope_base;
  const void* feats;      /* [N, n_feat, H] in dtype */
  const int32_t* positions;   /* [N] */
  const int32_t* dst_rows;    /* [N] */
  const void* w_fc;       /* [H, n_feat H] in dtype */
  const dmtp_layer* layers;   /* HOST array: g_attn and wqkv of each drafter layer */
  int32_t ctx_rows;       /* rows of every cache */
  void* const* k_cache;   /* HOST array of n_layers device pointers [ctx_rows, Hkv, d] */
  void* const* v_cache;   /* HOST array of n_layers device pointers [ctx_rows, Hkv, d] */
  float* ctx_out;         /* [N, H] or NULL */
} dmtp_ctx_desc;

size_t dmtp_ctx_kv_ws(const dmtp_ctx_desc* d);
int dmtp_ctx_kv(const dmtp_ctx_desc* d, void* ws, size_t ws_bytes, hipStream_t stream);

/* -------------------------------------------------------------- LM head ----
 * The shared vocabulary head ("DFlash vs MTP": shared output head; DMTP blog
 * section 6.5: it reads the whole [V, H] matrix for every row).  The M rows
 * are the concatenation of up to 4 segments.  A segment with g_norm != NULL
 * holds float32 hidden rows that are first mapped to RMSNorm(x; g_norm) and
 * rounded to dtype; otherwise its rows are already the head input, in dtype.
 * logits = W x (W [V, H]).  Per row m:
 *   temperature[m] == 0 (or temperature == NULL): token = argmax (lowest
 *       index among equal maxima), gap = top-1 minus top-2 logit;
 *   temperature[m] > 0 and draw_key[m] != DMTP_NO_DRAW: token is a draw from
 *       softmax(logits / t) in two levels: first the block b of
 *       DMTP_DRAW_BLOCK consecutive entries that maximises log Z_b + g1_b
 *       (Z_b the block's softmax mass), then the entry j of block b that
 *       maximises logits_j / t + g0_j.  gL_i is the Gumbel noise of level L of
 *       Philox4x64-10 draw (seed, draw_key[m]): word i of counter
 *       (i >> 3, key, L, 0) under key (seed, 0), 64-bit output (i & 7) >> 1,
 *       low half if i even; g = -log(-log1p(-(x + 1/2) 2^-32)).  The two
 *       noises are independent, so j is drawn with probability softmax_j
 *       (Gumbel-max identity, applied to the blocks and within the block).
 *       gap = the smaller of the two levels' top-2 score gaps.  The block
 *       masses come from one pass over the stored logits row, so such rows
 *       need store_row[m] >= 0 (else token = -1).
 *   temperature[m] > 0 and draw_key[m] == DMTP_NO_DRAW: argmax, as greedy.
 *   row_max = max logit; lse = logsumexp(logits / t) (t = 1 when 0).
 *   store_row[m] >= 0 writes the float32 logits row to logits[store_row[m]].
 *   plant_row[m] in [0, M) replaces the row's token by the argmax of row
 *       plant_row[m] of the same call (a workload whose first candidate is
 *       set to the target's choice).
 * Ids, offsets and row indices read from device memory are range-checked in
 * the kernels: an out-of-range embedding id reads a zero row, an
 * out-of-range store or plant index is ignored, so bad data never leads to
 * an out-of-bounds access.
 * A row's results do not depend on the other rows.  With bf16, H a multiple
 * of 512 and at most 2048, a call of at most 32 rows streams the weights with
 * H split into four quarters whose partial sums are added in order, while
 * larger calls sum over H in one sequence: a row's logit statistics then
 * agree between the two to float32 rounding, and tokens agree unless the
 * top-2 gap is within that rounding.  Within either case they do not depend
 * on M. */
typedef struct {
  const void* x;          /* [n, ld] rows */
  int32_t n;              /* rows in this segment (may be 0) */
  int32_t ld;             /* row stride in elements, >= H */
  int32_t dtype;          /* DMTP_F32 when g_norm is set, else the head dtype */
  const float* g_norm;    /* [H] or NULL */
} dmtp_head_segment;

typedef struct {
  int32_t H;              /* multiple of 64 */
  int32_t V;              /* >= 2 */
  int32_t dtype;          /* dtype of W and of the head input */
  float eps;
  int32_t n_seg;          /* 1 .. 4 */
  dmtp_head_segment seg[4];
  const void* W;          /* [V, H] */
  const float* temperature;   /* [M] or NULL: all greedy */
  const uint64_t* draw_key;   /* [M], required when temperature != NULL */
  uint64_t seed;
  const int32_t* plant_row;   /* [M] or NULL */
  const int32_t* store_row;   /* [M] or NULL */
  float* logits;              /* [logits_rows, V] */
  int32_t logits_rows;        /* store_row values >= logits_rows are not stored */
  void* prepared;             /* optional [M, H] in dtype: the head input rows */
  int32_t* token;             /* [M] */
  float* row_max;             /* [M] or NULL */
  float* lse;                 /* [M] or NULL */
  float* gap;                 /* [M] or NULL */
  /* Optional profiling hook: when both are set (hipEvent_t handles created
   * with timing enabled), the bf16 vocabulary GEMM kernel of this call is
   * launched with them as its start and stop events, taken from that
   * kernel's own dispatch, so hipEventElapsedTime(start, stop) is its
   * duration and no extra command enters the stream.  Ignored by the float32
   * path (which then records neither). */
  void* gemm_start_event;
  void* gemm_stop_event;
  /* Optional: W in the packed layout written by dmtp_head_pack (bf16 only),
   * 16-byte aligned.  The matrix-core GEMMs of bf16 calls with H a multiple
   * of 128 (more than 32 input rows, or any number when H is above 2048) then
   * stream their weight stages from it, each one contiguous 16 KB block,
   * instead of 128 runs of 128 bytes of W; results are bit-identical.  The
   * weight-streaming kernel of calls of at most 32 rows (H up to 2048) reads
   * W, which stays required.  NULL: W only. */
  const void* w_packed;
} dmtp_head_desc;

size_t dmtp_lm_head_ws(const dmtp_head_desc* d);
int dmtp_lm_head(const dmtp_head_desc* d, void* ws, size_t ws_bytes, hipStream_t stream);

/* ----------------------------------------------------- packed head weight ----
 * Not a step of the pages: a one-time copy of the shared head matrix W
 * [V, H] (bf16, H a multiple of 64) into the order in which the LM-head GEMM
 * streams it, made when the weights are loaded and passed to dmtp_lm_head as
 * w_packed.  Vocabulary tile t (rows 128 t .. 128 t + 127; rows at or past V
 * are zeros) occupies bytes [t 256 H, (t + 1) 256 H) of out; within it, block
 * s (H / 64 blocks of 16384 bytes) holds columns 64 s .. 64 s + 63 of the
 * tile's rows as 1024 pieces of 8 elements: piece 8 r + j is columns
 * 64 s + 8 (j ^ ((r >> 1) & 7)) .. + 7 of row 128 t + r.  That is the image
 * of the GEMM's LDS stage, so a stage is one contiguous copy.
 * dmtp_head_pack_bytes: the size of out, ceil(V / 128) 256 H bytes (0 for an
 * unsupported V or H).  dmtp_head_pack: W and out on the current device,
 * 16-byte aligned, out_bytes at least that size; dtype must be DMTP_BF16.
 * The copy is enqueued on stream; errors as for the other calls. */
size_t dmtp_head_pack_bytes(int32_t V, int32_t H);
int dmtp_head_pack(const void* W, int32_t V, int32_t H, int32_t dtype, void* out, size_t out_bytes,
                   hipStream_t stream);

/* --------------------------------------------------------------- verify ----
 * Block verification (DMTP blog section 5 step 3; the colibri notes on
 * verify semantics; Leviathan et al. as cited by "DFlash vs MTP").  Per
 * sequence b the candidates are d_0 = t1[b], d_i = drafts[b][i-1]; target row
 * i (i = 0..K) is the target after the prefix and d_0 .. d_{i-1}.
 *   temperature[b] == 0: L = first i < K with d_i != target[b][i] (else K);
 *       commit d_0 .. d_{L-1}, target[b][L].
 *   temperature[b] = t > 0: with p_i = softmax(lp_i / t), q_i =
 *       softmax(lq_i / t) from the float32 logits rows of the sequence
 *       (logits[b][i] = lq_i for i < K, logits[b][K + i] = lp_i), accept d_i
 *       iff u_acc[b][i] < p_i(d_i) / q_i(d_i); at the first rejection i draw
 *       the correction from normalize(max(0, p_i - q_i)) (from p_i if that is
 *       zero); if all K are accepted draw the bonus from p_K.  Draws are
 *       the two-level Gumbel-max draws of dmtp_lm_head over these weights
 *       (block masses of max(0, p_i - q_i) or of p, then an entry of the
 *       chosen block), with draw (seed, final_key[b]).  Needs the lse of
 *       every row (lse of logits / t).
 *   target_only != 0 (DMTP blog section 5, the note on target-only
 *       verification; colibri: a sampled pick equal to the next draft
 *       accepts it): every sequence, whatever its temperature, is verified
 *       against target[b][i], which then holds the target's own pick at row
 *       i -- a draw from softmax(lp_i / t) (dmtp_lm_head with a draw key), or
 *       the argmax at t = 0.  L = first i < K with d_i != target[b][i] (else
 *       K); commit d_0 .. d_{L-1}, target[b][L].  temperature, logits, lse,
 *       u_acc and final_key are not read.
 * out_tokens [B, K+1] is -1 padded, n_out = accept_len + 1. */
typedef struct {
  int32_t B, K, V;
  const int32_t* t1;          /* [B] */
  const int32_t* drafts;      /* [B, K - 1] */
  const int32_t* target;      /* [B, K + 1] target argmax per row */
  const float* temperature;   /* [B] or NULL: all greedy */
  const float* logits;        /* [B, 2K + 1, V], rows of sampled sequences only */
  const float* t1_lse;        /* [B] */
  const float* draft_lse;     /* [B, K - 1] */
  const float* target_lse;    /* [B, K + 1] */
  const float* u_acc;         /* [B, K] uniforms in [0, 1) */
  uint64_t seed;
  const uint64_t* final_key;  /* [B] */
  int32_t* accept_len;        /* [B] */
  int32_t* out_tokens;        /* [B, K + 1] */
  int32_t* n_out;             /* [B] */
  int32_t target_only;        /* 0: greedy (t = 0) / rejection (t > 0); 1: target-only */
  /* Optional profiling hook: when both are set (hipEvent_t handles created
   * with timing enabled), the pass over the drawn rows' logits (the block
   * masses of max(0, p - q) and of p) is launched with them as its start and
   * stop events, taken from that kernel's own dispatch.  Ignored when the
   * call has no such pass (greedy or target-only; then neither is
   * recorded). */
  void* mass_start_event;
  void* mass_stop_event;
} dmtp_verify_desc;

size_t dmtp_verify_ws(const dmtp_verify_desc* d);
int dmtp_verify(const dmtp_verify_desc* d, void* ws, size_t ws_bytes, hipStream_t stream);

/* ----------------------------------------------------- acceptance stats ----
 * Acceptance statistics of verify rounds (DMTP blog section 7: per-verify
 * acceptance length and its histogram; section 7 "Position-Wise Acceptance":
 * cumulative P(L >= k) and conditional acceptance).  Adds the B accepted
 * lengths to a running histogram and, optionally, summarises it:
 *   hist[k] += #{b : accept_len[b] == k}, k = 0..K   (lengths outside [0, K]
 *       are not counted; hist is caller-owned device memory, accumulated
 *       across calls -- zero it before the first)
 *   summary (NULL to skip), from the updated histogram, N = sum_k hist[k]:
 *     [0]         per-verify length 1 + sum_k k hist[k] / N (the committed
 *                 correction/bonus token included)
 *     [1]         first-candidate acceptance 1 - hist[0] / N
 *     [2 + k - 1] cumulative P(L >= k), k = 1..K
 *     [2 + K + k - 1] conditional P(L >= k | L >= k-1), k = 1..K
 *                 (NaN where the condition has no rounds; all NaN when N = 0)
 * Needs no workspace.  Integer counts make the histogram exact and the result
 * independent of the order of rows. */
typedef struct {
  int32_t B;                  /* >= 0 rows in this call */
  int32_t K;                  /* 1 .. 64 candidates per round */
  const int32_t* accept_len;  /* [B] */
  int64_t* hist;              /* [K + 1], accumulated */
  double* summary;            /* [2 + 2K] or NULL */
} dmtp_stats_desc;

int dmtp_accept_stats(const dmtp_stats_desc* d, hipStream_t stream);

/* ------------------------------------------------------------- helpers ---- */
const char* dmtp_status_str(int status);
const char* dmtp_version(void);
/* sizeof of the descriptor structs, for bindings to check their layout:
 * which = 0 rows, 1 fuse, 2 layer, 3 draft, 4 head segment, 5 head, 6 verify,
 * 7 stats, 8 MTP block, 9 context K/V */
size_t dmtp_struct_size(int which);

#ifdef __cplusplus
}
#endif

#endif /* DMTP_H */

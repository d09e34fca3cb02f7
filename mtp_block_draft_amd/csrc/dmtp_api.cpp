// The C ABI: argument validation on the host (before anything is enqueued),
// workspace planning, and the kernel sequence of each call.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

#include "dmtp.h"
#include "kernels.hpp"

namespace {

using namespace dmtp;

constexpr size_t kAlign = 256;
size_t al(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool valid_dtype(int t) { return t == DMTP_F32 || t == DMTP_BF16; }
size_t esize(int t) { return t == DMTP_BF16 ? 2 : 4; }

#define CHECK(cond, code) \
  do {                    \
    if (!(cond)) return (code); \
  } while (0)

// --- device check: gfx950 only (cached per device ordinal)
std::atomic<int> g_arch_ok[64];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DMTP_E_DEVICE;
  if (dev < 0 || dev >= 64) return DMTP_E_DEVICE;
  int s = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (s == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DMTP_E_DEVICE;
    s = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_arch_ok[dev].store(s, std::memory_order_relaxed);
  }
  return s == 1 ? DMTP_OK : DMTP_E_DEVICE;
}

int check_rows(const dmtp_rows& r, bool allow_absent) {
  if (!r.rows && !r.ids) return allow_absent ? DMTP_OK : DMTP_E_NULL;
  if (r.rows && r.ids) return DMTP_E_ARG;
  if (r.rows) {
    CHECK(valid_dtype(r.dtype), DMTP_E_DTYPE);
    CHECK(aligned16(r.rows), DMTP_E_ALIGN);
  } else {
    CHECK(r.table != nullptr, DMTP_E_NULL);
    CHECK(r.table_rows >= 1, DMTP_E_SHAPE);
    CHECK(aligned16(r.table), DMTP_E_ALIGN);
  }
  return DMTP_OK;
}

// ---------------------------------------------------------------- fuse ----
int validate_fuse(const dmtp_fuse_desc* d) {
  CHECK(d != nullptr, DMTP_E_NULL);
  CHECK(d->rows >= 1 && d->rows <= (1 << 20), DMTP_E_SHAPE);
  CHECK(d->H >= 64 && d->H <= 16384 && d->H % 64 == 0, DMTP_E_SHAPE);
  CHECK(valid_dtype(d->w_dtype), DMTP_E_DTYPE);
  CHECK(d->eps >= 0.f, DMTP_E_ARG);
  int e;
  if ((e = check_rows(d->x1, false)) != DMTP_OK) return e;
  if ((e = check_rows(d->x2, false)) != DMTP_OK) return e;
  if ((e = check_rows(d->res, true)) != DMTP_OK) return e;
  CHECK(d->g1 && d->g2 && d->W && d->out, DMTP_E_NULL);
  CHECK(aligned16(d->g1) && aligned16(d->g2) && aligned16(d->W) && aligned16(d->out), DMTP_E_ALIGN);
  return DMTP_OK;
}

size_t fuse_ws(const dmtp_fuse_desc* d) {
  if (fuse_fits(*d)) return al(fuse_fused_ws(*d));
  return al((size_t)d->rows * 2 * d->H * 4) +
         al(gemm_ws_bytes(d->rows, d->H, 2 * d->H, d->w_dtype == DMTP_F32));
}

// ---------------------------------------------------------- block draft ----
int check_layers(const dmtp_layer* layers, int n_layers, bool has_ctx);

int validate_draft(const dmtp_draft_desc* d) {
  CHECK(d != nullptr, DMTP_E_NULL);
  CHECK(d->B >= 1 && d->B <= 4096, DMTP_E_SHAPE);
  CHECK(d->H >= 64 && d->H <= 16384 && d->H % 64 == 0, DMTP_E_SHAPE);
  CHECK(d->d == 64 || d->d == 128, DMTP_E_SHAPE);
  CHECK(d->Hkv >= 1 && d->Hq >= d->Hkv && d->Hq % d->Hkv == 0 && d->Hq <= 256, DMTP_E_SHAPE);
  CHECK((d->Hq * d->d) % 64 == 0, DMTP_E_SHAPE);
  CHECK(d->F >= 64 && d->F % 64 == 0 && d->F <= 65536, DMTP_E_SHAPE);
  CHECK(d->n_layers >= 1 && d->n_layers <= 64, DMTP_E_SHAPE);
  CHECK(d->K >= 2 && d->K <= 32, DMTP_E_SHAPE);
  CHECK(d->n_anchor == 1 || d->n_anchor == 2, DMTP_E_SHAPE);
  const int S = d->K - 1 + d->n_anchor;
  CHECK(valid_dtype(d->dtype), DMTP_E_DTYPE);
  // query rows per kv head that fit one workgroup's LDS
  CHECK(S * (d->Hq / d->Hkv) <= attn_max_nq(d->d, d->dtype == DMTP_F32), DMTP_E_SHAPE);
  CHECK(d->eps >= 0.f && d->rope_base > 1.f, DMTP_E_ARG);
  CHECK(d->window >= 0 && d->max_ctx >= 0 && d->ctx_rows >= 0, DMTP_E_SHAPE);
  CHECK(d->V >= 2 && d->mask_id >= 0 && d->mask_id < d->V, DMTP_E_SHAPE);
  CHECK(d->x_t1 && d->emb && d->cu_ctx && d->layers && d->g_final && d->out, DMTP_E_NULL);
  if (d->n_anchor == 2) CHECK(d->anchor_ids != nullptr, DMTP_E_NULL);
  CHECK(aligned16(d->x_t1) && aligned16(d->emb) && aligned16(d->g_final) && aligned16(d->out),
        DMTP_E_ALIGN);
  return check_layers(d->layers, d->n_layers, d->max_ctx > 0 && d->ctx_rows > 0);
}

// Shapes of a stack of decoder layers over B sequences of S rows (the drafter's
// slots, or the MTP block's new rows).
struct Stack {
  int B, S, H, Hq, Hkv, d, F, n_layers, dtype;
  float eps, rope_base;
  int window, max_ctx, ctx_rows;
  const dmtp_layer* layers;
  const int32_t* cu_ctx;
  int causal;
  void* attn_ev[2];   // optional start/stop events of layer 0's context attention
};

Stack stack_of(const dmtp_draft_desc* d) {
  return Stack{d->B, d->K - 1 + d->n_anchor, d->H, d->Hq, d->Hkv, d->d, d->F, d->n_layers,
               d->dtype, d->eps, d->rope_base, d->window, d->max_ctx, d->ctx_rows, d->layers,
               d->cu_ctx, 0, {d->attn_start_event, d->attn_stop_event}};
}

Stack stack_of(const dmtp_mtp_desc* d) {
  return Stack{d->B, d->S, d->H, d->Hq, d->Hkv, d->d, d->F, d->n_layers, d->dtype, d->eps,
               d->rope_base, 0, d->max_ctx, d->ctx_rows, d->layers, d->cu_ctx, 1, {nullptr, nullptr}};
}

struct DraftWs {
  size_t X, xh, qkv, q, kb, vb, o, gate, up, act, gemm, gemm2, attn, total;
  AttnPlan plan;
};

DraftWs stack_ws(const Stack& d) {
  DraftWs w;
  const int S = d.S;
  const size_t R = (size_t)d.B * S;
  const int qkv_n = (d.Hq + 2 * d.Hkv) * d.d;
  w.plan = attn_plan(d.B, d.Hq, d.Hkv, S, d.d, d.max_ctx, d.window, d.dtype == DMTP_F32, d.ctx_rows);
  w.plan.causal = d.causal;
  size_t gemm_max = 0;
  const int wf32 = d.dtype == DMTP_F32;
  auto upd = [&](int M, int N, int K) {
    const size_t b = gemm_ws_bytes(M, N, K, wf32);
    if (b > gemm_max) gemm_max = b;
  };
  upd((int)R, qkv_n, d.H);
  upd((int)R, d.H, d.Hq * d.d);
  upd((int)R, 2 * d.F, d.H);   // gate and up as one GEMM (bf16 weights)
  upd((int)R, d.F, d.H);
  upd((int)R, d.H, d.F);
  size_t o = 0;
  w.X = o; o = al(o + R * d.H * 4);
  w.xh = o; o = al(o + R * d.H * 4);
  w.qkv = o; o = al(o + R * qkv_n * 4);
  w.q = o; o = al(o + R * d.Hq * d.d * 4);
  w.kb = o; o = al(o + R * d.Hkv * d.d * 4);
  w.vb = o; o = al(o + R * d.Hkv * d.d * 4);
  w.o = o; o = al(o + R * d.Hq * d.d * 4);
  w.gate = o; o = al(o + R * 2 * d.F * 4);   // [R, 2F]: gate columns, then up columns
  w.up = o; o = al(o + R * d.F * 4);
  w.act = o; o = al(o + R * d.F * 4);
  w.gemm = o; o = al(o + gemm_max);
  w.gemm2 = o; o = al(o + gemm_max);   // the up projection's partials (live with the gate's)
  w.attn = o; o = al(o + attn_ws_bytes(w.plan));
  w.total = o;
  return w;
}

DraftWs draft_ws(const dmtp_draft_desc* d) { return stack_ws(stack_of(d)); }

// The layers of a stack over X [B S, H] (float32, in the workspace), whose
// first-layer norm planes are already in xh.  Layer l's rotated block keys and
// values go to k_new[l] / v_new[l] when those are given.  On return *last is
// the residual stream after the last layer, as a split result not yet summed.
hipError_t run_stack(const Stack& d, const DraftWs& w, char* b, void* const* k_new,
                     void* const* v_new, SplitOut* last, hipStream_t stream) {
  float* X = (float*)(b + w.X);
  uint16_t* xh = (uint16_t*)(b + w.xh);   // bf16 planes [2][R][H]
  float* qkv = (float*)(b + w.qkv);
  float* q = (float*)(b + w.q);
  float* kb = (float*)(b + w.kb);
  float* vb = (float*)(b + w.vb);
  uint16_t* o = (uint16_t*)(b + w.o);     // bf16 planes [2][R][Hq d]
  float* gate = (float*)(b + w.gate);
  float* up = (float*)(b + w.up);
  uint16_t* act = (uint16_t*)(b + w.act); // bf16 planes [2][R][F]
  float* gws = (float*)(b + w.gemm);
  float* gws2 = (float*)(b + w.gemm2);
  float* aws = (float*)(b + w.attn);
  const int S = d.S;
  const int R = d.B * S;
  const int qkv_n = (d.Hq + 2 * d.Hkv) * d.d;
  const int wf32 = d.dtype == DMTP_F32;
  const size_t pst_h = (size_t)R * d.H, pst_o = (size_t)R * d.Hq * d.d;
  const int od = d.Hq * d.d;
  hipError_t h = hipSuccess;
  for (int l = 0; l < d.n_layers && h == hipSuccess; ++l) {
    const dmtp_layer& L = d.layers[l];
    SplitOut sq, so, sg, su, sd;
    GemmArgs g1{xh, pst_h, (size_t)d.H, R, L.wqkv, wf32, (size_t)d.H, qkv_n, d.H, qkv,
                (size_t)qkv_n, nullptr, 0};
    if ((h = gemm_deferred(g1, gws, stream, &sq)) != hipSuccess) break;
    if ((h = rope_split(sq, d.cu_ctx, d.ctx_rows, d.B, S, d.Hq, d.Hkv, d.d, d.rope_base, q, kb, vb,
                        stream)) != hipSuccess)
      break;
    if ((k_new || v_new) &&
        (h = export_kv(kb, vb, d.B, S, d.Hkv, d.d, d.dtype, k_new ? k_new[l] : nullptr,
                       v_new ? v_new[l] : nullptr, stream)) != hipSuccess)
      break;
    const bool ev = l == 0 && d.attn_ev[0] && d.attn_ev[1];
    if ((h = attention(w.plan, q, kb, vb, L.ctx_k, L.ctx_v, d.cu_ctx, d.ctx_rows, aws, o, stream,
                       ev ? (hipEvent_t)d.attn_ev[0] : nullptr, ev ? (hipEvent_t)d.attn_ev[1] : nullptr)) !=
        hipSuccess)
      break;
    GemmArgs g2{o, pst_o, (size_t)od, R, L.wo, wf32, (size_t)od, d.H, od, X, (size_t)d.H, X,
                (size_t)d.H};
    if ((h = gemm_deferred(g2, gws, stream, &so)) != hipSuccess) break;
    if ((h = residual_rmsnorm(so, X, (size_t)d.H, 1, L.g_ffn, d.eps, xh, R, d.H, stream)) !=
        hipSuccess)
      break;
    // gate and up projections of the same rows; bf16 weights as one GEMM over
    // [Wg; Wu] (columns [0, F) the gate, [F, 2F) the up projection), whose
    // epilogue applies the SwiGLU where the product needs no K split
    bool act_done = false;
    if (!wf32) {
      GemmArgs g3{xh, pst_h, (size_t)d.H, R, L.wg, wf32, (size_t)d.H, 2 * d.F, d.H, gate,
                  (size_t)2 * d.F, nullptr, 0};
      g3.B2 = L.wu;
      g3.N1 = d.F;
      h = gemm_swiglu(g3, act, stream);
      if (h == hipSuccess) {
        act_done = true;
      } else if (h == hipErrorNotSupported) {
        SplitOut sgu;
        if ((h = gemm_deferred(g3, gws, stream, &sgu)) != hipSuccess) break;
        sg = sgu;
        su = sgu;
        su.C = sgu.C + d.F;
        if (su.splits > 1) su.part = sgu.part + d.F;
      } else {
        break;
      }
    } else {
      GemmArgs g3{xh, pst_h, (size_t)d.H, R, L.wg, wf32, (size_t)d.H, d.F, d.H, gate,
                  (size_t)d.F, nullptr, 0};
      if ((h = gemm_deferred(g3, gws, stream, &sg)) != hipSuccess) break;
      GemmArgs g4{xh, pst_h, (size_t)d.H, R, L.wu, wf32, (size_t)d.H, d.F, d.H, up,
                  (size_t)d.F, nullptr, 0};
      if ((h = gemm_deferred(g4, gws2, stream, &su)) != hipSuccess) break;
    }
    if (!act_done && (h = swiglu(sg, su, act, R, d.F, stream)) != hipSuccess) break;
    const size_t pst_f = (size_t)R * d.F;
    GemmArgs g5{act, pst_f, (size_t)d.F, R, L.wd, wf32, (size_t)d.F, d.H, d.F, X,
                (size_t)d.H, X, (size_t)d.H};
    if ((h = gemm_deferred(g5, gws, stream, &sd)) != hipSuccess) break;
    if (l + 1 < d.n_layers)
      h = residual_rmsnorm(sd, X, (size_t)d.H, 1, d.layers[l + 1].g_attn, d.eps, xh, R, d.H, stream);
    else
      *last = sd;
  }
  return h;
}

int check_layers(const dmtp_layer* layers, int n_layers, bool has_ctx) {
  for (int l = 0; l < n_layers; ++l) {
    const dmtp_layer& L = layers[l];
    CHECK(L.g_attn && L.wqkv && L.wo && L.g_ffn && L.wg && L.wu && L.wd, DMTP_E_NULL);
    CHECK(aligned16(L.g_attn) && aligned16(L.wqkv) && aligned16(L.wo) && aligned16(L.g_ffn) &&
              aligned16(L.wg) && aligned16(L.wu) && aligned16(L.wd),
          DMTP_E_ALIGN);
    if (has_ctx) {
      CHECK(L.ctx_k && L.ctx_v, DMTP_E_NULL);
      CHECK(aligned16(L.ctx_k) && aligned16(L.ctx_v), DMTP_E_ALIGN);
    }
  }
  return DMTP_OK;
}

// ------------------------------------------------------------ MTP block ----
int validate_mtp(const dmtp_mtp_desc* d) {
  CHECK(d != nullptr, DMTP_E_NULL);
  CHECK(d->B >= 1 && d->B <= 4096, DMTP_E_SHAPE);
  CHECK(d->S >= 1 && d->S <= 64, DMTP_E_SHAPE);
  CHECK(d->H >= 64 && d->H <= 16384 && d->H % 64 == 0, DMTP_E_SHAPE);
  CHECK(d->d == 64 || d->d == 128, DMTP_E_SHAPE);
  CHECK(d->Hkv >= 1 && d->Hq >= d->Hkv && d->Hq % d->Hkv == 0 && d->Hq <= 256, DMTP_E_SHAPE);
  CHECK((d->Hq * d->d) % 64 == 0, DMTP_E_SHAPE);
  CHECK(d->F >= 64 && d->F % 64 == 0 && d->F <= 65536, DMTP_E_SHAPE);
  CHECK(d->n_layers >= 1 && d->n_layers <= 64, DMTP_E_SHAPE);
  CHECK(valid_dtype(d->dtype), DMTP_E_DTYPE);
  CHECK(d->S * (d->Hq / d->Hkv) <= attn_max_nq(d->d, d->dtype == DMTP_F32), DMTP_E_SHAPE);
  CHECK(d->eps >= 0.f && d->rope_base > 1.f, DMTP_E_ARG);
  CHECK(d->max_ctx >= 0 && d->ctx_rows >= 0, DMTP_E_SHAPE);
  CHECK(d->x && d->cu_ctx && d->layers && d->out, DMTP_E_NULL);
  CHECK(aligned16(d->x) && aligned16(d->out), DMTP_E_ALIGN);
  for (int l = 0; l < d->n_layers; ++l) {
    if (d->k_new && d->k_new[l]) CHECK(aligned16(d->k_new[l]), DMTP_E_ALIGN);
    if (d->v_new && d->v_new[l]) CHECK(aligned16(d->v_new[l]), DMTP_E_ALIGN);
  }
  return check_layers(d->layers, d->n_layers, d->max_ctx > 0 && d->ctx_rows > 0);
}

// ---------------------------------------------------------- context K/V ----
int validate_ctx(const dmtp_ctx_desc* d) {
  CHECK(d != nullptr, DMTP_E_NULL);
  CHECK(d->N >= 1 && d->N <= 65536, DMTP_E_SHAPE);
  CHECK(d->n_feat >= 1 && d->n_feat <= 8, DMTP_E_SHAPE);
  CHECK(d->H >= 64 && d->H <= 16384 && d->H % 64 == 0, DMTP_E_SHAPE);
  CHECK(d->d == 64 || d->d == 128, DMTP_E_SHAPE);
  CHECK(d->Hkv >= 1 && d->Hq >= d->Hkv && d->Hq % d->Hkv == 0 && d->Hq <= 256, DMTP_E_SHAPE);
  CHECK(d->n_layers >= 1 && d->n_layers <= 64, DMTP_E_SHAPE);
  CHECK(valid_dtype(d->dtype), DMTP_E_DTYPE);
  CHECK(d->eps >= 0.f && d->rope_base > 1.f, DMTP_E_ARG);
  CHECK(d->ctx_rows >= 0, DMTP_E_SHAPE);
  CHECK(d->feats && d->positions && d->dst_rows && d->w_fc && d->layers && d->k_cache &&
            d->v_cache,
        DMTP_E_NULL);
  CHECK(aligned16(d->feats) && aligned16(d->w_fc), DMTP_E_ALIGN);
  if (d->ctx_out) CHECK(aligned16(d->ctx_out), DMTP_E_ALIGN);
  for (int l = 0; l < d->n_layers; ++l) {
    const dmtp_layer& L = d->layers[l];
    CHECK(L.g_attn && L.wqkv && d->k_cache[l] && d->v_cache[l], DMTP_E_NULL);
    CHECK(aligned16(L.g_attn) && aligned16(L.wqkv), DMTP_E_ALIGN);
  }
  return DMTP_OK;
}

struct CtxWs {
  size_t planes, c, xh, kv, gemm, total;
};

CtxWs ctx_ws(const dmtp_ctx_desc* d) {
  CtxWs w;
  const size_t N = d->N, H = d->H, KF = (size_t)d->n_feat * d->H, nkv = (size_t)2 * d->Hkv * d->d;
  const int wf32 = d->dtype == DMTP_F32;
  size_t g = gemm_ws_bytes(d->N, d->H, (int)KF, wf32);
  const size_t g2 = gemm_ws_bytes(d->N, (int)nkv, d->H, wf32);
  if (g2 > g) g = g2;
  size_t o = 0;
  w.planes = o; o = al(o + 2 * N * KF * 2);
  w.c = o; o = al(o + N * H * 4);
  w.xh = o; o = al(o + 2 * N * H * 2);
  w.kv = o; o = al(o + N * nkv * 4);
  w.gemm = o; o = al(o + g);
  w.total = o;
  return w;
}

// -------------------------------------------------------------- LM head ----
int validate_head(const dmtp_head_desc* d, int* M_out) {
  CHECK(d != nullptr, DMTP_E_NULL);
  CHECK(d->H >= 64 && d->H <= 16384 && d->H % 64 == 0, DMTP_E_SHAPE);
  CHECK(d->V >= 2 && d->V <= (1 << 26), DMTP_E_SHAPE);
  CHECK(valid_dtype(d->dtype), DMTP_E_DTYPE);
  CHECK(d->eps >= 0.f, DMTP_E_ARG);
  CHECK(d->n_seg >= 1 && d->n_seg <= 4, DMTP_E_SHAPE);
  long M = 0;
  for (int i = 0; i < d->n_seg; ++i) {
    const dmtp_head_segment& s = d->seg[i];
    CHECK(s.n >= 0, DMTP_E_SHAPE);
    if (s.n == 0) continue;
    CHECK(s.x != nullptr, DMTP_E_NULL);
    CHECK(s.ld >= d->H, DMTP_E_SHAPE);
    CHECK(valid_dtype(s.dtype), DMTP_E_DTYPE);
    if (s.g_norm) {
      CHECK(s.dtype == DMTP_F32, DMTP_E_DTYPE);
      CHECK(aligned16(s.g_norm), DMTP_E_ALIGN);
    } else {
      CHECK(s.dtype == d->dtype, DMTP_E_DTYPE);
    }
    CHECK(aligned16(s.x) && ((size_t)s.ld * esize(s.dtype)) % 16 == 0, DMTP_E_ALIGN);
    M += s.n;
  }
  CHECK(M >= 1 && M <= 65536, DMTP_E_SHAPE);
  CHECK(d->W && d->token, DMTP_E_NULL);
  CHECK(aligned16(d->W), DMTP_E_ALIGN);
  if (d->temperature) CHECK(d->draw_key && d->store_row && d->logits, DMTP_E_NULL);
  if (d->store_row) CHECK(d->logits != nullptr && d->logits_rows >= 1, DMTP_E_NULL);
  if (d->prepared) CHECK(aligned16(d->prepared), DMTP_E_ALIGN);
  if (d->w_packed) {
    CHECK(d->dtype == DMTP_BF16, DMTP_E_DTYPE);
    CHECK(aligned16(d->w_packed), DMTP_E_ALIGN);
  }
  *M_out = (int)M;
  return DMTP_OK;
}

// --------------------------------------------------------------- verify ----
int validate_verify(const dmtp_verify_desc* d) {
  CHECK(d != nullptr, DMTP_E_NULL);
  CHECK(d->B >= 1 && d->B <= (1 << 20), DMTP_E_SHAPE);
  CHECK(d->K >= 1 && d->K <= 32, DMTP_E_SHAPE);
  CHECK(d->V >= 2 && d->V <= (1 << 26), DMTP_E_SHAPE);
  CHECK(d->t1 && d->target && d->accept_len && d->out_tokens && d->n_out, DMTP_E_NULL);
  if (d->K > 1) CHECK(d->drafts != nullptr, DMTP_E_NULL);
  CHECK(d->target_only == 0 || d->target_only == 1, DMTP_E_ARG);
  if (d->temperature && !d->target_only) {
    CHECK(d->logits && d->t1_lse && d->target_lse && d->u_acc && d->final_key, DMTP_E_NULL);
    if (d->K > 1) CHECK(d->draft_lse != nullptr, DMTP_E_NULL);
  }
  return DMTP_OK;
}

int validate_stats(const dmtp_stats_desc* d) {
  CHECK(d != nullptr, DMTP_E_NULL);
  CHECK(d->B >= 0 && d->B <= (1 << 30), DMTP_E_SHAPE);
  CHECK(d->K >= 1 && d->K <= accept_stats_max_k(), DMTP_E_SHAPE);
  CHECK(d->hist != nullptr, DMTP_E_NULL);
  if (d->B > 0) CHECK(d->accept_len != nullptr, DMTP_E_NULL);
  CHECK(((uintptr_t)d->hist & 7u) == 0 && ((uintptr_t)d->summary & 7u) == 0, DMTP_E_ALIGN);
  return DMTP_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? DMTP_OK : DMTP_E_LAUNCH; }

// ----------------------------------------------- static scratch buffer ----
// The workspace of dmtp_fuse_noalloc: one array per GPU (each device holds its
// own copy at its own address).  In host code `scratch` names a host-side
// stand-in, never the device memory: every use goes through the device
// address looked up once per device below.
static __device__ __align__(256) unsigned char scratch[DMTP_SCRATCH_BYTES];

std::atomic<void*> g_scratch_ptr[64];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array, or nullptr.
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
    g_scratch_ptr[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

}  // namespace

extern "C" {

size_t dmtp_fuse_ws(const dmtp_fuse_desc* d) {
  if (validate_fuse(d) != DMTP_OK) return 0;
  return fuse_ws(d);
}

int dmtp_fuse(const dmtp_fuse_desc* d, void* ws, size_t ws_bytes, hipStream_t stream) {
  int e = validate_fuse(d);
  if (e != DMTP_OK) return e;
  const size_t need = fuse_ws(d);
  CHECK(ws_bytes >= need, DMTP_E_WORKSPACE);
  CHECK(ws != nullptr, DMTP_E_NULL);
  CHECK(((uintptr_t)ws % kAlign) == 0, DMTP_E_ALIGN);
  if ((e = check_device()) != DMTP_OK) return e;
  // at most 32 rows with bf16 weights: the norms are folded into the
  // weight-streaming GEMM (two launches)
  if (fuse_fits(*d)) return launch_status(fuse_fused(*d, ws, stream));
  uint16_t* cat = (uint16_t*)ws;   // bf16 planes [2][rows][2H]
  float* part = (float*)((char*)ws + al((size_t)d->rows * 2 * d->H * 4));
  hipError_t h = fuse_prep(*d, cat, stream);
  if (h != hipSuccess) return DMTP_E_LAUNCH;
  const bool has_res = d->res.rows || d->res.ids;
  GemmArgs g{cat, (size_t)d->rows * 2 * d->H, (size_t)2 * d->H, d->rows, d->W,
             d->w_dtype == DMTP_F32, (size_t)2 * d->H, d->H, 2 * d->H, d->out, (size_t)d->H,
             has_res ? d->out : nullptr, (size_t)d->H};
  return launch_status(gemm(g, part, stream));
}

int dmtp_fuse_noalloc(const dmtp_fuse_desc* d, hipStream_t stream) {
  int e = validate_fuse(d);
  if (e != DMTP_OK) return e;
  if (fuse_ws(d) > DMTP_SCRATCH_BYTES) return DMTP_E_SCRATCH;
  if ((e = check_device()) != DMTP_OK) return e;
  void* ws = scratch_ptr();
  if (ws == nullptr) return DMTP_E_DEVICE;
  return dmtp_fuse(d, ws, DMTP_SCRATCH_BYTES, stream);
}

size_t dmtp_block_draft_ws(const dmtp_draft_desc* d) {
  if (validate_draft(d) != DMTP_OK) return 0;
  return draft_ws(d).total;
}

int dmtp_block_draft(const dmtp_draft_desc* d, void* ws, size_t ws_bytes, hipStream_t stream) {
  int e = validate_draft(d);
  if (e != DMTP_OK) return e;
  const Stack st = stack_of(d);
  const DraftWs w = stack_ws(st);
  CHECK(ws_bytes >= w.total, DMTP_E_WORKSPACE);
  CHECK(ws != nullptr, DMTP_E_NULL);
  CHECK(((uintptr_t)ws % kAlign) == 0, DMTP_E_ALIGN);
  if ((e = check_device()) != DMTP_OK) return e;
  char* b = (char*)ws;
  float* X = (float*)(b + w.X);
  uint16_t* xh = (uint16_t*)(b + w.xh);
  // the slots and their RMSNorm for the first layer; later layers get theirs
  // from the previous layer's residual update
  hipError_t h = build_slots(*d, X, d->layers[0].g_attn, xh, stream);
  SplitOut last{};
  if (h == hipSuccess) h = run_stack(st, w, b, nullptr, nullptr, &last, stream);
  if (h == hipSuccess)
    h = final_norm_mask(last, d->g_final, d->eps, d->B, st.S, d->n_anchor, d->K, d->H, d->dtype,
                        d->out, stream);
  return launch_status(h);
}

size_t dmtp_mtp_block_ws(const dmtp_mtp_desc* d) {
  if (validate_mtp(d) != DMTP_OK) return 0;
  return stack_ws(stack_of(d)).total;
}

int dmtp_mtp_block(const dmtp_mtp_desc* d, void* ws, size_t ws_bytes, hipStream_t stream) {
  int e = validate_mtp(d);
  if (e != DMTP_OK) return e;
  const Stack st = stack_of(d);
  const DraftWs w = stack_ws(st);
  CHECK(ws_bytes >= w.total, DMTP_E_WORKSPACE);
  CHECK(ws != nullptr, DMTP_E_NULL);
  CHECK(((uintptr_t)ws % kAlign) == 0, DMTP_E_ALIGN);
  if ((e = check_device()) != DMTP_OK) return e;
  char* b = (char*)ws;
  float* X = (float*)(b + w.X);
  uint16_t* xh = (uint16_t*)(b + w.xh);
  const int R = d->B * d->S;
  // X = x and the first layer's norm planes in one pass
  hipError_t h = residual_rmsnorm(split_out_plain(d->x, (size_t)d->H, R, d->H), X, (size_t)d->H, 1,
                                  d->layers[0].g_attn, d->eps, xh, R, d->H, stream);
  SplitOut last{};
  if (h == hipSuccess) h = run_stack(st, w, b, d->k_new, d->v_new, &last, stream);
  if (h == hipSuccess) h = finish_rows(last, d->out, (size_t)d->H, R, d->H, stream);
  return launch_status(h);
}

size_t dmtp_ctx_kv_ws(const dmtp_ctx_desc* d) {
  if (validate_ctx(d) != DMTP_OK) return 0;
  return ctx_ws(d).total;
}

int dmtp_ctx_kv(const dmtp_ctx_desc* d, void* ws, size_t ws_bytes, hipStream_t stream) {
  int e = validate_ctx(d);
  if (e != DMTP_OK) return e;
  const CtxWs w = ctx_ws(d);
  CHECK(ws_bytes >= w.total, DMTP_E_WORKSPACE);
  CHECK(ws != nullptr, DMTP_E_NULL);
  CHECK(((uintptr_t)ws % kAlign) == 0, DMTP_E_ALIGN);
  if ((e = check_device()) != DMTP_OK) return e;
  char* b = (char*)ws;
  uint16_t* planes = (uint16_t*)(b + w.planes);
  float* c = d->ctx_out ? d->ctx_out : (float*)(b + w.c);
  uint16_t* xh = (uint16_t*)(b + w.xh);
  float* kv = (float*)(b + w.kv);
  float* gws = (float*)(b + w.gemm);
  const int N = d->N, H = d->H, KF = d->n_feat * d->H, nkv = 2 * d->Hkv * d->d;
  const int wf32 = d->dtype == DMTP_F32;
  hipError_t h = hipSuccess;
  // the projection's split-K partials are added by the first layer's norm,
  // which also writes the finished rows to c; the K/V projection rotates and
  // scatters in its own epilogue (three launches for one layer), or, where it
  // cannot, the cache scatter adds its partials
  SplitOut sc{};
  if (wf32) {
    // float32 features and weights: the two-plane product
    h = to_planes(d->feats, d->dtype, (size_t)N * KF, planes, stream);
    if (h == hipSuccess) {
      GemmArgs g{planes, (size_t)N * KF, (size_t)KF, N, d->w_fc, wf32, (size_t)KF, H, KF, c,
                 (size_t)H, nullptr, 0};
      h = gemm_deferred(g, gws, stream, &sc);
    }
  } else {
    // bf16 features enter the projection as they are (one plane)
    GemmArgs g{(const uint16_t*)d->feats, 0, (size_t)KF, N, d->w_fc, wf32, (size_t)KF, H, KF, c,
               (size_t)H, nullptr, 0};
    g.a_planes = 1;
    h = gemm_deferred(g, gws, stream, &sc);
  }
  for (int l = 0; l < d->n_layers && h == hipSuccess; ++l) {
    const dmtp_layer& L = d->layers[l];
    // RMSNorm(c; g_attn) as planes; the first layer finishes c itself
    const int finish_c = l == 0 && sc.splits > 1;
    if ((h = residual_rmsnorm(l == 0 ? sc : split_out_plain(c, (size_t)H, N, H), finish_c ? c : nullptr,
                              (size_t)H, finish_c, L.g_attn, d->eps, xh, N, H, stream)) != hipSuccess)
      break;
    const char* wkv = (const char*)L.wqkv + (size_t)d->Hq * d->d * H * esize(d->dtype);
    GemmArgs g{xh, (size_t)N * H, (size_t)H, N, wkv, wf32, (size_t)H, nkv, H, kv, (size_t)nkv,
               nullptr, 0};
    // bf16 weights: the K/V GEMM's epilogue rotates and scatters (no split);
    // otherwise the scatter adds the split product's partials itself
    h = gemm_rope_scatter(g, d->positions, d->dst_rows, d->Hkv, d->d, d->rope_base, d->dtype,
                          d->ctx_rows, d->k_cache[l], d->v_cache[l], stream);
    if (h != hipErrorNotSupported) continue;
    SplitOut skv{};
    if ((h = gemm_deferred(g, gws, stream, &skv)) != hipSuccess) break;
    h = rope_scatter(skv, d->positions, d->dst_rows, N, d->Hkv, d->d, d->rope_base, d->dtype,
                     d->ctx_rows, d->k_cache[l], d->v_cache[l], stream);
  }
  return launch_status(h);
}

size_t dmtp_lm_head_ws(const dmtp_head_desc* d) {
  int M = 0;
  if (validate_head(d, &M) != DMTP_OK) return 0;
  return lm_head_ws_bytes(*d, M);
}

int dmtp_lm_head(const dmtp_head_desc* d, void* ws, size_t ws_bytes, hipStream_t stream) {
  int M = 0;
  int e = validate_head(d, &M);
  if (e != DMTP_OK) return e;
  CHECK(ws_bytes >= lm_head_ws_bytes(*d, M), DMTP_E_WORKSPACE);
  CHECK(ws != nullptr, DMTP_E_NULL);
  CHECK(((uintptr_t)ws % kAlign) == 0, DMTP_E_ALIGN);
  if ((e = check_device()) != DMTP_OK) return e;
  return launch_status(lm_head_run(*d, M, ws, stream));
}

size_t dmtp_head_pack_bytes(int32_t V, int32_t H) {
  if (V < 2 || V > (1 << 26) || H < 64 || H > 16384 || H % 64 != 0) return 0;
  return head_pack_bytes(V, H);
}

int dmtp_head_pack(const void* W, int32_t V, int32_t H, int32_t dtype, void* out, size_t out_bytes,
                   hipStream_t stream) {
  CHECK(W != nullptr && out != nullptr, DMTP_E_NULL);
  CHECK(V >= 2 && V <= (1 << 26) && H >= 64 && H <= 16384 && H % 64 == 0, DMTP_E_SHAPE);
  CHECK(dtype == DMTP_BF16, DMTP_E_DTYPE);
  CHECK(aligned16(W) && aligned16(out), DMTP_E_ALIGN);
  CHECK(out_bytes >= head_pack_bytes(V, H), DMTP_E_WORKSPACE);
  int e = check_device();
  if (e != DMTP_OK) return e;
  return launch_status(head_pack_run(W, V, H, out, stream));
}

size_t dmtp_verify_ws(const dmtp_verify_desc* d) {
  if (validate_verify(d) != DMTP_OK) return 0;
  return verify_ws_bytes(*d);
}

int dmtp_verify(const dmtp_verify_desc* d, void* ws, size_t ws_bytes, hipStream_t stream) {
  int e = validate_verify(d);
  if (e != DMTP_OK) return e;
  CHECK(ws_bytes >= verify_ws_bytes(*d), DMTP_E_WORKSPACE);
  CHECK(ws != nullptr, DMTP_E_NULL);
  CHECK(((uintptr_t)ws % kAlign) == 0, DMTP_E_ALIGN);
  if ((e = check_device()) != DMTP_OK) return e;
  return launch_status(verify_run(*d, ws, stream));
}

int dmtp_accept_stats(const dmtp_stats_desc* d, hipStream_t stream) {
  int e = validate_stats(d);
  if (e != DMTP_OK) return e;
  if ((e = check_device()) != DMTP_OK) return e;
  return launch_status(accept_stats_run(*d, stream));
}

const char* dmtp_status_str(int s) {
  switch (s) {
    case DMTP_OK: return "ok";
    case DMTP_E_NULL: return "a required pointer is NULL";
    case DMTP_E_SHAPE: return "a size is outside the supported range";
    case DMTP_E_DTYPE: return "unsupported dtype";
    case DMTP_E_WORKSPACE: return "workspace smaller than the *_ws() query";
    case DMTP_E_ALIGN: return "pointer not aligned (16 bytes; workspace 256 bytes)";
    case DMTP_E_DEVICE: return "current device is not gfx950";
    case DMTP_E_LAUNCH: return "kernel launch failed";
    case DMTP_E_ARG: return "inconsistent arguments";
    case DMTP_E_SCRATCH: return "needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

const char* dmtp_version(void) { return "dmtp 0.8.0 (gfx950, ABI 8)"; }

size_t dmtp_struct_size(int which) {
  switch (which) {
    case 0: return sizeof(dmtp_rows);
    case 1: return sizeof(dmtp_fuse_desc);
    case 2: return sizeof(dmtp_layer);
    case 3: return sizeof(dmtp_draft_desc);
    case 4: return sizeof(dmtp_head_segment);
    case 5: return sizeof(dmtp_head_desc);
    case 6: return sizeof(dmtp_verify_desc);
    case 7: return sizeof(dmtp_stats_desc);
    case 8: return sizeof(dmtp_mtp_desc);
    case 9: return sizeof(dmtp_ctx_desc);
    default: return 0;
  }
}

}  // extern "C"

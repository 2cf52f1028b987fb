// C ABI of the speculation-step library: context, workspace, argument checks
// and the fixed launch sequence of each entry point.  The host only enqueues
// work on the caller's stream; nothing here reads device data back, so every
// entry point can be captured in a HIP graph.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/spec.h"
#include "kernels.h"
#include "launch.h"

using namespace spec;

namespace spec {
thread_local LaunchTiming* launch_timing = nullptr;
}  // namespace spec

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Workspace {
  // activations (storage type)
  void *g, *c, *q, *o, *h1, *mn, *s, *hout[2], *nrm, *lowrank;
  // float32 buffers
  float *logits, *P, *attn_part, *cand_logits, *logp;
  void *topk_part, *verify_part;
  // int buffers
  int *ids, *cand_ids;
  int *tr_tok, *tr_par, *tr_slot, *tr_src, *tr_active, *tr_beam;
  float* tr_score;
  int *row_tok, *row_pos, *row_slot, *row_src, *row_anc;
};

}  // namespace

struct spec_ctx {
  spec_config cfg;
  bool bf16;
  int esz;
  int m_max;        // rows of one pass
  int r_max;        // rows per sequence in one pass
  int anc_w;        // width of the per-row extra-slot lists built by build_tree
  int cmax;         // candidates per sequence
  int att_nch, att_chunk;
  size_t p_floats, attn_floats, topk_bytes, verify_bytes;
  int verify_nch_max;
  void* base = nullptr;
  size_t bytes = 0;
  Workspace ws;
  std::string err;
  // kernel timing (spec_profile_*)
  bool prof = false;
  static constexpr int kProfCap = 4096;
  std::vector<hipEvent_t> ev[SPEC_PROF_NLABELS][2];
  int used[SPEC_PROF_NLABELS] = {};
};

namespace {

spec_status fail(spec_ctx* c, spec_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (c) c->err = buf;
  return st;
}

#define SPEC_HIP(ctx, expr)                                                                  \
  do {                                                                                       \
    hipError_t e_ = (expr);                                                                  \
    if (e_ != hipSuccess)                                                                    \
      return fail(ctx, SPEC_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));            \
  } while (0)

#define SPEC_REQ(ctx, cond, code, ...) \
  do {                                 \
    if (!(cond)) return fail(ctx, code, __VA_ARGS__); \
  } while (0)

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Times one labelled launch sequence when profiling is on: the kernels
// enqueued inside the scope carry the start/stop events in their dispatch
// packets (SPEC_LAUNCH); a scope that enqueued nothing records both events
// directly.
struct ProfScope {
  spec_ctx* c;
  int label;
  int slot = -1;
  hipStream_t s;
  LaunchTiming lt{nullptr, nullptr};
  LaunchTiming* prev = nullptr;
  ProfScope(spec_ctx* c_, int label_, hipStream_t s_) : c(c_), label(label_), s(s_) {
    if (c->prof && c->used[label] < spec_ctx::kProfCap) {
      slot = c->used[label]++;
      lt = {c->ev[label][0][slot], c->ev[label][1][slot]};
      prev = launch_timing;
      launch_timing = &lt;
    }
  }
  ~ProfScope() {
    if (slot < 0) return;
    launch_timing = prev;
    if (lt.start) {
      (void)hipEventRecord(lt.start, s);
      (void)hipEventRecord(lt.stop, s);
    }
  }
};

struct GemmShape {
  int N, K;
};

// Largest split-partial buffer any GEMM of the pass needs at any row count.
size_t max_partials(const spec_config& c, bool bf16, int m_max, int m_root) {
  const int H = c.hidden, I = c.intermediate, nqd = c.n_q_heads * c.head_dim;
  const int qkvN = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  GemmShape shapes[] = {{H, 3 * H}, {qkvN, 2 * H}, {qkvN, H}, {H, nqd}, {2 * I, H}, {H, I},
                        {c.cand_rank ? c.cand_rank : 1, H}, {c.cand_rank ? c.vocab : c.draft_vocab, H}};
  size_t best = 0;
  for (int M = 1; M <= std::max(m_max, m_root); ++M) {
    for (const auto& sh : shapes) {
      const GemmPlan p = gemm_plan(M, sh.N, sh.K, bf16);
      best = std::max(best, (size_t)p.nsplit * M * sh.N);
    }
  }
  return best;
}

}  // namespace

extern "C" {

const char* spec_version(void) { return "spec_mi355x 0.1 (gfx950)"; }

// Message of the last failed context-free call on this thread.
static thread_local std::string g_static_err = "no error";

const char* spec_last_error(const spec_ctx* ctx) { return ctx ? ctx->err.c_str() : g_static_err.c_str(); }

int64_t spec_workspace_bytes(const spec_ctx* ctx) { return ctx ? (int64_t)ctx->bytes : 0; }

spec_status spec_create(const spec_config* cfg_in, spec_ctx** out) {
  if (!cfg_in || !out) return SPEC_EINVAL;
  *out = nullptr;
  const spec_config c = *cfg_in;
  if (c.dtype != SPEC_F32 && c.dtype != SPEC_BF16) return SPEC_EINVAL;
  const bool bf16 = c.dtype == SPEC_BF16;
  if (c.hidden <= 0 || c.n_q_heads <= 0 || c.n_kv_heads <= 0 || c.intermediate <= 0 ||
      c.vocab <= 0 || c.draft_vocab <= 0 || c.draft_vocab > c.vocab || c.top_k <= 0 ||
      c.depth <= 0 || c.total_tokens <= 0 || c.max_batch <= 0 || c.max_new <= 0 ||
      c.kv_capacity <= 0 || c.sliding_window < 0 || c.n_q_heads % c.n_kv_heads)
    return SPEC_EINVAL;
  const int G = c.n_q_heads / c.n_kv_heads;
  const int r_max = std::max(c.max_new, c.top_k);
  const int kmul = bf16 ? 32 : 4;
  if ((c.head_dim != 64 && c.head_dim != 128) || c.top_k > 16 || c.total_tokens + 1 > 64 ||
      c.depth > c.total_tokens || G > (bf16 ? 32 : 64) || r_max > 64 || c.hidden % kmul ||
      c.intermediate % kmul || (c.n_q_heads * c.head_dim) % kmul || c.max_new > 64 ||
      c.hidden > (bf16 ? 8192 : 4096))
    return SPEC_EUNSUPPORTED;
  if (c.cand_rank) {
    if (c.cand_rank % kmul || c.num_candidates <= 0 || c.num_candidates > 256 ||
        c.num_candidates > c.vocab || c.num_candidates < c.top_k || c.draft_vocab != c.vocab)
      return SPEC_EUNSUPPORTED;
  }
  const int cmax = c.top_k + (c.depth - 1) * c.top_k * c.top_k;
  if (cmax > 4096) return SPEC_EUNSUPPORTED;

  spec_ctx* ctx = new spec_ctx();
  ctx->cfg = c;
  ctx->bf16 = bf16;
  ctx->esz = bf16 ? 2 : 4;
  ctx->r_max = r_max;
  ctx->m_max = c.max_batch * r_max;
  ctx->anc_w = c.max_new + c.depth;
  ctx->cmax = cmax;
  const int M = ctx->m_max;
  const int H = c.hidden, I = c.intermediate, nqd = c.n_q_heads * c.head_dim;
  const int Vz = c.cand_rank ? c.vocab : c.draft_vocab;  // width of the score rows
  const size_t e = ctx->esz;

  ctx->p_floats = max_partials(c, bf16, M, c.max_batch * c.max_new);
  attn_plan(c.max_batch, c.n_kv_heads, c.kv_capacity, c.sliding_window, &ctx->att_nch,
            &ctx->att_chunk);
  ctx->attn_floats = attn_part_floats(c.max_batch, c.n_kv_heads, r_max, c.n_q_heads, c.head_dim,
                                      ctx->att_nch);
  size_t tk = 0;
  const int nmax = std::max(std::max(c.vocab, c.draft_vocab), 256);
  for (int m = 1; m <= M; ++m) {
    int nch, ch;
    topk_plan(m, nmax, &nch, &ch);
    tk = std::max(tk, topk_part_bytes(m, nch, 16));
    // records of the fused LM-head top-k (one per row and workgroup strip)
    const GemmPlan lp = gemm_plan(m, c.draft_vocab, H, true);
    if (bf16 && !c.cand_rank && lp.nsplit == 1 && !lp.tile)
      tk = std::max(tk, topk_part_bytes(m, gemm_strips(m, c.draft_vocab), 8));
    // strip records of the tiled LM head (one per row and 128-column strip)
    if (bf16 && !c.cand_rank && lp.nsplit == 1 && lp.tile)
      tk = std::max(tk, (size_t)m * gemm_tile_strips(c.draft_vocab) * 8);
    // EAGLE-4: strip records of the candidate scores (one per row and
    // 128-column strip, from the tiled score GEMM or the records epilogue)
    if (bf16 && c.cand_rank) tk = std::max(tk, (size_t)m * gemm_tile_strips(c.vocab) * 8);
  }
  ctx->topk_bytes = tk;
  {
    size_t vb = 0;
    for (int b = 1; b <= c.max_batch; ++b)
      vb = std::max({vb, verify_ws_bytes(verify_plan(b, c.total_tokens, c.depth, c.vocab), b,
                                         c.total_tokens),
                     sample_ws_bytes(sample_plan(b, c.vocab), b, c.total_tokens)});
    ctx->verify_bytes = vb;
  }
  const int nc = c.cand_rank ? c.num_candidates : 1;
  struct Item {
    void** ptr;
    size_t bytes;
  };
  Workspace& w = ctx->ws;
  Item items[] = {
      {&w.g, (size_t)M * H * e},
      {&w.c, (size_t)M * 2 * H * e},
      {&w.q, (size_t)M * nqd * e},
      {&w.o, (size_t)M * nqd * e},
      {&w.h1, (size_t)M * H * e},
      {&w.mn, (size_t)M * H * e},
      {&w.s, (size_t)M * I * e},
      {&w.hout[0], (size_t)M * H * e},
      {&w.hout[1], (size_t)M * H * e},
      {&w.nrm, (size_t)M * H * e},
      {&w.lowrank, (size_t)M * std::max(c.cand_rank, 1) * e},
      {(void**)&w.logits, (size_t)M * Vz * 4},
      {(void**)&w.P, ctx->p_floats * 4},
      {(void**)&w.attn_part, ctx->attn_floats * 4},
      {(void**)&w.cand_logits, (size_t)M * nc * 4},
      {(void**)&w.logp, (size_t)M * c.top_k * 4},
      {&w.topk_part, ctx->topk_bytes},
      {&w.verify_part, ctx->verify_bytes},
      {(void**)&w.ids, (size_t)M * c.top_k * 4},
      {(void**)&w.cand_ids, (size_t)M * nc * 4},
      {(void**)&w.tr_tok, (size_t)c.max_batch * cmax * 4},
      {(void**)&w.tr_par, (size_t)c.max_batch * cmax * 4},
      {(void**)&w.tr_slot, (size_t)c.max_batch * cmax * 4},
      {(void**)&w.tr_src, (size_t)c.max_batch * cmax * 4},
      {(void**)&w.tr_score, (size_t)c.max_batch * cmax * 4},
      {(void**)&w.tr_active, (size_t)c.max_batch * 4},
      {(void**)&w.tr_beam, (size_t)c.max_batch * c.top_k * 4},
      {(void**)&w.row_tok, (size_t)M * 4},
      {(void**)&w.row_pos, (size_t)M * 4},
      {(void**)&w.row_slot, (size_t)M * 4},
      {(void**)&w.row_src, (size_t)M * 4},
      {(void**)&w.row_anc, (size_t)M * ctx->anc_w * 4},
  };
  size_t total = 0;
  for (auto& it : items) total += align_up(it.bytes);
  void* base = nullptr;
  if (hipMalloc(&base, total) != hipSuccess) {
    delete ctx;
    return SPEC_ENOMEM;
  }
  ctx->base = base;
  ctx->bytes = total;
  size_t off = 0;
  for (auto& it : items) {
    *it.ptr = (char*)base + off;
    off += align_up(it.bytes);
  }
  *out = ctx;
  return SPEC_OK;
}

void spec_destroy(spec_ctx* ctx) {
  if (!ctx) return;
  for (auto& lab : ctx->ev)
    for (auto& vec : lab)
      for (hipEvent_t e : vec) (void)hipEventDestroy(e);
  if (ctx->base) (void)hipFree(ctx->base);
  delete ctx;
}

spec_status spec_profile_enable(spec_ctx* ctx, int32_t enable) {
  if (!ctx || enable < 0 || enable > 2) return SPEC_EINVAL;
  if (enable && ctx->ev[0][0].empty()) {
    for (auto& lab : ctx->ev)
      for (auto& vec : lab) {
        vec.resize(spec_ctx::kProfCap);
        for (auto& e : vec) SPEC_HIP(ctx, hipEventCreate(&e));
      }
  }
  ctx->prof = enable != 0;
  if (enable == 1)
    for (int& u : ctx->used) u = 0;
  return SPEC_OK;
}

spec_status spec_profile_read(spec_ctx* ctx, int32_t label, int32_t* launches, double* total_ms) {
  if (!ctx || label < 0 || label >= SPEC_PROF_NLABELS || !launches || !total_ms) return SPEC_EINVAL;
  double tot = 0.0;
  const int n = ctx->used[label];
  for (int i = 0; i < n; ++i) {
    SPEC_HIP(ctx, hipEventSynchronize(ctx->ev[label][1][i]));
    float ms = 0.f;
    SPEC_HIP(ctx, hipEventElapsedTime(&ms, ctx->ev[label][0][i], ctx->ev[label][1][i]));
    tot += ms;
  }
  *launches = n;
  *total_ms = tot;
  return SPEC_OK;
}

}  // extern "C"

namespace {

struct PassIO {
  int B, R, mode;
  const void* hidden;   // [M, 3H] (mode 0) or rows indexed by src (mode 1)
  const int* src;       // mode 1: hidden row of each pass row, or null
  const int *tok, *pos, *slot, *ctx_len, *anc;
  int A;
  int k_out;
  int* ids;
  float* logp;
  int ld_out;
  void* hidden_out;
  float* logits_out;     // null: workspace
  int* cand_ids_out;     // null: workspace
  float* cand_logits_out;
  // chain trees: the caller merges the fused LM head's records itself (then
  // *merge_deferred is set), and may have built this pass's prologue already
  bool defer_merge = false;
  bool* merge_deferred = nullptr;
  bool skip_prologue = false;
};

spec_status check_weights(spec_ctx* ctx, const spec_weights* w) {
  SPEC_REQ(ctx, w, SPEC_EINVAL, "null weights");
  const void* req[] = {w->fc, w->embed, w->input_norm, w->hidden_norm, w->post_attn_norm,
                       w->final_norm, w->wqkv, w->wo, w->w_gate_up, w->w_down, w->lm_head};
  for (const void* p : req) {
    SPEC_REQ(ctx, p, SPEC_EINVAL, "a required weight pointer is null");
    SPEC_REQ(ctx, aligned16(p), SPEC_EINVAL, "weights must be 16-byte aligned");
  }
  if (ctx->cfg.draft_vocab < ctx->cfg.vocab && !ctx->cfg.cand_rank)
    SPEC_REQ(ctx, w->d2t, SPEC_EINVAL, "a trimmed draft vocabulary needs d2t");
  if (ctx->cfg.fc_norm)
    SPEC_REQ(ctx, w->fc_norm && aligned16(w->fc_norm), SPEC_EINVAL,
             "fc_norm needs a 16-byte aligned fc_norm gain");
  if (ctx->cfg.cand_rank) {
    SPEC_REQ(ctx, w->cand_down && w->cand_up, SPEC_EINVAL, "candidate head factors are null");
    SPEC_REQ(ctx, aligned16(w->cand_down) && aligned16(w->cand_up), SPEC_EINVAL,
             "weights must be 16-byte aligned");
  }
  return SPEC_OK;
}

spec_status check_kv(spec_ctx* ctx, const spec_kv* kv, int B, int layers_min) {
  const spec_config& c = ctx->cfg;
  SPEC_REQ(ctx, kv && kv->k && kv->v, SPEC_EINVAL, "null KV cache");
  SPEC_REQ(ctx, kv->n_kv_heads == c.n_kv_heads && kv->head_dim == c.head_dim, SPEC_EINVAL,
           "KV cache heads/head_dim do not match the config");
  SPEC_REQ(ctx, kv->batch >= B && kv->num_layers >= layers_min && kv->slots > 0, SPEC_EINVAL,
           "KV cache too small for this call");
  SPEC_REQ(ctx, aligned16(kv->k) && aligned16(kv->v), SPEC_EINVAL, "KV must be 16-byte aligned");
  const int64_t e = ctx->esz;
  SPEC_REQ(ctx, (kv->stride_head * e) % 16 == 0 && (kv->stride_seq * e) % 16 == 0 &&
                    (kv->stride_layer * e) % 16 == 0,
           SPEC_EINVAL, "KV strides must keep 16-byte alignment");
  if (!kv->block_table) {
    SPEC_REQ(ctx, kv->stride_head >= (int64_t)kv->slots * kv->head_dim, SPEC_EINVAL,
             "KV head stride smaller than slots * head_dim");
    return SPEC_OK;
  }
  SPEC_REQ(ctx, kv->block_size > 0 && kv->max_blocks > 0 && kv->num_blocks > 0 &&
                    (int64_t)kv->max_blocks * kv->block_size == kv->slots,
           SPEC_EINVAL, "paged KV: slots must equal max_blocks * block_size");
  SPEC_REQ(ctx, kv->stride_head >= (int64_t)kv->block_size * kv->head_dim &&
                    kv->stride_seq >= (int64_t)kv->n_kv_heads * kv->stride_head,
           SPEC_EINVAL, "paged KV: block strides smaller than a block");
  SPEC_REQ(ctx, ctx->att_chunk / kv->block_size + 2 <= kAttnMaxChunkPages, SPEC_EUNSUPPORTED,
           "paged KV: block_size %d too small for attention chunks of %d keys", kv->block_size,
           ctx->att_chunk);
  return SPEC_OK;
}

KvPages kv_pages(const spec_kv* kv) {
  KvPages pg;
  if (kv->block_table) {
    pg.tbl = kv->block_table;
    pg.bs = kv->block_size;
    pg.mb = kv->max_blocks;
    pg.nblk = kv->num_blocks;
  }
  return pg;
}

// Split-K depth of a GEMM whose partials one resid_norm workgroup per row
// sums: as many H-wide float32 partials as kResidNormSplit rows of 4096 (the
// bound resid_norm_ok applies at few rows), so narrower layers split deeper.
static int resid_norm_split(int H) { return std::max(1, kResidNormSplit * 4096 / std::max(1, H)); }

spec_status run_pass(spec_ctx* ctx, const spec_weights* w, const spec_kv* kv, const PassIO& io,
                     hipStream_t s) {
  const spec_config& c = ctx->cfg;
  const bool bf = ctx->bf16;
  Workspace& ws = ctx->ws;
  const int M = io.B * io.R;
  const int H = c.hidden, I = c.intermediate, nq = c.n_q_heads, nkv = c.n_kv_heads,
            hd = c.head_dim, nqd = nq * hd;
  const int qkvN = (nq + 2 * nkv) * hd;
  float* P = ws.P;

  // S1 (initial mode): FC fusion of the aux states; S2: prologue
  if (io.mode == 0) {
    const GemmPlan p = gemm_plan(M, H, 3 * H, bf);
    SPEC_HIP(ctx, gemm(bf, io.hidden, 3 * H, w->fc, 3 * H, P, M, H, 3 * H, p, s));
    if (c.fc_norm) {  // EAGLE-3.1: the layer input is the normalised fusion
      SPEC_HIP(ctx, gemm_epilogue(bf, EPI_STORE, ws.h1, nullptr, P, p.nsplit, M, H, s));
      SPEC_HIP(ctx, rmsnorm(bf, ws.h1, w->fc_norm, c.rms_eps, M, H, ws.g, s));
    } else {
      SPEC_HIP(ctx, gemm_epilogue(bf, EPI_STORE, ws.g, nullptr, P, p.nsplit, M, H, s));
    }
    SPEC_HIP(ctx, prologue(bf, w->embed, c.vocab, io.tok, ws.g, nullptr, w->input_norm,
                           w->hidden_norm, c.rms_eps, M, H, ws.g, ws.c, s));
  } else if (!io.skip_prologue) {
    SPEC_HIP(ctx, prologue(bf, w->embed, c.vocab, io.tok, io.hidden, io.src, w->input_norm,
                           w->hidden_norm, c.rms_eps, M, H, ws.g, ws.c, s));
  }
  // S3 + S4: QKV, RoPE, K/V store
  KvView kvv{kv->k, kv->v, kv->stride_seq, kv->stride_head, kv->slots, kv_pages(kv)};
  {
    const GemmPlan p = gemm_plan(M, qkvN, 2 * H, bf);
    SPEC_HIP(ctx, gemm(bf, ws.c, 2 * H, w->wqkv, 2 * H, P, M, qkvN, 2 * H, p, s));
    SPEC_HIP(ctx, qkv_epilogue(bf, P, p.nsplit, M, nq, nkv, hd, io.pos, io.slot, io.R,
                               c.rope_base, ws.q, kvv, s));
  }
  // S5: tree-masked attention
  {
    AttnArgs a;
    a.q = ws.q;
    a.kv = kvv;
    a.ctx_len = io.ctx_len;
    a.pos = io.pos;
    a.anc = io.anc;
    a.A = io.A;
    a.B = io.B;
    a.R = io.R;
    a.nq = nq;
    a.nkv = nkv;
    a.hd = hd;
    a.window = c.sliding_window;
    a.out = ws.o;
    a.part = ws.attn_part;
    a.nchunks = ctx->att_nch;
    a.chunk = ctx->att_chunk;
    ProfScope ps(ctx, SPEC_PROF_ATTENTION, s);
    SPEC_HIP(ctx, attention(bf, a, s));
  }
  // S6: O projection + residual; S7: post-attention norm, SwiGLU MLP, residual
  // (at few rows the O and down GEMMs split K less, so that one launch per row
  // can sum the splits and take the norm)
  {
    const GemmPlan p = gemm_plan(M, H, nqd, bf, resid_norm_split(H));
    SPEC_HIP(ctx, gemm(bf, ws.o, nqd, w->wo, nqd, P, M, H, nqd, p, s));
    if (resid_norm_ok(bf, M, H, p.nsplit, P, ws.g, ws.h1, w->post_attn_norm, ws.mn)) {
      SPEC_HIP(ctx, resid_norm(bf, P, p.nsplit, M, H, ws.g, ws.h1, w->post_attn_norm, c.rms_eps,
                               ws.mn, s));
    } else {
      SPEC_HIP(ctx, gemm_epilogue(bf, EPI_RESID, ws.h1, ws.g, P, p.nsplit, M, H, s));
      SPEC_HIP(ctx, rmsnorm(bf, ws.h1, w->post_attn_norm, c.rms_eps, M, H, ws.mn, s));
    }
  }
  {
    const GemmPlan p = gemm_plan(M, 2 * I, H, bf);
    if (bf && gemm_tile_swiglu_ok(M, 2 * I, H, p)) {
      SPEC_HIP(ctx, gemm_tile_swiglu(ws.mn, H, w->w_gate_up, H, ws.s, M, 2 * I, H, p, s));
    } else {
      SPEC_HIP(ctx, gemm(bf, ws.mn, H, w->w_gate_up, H, P, M, 2 * I, H, p, s));
      SPEC_HIP(ctx, gemm_epilogue(bf, EPI_SWIGLU, ws.s, nullptr, P, p.nsplit, M, I, s));
    }
  }
  {
    const GemmPlan p = gemm_plan(M, H, I, bf, resid_norm_split(H));
    SPEC_HIP(ctx, gemm(bf, ws.s, I, w->w_down, I, P, M, H, I, p, s));
    // S8: final norm (then the LM head; S9: top-k with log-probs)
    if (resid_norm_ok(bf, M, H, p.nsplit, P, ws.h1, io.hidden_out, w->final_norm, ws.nrm)) {
      SPEC_HIP(ctx, resid_norm(bf, P, p.nsplit, M, H, ws.h1, io.hidden_out, w->final_norm,
                               c.rms_eps, ws.nrm, s));
    } else {
      SPEC_HIP(ctx, gemm_epilogue(bf, EPI_RESID, io.hidden_out, ws.h1, P, p.nsplit, M, H, s));
      SPEC_HIP(ctx, rmsnorm(bf, io.hidden_out, w->final_norm, c.rms_eps, M, H, ws.nrm, s));
    }
    if (c.norm_output)  // EAGLE-3.1: the recurrent output is the normed row
      SPEC_HIP(ctx, hipMemcpyAsync(io.hidden_out, ws.nrm, (size_t)M * H * ctx->esz,
                                   hipMemcpyDeviceToDevice, s));
  }
  if (!c.cand_rank) {
    const int Vd = c.draft_vocab;
    const GemmPlan p = gemm_plan(M, Vd, H, bf);
    const int km = io.k_out == 1 ? 1 : (io.k_out <= 8 ? 8 : 0);
    if (bf && p.nsplit == 1 && !p.tile && km) {
      // LM head with the top-k fused into its epilogue; logits only if asked for
      {
        ProfScope ps(ctx, SPEC_PROF_LM_HEAD, s);
        SPEC_HIP(ctx, gemm_lmhead_topk(ws.nrm, H, w->lm_head, H, io.logits_out, M, Vd, H, km,
                                       ws.topk_part, s));
      }
      if (io.defer_merge && km == 1) {
        *io.merge_deferred = true;
        return SPEC_OK;
      }
      ProfScope ps(ctx, SPEC_PROF_TOPK, s);
      SPEC_HIP(ctx, topk_merge_records(M, Vd, io.k_out, km, gemm_strips(M, Vd), ws.topk_part,
                                       w->d2t, io.ids, io.ld_out, io.logp, io.ld_out, s));
      return SPEC_OK;
    }
    float* z = io.logits_out ? io.logits_out : ws.logits;
    if (bf && p.tile && p.nsplit == 1 && io.k_out <= 8) {
      // tiled LM head writing per-strip (max, sum exp) records; the top-k
      // rescans only the k best strips of each row
      {
        ProfScope ps(ctx, SPEC_PROF_LM_HEAD_TILED, s);
        SPEC_HIP(ctx, gemm_tile_records(ws.nrm, H, w->lm_head, H, z, M, Vd, H, ws.topk_part, s));
      }
      ProfScope ps(ctx, SPEC_PROF_TOPK, s);
      SPEC_HIP(ctx, topk_merge_strips(z, M, Vd, io.k_out, gemm_tile_strips(Vd), 128,
                                      ws.topk_part, w->d2t, io.ids, io.ld_out, io.logp, io.ld_out,
                                      s));
      return SPEC_OK;
    }
    if (io.k_out <= 8 && (size_t)M * gemm_tile_strips(Vd) * 8 <= ctx->topk_bytes) {
      // logits with per-strip (max, sum exp) records as the partials are
      // summed; the top-k rescans only the k best strips of each row
      float* src = p.nsplit == 1 ? z : P;
      {
        ProfScope ps(ctx, SPEC_PROF_LM_HEAD, s);
        SPEC_HIP(ctx, gemm(bf, ws.nrm, H, w->lm_head, H, src, M, Vd, H, p, s, 1));
      }
      SPEC_HIP(ctx, gemm_epilogue_records(src, p.nsplit, M, Vd, z, ws.topk_part, s));
      ProfScope ps(ctx, SPEC_PROF_TOPK, s);
      SPEC_HIP(ctx, topk_merge_strips(z, M, Vd, io.k_out, gemm_tile_strips(Vd), 128,
                                      ws.topk_part, w->d2t, io.ids, io.ld_out, io.logp, io.ld_out,
                                      s));
      return SPEC_OK;
    }
    if (p.nsplit == 1) {
      ProfScope ps(ctx, SPEC_PROF_LM_HEAD, s);
      SPEC_HIP(ctx, gemm(bf, ws.nrm, H, w->lm_head, H, z, M, Vd, H, p, s, 1));
    } else {
      {
        ProfScope ps(ctx, SPEC_PROF_LM_HEAD, s);
        SPEC_HIP(ctx, gemm(bf, ws.nrm, H, w->lm_head, H, P, M, Vd, H, p, s, 1));
      }
      SPEC_HIP(ctx, gemm_epilogue(bf, EPI_F32, z, nullptr, P, p.nsplit, M, Vd, s));
    }
    int nch, ch;
    topk_plan(M, Vd, &nch, &ch);
    ProfScope ps(ctx, SPEC_PROF_TOPK, s);
    SPEC_HIP(ctx, topk(z, M, Vd, Vd, io.k_out, w->d2t, io.ids, io.ld_out, io.logp, io.ld_out,
                       ws.topk_part, nch, ch, s));
    return SPEC_OK;
  }
  // S8': EAGLE-4 candidate head
  const int V = c.vocab, r = c.cand_rank, K = c.num_candidates;
  float* sc = io.logits_out ? io.logits_out : ws.logits;
  int* cid = io.cand_ids_out ? io.cand_ids_out : ws.cand_ids;
  float* cz = io.cand_logits_out ? io.cand_logits_out : ws.cand_logits;
  {
    const GemmPlan p = gemm_plan(M, r, H, bf);
    SPEC_HIP(ctx, gemm(bf, ws.nrm, H, w->cand_down, H, P, M, r, H, p, s));
    SPEC_HIP(ctx, gemm_epilogue(bf, EPI_STORE, ws.lowrank, nullptr, P, p.nsplit, M, r, s));
  }
  {
    const GemmPlan p = gemm_plan(M, V, r, bf);
    if (bf && p.tile && p.nsplit == 1) {
      // tiled score GEMM writing every 128-column strip's maximum with the
      // scores: the retrieval then reads only the strips that can hold one
      // of the K best
      {
        ProfScope ps(ctx, SPEC_PROF_LM_HEAD, s);
        SPEC_HIP(ctx, gemm_tile_records(ws.lowrank, r, w->cand_up, r, sc, M, V, r, ws.topk_part, s));
      }
      SPEC_HIP(ctx, topk_large_strips(sc, M, V, K, ws.topk_part, gemm_tile_strips(V), cid, s));
    } else if (bf) {
      // weight-streaming score GEMM, then one pass over its output (or the
      // split-K sum) writing the strip records, so that the retrieval again
      // reads only the strips that can hold one of the K best
      if (p.nsplit == 1) {
        {
          ProfScope ps(ctx, SPEC_PROF_LM_HEAD, s);
          SPEC_HIP(ctx, gemm(bf, ws.lowrank, r, w->cand_up, r, sc, M, V, r, p, s, 1));
        }
        SPEC_HIP(ctx, gemm_epilogue_records(sc, 1, M, V, sc, ws.topk_part, s));
      } else {
        {
          ProfScope ps(ctx, SPEC_PROF_LM_HEAD, s);
          SPEC_HIP(ctx, gemm(bf, ws.lowrank, r, w->cand_up, r, P, M, V, r, p, s, 1));
        }
        SPEC_HIP(ctx, gemm_epilogue_records(P, p.nsplit, M, V, sc, ws.topk_part, s));
      }
      SPEC_HIP(ctx, topk_large_strips(sc, M, V, K, ws.topk_part, gemm_tile_strips(V), cid, s));
    } else {
      if (p.nsplit == 1) {
        ProfScope ps(ctx, SPEC_PROF_LM_HEAD, s);
        SPEC_HIP(ctx, gemm(bf, ws.lowrank, r, w->cand_up, r, sc, M, V, r, p, s, 1));
      } else {
        {
          ProfScope ps(ctx, SPEC_PROF_LM_HEAD, s);
          SPEC_HIP(ctx, gemm(bf, ws.lowrank, r, w->cand_up, r, P, M, V, r, p, s, 1));
        }
        SPEC_HIP(ctx, gemm_epilogue(bf, EPI_F32, sc, nullptr, P, p.nsplit, M, V, s));
      }
      SPEC_HIP(ctx, topk_large(sc, M, V, K, cid, nullptr, s));
    }
  }
  SPEC_HIP(ctx, gather_dot(bf, ws.nrm, w->lm_head, H, V, cid, M, K, cz, s));
  {
    int nch, ch;
    topk_plan(M, K, &nch, &ch);
    SPEC_HIP(ctx, topk_rows(cz, M, K, K, io.k_out, nullptr, cid, io.ids, io.ld_out, io.logp,
                            io.ld_out, ws.topk_part, nch, ch, s));
  }
  return SPEC_OK;
}

TreeState tree_state(spec_ctx* ctx) {
  Workspace& w = ctx->ws;
  TreeState st;
  st.tok = w.tr_tok;
  st.parent = w.tr_par;
  st.slot = w.tr_slot;
  st.src = w.tr_src;
  st.score = w.tr_score;
  st.active = w.tr_active;
  st.beam = w.tr_beam;
  st.cmax = ctx->cmax;
  return st;
}

spec_status check_tree(spec_ctx* ctx, const spec_tree* t, bool full) {
  SPEC_REQ(ctx, t && t->tokens && t->parent && t->num_nodes, SPEC_EINVAL, "null tree arrays");
  if (full)
    SPEC_REQ(ctx, t->depth && t->position && t->draft_slot && t->score && t->anc_mask,
             SPEC_EINVAL, "null tree arrays");
  return SPEC_OK;
}

TreeOut tree_out(const spec_tree* t) {
  return TreeOut{t->tokens, t->parent, t->depth, t->position, t->draft_slot, t->num_nodes,
                 t->score, t->anc_mask};
}

}  // namespace

// hipStream_t is a pointer type; the ABI takes it as void*.
#define STREAM(s) ((hipStream_t)(s))

extern "C" {

spec_status spec_draft_step(spec_ctx* ctx, const spec_weights* w, const spec_kv* draft_kv,
                            int32_t B, int32_t rows_per_seq, int32_t mode, const void* hidden_in,
                            const int32_t* tokens, const int32_t* positions, const int32_t* kv_slot,
                            const int32_t* ctx_len, const int32_t* anc_slots, int32_t anc_width,
                            int32_t k_out, int32_t* topk_ids, float* topk_logp, void* hidden_out,
                            float* logits_out, int32_t* cand_ids_out, float* cand_logits_out,
                            void* stream) {
  if (!ctx) return SPEC_EINVAL;
  spec_status st = check_weights(ctx, w);
  if (st) return st;
  st = check_kv(ctx, draft_kv, B, 1);
  if (st) return st;
  const spec_config& c = ctx->cfg;
  SPEC_REQ(ctx, B > 0 && B <= c.max_batch, SPEC_EINVAL, "B=%d outside [1, max_batch]", B);
  SPEC_REQ(ctx, rows_per_seq > 0 && rows_per_seq <= ctx->r_max, SPEC_EUNSUPPORTED,
           "rows_per_seq=%d above max(max_new, top_k)", rows_per_seq);
  SPEC_REQ(ctx, mode == 0 || mode == 1, SPEC_EINVAL, "mode must be 0 or 1");
  SPEC_REQ(ctx, k_out > 0 && k_out <= c.top_k, SPEC_EINVAL, "k_out outside [1, top_k]");
  SPEC_REQ(ctx, anc_width >= 0 && anc_width <= 64, SPEC_EUNSUPPORTED, "anc_width above 64");
  SPEC_REQ(ctx, hidden_in && aligned16(hidden_in) && hidden_out && aligned16(hidden_out) &&
                    tokens && positions && kv_slot && ctx_len && topk_ids && topk_logp &&
                    (anc_width == 0 || anc_slots),
           SPEC_EINVAL, "null or misaligned argument");
  PassIO io{};
  io.B = B;
  io.R = rows_per_seq;
  io.mode = mode;
  io.hidden = hidden_in;
  io.src = nullptr;
  io.tok = tokens;
  io.pos = positions;
  io.slot = kv_slot;
  io.ctx_len = ctx_len;
  io.anc = anc_slots;
  io.A = anc_width;
  io.k_out = k_out;
  io.ids = topk_ids;
  io.logp = topk_logp;
  io.ld_out = k_out;
  io.hidden_out = hidden_out;
  io.logits_out = logits_out;
  io.cand_ids_out = cand_ids_out;
  io.cand_logits_out = cand_logits_out;
  return run_pass(ctx, w, draft_kv, io, STREAM(stream));
}

spec_status spec_topk_logprobs(spec_ctx* ctx, int32_t M, int32_t n, const float* logits, int32_t k,
                               const int32_t* id_map, int32_t* ids_out, float* logp_out,
                               void* stream) {
  if (!ctx) return SPEC_EINVAL;
  SPEC_REQ(ctx, M > 0 && n > 0 && k > 0 && k <= 16 && k <= n, SPEC_EINVAL, "bad sizes");
  SPEC_REQ(ctx, logits && ids_out && logp_out, SPEC_EINVAL, "null argument");
  int nch, ch;
  topk_plan(M, n, &nch, &ch);
  SPEC_REQ(ctx, topk_part_bytes(M, nch, 16) <= ctx->topk_bytes, SPEC_EUNSUPPORTED,
           "M x n larger than the workspace was sized for");
  SPEC_HIP(ctx, topk(logits, M, n, n, k, id_map, ids_out, k, logp_out, k, ctx->ws.topk_part, nch,
                     ch, STREAM(stream)));
  return SPEC_OK;
}

spec_status spec_retrieve_candidates(spec_ctx* ctx, int32_t M, int32_t n, const float* scores,
                                     int32_t K, int32_t* ids_out, void* stream) {
  if (!ctx) return SPEC_EINVAL;
  SPEC_REQ(ctx, M > 0 && n > 0 && K > 0 && K <= 256 && K <= n, SPEC_EINVAL, "bad sizes");
  SPEC_REQ(ctx, scores && ids_out, SPEC_EINVAL, "null argument");
  SPEC_HIP(ctx, topk_large(scores, M, n, K, ids_out, nullptr, STREAM(stream)));
  return SPEC_OK;
}

spec_status spec_tree_from_topk(spec_ctx* ctx, int32_t B, int32_t n_new, const int32_t* in_tokens,
                                const int32_t* ctx_len, const int32_t* topk_ids,
                                const float* topk_logp, spec_tree* out, void* stream) {
  if (!ctx) return SPEC_EINVAL;
  const spec_config& c = ctx->cfg;
  SPEC_REQ(ctx, B > 0 && B <= c.max_batch && n_new > 0 && n_new <= c.max_new, SPEC_EINVAL,
           "bad B or n_new");
  SPEC_REQ(ctx, in_tokens && ctx_len && topk_ids && topk_logp, SPEC_EINVAL, "null argument");
  spec_status st = check_tree(ctx, out, true);
  if (st) return st;
  hipStream_t s = STREAM(stream);
  Workspace& w = ctx->ws;
  const int k = c.top_k, D = c.depth;
  PassRows rows{w.row_tok, w.row_pos, w.row_slot, w.row_src, w.row_anc, ctx->anc_w};
  TreeState ts = tree_state(ctx);
  SPEC_HIP(ctx, tree_root_setup(B, n_new, in_tokens, ctx_len, k, D, c.kv_capacity, ts, rows, s));
  for (int d = 1; d <= D; ++d) {
    const size_t off = (size_t)(d - 1) * B * k * k;
    SPEC_HIP(ctx, tree_expand(d, B, n_new, ctx_len, in_tokens, k, D, c.total_tokens,
                              topk_ids + off, topk_logp + off, k, k, 0, ts, rows, tree_out(out), s));
  }
  return SPEC_OK;
}

spec_status spec_tree_candidates(spec_ctx* ctx, int32_t B, int32_t* tokens, int32_t* parent,
                                 int32_t* slot, float* score, void* stream) {
  if (!ctx) return SPEC_EINVAL;
  const spec_config& c = ctx->cfg;
  SPEC_REQ(ctx, B > 0 && B <= c.max_batch, SPEC_EINVAL, "bad B");
  SPEC_REQ(ctx, tokens && parent && slot && score, SPEC_EINVAL, "null argument");
  Workspace& w = ctx->ws;
  hipStream_t s = STREAM(stream);
  const size_t n = (size_t)B * ctx->cmax * 4;  // [B, C] rows, contiguous in the workspace
  SPEC_HIP(ctx, hipMemcpyAsync(tokens, w.tr_tok, n, hipMemcpyDeviceToDevice, s));
  SPEC_HIP(ctx, hipMemcpyAsync(parent, w.tr_par, n, hipMemcpyDeviceToDevice, s));
  SPEC_HIP(ctx, hipMemcpyAsync(slot, w.tr_slot, n, hipMemcpyDeviceToDevice, s));
  SPEC_HIP(ctx, hipMemcpyAsync(score, w.tr_score, n, hipMemcpyDeviceToDevice, s));
  return SPEC_OK;
}

spec_status spec_build_tree(spec_ctx* ctx, const spec_weights* w, const spec_kv* draft_kv,
                            int32_t B, int32_t n_new, const void* aux_hidden,
                            const int32_t* in_tokens, const int32_t* ctx_len, spec_tree* out,
                            void* stream) {
  if (!ctx) return SPEC_EINVAL;
  spec_status st = check_weights(ctx, w);
  if (st) return st;
  st = check_kv(ctx, draft_kv, B, 1);
  if (st) return st;
  st = check_tree(ctx, out, true);
  if (st) return st;
  const spec_config& c = ctx->cfg;
  SPEC_REQ(ctx, B > 0 && B <= c.max_batch && n_new > 0 && n_new <= c.max_new, SPEC_EINVAL,
           "bad B or n_new");
  SPEC_REQ(ctx, n_new + c.depth <= 64, SPEC_EUNSUPPORTED,
           "n_new + depth = %d above 64 (extra keys per row)", n_new + c.depth);
  SPEC_REQ(ctx, draft_kv->slots >= c.kv_capacity, SPEC_EINVAL, "draft KV has fewer slots than kv_capacity");
  SPEC_REQ(ctx, aux_hidden && aligned16(aux_hidden) && in_tokens && ctx_len, SPEC_EINVAL,
           "null or misaligned argument");
  hipStream_t s = STREAM(stream);
  Workspace& ws = ctx->ws;
  const int k = c.top_k, D = c.depth;
  PassRows rows{ws.row_tok, ws.row_pos, ws.row_slot, ws.row_src, ws.row_anc, ctx->anc_w};
  TreeState ts = tree_state(ctx);
  SPEC_HIP(ctx, tree_root_setup(B, n_new, in_tokens, ctx_len, k, D, c.kv_capacity, ts, rows, s));
  bool pro_done = false;  // the previous chain tail built this pass's prologue
  for (int d = 1; d <= D; ++d) {
    PassIO io{};
    bool deferred = false;
    io.defer_merge = k == 1;
    io.merge_deferred = &deferred;
    io.skip_prologue = pro_done;
    io.B = B;
    io.R = d == 1 ? n_new : k;
    io.mode = d == 1 ? 0 : 1;
    io.hidden = d == 1 ? aux_hidden : ws.hout[(d - 2) & 1];
    io.src = d == 1 ? nullptr : ws.row_src;
    io.tok = ws.row_tok;
    io.pos = ws.row_pos;
    io.slot = ws.row_slot;
    io.ctx_len = ctx_len;
    io.anc = ws.row_anc;
    io.A = ctx->anc_w;
    io.k_out = k;
    io.ids = ws.ids;
    io.logp = ws.logp;
    io.ld_out = k;
    io.hidden_out = ws.hout[(d - 1) & 1];
    st = run_pass(ctx, w, draft_kv, io, s);
    if (st) return st;
    if (deferred) {
      const int M = B * io.R;
      SPEC_HIP(ctx, chain_tail(ctx->bf16, d, B, M, n_new, ctx_len, in_tokens, D, c.total_tokens,
                               c.draft_vocab, gemm_strips(M, c.draft_vocab), ws.topk_part, w->d2t,
                               ws.ids, ws.logp, ts, rows, tree_out(out), w->embed, c.vocab,
                               io.hidden_out, w->input_norm, w->hidden_norm, c.rms_eps, c.hidden,
                               ws.g, ws.c, s));
      pro_done = d < D;
    } else {
      SPEC_HIP(ctx, tree_expand(d, B, n_new, ctx_len, in_tokens, k, D, c.total_tokens, ws.ids,
                                ws.logp, k, n_new, n_new - 1, ts, rows, tree_out(out), s));
      pro_done = false;
    }
  }
  return SPEC_OK;
}

spec_status spec_verify_tree(spec_ctx* ctx, int32_t B, const spec_tree* tree,
                             const float* target_logits, int32_t mode, float temperature,
                             const float* accept_u, uint64_t seed, int32_t* out_tokens,
                             int32_t* accepted_len, int32_t* accepted_nodes, void* stream) {
  if (!ctx) return SPEC_EINVAL;
  const spec_config& c = ctx->cfg;
  spec_status st = check_tree(ctx, tree, false);
  if (st) return st;
  SPEC_REQ(ctx, B > 0 && B <= c.max_batch, SPEC_EINVAL, "bad B");
  SPEC_REQ(ctx, mode == SPEC_VERIFY_GREEDY || mode == SPEC_VERIFY_STOCHASTIC, SPEC_EINVAL,
           "bad mode");
  SPEC_REQ(ctx, target_logits && out_tokens && accepted_len && accepted_nodes, SPEC_EINVAL,
           "null argument");
  if (mode == SPEC_VERIFY_STOCHASTIC)
    SPEC_REQ(ctx, accept_u && temperature > 0.f, SPEC_EINVAL,
             "stochastic verification needs accept_u and temperature > 0");
  const VerifyPlan vp = verify_plan(B, c.total_tokens, c.depth, c.vocab);
  SPEC_REQ(ctx, verify_ws_bytes(vp, B, c.total_tokens) <= ctx->verify_bytes, SPEC_EUNSUPPORTED,
           "workspace too small");
  ProfScope ps(ctx, SPEC_PROF_VERIFY, STREAM(stream));
  SPEC_HIP(ctx, verify(B, c.total_tokens, c.depth, c.top_k, c.vocab, tree->tokens, tree->parent,
                       tree->num_nodes, target_logits, mode, temperature, accept_u, seed,
                       out_tokens, accepted_len, accepted_nodes, ctx->ws.verify_part, vp,
                       STREAM(stream)));
  return SPEC_OK;
}

spec_status spec_verify_tree_static(int32_t B, int32_t total_tokens, int32_t depth, int32_t top_k,
                                    int32_t vocab, const spec_tree* tree, const float* target_logits,
                                    int32_t mode, float temperature, const float* accept_u,
                                    uint64_t seed, int32_t* out_tokens, int32_t* accepted_len,
                                    int32_t* accepted_nodes, void* stream) {
  auto bad = [](spec_status st, const char* msg) {
    g_static_err = msg;
    return st;
  };
  if (B <= 0 || total_tokens <= 0 || depth <= 0 || depth > total_tokens || top_k <= 0 ||
      vocab <= 0)
    return bad(SPEC_EINVAL, "spec_verify_tree_static: sizes must be positive, depth <= total_tokens");
  if (total_tokens + 1 > 64 || top_k > 64)
    return bad(SPEC_EUNSUPPORTED, "spec_verify_tree_static: total_tokens + 1 and top_k must be <= 64");
  if (!tree || !tree->tokens || !tree->parent || !tree->num_nodes || !target_logits ||
      !out_tokens || !accepted_len || !accepted_nodes)
    return bad(SPEC_EINVAL, "spec_verify_tree_static: null argument");
  if (mode != SPEC_VERIFY_GREEDY && mode != SPEC_VERIFY_STOCHASTIC)
    return bad(SPEC_EINVAL, "spec_verify_tree_static: bad mode");
  if (mode == SPEC_VERIFY_STOCHASTIC && (!accept_u || !(temperature > 0.f)))
    return bad(SPEC_EINVAL,
               "spec_verify_tree_static: stochastic verification needs accept_u and temperature > 0");
  const VerifyPlan vp = verify_plan(B, total_tokens, depth, vocab);
  if (verify_ws_bytes(vp, B, total_tokens) > kStaticVerifyScratchBytes) {
    char buf[160];
    snprintf(buf, sizeof buf,
             "spec_verify_tree_static: B=%d, total_tokens=%d, vocab=%d need %zu scratch bytes "
             "(at most %zu)",
             B, total_tokens, vocab, verify_ws_bytes(vp, B, total_tokens),
             kStaticVerifyScratchBytes);
    return bad(SPEC_EUNSUPPORTED, buf);
  }
  void* ws = nullptr;
  hipError_t e = static_verify_scratch(&ws);
  if (e == hipSuccess)
    e = verify(B, total_tokens, depth, top_k, vocab, tree->tokens, tree->parent, tree->num_nodes,
               target_logits, mode, temperature, accept_u, seed, out_tokens, accepted_len,
               accepted_nodes, ws, vp, STREAM(stream));
  if (e != hipSuccess) {
    g_static_err = std::string("spec_verify_tree_static: ") + hipGetErrorString(e);
    return SPEC_EHIP;
  }
  return SPEC_OK;
}

spec_status spec_decode_metadata(spec_ctx* ctx, int32_t B, const int32_t* cu_num_scheduled_tokens,
                                 const int32_t* num_draft_tokens, int32_t* cu_num_draft_tokens,
                                 int32_t* logits_indices, int32_t* target_logits_indices,
                                 int32_t* bonus_logits_indices, void* stream) {
  if (!ctx) return SPEC_EINVAL;
  SPEC_REQ(ctx, B > 0, SPEC_EINVAL, "bad B");
  SPEC_REQ(ctx, cu_num_scheduled_tokens && num_draft_tokens && cu_num_draft_tokens &&
                    logits_indices && target_logits_indices && bonus_logits_indices,
           SPEC_EINVAL, "null argument");
  SPEC_HIP(ctx, sample_metadata(B, cu_num_scheduled_tokens, num_draft_tokens, cu_num_draft_tokens,
                                logits_indices, target_logits_indices, bonus_logits_indices,
                                STREAM(stream)));
  return SPEC_OK;
}

spec_status spec_rejection_sample(spec_ctx* ctx, int32_t B, int32_t max_spec_len,
                                  const int32_t* cu_num_draft_tokens,
                                  const int32_t* draft_token_ids, const float* logits,
                                  int32_t num_logits_rows, const int32_t* target_logits_indices,
                                  const int32_t* bonus_logits_indices, const float* temperature,
                                  const int32_t* top_k, const float* top_p, const float* uniform,
                                  uint64_t seed, int32_t* out_tokens, int32_t* num_accepted,
                                  void* stream) {
  if (!ctx) return SPEC_EINVAL;
  const spec_config& c = ctx->cfg;
  SPEC_REQ(ctx, B > 0 && B <= c.max_batch, SPEC_EINVAL, "bad B");
  SPEC_REQ(ctx, max_spec_len >= 0 && max_spec_len <= c.total_tokens, SPEC_EUNSUPPORTED,
           "max_spec_len=%d outside [0, total_tokens]", max_spec_len);
  SPEC_REQ(ctx, num_logits_rows > 0, SPEC_EINVAL, "num_logits_rows must be positive");
  SPEC_REQ(ctx, c.vocab <= (1 << 18), SPEC_EUNSUPPORTED, "vocab above 2^18");
  SPEC_REQ(ctx, cu_num_draft_tokens && logits && bonus_logits_indices && temperature &&
                    out_tokens && num_accepted,
           SPEC_EINVAL, "null argument");
  SPEC_REQ(ctx, max_spec_len == 0 || (draft_token_ids && target_logits_indices), SPEC_EINVAL,
           "null draft arrays");
  const SamplePlan sp = sample_plan(B, c.vocab);
  SPEC_REQ(ctx, sample_ws_bytes(sp, B, max_spec_len) <= ctx->verify_bytes, SPEC_EUNSUPPORTED,
           "workspace too small");
  ProfScope ps(ctx, SPEC_PROF_VERIFY, STREAM(stream));
  SPEC_HIP(ctx, rejection_sample(B, max_spec_len, c.vocab, num_logits_rows, cu_num_draft_tokens,
                                 draft_token_ids, logits, target_logits_indices,
                                 bonus_logits_indices, temperature, top_k, top_p, uniform, seed,
                                 out_tokens, num_accepted, ctx->ws.verify_part, sp,
                                 STREAM(stream)));
  return SPEC_OK;
}

spec_status spec_target_forward(spec_ctx* ctx, const spec_target_weights* tw,
                                const spec_kv* kv, int32_t B, const spec_tree* tree,
                                const int32_t* ctx_len, float* logits, void* aux_hidden,
                                void* stream) {
  if (!ctx) return SPEC_EINVAL;
  const spec_config& c = ctx->cfg;
  const bool bf = ctx->bf16;
  const int N1 = c.total_tokens + 1, L = tw ? tw->num_layers : 0;
  SPEC_REQ(ctx, tw && tw->embed && tw->final_norm && tw->lm_head && tw->layers, SPEC_EINVAL,
           "null target weights");
  SPEC_REQ(ctx, L >= 7, SPEC_EUNSUPPORTED, "the aux layers (2, L/2, L-3) need L >= 7 (L=%d)", L);
  for (int l = 0; l < L; ++l) {
    const spec_target_layer& y = tw->layers[l];
    const void* req[] = {y.attn_norm, y.wqkv, y.wo, y.mlp_norm, y.w_gate_up, y.w_down};
    for (const void* p : req)
      SPEC_REQ(ctx, p && aligned16(p), SPEC_EINVAL, "target layer %d: null or unaligned weight", l);
  }
  SPEC_REQ(ctx, B > 0 && B <= c.max_batch, SPEC_EINVAL, "bad B");
  SPEC_REQ(ctx, c.max_new >= N1 && c.sliding_window == 0 && c.draft_vocab == c.vocab &&
                    !c.cand_rank,
           SPEC_EUNSUPPORTED,
           "target forward needs max_new >= total_tokens + 1, no window, a full LM head");
  SPEC_REQ(ctx, logits && aux_hidden && ctx_len, SPEC_EINVAL, "null argument");
  spec_status st = check_tree(ctx, tree, false);
  if (st) return st;
  st = check_kv(ctx, kv, B, L);
  if (st) return st;
  SPEC_REQ(ctx, (int64_t)ctx->att_nch * ctx->att_chunk >= kv->slots, SPEC_EUNSUPPORTED,
           "target KV slots (%d) beyond the attention plan: create the context with kv_capacity "
           ">= the slots", kv->slots);
  hipStream_t s = STREAM(stream);
  Workspace& ws = ctx->ws;
  // a node's extra keys are its ancestors and itself: at most N1 of them for
  // any tree (a chain of N1 tokens, a prompt's prefill, is deeper than the
  // draft's trees); M * N1 fits the row_anc workspace since N1 <= max_new
  const int M = B * N1, A = N1;
  const int H = c.hidden, I = c.intermediate, nq = c.n_q_heads, nkv = c.n_kv_heads,
            hd = c.head_dim, nqd = nq * hd, V = c.vocab;
  const int qkvN = (nq + 2 * nkv) * hd;
  const size_t esz = ctx->esz;
  float* P = ws.P;
  SPEC_HIP(ctx, target_rows(B, N1, A, tree->tokens, tree->position, tree->num_nodes,
                            (const unsigned long long*)tree->anc_mask, ctx_len, V, kv->slots,
                            ws.row_tok, ws.row_pos, ws.row_slot, ws.row_anc, s));
  void* h = ws.hout[0];
  void* h_next = ws.hout[1];
  SPEC_HIP(ctx, gather_rows(tw->embed, ws.row_tok, M, H * (int)esz, h, s));
  const int aux_ids[3] = {2, L / 2, L - 3};
  for (int l = 0; l < L; ++l) {
    const spec_target_layer& y = tw->layers[l];
    for (int a = 0; a < 3; ++a)  // the state entering an aux layer
      if (aux_ids[a] == l)
        SPEC_HIP(ctx, hipMemcpy2DAsync((char*)aux_hidden + (size_t)a * H * esz, 3 * H * esz, h,
                                       H * esz, H * esz, M, hipMemcpyDeviceToDevice, s));
    SPEC_HIP(ctx, rmsnorm(bf, h, y.attn_norm, c.rms_eps, M, H, ws.nrm, s));
    KvView kvv{(char*)kv->k + (size_t)l * kv->stride_layer * esz,
               (char*)kv->v + (size_t)l * kv->stride_layer * esz, kv->stride_seq, kv->stride_head,
               kv->slots, kv_pages(kv)};
    {
      const GemmPlan p = gemm_plan(M, qkvN, H, bf);
      SPEC_HIP(ctx, gemm(bf, ws.nrm, H, y.wqkv, H, P, M, qkvN, H, p, s));
      SPEC_HIP(ctx, qkv_epilogue(bf, P, p.nsplit, M, nq, nkv, hd, ws.row_pos, ws.row_slot, N1,
                                 c.rope_base, ws.q, kvv, s));
    }
    {
      AttnArgs a;
      a.q = ws.q;
      a.kv = kvv;
      a.ctx_len = ctx_len;
      a.pos = ws.row_pos;
      a.anc = ws.row_anc;
      a.A = A;
      a.B = B;
      a.R = N1;
      a.nq = nq;
      a.nkv = nkv;
      a.hd = hd;
      a.window = 0;
      a.out = ws.o;
      a.part = ws.attn_part;
      a.nchunks = ctx->att_nch;
      a.chunk = ctx->att_chunk;
      ProfScope ps(ctx, SPEC_PROF_ATTENTION, s);
      SPEC_HIP(ctx, attention(bf, a, s));
    }
    {
      const GemmPlan p = gemm_plan(M, H, nqd, bf, resid_norm_split(H));
      SPEC_HIP(ctx, gemm(bf, ws.o, nqd, y.wo, nqd, P, M, H, nqd, p, s));
      if (resid_norm_ok(bf, M, H, p.nsplit, P, h, ws.h1, y.mlp_norm, ws.mn)) {
        SPEC_HIP(ctx, resid_norm(bf, P, p.nsplit, M, H, h, ws.h1, y.mlp_norm, c.rms_eps, ws.mn, s));
      } else {
        SPEC_HIP(ctx, gemm_epilogue(bf, EPI_RESID, ws.h1, h, P, p.nsplit, M, H, s));
        SPEC_HIP(ctx, rmsnorm(bf, ws.h1, y.mlp_norm, c.rms_eps, M, H, ws.mn, s));
      }
    }
    {
      const GemmPlan p = gemm_plan(M, 2 * I, H, bf);
      if (bf && gemm_tile_swiglu_ok(M, 2 * I, H, p)) {
        SPEC_HIP(ctx, gemm_tile_swiglu(ws.mn, H, y.w_gate_up, H, ws.s, M, 2 * I, H, p, s));
      } else {
        SPEC_HIP(ctx, gemm(bf, ws.mn, H, y.w_gate_up, H, P, M, 2 * I, H, p, s));
        SPEC_HIP(ctx, gemm_epilogue(bf, EPI_SWIGLU, ws.s, nullptr, P, p.nsplit, M, I, s));
      }
    }
    {
      const GemmPlan p = gemm_plan(M, H, I, bf);
      SPEC_HIP(ctx, gemm(bf, ws.s, I, y.w_down, I, P, M, H, I, p, s));
      SPEC_HIP(ctx, gemm_epilogue(bf, EPI_RESID, h_next, ws.h1, P, p.nsplit, M, H, s));
    }
    std::swap(h, h_next);
  }
  SPEC_HIP(ctx, rmsnorm(bf, h, tw->final_norm, c.rms_eps, M, H, ws.nrm, s));
  const GemmPlan p = gemm_plan(M, V, H, bf);
  ProfScope ps(ctx, SPEC_PROF_LM_HEAD, s);
  if (p.nsplit == 1) {
    SPEC_HIP(ctx, gemm(bf, ws.nrm, H, tw->lm_head, H, logits, M, V, H, p, s, 1));
  } else {
    SPEC_HIP(ctx, gemm(bf, ws.nrm, H, tw->lm_head, H, P, M, V, H, p, s, 1));
    SPEC_HIP(ctx, gemm_epilogue(bf, EPI_F32, logits, nullptr, P, p.nsplit, M, V, s));
  }
  return SPEC_OK;
}

spec_status spec_compact_kv(spec_ctx* ctx, const spec_kv* kv, int32_t B, const int32_t* tree_base,
                            const int32_t* accepted_nodes, const int32_t* accepted_len,
                            int32_t max_accept, void* stream) {
  if (!ctx) return SPEC_EINVAL;
  spec_status st = check_kv(ctx, kv, B, 1);
  if (st) return st;
  SPEC_REQ(ctx, B > 0 && tree_base && accepted_nodes && accepted_len, SPEC_EINVAL,
           "null argument");
  SPEC_REQ(ctx, max_accept > 0 && max_accept <= 64, SPEC_EUNSUPPORTED, "max_accept outside [1, 64]");
  KvFull f{kv->k, kv->v, kv->num_layers, kv->batch, kv->n_kv_heads, kv->slots, kv->head_dim,
           kv->stride_layer, kv->stride_seq, kv->stride_head, kv_pages(kv)};
  SPEC_HIP(ctx, compact(ctx->bf16, f, B, tree_base, accepted_nodes, accepted_len, max_accept,
                        STREAM(stream)));
  return SPEC_OK;
}

}  // extern "C"

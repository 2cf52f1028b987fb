/*
 * spec.h - C ABI of the MI355X speculation-step library (libspec_mi355x.so).
 *
 * One speculation step of EAGLE-3 (and its EAGLE-4 variant) on one GPU:
 *   spec_build_tree   draft side: FC fusion of the three auxiliary target
 *                     hidden states, one draft decoder layer, LM head (or the
 *                     EAGLE-4 low-rank candidate head), top-k tree expansion;
 *   spec_verify_tree  greedy longest-accepted-path or stochastic rejection
 *                     sampling against the target's logits;
 *   spec_compact_kv   move the accepted nodes' K/V next to the root.
 * Stage-level entry points expose single steps of the same path:
 *   spec_draft_step, spec_topk_logprobs, spec_retrieve_candidates,
 *   spec_tree_from_topk.
 * Target side: spec_target_forward (tree-masked target layers, logits and
 * aux states of every tree node).
 * Flat batches of variable-length draft chains with per-request sampling
 * parameters: spec_decode_metadata (index bookkeeping) and
 * spec_rejection_sample (greedy / random acceptance with temperature, top-k
 * and top-p).
 *
 * Sources: "Speculative Decoding (EAGLE3) in the vLLM Neuron Framework"
 * (sections "What is EAGLE3?", "Eagle3 Draft Model Architecture", "The
 * propose() Method", "Rejection Sampling", "KV Cache Sharing", "Design
 * Choices"); "Eaglet" (section "Approach 1: YAML Recipe": draft_top_k,
 * draft_depth, total_draft_tokens); NeMo AutoModel "eagle4" page
 * (Eagle4CandidateHeadConfig rank / num_candidates, Eagle4Config
 * sliding_window).
 *
 * Conventions for every call
 *  - All tensors are caller-owned DEVICE memory unless a parameter says host.
 *    Matrices are row-major [rows, cols]; linear weights are [out, in].
 *  - Floating tensors are float32 or bfloat16 according to spec_config.dtype
 *    ("storage type"); logits, log-probs, scores and uniforms are float32;
 *    ids, positions, slots and counts are int32.
 *  - `stream` is a hipStream_t (void* here so the header needs no HIP headers);
 *    NULL is the default stream.  Calls only enqueue work: they never
 *    allocate, free or synchronise after spec_create.
 *  - Return codes: SPEC_OK, or SPEC_EINVAL (null pointer, bad size) /
 *    SPEC_EUNSUPPORTED (a size outside the compiled limits) detected on the
 *    host before anything is launched, or SPEC_EHIP if a launch failed;
 *    spec_last_error() then holds a message.  Device-side ids and slots are
 *    preconditions; kernels clamp them so that bad values cannot fault, but
 *    results are then unspecified.
 *  - One context per stream: a context's workspace is reused by every call.
 */
#ifndef SPEC_MI355X_H
#define SPEC_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPEC_OK = 0,
  SPEC_EINVAL = -1,
  SPEC_EUNSUPPORTED = -2,
  SPEC_EHIP = -3,
  SPEC_ENOMEM = -4
} spec_status;

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;
typedef enum { SPEC_VERIFY_GREEDY = 0, SPEC_VERIFY_STOCHASTIC = 1 } spec_verify_mode;

typedef struct spec_ctx spec_ctx;

/* Shapes of the draft and of the tree; copied by spec_create.
 * Limits: head_dim in {64, 128}; n_q_heads a multiple of n_kv_heads with
 * n_q_heads/n_kv_heads <= 32 (bf16) / 64 (f32); top_k <= 16; max_new <= 64;
 * total_tokens + 1 <= 64; depth <= total_tokens (spec_build_tree further
 * needs n_new + depth <= 64);
 * hidden, intermediate, n_q_heads*head_dim and cand_rank multiples of 32 for
 * bf16 (of 4 for f32); hidden <= 8192 (bf16) / 4096 (f32);
 * top_k <= num_candidates <= 256 when cand_rank > 0. */
typedef struct spec_config {
  int32_t hidden;          /* H */
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t intermediate;    /* I: MLP width */
  int32_t vocab;           /* V: target vocabulary (embedding rows, verify width) */
  int32_t draft_vocab;     /* Vd: LM-head rows; < V for a trimmed vocabulary with d2t */
  int32_t cand_rank;       /* r of the EAGLE-4 candidate head; 0 = EAGLE-3 head */
  int32_t num_candidates;  /* K candidates kept from the low-rank scores */
  int32_t sliding_window;  /* W keys per query including itself; 0 = full causal */
  float rope_base;         /* RoPE base (rotate-half form) */
  float rms_eps;           /* RMSNorm epsilon */
  int32_t top_k;           /* draft_top_k (1 = chain) */
  int32_t depth;           /* draft_depth (chain: num_speculative_tokens) */
  int32_t total_tokens;    /* total_draft_tokens N; the tree has N+1 nodes */
  int32_t max_batch;       /* largest B any call will pass */
  int32_t max_new;         /* largest n_new (rows per sequence in the root pass) */
  int32_t kv_capacity;     /* S: draft-KV slots per sequence */
  int32_t dtype;           /* spec_dtype: storage type of weights/activations/KV */
  /* EAGLE-3.1 normalisation (AMD Quark "EAGLE-3" page, "Background: EAGLE-3
   * and EAGLE-3.1": fc_norm, norm_output; placement not stated there).
   * fc_norm != 0: the FC output of the initial pass is RMS-normalised with
   * spec_weights.fc_norm before it enters the layer (input and residual).
   * norm_output != 0: the recurrent output hidden_out is the final-normed
   * row (the LM head's input) instead of the pre-norm state. */
  int32_t fc_norm;
  int32_t norm_output;
} spec_config;

/* Draft weights (device, storage type unless stated).  The QKV rows are
 * [q heads | k heads | v heads], each head_dim wide; w_gate_up rows are
 * [gate (I) | up (I)]. */
typedef struct spec_weights {
  const void* fc;             /* [H, 3H]  fusion of the low|mid|high aux states */
  const void* embed;          /* [V, H]   token embedding */
  const void* input_norm;     /* [H]      RMSNorm gain on the embedding */
  const void* hidden_norm;    /* [H]      RMSNorm gain on the hidden input */
  const void* post_attn_norm; /* [H] */
  const void* final_norm;     /* [H] */
  const void* wqkv;           /* [(nq+2nkv)*hd, 2H] */
  const void* wo;             /* [H, nq*hd] */
  const void* w_gate_up;      /* [2I, H] */
  const void* w_down;         /* [H, I] */
  const void* lm_head;        /* [Vd, H]; with a candidate head [V, H] */
  const int32_t* d2t;         /* [Vd] draft id -> target id, or NULL when Vd == V */
  const void* cand_down;      /* [r, H]  efficient_lm_head_down_proj, or NULL */
  const void* cand_up;        /* [V, r]  efficient_lm_head, or NULL */
  const void* fc_norm;        /* [H]     RMSNorm gain on the FC output (config fc_norm), or NULL */
} spec_weights;

/* A KV cache laid out [layers][batch][n_kv_heads][slots][head_dim] in the
 * storage type; the strides (in elements) allow any layout whose rows of
 * head_dim are contiguous.  The draft KV has one layer; keys are stored
 * after RoPE. */
typedef struct spec_kv {
  void* k;
  void* v;
  int32_t num_layers;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t slots;
  int32_t head_dim;
  int64_t stride_layer;
  int64_t stride_seq;
  int64_t stride_head;
  /* Paged caches (vLLM Neuron page, "KV Cache Sharing": physical slot =
   * block_table[pos / block_size] * block_size + pos % block_size).  NULL
   * block_table: the contiguous layout above.  Otherwise k and v are pools
   * [layers][num_blocks][n_kv_heads][block_size][head_dim]; stride_seq is the
   * stride of one block, stride_head the stride of a head inside a block;
   * block_table is [batch][max_blocks] int32 on the device; slots must equal
   * max_blocks * block_size (the logical slots of a sequence).  Block ids
   * outside [0, num_blocks) are clamped.  The blocks a call writes (new
   * rows, compaction) must not be shared between sequences. */
  const int32_t* block_table;
  int32_t block_size;
  int32_t max_blocks;
  int32_t num_blocks;
} spec_kv;

/* The draft tree of each sequence, N+1 nodes; node 0 is the root (the last
 * input token), nodes 1..num_nodes are drafts in candidate order (parents
 * before children).  Unused nodes hold -1 (tokens, parent, depth, position,
 * draft_slot), 0 (score) and 0 (anc_mask). */
typedef struct spec_tree {
  int32_t* tokens;      /* [B, N+1] target-vocabulary ids */
  int32_t* parent;      /* [B, N+1] node index, -1 for the root */
  int32_t* depth;       /* [B, N+1] root 0 */
  int32_t* position;    /* [B, N+1] ctx_len + n_new - 1 + depth */
  int32_t* draft_slot;  /* [B, N+1] draft-KV slot of nodes that were expanded, else -1 */
  int32_t* num_nodes;   /* [B] drafts kept (0 when the sequence is past the capacity cutoff) */
  float* score;         /* [B, N+1] cumulative draft log-prob, root 0 */
  uint64_t* anc_mask;   /* [B, N+1] bit j set iff node j is the node, an ancestor or the root */
} spec_tree;

/* Allocate a context and its workspace (the only allocation of the library). */
spec_status spec_create(const spec_config* cfg, spec_ctx** out);
void spec_destroy(spec_ctx* ctx);
const char* spec_last_error(const spec_ctx* ctx);  /* NULL: last context-free call's error */
int64_t spec_workspace_bytes(const spec_ctx* ctx);
const char* spec_version(void);

/* One draft pass over M = B * rows_per_seq rows (vLLM Neuron page, "Eagle3
 * Draft Model Architecture": initial and recurrent forward modes).  Row r
 * belongs to sequence r / rows_per_seq.
 *   mode 0: hidden_in is [M, 3H], the concatenated low|mid|high aux states;
 *   mode 1: hidden_in is [M, H], the pre-norm state of an earlier pass.
 *   tokens[M], positions[M]: input token and RoPE position of each row;
 *   kv_slot[M]: draft-KV slot the row's K/V is written to (-1: not written);
 *   ctx_len[B]: context slots [0, ctx_len) every row of the sequence sees;
 *   anc_slots[M, anc_width]: further visible slots, -1 padded; the valid
 *     entries of a row hold consecutive positions ending at the row's own
 *     position, in order (root rows, ancestors, the row itself);
 *   with sliding_window > 0 every row's position must be >= ctx_len - 1 of
 *     its sequence (the context span of a window is planned from the
 *     context's end; tree rows always satisfy this);
 *   k_out <= top_k: outputs topk_ids[M, k_out] (target ids, d2t applied) and
 *     topk_logp[M, k_out] (float32 log-probs), ordered by (logit desc, id asc);
 *   hidden_out[M, H]: pre-norm output state (storage type);
 *   logits_out: NULL, or [M, Vd] float32 logits (EAGLE-3 head) / [M, V]
 *     low-rank scores (candidate head);
 *   cand_ids_out / cand_logits_out: NULL, or [M, num_candidates] retrieved
 *     candidate ids and their exact logits (candidate head only).
 * K/V of all rows are written before any row attends. */
spec_status spec_draft_step(spec_ctx* ctx, const spec_weights* w, const spec_kv* draft_kv,
                            int32_t B, int32_t rows_per_seq, int32_t mode, const void* hidden_in,
                            const int32_t* tokens, const int32_t* positions, const int32_t* kv_slot,
                            const int32_t* ctx_len, const int32_t* anc_slots, int32_t anc_width,
                            int32_t k_out, int32_t* topk_ids, float* topk_logp, void* hidden_out,
                            float* logits_out, int32_t* cand_ids_out, float* cand_logits_out,
                            void* stream);

/* Top-k and log-probabilities of M rows of float32 logits [M, n]:
 * ids ordered by (value desc, position asc), log-prob = z - logsumexp(row)
 * with the sum accumulated in float64; ids_out = id_map[position] when
 * id_map (device, [n]) is given, else the position.  k <= 16. */
spec_status spec_topk_logprobs(spec_ctx* ctx, int32_t M, int32_t n, const float* logits, int32_t k,
                               const int32_t* id_map, int32_t* ids_out, float* logp_out, void* stream);

/* Candidate retrieval of the EAGLE-4 head (NeMo AutoModel "eagle4" page,
 * Eagle4CandidateHeadConfig: the num_candidates best of the low-rank scores
 * are kept for exact rescoring): for each of M rows of float32 scores [M, n]
 * (device), the positions of the K best, best first by (score desc,
 * position asc), into ids_out [M, K] (device).  K <= 256 and K <= n.  Uses
 * no workspace; asynchronous on stream. */
spec_status spec_retrieve_candidates(spec_ctx* ctx, int32_t M, int32_t n, const float* scores,
                                     int32_t K, int32_t* ids_out, void* stream);

/* Tree expansion and selection with the draft given as a table: pass d
 * (1 = root), sequence b and beam rank j produce topk_ids[d-1][b][j][:] and
 * topk_logp[d-1][b][j][:] (arrays [depth, B, top_k, top_k]; the root pass
 * uses rank 0).  Same selection rule and outputs as spec_build_tree. */
spec_status spec_tree_from_topk(spec_ctx* ctx, int32_t B, int32_t n_new, const int32_t* in_tokens,
                                const int32_t* ctx_len, const int32_t* topk_ids,
                                const float* topk_logp, spec_tree* out, void* stream);

/* The candidate table that the last spec_build_tree (or spec_tree_from_topk)
 * call left in the context: the candidates the tree of total_draft_tokens is
 * selected from ("Eaglet", "Approach 1: YAML Recipe").  For sequence b and
 * candidate c, in append order (depth by depth, beam node by beam node,
 * child rank by child rank): tokens[b, c] (target ids), parent[b, c]
 * (candidate index of the parent, -1 at depth 1), slot[b, c] (the draft-KV
 * slot of a candidate that was expanded, else -1) and score[b, c]
 * (cumulative log-prob).  Arrays are [B, C] with C = top_k + (depth - 1) *
 * top_k^2; entries of sequences past the capacity cutoff are unspecified.
 * Device-to-device copies, asynchronous on stream. */
spec_status spec_tree_candidates(spec_ctx* ctx, int32_t B, int32_t* tokens, int32_t* parent,
                                 int32_t* slot, float* score, void* stream);

/* Draft side of one step for B sequences ("Eaglet": tree of draft_top_k,
 * draft_depth, total_draft_tokens; vLLM Neuron page, "The propose() Method").
 *   aux_hidden[B, n_new, 3H]: concatenated aux states of the new rows;
 *   in_tokens[B, n_new]: their (shifted) input ids; the last one is the root;
 *   ctx_len[B]: tokens already in the draft KV.
 * The root pass runs the new rows at positions/slots ctx_len + i; each of
 * the depth-1 expansion passes runs the top_k beam nodes of the previous
 * depth; the tree is the best total_tokens candidates by cumulative log-prob.
 * A sequence with ctx_len + n_new + (depth-1)*top_k > kv_capacity gets no
 * drafts and no KV writes (the page's position-aware cutoff). */
spec_status spec_build_tree(spec_ctx* ctx, const spec_weights* w, const spec_kv* draft_kv,
                            int32_t B, int32_t n_new, const void* aux_hidden,
                            const int32_t* in_tokens, const int32_t* ctx_len, spec_tree* out,
                            void* stream);

/* Verification of the trees against target logits [B, N+1, V] float32 (row
 * n = tree node n) (vLLM Neuron page, "Rejection Sampling").
 *   mode SPEC_VERIFY_GREEDY: walk from the root to the child whose token is
 *     the current node's argmax (first index on ties); emit the accepted
 *     tokens, then the argmax at the last accepted node.
 *   mode SPEC_VERIFY_STOCHASTIC: at the current node test the children in
 *     node order with Z = 1 (a node may have at most top_k children, as
 *     every tree spec_build_tree makes; accept_u has one draw per child
 *     ordinal): accept child c_i iff accept_u[b, cur, i] <=
 *     p(c_i) / Z, else Z -= p(c_i), with p = softmax(logits / temperature);
 *     if none is accepted emit argmax over non-children of
 *     l/T - log(-log U) with U from Philox4x32-10 keyed by seed and counter
 *     (v >> 2, cur, b, 0), word v & 3, U = ((x >> 8) + 0.5) * 2^-24.
 *   accept_u: [B, N+1, top_k] float32 (stochastic only, else NULL).
 * Outputs: out_tokens[B, depth+1] (-1 padded), accepted_len[B],
 * accepted_nodes[B, depth] (-1 padded). */
spec_status spec_verify_tree(spec_ctx* ctx, int32_t B, const spec_tree* tree,
                             const float* target_logits, int32_t mode, float temperature,
                             const float* accept_u, uint64_t seed, int32_t* out_tokens,
                             int32_t* accepted_len, int32_t* accepted_nodes, void* stream);

/* Allocation-free variant of spec_verify_tree, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It takes no context: the tree shape
 * (total_tokens N, depth, top_k, vocab) is passed in, and the arguments,
 * modes, outputs and results are those of spec_verify_tree.  The call
 * allocates nothing: its scratch (statistics records per node and
 * vocabulary chunk, Gumbel records, stop nodes) lives in one fixed device
 * array of 1 MiB per GPU, held until the process ends; shapes that need more
 * (about B * (N + 1) * 16 bytes plus a little, at least 32 KiB) are rejected
 * with SPEC_EUNSUPPORTED.  Every call on one GPU shares that array and may
 * overwrite what the previous call left there: calls that overlap on one
 * GPU (concurrent streams, several host threads) race and must be
 * serialised by the caller.  Errors: SPEC_EINVAL / SPEC_EUNSUPPORTED before
 * any launch, SPEC_EHIP if a launch failed; spec_last_error(NULL) returns the
 * message of the last failed context-free call on the calling thread. */
spec_status spec_verify_tree_static(int32_t B, int32_t total_tokens, int32_t depth, int32_t top_k,
                                    int32_t vocab, const spec_tree* tree, const float* target_logits,
                                    int32_t mode, float temperature, const float* accept_u,
                                    uint64_t seed, int32_t* out_tokens, int32_t* accepted_len,
                                    int32_t* accepted_nodes, void* stream);

/* Index bookkeeping of a flat batch of variable-length draft chains (vLLM
 * Neuron page, "SpecDecodeMetadata: Index Bookkeeping"): request r has
 * n_r = num_draft_tokens[r] drafts (negative counts read as 0) and logits at
 * its last n_r + 1 scheduled positions, cu_num_scheduled_tokens[r] - n_r - 1
 * + j for j = 0..n_r.  Outputs (device, caller-owned, T = sum of n_r):
 *   cu_num_draft_tokens[B]   inclusive prefix sums of n_r;
 *   logits_indices[T + B]    those positions, request by request;
 *   target_logits_indices[T] entries of logits_indices at draft positions;
 *   bonus_logits_indices[B]  the entry of each request's last position.
 * One workgroup; no host synchronisation. */
spec_status spec_decode_metadata(spec_ctx* ctx, int32_t B, const int32_t* cu_num_scheduled_tokens,
                                 const int32_t* num_draft_tokens, int32_t* cu_num_draft_tokens,
                                 int32_t* logits_indices, int32_t* target_logits_indices,
                                 int32_t* bonus_logits_indices, void* stream);

/* Rejection sampling of a flat batch (vLLM Neuron page, "Rejection
 * Sampling", CPU rejection sampler: mixed greedy / random requests with
 * per-request temperature, top-k and top-p, draft_prob = 1).
 *   cu_num_draft_tokens[B]: inclusive prefix sums of the per-request draft
 *     counts n_r (0 <= n_r <= max_spec_len <= total_tokens);
 *   draft_token_ids[T]: drafts of request r at [cu[r] - n_r, cu[r]), ids in
 *     [0, vocab) (an id outside is never accepted by a random request);
 *   logits[num_logits_rows, vocab] float32: draft j of request r is verified
 *     against row target_logits_indices[cu[r] - n_r + j], the bonus position
 *     is row bonus_logits_indices[r] (indices clamped to the rows);
 *   temperature[B]: 0 = greedy (argmax, first index on ties; top-k/top-p
 *     ignored); top_k[B] (<= 0 or >= vocab: off) and top_p[B] (>= 1: off)
 *     may be NULL (off for every request);
 *   uniform[T]: the acceptance draws; NULL makes every request greedy.
 * A random request ranks tokens by (logit desc, id asc), keeps the first
 * top_k, then the shortest prefix of those whose mass (renormalised over the
 * top-k set) reaches top_p, and samples from p_f = softmax(l / T) over the
 * kept tokens: draft j is accepted iff uniform <= p_f(draft); at the first
 * rejection the emitted token is argmax over kept v != draft of
 * l/T - log(-log U), after n_r acceptances the bonus is the same argmax at
 * the bonus row without exclusion; U from Philox4x32-10 keyed by seed with
 * counter (v >> 2, j, r, 0) (j = n_r at the bonus row), word v & 3,
 * U = ((x >> 8) + 0.5) * 2^-24.  Masses are exp(l/T - max) in float32
 * summed in float64.
 * Outputs: out_tokens[B, max_spec_len + 1] (accepted drafts, the emitted
 * token, -1 padding) and num_accepted[B].  vocab <= 2^18. */
spec_status spec_rejection_sample(spec_ctx* ctx, int32_t B, int32_t max_spec_len,
                                  const int32_t* cu_num_draft_tokens,
                                  const int32_t* draft_token_ids, const float* logits,
                                  int32_t num_logits_rows, const int32_t* target_logits_indices,
                                  const int32_t* bonus_logits_indices, const float* temperature,
                                  const int32_t* top_k, const float* top_p, const float* uniform,
                                  uint64_t seed, int32_t* out_tokens, int32_t* num_accepted,
                                  void* stream);

/* Weights of one decoder layer of a Llama-style target (device pointers,
 * storage type). */
typedef struct spec_target_layer {
  const void* attn_norm;   /* [H]  RMSNorm gain before attention */
  const void* wqkv;        /* [(nq+2nkv)*hd, H] */
  const void* wo;          /* [H, nq*hd] */
  const void* mlp_norm;    /* [H]  RMSNorm gain before the MLP */
  const void* w_gate_up;   /* [2I, H] gate rows first */
  const void* w_down;      /* [H, I] */
} spec_target_layer;

typedef struct spec_target_weights {
  const void* embed;                /* [V, H] */
  const void* final_norm;           /* [H] */
  const void* lm_head;              /* [V, H] */
  int32_t num_layers;               /* L >= 7 */
  const spec_target_layer* layers;  /* host array of L layers */
} spec_target_weights;

/* The target's verification forward over the draft trees (vLLM Neuron page:
 * "What is Speculative Decoding?" - one target pass over the original token
 * and every draft; "Auxiliary Hidden State Extraction" - the hidden states
 * entering layers (2, L/2, L-3) are captured for the draft; "KV Cache
 * Sharing").  Every node n of sequence b is one row at its tree position; it
 * writes its K/V at slot ctx_len[b] + n of every target_kv layer and attends
 * to the context slots [0, ctx_len[b]) and to the slots of its ancestors and
 * itself (anc_mask, any of its N+1 bits: the tree may be deeper than the
 * config's depth, e.g. a chain of N+1 prompt tokens); nodes past num_nodes
 * see the context only and write no K/V.  Each layer: RMSNorm, QKV of the H-wide state, RoPE, GQA attention,
 * O projection + residual, RMSNorm, SwiGLU MLP + residual; then the final
 * norm and the LM head.
 * The context's config gives the target's shapes (vocab = draft_vocab = V,
 * sliding_window 0) and the tree (total_tokens N, depth); it must be created
 * with max_new >= N + 1 (rows per sequence of the forward) and kv_capacity
 * >= the target cache's slots.  Any tree of up to 64 nodes is served (the
 * attention takes the nodes' query vectors in groups of rows).
 * Outputs: logits [B, N+1, V] float32 (the verify step's target logits) and
 * aux_hidden [B, N+1, 3H] in the storage type (low | mid | high). */
spec_status spec_target_forward(spec_ctx* ctx, const spec_target_weights* w,
                                const spec_kv* target_kv, int32_t B, const spec_tree* tree,
                                const int32_t* ctx_len, float* logits, void* aux_hidden,
                                void* stream);

/* KV compaction of the accepted path (vLLM Neuron page, "KV Cache Sharing":
 * the draft and target layers share one cache addressed by slot, so the
 * accepted tokens' rows must sit at the slots that follow the root before
 * the next step), every layer of `kv`: for each
 * sequence b and j < accepted_len[b], the row at slot tree_base[b] +
 * accepted_nodes[b, j] moves to slot tree_base[b] + 1 + j.  All rows of a
 * sequence are read before any is written, so overlapping source and
 * destination slots are safe.  accepted_nodes is [B, max_accept]. */
spec_status spec_compact_kv(spec_ctx* ctx, const spec_kv* kv, int32_t B, const int32_t* tree_base,
                            const int32_t* accepted_nodes, const int32_t* accepted_len,
                            int32_t max_accept, void* stream);

/* Kernel timing for measurement tools.  While enabled, every labelled launch
 * sequence is timed by a pair of hipEvents that its kernels record from their
 * own dispatch packets (hipExtLaunchKernel: start as the first kernel begins,
 * stop as the last one ends), so timing adds no commands to the stream; at
 * most 4096 sequences per label are kept.  enable: 1 starts timing and
 * resets the counts, 2 resumes timing and keeps them, 0 stops timing (what
 * was recorded stays readable); the event pool is created on first use (the
 * only other host-side allocation of the library).  spec_profile_read waits
 * for the recorded events and returns the number of timed sequences and their
 * summed duration in milliseconds.  Not for use under stream capture. */
typedef enum {
  SPEC_PROF_LM_HEAD = 0,    /* LM-head GEMM up to 64 rows (EAGLE-3) or low-rank score GEMM (EAGLE-4) */
  SPEC_PROF_ATTENTION = 1,  /* context attention + combine */
  SPEC_PROF_VERIFY = 2,     /* verify statistics + walk */
  SPEC_PROF_TOPK = 3,       /* vocab top-k + log-probs */
  SPEC_PROF_LM_HEAD_TILED = 4, /* LM-head GEMM of passes above 64 rows (tree beam passes) */
  SPEC_PROF_NLABELS = 5
} spec_prof_label;
spec_status spec_profile_enable(spec_ctx* ctx, int32_t enable);
spec_status spec_profile_read(spec_ctx* ctx, int32_t label, int32_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_MI355X_H */

// Internal launch interface of the speculation-step kernels (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spec {

// ---------------------------------------------------------------- GEMM
// P[split][M][N] (float32) = X[M, K] . W[N, K]^T over the split's K range.
struct GemmPlan {
  int nsplit = 1;
  int kc = 0;         // K elements per split
  bool tile = false;  // LDS-tiled kernel (beam passes, M > 64) instead of weight streaming
  int bn = 128;       // tiled kernel: weight rows per tile (128, 112 or 96)
};
// max_split caps the split-K depth of the weight-streaming kernel (M <= 64).
GemmPlan gemm_plan(int M, int N, int K, bool bf16, int max_split = 32);
// LDS-tiled GEMM for M > 64 and K % 64 == 0 (gemm_tile.hip).
bool gemm_tile_ok(int M, int K);
GemmPlan gemm_tile_plan(int M, int N, int K);
hipError_t gemm_tile(const void* X, int ldx, const void* W, int ldw, float* P, int M, int N, int K,
                     const GemmPlan& plan, hipStream_t s);
// Unsplit tiled LM head: logits z[M, N] plus one record (max, sum of
// exp(v - max)) per row and 128-column strip, float2 [M][strips], for the
// vocab top-k.
int gemm_tile_strips(int N);
// gate|up projection with the SwiGLU fused: W [gate (N/2) | up (N/2)] rows,
// Y[M][N/2] = bf16(silu(X.gate^T) * X.up^T) with no partials, where the plan
// is one unsplit launch of 96-row tiles, at most one per CU (_ok says so).
bool gemm_tile_swiglu_ok(int M, int N, int K, const GemmPlan& plan);
hipError_t gemm_tile_swiglu(const void* X, int ldx, const void* W, int ldw, void* Y, int M, int N,
                            int K, const GemmPlan& plan, hipStream_t s);
hipError_t gemm_tile_records(const void* X, int ldx, const void* W, int ldw, float* z, int M,
                             int N, int K, void* rec, hipStream_t s);
// tag 1 launches a separately named instance (the LM head and score GEMMs).
hipError_t gemm(bool bf16, const void* X, int ldx, const void* W, int ldw, float* P, int M, int N,
                int K, const GemmPlan& plan, hipStream_t s, int tag = 0);

// LM head with the vocab top-k fused into its epilogue (nsplit must be 1):
// each workgroup writes, per row, its columns' top-km list and (sum exp, max)
// record into `part` (km = 1 or 8 >= k); logits are also stored when z != null.
// Returns hipErrorInvalidValue when the shape does not run unsplit.
int gemm_strips(int M, int N);
hipError_t gemm_lmhead_topk(const void* X, int ldx, const void* W, int ldw, float* z, int M, int N,
                            int K, int km, void* part, hipStream_t s);

enum EpiOp { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_F32 = 3 };
// Sum the nsplit partials and apply the op.  EPI_SWIGLU reads 2N columns of P
// (gate | up) and writes N; EPI_F32 writes float32 sums to Y.
hipError_t gemm_epilogue(bool bf16, int op, void* Y, const void* R, const float* P, int nsplit,
                         int M, int N, hipStream_t s);
// Float32 logits z[M, N] = the sum of the nsplit partials, plus one (max, sum
// exp) record per row and 128-column strip (float2 [M][ceil(N / 128)]) for
// topk_merge_strips.  P may be z itself when nsplit == 1.
hipError_t gemm_epilogue_records(const float* P, int nsplit, int M, int N, float* z, void* rec,
                                 hipStream_t s);

// Paged KV (vLLM Neuron page, "KV Cache Sharing": the physical slot of a
// logical position is block_table[pos / block_size] * block_size + pos %
// block_size).  tbl == nullptr: contiguous caches, slot s of sequence b at
// b * stride_seq + s * hd.  Otherwise the pool holds nblk blocks of bs slots,
// stride_seq apart, and slot s of sequence b lies in block tbl[b * mb + s / bs]
// at offset s % bs; slots and block ids are clamped into the table and the
// pool, so no value in them addresses memory outside the caches.
struct KvPages {
  const int* tbl = nullptr;
  int bs = 0, mb = 0, nblk = 0;
};
__device__ __forceinline__ int64_t kv_slot_off(const KvPages& pg, int b, int s, int64_t sseq,
                                               int hd) {
  if (!pg.tbl) return (int64_t)b * sseq + (int64_t)s * hd;
  const int cap = pg.mb * pg.bs;
  s = s < 0 ? 0 : (s >= cap ? cap - 1 : s);
  const int page = s / pg.bs;
  int blk = pg.tbl[(int64_t)b * pg.mb + page];
  blk = blk < 0 ? 0 : (blk >= pg.nblk ? pg.nblk - 1 : blk);
  return (int64_t)blk * sseq + (int64_t)(s - page * pg.bs) * hd;
}

// Pages one attention chunk may touch (paged caches need att_chunk / block_size + 2
// at most this many).
constexpr int kAttnMaxChunkPages = 512;

struct KvView {
  void* k;
  void* v;
  int64_t stride_seq, stride_head;  // elements (paged: block stride, head stride in a block)
  int slots;
  KvPages pg;
};
// QKV epilogue: sum partials, round, RoPE on q and k at pos[m], store q to
// qout[M, nq, hd], k/v to the cache at (m / rows_per_seq, head, slot[m]).
hipError_t qkv_epilogue(bool bf16, const float* P, int nsplit, int M, int nq, int nkv, int hd,
                        const int* pos, const int* slot, int rows_per_seq, float rope_base,
                        void* qout, KvView kv, hipStream_t s);

// ------------------------------------------------------------- norms
// c[r] = [rms(embed[tok[r]]) * w_in | rms(g[r]) * w_hid];  g[r] = hid[src ? src[r] : r]
// is also copied to gout (the residual of the layer).
hipError_t prologue(bool bf16, const void* embed, int V, const int* tok, const void* hid,
                    const int* src, const void* w_in, const void* w_hid, float eps, int M, int H,
                    void* gout, void* cout, hipStream_t s);
// Split-K sum + residual (stored in y) and RMSNorm of the rounded rows (to
// yn) in one launch, one workgroup per row; resid_norm_ok tells whether the
// row count, shape and alignment make it the better choice (else
// gemm_epilogue + rmsnorm).
bool resid_norm_ok(bool bf16, int M, int H, int nsplit, const void* P, const void* R,
                   const void* y, const void* w, const void* yn);
// Split-K depth at which a GEMM feeding resid_norm keeps it worthwhile at few rows.
constexpr int kResidNormSplit = 8;
hipError_t resid_norm(bool bf16, const float* P, int nsplit, int M, int H, const void* R, void* y,
                      const void* w, float eps, void* yn, hipStream_t s);
hipError_t rmsnorm(bool bf16, const void* x, const void* w, float eps, int M, int H, void* y,
                   hipStream_t s);

// --------------------------------------------------------- attention
struct AttnArgs {
  const void* q;        // [M, nq, hd]
  KvView kv;
  const int* ctx_len;   // [B]
  const int* pos;       // [M]
  const int* anc;       // [M, A]
  int A;
  int B, R, nq, nkv, hd, window;
  void* out;            // [M, nq*hd]
  float* part;          // workspace
  int nchunks, chunk;
};
void attn_plan(int B, int nkv, int slots, int window, int* nchunks, int* chunk);
size_t attn_part_floats(int B, int nkv, int R, int nq, int hd, int nchunks);
hipError_t attention(bool bf16, const AttnArgs& a, hipStream_t s);

// -------------------------------------------------------------- top-k
void topk_plan(int M, int n, int* nch, int* chunk);
size_t topk_part_bytes(int M, int nch, int kmax);
// ids = id_map ? id_map[pos] : pos, logp = z - lse.
hipError_t topk(const float* z, int M, int n, int ldz, int k, const int* id_map, int* ids,
                int ldi, float* logp, int ldl, void* part, int nch, int chunk, hipStream_t s);
// As topk, with per-row ids rowmap[M, n] used as tie-break and as output ids.
hipError_t topk_rows(const float* z, int M, int n, int ldz, int k, const int* id_map,
                     const int* rowmap, int* ids, int ldi, float* logp, int ldl, void* part,
                     int nch, int chunk, hipStream_t s);
// Top-k (k <= 8) and log-probs from the strip records of gemm_tile_records
// (strip width sw = 128 columns of the logits z[M, n]).
hipError_t topk_merge_strips(const float* z, int M, int n, int k, int nstrip, int sw,
                             const void* rec, const int* id_map, int* ids, int ldi, float* logp,
                             int ldl, hipStream_t s);
// Merge of the per-strip records written by the fused LM-head GEMM (km = 1 or 8
// entries per record, layout as the topk partials): ids and log-probs per row.
hipError_t topk_merge_records(int M, int n, int k, int km, int nch, void* part, const int* id_map,
                              int* ids, int ldi, float* logp, int ldl, hipStream_t s);
// Candidate retrieval: the best K (value desc, id asc) of each row, K <= 256.
hipError_t topk_large(const float* z, int M, int n, int K, int* ids, void* part, hipStream_t s);
// The same with the maximum of every 128-column strip of each row already
// known (rec: float2 [M][nstrip], .x the maximum, as gemm_tile_records
// writes; nstrip = ceil(n / 128)): only the strips that can hold one of the
// K best are read.
hipError_t topk_large_strips(const float* z, int M, int n, int K, const void* rec, int nstrip,
                             int* ids, hipStream_t s);
// Gathered exact rescoring: out[m, j] = dot(x[m], W[ids[m, j]]) (float32 accumulate).
hipError_t gather_dot(bool bf16, const void* x, const void* W, int H, int V, const int* ids, int M,
                      int K, float* out, hipStream_t s);

// --------------------------------------------------------------- tree
struct TreeState {   // workspace arrays, per sequence CMAX candidates
  int* tok;
  int* parent;
  int* slot;
  int* src;
  float* score;
  int* active;      // [B]
  int* beam;        // [B, k] candidate index of each beam node of the current pass
  int cmax;
};
struct TreeOut {
  int* tokens; int* parent; int* depth; int* position; int* draft_slot; int* num_nodes;
  float* score; uint64_t* anc_mask;
};
struct PassRows {    // inputs of the next draft pass
  int* tok; int* pos; int* slot; int* src; int* anc; int A;
};
hipError_t tree_root_setup(int B, int n_new, const int* in_tokens, const int* ctx_len, int k, int D,
                           int cap, TreeState st, PassRows rows, hipStream_t s);
// Consume pass d's top-k (ids/logp rows of width ld), append candidates,
// select the next beam (writes `next`) or, at d == D, the final tree.
hipError_t tree_expand(int d, int B, int n_new, const int* ctx_len, const int* in_tokens, int k,
                       int D, int N, const int* ids, const float* logp, int ld, int root_stride,
                       int root_off, TreeState st, PassRows next, TreeOut out, hipStream_t s);
// Chain passes (top_k 1) whose LM head left per-strip records (km 1) in part:
// the record merge of each sequence's expanding row (ids/logp, width 1), the
// tree step, and - before the last pass - the next pass's prologue (embed,
// hid = this pass's hidden output, norms, into gout/cout), in one launch.
hipError_t chain_tail(bool bf16, int d, int B, int M, int n_new, const int* ctx_len,
                      const int* in_tokens, int D, int N, int nvocab, int nch, const void* part,
                      const int* id_map, int* ids, float* logp, TreeState st, PassRows next,
                      TreeOut out, const void* embed, int V, const void* hid, const void* w_in,
                      const void* w_hid, float eps, int H, void* gout, void* cout, hipStream_t s);

// ------------------------------------------------------------- verify
struct VerifyPlan {
  int nch, chunk;    // statistics pass: vocab chunks per node row
  int gch, gchunk;   // Gumbel pass: vocab chunks per stop row
  bool level;        // level mode: statistics only of the rows the walks reach
  int lch, lchunk;   // level mode: vocab chunks per current row
};
// Level mode is chosen when the tree's rows outweigh the D + 2 launches it
// takes.
VerifyPlan verify_plan(int B, int N, int D, int V);
size_t verify_ws_bytes(const VerifyPlan& p, int B, int N);
hipError_t verify(int B, int N, int D, int k, int V, const int* tokens, const int* parent,
                  const int* num_nodes, const float* logits, int mode, float temperature,
                  const float* accept_u, uint64_t seed, int* out_tokens, int* accepted_len,
                  int* accepted_nodes, void* ws, const VerifyPlan& p, hipStream_t s);
// Fixed device scratch of the allocation-free verification entry point (one
// copy per GPU) and its device address on the current device.
constexpr size_t kStaticVerifyScratchBytes = size_t(1) << 20;
hipError_t static_verify_scratch(void** out);

// ------------------------------------------------------------ target forward
// Rows of the target's verification forward: token, position, KV slot and
// the A-wide list of visible tree slots of every node (target.hip).
hipError_t target_rows(int B, int N1, int A, const int* tokens, const int* position,
                       const int* num_nodes, const unsigned long long* anc_mask,
                       const int* ctx_len, int V, int S, int* tok, int* pos, int* slot, int* anc,
                       hipStream_t s);
// h[m] = embed[tok[m]] (row_bytes a multiple of 16).
hipError_t gather_rows(const void* embed, const int* tok, int M, int row_bytes, void* h,
                       hipStream_t s);

// ------------------------------------------------------------ flat-batch sampling
struct SamplePlan {
  int gch, gchunk;   // Gumbel pass: vocab chunks per request's stop row
};
SamplePlan sample_plan(int B, int V);
size_t sample_ws_bytes(const SamplePlan& p, int B, int L);
hipError_t sample_metadata(int B, const int* cu_sched, const int* nd, int* cu_nd, int* logits_idx,
                           int* tgt_idx, int* bonus_idx, hipStream_t s);
hipError_t rejection_sample(int B, int L, int V, int nrows, const int* cu_nd, const int* drafts,
                            const float* logits, const int* tgt_idx, const int* bonus_idx,
                            const float* temperature, const int* top_k, const float* top_p,
                            const float* uniform, uint64_t seed, int* out_tokens,
                            int* num_accepted, void* ws, const SamplePlan& p, hipStream_t s);

// ------------------------------------------------------------ compact
struct KvFull {
  void* k; void* v; int layers; int batch; int nkv; int slots; int hd;
  int64_t stride_layer, stride_seq, stride_head;
  KvPages pg;
};
hipError_t compact(bool bf16, KvFull kv, int B, const int* base, const int* nodes,
                   const int* alen, int max_accept, hipStream_t s);

}  // namespace spec

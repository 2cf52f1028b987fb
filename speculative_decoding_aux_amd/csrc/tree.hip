// Draft-tree bookkeeping: one workgroup per sequence.
//
// Candidates of a sequence are stored in append order (depth-major, beam
// order, child rank): depth 1 at [0, k), depth d >= 2 at
// [k + (d-2) k^2, k + (d-1) k^2).  After pass d the children of that pass are
// appended with score = parent score + log-prob (float32); the beam of the
// next pass is the top-k depth-d candidates by (score desc, index asc); beam
// node j runs at position ctx + n_new - 1 + d and slot ctx + n_new + (d-1) k + j
// and sees the root rows, its ancestors' slots and its own slot.  After the
// last pass the tree is the top-N candidates by (score desc, index asc),
// emitted in index order (parents precede children; log-probs <= 0 make the
// set ancestor-closed).  A sequence past the capacity cutoff keeps only its
// root and writes no KV.
#include "common.h"
#include "kernels.h"
#include "norm_common.h"
#include "topk_common.h"
#include "topk_merge.h"

namespace spec {

namespace {

SPEC_DEV int cand_depth(int c, int k) { return c < k ? 1 : 2 + (c - k) / (k * k); }

__global__ void root_setup_kernel(int B, int n_new, const int* __restrict__ in_tokens,
                                  const int* __restrict__ ctx_len, int k, int D, int cap,
                                  int* __restrict__ active, int* __restrict__ tok,
                                  int* __restrict__ pos, int* __restrict__ slot,
                                  int* __restrict__ src, int* __restrict__ anc, int A) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= B * n_new) return;
  const int b = idx / n_new, i = idx % n_new;
  const int ctx = ctx_len[b];
  const int act = (ctx >= 0 && ctx + n_new + (D - 1) * k <= cap) ? 1 : 0;
  if (i == 0) active[b] = act;
  tok[idx] = in_tokens[idx];
  pos[idx] = ctx + i;
  slot[idx] = act ? ctx + i : -1;
  src[idx] = idx;
  for (int j = 0; j < A; ++j) anc[(int64_t)idx * A + j] = (act && j <= i) ? ctx + j : -1;
}

// Tree step of sequence b after pass d, by a 256-thread block (every thread
// calls it).  The sequence's candidate arrays are mirrored in LDS for the
// step (one coalesced read of the candidates so far), so the ancestor walks
// and the ranking read LDS, not dependent global loads; every global write
// goes to the mirror too.  Dynamic LDS: expand_lds_ints(cmax) ints.
SPEC_DEV void expand_seq(int b, int d, int n_new, const int* __restrict__ ctx_len,
                         const int* __restrict__ in_tokens, int k, int D, int N,
                         const int* __restrict__ ids, const float* __restrict__ logp, int ld,
                         int root_stride, int root_off, TreeState st, int* __restrict__ beam,
                         PassRows nx, TreeOut out) {
  extern __shared__ int sh[];
  const int t = threadIdx.x;
  const int cmax = st.cmax;
  // node_of | counts[256] | scores | parent, slot, token, source, score mirrors | beam[64]
  int* node_of = sh;
  int* counts = sh + cmax;
  float* ss = (float*)(sh + cmax + 256);
  int* lpar = sh + 2 * cmax + 256;
  int* lslot = lpar + cmax;
  int* ltok = lslot + cmax;
  int* lsrc = ltok + cmax;
  float* lsc = (float*)(lsrc + cmax);
  int* lbm = (int*)(lsc + cmax);
  int* ctok = st.tok + (int64_t)b * cmax;
  int* cpar = st.parent + (int64_t)b * cmax;
  int* cslot = st.slot + (int64_t)b * cmax;
  int* csrc = st.src + (int64_t)b * cmax;
  float* csc = st.score + (int64_t)b * cmax;
  int* bm = beam + (int64_t)b * k;
  const int act = st.active[b];
  const int ctx = ctx_len[b];
  const int K2 = k * k;

  if (act) {
    // 0. mirror the candidates of passes 1 .. d-1 and the current beam
    const int have = d == 1 ? 0 : k + (d - 2) * K2;
    for (int x = t; x < have; x += blockDim.x) {
      lpar[x] = cpar[x];
      lslot[x] = cslot[x];
      ltok[x] = ctok[x];
      lsrc[x] = csrc[x];
      lsc[x] = csc[x];
    }
    if (d > 1)
      for (int j = t; j < k; j += blockDim.x) lbm[j] = bm[j];
    __syncthreads();
    // 1. append the children produced by pass d
    if (d == 1) {
      const int row = b * root_stride + root_off;
      if (t < k) {
        const int tk = ids[(int64_t)row * ld + t];
        const float sc = logp[(int64_t)row * ld + t];
        ctok[t] = ltok[t] = tk;
        cpar[t] = lpar[t] = -1;
        cslot[t] = lslot[t] = -1;
        csrc[t] = lsrc[t] = row;
        csc[t] = lsc[t] = sc;
      }
    } else {
      for (int x = t; x < K2; x += blockDim.x) {
        const int jb = x / k, jc = x % k;
        const int row = b * k + jb;
        const int p = lbm[jb];
        const int c = have + x;
        const int tk = ids[(int64_t)row * ld + jc];
        const float sc = lsc[p] + logp[(int64_t)row * ld + jc];
        ctok[c] = ltok[c] = tk;
        cpar[c] = lpar[c] = p;
        cslot[c] = lslot[c] = -1;
        csrc[c] = lsrc[c] = row;
        csc[c] = lsc[c] = sc;
      }
    }
    __syncthreads();
  }

  if (d < D) {
    // 2. beam of the next pass among the depth-d candidates
    const int lo = d == 1 ? 0 : k + (d - 2) * K2;
    const int cnt = d == 1 ? k : K2;
    if (act) {
      for (int x = t; x < cnt; x += blockDim.x) ss[x] = lsc[lo + x];
      __syncthreads();
      for (int x = t; x < cnt; x += blockDim.x) {
        const float sc = ss[x];
        int rank = 0;
        for (int y = 0; y < cnt; ++y) rank += better(ss[y], y, sc, x) ? 1 : 0;
        if (rank < k) bm[rank] = lbm[rank] = lo + x;
      }
      __syncthreads();
    }
    for (int j = t; j < k; j += blockDim.x) {
      const int r = b * k + j;
      nx.pos[r] = ctx + n_new - 1 + d;
      if (act) {
        const int c = lbm[j];
        const int sl = ctx + n_new + (d - 1) * k + j;
        cslot[c] = sl;  // the mirror is not read again in this step
        nx.tok[r] = ltok[c];
        nx.slot[r] = sl;
        nx.src[r] = lsrc[c];
        int* a = nx.anc + (int64_t)r * nx.A;
        for (int i = 0; i < n_new; ++i) a[i] = ctx + i;
        // ancestors of a depth-d candidate sit at depths 1 .. d-1, then itself
        for (int p = lpar[c]; p >= 0; p = lpar[p]) a[n_new + cand_depth(p, k) - 1] = lslot[p];
        a[n_new + d - 1] = sl;
        int na = n_new + d;
        for (; na < nx.A; ++na) a[na] = -1;
      } else {
        nx.tok[r] = 0;
        nx.slot[r] = -1;
        nx.src[r] = d == 1 ? b * root_stride : b * k;
        int* a = nx.anc + (int64_t)r * nx.A;
        for (int i = 0; i < nx.A; ++i) a[i] = -1;
      }
    }
    return;
  }

  // 3. final selection (d == D)
  const int n1 = N + 1;
  const int ncand = act ? k + (D - 1) * K2 : 0;
  for (int c = t; c < ncand; c += blockDim.x) ss[c] = lsc[c];
  __syncthreads();
  for (int c = t; c < ncand; c += blockDim.x) {
    const float sc = ss[c];
    int rank = 0;
    for (int y = 0; y < ncand; ++y) rank += better(ss[y], y, sc, c) ? 1 : 0;
    node_of[c] = rank < N ? 1 : 0;
  }
  __syncthreads();
  // exclusive scan of the selection flags in index order
  const int seg = (ncand + blockDim.x - 1) / blockDim.x;
  int local = 0;
  for (int c = t * seg; c < min(ncand, (t + 1) * seg); ++c) local += node_of[c];
  counts[t] = local;
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int i = 0; i < (int)blockDim.x; ++i) {
      const int v = counts[i];
      counts[i] = run;
      run += v;
    }
  }
  __syncthreads();
  int next = counts[t];
  for (int c = t * seg; c < min(ncand, (t + 1) * seg); ++c) {
    if (node_of[c]) {
      node_of[c] = 1 + next;
      ++next;
    } else {
      node_of[c] = -1;
    }
  }
  __syncthreads();
  const int64_t ob = (int64_t)b * n1;
  for (int n = t; n < n1; n += blockDim.x) {
    out.tokens[ob + n] = -1;
    out.parent[ob + n] = -1;
    out.depth[ob + n] = -1;
    out.position[ob + n] = -1;
    out.draft_slot[ob + n] = -1;
    out.score[ob + n] = 0.f;
    out.anc_mask[ob + n] = 0ull;
  }
  __syncthreads();
  if (t == 0) {
    out.tokens[ob] = in_tokens[b * n_new + n_new - 1];
    out.depth[ob] = 0;
    out.position[ob] = ctx + n_new - 1;
    out.draft_slot[ob] = act ? ctx + n_new - 1 : -1;
    out.anc_mask[ob] = 1ull;
    out.num_nodes[b] = min(N, ncand);
  }
  for (int c = t; c < ncand; c += blockDim.x) {
    const int n = node_of[c];
    if (n < 0) continue;
    const int pc = lpar[c];
    const int dep = cand_depth(c, k);
    out.tokens[ob + n] = ltok[c];
    out.parent[ob + n] = pc < 0 ? 0 : node_of[pc];
    out.depth[ob + n] = dep;
    out.position[ob + n] = ctx + n_new - 1 + dep;
    out.draft_slot[ob + n] = lslot[c];
    out.score[ob + n] = lsc[c];
    uint64_t mask = 1ull | (1ull << n);
    for (int p = pc; p >= 0; p = lpar[p]) mask |= 1ull << node_of[p];
    out.anc_mask[ob + n] = mask;
  }
}

__global__ __launch_bounds__(256) void tree_expand_kernel(
    int d, int n_new, const int* __restrict__ ctx_len, const int* __restrict__ in_tokens, int k,
    int D, int N, const int* __restrict__ ids, const float* __restrict__ logp, int ld,
    int root_stride, int root_off, TreeState st, int* __restrict__ beam, PassRows nx,
    TreeOut out) {
  expand_seq(blockIdx.x, d, n_new, ctx_len, in_tokens, k, D, N, ids, logp, ld, root_stride,
             root_off, st, beam, nx, out);
}

// Row inputs of the next pass (prologue_row arguments besides tokens and
// source rows, which the tree step writes).
template <typename T>
struct ChainPrologue {
  const T* embed;
  int V;
  const T* hid;
  const T* w_in;
  const T* w_hid;
  float eps;
  int H;
  T* gout;
  T* cout;
};

// Tail of a chain pass (top_k 1), one block per sequence: merge the LM-head
// records of the sequence's expanding row into its token and log-prob, run
// the tree step, and, before the last pass, build the next pass's row input
// (the prologue) - three launches' work in one.
template <typename T>
__global__ __launch_bounds__(256) void chain_tail_kernel(
    int d, int n_new, const int* __restrict__ ctx_len, const int* __restrict__ in_tokens, int D,
    int N, int nvocab, int nch, const float* __restrict__ pv, const int* __restrict__ pi,
    const topkdev::Part* __restrict__ pp, const int* __restrict__ id_map, int* __restrict__ ids,
    float* __restrict__ logp, TreeState st, int* __restrict__ beam, PassRows nx, TreeOut out,
    ChainPrologue<T> pro) {
  const int b = blockIdx.x;
  const int row = d == 1 ? b * n_new + n_new - 1 : b;
  topkdev::merge_row<1>(row, nvocab, 1, nch, pv, pi, pp, id_map, nullptr, ids, 1, logp, 1);
  __syncthreads();  // the row's id and log-prob (global, this block) are visible
  expand_seq(b, d, n_new, ctx_len, in_tokens, 1, D, N, ids, logp, 1, n_new, n_new - 1, st, beam,
             nx, out);
  if (d >= D) return;
  __syncthreads();  // the next pass's row inputs (global, this block) are visible
  normdev::prologue_row<T>(b, pro.embed, pro.V, nx.tok, pro.hid, nx.src, pro.w_in, pro.w_hid,
                           pro.eps, pro.H, pro.gout, pro.cout);
}

// Chain pass d < D (top_k 1), one block per sequence.  In a chain the
// depth-d candidate is index d - 1 and the only beam node, its slot is
// ctx + n_new + d - 1, and the slots of its ancestors follow the root rows',
// so the next row's visible slots are ctx .. ctx + n_new + d - 1: the tree
// step needs nothing back from the candidate arrays but the previous score.
// That score, the sequence state, the next row's hidden state and both norm
// weights are requested before the record merge, so they arrive with the
// records; the merged token comes through LDS.  Writes exactly what
// chain_tail_kernel writes for d < D.
template <typename T>
__global__ __launch_bounds__(256) void chain_step_kernel(
    int d, int n_new, const int* __restrict__ ctx_len, int nvocab, int nch,
    const float* __restrict__ pv, const int* __restrict__ pi, const topkdev::Part* __restrict__ pp,
    const int* __restrict__ id_map, int* __restrict__ ids, float* __restrict__ logp, TreeState st,
    int* __restrict__ beam, PassRows nx, ChainPrologue<T> pro) {
  __shared__ int bc[2];
  __shared__ double red[2][4];
  const int b = blockIdx.x, t = threadIdx.x;
  const int row = d == 1 ? b * n_new + n_new - 1 : b;
  const int act = st.active[b];
  const int ctx = ctx_len[b];
  const int c = d - 1;
  const int64_t cb = (int64_t)b * st.cmax;
  const float prev = (d > 1 && t == 0) ? st.score[cb + c - 1] : 0.f;
  const int src = act ? row : (d == 1 ? b * n_new : b);
  const int nvec = pro.H / normdev::V16<T>::N;
  u32x4_t gv[normdev::kVecPerThread], wi[normdev::kVecPerThread], wh[normdev::kVecPerThread];
  normdev::load_row<T>(pro.hid + (int64_t)src * pro.H, nvec, gv);
  normdev::load_row<T>(pro.w_in, nvec, wi);
  normdev::load_row<T>(pro.w_hid, nvec, wh);
  topkdev::merge_row<1>(row, nvocab, 1, nch, pv, pi, pp, id_map, nullptr, ids, 1, logp, 1, bc);
  __syncthreads();  // bc holds the row's token and log-prob
  const int tok = bc[0];
  const float lp = __int_as_float(bc[1]);
  const int sl = ctx + n_new + d - 1;
  if (t == 0) {
    if (act) {
      st.tok[cb + c] = tok;
      st.parent[cb + c] = d == 1 ? -1 : c - 1;
      st.slot[cb + c] = sl;
      st.src[cb + c] = row;
      st.score[cb + c] = d == 1 ? lp : prev + lp;
      beam[b] = c;
    }
    nx.pos[b] = ctx + n_new - 1 + d;
    nx.tok[b] = act ? tok : 0;
    nx.slot[b] = act ? sl : -1;
    nx.src[b] = src;
  }
  for (int i = t; i < nx.A; i += 256) nx.anc[(int64_t)b * nx.A + i] = (act && i < n_new + d) ? ctx + i : -1;
  // prologue of the next pass's row b (prologue_row with the hidden state and
  // weights already in registers)
  const int te = clampi(act ? tok : 0, 0, pro.V - 1);
  u32x4_t ev[normdev::kVecPerThread];
  normdev::load_row<T>(pro.embed + (int64_t)te * pro.H, nvec, ev);
  double se = wave_sum(normdev::sumsq<T>(ev)), sg = wave_sum(normdev::sumsq<T>(gv));
  const int w = t >> 6;
  if ((t & 63) == 0) {
    red[0][w] = se;
    red[1][w] = sg;
  }
  __syncthreads();
  se = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  sg = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const double ce = 1.0 / sqrt(se / pro.H + (double)pro.eps);
  const double cg = 1.0 / sqrt(sg / pro.H + (double)pro.eps);
  T* co = pro.cout + (int64_t)b * 2 * pro.H;
  normdev::scale_store<T>(ev, ce, wi, co, nvec);
  normdev::scale_store<T>(gv, cg, wh, co + pro.H, nvec);
  T* go = pro.gout + (int64_t)b * pro.H;
  if (go != pro.hid + (int64_t)src * pro.H) {
#pragma unroll
    for (int j = 0; j < normdev::kVecPerThread; ++j) {
      const int i = t + 256 * j;
      if (i < nvec) ((u32x4_t*)go)[i] = gv[j];
    }
  }
}

}  // namespace

hipError_t tree_root_setup(int B, int n_new, const int* in_tokens, const int* ctx_len, int k, int D,
                           int cap, TreeState st, PassRows rows, hipStream_t s) {
  const int n = B * n_new;
  SPEC_LAUNCH(root_setup_kernel, dim3((n + 255) / 256), dim3(256), 0, s, B, n_new,
                     in_tokens, ctx_len, k, D, cap, st.active, rows.tok, rows.pos, rows.slot,
                     rows.src, rows.anc, rows.A);
  return hipGetLastError();
}

// Dynamic LDS of expand_seq: node_of, scores and five candidate mirrors of
// cmax entries, 256 scan counts and the beam (k <= 64).
static size_t expand_lds_bytes(int cmax) { return (size_t)(7 * cmax + 256 + 64) * sizeof(int); }

hipError_t tree_expand(int d, int B, int n_new, const int* ctx_len, const int* in_tokens, int k,
                       int D, int N, const int* ids, const float* logp, int ld, int root_stride,
                       int root_off, TreeState st, PassRows next, TreeOut out, hipStream_t s) {
  const size_t lds = expand_lds_bytes(st.cmax);
  if (k > 64 || lds > 64 * 1024) return hipErrorInvalidValue;
  SPEC_LAUNCH(tree_expand_kernel, dim3(B), dim3(256), lds, s, d, n_new, ctx_len, in_tokens,
                     k, D, N, ids, logp, ld, root_stride, root_off, st, st.beam, next, out);
  return hipGetLastError();
}

hipError_t chain_tail(bool bf16, int d, int B, int M, int n_new, const int* ctx_len,
                      const int* in_tokens, int D, int N, int nvocab, int nch, const void* part,
                      const int* id_map, int* ids, float* logp, TreeState st, PassRows next,
                      TreeOut out, const void* embed, int V, const void* hid, const void* w_in,
                      const void* w_hid, float eps, int H, void* gout, void* cout, hipStream_t s) {
  if (M != B * (d == 1 ? n_new : 1)) return hipErrorInvalidValue;
  // record layout of the fused LM head (one entry per record): pv, pi [M][nch], pp [M][nch]
  const float* pv = (const float*)part;
  const int* pi = (const int*)(pv + (size_t)M * nch);
  const topkdev::Part* pp = (const topkdev::Part*)(pi + (size_t)M * nch);
  const size_t lds = expand_lds_bytes(st.cmax);
  if (lds > 64 * 1024) return hipErrorInvalidValue;
  if (bf16) {
    const ChainPrologue<bf16_t> pro{(const bf16_t*)embed, V, (const bf16_t*)hid,
                                    (const bf16_t*)w_in, (const bf16_t*)w_hid, eps, H,
                                    (bf16_t*)gout, (bf16_t*)cout};
    if (d < D) {
      SPEC_LAUNCH(chain_step_kernel<bf16_t>, dim3(B), dim3(256), 0, s, d, n_new, ctx_len, nvocab,
                  nch, pv, pi, pp, id_map, ids, logp, st, st.beam, next, pro);
      return hipGetLastError();
    }
    SPEC_LAUNCH(chain_tail_kernel<bf16_t>, dim3(B), dim3(256), lds, s, d, n_new, ctx_len,
                in_tokens, D, N, nvocab, nch, pv, pi, pp, id_map, ids, logp, st, st.beam, next,
                out, pro);
  } else {
    const ChainPrologue<float> pro{(const float*)embed, V, (const float*)hid, (const float*)w_in,
                                   (const float*)w_hid, eps, H, (float*)gout, (float*)cout};
    if (d < D) {
      SPEC_LAUNCH(chain_step_kernel<float>, dim3(B), dim3(256), 0, s, d, n_new, ctx_len, nvocab,
                  nch, pv, pi, pp, id_map, ids, logp, st, st.beam, next, pro);
      return hipGetLastError();
    }
    SPEC_LAUNCH(chain_tail_kernel<float>, dim3(B), dim3(256), lds, s, d, n_new, ctx_len,
                in_tokens, D, N, nvocab, nch, pv, pi, pp, id_map, ids, logp, st, st.beam, next,
                out, pro);
  }
  return hipGetLastError();
}

}  // namespace spec

// Set-up kernels of the target's verification forward over the draft tree
// (vLLM Neuron page: "What is Speculative Decoding?" - the target processes
// the original token and every draft token in one pass; "KV Cache Sharing" -
// each token's K/V goes to its own slot).  One row per tree node n of
// sequence b: the node's token, its position, KV slot ctx_len[b] + n, and the
// slots of its ancestors and itself (the bits of anc_mask) as the row's extra
// visible keys; nodes past num_nodes get token 0, the context alone, and no
// K/V write.  The layers themselves run on the draft layer's kernels.
#include "common.h"
#include "kernels.h"

namespace spec {

namespace {

__global__ __launch_bounds__(256) void target_rows_kernel(
    int B, int N1, int A, const int* __restrict__ tokens, const int* __restrict__ position,
    const int* __restrict__ num_nodes, const unsigned long long* __restrict__ anc_mask,
    const int* __restrict__ ctx_len, int V, int S, int* __restrict__ tok, int* __restrict__ pos,
    int* __restrict__ slot, int* __restrict__ anc) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= B * N1) return;
  const int b = m / N1, n = m % N1;
  const int nn = clampi(num_nodes[b], 0, N1 - 1);
  const int c = clampi(ctx_len[b], 0, S);
  const bool live = n <= nn;
  tok[m] = live ? clampi(tokens[m], 0, V - 1) : 0;
  pos[m] = live ? position[m] : c;
  slot[m] = live && c + n < S ? c + n : -1;
  const unsigned long long mask = live ? anc_mask[m] : 0ull;
  int k = 0;
  for (int j = 0; j < N1 && k < A; ++j)
    if ((mask >> j) & 1ull) anc[(int64_t)m * A + k++] = c + j < S ? c + j : -1;
  for (; k < A; ++k) anc[(int64_t)m * A + k] = -1;
}

// h[m] = embed[tok[m]], 16 bytes per thread and step.
__global__ __launch_bounds__(256) void gather_rows_kernel(const u32x4_t* __restrict__ embed,
                                                          const int* __restrict__ tok, int vec,
                                                          u32x4_t* __restrict__ h) {
  const int m = blockIdx.x;
  const u32x4_t* src = embed + (int64_t)tok[m] * vec;
  for (int i = threadIdx.x; i < vec; i += 256) h[(int64_t)m * vec + i] = src[i];
}

}  // namespace

hipError_t target_rows(int B, int N1, int A, const int* tokens, const int* position,
                       const int* num_nodes, const unsigned long long* anc_mask,
                       const int* ctx_len, int V, int S, int* tok, int* pos, int* slot, int* anc,
                       hipStream_t s) {
  const int M = B * N1;
  SPEC_LAUNCH(target_rows_kernel, dim3((M + 255) / 256), dim3(256), 0, s, B, N1, A, tokens,
              position, num_nodes, anc_mask, ctx_len, V, S, tok, pos, slot, anc);
  return hipGetLastError();
}

hipError_t gather_rows(const void* embed, const int* tok, int M, int row_bytes, void* h,
                       hipStream_t s) {
  SPEC_LAUNCH(gather_rows_kernel, dim3(M), dim3(256), 0, s, (const u32x4_t*)embed, tok,
              row_bytes / 16, (u32x4_t*)h);
  return hipGetLastError();
}

}  // namespace spec

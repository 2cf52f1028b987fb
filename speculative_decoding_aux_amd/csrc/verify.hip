// Verification of the draft trees against the target logits, and KV
// compaction of the accepted path.
//
// Stage 1, statistics (data-parallel over every tree node and a chunk of the
// vocabulary; the target logits are read once with 16-byte loads): greedy
// keeps the argmax (first index on ties), stochastic keeps the running max m
// of l/T and the sum of exp(l/T - m) in float64.
// Stage 2, walk (one wave per sequence): merge the chunk records of the nodes
// on the walk and run the acceptance walk from the root; greedy writes the
// bonus token, stochastic records the node where the walk stopped.
// Level mode (large rows): stages 1 and 2 run level by level, the statistics
// of only the node each walk has reached (at most depth + 1 rows a sequence
// instead of every node's).
// Stage 3, stochastic only: Gumbel-max over that node's row with its children
// excluded, which samples the residual distribution (or the node's own
// distribution when it has no children).  U is drawn in-kernel from
// Philox4x32-10 (key = seed, counter = (v >> 2, node, b, 0), word v & 3), so
// the noise costs no memory traffic and is drawn for B rows, not B (N + 1).
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace spec {

// Scratch of the allocation-free verification entry point: the per (node,
// vocabulary chunk) statistics records, the Gumbel records and the stop
// nodes.  Each GPU holds its own copy for the life of the process; host code
// never passes this name to a kernel, only the device address that
// hipGetSymbolAddress returns for it (static_verify_scratch).
static __device__ __align__(256) unsigned char scratch[kStaticVerifyScratchBytes];

namespace {

struct VPart {  // per (tree node, vocab chunk)
  double z;     // stochastic: sum exp(l/T - m)
  float m;      // stochastic: max l/T; greedy: max l
  int arg;      // greedy argmax id
};

struct GPart {  // per (sequence, vocab chunk) of the stop node's row
  float gs;     // best Gumbel score
  int gid;
};

// Statistics record of ids [lo, hi) of one logits row (lo a multiple of
// 1024), by a 256-thread block; valid in thread 0.
SPEC_DEV VPart chunk_stats(const float* __restrict__ lrow, int lo, int hi, int mode, float temp) {
  __shared__ float rf[4];
  __shared__ int ri[4];
  __shared__ double rz[4];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const bool vec = ((uintptr_t)lrow & 15) == 0;  // chunk starts are multiples of 1024
  VPart rec;
  if (mode == 0) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    auto visit = [&](float v, int x) {
      if (better(v, x, bv, bi)) {
        bv = v;
        bi = x;
      }
    };
    if (vec) {
      for_row_batches(lrow, lo, hi, [&](const float (&v)[16], int x0) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int x = x0 + 1024 * (e >> 2) + (e & 3);
          if (x < hi) visit(v[e], x);
        }
      });
    } else {
      for (int x = lo + t; x < hi; x += 256) visit(lrow[x], x);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (lane == 0) {
      rf[wave] = bv;
      ri[wave] = bi;
    }
    __syncthreads();
    if (t == 0) {
      for (int w = 1; w < 4; ++w)
        if (better(rf[w], ri[w], rf[0], ri[0])) {
          rf[0] = rf[w];
          ri[0] = ri[w];
        }
      rec.m = rf[0];
      rec.arg = ri[0];
      rec.z = 0.0;
    }
    return rec;
  }
  const float invT = 1.0f / temp;
  float m = -INFINITY;
  double zs = 0.0;
  if (vec) {
    for_row_batches(lrow, lo, hi, [&](const float (&v)[16], int) {
      if (temp == 1.0f) {
        lse_update16(v, m, zs);
      } else {
        float zv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) zv[e] = v[e] * invT;
        lse_update16(zv, m, zs);
      }
    });
  } else {
    for (int x = lo + t; x < hi; x += 256) {
      const float zv = temp == 1.0f ? lrow[x] : lrow[x] * invT;
      if (zv > m) {
        zs = (m == -INFINITY ? 0.0 : zs * exp((double)m - (double)zv)) + 1.0;
        m = zv;
      } else if (zv != -INFINITY) {
        zs += (double)expf(zv - m);
      }
    }
  }
  const float wm = wave_max(m);
  double wz = m == -INFINITY ? 0.0 : zs * exp((double)m - (double)wm);
  wz = wave_sum(wz);
  if (lane == 0) {
    rf[wave] = wm;
    rz[wave] = wz;
  }
  __syncthreads();
  if (t == 0) {
    float bm = -INFINITY;
    for (int w2 = 0; w2 < 4; ++w2) bm = fmaxf(bm, rf[w2]);
    double bz = 0.0;
    for (int w2 = 0; w2 < 4; ++w2)
      if (rf[w2] != -INFINITY) bz += rz[w2] * exp((double)rf[w2] - (double)bm);
    rec.m = bm;
    rec.z = bz;
    rec.arg = 0;
  }
  return rec;
}


__global__ __launch_bounds__(256) void verify_stats_kernel(int N, int V,
                                                           const int* __restrict__ num_nodes,
                                                           const float* __restrict__ logits,
                                                           int mode, float temp, int chunk,
                                                           VPart* __restrict__ part) {
  const int c = blockIdx.x, row = blockIdx.y, nch = gridDim.x;
  const int n1 = N + 1;
  const int b = row / n1, n = row % n1;
  if (n > num_nodes[b]) return;
  const int lo = c * chunk, hi = min(V, lo + chunk);
  const VPart rec = chunk_stats(logits + (int64_t)row * V, lo, hi, mode, temp);
  if (threadIdx.x == 0) part[(int64_t)row * nch + c] = rec;
}

// One step of the acceptance walk of sequence b at node cur, by one wave:
// merge cur's chunk records pb[0, nch) and return the accepted child (-1:
// none); greedy also leaves the argmax in *emit.  Lane l holds node l + 1's
// token tkl and parent prl (-2 past the tree's nn nodes).
SPEC_DEV int walk_step(int b, int cur, int n1, int nn, int k, int V, int tkl, int prl,
                       const float* __restrict__ logits, int mode, float temp,
                       const float* __restrict__ accept_u, int nch, const VPart* __restrict__ pb,
                       int* emit) {
  const int lane = threadIdx.x & 63;
  const int xl = lane + 1;
  // merge the chunk records of node cur
  float m = -INFINITY;
  int arg = 0x7fffffff;
  for (int c = lane; c < nch; c += 64) {
    const VPart p = pb[c];
    if (mode == 0) {
      if (better(p.m, p.arg, m, arg)) {
        m = p.m;
        arg = p.arg;
      }
    } else {
      m = fmaxf(m, p.m);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o, 64);
    const int oa = __shfl_xor(arg, o, 64);
    if (mode == 0) {
      if (better(om, oa, m, arg)) {
        m = om;
        arg = oa;
      }
    } else {
      m = fmaxf(m, om);
    }
  }
  int next = -1;
  if (mode == 0) {
    // child whose token is the argmax (first in node order)
    const unsigned long long bal = __ballot(xl <= nn && prl == cur && tkl == arg);
    if (bal) next = __ffsll((long long)bal);  // node lane + 1 of the lowest hit
    *emit = arg;
  } else {
    double z = 0.0;
    for (int c = lane; c < nch; c += 64) {
      const VPart p = pb[c];
      if (p.m != -INFINITY) z += p.z * exp((double)p.m - (double)m);
    }
    z = wave_sum(z);
    // each child's probability and uniform, loaded by its own lane (node
    // lane + 1; its rank among the children in node order picks the
    // uniform); then the children are tested one after another
    const unsigned long long kids = __ballot(xl <= nn && prl == cur);
    double p = 0.0;
    float u = 0.f;
    if ((kids >> lane) & 1) {
      const int tok = clampi(tkl, 0, V - 1);
      const float l = logits[(int64_t)(b * n1 + cur) * V + tok];
      const float zv = temp == 1.0f ? l : l * (1.0f / temp);
      p = exp((double)zv - (double)m) / z;
      const int ord = __popcll(kids & ((1ull << lane) - 1));
      u = accept_u[((int64_t)(b * n1 + cur)) * k + min(ord, k - 1)];
    }
    double zrem = 1.0;
    for (unsigned long long rem = kids; rem && next < 0; rem &= rem - 1) {
      const int i = __ffsll((long long)rem) - 1;
      const double pi = __shfl(p, i, 64);
      const float ui = __shfl(u, i, 64);
      if ((double)ui <= pi / zrem) {
        next = i + 1;
      } else {
        zrem -= pi;
      }
    }
  }
  return next;
}

__global__ __launch_bounds__(64) void verify_walk_kernel(
    int N, int D, int k, int V, const int* __restrict__ tokens, const int* __restrict__ parent,
    const int* __restrict__ num_nodes, const float* __restrict__ logits, int mode, float temp,
    const float* __restrict__ accept_u, int nch, const VPart* __restrict__ part,
    int* __restrict__ stop, int* __restrict__ out_tokens, int* __restrict__ accepted_len,
    int* __restrict__ accepted_nodes) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int n1 = N + 1;
  const int nn = min(num_nodes[b], N);
  const int* tk = tokens + (int64_t)b * n1;
  const int* pr = parent + (int64_t)b * n1;
  int cur = 0, depth = 0, emit = -1;
  for (int j = lane; j <= D; j += 64) out_tokens[(int64_t)b * (D + 1) + j] = -1;
  for (int j = lane; j < D; j += 64) accepted_nodes[(int64_t)b * D + j] = -1;
  // node lane + 1's token and parent, read once (nn <= 63: one node per lane)
  const int xl = lane + 1;
  const int tkl = xl <= nn ? tk[xl] : -1, prl = xl <= nn ? pr[xl] : -2;
  while (true) {
    const int next = walk_step(b, cur, n1, nn, k, V, tkl, prl, logits, mode, temp, accept_u, nch,
                               part + (int64_t)(b * n1 + cur) * nch, &emit);
    if (next < 0 || depth >= D) break;
    if (lane == 0) {
      out_tokens[(int64_t)b * (D + 1) + depth] = tk[next];
      accepted_nodes[(int64_t)b * D + depth] = next;
    }
    ++depth;
    cur = next;
  }
  if (lane == 0) {
    if (mode == 0) out_tokens[(int64_t)b * (D + 1) + depth] = emit;
    else stop[b] = cur;
    accepted_len[b] = depth;
  }
}

// Level mode (trees whose rows are large): launch r = 0..D+1 takes every
// walk from level r - 1 to level r and reads chunk c of the row of the node
// it reached, so only the rows of nodes the walks reach are read.  Launch r's
// workgroups (c, b) all repeat the step of sequence b from level r - 1 (the
// previous launch's records of that level: the kernel boundary makes them
// visible, no workgroup waits for another), workgroup c = 0 writes the step's
// outputs and the reached node; records and nodes alternate between two
// buffers by the parity of the level.  Launch D + 1 (one workgroup a
// sequence) only steps.  node[.][b] = -1 once b's walk has stopped.
__global__ __launch_bounds__(256) void verify_level_kernel(
    int r, int N, int D, int k, int V, const int* __restrict__ tokens,
    const int* __restrict__ parent, const int* __restrict__ num_nodes,
    const float* __restrict__ logits, int mode, float temp, const float* __restrict__ accept_u,
    int nch, int chunk, VPart* __restrict__ part0, VPart* __restrict__ part1,
    int* __restrict__ node0, int* __restrict__ node1, int* __restrict__ stop,
    int* __restrict__ out_tokens, int* __restrict__ accepted_len,
    int* __restrict__ accepted_nodes) {
  __shared__ int reached;
  const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int n1 = N + 1;
  int* nprev = (r & 1) ? node0 : node1;  // level r - 1
  int* ncur = (r & 1) ? node1 : node0;   // level r
  const VPart* pprev = (r & 1) ? part0 : part1;
  VPart* pcur = (r & 1) ? part1 : part0;
  int node;
  if (r == 0) {
    node = 0;
    if (c == 0) {
      for (int j = t; j <= D; j += 256) out_tokens[(int64_t)b * (D + 1) + j] = -1;
      for (int j = t; j < D; j += 256) accepted_nodes[(int64_t)b * D + j] = -1;
      if (t == 0) ncur[b] = 0;
    }
  } else {
    const int prev = nprev[b];
    if (prev < 0) {  // stopped before level r - 1 (uniform in the block)
      if (c == 0 && t == 0) ncur[b] = -1;
      return;
    }
    if (t < 64) {
      const int lane = t;
      const int nn = min(num_nodes[b], N);
      const int* tk = tokens + (int64_t)b * n1;
      const int* pr = parent + (int64_t)b * n1;
      const int xl = lane + 1;
      const int tkl = xl <= nn ? tk[xl] : -1, prl = xl <= nn ? pr[xl] : -2;
      int emit = -1;
      const int next = walk_step(b, prev, n1, nn, k, V, tkl, prl, logits, mode, temp, accept_u,
                                 nch, pprev + (int64_t)b * nch, &emit);
      const int go = (next >= 0 && r - 1 < D) ? next : -1;
      if (lane == 0) {
        reached = go;
        if (c == 0) {
          if (go >= 0) {
            out_tokens[(int64_t)b * (D + 1) + r - 1] = tk[go];
            accepted_nodes[(int64_t)b * D + r - 1] = go;
          } else {
            if (mode == 0) out_tokens[(int64_t)b * (D + 1) + r - 1] = emit;
            else stop[b] = prev;
            accepted_len[b] = r - 1;
          }
          ncur[b] = go;
        }
      }
    }
    __syncthreads();
    node = reached;
    if (node < 0 || r > D) return;  // uniform in the block
  }
  const int lo = c * chunk, hi = min(V, lo + chunk);
  const VPart rec = chunk_stats(logits + (int64_t)(b * n1 + node) * V, lo, hi, mode, temp);
  if (t == 0) pcur[(int64_t)b * nch + c] = rec;
}

// Gumbel-max over a chunk of the stop node's row, children excluded.
__global__ __launch_bounds__(256) void verify_gumbel_kernel(
    int N, int V, const int* __restrict__ tokens, const int* __restrict__ parent,
    const int* __restrict__ num_nodes, const float* __restrict__ logits, float temp,
    uint32_t seed_lo, uint32_t seed_hi, int chunk, const int* __restrict__ stop,
    GPart* __restrict__ gpart) {
  __shared__ int kids[64];
  __shared__ int nkids;
  __shared__ float rg[4];
  __shared__ int rgi[4];
  const int c = blockIdx.x, b = blockIdx.y, nch = gridDim.x;
  const int n1 = N + 1;
  const int nn = min(num_nodes[b], N);
  const int n = clampi(stop[b], 0, N);
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  if (t < 64) {  // node t + 1 (nn <= 63): one load per lane, children compacted in node order
    const int x = t + 1;
    const bool kid = x <= nn && parent[(int64_t)b * n1 + x] == n;
    const unsigned long long bal = __ballot(kid);
    if (kid) kids[__popcll(bal & ((1ull << t) - 1))] = tokens[(int64_t)b * n1 + x];
    if (t == 0) nkids = __popcll(bal);
  }
  __syncthreads();
  const int nk = nkids;
  const float* lrow = logits + (int64_t)(b * n1 + n) * V;
  const int lo = c * chunk, hi = min(V, lo + chunk);
  const float invT = 1.0f / temp;
  float gs = -INFINITY;
  int gi = 0x7fffffff;
  // 4 consecutive ids share one Philox block
  const int q0 = lo >> 2, q1 = (hi + 3) >> 2;
  for (int qd = q0 + t; qd < q1; qd += 256) {
    const u32x4 rnd = philox4x32_10(u32x4{(uint32_t)qd, (uint32_t)n, (uint32_t)b, 0u}, seed_lo,
                                    seed_hi);
    const uint32_t w[4] = {rnd.x, rnd.y, rnd.z, rnd.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int x = qd * 4 + e;
      if (x < lo || x >= hi) continue;
      const float l = lrow[x];
      const float sc = (temp == 1.0f ? l : l * invT) + gumbel_from_bits(w[e]);
      if (better(sc, x, gs, gi)) {
        bool child = false;
        for (int j = 0; j < nk; ++j) child |= kids[j] == x;
        if (!child) {
          gs = sc;
          gi = x;
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float og = __shfl_xor(gs, o, 64);
    const int oi = __shfl_xor(gi, o, 64);
    if (better(og, oi, gs, gi)) {
      gs = og;
      gi = oi;
    }
  }
  if (lane == 0) {
    rg[wave] = gs;
    rgi[wave] = gi;
  }
  __syncthreads();
  if (t == 0) {
    for (int w2 = 1; w2 < 4; ++w2)
      if (better(rg[w2], rgi[w2], rg[0], rgi[0])) {
        rg[0] = rg[w2];
        rgi[0] = rgi[w2];
      }
    gpart[(int64_t)b * nch + c] = GPart{rg[0], rgi[0]};
  }
}

// One wave per sequence: merge the Gumbel records and write the bonus token.
__global__ __launch_bounds__(64) void verify_emit_kernel(int D, int nch,
                                                         const GPart* __restrict__ gpart,
                                                         const int* __restrict__ accepted_len,
                                                         int* __restrict__ out_tokens) {
  const int b = blockIdx.x, lane = threadIdx.x;
  float gs = -INFINITY;
  int gi = 0x7fffffff;
  for (int c = lane; c < nch; c += 64) {
    const GPart p = gpart[(int64_t)b * nch + c];
    if (better(p.gs, p.gid, gs, gi)) {
      gs = p.gs;
      gi = p.gid;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float og = __shfl_xor(gs, o, 64);
    const int oi = __shfl_xor(gi, o, 64);
    if (better(og, oi, gs, gi)) {
      gs = og;
      gi = oi;
    }
  }
  if (lane == 0) out_tokens[(int64_t)b * (D + 1) + clampi(accepted_len[b], 0, D)] = gi;
}

// One block per (sequence, layer, group of HG kv-heads): for each head of the
// group, read every accepted row, then write (heads touch disjoint rows, so
// only the read-then-write order within a head needs the barrier).  Grouping
// heads keeps the block count near what the chip dispatches quickly when the
// cache has many layers and sequences.
template <int VEC_PER_ROW>
__global__ __launch_bounds__(256) void compact_kernel(char* __restrict__ kb, char* __restrict__ vb,
                                                      int64_t sl_bytes, int64_t ss_bytes,
                                                      int64_t sh_bytes, int slots, KvPages pg,
                                                      const int* __restrict__ base,
                                                      const int* __restrict__ nodes,
                                                      const int* __restrict__ alen, int max_accept,
                                                      int nkv, int hg) {
  const int b = blockIdx.x, layer = blockIdx.y, t = threadIdx.x;
  const int a = clampi(alen[b], 0, max_accept);
  const int bs = base[b];
  constexpr int kRow = VEC_PER_ROW * 16;
  constexpr int kPer = (2 * 64 * VEC_PER_ROW + 255) / 256;  // up to 64 rows of K and V
  const int total = 2 * a * VEC_PER_ROW;
  const int h1 = min(nkv, (blockIdx.z + 1) * hg);
  for (int h = blockIdx.z * hg; h < h1; ++h) {
    const int64_t off = layer * sl_bytes + h * sh_bytes;  // + the row of (b, slot)
    u32x4_t buf[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = t + 256 * i;
      if (e < total) {
        const int kv = e / (a * VEC_PER_ROW), rem = e % (a * VEC_PER_ROW);
        const int j = rem / VEC_PER_ROW, q = rem % VEC_PER_ROW;
        const int src = bs + nodes[(int64_t)b * max_accept + j];
        if (src >= 0 && src < slots) {
          const char* p = (kv ? vb : kb) + off + kv_slot_off(pg, b, src, ss_bytes, kRow) + q * 16;
          buf[i] = *(const u32x4_t*)p;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int e = t + 256 * i;
      if (e < total) {
        const int kv = e / (a * VEC_PER_ROW), rem = e % (a * VEC_PER_ROW);
        const int j = rem / VEC_PER_ROW, q = rem % VEC_PER_ROW;
        const int src = bs + nodes[(int64_t)b * max_accept + j];
        const int dst = bs + 1 + j;
        if (src >= 0 && src < slots && dst >= 0 && dst < slots) {
          char* p = (kv ? vb : kb) + off + kv_slot_off(pg, b, dst, ss_bytes, kRow) + q * 16;
          *(u32x4_t*)p = buf[i];
        }
      }
    }
  }
}

}  // namespace

VerifyPlan verify_plan(int B, int N, int D, int V) {
  VerifyPlan p;
  const int rows = B * (N + 1);
  // statistics: about 2048 blocks, chunks of at least 4096 ids
  int c = (2048 + rows - 1) / std::max(1, rows);
  c = std::max(1, std::min(c, std::max(1, (V + 4095) / 4096)));
  p.chunk = ((V + c - 1) / c + 1023) / 1024 * 1024;
  p.nch = (V + p.chunk - 1) / p.chunk;
  // Gumbel pass: about 1024 blocks over the B stop rows, chunks of >= 2048 ids
  int g = (1024 + B - 1) / std::max(1, B);
  g = std::max(1, std::min(g, std::max(1, (V + 2047) / 2048)));
  p.gchunk = ((V + g - 1) / g + 1023) / 1024 * 1024;
  p.gch = (V + p.gchunk - 1) / p.gchunk;
  // level mode once the rows of every node cost more than the D + 2 launches
  // it takes, a few microseconds each (about 32 MB of logits per launch)
  p.level = D >= 1 && (double)rows * V * 4.0 > (double)(D + 2) * 32.0 * (1 << 20);
  // level mode: about 1024 blocks over the B current rows, chunks of >= 4096 ids
  int lc = (1024 + B - 1) / std::max(1, B);
  lc = std::max(1, std::min(lc, std::max(1, (V + 4095) / 4096)));
  p.lchunk = ((V + lc - 1) / lc + 1023) / 1024 * 1024;
  p.lch = (V + p.lchunk - 1) / p.lchunk;
  return p;
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t verify_ws_bytes(const VerifyPlan& p, int B, int N) {
  // level mode: records and reached nodes of two levels
  const size_t recs = p.level ? 2 * (size_t)B * p.lch : (size_t)B * (N + 1) * p.nch;
  return align256(recs * sizeof(VPart)) + align256((size_t)B * p.gch * sizeof(GPart)) +
         3 * align256((size_t)B * sizeof(int));
}

hipError_t verify(int B, int N, int D, int k, int V, const int* tokens, const int* parent,
                  const int* num_nodes, const float* logits, int mode, float temperature,
                  const float* accept_u, uint64_t seed, int* out_tokens, int* accepted_len,
                  int* accepted_nodes, void* ws, const VerifyPlan& p, hipStream_t s) {
  const int rows = B * (N + 1);
  const size_t recs = p.level ? 2 * (size_t)B * p.lch : (size_t)rows * p.nch;
  char* w = (char*)ws;
  VPart* part = (VPart*)w;
  w += align256(recs * sizeof(VPart));
  GPart* gpart = (GPart*)w;
  w += align256((size_t)B * p.gch * sizeof(GPart));
  int* stop = (int*)w;
  w += align256((size_t)B * sizeof(int));
  int* node0 = (int*)w;
  w += align256((size_t)B * sizeof(int));
  int* node1 = (int*)w;
  hipError_t e = hipSuccess;
  if (p.level) {
    VPart* part1 = part + (size_t)B * p.lch;
    for (int r = 0; r <= D + 1 && e == hipSuccess; ++r) {
      SPEC_LAUNCH(verify_level_kernel, dim3(r <= D ? p.lch : 1, B), dim3(256), 0, s, r, N, D, k,
                  V, tokens, parent, num_nodes, logits, mode, temperature, accept_u, p.lch,
                  p.lchunk, part, part1, node0, node1, stop, out_tokens, accepted_len,
                  accepted_nodes);
      e = hipGetLastError();
    }
  } else {
    SPEC_LAUNCH(verify_stats_kernel, dim3(p.nch, rows), dim3(256), 0, s, N, V, num_nodes,
                logits, mode, temperature, p.chunk, part);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    SPEC_LAUNCH(verify_walk_kernel, dim3(B), dim3(64), 0, s, N, D, k, V, tokens, parent,
                num_nodes, logits, mode, temperature, accept_u, p.nch, (const VPart*)part, stop,
                out_tokens, accepted_len, accepted_nodes);
    e = hipGetLastError();
  }
  if (e != hipSuccess || mode == 0) return e;
  SPEC_LAUNCH(verify_gumbel_kernel, dim3(p.gch, B), dim3(256), 0, s, N, V, tokens, parent,
                     num_nodes, logits, temperature, (uint32_t)(seed & 0xffffffffu),
                     (uint32_t)(seed >> 32), p.gchunk, (const int*)stop, gpart);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  SPEC_LAUNCH(verify_emit_kernel, dim3(B), dim3(64), 0, s, D, p.gch, (const GPart*)gpart,
                     (const int*)accepted_len, out_tokens);
  return hipGetLastError();
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
hipError_t static_verify_scratch(void** out) {
  constexpr int kMaxDev = 64;
  static std::once_flag once[kMaxDev];
  static void* ptr[kMaxDev];
  static hipError_t err[kMaxDev];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::call_once(once[dev], [&] {
    void* p = nullptr;
    err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    ptr[dev] = err[dev] == hipSuccess ? p : nullptr;
  });
  if (err[dev] != hipSuccess) return err[dev];
  *out = ptr[dev];
  return hipSuccess;
}

hipError_t compact(bool bf16, KvFull kv, int B, const int* base, const int* nodes,
                   const int* alen, int max_accept, hipStream_t s) {
  const int esz = bf16 ? 2 : 4;
  const int row_bytes = kv.hd * esz;
  // heads per block: about 1024 blocks in all
  const int64_t units = (int64_t)B * kv.layers * kv.nkv;
  const int hg = (int)std::max<int64_t>(1, std::min<int64_t>(kv.nkv, units / 1024));
  const dim3 grid(B, kv.layers, (kv.nkv + hg - 1) / hg);
  const int64_t sl = kv.stride_layer * esz, ss = kv.stride_seq * esz, sh = kv.stride_head * esz;
  if (row_bytes == 256) {
    SPEC_LAUNCH(compact_kernel<16>, grid, dim3(256), 0, s, (char*)kv.k, (char*)kv.v, sl, ss,
                       sh, kv.slots, kv.pg, base, nodes, alen, max_accept, kv.nkv, hg);
  } else if (row_bytes == 128) {
    SPEC_LAUNCH(compact_kernel<8>, grid, dim3(256), 0, s, (char*)kv.k, (char*)kv.v, sl, ss,
                       sh, kv.slots, kv.pg, base, nodes, alen, max_accept, kv.nkv, hg);
  } else {
    SPEC_LAUNCH(compact_kernel<32>, grid, dim3(256), 0, s, (char*)kv.k, (char*)kv.v, sl, ss,
                       sh, kv.slots, kv.pg, base, nodes, alen, max_accept, kv.nkv, hg);
  }
  return hipGetLastError();
}

}  // namespace spec

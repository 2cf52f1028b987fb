// Rejection sampling of flat batches of variable-length draft chains with
// per-request temperature, top-k and top-p: the CPU rejection sampler of the
// vLLM Neuron design page ("Rejection Sampling"), on the flat index layout of
// its "SpecDecodeMetadata: Index Bookkeeping" section.
//
// Order and keys.  Tokens rank by (logit desc, id asc).  The 50-bit key
// (monotone(l) << 18) | (2^18 - 1 - id) is larger for a better token, so the
// kept set of a filter is {v : key(v) >= kstar} for the key kstar of its last
// kept token, and one 64-bit value per row describes it.
//
// Stage 1, one workgroup per (request, position j <= n_r): greedy rows keep
// the argmax (first index on ties) and whether draft j equals it.  Random
// rows find kstar of top-k (by count) and then of top-p (by mass, over the
// top-k set) by radix selection over key intervals: each level histograms the
// candidate interval into at most 2048 power-of-two-wide bins in LDS, keeps
// the bin where the running count or mass from the top crosses the target,
// and stops when that bin holds one token.  The first level (4096 bins of
// the top 12 key bits) counts the row in the same pass as the maximum; when
// the bins from the k-th best token's up hold at most the 8192 keys LDS
// takes, the second pass copies them there and both cuts are taken on that
// list, else the second pass histograms the masses and the cut bins are
// collected (or, when too full, rescanned) one at a time.  Masses are
// exp(l/T - max) in float32 summed in float64.  A draft is accepted iff
// u <= p_f(x).
// Stage 2, vocabulary chunks of each request's stop row (first rejection, or
// the bonus row): the Gumbel-max over the kept tokens with the rejected draft
// excluded, U from the Philox4x32-10 stream of the tree verifier with
// counter (v >> 2, j, r, 0).
// Stage 3, one wave per request: merge the chunk records and write the
// accepted drafts, the emitted token and -1 padding.
#include "common.h"
#include "kernels.h"

namespace spec {

namespace {

constexpr int kSelBins = 2048;
constexpr int kRowThreads = 1024;

struct SRow {                  // per (request, position)
  unsigned long long kstar;    // kept iff key >= kstar (0: every token)
  double skept;                // sum over kept tokens of exp(l/T - zmax)
  float zmax;                  // max of l/T
  int arg;                     // argmax of l (greedy)
  int acc;                     // draft at this position accepted
  int pad;
};

struct SPart {  // Gumbel record per (request, vocab chunk)
  float gs;
  int gid;
};

SPEC_DEV unsigned long long tok_key(float l, int v) {
  uint32_t b = l == 0.f ? 0u : __float_as_uint(l);  // -0 ranks with +0
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)b << 18) | (unsigned long long)(0x3FFFF - v);
}

// f(l, v) for every token of the row owned by this thread, four loads in
// flight per thread (16-byte loads when the row is 16-byte aligned and V a
// multiple of 4).
template <typename F>
SPEC_DEV void for_row(const float* __restrict__ row, int V, F&& f) {
  const int nt = blockDim.x;
  if ((V & 3) == 0 && ((uintptr_t)row & 15) == 0) {
    const float4* r4 = (const float4*)row;
    const int n4 = V >> 2;
    for (int q0 = threadIdx.x; q0 < n4; q0 += 4 * nt) {
      float4 w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = q0 + i * nt;
        w[i] = q < n4 ? r4[q] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = q0 + i * nt;
        if (q < n4) {
          f(w[i].x, 4 * q);
          f(w[i].y, 4 * q + 1);
          f(w[i].z, 4 * q + 2);
          f(w[i].w, 4 * q + 3);
        }
      }
    }
  } else {
    for (int v0 = threadIdx.x; v0 < V; v0 += 4 * nt) {
      float w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int v = v0 + i * nt;
        w[i] = v < V ? row[v] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (v0 + i * nt < V) f(w[i], v0 + i * nt);
    }
  }
}

SPEC_DEV unsigned long long wave_max_u64(unsigned long long x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long y = __shfl_xor(x, o, 64);
    x = y > x ? y : x;
  }
  return x;
}
SPEC_DEV unsigned long long wave_min_u64(unsigned long long x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long y = __shfl_xor(x, o, 64);
    x = y < x ? y : x;
  }
  return x;
}

SPEC_DEV float float_of_mono(uint32_t m) {
  return __uint_as_float((m & 0x80000000u) ? (m & 0x7FFFFFFFu) : ~m);
}
// logit and id of a key
SPEC_DEV void key_parts(unsigned long long k, float& l, int& v) {
  v = 0x3FFFF - (int)(k & 0x3FFFFull);
  l = float_of_mono((uint32_t)(k >> 18));
}

constexpr int kL0Bits = 12;            // static first level: top 12 bits of monotone(l)
constexpr int kL0Bins = 1 << kL0Bits;
constexpr int kL0Shift = 18 + 32 - kL0Bits;  // key >> kL0Shift = first-level bin
constexpr int kCap = 8192;             // candidates of one first-level bin kept in LDS

struct SelLds {
  unsigned int l0_cnt[kL0Bins];        // first level over the whole row
  double l0_mass[kL0Bins];
  unsigned int cnt[kSelBins];          // refinement levels
  double mass[kSelBins];
  unsigned long long cand[kCap];       // keys of one first-level bin
  unsigned long long red_u[kRowThreads / 64];
  double red_d[kRowThreads / 64];
  float red_f[kRowThreads / 64];
  int red_i[kRowThreads / 64];
  int ncand;
  int sel_bin;
  unsigned int sel_above_cnt;
  double sel_above_mass;
};

// Candidate sources: f(l, v) for every token of the row, or of the LDS list.
struct RowSrc {
  const float* row;
  int V;
  template <typename F>
  SPEC_DEV void operator()(F&& f) const { for_row(row, V, f); }
};
struct CandSrc {
  const unsigned long long* cand;
  int n;
  template <typename F>
  SPEC_DEV void operator()(F&& f) const {
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      float l;
      int v;
      key_parts(cand[i], l, v);
      f(l, v);
    }
  }
};

// Wave 0 walks nb bins from the top (bin nb-1 first): each lane sums a run
// of bins, the runs are scanned from the top, the crossing lane walks its
// run.  The picked bin is the first non-empty one at which the running count
// (or mass) reaches the target, the lowest non-empty bin when none does;
// s.sel_bin / sel_above_cnt / sel_above_mass get the bin and the totals of
// the bins above it.  Called by the whole block (ends with a barrier).
template <bool BY_MASS>
SPEC_DEV void scan_pick(const unsigned int* cnt, const double* mass, int nb, unsigned int need_cnt,
                        double need_mass, SelLds& s) {
  const int t = threadIdx.x;
  if (t < 64) {
    const int per = (nb + 63) / 64;
    const int b1 = nb - 1 - t * per;  // this lane's run: b1 down to b0
    const int b0 = max(0, b1 - per + 1);
    unsigned int c = 0;
    double m = 0.0;
    for (int b = b1; b >= b0; --b) {
      c += cnt[b];
      if (BY_MASS) m += mass[b];
    }
    unsigned int cx = c;
    double mx = m;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned int oc = __shfl_up(cx, o, 64);
      const double om = __shfl_up(mx, o, 64);
      if (t >= o) {
        cx += oc;
        mx += om;
      }
    }
    cx -= c;
    mx -= m;
    const bool reach = c > 0 && (BY_MASS ? (mx + m >= need_mass) : (cx + c >= need_cnt));
    const unsigned long long bal = __ballot(reach);
    const unsigned long long nz = __ballot(c > 0);
    const int lane = bal ? __ffsll((long long)bal) - 1 : (nz ? 63 - __clzll((long long)nz) : 0);
    if (t == lane) {
      unsigned int ca = cx;
      double ma = mx;
      int pick = -1, last = -1;
      for (int b = b1; b >= b0; --b) {
        const unsigned int cb = cnt[b];
        if (!cb) continue;
        const double mb = BY_MASS ? mass[b] : 0.0;
        last = b;
        if (bal && (BY_MASS ? (ma + mb >= need_mass) : (ca + cb >= need_cnt))) {
          pick = b;
          break;
        }
        ca += cb;
        ma += mb;
      }
      if (pick < 0 && last >= 0) {  // target not reached: the lowest non-empty bin
        pick = last;
        ca -= cnt[last];
        if (BY_MASS) ma -= mass[last];
      }
      if (pick < 0) pick = 0;  // no candidate at all (callers never ask for that)
      s.sel_bin = pick;
      s.sel_above_cnt = ca;
      s.sel_above_mass = ma;
    }
  }
  __syncthreads();
}

// Block-wide maximum of keys in [lo, hi] over a source.
template <typename Src>
SPEC_DEV unsigned long long max_key_in(const Src& src, unsigned long long lo,
                                       unsigned long long hi, SelLds& s) {
  unsigned long long best = 0;
  src([&](float l, int v) {
    const unsigned long long k = tok_key(l, v);
    if (k >= lo && k <= hi && k > best) best = k;
  });
  best = wave_max_u64(best);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s.red_u[w] = best;
  __syncthreads();
  unsigned long long b = 0;
  for (int i = 0; i < kRowThreads / 64; ++i) b = s.red_u[i] > b ? s.red_u[i] : b;
  return b;
}

// Sum of exp(l * invT - zmax) over a source's tokens with key in [lo, hi].
template <typename Src>
SPEC_DEV double mass_in(const Src& src, float invT, float zmax, unsigned long long lo,
                        unsigned long long hi, SelLds& s) {
  double acc = 0.0;
  src([&](float l, int v) {
    const unsigned long long k = tok_key(l, v);
    if (k >= lo && k <= hi && l != -INFINITY) acc += (double)expf(l * invT - zmax);
  });
  return block_sum(acc, s.red_d);
}

// Radix selection over the key interval [lo, hi] of a source (better tokens
// have larger keys).  BY_MASS = false: the key of the need_cnt-th best
// candidate.  BY_MASS = true: the key of the first candidate, best first, at
// which the running mass reaches need_mass (the last candidate when it never
// does); *mass_upto gets the mass up to and including it.
template <bool BY_MASS, typename Src>
SPEC_DEV unsigned long long radix_select(const Src& src, float invT, float zmax,
                                         unsigned long long lo, unsigned long long hi,
                                         unsigned int need_cnt, double need_mass,
                                         double* mass_upto, SelLds& s) {
  const int t = threadIdx.x;
  double above_mass = 0.0;
  while (true) {
    const unsigned long long span = hi - lo;
    int sh = 0;
    while ((span >> sh) >= (unsigned long long)kSelBins) ++sh;
    const int nb = (int)(span >> sh) + 1;
    for (int i = t; i < nb; i += kRowThreads) {
      s.cnt[i] = 0;
      if (BY_MASS) s.mass[i] = 0.0;
    }
    __syncthreads();
    src([&](float l, int v) {
      const unsigned long long k = tok_key(l, v);
      if (k >= lo && k <= hi) {
        const int bin = (int)((k - lo) >> sh);
        atomicAdd(&s.cnt[bin], 1u);
        if (BY_MASS && l != -INFINITY) atomicAdd(&s.mass[bin], (double)expf(l * invT - zmax));
      }
    });
    __syncthreads();
    scan_pick<BY_MASS>(s.cnt, s.mass, nb, need_cnt, need_mass, s);
    const int pick = s.sel_bin;
    const unsigned int cb = s.cnt[pick];
    const double mb = BY_MASS ? s.mass[pick] : 0.0;
    need_cnt -= s.sel_above_cnt;
    need_mass -= s.sel_above_mass;
    above_mass += s.sel_above_mass;
    const unsigned long long nlo = lo + ((unsigned long long)pick << sh);
    const unsigned long long nhi_full = nlo + ((1ull << sh) - 1);
    const unsigned long long nhi = nhi_full < hi ? nhi_full : hi;
    __syncthreads();  // everyone has read the selection before LDS is reused
    if (sh == 0) {
      if (BY_MASS) *mass_upto = above_mass + mb;
      return nlo;
    }
    if (cb == 1) {
      if (BY_MASS) *mass_upto = above_mass + mb;
      return max_key_in(src, nlo, nhi, s);
    }
    lo = nlo;
    hi = nhi;
  }
}

// Keys of the row's tokens in first-level bin b into s.cand (the bin holds
// at most kCap tokens); returns their number.
SPEC_DEV int collect_bin(const float* row, int V, int b, SelLds& s) {
  if (threadIdx.x == 0) s.ncand = 0;
  __syncthreads();
  for_row(row, V, [&](float l, int v) {
    const unsigned long long k = tok_key(l, v);
    const bool in = (int)(k >> kL0Shift) == b;
    const unsigned long long act = __ballot(true);
    const unsigned long long m = __ballot(in);
    if (m) {
      const int lane = threadIdx.x & 63;
      const int leader = __ffsll((long long)act) - 1;
      int base = 0;
      if (lane == leader) base = atomicAdd(&s.ncand, __popcll(m));
      base = __shfl(base, leader, 64);
      const int pos = base + __popcll(m & ((1ull << lane) - 1));
      if (in && pos < kCap) s.cand[pos] = k;
    }
  });
  __syncthreads();
  return min(s.ncand, kCap);
}

// Key interval of first-level bin b.
SPEC_DEV unsigned long long bin_lo(int b) { return (unsigned long long)b << kL0Shift; }
SPEC_DEV unsigned long long bin_hi(int b) { return (((unsigned long long)b + 1) << kL0Shift) - 1; }

__global__ __launch_bounds__(256) void sample_meta_kernel(int B, const int* __restrict__ cu_sched,
                                                          const int* __restrict__ nd,
                                                          int* __restrict__ cu_nd,
                                                          int* __restrict__ logits_idx,
                                                          int* __restrict__ tgt_idx,
                                                          int* __restrict__ bonus_idx) {
  __shared__ int part[4];
  __shared__ int carry_s;
  const int t = threadIdx.x, w = t >> 6, lane = t & 63;
  if (t == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < B; base += 256) {
    const int r = base + t;
    const int n = r < B ? max(0, nd[r]) : 0;
    int x = n;  // inclusive scan within the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) part[w] = x;
    __syncthreads();
    int off = carry_s;
    for (int i = 0; i < w; ++i) off += part[i];
    const int incl = off + x;  // drafts of requests 0..r
    if (r < B) {
      cu_nd[r] = incl;
      const int d0 = incl - n;    // first draft entry of request r
      const int o = d0 + r;       // first logits row of request r
      const int first = cu_sched[r] - (n + 1);
      for (int j = 0; j <= n; ++j) {
        logits_idx[o + j] = first + j;
        if (j < n) tgt_idx[d0 + j] = o + j;
      }
      bonus_idx[r] = o + n;
    }
    __syncthreads();
    if (t == 255) carry_s = incl;
    __syncthreads();
  }
}

__global__ __launch_bounds__(kRowThreads) void sample_row_kernel(
    int L, int V, int nrows, const int* __restrict__ cu_nd, const int* __restrict__ drafts,
    const float* __restrict__ logits, const int* __restrict__ tgt_idx,
    const int* __restrict__ bonus_idx, const float* __restrict__ temperature,
    const int* __restrict__ top_k, const float* __restrict__ top_p,
    const float* __restrict__ uniform, SRow* __restrict__ srow) {
  __shared__ SelLds s;
  const int r = blockIdx.x, j = blockIdx.y, t = threadIdx.x;
  const int start = r ? cu_nd[r - 1] : 0;
  const int n = min(max(cu_nd[r] - start, 0), L);
  if (j > n) return;
  const int rid = clampi(j < n ? tgt_idx[start + j] : bonus_idx[r], 0, nrows - 1);
  const float* row = logits + (int64_t)rid * V;
  const float T = temperature[r];
  const bool greedy = !(T > 0.f) || uniform == nullptr;
  const int x = j < n ? drafts[start + j] : -1;
  const int k = greedy || !top_k ? 0 : top_k[r];
  const float p = greedy || !top_p ? 1.0f : top_p[r];
  const bool use_k = k > 0 && k < V, use_p = p < 1.0f;
  const bool hist = use_k || use_p;  // the row needs the first-level histogram
  if (hist) {
    for (int i = t; i < kL0Bins; i += kRowThreads) {
      s.l0_cnt[i] = 0;
      s.l0_mass[i] = 0.0;
    }
    __syncthreads();
  }
  // pass 1: max / argmax, and the first-level counts (they need no maximum)
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for_row(row, V, [&](float l, int v) {
    if (better(l, v, bv, bi)) {
      bv = l;
      bi = v;
    }
    if (hist) atomicAdd(&s.l0_cnt[(int)(tok_key(l, v) >> kL0Shift)], 1u);
  });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  const int w = t >> 6;
  if ((t & 63) == 0) {
    s.red_f[w] = bv;
    s.red_i[w] = bi;
  }
  __syncthreads();  // also orders the counts before their use
  for (int i = 0; i < kRowThreads / 64; ++i)
    if (better(s.red_f[i], s.red_i[i], bv, bi)) {
      bv = s.red_f[i];
      bi = s.red_i[i];
    }
  SRow out;
  out.arg = bi;
  out.pad = 0;
  if (greedy) {
    out.kstar = 0;
    out.skept = 0.0;
    out.zmax = 0.f;
    out.acc = j < n && x == bi;
    if (t == 0) srow[r * (L + 1) + j] = out;
    return;
  }
  const float invT = 1.0f / T;
  const float zmax = bv * invT;
  // the first-level bin of the k-th best token, from the counts
  int bk = -1;
  unsigned int above = 0, cbk = 0;
  if (use_k) {
    scan_pick<false>(s.l0_cnt, s.l0_mass, kL0Bins, (unsigned int)k, 0.0, s);
    bk = s.sel_bin;
    above = s.sel_above_cnt;
    cbk = s.l0_cnt[bk];
  }
  // Top-k sets that fit in LDS: pass 2 collects the keys of every bin from
  // bk up (the whole top-k set and the rest of bin bk), and both cuts are
  // then taken on that list: no mass histogram and no further row pass.
  double S = 0.0;
  unsigned long long kstar = 0;  // kept iff key >= kstar
  if (use_k && above + cbk <= (unsigned int)kCap) {
    const unsigned long long glo = bin_lo(bk);
    if (t == 0) s.ncand = 0;
    __syncthreads();
    for_row(row, V, [&](float l, int v) {
      const unsigned long long key = tok_key(l, v);
      const bool in = key >= glo;
      const unsigned long long m = __ballot(in);
      if (m) {
        const int lane = t & 63;
        const int leader = __ffsll((long long)m) - 1;
        int base = 0;
        if (lane == leader) base = atomicAdd(&s.ncand, __popcll(m));
        base = __shfl(base, leader, 64);
        const int pos = base + __popcll(m & ((1ull << lane) - 1));
        if (in && pos < kCap) s.cand[pos] = key;
      }
    });
    __syncthreads();
    const CandSrc cs{s.cand, min(s.ncand, kCap)};
    const unsigned long long ktop = tok_key(bv, bi);  // the best key of the row
    double unused;
    kstar = radix_select<false>(cs, invT, zmax, glo, bin_hi(bk), (unsigned int)k - above, 0.0,
                                &unused, s);
    S = mass_in(cs, invT, zmax, kstar, ktop, s);
    if (use_p) {
      double upto = 0.0;
      kstar = radix_select<true>(cs, invT, zmax, kstar, ktop, 0u, (double)p * S, &upto, s);
      S = upto;
    }
  } else {
    // pass 2: the first-level masses and the row's mass
    double sum = 0.0;
    for_row(row, V, [&](float l, int v) {
      const double e = l == -INFINITY ? 0.0 : (double)expf(l * invT - zmax);
      sum += e;
      if (hist && e != 0.0) atomicAdd(&s.l0_mass[(int)(tok_key(l, v) >> kL0Shift)], e);
    });
    S = block_sum(sum, s.red_d);  // also orders the histogram before its use
    int cbin = -1;                // first-level bin whose keys are in s.cand
    int ncand = 0;
    if (use_k) {
      // the k-th best token in bin bk
      double above_mass = 0.0;
      for (int b = kL0Bins - 1 - t; b > bk; b -= kRowThreads) above_mass += s.l0_mass[b];
      above_mass = block_sum(above_mass, s.red_d);
      double unused;
      if (cbk <= (unsigned int)kCap) {
        ncand = collect_bin(row, V, bk, s);
        cbin = bk;
        const CandSrc cs{s.cand, ncand};
        kstar = radix_select<false>(cs, invT, zmax, bin_lo(bk), bin_hi(bk), (unsigned int)k - above,
                                    0.0, &unused, s);
        S = above_mass + mass_in(cs, invT, zmax, kstar, bin_hi(bk), s);
      } else {
        const RowSrc rs{row, V};
        kstar = radix_select<false>(rs, invT, zmax, bin_lo(bk), bin_hi(bk), (unsigned int)k - above,
                                    0.0, &unused, s);
        S = above_mass + mass_in(rs, invT, zmax, kstar, bin_hi(bk), s);
      }
      // the top-k set as a first-level histogram: bins below bk emptied, bin
      // bk reduced to its kept part
      for (int b = t; b < bk; b += kRowThreads) {
        s.l0_cnt[b] = 0;
        s.l0_mass[b] = 0.0;
      }
      __syncthreads();
      if (t == 0) {
        s.l0_cnt[bk] = (unsigned int)k - above;
        s.l0_mass[bk] = S - above_mass;
      }
      __syncthreads();
    }
    if (use_p) {
      const double target = (double)p * S;
      scan_pick<true>(s.l0_cnt, s.l0_mass, kL0Bins, 0u, target, s);
      const int bp = s.sel_bin;
      const double above_mass = s.sel_above_mass;
      const unsigned int cbp = s.l0_cnt[bp];
      __syncthreads();
      // in the top-k cut's bin only its kept part counts; its tokens are in
      // LDS when the top-k selection collected them, else the row is scanned
      const unsigned long long lo = bp == bk ? kstar : bin_lo(bp);
      const bool have = bp == cbin;
      double upto = 0.0;
      if (have || (bp != bk && cbp <= (unsigned int)kCap)) {
        if (!have) {
          ncand = collect_bin(row, V, bp, s);
          cbin = bp;
        }
        const CandSrc cs{s.cand, ncand};
        kstar = radix_select<true>(cs, invT, zmax, lo, bin_hi(bp), 0u, target - above_mass, &upto, s);
      } else {
        const RowSrc rs{row, V};
        kstar = radix_select<true>(rs, invT, zmax, lo, bin_hi(bp), 0u, target - above_mass, &upto, s);
      }
      S = above_mass + upto;
    }
  }
  out.kstar = kstar;
  out.skept = S;
  out.zmax = zmax;
  out.acc = 0;
  if (j < n) {
    const int xc = clampi(x, 0, V - 1);
    const float lx = row[xc];
    const bool kept = x == xc && (kstar == 0 || tok_key(lx, xc) >= kstar);
    const double px = kept && lx != -INFINITY ? (double)expf(lx * invT - zmax) / S : 0.0;
    out.acc = (double)uniform[start + j] <= px;
  }
  if (t == 0) srow[r * (L + 1) + j] = out;
}

// First position of request r whose draft was rejected, n when none was.
SPEC_DEV int stop_position(const SRow* srow, int r, int L, int n) {
  int js = n;
  for (int j = 0; j < n; ++j)
    if (!srow[r * (L + 1) + j].acc) {
      js = j;
      break;
    }
  return js;
}

__global__ __launch_bounds__(256) void sample_gumbel_kernel(
    int L, int V, int nrows, const int* __restrict__ cu_nd, const int* __restrict__ drafts,
    const float* __restrict__ logits, const int* __restrict__ tgt_idx,
    const int* __restrict__ bonus_idx, const float* __restrict__ temperature,
    const float* __restrict__ uniform, uint32_t seed_lo, uint32_t seed_hi, int chunk,
    const SRow* __restrict__ srow, SPart* __restrict__ gpart) {
  __shared__ float rg[4];
  __shared__ int rgi[4];
  const int c = blockIdx.x, r = blockIdx.y, nch = gridDim.x;
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const float T = temperature[r];
  if (!(T > 0.f) || uniform == nullptr) return;  // greedy: the emit stage takes the argmax
  const int start = r ? cu_nd[r - 1] : 0;
  const int n = min(max(cu_nd[r] - start, 0), L);
  const int js = stop_position(srow, r, L, n);
  const int rid = clampi(js < n ? tgt_idx[start + js] : bonus_idx[r], 0, nrows - 1);
  const int x = js < n ? drafts[start + js] : -1;
  const unsigned long long kstar = srow[r * (L + 1) + js].kstar;
  const float* row = logits + (int64_t)rid * V;
  const float invT = 1.0f / T;
  const int lo = c * chunk, hi = min(V, lo + chunk);
  float gs = -INFINITY;
  int gi = 0x7fffffff;
  const int q0 = lo >> 2, q1 = (hi + 3) >> 2;
  for (int qd = q0 + t; qd < q1; qd += 256) {
    const u32x4 rnd = philox4x32_10(u32x4{(uint32_t)qd, (uint32_t)js, (uint32_t)r, 0u}, seed_lo,
                                    seed_hi);
    const uint32_t wd[4] = {rnd.x, rnd.y, rnd.z, rnd.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = qd * 4 + e;
      if (v < lo || v >= hi || v == x) continue;
      const float l = row[v];
      if (kstar != 0 && tok_key(l, v) < kstar) continue;
      const float sc = l * invT + gumbel_from_bits(wd[e]);
      if (better(sc, v, gs, gi)) {
        gs = sc;
        gi = v;
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
    gpart[(int64_t)r * nch + c] = SPart{rg[0], rgi[0]};
  }
}

__global__ __launch_bounds__(64) void sample_emit_kernel(
    int L, int nch, const int* __restrict__ cu_nd, const int* __restrict__ drafts,
    const float* __restrict__ temperature, const float* __restrict__ uniform,
    const SRow* __restrict__ srow, const SPart* __restrict__ gpart, int* __restrict__ out_tokens,
    int* __restrict__ num_accepted) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const int start = r ? cu_nd[r - 1] : 0;
  const int n = min(max(cu_nd[r] - start, 0), L);
  const int js = stop_position(srow, r, L, n);
  int tok;
  const float T = temperature[r];
  if (!(T > 0.f) || uniform == nullptr) {
    tok = srow[r * (L + 1) + js].arg;
  } else {
    float gs = -INFINITY;
    int gi = 0x7fffffff;
    for (int c = lane; c < nch; c += 64) {
      const SPart q = gpart[(int64_t)r * nch + c];
      if (better(q.gs, q.gid, gs, gi)) {
        gs = q.gs;
        gi = q.gid;
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
    tok = gi == 0x7fffffff ? -1 : gi;
  }
  for (int jj = lane; jj <= L; jj += 64)
    out_tokens[(int64_t)r * (L + 1) + jj] = jj < js ? drafts[start + jj] : (jj == js ? tok : -1);
  if (lane == 0) num_accepted[r] = js;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

SamplePlan sample_plan(int B, int V) {
  SamplePlan p;
  int g = (1024 + B - 1) / std::max(1, B);
  g = std::max(1, std::min(g, std::max(1, (V + 2047) / 2048)));
  p.gchunk = ((V + g - 1) / g + 1023) / 1024 * 1024;
  p.gch = (V + p.gchunk - 1) / p.gchunk;
  return p;
}

size_t sample_ws_bytes(const SamplePlan& p, int B, int L) {
  return align256((size_t)B * (L + 1) * sizeof(SRow)) + align256((size_t)B * p.gch * sizeof(SPart));
}

hipError_t sample_metadata(int B, const int* cu_sched, const int* nd, int* cu_nd, int* logits_idx,
                           int* tgt_idx, int* bonus_idx, hipStream_t s) {
  SPEC_LAUNCH(sample_meta_kernel, dim3(1), dim3(256), 0, s, B, cu_sched, nd, cu_nd, logits_idx,
              tgt_idx, bonus_idx);
  return hipGetLastError();
}

hipError_t rejection_sample(int B, int L, int V, int nrows, const int* cu_nd, const int* drafts,
                            const float* logits, const int* tgt_idx, const int* bonus_idx,
                            const float* temperature, const int* top_k, const float* top_p,
                            const float* uniform, uint64_t seed, int* out_tokens,
                            int* num_accepted, void* ws, const SamplePlan& p, hipStream_t s) {
  char* w = (char*)ws;
  SRow* srow = (SRow*)w;
  w += align256((size_t)B * (L + 1) * sizeof(SRow));
  SPart* gpart = (SPart*)w;
  SPEC_LAUNCH(sample_row_kernel, dim3(B, L + 1), dim3(kRowThreads), 0, s, L, V, nrows, cu_nd,
              drafts, logits, tgt_idx, bonus_idx, temperature, top_k, top_p, uniform, srow);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SPEC_LAUNCH(sample_gumbel_kernel, dim3(p.gch, B), dim3(256), 0, s, L, V, nrows, cu_nd, drafts,
              logits, tgt_idx, bonus_idx, temperature, uniform, (uint32_t)(seed & 0xffffffffu),
              (uint32_t)(seed >> 32), p.gchunk, (const SRow*)srow, gpart);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  SPEC_LAUNCH(sample_emit_kernel, dim3(B), dim3(64), 0, s, L, p.gch, cu_nd, drafts, temperature,
              uniform, (const SRow*)srow, (const SPart*)gpart, out_tokens, num_accepted);
  return hipGetLastError();
}

}  // namespace spec

// Vocabulary-wide top-k with log-probabilities, candidate retrieval and the
// gathered exact rescoring of the EAGLE-4 candidate head.
//
// topk: rows are split into chunks; a workgroup scans one chunk with a sorted
// register list of KM (value, id) per thread plus an online (max, sum exp)
// (sum in float64), merges the 256 lists by k rounds of wave-wide "best head"
// selection, and writes a partial record (with 16-byte loads the lists hold
// the best element of each 16-value batch, and the k best batches are rescanned); a second kernel merges the chunk
// records of a row, takes logsumexp = max + log(sum) in float64 rounded once to
// float32, and emits log-prob = z - lse.  Order is (value desc, id asc).
#include "common.h"
#include "kernels.h"
#include "topk_common.h"
#include "topk_merge.h"

namespace spec {

namespace {

using namespace topkdev;

template <int KM>
__global__ __launch_bounds__(256) void topk_partial_kernel(const float* __restrict__ z, int n,
                                                           int ldz, int k, int chunk,
                                                           const int* __restrict__ rowmap,
                                                           float* __restrict__ pv,
                                                           int* __restrict__ pi,
                                                           Part* __restrict__ pp) {
  __shared__ float sv[4 * KM];
  __shared__ int si[4 * KM];
  __shared__ float smax[4];
  __shared__ double ssum[4];
  const int c = blockIdx.x, r = blockIdx.y, nch = gridDim.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float* row = z + (int64_t)r * ldz;
  const int* rm = rowmap ? rowmap + (int64_t)r * n : nullptr;
  const int lo = c * chunk, hi = min(n, lo + chunk);
  List<KM> L;
  L.init();
  float m = -INFINITY;
  double s = 0.0;
  auto visit = [&](float v, int id) {
    L.insert(v, id);
    if (v > m) {
      s = (m == -INFINITY ? 0.0 : s * (double)expf(m - v)) + 1.0;
      m = v;
    } else {
      s += (double)expf(v - m);
    }
  };
  // 16-byte path: each thread sees its values in batches of 16 and keeps the
  // KM best batches, ranked by their best element.  The k best elements of
  // the chunk lie in the k best batches (a batch holding one of them has a
  // best element at least as good; one holding none is worse than all of
  // them), so the batch bests are merged and then their batches rescanned.
  const bool vec = !rm && ((uintptr_t)row & 15) == 0;  // chunk starts are multiples of 256
  if (vec) {
    for_row_batches(row, lo, hi, [&](const float (&v)[16], int x0) {
      float bv = -INFINITY;
      int bi = kIdNone;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int x = x0 + 1024 * (e >> 2) + (e & 3);
        if (x < hi && better(v[e], x, bv, bi)) {
          bv = v[e];
          bi = x;
        }
      }
      if (bi != kIdNone) L.insert(bv, bi);
      lse_update16(v, m, s);
    });
  } else {
    for (int x = lo + threadIdx.x; x < hi; x += 256) visit(row[x], rm ? rm[x] : x);
  }
  // block max / sum
  float wm = wave_max(m);
  double ws = (m == -INFINITY) ? 0.0 : s * (double)expf(m - wm);
  ws = wave_sum(ws);
  if (lane == 0) {
    smax[wave] = wm;
    ssum[wave] = ws;
  }
  float wv[KM];
  int wi[KM];
  wave_merge<KM, KM>(L, k, wv, wi);
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < k) {
        sv[wave * KM + j] = wv[j];
        si[wave * KM + j] = wi[j];
      }
    }
  }
  __syncthreads();
  if (wave == 0) {
    float bm = -INFINITY;
    for (int w = 0; w < 4; ++w) bm = fmaxf(bm, smax[w]);
    double bs = 0.0;
    for (int w = 0; w < 4; ++w)
      if (smax[w] != -INFINITY) bs += ssum[w] * (double)expf(smax[w] - bm);
    List<1> one;
    one.init();
    if (lane < 4 * KM && (lane % KM) < k) {
      one.v[0] = sv[lane];
      one.i[0] = si[lane];
    }
    float ov[KM];
    int oi[KM];
    wave_merge<1, KM>(one, k, ov, oi);
    if (vec) {
      // rescan the k best batches: candidate q of lane = element q % 16 of batch q / 16
      constexpr int CPL = KM >= 4 ? KM / 4 : 1;
      List<CPL> cand;
      cand.init();
#pragma unroll
      for (int h = 0; h < CPL; ++h) {
        const int q = lane * CPL + h, j = q >> 4, e = q & 15;
        int bid = kIdNone;
#pragma unroll
        for (int jj = 0; jj < KM; ++jj)
          if (jj == j) bid = oi[jj];
        if (j < k && bid != kIdNone) {
          const int off = bid - lo;  // batch start: bid - 1024 i - e', i = (off >> 10) & 3, e' = off & 3
          const int x = bid - 1024 * ((off >> 10) & 3) - (off & 3) + 1024 * (e >> 2) + (e & 3);
          if (x < hi) cand.insert(row[x], x);
        }
      }
      wave_merge<CPL, KM>(cand, k, ov, oi);
    }
    const int64_t base = ((int64_t)r * nch + c) * KM;
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (j < k) {
          pv[base + j] = ov[j];
          pi[base + j] = oi[j];
        }
      }
      pp[(int64_t)r * nch + c] = Part{bs, bm, 0};
    }
  }
}

// Short rows (n <= kSmallRow, one chunk): one wave per row takes the k best
// and the log-probs in one launch (four rows per 256-thread block), with the
// partial kernel's per-value steps and the merge's output rule.
constexpr int kSmallRow = 512;

template <int KM>
__global__ __launch_bounds__(256) void topk_small_kernel(const float* __restrict__ z, int M, int n,
                                                         int ldz, int k,
                                                         const int* __restrict__ id_map,
                                                         const int* __restrict__ rowmap,
                                                         int* __restrict__ ids, int ldi,
                                                         float* __restrict__ logp, int ldl) {
  constexpr int U = kSmallRow / 64;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= M) return;  // whole waves
  const float* row = z + (int64_t)r * ldz;
  const int* rm = rowmap ? rowmap + (int64_t)r * n : nullptr;
  float v[U];
  int id[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {  // every load issued before the first is used
    const int x = min(lane + 64 * u, n - 1);
    v[u] = row[x];
    id[u] = rm ? rm[x] : x;
  }
  List<KM> L;
  L.init();
  float m = -INFINITY;
  double sm = 0.0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (lane + 64 * u >= n) continue;
    L.insert(v[u], id[u]);
    if (v[u] > m) {
      sm = (m == -INFINITY ? 0.0 : sm * (double)expf(m - v[u])) + 1.0;
      m = v[u];
    } else {
      sm += (double)expf(v[u] - m);
    }
  }
  const float wm = wave_max(m);
  double ws = m == -INFINITY ? 0.0 : sm * (double)expf(m - wm);
  ws = wave_sum(ws);
  const float lse = (float)((double)wm + log(ws));
  float ov[KM];
  int oi[KM];
  wave_merge<KM, KM>(L, k, ov, oi);
  if (lane < k) {
    float bv = 0.f;
    int bi = 0;
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j == lane) {
        bv = ov[j];
        bi = oi[j];
      }
    ids[(int64_t)r * ldi + lane] = rowmap ? bi : (id_map ? id_map[clampi(bi, 0, n - 1)] : bi);
    logp[(int64_t)r * ldl + lane] = bv - lse;
  }
}

// Merge of per-chunk records of a row (merge_row): one 256-thread block per row.
template <int KM>
__global__ __launch_bounds__(256) void topk_merge_kernel(int n, int k, int nch,
                                                         const float* __restrict__ pv,
                                                         const int* __restrict__ pi,
                                                         const Part* __restrict__ pp,
                                                         const int* __restrict__ id_map,
                                                         const int* __restrict__ rowmap,
                                                         int* __restrict__ ids, int ldi,
                                                         float* __restrict__ logp, int ldl) {
  merge_row<KM>(blockIdx.x, n, k, nch, pv, pi, pp, id_map, rowmap, ids, ldi, logp, ldl);
}

// ---- candidate retrieval: radix select of the K best per row ---------------
SPEC_DEV uint32_t okey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// In-place bitonic sort of P (a power of two, <= 4096) (value, id) pairs in
// LDS, best first by (value desc, id asc); 256 threads, barriers included.
SPEC_DEV void bitonic_desc(float* cv, int* ci, int P) {
  const int t = threadIdx.x;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int q = t; q < P; q += 256) {
        const int partner = q ^ stride;
        if (partner > q) {
          const bool desc = (q & size) == 0;
          const bool pb = better(cv[partner], ci[partner], cv[q], ci[q]);
          if (pb == desc) {
            const float tv = cv[q];
            cv[q] = cv[partner];
            cv[partner] = tv;
            const int ti = ci[q];
            ci[q] = ci[partner];
            ci[partner] = ti;
          }
        }
      }
      __syncthreads();
    }
  }
}

// Full-row radix select of the K best (K <= 256) of one row: four 8-bit
// histogram passes over the order-preserving keys, then the keys strictly
// above the threshold and the smallest ids at it, then a bitonic sort of the
// 256 slots.  LDS: hist[256], cv/ci[256], scan[256].
SPEC_DEV void radix_topk_row(const float* __restrict__ row, int n, int K, int* __restrict__ out,
                             int* hist, float* cv, int* ci, int* scan, int* sh /* >= 5 ints */) {
  const int t = threadIdx.x;
  int& sel_cnt = sh[0];
  int& need_s = sh[1];
  int& take_all = sh[2];
  uint32_t& prefix_s = *(uint32_t*)&sh[3];
  uint32_t& mask_s = *(uint32_t*)&sh[4];
  __syncthreads();
  if (t == 0) {
    prefix_s = 0;
    mask_s = 0;
    need_s = K;
  }
  __syncthreads();
  for (int p = 24; p >= 0; p -= 8) {
    hist[t] = 0;
    __syncthreads();
    const uint32_t pre = prefix_s, msk = mask_s;
    for (int x = t; x < n; x += 256) {
      const uint32_t key = okey(row[x]);
      if ((key & msk) == pre) atomicAdd(&hist[(key >> p) & 255], 1);
    }
    __syncthreads();
    if (t == 0) {
      int need = need_s, above = 0;
      int dd = 0;
      for (int d = 255; d >= 0; --d) {
        if (above + hist[d] >= need) {
          dd = d;
          break;
        }
        above += hist[d];
      }
      need_s = need - above;
      prefix_s = pre | ((uint32_t)dd << p);
      mask_s = msk | (255u << p);
      take_all = (p == 0) && (hist[dd] == need - above);
    }
    __syncthreads();
  }
  const uint32_t T = prefix_s;
  const int need_eq = need_s;
  if (t == 0) sel_cnt = 0;
  cv[t] = -INFINITY;
  ci[t] = kIdNone;
  __syncthreads();
  // strictly above the threshold: order does not matter (sorted below)
  for (int x = t; x < n; x += 256) {
    const float v = row[x];
    const uint32_t key = okey(v);
    if (key > T || (take_all && key == T)) {
      const int slot = atomicAdd(&sel_cnt, 1);
      cv[slot] = v;
      ci[slot] = x;
    }
  }
  __syncthreads();
  if (!take_all) {
    // ties at the threshold: the smallest ids first, in row order
    int taken = 0;
    const int base = sel_cnt;
    for (int x0 = 0; x0 < n && taken < need_eq; x0 += 256) {
      const int x = x0 + t;
      const int eq = (x < n && okey(row[x]) == T) ? 1 : 0;
      scan[t] = eq;
      __syncthreads();
      for (int o = 1; o < 256; o <<= 1) {
        const int add = t >= o ? scan[t - o] : 0;
        __syncthreads();
        scan[t] += add;
        __syncthreads();
      }
      const int before = scan[t] - eq;
      if (eq && taken + before < need_eq) {
        cv[base + taken + before] = row[x];
        ci[base + taken + before] = x;
      }
      const int tot = scan[255];
      __syncthreads();
      taken += tot;
    }
    __syncthreads();
  }
  bitonic_desc(cv, ci, 256);
  if (t < K) out[t] = ci[t];
}

// Candidate retrieval, K best of a row of n <= kLargeGroups * 16 scores.
// Pass 1 streams the row once (16-byte loads) and keeps the best value of
// every 16-value batch (group) in LDS.  The K best values of the row lie in
// the K best groups (a group holding one of them has a maximum at least that
// good), so a radix select over the group maxima gives a threshold; the
// groups at or above it (at most kLargeCand of them, else the full-row
// select runs) are rescanned and their values sorted.
// STRIPS: the score GEMM has already written every 128-column strip's
// maximum (rec[row][strip].x); by the same argument the K best values lie in
// the strips at or above the K-th best strip maximum, so pass 1 reads only
// those strips (at most kStripCand of them), in groups of 16 consecutive
// columns, instead of the whole row.
constexpr int kLargeGroups = 8192, kLargeCand = 256, kStripCand = 512, kStripW = 128;
template <bool STRIPS>
__global__ __launch_bounds__(256) void topk_large_kernel(const float* __restrict__ z, int n,
                                                         int K, const float2* __restrict__ rec,
                                                         int nstrip, int* __restrict__ ids) {
  __shared__ float gmax[kLargeGroups];
  __shared__ float cv[kLargeCand * 16];
  __shared__ int ci[kLargeCand * 16];
  __shared__ int hist[256], cg[kLargeCand];
  __shared__ int cstr[STRIPS ? kStripCand : 1];
  __shared__ int sh[8];
  const int r = blockIdx.x, t = threadIdx.x;
  const float* row = z + (int64_t)r * n;
  // K-th best key (okey) of vals[0, cnt) by radix select, left in sh[3]
  auto kth_key = [&](const float* vals, int cnt) {
    if (t == 0) {
      sh[3] = 0;  // prefix
      sh[4] = 0;  // mask
      sh[1] = K;  // still needed
    }
    __syncthreads();
    for (int p = 24; p >= 0; p -= 8) {
      hist[t] = 0;
      __syncthreads();
      const uint32_t pre = (uint32_t)sh[3], msk = (uint32_t)sh[4];
      for (int g = t; g < cnt; g += 256) {
        const uint32_t key = okey(vals[g]);
        if ((key & msk) == pre) atomicAdd(&hist[(key >> p) & 255], 1);
      }
      __syncthreads();
      // wave 0 finds the digit where the count from the top reaches `need`:
      // lane l sums digits 255 - 4 l down to 252 - 4 l, the lane sums are
      // scanned from the top and the crossing lane walks its four digits
      if (t < 64) {
        const int need = sh[1];
        const int d1 = 255 - 4 * t;
        const int c0 = hist[d1], c1 = hist[d1 - 1], c2 = hist[d1 - 2], c3 = hist[d1 - 3];
        const int c = c0 + c1 + c2 + c3;
        int cx = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int y = __shfl_up(cx, o, 64);
          if (t >= o) cx += y;
        }
        cx -= c;  // count of the digits above this lane's
        const unsigned long long bal = __ballot(cx < need && cx + c >= need);
        if (bal && t == __ffsll((long long)bal) - 1) {
          int above = cx, dd = d1 - 3;
          const int cs[4] = {c0, c1, c2, c3};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (above + cs[q] >= need) {
              dd = d1 - q;
              break;
            }
            above += cs[q];
          }
          sh[1] = need - above;
          sh[3] = (int)(pre | ((uint32_t)dd << p));
          sh[4] = (int)(msk | (255u << p));
        }
      }
      __syncthreads();
    }
    return (uint32_t)sh[3];
  };
  int G;       // groups of 16 values
  bool fast;
  if constexpr (!STRIPS) {
    G = (n + 4095) / 4096 * 256;  // batch j of thread t is group 256 j + t
    fast = ((uintptr_t)row & 15) == 0 && G <= kLargeGroups && K <= kLargeCand;
  } else {
    G = 0;
    fast = ((uintptr_t)row & 15) == 0 && nstrip == (n + kStripW - 1) / kStripW &&
           nstrip <= kLargeGroups && K <= kLargeCand;
  }
  // column of value e of group g
  auto gx = [&](int g, int e) -> int {
    if constexpr (STRIPS) return cstr[g >> 3] * kStripW + (g & 7) * 16 + e;
    else return (g >> 8) * 4096 + 4 * (g & 255) + 1024 * (e >> 2) + (e & 3);
  };
  if (fast) {
    if constexpr (!STRIPS) {
      for (int g = t; g < G; g += 256) gmax[g] = -INFINITY;
      __syncthreads();
      // two batches per thread per step (eight 16-byte loads in flight); the
      // batch at x0 = 4096 j + 4 t holds row[x0 + 1024 i + e] and is group 256 j + t
      for (int x0 = 4 * t; x0 < n; x0 += 8192) {
        float4 w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int x = x0 + 1024 * i;
          if (x + 3 < n) {
            w[i] = *(const float4*)(row + x);
          } else {
            w[i].x = x < n ? row[x] : -INFINITY;
            w[i].y = x + 1 < n ? row[x + 1] : -INFINITY;
            w[i].z = x + 2 < n ? row[x + 2] : -INFINITY;
            w[i].w = -INFINITY;
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float bm = -INFINITY;
#pragma unroll
          for (int i = 4 * h; i < 4 * h + 4; ++i)
            bm = fmaxf(fmaxf(bm, fmaxf(w[i].x, w[i].y)), fmaxf(w[i].z, w[i].w));
          const int xb = x0 + 4096 * h;
          if (xb < n) gmax[(xb >> 12) * 256 + t] = bm;
        }
      }
    } else {
      // the strips at or above the K-th best strip maximum
      const float2* pr = rec + (int64_t)r * nstrip;
      for (int q = t; q < nstrip; q += 256) gmax[q] = pr[q].x;
      __syncthreads();
      const uint32_t T1 = kth_key(gmax, nstrip);
      if (t == 0) sh[0] = 0;
      __syncthreads();
      for (int q = t; q < nstrip; q += 256)
        if (okey(gmax[q]) >= T1) {
          const int slot = atomicAdd(&sh[0], 1);
          if (slot < kStripCand) cstr[slot] = q;
        }
      __syncthreads();
      const int C1 = sh[0];
      fast = C1 <= kStripCand;
      if (fast) {
        // their groups of 16 consecutive columns (4 loads of 16 bytes each)
        G = C1 * (kStripW / 16);
        __syncthreads();  // every thread has read sh[0] and gmax
        for (int g = t; g < G; g += 256) {
          const int x0 = gx(g, 0);
          float bm = -INFINITY;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int x = x0 + 4 * i;
            float4 w;
            if (x + 3 < n) {
              w = *(const float4*)(row + x);
            } else {
              w.x = x < n ? row[x] : -INFINITY;
              w.y = x + 1 < n ? row[x + 1] : -INFINITY;
              w.z = x + 2 < n ? row[x + 2] : -INFINITY;
              w.w = -INFINITY;
            }
            bm = fmaxf(fmaxf(bm, fmaxf(w.x, w.y)), fmaxf(w.z, w.w));
          }
          gmax[g] = bm;
        }
      }
    }
  }
  if (fast) {
    // radix select of the K-th best group maximum (by key)
    kth_key(gmax, G);
    const uint32_t T = (uint32_t)sh[3];
    if (t == 0) sh[0] = 0;
    __syncthreads();
    for (int g = t; g < G; g += 256)
      if (okey(gmax[g]) >= T) {
        const int slot = atomicAdd(&sh[0], 1);
        if (slot < kLargeCand) cg[slot] = g;
      }
    __syncthreads();
    const int C = sh[0];
    if (C <= kLargeCand) {
      const int nc = C * 16;
      for (int q = t; q < nc; q += 256) {
        float v = -INFINITY;
        int id = kIdNone;
        const int g = cg[q >> 4], e = q & 15;
        const int x = gx(g, e);
        if (x < n) {
          v = row[x];
          id = x;
        }
        cv[q] = v;
        ci[q] = id;
      }
      // radix select of the K-th best candidate by the unique key
      // (okey(value) << 32) | ~id, 8 bits at a time from the top; it stops
      // once the picked digit holds exactly the number still needed, and the
      // K best are then the candidates whose key prefix is >= the picked one
      auto ckey = [&](int q) -> unsigned long long {
        return ((unsigned long long)okey(cv[q]) << 32) | (unsigned long long)(~(uint32_t)ci[q]);
      };
      if (t == 0) {
        sh[1] = K;  // still needed
        sh[5] = 0;  // done
      }
      unsigned long long pre = 0;  // picked digits so far (bits above p)
      int p = 56;
      for (;; p -= 8) {
        hist[t] = 0;
        __syncthreads();
        for (int q = t; q < nc; q += 256) {
          const unsigned long long k = ckey(q);
          if (p == 56 || (k >> (p + 8)) == pre) atomicAdd(&hist[(int)((k >> p) & 255)], 1);
        }
        __syncthreads();
        if (t < 64) {
          const int need = sh[1];
          const int d1 = 255 - 4 * t;
          const int c0 = hist[d1], c1 = hist[d1 - 1], c2 = hist[d1 - 2], c3 = hist[d1 - 3];
          const int c = c0 + c1 + c2 + c3;
          int cx = c;
#pragma unroll
          for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(cx, o, 64);
            if (t >= o) cx += y;
          }
          cx -= c;
          const unsigned long long bal = __ballot(cx < need && cx + c >= need);
          if (bal && t == __ffsll((long long)bal) - 1) {
            int above = cx, dd = d1 - 3;
            const int cs[4] = {c0, c1, c2, c3};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (above + cs[q] >= need) {
                dd = d1 - q;
                break;
              }
              above += cs[q];
            }
            sh[1] = need - above;
            sh[6] = dd;
            sh[5] = (hist[dd] == need - above) ? 1 : 0;
          }
        }
        __syncthreads();
        pre = (pre << 8) | (unsigned long long)sh[6];
        if (sh[5] || p == 0) break;
        __syncthreads();  // sh read by everyone before the next level writes it
      }
      // the K best: key prefix (bits >= p) >= pre; sort them (at most 256)
      __shared__ float sv[256];
      __shared__ int si[256];
      if (t == 0) sh[0] = 0;
      sv[t] = -INFINITY;
      si[t] = kIdNone;
      __syncthreads();
      for (int q = t; q < nc; q += 256)
        if ((ckey(q) >> p) >= pre) {
          const int slot = atomicAdd(&sh[0], 1);
          if (slot < 256) {
            sv[slot] = cv[q];
            si[slot] = ci[q];
          }
        }
      bitonic_desc(sv, si, 256);
      for (int q = t; q < K; q += 256) ids[(int64_t)r * K + q] = si[q];
      return;
    }
  }
  radix_topk_row(row, n, K, ids + (int64_t)r * K, hist, cv, ci, cg, sh);
}

template <typename T>
__global__ __launch_bounds__(256) void gather_dot_kernel(const T* __restrict__ x,
                                                         const T* __restrict__ W, int H, int V,
                                                         const int* __restrict__ ids, int K,
                                                         float* __restrict__ out) {
  const int m = blockIdx.y, j = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (j >= K) return;
  const int row = clampi(ids[(int64_t)m * K + j], 0, V - 1);
  const T* w = W + (int64_t)row * H;
  const T* xr = x + (int64_t)m * H;
  float a = 0.f;
  for (int i = lane; i < H; i += 64) a += St<T>::load(w, i) * St<T>::load(xr, i);
  a = wave_sum(a);
  if (lane == 0) out[(int64_t)m * K + j] = a;
}

// Exact rescoring, bf16, H a multiple of 512: one workgroup per row keeps the
// row's activation in registers (16-byte chunks at 8 lane + 512 i) and each
// wave walks candidates j = wave, wave + 4, ..., two at a time, with 16-byte
// weight loads.
template <int HC>  // H / 512 chunks per lane
__global__ __launch_bounds__(256) void gather_dot_vec_kernel(const bf16_t* __restrict__ x,
                                                             const bf16_t* __restrict__ W, int H,
                                                             int V, const int* __restrict__ ids,
                                                             int K, float* __restrict__ out) {
  const int m = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bf16_t* xr = x + (int64_t)m * H + lane * 8;
  float xf[HC][8];
#pragma unroll
  for (int i = 0; i < HC; ++i) {
    const u32x4_t w = *(const u32x4_t*)(xr + i * 512);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xf[i][2 * e] = __uint_as_float(w[e] << 16);
      xf[i][2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
  auto dot = [&](const u32x4_t (&wv)[HC]) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < HC; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a += xf[i][2 * e] * __uint_as_float(wv[i][e] << 16);
        a += xf[i][2 * e + 1] * __uint_as_float(wv[i][e] & 0xffff0000u);
      }
    return wave_sum(a);
  };
  for (int j = wave; j < K; j += 8) {
    const int j2 = j + 4;
    const int r1 = clampi(ids[(int64_t)m * K + j], 0, V - 1);
    const int r2 = clampi(ids[(int64_t)m * K + min(j2, K - 1)], 0, V - 1);
    u32x4_t w1[HC], w2[HC];
#pragma unroll
    for (int i = 0; i < HC; ++i) {
      w1[i] = *(const u32x4_t*)(W + (int64_t)r1 * H + lane * 8 + i * 512);
      w2[i] = *(const u32x4_t*)(W + (int64_t)r2 * H + lane * 8 + i * 512);
    }
    const float a1 = dot(w1), a2 = dot(w2);
    if (lane == 0) {
      out[(int64_t)m * K + j] = a1;
      if (j2 < K) out[(int64_t)m * K + j2] = a2;
    }
  }
}

// Vocab top-k from the per-strip records (max, sum exp(v - max)) of the tiled
// LM head, one 256-thread workgroup per row.  Strip order by (max desc, strip
// asc) is the order of the strips' best elements by (value desc, id asc), so
// the k best elements of the row lie in its k best strips: those are picked
// from the records and only their k * 128 logits are rescanned.  The row
// logsumexp comes from the records alone (merged across waves in float64).

// The same selection by one wave per row (four rows per 256-thread block):
// the row's records and its k best strips' logits each pass through the
// lanes once, with no exchange between waves and no barrier.
template <int KM>
__global__ __launch_bounds__(256) void topk_strip_merge_wave_kernel(
    int M, int n, int k, int nstrip, const float* __restrict__ z, const float2* __restrict__ rec,
    const int* __restrict__ id_map, int* __restrict__ ids, int ldi, float* __restrict__ logp,
    int ldl) {
  constexpr float kL2e = 1.4426950408889634f;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= M) return;  // whole waves
  const float2* pr = rec + (int64_t)r * nstrip;
  const float* row = z + (int64_t)r * n;
  List<KM> L;
  L.init();
  float m = -INFINITY, s = 0.f;
  // eight records per lane in flight at a time, then inserted
  for (int j0 = lane; j0 < nstrip; j0 += 64 * 8) {
    float2 p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) p[u] = pr[min(j0 + 64 * u, nstrip - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (j0 + 64 * u >= nstrip || p[u].x == -INFINITY) continue;
      L.insert(p[u].x, j0 + 64 * u);
      const float nm = fmaxf(m, p[u].x);
      s = (m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f((m - nm) * kL2e)) +
          p[u].y * __builtin_amdgcn_exp2f((p[u].x - nm) * kL2e);
      m = nm;
    }
  }
  float sv[KM];
  int si[KM];
  wave_merge<KM, KM>(L, k, sv, si);  // the k best strips, in every lane
  // candidate h of the lane: column lane + 64 (h & 1) of the (h / 2)-th best strip
  constexpr int CPL = KM * kStripW / 64;
  float cz[CPL];
  int cx[CPL];
#pragma unroll
  for (int h = 0; h < CPL; ++h) {
    const int st = (h >> 1) < k ? si[h >> 1] : kIdNone;
    cx[h] = st != kIdNone ? st * kStripW + lane + 64 * (h & 1) : n;
    cz[h] = row[min(cx[h], n - 1)];
  }
  // row logsumexp from the records (lanes combined in float64)
  const float wm = wave_max(m);
  double ws = m == -INFINITY ? 0.0 : (double)s * exp((double)m - (double)wm);
  ws = wave_sum(ws);
  const double lse = (double)wm + log(ws);
  List<KM> C;
  C.init();
#pragma unroll
  for (int h = 0; h < CPL; ++h)
    if (cx[h] < n) C.insert(cz[h], cx[h]);
  float ov[KM];
  int oi[KM];
  wave_merge<KM, KM>(C, k, ov, oi);
  if (lane < k) {
    float v = 0.f;
    int id = 0;
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j == lane) {
        v = ov[j];
        id = oi[j];
      }
    ids[(int64_t)r * ldi + lane] = id_map ? id_map[clampi(id, 0, n - 1)] : id;
    logp[(int64_t)r * ldl + lane] = (float)((double)v - lse);
  }
}

template <int KM>
__global__ __launch_bounds__(256) void topk_strip_merge_kernel(int n, int k, int nstrip,
                                                               const float* __restrict__ z,
                                                               const float2* __restrict__ rec,
                                                               const int* __restrict__ id_map,
                                                               int* __restrict__ ids, int ldi,
                                                               float* __restrict__ logp, int ldl) {
  constexpr float kL2e = 1.4426950408889634f;
  __shared__ float sv[4 * KM];
  __shared__ int si[4 * KM];
  __shared__ float smax[4], ssum[4];
  __shared__ int sel[KM];
  const int r = blockIdx.x, t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const float2* pr = rec + (int64_t)r * nstrip;
  const float* row = z + (int64_t)r * n;
  List<KM> L;
  L.init();
  float m = -INFINITY, s = 0.f;
  // eight records per thread in flight at a time (a row has ~1200 strips of
  // the 152K vocabulary), then inserted
  for (int j0 = t; j0 < nstrip; j0 += 256 * 8) {
    float2 p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      p[u] = j0 + 256 * u < nstrip ? pr[j0 + 256 * u] : make_float2(-INFINITY, 0.f);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (p[u].x == -INFINITY) continue;
      L.insert(p[u].x, j0 + 256 * u);
      const float nm = fmaxf(m, p[u].x);
      s = (m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f((m - nm) * kL2e)) +
          p[u].y * __builtin_amdgcn_exp2f((p[u].x - nm) * kL2e);
      m = nm;
    }
  }
  const float wm = wave_max(m);
  const float ws = wave_sum(m == -INFINITY ? 0.f : s * __builtin_amdgcn_exp2f((m - wm) * kL2e));
  float wv[KM];
  int wi[KM];
  wave_merge<KM, KM>(L, k, wv, wi);
  if (lane == 0) {
    smax[wave] = wm;
    ssum[wave] = ws;
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      sv[wave * KM + j] = j < k ? wv[j] : -INFINITY;
      si[wave * KM + j] = j < k ? wi[j] : kIdNone;
    }
  }
  __syncthreads();
  if (wave == 0) {  // the k best strips
    List<1> one;
    one.init();
    if (lane < 4 * KM) {
      one.v[0] = sv[lane];
      one.i[0] = si[lane];
    }
    float ov[KM];
    int oi[KM];
    wave_merge<1, KM>(one, k, ov, oi);
    if (lane < KM) {
      int id = kIdNone;
#pragma unroll
      for (int j = 0; j < KM; ++j)
        if (j == lane && j < k) id = oi[j];
      sel[lane] = id;
    }
  }
  __syncthreads();
  // candidate q = t + 256 h: column q % 128 of the (q / 128)-th best strip;
  // the loads go out first, the row logsumexp is taken while they fly
  constexpr int CPT = KM * kStripW / 256;
  float cz[CPT];
  int cx[CPT];
#pragma unroll
  for (int h = 0; h < CPT; ++h) {
    const int q = t + 256 * h, rank = q / kStripW;
    const int st = sel[rank];
    cx[h] = rank < k && st != kIdNone ? st * kStripW + q % kStripW : n;
    cz[h] = cx[h] < n ? row[cx[h]] : -INFINITY;
  }
  double lse = 0.0;
  if (wave == 0) {
    float bm = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) bm = fmaxf(bm, smax[w]);
    double bs = 0.0;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (smax[w] != -INFINITY) bs += (double)ssum[w] * exp((double)smax[w] - (double)bm);
    lse = (double)bm + log(bs);
  }
  List<KM < CPT ? KM : CPT> cand;
  cand.init();
#pragma unroll
  for (int h = 0; h < CPT; ++h)
    if (cx[h] < n) cand.insert(cz[h], cx[h]);
  float cv[KM];
  int cid[KM];
  wave_merge<KM < CPT ? KM : CPT, KM>(cand, k, cv, cid);
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      sv[wave * KM + j] = j < k ? cv[j] : -INFINITY;
      si[wave * KM + j] = j < k ? cid[j] : kIdNone;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  List<1> one;
  one.init();
  if (lane < 4 * KM) {
    one.v[0] = sv[lane];
    one.i[0] = si[lane];
  }
  float ov[KM];
  int oi[KM];
  wave_merge<1, KM>(one, k, ov, oi);
  if (lane < k) {
    float v = 0.f;
    int id = 0;
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j == lane) {
        v = ov[j];
        id = oi[j];
      }
    ids[(int64_t)r * ldi + lane] = id_map ? id_map[clampi(id, 0, n - 1)] : id;
    logp[(int64_t)r * ldl + lane] = (float)((double)v - lse);
  }
}

template <int KM>
hipError_t launch_topk(const float* z, int M, int n, int ldz, int k, const int* id_map,
                       const int* rowmap, int* ids, int ldi, float* logp, int ldl, void* part,
                       int nch, int chunk, hipStream_t s) {
  if (nch == 1 && n >= 1 && n <= kSmallRow) {
    SPEC_LAUNCH(topk_small_kernel<KM>, dim3((M + 3) / 4), dim3(256), 0, s, z, M, n, ldz, k, id_map,
                rowmap, ids, ldi, logp, ldl);
    return hipGetLastError();
  }
  float* pv = (float*)part;
  int* pi = (int*)(pv + (size_t)M * nch * KM);
  Part* pp = (Part*)(pi + (size_t)M * nch * KM);
  SPEC_LAUNCH(topk_partial_kernel<KM>, dim3(nch, M), dim3(256), 0, s, z, n, ldz, k, chunk,
                     rowmap, pv, pi, pp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SPEC_LAUNCH(topk_merge_kernel<KM>, dim3(M), dim3(256), 0, s, n, k, nch, pv, pi, pp,
                     id_map, rowmap, ids, ldi, logp, ldl);
  return hipGetLastError();
}

}  // namespace

void topk_plan(int M, int n, int* nch, int* chunk) {
  int c = (2048 + M - 1) / M;
  const int maxc = std::max(1, (n + 1023) / 1024);
  c = std::max(1, std::min(c, maxc));
  int ch = (n + c - 1) / c;
  ch = (ch + 255) / 256 * 256;
  *chunk = ch;
  *nch = (n + ch - 1) / ch;
}

size_t topk_part_bytes(int M, int nch, int kmax) {
  // 8-byte aligned: values + ids, then one Part per (row, chunk)
  size_t b = (size_t)M * nch * kmax * 8;
  b = (b + 15) / 16 * 16;
  return b + (size_t)M * nch * sizeof(Part);
}

hipError_t topk(const float* z, int M, int n, int ldz, int k, const int* id_map, int* ids,
                int ldi, float* logp, int ldl, void* part, int nch, int chunk, hipStream_t s) {
  return topk_rows(z, M, n, ldz, k, id_map, nullptr, ids, ldi, logp, ldl, part, nch, chunk, s);
}

// rowmap (optional, [M, n]): per-row ids used both as tie-break and as output.
hipError_t topk_rows(const float* z, int M, int n, int ldz, int k, const int* id_map,
                     const int* rowmap, int* ids, int ldi, float* logp, int ldl, void* part,
                     int nch, int chunk, hipStream_t s) {
  if (k <= 1)
    return launch_topk<1>(z, M, n, ldz, k, id_map, rowmap, ids, ldi, logp, ldl, part, nch, chunk, s);
  if (k <= 2)
    return launch_topk<2>(z, M, n, ldz, k, id_map, rowmap, ids, ldi, logp, ldl, part, nch, chunk, s);
  if (k <= 4)
    return launch_topk<4>(z, M, n, ldz, k, id_map, rowmap, ids, ldi, logp, ldl, part, nch, chunk, s);
  if (k <= 8)
    return launch_topk<8>(z, M, n, ldz, k, id_map, rowmap, ids, ldi, logp, ldl, part, nch, chunk, s);
  return launch_topk<16>(z, M, n, ldz, k, id_map, rowmap, ids, ldi, logp, ldl, part, nch, chunk, s);
}

hipError_t topk_merge_strips(const float* z, int M, int n, int k, int nstrip, int sw,
                             const void* rec, const int* id_map, int* ids, int ldi, float* logp,
                             int ldl, hipStream_t s) {
  if (k < 1 || k > 8 || sw != kStripW || nstrip != (n + kStripW - 1) / kStripW)
    return hipErrorInvalidValue;
  // up to 512 strips (vocabularies up to 65536) a wave per row; beyond, a
  // block per row, four waves sharing the records
  if (nstrip <= 512) {
    SPEC_LAUNCH(topk_strip_merge_wave_kernel<8>, dim3((M + 3) / 4), dim3(256), 0, s, M, n, k,
                nstrip, z, (const float2*)rec, id_map, ids, ldi, logp, ldl);
  } else {
    SPEC_LAUNCH(topk_strip_merge_kernel<8>, dim3(M), dim3(256), 0, s, n, k, nstrip, z,
                (const float2*)rec, id_map, ids, ldi, logp, ldl);
  }
  return hipGetLastError();
}

hipError_t topk_merge_records(int M, int n, int k, int km, int nch, void* part, const int* id_map,
                              int* ids, int ldi, float* logp, int ldl, hipStream_t s) {
  float* pv = (float*)part;
  int* pi = (int*)(pv + (size_t)M * nch * km);
  Part* pp = (Part*)(pi + (size_t)M * nch * km);
  if (km == 1) {
    SPEC_LAUNCH(topk_merge_kernel<1>, dim3(M), dim3(256), 0, s, n, k, nch, pv, pi, pp, id_map,
                       nullptr, ids, ldi, logp, ldl);
  } else {
    SPEC_LAUNCH(topk_merge_kernel<8>, dim3(M), dim3(256), 0, s, n, k, nch, pv, pi, pp, id_map,
                       nullptr, ids, ldi, logp, ldl);
  }
  return hipGetLastError();
}

hipError_t topk_large(const float* z, int M, int n, int K, int* ids, void* part, hipStream_t s) {
  (void)part;
  SPEC_LAUNCH(topk_large_kernel<false>, dim3(M), dim3(256), 0, s, z, n, K, nullptr, 0, ids);
  return hipGetLastError();
}

hipError_t topk_large_strips(const float* z, int M, int n, int K, const void* rec, int nstrip,
                             int* ids, hipStream_t s) {
  if (!rec || nstrip != (n + kStripW - 1) / kStripW) return hipErrorInvalidValue;
  SPEC_LAUNCH(topk_large_kernel<true>, dim3(M), dim3(256), 0, s, z, n, K, (const float2*)rec,
              nstrip, ids);
  return hipGetLastError();
}

hipError_t gather_dot(bool bf16, const void* x, const void* W, int H, int V, const int* ids, int M,
                      int K, float* out, hipStream_t s) {
  const bool al = ((uintptr_t)x & 15) == 0 && ((uintptr_t)W & 15) == 0;
  if (bf16 && al && H == 4096) {
    SPEC_LAUNCH(gather_dot_vec_kernel<8>, dim3(M), dim3(256), 0, s, (const bf16_t*)x,
                       (const bf16_t*)W, H, V, ids, K, out);
    return hipGetLastError();
  }
  if (bf16 && al && H == 2048) {
    SPEC_LAUNCH(gather_dot_vec_kernel<4>, dim3(M), dim3(256), 0, s, (const bf16_t*)x,
                       (const bf16_t*)W, H, V, ids, K, out);
    return hipGetLastError();
  }
  dim3 grid((K + 3) / 4, M);
  if (bf16) {
    SPEC_LAUNCH(gather_dot_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)x,
                       (const bf16_t*)W, H, V, ids, K, out);
  } else {
    SPEC_LAUNCH(gather_dot_kernel<float>, grid, dim3(256), 0, s, (const float*)x,
                       (const float*)W, H, V, ids, K, out);
  }
  return hipGetLastError();
}

}  // namespace spec

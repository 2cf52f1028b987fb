// Merge of the per-chunk top-k records of one row by a workgroup, shared by
// the vocab top-k kernels and the fused chain-pass tail.
#pragma once

#include "topk_common.h"

namespace spec {
namespace topkdev {

// Merge of per-chunk records (top-KM lists with ids, and (sum exp, max)) of
// row r by a 256-thread block: ids (through id_map, unless rowmap ids are
// already output ids) and log-probs of the row's k best.  Every thread of the
// block must call it (it meets at a barrier); on return the row's outputs are
// written by wave 0, and, given an LDS pair bcast, the best id and its
// log-prob (float bits) are stored there too (visible after a barrier).
template <int KM>
SPEC_DEV void merge_row(int r, int n, int k, int nch, const float* __restrict__ pv,
                        const int* __restrict__ pi, const Part* __restrict__ pp,
                        const int* __restrict__ id_map, const int* __restrict__ rowmap,
                        int* __restrict__ ids, int ldi, float* __restrict__ logp, int ldl,
                        int* bcast = nullptr) {
  __shared__ float sv[4 * KM];
  __shared__ int si[4 * KM];
  __shared__ float smax[4];
  __shared__ double ssum[4];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int total = nch * KM;
  const float* rv = pv + (int64_t)r * total;
  const int* ri = pi + (int64_t)r * total;
  List<KM> L;
  L.init();
  float m = -INFINITY;
  double s = 0.0;
  // rounds of U list entries and U chunk records per thread, every load of a
  // round issued before any is used (thread t takes entries t, t + 256, ...)
  constexpr int U = 8;
  const int rounds = (max(total, nch) + 256 * U - 1) / (256 * U);
  for (int rd = 0; rd < rounds; ++rd) {
    const int x0 = rd * 256 * U + t;
    float v[U];
    int id[U];
    Part q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int x = x0 + 256 * u;
      const bool ok = x < total && (x % KM) < k;
      v[u] = ok ? rv[x] : -INFINITY;
      id[u] = ok ? ri[x] : kIdNone;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = x0 + 256 * u;
      q[u] = c < nch ? pp[(int64_t)r * nch + c] : Part{0.0, -INFINITY, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) L.insert(v[u], id[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const Part p = q[u];
      if (p.m == -INFINITY) continue;
      if (p.m > m) {
        s = (m == -INFINITY ? 0.0 : s * exp((double)m - (double)p.m)) + p.s;
        m = p.m;
      } else {
        s += p.s * exp((double)p.m - (double)m);
      }
    }
  }
  const float wm = wave_max(m);
  double ws = m == -INFINITY ? 0.0 : s * exp((double)m - (double)wm);
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
  if (wave != 0) return;
  float bm = -INFINITY;
  for (int w = 0; w < 4; ++w) bm = fmaxf(bm, smax[w]);
  double bs = 0.0;
  for (int w = 0; w < 4; ++w)
    if (smax[w] != -INFINITY) bs += ssum[w] * exp((double)smax[w] - (double)bm);
  const float lse = (float)((double)bm + log(bs));
  List<1> one;
  one.init();
  if (lane < 4 * KM && (lane % KM) < k) {
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
    // with per-row ids the tie-break id is already the output id
    const int out = rowmap ? id : (id_map ? id_map[clampi(id, 0, n - 1)] : id);
    ids[(int64_t)r * ldi + lane] = out;
    logp[(int64_t)r * ldl + lane] = v - lse;
    if (bcast && lane == 0) {
      bcast[0] = out;
      bcast[1] = __float_as_int(v - lse);
    }
  }
}

}  // namespace topkdev
}  // namespace spec

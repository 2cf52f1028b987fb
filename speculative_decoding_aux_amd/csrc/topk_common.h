// Device helpers shared by the vocab top-k kernels and the fused LM-head
// epilogue: sorted per-thread (value desc, id asc) lists, wave-wide merges,
// and the per-chunk (sum exp, max) record of a logsumexp.
#pragma once

#include "common.h"

namespace spec {
namespace topkdev {

constexpr int kIdNone = 0x7fffffff;

template <int KM>
struct List {
  float v[KM];
  int i[KM];
  SPEC_DEV void init() {
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      v[j] = -INFINITY;
      i[j] = kIdNone;
    }
  }
  SPEC_DEV void insert(float x, int id) {
    if (!better(x, id, v[KM - 1], i[KM - 1])) return;
#pragma unroll
    for (int j = KM - 1; j >= 1; --j) {
      const bool bp = better(x, id, v[j - 1], i[j - 1]);
      const bool bc = better(x, id, v[j], i[j]);
      const float nv = bp ? v[j - 1] : (bc ? x : v[j]);
      const int ni = bp ? i[j - 1] : (bc ? id : i[j]);
      v[j] = nv;
      i[j] = ni;
    }
    if (better(x, id, v[0], i[0])) {
      v[0] = x;
      i[0] = id;
    }
  }
  SPEC_DEV void pop() {
#pragma unroll
    for (int j = 0; j < KM - 1; ++j) {
      v[j] = v[j + 1];
      i[j] = i[j + 1];
    }
    v[KM - 1] = -INFINITY;
    i[KM - 1] = kIdNone;
  }
};

// Wave-wide best (value, id) of each lane's head: within each row of 16 lanes
// by DPP exchanges, then the four rows' bests read back as scalars (the order
// (value desc, id asc) is total, so the combining order does not matter).
template <int CTRL>
SPEC_DEV void best_step(float& v, int& id) {
  const float ov = dpp_row<CTRL>(v);
  const int oi = dpp_row<CTRL>(id);
  if (better(ov, oi, v, id)) {
    v = ov;
    id = oi;
  }
}
SPEC_DEV void wave_best(float& v, int& id) {
  best_step<0xB1>(v, id);
  best_step<0x4E>(v, id);
  best_step<0x141>(v, id);
  best_step<0x140>(v, id);
  float bv = lane_f(v, 0);
  int bi = __builtin_amdgcn_readlane(id, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) {
    const float ov = lane_f(v, r);
    const int oi = __builtin_amdgcn_readlane(id, r);
    if (better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  v = bv;
  id = bi;
}

// Merge the lists of the wave: the k best go to (outv, outi) (valid in every lane).
template <int KM, int KO>
SPEC_DEV void wave_merge(List<KM>& L, int k, float (&outv)[KO], int (&outi)[KO]) {
#pragma unroll
  for (int r = 0; r < KO; ++r) {
    if (r < k) {
      float bv = L.v[0];
      int bi = L.i[0];
      wave_best(bv, bi);
      outv[r] = bv;
      outi[r] = bi;
      if (L.i[0] == bi && L.v[0] == bv) L.pop();
    }
  }
}

struct Part {   // per (row, chunk)
  double s;
  float m;
  int pad;
};


}  // namespace topkdev
}  // namespace spec

// Row helpers of the draft-layer prologue and RMSNorm (16-byte vectors of a
// row held in registers, 256 threads per row), shared by the norm kernels and
// the fused chain-pass tail.
#pragma once

#include "common.h"

namespace spec {
namespace normdev {

constexpr int kVecPerThread = 4;  // 256 threads x 4 x 16 B

template <typename T> struct V16;
template <> struct V16<float> {
  static constexpr int N = 4;
  static SPEC_DEV float get(const u32x4_t& w, int e) { return __uint_as_float(w[e]); }
  static SPEC_DEV void set(u32x4_t& w, int e, float v) { w[e] = __float_as_uint(v); }
};
template <> struct V16<bf16_t> {
  static constexpr int N = 8;
  static SPEC_DEV float get(const u32x4_t& w, int e) {
    const uint32_t x = w[e >> 1];
    return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
  }
  static SPEC_DEV void set(u32x4_t& w, int e, float v) {
    const uint32_t b = f32_to_bf16(v);
    w[e >> 1] = (e & 1) ? ((w[e >> 1] & 0xffffu) | (b << 16)) : ((w[e >> 1] & 0xffff0000u) | b);
  }
};

template <typename T>
SPEC_DEV void load_row(const T* x, int nvec, u32x4_t (&v)[kVecPerThread]) {
#pragma unroll
  for (int j = 0; j < kVecPerThread; ++j) {
    const int i = threadIdx.x + 256 * j;
    v[j] = i < nvec ? ((const u32x4_t*)x)[i] : u32x4_t{0u, 0u, 0u, 0u};
  }
}

template <typename T>
SPEC_DEV double sumsq(const u32x4_t (&v)[kVecPerThread]) {
  double a = 0.0;
#pragma unroll
  for (int j = 0; j < kVecPerThread; ++j)
#pragma unroll
    for (int e = 0; e < V16<T>::N; ++e) {
      const double x = V16<T>::get(v[j], e);
      a += x * x;
    }
  return a;
}

// y = x * scale * w for the vectors held in registers, stored with 16-byte stores.
template <typename T>
SPEC_DEV void scale_store(const u32x4_t (&v)[kVecPerThread], double sc, const T* w, T* y, int nvec) {
#pragma unroll
  for (int j = 0; j < kVecPerThread; ++j) {
    const int i = threadIdx.x + 256 * j;
    if (i >= nvec) continue;
    const u32x4_t wv = ((const u32x4_t*)w)[i];
    u32x4_t o = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < V16<T>::N; ++e)
      V16<T>::set(o, e, (float)((double)V16<T>::get(v[j], e) * sc * (double)V16<T>::get(wv, e)));
    ((u32x4_t*)y)[i] = o;
  }
}

// The same with the weight vectors already in registers (loaded by load_row).
template <typename T>
SPEC_DEV void scale_store(const u32x4_t (&v)[kVecPerThread], double sc, const u32x4_t (&wv)[kVecPerThread],
                          T* y, int nvec) {
#pragma unroll
  for (int j = 0; j < kVecPerThread; ++j) {
    const int i = threadIdx.x + 256 * j;
    if (i >= nvec) continue;
    u32x4_t o = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < V16<T>::N; ++e)
      V16<T>::set(o, e, (float)((double)V16<T>::get(v[j], e) * sc * (double)V16<T>::get(wv[j], e)));
    ((u32x4_t*)y)[i] = o;
  }
}

// Prologue of row r by a 256-thread block (every thread calls it: it meets at
// a barrier).
template <typename T>
SPEC_DEV void prologue_row(int r, const T* __restrict__ embed, int V, const int* __restrict__ tok,
                           const T* __restrict__ hid, const int* __restrict__ src,
                           const T* __restrict__ w_in, const T* __restrict__ w_hid, float eps,
                           int H, T* __restrict__ gout, T* __restrict__ cout) {
  __shared__ double red[2][4];
  const int nvec = H / V16<T>::N;
  const int t = clampi(tok[r], 0, V - 1);
  const T* e = embed + (int64_t)t * H;
  const T* g = hid + (int64_t)(src ? src[r] : r) * H;
  u32x4_t ev[kVecPerThread], gv[kVecPerThread];
  load_row<T>(e, nvec, ev);
  load_row<T>(g, nvec, gv);
  double se = wave_sum(sumsq<T>(ev)), sg = wave_sum(sumsq<T>(gv));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][w] = se;
    red[1][w] = sg;
  }
  __syncthreads();
  se = red[0][0] + red[0][1] + red[0][2] + red[0][3];
  sg = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  const double ce = 1.0 / sqrt(se / H + (double)eps);
  const double cg = 1.0 / sqrt(sg / H + (double)eps);
  T* c = cout + (int64_t)r * 2 * H;
  scale_store<T>(ev, ce, w_in, c, nvec);
  scale_store<T>(gv, cg, w_hid, c + H, nvec);
  T* go = gout + (int64_t)r * H;
  if (go != g) {
#pragma unroll
    for (int j = 0; j < kVecPerThread; ++j) {
      const int i = threadIdx.x + 256 * j;
      if (i < nvec) ((u32x4_t*)go)[i] = gv[j];
    }
  }
}

}  // namespace normdev
}  // namespace spec

// Fused draft-layer prologue and RMSNorm rows.
//
// Prologue (one block per row): gather the layer's hidden input g (the FC
// output in initial mode, a previous pass's pre-norm state in recurrent mode),
// keep it as the attention residual, and build the 2H-wide decoder input
// [RMSNorm(embed[token]) * w_in | RMSNorm(g) * w_hid].
// Rows are read once with 16-byte loads into registers (H <= 1024 vectors per
// row: 8192 bf16 or 4096 float32 values); the sums of squares and the scale
// 1/sqrt(mean + eps) are taken in float64 and each output is rounded once to
// the storage type.
#include "common.h"
#include "kernels.h"
#include "norm_common.h"

namespace spec {

namespace {

using namespace normdev;

template <typename T>
__global__ __launch_bounds__(256) void prologue_kernel(const T* __restrict__ embed, int V,
                                                       const int* __restrict__ tok,
                                                       const T* __restrict__ hid,
                                                       const int* __restrict__ src,
                                                       const T* __restrict__ w_in,
                                                       const T* __restrict__ w_hid, float eps,
                                                       int H, T* __restrict__ gout,
                                                       T* __restrict__ cout) {
  prologue_row<T>(blockIdx.x, embed, V, tok, hid, src, w_in, w_hid, eps, H, gout, cout);
}

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* __restrict__ x,
                                                      const T* __restrict__ w, float eps, int H,
                                                      T* __restrict__ y) {
  __shared__ double red[4];
  const int r = blockIdx.x;
  const int nvec = H / V16<T>::N;
  u32x4_t v[kVecPerThread];
  load_row<T>(x + (int64_t)r * H, nvec, v);
  const double s = wave_sum(sumsq<T>(v));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  const double tot = red[0] + red[1] + red[2] + red[3];
  scale_store<T>(v, 1.0 / sqrt(tot / H + (double)eps), w, y + (int64_t)r * H, nvec);
}

// Split-K reduction, residual and RMSNorm of one row in one pass (one 512-thread
// block per row): y = round(sum_s P[s][r] + resid[r]) is stored, and the row's
// RMSNorm of the rounded y (sum of squares in float64, as rmsnorm_kernel) goes
// to yn.  The splits are summed in order s = 0, 1, ... per element.
constexpr int kResidThreads = 512, kResidVec = 2;  // 512 threads x 2 x 16 B of output

template <typename T>
__global__ __launch_bounds__(kResidThreads) void resid_norm_kernel(
    const float* __restrict__ P, int nsplit, int M, int H, const T* __restrict__ R,
    T* __restrict__ y, const T* __restrict__ w, float eps, T* __restrict__ yn) {
  constexpr int NV = V16<T>::N;
  __shared__ double red[kResidThreads / 64];
  const int r = blockIdx.x;
  const int nvec = H / NV;
  const int64_t ss = (int64_t)M * H;
  u32x4_t v[kResidVec];
  double sq = 0.0;
#pragma unroll
  for (int j = 0; j < kResidVec; ++j) {
    const int i = threadIdx.x + kResidThreads * j;
    v[j] = u32x4_t{0u, 0u, 0u, 0u};
    if (i >= nvec) continue;
    float a[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) a[e] = 0.f;
    const float4* p = (const float4*)(P + (int64_t)r * H + (int64_t)i * NV);
    for (int sp0 = 0; sp0 < nsplit; sp0 += 8) {  // eight splits' loads in flight
      float4 x[8][NV / 4];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int q = 0; q < NV / 4; ++q)
          x[u][q] = sp0 + u < nsplit ? p[(sp0 + u) * (ss / 4) + q] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int q = 0; q < NV / 4; ++q) {
          a[4 * q] += x[u][q].x;
          a[4 * q + 1] += x[u][q].y;
          a[4 * q + 2] += x[u][q].z;
          a[4 * q + 3] += x[u][q].w;
        }
    }
    const u32x4_t rv = ((const u32x4_t*)(R + (int64_t)r * H))[i];
    u32x4_t o = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < NV; ++e) V16<T>::set(o, e, a[e] + V16<T>::get(rv, e));
    ((u32x4_t*)(y + (int64_t)r * H))[i] = o;
    v[j] = o;
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      const double x = V16<T>::get(o, e);
      sq += x * x;
    }
  }
  sq = wave_sum(sq);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = sq;
  __syncthreads();
  double tot = 0.0;
#pragma unroll
  for (int k = 0; k < kResidThreads / 64; ++k) tot += red[k];
  const double sc = 1.0 / sqrt(tot / H + (double)eps);
#pragma unroll
  for (int j = 0; j < kResidVec; ++j) {
    const int i = threadIdx.x + kResidThreads * j;
    if (i >= nvec) continue;
    const u32x4_t wv = ((const u32x4_t*)w)[i];
    u32x4_t o = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < NV; ++e)
      V16<T>::set(o, e, (float)((double)V16<T>::get(v[j], e) * sc * (double)V16<T>::get(wv, e)));
    ((u32x4_t*)(yn + (int64_t)r * H))[i] = o;
  }
}

}  // namespace

hipError_t prologue(bool bf16, const void* embed, int V, const int* tok, const void* hid,
                    const int* src, const void* w_in, const void* w_hid, float eps, int M, int H,
                    void* gout, void* cout, hipStream_t s) {
  if (bf16) {
    SPEC_LAUNCH(prologue_kernel<bf16_t>, dim3(M), dim3(256), 0, s, (const bf16_t*)embed, V,
                       tok, (const bf16_t*)hid, src, (const bf16_t*)w_in, (const bf16_t*)w_hid,
                       eps, H, (bf16_t*)gout, (bf16_t*)cout);
  } else {
    SPEC_LAUNCH(prologue_kernel<float>, dim3(M), dim3(256), 0, s, (const float*)embed, V,
                       tok, (const float*)hid, src, (const float*)w_in, (const float*)w_hid, eps,
                       H, (float*)gout, (float*)cout);
  }
  return hipGetLastError();
}

hipError_t rmsnorm(bool bf16, const void* x, const void* w, float eps, int M, int H, void* y,
                   hipStream_t s) {
  if (bf16) {
    SPEC_LAUNCH(rmsnorm_kernel<bf16_t>, dim3(M), dim3(256), 0, s, (const bf16_t*)x,
                       (const bf16_t*)w, eps, H, (bf16_t*)y);
  } else {
    SPEC_LAUNCH(rmsnorm_kernel<float>, dim3(M), dim3(256), 0, s, (const float*)x,
                       (const float*)w, eps, H, (float*)y);
  }
  return hipGetLastError();
}

// One workgroup per row pulls the row's nsplit partials alone: worth it with
// enough rows to spread over the chip, or with few partials per row (at most
// 8 splits of 4096 float32: below that the column-parallel epilogue plus a
// separate norm is faster).
bool resid_norm_ok(bool bf16, int M, int H, int nsplit, const void* P, const void* R,
                   const void* y, const void* w, const void* yn) {
  const int nv = bf16 ? 8 : 4;
  const auto al = [](const void* q) { return ((uintptr_t)q & 15u) == 0; };
  const bool few = (int64_t)nsplit * H * 4 <= (int64_t)kResidNormSplit * 4096 * 4;
  return (M >= 64 || few) && H % nv == 0 && H / nv <= kResidThreads * kResidVec && al(P) &&
         al(R) && al(y) && al(w) && al(yn);
}

hipError_t resid_norm(bool bf16, const float* P, int nsplit, int M, int H, const void* R, void* y,
                      const void* w, float eps, void* yn, hipStream_t s) {
  if (!resid_norm_ok(bf16, M, H, nsplit, P, R, y, w, yn) || nsplit < 1) return hipErrorInvalidValue;
  if (bf16) {
    SPEC_LAUNCH(resid_norm_kernel<bf16_t>, dim3(M), dim3(kResidThreads), 0, s, P, nsplit, M, H,
                (const bf16_t*)R, (bf16_t*)y, (const bf16_t*)w, eps, (bf16_t*)yn);
  } else {
    SPEC_LAUNCH(resid_norm_kernel<float>, dim3(M), dim3(kResidThreads), 0, s, P, nsplit, M, H,
                (const float*)R, (float*)y, (const float*)w, eps, (float*)yn);
  }
  return hipGetLastError();
}

}  // namespace spec

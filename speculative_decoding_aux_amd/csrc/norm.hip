// Fused draft-layer prologue and RMSNorm rows.
//
// Prologue (one block per row): gather the layer's hidden input g (the FC
// output in initial mode, a previous pass's pre-norm state in recurrent mode),
// keep it as the attention residual, and build the 2H-wide decoder input
// [RMSNorm(embed[token]) * w_in | RMSNorm(g) * w_hid].
// The sums of squares and the scale 1/sqrt(mean + eps) are taken in float64;
// each output is rounded once to the storage type.
#include "common.h"
#include "kernels.h"

namespace spec {

namespace {

template <typename T>
SPEC_DEV double row_rscale(const T* x, int H, float eps, double* red) {
  double ss = 0.0;
  for (int i = threadIdx.x; i < H; i += blockDim.x) {
    const double v = St<T>::load(x, i);
    ss += v * v;
  }
  const double tot = block_sum(ss, red);
  return 1.0 / sqrt(tot / H + (double)eps);
}

template <typename T>
__global__ __launch_bounds__(256) void prologue_kernel(const T* __restrict__ embed, int V,
                                                       const int* __restrict__ tok,
                                                       const T* __restrict__ hid,
                                                       const int* __restrict__ src,
                                                       const T* __restrict__ w_in,
                                                       const T* __restrict__ w_hid, float eps,
                                                       int H, T* __restrict__ gout,
                                                       T* __restrict__ cout) {
  __shared__ double red[16];
  const int r = blockIdx.x;
  const int t = clampi(tok[r], 0, V - 1);
  const T* e = embed + (int64_t)t * H;
  const T* g = hid + (int64_t)(src ? src[r] : r) * H;
  T* go = gout + (int64_t)r * H;
  T* c = cout + (int64_t)r * 2 * H;
  const double se = row_rscale(e, H, eps, red);
  const double sg = row_rscale(g, H, eps, red);
  for (int i = threadIdx.x; i < H; i += blockDim.x) {
    const float gv = St<T>::load(g, i);
    if (go != g) St<T>::store(go, i, gv);
    St<T>::store(c, i, (float)((double)St<T>::load(e, i) * se * (double)St<T>::load(w_in, i)));
    St<T>::store(c, H + i, (float)((double)gv * sg * (double)St<T>::load(w_hid, i)));
  }
}

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* __restrict__ x,
                                                      const T* __restrict__ w, float eps, int H,
                                                      T* __restrict__ y) {
  __shared__ double red[16];
  const int r = blockIdx.x;
  const T* xr = x + (int64_t)r * H;
  T* yr = y + (int64_t)r * H;
  const double sc = row_rscale(xr, H, eps, red);
  for (int i = threadIdx.x; i < H; i += blockDim.x)
    St<T>::store(yr, i, (float)((double)St<T>::load(xr, i) * sc * (double)St<T>::load(w, i)));
}

}  // namespace

hipError_t prologue(bool bf16, const void* embed, int V, const int* tok, const void* hid,
                    const int* src, const void* w_in, const void* w_hid, float eps, int M, int H,
                    void* gout, void* cout, hipStream_t s) {
  if (bf16) {
    hipLaunchKernelGGL(prologue_kernel<bf16_t>, dim3(M), dim3(256), 0, s, (const bf16_t*)embed, V,
                       tok, (const bf16_t*)hid, src, (const bf16_t*)w_in, (const bf16_t*)w_hid,
                       eps, H, (bf16_t*)gout, (bf16_t*)cout);
  } else {
    hipLaunchKernelGGL(prologue_kernel<float>, dim3(M), dim3(256), 0, s, (const float*)embed, V,
                       tok, (const float*)hid, src, (const float*)w_in, (const float*)w_hid, eps,
                       H, (float*)gout, (float*)cout);
  }
  return hipGetLastError();
}

hipError_t rmsnorm(bool bf16, const void* x, const void* w, float eps, int M, int H, void* y,
                   hipStream_t s) {
  if (bf16) {
    hipLaunchKernelGGL(rmsnorm_kernel<bf16_t>, dim3(M), dim3(256), 0, s, (const bf16_t*)x,
                       (const bf16_t*)w, eps, H, (bf16_t*)y);
  } else {
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(M), dim3(256), 0, s, (const float*)x,
                       (const float*)w, eps, H, (float*)y);
  }
  return hipGetLastError();
}

}  // namespace spec

// Peak probes: an HBM read stream, an HBM copy stream and a bf16 MFMA loop,
// each as plain as its resource allows, to measure what the GPU attains.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spec_peaks.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr uint32_t kSinkKey = 0x9e3779b9u;

__global__ __launch_bounds__(512) void peak_read_kernel(const u32x4* __restrict__ p, int64_t n,
                                                        uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n; i += stride) acc ^= p[i];
  const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (v == kSinkKey) sink[0] = v;
}

__global__ __launch_bounds__(512) void peak_copy_kernel(u32x4* __restrict__ q,
                                                        const u32x4* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    q[i] = a;
    q[i + stride] = b;
    q[i + 2 * stride] = c;
    q[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) q[i] = p[i];
}

// Eight independent accumulation chains per wave, written as one asm block so
// that the accumulators stay in place in AGPRs (compiled from builtins, this
// loop gets register copies between the MFMAs).  The s_nop after the loop
// covers the wait states before the accumulators are read back.
__global__ __launch_bounds__(256) void peak_mfma_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
    b[e] = (__bf16)(0.002f * (float)((lane * 3 + e) & 7));
  }
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {1.f, 0.f, 0.f, 0.f}, c2 = {2.f, 0.f, 0.f, 0.f},
        c3 = {3.f, 0.f, 0.f, 0.f}, c4 = {4.f, 0.f, 0.f, 0.f}, c5 = {5.f, 0.f, 0.f, 0.f},
        c6 = {6.f, 0.f, 0.f, 0.f}, c7 = {7.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
    asm volatile(
        "v_mfma_f32_16x16x32_bf16 %0, %8, %9, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %8, %9, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %8, %9, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %8, %9, %3\n\t"
        "v_mfma_f32_16x16x32_bf16 %4, %8, %9, %4\n\t"
        "v_mfma_f32_16x16x32_bf16 %5, %8, %9, %5\n\t"
        "v_mfma_f32_16x16x32_bf16 %6, %8, %9, %6\n\t"
        "v_mfma_f32_16x16x32_bf16 %7, %8, %9, %7"
        : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3), "+a"(c4), "+a"(c5), "+a"(c6), "+a"(c7)
        : "v"(a), "v"(b));
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  const f32x4 s = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" int32_t spec_peak_read(const void* src, int64_t bytes, uint32_t* sink, int32_t blocks,
                                  void* stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16 || !al16(src) || blocks < 1) return -1;
  hipLaunchKernelGGL(peak_read_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream,
                     (const u32x4*)src, bytes / 16, sink);
  return (int32_t)hipGetLastError();
}

extern "C" int32_t spec_peak_copy(void* dst, const void* src, int64_t bytes, int32_t blocks,
                                  void* stream) {
  if (!dst || !src || bytes <= 0 || bytes % 16 || !al16(src) || !al16(dst) || blocks < 1) return -1;
  const uintptr_t d = (uintptr_t)dst, s = (uintptr_t)src;
  if (d < s + (uintptr_t)bytes && s < d + (uintptr_t)bytes) return -1;
  hipLaunchKernelGGL(peak_copy_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream,
                     (u32x4*)dst, (const u32x4*)src, bytes / 16);
  return (int32_t)hipGetLastError();
}

extern "C" int32_t spec_peak_mfma(int32_t iters, float* sink, int32_t blocks, void* stream) {
  if (!sink || iters < 1 || blocks < 1) return -1;
  hipLaunchKernelGGL(peak_mfma_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return (int32_t)hipGetLastError();
}

extern "C" double spec_peak_mfma_flops(int32_t iters, int32_t blocks) {
  return (double)blocks * 4.0 * iters * 8.0 * 16.0 * 16.0 * 32.0 * 2.0;
}

// Weight-streaming GEMMs for the draft contractions (FC fusion, QKV, O,
// gate|up, down, LM head) and their split-K epilogues.
//
// Shapes: Y[M, N] = X[M, K] . W[N, K]^T with W row-major [out, in].  At the
// row counts of a speculation step (M = 1 .. 64 per block) the contraction is
// bound by streaming W from HBM, so the kernel is organised around the
// weight stream: a wave owns 16 output columns (16 rows of W) and a K range,
// issues 16-byte loads that cover 64 contiguous bytes of each of its 16 W rows
// per instruction, and feeds them to v_mfma_f32_16x16x32_bf16 with W as the
// A operand and up to 4 tiles of 16 X rows as B operands.  Split-K over the
// grid's y dimension keeps ~2048 workgroups in flight; partial sums go to a
// float32 buffer that the epilogue kernels reduce in a fixed order (the result
// is deterministic).
#include "common.h"
#include "kernels.h"

namespace spec {

namespace {

// v_mfma_f32_16x16x32_bf16 operand layout: lane l holds row (l & 15) of A
// (column (l & 15) of B) and K elements 8*(l >> 4) .. +8; the 4 accumulators
// of lane l are rows 4*(l >> 4) .. +4 of column (l & 15).
// TAG only separates kernel symbols (0: layer GEMMs, 1: LM head / scores) so
// that per-kernel traces attribute time to the dominant contraction.
template <int MT, int TAG>
__global__ __launch_bounds__(256) void gemm_bf16_stream(const bf16_t* __restrict__ X, int ldx,
                                                         const bf16_t* __restrict__ W, int ldw,
                                                         float* __restrict__ P, int M, int N, int K,
                                                         int kc) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * 64 + wave * 16;
  if (n0 >= N) return;
  const int split = blockIdx.y;
  const int k0 = split * kc;
  const int k1 = min(K, k0 + kc);
  const int m0 = blockIdx.z * (16 * MT);
  const int g = lane >> 4, c = lane & 15;

  const bf16_t* wp = W + (int64_t)min(n0 + c, N - 1) * ldw + g * 8;
  const bf16_t* xp[MT];
  bool xv[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = m0 + t * 16 + c;
    xv[t] = m < M;
    xp[t] = X + (int64_t)(xv[t] ? m : 0) * ldx + g * 8;
  }
  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // 128 K elements per step: 4 MFMAs, each over 32 consecutive K.
  int k = k0;
#pragma unroll 2
  for (; k + 128 <= k1; k += 128) {
    u32x4_t wr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wr[j] = __builtin_nontemporal_load((const u32x4_t*)(wp + k + j * 32));
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      u32x4_t xr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xr[j] = xv[t] ? *(const u32x4_t*)(xp[t] + k + j * 32) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wr[j]),
                                                         __builtin_bit_cast(bf16x8, xr[j]), acc[t],
                                                         0, 0, 0);
    }
  }
  // K tail in steps of 32
  for (; k < k1; k += 32) {
    const u32x4_t wr = *(const u32x4_t*)(wp + k);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const u32x4_t xr = xv[t] ? *(const u32x4_t*)(xp[t] + k) : u32x4_t{0u, 0u, 0u, 0u};
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wr),
                                                       __builtin_bit_cast(bf16x8, xr), acc[t], 0, 0,
                                                       0);
    }
  }
  // lane holds Y[n0 + 4g + r][m0 + 16t + c], r = 0..3
  const int nb = n0 + 4 * g;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = m0 + t * 16 + c;
    if (m >= M) continue;
    float* dst = P + ((int64_t)split * M + m) * N + nb;
    if (nb + 3 < N && (N & 3) == 0) {
      *(float4*)dst = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    } else {
      for (int r = 0; r < 4; ++r)
        if (nb + r < N) dst[r] = acc[t][r];
    }
  }
}

// float32 path: a 16-lane group owns one output column, lanes stride over K
// with float4 loads; up to 16 rows of X per block in registers.
__global__ __launch_bounds__(256) void gemm_f32_rows(const float* __restrict__ X, int ldx,
                                                      const float* __restrict__ W, int ldw,
                                                      float* __restrict__ P, int M, int N, int K) {
  const int grp = threadIdx.x >> 4, lane = threadIdx.x & 15;
  const int n = blockIdx.x * 16 + grp;
  const int m0 = blockIdx.y * 16;
  const int rows = min(16, M - m0);
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  if (n < N) {
    const float* w = W + (int64_t)n * ldw;
    for (int k = lane * 4; k < K; k += 64) {
      const float4 wv = *(const float4*)(w + k);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i < rows) {
          const float4 x = *(const float4*)(X + (int64_t)(m0 + i) * ldx + k);
          acc[i] += wv.x * x.x + wv.y * x.y + wv.z * x.z + wv.w * x.w;
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) acc[i] += __shfl_xor(acc[i], o, 16);
  }
  if (n < N && lane == 0) {
    for (int i = 0; i < rows; ++i) P[(int64_t)(m0 + i) * N + n] = acc[i];
  }
}

template <typename T, int OP>
__global__ __launch_bounds__(256) void epi_kernel(T* __restrict__ Y, const T* __restrict__ R,
                                                   const float* __restrict__ P, int nsplit, int M,
                                                   int N) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)M * N) return;
  const int m = int(idx / N), n = int(idx % N);
  const int ldp = OP == EPI_SWIGLU ? 2 * N : N;
  const int64_t ss = (int64_t)M * ldp;
  if (OP == EPI_SWIGLU) {
    float gsum = 0.f, usum = 0.f;
    const float* p = P + (int64_t)m * ldp + n;
    for (int s = 0; s < nsplit; ++s) {
      gsum += p[s * ss];
      usum += p[s * ss + N];
    }
    const float silu = gsum / (1.f + expf(-gsum));
    St<T>::store(Y, idx, silu * usum);
    return;
  }
  float sum = 0.f;
  const float* p = P + (int64_t)m * ldp + n;
  for (int s = 0; s < nsplit; ++s) sum += p[s * ss];
  if (OP == EPI_RESID) sum += St<T>::load(R, idx);
  St<T>::store(Y, idx, sum);
}

__global__ __launch_bounds__(256) void epi_f32(float* __restrict__ Y, const float* __restrict__ P,
                                               int nsplit, int64_t MN) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= MN) return;
  float sum = 0.f;
  for (int s = 0; s < nsplit; ++s) sum += P[s * MN + idx];
  Y[idx] = sum;
}

// One block per (row, head): thread i < hd/2 owns the rotation pair (i, i + hd/2).
template <typename T>
__global__ void qkv_epi_kernel(const float* __restrict__ P, int nsplit, int M, int nq, int nkv,
                               int hd, const int* __restrict__ pos, const int* __restrict__ slot,
                               int rows_per_seq, float rope_base, T* __restrict__ qout,
                               T* __restrict__ kc, T* __restrict__ vc, int64_t stride_seq,
                               int64_t stride_head, int slots) {
  const int m = blockIdx.x, h = blockIdx.y, i = threadIdx.x;
  const int half = hd >> 1;
  if (i >= half) return;
  const int N = (nq + 2 * nkv) * hd;
  const int64_t ss = (int64_t)M * N;
  const float* p = P + (int64_t)m * N + h * hd;
  float x1 = 0.f, x2 = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    x1 += p[s * ss + i];
    x2 += p[s * ss + i + half];
  }
  x1 = St<T>::round(x1);
  x2 = St<T>::round(x2);
  const int seq = m / rows_per_seq;
  const int sl = slot ? slot[m] : -1;
  if (h < nq + nkv) {
    const double inv = pow((double)rope_base, -2.0 * i / hd);
    double sn, cs;
    sincos((double)pos[m] * inv, &sn, &cs);
    const float c = (float)cs, sf = (float)sn;
    const float y1 = x1 * c - x2 * sf;
    const float y2 = x2 * c + x1 * sf;
    if (h < nq) {
      T* q = qout + ((int64_t)m * nq + h) * hd;
      St<T>::store(q, i, y1);
      St<T>::store(q, i + half, y2);
    } else if (sl >= 0 && sl < slots) {
      T* k = kc + seq * stride_seq + (int64_t)(h - nq) * stride_head + (int64_t)sl * hd;
      St<T>::store(k, i, y1);
      St<T>::store(k, i + half, y2);
    }
  } else if (sl >= 0 && sl < slots) {
    T* v = vc + seq * stride_seq + (int64_t)(h - nq - nkv) * stride_head + (int64_t)sl * hd;
    St<T>::store(v, i, x1);
    St<T>::store(v, i + half, x2);
  }
}

}  // namespace

GemmPlan gemm_plan(int M, int N, int K, bool bf16) {
  GemmPlan p;
  if (!bf16) {
    p.nsplit = 1;
    p.kc = K;
    return p;
  }
  const int strips = (N + 63) / 64;
  const int mblocks = (M + 63) / 64;
  const int target = 2048;
  int ns = (target + strips * mblocks - 1) / (strips * mblocks);
  const int kblocks = (K + 127) / 128;
  ns = std::max(1, std::min(ns, kblocks));
  const int kc = ((kblocks + ns - 1) / ns) * 128;
  p.kc = kc;
  p.nsplit = (K + kc - 1) / kc;
  return p;
}

template <int TAG>
static void launch_stream(const void* X, int ldx, const void* W, int ldw, float* P, int M, int N,
                          int K, const GemmPlan& plan, hipStream_t s) {
  const int strips = (N + 63) / 64;
  if (M <= 16) {
    hipLaunchKernelGGL((gemm_bf16_stream<1, TAG>), dim3(strips, plan.nsplit, 1), dim3(256), 0, s,
                       (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, P, M, N, K, plan.kc);
  } else if (M <= 32) {
    hipLaunchKernelGGL((gemm_bf16_stream<2, TAG>), dim3(strips, plan.nsplit, 1), dim3(256), 0, s,
                       (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, P, M, N, K, plan.kc);
  } else {
    hipLaunchKernelGGL((gemm_bf16_stream<4, TAG>), dim3(strips, plan.nsplit, (M + 63) / 64),
                       dim3(256), 0, s, (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, P, M, N, K,
                       plan.kc);
  }
}

hipError_t gemm(bool bf16, const void* X, int ldx, const void* W, int ldw, float* P, int M, int N,
                int K, const GemmPlan& plan, hipStream_t s, int tag) {
  if (!bf16) {
    dim3 grid((N + 15) / 16, (M + 15) / 16);
    hipLaunchKernelGGL(gemm_f32_rows, grid, dim3(256), 0, s, (const float*)X, ldx,
                       (const float*)W, ldw, P, M, N, K);
    return hipGetLastError();
  }
  if (tag == 1) {
    launch_stream<1>(X, ldx, W, ldw, P, M, N, K, plan, s);
  } else {
    launch_stream<0>(X, ldx, W, ldw, P, M, N, K, plan, s);
  }
  return hipGetLastError();
}

hipError_t gemm_epilogue(bool bf16, int op, void* Y, const void* R, const float* P, int nsplit,
                         int M, int N, hipStream_t s) {
  const int64_t total = (int64_t)M * N;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (op == EPI_F32) {
    hipLaunchKernelGGL(epi_f32, grid, dim3(256), 0, s, (float*)Y, P, nsplit, total);
    return hipGetLastError();
  }
#define SPEC_EPI(T)                                                                            \
  switch (op) {                                                                                \
    case EPI_STORE:                                                                            \
      hipLaunchKernelGGL((epi_kernel<T, EPI_STORE>), grid, dim3(256), 0, s, (T*)Y,             \
                         (const T*)R, P, nsplit, M, N);                                        \
      break;                                                                                   \
    case EPI_RESID:                                                                            \
      hipLaunchKernelGGL((epi_kernel<T, EPI_RESID>), grid, dim3(256), 0, s, (T*)Y,             \
                         (const T*)R, P, nsplit, M, N);                                        \
      break;                                                                                   \
    default:                                                                                   \
      hipLaunchKernelGGL((epi_kernel<T, EPI_SWIGLU>), grid, dim3(256), 0, s, (T*)Y,            \
                         (const T*)R, P, nsplit, M, N);                                        \
  }
  if (bf16) {
    SPEC_EPI(bf16_t)
  } else {
    SPEC_EPI(float)
  }
#undef SPEC_EPI
  return hipGetLastError();
}

hipError_t qkv_epilogue(bool bf16, const float* P, int nsplit, int M, int nq, int nkv, int hd,
                        const int* pos, const int* slot, int rows_per_seq, float rope_base,
                        void* qout, KvView kv, hipStream_t s) {
  dim3 grid(M, nq + 2 * nkv);
  dim3 block(hd / 2);
  if (bf16) {
    hipLaunchKernelGGL(qkv_epi_kernel<bf16_t>, grid, block, 0, s, P, nsplit, M, nq, nkv, hd, pos,
                       slot, rows_per_seq, rope_base, (bf16_t*)qout, (bf16_t*)kv.k,
                       (bf16_t*)kv.v, kv.stride_seq, kv.stride_head, kv.slots);
  } else {
    hipLaunchKernelGGL(qkv_epi_kernel<float>, grid, block, 0, s, P, nsplit, M, nq, nkv, hd, pos,
                       slot, rows_per_seq, rope_base, (float*)qout, (float*)kv.k, (float*)kv.v,
                       kv.stride_seq, kv.stride_head, kv.slots);
  }
  return hipGetLastError();
}

}  // namespace spec

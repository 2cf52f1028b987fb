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
#include "topk_common.h"

namespace spec {

namespace {

// v_mfma_f32_16x16x32_bf16 operand layout: lane l holds row (l & 15) of A
// (column (l & 15) of B) and K elements 8*(l >> 4) .. +8; the 4 accumulators
// of lane l are rows 4*(l >> 4) .. +4 of column (l & 15).
//
// A wave owns CW tiles of 16 output columns; each 128-K step issues 4*CW
// 16-byte loads per lane, and two steps are issued before their MFMAs, so a
// wave keeps 8*CW loads of the weight stream in flight.  Plain (temporal)
// loads measured faster than nontemporal ones on this stream.
// TAG only separates kernel symbols (0: layer GEMMs, 1: LM head / scores) so
// that per-kernel traces attribute time to the dominant contraction.
template <int MT, int CW>
SPEC_DEV void stream_acc(const bf16_t* __restrict__ X, int ldx, const bf16_t* __restrict__ W,
                         int ldw, int M, int N, int k0, int k1, int m0, int n0,
                         f32x4 (&acc)[CW][MT]) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const bf16_t* wp[CW];
#pragma unroll
  for (int w = 0; w < CW; ++w) wp[w] = W + (int64_t)min(n0 + 16 * w + c, N - 1) * ldw + g * 8;
  const bf16_t* xp[MT];
  bool xv[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = m0 + t * 16 + c;
    xv[t] = m < M;
    xp[t] = X + (int64_t)(xv[t] ? m : 0) * ldx + g * 8;
  }
#pragma unroll
  for (int w = 0; w < CW; ++w)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[w][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](const u32x4_t (&wr)[CW][4], int k) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      u32x4_t xr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xr[j] = xv[t] ? *(const u32x4_t*)(xp[t] + k + j * 32) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int w = 0; w < CW; ++w)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[w][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wr[w][j]),
                                                              __builtin_bit_cast(bf16x8, xr[j]),
                                                              acc[w][t], 0, 0, 0);
    }
  };
  int k = k0;
  // two 128-K steps per iteration: all their weight loads first
  for (; k + 256 <= k1; k += 256) {
    u32x4_t wa[CW][4], wb[CW][4];
#pragma unroll
    for (int w = 0; w < CW; ++w)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wa[w][j] = *(const u32x4_t*)(wp[w] + k + j * 32);
        wb[w][j] = *(const u32x4_t*)(wp[w] + k + 128 + j * 32);
      }
    step(wa, k);
    step(wb, k + 128);
  }
  for (; k + 128 <= k1; k += 128) {
    u32x4_t wa[CW][4];
#pragma unroll
    for (int w = 0; w < CW; ++w)
#pragma unroll
      for (int j = 0; j < 4; ++j) wa[w][j] = *(const u32x4_t*)(wp[w] + k + j * 32);
    step(wa, k);
  }
  // K tail in steps of 32
  for (; k < k1; k += 32) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const u32x4_t xr = xv[t] ? *(const u32x4_t*)(xp[t] + k) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int w = 0; w < CW; ++w)
        acc[w][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, *(const u32x4_t*)(wp[w] + k)), __builtin_bit_cast(bf16x8, xr),
            acc[w][t], 0, 0, 0);
    }
  }
}

// Block-shared activations for MT >= 2 (K % 512 == 0, 16-byte aligned X rows):
// the four waves of a block stream different weight rows against the same
// 16*MT X rows, so X comes into LDS once per block, 256 K at a time, by
// global_load_lds (two buffers, one LDS object each), instead of every wave
// reading it from L2.  Chunk j (16 bytes) of X row r of a buffer sits at
// position j ^ (r & 15), so the 16 rows of a fragment read hit 16 distinct
// 16-byte bank groups.  Per 256-K iteration a wave issues its weight loads,
// waits for its own DMA of the iteration (issued before them, at the end of
// the previous iteration), meets the other waves at a barrier, runs the
// MFMAs, and then issues the DMA of the next iteration: no MFMA operand wait
// ever has an LDS DMA behind it.  Past the last iteration the DMA repeats the
// last one, keeping every wave's load count uniform.
template <int MT, int CW>
SPEC_DEV void stream_acc_lds(const bf16_t* __restrict__ X, int ldx, const bf16_t* __restrict__ W,
                             int ldw, int M, int N, int k0, int kn, int m0, int n0,
                             f32x4 (&acc)[CW][MT], SPEC_LDS u32x4_t* xs0, SPEC_LDS u32x4_t* xs1) {
  constexpr int NXI = 2 * MT;  // DMA instructions per wave per iteration (16*MT rows x 32 chunks)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const bf16_t* wp[CW];
#pragma unroll
  for (int w = 0; w < CW; ++w) wp[w] = W + (int64_t)min(n0 + 16 * w + c, N - 1) * ldw + k0 + g * 8;
  const bf16_t* xsrc[NXI];
  int xdst[NXI];
#pragma unroll
  for (int j = 0; j < NXI; ++j) {
    xdst[j] = (wave * NXI + j) * 64;
    const int u = xdst[j] + lane, row = u >> 5, pos = u & 31;
    xsrc[j] = X + (int64_t)min(m0 + row, M - 1) * ldx + k0 + 8 * (pos ^ (row & 15));
  }
#pragma unroll
  for (int w = 0; w < CW; ++w)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[w][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nit = kn / 256;
  auto issue = [&](SPEC_LDS u32x4_t* xs, int it) __attribute__((always_inline)) {
    const int k = min(it, nit - 1) * 256;
#pragma unroll
    for (int j = 0; j < NXI; ++j) dma16(xsrc[j] + k, xs + xdst[j]);
  };
  auto body = [&](SPEC_LDS u32x4_t* xs, SPEC_LDS u32x4_t* xn, int it) __attribute__((always_inline)) {
    const int k = it * 256;
    u32x4_t wa[CW][4], wb[CW][4];
#pragma unroll
    for (int w = 0; w < CW; ++w)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        wa[w][j] = *(const u32x4_t*)(wp[w] + k + j * 32);
        wb[w][j] = *(const u32x4_t*)(wp[w] + k + 128 + j * 32);
      }
    // this wave's DMA of iteration it (older than the 8*CW weight loads) has
    // landed; after the barrier every wave's has, and every wave is done
    // with iteration it - 1, whose buffer the DMA below refills
    wait_vm_lgkm0<8 * CW>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        u32x4_t xr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) xr[j] = xs[(16 * t + c) * 32 + ((16 * h + 4 * j + g) ^ c)];
#pragma unroll
        for (int w = 0; w < CW; ++w)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[w][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, h ? wb[w][j] : wa[w][j]), __builtin_bit_cast(bf16x8, xr[j]),
                acc[w][t], 0, 0, 0);
      }
    }
    // the MFMAs (and so their weight-register waits) stay ahead of the DMA:
    // a wait for weights issued behind a pending DMA would have to wait for it
#pragma unroll
    for (int w = 0; w < CW; ++w)
#pragma unroll
      for (int t = 0; t < MT; ++t) asm volatile("" : "+v"(acc[w][t]) :: "memory");
    issue(xn, it + 1);
    asm volatile("" ::: "memory");  // the next weight loads stay behind this DMA
  };
  issue(xs0, 0);
  for (int it = 0; it < nit; it += 2) {
    body(xs0, xs1, it);
    body(xs1, xs0, it + 1);
  }
  wait_vm_lgkm0<0>();  // the repeated DMA past the end
}

// lane holds Y[n0 + 16w + 4g + r][m0 + 16t + c], r = 0..3
template <int MT, int CW>
SPEC_DEV void store_tiles(const f32x4 (&acc)[CW][MT], float* __restrict__ P, int M, int N, int m0,
                          int n0) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
#pragma unroll
  for (int w = 0; w < CW; ++w) {
    const int nb = n0 + 16 * w + 4 * g;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = m0 + t * 16 + c;
      if (m >= M || nb >= N) continue;
      float* dst = P + (int64_t)m * N + nb;
      if (nb + 3 < N && (N & 3) == 0) {
        *(float4*)dst = make_float4(acc[w][t][0], acc[w][t][1], acc[w][t][2], acc[w][t][3]);
      } else {
        for (int r = 0; r < 4; ++r)
          if (nb + r < N) dst[r] = acc[w][t][r];
      }
    }
  }
}

template <int MT, int TAG, int CW, bool XL>
__global__ __launch_bounds__(256) void gemm_bf16_stream(const bf16_t* __restrict__ X, int ldx,
                                                         const bf16_t* __restrict__ W, int ldw,
                                                         float* __restrict__ P, int M, int N, int K,
                                                         int kc) {
  __shared__ u32x4_t xs0[XL ? 16 * MT * 32 : 1], xs1[XL ? 16 * MT * 32 : 1];
  const int wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * (64 * CW) + wave * (16 * CW);
  const int split = blockIdx.y;
  const int k0 = split * kc;
  const int k1 = min(K, k0 + kc);
  const int m0 = blockIdx.z * (16 * MT);
  f32x4 acc[CW][MT];
  if constexpr (XL) {
    // every wave takes part in the block's shared X loads (one past N streams
    // the clamped last weight rows and stores nothing)
    stream_acc_lds<MT, CW>(X, ldx, W, ldw, M, N, k0, k1 - k0, m0, n0, acc,
                           (SPEC_LDS u32x4_t*)xs0, (SPEC_LDS u32x4_t*)xs1);
    if (n0 < N) store_tiles<MT, CW>(acc, P + (int64_t)split * M * N, M, N, m0, n0);
  } else {
    if (n0 >= N) return;
    stream_acc<MT, CW>(X, ldx, W, ldw, M, N, k0, k1, m0, n0, acc);
    store_tiles<MT, CW>(acc, P + (int64_t)split * M * N, M, N, m0, n0);
  }
}

// LM head with the vocab top-k fused: after the (unsplit) contraction each
// lane reduces its CW*4 columns of a row to a top-KM list and a (max, sum exp)
// pair, the four lane groups of a wave merge by shuffles, and the four waves
// through LDS; one record per (row, workgroup) goes to the partial buffer in
// the layout the record merge reads (pv/pi [M][nch][KM], pp [M][nch]).
template <int MT, int CW, int KM, bool XL>
__global__ __launch_bounds__(256) void gemm_lmhead_topk_kernel(
    const bf16_t* __restrict__ X, int ldx, const bf16_t* __restrict__ W, int ldw,
    float* __restrict__ z, int M, int N, int K, float* __restrict__ pv, int* __restrict__ pi,
    topkdev::Part* __restrict__ pp) {
  using topkdev::List;
  __shared__ u32x4_t xs0[XL ? 16 * MT * 32 : 1], xs1[XL ? 16 * MT * 32 : 1];
  __shared__ float tv[4][16 * MT][KM];
  __shared__ int ti[4][16 * MT][KM];
  __shared__ float tm[4][16 * MT];
  __shared__ float ts[4][16 * MT];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const int strip = blockIdx.x, nch = gridDim.x;
  const int n0 = strip * (64 * CW) + wave * (16 * CW);
  const int m0 = blockIdx.z * (16 * MT);
  const bool active = n0 < N;  // no early return: the block meets at a barrier
  f32x4 acc[CW][MT];
  if constexpr (XL) {
    // every wave takes part in the shared X loads (an inactive one streams
    // the clamped last weight rows and stores nothing)
    stream_acc_lds<MT, CW>(X, ldx, W, ldw, M, N, 0, K, m0, n0, acc, (SPEC_LDS u32x4_t*)xs0,
                           (SPEC_LDS u32x4_t*)xs1);
    if (active && z) store_tiles<MT, CW>(acc, z, M, N, m0, n0);
  } else if (active) {
    stream_acc<MT, CW>(X, ldx, W, ldw, M, N, 0, K, m0, n0, acc);
    if (z) store_tiles<MT, CW>(acc, z, M, N, m0, n0);
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    List<KM> L;
    L.init();
    float lm = -INFINITY, ls = 0.f;
    if (active) {
#pragma unroll
      for (int w = 0; w < CW; ++w)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int n = n0 + 16 * w + 4 * g + r;
          if (n < N) {
            L.insert(acc[w][t][r], n);
            lm = fmaxf(lm, acc[w][t][r]);
          }
        }
#pragma unroll
      for (int w = 0; w < CW; ++w)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n0 + 16 * w + 4 * g + r < N) ls += expf(acc[w][t][r] - lm);
    }
    // merge the four lane groups holding the same row
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
      const float om = xor_hi(lm, o), os = xor_hi(ls, o);
      const float mx = fmaxf(lm, om);
      ls = (lm == -INFINITY ? 0.f : ls * expf(lm - mx)) + (om == -INFINITY ? 0.f : os * expf(om - mx));
      lm = mx;
      float pvv[KM];
      int pii[KM];
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        pvv[j] = xor_hi(L.v[j], o);
        pii[j] = xor_hi(L.i[j], o);
      }
#pragma unroll
      for (int j = 0; j < KM; ++j) L.insert(pvv[j], pii[j]);
    }
    if (g == 0) {
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        tv[wave][16 * t + c][j] = L.v[j];
        ti[wave][16 * t + c][j] = L.i[j];
      }
      tm[wave][16 * t + c] = lm;
      ts[wave][16 * t + c] = ls;
    }
  }
  __syncthreads();
  const int row = threadIdx.x;
  if (row < 16 * MT && m0 + row < M) {
    List<KM> L;
    L.init();
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      mx = fmaxf(mx, tm[w][row]);
#pragma unroll
      for (int j = 0; j < KM; ++j) L.insert(tv[w][row][j], ti[w][row][j]);
    }
    double sum = 0.0;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (tm[w][row] != -INFINITY) sum += (double)ts[w][row] * exp((double)tm[w][row] - (double)mx);
    const int m = m0 + row;
    const int64_t base = ((int64_t)m * nch + strip) * KM;
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      pv[base + j] = L.v[j];
      pi[base + j] = L.i[j];
    }
    pp[(int64_t)m * nch + strip] = topkdev::Part{sum, mx, 0};
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

// Split-K reduction: a block covers 32 consecutive outputs; thread group
// sg = threadIdx.x / 32 (8 groups) sums splits sg, sg+8, ... and the groups are
// combined through LDS in a fixed order, so results are deterministic.
constexpr int kEpiCols = 32, kEpiGroups = 8;

SPEC_DEV float split_sum(const float* __restrict__ p, int64_t sstride, int nsplit, int sg) {
  float a = 0.f;
  for (int s = sg; s < nsplit; s += kEpiGroups) a += p[s * sstride];
  return a;
}

template <typename T, int OP>
__global__ __launch_bounds__(256) void epi_kernel(T* __restrict__ Y, const T* __restrict__ R,
                                                   const float* __restrict__ P, int nsplit, int M,
                                                   int N) {
  __shared__ float red[2][kEpiGroups][kEpiCols];
  const int e = threadIdx.x % kEpiCols, sg = threadIdx.x / kEpiCols;
  const int64_t idx = (int64_t)blockIdx.x * kEpiCols + e;
  const bool ok = idx < (int64_t)M * N;
  const int m = ok ? int(idx / N) : 0, n = ok ? int(idx % N) : 0;
  const int ldp = OP == EPI_SWIGLU ? 2 * N : N;
  const int64_t ss = (int64_t)M * ldp;
  const float* p = P + (int64_t)m * ldp + n;
  red[0][sg][e] = ok ? split_sum(p, ss, nsplit, sg) : 0.f;
  if (OP == EPI_SWIGLU) red[1][sg][e] = ok ? split_sum(p + N, ss, nsplit, sg) : 0.f;
  __syncthreads();
  if (sg != 0 || !ok) return;
  float a = 0.f, u = 0.f;
#pragma unroll
  for (int j = 0; j < kEpiGroups; ++j) {
    a += red[0][j][e];
    if (OP == EPI_SWIGLU) u += red[1][j][e];
  }
  if (OP == EPI_SWIGLU) {
    const float silu = a / (1.f + expf(-a));
    St<T>::store(Y, idx, silu * u);
    return;
  }
  if (OP == EPI_RESID) a += St<T>::load(R, idx);
  St<T>::store(Y, idx, a);
}

__global__ __launch_bounds__(256) void epi_f32(float* __restrict__ Y, const float* __restrict__ P,
                                               int nsplit, int64_t MN) {
  __shared__ float red[kEpiGroups][kEpiCols];
  const int e = threadIdx.x % kEpiCols, sg = threadIdx.x / kEpiCols;
  const int64_t idx = (int64_t)blockIdx.x * kEpiCols + e;
  const bool ok = idx < MN;
  red[sg][e] = ok ? split_sum(P + idx, MN, nsplit, sg) : 0.f;
  __syncthreads();
  if (sg != 0 || !ok) return;
  float a = 0.f;
#pragma unroll
  for (int j = 0; j < kEpiGroups; ++j) a += red[j][e];
  Y[idx] = a;
}

// Split-K LM head whose logits are materialised: z = the sum of the nsplit
// partials (in split order) and one (max, sum of exp(v - max)) record per row
// and 128-column strip, the layout the strip top-k reads (with z == P and one
// split, only the records of an output already written).  One wave per
// (row, strip), two columns per lane.
__global__ __launch_bounds__(256) void epi_f32_rec_kernel(float* __restrict__ z,
                                                          const float* __restrict__ P, int nsplit,
                                                          int M, int N, int nstrip,
                                                          float2* __restrict__ rec) {
  constexpr float kL2e = 1.4426950408889634f;
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (row, strip)
  if (w >= (int64_t)M * nstrip) return;                             // uniform in the wave
  const int m = int(w / nstrip), st = int(w % nstrip);
  const int64_t ss = (int64_t)M * N;
  float v[2];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = st * 128 + 2 * lane + j;
    v[j] = 0.f;
    if (n < N) {
      const float* p = P + (int64_t)m * N + n;
      float a = 0.f;
      for (int sp = 0; sp < nsplit; ++sp) a += p[sp * ss];
      if (z != P) z[(int64_t)m * N + n] = a;  // z == P: records of a finished output
      v[j] = a;
      mx = fmaxf(mx, a);
    }
  }
  mx = wave_max(mx);
  float sum = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (st * 128 + 2 * lane + j < N) sum += __builtin_amdgcn_exp2f((v[j] - mx) * kL2e);
  }
  sum = wave_sum(sum);
  if (lane == 0) rec[(int64_t)m * nstrip + st] = make_float2(mx, sum);
}

// Few splits over many outputs: one thread per 4 consecutive outputs (16-byte
// partial loads), splits summed in order from 0 - the same additions, in the
// same order, as epi_kernel for nsplit <= kEpiGroups.
template <typename T> struct Vec4;
template <> struct Vec4<float> {
  static SPEC_DEV float4 load(const float* p) { return *(const float4*)p; }
  static SPEC_DEV void store(float* p, float4 v) { *(float4*)p = v; }
};
template <> struct Vec4<bf16_t> {
  static SPEC_DEV float4 load(const bf16_t* p) {
    const uint2 w = *(const uint2*)p;
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
  }
  static SPEC_DEV void store(bf16_t* p, float4 v) {
    uint2 w;
    w.x = (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
    w.y = (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16);
    *(uint2*)p = w;
  }
};

SPEC_DEV float4 split_sum4(const float* __restrict__ p, int64_t sstride, int nsplit) {
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < nsplit; ++s) {
    const float4 v = *(const float4*)(p + s * sstride);
    a.x += v.x;
    a.y += v.y;
    a.z += v.z;
    a.w += v.w;
  }
  return a;
}

template <typename T, int OP>
__global__ __launch_bounds__(256) void epi_vec_kernel(T* __restrict__ Y, const T* __restrict__ R,
                                                       const float* __restrict__ P, int nsplit,
                                                       int M, int N) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= (int64_t)M * N) return;
  const int m = int(e / N), n = int(e % N);
  const int ldp = OP == EPI_SWIGLU ? 2 * N : N;
  const int64_t ss = (int64_t)M * ldp;
  const float* p = P + (int64_t)m * ldp + n;
  float4 a = split_sum4(p, ss, nsplit);
  if (OP == EPI_SWIGLU) {
    const float4 u = split_sum4(p + N, ss, nsplit);
    a.x = a.x / (1.f + expf(-a.x)) * u.x;
    a.y = a.y / (1.f + expf(-a.y)) * u.y;
    a.z = a.z / (1.f + expf(-a.z)) * u.z;
    a.w = a.w / (1.f + expf(-a.w)) * u.w;
  } else if (OP == EPI_RESID) {
    const float4 r = Vec4<T>::load(R + e);
    a.x += r.x;
    a.y += r.y;
    a.z += r.z;
    a.w += r.w;
  }
  Vec4<T>::store(Y + e, a);
}

// One block per (row, head): 4 split groups x 64 threads; thread i < hd/2 of
// group 0 owns the rotation pair (i, i + hd/2).
template <typename T>
__global__ __launch_bounds__(256) void qkv_epi_kernel(
    const float* __restrict__ P, int nsplit, int M, int nq, int nkv, int hd,
    const int* __restrict__ pos, const int* __restrict__ slot, int rows_per_seq, float rope_base,
    T* __restrict__ qout, T* __restrict__ kc, T* __restrict__ vc, int64_t stride_seq,
    int64_t stride_head, int slots, KvPages pg) {
  __shared__ float red[2][4][64];
  const int m = blockIdx.x, h = blockIdx.y, i = threadIdx.x & 63, sg = threadIdx.x >> 6;
  const int half = hd >> 1;
  const int N = (nq + 2 * nkv) * hd;
  const int64_t ss = (int64_t)M * N;
  const float* p = P + (int64_t)m * N + h * hd;
  float x1 = 0.f, x2 = 0.f;
  if (i < half) {
    for (int s = sg; s < nsplit; s += 4) {
      x1 += p[s * ss + i];
      x2 += p[s * ss + i + half];
    }
  }
  red[0][sg][i] = x1;
  red[1][sg][i] = x2;
  __syncthreads();
  if (sg != 0 || i >= half) return;
  x1 = red[0][0][i] + red[0][1][i] + red[0][2][i] + red[0][3][i];
  x2 = red[1][0][i] + red[1][1][i] + red[1][2][i] + red[1][3][i];
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
      T* k = kc + kv_slot_off(pg, seq, sl, stride_seq, hd) + (int64_t)(h - nq) * stride_head;
      St<T>::store(k, i, y1);
      St<T>::store(k, i + half, y2);
    }
  } else if (sl >= 0 && sl < slots) {
    T* v = vc + kv_slot_off(pg, seq, sl, stride_seq, hd) + (int64_t)(h - nq - nkv) * stride_head;
    St<T>::store(v, i, x1);
    St<T>::store(v, i + half, x2);
  }
}

// The same epilogue for many rows (M >= 64): a block covers one row and HPB
// of its heads, a group of hd/2 threads per head at a time, and each thread
// takes its rotation pair's angle once for all its heads.  Splits are summed
// in order s = 0, 1, ...
template <typename T>
__global__ __launch_bounds__(256) void qkv_epi_rows_kernel(
    const float* __restrict__ P, int nsplit, int M, int nq, int nkv, int hd,
    const int* __restrict__ pos, const int* __restrict__ slot, int rows_per_seq, float rope_base,
    T* __restrict__ qout, T* __restrict__ kc, T* __restrict__ vc, int64_t stride_seq,
    int64_t stride_head, int slots, KvPages pg, int hpb) {
  const int m = blockIdx.x, half = hd >> 1;
  const int par = blockDim.x / half;  // heads in flight per block
  const int i = threadIdx.x % half, hs = threadIdx.x / half;
  const int NH = nq + 2 * nkv, N = NH * hd;
  const int64_t ss = (int64_t)M * N;
  const double inv = pow((double)rope_base, -2.0 * i / hd);
  double sn, cs;
  sincos((double)pos[m] * inv, &sn, &cs);
  const float c = (float)cs, sf = (float)sn;
  const int seq = m / rows_per_seq;
  const int sl = slot ? slot[m] : -1;
  const int h1 = min(NH, (blockIdx.y + 1) * hpb);
  for (int h = blockIdx.y * hpb + hs; h < h1; h += par) {
    const float* p = P + (int64_t)m * N + h * hd;
    float x1 = 0.f, x2 = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) {
      x1 += p[sp * ss + i];
      x2 += p[sp * ss + i + half];
    }
    x1 = St<T>::round(x1);
    x2 = St<T>::round(x2);
    if (h < nq + nkv) {
      const float y1 = x1 * c - x2 * sf;
      const float y2 = x2 * c + x1 * sf;
      if (h < nq) {
        T* q = qout + ((int64_t)m * nq + h) * hd;
        St<T>::store(q, i, y1);
        St<T>::store(q, i + half, y2);
      } else if (sl >= 0 && sl < slots) {
        T* k = kc + kv_slot_off(pg, seq, sl, stride_seq, hd) + (int64_t)(h - nq) * stride_head;
        St<T>::store(k, i, y1);
        St<T>::store(k, i + half, y2);
      }
    } else if (sl >= 0 && sl < slots) {
      T* v = vc + kv_slot_off(pg, seq, sl, stride_seq, hd) + (int64_t)(h - nq - nkv) * stride_head;
      St<T>::store(v, i, x1);
      St<T>::store(v, i + half, x2);
    }
  }
}

}  // namespace

// Columns per wave: 16 for the very wide LM head at M <= 32 (one long K sweep
// per wave, no split, twice the strips), 32 otherwise (twice the loads in
// flight, and each activation fragment feeds two weight tiles).  With the
// top-k fused into the epilogue always 32: every strip adds a record list per
// row that the merge reads, and the weight stream runs as fast either way.
static constexpr int kMaxSplit = 32;  // bounds the epilogue's reduction depth
static int gemm_cw(int M, int N) { return (M <= 32 && N >= 65536) ? 1 : 2; }
static int lmhead_cw(int, int) { return 2; }

GemmPlan gemm_plan(int M, int N, int K, bool bf16, int max_split) {
  GemmPlan p;
  if (bf16 && gemm_tile_ok(M, K)) {
    p = gemm_tile_plan(M, N, K);
    p.tile = true;
    return p;
  }
  if (!bf16) {
    p.nsplit = 1;
    p.kc = K;
    return p;
  }
  const int cw = gemm_cw(M, N);
  const int strips = (N + 64 * cw - 1) / (64 * cw);
  const int mblocks = (M + 63) / 64;
  // workgroups in flight: 512 of four waves stream the weights at full rate
  // beyond 16 rows, 768 at up to 16 rows (shorter MFMA work per weight byte);
  // more only add split-K partials
  const int target = M <= 16 ? 768 : 512;
  int ns = (target + strips * mblocks - 1) / (strips * mblocks);
  // K in blocks of 512 where the activation rows go through LDS (see
  // stream_acc_lds: K steps in pairs of 256), else of 128
  const int kb = K % 512 == 0 ? 512 : 128;
  const int kblocks = (K + kb - 1) / kb;
  ns = std::max(1, std::min(std::min(ns, kblocks), std::min(kMaxSplit, std::max(1, max_split))));
  // vocab-wide heads have >= 1024 strips already: no split, so the top-k can
  // be fused into the epilogue and no M x N partials are written
  if (N >= 65536) ns = 1;
  const int kc = ((kblocks + ns - 1) / ns) * kb;
  p.kc = kc;
  p.nsplit = (K + kc - 1) / kc;
  return p;
}

template <int TAG, int CW>
static void launch_stream(const void* X, int ldx, const void* W, int ldw, float* P, int M, int N,
                          int K, const GemmPlan& plan, hipStream_t s) {
  const int strips = (N + 64 * CW - 1) / (64 * CW);
  // X through LDS once per block (the four waves share its rows) where every
  // split's K range is whole pairs of 256-wide steps
  const bool xl = K % 512 == 0 && plan.kc % 512 == 0 && ldx % 8 == 0 && ((uintptr_t)X & 15) == 0;
#define SPEC_STREAM(MT, XLV, GZ)                                                                \
  SPEC_LAUNCH((gemm_bf16_stream<MT, TAG, CW, XLV>), dim3(strips, plan.nsplit, GZ), dim3(256), 0, \
              s, (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, P, M, N, K, plan.kc)
  if (M <= 16) {
    if (xl) SPEC_STREAM(1, true, 1);
    else SPEC_STREAM(1, false, 1);
  } else if (M <= 32) {
    if (xl) SPEC_STREAM(2, true, 1);
    else SPEC_STREAM(2, false, 1);
  } else {
    if (xl) SPEC_STREAM(4, true, (M + 63) / 64);
    else SPEC_STREAM(4, false, (M + 63) / 64);
  }
#undef SPEC_STREAM
}

hipError_t gemm(bool bf16, const void* X, int ldx, const void* W, int ldw, float* P, int M, int N,
                int K, const GemmPlan& plan, hipStream_t s, int tag) {
  if (!bf16) {
    dim3 grid((N + 15) / 16, (M + 15) / 16);
    SPEC_LAUNCH(gemm_f32_rows, grid, dim3(256), 0, s, (const float*)X, ldx,
                       (const float*)W, ldw, P, M, N, K);
    return hipGetLastError();
  }
  if (plan.tile) return gemm_tile(X, ldx, W, ldw, P, M, N, K, plan, s);
  const bool cw1 = gemm_cw(M, N) == 1;
  if (tag == 1) {
    if (cw1) launch_stream<1, 1>(X, ldx, W, ldw, P, M, N, K, plan, s);
    else launch_stream<1, 2>(X, ldx, W, ldw, P, M, N, K, plan, s);
  } else {
    if (cw1) launch_stream<0, 1>(X, ldx, W, ldw, P, M, N, K, plan, s);
    else launch_stream<0, 2>(X, ldx, W, ldw, P, M, N, K, plan, s);
  }
  return hipGetLastError();
}

int gemm_strips(int M, int N) {
  const int cw = lmhead_cw(M, N);
  return (N + 64 * cw - 1) / (64 * cw);
}

template <int MT, int CW, bool XL>
static void launch_lmhead_x(const void* X, int ldx, const void* W, int ldw, float* z, int M, int N,
                            int K, int km, float* pv, int* pi, topkdev::Part* pp, hipStream_t s) {
  const dim3 grid((N + 64 * CW - 1) / (64 * CW), 1, (M + 16 * MT - 1) / (16 * MT));
  if (km == 1) {
    SPEC_LAUNCH((gemm_lmhead_topk_kernel<MT, CW, 1, XL>), grid, dim3(256), 0, s,
                (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, z, M, N, K, pv, pi, pp);
  } else {
    SPEC_LAUNCH((gemm_lmhead_topk_kernel<MT, CW, 8, XL>), grid, dim3(256), 0, s,
                (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, z, M, N, K, pv, pi, pp);
  }
}

// X through LDS (see stream_acc_lds) where the block holds two or more
// 16-row tiles and the shape allows it.
template <int MT, int CW>
static void launch_lmhead(const void* X, int ldx, const void* W, int ldw, float* z, int M, int N,
                          int K, int km, float* pv, int* pi, topkdev::Part* pp, hipStream_t s) {
  if (MT >= 2 && K % 512 == 0 && ldx % 8 == 0 && ((uintptr_t)X & 15) == 0)
    launch_lmhead_x<MT, CW, MT >= 2>(X, ldx, W, ldw, z, M, N, K, km, pv, pi, pp, s);
  else
    launch_lmhead_x<MT, CW, false>(X, ldx, W, ldw, z, M, N, K, km, pv, pi, pp, s);
}

hipError_t gemm_lmhead_topk(const void* X, int ldx, const void* W, int ldw, float* z, int M, int N,
                            int K, int km, void* part, hipStream_t s) {
  const GemmPlan plan = gemm_plan(M, N, K, true);
  if (plan.nsplit != 1 || plan.tile || (km != 1 && km != 8)) return hipErrorInvalidValue;
  const int nch = gemm_strips(M, N);
  float* pv = (float*)part;
  int* pi = (int*)(pv + (size_t)M * nch * km);
  topkdev::Part* pp = (topkdev::Part*)(pi + (size_t)M * nch * km);
  const bool cw1 = lmhead_cw(M, N) == 1;
  if (M <= 16) {
    if (cw1) launch_lmhead<1, 1>(X, ldx, W, ldw, z, M, N, K, km, pv, pi, pp, s);
    else launch_lmhead<1, 2>(X, ldx, W, ldw, z, M, N, K, km, pv, pi, pp, s);
  } else if (M <= 32) {
    if (cw1) launch_lmhead<2, 1>(X, ldx, W, ldw, z, M, N, K, km, pv, pi, pp, s);
    else launch_lmhead<2, 2>(X, ldx, W, ldw, z, M, N, K, km, pv, pi, pp, s);
  } else {
    if (cw1) launch_lmhead<4, 1>(X, ldx, W, ldw, z, M, N, K, km, pv, pi, pp, s);
    else launch_lmhead<4, 2>(X, ldx, W, ldw, z, M, N, K, km, pv, pi, pp, s);
  }
  return hipGetLastError();
}

hipError_t gemm_epilogue_records(const float* P, int nsplit, int M, int N, float* z, void* rec,
                                 hipStream_t s) {
  const int nstrip = (N + 127) / 128;
  const int64_t waves = (int64_t)M * nstrip;
  SPEC_LAUNCH(epi_f32_rec_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, z, P, nsplit,
              M, N, nstrip, (float2*)rec);
  return hipGetLastError();
}

hipError_t gemm_epilogue(bool bf16, int op, void* Y, const void* R, const float* P, int nsplit,
                         int M, int N, hipStream_t s) {
  const int64_t total = (int64_t)M * N;
  const dim3 grid((unsigned)((total + kEpiCols - 1) / kEpiCols));
  // vector path: few splits, many outputs, rows of whole 4-vectors, aligned
  const auto al = [](const void* q, int b) { return ((uintptr_t)q & (b - 1)) == 0; };
  const int eb = op == EPI_F32 || !bf16 ? 16 : 8;
  if (nsplit <= kEpiGroups && total >= 65536 && N % 4 == 0 && al(P, 16) && al(Y, eb) &&
      (op != EPI_RESID || al(R, eb))) {
    const dim3 vgrid((unsigned)((total / 4 + 255) / 256));
#define SPEC_EPIV(T, OPV)                                                                       \
  SPEC_LAUNCH((epi_vec_kernel<T, OPV>), vgrid, dim3(256), 0, s, (T*)Y, (const T*)R, P,  \
                     nsplit, M, N)
    if (op == EPI_F32) SPEC_EPIV(float, EPI_STORE);
    else if (bf16 && op == EPI_STORE) SPEC_EPIV(bf16_t, EPI_STORE);
    else if (bf16 && op == EPI_RESID) SPEC_EPIV(bf16_t, EPI_RESID);
    else if (bf16) SPEC_EPIV(bf16_t, EPI_SWIGLU);
    else if (op == EPI_STORE) SPEC_EPIV(float, EPI_STORE);
    else if (op == EPI_RESID) SPEC_EPIV(float, EPI_RESID);
    else SPEC_EPIV(float, EPI_SWIGLU);
#undef SPEC_EPIV
    return hipGetLastError();
  }
  if (op == EPI_F32) {
    SPEC_LAUNCH(epi_f32, grid, dim3(256), 0, s, (float*)Y, P, nsplit, total);
    return hipGetLastError();
  }
#define SPEC_EPI(T)                                                                            \
  switch (op) {                                                                                \
    case EPI_STORE:                                                                            \
      SPEC_LAUNCH((epi_kernel<T, EPI_STORE>), grid, dim3(256), 0, s, (T*)Y,             \
                         (const T*)R, P, nsplit, M, N);                                        \
      break;                                                                                   \
    case EPI_RESID:                                                                            \
      SPEC_LAUNCH((epi_kernel<T, EPI_RESID>), grid, dim3(256), 0, s, (T*)Y,             \
                         (const T*)R, P, nsplit, M, N);                                        \
      break;                                                                                   \
    default:                                                                                   \
      SPEC_LAUNCH((epi_kernel<T, EPI_SWIGLU>), grid, dim3(256), 0, s, (T*)Y,            \
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
  const int NH = nq + 2 * nkv;
  if (M >= 64 && hd % 2 == 0 && hd <= 256 && 256 % (hd / 2) == 0) {
    // four blocks per row (about a dozen heads each)
    const int hpb = (NH + 3) / 4;
    const dim3 grid(M, (NH + hpb - 1) / hpb);
    if (bf16) {
      SPEC_LAUNCH(qkv_epi_rows_kernel<bf16_t>, grid, dim3(256), 0, s, P, nsplit, M, nq, nkv, hd,
                  pos, slot, rows_per_seq, rope_base, (bf16_t*)qout, (bf16_t*)kv.k,
                  (bf16_t*)kv.v, kv.stride_seq, kv.stride_head, kv.slots, kv.pg, hpb);
    } else {
      SPEC_LAUNCH(qkv_epi_rows_kernel<float>, grid, dim3(256), 0, s, P, nsplit, M, nq, nkv, hd,
                  pos, slot, rows_per_seq, rope_base, (float*)qout, (float*)kv.k, (float*)kv.v,
                  kv.stride_seq, kv.stride_head, kv.slots, kv.pg, hpb);
    }
    return hipGetLastError();
  }
  dim3 grid(M, NH);
  dim3 block(256);
  if (bf16) {
    SPEC_LAUNCH(qkv_epi_kernel<bf16_t>, grid, block, 0, s, P, nsplit, M, nq, nkv, hd, pos,
                       slot, rows_per_seq, rope_base, (bf16_t*)qout, (bf16_t*)kv.k,
                       (bf16_t*)kv.v, kv.stride_seq, kv.stride_head, kv.slots, kv.pg);
  } else {
    SPEC_LAUNCH(qkv_epi_kernel<float>, grid, block, 0, s, P, nsplit, M, nq, nkv, hd, pos,
                       slot, rows_per_seq, rope_base, (float*)qout, (float*)kv.k, (float*)kv.v,
                       kv.stride_seq, kv.stride_head, kv.slots, kv.pg);
  }
  return hipGetLastError();
}

}  // namespace spec

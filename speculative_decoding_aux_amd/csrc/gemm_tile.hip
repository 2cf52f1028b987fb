// LDS-tiled MFMA GEMM for the beam passes of tree workloads (M > 64 rows):
// P[split][M][N] = X[M, K] . W[N, K]^T over the split's K range.
//
// A 256-thread block owns a BN x BM output tile (BN weight rows x BM X rows)
// and walks K in 64-wide tiles staged through LDS; while the MFMAs consume the
// current tile, each thread's 16-byte global loads of the next tile are in
// flight.  Four waves in a 2 x 2 layout each own a 64 (N) x BM/2 (M) tile of
// v_mfma_f32_16x16x32_bf16 accumulators, so every weight tile of the block is
// read from HBM once for all BM rows.  LDS rows are padded to 72 elements
// (144 B), which makes the 16-lane 16-byte fragment reads conflict-free.
#include "common.h"
#include "kernels.h"

namespace spec {

namespace {

constexpr int kBK = 64;
constexpr int kPitch = kBK + 8;  // bf16 elements per LDS row

template <int BN, int BM>
__global__ __launch_bounds__(256) void gemm_tile_kernel(const bf16_t* __restrict__ X, int ldx,
                                                         const bf16_t* __restrict__ W, int ldw,
                                                         float* __restrict__ P, int M, int N, int K,
                                                         int kc) {
  constexpr int WN = BN / 2, WM = BM / 2;  // wave tile
  constexpr int FA = WN / 16, FB = WM / 16;
  constexpr int CW = BN * kBK / 8 / 256;   // 16-byte chunks per thread per tile
  constexpr int CX = BM * kBK / 8 / 256;
  __shared__ bf16_t ws[BN * kPitch];
  __shared__ bf16_t xs[BM * kPitch];
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const int wn = wave & 1, wm = wave >> 1;
  const int g = lane >> 4, c = lane & 15;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.z * BM;
  const int k0 = blockIdx.y * kc, k1 = min(K, k0 + kc);

  f32x4 acc[FA][FB];
#pragma unroll
  for (int a = 0; a < FA; ++a)
#pragma unroll
    for (int b = 0; b < FB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4_t rw[CW], rx[CX];
  auto load = [&](int k) {
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const int q = t + 256 * i, row = q >> 3, ch = q & 7;
      const int n = n0 + row;
      rw[i] = n < N ? *(const u32x4_t*)(W + (int64_t)n * ldw + k + ch * 8) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < CX; ++i) {
      const int q = t + 256 * i, row = q >> 3, ch = q & 7;
      const int m = m0 + row;
      rx[i] = m < M ? *(const u32x4_t*)(X + (int64_t)m * ldx + k + ch * 8) : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const int q = t + 256 * i, row = q >> 3, ch = q & 7;
      *(u32x4_t*)(ws + row * kPitch + ch * 8) = rw[i];
    }
#pragma unroll
    for (int i = 0; i < CX; ++i) {
      const int q = t + 256 * i, row = q >> 3, ch = q & 7;
      *(u32x4_t*)(xs + row * kPitch + ch * 8) = rx[i];
    }
  };

  if (k0 < k1) {
    load(k0);
    stash();
  }
  __syncthreads();
  for (int k = k0; k < k1; k += kBK) {
    const bool more = k + kBK < k1;
    if (more) load(k + kBK);
#pragma unroll
    for (int s = 0; s < kBK / 32; ++s) {
      u32x4_t fa[FA], fb[FB];
#pragma unroll
      for (int a = 0; a < FA; ++a)
        fa[a] = *(const u32x4_t*)(ws + (wn * WN + a * 16 + c) * kPitch + s * 32 + g * 8);
#pragma unroll
      for (int b = 0; b < FB; ++b)
        fb[b] = *(const u32x4_t*)(xs + (wm * WM + b * 16 + c) * kPitch + s * 32 + g * 8);
#pragma unroll
      for (int a = 0; a < FA; ++a)
#pragma unroll
        for (int b = 0; b < FB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fa[a]),
                                                              __builtin_bit_cast(bf16x8, fb[b]),
                                                              acc[a][b], 0, 0, 0);
    }
    __syncthreads();
    if (more) {
      stash();
      __syncthreads();
    }
  }
  // lane holds Y[m0 + wm*WM + 16b + c][n0 + wn*WN + 16a + 4g + r]
  float* Pb = P + (int64_t)blockIdx.y * M * N;
#pragma unroll
  for (int b = 0; b < FB; ++b) {
    const int m = m0 + wm * WM + 16 * b + c;
    if (m >= M) continue;
#pragma unroll
    for (int a = 0; a < FA; ++a) {
      const int n = n0 + wn * WN + 16 * a + 4 * g;
      float* dst = Pb + (int64_t)m * N + n;
      if (n + 3 < N && (N & 3) == 0) {
        *(float4*)dst = make_float4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]);
      } else {
        for (int r = 0; r < 4; ++r)
          if (n + r < N) dst[r] = acc[a][b][r];
      }
    }
  }
}

}  // namespace

constexpr int kTileBN = 128, kTileBM = 256;

bool gemm_tile_ok(int M, int K) { return M > 64 && K % kBK == 0; }

GemmPlan gemm_tile_plan(int M, int N, int K) {
  GemmPlan p;
  const int strips = (N + kTileBN - 1) / kTileBN;
  const int mblocks = (M + kTileBM - 1) / kTileBM;
  const int ktiles = K / kBK;
  // enough blocks for 256 CUs, but at least 8 K tiles per split
  int ns = (512 + strips * mblocks - 1) / (strips * mblocks);
  ns = std::max(1, std::min(ns, std::max(1, ktiles / 8)));
  const int per = (ktiles + ns - 1) / ns;
  p.kc = per * kBK;
  p.nsplit = (ktiles + per - 1) / per;
  return p;
}

hipError_t gemm_tile(const void* X, int ldx, const void* W, int ldw, float* P, int M, int N, int K,
                     const GemmPlan& plan, hipStream_t s) {
  const dim3 grid((N + kTileBN - 1) / kTileBN, plan.nsplit, (M + kTileBM - 1) / kTileBM);
  hipLaunchKernelGGL((gemm_tile_kernel<kTileBN, kTileBM>), grid, dim3(256), 0, s, (const bf16_t*)X,
                     ldx, (const bf16_t*)W, ldw, P, M, N, K, plan.kc);
  return hipGetLastError();
}

}  // namespace spec

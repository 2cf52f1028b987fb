// LDS-tiled MFMA GEMM for the beam passes of tree workloads (M > 64 rows):
// P[split][M][N] = X[M, K] . W[N, K]^T over the split's K range.
//
// A 512-thread block owns a BN x BM output tile (BN weight rows x BM X rows),
// so each weight tile is read from HBM once for all BM rows, and walks K in
// BK-wide stages that global_load_lds_dwordx4 brings straight into LDS.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace spec {

namespace {

// NTH threads own a BN x BM output tile and walk K in BK-wide stages.  Each
// stage is brought into LDS by global_load_lds_dwordx4 (no staging registers),
// NS stages deep: NS - 1 are in flight while the MFMAs consume one.  A stage
// row is BK * 2 bytes (CH = BK / 8 chunks of 16 bytes); chunk j of row r is
// stored at position j ^ swz(r), swz(r) = (r >> 2) & 3 for 4 chunks and
// (r >> 1) & 7 for 8, so the 16-lane fragment reads of 16 consecutive rows hit
// 16 distinct 16-byte bank groups.
// Synchronisation is a raw s_waitcnt vmcnt lgkmcnt(0) + s_barrier (a
// workgroup fence would drain every stage in flight; lgkmcnt(0) makes the
// reads of the stage before complete, so the refill after the barrier cannot
// overtake them), with compiler fences so that no LDS access moves across it.  Each stage lives in its own LDS object
// and every wave issues the same DMA count per stage, unconditionally (past
// the end the last stage is loaded again), so the compiler can tell a stage's
// reads from the other stages' DMA and adds no wait of its own.
template <int CH>
SPEC_DEV int chunk_swz(int row) {
  return CH == 4 ? (row >> 2) & 3 : (row >> 1) & 7;
}

template <int BN, int BM, int BK, int NTH, int NS>
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2))) void gemm_dma_kernel(
    const bf16_t* __restrict__ X, int ldx, const bf16_t* __restrict__ W, int ldw,
    float* __restrict__ P, int M, int N, int K, int kc) {
  constexpr int NWAVE = NTH / 64;
  constexpr int WGN = BN / 64, WGM = NWAVE / WGN;  // wave grid
  constexpr int WM = BM / WGM;                     // X rows per wave
  constexpr int FA = 4, FB = WM / 16;
  constexpr int CH = BK / 8;                       // 16-byte chunks per stage row
  // wave-level DMA instructions per stage, dealt round-robin to the waves
  // (repeats load the same bytes)
  constexpr int IW = BN * CH / 64, IX = BM * CH / 64;
  constexpr int NW = (IW + NWAVE - 1) / NWAVE, NX = (IX + NWAVE - 1) / NWAVE, NI = NW + NX;
  static_assert(FB >= 1 && WGN * WGM == NWAVE && BM % (16 * WGM) == 0, "tile shape");
  static_assert((BK == 32 || BK == 64) && NS >= 2 && NS <= 4, "stages");
  // one LDS object per stage
  __shared__ u32x4_t w0[BN * CH], w1[BN * CH], w2[NS > 2 ? BN * CH : 1], w3[NS > 3 ? BN * CH : 1];
  __shared__ u32x4_t x0[BM * CH], x1[BM * CH], x2[NS > 2 ? BM * CH : 1], x3[NS > 3 ? BM * CH : 1];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wn = wave % WGN, wm = wave / WGN;
  const int g = lane >> 4, c = lane & 15;
  // Block order: workgroups are dealt to the 8 XCDs round-robin, so ids b and
  // b + 8 share an XCD (and its L2).  The row blocks of one weight strip get
  // ids 8 apart and run together there, and the strip is read from HBM once.
  // The grid is (strips x row blocks, splits): blockIdx.x carries both.
  const int nstrip = (N + BN - 1) / BN, nmb = (M + BM - 1) / BM;
  int strip = blockIdx.x, mb = 0;
  if (nmb > 1) {
    const int b = blockIdx.x;
    const int grp = b / (8 * nmb), rem = b % (8 * nmb);
    strip = grp * 8 + rem % 8;
    mb = rem / 8;
    if (strip >= nstrip) {  // the last group is short: spread its ids over what is left
      const int base = (nstrip / 8) * 8, left = nstrip - base;
      const int q = b - base * nmb;
      strip = base + q % left;
      mb = q / left;
    }
  }
  const int n0 = strip * BN, m0 = mb * BM;
  const int k0 = blockIdx.y * kc, k1 = min(K, k0 + kc);
  const int T = max(0, (k1 - k0) / BK);

  // DMA sources: LDS unit u (row u / CH, position u % CH) holds chunk
  // (u % CH) ^ swz(row)
  const bf16_t* gw[NW];
  const bf16_t* gx[NX];
  int uw[NW], ux[NX];
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    uw[j] = ((wave * NW + j) % IW) * 64;
    const int u = uw[j] + lane, row = u / CH;
    const int ch = (u % CH) ^ chunk_swz<CH>(row);
    gw[j] = W + (int64_t)min(n0 + row, N - 1) * ldw + k0 + ch * 8;
  }
#pragma unroll
  for (int j = 0; j < NX; ++j) {
    ux[j] = ((wave * NX + j) % IX) * 64;
    const int u = ux[j] + lane, row = u / CH;
    const int ch = (u % CH) ^ chunk_swz<CH>(row);
    gx[j] = X + (int64_t)min(m0 + row, M - 1) * ldx + k0 + ch * 8;
  }
  auto wbuf = [](auto sc) -> SPEC_LDS u32x4_t* {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return (SPEC_LDS u32x4_t*)w0;
    else if constexpr (S == 1) return (SPEC_LDS u32x4_t*)w1;
    else if constexpr (S == 2) return (SPEC_LDS u32x4_t*)w2;
    else return (SPEC_LDS u32x4_t*)w3;
  };
  auto xbuf = [](auto sc) -> SPEC_LDS u32x4_t* {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return (SPEC_LDS u32x4_t*)x0;
    else if constexpr (S == 1) return (SPEC_LDS u32x4_t*)x1;
    else if constexpr (S == 2) return (SPEC_LDS u32x4_t*)x2;
    else return (SPEC_LDS u32x4_t*)x3;
  };
  auto issue = [&](auto sc, int i) {
    const int k = min(i, T - 1) * BK;
#pragma unroll
    for (int j = 0; j < NW; ++j) dma16(gw[j] + k, wbuf(sc) + uw[j]);
#pragma unroll
    for (int j = 0; j < NX; ++j) dma16(gx[j] + k, xbuf(sc) + ux[j]);
  };

  f32x4 acc[FA][FB];
#pragma unroll
  for (int a = 0; a < FA; ++a)
#pragma unroll
    for (int b = 0; b < FB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int sw = chunk_swz<CH>(c);  // rows of a fragment start at multiples of 16
  const int rowa = (wn * 64 + c) * CH, rowb = (wm * WM + c) * CH;

  // stage i: wait for this wave's DMA of stage i (the NS - 2 stages after it
  // may still be pending), barrier (every wave's DMA of stage i has landed and
  // every wave is done reading stage i - 1), refill stage i - 1's buffer with
  // stage i + NS - 1, compute stage i.  Past T only the refill runs.
  auto step = [&](auto sc, auto sn, int i) {
    wait_vm_lgkm0<(NS - 2) * NI>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(sn, i + NS - 1);
    if (i < T) {
#pragma unroll
      for (int ks = 0; ks < BK / 32; ++ks) {
        const int pos = (ks * 4 + g) ^ sw;
        u32x4_t fa[FA], fb[FB];
#pragma unroll
        for (int a = 0; a < FA; ++a) fa[a] = wbuf(sc)[rowa + a * 16 * CH + pos];
#pragma unroll
        for (int b = 0; b < FB; ++b) fb[b] = xbuf(sc)[rowb + b * 16 * CH + pos];
#pragma unroll
        for (int a = 0; a < FA; ++a)
#pragma unroll
          for (int b = 0; b < FB; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fa[a]),
                                                                __builtin_bit_cast(bf16x8, fb[b]),
                                                                acc[a][b], 0, 0, 0);
      }
    }
    asm volatile("" ::: "memory");
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  if (T > 0) {
    issue(S0{}, 0);
    if constexpr (NS == 4) {
      issue(S1{}, 1);
      issue(S2{}, 2);
      for (int i = 0; i < T; i += 4) {
        step(S0{}, S3{}, i);
        step(S1{}, S0{}, i + 1);
        step(S2{}, S1{}, i + 2);
        step(S3{}, S2{}, i + 3);
      }
    } else if constexpr (NS == 3) {
      issue(S1{}, 1);
      for (int i = 0; i < T; i += 3) {
        step(S0{}, S2{}, i);
        step(S1{}, S0{}, i + 1);
        step(S2{}, S1{}, i + 2);
      }
    } else {
      for (int i = 0; i < T; i += 2) {
        step(S0{}, S1{}, i);
        step(S1{}, S0{}, i + 1);
      }
    }
    wait_vm_lgkm0<0>();  // the repeated loads past the end
  }
  // lane holds Y[m0 + wm*WM + 16b + c][n0 + wn*64 + 16a + 4g + r]
  float* Pb = P + (int64_t)blockIdx.y * M * N;
#pragma unroll
  for (int b = 0; b < FB; ++b) {
    const int m = m0 + wm * WM + 16 * b + c;
    if (m >= M) continue;
#pragma unroll
    for (int a = 0; a < FA; ++a) {
      const int n = n0 + wn * 64 + 16 * a + 4 * g;
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

// Beam-pass tile: 128 weight rows x 256 X rows, K stages of 64, three stages
// (144 KB of LDS, one block per CU, two waves per SIMD).
constexpr int kTileBN = 128, kTileBM = 256, kTileBK = 64, kTileThreads = 512, kTileStages = 3;

bool gemm_tile_ok(int M, int K) { return M > 64 && K % kTileBK == 0; }

GemmPlan gemm_tile_plan(int M, int N, int K) {
  GemmPlan p;
  const int strips = (N + kTileBN - 1) / kTileBN;
  const int mblocks = (M + kTileBM - 1) / kTileBM;
  const int ktiles = K / kTileBK;
  // One block per CU: split K only while the grid is short of 256 blocks
  // (every split costs an M x N float32 partial), keeping >= 4 stages per split.
  int ns = 256 / std::max(1, strips * mblocks);
  ns = std::max(1, std::min(ns, std::max(1, ktiles / 4)));
  const int per = (ktiles + ns - 1) / ns;
  p.kc = per * kTileBK;
  p.nsplit = (ktiles + per - 1) / per;
  return p;
}

hipError_t gemm_tile(const void* X, int ldx, const void* W, int ldw, float* P, int M, int N, int K,
                     const GemmPlan& plan, hipStream_t s) {
  if (M <= 0 || N <= 0 || K % kTileBK != 0 || plan.kc % kTileBK != 0) return hipErrorInvalidValue;
  const dim3 grid(((N + kTileBN - 1) / kTileBN) * ((M + kTileBM - 1) / kTileBM), plan.nsplit, 1);
  hipLaunchKernelGGL((gemm_dma_kernel<kTileBN, kTileBM, kTileBK, kTileThreads, kTileStages>), grid,
                     dim3(kTileThreads), 0, s, (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, P, M,
                     N, K, plan.kc);
  return hipGetLastError();
}

}  // namespace spec

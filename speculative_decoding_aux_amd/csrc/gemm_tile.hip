// LDS-tiled MFMA GEMM for the beam passes of tree workloads (M > 64 rows):
// P[split][M][N] = X[M, K] . W[N, K]^T over the split's K range.
//
// A 512-thread block owns a BN x BM output tile (BN weight rows x BM X rows),
// so each weight tile is read from HBM once for all BM rows, and walks K in
// BK-wide stages that global_load_lds_dwordx4 brings straight into LDS.
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"
#include "topk_common.h"

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
// overtake them), with compiler fences so that no LDS access moves across it.
// Each stage lives in its own LDS object and every wave issues the same DMA
// count per stage, unconditionally (past the last step the last stage is
// loaded again), so the compiler can tell a stage's reads from the other
// stages' DMA and adds no wait of its own.
template <int CH>
SPEC_DEV int chunk_swz(int row) {
  return CH == 4 ? (row >> 2) & 3 : (row >> 1) & 7;
}

// s_waitcnt lgkmcnt(0) with no vector-memory wait (vmcnt and expcnt at their
// maxima).
SPEC_DEV void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

SPEC_DEV void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int... I, class F>
SPEC_DEV void unroll_seq(std::integer_sequence<int, I...>, F f) {
  (f(std::integral_constant<int, I>{}), ...);
}

// One output tile: weight rows n0.., X rows m0.., K range k0 .. k0 + T * BK.
struct TileGeo {
  int n0, m0, k0, T, split, strip;
};

// Tile t of the launch: t = split * (strips * row blocks) + r.  Workgroups are
// dealt to the 8 XCDs round-robin, so block ids b and b + 8 share an XCD (and
// its L2); with a grid that is a multiple of 8 the same holds for the tiles
// t and t + 8 that a persistent block takes in turn.  The row blocks of one
// weight strip get r values 8 apart, so they run together on one XCD and the
// strip is read from HBM once.
template <int BN, int BM, int BK>
SPEC_DEV TileGeo tile_geo(int t, int M, int N, int K, int kc) {
  const int nstrip = (N + BN - 1) / BN, nmb = (M + BM - 1) / BM, per = nstrip * nmb;
  TileGeo q;
  q.split = t / per;
  const int r = t - q.split * per;
  int strip = r, mb = 0;
  if (nmb > 1) {
    const int grp = r / (8 * nmb);
    if ((grp + 1) * 8 <= nstrip) {  // a full group of 8 strips
      const int rem = r % (8 * nmb);
      strip = grp * 8 + rem % 8;
      mb = rem / 8;
    } else {  // the last group is short: its ids cover the strips that are left
      const int base = grp * 8, left = nstrip - base;
      const int u = r - base * nmb;
      strip = base + u % left;
      mb = u / left;
    }
  }
  q.strip = strip;
  q.n0 = strip * BN;
  q.m0 = mb * BM;
  q.k0 = q.split * kc;
  q.T = (min(K, q.k0 + kc) - q.k0) / BK;
  return q;
}

// PERSIST (more tiles than CUs): block b takes the tiles b, b + G, b + 2G, ...
// (G = grid size) and runs their K steps as one stream, so the DMA of the next
// tile's first stages is in flight while a tile's results are written out.
// Otherwise every block owns one tile.
// REC (unsplit launches, BN = 128): also write, per row and BN-column strip,
// the record (max, sum of exp(v - max)) that the vocab top-k merges.
// SWI (unsplit, one tile per block, two waves across): W is [gate (N/2) |
// up (N/2)] and tile s takes gate rows s*BN/2 .. and the same up rows, the
// first wave across holding gate and the second up; the epilogue writes
// silu(gate) * up as bf16 to Y[M][N/2] (the up values cross through LDS).
template <int BN, int BM, int BK, int NTH, int NS, bool REC, bool PERSIST, bool SWI = false>
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2))) void gemm_dma_kernel(
    const bf16_t* __restrict__ X, int ldx, const bf16_t* __restrict__ W, int ldw,
    float* __restrict__ P, int M, int N, int K, int kc, int ntiles, float2* __restrict__ rec,
    bf16_t* __restrict__ Y) {
  constexpr int NWAVE = NTH / 64;
  constexpr int WGN = BN % 64 == 0 ? BN / 64 : (BN % 32 == 0 ? 2 : 1), WGM = NWAVE / WGN;  // wave grid
  constexpr int WN = BN / WGN, WM = BM / WGM;  // weight rows and X rows per wave
  constexpr int FA = WN / 16, FB = WM / 16;
  constexpr int CH = BK / 8;                       // 16-byte chunks per stage row
  // wave-level DMA instructions per stage, dealt round-robin to the waves
  // (repeats load the same bytes)
  constexpr int IW = BN * CH / 64, IX = BM * CH / 64;
  constexpr int NW = (IW + NWAVE - 1) / NWAVE, NX = (IX + NWAVE - 1) / NWAVE, NI = NW + NX;
  static_assert(FA >= 1 && FB >= 1 && WGN * WGM == NWAVE && BN % (16 * WGN) == 0 &&
                    BM % (16 * WGM) == 0,
                "tile shape");
  static_assert((BK == 32 || BK == 64) && NS >= 2 && NS <= 6, "stages");
  static_assert(!REC || (WGN == 2 && WN == 64), "strip records assume two waves across the strip");
  static_assert(!SWI || (WGN == 2 && !REC && !PERSIST && NS >= 2 && WGM * WM * WN * 4 <= 2 * BM * BK * 2),
                "SwiGLU epilogue: gate and up waves, one tile per block, up values fit two X stages");
  // one LDS object per stage, and the records' exchange (the (max, sum) of
  // the wn = 1 half of each row)
  __shared__ u32x4_t w0[BN * CH], w1[BN * CH], w2[NS > 2 ? BN * CH : 1],
      w3[NS > 3 ? BN * CH : 1], w4[NS > 4 ? BN * CH : 1], w5[NS > 5 ? BN * CH : 1];
  __shared__ u32x4_t x0[BM * CH], x1[BM * CH], x2[NS > 2 ? BM * CH : 1], x3[NS > 3 ? BM * CH : 1],
      x4[NS > 4 ? BM * CH : 1], x5[NS > 5 ? BM * CH : 1];
  __shared__ float2 xr[REC ? BM : 1];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wn = wave % WGN, wm = wave / WGN;
  const int g = lane >> 4, c = lane & 15;
  const int G = gridDim.x, b0 = blockIdx.x;
  // tiles of this block (the grid is <= ntiles; one each unless PERSIST)
  const int J = PERSIST ? (ntiles - 1 - b0) / G + 1 : 1;
  const int nstrip = (N + BN - 1) / BN;

  // DMA slots: LDS unit u (row u / CH, position u % CH) holds chunk
  // (u % CH) ^ swz(row) of that row
  int uw[NW], ux[NX], rw[NW], rx[NX], ow[NW], ox[NX];
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    uw[j] = ((wave * NW + j) % IW) * 64;
    const int u = uw[j] + lane;
    rw[j] = u / CH;
    ow[j] = ((u % CH) ^ chunk_swz<CH>(rw[j])) * 8;
  }
#pragma unroll
  for (int j = 0; j < NX; ++j) {
    ux[j] = ((wave * NX + j) % IX) * 64;
    const int u = ux[j] + lane;
    rx[j] = u / CH;
    ox[j] = ((u % CH) ^ chunk_swz<CH>(rx[j])) * 8;
  }
  const bf16_t* gw[NW];
  const bf16_t* gx[NX];
  auto point = [&](const TileGeo& q) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      int row = min(q.n0 + rw[j], N - 1);
      if constexpr (SWI) {  // local rows [0, BN/2) gate, [BN/2, BN) the matching up rows
        const int r = rw[j] % BN, hn = N / 2;
        row = min(r < BN / 2 ? q.n0 / 2 + r : hn + q.n0 / 2 + r - BN / 2, N - 1);
      }
      gw[j] = W + (int64_t)row * ldw + q.k0 + ow[j];
    }
#pragma unroll
    for (int j = 0; j < NX; ++j) gx[j] = X + (int64_t)min(q.m0 + rx[j], M - 1) * ldx + q.k0 + ox[j];
  };
  auto wbuf = [](auto sc) -> SPEC_LDS u32x4_t* {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return (SPEC_LDS u32x4_t*)w0;
    else if constexpr (S == 1) return (SPEC_LDS u32x4_t*)w1;
    else if constexpr (S == 2) return (SPEC_LDS u32x4_t*)w2;
    else if constexpr (S == 3) return (SPEC_LDS u32x4_t*)w3;
    else if constexpr (S == 4) return (SPEC_LDS u32x4_t*)w4;
    else return (SPEC_LDS u32x4_t*)w5;
  };
  auto xbuf = [](auto sc) -> SPEC_LDS u32x4_t* {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return (SPEC_LDS u32x4_t*)x0;
    else if constexpr (S == 1) return (SPEC_LDS u32x4_t*)x1;
    else if constexpr (S == 2) return (SPEC_LDS u32x4_t*)x2;
    else if constexpr (S == 3) return (SPEC_LDS u32x4_t*)x3;
    else if constexpr (S == 4) return (SPEC_LDS u32x4_t*)x4;
    else return (SPEC_LDS u32x4_t*)x5;
  };

  int S = 0;  // K steps of all the block's tiles
  for (int j = 0; j < J; ++j) S += tile_geo<BN, BM, BK>(b0 + j * G, M, N, K, kc).T;
  // issue cursor: tile ij of the block, K step ii; it stays on the last step
  // once the block's stream is exhausted
  int ij = 0, ii = 0;
  TileGeo iq = tile_geo<BN, BM, BK>(b0, M, N, K, kc);
  const TileGeo q0 = iq;
  point(iq);
  auto issue = [&](auto sc) __attribute__((always_inline)) {
    const int k = ii * BK;
#pragma unroll
    for (int j = 0; j < NW; ++j) dma16(gw[j] + k, wbuf(sc) + uw[j]);
#pragma unroll
    for (int j = 0; j < NX; ++j) dma16(gx[j] + k, xbuf(sc) + ux[j]);
    if (ii + 1 < iq.T) {
      ++ii;
    } else if (ij + 1 < J) {
      ++ij;
      ii = 0;
      iq = tile_geo<BN, BM, BK>(b0 + ij * G, M, N, K, kc);
      point(iq);
    }
  };

  f32x4 acc[FA][FB];
#pragma unroll
  for (int a = 0; a < FA; ++a)
#pragma unroll
    for (int b = 0; b < FB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int sw = chunk_swz<CH>(c);  // rows of a fragment start at multiples of 16
  const int rowa = (wn * WN + c) * CH, rowb = (wm * WM + c) * CH;

  // lane holds Y[m0 + wm*WM + 16b + c][n0 + wn*64 + 16a + 4g + r]
  auto epilogue = [&](const TileGeo& q) __attribute__((always_inline)) {
    if constexpr (SWI) {
      // the up wave (wn = 1) of each row block hands its values to the gate
      // wave (wn = 0) through the (now idle) X stages; then silu(g) * u
      float* ex = (float*)(wm < WGM / 2 ? (SPEC_LDS u32x4_t*)x0 : (SPEC_LDS u32x4_t*)x1) +
                  (wm % (WGM / 2)) * WM * WN;
      block_barrier();  // every wave is done with the stages
      if (wn == 1) {
#pragma unroll
        for (int b = 0; b < FB; ++b)
#pragma unroll
          for (int a = 0; a < FA; ++a)
            *(f32x4*)(ex + (16 * b + c) * WN + 16 * a + 4 * g) = acc[a][b];
      }
      wait_lgkm0();
      block_barrier();
      if (wn == 0) {
        const int hn = N / 2;
#pragma unroll
        for (int b = 0; b < FB; ++b) {
          const int m = q.m0 + wm * WM + 16 * b + c;
          if (m >= M) continue;
#pragma unroll
          for (int a = 0; a < FA; ++a) {
            const int n = q.n0 / 2 + 16 * a + 4 * g;
            const f32x4 u = *(const f32x4*)(ex + (16 * b + c) * WN + 16 * a + 4 * g);
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float gt = acc[a][b][r];
              v[r] = gt / (1.f + expf(-gt)) * u[r];
            }
            bf16_t* dst = Y + (int64_t)m * hn + n;
            if (n + 3 < hn) {
              uint2 w2;
              w2.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
              w2.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
              *(uint2*)dst = w2;
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (n + r < hn) dst[r] = f32_to_bf16(v[r]);
            }
          }
        }
      }
      return;
    }
    float* Pb = P + (int64_t)q.split * M * N;
#pragma unroll
    for (int b = 0; b < FB; ++b) {
      const int m = q.m0 + wm * WM + 16 * b + c;
      if (m >= M) continue;
#pragma unroll
      for (int a = 0; a < FA; ++a) {
        const int n = q.n0 + wn * WN + 16 * a + 4 * g;
        float* dst = Pb + (int64_t)m * N + n;
        if (n + 3 < N && (N & 3) == 0) {
          *(float4*)dst = make_float4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) dst[r] = acc[a][b][r];
        }
      }
    }
    if constexpr (REC) {
      // (max, sum exp) per row over the strip: the lane's 16 values, the four
      // lane groups of the wave by shuffles, the two waves of a row via LDS
      constexpr float kL2e = 1.4426950408889634f;
      const bool full = q.n0 + BN <= N;
      const int nl = N - (q.n0 + wn * WN + 4 * g);  // this lane's columns below N: 16a + r < nl
      float rm[FB], rs[FB];
#pragma unroll
      for (int b = 0; b < FB; ++b) {
        float m = -INFINITY, sum = 0.f;
#pragma unroll
        for (int a = 0; a < FA; ++a)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (full || 16 * a + r < nl) m = fmaxf(m, acc[a][b][r]);
        if (m != -INFINITY) {
          const float mo = m * kL2e;
#pragma unroll
          for (int a = 0; a < FA; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (full || 16 * a + r < nl)
                sum += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[a][b][r], kL2e, -mo));
        }
#pragma unroll
        for (int o = 16; o <= 32; o <<= 1) {
          const float om = xor_hi(m, o), os = xor_hi(sum, o);
          const float nm = fmaxf(m, om);
          if (nm != -INFINITY)
            sum = (m == -INFINITY ? 0.f : sum * __builtin_amdgcn_exp2f((m - nm) * kL2e)) +
                  (om == -INFINITY ? 0.f : os * __builtin_amdgcn_exp2f((om - nm) * kL2e));
          m = nm;
        }
        rm[b] = m;
        rs[b] = sum;
        if (wn == 1 && g == 0) xr[wm * WM + 16 * b + c] = make_float2(m, sum);
      }
      wait_lgkm0();
      block_barrier();
      if (wn == 0 && g == 0) {
#pragma unroll
        for (int b = 0; b < FB; ++b) {
          const int row = wm * WM + 16 * b + c, m = q.m0 + row;
          const float2 o = xr[row];
          const float nm = fmaxf(rm[b], o.x);
          float sum = 0.f;
          if (nm != -INFINITY)
            sum = (rm[b] == -INFINITY ? 0.f : rs[b] * __builtin_amdgcn_exp2f((rm[b] - nm) * kL2e)) +
                  (o.x == -INFINITY ? 0.f : o.y * __builtin_amdgcn_exp2f((o.x - nm) * kL2e));
          if (m < M) rec[(int64_t)m * nstrip + q.strip] = make_float2(nm, sum);
        }
      }
    }
  };

  // K step s of the block's stream: wait for this wave's DMA of step s (the
  // NS - 2 steps after it may still be pending), barrier (every wave's DMA of
  // step s has landed and every wave is done reading the previous stage),
  // refill the previous stage's buffer with step s + NS - 1, compute step s.
  // After a tile's last step the tile is written out while the next tile's
  // first stages load; then every access of the wave is waited for (loads and
  // stores may complete out of order, so no partial count is safe past a
  // store).  The block's last tile is written out after the stream, when no
  // loads are left to overlap.
  int ci = 0, cj = 0;
  TileGeo cq = q0;
  auto step = [&](auto sc, auto sn, int s) __attribute__((always_inline)) {
    wait_vm_lgkm0<(NS - 2) * NI>();
    block_barrier();
    issue(sn);
    if (s < S) {
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
      if (PERSIST && ++ci == cq.T && cj + 1 < J) {
        epilogue(cq);
#pragma unroll
        for (int a = 0; a < FA; ++a)
#pragma unroll
          for (int b = 0; b < FB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        ci = 0;
        cq = tile_geo<BN, BM, BK>(b0 + ++cj * G, M, N, K, kc);
        wait_vm_lgkm0<0>();
      }
    }
    asm volatile("" ::: "memory");
  };
  unroll_seq(std::make_integer_sequence<int, NS - 1>{}, [&](auto sc) { issue(sc); });
  for (int s = 0; s < S; s += NS) {
    unroll_seq(std::make_integer_sequence<int, NS>{}, [&](auto sc) {
      constexpr int i = decltype(sc)::value;
      step(sc, std::integral_constant<int, (i + NS - 1) % NS>{}, s + i);
    });
  }
  wait_vm_lgkm0<0>();  // the repeated loads past the end
  epilogue(cq);        // the block's last tile
}

}  // namespace

// Beam-pass tile: 128 (or 96, 112 or 64) weight rows x 256 X rows, K stages of 64,
// three stages (up to 144 KB of LDS, one block per CU, two waves per SIMD).
constexpr int kTileBN = 128, kTileBM = 256, kTileBK = 64, kTileThreads = 512, kTileStages = 3;
constexpr int kTileBNNarrow = 96, kTileBN112 = 112, kTileBN64 = 64;

bool gemm_tile_ok(int M, int K) { return M > 64 && K % kTileBK == 0; }

GemmPlan gemm_tile_plan(int M, int N, int K) {
  // One block per CU: split K only while the grid is short of 256 blocks
  // (every split costs an M x N float32 partial), keeping >= 4 stages per split.
  // Of the strip widths, the one with the least work on the busiest CU:
  // rounds of tiles x (strip width + a fixed cost per step of 32 rows) x (steps
  // per tile + 6 for filling the stages and writing the tile).
  GemmPlan best;
  int64_t best_cost = 0;
  for (const int bn : {kTileBN, kTileBNNarrow, kTileBN112, kTileBN64}) {
    GemmPlan p;
    p.bn = bn;
    const int strips = (N + bn - 1) / bn;
    const int mblocks = (M + kTileBM - 1) / kTileBM;
    const int ktiles = K / kTileBK;
    int ns = 256 / std::max(1, strips * mblocks);
    ns = std::max(1, std::min(ns, std::max(1, ktiles / 4)));
    const int per = (ktiles + ns - 1) / ns;
    p.kc = per * kTileBK;
    p.nsplit = (ktiles + per - 1) / per;
    const int64_t tiles = (int64_t)strips * mblocks * p.nsplit;
    const int64_t cost = (tiles + 255) / 256 * (bn + 32) * (per + 6);
    if (bn == kTileBN || cost < best_cost) {
      best = p;
      best_cost = cost;
    }
  }
  return best;
}

namespace {

// Persistent grid: one block per CU (a block takes 144 KB of LDS), a multiple
// of 8 so that a block's successive tiles stay on one XCD.
int tile_grid(int ntiles) {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8)
      n = 8;
    cus[dev] = n / 8 * 8;
  }
  return std::min(ntiles, cus[dev]);
}

template <bool REC, int BN, bool SWI = false>
hipError_t launch_tile(const void* X, int ldx, const void* W, int ldw, float* P, int M, int N,
                       int K, int kc, int nsplit, float2* rec, hipStream_t s,
                       bf16_t* Y = nullptr) {
  if (M <= 0 || N <= 0 || K % kTileBK != 0 || kc % kTileBK != 0 || kc <= 0 || nsplit < 1 ||
      (int64_t)(nsplit - 1) * kc >= K)
    return hipErrorInvalidValue;
  const int ntiles = ((N + BN - 1) / BN) * ((M + kTileBM - 1) / kTileBM) * nsplit;
  const int grid = tile_grid(ntiles);
  if constexpr (SWI) {
    if (grid < ntiles || nsplit != 1 || N % BN != 0 || !Y) return hipErrorInvalidValue;
    SPEC_LAUNCH((gemm_dma_kernel<BN, kTileBM, kTileBK, kTileThreads, kTileStages, false, false, true>),
                dim3(ntiles), dim3(kTileThreads), 0, s, (const bf16_t*)X, ldx, (const bf16_t*)W,
                ldw, P, M, N, K, kc, ntiles, rec, Y);
  } else if (grid < ntiles) {
    SPEC_LAUNCH((gemm_dma_kernel<BN, kTileBM, kTileBK, kTileThreads, kTileStages, REC, true>),
                dim3(grid), dim3(kTileThreads), 0, s, (const bf16_t*)X, ldx, (const bf16_t*)W,
                ldw, P, M, N, K, kc, ntiles, rec, Y);
  } else {
    SPEC_LAUNCH((gemm_dma_kernel<BN, kTileBM, kTileBK, kTileThreads, kTileStages, REC, false>),
                dim3(ntiles), dim3(kTileThreads), 0, s, (const bf16_t*)X, ldx, (const bf16_t*)W,
                ldw, P, M, N, K, kc, ntiles, rec, Y);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_tile(const void* X, int ldx, const void* W, int ldw, float* P, int M, int N, int K,
                     const GemmPlan& plan, hipStream_t s) {
  if (plan.bn == kTileBNNarrow)
    return launch_tile<false, kTileBNNarrow>(X, ldx, W, ldw, P, M, N, K, plan.kc, plan.nsplit,
                                             nullptr, s);
  if (plan.bn == kTileBN112)
    return launch_tile<false, kTileBN112>(X, ldx, W, ldw, P, M, N, K, plan.kc, plan.nsplit,
                                          nullptr, s);
  if (plan.bn == kTileBN64)
    return launch_tile<false, kTileBN64>(X, ldx, W, ldw, P, M, N, K, plan.kc, plan.nsplit,
                                         nullptr, s);
  return launch_tile<false, kTileBN>(X, ldx, W, ldw, P, M, N, K, plan.kc, plan.nsplit, nullptr, s);
}

int gemm_tile_strips(int N) { return (N + kTileBN - 1) / kTileBN; }

bool gemm_tile_swiglu_ok(int M, int N, int K, const GemmPlan& plan) {
  if (!plan.tile || plan.nsplit != 1 || plan.bn != kTileBNNarrow || N % kTileBNNarrow != 0 ||
      K % kTileBK != 0)
    return false;
  const int ntiles = (N / kTileBNNarrow) * ((M + kTileBM - 1) / kTileBM);
  return tile_grid(ntiles) >= ntiles;
}

hipError_t gemm_tile_swiglu(const void* X, int ldx, const void* W, int ldw, void* Y, int M, int N,
                            int K, const GemmPlan& plan, hipStream_t s) {
  if (!gemm_tile_swiglu_ok(M, N, K, plan)) return hipErrorInvalidValue;
  return launch_tile<false, kTileBNNarrow, true>(X, ldx, W, ldw, nullptr, M, N, K, plan.kc, 1,
                                                 nullptr, s, (bf16_t*)Y);
}

hipError_t gemm_tile_records(const void* X, int ldx, const void* W, int ldw, float* z, int M,
                             int N, int K, void* rec, hipStream_t s) {
  return launch_tile<true, kTileBN>(X, ldx, W, ldw, z, M, N, K, K, 1, (float2*)rec, s);
}

}  // namespace spec

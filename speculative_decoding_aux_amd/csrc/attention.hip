// Tree-masked GQA decode attention of the draft layer.
//
// The visible keys of a row are the sequence's context slots [lo, ctx_len)
// (lo = pos - W + 1 under a sliding window of W keys, else 0) plus the row's
// own list of extra slots (root rows, tree ancestors, itself) whose positions
// run consecutively up to the row's position.  Every row of a sequence shares
// the context, so the context is split into chunks and each workgroup streams
// one chunk of one (sequence, kv-head) once for all R rows x G q-heads of that
// kv-head (online softmax in float32, partial (max, sum, O) per query vector).
// A combine kernel merges the chunk partials with the few extra keys of each
// row and normalises.  When one workgroup can take a (sequence, kv-head)'s
// whole context (all rows in one launch, a short context per wave), it also
// attends the rows' extra keys and writes the normalised output itself: no
// partials and no combine launch.  Scores are q.k / sqrt(hd).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace spec {

namespace {

constexpr int kTile = 64;  // keys per tile (one per lane)

// Element e of a 16-byte vector holding 8 bf16 or 4 float32 values.
template <typename T> SPEC_DEV float unpack(const u32x4_t& w, int e);
template <> SPEC_DEV float unpack<float>(const u32x4_t& w, int e) { return __uint_as_float(w[e]); }
template <> SPEC_DEV float unpack<bf16_t>(const u32x4_t& w, int e) {
  const uint32_t x = w[e >> 1];
  return __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
}

// N consecutive values (N = 1 or 2) as floats, by one load or store.
template <typename T, int N>
SPEC_DEV void load_dims(const T* p, float (&x)[N]) {
  if constexpr (N == 1) {
    x[0] = St<T>::load(p, 0);
  } else if constexpr (std::is_same<T, float>::value) {
    const float2 v = *(const float2*)p;
    x[0] = v.x;
    x[1] = v.y;
  } else {
    const uint32_t v = *(const uint32_t*)p;
    x[0] = __uint_as_float(v << 16);
    x[1] = __uint_as_float(v & 0xffff0000u);
  }
}
template <typename T, int N>
SPEC_DEV void store_dims(T* p, const float (&x)[N]) {
  if constexpr (N == 1) {
    St<T>::store(p, 0, x[0]);
  } else if constexpr (std::is_same<T, float>::value) {
    *(float2*)p = make_float2(x[0], x[1]);
  } else {
    *(uint32_t*)p = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
  }
}

// Final attention output of one query vector (row r, q-head h), computed by
// one wave: merge the context-chunk records with the row's extra keys.  Lane l
// holds dims DPL*l .. DPL*l + DPL - 1 (DPL = HD / 64) of q, of the output and
// of every K and V row it reads, so an extra key's score is a wave-wide sum
// and a row is one coalesced load of DPL consecutive values per lane.  Extra keys go in batches of eight (their K and V rows
// loaded together); the loads that depend on nothing (q, the extra-key
// slots, the first chunk records) are issued first and the first batch's rows
// as soon as the slots arrive, so the wave waits on two round trips to memory.
template <typename T, int HD>
SPEC_DEV void combine_qv(int r, int h, const T* __restrict__ q, const T* __restrict__ kc,
                         const T* __restrict__ vc, int64_t sseq, int64_t shead, int S, KvPages pg,
                         const int* __restrict__ pos, const int* __restrict__ anc, int A, int R,
                         int nq, int nkv, int window, int nch, const float* __restrict__ part,
                         T* __restrict__ out) {
  constexpr int DPL = HD / 64;  // dims per lane
  constexpr int PC = 32;        // chunk records prefetched (the first round trip)
  constexpr int CG = 16;        // chunk records in flight per group after them
  constexpr int KB = 8;         // extra keys per batch
  const int lane = threadIdx.x & 63;
  const int G = nq / nkv, kvh = h / G;
  const int b = r / R, qv = (r % R) * G + h % G, QV = R * G;
  const float inv_sqrt = 1.0f / sqrtf((float)HD);
  const float* pb = part + ((int64_t)(b * nkv + kvh) * nch * QV + qv) * (HD + 2);
  const int64_t cstride = (int64_t)QV * (HD + 2);
  // round trip 1: slots, q, chunk records
  const int sl = lane < A ? anc[(int64_t)r * A + lane] : -1;
  const int pq = pos[r];
  float qr[DPL];
  load_dims<T, DPL>(q + ((int64_t)r * nq + h) * HD + DPL * lane, qr);
  float pm = -INFINITY, pl = 0.f;
  if (lane < nch) {
    pm = pb[lane * cstride + HD];
    pl = pb[lane * cstride + HD + 1];
  }
  float po[PC][DPL];
#pragma unroll
  for (int c = 0; c < PC; ++c) {
    if (c < nch) {
      load_dims<float, DPL>(pb + c * cstride + DPL * lane, po[c]);
    } else {
#pragma unroll
      for (int i = 0; i < DPL; ++i) po[c][i] = 0.f;
    }
  }
  // extra keys: valid entries hold consecutive positions ending at pos[r]
  const unsigned long long vmask = __ballot(sl >= 0);
  const int nvalid = __popcll(vmask);
  const int rank = __popcll(vmask & ((1ull << lane) - 1ull));
  const bool vis = sl >= 0 && sl < S && (window <= 0 || pq - (nvalid - 1 - rank) > pq - window);
  const unsigned long long kmask = __ballot(vis);
  // each lane's own extra slot as an element offset (a page lookup when paged)
  const long long soff = vis ? (long long)kv_slot_off(pg, b, sl, sseq, HD) : 0ll;
  const T* kb = kc + kvh * shead;
  const T* vb = vc + kvh * shead;
  float kv[KB][DPL], vv[KB][DPL];
  auto load_batch = [&](int j0) {
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int j = j0 + u;
      const bool ok = j < 64 && ((kmask >> j) & 1ull);
      const int64_t row = (int64_t)__shfl(soff, j & 63, 64) + DPL * lane;
      if (ok) {
        load_dims<T, DPL>(kb + row, kv[u]);
        load_dims<T, DPL>(vb + row, vv[u]);
      } else {
#pragma unroll
        for (int i = 0; i < DPL; ++i) kv[u][i] = vv[u][i] = 0.f;
      }
    }
  };
  // round trip 2: the first batch of extra keys
  load_batch(0);
  // context chunks: their maximum, then the rescaled sums
  float m = pm;
  for (int c = lane + 64; c < nch; c += 64) m = fmaxf(m, pb[c * cstride + HD]);
  m = wave_max(m);
  float l = 0.f;
  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] = 0.f;
  if (m != -INFINITY) {
    float lc = pm == -INFINITY ? 0.f : pl * expf(pm - m);
    for (int c = lane + 64; c < nch; c += 64) {
      const float mc = pb[c * cstride + HD];
      if (mc != -INFINITY) lc += pb[c * cstride + HD + 1] * expf(mc - m);
    }
    l = wave_sum_uniform(lc);
#pragma unroll
    for (int c = 0; c < PC; ++c) {
      const float mc = __shfl(pm, c, 64);
      if (c < nch && mc != -INFINITY) {
        const float w = expf(mc - m);
#pragma unroll
        for (int i = 0; i < DPL; ++i) o[i] += po[c][i] * w;
      }
    }
    // the remaining chunk records, CG chunks' loads in flight at a time (the
    // maxima of the first 64 chunks are already in the lanes)
    for (int c0 = PC; c0 < nch; c0 += CG) {
      float mq[CG], oq[CG][DPL];
#pragma unroll
      for (int u = 0; u < CG; ++u) {
        const int c = c0 + u;
        const float sm = __shfl(pm, c & 63, 64);
        mq[u] = c >= nch ? -INFINITY : (c < 64 ? sm : pb[c * cstride + HD]);
        if (c < nch) {
          load_dims<float, DPL>(pb + c * cstride + DPL * lane, oq[u]);
        } else {
#pragma unroll
          for (int i = 0; i < DPL; ++i) oq[u][i] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < CG; ++u) {
        if (mq[u] == -INFINITY) continue;
        const float w = expf(mq[u] - m);
#pragma unroll
        for (int i = 0; i < DPL; ++i) o[i] += oq[u][i] * w;
      }
    }
  }
  // extra keys, batch by batch: scores, running max, rescale, accumulate
#pragma unroll 1
  for (int j0 = 0; j0 < 64 && (kmask >> j0); j0 += KB) {
    if (j0 > 0) load_batch(j0);
    float s[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) a += qr[i] * kv[u][i];
      s[u] = wave_sum_uniform(a) * inv_sqrt;
    }
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < KB; ++u)
      if (j0 + u < 64 && ((kmask >> (j0 + u)) & 1ull)) bm = fmaxf(bm, s[u]);
    const float mn = fmaxf(m, bm);
    if (mn == -INFINITY) continue;
    if (mn != m) {
      const float alpha = m == -INFINITY ? 0.f : expf(m - mn);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[i] *= alpha;
      m = mn;
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (!(j0 + u < 64 && ((kmask >> (j0 + u)) & 1ull))) continue;
      const float p = expf(s[u] - m);
      l += p;
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[i] += p * vv[u][i];
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] *= inv;
  store_dims<T, DPL>(out + ((int64_t)r * nq + h) * HD + DPL * lane, o);
}

// One wave per (row, q-head).
template <typename T, int HD>
__global__ __launch_bounds__(64) void attn_combine_kernel(const T* __restrict__ q,
                                                          const T* __restrict__ kc,
                                                          const T* __restrict__ vc, int64_t sseq,
                                                          int64_t shead, int S, KvPages pg,
                                                          const int* __restrict__ pos,
                                                          const int* __restrict__ anc, int A,
                                                          int R, int nq, int nkv, int window,
                                                          int nch, const float* __restrict__ part,
                                                          T* __restrict__ out) {
  combine_qv<T, HD>(blockIdx.x, blockIdx.y, q, kc, vc, sseq, shead, S, pg, pos, anc, A, R, nq, nkv,
                    window, nch, part, out);
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_ctx_kernel(const T* __restrict__ q,
                                                       const T* __restrict__ kc,
                                                       const T* __restrict__ vc, int64_t sseq,
                                                       int64_t shead, int S, KvPages pg,
                                                       const int* __restrict__ ctx_len,
                                                       const int* __restrict__ pos, int R, int r0,
                                                       int Rg, int nq, int nkv, int window,
                                                       int chunk, float* __restrict__ part) {
  extern __shared__ float smem[];
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int nch = gridDim.x;
  const int G = nq / nkv;
  // rows r0 .. r0 + Rg - 1 of each sequence (see attn_ctx_mfma_kernel)
  const int QV = Rg * G, QVF = R * G;
  float* qs = smem;                  // [QV][HD]
  float* sc = qs + QV * HD;          // [QV][kTile]
  float* mrow = sc + QV * kTile;     // [QV]
  float* lrow = mrow + QV;
  float* srow = lrow + QV;
  int* lo = (int*)(srow + QV);       // [QV]
  float* red = (float*)(lo + QV);    // [NG][QV][HD] when the keys are split
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float inv_sqrt = 1.0f / sqrtf((float)HD);

  const int ctx = clampi(ctx_len[b], 0, S);
  int minpos = 0x7fffffff;
  for (int r = 0; r < R; ++r) minpos = min(minpos, pos[b * R + r]);
  const int start = window > 0 ? max(0, minpos - window + 1) : 0;
  const int k0 = start + c * chunk;
  const int k1 = min(ctx, k0 + chunk);

  for (int i = threadIdx.x; i < QV * HD; i += blockDim.x) {
    const int qv = i / HD, d = i % HD;
    const int r = r0 + qv / G, h = kvh * G + qv % G;
    qs[i] = St<T>::load(q, ((int64_t)(b * R + r) * nq + h) * HD + d);
  }
  for (int i = threadIdx.x; i < QV; i += blockDim.x) {
    mrow[i] = -INFINITY;
    lrow[i] = 0.f;
    lo[i] = window > 0 ? max(0, pos[b * R + r0 + i / G] - window + 1) : 0;
  }
  __syncthreads();

  const T* kb = kc + kvh * shead;  // rows at kv_slot_off(pg, b, key, ...)
  const T* vb = vc + kvh * shead;
  constexpr int NG = 256 / HD;          // PV thread groups
  const int d = threadIdx.x % HD, grp = threadIdx.x / HD;
  constexpr int NJ = (64 + NG - 1) / NG;  // accumulators per thread, enough for 64 vectors
  // the ones this thread's group uses (uniform across a wave: a group is one
  // or two whole waves), so the unused ones are skipped by scalar branches
  const int jn = __builtin_amdgcn_readfirstlane(QV > grp ? (QV - grp + NG - 1) / NG : 0);
  // few query vectors (at most half the groups): every group takes every
  // vector over its own keys (key % NG == group), the groups summed at the end
  const bool ksplit = 2 * QV <= NG;
  float acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = 0.f;

  for (int t0 = k0; t0 < k1; t0 += kTile) {
    // scores: lane = key, wave w takes query vectors w, w+4, ...
    const int key = t0 + lane;
    const bool kok = key < k1;
    float kv[HD];
    if (kok) {
      // 16-byte loads of the key row
      const u32x4_t* kr = (const u32x4_t*)(kb + kv_slot_off(pg, b, key, sseq, HD));
      constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte vector
#pragma unroll
      for (int vq = 0; vq < HD / EPV; ++vq) {
        const u32x4_t w = kr[vq];
#pragma unroll
        for (int e = 0; e < EPV; ++e) kv[vq * EPV + e] = unpack<T>(w, e);
      }
    }
    for (int qv = wave; qv < QV; qv += 4) {
      float s = -INFINITY;
      if (kok && key >= lo[qv]) {
        float a = 0.f;
        const float* qq = qs + qv * HD;
#pragma unroll
        for (int e = 0; e < HD; ++e) a += qq[e] * kv[e];
        s = a * inv_sqrt;
      }
      const float mt = wave_max(s);
      const float mo = mrow[qv];
      const float mn = fmaxf(mo, mt);
      const float p = s == -INFINITY ? 0.f : expf(s - mn);
      const float ps = wave_sum(p);
      sc[qv * kTile + lane] = p;
      if (lane == 0) {
        const float scale = mo == -INFINITY ? (mn == -INFINITY ? 1.f : 0.f) : expf(mo - mn);
        srow[qv] = scale;
        lrow[qv] = lrow[qv] * scale + ps;
        mrow[qv] = mn;
      }
    }
    __syncthreads();
    // O[qv][d] = O * scale + sum_key p[qv][key] * V[key][d]
    const int nk = min(kTile, k1 - t0);
    if (ksplit) {
      constexpr int KPG = kTile / NG;  // keys per group per tile
#pragma unroll
      for (int qv = 0; qv < NG / 2; ++qv)
        if (qv < QV) acc[qv] *= srow[qv];
      float vk[KPG];
#pragma unroll
      for (int u = 0; u < KPG; ++u) {
        const int kk = grp + NG * u;
        vk[u] = kk < nk ? St<T>::load(vb, kv_slot_off(pg, b, t0 + kk, sseq, HD) + d) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < KPG; ++u) {
        const int kk = grp + NG * u;
        if (kk >= nk) break;
#pragma unroll
        for (int qv = 0; qv < NG / 2; ++qv)
          if (qv < QV) acc[qv] += sc[qv * kTile + kk] * vk[u];
      }
      __syncthreads();
      continue;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j >= jn) break;
      acc[j] *= srow[grp + j * NG];
    }
    // V rows in batches of 8 keys: the loads of a batch are independent
    for (int kk0 = 0; kk0 < nk; kk0 += 8) {
      float v8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v8[u] = kk0 + u < nk ? St<T>::load(vb, kv_slot_off(pg, b, t0 + kk0 + u, sseq, HD) + d) : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (kk0 + u >= nk) break;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if (j >= jn) break;
          acc[j] += sc[(grp + j * NG) * kTile + kk0 + u] * v8[u];
        }
      }
    }
    __syncthreads();
  }
  // partial record per query vector: O[HD], m, l
  float* pb = part + (((int64_t)(b * nkv + kvh) * nch + c) * QVF + r0 * G) * (HD + 2);
  if (ksplit) {
#pragma unroll
    for (int qv = 0; qv < NG / 2; ++qv)
      if (qv < QV) red[(grp * QV + qv) * HD + d] = acc[qv];
    __syncthreads();
    for (int i = threadIdx.x; i < QV * HD; i += blockDim.x) {
      float o = 0.f;
#pragma unroll
      for (int gg = 0; gg < NG; ++gg) o += red[gg * QV * HD + i];
      pb[(i / HD) * (HD + 2) + i % HD] = o;
    }
  } else {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (j >= jn) break;
      pb[(grp + j * NG) * (HD + 2) + d] = acc[j];
    }
  }
  for (int i = threadIdx.x; i < QV; i += blockDim.x) {
    pb[i * (HD + 2) + HD] = mrow[i];
    pb[i * (HD + 2) + HD + 1] = lrow[i];
  }
}


// ---- bf16 context attention on MFMA -----------------------------------------
// Each wave walks blocks of 16 keys, wave w taking blocks w, w + NW, ... of
// the chunk (NW = 4 or 8 waves), one block ahead of use: the V rows go into a
// wave-private LDS stage by global_load_lds_dwordx4 (two stages per wave, 8 KB
// per wave at hd 128) and the K rows load straight into registers in MFMA fragment layout as
// soon as the previous block's scores are done, so the key loop has no
// workgroup barrier, every load is 16 bytes wide and several workgroups share
// a CU.
// S^T = K . Q^T (16x16x32 bf16 MFMA) takes K rows as the A operand (lane:
// key = lane&15, 8 dims at 8*(lane>>4)) and the query vectors as B, so the
// score tile lands with key 4*(lane>>4)+i and query column lane&15 - exactly
// the B-operand layout of the 16x16x16 bf16 MFMA of O^T = V^T . P^T over the
// 16 keys.  The V^T fragment of 16 dims takes keys 4g..4g+3 at dim lane&15
// from LDS with 2-byte reads; V row r keeps its 16-byte chunk j at position
// j ^ 2((r >> 2) & 3), so the four key rows of one read hit distinct bank
// groups.  P goes in as two bf16 parts (hi + lo), keeping the float32 softmax
// weights to about 16 bits.  The query fragments sit in LDS, shared by the
// waves.  Online softmax runs per query column (shuffles across the four
// lane groups); the waves are merged pairwise through LDS at the end.
typedef short s16x4 __attribute__((ext_vector_type(4)));

SPEC_DEV uint2 pack4(const float (&v)[4]) {
  return make_uint2((uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16),
                    (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16));
}

SPEC_DEV int v_swz(int r) { return 2 * ((r >> 2) & 3); }

template <int HD, int QT, int NW, bool FUSE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW == 8 ? 2 : 3))) void attn_ctx_mfma_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    int64_t sseq, int64_t shead, int S, KvPages pg, const int* __restrict__ ctx_len,
    const int* __restrict__ pos, int R, int r0, int Rg, int nq, int nkv, int window, int chunk,
    const int* __restrict__ anc, int A, float* __restrict__ part, bf16_t* __restrict__ out) {
  constexpr int DS = HD / 32;        // 32-dim steps of S^T
  constexpr int DT = HD / 16;        // 16-dim tiles of O^T
  constexpr int CH = HD / 8;         // 16-byte chunks per row
  constexpr int BLK = 16 * CH;       // 16-byte units per 16-row V block
  constexpr int NI = BLK / 64;       // DMA instructions per V block
  constexpr int NL = DS + NI;        // vector loads per block (K fragments + V DMA)
  constexpr int KS = NW * 16;        // keys from one of a wave's blocks to its next
  static_assert(NL < 64 && NI < 64, "vmcnt range");
  static_assert(HD == 64 || HD == 128, "head dim");
  static_assert(NW == 4 || NW == 8, "waves");
  // two V stages, one LDS object each; a wave owns BLK units of each
  __shared__ u32x4_t v0s[NW * BLK], v1s[NW * BLK];
  // query fragments (B operand of S^T), [t][ds][lane], shared by the waves
  __shared__ u32x4_t qsh[QT * DS * 64];
  // merge buffers: slots of [QT][DT][64] accumulators in the V stages (free
  // after the key loop), [NW / 2][QT][64] max and sum
  constexpr int SLOT = QT * DT * 64;
  constexpr int CAP = NW * BLK / SLOT;  // merge slots per V stage
  static_assert(CAP >= 1 && 2 * CAP >= NW / 2, "merge slots fit in the V stages");
  __shared__ float mm[NW / 2 * QT * 64], ml[NW / 2 * QT * 64];
  // paged caches: the blocks of the pages this chunk touches, read once;
  // with eight waves the table also pads the workgroup's LDS past half of a
  // CU's 160 KB, so no CU takes two of them
  constexpr int LDS0 = 2 * NW * BLK * 16 + QT * DS * 64 * 16 + 2 * (NW / 2) * QT * 64 * 4;
  constexpr int PTAB = NW == 8 && (84 * 1024 - LDS0) / 4 > kAttnMaxChunkPages
                           ? (84 * 1024 - LDS0) / 4
                           : kAttnMaxChunkPages;
  __shared__ int ptab[PTAB];
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int nch = gridDim.x;
  // this launch's query vectors: rows r0 .. r0 + Rg - 1 of each sequence
  // (local index qv = (r - r0) * G + head), recorded at r * G + head of the
  // R * G vectors of the sequence
  const int G = nq / nkv, QV = Rg * G, QVF = R * G;
  const int lane = threadIdx.x & 63, g = lane >> 4, col = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // scores in log2 units (x * log2 e / sqrt(hd)), so the softmax uses the
  // hardware exp2; the records store the running max back in natural units
  const float scale = 1.4426950408889634f / sqrtf((float)HD);

  const int ctx = clampi(ctx_len[b], 0, S);
  int minpos = 0x7fffffff;
  for (int r = 0; r < R; ++r) minpos = min(minpos, pos[b * R + r]);
  const int start = window > 0 ? max(0, minpos - window + 1) : 0;
  const int k0 = start + c * chunk;
  const int k1 = min(ctx, k0 + chunk);
  const int first = k0 + wave * 16;
  const int nblk = first < k1 ? (k1 - first + KS - 1) / KS : 0;

  // every key the kernel touches lies in [kmin, kmax] (clamped reads past
  // the end included)
  const int kmax = max(k1 - 1, 0), kmin = min(k0, kmax);
  const int pg0 = pg.tbl ? kmin / pg.bs : 0;
  const int npg = pg.tbl ? min(kmax / pg.bs - pg0 + 1, kAttnMaxChunkPages) : 0;
  for (int i = threadIdx.x; i < npg; i += 64 * NW) {
    const int page = min(pg0 + i, pg.mb - 1);
    const int blk = pg.tbl[(int64_t)b * pg.mb + page];
    ptab[i] = blk < 0 ? 0 : (blk >= pg.nblk ? pg.nblk - 1 : blk);
  }
  // element offset of key row `key` of this sequence (head 0)
  auto koff = [&](int key) -> int64_t {
    if (!pg.tbl) return (int64_t)b * sseq + (int64_t)key * HD;
    const int page = key / pg.bs;
    const int i = min(max(page - pg0, 0), npg - 1);
    return (int64_t)ptab[i] * sseq + (int64_t)(key - page * pg.bs) * HD;
  };

  int loq[QT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    const int qv = t * 16 + col;
    const bool ok = qv < QV;
    const int r = r0 + (ok ? qv / G : 0), h = kvh * G + (ok ? qv % G : 0);
    if (wave == 0) {
      const bf16_t* qp = q + ((int64_t)(b * R + r) * nq + h) * HD + g * 8;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        qsh[(t * DS + ds) * 64 + lane] = ok ? *(const u32x4_t*)(qp + ds * 32) : u32x4_t{0u, 0u, 0u, 0u};
    }
    loq[t] = ok ? (window > 0 ? max(0, pos[b * R + r] - window + 1) : 0) : 0x7fffffff;
  }
  __syncthreads();
  float mrun[QT], lrun[QT];
  f32x4 o[QT][DT];
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    mrun[t] = -INFINITY;
    lrun[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const bf16_t* kb = kc + kvh * shead;  // key rows at koff(key)
  const bf16_t* vb = vc + kvh * shead;

  auto vbuf = [](auto sc) -> SPEC_LDS u32x4_t* {
    if constexpr (decltype(sc)::value == 0) return (SPEC_LDS u32x4_t*)v0s;
    else return (SPEC_LDS u32x4_t*)v1s;
  };
  u32x4_t kf[DS];  // K fragments: loaded for block i + 1 once block i's scores are done
  auto issue_k = [&](int i) {
    const int base = first + min(i, max(nblk - 1, 0)) * KS;
    const bf16_t* kp = kb + koff(min(base + col, max(k1 - 1, 0))) + g * 8;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) kf[ds] = *(const u32x4_t*)(kp + ds * 32);
  };
  // V rows of block i (past the end: the last block again, never used)
  auto issue_v = [&](auto sc, int i) {
    const int base = first + min(i, max(nblk - 1, 0)) * KS;
    // unit u of a block is row u / CH at position u % CH, holding chunk
    // (u % CH) ^ v_swz(row)
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int u = j * 64 + lane, row = u / CH;
      const int key = min(base + row, kmax);
      dma16(vb + koff(key) + ((u % CH) ^ v_swz(row)) * 8, vbuf(sc) + wave * BLK + j * 64);
    }
  };

  // One 16-key block: V rows in LDS at vs, K fragments in kf.  S^T tiles by
  // MFMA, then after_s() (the K fragments are free), then the online softmax
  // per query column over the keys vis(t, e) admits (key 4g + e of the block
  // for this lane's query vector of tile t) and O^T += V^T . P^T.
  auto attend = [&](const SPEC_LDS bf16_t* vs, auto after_s, auto vis) {
    f32x4 sc4[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      sc4[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        sc4[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, kf[ds]),
            __builtin_bit_cast(bf16x8, qsh[(t * DS + ds) * 64 + lane]), sc4[t], 0, 0, 0);
    }
    after_s();
    uint2 pf[QT], pl[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      float v[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = vis(t, e) ? sc4[t][e] * scale : -INFINITY;
        tmax = fmaxf(tmax, v[e]);
      }
      {
        float a, bb;
        swap16(tmax, a, bb);
        tmax = fmaxf(a, bb);
        swap32(tmax, a, bb);
        tmax = fmaxf(a, bb);
      }
      const float mnew = fmaxf(mrun[t], tmax);
      const float alpha = mrun[t] == -INFINITY ? (mnew == -INFINITY ? 1.f : 0.f)
                                               : __builtin_amdgcn_exp2f(mrun[t] - mnew);
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = v[e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(v[e] - mnew);
        psum += v[e];
      }
      {
        float a, bb;
        swap16(psum, a, bb);
        psum = a + bb;
        swap32(psum, a, bb);
        psum = a + bb;
      }
      lrun[t] = lrun[t] * alpha + psum;
      mrun[t] = mnew;
      // P = P_hi + P_lo in two bf16 parts (about 16 significant bits), so the
      // products with V carry the float32 softmax weights, not bf16-rounded ones
      pf[t] = pack4(v);
      float vlo[4];
      vlo[0] = v[0] - __uint_as_float(pf[t].x << 16);
      vlo[1] = v[1] - __uint_as_float(pf[t].x & 0xffff0000u);
      vlo[2] = v[2] - __uint_as_float(pf[t].y << 16);
      vlo[3] = v[3] - __uint_as_float(pf[t].y & 0xffff0000u);
      pl[t] = pack4(vlo);
      // the accumulators need rescaling only when some query's max moved
      if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[t][dt] *= alpha;
      }
    }
    // V^T fragment of dims dt*16 + col, keys 4g..4g+3, by one transposed LDS
    // read (ds_read_b64_tr_b16): within each 16-lane group, lane s points at
    // key 4g + s/4, dims dt*16 + 4(s%4) .. +3, and lane t receives dim
    // dt*16 + t of the group's four keys
    const int trow = 4 * g + (col >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d0 = dt * 16 + 4 * (col & 3);
      SPEC_LDS s16x4* ap =
          (SPEC_LDS s16x4*)(vs + (trow * CH + ((d0 >> 3) ^ v_swz(trow))) * 8 + (d0 & 7));
      const uint2 vf = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(ap));
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vf),
                                                            __builtin_bit_cast(s16x4, pf[t]),
                                                            o[t][dt], 0, 0, 0);
        o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vf),
                                                            __builtin_bit_cast(s16x4, pl[t]),
                                                            o[t][dt], 0, 0, 0);
      }
    }
  };

  auto block = [&](auto sc, auto sn, int i) {
    // refill the other V stage (read by this wave's previous block, whose LDS
    // reads have completed) with block i + 1, then wait for everything issued
    // before it: this block's V stage and K fragments
    wait_vm_lgkm0<NL>();
    asm volatile("" ::: "memory");
    issue_v(sn, i + 1);
    wait_vm_lgkm0<NI>();
    asm volatile("" ::: "memory");
    if (i >= nblk) return;
    const int kb0 = first + i * KS;
    attend((const SPEC_LDS bf16_t*)(vbuf(sc) + wave * BLK), [&] { issue_k(i + 1); },
           [&](int t, int e) {
             const int key = kb0 + 4 * g + e;
             return key < k1 && key >= loq[t];
           });
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  if (nblk > 0) {
    issue_v(S0{}, 0);
    issue_k(0);
    for (int i = 0; i < nblk; i += 2) {
      block(S0{}, S1{}, i);
      block(S1{}, S0{}, i + 1);
    }
  }
  wait_vm_lgkm0<0>();  // the repeated loads past the end

  if constexpr (FUSE) {
    // The whole context is this workgroup's (one chunk): the rows' extra keys
    // (root rows, tree ancestors, itself) are attended here as well, wave w
    // taking rows w, w + NW, ...  A row's list holds its slots (-1: none)
    // with consecutive positions ending at the row's own; lane l takes entry
    // l, and the keys go in blocks of 16 through the same MFMA step, visible
    // to the query vectors of that row only.
    for (int rr = wave; rr < Rg; rr += NW) {
      const int grow = b * R + r0 + rr;
      const int pq = pos[grow];
      const int sl = lane < A ? anc[(int64_t)grow * A + lane] : -1;
      const unsigned long long vmask = __ballot(sl >= 0);
      const int nvalid = __popcll(vmask);
      const int rank = __popcll(vmask & ((1ull << lane) - 1ull));
      const bool vis = sl >= 0 && sl < S && (window <= 0 || pq - (nvalid - 1 - rank) > pq - window);
      const unsigned long long kmask = __ballot(vis);
      // each lane's entry as an element offset (an in-range row when hidden)
      const int64_t soff = kv_slot_off(pg, b, vis ? sl : 0, sseq, HD);
      for (int j0 = 0; j0 < 64 && (kmask >> j0) != 0ull; j0 += 16) {
        wait_vm_lgkm0<0>();  // the stage's previous reads are done
        asm volatile("" ::: "memory");
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int u = j * 64 + lane, row = u / CH;
          const int64_t ro = __shfl(soff, (j0 + row) & 63, 64);
          dma16(vb + ro + ((u % CH) ^ v_swz(row)) * 8, vbuf(S0{}) + wave * BLK + j * 64);
        }
        {
          const bf16_t* kp = kb + __shfl(soff, (j0 + col) & 63, 64) + g * 8;
#pragma unroll
          for (int ds = 0; ds < DS; ++ds) kf[ds] = *(const u32x4_t*)(kp + ds * 32);
        }
        wait_vm_lgkm0<0>();
        asm volatile("" ::: "memory");
        attend((const SPEC_LDS bf16_t*)(vbuf(S0{}) + wave * BLK), [] {}, [&](int t, int e) {
          const int qv = t * 16 + col, key = j0 + 4 * g + e;
          return qv < QV && qv / G == rr && key < 64 && ((kmask >> key) & 1ull);
        });
      }
    }
    wait_vm_lgkm0<0>();
  }
  __syncthreads();  // every wave is done with the V stages
  auto slotp = [&](int sl) -> f32x4* {
    return (f32x4*)(sl < CAP ? v0s : v1s) + (sl % CAP) * SLOT;
  };

  // merge the waves pairwise through LDS, the upper half into the lower
#pragma unroll
  for (int half = NW / 2; half >= 1; half /= 2) {
    if (wave >= half && wave < 2 * half) {
      const int slot = wave - half;
      f32x4* mo = slotp(slot);
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        mm[(slot * QT + t) * 64 + lane] = mrun[t];
        ml[(slot * QT + t) * 64 + lane] = lrun[t];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) mo[(t * DT + dt) * 64 + lane] = o[t][dt];
      }
    }
    __syncthreads();
    if (wave < half) {
      const f32x4* mo = slotp(wave);
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        const float mb = mm[(wave * QT + t) * 64 + lane], lb = ml[(wave * QT + t) * 64 + lane];
        const float M = fmaxf(mrun[t], mb);
        const float ea = mrun[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun[t] - M);
        const float eb = mb == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mb - M);
        lrun[t] = lrun[t] * ea + lb * eb;
        mrun[t] = M;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[t][dt] = o[t][dt] * ea + mo[(t * DT + dt) * 64 + lane] * eb;
      }
    }
    __syncthreads();
  }
  if (wave == 0) {
    if constexpr (FUSE) {
      // normalised output of each query vector: dims dt*16 + 4g .. +3
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        const int qv = t * 16 + col;
        if (qv >= QV) continue;
        const int r = r0 + qv / G, h = kvh * G + qv % G;
        const float inv = lrun[t] > 0.f ? 1.f / lrun[t] : 0.f;
        bf16_t* op = out + ((int64_t)(b * R + r) * nq + h) * HD + 4 * g;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const float w[4] = {o[t][dt][0] * inv, o[t][dt][1] * inv, o[t][dt][2] * inv,
                              o[t][dt][3] * inv};
          *(uint2*)(op + dt * 16) = pack4(w);
        }
      }
    } else {
      float* pb = part + (((int64_t)(b * nkv + kvh) * nch + c) * QVF + r0 * G) * (HD + 2);
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        const int qv = t * 16 + col;
        if (qv >= QV) continue;
        float* rec = pb + (int64_t)qv * (HD + 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) rec[dt * 16 + 4 * g + i] = o[t][dt][i];
        if (g == 0) {
          rec[HD] = mrun[t] * 0.6931471805599453f;  // log2 units -> natural
          rec[HD + 1] = lrun[t];
        }
      }
    }
  }
}

// One-chunk attention: at most this many 16-key blocks per wave.
constexpr int kFuseMaxBlocks = 24;

int cu_count() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 1;
    cus[dev] = n;
  }
  return cus[dev];
}

template <int HD, int QT, int NW, bool FUSE>
void launch_ctx(const AttnArgs& a, dim3 grid, size_t lds, int r0, int Rg, int chunk,
                hipStream_t s) {
  SPEC_LAUNCH((attn_ctx_mfma_kernel<HD, QT, NW, FUSE>), grid, dim3(64 * NW), lds, s,
              (const bf16_t*)a.q, (const bf16_t*)a.kv.k, (const bf16_t*)a.kv.v, a.kv.stride_seq,
              a.kv.stride_head, a.kv.slots, a.kv.pg, a.ctx_len, a.pos, a.R, r0, Rg, a.nq, a.nkv,
              a.window, chunk, a.anc, a.A, a.part, (bf16_t*)a.out);
}

template <typename T, int HD>
hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  const int G = a.nq / a.nkv;
  const bool mfma = std::is_same<T, bf16_t>::value;
  if (mfma) {
    // All of a sequence's rows in one launch and a short context per wave:
    // one workgroup per (sequence, kv-head) takes the whole context and the
    // rows' extra keys and writes the output (no chunk records, no combine).
    // Eight waves when the workgroups fit the CUs one each (their LDS keeps
    // a second one off a CU), else four, two per CU.
    const int span = a.window > 0 ? std::min(a.window, a.kv.slots) : a.kv.slots;
    const int nw = a.B * a.nkv <= cu_count() ? 8 : 4;
    const bool pages_ok = !a.kv.pg.tbl || span / a.kv.pg.bs + 2 <= kAttnMaxChunkPages;
    if (a.R * G <= 32 && a.A <= 64 && pages_ok && span <= nw * 16 * kFuseMaxBlocks) {
      const int chunk = (span + nw * 16 - 1) / (nw * 16) * (nw * 16);
      const dim3 grid(1, a.nkv, a.B);
      const bool one = a.R * G <= 16;
      if (nw == 8) {
        if (one) launch_ctx<HD, 1, 8, true>(a, grid, 0, 0, a.R, chunk, s);
        else launch_ctx<HD, 2, 8, true>(a, grid, 0, 0, a.R, chunk, s);
      } else {
        if (one) launch_ctx<HD, 1, 4, true>(a, grid, 0, 0, a.R, chunk, s);
        else launch_ctx<HD, 2, 4, true>(a, grid, 0, 0, a.R, chunk, s);
      }
      return hipGetLastError();
    }
  }
  const dim3 grid(a.nchunks, a.nkv, a.B);
  // query vectors go in groups of rows: up to 32 vectors per launch on the
  // bf16 MFMA path (two 16-vector tiles), 64 on the scalar path; each group
  // streams the context chunk again, so one group is the common case (the
  // draft's beam rows) and several only serve large trees (the target's
  // verification forward)
  const int rg = std::max(1, (mfma ? 32 : 64) / G);
  for (int r0 = 0; r0 < a.R; r0 += rg) {
    const int Rg = std::min(rg, a.R - r0);
    const int QV = Rg * G;
    if (mfma && QV <= 16) {
      launch_ctx<HD, 1, 4, false>(a, grid, 0, r0, Rg, a.chunk, s);
    } else if (mfma) {
      launch_ctx<HD, 2, 4, false>(a, grid, 0, r0, Rg, a.chunk, s);
    } else {
      const size_t lds = (size_t)QV * (HD + kTile + 3) * sizeof(float) + QV * sizeof(int) +
                         (2 * QV <= 256 / HD ? (size_t)(256 / HD) * QV * HD * sizeof(float) : 0);
      SPEC_LAUNCH((attn_ctx_kernel<T, HD>), grid, dim3(256), lds, s, (const T*)a.q,
                  (const T*)a.kv.k, (const T*)a.kv.v, a.kv.stride_seq, a.kv.stride_head,
                  a.kv.slots, a.kv.pg, a.ctx_len, a.pos, a.R, r0, Rg, a.nq, a.nkv, a.window,
                  a.chunk, a.part);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SPEC_LAUNCH((attn_combine_kernel<T, HD>), dim3(a.B * a.R, a.nq), dim3(64), 0, s,
                     (const T*)a.q, (const T*)a.kv.k, (const T*)a.kv.v, a.kv.stride_seq,
                     a.kv.stride_head, a.kv.slots, a.kv.pg, a.pos, a.anc, a.A, a.R, a.nq, a.nkv,
                     a.window,
                     a.nchunks, a.part, (T*)a.out);
  return hipGetLastError();
}

}  // namespace

void attn_plan(int B, int nkv, int slots, int window, int* nchunks, int* chunk) {
  const int span = window > 0 ? std::min(window, slots) : slots;
  const int units = std::max(1, B * nkv);
  // about two workgroups per CU; chunks of at least 128 keys (two 16-key
  // blocks per wave), so the combine step has few records per row to merge
  int nc = (512 + units - 1) / units;
  const int max_nc = std::max(1, (span + 127) / 128);
  nc = std::max(1, std::min(nc, max_nc));
  int ch = (span + nc - 1) / nc;
  ch = (ch + 63) / 64 * 64;  // whole 16-key blocks for each of the 4 waves
  *chunk = ch;
  *nchunks = (span + ch - 1) / ch;
}

size_t attn_part_floats(int B, int nkv, int R, int nq, int hd, int nchunks) {
  return (size_t)B * nkv * nchunks * R * (nq / nkv) * (hd + 2);
}

hipError_t attention(bool bf16, const AttnArgs& a, hipStream_t s) {
  if (bf16) return a.hd == 128 ? launch_attn<bf16_t, 128>(a, s) : launch_attn<bf16_t, 64>(a, s);
  return a.hd == 128 ? launch_attn<float, 128>(a, s) : launch_attn<float, 64>(a, s);
}

}  // namespace spec

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
// row and normalises.  Scores are q.k / sqrt(hd).
#include "common.h"
#include "kernels.h"

namespace spec {

namespace {

constexpr int kTile = 64;  // keys per tile (one per lane)

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_ctx_kernel(const T* __restrict__ q,
                                                       const T* __restrict__ kc,
                                                       const T* __restrict__ vc, int64_t sseq,
                                                       int64_t shead, int S,
                                                       const int* __restrict__ ctx_len,
                                                       const int* __restrict__ pos, int R, int nq,
                                                       int nkv, int window, int chunk,
                                                       float* __restrict__ part) {
  extern __shared__ float smem[];
  const int c = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int nch = gridDim.x;
  const int G = nq / nkv;
  const int QV = R * G;
  float* qs = smem;                  // [QV][HD]
  float* sc = qs + QV * HD;          // [QV][kTile]
  float* mrow = sc + QV * kTile;     // [QV]
  float* lrow = mrow + QV;
  float* srow = lrow + QV;
  int* lo = (int*)(srow + QV);       // [QV]
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
    const int r = qv / G, h = kvh * G + qv % G;
    qs[i] = St<T>::load(q, ((int64_t)(b * R + r) * nq + h) * HD + d);
  }
  for (int i = threadIdx.x; i < QV; i += blockDim.x) {
    mrow[i] = -INFINITY;
    lrow[i] = 0.f;
    lo[i] = window > 0 ? max(0, pos[b * R + i / G] - window + 1) : 0;
  }
  __syncthreads();

  const T* kb = kc + b * sseq + kvh * shead;
  const T* vb = vc + b * sseq + kvh * shead;
  constexpr int NG = 256 / HD;          // PV thread groups
  const int d = threadIdx.x % HD, grp = threadIdx.x / HD;
  float acc[(64 + NG - 1) / NG];
#pragma unroll
  for (int j = 0; j < (64 + NG - 1) / NG; ++j) acc[j] = 0.f;

  for (int t0 = k0; t0 < k1; t0 += kTile) {
    // scores: lane = key, wave w takes query vectors w, w+4, ...
    const int key = t0 + lane;
    const bool kok = key < k1;
    float kv[HD];
    if (kok) {
      const T* kr = kb + (int64_t)key * HD;
#pragma unroll
      for (int e = 0; e < HD; ++e) kv[e] = St<T>::load(kr, e);
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
#pragma unroll
    for (int j = 0; j < (64 + NG - 1) / NG; ++j) {
      const int qv = grp + j * NG;
      if (qv < QV) acc[j] *= srow[qv];
    }
    for (int kk = 0; kk < nk; ++kk) {
      const float v = St<T>::load(vb, (int64_t)(t0 + kk) * HD + d);
#pragma unroll
      for (int j = 0; j < (64 + NG - 1) / NG; ++j) {
        const int qv = grp + j * NG;
        if (qv < QV) acc[j] += sc[qv * kTile + kk] * v;
      }
    }
    __syncthreads();
  }
  // partial record per query vector: O[HD], m, l
  float* pb = part + (((int64_t)(b * nkv + kvh) * nch + c) * QV) * (HD + 2);
#pragma unroll
  for (int j = 0; j < (64 + NG - 1) / NG; ++j) {
    const int qv = grp + j * NG;
    if (qv < QV) pb[qv * (HD + 2) + d] = acc[j];
  }
  for (int i = threadIdx.x; i < QV; i += blockDim.x) {
    pb[i * (HD + 2) + HD] = mrow[i];
    pb[i * (HD + 2) + HD + 1] = lrow[i];
  }
}

// One wave per (row, q-head).
template <typename T, int HD>
__global__ __launch_bounds__(64) void attn_combine_kernel(const T* __restrict__ q,
                                                          const T* __restrict__ kc,
                                                          const T* __restrict__ vc, int64_t sseq,
                                                          int64_t shead, int S,
                                                          const int* __restrict__ pos,
                                                          const int* __restrict__ anc, int A,
                                                          int R, int nq, int nkv, int window,
                                                          int nch, const float* __restrict__ part,
                                                          T* __restrict__ out) {
  constexpr int DPL = HD / 64;  // dims per lane
  const int r = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int G = nq / nkv, kvh = h / G;
  const int b = r / R, qv = (r % R) * G + h % G, QV = R * G;
  const float inv_sqrt = 1.0f / sqrtf((float)HD);
  float qd[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) qd[i] = St<T>::load(q, ((int64_t)r * nq + h) * HD + lane + 64 * i);

  const float* pb = part + ((int64_t)(b * nkv + kvh) * nch * QV + qv) * (HD + 2);
  const int64_t cstride = (int64_t)QV * (HD + 2);
  float m = -INFINITY;
  for (int c = 0; c < nch; ++c) m = fmaxf(m, pb[c * cstride + HD]);

  // extra keys: valid entries hold consecutive positions ending at pos[r]
  const int* ar = anc + (int64_t)r * A;
  int nvalid = 0;
  for (int j = 0; j < A; ++j) nvalid += ar[j] >= 0;
  const int pq = pos[r];
  const T* kb = kc + b * sseq + kvh * shead;
  const T* vb = vc + b * sseq + kvh * shead;
  __shared__ float sx[64];
  int jv = 0;
  for (int j = 0; j < A && jv < 64; ++j) {
    const int sl = ar[j];
    if (sl < 0) continue;
    const int pk = pq - (nvalid - 1 - jv);
    float s = -INFINITY;
    if (sl < S && (window <= 0 || pk > pq - window)) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) a += qd[i] * St<T>::load(kb, (int64_t)sl * HD + lane + 64 * i);
      s = wave_sum(a) * inv_sqrt;
    }
    sx[jv++] = s;
    m = fmaxf(m, s);
  }
  float l = 0.f;
  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] = 0.f;
  if (m != -INFINITY) {
    for (int c = 0; c < nch; ++c) {
      const float mc = pb[c * cstride + HD];
      if (mc == -INFINITY) continue;
      const float w = expf(mc - m);
      l += pb[c * cstride + HD + 1] * w;
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[i] += pb[c * cstride + lane + 64 * i] * w;
    }
    jv = 0;
    for (int j = 0; j < A && jv < 64; ++j) {
      const int sl = ar[j];
      if (sl < 0) continue;
      const float s = sx[jv++];
      if (s == -INFINITY) continue;
      const float w = expf(s - m);
      l += w;
#pragma unroll
      for (int i = 0; i < DPL; ++i) o[i] += w * St<T>::load(vb, (int64_t)sl * HD + lane + 64 * i);
    }
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int i = 0; i < DPL; ++i) St<T>::store(out, ((int64_t)r * nq + h) * HD + lane + 64 * i, o[i] * inv);
}

template <typename T, int HD>
hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  const int G = a.nq / a.nkv;
  const int QV = a.R * G;
  const size_t lds = (size_t)QV * (HD + kTile + 3) * sizeof(float) + QV * sizeof(int);
  hipLaunchKernelGGL((attn_ctx_kernel<T, HD>), dim3(a.nchunks, a.nkv, a.B), dim3(256), lds, s,
                     (const T*)a.q, (const T*)a.kv.k, (const T*)a.kv.v, a.kv.stride_seq,
                     a.kv.stride_head, a.kv.slots, a.ctx_len, a.pos, a.R, a.nq, a.nkv, a.window,
                     a.chunk, a.part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_combine_kernel<T, HD>), dim3(a.B * a.R, a.nq), dim3(64), 0, s,
                     (const T*)a.q, (const T*)a.kv.k, (const T*)a.kv.v, a.kv.stride_seq,
                     a.kv.stride_head, a.kv.slots, a.pos, a.anc, a.A, a.R, a.nq, a.nkv, a.window,
                     a.nchunks, a.part, (T*)a.out);
  return hipGetLastError();
}

}  // namespace

void attn_plan(int B, int nkv, int slots, int window, int* nchunks, int* chunk) {
  const int span = window > 0 ? std::min(window, slots) : slots;
  const int units = std::max(1, B * nkv);
  int nc = (1024 + units - 1) / units;
  const int max_nc = std::max(1, (span + 255) / 256);
  nc = std::max(1, std::min(nc, max_nc));
  int ch = (span + nc - 1) / nc;
  ch = (ch + kTile - 1) / kTile * kTile;
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

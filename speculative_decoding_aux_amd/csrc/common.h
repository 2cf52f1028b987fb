// Shared device helpers for the gfx950 speculation-step kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

#define SPEC_DEV __device__ __forceinline__

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));  // 16-byte load unit

constexpr int kWave = 64;

#define SPEC_LDS __attribute__((address_space(3)))

// 16 bytes per lane from global memory straight into LDS
// (global_load_lds_dwordx4): lane i's bytes land at dst + 16 i, dst uniform.
// Completion is counted by vmcnt like any vector load.
SPEC_DEV void dma16(const void* src, SPEC_LDS void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt in bits [3:0] and
// [15:14], expcnt [6:4], lgkmcnt [11:8]): at most N vector loads of this wave
// outstanding, and every LDS access issued so far complete.
template <int N>
SPEC_DEV void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

SPEC_DEV float bf16_to_f32(bf16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// float -> bfloat16, round to nearest even (NaN stays NaN).
SPEC_DEV bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return bf16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return bf16_t(u >> 16);
}

// Storage-type traits: T is float (fp32 workloads) or bf16_t.
template <typename T> struct St;
template <> struct St<float> {
  static SPEC_DEV float load(const float* p, int64_t i) { return p[i]; }
  static SPEC_DEV void store(float* p, int64_t i, float v) { p[i] = v; }
  static SPEC_DEV float round(float v) { return v; }
};
template <> struct St<bf16_t> {
  static SPEC_DEV float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  static SPEC_DEV void store(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
  static SPEC_DEV float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};

// ---- wavefront reductions (64 lanes) --------------------------------------
SPEC_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
SPEC_DEV double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
// Lane exchange within rows of 16 lanes by DPP (no LDS round trip):
// CTRL 0xB1 / 0x4E swap lanes xor 1 / xor 2 within quads, 0x141 mirrors each
// half-row (lane i <-> 7 - i), 0x140 each row (i <-> 15 - i).  Applied in that
// order they pair every lane with one lane of each other quad, half-row and
// row half, so a commutative, associative reduction reaches the whole row.
template <int CTRL>
SPEC_DEV int dpp_row(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
SPEC_DEV float dpp_row(float x) {
  return __int_as_float(dpp_row<CTRL>(__float_as_int(x)));
}
SPEC_DEV float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Row-pair and half-wave exchanges (gfx950 permlane swaps, no LDS round
// trip): with both operands x, permlane16_swap returns rows (x0, x0, x2, x2)
// and (x1, x1, x3, x3) of 16 lanes, permlane32_swap the halves (xlo, xlo) and
// (xhi, xhi).  Combining the two results commutatively equals combining each
// lane with lane ^ 16 (^ 32); the partner value itself is picked by row parity.
SPEC_DEV void swap16(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
SPEC_DEV void swap32(float x, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
// x of lane ^ 16 and lane ^ 32
SPEC_DEV float xor16(float x) {
  float a, b;
  swap16(x, a, b);
  return ((threadIdx.x >> 4) & 1) ? a : b;
}
SPEC_DEV float xor32(float x) {
  float a, b;
  swap32(x, a, b);
  return ((threadIdx.x >> 5) & 1) ? a : b;
}
SPEC_DEV int xor16(int x) { return __float_as_int(xor16(__int_as_float(x))); }
SPEC_DEV int xor32(int x) { return __float_as_int(xor32(__int_as_float(x))); }
// lane ^ o for o = 16 or 32 (uniform)
template <typename V>
SPEC_DEV V xor_hi(V x, int o) {
  return o == 16 ? xor16(x) : xor32(x);
}

SPEC_DEV float wave_max(float v) {
  v = fmaxf(v, dpp_row<0xB1>(v));
  v = fmaxf(v, dpp_row<0x4E>(v));
  v = fmaxf(v, dpp_row<0x141>(v));
  v = fmaxf(v, dpp_row<0x140>(v));
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

// Wave-wide sum by DPP row reductions and four lane reads: the same value in
// every lane (the row sums are added in the order of rows 0..3).
SPEC_DEV float wave_sum_uniform(float v) {
  v += dpp_row<0xB1>(v);
  v += dpp_row<0x4E>(v);
  v += dpp_row<0x141>(v);
  v += dpp_row<0x140>(v);
  return ((lane_f(v, 0) + lane_f(v, 16)) + lane_f(v, 32)) + lane_f(v, 48);
}

// Block-wide sum of one float (blockDim.x a multiple of 64, <= 1024).
SPEC_DEV float block_sum(float v, float* red /* >= 16 floats of LDS */) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  const int nw = blockDim.x >> 6;
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}
SPEC_DEV double block_sum(double v, double* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  const int nw = blockDim.x >> 6;
  double t = 0.0;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// (value desc, id asc) ordering used by every top-k and argmax (bitwise
// combination: both comparisons are evaluated, so no branch is emitted).
SPEC_DEV bool better(float va, int ia, float vb, int ib) {
  return (va > vb) | ((va == vb) & (ia < ib));
}

// ---- Philox4x32-10 (Salmon, Moraes, Dror, Shaw; SC'11) ----------------------
struct u32x4 { uint32_t x, y, z, w; };
SPEC_DEV u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = 0xD2511F53u * c.x, hi0 = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo1 = 0xCD9E8D57u * c.z, hi1 = __umulhi(0xCD9E8D57u, c.z);
    c = u32x4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}
// Gumbel noise -log(-log U) for U = ((x >> 8) + 0.5) * 2^-24 in (0, 1).
// U = (2m+1) * 2^-25 with m = x >> 8.  Below 1/2 that value is exact in
// float32 and -log U is taken directly; above, 1 - U = (2^25 - 2m - 1) * 2^-25
// is exact and -log U = -log1p(-(1 - U)) avoids the cancellation near 1.
SPEC_DEV float gumbel_from_bits(uint32_t x) {
  const uint32_t m = x >> 8;
  float e;
  if (m < (1u << 23)) {
    e = -logf(float(2u * m + 1u) * 2.98023223876953125e-8f);
  } else {
    e = -log1pf(-float((1u << 25) - 2u * m - 1u) * 2.98023223876953125e-8f);
  }
  return -logf(e);
}

SPEC_DEV int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// The float32 values row[lo, hi) owned by this thread of a 256-thread block,
// in batches of 16 read by four 16-byte loads in flight (lo a multiple of 4,
// row 16-byte aligned): f(v, x0) with v[4 i + e] = row[x0 + 1024 i + e], and
// -inf where that index is >= hi.  Batches come in increasing x0.
template <typename F>
SPEC_DEV void for_row_batches(const float* __restrict__ row, int lo, int hi, F&& f) {
  for (int x0 = lo + 4 * (int)threadIdx.x; x0 < hi; x0 += 4096) {
    float v[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int x = x0 + 1024 * i;
      float4 w;
      if (x + 3 < hi) {
        w = *(const float4*)(row + x);
      } else {
        w.x = x < hi ? row[x] : -INFINITY;
        w.y = x + 1 < hi ? row[x + 1] : -INFINITY;
        w.z = x + 2 < hi ? row[x + 2] : -INFINITY;
        w.w = -INFINITY;
      }
      v[4 * i] = w.x;
      v[4 * i + 1] = w.y;
      v[4 * i + 2] = w.z;
      v[4 * i + 3] = w.w;
    }
    f(v, x0);
  }
}

// Online (max m, sum s of exp(v - m)) update with a batch of 16 values:
// one rescale per batch at most.  Each term is exp2((v - m) log2 e) (the
// difference taken first, so the batch maximum's term is exactly 1); the 16
// terms are summed in float32 and the batch sum is added in float64.
SPEC_DEV void lse_update16(const float (&v)[16], float& m, double& s) {
  constexpr float kL2e = 1.4426950408889634f;
  float bm = v[0];
#pragma unroll
  for (int e = 1; e < 16; ++e) bm = fmaxf(bm, v[e]);
  if (bm == -INFINITY) return;
  if (bm > m) {
    s = m == -INFINITY ? 0.0 : s * exp((double)m - (double)bm);
    m = bm;
  }
  float a = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) a += __builtin_amdgcn_exp2f((v[e] - m) * kL2e);
  s += (double)a;
}

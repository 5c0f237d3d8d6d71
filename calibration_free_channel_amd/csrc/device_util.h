// Device helpers shared by the decode and dense kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace cfr {
namespace {

constexpr float kInvSqrt128f = 0.08838834764831845f;  // 1/sqrt(128) rounded to float
constexpr float kTwo32 = 4294967296.0f;                // 2^32: fixed-point scale of the screen sums

__device__ __forceinline__ float f16f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ float lo16(uint32_t w) { return f16f((uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float hi16(uint32_t w) { return f16f((uint16_t)(w >> 16)); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// silu(z) = z / (1 + e^-z) through the hardware exp2 and reciprocal (about
// one ulp each; the method's tolerances are far wider).
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// float -> 64-bit two's complement fixed point with 32 fraction bits, rounded
// to nearest; exact in float32 arithmetic for |v| < 2^31: v = fl + fr with
// fl = floor(v) and fr in [0, 1), and fr * 2^32 is an exact float.
__device__ __forceinline__ unsigned long long to_fix(float v) {
  const float fl = floorf(v);
  const float fr = v - fl;
  const uint32_t hi = (uint32_t)(int)fl;
  const uint32_t lo = (uint32_t)rintf(fr * kTwo32);
  return ((unsigned long long)hi << 32) | lo;
}

// fixed point -> float (one rounding)
__device__ __forceinline__ float from_fix(unsigned long long x) {
  return fmaf((float)(int)(x >> 32), kTwo32, (float)(uint32_t)x) * (1.0f / kTwo32);
}

__device__ __forceinline__ int clamp_expert(int e, int E, int32_t* status) {
  if (e < 0 || e >= E) {
    atomicOr(status, 1);
    e = e < 0 ? 0 : E - 1;
  }
  return e;
}

// Order-preserving map of a float to an unsigned key: a larger float gives a
// larger key (negative values below positive ones).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Value of lane (lane ^ H) in a wave64, through register-level exchanges:
// DPP quad permutes for H = 1, 2, DPP row shifts for H = 4, 8 and the gfx950
// permlane swaps for H = 16, 32 (no trip through the LDS crossbar).
template <int H>
__device__ __forceinline__ int xor_lane(int v) {
  const int lane = threadIdx.x & 63;
  if constexpr (H == 1) {
    return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (H == 2) {
    return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else if constexpr (H == 4 || H == 8) {
    const int up = __builtin_amdgcn_update_dpp(0, v, 0x100 + H, 0xF, 0xF, false);  // row_shl:H
    const int dn = __builtin_amdgcn_update_dpp(0, v, 0x110 + H, 0xF, 0xF, false);  // row_shr:H
    return (lane & H) ? dn : up;
  } else if constexpr (H == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}

template <int H>
__device__ __forceinline__ float xor_lane_f(float v) {
  return __int_as_float(xor_lane<H>(__float_as_int(v)));
}

// Butterfly sum over the wave; every lane ends with the same total.
__device__ __forceinline__ float wave_sum(float v) {
  v += xor_lane_f<1>(v);
  v += xor_lane_f<2>(v);
  v += xor_lane_f<4>(v);
  v += xor_lane_f<8>(v);
  v += xor_lane_f<16>(v);
  v += xor_lane_f<32>(v);
  return v;
}

// Inclusive prefix sum over a wave64 (DPP row shifts and row broadcasts).
__device__ __forceinline__ int wave_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every outstanding global load of the wave; these kernels exchange data
// through LDS alone, so loads issued early stay in flight across barriers.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  // compiler-only barrier: global loads issued before stay before (nothing
  // waits for them here), so they remain in flight across the barrier
  asm volatile("" ::: "memory");
}

// Inclusive prefix sum over the NT threads of a workgroup.  sh: NT/64 ints
// that nobody else uses between the two barriers inside.
template <int NT>
__device__ __forceinline__ int block_scan(int v, int* sh) {
  static_assert(NT % 256 == 0 && NT <= 1024, "whole groups of four waves");
  constexpr int NQ = NT / 256;  // int4 groups of wave totals
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_scan(v);
  if (lane == 63) sh[w] = v;
  lds_barrier();
  int add = 0;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int4 p = reinterpret_cast<const int4*>(sh)[q];
    add += (4 * q < w ? p.x : 0) + (4 * q + 1 < w ? p.y : 0) + (4 * q + 2 < w ? p.z : 0) +
           (4 * q + 3 < w ? p.w : 0);
  }
  lds_barrier();
  return v + add;
}

// Output-unit score of one candidate from its fixed-point screen sums (the
// up sum carries ||d_j||) and routing weight w: sets g_hat, v_hat' = ||d_j||
// v_hat, p' = silu(g_hat) v_hat' = ||d_j|| p and s = w |p'| = w ||d_j|| |p|,
// and returns the order-preserving key of s.
__device__ __forceinline__ uint32_t score_key(unsigned long long g, unsigned long long v, float w,
                                              float& gh, float& vh, float& p, float& sc) {
  gh = from_fix(g) * kInvSqrt128f;
  vh = from_fix(v) * kInvSqrt128f;
  p = silu(gh) * vh;
  sc = w * fabsf(p);
  return order_key(sc);
}

// Eight consecutive weights h .. h + 7 (h a multiple of 8) of one resident
// row, as one lane holds them.  BF16 rows: 16 bytes.  4-bit rows (a row
// record of H/2 bytes of codes, value h in byte h/2, even h in the low
// nibble, then H/128 fp16 group scales, then H/128 byte zero points):
// w = scale (q - zero), the eight in one group of 128.
template <bool Q4>
struct Chunk8;

// Row chunks are loaded non-temporally: a call streams each kept row once
// per token that keeps it, while the screen sums, the token and the kept
// list are read again by every workgroup, and the rows should not push those
// out of L2.  Measured: the select 11.3 -> 10.7 us at the Qwen3-30B-A3B
// layer, batch 1, and 67.7 -> 62.4 us per call at the Qwen3-235B-A22B layer,
// batch 8.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <>
struct Chunk8<false> {
  uint4 w;
  __device__ __forceinline__ void load(const uint8_t* row, int H, int h) {
    (void)H;
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row + 2 * (size_t)h));
    w = make_uint4(v.x, v.y, v.z, v.w);
  }
  __device__ __forceinline__ void clear() { w = make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ void vals(float* v) const {
    const uint32_t q[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) v[2 * p] = bf_lo(q[p]), v[2 * p + 1] = bf_hi(q[p]);
  }
};

template <>
struct Chunk8<true> {
  uint32_t q;
  uint16_t s;
  uint8_t z;
  __device__ __forceinline__ void load(const uint8_t* row, int H, int h) {
    q = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(row + (h >> 1)));  // streamed, as above
    s = *reinterpret_cast<const uint16_t*>(row + (H >> 1) + 2 * (h >> 7));
    z = row[(H >> 1) + (H >> 6) + (h >> 7)];
  }
  __device__ __forceinline__ void clear() { q = 0u, s = 0, z = 0; }
  __device__ __forceinline__ void vals(float* v) const {
    const float sc = f16f(s), zf = (float)z;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ((float)((q >> (4 * i)) & 15u) - zf) * sc;
  }
};

}  // namespace
}  // namespace cfr

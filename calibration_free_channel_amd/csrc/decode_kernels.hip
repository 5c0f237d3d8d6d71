// Decode kernels of the channel-selection reader for gfx950 (CDNA4, wave64).
//
// Per token and layer ([zh §方法步骤详情] decode steps (1)-(4); [zh §核心方法];
// [ko §어떻게 쓰나]; zh/ko = the Chinese/Korean summary pages of "Channel
// Selection for Mixture-of-Experts Decoding Needs No Calibration Data"), three
// kernels; a kernel boundary is the only grid-wide synchronisation:
//
//   1 k_screen   one workgroup per (token, routed slot, 128-block, half):
//                rotate the block of x (float32 butterfly of H_128 sigma x),
//                pick its n_screen coordinates of largest |value| (ties to the
//                lower index), read the whole half-units of those coordinates
//                (coalesced: every sketch byte is fetched by exactly one
//                workgroup), decode the base-3 codes through an LDS table and
//                add alpha_b * sum_i c_i x_i for every channel of the half into
//                a 64-bit fixed-point accumulator.  Integer addition is
//                associative, so the sum over blocks is bit-reproducible
//                whatever the order the workgroups finish in.
//   2 k_select   per token, G gather workgroups and Z recovery workgroups.
//                Each finalises g_hat, v_hat, p = silu(g_hat) v_hat and the
//                output-unit score s = w ||d|| |p| of every candidate,
//                finds the exact top-k (radix select on order-preserving
//                keys, ties to the lower candidate index) and ranks the kept
//                candidates in index order.  A gather workgroup then loads the
//                native gate, up and down rows of its share of the kept
//                channels at once (one memory latency), computes
//                a_j = silu(g_j.x)(v_j.x) and writes the partial output
//                sum_j w a_j d_j over its share.  A recovery workgroup reads
//                b_j of the skipped candidates in its candidate range and
//                writes the partial recovery vector z = sum w p_j b_j.
//   3 k_reduce   per hidden slice: y = sum of the partial outputs + U z, and
//                clears the screen accumulators for the next call.
//
// In-kernel grid barriers and last-arriver counters were measured slower on
// MI355X than a kernel boundary (agent-scope atomics on one address
// serialise), so no kernel waits for another workgroup.
#include <hip/hip_runtime.h>

#include "kernels.h"

// Optional device-side phase trace: a build that defines CFR_TRACE_PHASE(k, i)
// records a timestamp at each numbered phase of each kernel.  Empty otherwise.
#ifndef CFR_TRACE_PHASE
#define CFR_TRACE_PHASE(kernel, phase) \
  do {                                  \
  } while (0)
#endif

namespace cfr {

namespace {

constexpr float kInvSqrt128f = 0.08838834764831845f;  // 1/sqrt(128) rounded to float
constexpr float kTwo32 = 4294967296.0f;                // 2^32: fixed-point scale of the screen sums
constexpr int kCB = 8;  // screened coordinates whose code words are in flight together

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

// Dispatch places workgroup i on XCD i % 8; item (i % 8) * per_xcd + i / 8
// gives each XCD a contiguous range of items (performance only).
__device__ __forceinline__ int xcd_item(int id, int per_xcd) {
  return (id & 7) * per_xcd + (id >> 3);
}

}  // namespace

// ===========================================================================
// 1: rotate + select + screen
// ===========================================================================
struct ScreenArgs {
  const float* x;
  const int32_t* ids;
  const float* gw;
  const float* sigma;
  const uint8_t* codes;
  const uint16_t* scales;
  const float* norms;
  unsigned long long* acc;
  float* wn;
  float* xrot;
  uint8_t* sel;
  int32_t* status;
  int H, E, I, top, ncp, nblk, ns, lp, unit, nd, ng, items, per_xcd, dbg;
};

// Wave 0 rotates one 128-block held as two values per lane (lane l holds
// coordinates l and l + 64) and picks the n_screen coordinates of largest
// magnitude, ties to the lower index.  The float32 butterfly runs the stages
// h = 1 .. 32 across lanes and h = 64 inside the lane, in that order, with the
// lower element of each pair taking a + b and the upper a - b.  The n_screen-th
// largest magnitude T is found bit by bit from wave ballots (all in
// registers); the kept coordinates are then compacted in ascending order into
// rec (byte offset of the coordinate's unit, value bits) and, when asked, sel.
__device__ __forceinline__ void rotate_select(float v0, float v1, int NS, int unit, int2* rec,
                                              uint8_t* sel_out, float* xrot_out) {
  const int lane = threadIdx.x & 63;
  auto stage = [&](float o0, float o1, int h) {
    if (lane & h) {
      v0 = o0 - v0;
      v1 = o1 - v1;
    } else {
      v0 = v0 + o0;
      v1 = v1 + o1;
    }
  };
  stage(xor_lane_f<1>(v0), xor_lane_f<1>(v1), 1);
  stage(xor_lane_f<2>(v0), xor_lane_f<2>(v1), 2);
  stage(xor_lane_f<4>(v0), xor_lane_f<4>(v1), 4);
  stage(xor_lane_f<8>(v0), xor_lane_f<8>(v1), 8);
  stage(xor_lane_f<16>(v0), xor_lane_f<16>(v1), 16);
  stage(xor_lane_f<32>(v0), xor_lane_f<32>(v1), 32);
  {
    const float u = v0;
    v0 = u + v1;
    v1 = u - v1;
  }
  if (xrot_out) {
    xrot_out[lane] = v0;
    xrot_out[lane + 64] = v1;
  }
  const uint32_t k0 = __float_as_uint(v0) & 0x7FFFFFFFu;
  const uint32_t k1 = __float_as_uint(v1) & 0x7FFFFFFFu;
  uint32_t T = 0;
  for (int bit = 30; bit >= 0; --bit) {
    const uint32_t cand = T | (1u << bit);
    const int cnt = __popcll(__ballot(k0 >= cand)) + __popcll(__ballot(k1 >= cand));
    if (cnt >= NS) T = cand;
  }
  const unsigned long long lt = (1ull << lane) - 1ull;
  const unsigned long long gt0 = __ballot(k0 > T), gt1 = __ballot(k1 > T);
  const unsigned long long eq0 = __ballot(k0 == T), eq1 = __ballot(k1 == T);
  const int need = NS - __popcll(gt0) - __popcll(gt1);
  const bool s0 = k0 > T || (k0 == T && __popcll(eq0 & lt) < need);
  const bool s1 = k1 > T || (k1 == T && __popcll(eq0) + __popcll(eq1 & lt) < need);
  const unsigned long long m0 = __ballot(s0), m1 = __ballot(s1);
  const int p0 = __popcll(m0 & lt), p1 = __popcll(m0) + __popcll(m1 & lt);
  if (s0) {
    rec[p0] = make_int2(lane * unit, __float_as_int(v0));
    if (sel_out) sel_out[p0] = (uint8_t)lane;
  }
  if (s1) {
    rec[p1] = make_int2((lane + 64) * unit, __float_as_int(v1));
    if (sel_out) sel_out[p1] = (uint8_t)(lane + 64);
  }
}

template <int NT>
__global__ __launch_bounds__(NT) void k_screen(ScreenArgs a) {
  __shared__ uint4 lut[256];
  __shared__ int2 rec[128];
  extern __shared__ __align__(16) float red[];  // [ng][nd * 20]
  CFR_TRACE_PHASE(0, 0);
  const int item = xcd_item(blockIdx.x, a.per_xcd);
  if (item >= a.items) return;
  const int m = item & 1;          // 0 gate, 1 up
  const int rb = item >> 1;
  const int b = rb % a.nblk;       // block
  const int ts = rb / a.nblk;      // token * top + slot
  const int s = ts % a.top, t = ts / a.top;
  const int tid = threadIdx.x, lane = tid & 63;
  const int H = a.H, I = a.I, NS = a.ns;
  // token block and signs (wave 0) first: the rotation waits on them; then
  // the routed expert and everything that depends on it
  float x0 = 0.f, x1 = 0.f, g0 = 0.f, g1 = 0.f;
  if (tid < 64) {
    const float* xb = a.x + (size_t)t * H + b * 128;
    x0 = xb[lane];
    x1 = xb[lane + 64];
    g0 = a.sigma[b * 128 + lane];
    g1 = a.sigma[b * 128 + 64 + lane];
  }
  const int e = clamp_expert(a.ids[ts], a.E, a.status);
  CFR_TRACE_PHASE(0, 5);
  // scales of the channels this thread finalises (used at the end)
  constexpr int MAXJ = kMaxInter / NT;
  uint16_t al[MAXJ];
  const uint16_t* sp = a.scales + (((size_t)e * a.nblk + b) * 2 + m) * I;
#pragma unroll
  for (int q = 0; q < MAXJ; ++q) {
    const int j = tid + q * NT;
    al[q] = sp[j < I ? j : I - 1];  // unconditional (clamped): no branch waits on it
  }
  // routing weight times down-column norm of every channel of this slot, for
  // the score: loaded now by one workgroup per slot, stored at the end
  const bool wn_writer = b == 0 && m == 1;
  float nw[MAXJ];
  float wslot = 0.f;
  if (wn_writer) {
    wslot = a.gw[ts];
#pragma unroll
    for (int q = 0; q < MAXJ; ++q) {
      const int j = tid + q * NT;
      nw[q] = a.norms[(size_t)e * I + (j < I ? j : I - 1)];
    }
  }
  // code table: byte q -> its five codes c_t = digit_t - 1 as fp16 (entries
  // 243..255 never occur in a packed unit and decode to zero)
  if (tid < 256) {
    uint32_t h[5] = {0u, 0u, 0u, 0u, 0u};
    if (tid < 243) {
      int q = tid;
#pragma unroll
      for (int d = 0; d < 5; ++d) {
        const int dig = q % 3;
        q /= 3;
        h[d] = dig == 0 ? 0xBC00u : (dig == 2 ? 0x3C00u : 0u);
      }
    }
    lut[tid] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4], 0u);
  }
  // decode step (1): rotation and the partial-screen coordinates
  const bool writer = a.dbg && s == 0 && m == 0;
  if (tid < 64)
    rotate_select(x0 * g0, x1 * g1, NS, a.unit, rec,
                  writer ? a.sel + ((size_t)t * a.nblk + b) * NS : nullptr,
                  writer ? a.xrot + (size_t)t * H + b * 128 : nullptr);
  CFR_TRACE_PHASE(0, 6);
  lds_barrier();
  CFR_TRACE_PHASE(0, 1);

  // screen: thread (g, d) takes code word d (channels 20d .. 20d+19 of the
  // half) at every ng-th screened coordinate starting at g
  const int ND = a.nd, NG = a.ng;
  const int g = tid / ND, d = tid - g * ND;
  float acc[20];
#pragma unroll
  for (int q = 0; q < 20; ++q) acc[q] = 0.f;
  if (g < NG) {
    // uniform base of this (expert, block) and 32-bit per-coordinate offsets
    const uint8_t* ub = a.codes + ((size_t)e * a.nblk + b) * 128 * a.unit;
    const uint32_t col = (uint32_t)(m * a.lp + 4 * d);
    for (int c0 = g; c0 < NS; c0 += NG * kCB) {
      uint32_t wv[kCB];
      float xv[kCB];
#pragma unroll
      for (int u = 0; u < kCB; ++u) {
        const int c = c0 + u * NG;
        const int2 rc = rec[c < NS ? c : NS - 1];  // clamped; past the list x = 0
        wv[u] = *reinterpret_cast<const uint32_t*>(ub + ((uint32_t)rc.x + col));
        xv[u] = c < NS ? __int_as_float(rc.y) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kCB; ++u) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const uint4 cw = lut[(wv[u] >> (8 * kb)) & 0xFFu];
          acc[5 * kb + 0] = fmaf(lo16(cw.x), xv[u], acc[5 * kb + 0]);
          acc[5 * kb + 1] = fmaf(hi16(cw.x), xv[u], acc[5 * kb + 1]);
          acc[5 * kb + 2] = fmaf(lo16(cw.y), xv[u], acc[5 * kb + 2]);
          acc[5 * kb + 3] = fmaf(hi16(cw.y), xv[u], acc[5 * kb + 3]);
          acc[5 * kb + 4] = fmaf(lo16(cw.z), xv[u], acc[5 * kb + 4]);
        }
      }
    }
    CFR_TRACE_PHASE(0, 2);
    float* my = red + (size_t)g * ND * 20 + d * 20;
#pragma unroll
    for (int q = 0; q < 20; q += 4) *reinterpret_cast<float4*>(my + q) = make_float4(acc[q], acc[q + 1], acc[q + 2], acc[q + 3]);
  }
  lds_barrier();
  CFR_TRACE_PHASE(0, 3);
  // channel j = 20 d + i sits at red[g][j]: sum the coordinate groups, scale
  // by alpha_b and add to the fixed-point accumulator
  unsigned long long* ap = a.acc + ((size_t)t * 2 + m) * a.ncp + (size_t)s * I;
#pragma unroll
  for (int q = 0; q < MAXJ; ++q) {
    const int j = tid + q * NT;
    if (j < I) {
      float S = 0.f;
      const float* rj = red + j;
      int gg = 0;
      for (; gg + 4 <= NG; gg += 4) {  // four LDS reads in flight
        const float r0 = rj[(size_t)gg * ND * 20], r1 = rj[(size_t)(gg + 1) * ND * 20];
        const float r2 = rj[(size_t)(gg + 2) * ND * 20], r3 = rj[(size_t)(gg + 3) * ND * 20];
        S += (r0 + r1) + (r2 + r3);
      }
      for (; gg < NG; ++gg) S += rj[(size_t)gg * ND * 20];
      atomicAdd(ap + j, to_fix(f16f(al[q]) * S));
    }
  }
  if (wn_writer) {
    float* wo = a.wn + (size_t)t * a.ncp + (size_t)s * I;
#pragma unroll
    for (int q = 0; q < MAXJ; ++q) {
      const int j = tid + q * NT;
      if (j < I) wo[j] = wslot * nw[q];
    }
  }
  CFR_TRACE_PHASE(0, 4);
}

// ===========================================================================
// 2: finalise scores, exact top-k, gather kept channels / recovery partials
// ===========================================================================
struct SelectArgs {
  const float* x;
  const int32_t* ids;
  const float* gw;
  const uint16_t* w3;
  const uint16_t* bmat;
  const unsigned long long* acc;
  const float* wn;
  float* ypart;
  float* zpart;
  float* ghat;   // debug outputs (written by workgroup 0 of each token when dbg)
  float* vhat;
  float* score;
  int32_t* kept;
  int32_t* status;
  int H, E, I, top, nc, ncp, k, rank, G, Z, cpw, chan, dense, dbg;
};

// misc slots
constexpr int kMiscDigit = 16, kMiscNeed = 17, kMiscCount = 18, kMiscSlot = 19;
constexpr int kDirectMax = 32;  // boundary sets up to this size are ranked directly

template <int NT, int PER, int NCH>
__global__ __launch_bounds__(NT) void k_select(SelectArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NW = NT / 64;
  CFR_TRACE_PHASE(1, 0);
  const int wgs = a.G + a.Z;
  const int t = blockIdx.x / wgs, w = blockIdx.x - t * wgs;
  const bool recover = w >= a.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, I = a.I, nc = a.nc, k = a.k;
  const GatherLds L(H, a.ncp, NT, a.chan);
  float* xs = reinterpret_cast<float*>(smem + L.xs);
  float* pvl = reinterpret_cast<float*>(smem + L.pv);
  uint8_t* flags = smem + L.flags;
  float* yred = reinterpret_cast<float*>(smem + L.yred);
  int* hist = reinterpret_cast<int*>(smem + L.hist);
  int* list = reinterpret_cast<int*>(smem + L.list);
  int* misc = reinterpret_cast<int*>(smem + L.misc);
  uint32_t* bkey = reinterpret_cast<uint32_t*>(smem + L.bkey);
  int* bidx = reinterpret_cast<int*>(smem + L.bidx);
  int* sl_e = reinterpret_cast<int*>(smem + L.slot_e);
  float* sl_w = reinterpret_cast<float*>(smem + L.slot_w);
  float* zred = reinterpret_cast<float*>(smem + L.zred);

  const bool all = a.dense || k == nc;
  const bool partial = !all && k > 0;
  const int kk = all ? nc : k;  // kept candidates
  const int c0 = tid * PER;     // this thread's candidates: [c0, c0 + PER)

  // ---- loads, all issued up front in straight-line code at clamped
  // addresses (a guarded load compiles to a branch that waits on it):
  // screen sums, w ||d||, routing and the token ----
  static_assert(kMaxHidden <= 2 * NT * 4, "the token is two float4 per thread at most");
  ulonglong2 gq[PER / 2], vq[PER / 2];
  float4 wq[PER / 4];
  if (!a.dense) {
    const ulonglong2* ag = reinterpret_cast<const ulonglong2*>(a.acc + (size_t)t * 2 * a.ncp + c0);
    const ulonglong2* av = reinterpret_cast<const ulonglong2*>(a.acc + ((size_t)t * 2 + 1) * a.ncp + c0);
    const float4* wp = reinterpret_cast<const float4*>(a.wn + (size_t)t * a.ncp + c0);
#pragma unroll
    for (int u = 0; u < PER / 2; ++u) {
      gq[u] = ag[u];
      vq[u] = av[u];
    }
#pragma unroll
    for (int u = 0; u < PER / 4; ++u) wq[u] = wp[u];
  }
  const int rslot = tid < a.top ? tid : a.top - 1;
  const int id_raw = a.ids[t * a.top + rslot];
  const float gw_raw = a.gw[t * a.top + rslot];
  // the token, for the gather (written to LDS after the selection)
  const float* xt = a.x + (size_t)t * H;
  const int hx0 = tid * 4, hx1 = (tid + NT) * 4;
  const float4 xr0 = *reinterpret_cast<const float4*>(xt + (hx0 < H ? hx0 : H - 4));
  const float4 xr1 = *reinterpret_cast<const float4*>(xt + (hx1 < H ? hx1 : H - 4));
  if (partial)
    for (int q = tid; q < 2048; q += NT) hist[q] = 0;
  uint32_t key[PER];
  float pr[PER];
  if (!a.dense) {
    const bool dbg = a.dbg && w == 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const float gh = from_fix((i & 1) ? gq[i / 2].y : gq[i / 2].x) * kInvSqrt128f;
      const float vh = from_fix((i & 1) ? vq[i / 2].y : vq[i / 2].x) * kInvSqrt128f;
      const float4 w4 = wq[i / 4];
      const float wn = (i & 3) == 0 ? w4.x : (i & 3) == 1 ? w4.y : (i & 3) == 2 ? w4.z : w4.w;
      const float p = silu(gh) * vh;
      const float sc = wn * fabsf(p);
      const int c = c0 + i;
      key[i] = c < nc ? order_key(sc) : 0u;  // padding ranks below every real candidate
      pr[i] = p;
      if (dbg && c < nc) {
        a.ghat[(size_t)t * nc + c] = gh;
        a.vhat[(size_t)t * nc + c] = vh;
        a.score[(size_t)t * nc + c] = sc;
      }
    }
  }
  if (tid < a.top) {
    sl_e[tid] = clamp_expert(id_raw, a.E, a.status);
    sl_w[tid] = gw_raw;
  }
  if (tid == 0) misc[kMiscSlot] = 0;
  lds_barrier();
  CFR_TRACE_PHASE(1, 1);

  // ---- exact top-k: radix select over 11, 11 and 10 key bits ----
  // After a pass, candidates whose masked key exceeds `prefix` are kept; the
  // `need` remaining places go to the boundary set (masked key == prefix):
  //   mode 0  the whole boundary set (its size equals need)
  //   mode 1  the members ranked directly (flag 2 = kept, 1 = not)
  //   mode 2  all boundary keys are equal: the lowest candidate indices
  uint32_t prefix = 0, mask = 0;
  int need = kk, mode = 0;
  if (partial) {
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const int nbins = pass == 2 ? 1024 : 2048;
      const uint32_t dm = (uint32_t)nbins - 1u;
      if (pass > 0) {
        for (int q = tid; q < nbins; q += NT) hist[q] = 0;
        lds_barrier();
      }
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (c0 + i < nc && (key[i] & mask) == prefix) atomicAdd(&hist[(key[i] >> shift) & dm], 1);
      lds_barrier();
      // thread tid owns bins [base, base + bpt), highest bins first
      const int bpt = nbins / NT;
      const int base = nbins - (tid + 1) * bpt;
      int own = 0;
      for (int q = 0; q < bpt; ++q) own += hist[base + q];
      const int incl = block_scan<NT>(own, misc);
      if (incl >= need && incl - own < need) {
        int cum = incl - own;
        for (int q = bpt - 1; q >= 0; --q) {
          const int hb = hist[base + q];
          if (cum < need && cum + hb >= need) {
            misc[kMiscDigit] = base + q;
            misc[kMiscNeed] = need - cum;
            misc[kMiscCount] = hb;
          }
          cum += hb;
        }
      }
      lds_barrier();
      prefix |= (uint32_t)misc[kMiscDigit] << shift;
      mask |= dm << shift;
      need = misc[kMiscNeed];
      const int cnt = misc[kMiscCount];
      if (cnt == need) {
        mode = 0;
        break;
      }
      if (cnt <= kDirectMax) {
        // rank the boundary set directly (key descending, index ascending)
#pragma unroll
        for (int i = 0; i < PER; ++i)
          if (c0 + i < nc && (key[i] & mask) == prefix) {
            const int slot = atomicAdd(&misc[kMiscSlot], 1);
            bkey[slot] = key[i];
            bidx[slot] = c0 + i;
            flags[c0 + i] = 1;
          }
        lds_barrier();
        if (tid < cnt) {
          const uint32_t ki = bkey[tid];
          const int ii = bidx[tid];
          int rk = 0;
#pragma unroll 8
          for (int q = 0; q < kDirectMax; ++q)
            if (q < cnt) {
              const uint32_t kq = bkey[q];
              rk += kq > ki || (kq == ki && bidx[q] < ii);
            }
          if (rk < need) flags[ii] = 2;
        }
        lds_barrier();
        mode = 1;
        break;
      }
      mode = 2;
    }
  }

  CFR_TRACE_PHASE(1, 2);
  // ---- kept flags and ranks in ascending candidate order ----
  bool on[PER];
  if (all) {
#pragma unroll
    for (int i = 0; i < PER; ++i) on[i] = c0 + i < nc;
  } else if (!partial) {
#pragma unroll
    for (int i = 0; i < PER; ++i) on[i] = false;
  } else {
    int eq_before = 0;
    if (mode == 2) {
      int neq = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) neq += c0 + i < nc && (key[i] & mask) == prefix;
      eq_before = block_scan<NT>(neq, misc) - neq;
    }
    int eq_seen = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint32_t km = key[i] & mask;
      bool o = c0 + i < nc && km > prefix;
      if (c0 + i < nc && km == prefix) {
        if (mode == 0) o = true;
        else if (mode == 1) o = flags[c0 + i] == 2;
        else o = eq_before + (eq_seen++) < need;
      }
      on[i] = o;
    }
  }
  int mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) mine += on[i];
  int rnk = block_scan<NT>(mine, misc) - mine;
  const int r0 = recover ? 0 : min(w * a.chan, kk);
  const int r1 = recover ? 0 : min(r0 + a.chan, kk);
  {
    const bool dbg = a.dbg && w == 0;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (on[i]) {
        if (rnk >= r0 && rnk < r1) list[rnk - r0] = c0 + i;
        if (dbg) a.kept[(size_t)t * nc + rnk] = c0 + i;
        ++rnk;
      }
  }
  if (recover) {
    // p and the kept flags of every candidate, for the recovery ranges
#pragma unroll
    for (int i = 0; i < PER; i += 4) {
      *reinterpret_cast<float4*>(pvl + c0 + i) = make_float4(pr[i], pr[i + 1], pr[i + 2], pr[i + 3]);
      *reinterpret_cast<uint32_t*>(flags + c0 + i) =
          (uint32_t)on[i] | ((uint32_t)on[i + 1] << 8) | ((uint32_t)on[i + 2] << 16) | ((uint32_t)on[i + 3] << 24);
    }
  }
  lds_barrier();
  CFR_TRACE_PHASE(1, 3);

  if (!recover) {
    if (hx0 < H) *reinterpret_cast<float4*>(xs + hx0) = xr0;
    if (hx1 < H) *reinterpret_cast<float4*>(xs + hx1) = xr1;
    lds_barrier();
    // ---- decode step (3): exact kept channels from native BF16 rows ----
    // wave v takes list entries [v cpw, (v+1) cpw), two channels at a time
    // when registers allow, all rows of both in flight together
    float yv[NCH][8];
#pragma unroll
    for (int q = 0; q < NCH; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i) yv[q][i] = 0.f;
    const int nmine = r1 - r0;
    constexpr bool kPair = NCH <= 4;
    const int qend = min((wave + 1) * a.cpw, nmine);
    for (int q0 = wave * a.cpw; q0 < qend; q0 += kPair ? 2 : 1) {
      const bool two = kPair && q0 + 1 < qend;
      const int cA = list[q0], cB = two ? list[q0 + 1] : cA;
      const int sA = cA / I, sB = cB / I;
      const uint16_t* rowA = a.w3 + ((size_t)sl_e[sA] * I + (cA - sA * I)) * 3 * H;
      const uint16_t* rowB = a.w3 + ((size_t)sl_e[sB] * I + (cB - sB * I)) * 3 * H;
      uint4 gq[2][NCH], uq[2][NCH], dq[2][NCH];
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const int h = min(ch * 512 + lane * 8, H - 8);  // clamped; the tail is masked below
        gq[0][ch] = *reinterpret_cast<const uint4*>(rowA + h);
        uq[0][ch] = *reinterpret_cast<const uint4*>(rowA + H + h);
        dq[0][ch] = *reinterpret_cast<const uint4*>(rowA + 2 * H + h);
      }
      if (two) {  // wave-uniform
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
          const int h = min(ch * 512 + lane * 8, H - 8);
          gq[1][ch] = *reinterpret_cast<const uint4*>(rowB + h);
          uq[1][ch] = *reinterpret_cast<const uint4*>(rowB + H + h);
          dq[1][ch] = *reinterpret_cast<const uint4*>(rowB + 2 * H + h);
        }
      } else {
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) gq[1][ch] = uq[1][ch] = dq[1][ch] = make_uint4(0u, 0u, 0u, 0u);
      }
      float gs[2] = {0.f, 0.f}, vs[2] = {0.f, 0.f};
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const int h = ch * 512 + lane * 8;
        if (h < H) {
          const float4 xa = *reinterpret_cast<const float4*>(xs + h);
          const float4 xb = *reinterpret_cast<const float4*>(xs + h + 4);
          const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const uint32_t gw4[4] = {gq[r][ch].x, gq[r][ch].y, gq[r][ch].z, gq[r][ch].w};
            const uint32_t uw4[4] = {uq[r][ch].x, uq[r][ch].y, uq[r][ch].z, uq[r][ch].w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              gs[r] = fmaf(bf_lo(gw4[p]), xv[2 * p], gs[r]);
              gs[r] = fmaf(bf_hi(gw4[p]), xv[2 * p + 1], gs[r]);
              vs[r] = fmaf(bf_lo(uw4[p]), xv[2 * p], vs[r]);
              vs[r] = fmaf(bf_hi(uw4[p]), xv[2 * p + 1], vs[r]);
            }
          }
        }
      }
      const float cfA = sl_w[sA] * silu(wave_sum(gs[0])) * wave_sum(vs[0]);
      const float cfB = two ? sl_w[sB] * silu(wave_sum(gs[1])) * wave_sum(vs[1]) : 0.f;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const uint32_t d0[4] = {dq[0][ch].x, dq[0][ch].y, dq[0][ch].z, dq[0][ch].w};
        const uint32_t d1[4] = {dq[1][ch].x, dq[1][ch].y, dq[1][ch].z, dq[1][ch].w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          yv[ch][2 * p] = fmaf(cfA, bf_lo(d0[p]), yv[ch][2 * p]);
          yv[ch][2 * p + 1] = fmaf(cfA, bf_hi(d0[p]), yv[ch][2 * p + 1]);
          yv[ch][2 * p] = fmaf(cfB, bf_lo(d1[p]), yv[ch][2 * p]);
          yv[ch][2 * p + 1] = fmaf(cfB, bf_hi(d1[p]), yv[ch][2 * p + 1]);
        }
      }
    }
    CFR_TRACE_PHASE(1, 4);
    // ---- partial output: only waves that took channels contribute ----
    // waves [0, NW/2) store their rows into NW/2 slots, the others add theirs
    constexpr int SL = NW / 2;
    const int used = min(NW, (nmine + a.cpw - 1) / a.cpw);  // waves holding channels
    const int slot = wave % SL;
    if (wave < SL) {
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const int h = ch * 512 + lane * 8;
        if (h < H) {
          float* o = yred + (size_t)slot * H + h;
          *reinterpret_cast<float4*>(o) = make_float4(yv[ch][0], yv[ch][1], yv[ch][2], yv[ch][3]);
          *reinterpret_cast<float4*>(o + 4) = make_float4(yv[ch][4], yv[ch][5], yv[ch][6], yv[ch][7]);
        }
      }
    }
    lds_barrier();
    if (wave >= SL && wave < used) {
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const int h = ch * 512 + lane * 8;
        if (h < H) {
          float* o = yred + (size_t)slot * H + h;
          float4 p0 = *reinterpret_cast<float4*>(o);
          float4 p1 = *reinterpret_cast<float4*>(o + 4);
          p0.x += yv[ch][0];
          p0.y += yv[ch][1];
          p0.z += yv[ch][2];
          p0.w += yv[ch][3];
          p1.x += yv[ch][4];
          p1.y += yv[ch][5];
          p1.z += yv[ch][6];
          p1.w += yv[ch][7];
          *reinterpret_cast<float4*>(o) = p0;
          *reinterpret_cast<float4*>(o + 4) = p1;
        }
      }
    }
    lds_barrier();
    const int nsl = min(SL, max(used, 1));  // slots that received rows
    float* yp = a.ypart + ((size_t)t * a.G + w) * H;
    for (int h = tid * 4; h < H; h += NT * 4) {
      float4 v = *reinterpret_cast<const float4*>(yred + h);
      for (int q = 1; q < nsl; ++q) {
        const float4 u = *reinterpret_cast<const float4*>(yred + (size_t)q * H + h);
        v.x += u.x;
        v.y += u.y;
        v.z += u.z;
        v.w += u.w;
      }
      *reinterpret_cast<float4*>(yp + h) = v;
    }
    CFR_TRACE_PHASE(1, 5);
    return;
  }

  // ---- decode step (4), first half: z over this workgroup's candidate range ----
  // R8 threads per candidate, each 8 coefficients (one uint4) of b_j
  const int zr = w - a.G;
  const int R = a.rank, R8 = R / 8;
  const int zper = (nc + a.Z - 1) / a.Z;
  const int cb0 = min(zr * zper, nc), cb1 = min(cb0 + zper, nc);
  const int cpp = NT / R8;  // candidates per pass
  const int cl = tid / R8, r8 = tid - cl * R8;
  float zacc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) zacc[d] = 0.f;
  if (cl < cpp) {
    for (int cb = cb0 + cl; cb < cb1; cb += cpp * 4) {
      uint4 bq[4];
      float cf[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int cnd = cb + u * cpp;
        const int cc = cnd < cb1 ? cnd : cb1 - 1;  // clamped: loads always issued
        const int s = cc / I, j = cc - s * I;
        bq[u] = reinterpret_cast<const uint4*>(a.bmat + ((size_t)sl_e[s] * I + j) * R)[r8];
        cf[u] = (cnd < cb1 && !flags[cc]) ? sl_w[s] * pvl[cc] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t bw[4] = {bq[u].x, bq[u].y, bq[u].z, bq[u].w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          zacc[2 * d] = fmaf(cf[u], lo16(bw[d]), zacc[2 * d]);
          zacc[2 * d + 1] = fmaf(cf[u], hi16(bw[d]), zacc[2 * d + 1]);
        }
      }
    }
  }
#pragma unroll
  for (int d = 0; d < 8; ++d) zred[(size_t)tid * 8 + d] = cl < cpp ? zacc[d] : 0.f;
  lds_barrier();
  // component r = 8 r8 + d sums zred[(cl R8 + r8) 8 + d] over cl < cpp: tpo
  // consecutive threads per component (a power of two, at most 64) each sum a
  // strided share, then a lane butterfly combines them
  int tpo = 1;
  while (tpo * 2 * R <= NT && tpo < 64) tpo *= 2;
  const int r = tid / tpo, jq = tid - r * tpo;
  float z = 0.f;
  if (r < R) {
    const int rr8 = r >> 3, d = r & 7;
    for (int q0 = jq; q0 < cpp; q0 += tpo * 4) {
      float zz[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = q0 + u * tpo;
        zz[u] = zred[(size_t)((q < cpp ? q : 0) * R8 + rr8) * 8 + d];
        zz[u] = q < cpp ? zz[u] : 0.f;
      }
      z += (zz[0] + zz[1]) + (zz[2] + zz[3]);
    }
  }
  if (tpo > 1) z += xor_lane_f<1>(z);
  if (tpo > 2) z += xor_lane_f<2>(z);
  if (tpo > 4) z += xor_lane_f<4>(z);
  if (tpo > 8) z += xor_lane_f<8>(z);
  if (tpo > 16) z += xor_lane_f<16>(z);
  if (tpo > 32) z += xor_lane_f<32>(z);
  if (r < R && jq == 0) a.zpart[((size_t)t * a.Z + zr) * R + r] = z;
  CFR_TRACE_PHASE(1, 6);
}

// ===========================================================================
// 3: y = sum of the partial outputs + U z; clear the screen accumulators
// ===========================================================================
struct ReduceArgs {
  const float* ypart;
  const float* zpart;
  const uint16_t* U;
  float* y;
  unsigned long long* acc;
  int H, G, Z, rank, ncp, nslices, clear;
};

constexpr int kReduceThreads = 256;
constexpr int kReduceParts = kReduceThreads / kReduceSlice;  // 8
constexpr int kReducePer = kMaxGatherWgs / kReduceParts;     // partial rows per thread, at most

__global__ __launch_bounds__(kReduceThreads) void k_reduce(ReduceArgs a) {
  __shared__ float part[kReduceParts][kReduceSlice];
  __shared__ float zs[64];
  CFR_TRACE_PHASE(2, 0);
  const int t = blockIdx.x / a.nslices, sl = blockIdx.x - t * a.nslices;
  const int tid = threadIdx.x;
  const int H = a.H, h0 = sl * kReduceSlice;
  const int hl = tid % kReduceSlice, pt = tid / kReduceSlice;
  // U rows of this slice, the recovery partials and the output partials:
  // all issued before any is summed
  uint4 uq[8];
  const bool rec = a.Z > 0;
  if (rec && tid < kReduceSlice) {
    const uint4* up = reinterpret_cast<const uint4*>(a.U + (size_t)(h0 + tid) * a.rank);
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) uq[r8] = up[r8 * 8 < a.rank ? r8 : 0];
  }
  float zv[kMaxRecoverWgs];
  if (rec && tid < a.rank) {
    const float* zp = a.zpart + (size_t)t * a.Z * a.rank + tid;
#pragma unroll
    for (int q = 0; q < kMaxRecoverWgs; ++q) zv[q] = zp[(size_t)(q < a.Z ? q : 0) * a.rank];
  }
  const float* yp = a.ypart + (size_t)t * a.G * H + h0 + hl;
  float pv[kReducePer];
#pragma unroll
  for (int u = 0; u < kReducePer; ++u) {
    const int wq = pt + u * kReduceParts;
    pv[u] = yp[(size_t)(wq < a.G ? wq : 0) * H];
  }
  float v = 0.f;
#pragma unroll
  for (int u = 0; u < kReducePer; ++u) v += pt + u * kReduceParts < a.G ? pv[u] : 0.f;
  CFR_TRACE_PHASE(2, 1);
  part[pt][hl] = v;
  if (tid < 64) {
    float z = 0.f;
    if (rec && tid < a.rank)
#pragma unroll
      for (int q = 0; q < kMaxRecoverWgs; ++q) z += q < a.Z ? zv[q] : 0.f;
    zs[tid] = z;
  }
  lds_barrier();
  if (tid < kReduceSlice) {
    float o = 0.f;
#pragma unroll
    for (int q = 0; q < kReduceParts; ++q) o += part[q][tid];
    if (rec) {
#pragma unroll
      for (int r8 = 0; r8 < 8; ++r8)
        if (r8 * 8 < a.rank) {
          const uint32_t uw[4] = {uq[r8].x, uq[r8].y, uq[r8].z, uq[r8].w};
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            o = fmaf(lo16(uw[d]), zs[r8 * 8 + 2 * d], o);
            o = fmaf(hi16(uw[d]), zs[r8 * 8 + 2 * d + 1], o);
          }
        }
    }
    a.y[(size_t)t * H + h0 + tid] = o;
  }
  CFR_TRACE_PHASE(2, 2);
  if (a.clear) {
    // the screen accumulators of this token (gate then up, ncp each), split
    // over its slices
    const int n = 2 * a.ncp;
    const int per = (n + a.nslices - 1) / a.nslices;
    const int b0 = sl * per, b1 = min(b0 + per, n);
    ulonglong2* ap = reinterpret_cast<ulonglong2*>(a.acc + (size_t)t * n);
    for (int q = b0 / 2 + tid; q < b1 / 2; q += kReduceThreads) ap[q] = make_ulonglong2(0ull, 0ull);
  }
  CFR_TRACE_PHASE(2, 3);
}

// ===========================================================================
// host side
// ===========================================================================
static int hip_fail(hipError_t e, const char* what) {
  return fail(CFR_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

Plan make_plan(const cfr_config& c, int batch, int k, bool dense) {
  Plan p;
  const int nblk = c.hidden / kBlock, nbytes = (c.inter + 4) / 5, nc = c.top * c.inter;
  // screen
  p.nd = (nbytes + 3) / 4;
  p.ng = kScreenThreads / p.nd;
  if (p.ng < 1) p.ng = 1;
  p.items1 = batch * c.top * nblk * 2;
  p.per_xcd1 = (p.items1 + 7) / 8;
  p.lds1 = (size_t)p.ng * p.nd * 20 * 4;
  // select/gather: about 240 gather workgroups over the batch plus 16
  // recovery workgroups, so the whole grid fits one workgroup per CU
  const SelectGeom g = select_geom(nc);
  p.nt2 = g.nt;
  p.per = g.per;
  p.ncp = g.nt * g.per;
  const int NW = p.nt2 / 64;
  const int kk = dense ? nc : k;
  int gmax = (kMaxGatherWgs - kMaxRecoverWgs) / batch;
  if (gmax < 1) gmax = 1;
  p.chan = (kk + gmax - 1) / gmax;
  if (p.chan < 1) p.chan = 1;
  p.cpw = (p.chan + NW - 1) / NW;
  p.G = (kk + p.chan - 1) / p.chan;
  if (p.G < 1) p.G = 1;
  int z = kMaxRecoverWgs / batch;
  if (z < 1) z = 1;
  p.Z = (!dense && c.rank > 0 && k < nc) ? z : 0;
  if (p.Z > nc) p.Z = nc;
  p.nch = 1;
  while (p.nch * 512 < c.hidden) p.nch *= 2;
  p.lds2 = GatherLds(c.hidden, p.ncp, p.nt2, p.chan).total;
  // reduce
  p.nslices = c.hidden / kReduceSlice;
  return p;
}

size_t max_lds_needed(const cfr_config& c) {
  size_t m = 0;
  const int nc = c.top * c.inter;
  for (int b = 1; b <= c.max_batch; ++b)
    for (int kk : {0, 1, nc / 2, nc}) {
      const Plan p = make_plan(c, b, kk, false);
      if (p.lds1 + 8192 > m) m = p.lds1 + 8192;  // + the screen kernel's static LDS
      if (p.lds2 > m) m = p.lds2;
    }
  const Plan d = make_plan(c, 1, nc, true);
  if (d.lds2 > m) m = d.lds2;
  return m;
}

// Lets a kernel take dynamic LDS up to the workgroup limit minus its static
// LDS.  A failure here would surface as the launch error, so it is cleared.
template <typename K>
static void allow_lds(K kernel) {
  hipFuncAttributes fa{};
  size_t stat = 0;
  if (hipFuncGetAttributes(&fa, (const void*)kernel) == hipSuccess) stat = fa.sharedSizeBytes;
  (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(kMaxLds - stat));
  (void)hipGetLastError();
}

template <int NT, int PER, int NCH>
static hipError_t launch_select_t(const SelectArgs& a, const Plan& p, int batch, hipStream_t st) {
  static bool attr = false;
  if (!attr) {
    allow_lds(k_select<NT, PER, NCH>);
    attr = true;
  }
  k_select<NT, PER, NCH><<<batch * (p.G + p.Z), NT, p.lds2, st>>>(a);
  return hipGetLastError();
}

template <int NT, int PER>
static hipError_t launch_select_n(const SelectArgs& a, const Plan& p, int batch, hipStream_t st) {
  switch (p.nch) {
    case 1: return launch_select_t<NT, PER, 1>(a, p, batch, st);
    case 2: return launch_select_t<NT, PER, 2>(a, p, batch, st);
    case 4: return launch_select_t<NT, PER, 4>(a, p, batch, st);
    default: return launch_select_t<NT, PER, 8>(a, p, batch, st);
  }
}

static hipError_t launch_select(const SelectArgs& a, const Plan& p, int batch, hipStream_t st) {
  switch (p.per) {  // select_geom: 512 threads, 4..32 candidates each
    case 4: return launch_select_n<512, 4>(a, p, batch, st);
    case 8: return launch_select_n<512, 8>(a, p, batch, st);
    case 12: return launch_select_n<512, 12>(a, p, batch, st);
    case 16: return launch_select_n<512, 16>(a, p, batch, st);
    case 24: return launch_select_n<512, 24>(a, p, batch, st);
    default: return launch_select_n<512, 32>(a, p, batch, st);
  }
}

static hipError_t launch_screen(const ScreenArgs& a, const Plan& p, hipStream_t st) {
  static bool attr = false;
  if (!attr) {
    allow_lds(k_screen<kScreenThreads>);
    attr = true;
  }
  k_screen<kScreenThreads><<<8 * p.per_xcd1, kScreenThreads, p.lds1, st>>>(a);
  return hipGetLastError();
}

static hipError_t launch_reduce(const ReduceArgs& a, int batch, hipStream_t st) {
  k_reduce<<<batch * a.nslices, kReduceThreads, 0, st>>>(a);
  return hipGetLastError();
}

int launch_decode(cfr_reader* r, const float* x, const int32_t* ids, const float* gw, int batch,
                  int k, float* y, hipStream_t st, const DebugOut* dbg, hipEvent_t* ev) {
  const cfr_config& c = r->cfg;
  const Plan p = make_plan(c, batch, k, false);
  auto mark = [&](int i) {
    if (ev) (void)hipEventRecord(ev[i], st);
  };
  hipError_t e;
  mark(0);
  ScreenArgs A{x, ids, gw, r->sigma, r->codes, r->scales, r->norms, r->acc, r->wn, r->xrot,
               r->sel, r->status, c.hidden, c.n_experts, c.inter, c.top, r->ncp, r->nblk,
               c.n_screen, r->lp, r->unit, p.nd, p.ng, p.items1, p.per_xcd1, dbg != nullptr};
  if ((e = launch_screen(A, p, st)) != hipSuccess) return hip_fail(e, "screen launch");
  mark(1);
  SelectArgs B{x, ids, gw, r->w3, r->b, r->acc, r->wn, r->ypart, r->zpart, r->ghat, r->vhat,
               r->score, r->kept, r->status, c.hidden, c.n_experts, c.inter, c.top, r->ncand,
               r->ncp, k, c.rank, p.G, p.Z, p.cpw, p.chan, 0, dbg != nullptr};
  if ((e = launch_select(B, p, batch, st)) != hipSuccess) return hip_fail(e, "select launch");
  mark(2);
  ReduceArgs C{r->ypart, r->zpart, r->u, y, r->acc, c.hidden, p.G, p.Z, c.rank, r->ncp,
               p.nslices, 1};
  if ((e = launch_reduce(C, batch, st)) != hipSuccess) return hip_fail(e, "reduce launch");
  mark(3);
  if (dbg) {
    const int H = c.hidden, nblk = r->nblk, nsc = batch * r->ncand;
    auto cp = [&](void* dst, const void* src, size_t bytes) -> hipError_t {
      return dst ? hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st) : hipSuccess;
    };
    if ((e = cp(dbg->xrot, r->xrot, sizeof(float) * batch * H)) != hipSuccess ||
        (e = cp(dbg->sel, r->sel, (size_t)batch * nblk * c.n_screen)) != hipSuccess ||
        (e = cp(dbg->ghat, r->ghat, sizeof(float) * nsc)) != hipSuccess ||
        (e = cp(dbg->vhat, r->vhat, sizeof(float) * nsc)) != hipSuccess ||
        (e = cp(dbg->score, r->score, sizeof(float) * nsc)) != hipSuccess)
      return hip_fail(e, "debug copy");
    if (dbg->kept && k > 0) {
      e = hipMemcpy2DAsync(dbg->kept, sizeof(int32_t) * k, r->kept, sizeof(int32_t) * r->ncand,
                           sizeof(int32_t) * k, batch, hipMemcpyDeviceToDevice, st);
      if (e != hipSuccess) return hip_fail(e, "debug copy kept");
    }
  }
  return CFR_OK;
}

int launch_dense(cfr_reader* r, const float* x, const int32_t* ids, const float* gw, int batch,
                 float* y, hipStream_t st) {
  const cfr_config& c = r->cfg;
  const int nc = r->ncand;
  const Plan p = make_plan(c, batch, nc, true);
  SelectArgs B{x, ids, gw, r->w3, r->b, r->acc, r->wn, r->ypart, r->zpart, nullptr, nullptr,
               nullptr, nullptr, r->status, c.hidden, c.n_experts, c.inter, c.top, nc, r->ncp,
               nc, 0, p.G, 0, p.cpw, p.chan, 1, 0};
  hipError_t e;
  if ((e = launch_select(B, p, batch, st)) != hipSuccess) return hip_fail(e, "dense launch");
  ReduceArgs C{r->ypart, r->zpart, r->u, y, r->acc, c.hidden, p.G, 0, c.rank, r->ncp,
               p.nslices, 0};
  if ((e = launch_reduce(C, batch, st)) != hipSuccess) return hip_fail(e, "dense reduce launch");
  return CFR_OK;
}

}  // namespace cfr

// Decode kernels of the channel-selection reader for gfx950 (CDNA4, wave64).
//
// Per token and layer ([zh §方法步骤详情] decode steps (1)-(4); [zh §核心方法];
// [ko §어떻게 쓰나]; zh/ko = the Chinese/Korean summary pages of "Channel
// Selection for Mixture-of-Experts Decoding Needs No Calibration Data"), three
// kernels; a kernel boundary is the only grid-wide synchronisation:
//
//   1 k_screen   one workgroup per (token, routed slot, group of bg
//                128-blocks, half): rotate each block of x (float32
//                butterfly of H_128 sigma x), pick its n_screen coordinates of
//                largest |value| (ties to the lower index), read the whole
//                half-units of those coordinates (coalesced: every sketch
//                byte is fetched by exactly one workgroup), decode the base-3
//                codes through an LDS table of digits and add
//                sum_b alpha_b sum_i c_i x_i over the group's blocks for every
//                channel of the half into a 64-bit fixed-point accumulator.
//                Integer addition is associative, so the sum over groups is
//                bit-reproducible whatever the order the workgroups finish in.
//                bg = 1 at batch 1 (most workgroups, shortest chains); at
//                larger batches groups of 2-8 blocks cut the atomics.
//   2 k_select   per token, G gather workgroups and Z recovery workgroups.
//                Each finalises g_hat, v_hat, p = silu(g_hat) v_hat and the
//                output-unit score s = w ||d|| |p| of every candidate,
//                finds the exact top-k (one histogram pass over the keys'
//                distance below the largest, the boundary bin ranked
//                directly, or radix passes when it is large; ties to the
//                lower candidate index) and ranks the kept candidates.  A gather workgroup then loads the
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

#include <algorithm>
#include <type_traits>

#include "device_util.h"
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

// Buffer resource over `bytes` bytes at p (gfx9 layout): a raw buffer load at
// an offset past the end returns zeros without a memory access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kNoLoad = 0x80000000u;  // offset past the end of any buffer here

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
  const uint16_t* rho;  // [E][nblk][2][I] fp16 (expected-error ranking only)
  unsigned long long* acc;
  float* var;  // [B][2][ncp] sketch-error variances of g_hat and v_hat' (expected-error ranking)
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
  // Once exactly NS magnitudes are >= a prefix, those NS are the kept set
  // (every later T lies between that prefix and their minimum), so the search
  // stops there.  The whole block (NS = 128) needs no search: T = 0 keeps all.
  uint32_t T = 0;
#pragma unroll
  for (int bit = 30; bit >= 0 && NS < 128; --bit) {
    const uint32_t cand = T | (1u << bit);
    const int cnt = __popcll(__ballot(k0 >= cand)) + __popcll(__ballot(k1 >= cand));
    if (cnt >= NS) T = cand;
    if (cnt == NS) break;
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

// NG: threads per code word (a power of two, at most 16), CPB: screened
// coordinates per thread whose code words are in flight together.  VAR (the
// expected-error ranking, whole sketch): the workgroup also writes, for its
// 1/nblk share of the half's channels, the sketch-error variance
// sum_b rho_b ||x_b||^2 (times ||d_j||^2 for the up half: the variance of
// v_hat'), every term from stored values, so no accumulation across
// workgroups is needed.
template <int NT, int NG, int CPB, bool VAR, int BG, int BC>
__global__ __launch_bounds__(NT) void k_screen(ScreenArgs a) {
  static_assert(NG >= 1 && NG <= 16 && (NG & (NG - 1)) == 0, "word groups within a row of lanes");
  static_assert(BG == 1 || (!VAR && BG <= NT / 64), "block groups: score ranking, one wave per block");
  static_assert(BG % BC == 0 && (BG > 1 || BC == 1), "blocks of a group in whole chunks");
  __shared__ uint2 lut[256];
  __shared__ int2 rec[BG][128];
  __shared__ float qn2[VAR ? kMaxHidden / 128 : 1];  // ||x_b||^2 of every block (VAR)
  CFR_TRACE_PHASE(0, 0);
  const int item = xcd_item(blockIdx.x, a.per_xcd);
  if (item >= a.items) return;
  // a workgroup screens the BG blocks [b, b + nbh) of one half (BG > 1 at
  // batch sizes where the atomics' count, not latency, bounds the kernel:
  // the blocks are summed in registers before one atomic per channel)
  const int nbg = (a.nblk + BG - 1) / BG;
  const int m = item & 1;          // 0 gate, 1 up
  const int rb = item >> 1;
  const int b = (rb % nbg) * BG;   // first block
  const int nbh = min(BG, a.nblk - b);
  const int ts = rb / nbg;         // token * top + slot
  const int s = ts % a.top, t = ts / a.top;
  const int tid = threadIdx.x, lane = tid & 63, wvi = tid >> 6;
  const int H = a.H, I = a.I, NS = a.ns;
  // token block and signs (wave v: block b + v) first: the rotation waits on
  // them; then the routed expert and everything that depends on it
  float x0 = 0.f, x1 = 0.f, g0 = 0.f, g1 = 0.f;
  if (wvi < nbh) {
    const int bb = b + wvi;
    const float* xb = a.x + (size_t)t * H + bb * 128;
    x0 = xb[lane];
    x1 = xb[lane + 64];
    g0 = a.sigma[bb * 128 + lane];
    g1 = a.sigma[bb * 128 + 64 + lane];
  }
  // VAR: the token, four coordinates per thread and chunk, for the block
  // norms (before the loads that wait on the routed expert)
  float4 q0 = make_float4(0.f, 0.f, 0.f, 0.f), q1 = q0;
  if constexpr (VAR) {
    const float* xt = a.x + (size_t)t * H;
    const int h0 = 4 * tid, h1 = 4 * (tid + NT);
    q0 = *reinterpret_cast<const float4*>(xt + (h0 < H ? h0 : H - 4));
    q1 = *reinterpret_cast<const float4*>(xt + (h1 < H ? h1 : H - 4));
  }
  const int e = clamp_expert(a.ids[ts], a.E, a.status);
  CFR_TRACE_PHASE(0, 5);
  // thread (d, g) = tid: code word d (channels 20d .. 20d+19 of the half),
  // lane g of the NG consecutive lanes that share it; after the decode, lane g
  // finalises channels 20d + g + NG r (r < RPL): their scales, loaded now
  constexpr int RPL = (20 + NG - 1) / NG;
  const int d = tid / NG, g = tid & (NG - 1);
  // (a block group loads each chunk's scales with its words)
  auto load_scales = [&](int bi, uint16_t* al) {
    const uint16_t* sp = a.scales + (((size_t)e * a.nblk + b + bi) * 2 + m) * I;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const int j = 20 * d + g + NG * r;
      al[r] = sp[j < I ? j : I - 1];  // unconditional (clamped): no branch waits on it
    }
  };
  uint16_t al[RPL];
  if constexpr (BG == 1) load_scales(0, al);
  // VAR: this workgroup owns channels [b vper, (b + 1) vper) of the half;
  // thread tid < vper loads channel b vper + tid's rho in every block and
  // ||d_j|| now, as buffer loads that the other threads point past the end
  // (issued by every thread: no wait depends on which path a thread took);
  // channels past NT of the share, if any, are done at the end
  constexpr int VB = VAR ? kMaxHidden / 128 : 1;
  const int vper = (I + a.nblk - 1) / a.nblk;
  const bool vown = VAR && tid < vper && b * vper + tid < I;
  uint16_t vrho[VB];
  float vdn = 1.f;
  if constexpr (VAR) {
    const __amdgpu_buffer_rsrc_t rrs = buffer_rsrc(a.rho + (size_t)e * a.nblk * 2 * I, (uint32_t)(a.nblk * 2 * I * 2));
    const __amdgpu_buffer_rsrc_t drs = buffer_rsrc(a.norms + (size_t)e * I, (uint32_t)I * 4u);
    const uint32_t jb = (uint32_t)(m * I + b * vper + tid) * 2u;
#pragma unroll
    for (int q = 0; q < VB; ++q)
      vrho[q] = __builtin_amdgcn_raw_buffer_load_b16(rrs, vown && q < a.nblk ? jb + (uint32_t)q * 4u * I : kNoLoad,
                                                     0, 0);
    vdn = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                        drs, vown ? (uint32_t)(b * vper + tid) * 4u : kNoLoad, 0, 0));
  }
  // the up half carries ||d_j|| into its sums (v_hat' = ||d_j|| v_hat), so the
  // score needs no per-candidate norm read later: those norms, loaded now
  float nrm[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) nrm[r] = 1.f;
  if (m == 1) {
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const int j = 20 * d + g + NG * r;
      nrm[r] = a.norms[(size_t)e * I + (j < I ? j : I - 1)];
    }
  }
  // code table: byte q -> its five base-3 digits d_t = c_t + 1, one byte each
  // (entries 243..255 never occur in a packed unit and decode to codes 0)
  if (tid < 256) {
    uint32_t dg[5] = {1u, 1u, 1u, 1u, 1u};
    if (tid < 243) {
      int q = tid;
#pragma unroll
      for (int d = 0; d < 5; ++d) {
        dg[d] = (uint32_t)(q % 3);
        q /= 3;
      }
    }
    lut[tid] = make_uint2(dg[0] | (dg[1] << 8) | (dg[2] << 16) | (dg[3] << 24), dg[4]);
  }
  // decode step (1): rotation and the partial-screen coordinates
  const bool writer = a.dbg && s == 0 && m == 0;
  if (wvi < nbh) {
    rotate_select(x0 * g0, x1 * g1, NS, a.unit, rec[wvi],
                  writer ? a.sel + ((size_t)t * a.nblk + b + wvi) * NS : nullptr,
                  writer ? a.xrot + (size_t)t * H + (b + wvi) * 128 : nullptr);
  }
  if constexpr (VAR) {
    // ||x_b||^2 of every block: 32 lanes hold one block's 128 coordinates
    static_assert(kMaxHidden <= 8 * NT, "the token is two float4 per thread at most");
    const int h0 = 4 * tid, h1 = 4 * (tid + NT);
    float s0 = h0 < H ? q0.x * q0.x + q0.y * q0.y + q0.z * q0.z + q0.w * q0.w : 0.f;
    float s1 = h1 < H ? q1.x * q1.x + q1.y * q1.y + q1.z * q1.z + q1.w * q1.w : 0.f;
    s0 += xor_lane_f<1>(s0);
    s1 += xor_lane_f<1>(s1);
    s0 += xor_lane_f<2>(s0);
    s1 += xor_lane_f<2>(s1);
    s0 += xor_lane_f<4>(s0);
    s1 += xor_lane_f<4>(s1);
    s0 += xor_lane_f<8>(s0);
    s1 += xor_lane_f<8>(s1);
    s0 += xor_lane_f<16>(s0);
    s1 += xor_lane_f<16>(s1);
    if ((lane & 31) == 0) {
      if (h0 < H) qn2[h0 >> 7] = s0;
      if (h1 < H) qn2[h1 >> 7] = s1;
    }
  }
  CFR_TRACE_PHASE(0, 6);
  lds_barrier();
  CFR_TRACE_PHASE(0, 1);

  // screen: thread (d, g) decodes code word d at screened coordinates
  // g, g + NG, g + 2 NG, ..., all its words in flight together (CPB at a time)
  const int ND = a.nd;
  const bool active = d < ND;
  const uint32_t col = (uint32_t)(m * a.lp + 4 * d);
  constexpr int NA = 21;  // sums per thread
  // thread's codes decoded into its word's 20 channels, x-weighted: the
  // table gives the digits d = c + 1, so the sums are sum d x and acc[20]
  // carries sum x, taken off at the end (each digit is one byte-to-float
  // conversion; measured faster than fp16 codes, whose table reads take
  // twice the LDS bandwidth, and than digits computed from the byte)
  auto decode_words = [&](const uint32_t* wq, const float* xq, float* acc) {
#pragma unroll
    for (int u = 0; u < CPB; ++u) {
      acc[20] += xq[u];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint2 cw = lut[(wq[u] >> (8 * kb)) & 0xFFu];
        acc[5 * kb + 0] = fmaf((float)(cw.x & 0xFFu), xq[u], acc[5 * kb + 0]);
        acc[5 * kb + 1] = fmaf((float)((cw.x >> 8) & 0xFFu), xq[u], acc[5 * kb + 1]);
        acc[5 * kb + 2] = fmaf((float)((cw.x >> 16) & 0xFFu), xq[u], acc[5 * kb + 2]);
        acc[5 * kb + 3] = fmaf((float)(cw.x >> 24), xq[u], acc[5 * kb + 3]);
        acc[5 * kb + 4] = fmaf((float)(cw.y & 0xFFu), xq[u], acc[5 * kb + 4]);
      }
    }
  };
  // sum over the NG lanes of each word (register butterfly, every lane ends
  // with the totals)
  auto word_sums = [&](float* acc) {
#pragma unroll
    for (int q = 0; q < NA; ++q) {
      if constexpr (NG > 1) acc[q] += xor_lane_f<1>(acc[q]);
      if constexpr (NG > 2) acc[q] += xor_lane_f<2>(acc[q]);
      if constexpr (NG > 4) acc[q] += xor_lane_f<4>(acc[q]);
      if constexpr (NG > 8) acc[q] += xor_lane_f<8>(acc[q]);
    }
  };
  // lane g's value of its r-th channel 20 d + g + NG r
  auto lane_value = [&](const float* acc, int r) {
    float v = acc[(NG * r < 20) ? NG * r : 19];
#pragma unroll
    for (int q = 1; q < NG; ++q)
      if (NG * r + q < 20) v = g == q ? acc[NG * r + q] : v;
    v -= acc[20];
    return v;
  };
  // per lane channel: alpha-scaled sum over the workgroup's blocks (the
  // up half times ||d_j||), before the fixed-point accumulator
  float tot[RPL];
  if constexpr (BG == 1) {
    // screen: thread (d, g) decodes code word d at screened coordinates
    // g, g + NG, g + 2 NG, ..., all its words in flight together (CPB at a time)
    float acc[NA];
#pragma unroll
    for (int q = 0; q < NA; ++q) acc[q] = 0.f;
    if (active) {
      // uniform base of this (expert, block) and 32-bit per-coordinate offsets
      const uint8_t* ub = a.codes + ((size_t)e * a.nblk + b) * 128 * a.unit;
      for (int c0 = g; c0 < NS; c0 += NG * CPB) {
        uint32_t wq[CPB];
        float xq[CPB];
#pragma unroll
        for (int u = 0; u < CPB; ++u) {
          const int c = c0 + u * NG;
          const int2 rc = rec[0][c < NS ? c : NS - 1];  // clamped; past the list x = 0
          wq[u] = *reinterpret_cast<const uint32_t*>(ub + ((uint32_t)rc.x + col));
          xq[u] = c < NS ? __int_as_float(rc.y) : 0.f;
        }
        decode_words(wq, xq, acc);
      }
    }
    CFR_TRACE_PHASE(0, 2);
    word_sums(acc);
    CFR_TRACE_PHASE(0, 3);
    // Every loaded value is consumed before the first atomic or store: on this
    // target the in-order memory counter also counts stores and atomics, so a
    // wait for a load placed after them would wait for them as well.
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      tot[r] = f16f(al[r]) * nrm[r] * lane_value(acc, r);
      asm volatile("" ::"v"(tot[r]));
    }
  } else {
    // the group's blocks BC at a time (the host picks BG only when one batch
    // of CPB coordinates covers n_screen), every word of the BC blocks in
    // flight together; each block's sums scaled by its alpha and added up
    float sum[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) sum[r] = 0.f;
    // chunk by chunk: the chunk's words and scales, then its decode (a
    // prefetch of the next chunk measured slower: the registers it holds
    // cost a wave per SIMD).  Blocks past a group cut short by nblk re-read
    // the group's last block and get x = 0, so every load is in bounds and
    // an active thread issues the same loads on every path (threads past the
    // half's words skip the whole loop)
    if (active) {
#pragma unroll 1
      for (int i0 = 0; i0 < BG; i0 += BC) {
        uint32_t wq[BC][CPB];
        uint16_t aq[BC][RPL];
#pragma unroll
        for (int i = 0; i < BC; ++i) {
          const int bi = min(i0 + i, nbh - 1);
          const uint8_t* ub = a.codes + ((size_t)e * a.nblk + b + bi) * 128 * a.unit;
#pragma unroll
          for (int u = 0; u < CPB; ++u) {
            const int c = g + u * NG;
            const int2 rc = rec[bi][c < NS ? c : NS - 1];  // clamped; past the list x = 0
            wq[i][u] = *reinterpret_cast<const uint32_t*>(ub + ((uint32_t)rc.x + col));
          }
          load_scales(bi, aq[i]);
        }
        CFR_TRACE_PHASE(0, 2);
#pragma unroll
        for (int i = 0; i < BC; ++i) {
          const int bi = min(i0 + i, nbh - 1);
          float xq[CPB];
#pragma unroll
          for (int u = 0; u < CPB; ++u) {
            const int c = g + u * NG;
            xq[u] = (c < NS && i0 + i < nbh) ? __int_as_float(rec[bi][c < NS ? c : NS - 1].y) : 0.f;
          }
          float acc[NA];
#pragma unroll
          for (int q = 0; q < NA; ++q) acc[q] = 0.f;
          decode_words(wq[i], xq, acc);
          word_sums(acc);
#pragma unroll
          for (int r = 0; r < RPL; ++r) sum[r] = fmaf(f16f(aq[i][r]), lane_value(acc, r), sum[r]);
        }
      }
    }
    CFR_TRACE_PHASE(0, 3);
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      tot[r] = nrm[r] * sum[r];
      asm volatile("" ::"v"(tot[r]));
    }
  }
  float vsum = 0.f;
  if constexpr (VAR) {
    // block order, the same in whichever workgroup owns the channel
#pragma unroll
    for (int q = 0; q < VB; ++q) vsum += q < a.nblk ? f16f(vrho[q]) * qn2[q] : 0.f;
    if (m == 1) vsum *= vdn * vdn;
    asm volatile("" ::"v"(vsum));
  }
  unsigned long long* ap = a.acc + ((size_t)t * 2 + m) * a.ncp + (size_t)s * I;
  if (active) {
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const int i = g + NG * r, j = 20 * d + i;
      if (i < 20 && j < I) atomicAdd(ap + j, to_fix(tot[r]));
    }
  }
  if constexpr (VAR) {
    float* vo = a.var + ((size_t)t * 2 + m) * a.ncp + (size_t)s * I;
    if (vown) vo[b * vper + tid] = vsum;
    // the rest of a share wider than the workgroup (not at the configured
    // shapes): the same sum with plain loads
    for (int c = NT + tid; c < vper && b * vper + c < I; c += NT) {
      const int j = b * vper + c;
      const uint16_t* rp = a.rho + ((size_t)e * a.nblk * 2 + m) * I + j;
      float v = 0.f;
      for (int q = 0; q < a.nblk; ++q) v += f16f(rp[(size_t)q * 2 * I]) * qn2[q];
      if (m == 1) {
        const float dn = a.norms[(size_t)e * I + j];
        v *= dn * dn;
      }
      vo[j] = v;
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
  const uint8_t* w3;  // [E][I][3] rows of rowq bytes (BF16, or 4-bit records)
  const uint16_t* bmat;
  const unsigned long long* acc;
  const float* norms;  // ||d_j|| [E][I]
  float* ypart;
  float* zpart;
  float* ghat;   // debug outputs (written by workgroup 0 of each token when dbg)
  float* vhat;
  float* score;
  int32_t* kept;
  int32_t* status;
  int H, E, I, top, nc, ncp, k, rank, G, Z, cpw, chan, dbg;
  float invI;   // 1 / I rounded to float (exact slot division below 2^17)
  int cps_mul;  // I % 128 == 0: ceil(2^16 / (I / 128)), else 0
  const float* var;  // [B][2][ncp] sketch-error variances (expected-error ranking)
  int rowq = 0;      // bytes of one resident row
};

// misc slots
constexpr int kMiscDigit = 16, kMiscNeed = 17, kMiscCount = 18, kMiscSlot = 19, kMiscDT = 20,
              kMiscCT = 21, kMiscMax = 32;
constexpr int kDirectMax = 64;  // boundary sets up to this size are ranked directly
// First selection pass: candidates are binned by how far their key lies below
// the largest key, 2^kBinShift key units per bin (1/128 of an octave of the
// score for positive scores); the last bin collects everything further down.
constexpr int kBinShift = 16;
constexpr int kBins = 2048;

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)xor_lane<1>((int)v));
  v = max(v, (uint32_t)xor_lane<2>((int)v));
  v = max(v, (uint32_t)xor_lane<4>((int)v));
  v = max(v, (uint32_t)xor_lane<8>((int)v));
  v = max(v, (uint32_t)xor_lane<16>((int)v));
  v = max(v, (uint32_t)xor_lane<32>((int)v));
  return v;
}

__device__ __forceinline__ int lanes_below(unsigned long long m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The expected-error ranking ([zh §方法步骤详情] decode step (2), budgets from
// 28.7%): with the sketch-error variances of g_hat and of v_hat' (the
// latter carrying ||d_j||^2), the first-order variance of the activation
// Var[a'] = (phi'(g_hat) v_hat')^2 var_g + phi(g_hat)^2 var_v' and
// e = w sqrt(p'^2 + Var[a']) = w ||d_j|| sqrt(p^2 + Var[a]); returns its key.
__device__ __forceinline__ uint32_t error_key(unsigned long long g, unsigned long long v, float vg,
                                              float vv, float w, float& gh, float& vh, float& p,
                                              float& sc) {
  gh = from_fix(g) * kInvSqrt128f;
  vh = from_fix(v) * kInvSqrt128f;
  const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gh));  // sigma(g_hat)
  const float phi = gh * sg;
  const float dphi = sg * (1.0f + gh * (1.0f - sg));
  p = phi * vh;
  const float t = dphi * vh;
  sc = w * sqrtf(p * p + t * t * vg + phi * phi * vv);
  return order_key(sc);
}


// One wave finds the bin where the running count over bins 0, 1, ... first
// reaches need (need >= 1 and at most the total count), and writes the bin,
// the places left in it and its size to misc.  Lane l first sums the NB/64
// consecutive bins it owns; then the lanes take one bin each of the lane
// range where the count crosses.
template <int NB>
__device__ __forceinline__ void find_crossing_wave(const int* hist, int need, int* misc) {
  constexpr int BPL = NB / 64;
  static_assert(BPL % 4 == 0 && BPL <= 64, "whole int4 groups per lane");
  const int lane = threadIdx.x & 63;
  const int4* hp = reinterpret_cast<const int4*>(hist + lane * BPL);
  int own = 0;
#pragma unroll
  for (int q = 0; q < BPL / 4; ++q) {
    const int4 v = hp[q];
    own += (v.x + v.y) + (v.z + v.w);
  }
  const int incl = wave_scan(own);
  const int L = max(__builtin_ffsll((long long)__ballot(incl >= need)) - 1, 0);  // first lane reaching need
  const int before = __builtin_amdgcn_readlane(incl - own, L);
  const int hb = lane < BPL ? hist[L * BPL + lane] : 0;
  const int run = wave_scan(hb) + before;  // count through this bin
  const int b = __builtin_ffsll((long long)__ballot(lane < BPL && run >= need)) - 1;
  if (lane == b) {
    misc[kMiscDigit] = L * BPL + b;
    misc[kMiscNeed] = need - (run - hb);
    misc[kMiscCount] = hb;
  }
}

// Ranks of flagged candidates in ascending candidate order, the order
// (pair slot i, wave, lane, j) for pair P = i NT + tid holding candidates 2P
// and 2P + 1: out[i] = flagged candidates before candidate 2P.  wc: P2 * NW
// ints not reused before the next barrier.  One barrier inside; every wave
// scans the per-(slot, wave) counts itself (lane l holds entries 2l, 2l + 1).
template <int NT, int PER>
__device__ __forceinline__ void ordered_counts(const bool (&f)[PER], int* wc, int (&out)[PER / 2]) {
  constexpr int NW = NT / 64, P2 = PER / 2;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  unsigned long long b0[P2], b1[P2];
#pragma unroll
  for (int i = 0; i < P2; ++i) {
    b0[i] = __ballot(f[2 * i]);
    b1[i] = __ballot(f[2 * i + 1]);
    if (lane == 0) wc[i * NW + wave] = __popcll(b0[i]) + __popcll(b1[i]);
  }
  lds_barrier();
  const int q0 = 2 * lane < P2 * NW ? wc[2 * lane] : 0;
  const int q1 = 2 * lane + 1 < P2 * NW ? wc[2 * lane + 1] : 0;
  const int incl = wave_scan(q0 + q1);
  const int excl = incl - q0 - q1;
#pragma unroll
  for (int i = 0; i < P2; ++i) {
    const int qq = i * NW + wave;
    const int base = __builtin_amdgcn_readlane(excl, qq >> 1) + ((qq & 1) ? __builtin_amdgcn_readlane(q0, qq >> 1) : 0);
    out[i] = base + lanes_below(b0[i]) + lanes_below(b1[i]);
  }
}

// Writes the flagged candidates to kept_out in ascending order (at most kk).
template <int NT, int PER>
__device__ __forceinline__ void write_kept_debug(const bool (&f)[PER], int* wc, int32_t* kept_out, int kk) {
  int rk[PER / 2];
  ordered_counts<NT, PER>(f, wc, rk);
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < PER / 2; ++i) {
    const int rA = rk[i], rB = rA + (int)f[2 * i];
    const int c = 2 * (i * NT + tid);
    if (f[2 * i] && rA < kk) kept_out[rA] = c;
    if (f[2 * i + 1] && rB < kk) kept_out[rB] = c + 1;
  }
}

// VAR: rank by the expected squared error of skipping (error_key) instead of
// the output-unit score.
template <int NT, int PER, int NCH, bool VAR, bool Q4>
__global__ __launch_bounds__(NT) void k_select(SelectArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NW = NT / 64, P2 = PER / 2;
  static_assert(PER % 2 == 0, "candidates are taken in pairs");
  static_assert(P2 * NW <= 128, "two wave counts per lane");
  CFR_TRACE_PHASE(1, 0);
  const int wgs = a.G + a.Z;
  const int t = blockIdx.x / wgs, w = blockIdx.x - t * wgs;
  const bool recover = w >= a.G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H, I = a.I, nc = a.nc, k = a.k;
  const GatherLds L(H, a.ncp, NT, a.chan);
  float* xs = reinterpret_cast<float*>(smem + L.xs);
  float* pvl = reinterpret_cast<float*>(smem + L.pv);
  uint8_t* flags = smem + L.flags;
  uint32_t* dl = reinterpret_cast<uint32_t*>(smem + L.dl);
  float* yred = reinterpret_cast<float*>(smem + L.yred);
  int* hist = reinterpret_cast<int*>(smem + L.hist);
  int* list = reinterpret_cast<int*>(smem + L.list);
  int* misc = reinterpret_cast<int*>(smem + L.misc);
  int2* bmem = reinterpret_cast<int2*>(smem + L.bmem);
  int* wcnt = reinterpret_cast<int*>(smem + L.wcnt);
  int* sl_e = reinterpret_cast<int*>(smem + L.slot_e);
  float* sl_w = reinterpret_cast<float*>(smem + L.slot_w);
  float* zw = reinterpret_cast<float*>(smem + L.zred);

  const bool all = k == nc;
  const bool partial = !all && k > 0;
  const int kk = all ? nc : k;  // kept candidates
  const int r0 = recover ? 0 : min(w * a.chan, kk);
  const int r1 = recover ? 0 : min(r0 + a.chan, kk);
  const bool dbgw = a.dbg && w == 0;
  // slot of candidate c (c < 2^17): exact through the float reciprocal of I
  auto slot_of = [&](int c) { return (int)(((float)c + 0.5f) * a.invI); };

  // ---- loads, all issued up front in straight-line code at clamped
  // addresses (a guarded load compiles to a branch that waits on it): the
  // screen sums of this thread's candidate pairs (the up sums carry ||d||),
  // routing, the token.  Pair P = i NT + tid holds candidates 2P and 2P + 1. ----
  static_assert(kMaxHidden <= 2 * NT * 4, "the token is two float4 per thread at most");
  // the token's routing weights first, lane s holding slot s's (for the
  // scores): loads complete in issue order, so waiting for these must not
  // wait for the screen sums issued after them
  const float gwl = a.gw[t * a.top + min(lane, a.top - 1)];
  ulonglong2 gq[P2], vq[P2];
  float2 gvq[VAR ? P2 : 1], vvq[VAR ? P2 : 1];
  float2 wq[P2];
  {
    const __amdgpu_buffer_rsrc_t ars = buffer_rsrc(a.acc + (size_t)t * 2 * a.ncp, (uint32_t)(a.ncp * 16));
    const uint32_t vofs = (uint32_t)a.ncp * 8u;
#pragma unroll
    for (int i = 0; i < P2; ++i) {
      const uint32_t o = (uint32_t)(i * NT + tid) * 16u;
      const auto g4 = __builtin_amdgcn_raw_buffer_load_b128(ars, o, 0, 0);
      const auto v4 = __builtin_amdgcn_raw_buffer_load_b128(ars, o + vofs, 0, 0);
      gq[i] = make_ulonglong2(((unsigned long long)g4[1] << 32) | g4[0], ((unsigned long long)g4[3] << 32) | g4[2]);
      vq[i] = make_ulonglong2(((unsigned long long)v4[1] << 32) | v4[0], ((unsigned long long)v4[3] << 32) | v4[2]);
    }
    if constexpr (VAR) {
      const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(a.var + (size_t)t * 2 * a.ncp, (uint32_t)(a.ncp * 8));
      const uint32_t wofs = (uint32_t)a.ncp * 4u;
#pragma unroll
      for (int i = 0; i < P2; ++i) {
        const uint32_t o = (uint32_t)(i * NT + tid) * 8u;
        const auto g2 = __builtin_amdgcn_raw_buffer_load_b64(vrs, o, 0, 0);
        const auto v2 = __builtin_amdgcn_raw_buffer_load_b64(vrs, o + wofs, 0, 0);
        gvq[i] = make_float2(__uint_as_float(g2[0]), __uint_as_float(g2[1]));
        vvq[i] = make_float2(__uint_as_float(v2[0]), __uint_as_float(v2[1]));
      }
    }
  }
  const int rslot = tid < a.top ? tid : a.top - 1;
  const int id_raw = a.ids[t * a.top + rslot];
  const float gw_raw = a.gw[t * a.top + rslot];
  const float* xt = a.x + (size_t)t * H;
  const int hx0 = tid * 4, hx1 = (tid + NT) * 4;
  const float4 xr0 = *reinterpret_cast<const float4*>(xt + (hx0 < H ? hx0 : H - 4));
  const float4 xr1 = *reinterpret_cast<const float4*>(xt + (hx1 < H ? hx1 : H - 4));
  if (partial)
    for (int q = tid; q < kBins; q += NT) hist[q] = 0;

  // ---- scores: s = w ||d|| |silu(g_hat) v_hat| as order-preserving keys;
  // padding candidates (index >= nc) get key 0, below every real one ----
  uint32_t key[PER];
  float pr[PER];
  uint32_t kmax = 0u;
  {
#pragma unroll
    for (int i = 0; i < P2; ++i) {
      if (a.cps_mul) {
        // I a multiple of 128: the wave's 128 candidates of pair slot i (chunk
        // q = i NW + wave) lie in routed slot q / (I / 128), scalar arithmetic
        const int q = i * NW + wave;
        const int sl = min((q * a.cps_mul) >> 16, a.top - 1);
        const float wv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gwl), sl));
        wq[i] = make_float2(wv, wv);
      } else {
        const int c2 = 2 * (i * NT + tid);
        wq[i] = make_float2(__shfl(gwl, min(slot_of(c2), a.top - 1)),
                            __shfl(gwl, min(slot_of(c2 + 1), a.top - 1)));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float gh, vh, p, sc;
        uint32_t k0;
        if constexpr (VAR)
          k0 = error_key(j ? gq[i].y : gq[i].x, j ? vq[i].y : vq[i].x, j ? gvq[i].y : gvq[i].x,
                         j ? vvq[i].y : vvq[i].x, j ? wq[i].y : wq[i].x, gh, vh, p, sc);
        else
          k0 = score_key(j ? gq[i].y : gq[i].x, j ? vq[i].y : vq[i].x, j ? wq[i].y : wq[i].x, gh, vh, p,
                         sc);
        const int c = 2 * (i * NT + tid) + j;
        const uint32_t kv = c < nc ? k0 : 0u;
        key[2 * i + j] = kv;
        pr[2 * i + j] = p;
        kmax = max(kmax, kv);
      }
    }
    kmax = wave_max_u32(kmax);
  }
  if (lane == 0) misc[kMiscMax + wave] = (int)kmax;
  if (tid < a.top) {
    sl_e[tid] = clamp_expert(id_raw, a.E, a.status);
    sl_w[tid] = gw_raw;
  }
  if (tid == 0) misc[kMiscSlot] = 0;
  lds_barrier();
  CFR_TRACE_PHASE(1, 1);
  if (dbgw) {
    // debug copies of g_hat, v_hat and the scores: a separate pass that reads
    // the sums again (kept out of the loop above, whose loads it would stall)
    for (int c = tid; c < nc; c += NT) {
      const int sl = slot_of(c);
      float gh, vh, p, sc;
      const unsigned long long* at = a.acc + (size_t)t * 2 * a.ncp + c;
      if constexpr (VAR) {
        const float* vt = a.var + (size_t)t * 2 * a.ncp + c;
        error_key(at[0], at[a.ncp], vt[0], vt[a.ncp], sl_w[sl], gh, vh, p, sc);
      } else {
        score_key(at[0], at[a.ncp], sl_w[sl], gh, vh, p, sc);
      }
      const float nd = a.norms[(size_t)sl_e[sl] * I + (c - sl * I)];
      a.ghat[(size_t)t * nc + c] = gh;
      a.vhat[(size_t)t * nc + c] = nd > 0.f ? vh / nd : 0.f;
      a.score[(size_t)t * nc + c] = sc;
    }
  }

  // ---- exact top-k ----
  // Distance below the largest key M, d = M - key: a smaller d is a larger
  // score; among equal d the lower candidate index wins.  Pass 1 counts the
  // bins min(d >> kBinShift, last) and finds the bin b* where the running
  // count reaches k: bins before it are kept (S1), bins after it are not.
  uint32_t M = 0u;
#pragma unroll
  for (int q = 0; q < NW; q += 4) {
    const int4 m4 = *reinterpret_cast<const int4*>(misc + kMiscMax + q);
    M = max(M, max(max((uint32_t)m4.x, (uint32_t)m4.y), max((uint32_t)m4.z, (uint32_t)m4.w)));
  }
  uint32_t bin[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    key[q] = M - key[q];  // key now holds d
    bin[q] = min(key[q] >> kBinShift, (uint32_t)(kBins - 1));
  }
  if (recover && partial) {
    // d and p of every candidate, for the recovery threads' early b requests
#pragma unroll
    for (int i = 0; i < P2; ++i) {
      const int P = i * NT + tid;
      *reinterpret_cast<uint2*>(dl + 2 * P) = make_uint2(key[2 * i], key[2 * i + 1]);
      *reinterpret_cast<float2*>(pvl + 2 * P) = make_float2(pr[2 * i], pr[2 * i + 1]);
    }
  }
  int bstar = 0, need = kk, cnt = 0;
  if (partial) {
#pragma unroll
    for (int q = 0; q < PER; ++q) atomicAdd(&hist[bin[q]], 1);
    lds_barrier();
    if (wave == 0) find_crossing_wave<kBins>(hist, kk, misc);
    lds_barrier();
    bstar = misc[kMiscDigit];
    need = misc[kMiscNeed];
    cnt = misc[kMiscCount];
  }
  CFR_TRACE_PHASE(1, 2);

  // recovery geometry: Rp = rank / 8 rounded up to a power of two threads
  // per candidate, each 8 coefficients (one uint4) of b_j; thread (zcl, zr8)
  // takes candidates zcb0 + zcl + u zcpp of this workgroup's range
  int rp_log = 0;
  while ((8 << rp_log) < a.rank) ++rp_log;
  const int R8 = a.rank >> 3;
  const int zcpp = NT >> rp_log;
  const int zcl = tid >> rp_log, zr8 = tid & ((1 << rp_log) - 1);
  int zcb0 = 0, zcb1 = 0;
  if (recover) {
    const int zper = (nc + a.Z - 1) / a.Z;
    zcb0 = min((w - a.G) * zper, nc);
    zcb1 = min(zcb0 + zper, nc);
  }
  const __amdgpu_buffer_rsrc_t brs = buffer_rsrc(a.bmat, (uint32_t)((size_t)a.E * I * a.rank * 2));
  // byte offset of this thread's uint4 of b_j for candidate cc
  auto brow = [&](int cc) -> uint32_t {
    const int sl = slot_of(cc);
    return (uint32_t)((((size_t)sl_e[sl] * I + (cc - sl * I)) * a.rank + zr8 * 8) * 2);
  };
  uint4 zb[4];
  float zn[4];  // ||d_j|| of the first-pass candidates (p = p' / ||d_j||)
  auto norm_of = [&](int cc) {
    const int sl = slot_of(cc);
    return a.norms[(size_t)sl_e[sl] * I + (cc - sl * I)];
  };

  const bool fast = partial && cnt <= kDirectMax;
  if (fast) {
    // ---- the usual case: a boundary bin small enough to rank directly ----
    // S1 (n1 candidates) takes ranks [0, n1) in candidate order; b*'s members
    // are ranked by (d, index) and the first `need` take ranks [n1, k).
    const int n1 = kk - need;
    bool s1[PER], mem[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      s1[q] = bin[q] < (uint32_t)bstar;
      mem[q] = bin[q] == (uint32_t)bstar;
    }
    if (recover) {
      // b rows of the first pass, except candidates surely kept
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int cnd = zcb0 + zcl + u * zcpp;
        const int cc = min(cnd, max(zcb1 - 1, 0));
        const bool ld = cnd < zcb1 && zr8 < R8 && (dl[cc] >> kBinShift) >= (uint32_t)bstar;
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(brs, ld ? brow(cc) : kNoLoad, 0, 0);
        zb[u] = make_uint4(v[0], v[1], v[2], v[3]);
        zn[u] = norm_of(cc);
      }
      asm volatile("" ::: "memory");  // keeps the requests here, ahead of the barriers below
    }
    // S1 counts per (pair slot, wave) for the ranks (gather workgroups)
    unsigned long long ba[PER];
    if (!recover) {
#pragma unroll
      for (int i = 0; i < P2; ++i) {
        ba[2 * i] = __ballot(s1[2 * i]);
        ba[2 * i + 1] = __ballot(s1[2 * i + 1]);
        if (lane == 0) wcnt[i * NW + wave] = __popcll(ba[2 * i]) + __popcll(ba[2 * i + 1]);
      }
    }
    // b*'s members into bmem (a few per workgroup: one LDS atomic each)
#pragma unroll
    for (int q = 0; q < PER; ++q)
      if (mem[q]) {
        const int slot = atomicAdd(&misc[kMiscSlot], 1);
        if (slot < kDirectMax) bmem[slot] = make_int2((int)key[q], 2 * ((q >> 1) * NT + tid) + (q & 1));
      }
    const bool wantflags = recover || dbgw;
    if (wantflags) {
#pragma unroll
      for (int i = 0; i < P2; ++i)
        *reinterpret_cast<uint16_t*>(flags + 2 * (i * NT + tid)) =
            (uint16_t)((uint32_t)s1[2 * i] | ((uint32_t)s1[2 * i + 1] << 8));
    }
    if (!recover) {
      if (hx0 < H) *reinterpret_cast<float4*>(xs + hx0) = xr0;
      if (hx1 < H) *reinterpret_cast<float4*>(xs + hx1) = xr1;
    }
    CFR_TRACE_PHASE(1, 7);
    lds_barrier();
    if (!recover && r0 < n1) {
      // every wave scans the counts itself (lane l holds entries 2l, 2l + 1)
      // and writes its S1 candidates whose rank falls in [r0, min(r1, n1))
      const int hi = min(r1, n1);
      const int q0 = 2 * lane < P2 * NW ? wcnt[2 * lane] : 0;
      const int q1 = 2 * lane + 1 < P2 * NW ? wcnt[2 * lane + 1] : 0;
      const int incl = wave_scan(q0 + q1);
      const int excl = incl - q0 - q1;
#pragma unroll
      for (int i = 0; i < P2; ++i) {
        const int qq = i * NW + wave;
        const int base = __builtin_amdgcn_readlane(excl, qq >> 1) + ((qq & 1) ? __builtin_amdgcn_readlane(q0, qq >> 1) : 0);
        const int n = __popcll(ba[2 * i]) + __popcll(ba[2 * i + 1]);
        if (base < hi && base + n > r0) {  // wave-uniform
          const int rA = base + lanes_below(ba[2 * i]) + lanes_below(ba[2 * i + 1]);
          const int rB = rA + (int)s1[2 * i];
          const int c = 2 * (i * NT + tid);
          if (s1[2 * i] && rA >= r0 && rA < hi) list[rA - r0] = c;
          if (s1[2 * i + 1] && rB >= r0 && rB < hi) list[rB - r0] = c + 1;
        }
      }
    }
    if (wave == 0 && (r1 > n1 || wantflags)) {
      // one member per lane; each compares itself with every other member
      // through lane broadcasts
      const int2 me = bmem[lane < cnt ? lane : 0];
      const uint32_t md = lane < cnt ? (uint32_t)me.x : 0xFFFFFFFFu;
      const int mi = lane < cnt ? me.y : 0x7FFFFFFF;
      const int n = __builtin_amdgcn_readfirstlane(cnt);
      int rk = 0;
      for (int q = 0; q < n; ++q) {
        const uint32_t od = (uint32_t)__builtin_amdgcn_readlane((int)md, q);
        const int oi = __builtin_amdgcn_readlane(mi, q);
        rk += (int)((od < md) | ((od == md) & (oi < mi)));
      }
      if (lane < cnt && rk < need) {
        const int r = n1 + rk;
        if (r >= r0 && r < r1) list[r - r0] = mi;
        if (wantflags) flags[mi] = 1;
      }
    }
    lds_barrier();
    if (dbgw) {
      // the debug copy of the kept list, in candidate order
      bool on[PER];
#pragma unroll
      for (int q = 0; q < PER; ++q) on[q] = flags[2 * ((q >> 1) * NT + tid) + (q & 1)] != 0;
      write_kept_debug<NT, PER>(on, wcnt + 128, a.kept + (size_t)t * nc, kk);
    }
  } else {
    // ---- general case: keep all, keep none, or a large boundary bin ----
    uint32_t dT = 0u;
    int cT = -1;
    if (partial) {
      // boundary set: d in bin b* with (d & mask) == prefix
      uint32_t prefix = 0u, mask = 0u;
      auto member = [&](int q) { return bin[q] == (uint32_t)bstar && (key[q] & mask) == prefix; };
      // 0: the whole boundary set is kept; 1: rank it directly; 2: equal keys
      int mode = cnt == need ? 0 : -1;
      for (int pass = 0; pass < 3 && mode < 0; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nbins = pass == 2 ? 1024 : 2048;
        const uint32_t dm = (uint32_t)nbins - 1u;
        for (int q = tid; q < nbins; q += NT) hist[q] = 0;
        lds_barrier();
#pragma unroll
        for (int q = 0; q < PER; ++q)
          if (member(q)) atomicAdd(&hist[(key[q] >> shift) & dm], 1);
        lds_barrier();
        if (wave == 0) {
          if (pass == 2) find_crossing_wave<1024>(hist, need, misc);
          else find_crossing_wave<2048>(hist, need, misc);
        }
        lds_barrier();
        prefix |= (uint32_t)misc[kMiscDigit] << shift;
        mask |= dm << shift;
        need = misc[kMiscNeed];
        cnt = misc[kMiscCount];
        mode = cnt == need ? 0 : (cnt <= kDirectMax ? 1 : (pass == 2 ? 2 : -1));
      }
      if (mode == 0) {
        // every d of the boundary set is kept: the boundary is its largest d
        dT = mask == 0u ? (bstar == kBins - 1 ? 0xFFFFFFFFu : (((uint32_t)bstar + 1u) << kBinShift) - 1u)
                        : (prefix | ~mask);
        cT = 0x7FFFFFFF;
      } else if (mode == 1) {
        // rank the members (d ascending, index ascending); the need-th is the boundary
#pragma unroll
        for (int q = 0; q < PER; ++q)
          if (member(q)) {
            const int slot = atomicAdd(&misc[kMiscSlot], 1);
            if (slot < kDirectMax) bmem[slot] = make_int2((int)key[q], 2 * ((q >> 1) * NT + tid) + (q & 1));
          }
        lds_barrier();
        if (wave == 0) {
          const int2 me = bmem[lane < cnt ? lane : 0];
          const uint32_t md = lane < cnt ? (uint32_t)me.x : 0xFFFFFFFFu;
          const int mi = lane < cnt ? me.y : 0x7FFFFFFF;
          const int n = __builtin_amdgcn_readfirstlane(cnt);
          int rk = 0;
          for (int q = 0; q < n; ++q) {
            const uint32_t od = (uint32_t)__builtin_amdgcn_readlane((int)md, q);
            const int oi = __builtin_amdgcn_readlane(mi, q);
            rk += (int)((od < md) | ((od == md) & (oi < mi)));
          }
          if (lane < cnt && rk == need - 1) {
            misc[kMiscDT] = (int)md;
            misc[kMiscCT] = mi;
          }
        }
        lds_barrier();
        dT = (uint32_t)misc[kMiscDT];
        cT = misc[kMiscCT];
      } else {
        // all members share one d: the need lowest indices among them
        dT = prefix;
        bool mb[PER];
#pragma unroll
        for (int q = 0; q < PER; ++q) mb[q] = member(q);
        int ob[P2];
        ordered_counts<NT, PER>(mb, wcnt + 128, ob);
#pragma unroll
        for (int i = 0; i < P2; ++i) {
          const int o1 = ob[i] + (int)mb[2 * i];
          if (mb[2 * i] && ob[i] == need - 1) misc[kMiscCT] = 2 * (i * NT + tid);
          if (mb[2 * i + 1] && o1 == need - 1) misc[kMiscCT] = 2 * (i * NT + tid) + 1;
        }
        lds_barrier();
        cT = misc[kMiscCT];
      }
    }
    // kept flags and ranks in ascending candidate order
    bool on[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int c = 2 * ((q >> 1) * NT + tid) + (q & 1);
      on[q] = all ? c < nc : (partial && ((key[q] < dT) | ((key[q] == dT) & (c <= cT))));
    }
    if (recover) {
#pragma unroll
      for (int i = 0; i < P2; ++i) {
        const int P = i * NT + tid;
        *reinterpret_cast<uint16_t*>(flags + 2 * P) = (uint16_t)((uint32_t)on[2 * i] | ((uint32_t)on[2 * i + 1] << 8));
        *reinterpret_cast<float2*>(pvl + 2 * P) = make_float2(pr[2 * i], pr[2 * i + 1]);
      }
    }
    if (!recover) {
      if (hx0 < H) *reinterpret_cast<float4*>(xs + hx0) = xr0;
      if (hx1 < H) *reinterpret_cast<float4*>(xs + hx1) = xr1;
    }
    int rk[P2];
    ordered_counts<NT, PER>(on, wcnt, rk);  // one barrier inside
#pragma unroll
    for (int i = 0; i < P2; ++i) {
      const int rA = rk[i], rB = rA + (int)on[2 * i];
      const int c = 2 * (i * NT + tid);
      if (on[2 * i]) {
        if (rA >= r0 && rA < r1) list[rA - r0] = c;
        if (dbgw && rA < kk) a.kept[(size_t)t * nc + rA] = c;
      }
      if (on[2 * i + 1]) {
        if (rB >= r0 && rB < r1) list[rB - r0] = c + 1;
        if (dbgw && rB < kk) a.kept[(size_t)t * nc + rB] = c + 1;
      }
    }
    lds_barrier();
    if (recover) {
      // b rows of the first pass, kept candidates skipped
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int cnd = zcb0 + zcl + u * zcpp;
        const int cc = min(cnd, max(zcb1 - 1, 0));
        const bool ld = cnd < zcb1 && zr8 < R8 && !flags[cc];
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(brs, ld ? brow(cc) : kNoLoad, 0, 0);
        zb[u] = make_uint4(v[0], v[1], v[2], v[3]);
        zn[u] = norm_of(cc);
      }
    }
  }
  CFR_TRACE_PHASE(1, 3);

  if (!recover) {
    // ---- decode step (3): exact kept channels from the resident rows
    // (native BF16, or 4-bit records dequantized on the fly) ----
    // wave v takes list entries [v cpw, (v+1) cpw), two channels at a time
    // when registers allow, all rows in flight together
    float yv[NCH][8];
#pragma unroll
    for (int q = 0; q < NCH; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i) yv[q][i] = 0.f;
    const int nmine = r1 - r0;
    constexpr bool kPair = NCH <= 4;
    constexpr int NR = kPair ? 2 : 1;
    const int qend = min((wave + 1) * a.cpw, nmine);
    for (int q0 = wave * a.cpw; q0 < qend; q0 += NR) {
      const bool two = kPair && q0 + 1 < qend;
      int cc[NR];
      cc[0] = list[q0];
      if constexpr (kPair) cc[NR - 1] = two ? list[q0 + 1] : cc[0];
      Chunk8<Q4> gq2[NR][NCH], uq2[NR][NCH], dq2[NR][NCH];
      int sr[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        sr[r] = slot_of(cc[r]);
        const uint8_t* row = a.w3 + ((size_t)sl_e[sr[r]] * I + (cc[r] - sr[r] * I)) * 3 * a.rowq;
        if (r == 0 || two) {  // wave-uniform
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch) {
            const int h = min(ch * 512 + lane * 8, H - 8);  // clamped; the tail is masked below
            gq2[r][ch].load(row, H, h);
            uq2[r][ch].load(row + a.rowq, H, h);
            dq2[r][ch].load(row + 2 * a.rowq, H, h);
          }
        } else {
#pragma unroll
          for (int ch = 0; ch < NCH; ++ch) gq2[r][ch].clear(), uq2[r][ch].clear(), dq2[r][ch].clear();
        }
      }
      float gs[NR], vs[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) gs[r] = vs[r] = 0.f;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const int h = ch * 512 + lane * 8;
        if (h < H) {
          const float4 xa = *reinterpret_cast<const float4*>(xs + h);
          const float4 xb = *reinterpret_cast<const float4*>(xs + h + 4);
          const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            float gv[8], uv[8];
            gq2[r][ch].vals(gv);
            uq2[r][ch].vals(uv);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              gs[r] = fmaf(gv[i], xv[i], gs[r]);
              vs[r] = fmaf(uv[i], xv[i], vs[r]);
            }
          }
        }
      }
      float cf[NR];
      cf[0] = sl_w[sr[0]] * silu(wave_sum(gs[0])) * wave_sum(vs[0]);
      if constexpr (kPair) cf[NR - 1] = two ? sl_w[sr[NR - 1]] * silu(wave_sum(gs[NR - 1])) * wave_sum(vs[NR - 1]) : 0.f;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          float dv[8];
          dq2[r][ch].vals(dv);
#pragma unroll
          for (int i = 0; i < 8; ++i) yv[ch][i] = fmaf(cf[r], dv[i], yv[ch][i]);
        }
    }
    CFR_TRACE_PHASE(1, 4);
    // ---- partial output: only waves that took channels contribute ----
    // With one LDS slot per wave (rows up to 2048 wide) each such wave stores
    // its rows in its slot; otherwise waves [0, NW/2) store and the others
    // add theirs.  The slots are then summed in a fixed order.
    constexpr int SL = NCH <= 4 ? NW : NW / 2;
    const int used = min(NW, (nmine + a.cpw - 1) / a.cpw);  // waves holding channels
    const int slot = wave % SL;
    if (wave < SL && (SL == NW ? wave < used : true)) {
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
    if constexpr (SL < NW) {
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
    }
    lds_barrier();
    const int nsl = min(SL, used);  // slots that received rows
    float* yp = a.ypart + ((size_t)t * a.G + w) * H;
    for (int h = tid * 4; h < H; h += NT * 4) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int q = 0; q < nsl; ++q) {
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
  // z = sum over skipped candidates of w p_j b_j; the first pass was
  // requested during the selection, later passes skip kept candidates' rows
  float zacc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) zacc[d] = 0.f;
  auto zadd = [&](const uint4& bq, float cf) {
    const uint32_t bw[4] = {bq.x, bq.y, bq.z, bq.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      zacc[2 * d] = fmaf(cf, lo16(bw[d]), zacc[2 * d]);
      zacc[2 * d + 1] = fmaf(cf, hi16(bw[d]), zacc[2 * d + 1]);
    }
  };
  // w p_j b_j with p_j = p'_j / ||d_j|| (a zero norm means b_j = U^T d_j = 0)
  auto coef = [&](bool skip, int cc, float nd) {
    return (skip && nd > 0.f) ? sl_w[slot_of(cc)] * (pvl[cc] / nd) : 0.f;
  };
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int cnd = zcb0 + zcl + u * zcpp;
    const int cc = min(cnd, max(zcb1 - 1, 0));
    zadd(zb[u], coef(cnd < zcb1 && !flags[cc], cc, zn[u]));
  }
  CFR_TRACE_PHASE(1, 4);
  for (int cb = zcb0 + zcl + 4 * zcpp; cb < zcb1; cb += 4 * zcpp) {
    uint4 bq[4];
    float cf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int cnd = cb + u * zcpp;
      const int cc = cnd < zcb1 ? cnd : zcb1 - 1;
      const bool skip = cnd < zcb1 && !flags[cc];
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(brs, (skip && zr8 < R8) ? brow(cc) : kNoLoad, 0, 0);
      bq[u] = make_uint4(v[0], v[1], v[2], v[3]);
      cf[u] = coef(skip, cc, norm_of(cc));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) zadd(bq[u], cf[u]);
  }
  // sum over the candidates of the wave (lanes with equal zr8), then over waves
  auto zfold = [&](auto hc) {
    constexpr int HH = decltype(hc)::value;
#pragma unroll
    for (int d = 0; d < 8; ++d) zacc[d] += xor_lane_f<HH>(zacc[d]);
  };
  if (rp_log == 0) zfold(std::integral_constant<int, 1>{});
  if (rp_log <= 1) zfold(std::integral_constant<int, 2>{});
  if (rp_log <= 2) zfold(std::integral_constant<int, 4>{});
  if (rp_log <= 3) zfold(std::integral_constant<int, 8>{});
  zfold(std::integral_constant<int, 16>{});
  zfold(std::integral_constant<int, 32>{});
  if (lane < (1 << rp_log) && lane < R8) {
#pragma unroll
    for (int d = 0; d < 8; ++d) zw[wave * 64 + lane * 8 + d] = zacc[d];
  }
  lds_barrier();
  CFR_TRACE_PHASE(1, 5);
  if (tid < a.rank) {
    float z = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) z += zw[v * 64 + tid];
    a.zpart[((size_t)t * a.Z + (w - a.G)) * a.rank + tid] = z;
  }
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
  const float* resid = nullptr;  // non-null: y = resid + output (resid may be y)
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
  // the residual last: the waits above do not wait for it
  float rv = 0.f;
  if (a.resid && tid < kReduceSlice) rv = a.resid[(size_t)t * H + h0 + tid];
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
    // the residual is added to the finished output, as a separate add would
    a.y[(size_t)t * H + h0 + tid] = a.resid ? rv + o : o;
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
// Multiplier m with floor(q / (I / 128)) == (q m) >> 16 for the chunk
// indices q < 2048 used here (I / 128 <= 32); 0 when I is not a multiple of 128.
static int cps_mul(int inter) {
  if (inter % 128) return 0;
  const int cps = inter / 128;
  return (65536 + cps - 1) / cps;
}

static int hip_fail(hipError_t e, const char* what) {
  return fail(CFR_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Zero fill of a device buffer (a kernel rather than a memset node, so that
// a caller may capture it in a graph)
__global__ void k_zero(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  const int blocks = (int)std::min<size_t>((n16 + 255) / 256, 1024);
  if (blocks > 0) k_zero<<<blocks, 256, 0, st>>>(static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

size_t decode_sums_bytes(const cfr_reader& r, int batch) {
  return (sizeof(unsigned long long) * batch * 2 * r.ncp + 255) / 256 * 256;
}

size_t carve_decode_workspace(const cfr_reader& r, int batch, bool debug, char* base, Workspace* w,
                              bool shared) {
  const cfr_config& c = r.cfg;
  const size_t B = batch, H = c.hidden, nc = r.ncand, R = c.rank > 0 ? c.rank : 1;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += (bytes + 255) / 256 * 256;
    return base ? base + at : nullptr;
  };
  Workspace v;
  // the screen sums first: they must be zero when a decode starts, and the
  // reduce kernel leaves them zero
  v.acc = reinterpret_cast<unsigned long long*>(take(sizeof(unsigned long long) * B * 2 * r.ncp));
  v.var = reinterpret_cast<float*>(
      take(c.ranking == CFR_RANK_EXPECTED_ERROR ? sizeof(float) * B * 2 * r.ncp : 0));
  // the gather workgroups of the whole call number at most kMaxGatherWgs
  v.ypart = reinterpret_cast<float*>(take(sizeof(float) * (size_t)kMaxGatherWgs * H));
  v.zpart = reinterpret_cast<float*>(take(sizeof(float) * B * kMaxRecoverWgs * R));
  if (debug) {
    v.xrot = reinterpret_cast<float*>(take(sizeof(float) * B * H));
    v.sel = reinterpret_cast<uint8_t*>(take(B * r.nblk * c.n_screen));
    v.ghat = reinterpret_cast<float*>(take(sizeof(float) * B * nc));
    v.vhat = reinterpret_cast<float*>(take(sizeof(float) * B * nc));
    v.score = reinterpret_cast<float*>(take(sizeof(float) * B * nc));
    v.kept = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * B * nc));
  }
  if (shared) {
    const size_t nb = std::min<size_t>(B, kMaxSharedBatch) * nc;  // union candidates, at most
    v.bscore = reinterpret_cast<float*>(take(sizeof(float) * nb));
    v.meta = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * (1 + std::min<size_t>(B, kMaxSharedBatch) * c.top)));
    v.klist = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * nb));
    v.kflag = reinterpret_cast<uint8_t*>(take(nb));
    v.coef = reinterpret_cast<float*>(take(sizeof(float) * nb * std::min<size_t>(B, kMaxSharedBatch)));
    v.krow = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * nb));
    v.ghist = reinterpret_cast<int32_t*>(take(sizeof(int32_t) * 4096));
  }
  if (w) *w = v;
  return o;
}

Plan make_plan(const cfr_config& c, int batch, int k) {
  Plan p;
  const int nblk = c.hidden / kBlock, nbytes = (c.inter + 4) / 5, nc = c.top * c.inter;
  // screen
  p.nd = (nbytes + 3) / 4;
  p.ng = 16;  // threads per code word: a power of two with ng * nd <= threads
  while (p.ng > 1 && p.ng * p.nd > kScreenThreads) p.ng /= 2;
  // several blocks per workgroup when the batch makes the screen's atomics
  // count (the score ranking, one batch of CPB coordinates per thread
  // covering n_screen; CPB 5, 10, 20 for ng 16, 8, 4): the largest group of
  // 2, 4 or 8 blocks that leaves kScreenMinWgs workgroups (measured best at
  // the Qwen3-30B-A3B layer, batch 4, and the Qwen3-235B-A22B layer, batch 8)
  p.bg = 1;
  if (batch >= 2 && c.ranking == CFR_RANK_SCORE && p.ng >= 4) {
    const int cpb = p.ng == 16 ? 5 : (p.ng == 8 ? 10 : 20);
    if (c.n_screen <= p.ng * cpb)
      while (p.bg < 8 && batch * c.top * 2 * ((nblk + 2 * p.bg - 1) / (2 * p.bg)) >= kScreenMinWgs) p.bg *= 2;
  }
  p.items1 = batch * c.top * ((nblk + p.bg - 1) / p.bg) * 2;
  p.per_xcd1 = (p.items1 + 7) / 8;
  p.lds1 = 0;
  // select/gather: about 240 gather workgroups over the batch plus 16
  // recovery workgroups, so the whole grid fits one workgroup per CU
  const SelectGeom g = select_geom(nc);
  p.nt2 = g.nt;
  p.per = g.per;
  p.ncp = g.nt * g.per;
  const int NW = p.nt2 / 64;
  const int kk = k;
  int gmax = (kMaxGatherWgs - kMaxRecoverWgs) / batch;
  if (gmax < 1) gmax = 1;
  p.chan = (kk + gmax - 1) / gmax;
  if (p.chan < 1) p.chan = 1;
  p.cpw = (p.chan + NW - 1) / NW;
  p.G = (kk + p.chan - 1) / p.chan;
  if (p.G < 1) p.G = 1;
  int z = kMaxRecoverWgs / batch;
  if (z < 1) z = 1;
  p.Z = (c.rank > 0 && k < nc) ? z : 0;
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
      const Plan p = make_plan(c, b, kk);
      // + the screen kernel's static LDS: code table, bg blocks' coordinate
      // lists, block norms
      const size_t st1 = 2048 + 1024 * (size_t)p.bg + 4 * (kMaxHidden / 128);
      if (p.lds1 + st1 > m) m = p.lds1 + st1;
      if (p.lds2 > m) m = p.lds2;
    }
  const DensePlan d = make_dense_plan(c, 1);
  if (d.lds > m) m = d.lds;
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

template <int NT, int PER, int NCH, bool VAR, bool Q4>
static hipError_t launch_select_t(const SelectArgs& a, const Plan& p, int batch, hipStream_t st) {
  static OncePerDevice attr;
  attr([] { allow_lds(k_select<NT, PER, NCH, VAR, Q4>); });
  k_select<NT, PER, NCH, VAR, Q4><<<batch * (p.G + p.Z), NT, p.lds2, st>>>(a);
  return hipGetLastError();
}

template <int PER, bool VAR, bool Q4>
static hipError_t launch_select_n(const SelectArgs& a, const Plan& p, int batch, hipStream_t st) {
  switch (p.nch) {
    case 1: return launch_select_t<512, PER, 1, VAR, Q4>(a, p, batch, st);
    case 2: return launch_select_t<512, PER, 2, VAR, Q4>(a, p, batch, st);
    case 4: return launch_select_t<512, PER, 4, VAR, Q4>(a, p, batch, st);
    default: return launch_select_t<512, PER, 8, VAR, Q4>(a, p, batch, st);
  }
}

template <bool VAR, bool Q4>
static hipError_t launch_select_v(const SelectArgs& a, const Plan& p, int batch, hipStream_t st) {
  switch (p.per) {  // select_geom: 512 threads, 2..32 candidates each
    case 2: return launch_select_n<2, VAR, Q4>(a, p, batch, st);
    case 4: return launch_select_n<4, VAR, Q4>(a, p, batch, st);
    case 6: return launch_select_n<6, VAR, Q4>(a, p, batch, st);
    case 8: return launch_select_n<8, VAR, Q4>(a, p, batch, st);
    case 12: return launch_select_n<12, VAR, Q4>(a, p, batch, st);
    case 16: return launch_select_n<16, VAR, Q4>(a, p, batch, st);
    case 24: return launch_select_n<24, VAR, Q4>(a, p, batch, st);
    default: return launch_select_n<32, VAR, Q4>(a, p, batch, st);
  }
}

// 4-bit rows are read with the output-unit score only (the configuration
// refuses them with the expected-error ranking)
static hipError_t launch_select(const SelectArgs& a, const Plan& p, int batch, bool q4, hipStream_t st) {
  if (q4) return launch_select_v<false, true>(a, p, batch, st);
  return a.var ? launch_select_v<true, false>(a, p, batch, st) : launch_select_v<false, false>(a, p, batch, st);
}

// CPB: coordinates per thread batch, the n_screen = 80 share of one thread in
// one batch
// blocks of a group whose words are in flight together (at most 40 words
// per thread)
constexpr int screen_chunk(int ng, int bg) { return ng >= 8 ? 2 : (bg == 2 ? 2 : 1); }

template <int NG, int CPB, bool VAR, int BG, int BC>
static hipError_t launch_screen_t(const ScreenArgs& a, const Plan& p, hipStream_t st) {
  k_screen<kScreenThreads, NG, CPB, VAR, BG, BC><<<8 * p.per_xcd1, kScreenThreads, 0, st>>>(a);
  return hipGetLastError();
}

// (the whole sketch, VAR: a thread's share of all 128 coordinates in one batch)
template <bool VAR>
static hipError_t launch_screen_v(const ScreenArgs& a, const Plan& p, hipStream_t st) {
  if constexpr (!VAR) {
    if (p.bg > 1) {  // the (ng, bg) pairs make_plan can choose
      switch (p.ng * 16 + p.bg) {
        case 16 * 16 + 2: return launch_screen_t<16, 5, false, 2, screen_chunk(16, 2)>(a, p, st);
        case 16 * 16 + 4: return launch_screen_t<16, 5, false, 4, screen_chunk(16, 4)>(a, p, st);
        case 16 * 16 + 8: return launch_screen_t<16, 5, false, 8, screen_chunk(16, 8)>(a, p, st);
        case 8 * 16 + 2: return launch_screen_t<8, 10, false, 2, screen_chunk(8, 2)>(a, p, st);
        case 8 * 16 + 4: return launch_screen_t<8, 10, false, 4, screen_chunk(8, 4)>(a, p, st);
        case 8 * 16 + 8: return launch_screen_t<8, 10, false, 8, screen_chunk(8, 8)>(a, p, st);
        case 4 * 16 + 2: return launch_screen_t<4, 20, false, 2, screen_chunk(4, 2)>(a, p, st);
        case 4 * 16 + 4: return launch_screen_t<4, 20, false, 4, screen_chunk(4, 4)>(a, p, st);
        case 4 * 16 + 8: return launch_screen_t<4, 20, false, 8, screen_chunk(4, 8)>(a, p, st);
        default: return hipErrorInvalidConfiguration;
      }
    }
  }
  if (p.bg != 1) return hipErrorInvalidConfiguration;
  switch (p.ng) {
    case 16: return launch_screen_t<16, VAR ? 8 : 5, VAR, 1, 1>(a, p, st);
    case 8: return launch_screen_t<8, VAR ? 16 : 10, VAR, 1, 1>(a, p, st);
    case 4: return launch_screen_t<4, 20, VAR, 1, 1>(a, p, st);
    case 2: return launch_screen_t<2, 20, VAR, 1, 1>(a, p, st);
    default: return launch_screen_t<1, 20, VAR, 1, 1>(a, p, st);
  }
}

static hipError_t launch_screen(const ScreenArgs& a, const Plan& p, hipStream_t st) {
  return a.var ? launch_screen_v<true>(a, p, st) : launch_screen_v<false>(a, p, st);
}

static hipError_t launch_reduce(const ReduceArgs& a, int batch, hipStream_t st) {
  k_reduce<<<batch * a.nslices, kReduceThreads, 0, st>>>(a);
  return hipGetLastError();
}

int launch_decode(cfr_reader* r, const float* x, const int32_t* ids, const float* gw, int batch,
                  int k, float* y, hipStream_t st, const DebugOut* dbg, hipEvent_t* ev, int only,
                  const float* resid, const Workspace* wsp) {
  const cfr_config& c = r->cfg;
  const Workspace& W = wsp ? *wsp : r->wk;
  const Plan p = make_plan(c, batch, k);
  auto mark = [&](int i) {
    if (ev) (void)hipEventRecord(ev[i], st);
  };
  hipError_t e;
  mark(0);
  // the sketch-error variances, with the expected-error ranking only
  float* var = c.ranking == CFR_RANK_EXPECTED_ERROR ? W.var : nullptr;
  ScreenArgs A{x, ids, gw, r->sigma, r->codes, r->scales, r->norms, r->rho, W.acc, var, W.xrot,
               W.sel, r->status, c.hidden, c.n_experts, c.inter, c.top, r->ncp, r->nblk,
               c.n_screen, r->lp, r->unit, p.nd, p.ng, p.items1, p.per_xcd1, dbg != nullptr};
  if (only < 0 || only == 0)
    if ((e = launch_screen(A, p, st)) != hipSuccess) return hip_fail(e, "screen launch");
  mark(1);
  SelectArgs B{x, ids, gw, r->w3, r->b, W.acc, r->norms, W.ypart, W.zpart, W.ghat, W.vhat,
               W.score, W.kept, r->status, c.hidden, c.n_experts, c.inter, c.top, r->ncand,
               r->ncp, k, c.rank, p.G, p.Z, p.cpw, p.chan, dbg != nullptr, 1.0f / (float)c.inter,
               cps_mul(c.inter), var};
  B.rowq = row_bytes(c.hidden, q4_rows(c));
  if (only < 0 || only == 1)
    if ((e = launch_select(B, p, batch, q4_rows(c), st)) != hipSuccess) return hip_fail(e, "select launch");
  mark(2);
  ReduceArgs C{W.ypart, W.zpart, r->u, y, W.acc, c.hidden, p.G, p.Z, c.rank, r->ncp,
               p.nslices, 1, resid};
  if (only < 0 || only == 2)
    if ((e = launch_reduce(C, batch, st)) != hipSuccess) return hip_fail(e, "reduce launch");
  mark(3);
  if (dbg) {
    const int H = c.hidden, nblk = r->nblk, nsc = batch * r->ncand;
    auto cp = [&](void* dst, const void* src, size_t bytes) -> hipError_t {
      return dst ? hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st) : hipSuccess;
    };
    if ((e = cp(dbg->xrot, W.xrot, sizeof(float) * batch * H)) != hipSuccess ||
        (e = cp(dbg->sel, W.sel, (size_t)batch * nblk * c.n_screen)) != hipSuccess ||
        (e = cp(dbg->ghat, W.ghat, sizeof(float) * nsc)) != hipSuccess ||
        (e = cp(dbg->vhat, W.vhat, sizeof(float) * nsc)) != hipSuccess ||
        (e = cp(dbg->score, W.score, sizeof(float) * nsc)) != hipSuccess)
      return hip_fail(e, "debug copy");
    if (dbg->kept && k > 0) {
      e = hipMemcpy2DAsync(dbg->kept, sizeof(int32_t) * k, W.kept, sizeof(int32_t) * r->ncand,
                           sizeof(int32_t) * k, batch, hipMemcpyDeviceToDevice, st);
      if (e != hipSuccess) return hip_fail(e, "debug copy kept");
    }
  }
  return CFR_OK;
}

int launch_decode_shared(cfr_reader* r, const float* x, const int32_t* ids, const float* gw, int batch,
                         int k, float* y, hipStream_t st, const float* resid, float* bscore_out,
                         int32_t* kept_out, int32_t* meta_out) {
  const cfr_config& c = r->cfg;
  const Workspace& W = r->wk;
  const Plan p = make_plan(c, batch, k);
  hipError_t e;
  ScreenArgs A{x, ids, gw, r->sigma, r->codes, r->scales, r->norms, r->rho, W.acc, nullptr, W.xrot,
               W.sel, r->status, c.hidden, c.n_experts, c.inter, c.top, r->ncp, r->nblk,
               c.n_screen, r->lp, r->unit, p.nd, p.ng, p.items1, p.per_xcd1, 0};
  if ((e = launch_screen(A, p, st)) != hipSuccess) return hip_fail(e, "screen launch");
  const SharedPlan sp = make_shared_plan(c, batch, k);
  if ((e = launch_shared_select(*r, x, ids, gw, batch, k, W, sp, st)) != hipSuccess)
    return hip_fail(e, "shared selection launch");
  ReduceArgs C{W.ypart, W.zpart, r->u, y, W.acc, c.hidden, sp.G, sp.Z, c.rank, r->ncp,
               c.hidden / kReduceSlice, 1, resid};
  if ((e = launch_reduce(C, batch, st)) != hipSuccess) return hip_fail(e, "reduce launch");
  const size_t nb = (size_t)batch * r->ncand;
  auto cp = [&](void* dst, const void* src, size_t bytes) -> hipError_t {
    return dst ? hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st) : hipSuccess;
  };
  if ((e = cp(bscore_out, W.bscore, sizeof(float) * nb)) != hipSuccess ||
      (e = cp(kept_out, W.klist, sizeof(int32_t) * k)) != hipSuccess ||
      (e = cp(meta_out, W.meta, sizeof(int32_t) * (1 + (size_t)batch * c.top))) != hipSuccess)
    return hip_fail(e, "debug copy");
  return CFR_OK;
}

int launch_dense(cfr_reader* r, const float* x, const int32_t* ids, const float* gw, int batch,
                 float* y, hipStream_t st, const float* resid) {
  const cfr_config& c = r->cfg;
  const DensePlan p = make_dense_plan(c, batch);
  const Workspace& W = r->wk;
  hipError_t e;
  if ((e = launch_dense_block(x, ids, gw, r->w3, W.ypart, r->status, c, batch, p, st)) != hipSuccess)
    return hip_fail(e, "dense launch");
  ReduceArgs C{W.ypart, W.zpart, r->u, y, W.acc, c.hidden, p.G, 0, c.rank, r->ncp,
               c.hidden / kReduceSlice, 0, resid};
  if ((e = launch_reduce(C, batch, st)) != hipSuccess) return hip_fail(e, "dense reduce launch");
  return CFR_OK;
}

}  // namespace cfr

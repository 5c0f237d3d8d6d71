// Decode kernels of the channel-selection reader for gfx950 (CDNA4, wave64).
//
// Per token and layer ([zh §方法步骤详情] decode steps (1)-(4); [zh §核心方法];
// [ko §어떻게 쓰나]; zh/ko = the Chinese/Korean summary pages of "Channel
// Selection for Mixture-of-Experts Decoding Needs No Calibration Data"), three
// kernels separated by the only two global dependencies of the method:
//
//   A  k_screen_score   rotate x (float32 butterfly, H_128 sigma x per block),
//                       pick the n_screen coordinates of largest |v| per block
//                       (LDS radix select), read the codes of those coordinates
//                       for a slice of channels of one routed expert, and emit
//                       g_hat, v_hat, p = silu(g_hat) v_hat and the output-unit
//                       score s = w ||d|| |p| of every channel in the slice.
//   B  k_select_exact   every workgroup finds the exact top-k threshold of its
//                       token from all scores (radix select, ties to the lower
//                       candidate index), takes its share of the kept channels,
//                       computes a_j = silu(g_j.x)(v_j.x) from the native BF16
//                       rows and w a_j, and a partial recovery vector
//                       z = sum over its skipped candidates of w p b.
//   C  k_down_recover   per hidden slice: y = sum over kept of (w a_j) d_j
//                       (transposed down rows) + U z.
//
// Each workgroup of A owns whole channels (all blocks, all screened
// coordinates), so no partial sums cross workgroups before the top-k.
// Cross-workgroup handoff goes through kernel boundaries: on MI355X a kernel
// boundary costs less than an in-kernel grid barrier, whose agent-scope
// release has to write back every XCD's L2.
//
// Workgroups are mapped XCD-aware: dispatch places workgroup i on XCD i % 8,
// so work item (i % 8) * per_xcd + i / 8 gives each XCD a contiguous range of
// items.  In A that puts all slices of one routed expert on one XCD (its L2
// then fetches each 32-byte sector of a sketch unit once); in C adjacent
// hidden slices of a row land in the same L2.  The mapping only affects
// performance, never correctness.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace cfr {

namespace {

constexpr float kInvSqrt128f = 0.08838834764831845f;  // 1/sqrt(128) rounded to float
constexpr int kThreads = 256;
constexpr int kMaxS1024 = 8;  // widest slice that still fits 128 VGPRs at 1024 threads
constexpr int kMaxS = 13;  // bytes per half handled by one screen workgroup

__device__ __forceinline__ float f16f(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ int clamp_expert(int e, int E, int32_t* status) {
  if (e < 0 || e >= E) {
    atomicOr(status, 1);
    e = e < 0 ? 0 : E - 1;
  }
  return e;
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

// Inclusive prefix sum over a 256-thread block (4 waves) with one barrier;
// sh (4 ints) must not be written again before the caller's next barrier.
__device__ __forceinline__ int block_scan_256(int v, int* sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_scan(v);
  if (lane == 63) sh[w] = v;
  __syncthreads();
  int add = 0;
  for (int q = 0; q < w; ++q) add += sh[q];
  return v + add;
}

__device__ __forceinline__ int xcd_item(int id, int per_xcd) {
  return (id & 7) * per_xcd + (id >> 3);
}

}  // namespace

// ===========================================================================
// A: rotate + select + screen + score
// ===========================================================================
struct ScreenArgs {
  const float* x;
  const int32_t* ids;
  const float* gw;
  const float* sigma;
  const uint8_t* codes;
  const uint16_t* scales;
  const float* norms;
  float* xrot;
  uint8_t* sel;
  float* ghat;
  float* vhat;
  float* pact;
  float* score;
  int32_t* status;
  int H, E, I, top, nblk, n_screen, lp, unit, n_slices, items, per_xcd, dbg;
};

// One wave rotates and screens one 128-block held as two values per lane
// (lane l holds coordinates l and l + 64).  The float32 butterfly runs the
// stages h = 1 .. 32 across lanes and h = 64 inside the lane, in that order,
// with the lower element of each pair taking a + b and the upper a - b.
// The n_screen largest |v| (ties to the lower index) are found by a
// bit-by-bit search of the n_screen-th largest magnitude over wave ballots,
// then compacted in ascending coordinate order.
__device__ __forceinline__ void rotate_select_block(float v0, float v1, int b, int NS,
                                                    uint8_t* sl, int2* rec, int unit,
                                                    float* xrot_out) {
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
  if (s0) {
    const int pos = __popcll(m0 & lt);
    if (pos < NS) {
      sl[b * NS + pos] = (uint8_t)lane;
      rec[b * NS + pos] = make_int2(lane * unit, __float_as_int(v0));
    }
  }
  if (s1) {
    const int pos = __popcll(m0) + __popcll(m1 & lt);
    if (pos < NS) {
      sl[b * NS + pos] = (uint8_t)(lane + 64);
      rec[b * NS + pos] = make_int2((lane + 64) * unit, __float_as_int(v1));
    }
  }
}

template <int S, int NT>
__global__ __launch_bounds__(NT) void k_screen_score(ScreenArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int item = xcd_item(blockIdx.x, a.per_xcd);
  if (item >= a.items) return;
  const int c = item % a.n_slices;
  const int ts = item / a.n_slices;
  const int s = ts % a.top, t = ts / a.top;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int NW = NT / 64;
  const int H = a.H, I = a.I, nblk = a.nblk, NS = a.n_screen;
  constexpr int NCH = 5 * S;  // channels per half in this slice
  const ScreenLds L(nblk, NS, S, NT);
  uint4* lut = reinterpret_cast<uint4*>(smem + L.lut);
  uint8_t* sl = smem + L.sl;
  int2* rec = reinterpret_cast<int2*>(smem + L.rec);  // (unit byte offset, x bits) per screened coordinate
  float* sc = reinterpret_cast<float*>(smem + L.sc);
  float* red = reinterpret_cast<float*>(smem + L.red);

  // token and signs of this wave's first blocks: independent of the routing
  const float* xt = a.x + (size_t)t * H;
  float xv0[4], xv1[4], sg0[4], sg1[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {  // clamped addresses: every load is issued, none waits
    const int b = min(wave + u * NW, nblk - 1);
    xv0[u] = xt[b * 128 + lane];
    xv1[u] = xt[b * 128 + 64 + lane];
    sg0[u] = a.sigma[b * 128 + lane];
    sg1[u] = a.sigma[b * 128 + 64 + lane];
  }
  const int e = clamp_expert(a.ids[t * a.top + s], a.E, a.status);
  const float wgt = a.gw[t * a.top + s];
  const int b0 = c * S;   // first byte of the slice inside each half
  const int j0 = 5 * b0;  // first channel of the slice

  // scales of the slice for every block and half: the first batch is
  // loaded now and stored after the rotation, so its latency hides there
  const int nsc = nblk * 2 * NCH;
  uint16_t hv[4];
  auto load_scales = [&](int q0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = q0 + tid + u * NT;
      const int jj = q % NCH, bm = q / NCH;  // bm = block * 2 + half
      const int j = j0 + jj;
      const bool ok = q < nsc && j < I;
      const size_t ix = ok ? ((size_t)e * nblk + (bm >> 1)) * 2 * I + (bm & 1) * I + j : 0;
      hv[u] = a.scales[ix];
      hv[u] = ok ? hv[u] : (uint16_t)0;
    }
  };
  auto store_scales = [&](int q0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = q0 + tid + u * NT;
      if (q < nsc) sc[q] = f16f(hv[u]);
    }
  };
  load_scales(0);
  float nrm = 0.f;
  if (tid < NCH && j0 + tid < I) nrm = a.norms[(size_t)e * I + j0 + tid];

  // code table: byte q -> its five codes c_t = digit_t - 1 as fp16 (entries
  // 243..255 never occur in a packed unit and decode to zero)
  if (tid < 256) {  // NT >= 512
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

  // ---- decode step (1): rotation and the partial-screen coordinates ----
  const bool writer = a.dbg && c == 0 && s == 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int b = wave + u * NW;
    if (b < nblk)
      rotate_select_block(xv0[u] * sg0[u], xv1[u] * sg1[u], b, NS, sl, rec, a.unit,
                          writer ? a.xrot + (size_t)t * H + b * 128 : nullptr);
  }
  for (int b = wave + 4 * NW; b < nblk; b += NW) {  // hidden above 4096
    const float v0 = xt[b * 128 + lane] * a.sigma[b * 128 + lane];
    const float v1 = xt[b * 128 + 64 + lane] * a.sigma[b * 128 + 64 + lane];
    rotate_select_block(v0, v1, b, NS, sl, rec, a.unit,
                        writer ? a.xrot + (size_t)t * H + b * 128 : nullptr);
  }
  __syncthreads();
  store_scales(0);
  for (int q0 = NT * 4; q0 < nsc; q0 += NT * 4) {  // large layers only
    load_scales(q0);
    store_scales(q0);
  }
  __syncthreads();
  if (writer)
    for (int q = tid; q < nblk * NS; q += NT) a.sel[(size_t)t * nblk * NS + q] = sl[q];

  // ---- screen: codes of the slice at the screened coordinates ----
  // group g = (block, half) with tpg threads; each thread takes every
  // tpg-th screened coordinate of its block.
  const int groups = 2 * nblk;
  int tpg = 1;
  while (tpg * 2 * groups <= NT) tpg *= 2;
  const int g = tid / tpg, lg = tid % tpg;
  float acc[NCH];
#pragma unroll
  for (int q = 0; q < NCH; ++q) acc[q] = 0.f;
  const int nbytes = (I + 4) / 5;
  const int nb_slice = min(S, nbytes - b0);  // bytes of this slice inside a half
  if (g < groups) {
    const int b = g >> 1, m = g & 1;
    const uint8_t* ubase = a.codes + ((size_t)e * nblk + b) * 128 * a.unit + m * a.lp + (b0 & ~3);
    const int sh = (b0 & 3) * 8;
    constexpr int ND = (S + 6) / 4;  // dwords covering S bytes at any 4-byte phase
    constexpr int CB = 5;            // coordinates whose codes are in flight together
    for (int q0 = lg; q0 < NS; q0 += tpg * CB) {
      // all records first, then all code loads: one LDS and one memory latency per batch
      int2 rc[CB];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const int q = q0 + u * tpg;
        rc[u] = rec[b * NS + (q < NS ? q : NS - 1)];
      }
      uint32_t w[CB][ND];
      float xv[CB];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const uint32_t* wp = reinterpret_cast<const uint32_t*>(ubase + rc[u].x);
#pragma unroll
        for (int d = 0; d < ND; ++d) w[u][d] = wp[d];
        xv[u] = q0 + u * tpg < NS ? __int_as_float(rc[u].y) : 0.f;  // past the list: x = 0
      }
#pragma unroll
      for (int u = 0; u < CB; ++u) {
#pragma unroll
        for (int k = 0; k < S; ++k) {
          const int bit = sh + 8 * k;
          const int wi = bit >> 5, bo = bit & 31;
          const uint32_t byte = wi < ND ? (w[u][wi < ND ? wi : 0] >> bo) & 0xFFu : 121u;
          if (k < nb_slice) {
            const uint4 cw = lut[byte];
            const uint32_t hw[3] = {cw.x, cw.y, cw.z};
#pragma unroll
            for (int d = 0; d < 5; ++d) {
              const uint16_t hb = (uint16_t)(hw[d >> 1] >> ((d & 1) * 16));
              acc[5 * k + d] = fmaf((float)__builtin_bit_cast(_Float16, hb), xv[u], acc[5 * k + d]);
            }
          }
        }
      }
    }
  }
  if (g < groups) {
#pragma unroll
    for (int q = 0; q < NCH; ++q) red[(size_t)tid * NCH + q] = acc[q];
  }
  __syncthreads();
  if (g < groups)
    for (int jj = lg; jj < NCH; jj += tpg) {
      float v = 0.f;
      for (int l = 0; l < tpg; ++l) v += red[(size_t)(g * tpg + l) * NCH + jj];
      sc[g * NCH + jj] *= v;  // alpha_b * sum over screened coordinates
    }
  __syncthreads();
  if (tid < NCH && j0 + tid < I) {
    float gs = 0.f, vs = 0.f;
    for (int b = 0; b < nblk; ++b) {
      gs += sc[(2 * b) * NCH + tid];
      vs += sc[(2 * b + 1) * NCH + tid];
    }
    gs *= kInvSqrt128f;
    vs *= kInvSqrt128f;
    const float p = silu(gs) * vs;
    const size_t o = (size_t)t * a.top * I + (size_t)s * I + j0 + tid;
    a.ghat[o] = gs;
    a.vhat[o] = vs;
    a.pact[o] = p;
    a.score[o] = fabsf(wgt) * nrm * fabsf(p);  // routing weights are non-negative; |w| keeps the sign bit clear
  }
}

// ===========================================================================
// B: exact top-k (redundant per workgroup) + exact kept channels + recovery z
// ===========================================================================
struct SelectArgs {
  const float* x;
  const int32_t* ids;
  const float* gw;
  const uint16_t* w3;
  const uint16_t* bmat;
  const float* score;
  const float* pact;
  int32_t* kept;
  int32_t* rowidx;
  float* coef;
  float* zpart;
  int32_t* status;
  int H, E, I, top, ncand, k, rank, G, share_max, ZW;
  int dense;  // 1: every candidate is kept (the dense baseline); scores unused
};

template <int KPT>
__global__ __launch_bounds__(kThreads) void k_select_exact(SelectArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int t = blockIdx.x / a.G, w = blockIdx.x % a.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, I = a.I, nc = a.ncand, k = a.k;
  const SelectLds L(H, nc, a.share_max, a.rank);
  float* xs = reinterpret_cast<float*>(smem + L.xs);
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem + L.keys);
  uint8_t* flags = smem + L.flags;
  int* list = reinterpret_cast<int*>(smem + L.list);
  float* zred = reinterpret_cast<float*>(smem + L.zred);
  int* hist = reinterpret_cast<int*>(smem + L.hist);  // 4096 bins, then 2 x 1024 bins
  int* hist1 = hist + 4096;
  int* hist2 = hist1 + 1024;
  int* misc = reinterpret_cast<int*>(smem + L.misc);
  // misc: [0..3] [4..7] [12..15] scan scratch, [8] digit [9] need [10] bin count,
  // [11] gather slot, [16] [17] boundary key and count, [20..35] routed expert
  // of each slot, [36..51] its weight; bkey/bidx: the boundary bin's elements
  int* sl_e = misc + 20;
  float* sl_w = reinterpret_cast<float*>(misc + 36);
  uint32_t* bkey = reinterpret_cast<uint32_t*>(misc + 64);
  int* bidx = misc + 128;

  const bool partial = !a.dense && k > 0 && k < nc;
  const bool all = a.dense || k == nc;
  const int per = (nc + kThreads - 1) / kThreads;  // candidates per thread (uniform)
  // loads first, all issued before any is consumed: routing of the token,
  // the token itself, its scores
  const int tsl = min(tid, a.top - 1);
  const int id_raw = a.ids[t * a.top + tsl];
  const float gw_raw = a.gw[t * a.top + tsl];
  const float* xt = a.x + (size_t)t * H;
  {
    // four named registers rather than an array: the array form ends up on
    // the stack once its stores sit below the score loads
    const int xq0 = min(tid * 4, H - 4), xq1 = min((tid + kThreads) * 4, H - 4);
    const int xq2 = min((tid + 2 * kThreads) * 4, H - 4), xq3 = min((tid + 3 * kThreads) * 4, H - 4);
    const float4 xr0 = *reinterpret_cast<const float4*>(xt + xq0);
    const float4 xr1 = *reinterpret_cast<const float4*>(xt + xq1);
    const float4 xr2 = *reinterpret_cast<const float4*>(xt + xq2);
    const float4 xr3 = *reinterpret_cast<const float4*>(xt + xq3);
    // all KPT score loads are issued unguarded (clamped addresses) and only
    // consumed after the token's stores, so one memory latency covers them
    float v[KPT];
    if (partial) {
      const float* sct = a.score + (size_t)t * nc;
#pragma unroll
      for (int u = 0; u < KPT; ++u) v[u] = sct[min(tid + u * kThreads, nc - 1)];
    }
    if (tid < a.top) {
      sl_e[tid] = clamp_expert(id_raw, a.E, a.status);
      sl_w[tid] = gw_raw;
    }
    // clamped like the loads: duplicate addresses store equal values
    *reinterpret_cast<float4*>(xs + xq0) = xr0;
    *reinterpret_cast<float4*>(xs + xq1) = xr1;
    *reinterpret_cast<float4*>(xs + xq2) = xr2;
    *reinterpret_cast<float4*>(xs + xq3) = xr3;
    for (int q = (tid + 4 * kThreads) * 4; q < H; q += kThreads * 4)  // hidden above 4096
      *reinterpret_cast<float4*>(xs + q) = *reinterpret_cast<const float4*>(xt + q);
    if (partial) {
      // keys padded to 256 * per entries; padding keys are 0, the smallest key,
      // and sit at the highest indices, so the tie rule never keeps them
#pragma unroll
      for (int u = 0; u < KPT; ++u)
        if (u < per) keys[tid + u * kThreads] = tid + u * kThreads < nc ? __float_as_uint(v[u]) : 0u;
#pragma unroll
      for (int q = 0; q < 16; ++q) hist[tid * 16 + q] = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) hist1[tid * 8 + q] = 0;  // both 1024-bin histograms
      if (tid == 0) misc[11] = 0;
    }
  }
  __syncthreads();
  // each thread owns a contiguous chunk of `per` (<= KPT) candidates, in
  // registers; `per` is uniform, so every guard below is a scalar branch
  const int lo = tid * per;
  const int nreal = max(0, min(per, nc - lo));  // real candidates of this chunk
  uint32_t kr[KPT];
#pragma unroll
  for (int q = 0; q < KPT; ++q) kr[q] = (partial && q < per) ? keys[lo + q] : 0u;
  uint32_t prefix = 0, mask = 0;
  int need = k;
  if (partial) {
    // exact k-th largest key.  Scores are non-negative, so bits 30..19
    // (exponent and 4 mantissa bits) order them; one pass over those 12 bits
    // finds the boundary bin; a bin of at most 64 keys is then ranked
    // directly, a larger one (many near-equal scores) is refined by two more
    // passes over bits 18..9 and 8..0.
#pragma unroll
    for (int q = 0; q < KPT; ++q)
      if (q < per) atomicAdd(&hist[(kr[q] >> 19) & 0xFFFu], 1);
    __syncthreads();
    {
      const int base = 16 * (255 - tid);  // thread tid holds bins [base, base + 16), descending digits
      int bins[16], own = 0;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const uint4 hq = *reinterpret_cast<const uint4*>(hist + base + 4 * q4);
        bins[4 * q4] = (int)hq.x;
        bins[4 * q4 + 1] = (int)hq.y;
        bins[4 * q4 + 2] = (int)hq.z;
        bins[4 * q4 + 3] = (int)hq.w;
        own += (int)(hq.x + hq.y + hq.z + hq.w);
      }
      const int incl = block_scan_256(own, misc);
      if (incl >= need && incl - own < need) {
        int cum = incl - own;
#pragma unroll
        for (int q = 15; q >= 0; --q) {
          if (cum < need && cum + bins[q] >= need) {
            misc[8] = base + q;
            misc[9] = need - cum;
            misc[10] = bins[q];
          }
          cum += bins[q];
        }
      }
    }
    __syncthreads();
    prefix = (uint32_t)misc[8] << 19;
    mask = 0x7FF80000u;
    need = misc[9];
    const int cb = misc[10];
    if (cb != need && cb <= 64) {
      // rank the boundary bin's keys directly (key descending, index ascending)
#pragma unroll
      for (int q = 0; q < KPT; ++q)
        if (q < per && (kr[q] & mask) == prefix) {
          const int slot = atomicAdd(&misc[11], 1);
          bkey[slot] = kr[q];
          bidx[slot] = lo + q;
        }
      __syncthreads();
      if (tid < cb) {
        const uint32_t ki = bkey[tid];
        const int ii = bidx[tid];
        int gt = 0, eqb = 0;
        for (int jx = 0; jx < cb; ++jx) {
          const uint32_t kj = bkey[jx];
          gt += kj > ki;
          eqb += kj == ki && bidx[jx] < ii;
        }
        if (gt + eqb == need - 1) {
          misc[16] = (int)ki;
          misc[17] = need - gt;
        }
      }
      __syncthreads();
      prefix = (uint32_t)misc[16];
      mask = 0xFFFFFFFFu;
      need = misc[17];
    } else if (cb != need) {
      for (int pass = 1; pass < 3; ++pass) {  // bits 18..9, then 8..0
        const int shift = pass == 1 ? 9 : 0;
        const uint32_t dm = pass == 1 ? 0x3FFu : 0x1FFu;
        int* hcur = pass == 1 ? hist1 : hist2;
#pragma unroll
        for (int q = 0; q < KPT; ++q)
          if (q < per && (kr[q] & mask) == prefix) atomicAdd(&hcur[(kr[q] >> shift) & dm], 1);
        __syncthreads();
        const int base = 4 * (255 - tid);
        const uint4 hq = *reinterpret_cast<const uint4*>(hcur + base);
        const int bins[4] = {(int)hq.x, (int)hq.y, (int)hq.z, (int)hq.w};
        const int own = bins[0] + bins[1] + bins[2] + bins[3];
        const int incl = block_scan_256(own, misc + (pass == 1 ? 4 : 12));
        if (incl >= need && incl - own < need) {
          int cum = incl - own;
#pragma unroll
          for (int q = 3; q >= 0; --q) {
            if (cum < need && cum + bins[q] >= need) {
              misc[8] = base + q;
              misc[9] = need - cum;
            }
            cum += bins[q];
          }
        }
        __syncthreads();
        prefix |= (uint32_t)misc[8] << shift;
        mask |= dm << shift;
        need = misc[9];
        __syncthreads();
      }
      mask = 0xFFFFFFFFu;  // bit 31 is clear in every key
    }
  }
  // kept flags and ranks in ascending candidate order
  int ngt = 0, neq = 0;
  if (partial)
#pragma unroll
    for (int q = 0; q < KPT; ++q)
      if (q < per) {
        const uint32_t kv = kr[q] & mask;
        ngt += kv > prefix;
        neq += kv == prefix;
      }
  __syncthreads();
  const int eq_incl = block_scan_256(neq, misc);  // scratch [0..3]
  const int eq_before = eq_incl - neq;
  int take_eq = 0;
  if (partial) take_eq = max(0, min(neq, need - eq_before));
  const int mine = partial ? ngt + take_eq : (all ? nreal : 0);
  const int pos_incl = block_scan_256(mine, misc + 4);  // scratch [4..7]
  int rnk = pos_incl - mine;
  const int share = (k + a.G - 1) / a.G;
  const int r0 = min(w * share, k), r1 = min(r0 + share, k);
  if (partial) {
    int eq_seen = 0;
#pragma unroll
    for (int q = 0; q < KPT; ++q)
      if (q < per) {
        const uint32_t kv = kr[q] & mask;
        const bool eq = kv == prefix;
        const bool on = kv > prefix || (eq && eq_seen < take_eq);
        eq_seen += eq;
        flags[lo + q] = on;
        if (on && rnk >= r0 && rnk < r1) list[rnk - r0] = lo + q;
        rnk += on;
      }
  } else {
    for (int q = 0; q < per; ++q) {
      const bool on = all && q < nreal;
      flags[lo + q] = on;
      if (on && rnk >= r0 && rnk < r1) list[rnk - r0] = lo + q;
      rnk += on;
    }
  }
  __syncthreads();

  // ---- decode step (3): exact kept channels from native BF16 rows ----
  // one kept channel per wave; all of its gate and up loads in flight together
  for (int q = wave; q < r1 - r0; q += 4) {
    const int cnd = list[q];
    const int sl = cnd / I, j = cnd % I;
    const size_t row = (size_t)sl_e[sl] * I + j;
    const uint16_t* gr = a.w3 + row * 3 * H;
    float gsum = 0.f, vsum = 0.f;
    for (int hb = 0; hb < H; hb += 512 * 8) {
      uint4 gq[8], vq[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int h = min(hb + u * 512 + lane * 8, H - 8);  // clamped; the tail is skipped below
        gq[u] = *reinterpret_cast<const uint4*>(gr + h);
        vq[u] = *reinterpret_cast<const uint4*>(gr + H + h);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int h = hb + u * 512 + lane * 8;
        if (h < H) {
          const float4 x0 = *reinterpret_cast<const float4*>(xs + h);
          const float4 x1 = *reinterpret_cast<const float4*>(xs + h + 4);
          gsum = fmaf(__uint_as_float(gq[u].x << 16), x0.x, gsum);
          gsum = fmaf(__uint_as_float(gq[u].x & 0xFFFF0000u), x0.y, gsum);
          gsum = fmaf(__uint_as_float(gq[u].y << 16), x0.z, gsum);
          gsum = fmaf(__uint_as_float(gq[u].y & 0xFFFF0000u), x0.w, gsum);
          gsum = fmaf(__uint_as_float(gq[u].z << 16), x1.x, gsum);
          gsum = fmaf(__uint_as_float(gq[u].z & 0xFFFF0000u), x1.y, gsum);
          gsum = fmaf(__uint_as_float(gq[u].w << 16), x1.z, gsum);
          gsum = fmaf(__uint_as_float(gq[u].w & 0xFFFF0000u), x1.w, gsum);
          vsum = fmaf(__uint_as_float(vq[u].x << 16), x0.x, vsum);
          vsum = fmaf(__uint_as_float(vq[u].x & 0xFFFF0000u), x0.y, vsum);
          vsum = fmaf(__uint_as_float(vq[u].y << 16), x0.z, vsum);
          vsum = fmaf(__uint_as_float(vq[u].y & 0xFFFF0000u), x0.w, vsum);
          vsum = fmaf(__uint_as_float(vq[u].z << 16), x1.x, vsum);
          vsum = fmaf(__uint_as_float(vq[u].z & 0xFFFF0000u), x1.y, vsum);
          vsum = fmaf(__uint_as_float(vq[u].w << 16), x1.z, vsum);
          vsum = fmaf(__uint_as_float(vq[u].w & 0xFFFF0000u), x1.w, vsum);
        }
      }
    }
    gsum = wave_sum(gsum);
    vsum = wave_sum(vsum);
    if (lane == 0) {
      const size_t o = (size_t)t * nc + r0 + q;
      a.coef[o] = sl_w[sl] * silu(gsum) * vsum;
      a.rowidx[o] = (int32_t)row;
      a.kept[o] = cnd;
    }
  }

  // ---- decode step (4), first half: z over a range of skipped candidates ----
  // the first ZW workgroups of the token each take nc/ZW candidates; a
  // thread handles 8 coefficients (one uint4) of one candidate at a time
  if (a.rank > 0 && !all && w < a.ZW) {
    const int R = a.rank, R8 = R / 8;
    const int zper = (nc + a.ZW - 1) / a.ZW;
    const int c0 = min(w * zper, nc), c1 = min(c0 + zper, nc);
    const int cpp = kThreads / R8;  // candidates per pass
    const int cl = tid / R8, r8 = tid % R8;
    float zacc[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) zacc[d] = 0.f;
    if (cl < cpp)
      for (int cb = c0 + cl; cb < c1; cb += cpp * 4) {
        float cf[4];
        uint4 bq[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int cnd = cb + u * cpp;
          const int cc = cnd < c1 ? cnd : c1 - 1;  // clamped: loads always issued
          const int sl = cc / I, j = cc % I;
          const float pv = a.pact[(size_t)t * nc + cc];
          bq[u] = reinterpret_cast<const uint4*>(a.bmat + ((size_t)sl_e[sl] * I + j) * R)[r8];
          cf[u] = (cnd < c1 && !flags[cc]) ? sl_w[sl] * pv : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint32_t bw[4] = {bq[u].x, bq[u].y, bq[u].z, bq[u].w};
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            zacc[2 * d] = fmaf(cf[u], f16f((uint16_t)(bw[d] & 0xFFFFu)), zacc[2 * d]);
            zacc[2 * d + 1] = fmaf(cf[u], f16f((uint16_t)(bw[d] >> 16)), zacc[2 * d + 1]);
          }
        }
      }
    // reduce over candidates: lanes with equal r8 inside a wave, then waves
    for (int q = 0; q < R * 4; q += kThreads)
      if (q + tid < R * 4) zred[q + tid] = 0.f;
    __syncthreads();
    // lanes 0..R8-1 of each wave end with its sums when R8 is a power of two;
    // otherwise fall back to shared-memory atomics
    const bool pow2 = (R8 & (R8 - 1)) == 0;
    if (pow2) {
#pragma unroll
      for (int d = 0; d < 8; ++d) {  // butterfly over lanes of equal r8
        float v = zacc[d];
        if (R8 <= 1) v += xor_lane_f<1>(v);
        if (R8 <= 2) v += xor_lane_f<2>(v);
        if (R8 <= 4) v += xor_lane_f<4>(v);
        if (R8 <= 8) v += xor_lane_f<8>(v);
        v += xor_lane_f<16>(v);
        v += xor_lane_f<32>(v);
        zacc[d] = v;
      }
      if (lane < R8 && cl < cpp)
#pragma unroll
        for (int d = 0; d < 8; ++d) zred[wave * R + r8 * 8 + d] = zacc[d];
    } else if (cl < cpp) {
#pragma unroll
      for (int d = 0; d < 8; ++d) atomicAdd(&zred[r8 * 8 + d], zacc[d]);
    }
    __syncthreads();
    if (tid < R)
      a.zpart[((size_t)t * a.ZW + w) * R + tid] =
          pow2 ? zred[tid] + zred[R + tid] + zred[2 * R + tid] + zred[3 * R + tid] : zred[tid];
  }
}

// ===========================================================================
// C: y = sum over kept of (w a_j) d_j + U z, per hidden slice
// ===========================================================================
struct DownArgs {
  const uint16_t* w3;
  const uint16_t* U;
  const int32_t* rowidx;
  const float* coef;
  const float* zpart;
  float* y;
  int H, ncand, k, rank, nz, nhs, items, per_xcd;
};

template <int HS>
__global__ __launch_bounds__(kThreads) void k_down_recover(DownArgs a) {
  __shared__ float zl[16 * 64];
  __shared__ float zs[64];
  __shared__ float part[4][HS];
  const int item = xcd_item(blockIdx.x, a.per_xcd);
  if (item >= a.items) return;
  const int t = item / a.nhs, hs = item % a.nhs;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, h0 = hs * HS;
  // this slice's rows of U, needed last, loaded first (thread tid < HS owns hidden h0 + tid)
  uint4 uq[8];
  if (a.nz > 0) {
    const uint4* up = reinterpret_cast<const uint4*>(a.U + (size_t)(h0 + (tid < HS ? tid : 0)) * a.rank);
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) uq[r8] = up[r8 * 8 < a.rank ? r8 : 0];
  }
  const int nzv = a.nz * a.rank;  // at most 16 * 64 partial values
  {
    float zv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = tid + u * kThreads;
      zv[u] = nzv > 0 ? a.zpart[(size_t)t * nzv + (q < nzv ? q : nzv - 1)] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = tid + u * kThreads;
      if (q < nzv) zl[q] = zv[u];
    }
  }
  constexpr int RB = HS >= 64 ? 1 : 64 / HS;  // kept rows in flight per thread
  float acc[HS];
#pragma unroll
  for (int q = 0; q < HS; ++q) acc[q] = 0.f;
  const int32_t* ri = a.rowidx + (size_t)t * a.ncand;
  const float* cfp = a.coef + (size_t)t * a.ncand;
  for (int rb = tid; rb < a.k; rb += kThreads * RB) {
    int rows[RB];
    float cf[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) {  // clamped: every load is issued; extra ranks get weight 0
      const int r = rb + u * kThreads;
      const int rc = r < a.k ? r : a.k - 1;
      rows[u] = ri[rc];
      cf[u] = cfp[rc];
      cf[u] = r < a.k ? cf[u] : 0.f;
    }
    uint4 dv[RB][HS / 8];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const uint16_t* d = a.w3 + ((size_t)rows[u] * 3 + 2) * H + h0;
#pragma unroll
      for (int q = 0; q < HS / 8; ++q) dv[u][q] = *reinterpret_cast<const uint4*>(d + 8 * q);
    }
#pragma unroll
    for (int u = 0; u < RB; ++u)
#pragma unroll
      for (int q = 0; q < HS / 8; ++q) {
        const uint32_t dw[4] = {dv[u][q].x, dv[u][q].y, dv[u][q].z, dv[u][q].w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          acc[8 * q + 2 * p] = fmaf(cf[u], __uint_as_float(dw[p] << 16), acc[8 * q + 2 * p]);
          acc[8 * q + 2 * p + 1] = fmaf(cf[u], __uint_as_float(dw[p] & 0xFFFF0000u), acc[8 * q + 2 * p + 1]);
        }
      }
  }
#pragma unroll
  for (int q = 0; q < HS; ++q) acc[q] = wave_sum(acc[q]);
  if (lane == 0)
#pragma unroll
    for (int q = 0; q < HS; ++q) part[wave][q] = acc[q];
  __syncthreads();
  if (tid < 64) {
    float z = 0.f;
    if (tid < a.rank)
      for (int q = 0; q < a.nz; ++q) z += zl[q * a.rank + tid];
    zs[tid] = z;
  }
  __syncthreads();
  if (tid < HS) {
    const int h = h0 + tid;
    float v = part[0][tid] + part[1][tid] + part[2][tid] + part[3][tid];
    if (a.nz > 0) {
#pragma unroll
      for (int r8 = 0; r8 < 8; ++r8)
        if (r8 * 8 < a.rank) {
          const uint32_t uw[4] = {uq[r8].x, uq[r8].y, uq[r8].z, uq[r8].w};
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            v = fmaf(f16f((uint16_t)(uw[d] & 0xFFFFu)), zs[r8 * 8 + 2 * d], v);
            v = fmaf(f16f((uint16_t)(uw[d] >> 16)), zs[r8 * 8 + 2 * d + 1], v);
          }
        }
    }
    a.y[(size_t)t * H + h] = v;
  }
}

// ===========================================================================
// host side
// ===========================================================================
static int hip_fail(hipError_t e, const char* what) {
  return fail(CFR_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

Plan make_plan(const cfr_config& c, int batch, int k) {
  Plan p;
  const int nblk = c.hidden / kBlock, nbytes = (c.inter + 4) / 5, nc = c.top * c.inter;
  // A: about 32 slices per routed expert, i.e. one workgroup per CU at batch 1
  p.S = (nbytes + 31) / 32;
  if (p.S < 1) p.S = 1;
  if (p.S > kMaxS) p.S = kMaxS;
  p.n_slices = (nbytes + p.S - 1) / p.S;
  p.itemsA = batch * c.top * p.n_slices;
  p.per_xcdA = (p.itemsA + 7) / 8;
  p.ntA = 1024;
  p.ldsA = ScreenLds(nblk, c.n_screen, p.S, 1024).total;
  if (p.S > kMaxS1024 || p.ldsA > kMaxLds) {
    p.ntA = 512;
    p.ldsA = ScreenLds(nblk, c.n_screen, p.S, 512).total;
  }
  // B: workgroups per token; about one kept channel per wave at batch 1
  int g = 256 / batch;
  if (g < 4) g = 4;
  const int per4 = ((k > 0 ? k : 1) + 3) / 4;
  if (g > per4) g = per4 < 4 ? 4 : per4;
  p.G = g;
  p.share_max = (k + g - 1) / g;
  p.ZW = g < 16 ? g : 16;
  p.ldsB = SelectLds(c.hidden, nc, p.share_max, c.rank).total;
  // C: hidden slices per token (8..64 hidden units each)
  int hsl = 8;
  while ((long)batch * (c.hidden / hsl) > 512 && hsl < 64) hsl *= 2;
  p.HS = hsl;
  p.nhs = c.hidden / hsl;
  p.itemsC = batch * p.nhs;
  p.per_xcdC = (p.itemsC + 7) / 8;
  return p;
}

size_t max_lds_needed(const cfr_config& c) {
  size_t m = 0;
  for (int b = 1; b <= c.max_batch; ++b) {
    const Plan p = make_plan(c, b, c.top * c.inter);
    if (p.ldsA > m) m = p.ldsA;
    if (p.ldsB > m) m = p.ldsB;
  }
  return m;
}

size_t zpart_rows(const cfr_config& c) { return (size_t)c.max_batch * 16; }

template <int S, int NT>
static hipError_t launch_A_nt(const ScreenArgs& a, const Plan& p, hipStream_t st) {
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)k_screen_score<S, NT>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    attr = true;
  }
  k_screen_score<S, NT><<<8 * p.per_xcdA, NT, p.ldsA, st>>>(a);
  return hipGetLastError();
}

template <int S>
static hipError_t launch_A(const ScreenArgs& a, const Plan& p, hipStream_t st) {
  if constexpr (S <= kMaxS1024) {
    if (p.ntA == 1024) return launch_A_nt<S, 1024>(a, p, st);
  }
  return launch_A_nt<S, 512>(a, p, st);
}

template <int HS>
static hipError_t launch_C(const DownArgs& a, const Plan& p, hipStream_t st) {
  k_down_recover<HS><<<8 * p.per_xcdC, kThreads, 0, st>>>(a);
  return hipGetLastError();
}

static hipError_t launch_C_any(const DownArgs& a, const Plan& p, hipStream_t st) {
  switch (p.HS) {
    case 8: return launch_C<8>(a, p, st);
    case 16: return launch_C<16>(a, p, st);
    case 32: return launch_C<32>(a, p, st);
    default: return launch_C<64>(a, p, st);
  }
}

template <int KPT>
static hipError_t launch_B_k(const SelectArgs& a, const Plan& p, int batch, hipStream_t st) {
  static bool attr = false;
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)k_select_exact<KPT>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, kMaxLds);
    attr = true;
  }
  k_select_exact<KPT><<<batch * p.G, kThreads, p.ldsB, st>>>(a);
  return hipGetLastError();
}

static hipError_t launch_B(const SelectArgs& a, const Plan& p, int batch, hipStream_t st) {
  const int per = a.dense ? 1 : (a.ncand + kThreads - 1) / kThreads;
  if (per <= 1) return launch_B_k<1>(a, p, batch, st);
  if (per <= 4) return launch_B_k<4>(a, p, batch, st);
  if (per <= 16) return launch_B_k<16>(a, p, batch, st);
  if (per <= 32) return launch_B_k<32>(a, p, batch, st);
  return launch_B_k<64>(a, p, batch, st);
}

int launch_decode(cfr_reader* r, const float* x, const int32_t* ids, const float* gw, int batch,
                  int k, float* y, hipStream_t st, const DebugOut* dbg, hipEvent_t* ev) {
  const cfr_config& c = r->cfg;
  const Plan p = make_plan(c, batch, k);
  auto mark = [&](int i) {
    if (ev) (void)hipEventRecord(ev[i], st);
  };
  ScreenArgs A{x, ids, gw, r->sigma, r->codes, r->scales, r->norms, r->xrot, r->sel, r->ghat,
               r->vhat, r->pact, r->score, r->status, c.hidden, c.n_experts, c.inter, c.top,
               r->nblk, c.n_screen, r->lp, r->unit, p.n_slices, p.itemsA, p.per_xcdA,
               dbg != nullptr};
  hipError_t e = hipSuccess;
  mark(0);
  switch (p.S) {
#define CFR_CASE(v) \
  case v:           \
    e = launch_A<v>(A, p, st); \
    break;
    CFR_CASE(1) CFR_CASE(2) CFR_CASE(3) CFR_CASE(4) CFR_CASE(5) CFR_CASE(6) CFR_CASE(7)
    CFR_CASE(8) CFR_CASE(9) CFR_CASE(10) CFR_CASE(11) CFR_CASE(12) CFR_CASE(13)
#undef CFR_CASE
    default:
      return fail(CFR_EUNSUPPORTED, "screen slice width");
  }
  if (e != hipSuccess) return hip_fail(e, "screen launch");
  mark(1);
  SelectArgs B{x, ids, gw, r->w3, r->b, r->score, r->pact, r->kept, r->rowidx, r->coef,
               r->zpart, r->status, c.hidden, c.n_experts, c.inter, c.top, r->ncand, k,
               c.rank, p.G, p.share_max, p.ZW, 0};
  if ((e = launch_B(B, p, batch, st)) != hipSuccess) return hip_fail(e, "select launch");
  mark(2);
  const int nz = (c.rank > 0 && k < r->ncand) ? p.ZW : 0;
  DownArgs C{r->w3, r->u, r->rowidx, r->coef, r->zpart, y, c.hidden, r->ncand, k,
             c.rank, nz, p.nhs, p.itemsC, p.per_xcdC};
  if ((e = launch_C_any(C, p, st)) != hipSuccess) return hip_fail(e, "down launch");
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
  Plan p = make_plan(c, batch, nc);
  // the dense block keeps every candidate: one wave per channel
  p.G = (nc + 3) / 4;
  p.share_max = 4;
  p.ldsB = SelectLds(c.hidden, nc, p.share_max, 0).total;
  SelectArgs B{x, ids, gw, r->w3, r->b, r->score, r->pact, r->kept, r->rowidx, r->coef,
               r->zpart, r->status, c.hidden, c.n_experts, c.inter, c.top, nc, nc, 0, p.G,
               p.share_max, 0, 1};
  hipError_t e;
  if ((e = launch_B(B, p, batch, st)) != hipSuccess) return hip_fail(e, "dense launch");
  DownArgs C{r->w3, r->u, r->rowidx, r->coef, r->zpart, y, c.hidden, nc, nc, 0, 0,
             p.nhs, p.itemsC, p.per_xcdC};
  if ((e = launch_C_any(C, p, st)) != hipSuccess) return hip_fail(e, "dense down launch");
  return CFR_OK;
}

}  // namespace cfr

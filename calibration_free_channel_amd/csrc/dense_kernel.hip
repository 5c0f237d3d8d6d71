// Dense BF16 routed-expert block for gfx950: the baseline the reader is
// measured against, and the k = all limit of its exact part.
//
// For each token and each channel j of its routed experts (gated MLP of the
// MoE layer, [zh §前置知识 / Mixture-of-Experts (MoE)]; zh = the Chinese
// summary page of "Channel Selection for Mixture-of-Experts Decoding Needs No
// Calibration Data"): a_j = silu(g_j . x)(v_j . x), y = sum_j w_j a_j d_j.
//
// The block is a pure HBM stream: every routed channel's gate, up and
// (transposed) down rows are read once, 3 H BF16 values that lie next to each
// other in the [E][I][3][H] layout.  One launch of G workgroups per token,
// each over a contiguous range of the token's top * inter channels; a wave
// takes its channels U at a time with every row of the U in flight together
// (one memory latency per U channels; the CU's other waves hide it), and the
// workgroup writes its partial output.  The reduce kernel of the decode sums
// the G partials (and adds the residual when asked).
#include <hip/hip_runtime.h>

#include "device_util.h"
#include "kernels.h"

namespace cfr {

namespace {

struct DenseArgs {
  const float* x;       // [B][H]
  const int32_t* ids;   // [B][top]
  const float* gw;      // [B][top]
  const uint16_t* w3;   // [E][I][3][H] bf16
  float* ypart;         // [B][G][H]
  int32_t* status;
  int H, E, I, top, nc, G, chan, cpw;
};

constexpr int kDenseThreads = 512;
constexpr int kDenseWaves = kDenseThreads / 64;

// NCH: 512-wide chunks covering a row (H <= 512 NCH); U: channels a wave has
// in flight at once.
template <int NCH, int U>
__global__ __launch_bounds__(kDenseThreads) void k_dense(DenseArgs a) {
  extern __shared__ float4 dense_lds[];
  float* xs = reinterpret_cast<float*>(dense_lds);  // [H]
  float* yred = xs + a.H;                           // [NW / 2][H]
  __shared__ int sl_e[kMaxTop];
  __shared__ float sl_w[kMaxTop];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x / a.G, w = blockIdx.x - t * a.G;
  const int H = a.H, I = a.I;
  for (int h = tid * 4; h < H; h += kDenseThreads * 4)
    *reinterpret_cast<float4*>(xs + h) = *reinterpret_cast<const float4*>(a.x + (size_t)t * H + h);
  if (tid < a.top) {
    sl_e[tid] = clamp_expert(a.ids[t * a.top + tid], a.E, a.status);
    sl_w[tid] = a.gw[t * a.top + tid];
  }
  lds_barrier();

  const int c0 = w * a.chan, c1 = min(a.nc, c0 + a.chan);
  const int q0 = c0 + wave * a.cpw, q1 = min(c1, q0 + a.cpw);
  float yv[NCH][8];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
    for (int i = 0; i < 8; ++i) yv[ch][i] = 0.f;

  for (int q = q0; q < q1; q += U) {
    uint4 gq[U][NCH], uq[U][NCH], dq[U][NCH];
    int sr[U];
    // every row of the U channels issued before any is used; a channel past
    // the wave's range re-reads the last one and gets coefficient 0
#pragma unroll
    for (int r = 0; r < U; ++r) {
      const int cc = min(q + r, q1 - 1);
      sr[r] = cc / I;
      const uint16_t* row = a.w3 + ((size_t)sl_e[sr[r]] * I + (cc - sr[r] * I)) * 3 * H;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const int h = min(ch * 512 + lane * 8, H - 8);  // clamped; the tail is masked below
        gq[r][ch] = *reinterpret_cast<const uint4*>(row + h);
        uq[r][ch] = *reinterpret_cast<const uint4*>(row + H + h);
        dq[r][ch] = *reinterpret_cast<const uint4*>(row + 2 * H + h);
      }
    }
    float gs[U], vs[U];
#pragma unroll
    for (int r = 0; r < U; ++r) gs[r] = vs[r] = 0.f;
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const int h = ch * 512 + lane * 8;
      if (h < H) {
        const float4 xa = *reinterpret_cast<const float4*>(xs + h);
        const float4 xb = *reinterpret_cast<const float4*>(xs + h + 4);
        const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
        for (int r = 0; r < U; ++r) {
          const uint32_t g4[4] = {gq[r][ch].x, gq[r][ch].y, gq[r][ch].z, gq[r][ch].w};
          const uint32_t u4[4] = {uq[r][ch].x, uq[r][ch].y, uq[r][ch].z, uq[r][ch].w};
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            gs[r] = fmaf(bf_lo(g4[p]), xv[2 * p], gs[r]);
            gs[r] = fmaf(bf_hi(g4[p]), xv[2 * p + 1], gs[r]);
            vs[r] = fmaf(bf_lo(u4[p]), xv[2 * p], vs[r]);
            vs[r] = fmaf(bf_hi(u4[p]), xv[2 * p + 1], vs[r]);
          }
        }
      }
    }
    float cf[U];
#pragma unroll
    for (int r = 0; r < U; ++r) {
      const float c = sl_w[sr[r]] * silu(wave_sum(gs[r])) * wave_sum(vs[r]);
      cf[r] = q + r < q1 ? c : 0.f;
    }
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
      for (int r = 0; r < U; ++r) {
        const uint32_t d4[4] = {dq[r][ch].x, dq[r][ch].y, dq[r][ch].z, dq[r][ch].w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          yv[ch][2 * p] = fmaf(cf[r], bf_lo(d4[p]), yv[ch][2 * p]);
          yv[ch][2 * p + 1] = fmaf(cf[r], bf_hi(d4[p]), yv[ch][2 * p + 1]);
        }
      }
  }

  // partial output of the workgroup: waves [0, NW/2) store their rows, the
  // others add theirs, then the NW/2 slots are summed in a fixed order
  constexpr int SL = kDenseWaves / 2;
  const int slot = wave % SL;
  auto rows = [&](bool add) {
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
      const int h = ch * 512 + lane * 8;
      if (h < H) {
        float4* o = reinterpret_cast<float4*>(yred + (size_t)slot * H + h);
        float4 p0 = make_float4(yv[ch][0], yv[ch][1], yv[ch][2], yv[ch][3]);
        float4 p1 = make_float4(yv[ch][4], yv[ch][5], yv[ch][6], yv[ch][7]);
        if (add) {
          const float4 r0 = o[0], r1 = o[1];
          p0.x += r0.x, p0.y += r0.y, p0.z += r0.z, p0.w += r0.w;
          p1.x += r1.x, p1.y += r1.y, p1.z += r1.z, p1.w += r1.w;
        }
        o[0] = p0;
        o[1] = p1;
      }
    }
  };
  if (wave < SL) rows(false);
  lds_barrier();
  if (wave >= SL) rows(true);
  lds_barrier();
  float* yp = a.ypart + ((size_t)t * a.G + w) * H;
  for (int h = tid * 4; h < H; h += kDenseThreads * 4) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int q = 0; q < SL; ++q) {
      const float4 u = *reinterpret_cast<const float4*>(yred + (size_t)q * H + h);
      v.x += u.x, v.y += u.y, v.z += u.z, v.w += u.w;
    }
    *reinterpret_cast<float4*>(yp + h) = v;
  }
}

template <int NCH, int U>
hipError_t launch_dense_t(const DenseArgs& a, int batch, size_t lds, hipStream_t st) {
  static OncePerDevice attr;
  attr([] {
    (void)hipFuncSetAttribute((const void*)k_dense<NCH, U>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)(kMaxLds - 1024));
    (void)hipGetLastError();
  });
  k_dense<NCH, U><<<batch * a.G, kDenseThreads, lds, st>>>(a);
  return hipGetLastError();
}

template <int NCH>
hipError_t launch_dense_u(const DenseArgs& a, int u, int batch, size_t lds, hipStream_t st) {
  if constexpr (NCH >= 8) {
    return launch_dense_t<NCH, 1>(a, batch, lds, st);
  } else {
    switch (u) {
      case 1: return launch_dense_t<NCH, 1>(a, batch, lds, st);
      case 2: return launch_dense_t<NCH, 2>(a, batch, lds, st);
      default: return launch_dense_t<NCH, 3>(a, batch, lds, st);
    }
  }
}

}  // namespace

DensePlan make_dense_plan(const cfr_config& c, int batch) {
  DensePlan p;
  const int nc = c.top * c.inter;
  int g = kMaxGatherWgs / batch;
  if (g < 1) g = 1;
  p.chan = (nc + g - 1) / g;
  p.G = (nc + p.chan - 1) / p.chan;
  p.cpw = (p.chan + kDenseWaves - 1) / kDenseWaves;
  p.nch = 1;
  while (p.nch * 512 < c.hidden) p.nch *= 2;
  p.u = p.nch >= 8 ? 1 : (p.cpw < 3 ? p.cpw : 3);
  p.lds = sizeof(float) * (size_t)c.hidden * (1 + kDenseWaves / 2);
  return p;
}

hipError_t launch_dense_block(const float* x, const int32_t* ids, const float* gw, const uint16_t* w3,
                              float* ypart, int32_t* status, const cfr_config& c, int batch,
                              const DensePlan& p, hipStream_t st) {
  DenseArgs a{x, ids, gw, w3, ypart, status, c.hidden, c.n_experts, c.inter, c.top,
              c.top * c.inter, p.G, p.chan, p.cpw};
  switch (p.nch) {
    case 1: return launch_dense_u<1>(a, p.u, batch, p.lds, st);
    case 2: return launch_dense_u<2>(a, p.u, batch, p.lds, st);
    case 4: return launch_dense_u<4>(a, p.u, batch, p.lds, st);
    default: return launch_dense_u<8>(a, p.u, batch, p.lds, st);
  }
}

}  // namespace cfr

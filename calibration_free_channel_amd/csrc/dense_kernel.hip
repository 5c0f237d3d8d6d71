// Dense BF16 routed-expert block for gfx950: the baseline the reader is
// measured against, and the k = all limit of its exact part.
//
// For each token and each channel j of its routed experts (gated MLP of the
// MoE layer, [zh §前置知识 / Mixture-of-Experts (MoE)]; zh = the Chinese
// summary page of "Channel Selection for Mixture-of-Experts Decoding Needs No
// Calibration Data"): a_j = silu(g_j . x)(v_j . x), y = sum_j w_j a_j d_j.
//
// The block is a pure HBM stream: every routed channel's gate, up and
// (transposed) down rows are read once, three rows that lie next to each
// other in the [E][I][3] row layout (native BF16, or 4-bit records
// dequantized on the fly).  One launch of G workgroups per token,
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
  const uint8_t* w3;    // [E][I][3] rows of rowq bytes (BF16, or 4-bit records)
  float* ypart;         // [B][G][H]
  int32_t* status;
  int H, E, I, top, nc, G, chan, cpw, rowq;
};

constexpr int kDenseThreads = 512;
constexpr int kDenseWaves = kDenseThreads / 64;

// NCH: 512-wide chunks covering a row (H <= 512 NCH); U: channels a wave has
// in flight at once.
template <int NCH, int U, bool Q4>
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
    Chunk8<Q4> gq[U][NCH], uq[U][NCH], dq[U][NCH];
    int sr[U];
    // every row of the U channels issued before any is used; a channel past
    // the wave's range re-reads the last one and gets coefficient 0
#pragma unroll
    for (int r = 0; r < U; ++r) {
      const int cc = min(q + r, q1 - 1);
      sr[r] = cc / I;
      const uint8_t* row = a.w3 + ((size_t)sl_e[sr[r]] * I + (cc - sr[r] * I)) * 3 * a.rowq;
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const int h = min(ch * 512 + lane * 8, H - 8);  // clamped; the tail is masked below
        gq[r][ch].load(row, H, h);
        uq[r][ch].load(row + a.rowq, H, h);
        dq[r][ch].load(row + 2 * a.rowq, H, h);
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
          float gv[8], uv[8];
          gq[r][ch].vals(gv);
          uq[r][ch].vals(uv);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            gs[r] = fmaf(gv[i], xv[i], gs[r]);
            vs[r] = fmaf(uv[i], xv[i], vs[r]);
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
        float dv[8];
        dq[r][ch].vals(dv);
#pragma unroll
        for (int i = 0; i < 8; ++i) yv[ch][i] = fmaf(cf[r], dv[i], yv[ch][i]);
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

template <int NCH, int U, bool Q4>
hipError_t launch_dense_t(const DenseArgs& a, int batch, size_t lds, hipStream_t st) {
  static OncePerDevice attr;
  attr([] {
    (void)hipFuncSetAttribute((const void*)k_dense<NCH, U, Q4>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)(kMaxLds - 1024));
    (void)hipGetLastError();
  });
  k_dense<NCH, U, Q4><<<batch * a.G, kDenseThreads, lds, st>>>(a);
  return hipGetLastError();
}

template <int NCH, bool Q4>
hipError_t launch_dense_u(const DenseArgs& a, int u, int batch, size_t lds, hipStream_t st) {
  if constexpr (NCH >= 8) {
    return launch_dense_t<NCH, 1, Q4>(a, batch, lds, st);
  } else {
    switch (u) {
      case 1: return launch_dense_t<NCH, 1, Q4>(a, batch, lds, st);
      case 2: return launch_dense_t<NCH, 2, Q4>(a, batch, lds, st);
      default: return launch_dense_t<NCH, 3, Q4>(a, batch, lds, st);
    }
  }
}

template <bool Q4>
hipError_t launch_dense_q(const DenseArgs& a, int nch, int u, int batch, size_t lds, hipStream_t st) {
  switch (nch) {
    case 1: return launch_dense_u<1, Q4>(a, u, batch, lds, st);
    case 2: return launch_dense_u<2, Q4>(a, u, batch, lds, st);
    case 4: return launch_dense_u<4, Q4>(a, u, batch, lds, st);
    default: return launch_dense_u<8, Q4>(a, u, batch, lds, st);
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

hipError_t launch_dense_block(const float* x, const int32_t* ids, const float* gw, const uint8_t* w3,
                              float* ypart, int32_t* status, const cfr_config& c, int batch,
                              const DensePlan& p, hipStream_t st) {
  const bool q4 = q4_rows(c);
  DenseArgs a{x, ids, gw, w3, ypart, status, c.hidden, c.n_experts, c.inter, c.top,
              c.top * c.inter, p.G, p.chan, p.cpw, row_bytes(c.hidden, q4)};
  return q4 ? launch_dense_q<true>(a, p.nch, p.u, batch, p.lds, st)
            : launch_dense_q<false>(a, p.nch, p.u, batch, p.lds, st);
}

}  // namespace cfr

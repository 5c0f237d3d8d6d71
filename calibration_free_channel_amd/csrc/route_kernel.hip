// Softmax top-k router of a MoE layer for gfx950: the experts a token
// activates and their weights, the inputs of the reader's decode.
//
// The router activates a few experts per token, e.g. 8 of 128
// ([zh §前置知识 / Mixture-of-Experts (MoE)]); a channel's routing weight is
// its expert's ([zh §核心方法]).  Reading (Qwen3 convention): logits =
// W_router x, softmax over all experts, keep the `top` largest (ties to the
// lower expert index), renormalise the kept probabilities to sum to one.
// The full softmax denominator cancels in the renormalisation, so the weights
// are a softmax over the kept logits alone.
#include <hip/hip_runtime.h>

#include <math.h>

#include "kernels.h"

namespace cfr {

namespace {

constexpr int kRouteThreads = 512;  // eight experts per workgroup, one per wave

__device__ __forceinline__ float route_wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Logits: grid (ceil(E / 8), batch); wave w of workgroup g computes expert
// 8 g + w for token blockIdx.y, lane l the 8-element chunks l, l + 64, ...
// of the token and of its row: the token's chunks first, then the row's, all
// in flight together.  With eps >= 0 the router reads h = x / sqrt(mean(x^2)
// + eps) (RMSNorm, unit weights): every wave forms sum x^2 over the same
// chunks in the same order, so each gets the same scale; workgroup 0's first
// wave writes h.
__global__ __launch_bounds__(kRouteThreads) void k_route_logits(const float* x, const uint16_t* router,
                                                                int H, int E, float eps, float* h,
                                                                float* logits) {
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * (kRouteThreads / 64) + (threadIdx.x >> 6);
  const float* xt = x + (size_t)t * H;
  constexpr int CH = kMaxHidden / 512;  // chunks per lane, at most
  const int nch = H / 8;
  float4 xa[CH], xb[CH];
#pragma unroll
  for (int q = 0; q < CH; ++q) {
    const int c = min(lane + 64 * q, nch - 1);
    xa[q] = *reinterpret_cast<const float4*>(xt + 8 * c);
    xb[q] = *reinterpret_cast<const float4*>(xt + 8 * c + 4);
  }
  const uint4* row = reinterpret_cast<const uint4*>(router + (size_t)min(e, E - 1) * H);
  uint4 wv[CH];
#pragma unroll
  for (int q = 0; q < CH; ++q) wv[q] = row[min(lane + 64 * q, nch - 1)];
  float scale = 1.f;
  if (eps >= 0.f) {
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < CH; ++q)
      if (lane + 64 * q < nch) {
        ss = fmaf(xa[q].x, xa[q].x, ss);
        ss = fmaf(xa[q].y, xa[q].y, ss);
        ss = fmaf(xa[q].z, xa[q].z, ss);
        ss = fmaf(xa[q].w, xa[q].w, ss);
        ss = fmaf(xb[q].x, xb[q].x, ss);
        ss = fmaf(xb[q].y, xb[q].y, ss);
        ss = fmaf(xb[q].z, xb[q].z, ss);
        ss = fmaf(xb[q].w, xb[q].w, ss);
      }
    scale = rsqrtf(route_wave_sum(ss) / (float)H + eps);
    if (blockIdx.x == 0 && threadIdx.x < 64) {
      float* ht = h + (size_t)t * H;
#pragma unroll
      for (int q = 0; q < CH; ++q) {
        const int c = lane + 64 * q;
        if (c >= nch) continue;
        *reinterpret_cast<float4*>(ht + 8 * c) =
            make_float4(xa[q].x * scale, xa[q].y * scale, xa[q].z * scale, xa[q].w * scale);
        *reinterpret_cast<float4*>(ht + 8 * c + 4) =
            make_float4(xb[q].x * scale, xb[q].y * scale, xb[q].z * scale, xb[q].w * scale);
      }
    }
  }
  if (e >= E) return;
  float acc = 0.f;
#pragma unroll
  for (int q = 0; q < CH; ++q) {
    if (lane + 64 * q >= nch) continue;
    const uint32_t w4[4] = {wv[q].x, wv[q].y, wv[q].z, wv[q].w};
    const float xv[8] = {xa[q].x * scale, xa[q].y * scale, xa[q].z * scale, xa[q].w * scale,
                         xb[q].x * scale, xb[q].y * scale, xb[q].z * scale, xb[q].w * scale};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(__uint_as_float(w4[i] << 16), xv[2 * i], acc);
      acc = fmaf(__uint_as_float(w4[i] & 0xFFFF0000u), xv[2 * i + 1], acc);
    }
  }
  acc = route_wave_sum(acc);
  if (lane == 0) logits[(size_t)t * E + e] = acc;
}

// Top experts by logit (ties to the lower index) and their weights, a
// softmax over the kept logits: one wave per token.  Each expert's rank is
// the number of experts ahead of it (a larger logit, or an equal one with a
// lower index), counted against the logits staged in LDS; the top ranks
// write themselves.
__global__ __launch_bounds__(64) void k_route_topk(const float* logits, int E, int top, int32_t* ids,
                                                   float* gw) {
  extern __shared__ float4 lg4[];  // the logits, padded to a multiple of 4 with -inf
  __shared__ float selv[kMaxTop];
  float* lg = reinterpret_cast<float*>(lg4);
  const int t = blockIdx.x, lane = threadIdx.x;
  const int E4 = (E + 3) / 4;
  const float* lt = logits + (size_t)t * E;
  for (int base = 0; base < 4 * E4; base += 256) {
    // four loads per lane in flight (clamped addresses), then the stores
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = lt[min(base + lane + 64 * i, E - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = base + lane + 64 * i;
      if (e < 4 * E4) lg[e] = e < E ? v[i] : -INFINITY;
    }
  }
  __syncthreads();
  for (int e = lane; e < E; e += 64) {
    const float v = lg[e];
    int rank = 0;
#pragma unroll 4
    for (int q = 0; q < E4; ++q) {
      const float4 o = lg4[q];  // the same address in every lane: a broadcast read
      const int b = 4 * q;
      rank += (o.x > v) | ((o.x == v) & (b < e));
      rank += (o.y > v) | ((o.y == v) & (b + 1 < e));
      rank += (o.z > v) | ((o.z == v) & (b + 2 < e));
      rank += (o.w > v) | ((o.w == v) & (b + 3 < e));
    }
    if (rank < top) {
      ids[(size_t)t * top + rank] = e;
      selv[rank] = v;
    }
  }
  __syncthreads();
  const float ev = lane < top ? __expf(selv[lane] - selv[0]) : 0.f;
  const float sum = route_wave_sum(ev);
  if (lane < top) gw[(size_t)t * top + lane] = ev / sum;
}

}  // namespace

size_t route_lds_bytes(const cfr_config& c) { return (size_t)(c.n_experts + 3) / 4 * 16; }

hipError_t launch_route(const float* x, const uint16_t* router, const cfr_config& c, int batch, float eps,
                        float* h, float* logits, int32_t* ids, float* gw, hipStream_t st) {
  static OncePerDevice attr;
  attr([] {
    (void)hipFuncSetAttribute((const void*)k_route_topk, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)(kMaxLds - kMaxTop * 4));
    (void)hipGetLastError();
  });
  const int per = kRouteThreads / 64;
  k_route_logits<<<dim3((c.n_experts + per - 1) / per, batch), kRouteThreads, 0, st>>>(x, router, c.hidden,
                                                                                      c.n_experts, eps, h, logits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_route_topk<<<batch, 64, route_lds_bytes(c), st>>>(logits, c.n_experts, c.top, ids, gw);
  return hipGetLastError();
}

}  // namespace cfr

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
//
// One launch: the workgroups of a token compute its logits, and the last of
// them to finish (a per-token arrival counter, which that workgroup sets back
// to zero for the next call) picks the top experts and their weights.
#include <hip/hip_runtime.h>

#include <math.h>

#include "kernels.h"

namespace cfr {

namespace {

constexpr int kRouteThreads = 512;  // eight experts per workgroup, one per wave

// Total order on logits: a larger float gives a larger key; NaN takes key 0,
// below every other value (including -inf), so the ranks below always form a
// permutation of the experts.
__device__ __forceinline__ uint32_t route_key(float f) {
  const uint32_t u = __float_as_uint(f);
  if (f != f) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// the float a key came from (NaN for key 0)
__device__ __forceinline__ float route_unkey(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ float route_wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Grid (ceil(E / 8), batch); wave w of workgroup g computes expert 8 g + w for
// token blockIdx.y, lane l the 8-element chunks l, l + 64, ... (CH of them,
// clamped to the last) of the token and of its row: the token's chunks first,
// then the row's, all in flight together.  With eps >= 0 the router reads
// h = x / sqrt(mean(x^2) + eps) (RMSNorm, unit weights): every wave forms
// sum x^2 over the same chunks in the same order, so each gets the same
// scale; workgroup 0's first wave writes h.
template <int CH>
__global__ __launch_bounds__(kRouteThreads) void k_route(const float* x, const uint16_t* router, int H, int E,
                                                         int top, float eps, float* h, float* logits,
                                                         int* arrived, int32_t* ids, float* gw,
                                                         int32_t* status) {
  // the last workgroup: the logits' order keys padded to a multiple of 4 with
  // key 0, then each expert's rank
  extern __shared__ uint4 lg4[];
  __shared__ int last;
  __shared__ float selv[kMaxTop];
  const int t = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * (kRouteThreads / 64) + (threadIdx.x >> 6);
  const float* xt = x + (size_t)t * H;
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
  // Hand-over between the workgroups of a token, through device-scope atomic
  // read-modify-writes only (performed where every workgroup sees them, so no
  // cache write-back is needed, which a release fence would force on every
  // dirty line of the L2): each wave swaps its logit in and waits for the
  // swap to complete before the barrier; then the workgroup counts itself in;
  // the last to count reads the logits back with atomics and zeroes the
  // counter.
  float* lt = logits + (size_t)t * E;
  if (e < E && lane == 0) atomicExch(lt + e, acc);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) last = atomicAdd(arrived + t, 1) == (int)gridDim.x - 1;
  __syncthreads();
  if (!last) return;
  const int E4 = (E + 3) / 4;
  uint32_t* lg = reinterpret_cast<uint32_t*>(lg4);
  int* rank = reinterpret_cast<int*>(lg4 + E4);
  bool bad = false;
  for (int i = threadIdx.x; i < 4 * E4; i += kRouteThreads) {
    const float v = i < E ? __uint_as_float(atomicOr(reinterpret_cast<unsigned*>(lt) + i, 0u)) : 0.f;
    bad |= !isfinite(v);
    lg[i] = i < E ? route_key(v) : 0u;
    if (i < E) rank[i] = 0;
  }
  // a non-finite logit (from a non-finite token, or inf * 0 in the norm):
  // bit 1 of the reader's status word
  if (bad) atomicOr(status, 2);
  if (threadIdx.x == 0) atomicExch(arrived + t, 0);  // no workgroup of this launch counts again
  __syncthreads();
  // rank of expert e = the experts ahead of it (a larger key, or an equal one
  // with a lower index); P threads count it, each over its share of the keys
  // (read four at a time), and add their counts in LDS.  Padding (index >= E,
  // key 0) is never ahead of an expert.
  const int P = max(1, min(16, kRouteThreads / E));
  const int L = (E4 + P - 1) / P;
  for (int idx = threadIdx.x; idx < E * P; idx += kRouteThreads) {
    const int j = idx / P, part = idx - j * P;
    const uint32_t v = lg[j];
    const int q1 = min(E4, (part + 1) * L);
    int cnt = 0;
    for (int q = part * L; q < q1; ++q) {
      const uint4 o = lg4[q];
      const int i = 4 * q;
      cnt += (o.x > v) | ((o.x == v) & (i < j));
      cnt += (o.y > v) | ((o.y == v) & (i + 1 < j));
      cnt += (o.z > v) | ((o.z == v) & (i + 2 < j));
      cnt += (o.w > v) | ((o.w == v) & (i + 3 < j));
    }
    if (cnt) atomicAdd(rank + j, cnt);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < E; j += kRouteThreads) {
    const int k = rank[j];
    if (k < top) {
      ids[(size_t)t * top + k] = j;
      selv[k] = route_unkey(lg[j]);
    }
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const float ev = lane < top ? __expf(selv[lane] - selv[0]) : 0.f;
  const float sum = route_wave_sum(ev);
  if (lane < top) gw[(size_t)t * top + lane] = ev / sum;
}

template <int CH>
hipError_t launch_route_t(const float* x, const uint16_t* router, const cfr_config& c, int batch, float eps,
                          float* h, float* logits, int* arrived, int32_t* ids, float* gw, int32_t* status,
                          hipStream_t st) {
  static OncePerDevice attr;
  attr([] {
    (void)hipFuncSetAttribute((const void*)k_route<CH>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)(kMaxLds - 128));
    (void)hipGetLastError();
  });
  const int per = kRouteThreads / 64;
  k_route<CH><<<dim3((c.n_experts + per - 1) / per, batch), kRouteThreads, route_lds_bytes(c), st>>>(
      x, router, c.hidden, c.n_experts, c.top, eps, h, logits, arrived, ids, gw, status);
  return hipGetLastError();
}

}  // namespace

size_t route_lds_bytes(const cfr_config& c) {
  return (size_t)(c.n_experts + 3) / 4 * 16 + (size_t)c.n_experts * 4;
}

hipError_t launch_route(const float* x, const uint16_t* router, const cfr_config& c, int batch, float eps,
                        float* h, float* logits, int* arrived, int32_t* ids, float* gw, int32_t* status,
                        hipStream_t st) {
  // chunks of 8 per lane: the fewest of 1, 2, 4, 8 that cover hidden / 8
  static_assert(kMaxHidden / 8 <= 64 * 8, "eight chunks per lane cover the largest token");
  const int need = (c.hidden / 8 + 63) / 64;
  if (need <= 1) return launch_route_t<1>(x, router, c, batch, eps, h, logits, arrived, ids, gw, status, st);
  if (need <= 2) return launch_route_t<2>(x, router, c, batch, eps, h, logits, arrived, ids, gw, status, st);
  if (need <= 4) return launch_route_t<4>(x, router, c, batch, eps, h, logits, arrived, ids, gw, status, st);
  return launch_route_t<8>(x, router, c, batch, eps, h, logits, arrived, ids, gw, status, st);
}

}  // namespace cfr

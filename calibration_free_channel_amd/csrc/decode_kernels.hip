// Decode kernels of the channel-selection reader for gfx950 (CDNA4, wave64).
//
// Per token and layer ([zh §方法步骤详情] decode steps (1)-(4); [zh §核心方法];
// [ko §어떻게 쓰나]; zh/ko = the Chinese/Korean summary pages of "Channel
// Selection for Mixture-of-Experts Decoding Needs No Calibration Data"):
//   k_rotate_select   v = H_128 (sigma * x) per block (float32 butterfly) and
//                     the n_screen coordinates of largest |v| per block
//   k_screen          per (token, routed slot, block): sum over screened
//                     coordinates of code * v, times the block's fp16 scale
//   k_score           g_hat, v_hat (sum over blocks, / sqrt 128), p = silu(g_hat) v_hat,
//                     s = w ||d|| |p|
//   k_topk            exact top-k per token: radix select on the score bits,
//                     ties to the lower candidate index, ascending compaction
//   k_exact_act       kept channels: a = silu(g.x) (v.x) from native BF16 rows
//   k_down_partial    partial y over chunks of kept channels (transposed down rows)
//   k_recover_partial partial z = sum over skipped of w p b
//   k_finalize        y = sum of partials + U z
// The whole path is HBM-bandwidth bound at batch 1 (about 2 flops per byte),
// so it uses vector ALU and wave reductions, not matrix cores.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace cfr {

namespace {

constexpr float kInvSqrt128f = 0.08838834764831845f;  // 1/sqrt(128) rounded to float
constexpr int kDownChunk = 32;    // kept channels per down-projection work item
constexpr int kDownSlice = 512;   // hidden units per down-projection work item
constexpr int kZChunk = 256;      // candidates per recovery work item

__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

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

__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Inclusive scan of one int per thread over a 1024-thread block (16 waves).
__device__ int block_scan_1024(int v, int* sh /* >= 16 ints */) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63) sh[w] = v;
  __syncthreads();
  if (w == 0) {
    int t = lane < 16 ? sh[lane] : 0;
    for (int off = 1; off < 16; off <<= 1) {
      int o = __shfl_up(t, off, 64);
      if (lane >= off) t += o;
    }
    if (lane < 16) sh[lane] = t;
  }
  __syncthreads();
  int add = w > 0 ? sh[w - 1] : 0;
  __syncthreads();
  return v + add;
}

}  // namespace

// ---------------------------------------------------------------------------
// decode step (1a): rotate and select.  grid (nblk, B), 128 threads.
__global__ __launch_bounds__(128) void k_rotate_select(const float* __restrict__ x,
                                                       const float* __restrict__ sigma,
                                                       float* __restrict__ xrot,
                                                       uint8_t* __restrict__ sel, int H, int nblk,
                                                       int n_screen) {
  const int b = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
  __shared__ float s[128];
  __shared__ unsigned long long bal[2];
  const size_t off = (size_t)t * H + (size_t)b * 128 + tid;
  float v = x[off] * sigma[b * 128 + tid];
  for (int h = 1; h < 128; h <<= 1) {
    s[tid] = v;
    __syncthreads();
    float o = s[tid ^ h];
    v = (tid & h) ? (o - v) : (v + o);
    __syncthreads();
  }
  xrot[off] = v;
  const float a = fabsf(v);
  s[tid] = a;
  __syncthreads();
  int rank = 0;
  for (int j = 0; j < 128; ++j) {
    float aj = s[j];
    rank += (aj > a) || (aj == a && j < tid);
  }
  const bool on = rank < n_screen;
  const unsigned long long m = __ballot(on);
  const int lane = tid & 63, w = tid >> 6;
  if (lane == 0) bal[w] = m;
  __syncthreads();
  const int pos = __popcll(m & ((1ull << lane) - 1ull)) + (w ? __popcll(bal[0]) : 0);
  // ranks form a permutation for finite inputs; the bound keeps NaN inputs in range
  if (on && pos < n_screen) sel[((size_t)t * nblk + b) * n_screen + pos] = (uint8_t)tid;
}

// ---------------------------------------------------------------------------
// decode step (1b): partial screen.  grid (nblk, top, B), G*D threads where
// D = unit/4 dwords per unit and G coordinate groups.  Each thread owns one
// dword (four bytes = twenty channel codes) of the unit and accumulates over
// its group's screened coordinates; groups are then summed through LDS and
// scaled by the block's fp16 scale.
__global__ __launch_bounds__(512) void k_screen(const uint8_t* __restrict__ codes,
                                                const uint16_t* __restrict__ scales,
                                                const float* __restrict__ xrot,
                                                const uint8_t* __restrict__ sel,
                                                const int32_t* __restrict__ ids,
                                                float* __restrict__ part, int32_t* status, int H,
                                                int E, int I, int top, int nblk, int n_screen,
                                                int lp, int unit, int G) {
  extern __shared__ float red[];  // [G][D*20]
  const int b = blockIdx.x, s = blockIdx.y, t = blockIdx.z;
  const int D = unit >> 2;
  const int tid = threadIdx.x, d = tid % D, g = tid / D;
  const int e = clamp_expert(ids[t * top + s], E, status);
  float acc[20];
#pragma unroll
  for (int q = 0; q < 20; ++q) acc[q] = 0.f;
  const uint32_t* base = reinterpret_cast<const uint32_t*>(codes + ((size_t)e * nblk + b) * 128 * unit);
  const uint8_t* selp = sel + ((size_t)t * nblk + b) * n_screen;
  const float* xr = xrot + (size_t)t * H + (size_t)b * 128;
  if (g < G) {
    for (int i = g; i < n_screen; i += G) {
      const int c = selp[i] & 127;
      const float xv = xr[c];
      uint32_t w = base[(size_t)c * D + d];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        uint32_t q = (w >> (8 * kb)) & 255u;
#pragma unroll
        for (int dd = 0; dd < 5; ++dd) {
          const uint32_t r = q % 3u;
          q /= 3u;
          acc[kb * 5 + dd] += (r == 2u) ? xv : ((r == 0u) ? -xv : 0.f);
        }
      }
    }
    float* my = red + (size_t)g * D * 20 + d * 20;
#pragma unroll
    for (int q = 0; q < 20; ++q) my[q] = acc[q];
  }
  __syncthreads();
  const int nout = D * 20;
  float* out = part + (((size_t)t * top + s) * nblk + b) * 2 * I;
  const uint16_t* sc = scales + ((size_t)e * nblk + b) * 2 * I;
  for (int o = tid; o < nout; o += blockDim.x) {
    const int p = o / 5, digit = o % 5;
    const int half = p / lp;
    if (half >= 2) continue;
    const int ch = 5 * (p % lp) + digit;
    if (ch >= I) continue;
    float v = 0.f;
    for (int gg = 0; gg < G; ++gg) v += red[(size_t)gg * nout + o];
    out[half * I + ch] = v * f16f(sc[half * I + ch]);
  }
}

// ---------------------------------------------------------------------------
// decode step (2a): estimates and scores.  One thread per (token, candidate).
__global__ __launch_bounds__(256) void k_score(const float* __restrict__ part,
                                               const float* __restrict__ norms,
                                               const int32_t* __restrict__ ids,
                                               const float* __restrict__ gw,
                                               float* __restrict__ ghat, float* __restrict__ vhat,
                                               float* __restrict__ pact,
                                               float* __restrict__ score, int32_t* status, int E,
                                               int I, int top, int nblk, int ncand, int batch) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= batch * ncand) return;
  const int t = idx / ncand, c = idx % ncand, s = c / I, j = c % I;
  const int e = clamp_expert(ids[t * top + s], E, status);
  const float* pp = part + ((size_t)t * top + s) * nblk * 2 * I;
  float g = 0.f, v = 0.f;
  for (int b = 0; b < nblk; ++b) {
    g += pp[(size_t)b * 2 * I + j];
    v += pp[(size_t)b * 2 * I + I + j];
  }
  g *= kInvSqrt128f;
  v *= kInvSqrt128f;
  const float p = silu(g) * v;
  ghat[idx] = g;
  vhat[idx] = v;
  pact[idx] = p;
  score[idx] = gw[t * top + s] * norms[(size_t)e * I + j] * fabsf(p);
}

// ---------------------------------------------------------------------------
// decode step (2b): exact top-k per token.  grid (B), 1024 threads.
// Scores are non-negative floats, so their bit patterns order like their
// values; a 4-pass MSB-first radix select finds the k-th largest key T and
// how many keys equal to T are kept (lowest indices first).
__global__ __launch_bounds__(1024) void k_topk(const float* __restrict__ score,
                                               int32_t* __restrict__ kept,
                                               uint8_t* __restrict__ keptf, int ncand, int k) {
  __shared__ int hist[256];
  __shared__ int scan_sh[16];
  __shared__ int sel_digit, sel_kk;
  const int t = blockIdx.x, tid = threadIdx.x;
  const uint32_t* key = reinterpret_cast<const uint32_t*>(score + (size_t)t * ncand);
  int32_t* kout = kept + (size_t)t * ncand;
  uint8_t* fout = keptf + (size_t)t * ncand;
  const int per = (ncand + 1023) / 1024;
  const int lo = min(tid * per, ncand), hi = min(lo + per, ncand);

  uint32_t prefix = 0, mask = 0;
  int kk = k;
  if (k > 0 && k < ncand) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int i = lo; i < hi; ++i) {
        uint32_t kv = key[i];
        if ((kv & mask) == prefix) atomicAdd(&hist[(kv >> shift) & 255u], 1);
      }
      __syncthreads();
      // suffix counts: thread d holds count of digits >= 255 - d
      int own = tid < 256 ? hist[255 - tid] : 0;
      int incl = block_scan_1024(own, scan_sh);
      if (tid < 256 && incl >= kk && incl - own < kk) {
        sel_digit = 255 - tid;
        sel_kk = kk - (incl - own);
      }
      __syncthreads();
      prefix |= (uint32_t)sel_digit << shift;
      mask |= 255u << shift;
      kk = sel_kk;
      __syncthreads();
    }
  }
  // count per thread, then scan for equal keys and for output positions
  int ngt = 0, neq = 0;
  if (k == ncand) {
    ngt = hi - lo;
  } else if (k > 0) {
    for (int i = lo; i < hi; ++i) {
      uint32_t kv = key[i];
      ngt += kv > prefix;
      neq += kv == prefix;
    }
  }
  const int eq_incl = block_scan_1024(neq, scan_sh);
  int eq_before = eq_incl - neq;
  int take_eq = 0;
  if (k > 0 && k < ncand) take_eq = max(0, min(neq, kk - eq_before));
  const int mine = ngt + take_eq;
  const int pos_incl = block_scan_1024(mine, scan_sh);
  int pos = pos_incl - mine;
  int eq_seen = 0;
  for (int i = lo; i < hi; ++i) {
    bool on;
    if (k == ncand) {
      on = true;
    } else if (k == 0) {
      on = false;
    } else {
      uint32_t kv = key[i];
      on = kv > prefix;
      if (kv == prefix) {
        on = eq_seen < take_eq;
        ++eq_seen;
      }
    }
    fout[i] = on ? 1 : 0;
    if (on) kout[pos++] = i;
  }
}

// ---------------------------------------------------------------------------
// decode step (3a): exact activations of kept channels from native rows.
// grid (ceil(k/4), B), 256 threads = 4 waves, one kept channel per wave.
// kept == nullptr means candidate idx itself (the dense baseline).
__global__ __launch_bounds__(256) void k_exact_act(const uint16_t* __restrict__ w3,
                                                   const float* __restrict__ x,
                                                   const int32_t* __restrict__ kept,
                                                   const int32_t* __restrict__ ids,
                                                   const float* __restrict__ gw,
                                                   float* __restrict__ coef, int32_t* status,
                                                   int H, int E, int I, int top, int ncand, int k) {
  const int t = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int idx = blockIdx.x * 4 + wave;
  if (idx >= k) return;
  const int c = kept ? kept[(size_t)t * ncand + idx] : idx;
  const int s = c / I, j = c % I;
  const int e = clamp_expert(ids[t * top + s], E, status);
  const uint16_t* row = w3 + ((size_t)e * I + j) * 3 * H;
  const float* xt = x + (size_t)t * H;
  float g = 0.f, v = 0.f;
  for (int h = lane * 8; h < H; h += 512) {
    const uint4 gq = *reinterpret_cast<const uint4*>(row + h);
    const uint4 vq = *reinterpret_cast<const uint4*>(row + H + h);
    const float4 x0 = *reinterpret_cast<const float4*>(xt + h);
    const float4 x1 = *reinterpret_cast<const float4*>(xt + h + 4);
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    const uint32_t gw4[4] = {gq.x, gq.y, gq.z, gq.w};
    const uint32_t vw4[4] = {vq.x, vq.y, vq.z, vq.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      g += __uint_as_float(gw4[q] << 16) * xs[2 * q] + __uint_as_float(gw4[q] & 0xFFFF0000u) * xs[2 * q + 1];
      v += __uint_as_float(vw4[q] << 16) * xs[2 * q] + __uint_as_float(vw4[q] & 0xFFFF0000u) * xs[2 * q + 1];
    }
  }
  g = wave_sum(g);
  v = wave_sum(v);
  if (lane == 0) coef[(size_t)t * ncand + idx] = gw[t * top + s] * silu(g) * v;
}

// ---------------------------------------------------------------------------
// decode step (3b): partial y over a chunk of kept channels.
// grid (ceil(H/512), nchunks, B), 256 threads, two hidden units per thread.
__global__ __launch_bounds__(256) void k_down_partial(const uint16_t* __restrict__ w3,
                                                      const int32_t* __restrict__ kept,
                                                      const int32_t* __restrict__ ids,
                                                      const float* __restrict__ coef,
                                                      float* __restrict__ ypart, int32_t* status,
                                                      int H, int E, int I, int top, int ncand,
                                                      int k, int max_chunks) {
  const int t = blockIdx.z, ch = blockIdx.y;
  const int h0 = blockIdx.x * kDownSlice + threadIdx.x * 2;
  const int i0 = ch * kDownChunk, i1 = min(k, i0 + kDownChunk);
  float a0 = 0.f, a1 = 0.f;
  if (h0 < H) {
    for (int idx = i0; idx < i1; ++idx) {
      const int c = kept ? kept[(size_t)t * ncand + idx] : idx;
      const int s = c / I, j = c % I;
      const int e = clamp_expert(ids[t * top + s], E, status);
      const float cf = coef[(size_t)t * ncand + idx];
      const uint32_t dq = *reinterpret_cast<const uint32_t*>(w3 + (((size_t)e * I + j) * 3 + 2) * H + h0);
      a0 += cf * __uint_as_float(dq << 16);
      a1 += cf * __uint_as_float(dq & 0xFFFF0000u);
    }
    float* yp = ypart + ((size_t)t * max_chunks + ch) * H + h0;
    yp[0] = a0;
    yp[1] = a1;
  }
}

// ---------------------------------------------------------------------------
// decode step (4a): partial recovery vector z over a chunk of candidates.
// grid (nz, B), 256 threads = 4 candidate groups x 64 rank lanes.
__global__ __launch_bounds__(256) void k_recover_partial(const uint16_t* __restrict__ bmat,
                                                         const uint8_t* __restrict__ keptf,
                                                         const float* __restrict__ pact,
                                                         const int32_t* __restrict__ ids,
                                                         const float* __restrict__ gw,
                                                         float* __restrict__ zpart,
                                                         int32_t* status, int E, int I, int top,
                                                         int ncand, int rank, int max_zchunks) {
  __shared__ float red[4][64];
  const int t = blockIdx.y, zc = blockIdx.x;
  const int r = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int c0 = zc * kZChunk, c1 = min(ncand, c0 + kZChunk);
  float acc = 0.f;
  if (r < rank) {
    for (int c = c0 + grp; c < c1; c += 4) {
      if (keptf[(size_t)t * ncand + c]) continue;
      const int s = c / I, j = c % I;
      const int e = clamp_expert(ids[t * top + s], E, status);
      const float cf = gw[t * top + s] * pact[(size_t)t * ncand + c];
      acc += cf * f16f(bmat[((size_t)e * I + j) * rank + r]);
    }
  }
  red[grp][r] = acc;
  __syncthreads();
  if (grp == 0 && r < rank)
    zpart[((size_t)t * max_zchunks + zc) * rank + r] = red[0][r] + red[1][r] + red[2][r] + red[3][r];
}

// ---------------------------------------------------------------------------
// y = sum of partial y + U z.  grid (ceil(H/256), B), 256 threads.
__global__ __launch_bounds__(256) void k_finalize(const float* __restrict__ ypart,
                                                  const float* __restrict__ zpart,
                                                  const uint16_t* __restrict__ U,
                                                  float* __restrict__ y, int H, int rank,
                                                  int nchunks, int nz, int max_chunks,
                                                  int max_zchunks) {
  __shared__ float z[64];
  const int t = blockIdx.y, tid = threadIdx.x;
  if (tid < 64) {
    float a = 0.f;
    if (tid < rank)
      for (int q = 0; q < nz; ++q) a += zpart[((size_t)t * max_zchunks + q) * rank + tid];
    z[tid] = a;
  }
  __syncthreads();
  const int h = blockIdx.x * 256 + tid;
  if (h >= H) return;
  float acc = 0.f;
  for (int q = 0; q < nchunks; ++q) acc += ypart[((size_t)t * max_chunks + q) * H + h];
  if (nz > 0)
    for (int rr = 0; rr < rank; ++rr) acc += f16f(U[(size_t)h * rank + rr]) * z[rr];
  y[(size_t)t * H + h] = acc;
}

// ---------------------------------------------------------------------------
static int hip_fail(hipError_t e, const char* what) {
  return fail(CFR_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

int launch_decode(cfr_reader* r, const float* x, const int32_t* ids, const float* gw, int batch,
                  int k, float* y, hipStream_t st, const DebugOut* dbg, hipEvent_t* ev) {
  const cfr_config& c = r->cfg;
  const int H = c.hidden, E = c.n_experts, I = c.inter, top = c.top, nblk = r->nblk;
  const int ncand = r->ncand;
  const int D = r->unit / 4;
  int G = 512 / D;
  if (G < 1) G = 1;
  if (G > c.n_screen) G = c.n_screen;
  const size_t lds = (size_t)G * D * 20 * sizeof(float);

  auto mark = [&](int i) {
    if (ev) (void)hipEventRecord(ev[i], st);
  };
  mark(0);
  k_rotate_select<<<dim3(nblk, batch), 128, 0, st>>>(x, r->sigma, r->xrot, r->sel, H, nblk,
                                                     c.n_screen);
  mark(1);
  k_screen<<<dim3(nblk, top, batch), G * D, lds, st>>>(r->codes, r->scales, r->xrot, r->sel, ids,
                                                       r->part, r->status, H, E, I, top, nblk,
                                                       c.n_screen, r->lp, r->unit, G);
  mark(2);
  const int nsc = batch * ncand;
  k_score<<<(nsc + 255) / 256, 256, 0, st>>>(r->part, r->norms, ids, gw, r->ghat, r->vhat,
                                             r->pact, r->score, r->status, E, I, top, nblk, ncand,
                                             batch);
  mark(3);
  k_topk<<<batch, 1024, 0, st>>>(r->score, r->kept, r->keptf, ncand, k);
  mark(4);
  int nchunks = 0, nz = 0;
  if (k > 0) {
    nchunks = (k + kDownChunk - 1) / kDownChunk;
    k_exact_act<<<dim3((k + 3) / 4, batch), 256, 0, st>>>(r->w3, x, r->kept, ids, gw, r->coef,
                                                          r->status, H, E, I, top, ncand, k);
  }
  mark(5);
  if (k > 0) {
    k_down_partial<<<dim3((H + kDownSlice - 1) / kDownSlice, nchunks, batch), 256, 0, st>>>(
        r->w3, r->kept, ids, r->coef, r->ypart, r->status, H, E, I, top, ncand, k, r->max_chunks);
  }
  mark(6);
  if (k < ncand && c.rank > 0) {
    nz = (ncand + kZChunk - 1) / kZChunk;
    k_recover_partial<<<dim3(nz, batch), 256, 0, st>>>(r->b, r->keptf, r->pact, ids, gw, r->zpart,
                                                        r->status, E, I, top, ncand, c.rank,
                                                        r->max_zchunks);
  }
  mark(7);
  k_finalize<<<dim3((H + 255) / 256, batch), 256, 0, st>>>(r->ypart, r->zpart, r->u, y, H, c.rank,
                                                           nchunks, nz, r->max_chunks,
                                                           r->max_zchunks);
  mark(8);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (dbg) {
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
      e = hipMemcpy2DAsync(dbg->kept, sizeof(int32_t) * k, r->kept, sizeof(int32_t) * ncand,
                           sizeof(int32_t) * k, batch, hipMemcpyDeviceToDevice, st);
      if (e != hipSuccess) return hip_fail(e, "debug copy kept");
    }
  }
  return CFR_OK;
}

int launch_dense(cfr_reader* r, const float* x, const int32_t* ids, const float* gw, int batch,
                 float* y, hipStream_t st) {
  const cfr_config& c = r->cfg;
  const int H = c.hidden, E = c.n_experts, I = c.inter, top = c.top, ncand = r->ncand;
  const int k = ncand, nchunks = (k + kDownChunk - 1) / kDownChunk;
  k_exact_act<<<dim3((k + 3) / 4, batch), 256, 0, st>>>(r->w3, x, nullptr, ids, gw, r->coef,
                                                        r->status, H, E, I, top, ncand, k);
  k_down_partial<<<dim3((H + kDownSlice - 1) / kDownSlice, nchunks, batch), 256, 0, st>>>(
      r->w3, nullptr, ids, r->coef, r->ypart, r->status, H, E, I, top, ncand, k, r->max_chunks);
  k_finalize<<<dim3((H + 255) / 256, batch), 256, 0, st>>>(r->ypart, r->zpart, r->u, y, H, c.rank,
                                                           nchunks, 0, r->max_chunks,
                                                           r->max_zchunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "dense launch");
  return CFR_OK;
}

}  // namespace cfr

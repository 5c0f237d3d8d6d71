// Batch-shared channel selection for gfx950: one exact top-k for the whole
// batch, each kept channel's native rows read once and applied to every token
// routed to its expert.
//
// The pages leave selecting channels jointly for the batch as future work
// ([zh §未来方向] direction (1); [ko §전제와 한계]; zh/ko = the Chinese/Korean
// summary pages of "Channel Selection for Mixture-of-Experts Decoding Needs No
// Calibration Data").  Reading (the oracle's): the candidates are the channels
// of the batch's distinct routed experts, union candidate u * I + j for the
// u-th distinct expert in ascending id order; a candidate's batch score is the
// sum over the (token, slot) pairs routed to its expert, token-major, of the
// per-token output-unit score w ||d_j|| |silu(g_hat_j) v_hat_j|; the k largest
// are kept (ties to the lower union candidate); every token recovers its own
// skipped channels with its own p_j.
//
// After the screen kernel (per token, as in the per-token decode):
//   k_bscore  one thread per union candidate: the batch score, from the
//             screen sums of every (token, slot) routed to its expert;
//   k_btopk   one workgroup: the bin of the k-th largest batch score from
//             the histogram k_bscore accumulates (1/8 octave per bin), the
//             bin's keys ranked in LDS digit by digit, then the kept list in
//             ascending order with each one's row, and a kept flag per union
//             candidate;
//   k_bact    one wave per four kept channels: their gate and up rows give
//             w a_j for every token routed to the channel's expert (a
//             coefficient per kept channel and token, 0 where not routed);
//             and B Z recovery workgroups: each token's partial z over its
//             skipped candidates;
//   k_bdown   one workgroup per (512 hidden units, range of kept channels):
//             sum over the range of coefficient x down row, per token.
// The decode's reduce kernel then sums the partials per token.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_util.h"
#include "kernels.h"

namespace cfr {

namespace {

constexpr int kMaxEntries = kMaxSharedBatch * kMaxTop;  // (token, slot) pairs of a batch

__device__ __forceinline__ int lanes_below_mask(unsigned long long m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The batch's distinct routed experts, in LDS.
struct SharedLds {
  int ent_e[kMaxEntries];  // expert of pair i = t top + s (clamped)
  int ent_u[kMaxEntries];  // its position in the union
  int first[kMaxEntries];  // 1: the first pair routed to that expert
  int uexp[kMaxEntries];   // the u-th distinct expert, ascending
  int ucnt[kMaxEntries];   // pairs routed to the u-th expert
  int ustart[kMaxEntries]; // where they start in ulist
  int ulist[kMaxEntries];  // pairs grouped by union position, ascending within a group
  int nu;
};

// Every thread of the workgroup calls it; returns the union's size.  Up to
// 64 pairs, wave 0 builds it in registers (lane i holds pair i; the other
// pairs come through lane reads); more pairs go through LDS loops.
template <int NT>
__device__ int build_union(const int32_t* ids, int n, int E, int32_t* status, SharedLds& L) {
  const int tid = threadIdx.x;
  if (n <= 64) {
    if (tid < 64) {
      const int lane = tid;
      const int e = lane < n ? clamp_expert(ids[lane], E, status) : 0x7FFFFFFF;
      int first = lane < n ? 1 : 0;
      for (int j = 0; j < n; ++j) {
        const int ej = __builtin_amdgcn_readlane(e, j);
        first &= !(j < lane && ej == e);
      }
      int rank = 0, cnt = 0;
      for (int j = 0; j < n; ++j) {
        const int ej = __builtin_amdgcn_readlane(e, j);
        const int fj = __builtin_amdgcn_readlane(first, j);
        rank += (fj && ej < e) ? 1 : 0;
        cnt += ej == e ? 1 : 0;
      }
      // start of each union position's group: the pairs of lower positions
      int start = 0, pos = 0;
      for (int j = 0; j < n; ++j) {
        const int ej = __builtin_amdgcn_readlane(e, j);
        start += ej < e ? 1 : 0;
        pos += (j < lane && ej == e) ? 1 : 0;
      }
      const int nu = __popcll(__ballot(first != 0));
      if (lane < n) {
        L.ent_e[lane] = e;
        L.ent_u[lane] = rank;
        L.first[lane] = first;
        L.ulist[start + pos] = lane;
        if (first) {
          L.uexp[rank] = e;
          L.ucnt[rank] = cnt;
          L.ustart[rank] = start;
        }
      }
      if (lane == 0) L.nu = nu;
    }
    lds_barrier();
    return L.nu;
  }
  for (int i = tid; i < n; i += NT) L.ent_e[i] = clamp_expert(ids[i], E, status);
  lds_barrier();
  for (int i = tid; i < n; i += NT) {
    const int e = L.ent_e[i];
    int f = 1;
    for (int j = 0; j < i; ++j) f &= L.ent_e[j] != e;
    L.first[i] = f;
  }
  lds_barrier();
  for (int i = tid; i < n; i += NT) {
    const int e = L.ent_e[i];
    int rank = 0, cnt = 0;
    for (int j = 0; j < n; ++j) {
      rank += (L.first[j] && L.ent_e[j] < e) ? 1 : 0;
      cnt += L.ent_e[j] == e ? 1 : 0;
    }
    L.ent_u[i] = rank;
    if (L.first[i]) {
      L.uexp[rank] = e;
      L.ucnt[rank] = cnt;
    }
  }
  lds_barrier();
  if (tid == 0) {
    int nu = 0;
    for (int j = 0; j < n; ++j) nu += L.first[j];
    int o = 0;
    for (int u = 0; u < nu; ++u) {
      L.ustart[u] = o;
      o += L.ucnt[u];
    }
    L.nu = nu;
  }
  lds_barrier();
  for (int i = tid; i < n; i += NT) {
    const int u = L.ent_u[i];
    int pos = 0;
    for (int j = 0; j < i; ++j) pos += L.ent_u[j] == u ? 1 : 0;
    L.ulist[L.ustart[u] + pos] = i;
  }
  lds_barrier();
  return L.nu;
}

// ---------------------------------------------------------------------------
// k_bscore: batch scores of the union candidates
// ---------------------------------------------------------------------------
struct BScoreArgs {
  const int32_t* ids;
  const float* gw;
  const unsigned long long* acc;  // [B][2][ncp] screen sums (the up sums carry ||d||)
  float* bscore;                  // [B top I] (the first nu * I used)
  int32_t* meta;                  // [0] = nu, [1 + u] = u-th distinct expert
  int32_t* ghist;                 // [kHistBins] counts of key >> kHistShift (zero on entry)
  int32_t* status;
  int E, I, top, n, ncp;
};

constexpr int kBScoreThreads = 256;
constexpr int kBScoreUnroll = 4;  // pairs of one expert whose sums are in flight together
constexpr int kHistShift = 20;    // histogram bin = order key >> 20 (1/8 octave of the score)
constexpr int kHistBins = 4096;

__global__ __launch_bounds__(kBScoreThreads) void k_bscore(BScoreArgs a) {
  __shared__ SharedLds L;
  __shared__ int lh[kHistBins];
  const int tid = threadIdx.x;
  for (int b = tid; b < kHistBins; b += kBScoreThreads) lh[b] = 0;
  const int nu = build_union<kBScoreThreads>(a.ids, a.n, a.E, a.status, L);  // barriers inside
  if (blockIdx.x == 0) {
    if (tid == 0) a.meta[0] = nu;
    for (int u = tid; u < nu; u += kBScoreThreads) a.meta[1 + u] = L.uexp[u];
  }
  const int cand = blockIdx.x * kBScoreThreads + tid;
  const bool valid = cand < nu * a.I;
  const int cc = valid ? cand : 0;
  const int ux = cc / a.I, j = cc - ux * a.I;
  const int cnt = L.ucnt[ux], st = L.ustart[ux];
  float S = 0.f;
  for (int q0 = 0; q0 < cnt; q0 += kBScoreUnroll) {
    unsigned long long g[kBScoreUnroll], v[kBScoreUnroll];
    float w[kBScoreUnroll];
#pragma unroll
    for (int u = 0; u < kBScoreUnroll; ++u) {
      const int i = L.ulist[st + min(q0 + u, cnt - 1)];
      const int t = i / a.top, s = i - t * a.top;
      const size_t c = (size_t)s * a.I + j;
      g[u] = a.acc[((size_t)t * 2) * a.ncp + c];
      v[u] = a.acc[((size_t)t * 2 + 1) * a.ncp + c];
      w[u] = a.gw[i];
    }
#pragma unroll
    for (int u = 0; u < kBScoreUnroll; ++u) {
      float gh, vh, p, sc;
      (void)score_key(g[u], v[u], w[u], gh, vh, p, sc);
      if (q0 + u < cnt) S += sc;  // token-major: pairs in ascending order
    }
  }
  if (valid) {
    a.bscore[cand] = S;
    atomicAdd(&lh[order_key(S) >> kHistShift], 1);
  }
  lds_barrier();
  for (int b = tid; b < kHistBins; b += kBScoreThreads)
    if (lh[b]) atomicAdd(&a.ghist[b], lh[b]);
}

// ---------------------------------------------------------------------------
// k_btopk: exact top-k of the batch scores (one workgroup)
// ---------------------------------------------------------------------------
struct BTopkArgs {
  const float* bscore;
  const int32_t* meta;
  int32_t* ghist;  // read, then cleared for the next call
  int32_t* klist;  // [k] kept union candidates, ascending
  int32_t* krow;   // [k] their row e I + j
  uint8_t* kflag;  // [nu I] 1 = kept
  int I, k;
};

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kTopkUnroll = 8;    // keys per thread whose loads are in flight together
constexpr int kTopkList = 8192;   // keys of the boundary bin held in LDS, at most

// One workgroup.  The histogram of the batch scores' keys (k_bscore) gives
// the bin holding the k-th largest; the keys of that bin are gathered into
// LDS and ranked there digit by digit (a boundary bin larger than the LDS
// list is ranked with passes over all keys instead), giving the k-th largest
// key T and how many keys equal to T are kept (those of lowest index); a
// last walk over all keys, each wave over a contiguous range, writes the
// kept list in ascending order.
__global__ __launch_bounds__(kTopkThreads) void k_btopk(BTopkArgs a) {
  __shared__ uint32_t lkey[kTopkList];
  __shared__ int cw[kTopkWaves][2];
  __shared__ __align__(16) int sh[kTopkWaves];
  __shared__ int cnt16[16];
  __shared__ int res[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nu = a.meta[0];
  const int n = nu * a.I;
  const int kk = min(a.k, n);
  // the histogram, four bins per thread from the top, cleared once read
  constexpr int PB = kHistBins / kTopkThreads;
  int hc[PB], own = 0;
#pragma unroll
  for (int q = 0; q < PB; ++q) {
    const int b = kHistBins - 1 - (tid * PB + q);
    hc[q] = a.ghist[b];
    own += hc[q];
  }
#pragma unroll
  for (int q = 0; q < PB; ++q) a.ghist[kHistBins - 1 - (tid * PB + q)] = 0;
  const bool all = kk >= n, none = kk == 0;
  if (tid == 0) res[0] = res[1] = res[2] = 0;
  const int incl = block_scan<kTopkThreads>(own, sh);  // barriers inside
  uint32_t T = 0;
  int keep_ties = 0;
  if (!all && !none) {
    int run = incl - own;
#pragma unroll
    for (int q = 0; q < PB; ++q) {
      if (run < kk && run + hc[q] >= kk) {
        res[0] = kHistBins - 1 - (tid * PB + q);  // boundary bin
        res[1] = run;                            // keys in higher bins
      }
      run += hc[q];
    }
    if (tid == 0) cnt16[0] = 0;
    lds_barrier();
    const uint32_t bin = (uint32_t)res[0];
    int need = kk - res[1];
    // gather the boundary bin's keys
    for (int c0 = 0; c0 < n; c0 += kTopkThreads * kTopkUnroll) {
      float v[kTopkUnroll];
#pragma unroll
      for (int u = 0; u < kTopkUnroll; ++u) v[u] = a.bscore[min(c0 + u * kTopkThreads + tid, n - 1)];
#pragma unroll
      for (int u = 0; u < kTopkUnroll; ++u) {
        const int c = c0 + u * kTopkThreads + tid;
        const uint32_t key = order_key(v[u]);
        if (c < n && (key >> kHistShift) == bin) {
          const int at = atomicAdd(&cnt16[0], 1);
          if (at < kTopkList) lkey[at] = key;
        }
      }
    }
    lds_barrier();
    const int m = cnt16[0];
    const bool in_lds = m <= kTopkList;
    lds_barrier();
    // rank inside the bin: digits of 4 bits below the bin's, from the top
    uint32_t prefix = bin;
    for (int p = kHistShift / 4 - 1; p >= 0; --p) {
      const int sh4 = 4 * p;
      if (tid < 16) cnt16[tid] = 0;
      lds_barrier();
      if (in_lds) {
        for (int q = tid; q < m; q += kTopkThreads) {
          const uint32_t key = lkey[q];
          if ((key >> (sh4 + 4)) == prefix) atomicAdd(&cnt16[(key >> sh4) & 15u], 1);
        }
      } else {
        for (int c0 = 0; c0 < n; c0 += kTopkThreads * kTopkUnroll) {
          float v[kTopkUnroll];
#pragma unroll
          for (int u = 0; u < kTopkUnroll; ++u) v[u] = a.bscore[min(c0 + u * kTopkThreads + tid, n - 1)];
#pragma unroll
          for (int u = 0; u < kTopkUnroll; ++u) {
            const uint32_t key = order_key(v[u]);
            if (c0 + u * kTopkThreads + tid < n && (key >> (sh4 + 4)) == prefix)
              atomicAdd(&cnt16[(key >> sh4) & 15u], 1);
          }
        }
      }
      lds_barrier();
      if (tid == 0) {
        int run = 0;
        for (int d = 15; d >= 0; --d) {
          if (run + cnt16[d] >= need) {
            res[2] = d;
            res[3] = run;
            break;
          }
          run += cnt16[d];
        }
      }
      lds_barrier();
      prefix = (prefix << 4) | (uint32_t)res[2];
      need -= res[3];
      lds_barrier();
    }
    T = prefix;
    keep_ties = need;  // >= 1: the keep_ties ties (keys equal to T) of lowest index
  }
  // kept list in ascending order: wave w owns [w S, (w + 1) S), 64 keys a
  // step (lane l the l-th); ranks of kept keys and of ties from ballots and
  // the per-wave counts
  const int S = ((n + kTopkWaves - 1) / kTopkWaves + 63) / 64 * 64;
  const int sb = min(wave * S, n), se = min(sb + S, n);
  int wgt = 0, wtie = 0;
  for (int c0 = sb; c0 < se; c0 += 64 * kTopkUnroll) {
    float v[kTopkUnroll];
#pragma unroll
    for (int u = 0; u < kTopkUnroll; ++u) v[u] = a.bscore[min(c0 + u * 64 + lane, n - 1)];
#pragma unroll
    for (int u = 0; u < kTopkUnroll; ++u) {
      const bool in = c0 + u * 64 + lane < se;
      const uint32_t key = order_key(v[u]);
      wgt += __popcll(__ballot(in && key > T));
      wtie += __popcll(__ballot(in && key == T));
    }
  }
  if (lane == 0) {
    cw[wave][0] = wgt;
    cw[wave][1] = wtie;
  }
  lds_barrier();
  int gt0 = 0, tie0 = 0;
  for (int q = 0; q < wave; ++q) {
    gt0 += cw[q][0];
    tie0 += cw[q][1];
  }
  // a wave's kept keys start after the kept keys of the waves before it
  int pos = all ? sb : (none ? 0 : gt0 + min(tie0, keep_ties));
  int tie_rank = tie0;
  const int* uexp = a.meta + 1;
  for (int c0 = sb; c0 < se; c0 += 64 * kTopkUnroll) {
    float v[kTopkUnroll];
#pragma unroll
    for (int u = 0; u < kTopkUnroll; ++u) v[u] = a.bscore[min(c0 + u * 64 + lane, n - 1)];
#pragma unroll
    for (int u = 0; u < kTopkUnroll; ++u) {
      const int c = c0 + u * 64 + lane;
      const bool in = c < se;
      const uint32_t key = order_key(v[u]);
      const bool tie = in && !all && key == T;
      const unsigned long long tb = __ballot(tie);
      const bool kp = in && (all || (!none && (key > T || (tie && tie_rank + lanes_below_mask(tb) < keep_ties))));
      const unsigned long long kb = __ballot(kp);
      if (in) a.kflag[c] = kp ? 1 : 0;
      if (kp) {
        const int at = pos + lanes_below_mask(kb);
        a.klist[at] = c;
        const int ux = c / a.I;
        a.krow[at] = uexp[ux] * a.I + (c - ux * a.I);
      }
      pos += __popcll(kb);
      tie_rank += __popcll(tb);
    }
  }
}

// ---------------------------------------------------------------------------
// k_bact: coefficients w a_j of the kept channels per token, and the
// per-token recovery partials
// ---------------------------------------------------------------------------
struct BActArgs {
  const float* x;       // [B][H]
  const int32_t* ids;   // [B][top]
  const float* gw;      // [B][top]
  const uint16_t* w3;   // [E][I][3][H]
  const uint16_t* bmat; // [E][I][rank] fp16
  const float* norms;   // [E][I]
  const unsigned long long* acc;
  const int32_t* klist;
  const int32_t* krow;
  const uint8_t* kflag;
  float* coef;   // [k][B]
  float* zpart;  // [B][Z][rank]
  int32_t* status;
  int H, E, I, top, B, n, ncp, k, rank, Ga, Z;
};

constexpr int kBActThreads = 256;
constexpr int kBActWaves = kBActThreads / 64;
constexpr int kBActU = 4;  // kept channels per wave, rows in flight together
constexpr int kBRecUnroll = 2;  // candidates per thread with loads in flight together

template <int NCH>
__global__ __launch_bounds__(kBActThreads) void k_bact(BActArgs a) {
  extern __shared__ float4 bact_lds[];  // [B][H] the tokens (activation workgroups)
  __shared__ SharedLds L;
  __shared__ float zw[kBActWaves][kMaxRank];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H, I = a.I, B = a.B;
  const int w = blockIdx.x;
  if (w < a.Ga) {
    float* xs = reinterpret_cast<float*>(bact_lds);
    {
      // the B tokens (at most 8 x 4096 floats: 32 float4 per thread), every
      // load issued before the first store
      constexpr int XU = kMaxSharedBatch * kMaxHidden / 4 / kBActThreads;
      float4 xv[XU];
#pragma unroll
      for (int u = 0; u < XU; ++u) {
        const int h = (u * kBActThreads + tid) * 4;
        xv[u] = *reinterpret_cast<const float4*>(a.x + min(h, B * H - 4));
      }
#pragma unroll
      for (int u = 0; u < XU; ++u) {
        const int h = (u * kBActThreads + tid) * 4;
        if (h < B * H) *reinterpret_cast<float4*>(xs + h) = xv[u];
      }
    }
    const int nu = build_union<kBActThreads>(a.ids, a.n, a.E, a.status, L);  // barriers inside
    const int kk = min(a.k, nu * I);
    const int q0 = (w * kBActWaves + wave) * kBActU;
    if (q0 >= kk) return;
    const int nq = min(kBActU, kk - q0);
    int ux[kBActU];
    uint4 gq[kBActU][NCH], uq[kBActU][NCH];
#pragma unroll
    for (int r = 0; r < kBActU; ++r) {
      const int c = a.klist[q0 + min(r, nq - 1)];
      ux[r] = c / I;
      const uint16_t* row = a.w3 + (size_t)a.krow[q0 + min(r, nq - 1)] * 3 * H;  // BF16 rows
#pragma unroll
      for (int ch = 0; ch < NCH; ++ch) {
        const int h = min(ch * 512 + lane * 8, H - 8);  // clamped; the tail is masked below
        // streamed, like the row chunks of the per-token gather
        const u32x4_t g4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row + h));
        const u32x4_t u4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row + H + h));
        gq[r][ch] = make_uint4(g4.x, g4.y, g4.z, g4.w);
        uq[r][ch] = make_uint4(u4.x, u4.y, u4.z, u4.w);
      }
    }
#pragma unroll
    for (int r = 0; r < kBActU; ++r) {
      if (r >= nq) break;  // wave-uniform
      float cv[kMaxSharedBatch];
#pragma unroll
      for (int t = 0; t < kMaxSharedBatch; ++t) cv[t] = 0.f;
      const int cnt = L.ucnt[ux[r]], st = L.ustart[ux[r]];
      for (int e = 0; e < cnt; ++e) {
        const int i = L.ulist[st + e];
        const int t = i / a.top;
        const float* xt = xs + (size_t)t * H;
        float gs = 0.f, vs = 0.f;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
          const int h = ch * 512 + lane * 8;
          if (h < H) {
            const float4 xa = *reinterpret_cast<const float4*>(xt + h);
            const float4 xb = *reinterpret_cast<const float4*>(xt + h + 4);
            const float xv[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
            const uint32_t g4[4] = {gq[r][ch].x, gq[r][ch].y, gq[r][ch].z, gq[r][ch].w};
            const uint32_t u4[4] = {uq[r][ch].x, uq[r][ch].y, uq[r][ch].z, uq[r][ch].w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              gs = fmaf(bf_lo(g4[p]), xv[2 * p], gs);
              gs = fmaf(bf_hi(g4[p]), xv[2 * p + 1], gs);
              vs = fmaf(bf_lo(u4[p]), xv[2 * p], vs);
              vs = fmaf(bf_hi(u4[p]), xv[2 * p + 1], vs);
            }
          }
        }
        const float av = a.gw[i] * silu(wave_sum(gs)) * wave_sum(vs);
#pragma unroll
        for (int tt = 0; tt < kMaxSharedBatch; ++tt) cv[tt] += tt == t ? av : 0.f;
      }
#pragma unroll
      for (int t = 0; t < kMaxSharedBatch; ++t)
        if (lane == t && t < B) a.coef[(size_t)(q0 + r) * B + t] = cv[t];
    }
    return;
  }

  // recovery workgroup zq of token t: candidates [zq cz, (zq + 1) cz) of the
  // token's top * I, every load issued before any is used (a kept
  // candidate's b row is read at a clamped address and weighted 0)
  const int nu = build_union<kBActThreads>(a.ids, a.n, a.E, a.status, L);
  (void)nu;
  const int t = (w - a.Ga) / a.Z, zq = (w - a.Ga) - t * a.Z;
  const int nc = a.top * I, cz = (nc + a.Z - 1) / a.Z;
  const int R = a.rank;
  float z[kMaxRank];
#pragma unroll
  for (int r = 0; r < kMaxRank; ++r) z[r] = 0.f;
  const int cb = zq * cz, ce = min(nc, cb + cz);
  for (int c0 = cb + tid; c0 < ce; c0 += kBActThreads * kBRecUnroll) {
    uint4 bq[kBRecUnroll][kMaxRank / 8];
    float coef[kBRecUnroll];
#pragma unroll
    for (int u = 0; u < kBRecUnroll; ++u) {
      const int cr = c0 + u * kBActThreads;
      const int c = min(cr, ce - 1);
      const int s = c / I, j = c - s * I;
      const int i = t * a.top + s;
      const int ux = L.ent_u[i], e = L.ent_e[i];
      const uint8_t kept = a.kflag[(size_t)ux * I + j];
      const unsigned long long g = a.acc[((size_t)t * 2) * a.ncp + c];
      const unsigned long long v = a.acc[((size_t)t * 2 + 1) * a.ncp + c];
      const float nd = a.norms[(size_t)e * I + j];
      const float wi = a.gw[i];
      const uint4* bp = reinterpret_cast<const uint4*>(a.bmat + ((size_t)e * I + j) * R);
#pragma unroll
      for (int r8 = 0; r8 < kMaxRank / 8; ++r8) bq[u][r8] = bp[r8 * 8 < R ? r8 : 0];
      float gh, vh, p, sc;
      (void)score_key(g, v, wi, gh, vh, p, sc);
      // p' = ||d_j|| p; a zero norm means b_j = U^T d_j = 0
      coef[u] = (cr < ce && !kept && nd > 0.f) ? wi * (p / nd) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kBRecUnroll; ++u) {
#pragma unroll
      for (int r8 = 0; r8 < kMaxRank / 8; ++r8) {
        if (r8 * 8 < R) {
          const uint32_t bw[4] = {bq[u][r8].x, bq[u][r8].y, bq[u][r8].z, bq[u][r8].w};
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            z[r8 * 8 + 2 * d] = fmaf(coef[u], lo16(bw[d]), z[r8 * 8 + 2 * d]);
            z[r8 * 8 + 2 * d + 1] = fmaf(coef[u], hi16(bw[d]), z[r8 * 8 + 2 * d + 1]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kMaxRank; ++r) {
    if (r < R) {
      const float v = wave_sum(z[r]);
      if (lane == 0) zw[wave][r] = v;
    }
  }
  lds_barrier();
  if (tid < R) {
    float v = 0.f;
#pragma unroll
    for (int q = 0; q < kBActWaves; ++q) v += zw[q][tid];
    a.zpart[((size_t)t * a.Z + zq) * R + tid] = v;
  }
}

// ---------------------------------------------------------------------------
// k_bdown: partial outputs, sum over a range of kept channels of
// coefficient x down row, per token
// ---------------------------------------------------------------------------
struct BDownArgs {
  const uint16_t* w3;
  const int32_t* krow;
  const int32_t* meta;
  const float* coef;  // [k][B]
  float* ypart;       // [B][G][H]
  int H, I, B, k, G, qc, nhs;
};

constexpr int kBDownThreads = 256;  // four waves, each over a quarter of the range
constexpr int kBDownWaves = kBDownThreads / 64;
constexpr int kBDownSlice = 512;    // hidden units per workgroup: 8 per lane (16-byte loads)
constexpr int kBDownRows = 8;       // down rows in flight per wave

// Workgroup (range g of qc kept channels, hidden slice hs): wave v sums
// channels v, v + 4, ... of the range into its registers (8 hidden units
// per lane, every token); the four waves' sums are added in LDS in a fixed
// order.
__global__ __launch_bounds__(kBDownThreads) void k_bdown(BDownArgs a) {
  __shared__ float red[kBDownWaves - 1][kMaxSharedBatch][kBDownSlice];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = blockIdx.x / a.nhs, hs = blockIdx.x - g * a.nhs;
  const int H = a.H, B = a.B;
  const int h0 = hs * kBDownSlice + lane * 8;
  const bool hown = h0 < H;
  const int kk = min(a.k, a.meta[0] * a.I);
  const int r0 = min(g * a.qc, kk), r1 = min(r0 + a.qc, kk);
  float y[kMaxSharedBatch][8];
#pragma unroll
  for (int t = 0; t < kMaxSharedBatch; ++t)
#pragma unroll
    for (int i = 0; i < 8; ++i) y[t][i] = 0.f;
  const uint16_t* dbase = a.w3 + 2 * H + min(h0, H - 8);
  for (int q0 = r0 + wave; q0 < r1; q0 += kBDownWaves * kBDownRows) {
    uint4 dq[kBDownRows];
    float cf[kBDownRows][kMaxSharedBatch];
#pragma unroll
    for (int u = 0; u < kBDownRows; ++u) {
      const int q = min(q0 + u * kBDownWaves, r1 - 1);
      const u32x4_t d4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(dbase + (size_t)a.krow[q] * 3 * H));
      dq[u] = make_uint4(d4.x, d4.y, d4.z, d4.w);  // streamed
#pragma unroll
      for (int t = 0; t < kMaxSharedBatch; ++t)
        cf[u][t] = (t < B && q0 + u * kBDownWaves < r1) ? a.coef[(size_t)q * B + t] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kBDownRows; ++u) {
      const uint32_t w4[4] = {dq[u].x, dq[u].y, dq[u].z, dq[u].w};
#pragma unroll
      for (int t = 0; t < kMaxSharedBatch; ++t)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          y[t][2 * p] = fmaf(cf[u][t], bf_lo(w4[p]), y[t][2 * p]);
          y[t][2 * p + 1] = fmaf(cf[u][t], bf_hi(w4[p]), y[t][2 * p + 1]);
        }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < kMaxSharedBatch; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) red[wave - 1][t][lane * 8 + i] = y[t][i];
  }
  __syncthreads();
  if (wave == 0 && hown) {
#pragma unroll
    for (int t = 0; t < kMaxSharedBatch; ++t) {
      if (t < B) {
        float* yp = a.ypart + ((size_t)t * a.G + g) * H + h0;
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = y[t][i] + red[0][t][lane * 8 + i] + red[1][t][lane * 8 + i] +
                                           red[2][t][lane * 8 + i];
        *reinterpret_cast<float4*>(yp) = make_float4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<float4*>(yp + 4) = make_float4(o[4], o[5], o[6], o[7]);
      }
    }
  }
}

template <int NCH>
hipError_t launch_bact_t(const BActArgs& a, size_t lds, hipStream_t st) {
  static OncePerDevice attr;
  attr([] {
    (void)hipFuncSetAttribute((const void*)k_bact<NCH>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)(kMaxSharedBatch * kMaxHidden * 4));
    (void)hipGetLastError();
  });
  k_bact<NCH><<<a.Ga + a.B * a.Z, kBActThreads, lds, st>>>(a);
  return hipGetLastError();
}

}  // namespace

SharedPlan make_shared_plan(const cfr_config& c, int batch, int k) {
  SharedPlan p;
  const int nmax = std::min(c.n_experts, batch * c.top);
  p.nscore = (nmax * c.inter + kBScoreThreads - 1) / kBScoreThreads;
  p.Ga = std::max(1, (k + kBActWaves * kBActU - 1) / (kBActWaves * kBActU));
  p.Z = c.rank > 0 ? kMaxRecoverWgs : 0;
  // partial outputs: G per token, batch G <= kMaxGatherWgs rows in all
  const int gmax = std::max(1, kMaxGatherWgs / batch);
  p.qc = std::max(64, (k + gmax - 1) / gmax);
  p.G = std::max(1, (k + p.qc - 1) / p.qc);
  p.nhs = (c.hidden + kBDownSlice - 1) / kBDownSlice;
  p.nch = 1;
  while (p.nch * 512 < c.hidden) p.nch *= 2;
  return p;
}

hipError_t launch_shared_select(const cfr_reader& r, const float* x, const int32_t* ids, const float* gw,
                                int batch, int k, const Workspace& W, const SharedPlan& p, hipStream_t st) {
  const cfr_config& c = r.cfg;
  const int n = batch * c.top;
  BScoreArgs s{ids, gw, W.acc, W.bscore, W.meta, W.ghist, r.status, c.n_experts, c.inter, c.top, n, r.ncp};
  k_bscore<<<p.nscore, kBScoreThreads, 0, st>>>(s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  BTopkArgs t{W.bscore, W.meta, W.ghist, W.klist, W.krow, W.kflag, c.inter, k};
  k_btopk<<<1, kTopkThreads, 0, st>>>(t);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const uint16_t* w3 = reinterpret_cast<const uint16_t*>(r.w3);  // BF16 rows (the API refuses 4-bit ones)
  BActArgs ba{x, ids, gw, w3, r.b, r.norms, W.acc, W.klist, W.krow, W.kflag, W.coef, W.zpart, r.status,
              c.hidden, c.n_experts, c.inter, c.top, batch, n, r.ncp, k, c.rank, p.Ga, p.Z};
  const size_t lds = sizeof(float) * (size_t)batch * c.hidden;
  switch (p.nch) {
    case 1: e = launch_bact_t<1>(ba, lds, st); break;
    case 2: e = launch_bact_t<2>(ba, lds, st); break;
    case 4: e = launch_bact_t<4>(ba, lds, st); break;
    default: e = launch_bact_t<8>(ba, lds, st); break;
  }
  if (e != hipSuccess) return e;
  BDownArgs bd{w3, W.krow, W.meta, W.coef, W.ypart, c.hidden, c.inter, batch, k, p.G, p.qc, p.nhs};
  k_bdown<<<p.G * p.nhs, kBDownThreads, 0, st>>>(bd);
  return hipGetLastError();
}

}  // namespace cfr

// Launchers of the device kernels (HIP translation units only).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>

#include "cfr_internal.h"

namespace cfr {

constexpr size_t kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int kScreenThreads = 512;     // screen workgroup size
constexpr int kScreenMinWgs = 512;     // screen workgroups a block group may leave at batch >= 2
constexpr int kMaxGatherWgs = 256;      // gather workgroups per call, summed over the batch
constexpr int kMaxRecoverWgs = 16;      // recovery workgroups per token
constexpr int kReduceSlice = 32;        // hidden units per reduce workgroup

__host__ __device__ inline size_t lds_align(size_t v) { return (v + 15) / 16 * 16; }

// Thread geometry of the select/gather kernel for nc candidates per token:
// nt threads, each owning `per` candidates taken in pairs (pair P = i nt + tid
// holds candidates 2P and 2P + 1, so a wave's loads of the screen sums are
// contiguous).  Per-token candidate arrays are padded to nt * per entries;
// the padding is never written and stays zero.
struct SelectGeom {
  int nt, per;
};
__host__ __device__ inline SelectGeom select_geom(int nc) {
  const int nt = 512;
  int per = (nc + nt - 1) / nt;
  per = (per + 1) / 2 * 2;
  if (per < 2) per = 2;
  if (per > 8 && per <= 12) per = 12;
  if (per > 12 && per <= 16) per = 16;
  if (per > 16 && per <= 24) per = 24;
  if (per > 24) per = 32;
  return {nt, per};
}

// LDS layout of the select/gather kernel (bytes); host and device share it.
//   xs     fp32 [H]          the token (gather workgroups)
//   pv     fp32 [ncp]        p of every candidate (recovery workgroups)
//   dl     u32 [ncp]         key distance d of every candidate (recovery)
//   flags  u8 [ncp]          kept flag of every candidate (recovery, debug)
//   yred   fp32 [S][H]       partial outputs, S = NT/64 slots for H <= 2048
//                            else NT/128 (gather workgroups; shares the
//                            space of pv, dl and flags)
//   hist   int [2048]        selection histogram
//   list   int [chan]        this workgroup's kept candidates, by rank
//   misc   int [64]          scan scratch and broadcast values
//   bmem   int2 [64]         the boundary set, when ranked directly
//   wcnt   int [256]         per-wave counts of the ordered prefix sums
//   slot   int [16] + fp32 [16]  routed expert and weight per slot
//   zred   fp32 [NT/64][64]  per-wave recovery sums
struct GatherLds {
  size_t xs, pv, dl, flags, yred, hist, list, misc, bmem, wcnt, slot_e, slot_w, zred, total;
  __host__ __device__ GatherLds(int H, int ncp, int nt, int chan) {
    size_t o = 0;
    xs = o;
    o += lds_align((size_t)H * 4);
    const size_t rec = 2 * lds_align((size_t)ncp * 4) + lds_align((size_t)ncp);
    const size_t red = (size_t)(H <= 2048 ? nt / 64 : nt / 128) * H * 4;
    pv = o;
    dl = o + lds_align((size_t)ncp * 4);
    flags = o + 2 * lds_align((size_t)ncp * 4);
    yred = o;
    o += rec > red ? rec : red;
    hist = o;
    o += 2048 * 4;
    list = o;
    o += lds_align((size_t)(chan > 0 ? chan : 1) * 4);
    misc = o;
    o += 64 * 4;
    bmem = o;
    o += 64 * 8;
    wcnt = o;
    o += 256 * 4;
    slot_e = o;
    o += 16 * 4;
    slot_w = o;
    o += 16 * 4;
    zred = o;
    o += (size_t)nt * 4;
    total = o;
  }
};

// Launch geometry of one decode call.
struct Plan {
  // screen: one workgroup per (token, routed slot, group of bg blocks, half)
  int items1 = 0, per_xcd1 = 0, bg = 1;
  int nd = 0;  // 32-bit code words per half-unit that hold codes
  int ng = 0;  // screened-coordinate groups per workgroup
  size_t lds1 = 0;
  // select/gather
  int nt2 = 512, per = 4, ncp = 0, nch = 1, cpw = 1, chan = 1, G = 1, Z = 0;
  size_t lds2 = 0;
  // reduce
  int nslices = 0;
};
Plan make_plan(const cfr_config& c, int batch, int k);
size_t max_lds_needed(const cfr_config& c);  // over every batch and k the config allows

// Intermediates copied out by the debug entry point (any may be null).
struct DebugOut {
  float* xrot = nullptr;
  uint8_t* sel = nullptr;
  float* ghat = nullptr;
  float* vhat = nullptr;
  float* score = nullptr;
  int32_t* kept = nullptr;
};

// only: -1 launches every stage; 0, 1 or 2 launches that stage's kernel alone
int launch_decode(cfr_reader* r, const float* x, const int32_t* ids, const float* gw, int batch,
                  int k, float* y, hipStream_t stream, const DebugOut* dbg,
                  hipEvent_t* stage_events = nullptr /* CFR_NUM_STAGES + 1 or null */, int only = -1,
                  const float* resid = nullptr /* non-null: y = resid + output */,
                  const Workspace* ws = nullptr /* null: the reader's own workspace */);
// Zero a device buffer (a multiple of 16 bytes) with a fill kernel on st.
hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);
// The decode's buffers for `batch` tokens carved from base (any size when
// base is null); returns the bytes they take.  debug: also the copies the
// debug entry point reads.
// shared: also the buffers of the batch-shared decode.
size_t carve_decode_workspace(const cfr_reader& r, int batch, bool debug, char* base, Workspace* w,
                              bool shared = false);
// Bytes at the start of that carve that must be zero when a decode starts
// (the screen sums; a decode leaves them zero).
size_t decode_sums_bytes(const cfr_reader& r, int batch);
// Kernel attributes (hipFuncSetAttribute) apply to the current device: a
// launcher sets them once per device, the first time it runs there.  Setting
// them twice (two threads at once) is harmless.
constexpr int kMaxDevices = 64;
struct OncePerDevice {
  std::atomic<bool> done[kMaxDevices] = {};
  template <typename F>
  void operator()(F&& set) {
    int d = 0;
    const bool known = hipGetDevice(&d) == hipSuccess && d >= 0 && d < kMaxDevices;
    if (known && done[d].load(std::memory_order_acquire)) return;
    set();
    if (known) done[d].store(true, std::memory_order_release);
  }
};

// Softmax top-k routing (route_kernel.hip): dynamic LDS bytes of the pick and the
// launch (logits into logits[batch][E]; arrived[batch] must be zero before
// the first call and is zero again after each).
size_t route_lds_bytes(const cfr_config& c);
// eps < 0: route on x; else on h = RMSNorm(x) (unit weights), written to h.
hipError_t launch_route(const float* x, const uint16_t* router, const cfr_config& c, int batch, float eps,
                        float* h, float* logits, int* arrived, int32_t* ids, float* gw, int32_t* status,
                        hipStream_t st);
int launch_dense(cfr_reader* r, const float* x, const int32_t* ids, const float* gw, int batch,
                 float* y, hipStream_t stream, const float* resid = nullptr);

// The dense block's streaming kernel (dense_kernel.hip): G workgroups per
// token over `chan` channels each, `cpw` per wave, u in flight per wave,
// writing G partial outputs per token into ypart[batch][G][H].
struct DensePlan {
  int G = 1, chan = 1, cpw = 1, nch = 1, u = 1;
  size_t lds = 0;
};
DensePlan make_dense_plan(const cfr_config& c, int batch);
hipError_t launch_dense_block(const float* x, const int32_t* ids, const float* gw, const uint8_t* w3,
                              float* ypart, int32_t* status, const cfr_config& c, int batch,
                              const DensePlan& p, hipStream_t st);

// Batch-shared selection (shared_kernels.hip): after the screen kernel, the
// batch scores (nscore workgroups), the batch top-k (one workgroup), the
// kept channels' coefficients (Ga workgroups) with batch * Z recovery
// workgroups writing zpart [batch][Z][rank], then G ranges of qc kept
// channels times nhs hidden slices writing ypart [batch][G][H], for the
// reduce kernel.
struct SharedPlan {
  int nscore = 1, Ga = 1, Z = 0, qc = 64, G = 1, nhs = 1, nch = 1;
};
SharedPlan make_shared_plan(const cfr_config& c, int batch, int k);
hipError_t launch_shared_select(const cfr_reader& r, const float* x, const int32_t* ids, const float* gw,
                                int batch, int k, const Workspace& W, const SharedPlan& p, hipStream_t st);
// Batch-shared decode (screen, shared selection, reduce); debug copies of the
// batch scores, kept list and union when the pointers are non-null.
int launch_decode_shared(cfr_reader* r, const float* x, const int32_t* ids, const float* gw, int batch,
                         int k, float* y, hipStream_t st, const float* resid, float* bscore_out,
                         int32_t* kept_out, int32_t* meta_out);

// Load step (3) on the device: U (fp16 [H][rank]) and b (fp16 [E][I][rank])
// from the resident down rows.  Synchronous.
int device_lowrank(cfr_reader* r);

}  // namespace cfr

// Launchers of the device kernels (HIP translation units only).
#pragma once

#include <hip/hip_runtime.h>

#include "cfr_internal.h"

namespace cfr {

constexpr size_t kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950

__host__ __device__ inline size_t lds_align(size_t v) { return (v + 15) / 16 * 16; }

// LDS layout of the screen kernel (bytes); host and device share it.
struct ScreenLds {
  size_t lut, sl, rec, sc, red, total;
  __host__ __device__ ScreenLds(int nblk, int n_screen, int S, int nthreads) {
    size_t o = 0;
    lut = o;  // 256 entries of five fp16 codes
    o += 256 * 16;
    sl = o;
    o += lds_align((size_t)nblk * n_screen);
    rec = o;
    o += lds_align((size_t)nblk * n_screen * 8);
    sc = o;
    o += lds_align((size_t)nblk * 2 * 5 * S * 4);
    red = o;
    o += lds_align((size_t)nthreads * 5 * S * 4);
    total = o;
  }
};

// LDS layout of the select/exact kernel (bytes).
struct SelectLds {
  size_t xs, keys, flags, list, zred, hist, misc, total;
  __host__ __device__ SelectLds(int H, int ncand, int share_max, int rank) {
    size_t o = 0;
    xs = o;
    o += lds_align((size_t)H * 4);
    const size_t npad = (size_t)256 * ((ncand + 255) / 256);  // whole chunks of 256 threads
    keys = o;
    o += lds_align(npad * 4);
    flags = o;
    o += lds_align(npad);
    list = o;
    o += lds_align((size_t)(share_max > 0 ? share_max : 1) * 4);
    zred = o;
    o += lds_align((size_t)4 * (rank > 0 ? rank : 1) * 4);
    hist = o;
    o += (4096 + 2048) * 4;
    misc = o;
    o += lds_align(192 * 4);
    total = o;
  }
};

// Launch geometry of one decode call.
struct Plan {
  int S = 1, n_slices = 1, itemsA = 0, per_xcdA = 0, ntA = 512;  // screen
  int G = 4, share_max = 0, ZW = 4;                          // select/exact
  int HS = 8, nhs = 0, itemsC = 0, per_xcdC = 0;             // down/recover
  size_t ldsA = 0, ldsB = 0;
};
Plan make_plan(const cfr_config& c, int batch, int k);
size_t max_lds_needed(const cfr_config& c);  // over every batch and k the config allows
size_t zpart_rows(const cfr_config& c);      // rows of the recovery partial buffer

// Intermediates copied out by the debug entry point (any may be null).
struct DebugOut {
  float* xrot = nullptr;
  uint8_t* sel = nullptr;
  float* ghat = nullptr;
  float* vhat = nullptr;
  float* score = nullptr;
  int32_t* kept = nullptr;
};

int launch_decode(cfr_reader* r, const float* x, const int32_t* ids, const float* gw, int batch,
                  int k, float* y, hipStream_t stream, const DebugOut* dbg,
                  hipEvent_t* stage_events = nullptr /* CFR_NUM_STAGES + 1 or null */);
int launch_dense(cfr_reader* r, const float* x, const int32_t* ids, const float* gw, int batch,
                 float* y, hipStream_t stream);

// Load step (3) on the device: U (fp16 [H][rank]) and b (fp16 [E][I][rank])
// from the resident down rows.  Synchronous.
int device_lowrank(cfr_reader* r);

}  // namespace cfr

// Launchers of the device kernels (HIP translation units only).
#pragma once

#include <hip/hip_runtime.h>

#include "cfr_internal.h"

namespace cfr {

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

// Internal declarations shared by the library's translation units.
#pragma once

#include <stdint.h>
#include <stddef.h>

#include <string>

#include "../../include/cfr.h"

namespace cfr {

constexpr int kBlock = 128;                      // rotation block
constexpr double kSqrt128 = 11.313708498984761;  // sqrt(128) rounded to the nearest double
constexpr int kMaxInter = 4096;
constexpr int kMaxTop = 16;
constexpr int kMaxRank = 64;
constexpr int kMaxBatch = 64;
constexpr int kMaxHidden = 4096;
constexpr int kMaxSharedBatch = 8;  // tokens of one batch-shared decode

// Error reporting (thread-local message).
int fail(int code, const std::string& msg);
void clear_error();

// Geometry of one sketch unit for I channels: each half (gate, up) holds five
// codes per byte, padded to a multiple of 16 bytes; the unit is padded to a
// multiple of 32 bytes (whole sectors).
inline int half_bytes(int inter) {
  int lp = (inter + 4) / 5;
  return (lp + 15) / 16 * 16;
}
inline int unit_bytes(int inter) { return (2 * half_bytes(inter) + 31) / 32 * 32; }

int validate_config(const cfr_config* c);

// Exact rows in 4 bits (cfr_config.exact_bits == 4) rather than BF16.
inline bool q4_rows(const cfr_config& c) { return c.exact_bits == 4; }
// Bytes of one resident row of H weights: BF16, or the 4-bit record (H/2
// bytes of codes, H/128 fp16 group scales, H/128 byte zero points) padded to
// a multiple of 16 bytes.
inline int row_bytes(int H, bool q4) { return q4 ? ((H / 2 + 3 * (H / 128)) + 15) / 16 * 16 : 2 * H; }

// Host pack (load steps 1, 2 and 4).  Writes into caller buffers; any may be null.
//   w3: [E][I][3][H] bf16 (gate row, up row, down column) — the resident layout.
int pack_host(const cfr_config& c, const uint16_t* gate, const uint16_t* up,
              const uint16_t* down, uint8_t* codes, uint16_t* scales, uint16_t* rho,
              float* norms, uint16_t* w3, float* sigma);

// The same from real-valued weights (a dequantized 4-bit checkpoint; no
// resident BF16 layout).
int pack_host_f32(const cfr_config& c, const float* gate, const float* up, const float* down,
                  uint8_t* codes, uint16_t* scales, uint16_t* rho, float* norms, float* sigma_out);
// Weights of one 4-bit row record of H weights (see row_bytes).
int dequant_q4_record(const uint8_t* rec, int H, float* out);

void sign_vector(uint64_t seed, int hidden, float* out);
uint16_t f64_to_f16_rne(double v);
double f16_to_f64(uint16_t h);

// The decode's per-call device buffers (views into one block of device
// memory: the reader's workspace, or the allocation-free entry point's
// static array).
struct Workspace {
  unsigned long long* acc = nullptr;  // [B][2][ncp] fixed-point screen sums (gate, up); zero between calls
  float* var = nullptr;               // [B][2][ncp] sketch-error variances (expected-error ranking)
  float* ypart = nullptr;             // [kMaxGatherWgs][H] partial outputs of the gather workgroups
  float* zpart = nullptr;             // [B][kMaxRecoverWgs][rank] partial recovery vectors
  float* xrot = nullptr;    // [B][H]   H_128 (sigma x) per block (debug copy only)
  uint8_t* sel = nullptr;   // [B][nblk][n_screen] (debug copy only)
  float* ghat = nullptr;    // [B][ncand] (debug copy only)
  float* vhat = nullptr;    // [B][ncand] (debug copy only)
  float* score = nullptr;   // [B][ncand] (debug copy only)
  int32_t* kept = nullptr;  // [B][ncand]  kept candidates by rank (debug copy only)
  // batch-shared selection (the reader's own workspace only)
  float* bscore = nullptr;  // [B top I] batch scores of the union candidates
  int32_t* meta = nullptr;  // [1 + B top] union size, then the union's experts ascending
  int32_t* klist = nullptr; // [B top I] kept union candidates, ascending
  uint8_t* kflag = nullptr; // [B top I] kept flag per union candidate
  float* coef = nullptr;    // [B top I][B] w a_j of each kept channel per token
  int32_t* krow = nullptr;  // [B top I] row e I + j of each kept union candidate
  int32_t* ghist = nullptr; // [4096] histogram of the batch scores' keys; zero between calls
};

}  // namespace cfr

// The reader object.  All pointers are device memory on cfg.device unless
// noted.  Workspace pointers are views into one allocation.
struct cfr_reader {
  cfr_config cfg;
  int nblk, lp, unit, ncand;
  int ncp = 0;  // candidates per token padded for the select kernel (select_geom)
  // resident state
  uint8_t* w3 = nullptr;       // [E][I][3] rows of row_bytes(H) bytes: BF16, or 4-bit records
  uint8_t* codes = nullptr;    // [E][nblk][128][unit]
  uint16_t* scales = nullptr;  // [E][nblk][2][I] fp16
  uint16_t* rho = nullptr;     // [E][nblk][2][I] fp16
  float* norms = nullptr;      // [E][I]
  uint16_t* u = nullptr;       // [H][rank] fp16
  uint16_t* b = nullptr;       // [E][I][rank] fp16
  float* sigma = nullptr;      // [H] +1 / -1
  uint16_t* router = nullptr;  // [E][H] bf16 or null
  // workspace (sized for cfg.max_batch); one allocation, zeroed once
  void* ws = nullptr;
  size_t ws_bytes = 0;
  float* rlog = nullptr;       // [B][E] router logits (cfr_reader_route)
  int32_t* rarr = nullptr;     // [B] workgroups of the route that have finished; zero between calls
  cfr::Workspace wk;           // the decode's buffers, views into ws
  int32_t* status = nullptr;   // [1]
};

// Host-only parts of the C ABI: errors, config validation, sizes, read
// accounting and the host pack entry point.  No HIP calls in this file.
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "cfr_internal.h"

namespace cfr {

static thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

void clear_error() { g_last_error.clear(); }

int validate_config(const cfr_config* c) {
  if (!c) return fail(CFR_EINVAL, "config is NULL");
  if (c->hidden <= 0 || c->hidden % kBlock != 0)
    return fail(CFR_EINVAL, "hidden must be a positive multiple of 128");
  if (c->hidden > kMaxHidden) return fail(CFR_EUNSUPPORTED, "hidden above 4096");
  if (c->n_experts <= 0) return fail(CFR_EINVAL, "n_experts must be positive");
  if (c->inter <= 0) return fail(CFR_EINVAL, "inter must be positive");
  if (c->inter > kMaxInter) return fail(CFR_EUNSUPPORTED, "inter above 4096");
  if (c->top <= 0 || c->top > c->n_experts) return fail(CFR_EINVAL, "top must be in 1..n_experts");
  if (c->top > kMaxTop) return fail(CFR_EUNSUPPORTED, "top above 16");
  if (c->rank < 0 || c->rank > c->hidden) return fail(CFR_EINVAL, "rank must be in 0..hidden");
  if (c->rank > kMaxRank) return fail(CFR_EUNSUPPORTED, "rank above 64");
  if (c->rank % 8 != 0) return fail(CFR_EUNSUPPORTED, "rank must be a multiple of 8");
  if ((int64_t)c->top * c->inter > 16384)
    return fail(CFR_EUNSUPPORTED, "top * inter above 16384 candidates per token");
  if (c->n_screen < 1 || c->n_screen > kBlock) return fail(CFR_EINVAL, "n_screen must be in 1..128");
  if (c->max_batch < 1) return fail(CFR_EINVAL, "max_batch must be at least 1");
  if (c->max_batch > kMaxBatch) return fail(CFR_EUNSUPPORTED, "max_batch above 64");
  if (c->device < 0) return fail(CFR_EINVAL, "device must be non-negative");
  if (c->ranking != CFR_RANK_SCORE && c->ranking != CFR_RANK_EXPECTED_ERROR)
    return fail(CFR_EINVAL, "ranking must be CFR_RANK_SCORE or CFR_RANK_EXPECTED_ERROR");
  if (c->ranking == CFR_RANK_EXPECTED_ERROR && c->n_screen != kBlock)
    return fail(CFR_EINVAL, "the expected-error ranking reads the whole sketch: n_screen must be 128");
  if (c->exact_bits != 0 && c->exact_bits != 16 && c->exact_bits != 4)
    return fail(CFR_EINVAL, "exact_bits must be 16 (or 0) or 4");
  if (c->exact_bits == 4 && c->ranking != CFR_RANK_SCORE)
    return fail(CFR_EUNSUPPORTED, "4-bit exact rows are read with the output-unit score ranking only");
  return CFR_OK;
}

static int64_t sect(int64_t nbytes) { return (nbytes + 31) / 32 * 32; }

}  // namespace cfr

using namespace cfr;

extern "C" {

const char* cfr_last_error(void) { return g_last_error.c_str(); }

int cfr_sizes_of(const cfr_config* c, cfr_sizes* out) {
  int rc = validate_config(c);
  if (rc) return rc;
  if (!out) return fail(CFR_EINVAL, "out is NULL");
  const int64_t E = c->n_experts, I = c->inter, H = c->hidden, nblk = H / kBlock;
  out->n_blocks = (int32_t)nblk;
  out->half_bytes = half_bytes(c->inter);
  out->unit_bytes = unit_bytes(c->inter);
  out->n_cand = c->top * c->inter;
  out->codes_bytes = E * nblk * kBlock * out->unit_bytes;
  out->scales_count = E * nblk * 2 * I;
  out->norms_count = E * I;
  out->u_count = H * c->rank;
  out->b_count = E * I * c->rank;
  out->weights_bytes = E * I * 3 * (int64_t)row_bytes((int)H, q4_rows(*c));
  return CFR_OK;
}

int cfr_read_bytes(const cfr_config* c, int32_t k, cfr_read_stats* out) {
  int rc = validate_config(c);
  if (rc) return rc;
  if (!out) return fail(CFR_EINVAL, "out is NULL");
  const int64_t I = c->inter, H = c->hidden, top = c->top, nblk = H / kBlock;
  if (k < 0 || k > top * I) return fail(CFR_EINVAL, "k must be in 0..top*inter");
  out->codes = top * nblk * c->n_screen * sect(unit_bytes(c->inter));
  out->scales = top * nblk * sect(2 * I * 2);
  out->norms = top * sect(I * 4);
  out->rho = c->ranking == CFR_RANK_EXPECTED_ERROR ? top * nblk * sect(2 * I * 2) : 0;
  out->exact = (int64_t)k * sect(3 * (int64_t)row_bytes((int)H, q4_rows(*c)));
  out->b = (top * I - k) * sect((int64_t)c->rank * 2);
  out->u = sect(H * (int64_t)c->rank * 2);
  out->total = out->codes + out->scales + out->norms + out->rho + out->exact + out->b + out->u;
  out->dense = top * 3 * I * (int64_t)row_bytes((int)H, q4_rows(*c));
  return CFR_OK;
}

int cfr_read_bytes_batch(const cfr_config* c, int32_t batch, int32_t k, const int32_t* ids,
                         const uint8_t* sel, const int32_t* kept, cfr_read_stats* out) {
  int rc = validate_config(c);
  if (rc) return rc;
  if (!out || !ids || !sel || (k > 0 && !kept)) return fail(CFR_EINVAL, "null argument");
  const int64_t E = c->n_experts, I = c->inter, H = c->hidden, top = c->top, nblk = H / kBlock;
  const int64_t ns = c->n_screen, nc = top * I;
  if (batch < 1) return fail(CFR_EINVAL, "batch must be at least 1");
  if (k < 0 || k > nc) return fail(CFR_EINVAL, "k must be in 0..top*inter");
  // one flag per sketch unit (expert, block, coordinate), per scale block
  // (expert, block), per expert, and per channel read exactly / skipped
  std::vector<uint8_t> unit_seen(E * nblk * kBlock, 0), block_seen(E * nblk, 0), expert_seen(E, 0);
  std::vector<uint8_t> exact_seen(E * I, 0), skip_seen(E * I, 0), kept_here(nc, 0);
  int64_t n_unit = 0, n_block = 0, n_expert = 0, n_exact = 0, n_skip = 0;
  for (int64_t t = 0; t < batch; ++t) {
    std::fill(kept_here.begin(), kept_here.end(), 0);
    for (int64_t q = 0; q < k; ++q) {
      const int32_t cand = kept[t * k + q];
      if (cand < 0 || cand >= nc) return fail(CFR_EINVAL, "kept candidate out of range");
      kept_here[cand] = 1;
    }
    for (int64_t s = 0; s < top; ++s) {
      const int32_t e = ids[t * top + s];
      if (e < 0 || e >= E) return fail(CFR_EINVAL, "expert id out of range");
      if (!expert_seen[e]) expert_seen[e] = 1, ++n_expert;
      for (int64_t b = 0; b < nblk; ++b) {
        if (!block_seen[e * nblk + b]) block_seen[e * nblk + b] = 1, ++n_block;
        const uint8_t* sb = sel + (t * nblk + b) * ns;
        for (int64_t q = 0; q < ns; ++q) {
          if (sb[q] >= kBlock) return fail(CFR_EINVAL, "screened coordinate out of range");
          uint8_t& u = unit_seen[(e * nblk + b) * kBlock + sb[q]];
          if (!u) u = 1, ++n_unit;
        }
      }
      for (int64_t j = 0; j < I; ++j) {
        const bool keep = kept_here[s * I + j] != 0;
        uint8_t& f = keep ? exact_seen[e * I + j] : skip_seen[e * I + j];
        if (!f) {
          f = 1;
          ++(keep ? n_exact : n_skip);
        }
      }
    }
  }
  out->codes = n_unit * sect(unit_bytes(c->inter));
  out->scales = n_block * sect(2 * I * 2);
  out->norms = n_expert * sect(I * 4);
  out->rho = c->ranking == CFR_RANK_EXPECTED_ERROR ? n_block * sect(2 * I * 2) : 0;
  out->exact = n_exact * sect(3 * (int64_t)row_bytes((int)H, q4_rows(*c)));
  out->b = n_skip * sect((int64_t)c->rank * 2);
  out->u = sect(H * (int64_t)c->rank * 2);
  out->total = out->codes + out->scales + out->norms + out->rho + out->exact + out->b + out->u;
  out->dense = n_expert * 3 * I * (int64_t)row_bytes((int)H, q4_rows(*c));
  return CFR_OK;
}

int cfr_read_bytes_shared(const cfr_config* c, int32_t batch, const int32_t* ids, const uint8_t* sel,
                          int32_t n_kept, cfr_read_stats* out) {
  int rc = validate_config(c);
  if (rc) return rc;
  if (!out || !ids || !sel) return fail(CFR_EINVAL, "null argument");
  const int64_t E = c->n_experts, I = c->inter, H = c->hidden, top = c->top, nblk = H / kBlock;
  const int64_t ns = c->n_screen;
  if (batch < 1) return fail(CFR_EINVAL, "batch must be at least 1");
  std::vector<uint8_t> unit_seen(E * nblk * kBlock, 0), block_seen(E * nblk, 0), expert_seen(E, 0);
  int64_t n_unit = 0, n_block = 0, n_expert = 0;
  for (int64_t t = 0; t < batch; ++t)
    for (int64_t s = 0; s < top; ++s) {
      const int32_t e = ids[t * top + s];
      if (e < 0 || e >= E) return fail(CFR_EINVAL, "expert id out of range");
      if (!expert_seen[e]) expert_seen[e] = 1, ++n_expert;
      for (int64_t b = 0; b < nblk; ++b) {
        if (!block_seen[e * nblk + b]) block_seen[e * nblk + b] = 1, ++n_block;
        const uint8_t* sb = sel + (t * nblk + b) * ns;
        for (int64_t q = 0; q < ns; ++q) {
          if (sb[q] >= kBlock) return fail(CFR_EINVAL, "screened coordinate out of range");
          uint8_t& u = unit_seen[(e * nblk + b) * kBlock + sb[q]];
          if (!u) u = 1, ++n_unit;
        }
      }
    }
  if (n_kept < 0 || n_kept > n_expert * I) return fail(CFR_EINVAL, "n_kept must be in 0..u*inter");
  out->codes = n_unit * sect(unit_bytes(c->inter));
  out->scales = n_block * sect(2 * I * 2);
  out->norms = n_expert * sect(I * 4);
  out->rho = 0;
  out->exact = (int64_t)n_kept * sect(3 * (int64_t)row_bytes((int)H, q4_rows(*c)));
  out->b = (n_expert * I - n_kept) * sect((int64_t)c->rank * 2);
  out->u = sect(H * (int64_t)c->rank * 2);
  out->total = out->codes + out->scales + out->norms + out->rho + out->exact + out->b + out->u;
  out->dense = n_expert * 3 * I * (int64_t)row_bytes((int)H, q4_rows(*c));
  return CFR_OK;
}

int cfr_pack_host(const cfr_config* c, const uint16_t* gate, const uint16_t* up,
                  const uint16_t* down, uint8_t* codes, uint16_t* scales, uint16_t* rho,
                  float* norms) {
  clear_error();
  int rc = validate_config(c);
  if (rc) return rc;
  if (!gate || !up || !down) return fail(CFR_EINVAL, "gate, up and down must be non-NULL");
  return pack_host(*c, gate, up, down, codes, scales, rho, norms, nullptr, nullptr);
}

}  // extern "C"

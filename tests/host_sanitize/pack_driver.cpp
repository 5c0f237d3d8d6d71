// Host-only driver of the C ABI's host entry points (config validation,
// sizes, read accounting, the sketch pack) for a build under AddressSanitizer
// and UndefinedBehaviorSanitizer.  Exits 0 when every check holds; a
// sanitizer report aborts it with a non-zero status.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "cfr.h"

static int failures = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

// float -> bf16 bits, round to nearest even (finite inputs)
static uint16_t bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

int main() {
  for (int shape = 0; shape < 3; ++shape) {
    cfr_config c{};
    const int H[3] = {256, 384, 128}, E[3] = {4, 3, 2}, I[3] = {64, 37, 250};
    c.hidden = H[shape];
    c.n_experts = E[shape];
    c.inter = I[shape];
    c.top = 2;
    c.rank = 8;
    c.n_screen = shape == 1 ? 128 : 80;
    c.max_batch = 2;
    c.device = 0;
    c.rot_seed = 12345u + shape;
    c.ranking = shape == 1 ? CFR_RANK_EXPECTED_ERROR : CFR_RANK_SCORE;
    cfr_sizes s{};
    CHECK(cfr_sizes_of(&c, &s) == CFR_OK);
    cfr_read_stats rb{};
    CHECK(cfr_read_bytes(&c, 5, &rb) == CFR_OK);
    CHECK(rb.total == rb.codes + rb.scales + rb.norms + rb.rho + rb.exact + rb.b + rb.u);
    CHECK(cfr_read_bytes(&c, c.top * c.inter + 1, &rb) == CFR_EINVAL);

    const size_t nw = (size_t)c.n_experts * c.inter * c.hidden;
    std::vector<uint16_t> gate(nw), up(nw), down(nw);
    uint64_t st = 0x9E3779B97F4A7C15ull + shape;
    auto uni = [&]() {
      st = st * 6364136223846793005ull + 1442695040888963407ull;
      return (float)((st >> 40) * (1.0 / 16777216.0)) - 0.5f;
    };
    for (size_t i = 0; i < nw; ++i) {
      gate[i] = bf16(0.04f * uni());
      up[i] = bf16(0.04f * uni());
      down[i] = bf16(0.04f * uni());
    }
    std::vector<uint8_t> codes((size_t)s.codes_bytes);
    std::vector<uint16_t> scales((size_t)s.scales_count), rho((size_t)s.scales_count);
    std::vector<float> norms((size_t)s.norms_count);
    CHECK(cfr_pack_host(&c, gate.data(), up.data(), down.data(), codes.data(), scales.data(), rho.data(),
                        norms.data()) == CFR_OK);
    // every packed byte is a base-3 number of five trits or padding zero
    for (uint8_t b : codes) CHECK(b < 243);
    for (float n : norms) CHECK(std::isfinite(n) && n > 0.f);
    // a NaN or an infinity anywhere is rejected
    gate[nw / 2] = 0x7FC0u;
    CHECK(cfr_pack_host(&c, gate.data(), up.data(), down.data(), codes.data(), scales.data(), rho.data(),
                        norms.data()) == CFR_EINVAL);
    gate[nw / 2] = 0;
    down[nw - 1] = 0xFF80u;
    CHECK(cfr_pack_host(&c, gate.data(), up.data(), down.data(), codes.data(), scales.data(), rho.data(),
                        norms.data()) == CFR_EINVAL);
    CHECK(cfr_pack_host(&c, nullptr, up.data(), down.data(), codes.data(), scales.data(), rho.data(),
                        norms.data()) == CFR_EINVAL);
  }
  cfr_config bad{};
  CHECK(cfr_sizes_of(&bad, nullptr) != CFR_OK);
  CHECK(cfr_sizes_of(nullptr, nullptr) == CFR_EINVAL);
  CHECK(std::strlen(cfr_last_error()) > 0);
  if (failures) std::fprintf(stderr, "%d checks failed\n", failures);
  return failures ? 1 : 0;
}

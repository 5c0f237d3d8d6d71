// Load-time pack on the host: rotation signs, rotated rows, TWN ternary
// codes, FP16 scales, rho, the base-3 coordinate-major sketch units, down
// norms and the resident [E][I][3][H] weight layout.
//
// Sources: [zh §方法步骤详情] load steps (1), (2) and (4); [zh §前置知识 /
// Hadamard旋转与三元Sketch]; [ko §어떻게 쓰나]  (zh = Chinese summary page,
// ko = Korean summary page of "Channel Selection for Mixture-of-Experts
// Decoding Needs No Calibration Data").
//
// Every floating-point step uses IEEE double in a fixed order and this file
// is compiled with -ffp-contract=off, so the result is a pure function of
// the BF16 inputs:
//   u      = H_128 (sigma * w_block)   in-place butterfly, h = 1, 2, ..., 64
//   S      = sum_i |u_i|                (i = 0..127 in order)
//   c_i    = sign(u_i) if 1280 |u_i| > 7 S else 0      (TWN, threshold 0.7 mean|u|)
//   alpha  = fp16_rne( A / (n * sqrt128) ),  A = sum of |u_i| over c_i != 0
//   rho    = fp16_rne( sum_i (u_i / sqrt128 - alpha c_i)^2 / 128 )
//   ||d_j|| = (float) sqrt( sum_h d_hj^2 )   (h in order)
#include <math.h>

#include <cmath>
#include <string.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "cfr_internal.h"

namespace cfr {

static inline double bf16_to_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

uint16_t f64_to_f16_rne(double v) {
  uint64_t x;
  memcpy(&x, &v, 8);
  uint16_t sign = (uint16_t)((x >> 48) & 0x8000u);
  uint64_t ax = x & 0x7FFFFFFFFFFFFFFFull;
  if (ax >= 0x7FF0000000000000ull) {  // inf or nan
    return (uint16_t)(sign | 0x7C00u | (ax > 0x7FF0000000000000ull ? 0x200u : 0u));
  }
  int e = (int)(ax >> 52) - 1023;
  uint64_t mant = ax & ((1ull << 52) - 1);
  if (e > 15) return (uint16_t)(sign | 0x7C00u);
  if (e >= -14) {  // normal range: keep 10 mantissa bits
    uint64_t keep = mant >> 42, rem = mant & ((1ull << 42) - 1), half = 1ull << 41;
    uint32_t h = ((uint32_t)(e + 15) << 10) | (uint32_t)keep;
    if (rem > half || (rem == half && (keep & 1))) h += 1;  // may carry into exponent / inf
    return (uint16_t)(sign | h);
  }
  if (e < -25) return sign;  // below half the smallest subnormal
  uint64_t sig = (1ull << 52) | mant;  // value = sig * 2^(e-52); unit 2^-24
  int shift = 28 - e;                  // 43..53
  uint64_t q = sig >> shift, rem = sig & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) q += 1;
  return (uint16_t)(sign | (uint16_t)q);
}

double f16_to_f64(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

// SplitMix64 (Steele, Lea, Flood 2014): state += golden gamma, then the
// variant-13 finalizer.  sigma_i = -1 when the top bit of output i is set.
void sign_vector(uint64_t seed, int hidden, float* out) {
  uint64_t state = seed;
  for (int i = 0; i < hidden; ++i) {
    state += 0x9E3779B97F4A7C15ull;
    uint64_t z = state;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z = z ^ (z >> 31);
    out[i] = (z >> 63) ? -1.0f : 1.0f;
  }
}

static void fwht128(double* v) {
  for (int h = 1; h < kBlock; h <<= 1)
    for (int i = 0; i < kBlock; ++i)
      if (!(i & h)) {
        double a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
}

namespace {

static inline double w_f64(uint16_t b) { return bf16_to_f64(b); }
static inline double w_f64(float f) { return (double)f; }

// T: uint16_t (BF16 bit patterns) or float (a dequantized 4-bit checkpoint)
template <typename T>
struct PackJob {
  const cfr_config* c;
  const T *gate, *up, *down;
  uint8_t* codes;
  uint16_t *scales, *rho, *w3;
  float* norms;
  const float* sigma;
  int nblk, lp, unit;
};

// One expert: sketch of gate and up, norms, resident layout (BF16 only).
template <typename T>
void pack_expert(const PackJob<T>& J, int e, std::vector<int8_t>& trits) {
  const int H = J.c->hidden, I = J.c->inter, nblk = J.nblk;
  const size_t row_stride = (size_t)H;
  double u[kBlock];
  for (int m = 0; m < 2; ++m) {
    const T* W = (m == 0 ? J.gate : J.up) + (size_t)e * I * H;
    // trits[b][i][j], coordinate-major like the units
    for (int j = 0; j < I; ++j) {
      const T* row = W + (size_t)j * row_stride;
      for (int b = 0; b < nblk; ++b) {
        for (int i = 0; i < kBlock; ++i)
          u[i] = (double)J.sigma[b * kBlock + i] * w_f64(row[b * kBlock + i]);
        fwht128(u);
        double S = 0.0;
        for (int i = 0; i < kBlock; ++i) S = S + fabs(u[i]);
        double A = 0.0;
        int n = 0;
        int8_t cc[kBlock];
        for (int i = 0; i < kBlock; ++i) {
          double a = fabs(u[i]);
          if (1280.0 * a > 7.0 * S) {
            cc[i] = u[i] > 0 ? 1 : -1;
            A = A + a;
            ++n;
          } else {
            cc[i] = 0;
          }
        }
        double alpha64 = n > 0 ? A / ((double)n * kSqrt128) : 0.0;
        uint16_t a16 = f64_to_f16_rne(alpha64);
        double alpha = f16_to_f64(a16);
        double acc = 0.0;
        for (int i = 0; i < kBlock; ++i) {
          double r = u[i] / kSqrt128;
          double d = r - alpha * (double)cc[i];
          acc = acc + d * d;
        }
        size_t sidx = (((size_t)e * nblk + b) * 2 + m) * I + j;
        if (J.scales) J.scales[sidx] = a16;
        if (J.rho) J.rho[sidx] = f64_to_f16_rne(acc / 128.0);
        int8_t* t = trits.data() + (size_t)b * kBlock * I;
        for (int i = 0; i < kBlock; ++i) t[(size_t)i * I + j] = cc[i];
      }
    }
    if (J.codes) {
      const int nbytes = (I + 4) / 5;
      for (int b = 0; b < nblk; ++b)
        for (int i = 0; i < kBlock; ++i) {
          uint8_t* unitp = J.codes + (((size_t)e * nblk + b) * kBlock + i) * J.unit;
          uint8_t* half = unitp + (size_t)m * J.lp;
          if (m == 0) memset(unitp, 0, J.unit);
          const int8_t* t = trits.data() + ((size_t)b * kBlock + i) * I;
          for (int q = 0; q < nbytes; ++q) {
            int v = 0, p3 = 1;
            for (int d = 0; d < 5; ++d) {
              int ch = 5 * q + d;
              int code = ch < I ? t[ch] : 0;
              v += (code + 1) * p3;
              p3 *= 3;
            }
            half[q] = (uint8_t)v;
          }
        }
    }
  }
  // down norms and the resident layout
  const T* D = J.down + (size_t)e * H * I;
  if (J.norms) {
    std::vector<double> acc(I, 0.0);
    for (int h = 0; h < H; ++h)
      for (int j = 0; j < I; ++j) {
        double d = w_f64(D[(size_t)h * I + j]);
        acc[j] = acc[j] + d * d;
      }
    for (int j = 0; j < I; ++j) J.norms[(size_t)e * I + j] = (float)sqrt(acc[j]);
  }
  if constexpr (sizeof(T) == 2) {
    if (!J.w3) return;
    for (int j = 0; j < I; ++j) {
      uint16_t* dst = J.w3 + ((size_t)e * I + j) * 3 * H;
      memcpy(dst, J.gate + ((size_t)e * I + j) * H, (size_t)H * 2);
      memcpy(dst + H, J.up + ((size_t)e * I + j) * H, (size_t)H * 2);
    }
    for (int h = 0; h < H; ++h)
      for (int j = 0; j < I; ++j)
        J.w3[(((size_t)e * I + j) * 3 + 2) * H + h] = D[(size_t)h * I + j];
  }
}

// True when any of n weights is an infinity or a NaN (for BF16: exponent
// field all ones).
static bool any_nonfinite(const uint16_t* a, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if ((a[i] & 0x7F80u) == 0x7F80u) return true;
  return false;
}
static bool any_nonfinite(const float* a, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!std::isfinite(a[i])) return true;
  return false;
}

template <typename T>
int pack_host_t(const cfr_config& c, const T* gate, const T* up, const T* down, uint8_t* codes,
                uint16_t* scales, uint16_t* rho, float* norms, uint16_t* w3, float* sigma_out) {
  // the sketch, the norms and the recovery basis are only defined for finite
  // weights: a NaN or an infinity is rejected before any work
  const size_t nw = (size_t)c.n_experts * c.inter * c.hidden;
  if (any_nonfinite(gate, nw) || any_nonfinite(up, nw) || any_nonfinite(down, nw))
    return fail(CFR_EINVAL, "weights contain NaN or infinity");
  PackJob<T> J;
  J.c = &c;
  J.gate = gate;
  J.up = up;
  J.down = down;
  J.codes = codes;
  J.scales = scales;
  J.rho = rho;
  J.w3 = w3;
  J.norms = norms;
  J.nblk = c.hidden / kBlock;
  J.lp = half_bytes(c.inter);
  J.unit = unit_bytes(c.inter);
  std::vector<float> sigma(c.hidden);
  sign_vector(c.rot_seed, c.hidden, sigma.data());
  if (sigma_out) memcpy(sigma_out, sigma.data(), sizeof(float) * c.hidden);
  J.sigma = sigma.data();

  unsigned nt = std::max(1u, std::min(std::thread::hardware_concurrency(), 16u));
  nt = std::min<unsigned>(nt, (unsigned)c.n_experts);
  std::vector<std::thread> pool;
  std::vector<int> errs(nt, 0);
  for (unsigned t = 0; t < nt; ++t) {
    pool.emplace_back([&, t]() {
      try {
        std::vector<int8_t> trits((size_t)J.nblk * kBlock * c.inter);
        for (int e = (int)t; e < c.n_experts; e += (int)nt) pack_expert(J, e, trits);
      } catch (...) {
        errs[t] = 1;
      }
    });
  }
  for (auto& th : pool) th.join();
  for (int e : errs)
    if (e) return fail(CFR_ENOMEM, "pack_host: host allocation failed");
  return CFR_OK;
}

}  // namespace

int pack_host(const cfr_config& c, const uint16_t* gate, const uint16_t* up,
              const uint16_t* down, uint8_t* codes, uint16_t* scales, uint16_t* rho,
              float* norms, uint16_t* w3, float* sigma_out) {
  return pack_host_t<uint16_t>(c, gate, up, down, codes, scales, rho, norms, w3, sigma_out);
}

int pack_host_f32(const cfr_config& c, const float* gate, const float* up, const float* down,
                  uint8_t* codes, uint16_t* scales, uint16_t* rho, float* norms, float* sigma_out) {
  return pack_host_t<float>(c, gate, up, down, codes, scales, rho, norms, nullptr, sigma_out);
}

// A 4-bit row record (cfr_build_reader_q4): weight h = scale_g (q_h - z_g),
// g = h / 128; every product is exact in float.  Zero points above 15 or
// non-finite scales are reported.
int dequant_q4_record(const uint8_t* rec, int H, float* out) {
  const int G = H / kBlock;
  for (int g = 0; g < G; ++g) {
    const uint16_t sb = (uint16_t)(rec[H / 2 + 2 * g] | (rec[H / 2 + 2 * g + 1] << 8));
    const double sc = f16_to_f64(sb);
    const int z = rec[H / 2 + 2 * G + g];
    if (z > 15 || !std::isfinite(sc)) return fail(CFR_EINVAL, "4-bit record: zero point above 15 or scale not finite");
    for (int i = 0; i < kBlock; ++i) {
      const int h = g * kBlock + i;
      const int q = (rec[h / 2] >> (4 * (h & 1))) & 15;
      out[h] = (float)(sc * (double)(q - z));
    }
  }
  return CFR_OK;
}

}  // namespace cfr

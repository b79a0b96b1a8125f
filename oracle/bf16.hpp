// CPU oracle — test infrastructure only. Nothing in the product path may include or link this.
//
// bfloat16 storage: 1 sign bit, 8 exponent bits, 7 stored mantissa bits (the upper half of an
// IEEE binary32). Conversions round to nearest, ties to even. Two entry points are needed:
//   * from float: the perturbed weight of a bf16 model is round_bf16(float(w) + float(+-eps)),
//     the float sum being rounded first (this project's reading of "bf16 weights with fp32
//     accumulate"; the pages fix no precision);
//   * from double: the oracle keeps activations in double and rounds a value once to bf16 where
//     the bf16 model feeds it to a matrix product, and once when it writes an updated weight.
#pragma once
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>

namespace oracle {

inline uint32_t f32_bits(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  return u;
}

inline float f32_from_bits(uint32_t u) {
  float x;
  std::memcpy(&x, &u, 4);
  return x;
}

inline float bf16_to_f32(uint16_t h) { return f32_from_bits(static_cast<uint32_t>(h) << 16); }

// Round a float to the nearest bf16, ties to even. NaN stays NaN (quiet), infinities stay.
inline uint16_t f32_to_bf16(float x) {
  const uint32_t u = f32_bits(x);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0) {
    return static_cast<uint16_t>((u >> 16) | 0x0040u);
  }
  // The discarded low half decides: above half rounds up, below rounds down, exactly half goes
  // to the even neighbour. Written as comparisons so a reader can check it against that rule.
  const uint32_t upper = u >> 16;
  const uint32_t lower = u & 0xffffu;
  uint32_t result = upper;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) result = upper + 1u;
  return static_cast<uint16_t>(result);
}

// Round a double to the nearest bf16 with a single rounding, ties to even.
// bf16 keeps 8 significant bits and the binary32 exponent range (normals down to 2^-126,
// subnormals with quantum 2^-133). The value is scaled to an integer count of quanta, rounded
// with nearbyint (round-half-even in the default rounding mode), and scaled back exactly.
inline uint16_t f64_to_bf16(double x) {
  if (std::isnan(x)) return 0x7fc0u;
  if (std::isinf(x)) return x > 0 ? 0x7f80u : 0xff80u;
  if (x == 0.0) return std::signbit(x) ? 0x8000u : 0x0000u;
  int e2;
  std::frexp(x, &e2);           // |x| = m * 2^e2 with m in [0.5, 1): leading bit is 2^(e2-1)
  int lead = e2 - 1;
  if (lead < -126) lead = -126;  // subnormal range shares the smallest normal quantum
  const double quantum = std::ldexp(1.0, lead - 7);
  const double count = std::nearbyint(x / quantum);
  const double y = count * quantum;
  // Overflow: anything that rounds to 2^128 or beyond is infinite.
  if (std::fabs(y) >= std::ldexp(1.0, 128)) return x > 0 ? 0x7f80u : 0xff80u;
  const float yf = static_cast<float>(y);  // exact: y has at most 8 significant bits
  return static_cast<uint16_t>(f32_bits(yf) >> 16);
}

inline double round_to_bf16(double x) { return bf16_to_f32(f64_to_bf16(x)); }

}  // namespace oracle

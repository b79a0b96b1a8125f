// CPU oracle — test infrastructure only. Nothing in the product path may include or link this.
//
// Counter-based Philox4x32-10 and the two derived streams the CD-RGE probe scheme needs:
// per-step probe seeds, and the Rademacher sign of one parameter under one probe.
//
// Source of the method: "Scaling Recurrent Neural Networks to a Billion Parameters with
// Zero-Order Optimization" (Chaubard & Kochenderfer, arXiv 2505.17852). The pith.science review
// page ("What carries the argument") states that the probes p_i are Rademacher vectors with
// entries in {-1,+1}; the review's "assumptions" list fixes E[p]=0 and E[pp^T]=I; the alex-wiki
// source note ("Method") says the directions come from reconstructible random seeds. The pages
// do not name a generator, so the generator and the bit mapping below are this project's reading:
//
//   * Philox4x32-10 exactly as defined by Salmon, Moraes, Dror and Shaw, "Parallel Random
//     Numbers: As Easy as 1, 2, 3" (SC'11): 4x32-bit counter, 2x32-bit key, 10 rounds, round
//     multipliers 0xD2511F53 / 0xCD9E8D57, Weyl key increments 0x9E3779B9 / 0xBB67AE85.
//   * probe seed i of step s:  x = Philox(key = base_seed, ctr = (i, lo32(s), hi32(s), 1)),
//     seed = x0 | x1 << 32.
//   * sign of element (tensor t, row r, column c) under probe seed S:
//     x = Philox(key = S, ctr = (c >> 7, r, t, 0)); word w = (c >> 5) & 3; j = c & 31;
//     bit = (x_w >> ((j >> 1) | ((j & 1) << 4))) & 1;  p = bit ? -1 : +1.
//     (Even columns of a 32-column group read the low half-word, odd columns the high half-word;
//     one Philox call therefore covers 128 consecutive columns of one row.)
#pragma once
#include <cstdint>

namespace oracle {

struct U32x4 {
  uint32_t w[4];
};

// One 32x32 -> 64-bit product split into (hi, lo).
inline void mulhilo32(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
  const uint64_t p = static_cast<uint64_t>(a) * static_cast<uint64_t>(b);
  *hi = static_cast<uint32_t>(p >> 32);
  *lo = static_cast<uint32_t>(p);
}

// Philox4x32 with 10 rounds (SC'11 definition). The key is bumped between rounds, so round r
// uses key + r * (0x9E3779B9, 0xBB67AE85).
inline U32x4 philox4x32_10(U32x4 ctr, uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  for (int round = 0; round < 10; ++round) {
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo32(M0, ctr.w[0], &hi0, &lo0);
    mulhilo32(M1, ctr.w[2], &hi1, &lo1);
    U32x4 next;
    next.w[0] = hi1 ^ ctr.w[1] ^ k0;
    next.w[1] = lo1;
    next.w[2] = hi0 ^ ctr.w[3] ^ k1;
    next.w[3] = lo0;
    ctr = next;
    k0 += W0;
    k1 += W1;
  }
  return ctr;
}

inline U32x4 philox_u64key(U32x4 ctr, uint64_t key) {
  return philox4x32_10(ctr, static_cast<uint32_t>(key), static_cast<uint32_t>(key >> 32));
}

// Seed of probe i at update step s (the "reconstructible seed" of the alex-wiki "Method" section).
inline uint64_t probe_seed(uint64_t base_seed, uint64_t step, uint32_t i) {
  U32x4 ctr{{i, static_cast<uint32_t>(step), static_cast<uint32_t>(step >> 32), 1u}};
  const U32x4 x = philox_u64key(ctr, base_seed);
  return static_cast<uint64_t>(x.w[0]) | (static_cast<uint64_t>(x.w[1]) << 32);
}

// Bit position inside a Philox word for column c (see the header comment).
inline uint32_t sign_bit_position(uint32_t c) {
  const uint32_t j = c & 31u;
  return (j >> 1) | ((j & 1u) << 4);
}

// Rademacher entry p(t, r, c) in {-1, +1} for a probe with the given seed.
inline int probe_sign(uint64_t seed, uint32_t tensor, uint32_t row, uint32_t col) {
  U32x4 ctr{{col >> 7, row, tensor, 0u}};
  const U32x4 x = philox_u64key(ctr, seed);
  const uint32_t word = x.w[(col >> 5) & 3u];
  const uint32_t bit = (word >> sign_bit_position(col)) & 1u;
  return bit ? -1 : +1;
}

}  // namespace oracle

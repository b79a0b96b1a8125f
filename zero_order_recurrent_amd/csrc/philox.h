// Counter-based Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
// 1, 2, 3", SC'11) for the CD-RGE probe streams. Usable on host and device.
//
// The pages ask for Rademacher probes regenerated from reconstructible seeds (pith.science review
// of arXiv 2505.17852, "What carries the argument"; alex-wiki source note, "Method") and fix no
// generator; the streams below are this library's definition, stated in include/cdrge.h:
//   seed_i of step s  = words 0|1<<32 of Philox(key = base_seed, ctr = (i, lo(s), hi(s), 1));
//   sign of (t, r, c) = bit ((c&31)>>1 | (c&1)<<4) of word (c>>5)&3 of
//                       Philox(key = seed_i, ctr = (c>>7, r, t, 0)); set bit -> -1.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cdrge {

struct PhiloxOut {
  uint32_t x, y, z, w;
};

#define CDRGE_HD __host__ __device__ __forceinline__

// a ^ b ^ c; one three-input bit operation (truth table 0x96) on the device.
CDRGE_HD uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
#else
  return a ^ b ^ c;
#endif
}

// Ten rounds; round r uses the key advanced r times by the Weyl constants. The 32 x 32 -> 64-bit
// products give both halves at once (one v_mad_u64_u32 each on the device).
CDRGE_HD PhiloxOut philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                            uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c0;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c2;
    const uint32_t n0 = xor3(static_cast<uint32_t>(p1 >> 32), c1, k0);
    const uint32_t n2 = xor3(static_cast<uint32_t>(p0 >> 32), c3, k1);
    c0 = n0;
    c1 = static_cast<uint32_t>(p1);
    c2 = n2;
    c3 = static_cast<uint32_t>(p0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return PhiloxOut{c0, c1, c2, c3};
}

CDRGE_HD uint64_t probe_seed(uint64_t base_seed, uint64_t step, uint32_t i) {
  const PhiloxOut o = philox10(i, static_cast<uint32_t>(step), static_cast<uint32_t>(step >> 32), 1u,
                               static_cast<uint32_t>(base_seed), static_cast<uint32_t>(base_seed >> 32));
  return static_cast<uint64_t>(o.x) | (static_cast<uint64_t>(o.y) << 32);
}

// The 128 sign bits of one row block: columns 128*blk .. 128*blk+127 of row r of tensor t.
CDRGE_HD PhiloxOut sign_block(uint64_t seed, uint32_t tensor, uint32_t row, uint32_t blk) {
  return philox10(blk, row, tensor, 0u, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
}

CDRGE_HD uint32_t pick_word(const PhiloxOut& o, uint32_t w) {
  return w == 0 ? o.x : (w == 1 ? o.y : (w == 2 ? o.z : o.w));
}

// Bit index inside a word for column c: even columns of a 32-column group read the low half-word
// (bits 0..15), odd columns the high half-word (bits 16..31).
CDRGE_HD uint32_t sign_bit_pos(uint32_t c) {
  const uint32_t j = c & 31u;
  return (j >> 1) | ((j & 1u) << 4);
}

}  // namespace cdrge

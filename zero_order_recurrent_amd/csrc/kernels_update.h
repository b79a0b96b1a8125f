// Seed-regenerating CD-RGE update, with 8-probe look-up tables:
//   theta_j <- R(theta_j - coef * sum_i p_i(j) d_i),   d_i = L(theta + eps p_i) - L(theta - eps p_i),
// R the rounding to the parameters' storage type (bf16 round-to-nearest-even, or none for fp32)
// (the update of the pith.science review, "What carries the argument", in the eta / (2 K eps)
// form of the alex-wiki source note, "Method"; the probes are regenerated from their seeds).
//
// Per element the sum over K probes costs K sign-adds when done probe by probe. Here the probes
// are taken 8 at a time: a table T_g[m] = sum_k (bit k of m ? -d_{8g+k} : d_{8g+k}) of all 256
// signed partial sums is built once per workgroup in LDS, and each element adds T_g at the 8-bit
// index formed by its 8 sign bits. The sign words arrive probe-major (one Philox block per probe
// and 128-column segment), so each quad of lanes (one lane per 32-column word of a segment)
// evaluates 8 probes' blocks, exchanges words with two DPP butterflies so that every lane holds
// its own word of all 8 probes, and transposes those 8 words bitwise (three swap stages) so that
// byte b of word k is the index of bit position 8b + k.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels_common.h"

namespace cdrge {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kUpdLutThreads = 256;
constexpr int kUpdLutStride = 256 + 16; // table copies 16 banks apart, so equal indices from
                                        // different lane groups hit different banks
constexpr int kUpdLutMaxProbes = 1024;
constexpr size_t kUpdLutMaxBytes = 144 * 1024;  // LDS of the tables

__device__ __forceinline__ uint32_t quad_xor1(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ uint32_t quad_xor2(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), 0x4E, 0xF, 0xF, true));
}

// Copies of each table (1, 2 or 4; lane group l of 16 lanes reads copy l % copies): as many as
// fit in kUpdLutMaxBytes for K probes.
inline int update_lut_copies(int K) {
  const size_t one = sizeof(float) * ((K + 7) / 8) * kUpdLutStride;
  return one * 4 <= kUpdLutMaxBytes ? 4 : (one * 2 <= kUpdLutMaxBytes ? 2 : 1);
}
// Dynamic LDS bytes for K probes: the seeds and loss differences of 8 ceil(K / 8) probes, then
// the tables.
inline size_t update_lut_bytes(int K) {
  const size_t kp = 8 * static_cast<size_t>((K + 7) / 8);
  return 12 * kp + sizeof(float) * ((K + 7) / 8) * update_lut_copies(K) * kUpdLutStride;
}

// The tensors of the flat parameter vector, as one index space of 128-column row segments.
constexpr int kUpdMaxTensors = 32;
struct UpdTensors {
  int64_t seg_end[kUpdMaxTensors];  // exclusive prefix sums of the tensors' segment counts
  int64_t off[kUpdMaxTensors];      // element offset of each tensor in theta
  int rows[kUpdMaxTensors], cols[kUpdMaxTensors];
  int n;
};

// One launch for all tensors, K <= kUpdLutMaxProbes; T is uint16_t (bf16 bit patterns) or
// float. A quad of lanes handles one 128-column segment (lane q: columns 32q .. 32q + 31);
// workgroups stride over the segments and the parameters of the next segment are requested
// before the current one is computed. Non-finite losses: nothing is written and flags[0] is
// raised.
template <typename T, int kCopies>
__global__ __launch_bounds__(kUpdLutThreads) void k_update_lut(
    T* __restrict__ theta_all, UpdTensors tens, const uint64_t* __restrict__ seeds,
    const float* __restrict__ losses, int K, float coef, uint32_t* __restrict__ flags) {
  constexpr int copies = kCopies;
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int kVec = 32 * sizeof(T) / 16;  // 16-byte pieces of a lane's 32 parameters
  extern __shared__ __align__(16) uint64_t upd_smem[];
  const int G = (K + 7) / 8;
  uint64_t* sseed = upd_smem;                                // [8 G]
  float* sdif = reinterpret_cast<float*>(upd_smem + 8 * G);  // [8 G]
  float* lut = sdif + 8 * G;  // [group][copy][kUpdLutStride], 256 entries used
  __shared__ int bad;
  const int tid = threadIdx.x;
  if (tid == 0) bad = 0;
  __syncthreads();
  for (int i = tid; i < 8 * G; i += kUpdLutThreads) {
    float dv = 0.f;
    uint64_t sd = 0;
    if (i < K) {
      const float lp = losses[2 * i], lm = losses[2 * i + 1];
      if (!isfinite(lp) || !isfinite(lm)) atomicOr(&bad, 1);
      dv = lp - lm;
      sd = seeds[i];
    }
    sdif[i] = dv;   // probes past K contribute nothing
    sseed[i] = sd;
  }
  __syncthreads();
  if (bad) {
    if (tid == 0 && blockIdx.x == 0) flags[0] = 1u;
    return;
  }
  for (int e = tid; e < G * 256; e += kUpdLutThreads) {
    const int g = e >> 8, m = e & 255;
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float dv = sdif[8 * g + k];
      t += ((m >> k) & 1) ? -dv : dv;   // sign bit set: p = -1
    }
    for (int cp = 0; cp < copies; ++cp) lut[(g * copies + cp) * kUpdLutStride + m] = t;
  }
  __syncthreads();

  const int lane = tid & 63, ell = tid & 3;
  const int odd1 = ell & 1, odd2 = (ell >> 1) & 1;
  const float* lcopy = lut + ((lane >> 4) & (copies - 1)) * kUpdLutStride;
  // 4x4 word transpose within the quad: v[w] = word w of the block this lane evaluated becomes
  // word `ell` of the block that quad lane w evaluated.
  auto qtrans = [&](uint32_t (&v)[4]) {
    uint32_t t[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) t[w] = quad_xor1(v[w ^ 1]);
#pragma unroll
    for (int w = 0; w < 4; ++w) v[w] = ((w & 1) != odd1) ? t[w] : v[w];
#pragma unroll
    for (int w = 0; w < 4; ++w) t[w] = quad_xor2(v[w ^ 2]);
#pragma unroll
    for (int w = 0; w < 4; ++w) v[w] = (((w >> 1) & 1) != odd2) ? t[w] : v[w];
  };

  const int64_t nseg = tens.seg_end[tens.n - 1];
  const int64_t quads = static_cast<int64_t>(gridDim.x) * (kUpdLutThreads / 4);
  // Locates a segment: tensor id, row, 128-column block, and this lane's first element.
  struct Seg {
    T* t;
    int r, blk, c0, cols;
    uint32_t id;
    int full;
  };
  auto locate = [&](int64_t seg) {
    int ti = 0;
    while (seg >= tens.seg_end[ti]) ++ti;
    const int64_t local = seg - (ti ? tens.seg_end[ti - 1] : 0);
    const int cols = tens.cols[ti];
    const int segs_per_row = (cols + 127) / 128;
    Seg g;
    g.r = static_cast<int>(local / segs_per_row);
    g.blk = static_cast<int>(local % segs_per_row);
    g.c0 = g.blk * 128 + 32 * ell;
    g.cols = cols;
    g.id = static_cast<uint32_t>(ti);
    g.t = theta_all + tens.off[ti] + static_cast<int64_t>(g.r) * cols + g.c0;
    g.full = (g.c0 + 32 <= cols) && ((reinterpret_cast<uintptr_t>(g.t) & 15u) == 0);
    return g;
  };
  auto load32 = [](const Seg& g, uint4 (&wv)[kVec]) {
    if (g.full) {
#pragma unroll
      for (int v = 0; v < kVec; ++v) wv[v] = reinterpret_cast<const uint4*>(g.t)[v];
    }
  };

  int64_t seg = static_cast<int64_t>(blockIdx.x) * (kUpdLutThreads / 4) + (tid >> 2);
  if (seg >= nseg) return;
  Seg cur = locate(seg);
  uint4 wv[kVec] = {};
  load32(cur, wv);
  for (; seg < nseg; seg += quads) {
    // request the next segment's parameters first
    const int64_t nxt = seg + quads;
    Seg next = cur;
    uint4 wn[kVec] = {};
    if (nxt < nseg) {
      next = locate(nxt);
      load32(next, wn);
    }
    float acc[32];
#pragma unroll
    for (int p = 0; p < 32; ++p) acc[p] = 0.f;
    for (int g = 0; g < G; ++g) {
      // this lane evaluates probes 8g + 2 ell and 8g + 2 ell + 1
      const PhiloxOut o0 = sign_block(sseed[8 * g + 2 * ell], cur.id, static_cast<uint32_t>(cur.r), static_cast<uint32_t>(cur.blk));
      const PhiloxOut o1 = sign_block(sseed[8 * g + 2 * ell + 1], cur.id, static_cast<uint32_t>(cur.r), static_cast<uint32_t>(cur.blk));
      uint32_t v0[4] = {o0.x, o0.y, o0.z, o0.w}, v1[4] = {o1.x, o1.y, o1.z, o1.w};
      qtrans(v0);
      qtrans(v1);
      // X[j]: word ell (this lane's 32 columns) of probe 8g + j
      uint32_t X[8] = {v0[0], v1[0], v0[1], v1[1], v0[2], v1[2], v0[3], v1[3]};
      // 8x8 bit transposes inside each byte: afterwards bit j of byte b of X[k] is bit 8b + k
      // of the word of probe 8g + j
      auto swap_bits = [](uint32_t& lo, uint32_t& hi, int sh, uint32_t msk) {
        const uint32_t x = ((lo >> sh) ^ hi) & msk;
        hi ^= x;
        lo ^= x << sh;
      };
      swap_bits(X[0], X[4], 4, 0x0F0F0F0Fu);
      swap_bits(X[1], X[5], 4, 0x0F0F0F0Fu);
      swap_bits(X[2], X[6], 4, 0x0F0F0F0Fu);
      swap_bits(X[3], X[7], 4, 0x0F0F0F0Fu);
      swap_bits(X[0], X[2], 2, 0x33333333u);
      swap_bits(X[1], X[3], 2, 0x33333333u);
      swap_bits(X[4], X[6], 2, 0x33333333u);
      swap_bits(X[5], X[7], 2, 0x33333333u);
      swap_bits(X[0], X[1], 1, 0x55555555u);
      swap_bits(X[2], X[3], 1, 0x55555555u);
      swap_bits(X[4], X[5], 1, 0x55555555u);
      swap_bits(X[6], X[7], 1, 0x55555555u);
      const float* lg = lcopy + g * (copies * kUpdLutStride);
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[8 * b + k] += lg[(X[k] >> (8 * b)) & 255u];
    }
    // Bit position p of the word is column 2 (p & 15) + (p >> 4): pair k of the 32 columns (16
    // 32-bit pairs) holds bit positions k (low half) and k + 16 (high half).
    if (cur.full) {
      if constexpr (kBf16) {
        uint32_t in[16] = {wv[0].x, wv[0].y, wv[0].z, wv[0].w, wv[1].x, wv[1].y, wv[1].z, wv[1].w,
                           wv[2].x, wv[2].y, wv[2].z, wv[2].w, wv[3].x, wv[3].y, wv[3].z, wv[3].w};
        uint32_t out[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const float lo = __uint_as_float(in[k] << 16) - coef * acc[k];
          const float hi = __uint_as_float(in[k] & 0xffff0000u) - coef * acc[k + 16];
          // packed round-to-nearest-even conversion (identical to f32_to_bf16_rne for non-NaN)
          const f32x2 v = {lo, hi};
          out[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
        }
#pragma unroll
        for (int v = 0; v < 4; ++v)
          reinterpret_cast<uint4*>(cur.t)[v] = make_uint4(out[4 * v], out[4 * v + 1], out[4 * v + 2], out[4 * v + 3]);
      } else {
        float in[32];
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          in[4 * v] = __uint_as_float(wv[v].x);
          in[4 * v + 1] = __uint_as_float(wv[v].y);
          in[4 * v + 2] = __uint_as_float(wv[v].z);
          in[4 * v + 3] = __uint_as_float(wv[v].w);
        }
#pragma unroll
        for (int cl = 0; cl < 32; ++cl) in[cl] -= coef * acc[(cl >> 1) + ((cl & 1) << 4)];
#pragma unroll
        for (int v = 0; v < 8; ++v)
          reinterpret_cast<float4*>(cur.t)[v] = make_float4(in[4 * v], in[4 * v + 1], in[4 * v + 2], in[4 * v + 3]);
      }
    } else {
#pragma unroll
      for (int p = 0; p < 32; ++p) {
        const int cl = 2 * (p & 15) + (p >> 4);
        if (cur.c0 + cl < cur.cols) {
          if constexpr (kBf16)
            cur.t[cl] = static_cast<uint16_t>(f32_to_bf16_rne(bf16_to_f32(cur.t[cl]) - coef * acc[p]));
          else
            cur.t[cl] = cur.t[cl] - coef * acc[p];
        }
      }
    }
    cur = next;
#pragma unroll
    for (int v = 0; v < kVec; ++v) wv[v] = wn[v];
  }
}

}  // namespace cdrge

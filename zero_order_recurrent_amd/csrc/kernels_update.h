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
// and 128-column segment), so the four lanes of a segment (one per 32-column word) evaluate 8
// probes' blocks, exchange words so that every lane holds its own word of all 8 probes, and
// transpose those 8 words bitwise (three swap stages) so that byte b of word k is the index of
// bit position 8b + k.
//
// Two kernels: k_update_perm (bf16, K <= 64: lanes of a segment 16 apart, permute-addressed
// tables, below) and k_update_lut (any dtype, K <= 1,024: a quad of adjacent lanes per segment,
// DPP exchanges, tables in 4, 2 or 1 copies).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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

// 128 bytes that lanes without a whole block of parameters load from (the loads are issued on
// every path, so that the count in flight never depends on it) and never use; never written.
// A distinct 16-byte piece per load: eight loads of one address from most lanes of a wave took
// the fp32 update at K = 512 from 62 to 109 us.
__device__ __align__(16) uint4 upd_dummy[8];

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
  // the tensor table, so that locating a segment issues no vector load (whose wait would also
  // wait for the previous segment's stores)
  __shared__ int64_t t_end[kUpdMaxTensors], t_off[kUpdMaxTensors];
  __shared__ int t_cols[kUpdMaxTensors];
  const int tid = threadIdx.x;
  if (tid == 0) bad = 0;
  if (tid < tens.n) {
    t_end[tid] = tens.seg_end[tid];
    t_off[tid] = tens.off[tid];
    t_cols[tid] = tens.cols[tid];
  }
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
  // Segments past the end are located as the last one and never written (full = 0).
  auto locate = [&](int64_t seg) {
    const bool valid = seg < nseg;
    const int64_t sg = valid ? seg : nseg - 1;
    int ti = 0;
    while (sg >= t_end[ti]) ++ti;
    const int64_t local = sg - (ti ? t_end[ti - 1] : 0);
    const int cols = t_cols[ti];
    const int segs_per_row = (cols + 127) / 128;
    Seg g;
    g.r = static_cast<int>(local / segs_per_row);
    g.blk = static_cast<int>(local % segs_per_row);
    g.c0 = g.blk * 128 + 32 * ell;
    g.cols = cols;
    g.id = static_cast<uint32_t>(ti);
    g.t = theta_all + t_off[ti] + static_cast<int64_t>(g.r) * cols + g.c0;
    g.full = valid && (g.c0 + 32 <= cols) && ((reinterpret_cast<uintptr_t>(g.t) & 15u) == 0);
    return g;
  };
  // Issued for every lane, so that the number of loads in flight does not depend on the path
  // taken; lanes without a whole 32-column piece read upd_dummy instead and do not use it.
  auto load32 = [&](const Seg& g, uint4 (&wv)[kVec]) {
    const uint4* src = g.full ? reinterpret_cast<const uint4*>(g.t) : upd_dummy;
#pragma unroll
    for (int v = 0; v < kVec; ++v) wv[v] = src[v];
  };

  int64_t seg = static_cast<int64_t>(blockIdx.x) * (kUpdLutThreads / 4) + (tid >> 2);
  if (seg >= nseg) return;
  Seg cur = locate(seg);
  uint4 wv[kVec];
  load32(cur, wv);
  for (; seg < nseg; seg += quads) {
    // request the next segment's parameters first (past the end: an unused, clamped one)
    const int64_t nxt = seg + quads;
    const Seg next = locate(nxt);
    uint4 wn[kVec];
    load32(next, wn);
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

// ---------------------------------------------------------------------------------------------
// The same update for bf16 parameters and K <= kUpdPermMaxProbes, with look-up addresses built by
// one byte permute.
//
// Table copy o = g C + c (probe group g, copy c of C) keeps its 256 entries 256 bytes apart:
// entry m at byte 65536 (o >> 6) + 256 m + 4 (o & 63). The byte address of a look-up is then the
// byte string [4 (o & 63), m, o >> 6, 0], which v_perm_b32 assembles from index byte m of a
// transposed sign word and a per-lane constant (no shift, no add). Lane l reads copy l % C; the
// copies are C consecutive banks, so only lanes a multiple of C apart can meet in a bank.
// Lanes form 4 rows of 16: the 16 lanes of a row take 16 consecutive 128-column segments, and
// row w computes block w (columns 32w .. 32w + 31) of each. The four lanes of a segment are 16
// apart, so a 4 x 4 exchange among them is two row swaps (v_permlane16_swap, v_permlane32_swap)
// per four registers. It serves the sign words, and the parameters: memory is accessed with lane
// (w, s) moving 16-byte piece w of each block of segment s (64 contiguous bytes per segment and
// instruction), and the exchange turns that into, or back from, the four pieces of block w.
// The Philox keys of every probe and round are precomputed in LDS (k0 + r 0x9E3779B9,
// k1 + r 0xBB67AE85), and each segment's parameters are requested one segment ahead, alternating
// between two register buffers.
constexpr int kUpdPermThreads = 1024;
constexpr int kUpdPermMaxProbes = 64;
// Copies per group: the largest power of two up to 32 with G C <= 128 (at most two 64 KB regions).
__host__ __device__ inline int update_perm_copies(int K) {
  const int G = (K + 7) / 8;
  int c = 32;
  while (c > 1 && G * c > 128) c >>= 1;
  return c;
}
__host__ __device__ inline int update_perm_regions(int K) {
  return ((K + 7) / 8 * update_perm_copies(K) + 63) / 64;
}
// Dynamic LDS: the tables, then the key schedules [8 G][10], the loss differences [8 G], a flag,
// and the tensor table (segment ends, offsets, column counts) that locates a segment without
// vector memory loads (whose wait would also wait for the previous segment's stores).
inline size_t update_perm_bytes(int K) {
  const size_t kp = 8 * static_cast<size_t>((K + 7) / 8);
  return 65536 * static_cast<size_t>(update_perm_regions(K)) + 80 * kp + 4 * kp + 16 +
         kUpdMaxTensors * (8 + 8 + 4);
}

__device__ __forceinline__ PhiloxOut philox10_ks(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 const uint2* ks) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint2 k = ks[r];
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c0;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c2;
    const uint32_t n0 = xor3(static_cast<uint32_t>(p1 >> 32), c1, k.x);
    const uint32_t n2 = xor3(static_cast<uint32_t>(p0 >> 32), c3, k.y);
    c0 = n0;
    c1 = static_cast<uint32_t>(p1);
    c2 = n2;
    c3 = static_cast<uint32_t>(p0);
  }
  return PhiloxOut{c0, c1, c2, c3};
}

// row_exchange of four 16-byte registers, one 32-bit component at a time.
__device__ __forceinline__ void row_exchange(uint4 (&p)[4]) {
  row_exchange(p[0].x, p[1].x, p[2].x, p[3].x);
  row_exchange(p[0].y, p[1].y, p[2].y, p[3].y);
  row_exchange(p[0].z, p[1].z, p[2].z, p[3].z);
  row_exchange(p[0].w, p[1].w, p[2].w, p[3].w);
}

// Keeps a parameter buffer in its registers up to this point (an empty asm that reads them). Put
// between a buffer's stores and its reload, it keeps the address arithmetic of the reload out of
// those registers: an ALU write there would first wait for the stores to complete, while the
// reload itself, a memory load, is ordered after them.
__device__ __forceinline__ void hold_buffer(const uint4 (&w)[4]) {
  asm volatile("" ::"v"(w[0].x), "v"(w[0].y), "v"(w[0].z), "v"(w[0].w), "v"(w[1].x), "v"(w[1].y),
               "v"(w[1].z), "v"(w[1].w), "v"(w[2].x), "v"(w[2].y), "v"(w[2].z), "v"(w[2].w),
               "v"(w[3].x), "v"(w[3].y), "v"(w[3].z), "v"(w[3].w));
}

// A float in LDS addressed by its byte address (the kernel has no static LDS, so its dynamic
// LDS, and with it the tables, starts at address 0).
typedef __attribute__((address_space(3))) const float LdsFloat;

//
// kG = ceil(K / 8), the number of 8-probe groups, fixed at compile time so that the group loop
// unrolls and the Philox rounds of one group interleave with the table look-ups of the previous
// one (lstm270m, K = 32: 0.357 -> 0.313 ms; charlm, K = 64: 0.053 -> 0.049 ms).
template <int kG>
__global__ __launch_bounds__(kUpdPermThreads) void k_update_perm(
    uint16_t* __restrict__ theta_all, UpdTensors tens, const uint64_t* __restrict__ seeds,
    const float* __restrict__ losses, int K, float coef, uint32_t* __restrict__ flags) {
  extern __shared__ __align__(16) uint64_t upd_smem[];
  char* const lds = reinterpret_cast<char*>(upd_smem);
  constexpr int G = kG;
  const int C = update_perm_copies(K), R = update_perm_regions(K);
  uint2* skeys = reinterpret_cast<uint2*>(lds + 65536 * R);
  float* sdif = reinterpret_cast<float*>(skeys + 80 * G);
  int* bad = reinterpret_cast<int*>(sdif + 8 * G);
  int64_t* t_end = reinterpret_cast<int64_t*>(sdif + 8 * G + 4);
  int64_t* t_off = t_end + kUpdMaxTensors;
  int* t_cols = reinterpret_cast<int*>(t_off + kUpdMaxTensors);
  const int tid = threadIdx.x;
  if (tid == 0) *bad = 0;
  if (tid < tens.n) {
    t_end[tid] = tens.seg_end[tid];
    t_off[tid] = tens.off[tid];
    t_cols[tid] = tens.cols[tid];
  }
  __syncthreads();
  for (int i = tid; i < 8 * G; i += kUpdPermThreads) {
    float dv = 0.f;
    if (i < K) {
      const float lp = losses[2 * i], lm = losses[2 * i + 1];
      if (!isfinite(lp) || !isfinite(lm)) atomicOr(bad, 1);
      dv = lp - lm;
    }
    sdif[i] = dv;  // probes past K contribute nothing
  }
  for (int i = tid; i < 80 * G; i += kUpdPermThreads) {
    const int pr = i / 10, r = i - 10 * pr;
    const uint64_t sd = pr < K ? seeds[pr] : 0;
    skeys[i] = make_uint2(static_cast<uint32_t>(sd) + static_cast<uint32_t>(r) * 0x9E3779B9u,
                          static_cast<uint32_t>(sd >> 32) + static_cast<uint32_t>(r) * 0xBB67AE85u);
  }
  __syncthreads();
  if (*bad) {
    if (tid == 0 && blockIdx.x == 0) flags[0] = 1u;
    return;
  }
  // float e of the table area is entry m = (e >> 6) & 255 of copy o = 64 (e >> 14) + (e & 63)
  float* lut = reinterpret_cast<float*>(lds);
  for (int e = tid; e < 16384 * R; e += kUpdPermThreads) {
    const int o = 64 * (e >> 14) + (e & 63), m = (e >> 6) & 255;
    if (o >= G * C) continue;
    const int g = o / C;
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float dv = sdif[8 * g + k];
      t += ((m >> k) & 1) ? -dv : dv;  // sign bit set: p = -1
    }
    lut[e] = t;
  }
  __syncthreads();

  const int lane = tid & 63, row = lane >> 4, wave = tid >> 6;
  const int cpy = lane & (C - 1);
  const int64_t nseg = tens.seg_end[tens.n - 1];
  struct Seg {
    uint16_t* tb;    // first parameter of the segment
    int r, blk;
    uint32_t id;
    uint32_t fmask;  // bit j < 4: block j is a whole, 16-byte aligned 32-column block; bit 4: valid
  };
  // segments past the end are located as the last one and flagged invalid (no load or store)
  auto locate = [&](int64_t seg) {
    Seg g;
    const bool valid = seg < nseg;
    const int64_t sg = valid ? seg : nseg - 1;
    int ti = 0;
    while (sg >= t_end[ti]) ++ti;
    const uint32_t local = static_cast<uint32_t>(sg - (ti ? t_end[ti - 1] : 0));
    const int cols = t_cols[ti];
    const uint32_t spr = static_cast<uint32_t>((cols + 127) / 128);
    const uint32_t r = local / spr;
    g.r = static_cast<int>(r);
    g.blk = static_cast<int>(local - r * spr);
    g.id = static_cast<uint32_t>(ti);
    g.tb = theta_all + t_off[ti] + static_cast<int64_t>(g.r) * cols + 128 * g.blk;
    const int rem = cols - 128 * g.blk;
    const bool aligned = (reinterpret_cast<uintptr_t>(g.tb) & 15u) == 0;
    g.fmask = valid ? (16u | (aligned ? (rem >= 128 ? 15u : (1u << (rem >> 5)) - 1u) : 0u)) : 0u;
    return g;
  };
  // Piece `row` of every block of the segment. Issued for every lane and every segment, so that
  // the number of loads in flight never depends on the path taken and the wait for a buffer never
  // waits for the loads into the other one; pieces of blocks that are not whole read upd_dummy
  // instead and are not used.
  auto load_pieces = [&](const Seg& g, uint4 (&wv)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t* src = ((g.fmask >> j) & 1u) ? g.tb + 32 * j + 8 * row : reinterpret_cast<const uint16_t*>(upd_dummy + j);
      wv[j] = *reinterpret_cast<const uint4*>(src);
    }
  };
  auto process = [&](const Seg& cur, uint4 (&wv)[4]) {
    float acc[32];
    // first_tag: std::true_type for group 0, whose look-ups initialise the sums
    auto group = [&](int g, auto first_tag) {
      constexpr bool kFirst = decltype(first_tag)::value;
      // row w evaluates probes 8g + 2w and 8g + 2w + 1 on this lane's segment
      const uint2* ks = skeys + (8 * g + 2 * row) * 10;
      const uint32_t blk = static_cast<uint32_t>(cur.blk), rr = static_cast<uint32_t>(cur.r);
      const PhiloxOut o0 = philox10_ks(blk, rr, cur.id, 0u, ks);
      const PhiloxOut o1 = philox10_ks(blk, rr, cur.id, 0u, ks + 10);
      uint32_t v0[4] = {o0.x, o0.y, o0.z, o0.w}, v1[4] = {o1.x, o1.y, o1.z, o1.w};
      // afterwards v[w] is word `row` (this lane's 32 columns) of the block of row w's probe
      row_exchange(v0[0], v0[1], v0[2], v0[3]);
      row_exchange(v1[0], v1[1], v1[2], v1[3]);
      // X[j]: word `row` of probe 8g + j
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
      const int o = g * C + cpy;
      const uint32_t y = (static_cast<uint32_t>(o & 63) << 2) | (static_cast<uint32_t>(o >> 6) << 16);
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          // address bytes: [y byte 0, byte b of X[k], y byte 2, 0]
          const uint32_t addr = __builtin_amdgcn_perm(X[k], y, 0x0C020400u | ((4u + b) << 8));
          const float v = *reinterpret_cast<const LdsFloat*>(static_cast<uintptr_t>(addr));
          if constexpr (kFirst)
            acc[8 * b + k] = v;
          else
            acc[8 * b + k] += v;
        }
    };
    group(0, std::true_type{});
#pragma unroll
    for (int g = 1; g < G; ++g) group(g, std::false_type{});

    // wv[v] becomes piece v of this lane's block; the results go back the same way
    row_exchange(wv);
    // Bit position p of the word is column 2 (p & 15) + (p >> 4): pair k of the 32 columns (16
    // 32-bit pairs) holds bit positions k (low half) and k + 16 (high half).
    const uint32_t in[16] = {wv[0].x, wv[0].y, wv[0].z, wv[0].w, wv[1].x, wv[1].y, wv[1].z, wv[1].w,
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
    for (int v = 0; v < 4; ++v) wv[v] = make_uint4(out[4 * v], out[4 * v + 1], out[4 * v + 2], out[4 * v + 3]);
    row_exchange(wv);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if ((cur.fmask >> j) & 1u) *reinterpret_cast<uint4*>(cur.tb + 32 * j + 8 * row) = wv[j];
    // a valid block that is not whole (a row's last columns, or unaligned): element by element
    if ((cur.fmask & 16u) && !((cur.fmask >> row) & 1u)) {
      const int c0 = 128 * cur.blk + 32 * row, cols = t_cols[cur.id];
      uint16_t* t = cur.tb + 32 * row;
#pragma unroll
      for (int p = 0; p < 32; ++p) {
        const int cl = 2 * (p & 15) + (p >> 4);
        if (c0 + cl < cols)
          t[cl] = static_cast<uint16_t>(f32_to_bf16_rne(bf16_to_f32(t[cl]) - coef * acc[p]));
      }
    }
  };

  // Every lane runs every iteration (the row swaps need all 64 lanes); the wave's first segment
  // decides the trip count.
  const int64_t stride = static_cast<int64_t>(gridDim.x) * (kUpdPermThreads / 4);
  int64_t base = static_cast<int64_t>(blockIdx.x) * (kUpdPermThreads / 4) + 16 * wave;
  if (base >= nseg) return;
  const int sl = lane & 15;
  Seg sa = locate(base + sl), sb;
  uint4 wa[4], wb[4];
  load_pieces(sa, wa);
  for (;;) {
    // the next segment (past the end: an invalid one) is requested before this one is computed
    base += stride;
    const bool more = base < nseg;
    sb = locate(base + sl);
    hold_buffer(wb);
    load_pieces(sb, wb);
    process(sa, wa);
    if (!more) break;
    base += stride;
    const bool more2 = base < nseg;
    sa = locate(base + sl);
    hold_buffer(wa);
    load_pieces(sa, wa);
    process(sb, wb);
    if (!more2) break;
  }
}

}  // namespace cdrge

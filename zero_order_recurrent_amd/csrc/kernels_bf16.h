// Perturbed logits + cross-entropy of the last LSTM layer for bf16 models on gfx950 matrix cores.
// One launch per timestep covers every probe pair of a chunk: both perturbed models' logits
// (W_out +- eps P) h_t + (b_out +- eps p), then the softmax cross-entropy against the next token
// (the pages' next-character objective: pith.science review, Figure 2 caption) accumulated per
// sequence. The perturbed output weights are formed exactly as in the gate kernel: a per-element
// bit select between the candidates bf16(W + eps) and bf16(W - eps), or, for the
// exact-perturbation model, W and the operand eps' P multiplied into the same accumulators.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "kernels_common.h"
#include "kernels_gates_bf16.h"

namespace cdrge {

constexpr int kCeThreads = 256;
constexpr int kCeCols = 128;        // batch columns per model
constexpr int kCeLdsStride = 40;    // bf16 per LDS row (32 + 8 pad)

// Per 32-bit pair of bf16 elements (2m, 2m+1): an all-ones half-word where the probe sign is -1.
// Column 2m of the 32-column group reads sign bit m, column 2m+1 bit m+16.
__device__ __forceinline__ uint32_t pair_mask(uint32_t word, int m) {
  return __builtin_amdgcn_perm(0u, word << (15 - m), 0x09090808u);
}

// ---------------------------------------------------------------------------------------------
// Perturbed logits + cross-entropy of the last layer at timestep t, for every probe pair.
// Tile: 64 logit rows (V <= 64, padded) x (128 columns of the +eps model, 128 of the -eps model).
// waves: (64-column half, model); each wave owns 64 x 64 = 4 x 4 MFMA tiles. The perturbed W_out
// tiles go through LDS (double-buffered); h goes from global memory straight into each wave's MFMA
// B registers (the k-chunk-major layout makes a lane's 8 values of a fragment 16 contiguous bytes),
// two chunks ahead. The softmax over the 64 rows of one column spans the 4 lane groups of a wave,
// reduced with cross-lane shuffles.
// seq[m][b] accumulates sum_t (logsumexp - logit of the next token) in float, in t order.
//
// kSplit: when the grid (column blocks x pairs) is too small to fill the chip, the reduction over
// H is split into gridDim.z slices of `kper` chunks; each workgroup writes its partial logits to
// zpart[slice][column][64] and k_ce_reduce finishes the sum (in slice order), the softmax and the
// cross-entropy.
// ---------------------------------------------------------------------------------------------
constexpr int kCeRows = 64;
// Split the reduction below this many workgroups (one per CU). Measured on MI355X: splitting
// charlm's 512 workgroups, or targeting 512 or 768, was slower than leaving 256+ unsplit.
constexpr int kCeTargetWorkgroups = 256;
constexpr size_t kCeLdsBytes = sizeof(uint16_t) * 2 * 2 * kCeRows * kCeLdsStride;

struct CeArgs {
  const uint16_t* wp;
  const uint16_t* wm;      // W_out candidates [V][H]
  const uint16_t* h;       // last layer h_t, [H / 32][ncols_pad][32] (k-chunk-major)
  const float* bout_m;     // per-model perturbed output bias [2P][64]
  const int32_t* tg;       // target of (b, t) at tg[b * tg_stride + t]; below zero: not scored
  int tg_stride;
  const uint64_t* seeds;
  float* seq;              // [2P][B]
  float* zpart;            // split: partial logits [slices][2P B][64]
  int pair0, H, B, V, T, t, ncols_pad;
  int kper;                // split: 32-wide chunks per slice (a multiple of 4)
  uint32_t tensor_wout;
  float eps;               // exact perturbation: the radius eps' (a bf16 value)
};

// grid: (ceil(B / 128), pairs in chunk, slices)
// kExact (exact-perturbation bf16): wp = wm = W_out itself; the LDS tile of side 0 holds W_out, that
// of side 1 the bf16 operand eps' P, and each wave multiplies both into its accumulators, the
// -eps model with the sign bits of eps' P flipped in registers: (W +- eps' P) h = W h +- eps' P h.
template <bool kSplit, bool kExact>
__global__ __launch_bounds__(kCeThreads) void k_logits_ce_bf16(CeArgs a) {
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* As = smem;                                  // [buf][side][64][40]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ch = wave & 1, side = wave >> 1;
  const int H = a.H;
  const int bcol0 = blockIdx.x * kCeCols;
  const int pr = blockIdx.y;
  const uint64_t seed = a.seeds[a.pair0 + pr];

  const bool former = tid < kCeRows;
  const bool frow_ok = tid < a.V;
  const int frow = frow_ok ? tid : 0;
  // h column of this lane in fragment j: model 2 pr + side, sequence bcol0 + 64 ch + 16 j + lane % 16.
  // Columns past the batch read the next model's columns or the padding (at least 256 columns
  // past the last model; their logits are not used).
  const uint32_t hcol0 = static_cast<uint32_t>((2 * pr + side) * a.B + bcol0 + 64 * ch + (lane & 15));
  const uint16_t* hlane = a.h + static_cast<int64_t>(hcol0) * kKChunk + 8 * (lane >> 4);
  const int64_t hchunk = static_cast<int64_t>(a.ncols_pad) * kKChunk;
  const int nch = H / kKChunk;
  const int c_begin = kSplit ? blockIdx.z * a.kper : 0;
  const int c_end = kSplit ? min(nch, c_begin + a.kper) : nch;
  uint4 rp[4], rm[4];
  PhiloxOut words{0, 0, 0, 0};

  auto load_w = [&](int c) {
    if (former) {
      const uint16_t* wp = a.wp + static_cast<int64_t>(frow) * H + kKChunk * c;
      const uint16_t* wm = a.wm + static_cast<int64_t>(frow) * H + kKChunk * c;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        rp[k] = frow_ok ? reinterpret_cast<const uint4*>(wp)[k] : make_uint4(0, 0, 0, 0);
        if constexpr (!kExact) rm[k] = frow_ok ? reinterpret_cast<const uint4*>(wm)[k] : make_uint4(0, 0, 0, 0);
      }
    }
  };
  // bf16 bits of eps' in both halves of a word (the exact-perturbation operand before signs)
  const uint32_t eps2 = (__float_as_uint(a.eps) >> 16) * 0x00010001u;
  // h fragments of chunk c (clamped to the last chunk of the range)
  auto load_h = [&](int c, bf16x8 (&b)[4]) {
    const uint16_t* src = hlane + hchunk * min(c, c_end - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const bf16x8*>(src + 16 * kKChunk * j);
  };
  auto form_store = [&](int c, int buf) {
    if (former) {
      if ((c & 3) == 0)  // c_begin is a multiple of 4
        words = sign_block(seed, a.tensor_wout, static_cast<uint32_t>(frow), static_cast<uint32_t>(c >> 2));
      const uint32_t w = pick_word(words, static_cast<uint32_t>(c & 3));
      const uint32_t p32[16] = {rp[0].x, rp[0].y, rp[0].z, rp[0].w, rp[1].x, rp[1].y, rp[1].z, rp[1].w,
                                rp[2].x, rp[2].y, rp[2].z, rp[2].w, rp[3].x, rp[3].y, rp[3].z, rp[3].w};
      const uint32_t m32[16] = {rm[0].x, rm[0].y, rm[0].z, rm[0].w, rm[1].x, rm[1].y, rm[1].z, rm[1].w,
                                rm[2].x, rm[2].y, rm[2].z, rm[2].w, rm[3].x, rm[3].y, rm[3].z, rm[3].w};
      uint32_t plus[16], minus[16];
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const uint32_t mask = pair_mask(w, m);
        if constexpr (kExact) {
          plus[m] = p32[m];                                    // W
          minus[m] = frow_ok ? eps2 | (mask & 0x80008000u) : 0u;  // eps' P (padding rows zero)
        } else {
          plus[m] = (mask & m32[m]) | (~mask & p32[m]);
          minus[m] = (mask & p32[m]) | (~mask & m32[m]);
        }
      }
      uint4* ap = reinterpret_cast<uint4*>(As + ((buf * 2 + 0) * kCeRows + tid) * kCeLdsStride);
      uint4* am = reinterpret_cast<uint4*>(As + ((buf * 2 + 1) * kCeRows + tid) * kCeLdsStride);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ap[k] = make_uint4(plus[4 * k], plus[4 * k + 1], plus[4 * k + 2], plus[4 * k + 3]);
        am[k] = make_uint4(minus[4 * k], minus[4 * k + 1], minus[4 * k + 2], minus[4 * k + 3]);
      }
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t pflip = side ? 0x80008000u : 0u;  // the -eps model's sign of eps' P
  auto mma = [&](int buf, const bf16x8 (&bfr)[4]) {
    if constexpr (kExact) {
      const uint16_t* AW = As + ((buf * 2 + 0) * kCeRows + (lane & 15)) * kCeLdsStride + 8 * (lane >> 4);
      const uint16_t* AP = As + ((buf * 2 + 1) * kCeRows + (lane & 15)) * kCeLdsStride + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 aw = *reinterpret_cast<const bf16x8*>(AW + 16 * i * kCeLdsStride);
        const u32x4 ap = *reinterpret_cast<const u32x4*>(AP + 16 * i * kCeLdsStride) ^ pflip;
        const bf16x8 apf = __builtin_bit_cast(bf16x8, ap);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw, bfr[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(apf, bfr[j], acc[i][j], 0, 0, 0);
        }
      }
    } else {
      const uint16_t* A = As + ((buf * 2 + side) * kCeRows + (lane & 15)) * kCeLdsStride + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 afr = *reinterpret_cast<const bf16x8*>(A + 16 * i * kCeLdsStride);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  // h of chunk c is in hb[(c - c_begin) % 2]; the request for chunk c + 2 goes out after chunk c
  // is multiplied (requests past the range repeat its last chunk and are not used).
  bf16x8 hb[2][4];
  load_w(c_begin);
  load_h(c_begin, hb[0]);
  load_h(c_begin + 1, hb[1]);
  form_store(c_begin, 0);
  __syncthreads();
  auto ce_step = [&](int c, auto par_tag) {
    constexpr int par = decltype(par_tag)::value;
    if (c + 1 < c_end) load_w(c + 1);
    mma(par, hb[par]);
    load_h(c + 2, hb[par]);
    if (c + 1 < c_end) form_store(c + 1, par ^ 1);
    __syncthreads();
  };
  int c = c_begin;
  for (; c + 2 <= c_end; c += 2) {
    ce_step(c, std::integral_constant<int, 0>{});
    ce_step(c + 1, std::integral_constant<int, 1>{});
  }
  if (c < c_end) ce_step(c, std::integral_constant<int, 0>{});

  const int m = 2 * pr + side;
  const int g = lane >> 4;
  if constexpr (kSplit) {
    // partial logits of rows 16 i + 4 g .. + 3 for this lane's four columns
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = bcol0 + 64 * ch + 16 * j + (lane & 15);
      if (b < a.B) {
        float4* dst = reinterpret_cast<float4*>(
            a.zpart + ((static_cast<int64_t>(blockIdx.z) * gridDim.y * 2 + m) * a.B + b) * kCeRows);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dst[4 * i + g] = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
    }
    return;
  }
  const float* bout = a.bout_m + static_cast<int64_t>(m) * kCeRows;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = 64 * ch + 16 * j + (lane & 15);
    const int b = bcol0 + n;
    const bool ok = b < a.B;
    const int y_raw = ok ? a.tg[static_cast<int64_t>(b) * a.tg_stride + a.t] : 0;
    const int y = min(y_raw, a.V - 1);
    float z[16];
    float zmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * i + 4 * g + r;
        const float v = (row < a.V) ? acc[i][j][r] + bout[row] : -INFINITY;
        z[4 * i + r] = v;
        zmax = fmaxf(zmax, v);
      }
    zmax = fmaxf(zmax, __shfl_xor(zmax, 16));
    zmax = fmaxf(zmax, __shfl_xor(zmax, 32));
    float sum = 0.f, zy = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * i + 4 * g + r;
        if (row < a.V) sum += __expf(z[4 * i + r] - zmax);
        if (row == y) zy = z[4 * i + r];
      }
    sum += __shfl_xor(sum, 16);
    sum += __shfl_xor(sum, 32);
    zy += __shfl_xor(zy, 16);
    zy += __shfl_xor(zy, 32);
    if (ok && g == 0) {
      const float l = (y_raw >= 0) ? (zmax + __logf(sum)) - zy : 0.f;
      float* dst = a.seq + static_cast<int64_t>(m) * a.B + b;
      *dst = (a.t == 0) ? l : *dst + l;
    }
  }
}

// Finishes the split logits: one wave per (model, sequence) column of the chunk, lane = logit
// row. z = bout + sum over slices (in slice order) of the partials, then the softmax
// cross-entropy against the target of (b, t) (none when it is below zero), accumulated into
// seq[m][b] over t.
// grid: ceil(2P B / 4) blocks of 256 threads.
__global__ __launch_bounds__(256) void k_ce_reduce(const float* __restrict__ zpart, int slices, int ncols,
                                                   int B, int V, int t, const float* __restrict__ bout_m,
                                                   const int32_t* __restrict__ tg, int tg_stride,
                                                   float* __restrict__ seq) {
  const int lane = threadIdx.x & 63;
  const int col = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (col >= ncols) return;
  const int m = col / B, b = col % B;
  float z = bout_m[static_cast<int64_t>(m) * kCeRows + lane];
  for (int sl = 0; sl < slices; ++sl) z += zpart[(static_cast<int64_t>(sl) * ncols + col) * kCeRows + lane];
  const bool row_ok = lane < V;
  float zmax = row_ok ? z : -INFINITY;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) zmax = fmaxf(zmax, __shfl_xor(zmax, o));
  float e = row_ok ? __expf(z - zmax) : 0.f;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) e += __shfl_xor(e, o);
  const int y_raw = tg[static_cast<int64_t>(b) * tg_stride + t];
  const int y = min(max(y_raw, 0), V - 1);
  const float zy = __shfl(z, y);
  if (lane == 0) {
    const float l = (y_raw >= 0) ? (zmax + __logf(e)) - zy : 0.f;
    float* dst = seq + static_cast<int64_t>(m) * B + b;
    *dst = (t == 0) ? l : *dst + l;
  }
}

}  // namespace cdrge

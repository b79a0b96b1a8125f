// fp32 models with many (model, sequence) columns: the gate product of one layer at one timestep
// for every perturbed model of a probe chunk, with the weights shared on the matrix cores.
//
// The persistent fp32 kernel (kernels_f32.h) gives each workgroup a few models and streams all of
// W through it every timestep, so a weight load feeds only as many multiply-adds as the
// workgroup has columns. Here a launch covers one (layer, timestep): workgroup (row slice, column
// block) computes 64 gate rows (16 hidden units x 4 gates) for 64 (model, sequence) columns, so
// each weight it stages feeds 64 columns and each activation 64 rows.
//
// Per model the gate pre-activations are (W + s eps P) [x; h] + b, with s = +1 for the +eps model
// of a pair and -1 for the -eps one and P the pair's Rademacher signs (pith.science review, "What
// carries the argument"; the perturbed recurrent forward of alex-wiki "Method"). They are computed
// as W [x; h] + s eps (P [x; h]) + b:
//   * W [x; h] is shared by all models: v_mfma_f32_16x16x4_f32 on fp32 operands staged in LDS;
//   * P [x; h] differs per pair: for every column and group of 4 K-columns that one nibble of a
//     sign word covers, the 16 signed sums +-x_a +-x_b +-x_c +-x_d are tabulated in LDS once per
//     32-wide K chunk, and each (row, column) adds the entry its nibble selects. Two adjacent
//     columns always belong to one probe pair and share the nibble, so one 8-byte read serves
//     both. The read's address is built by one byte permute: the nibble lands in address byte 1
//     (entries of one nibble value are one 256-byte row of 64 columns) and the column pair in
//     byte 0, so the tables start at LDS address 0 (the kernel has no static LDS).
// The perturbed biases come from a per-chunk table. The four gates of a hidden unit meet in one
// lane of the matrix-core output (local row 4u + g is gate g of unit u), so the LSTM cell runs in
// registers; c and h live in global memory as [H][columns], h ping-ponged per layer.
//
// The last layer also forms, for its 16 units, the partial logits of every column whose target at
// t is scored (the others add nothing to their loss):
// zpart[slice][column][v] = sum over its units u of fl(w_out[v][u] +- eps_vu) h[u][column], the
// perturbed output weight rounded once in fp32 as in the persistent kernel; k_ce_f32_sliced adds
// the slices in order, the perturbed output bias and the cross-entropy of the timestep.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels_common.h"

namespace cdrge {

constexpr int kSlUnits = 16;                 // hidden units per workgroup
constexpr int kSlRows = 4 * kSlUnits;        // gate rows per workgroup
constexpr int kSlCols = 64;                  // (model, sequence) columns per workgroup
constexpr int kSlThreads = 256;
constexpr int kSlMaxPairs = 32;              // probe pairs one column block can span (B = 1)
constexpr int kSlMaxV = 64;
constexpr int kSlPStride = 80;               // floats per row of the P x exchange buffer
// LDS map in bytes. The sign-sum tables are [8 nibble positions][16 values][64 columns] floats at
// address 0; after the K loop the same bytes hold the P x exchange buffer [64 rows][80] and the
// last layer's h [16 units][64 columns].
constexpr int kSlTabBytes = 8 * 16 * kSlCols * 4;                  // 32 KB
constexpr int kSlWOff = kSlTabBytes;                                // W^T chunk [2][32][64 rows]
constexpr int kSlXOff = kSlWOff + 2 * 32 * kSlRows * 4;             // activations [2][32][64 columns]
constexpr int kSlSOff = kSlXOff + 2 * 32 * kSlCols * 4;             // sign words [2][32 pairs][64 rows]
constexpr int kSlLdsBytes = kSlSOff + 2 * kSlMaxPairs * kSlRows * 4;  // 80 KB: two workgroups per CU
constexpr int kSlHsOff = kSlRows * kSlPStride * 4;                  // h [16][64] after the exchange buffer
// after the K loop the W^T buffers hold the last layer's output weights [16 units][64] and output
// sign words [pairs][64]
static_assert((kSlUnits * kSlMaxV + kSlMaxPairs * kSlCols) * 4 <= kSlXOff - kSlWOff, "logit staging");
// The direct variant (B a multiple of 16) has no tables, and a 64-column block spans at most two
// probe pairs (pairs start at multiples of 2B, a multiple of 32; blocks at multiples of 64): h
// [16][64] at 0, then W^T, activations and the sign words of up to 4 pairs (one per wave), 38 KB
// in all (four workgroups per CU).
constexpr int kSlDirWgs = 4;
constexpr int kSlDirMaxPairs = 4;
constexpr int kSlDirBase = 4096;
constexpr int kSlDirLdsBytes = kSlDirBase + (kSlSOff - kSlWOff) + 2 * kSlDirMaxPairs * kSlRows * 4;

typedef float f32x4_sl __attribute__((ext_vector_type(4)));
// Two floats in LDS by their byte address: the kernel has no static LDS, so its dynamic LDS (and
// the sign-sum tables at its start) begins at address 0; the host checks that before using the
// kernel.
typedef float f32x2_sl __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const f32x2_sl SlLdsFloat2;

struct F32SlArgs {
  const float* wt_ih;      // W_ih^T [in][4H] (k-major copy)
  const float* wt_hh;      // W_hh^T [H][4H]
  const uint32_t* sg_ih;   // sign words of W_ih for the chunk's pairs, [pairs][in / 32][4H]
  const uint32_t* sg_hh;   // [pairs][H / 32][4H]
  const float* bias_m;     // perturbed gate biases [2 pairs][L][4H]
  const float* x;          // layers above 0: input [in][ncp] (h of the layer below at t)
  const float* emb_m;      // layer 0: perturbed embeddings [2 pairs][V][E]
  const int32_t* tok;      // layer 0: token of (sequence b, t) at tok[b * in_stride + t]
  const float* h_prev;     // h of this layer at t - 1, [H][ncp] (unused when first)
  float* h_out;            // h of this layer at t, [H][ncp]
  float* c;                // cell state of this layer, [H][ncp], read (unless first) and written
  const float* wt_out;     // last layer: W_out^T [H][V]
  const uint32_t* sg_out;  // [pairs][H / 32][V]
  float* zpart;            // last layer: partial logits [H / 16][ncp][V]
  const int32_t* tg;       // last layer: target of (sequence b, t) at tg[b * tg_stride + t]
  float eps;
  int in, H, B, V, L, layer, t, ncols, ncp, pc, in_stride, tg_stride, first, last;
};

// grid (H / 16, ncp / 64), block 256, dynamic LDS kSlLdsBytes (kDirect: kSlDirLdsBytes). Requires
// in % 32 == 0, H % 32 == 0, V <= kSlMaxV, and for kDirect B % 16 == 0. Column s = m B + b is
// sequence b of model m (model 2q + side of pair q); columns at or past ncols are computed from
// whatever the padding holds and not written.
//
// kDirect: when B is a multiple of 16, every 16-column matrix-core tile lies in one model, so the
// perturbed weight itself can be the A operand: each lane forms fl(w +- eps p) for its element of
// the tile's model (the perturbed weight w + s eps p rounded once to fp32, as a perturbed copy of
// the parameters holds it) and the matrix cores multiply it with the activations. No sign-sum tables, no P x exchange, one barrier per K chunk.
template <bool kDirect>
__global__ __launch_bounds__(kSlThreads, kDirect ? kSlDirWgs : 2) void k_lstm_f32_sliced(F32SlArgs a) {
  extern __shared__ __align__(16) float sl_lds[];
  char* const lds = reinterpret_cast<char*>(sl_lds);
  // LDS offsets of the staged chunk (the direct variant has no tables in front of them)
  constexpr int kWOff = kDirect ? kSlDirBase : kSlWOff;
  constexpr int kXOff = kWOff + (kSlXOff - kSlWOff);
  constexpr int kSOff = kWOff + (kSlSOff - kSlWOff);
  constexpr int kHsOff = kDirect ? 0 : kSlHsOff;
  constexpr int kMaxPairs = kDirect ? kSlDirMaxPairs : kSlMaxPairs;  // sign-word pairs per LDS chunk
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H = a.H, G4 = 4 * H;
  const int u0 = blockIdx.x * kSlUnits;
  const int s0 = blockIdx.y * kSlCols;
  const int two_b = 2 * a.B;
  const int q_first = min(s0 / two_b, a.pc - 1);
  const int n_q = min(min(s0 + kSlCols - 1, a.ncols - 1) / two_b, a.pc - 1) - q_first + 1;
  const int kx = a.in / 32, kh = a.first ? 0 : H / 32, nch = kx + kh;

  // ---- staging of one 32-wide K chunk into registers, then into LDS buffer `buf` ----
  // W^T rows: element e = tid + 256 i is (k = e >> 6, position p = e & 63), p = 16 g + u for
  // gate g of unit u0 + u, i.e. W row g H + u0 + u; the LDS chunk is [k][p].
  // Activations: for the layer-0 input a thread gathers 8 consecutive embedding values of one
  // column (column tid & 63, k = 8 (tid >> 6) + i); otherwise column tid & 63, k = (tid >> 6) + 4 i.
  // Sign words: element e is (pair q_first + (e >> 6), position e & 63); the LDS chunk is [pair][p].
  struct Regs {
    float w[8], x[8];
    uint32_t s[8];
  };
  const int scol = tid & 63;
  const bool emb_in = a.layer == 0;
  int tok_row = 0;  // layer 0: row of emb_m of this thread's column
  {
    const int col = min(s0 + scol, a.ncols - 1);
    const int m = col / a.B, b = col - m * a.B;
    if (emb_in) {
      int tk = a.tok[static_cast<int64_t>(b) * a.in_stride + a.t];
      tk = min(max(tk, 0), a.V - 1);  // invalid tokens are reported through the loss
      tok_row = m * a.V + tk;
    }
  }
  // Global addresses are a wave-uniform base (the wave index comes from readfirstlane) plus a
  // 32-bit per-lane byte offset.
  const uint32_t lane_row = static_cast<uint32_t>((scol >> 4) * H + u0 + (scol & 15)) * 4u;  // W row of position scol
  const uint32_t lane_col = static_cast<uint32_t>(scol) * 4u;
  auto gload = [&](int kc, Regs& rg) {
    const bool xpart = kc < kx;
    const int cc = xpart ? kc : kc - kx;
    const float* wt = xpart ? a.wt_ih : a.wt_hh;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const char* base = reinterpret_cast<const char*>(wt + static_cast<int64_t>(32 * cc + wave + 4 * i) * G4);
      rg.w[i] = *reinterpret_cast<const float*>(base + lane_row);
    }
    if (xpart && emb_in) {
      const float4* src = reinterpret_cast<const float4*>(a.emb_m + static_cast<int64_t>(tok_row) * a.in + 32 * cc +
                                                          8 * wave);
      const float4 v0 = src[0], v1 = src[1];
      rg.x[0] = v0.x; rg.x[1] = v0.y; rg.x[2] = v0.z; rg.x[3] = v0.w;
      rg.x[4] = v1.x; rg.x[5] = v1.y; rg.x[6] = v1.z; rg.x[7] = v1.w;
    } else {
      const float* xs = xpart ? a.x : a.h_prev;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const char* base = reinterpret_cast<const char*>(xs + static_cast<int64_t>(32 * cc + wave + 4 * i) * a.ncp + s0);
        rg.x[i] = *reinterpret_cast<const float*>(base + lane_col);
      }
    }
    const uint32_t* sg = xpart ? a.sg_ih : a.sg_hh;
    const int nw = xpart ? kx : H / 32;
#pragma unroll
    for (int i = 0; i < kMaxPairs / 4; ++i) {
      const int qi = wave + 4 * i;  // wave-uniform
      rg.s[i] = 0u;
      if (qi < n_q) {
        const char* base = reinterpret_cast<const char*>(sg + (static_cast<int64_t>(q_first + qi) * nw + cc) * G4);
        rg.s[i] = *reinterpret_cast<const uint32_t*>(base + lane_row);
      }
    }
  };
  auto lstore = [&](int kc, int buf, const Regs& rg) {
    float* wk = reinterpret_cast<float*>(lds + kWOff) + buf * 32 * kSlRows;
    float* xk = reinterpret_cast<float*>(lds + kXOff) + buf * 32 * kSlCols;
    uint32_t* sk = reinterpret_cast<uint32_t*>(lds + kSOff) + buf * kMaxPairs * kSlRows;
#pragma unroll
    for (int i = 0; i < 8; ++i) wk[tid + 256 * i] = rg.w[i];
    if (kc < kx && emb_in) {
#pragma unroll
      for (int i = 0; i < 8; ++i) xk[(8 * wave + i) * kSlCols + scol] = rg.x[i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xk[(wave + 4 * i) * kSlCols + scol] = rg.x[i];
    }
#pragma unroll
    for (int i = 0; i < kMaxPairs / 4; ++i) {
      // pair qi's 64 words are stored with their 4-word groups permuted by qi (bits 2-5 of the
      // position xor 4 (qi & 15)), so that the 16-byte reads of lanes with different pairs fall
      // in different banks
      const int qi = wave + 4 * i;
      sk[qi * kSlRows + (scol ^ ((qi & 15) << 2))] = rg.s[i];
    }
  };

  // ---- sign-sum tables of one chunk: thread (column tid & 63, nibble positions 2 (tid >> 6)
  // and 2 (tid >> 6) + 1). Bit position p of a sign word is column 2 (p & 15) + (p >> 4) of the
  // chunk; entry v of nibble j is the sum over i < 4 of (bit i of v ? -x : x) at bit 4 j + i.
  auto build = [&](int buf) {
    const float* xk = reinterpret_cast<const float*>(lds + kXOff) + buf * 32 * kSlCols;
    float* tab = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * (tid >> 6) + jj;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = 4 * j + i;
        v[i] = xk[(2 * (p & 15) + (p >> 4)) * kSlCols + scol];
      }
      const float lo[4] = {v[0] + v[1], v[1] - v[0], v[0] - v[1], -v[0] - v[1]};
      const float hi[4] = {v[2] + v[3], v[3] - v[2], v[2] - v[3], -v[2] - v[3]};
#pragma unroll
      for (int m = 0; m < 16; ++m) tab[(j * 16 + m) * kSlCols + scol] = lo[m & 3] + hi[m >> 2];
    }
  };

  // ---- matrix-core role: wave w owns local rows 4 u + g for units u = 4 w .. 4 w + 3, as the
  // 16 rows of its A fragments (row i of the fragment: unit 4 w + i / 4, gate i % 4), and all 64
  // columns as four 16-column tiles.
  f32x4_sl acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4_sl{0.f, 0.f, 0.f, 0.f};
  const int fi = lane & 15, fk = lane >> 4;
  const int a_pos = (fi & 3) * 16 + 4 * wave + (fi >> 2);  // position p of the lane's A row
  const int a_off = fk * kSlRows + a_pos;
  const int b_off = fk * kSlCols + fi;
  // direct variant: the model of each 16-column tile, its pair within the block and its signed eps
  int tile_qi[4];
  float tile_e[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = min(min(s0 + 16 * j, a.ncols - 1) / a.B, 2 * a.pc - 1);
    tile_qi[j] = min((m >> 1) - q_first, kMaxPairs - 1);
    tile_e[j] = (m & 1) ? -a.eps : a.eps;
  }
  // B a multiple of 64: the block's 64 columns are sequences of one model (blocks start at
  // multiples of 64)
  const bool one_model = a.B % 64 == 0;
  // ---- sign-sum role: thread (column pair cp = tid & 31, row group rg = tid >> 5) owns columns
  // 2 cp, 2 cp + 1 and positions p = 8 rg + i. Columns 2k and 2k + 1 always belong to one probe
  // pair (a pair's 2B columns start at a multiple of 2B), so they share the nibble and one 8-byte
  // read returns both columns' entries.
  const int cp = tid & 31, rgp = tid >> 5;
  float2 accp[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) accp[i] = make_float2(0.f, 0.f);
  const int my_col = min(s0 + 2 * cp, a.ncols - 1);
  const int my_qi = min((my_col / two_b) - q_first, kSlMaxPairs - 1);
  const uint32_t col_byte = static_cast<uint32_t>(8 * cp);

  // Chunk kc + 1 is requested at the top of step kc and written to LDS buffer (kc + 1) & 1 at its
  // end.
  Regs rg;
  auto step = [&](int kc) {
    const int buf = kc & 1;
    if constexpr (!kDirect) {
      if (kc + 1 < nch) gload(kc + 1, rg);
    }
    if constexpr (kDirect) {
      // A = fl(w + e) per tile: e = +-eps by the tile's side, negated where the pair's sign bit
      // of (row, column) is set; bit position of chunk column c is (c >> 1) | ((c & 1) << 4)
      const float* wk = reinterpret_cast<const float*>(lds + kWOff) + buf * 32 * kSlRows;
      const float* xk = reinterpret_cast<const float*>(lds + kXOff) + buf * 32 * kSlCols;
      const uint32_t* sk = reinterpret_cast<const uint32_t*>(lds + kSOff) + buf * kMaxPairs * kSlRows;
      if (one_model) {
        // all four tiles in one model: one A value per K step feeds the four MFMAs
        const uint32_t word = sk[tile_qi[0] * kSlRows + (a_pos ^ ((tile_qi[0] & 15) << 2))];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const float av = wk[a_off + 4 * ks * kSlRows];
          const uint32_t c = static_cast<uint32_t>(4 * ks + fk);
          const uint32_t pos = (c >> 1) | ((c & 1u) << 4);
          const float e = __uint_as_float(__float_as_uint(tile_e[0]) ^ (((word >> pos) & 1u) << 31));
          const float ap = av + e;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(ap, xk[b_off + 4 * ks * kSlCols + 16 * j], acc[j], 0, 0, 0);
        }
        return;
      }
      uint32_t word[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) word[j] = sk[tile_qi[j] * kSlRows + (a_pos ^ ((tile_qi[j] & 15) << 2))];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const float av = wk[a_off + 4 * ks * kSlRows];
        const uint32_t c = static_cast<uint32_t>(4 * ks + fk);
        const uint32_t pos = (c >> 1) | ((c & 1u) << 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float e = __uint_as_float(__float_as_uint(tile_e[j]) ^ (((word[j] >> pos) & 1u) << 31));
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av + e, xk[b_off + 4 * ks * kSlCols + 16 * j], acc[j], 0, 0, 0);
        }
      }
      return;
    }
    build(buf);
    __syncthreads();
    {
      const float* wk = reinterpret_cast<const float*>(lds + kWOff) + buf * 32 * kSlRows;
      const float* xk = reinterpret_cast<const float*>(lds + kXOff) + buf * 32 * kSlCols;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const float av = wk[a_off + 4 * ks * kSlRows];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, xk[b_off + 4 * ks * kSlCols + 16 * j], acc[j], 0, 0, 0);
      }
    }
    {
      const char* sk = lds + kSOff + buf * kSlMaxPairs * kSlRows * 4 + my_qi * kSlRows * 4;
#pragma unroll
      for (int i4 = 0; i4 < 2; ++i4) {
        const uint4 w4 = *reinterpret_cast<const uint4*>(sk + 4 * ((8 * rgp + 4 * i4) ^ ((my_qi & 15) << 2)));
        const uint32_t ws[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const uint32_t me = ws[ii] & 0x0F0F0F0Fu, mo = (ws[ii] >> 4) & 0x0F0F0F0Fu;
          float2 sum = make_float2(0.f, 0.f);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            // address byte 1 = nibble j, byte 0 = 8 * column pair; the table of nibble position
            // j is 4 KB further
            const uint32_t sel = 0x0C0C0000u | ((4u + static_cast<uint32_t>(j >> 1)) << 8);
            const uint32_t addr = __builtin_amdgcn_perm((j & 1) ? mo : me, col_byte, sel);
            const f32x2_sl v = *reinterpret_cast<const SlLdsFloat2*>(static_cast<uintptr_t>(4096 * j) + addr);
            sum.x += v[0];
            sum.y += v[1];
          }
          accp[4 * i4 + ii].x += sum.x;
          accp[4 * i4 + ii].y += sum.y;
        }
      }
    }
    if (kc + 1 < nch) lstore(kc + 1, buf ^ 1, rg);
    __syncthreads();
  };
  // The epilogue's cell state and biases are requested before the K loop, so that their latency
  // overlaps it: lane (wave w, fi, fk) owns unit 4 w + fk of the slice for columns 16 j + fi.
  const int ul = 4 * wave + fk;  // unit within the slice
  const int unit = u0 + ul;
  float cpre[4], bpre[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = s0 + 16 * j + fi;
    const int m = min(col / a.B, 2 * a.pc - 1);
    const float* bs = a.bias_m + (static_cast<int64_t>(m) * a.L + a.layer) * G4 + unit;
#pragma unroll
    for (int r = 0; r < 4; ++r) bpre[j][r] = bs[r * H];
    cpre[j] = a.first ? 0.f : a.c[static_cast<int64_t>(unit) * a.ncp + col];
  }
  if constexpr (kDirect) {
    // one chunk ahead: a deeper request queue needs a second register set, and the 158 registers
    // it takes leave three workgroups per CU, which measured slower than four
    gload(0, rg);
    lstore(0, 0, rg);
    __syncthreads();
    for (int kc = 0; kc < nch; ++kc) {
      if (kc + 1 < nch) gload(kc + 1, rg);
      step(kc);
      if (kc + 1 < nch) lstore(kc + 1, (kc + 1) & 1, rg);
      __syncthreads();
    }
  } else {
    gload(0, rg);
    lstore(0, 0, rg);
    __syncthreads();
    for (int kc = 0; kc < nch; ++kc) step(kc);
  }

  // last layer: the output weights of the slice's units (W_out^T rows u0 .. u0 + 15; wave w
  // reads rows w + 4 i, lane = logit) and the output sign words of the block's pairs are
  // requested now, ahead of the cell, and staged in LDS after it
  constexpr int kOutW = kSlUnits / 4;
  float wo_r[kOutW];
  uint32_t so_r[kMaxPairs / 4];
  if (a.last) {
#pragma unroll
    for (int i = 0; i < kOutW; ++i)
      wo_r[i] = lane < a.V ? a.wt_out[static_cast<int64_t>(u0 + wave + 4 * i) * a.V + lane] : 0.f;
    const int wi = u0 >> 5;  // the 16 units lie in one 32-column sign word
#pragma unroll
    for (int i = 0; i < kMaxPairs / 4; ++i) {
      const int qi = wave + 4 * i;  // wave-uniform
      so_r[i] = 0u;
      if (qi < n_q && lane < a.V)
        so_r[i] = a.sg_out[(static_cast<int64_t>(q_first + qi) * (H >> 5) + wi) * a.V + lane];
    }
  }

  // ---- P x to the matrix-core layout, through LDS (the tables are no longer needed) ----
  float* pbuf = reinterpret_cast<float*>(lds);
  if constexpr (!kDirect) {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<float2*>(pbuf + (8 * rgp + i) * kSlPStride + 2 * cp) = accp[i];
    __syncthreads();
  }

  // ---- cell: lane holds gates 0..3 of unit 4 w + lane / 16 for columns 16 j + lane % 16 ----
  float* hs = reinterpret_cast<float*>(lds + kHsOff);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int cl = 16 * j + fi, col = s0 + cl;
    const int m = min(col / a.B, 2 * a.pc - 1);
    const float se = (m & 1) ? -a.eps : a.eps;  // +eps model: W + s eps P; -eps model: W - s eps P
    float g[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      g[r] = kDirect ? acc[j][r] + bpre[j][r] : fmaf(se, pbuf[(16 * r + ul) * kSlPStride + cl], acc[j][r]) + bpre[j][r];
    const int64_t at = static_cast<int64_t>(unit) * a.ncp + col;
    float cn, hn;
    lstm_cell(g[0], g[1], g[2], g[3], cpre[j], cn, hn);
    if (col < a.ncols) {
      a.c[at] = cn;
      a.h_out[at] = hn;
    }
    hs[ul * kSlCols + cl] = hn;
  }
  if (!a.last) return;

  // ---- partial logits of the slice's 16 units. The W^T buffers are free after the K loop: they
  // take the output weights [16 units][64] and the sign words [pair][64]. Item e of the block is
  // (column e / V, logit e % V), so that consecutive threads write consecutive floats of zpart
  // [slice][column][V] and every lane has work whatever V is.
  float* ws = reinterpret_cast<float*>(lds + kWOff);
  uint32_t* so = reinterpret_cast<uint32_t*>(lds + kWOff) + kSlUnits * kSlMaxV;
#pragma unroll
  for (int i = 0; i < kOutW; ++i) ws[(wave + 4 * i) * kSlCols + lane] = wo_r[i];
#pragma unroll
  for (int i = 0; i < kMaxPairs / 4; ++i) so[(wave + 4 * i) * kSlCols + lane] = so_r[i];
  __syncthreads();
  // units u0 .. u0 + 15 are columns 0-15 or 16-31 of their sign word; shifted right by `half`, the
  // bit of unit u0 + u is at (u & 1) 16 + (u >> 1) either way
  const uint32_t half = static_cast<uint32_t>(u0 & 16) >> 1;
  const int n_items = min(kSlCols, a.ncols - s0) * a.V;
  for (int e = tid; e < n_items; e += kSlThreads) {
    const int cl = static_cast<int>(static_cast<uint32_t>(e) / static_cast<uint32_t>(a.V));
    const int v = e - cl * a.V;
    const int col = s0 + cl;
    const int m = col / a.B;
    // a column whose target at t is not scored adds nothing to its loss: its logits are not formed
    if (a.tg[static_cast<int64_t>(col - m * a.B) * a.tg_stride + a.t] < 0) continue;
    // the -eps model of a pair takes the opposite sign: w - s eps = w + (-s) eps exactly
    const uint32_t word = (so[((m >> 1) - q_first) * kSlCols + v] >> half) ^ ((m & 1) ? 0xFFFFFFFFu : 0u);
    float z = 0.f;
#pragma unroll
    for (int u = 0; u < kSlUnits; ++u) {
      const float wp = ws[u * kSlCols + v] + signed_eps(a.eps, (word >> ((u & 1) * 16 + (u >> 1))) & 1u);
      z = fmaf(wp, hs[u * kSlCols + cl], z);
    }
    a.zpart[(static_cast<int64_t>(blockIdx.x) * a.ncp + col) * a.V + v] = z;
  }
}

// Logits and cross-entropy of timestep t: one wave per column, lane v holds logit v = bout_m[m][v]
// plus the slices of zpart in order; seq[column] accumulates logsumexp(z) - z[target] over the
// timesteps whose target is scored (target >= 0), starting from zero at t = 0. Block 256 (four
// columns), grid ceil(ncols / 4).
__global__ __launch_bounds__(256) void k_ce_f32_sliced(const float* __restrict__ zpart, const float* __restrict__ bout_m,
                                                       const int32_t* __restrict__ tg, int tg_stride, int t, int V,
                                                       int B, int n_slices, int ncols, int ncp, float* __restrict__ seq) {
  const int lane = threadIdx.x & 63;
  const int col = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (col >= ncols) return;  // whole waves
  const int m = col / B, b = col - m * B;
  const int y = tg[static_cast<int64_t>(b) * tg_stride + t];
  if (y < 0) {  // not scored: the column's partial logits were not formed
    if (lane == 0 && t == 0) seq[col] = 0.f;
    return;
  }
  const bool on = lane < V;
  float z = -INFINITY;
  if (on) {
    const float* zp = zpart + static_cast<int64_t>(col) * V + lane;
    const int64_t step = static_cast<int64_t>(ncp) * V;
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    int r = 0;
    // four independent loads in flight; the sum itself runs over the slices in order
    for (; r + 4 <= n_slices; r += 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) part[k] = zp[(r + k) * step];
      z = (r == 0) ? bout_m[static_cast<int64_t>(m) * V + lane] : z;
#pragma unroll
      for (int k = 0; k < 4; ++k) z += part[k];
    }
    if (r == 0) z = bout_m[static_cast<int64_t>(m) * V + lane];
    for (; r < n_slices; ++r) z += zp[r * step];
  }
  float zmax = z;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) zmax = fmaxf(zmax, __shfl_xor(zmax, o));
  float e = on ? expf(z - zmax) : 0.f;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) e += __shfl_xor(e, o);
  const float zy = __shfl(z, min(y, V - 1));
  if (lane == 0) seq[col] = (t == 0 ? 0.f : seq[col]) + ((zmax + logf(e)) - zy);
}

// Per-model perturbed copies of a small fp32 tensor [rows][cols]: out[(m rows + r) out_cols + c]
// = w[r][c] + s eps p(r, c), s = +1 for model 2q and -1 for 2q + 1 (pair q = pair0-relative),
// rounded once in fp32. One thread per (model, row, 32-column group).
__global__ void k_model_tensor_f32(const float* __restrict__ src, int rows, int cols, uint32_t tensor,
                                   const uint64_t* __restrict__ seeds, int pair0, int n_models, float eps,
                                   int out_cols, float* __restrict__ out) {
  const int groups = (cols + 31) / 32;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(n_models) * rows * groups) return;
  const int g = static_cast<int>(idx % groups);
  const int r = static_cast<int>((idx / groups) % rows);
  const int m = static_cast<int>(idx / (static_cast<int64_t>(groups) * rows));
  const uint64_t seed = seeds[pair0 + (m >> 1)];
  const float e = (m & 1) ? -eps : eps;
  const PhiloxOut o = sign_block(seed, tensor, static_cast<uint32_t>(r), static_cast<uint32_t>(g >> 2));
  const uint32_t word = pick_word(o, static_cast<uint32_t>(g & 3));
  for (int j = 0; j < 32; ++j) {
    const int c = g * 32 + j;
    if (c >= cols) break;
    const uint32_t bit = (word >> sign_bit_pos(static_cast<uint32_t>(c))) & 1u;
    out[(static_cast<int64_t>(m) * rows + r) * out_cols + c] = src[static_cast<int64_t>(r) * cols + c] + signed_eps(e, bit);
  }
}

}  // namespace cdrge

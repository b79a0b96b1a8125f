// bf16 models on gfx950 matrix cores: one launch per (layer, timestep) computes, for every probe
// pair of a chunk, the perturbed gate product of both models (theta + eps p_i and theta - eps p_i)
// and the fused LSTM cell update; one launch per timestep computes the perturbed logits and the
// cross-entropy of the last layer.
//
// The method evaluates complete recurrent forward passes at perturbed weights (alex-wiki source
// note on arXiv 2505.17852, "Method"); the weights are perturbed by +-eps p_i with Rademacher p_i
// (pith.science review, "What carries the argument"). Here the perturbed weight tile is never
// stored: the probe-independent candidates Wp = bf16(W + eps) and Wm = bf16(W - eps) are built
// once per step, and each probe's tile is a per-element bit select between them, driven by the
// Philox sign bits, done in registers on its way into LDS. The +eps and -eps models of a pair
// share the sign bits and the loaded candidates, so one workgroup computes both.
//
// Tile (one workgroup, 256 threads = 4 waves of 64):
//   rows   : 64 hidden units x 4 gates = 256 gate rows, interleaved so that local row 4u+g is
//            gate g (i, f, g, o) of unit u; a 16x16 MFMA accumulator then holds all four gates of
//            4 units in each lane, and the cell update runs in registers.
//   columns: 128 batch columns of the +eps model and the same 128 of the -eps model.
//   waves  : (row half, model); each wave owns a 128 x 128 block = 8 x 8 MFMA 16x16x32 tiles.
//   K loop : the concatenated reduction [x_t ; h_{t-1}] in chunks of 32, double-buffered in LDS.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels_common.h"

namespace cdrge {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGateThreads = 256;
constexpr int kUnitsPerTile = 64;
constexpr int kTileRows = 4 * kUnitsPerTile;   // 256 gate rows
constexpr int kTileCols = 128;                 // batch columns per model
constexpr int kKChunk = 32;
constexpr int kLdsStride = 40;                 // bf16 per LDS row: 32 + 8 padding (80 bytes)
constexpr int kHsStride = 72;                  // bf16 per row of the h transpose buffer
constexpr size_t kGateLdsBytes =
    sizeof(uint16_t) * (2 * 2 * kTileRows * kLdsStride + 2 * 2 * kTileCols * kLdsStride);

__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-x));
}
__device__ __forceinline__ float fast_tanh(float x) { return 2.f * fast_sigmoid(2.f * x) - 1.f; }

// Per 32-bit pair of bf16 elements (2m, 2m+1): an all-ones half-word where the probe sign is -1.
// Column 2m of the 32-column group reads sign bit m, column 2m+1 bit m+16.
__device__ __forceinline__ uint32_t pair_mask(uint32_t word, int m) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(word), m, 1));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(word), m + 16, 1));
  return (lo & 0x0000ffffu) | (hi & 0xffff0000u);
}

struct GateArgs {
  const uint16_t* wp_ih;
  const uint16_t* wm_ih;   // [4H][in] candidates of W_ih
  const uint16_t* wp_hh;
  const uint16_t* wm_hh;   // [4H][H] candidates of W_hh
  const uint16_t* emb_m;   // layer 0 input: per-model perturbed embedding [2P][V][E]
  const int32_t* tokens;   // [B][T+1]
  const uint16_t* x_h;     // layer > 0 input: previous layer's h_t, [Ncols][H]
  const uint16_t* h_prev;  // this layer's h_{t-1}, [Ncols][H] (unused when first)
  uint16_t* h_out;         // this layer's h_t, [Ncols][H]
  float* c;                // this layer's cell state, [H][Ncols], updated in place
  const float* bias_m;     // per-model perturbed gate bias [2P][L][4H]
  const uint64_t* seeds;
  int pair0, in, H, B, V, E, L, layer, t, T, Ncols, first;
  uint32_t tensor_ih, tensor_hh;
};

// grid: (H / 64, ceil(B / 128), pairs in chunk). Columns of model m (= 2q + side) are m*B + b.
__global__ __launch_bounds__(kGateThreads, 1) void k_lstm_gates_bf16(GateArgs a) {
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* As = smem;                                    // [buf][side][256][40]
  uint16_t* Bs = smem + 2 * 2 * kTileRows * kLdsStride;   // [buf][256][40]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rh = wave & 1, side = wave >> 1;
  const int H = a.H;
  const int u0 = blockIdx.x * kUnitsPerTile;
  const int bcol0 = blockIdx.y * kTileCols;
  const int pr = blockIdx.z;
  const uint64_t seed = a.seeds[a.pair0 + pr];

  // Formation: thread tid forms local row tid = 4*unit + gate.
  const int frow = (tid & 3) * H + u0 + (tid >> 2);
  // Operand B staging: thread loads 16 bytes (8 reduction columns, piece bq) of 4 tile columns.
  const int bq = tid & 3;
  int64_t bcol_g[4];
  int btok[4], bmodel[4];
  bool bvalid[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = (tid >> 2) + 64 * j;
    const int sd = n >> 7;
    const int b = bcol0 + (n & 127);
    bvalid[j] = b < a.B;
    bmodel[j] = 2 * pr + sd;
    bcol_g[j] = static_cast<int64_t>(bmodel[j]) * a.B + (bvalid[j] ? b : 0);
    int tok = bvalid[j] ? a.tokens[static_cast<int64_t>(b) * (a.T + 1) + a.t] : 0;
    btok[j] = min(max(tok, 0), a.V - 1);
  }

  const int kx = a.in / kKChunk;
  const int kh = a.first ? 0 : H / kKChunk;
  const int nch = kx + kh;

  uint4 rp[4], rm[4], rb[4];
  PhiloxOut words{0, 0, 0, 0};

  auto load = [&](int c) {
    const uint16_t* wp;
    const uint16_t* wm;
    if (c < kx) {
      wp = a.wp_ih + static_cast<int64_t>(frow) * a.in + kKChunk * c;
      wm = a.wm_ih + static_cast<int64_t>(frow) * a.in + kKChunk * c;
    } else {
      wp = a.wp_hh + static_cast<int64_t>(frow) * H + kKChunk * (c - kx);
      wm = a.wm_hh + static_cast<int64_t>(frow) * H + kKChunk * (c - kx);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      rp[k] = reinterpret_cast<const uint4*>(wp)[k];
      rm[k] = reinterpret_cast<const uint4*>(wm)[k];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t* src;
      if (c < kx) {
        src = (a.layer == 0)
                  ? a.emb_m + (static_cast<int64_t>(bmodel[j]) * a.V + btok[j]) * a.E + kKChunk * c + 8 * bq
                  : a.x_h + bcol_g[j] * H + kKChunk * c + 8 * bq;
      } else {
        src = a.h_prev + bcol_g[j] * H + kKChunk * (c - kx) + 8 * bq;
      }
      rb[j] = bvalid[j] ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
    }
  };

  auto form_store = [&](int c, int buf) {
    const int cc = (c < kx) ? c : c - kx;
    if ((cc & 3) == 0)
      words = sign_block(seed, (c < kx) ? a.tensor_ih : a.tensor_hh, static_cast<uint32_t>(frow),
                         static_cast<uint32_t>(cc >> 2));
    const uint32_t w = pick_word(words, static_cast<uint32_t>(cc & 3));
    const uint32_t p32[16] = {rp[0].x, rp[0].y, rp[0].z, rp[0].w, rp[1].x, rp[1].y, rp[1].z, rp[1].w,
                              rp[2].x, rp[2].y, rp[2].z, rp[2].w, rp[3].x, rp[3].y, rp[3].z, rp[3].w};
    const uint32_t m32[16] = {rm[0].x, rm[0].y, rm[0].z, rm[0].w, rm[1].x, rm[1].y, rm[1].z, rm[1].w,
                              rm[2].x, rm[2].y, rm[2].z, rm[2].w, rm[3].x, rm[3].y, rm[3].z, rm[3].w};
    uint32_t plus[16], minus[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const uint32_t mask = pair_mask(w, m);
      // sign -1: the +eps model takes w - eps (Wm), the -eps model takes w + eps (Wp).
      plus[m] = (mask & m32[m]) | (~mask & p32[m]);
      minus[m] = (mask & p32[m]) | (~mask & m32[m]);
    }
    uint4* ap = reinterpret_cast<uint4*>(As + ((buf * 2 + 0) * kTileRows + tid) * kLdsStride);
    uint4* am = reinterpret_cast<uint4*>(As + ((buf * 2 + 1) * kTileRows + tid) * kLdsStride);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      ap[k] = make_uint4(plus[4 * k], plus[4 * k + 1], plus[4 * k + 2], plus[4 * k + 3]);
      am[k] = make_uint4(minus[4 * k], minus[4 * k + 1], minus[4 * k + 2], minus[4 * k + 3]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = (tid >> 2) + 64 * j;
      *reinterpret_cast<uint4*>(Bs + (buf * 2 * kTileCols + n) * kLdsStride + 8 * bq) = rb[j];
    }
  };

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mma = [&](int buf) {
    const uint16_t* A = As + ((buf * 2 + side) * kTileRows + 128 * rh + (lane & 15)) * kLdsStride + 8 * (lane >> 4);
    const uint16_t* Bp = Bs + (buf * 2 * kTileCols + 128 * side + (lane & 15)) * kLdsStride + 8 * (lane >> 4);
    bf16x8 bfr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(Bp + 16 * j * kLdsStride);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16x8 afr = *reinterpret_cast<const bf16x8*>(A + 16 * i * kLdsStride);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  load(0);
  form_store(0, 0);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    if (c + 1 < nch) load(c + 1);
    mma(c & 1);
    if (c + 1 < nch) form_store(c + 1, (c + 1) & 1);
    __syncthreads();
  }

  // ---- fused LSTM cell: gates -> (c, h); h goes through LDS to leave as whole rows ----------
  uint16_t* Hs = smem;  // [256 tile columns][72], reused after the K loop
  const int m = 2 * pr + side;
  const int G = 4 * H;
  const float* bias = a.bias_m + (static_cast<int64_t>(m) * a.L + a.layer) * G;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ul = 32 * rh + 4 * i + (lane >> 4);
    const int u = u0 + ul;
    const float bi = bias[u], bf = bias[H + u], bg = bias[2 * H + u], bo = bias[3 * H + u];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = 16 * j + (lane & 15);
      const int b = bcol0 + n;
      if (b < a.B) {
        const int64_t gcol = static_cast<int64_t>(m) * a.B + b;
        const float ig = fast_sigmoid(acc[i][j][0] + bi);
        const float fg = fast_sigmoid(acc[i][j][1] + bf);
        const float gg = fast_tanh(acc[i][j][2] + bg);
        const float og = fast_sigmoid(acc[i][j][3] + bo);
        float* cp = a.c + static_cast<int64_t>(u) * a.Ncols + gcol;
        const float cprev = a.first ? 0.f : *cp;
        const float cn = fg * cprev + ig * gg;
        *cp = cn;
        const float hv = og * fast_tanh(cn);
        Hs[(128 * side + n) * kHsStride + ul] = static_cast<uint16_t>(f32_to_bf16_rne(hv));
      }
    }
  }
  __syncthreads();
  {
    const int n = tid;  // tile column
    const int sd = n >> 7;
    const int b = bcol0 + (n & 127);
    if (b < a.B) {
      const int64_t gcol = static_cast<int64_t>(2 * pr + sd) * a.B + b;
      const uint4* src = reinterpret_cast<const uint4*>(Hs + n * kHsStride);
      uint4* dst = reinterpret_cast<uint4*>(a.h_out + gcol * H + u0);
#pragma unroll
      for (int k = 0; k < 8; ++k) dst[k] = src[k];
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Perturbed logits + cross-entropy of the last layer at timestep t, for every probe pair.
// Tile: 64 logit rows (V <= 64, padded) x (128 columns of the +eps model, 128 of the -eps model).
// waves: (64-column half, model); each wave owns 64 x 64 = 4 x 4 MFMA tiles. The softmax over the
// 64 rows of one column spans the 4 lane groups of a wave, reduced with cross-lane shuffles.
// seq[m][b] accumulates sum_t (logsumexp - logit of the next token) in float, in t order.
// ---------------------------------------------------------------------------------------------
constexpr int kCeRows = 64;
constexpr size_t kCeLdsBytes =
    sizeof(uint16_t) * (2 * 2 * kCeRows * kLdsStride + 2 * 2 * kTileCols * kLdsStride);

struct CeArgs {
  const uint16_t* wp;
  const uint16_t* wm;      // W_out candidates [V][H]
  const uint16_t* h;       // last layer h_t [Ncols][H]
  const float* bout_m;     // per-model perturbed output bias [2P][64]
  const int32_t* tokens;   // [B][T+1]
  const uint64_t* seeds;
  float* seq;              // [2P][B]
  int pair0, H, B, V, T, t;
  uint32_t tensor_wout;
};

// grid: (ceil(B / 128), pairs in chunk)
__global__ __launch_bounds__(kGateThreads) void k_logits_ce_bf16(CeArgs a) {
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* As = smem;                                  // [buf][side][64][40]
  uint16_t* Bs = smem + 2 * 2 * kCeRows * kLdsStride;   // [buf][256][40]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ch = wave & 1, side = wave >> 1;
  const int H = a.H;
  const int bcol0 = blockIdx.x * kTileCols;
  const int pr = blockIdx.y;
  const uint64_t seed = a.seeds[a.pair0 + pr];

  const bool former = tid < kCeRows;
  const bool frow_ok = tid < a.V;
  const int frow = frow_ok ? tid : 0;
  const int bq = tid & 3;
  int64_t bcol_g[4];
  bool bvalid[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = (tid >> 2) + 64 * j;
    const int b = bcol0 + (n & 127);
    bvalid[j] = b < a.B;
    bcol_g[j] = static_cast<int64_t>(2 * pr + (n >> 7)) * a.B + (bvalid[j] ? b : 0);
  }
  const int nch = H / kKChunk;
  uint4 rp[4], rm[4], rb[4];
  PhiloxOut words{0, 0, 0, 0};

  auto load = [&](int c) {
    if (former) {
      const uint16_t* wp = a.wp + static_cast<int64_t>(frow) * H + kKChunk * c;
      const uint16_t* wm = a.wm + static_cast<int64_t>(frow) * H + kKChunk * c;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        rp[k] = frow_ok ? reinterpret_cast<const uint4*>(wp)[k] : make_uint4(0, 0, 0, 0);
        rm[k] = frow_ok ? reinterpret_cast<const uint4*>(wm)[k] : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint16_t* src = a.h + bcol_g[j] * H + kKChunk * c + 8 * bq;
      rb[j] = bvalid[j] ? *reinterpret_cast<const uint4*>(src) : make_uint4(0, 0, 0, 0);
    }
  };
  auto form_store = [&](int c, int buf) {
    if (former) {
      if ((c & 3) == 0)
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
        plus[m] = (mask & m32[m]) | (~mask & p32[m]);
        minus[m] = (mask & p32[m]) | (~mask & m32[m]);
      }
      uint4* ap = reinterpret_cast<uint4*>(As + ((buf * 2 + 0) * kCeRows + tid) * kLdsStride);
      uint4* am = reinterpret_cast<uint4*>(As + ((buf * 2 + 1) * kCeRows + tid) * kLdsStride);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ap[k] = make_uint4(plus[4 * k], plus[4 * k + 1], plus[4 * k + 2], plus[4 * k + 3]);
        am[k] = make_uint4(minus[4 * k], minus[4 * k + 1], minus[4 * k + 2], minus[4 * k + 3]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = (tid >> 2) + 64 * j;
      *reinterpret_cast<uint4*>(Bs + (buf * 2 * kTileCols + n) * kLdsStride + 8 * bq) = rb[j];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](int buf) {
    const uint16_t* A = As + ((buf * 2 + side) * kCeRows + (lane & 15)) * kLdsStride + 8 * (lane >> 4);
    const uint16_t* Bp =
        Bs + (buf * 2 * kTileCols + 128 * side + 64 * ch + (lane & 15)) * kLdsStride + 8 * (lane >> 4);
    bf16x8 bfr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(Bp + 16 * j * kLdsStride);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8 afr = *reinterpret_cast<const bf16x8*>(A + 16 * i * kLdsStride);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[j], acc[i][j], 0, 0, 0);
    }
  };

  load(0);
  form_store(0, 0);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    if (c + 1 < nch) load(c + 1);
    mma(c & 1);
    if (c + 1 < nch) form_store(c + 1, (c + 1) & 1);
    __syncthreads();
  }

  const int m = 2 * pr + side;
  const float* bout = a.bout_m + static_cast<int64_t>(m) * kCeRows;
  const int g = lane >> 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = 64 * ch + 16 * j + (lane & 15);
    const int b = bcol0 + n;
    const bool ok = b < a.B;
    int y = ok ? a.tokens[static_cast<int64_t>(b) * (a.T + 1) + a.t + 1] : 0;
    y = min(max(y, 0), a.V - 1);
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
      const float l = (zmax + __logf(sum)) - zy;
      float* dst = a.seq + static_cast<int64_t>(m) * a.B + b;
      *dst = (a.t == 0) ? l : *dst + l;
    }
  }
}

}  // namespace cdrge

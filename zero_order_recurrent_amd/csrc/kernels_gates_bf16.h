// Perturbed LSTM gate product + fused cell update for bf16 models on gfx950 matrix cores.
//
// One launch per (layer, timestep) computes, for every probe pair of a chunk, the gate
// pre-activations of both perturbed models (theta + eps p_i and theta - eps p_i),
//   G = (W_ih +- eps P_ih) x_t + (W_hh +- eps P_hh) h_{t-1} + (b +- eps p_b),
// and applies the LSTM cell to them in registers. This is the complete recurrent forward pass at
// perturbed weights that the method evaluates (alex-wiki source note on arXiv 2505.17852,
// "Method"), with Rademacher perturbations (pith.science review, "What carries the argument").
//
// The perturbed weight tile is never stored to memory: per step the probe-independent candidates
// Wp = bf16(W + eps) and Wm = bf16(W - eps) exist once in memory, and each probe's tile is a
// per-element bit select between them, driven by the probe's Philox sign bits, done in registers
// on the way into LDS. Both models of a pair share the loaded candidates and the sign bits.
//
// Workgroup tile (512 threads = 8 waves of 64 lanes, two per SIMD):
//   rows    128 gate rows = 32 hidden units x 4 gates, interleaved (local row 4u + g is gate g of
//           unit u) so that each lane's 16x16 accumulator holds all four gates of one unit;
//   columns 256 batch columns of the +eps model and the same 256 of the -eps model;
//   waves   (model, column quarter): each wave owns 128 x 64 = 8 x 4 MFMA 16x16x32 tiles
//           (128 accumulator registers per lane); the two waves of a SIMD overlap one's weight
//           select work with the other's MFMAs;
//   K loop  the concatenated reduction [x_t ; h_{t-1}] in chunks of 32. The activation operand
//           moves global -> LDS with direct 16-byte loads into an XOR-swizzled (bank-conflict-free)
//           three-stage ring, issued two chunks ahead; the weight candidates of the next chunk are
//           loaded coalesced into registers before the current chunk's MFMAs, then selected and
//           written to a padded two-stage LDS tile.
// The 1-D grid is ordered so that the 32 workgroups resident on one XCD at a time cover 8 row
// tiles x 4 column blocks, which keeps their shared weight and activation chunks in that XCD's L2.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels_common.h"

namespace cdrge {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGateThreads = 512;
constexpr int kUnitsPerTile = 32;
constexpr int kTileRows = 4 * kUnitsPerTile;   // 128 gate rows
constexpr int kTileCols = 256;                 // batch columns per model
constexpr int kKChunk = 32;
constexpr int kAStride = 40;                   // bf16 per LDS row of the weight tile (32 + 8 pad)
constexpr int kHsStride = 40;                  // bf16 per row of the h transpose buffer
constexpr int kAStageElems = 2 * kTileRows * kAStride;        // both models
constexpr int kBStageElems = 2 * kTileCols * kKChunk;         // 512 columns x 32, swizzled
constexpr int kAStages = 2;
constexpr int kBStages = 3;
constexpr size_t kGateBiasOffset = sizeof(uint16_t) * (kAStages * kAStageElems + kBStages * kBStageElems);
constexpr size_t kGateLdsBytes = kGateBiasOffset + sizeof(float) * 2 * 4 * kUnitsPerTile;  // + gate biases

__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-x));
}
__device__ __forceinline__ float fast_tanh(float x) { return 2.f * fast_sigmoid(2.f * x) - 1.f; }

// LSTM cell from the four gate pre-activations, with the reciprocals merged:
//   sigmoid(x) = 1/(1+e^-x), tanh(x) = (1-e^-2x)/(1+e^-2x),
//   c' = c sigmoid(f) + sigmoid(i) tanh(g) = (c A Gm + Gp F) / (F A Gm),
//   h  = sigmoid(o) tanh(c') = (1 - e^-2c') / (O (1 + e^-2c')),
// with A = 1+e^-i, F = 1+e^-f, Gp/Gm = 1 -/+ e^-2g, O = 1+e^-o. Arguments are clamped to
// [-15, 15] (sigmoid(-15) = 3e-7, tanh(15) = 1 in float), which bounds every product below 1e27;
// the clamp is written with comparisons so that a NaN argument stays NaN.
__device__ __forceinline__ float clamp15(float x) { return x < -15.f ? -15.f : (x > 15.f ? 15.f : x); }
__device__ __forceinline__ void lstm_cell(float gi, float gf, float gg, float go, float c, float& c_out,
                                          float& h_out) {
  const float A = 1.f + __expf(-clamp15(gi));
  const float F = 1.f + __expf(-clamp15(gf));
  const float eg = __expf(-2.f * clamp15(gg));
  const float O = 1.f + __expf(-clamp15(go));
  const float Gm = 1.f + eg, Gp = 1.f - eg;
  const float AG = A * Gm;
  const float cn = (c * AG + Gp * F) * __builtin_amdgcn_rcpf(F * AG);
  const float ec = __expf(-2.f * clamp15(cn));
  c_out = cn;
  h_out = (1.f - ec) * __builtin_amdgcn_rcpf(O * (1.f + ec));
}

// Position of 16-byte piece p (k = 8p..8p+7) of activation column c inside an LDS stage: each
// column takes 64 bytes and its pieces are XOR-swizzled with (c >> 2) & 3, so that the 16 lanes
// of one LDS phase, reading the same piece of 16 consecutive columns, cover all 64 banks once.
__device__ __forceinline__ int b_swizzle(int c) { return (c >> 2) & 3; }
__device__ __forceinline__ int b_piece_offset(int c, int p) { return c * 64 + 16 * (p ^ b_swizzle(c)); }

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
  int n_row_tiles, n_col_blocks, n_pairs, swizzle;
  uint32_t tensor_ih, tensor_hh;
};

// Row tile / column block / pair of this workgroup (see the header comment for the XCD order).
__device__ __forceinline__ void gate_tile_of_block(const GateArgs& a, int& rt, int& cb, int& pr) {
  const int L = blockIdx.x;
  int rtile, cw;
  if (a.swizzle) {
    const int n = gridDim.x;            // multiple of 8 * 32 when swizzling
    const int v = (L & 7) * (n >> 3) + (L >> 3);
    const int g = v >> 5, q = v & 31;
    const int n_rg = a.n_row_tiles >> 3;
    rtile = (g % n_rg) * 8 + (q & 7);
    cw = (g / n_rg) * 4 + (q >> 3);
  } else {
    rtile = L % a.n_row_tiles;
    cw = L / a.n_row_tiles;
  }
  rt = rtile;
  cb = cw % a.n_col_blocks;
  pr = cw / a.n_col_blocks;
}

__global__ __launch_bounds__(kGateThreads, 1) void k_lstm_gates_bf16(GateArgs a) {
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* As = smem;                                 // [2 stages][model][128][40]
  uint16_t* Bs = smem + kAStages * kAStageElems;       // [3 stages][512 cols][32] swizzled

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int side = wave >> 2, cq = wave & 3;
  const int H = a.H;
  int rt, cb, pr;
  gate_tile_of_block(a, rt, cb, pr);
  const int u0 = rt * kUnitsPerTile;
  const int bcol0 = cb * kTileCols;
  const uint64_t seed = a.seeds[a.pair0 + pr];

  // ---- weight operand: thread owns local row ra = tid/4 (4 lanes per row), piece q = tid%4 ----
  const int q = tid & 3;
  const int ra = tid >> 2;
  const int grow = (ra & 3) * H + u0 + (ra >> 2);

  // ---- activation operand: 4 direct 16-byte LDS loads per thread per chunk ----
  // Load k of wave w fills bytes [(4w + k) * 1024, +1024) of the stage: lane l -> column
  // (4w + k) * 16 + l / 4, stored slot l % 4, which holds piece (l % 4) ^ swizzle(column).
  // Element offsets are 32-bit (the host guarantees Ncols * H and 2P * V * E fit) from uniform bases.
  const uint16_t* xbase = (a.layer == 0) ? a.emb_m : a.x_h;
  uint32_t xoff[4], hoff[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int c = (4 * wave + k) * 16 + (lane >> 2);
    const int p = (lane & 3) ^ b_swizzle(c);
    const int sd = c >> 8;
    const int b = bcol0 + (c & 255);
    const int bs = (b < a.B) ? b : 0;    // columns past the batch read column 0 (results unused)
    const int m = 2 * pr + sd;
    const uint32_t gcol = static_cast<uint32_t>(m * a.B + bs);
    if (a.layer == 0) {
      int tok = a.tokens[static_cast<int64_t>(bs) * (a.T + 1) + a.t];
      tok = min(max(tok, 0), a.V - 1);
      xoff[k] = static_cast<uint32_t>((m * a.V + tok) * a.E + 8 * p);
    } else {
      xoff[k] = gcol * static_cast<uint32_t>(H) + 8 * p;
    }
    hoff[k] = gcol * static_cast<uint32_t>(H) + 8 * p;
  }

  const int kx = a.in / kKChunk;
  const int kh = a.first ? 0 : H / kKChunk;
  const int nch = kx + kh;

  uint4 wpr, wmr;  // weight candidates of row ra for the next chunk
  PhiloxOut oa{0, 0, 0, 0};

  auto issue_b = [&](int c, int stage) {
    const bool xpart = c < kx;
    const int cc = xpart ? c : c - kx;
    uint16_t* base = Bs + stage * kBStageElems + (4 * wave) * 512;  // 512 bf16 = 1024 bytes per load
    const uint16_t* src = xpart ? xbase : a.h_prev;
    const uint32_t kofs = static_cast<uint32_t>(kKChunk * cc);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t off = (xpart ? xoff[k] : hoff[k]) + kofs;
      __builtin_amdgcn_global_load_lds(src + off, (__attribute__((address_space(3))) void*)(base + k * 512), 16, 0, 0);
    }
  };
  auto load_w = [&](int c, uint4& wp_out, uint4& wm_out) {
    const bool xpart = c < kx;
    const int cc = xpart ? c : c - kx;
    const int ld = xpart ? a.in : H;
    const uint16_t* wp = xpart ? a.wp_ih : a.wp_hh;
    const uint16_t* wm = xpart ? a.wm_ih : a.wm_hh;
    const uint32_t off = static_cast<uint32_t>(grow * ld + kKChunk * cc + 8 * q);
    wp_out = *reinterpret_cast<const uint4*>(wp + off);
    wm_out = *reinterpret_cast<const uint4*>(wm + off);
  };
  // Philox words of the 128-column blocks used by chunks cc..cc+15 of a tensor: each lane of a
  // row's quad evaluates a different block (one call per lane per 16 chunks).
  auto philox_w = [&](int c) {
    const bool xpart = c < kx;
    const int cc = xpart ? c : c - kx;
    if ((cc & 15) == 0) {
      const uint32_t tensor = xpart ? a.tensor_ih : a.tensor_hh;
      oa = sign_block(seed, tensor, static_cast<uint32_t>(grow), static_cast<uint32_t>((cc >> 2) + q));
    }
  };
  // Selects the probe's weights for row ra of chunk c and writes both models' tiles to LDS.
  // The word of chunk c is word (cc & 3) of the block; the lanes keep their four words rotating by
  // one position per chunk (reset by philox_w), so it is always .x - no data-dependent selects.
  auto form_w = [&](int c, const uint4& wpv, const uint4& wmv, int stage) {
    const bool xpart = c < kx;
    const int cc = xpart ? c : c - kx;
    const int owner = (lane & ~3) | ((cc >> 2) & 3);  // the quad lane holding this block
    const uint32_t word = static_cast<uint32_t>(__shfl(static_cast<int>(oa.x), owner));
    oa = PhiloxOut{oa.y, oa.z, oa.w, oa.x};
    // Piece q covers columns 8q..8q+7 of the 32-column word: pairs 4q..4q+3, which read bits
    // 4q+p (even column) and 16+4q+p (odd column).
    const uint32_t t4 = word >> (4 * q);
    const uint32_t pv[4] = {wpv.x, wpv.y, wpv.z, wpv.w}, mv[4] = {wmv.x, wmv.y, wmv.z, wmv.w};
    uint32_t plus[4], minus[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // bits p and p+16 moved to 15 and 31, then replicated over each half-word
      const uint32_t mk = __builtin_amdgcn_perm(0u, t4 << (15 - p), 0x09090808u);
      plus[p] = (mk & mv[p]) | (~mk & pv[p]);   // sign -1: +eps model takes w - eps
      minus[p] = (mk & pv[p]) | (~mk & mv[p]);
    }
    uint16_t* st = As + stage * kAStageElems;
    *reinterpret_cast<uint4*>(st + (0 * kTileRows + ra) * kAStride + 8 * q) = make_uint4(plus[0], plus[1], plus[2], plus[3]);
    *reinterpret_cast<uint4*>(st + (1 * kTileRows + ra) * kAStride + 8 * q) = make_uint4(minus[0], minus[1], minus[2], minus[3]);
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mma = [&](int astage, int bstage) {
    const uint16_t* A = As + astage * kAStageElems + (side * kTileRows + (lane & 15)) * kAStride + 8 * (lane >> 4);
    const char* Bb = reinterpret_cast<const char*>(Bs + bstage * kBStageElems);
    bf16x8 afr[8], bfr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cidx = 256 * side + 64 * cq + 16 * j + (lane & 15);
      bfr[j] = *reinterpret_cast<const bf16x8*>(Bb + b_piece_offset(cidx, lane >> 4));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) afr[i] = *reinterpret_cast<const bf16x8*>(A + 16 * i * kAStride);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[i], bfr[j], acc[i][j], 0, 0, 0);
  };

  // One K step: chunk c is multiplied (A stage c&1, B stage c%3) while the loads of chunk c+1's
  // weights and chunk c+2's activations are in flight; then chunk c+1 is selected into A stage
  // (c+1)&1. The issue sequence has no branches (past the last chunk it reloads the last chunk
  // into a stage that is not read again, and the select writes an unused A stage), so at the
  // wait exactly the 4 activation loads of step c may still be outstanding.
  auto kstep = [&](int c) {
    load_w(min(c + 1, nch - 1), wpr, wmr);
    __builtin_amdgcn_sched_barrier(0);  // weights strictly before activations (wait accounting)
    issue_b(min(c + 2, nch - 1), (c + 2) % kBStages);
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMAs
    mma(c & 1, c % kBStages);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    philox_w(c + 1);
    form_w(c + 1, wpr, wmr, (c + 1) & 1);
    __syncthreads();
  };

  // Gate biases of both models for the tile's 32 units, [model][gate][unit], into LDS.
  float* bias_s = reinterpret_cast<float*>(reinterpret_cast<char*>(smem) + kGateBiasOffset);
  if (tid < 2 * 4 * kUnitsPerTile) {
    const int sd = tid >> 7, g = (tid >> 5) & 3, u = tid & 31;
    bias_s[tid] = a.bias_m[(static_cast<int64_t>(2 * pr + sd) * a.L + a.layer) * (4 * H) + g * H + u0 + u];
  }
  // Cell state of this lane's 8 x 4 cells, loaded now so its latency hides under the K loop.
  const int m_out = 2 * pr + side;
  const uint32_t ncols = static_cast<uint32_t>(a.Ncols);
  float cst[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = bcol0 + 64 * cq + 16 * j + (lane & 15);
      const uint32_t coff = static_cast<uint32_t>(u0 + 4 * i + (lane >> 4)) * ncols +
                            static_cast<uint32_t>(m_out * a.B + (b < a.B ? b : 0));
      cst[i][j] = a.first ? 0.f : a.c[coff];
    }

  // Prologue: activations of chunks 0 and 1 in flight, chunk 0 selected into A stage 0.
  issue_b(0, 0);
  load_w(0, wpr, wmr);
  if (nch > 1) {
    issue_b(1, 1);
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  philox_w(0);
  form_w(0, wpr, wmr, 0);
  __syncthreads();
  for (int c = 0; c < nch; ++c) kstep(c);
  // The last steps leave activation loads in flight; LDS is reused below.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // ---- fused LSTM cell; h leaves through LDS as whole 64-byte column segments ----------------
  uint16_t* Hs = smem;  // [512 columns][40], reused after the K loop
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int ul = 4 * i + (lane >> 4);
    const int u = u0 + ul;
    const float* bs = bias_s + side * 4 * kUnitsPerTile + ul;
    const float bi = bs[0], bf = bs[kUnitsPerTile], bg = bs[2 * kUnitsPerTile], bo = bs[3 * kUnitsPerTile];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cl = 64 * cq + 16 * j + (lane & 15);
      const int b = bcol0 + cl;
      if (b < a.B) {
        const uint32_t coff = static_cast<uint32_t>(u) * ncols + static_cast<uint32_t>(m_out * a.B + b);
        float cn, hv;
        lstm_cell(acc[i][j][0] + bi, acc[i][j][1] + bf, acc[i][j][2] + bg, acc[i][j][3] + bo, cst[i][j], cn, hv);
        a.c[coff] = cn;
        Hs[(256 * side + cl) * kHsStride + ul] = static_cast<uint16_t>(f32_to_bf16_rne(hv));
      }
    }
  }
  __syncthreads();
  {
    const int cidx = tid;  // 0..511
    const int sd = cidx >> 8;
    const int b = bcol0 + (cidx & 255);
    if (b < a.B) {
      const int64_t gcol = static_cast<int64_t>(2 * pr + sd) * a.B + b;
      const uint4* src = reinterpret_cast<const uint4*>(Hs + cidx * kHsStride);
      uint4* dst = reinterpret_cast<uint4*>(a.h_out + gcol * H + u0);
#pragma unroll
      for (int v = 0; v < 4; ++v) dst[v] = src[v];
    }
  }
}

}  // namespace cdrge

// fp32 models (small hidden sizes, long sequences, many probes). One persistent workgroup per
// (G probe pairs, NB sequences) runs the whole perturbed forward of the 2G models - every
// timestep, every layer, the logits and the cross-entropy - with the recurrent state in LDS. The
// models are independent, so no inter-workgroup synchronisation is needed and a probe chunk is
// one launch.
//
// Model (LSTM language model; the pages' "large LSTMs" on next-character prediction, pith.science
// review Figure 2 caption): gates = W_ih x + W_hh h + b in row order i, f, g, o; c = f c + i g;
// h = o tanh(c); logits = W_out h + b_out; loss = logsumexp - logit of the next token.
// Perturbed weight: float(w) + (+-eps) with the sign of probe p_i (include/cdrge.h), rounded once
// in fp32, as a Rademacher perturbation of every weight (pith.science review, "What carries the
// argument").
//
// Work split. A thread owns one weight row (a gate row, or a logit row and a slice of its
// columns) and computes that row's dot products for all 2G*NB (model, sequence) slots of the
// workgroup, so each weight is loaded once for 2G models. Weights are read from per-step k-major
// copies W^T (lanes hold consecutive rows, so every load is coalesced) and the sign bits from
// per-chunk tables of Philox words, one word per (pair, row, 32 columns), also row-fastest.
// Activations live in LDS as [k][slot], so a single broadcast read returns the inputs of every
// slot for one k.
//
// Gate rows use the identity (W + s eps P) x = W x + s eps (P x): the W x part is plain FMAs
// shared by both models of a pair, and P x comes from tables of signed partial sums: for every
// slot and every group of 4 columns that one nibble of a sign word covers, the 16 sums
// +-x_a +-x_b +-x_c +-x_d are built once per timestep and layer in LDS, and a row adds the entry
// its nibble selects. That is a quarter of a table read per column and slot instead of forming
// w + eps and w - eps per column and pair, about half the arithmetic. The result differs from
// summing fl(w +- eps) x only in rounding (the perturbed weight is not rounded to float before
// the product).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels_common.h"

namespace cdrge {

constexpr int kF32MaxThreads = 1024;
constexpr int kF32MaxLayers = 8;
constexpr int kF32MaxSeq = 8;  // NB: sequences per workgroup

// out[c][r] = in[r][c] for a row-major fp32 matrix [rows][cols]; 32 x 32 tiles through LDS.
// grid (ceil(cols / 32), ceil(rows / 32)), 256 threads.
__global__ __launch_bounds__(256) void k_transpose_f32(const float* __restrict__ in, int rows, int cols,
                                                       float* __restrict__ out) {
  __shared__ float tile[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int j = ty; j < 32; j += 8) {
    const int r = r0 + j, c = c0 + tx;
    if (r < rows && c < cols) tile[j][tx] = in[static_cast<int64_t>(r) * cols + c];
  }
  __syncthreads();
  for (int j = ty; j < 32; j += 8) {
    const int c = c0 + j, r = r0 + tx;
    if (r < rows && c < cols) out[static_cast<int64_t>(c) * rows + r] = tile[tx][j];
  }
}

struct F32Args {
  const float* theta;                       // flat parameters: embedding and biases are read here
  int64_t off_emb, off_bout, off_b[kF32MaxLayers];
  const float* wt_ih[kF32MaxLayers];        // W_ih^T [in_l][4H]
  const float* wt_hh[kF32MaxLayers];        // W_hh^T [H][4H]
  const float* wt_out;                      // W_out^T [H][V]
  const uint32_t* sg_ih[kF32MaxLayers];     // sign words [pairs][ceil(in_l / 32)][4H]
  const uint32_t* sg_hh[kF32MaxLayers];     // [pairs][ceil(H / 32)][4H]
  const uint32_t* sg_out;                   // [pairs][ceil(H / 32)][V]
  const int32_t* in;                        // input of (b, t) at in[b * in_stride + t]
  const int32_t* tg;                        // target at tg[b * tg_stride + t]; below zero: not scored
  int in_stride, tg_stride;
  const uint64_t* seeds;                    // all K seeds
  float* seq_out;                           // [2 pc][B]: per (model, sequence) sum over t of the CE
  float eps;
  int L, V, E, H, B, T;
  int pair0, pc;                            // the chunk's first pair and pair count
};

// Offsets (in floats) of the LDS regions; every region starts on a 16-byte boundary.
struct F32Lds {
  int h, c, xin, gbuf, bias, bout, z, loss, tab, tab_h, total;
};
__host__ __device__ inline int f32_pad4(int x) { return (x + 3) & ~3; }
__host__ __device__ inline F32Lds f32_lds_layout(int L, int V, int E, int H, int G, int NB, int NT) {
  const int M = 2 * G * NB, G4 = 4 * H;
  F32Lds o;
  int at = 0;
  o.h = at;    at += f32_pad4(L * H * M);                 // [L][H][M]
  o.c = at;    at += f32_pad4(L * H * M);                 // [L][H][M]
  o.xin = at;  at += f32_pad4(E * M);                     // [E][M]
  const int grows = G4 > NT ? (G4 > V ? G4 : V) : (NT > V ? NT : V);
  o.gbuf = at; at += f32_pad4(grows * M);                 // gates [4H][M], then logit partials [slice][V][M]
  o.bias = at; at += f32_pad4(L * G4 * 2 * G);            // [L][4H][2G]
  o.bout = at; at += f32_pad4(V * 2 * G);                 // [V][2G]
  o.z = at;    at += f32_pad4(V * M);                     // [V][M]
  o.loss = at; at += f32_pad4(M);                         // [M]
  // signed partial sums of the layer input and of h: [word][nibble][slot][16]
  const int wx = ((E > H ? E : H) + 31) >> 5, wh = (H + 31) >> 5;
  o.tab = at;  at += wx * 8 * M * 16;
  o.tab_h = at; at += wh * 8 * M * 16;
  o.total = at;
  return o;
}

// Threads of a workgroup: one per gate row, rounded up to whole waves, at most 1024.
inline int f32_threads(int H) {
  const int r = ((4 * H + 63) / 64) * 64;
  return r < kF32MaxThreads ? r : kF32MaxThreads;
}

template <int M>
__device__ __forceinline__ void f32_load_slots(const float* p, float (&v)[M]) {
  if constexpr (M % 4 == 0) {
#pragma unroll
    for (int i = 0; i < M / 4; ++i) {
      const float4 t = reinterpret_cast<const float4*>(p)[i];
      v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
    }
  } else {
    static_assert(M == 2, "slot counts are 2, 4, 8 or 16");
    const float2 t = *reinterpret_cast<const float2*>(p);
    v[0] = t.x; v[1] = t.y;
  }
}
template <int M>
__device__ __forceinline__ void f32_store_slots(float* p, const float (&v)[M]) {
  if constexpr (M % 4 == 0) {
#pragma unroll
    for (int i = 0; i < M / 4; ++i)
      reinterpret_cast<float4*>(p)[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
  } else {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  }
}

// One column k of the perturbed dot products of row r: for pair g with sign bit s (bit p of
// word[g]; set = -1), the +eps model takes w + s eps and the -eps model w - s eps.
template <int G, int NB>
__device__ __forceinline__ void f32_column(float (&acc)[2 * G * NB], float w, const float* xk,
                                           const uint32_t (&word)[G], uint32_t p, float eps) {
  constexpr int M = 2 * G * NB;
  float xv[M];
  f32_load_slots<M>(xk, xv);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float e = __uint_as_float(__float_as_uint(eps) ^ ((word[g] << (31u - p)) & 0x80000000u));
    const float wp = w + e, wm = w - e;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      acc[(2 * g) * NB + b] = fmaf(wp, xv[(2 * g) * NB + b], acc[(2 * g) * NB + b]);
      acc[(2 * g + 1) * NB + b] = fmaf(wm, xv[(2 * g + 1) * NB + b], acc[(2 * g + 1) * NB + b]);
    }
  }
}

// Tables of signed partial sums of x ([K][M] in LDS) for the nibbles of the sign words:
// tab[((w * 8 + j) * 16 + m) * M + s] = sum over i < 4 of (bit i of m ? -x : x)[col_i][s], where
// col_i is the column of bit position 4 j + i of word w (2 (p & 15) + (p >> 4) for p = 4 j + i);
// columns at or past K count as zero.
template <int M>
__device__ __forceinline__ void f32_build_tables(const float* x, int K, float* tab, int tid, int NT) {
  const int nw = (K + 31) >> 5;
  for (int i = tid; i < nw * 8 * M; i += NT) {
    const int sl = i % M, wj = i / M, j = wj & 7, w = wj >> 3;
    float v[4];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int p = 4 * j + ii;
      const int col = 32 * w + 2 * (p & 15) + (p >> 4);
      v[ii] = col < K ? x[col * M + sl] : 0.f;
    }
    // bits 0, 1 of m select the signs of v0, v1; bits 2, 3 those of v2, v3
    const float lo[4] = {v[0] + v[1], v[1] - v[0], v[0] - v[1], -v[0] - v[1]};
    const float hi[4] = {v[2] + v[3], v[3] - v[2], v[2] - v[3], -v[2] - v[3]};
    // the slots of one nibble value are contiguous, so that the 2 NB slots of a pair (which share
    // the pair's sign word) are read together
    float* dst = tab + static_cast<int64_t>(wj) * 16 * M + sl;
#pragma unroll
    for (int m = 0; m < 16; ++m) dst[m * M] = lo[m & 3] + hi[m >> 2];
  }
}

// accw[slot] += sum_k W[r][k] x[k][slot] and accp[slot] += sum_k p(r, k) x[k][slot] for
// k in [0, K), from W^T (wt[k * ld + r] = W[r][k]), the tensor's sign table with `ld` rows, the
// activations x ([K][M] in LDS) and their tables (f32_build_tables).
template <int G, int NB>
__device__ __forceinline__ void f32_row_dot_split(float (&accw)[2 * G * NB], float (&accp)[2 * G * NB],
                                                  const float* __restrict__ wt, const uint32_t* __restrict__ sg,
                                                  int ld, int r, int K, const float* x, const float* tab,
                                                  const int (&qg)[G]) {
  constexpr int M = 2 * G * NB;
  const int nw = (K + 31) >> 5;
  for (int kw = 0; kw < nw; ++kw) {
    uint32_t word[G];
#pragma unroll
    for (int g = 0; g < G; ++g) word[g] = (sg + (static_cast<int64_t>(qg[g]) * nw + kw) * ld)[r];
    const int k0 = 32 * kw;
    // W^T column k is a wave-uniform base (advanced by one row of W^T per column) plus this
    // lane's 32-bit byte offset; the activations of the 32 columns are at fixed offsets from xk
    const char* wcol = reinterpret_cast<const char*>(wt + static_cast<int64_t>(k0) * ld);
    const size_t wstep = sizeof(float) * static_cast<size_t>(ld);
    const uint32_t roff = static_cast<uint32_t>(r) * 4u;
    const float* xk = x + k0 * M;
    auto column = [&](int kk) {
      const float w = *reinterpret_cast<const float*>(wcol + roff);
      wcol += wstep;
      float xv[M];
      f32_load_slots<M>(xk + kk * M, xv);
#pragma unroll
      for (int i = 0; i < M; ++i) accw[i] = fmaf(w, xv[i], accw[i]);
    };
    if (k0 + 32 <= K) {
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) column(kk);
    } else {
      for (int kk = 0; kk < K - k0; ++kk) column(kk);
    }
    const float* tw = tab + kw * 8 * M * 16;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint32_t nib = (word[g] >> (4 * j)) & 15u;
        float tv[2 * NB];
        f32_load_slots<2 * NB>(tw + (j * 16 + nib) * M + 2 * g * NB, tv);
#pragma unroll
        for (int i = 0; i < 2 * NB; ++i) accp[2 * g * NB + i] += tv[i];
      }
    }
  }
}

// grid (ceil(pc / G), ceil(B / NB)); block f32_threads(H); dynamic LDS f32_lds_layout(...).total
// floats. Slot (g, s, b) = (2g + s) NB + b is sequence b0 + b of model (pair q0 + g, side s).
// A workgroup whose last pair slot has no pair (pc odd) repeats its previous pair there and does
// not write it; slots past the batch compute on zero inputs and are not written either.
template <int G, int NB>
__global__ __launch_bounds__(kF32MaxThreads) void k_lstm_f32(F32Args a) {
  constexpr int M = 2 * G * NB;
  extern __shared__ __align__(16) float lds[];
  const int tid = threadIdx.x, NT = blockDim.x;
  const int L = a.L, V = a.V, E = a.E, H = a.H, G4 = 4 * H;
  const F32Lds lay = f32_lds_layout(L, V, E, H, G, NB, NT);
  float* h = lds + lay.h;
  float* c = lds + lay.c;
  float* xin = lds + lay.xin;
  float* gbuf = lds + lay.gbuf;
  float* bias = lds + lay.bias;
  float* bout = lds + lay.bout;
  float* z = lds + lay.z;
  float* loss = lds + lay.loss;
  float* tab = lds + lay.tab;
  float* tab_h = lds + lay.tab_h;

  const int q0 = blockIdx.x * G;
  const int b0 = blockIdx.y * NB;
  const int nb = min(NB, a.B - b0);
  int qg[G];
  uint64_t seed[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    qg[g] = min(q0 + g, a.pc - 1);
    seed[g] = a.seeds[a.pair0 + qg[g]];
  }

  for (int i = tid; i < L * H * M; i += NT) {
    h[i] = 0.f;
    c[i] = 0.f;
  }
  if (tid < M) loss[tid] = 0.f;
  // Perturbed biases of both models of every pair, once.
  for (int i = tid; i < L * G4 * G; i += NT) {
    const int g = i % G, r = (i / G) % G4, l = i / (G * G4);
    const PhiloxOut o = sign_block(seed[g], 3u + 3u * l, 0u, static_cast<uint32_t>(r >> 7));
    const uint32_t bit = (pick_word(o, (r >> 5) & 3) >> sign_bit_pos(r)) & 1u;
    const float e = signed_eps(a.eps, bit);
    const float w = a.theta[a.off_b[l] + r];
    bias[(l * G4 + r) * 2 * G + 2 * g] = w + e;
    bias[(l * G4 + r) * 2 * G + 2 * g + 1] = w - e;
  }
  for (int i = tid; i < V * G; i += NT) {
    const int g = i % G, v = i / G;
    const PhiloxOut o = sign_block(seed[g], 2u + 3u * L, 0u, static_cast<uint32_t>(v >> 7));
    const uint32_t bit = (pick_word(o, (v >> 5) & 3) >> sign_bit_pos(v)) & 1u;
    const float e = signed_eps(a.eps, bit);
    const float w = a.theta[a.off_bout + v];
    bout[v * 2 * G + 2 * g] = w + e;
    bout[v * 2 * G + 2 * g + 1] = w - e;
  }

  const int nsl = max(1, NT / V);            // column slices of the logits
  const int kper = (H + nsl - 1) / nsl;
  for (int t = 0; t < a.T; ++t) {
    // Layer-0 input: the perturbed embedding rows of the current tokens.
    for (int i = tid; i < E * M; i += NT) {
      const int slot = i % M, e = i / M;
      const int g = slot / (2 * NB), s = (slot / NB) & 1, b = slot % NB;
      float v = 0.f;
      if (b < nb) {
        int tok = a.in[static_cast<int64_t>(b0 + b) * a.in_stride + t];
        tok = min(max(tok, 0), V - 1);  // invalid tokens are reported through the loss (NaN)
        const PhiloxOut o = sign_block(seed[g], 0u, static_cast<uint32_t>(tok), static_cast<uint32_t>(e >> 7));
        const uint32_t bit = (pick_word(o, (e >> 5) & 3) >> sign_bit_pos(e)) & 1u;
        const float ee = signed_eps(a.eps, bit);
        const float w = a.theta[a.off_emb + static_cast<int64_t>(tok) * E + e];
        v = s ? w - ee : w + ee;
      }
      xin[e * M + slot] = v;
    }
    __syncthreads();
    for (int l = 0; l < L; ++l) {
      const int in = (l == 0) ? E : H;
      const float* x = (l == 0) ? xin : h + (l - 1) * H * M;
      const float* hl = h + l * H * M;
      f32_build_tables<M>(x, in, tab, tid, NT);
      if (t > 0) f32_build_tables<M>(hl, H, tab_h, tid, NT);
      __syncthreads();
      for (int r = tid; r < G4; r += NT) {
        float accw[M], accp[M];
#pragma unroll
        for (int i = 0; i < M; ++i) accw[i] = accp[i] = 0.f;
        f32_row_dot_split<G, NB>(accw, accp, a.wt_ih[l], a.sg_ih[l], G4, r, in, x, tab, qg);
        if (t > 0) f32_row_dot_split<G, NB>(accw, accp, a.wt_hh[l], a.sg_hh[l], G4, r, H, hl, tab_h, qg);
        const float* bs = bias + (l * G4 + r) * 2 * G;
        float acc[M];
#pragma unroll
        for (int i = 0; i < M; ++i) {
          const float se = ((i / NB) & 1) ? -a.eps : a.eps;  // +eps model: w + s eps; -eps model: w - s eps
          acc[i] = fmaf(se, accp[i], accw[i]) + bs[i / NB];
        }
        f32_store_slots<M>(gbuf + r * M, acc);
      }
      __syncthreads();
      float* cl = c + l * H * M;
      float* hw = h + l * H * M;
      for (int i = tid; i < H * M; i += NT) {
        const float gi = gbuf[i], gf = gbuf[H * M + i], gg = gbuf[2 * H * M + i], go = gbuf[3 * H * M + i];
        const float ig = 1.f / (1.f + expf(-gi));
        const float fg = 1.f / (1.f + expf(-gf));
        const float gt = tanhf(gg);
        const float og = 1.f / (1.f + expf(-go));
        const float cn = fg * cl[i] + ig * gt;
        cl[i] = cn;
        hw[i] = og * tanhf(cn);
      }
      __syncthreads();
    }
    // Logits: thread (row v, column slice j) forms a partial dot product over its slice.
    const float* hl = h + (L - 1) * H * M;
    for (int i = tid; i < nsl * V; i += NT) {
      const int v = i % V, j = i / V;
      const int k0 = j * kper, k1 = min(H, k0 + kper);
      const int nw = (H + 31) >> 5;
      float acc[M];
#pragma unroll
      for (int i = 0; i < M; ++i) acc[i] = 0.f;
      uint32_t word[G];
      const float* wo = a.wt_out + static_cast<int64_t>(k0) * V + v;  // W_out^T column k, row v
      // columns in groups of 8: the group's weights and the (at most two) sign words its columns
      // fall in are requested together
      for (int kb = k0; kb < k1; kb += 8) {
        float wk[8];
        uint32_t wa[G], wb[G];
        const int kl = min(kb + 7, k1 - 1);
#pragma unroll
        for (int i = 0; i < 8; ++i) wk[i] = kb + i < k1 ? wo[static_cast<int64_t>(kb - k0 + i) * V] : 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const uint32_t* sg = a.sg_out + static_cast<int64_t>(qg[g]) * nw * V + v;
          wa[g] = sg[static_cast<int64_t>(kb >> 5) * V];
          wb[g] = sg[static_cast<int64_t>(kl >> 5) * V];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int k = kb + i;
          if (k >= k1) break;
#pragma unroll
          for (int g = 0; g < G; ++g) word[g] = (k >> 5) == (kb >> 5) ? wa[g] : wb[g];
          f32_column<G, NB>(acc, wk[i], hl + k * M, word, sign_bit_pos(static_cast<uint32_t>(k)), a.eps);
        }
      }
      f32_store_slots<M>(gbuf + (j * V + v) * M, acc);
    }
    __syncthreads();
    for (int i = tid; i < V * M; i += NT) {
      const int v = i / M, slot = i % M;
      float s = bout[v * 2 * G + slot / NB];
      for (int j = 0; j < nsl; ++j) s += gbuf[(j * V + v) * M + slot];
      z[i] = s;
    }
    __syncthreads();
    // Cross-entropy per slot, one wave per slot (lane l: logits l, l + 64, ...; NT is whole
    // waves). The next writes of z and gbuf come after the next barriers.
    for (int slot = tid >> 6; slot < M; slot += NT >> 6) {
      const int lane = tid & 63, b = slot % NB;
      if (b >= nb) continue;  // whole waves
      float zmax = -INFINITY;
      for (int v = lane; v < V; v += 64) zmax = fmaxf(zmax, z[v * M + slot]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) zmax = fmaxf(zmax, __shfl_xor(zmax, o));
      float sum = 0.f;
      for (int v = lane; v < V; v += 64) sum += expf(z[v * M + slot] - zmax);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
      if (lane == 0) {
        const int y = a.tg[static_cast<int64_t>(b0 + b) * a.tg_stride + t];
        if (y >= 0) loss[slot] += (zmax + logf(sum)) - z[min(y, V - 1) * M + slot];
      }
    }
  }
  __syncthreads();
  if (tid < M) {
    const int slot = tid, g = slot / (2 * NB), s = (slot / NB) & 1, b = slot % NB;
    if (b < nb && q0 + g < a.pc)
      a.seq_out[static_cast<int64_t>(2 * (q0 + g) + s) * a.B + b0 + b] = loss[slot];
  }
}

// Sequences per workgroup for a batch of B, and pairs per workgroup for a chunk of P pairs: two
// pairs share each weight load when the chunk has enough pairs to fill the chip twice over.
inline int f32_nb(int B) { return B >= 8 ? 8 : (B >= 4 ? 4 : (B >= 2 ? 2 : 1)); }
inline int f32_g(int NB, int P) { return (NB <= 4 && P >= 512) ? 2 : 1; }

typedef void (*F32Kernel)(F32Args);
inline F32Kernel f32_kernel(int G, int NB) {
  if (G == 2) {
    switch (NB) {
      case 1: return k_lstm_f32<2, 1>;
      case 2: return k_lstm_f32<2, 2>;
      default: return k_lstm_f32<2, 4>;
    }
  }
  switch (NB) {
    case 1: return k_lstm_f32<1, 1>;
    case 2: return k_lstm_f32<1, 2>;
    case 4: return k_lstm_f32<1, 4>;
    default: return k_lstm_f32<1, 8>;
  }
}

}  // namespace cdrge

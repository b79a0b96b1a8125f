// fp32 models (small hidden sizes, long sequences, many probes): one persistent workgroup per
// (probe pair, group of up to 8 sequences) runs the whole perturbed forward of both the +eps and
// the -eps model - every timestep, every layer, the logits and the cross-entropy - with the
// recurrent state in LDS. The models are independent, so no inter-workgroup synchronisation is
// needed and a whole probe chunk is one launch.
//
// Model (LSTM language model; the pages' "large LSTMs" on next-character prediction, pith.science
// review Figure 2 caption): gates = W_ih x + W_hh h + b in row order i, f, g, o; c = f c + i g;
// h = o tanh(c); logits = W_out h + b_out; loss = logsumexp - logit of the next token.
// Perturbed weight: float(w) + (+-eps) with the sign of probe p_i (include/cdrge.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels_common.h"

namespace cdrge {

constexpr int kF32Threads = 256;
constexpr int kF32MaxSeq = 8;  // sequences per workgroup

struct F32Model {
  const float* theta;  // flat parameters
  int64_t off_emb, off_wout, off_bout;
  int64_t off_wih[8], off_whh[8], off_b[8];
  int L, V, E, H, B, T;
};

// Dot products of one weight row (perturbed both ways) with the inputs of both models for nb
// sequences: acc[s][b] += sum_k (w_k + s*e_k) * x[s][b][k], k in [0, n), ascending.
__device__ __forceinline__ void f32_row_dot(const float* __restrict__ wrow, int n, uint64_t seed,
                                            uint32_t tensor, uint32_t row, float eps,
                                            const float* __restrict__ x, int x_stride_seq,
                                            int x_stride_side, int nb, float (&acc)[2][kF32MaxSeq]) {
  PhiloxOut o{0, 0, 0, 0};
  for (int k = 0; k < n; ++k) {
    if ((k & 127) == 0) o = sign_block(seed, tensor, row, static_cast<uint32_t>(k >> 7));
    const uint32_t word = pick_word(o, static_cast<uint32_t>((k >> 5) & 3));
    const uint32_t bit = (word >> sign_bit_pos(static_cast<uint32_t>(k))) & 1u;
    const float w = wrow[k];
    const float e = signed_eps(eps, bit);
    const float wp = w + e;
    const float wm = w - e;
#pragma unroll
    for (int b = 0; b < kF32MaxSeq; ++b) {
      if (b < nb) {
        acc[0][b] = fmaf(wp, x[b * x_stride_seq + k], acc[0][b]);
        acc[1][b] = fmaf(wm, x[x_stride_side + b * x_stride_seq + k], acc[1][b]);
      }
    }
  }
}

// grid: (pairs in chunk, ceil(B / S)), S = min(B, kF32MaxSeq). Dynamic LDS: see layout below.
// seq_out[(2 q + s) * B + b] = sum_t cross-entropy of model (pair q, side s) on sequence b.
__global__ __launch_bounds__(kF32Threads) void k_lstm_f32(F32Model m, const int32_t* __restrict__ tokens,
                                                        const uint64_t* __restrict__ seeds, int pair0,
                                                        float eps, float* __restrict__ seq_out) {
  extern __shared__ float lds[];
  const int tid = threadIdx.x;
  const int q = blockIdx.x;
  const int S = min(kF32MaxSeq, m.B);  // sequences per workgroup (LDS is laid out for S)
  const int b0 = blockIdx.y * S;
  const int nb = min(S, m.B - b0);
  const uint64_t seed = seeds[pair0 + q];
  const int L = m.L, V = m.V, E = m.E, H = m.H, G = 4 * H;
  const int X = max(E, H);

  // LDS layout (floats). Per-side blocks are [S][len].
  float* h = lds;                                  // [L][2][S][H]
  float* c = h + L * 2 * S * H;           // [L][2][S][H]
  float* gates = c + L * 2 * S * H;       // [2][S][G]
  float* xin = gates + 2 * S * G;         // [2][S][X]
  float* bias = xin + 2 * S * X;          // [L][2][G]
  float* bout = bias + L * 2 * G;                  // [2][V]
  float* z = bout + 2 * V;                         // [2][S][V]
  float* loss = z + 2 * S * V;            // [2][S]

  for (int i = tid; i < L * 2 * S * H; i += kF32Threads) {
    h[i] = 0.f;
    c[i] = 0.f;
  }
  if (tid < 2 * S) loss[tid] = 0.f;
  // Perturbed biases of both models, once.
  for (int l = 0; l < L; ++l) {
    for (int r = tid; r < G; r += kF32Threads) {
      const PhiloxOut o = sign_block(seed, 3u + 3u * l, 0u, static_cast<uint32_t>(r >> 7));
      const uint32_t bit = (pick_word(o, (r >> 5) & 3) >> sign_bit_pos(r)) & 1u;
      const float e = signed_eps(eps, bit);
      const float w = m.theta[m.off_b[l] + r];
      bias[(l * 2 + 0) * G + r] = w + e;
      bias[(l * 2 + 1) * G + r] = w - e;
    }
  }
  for (int v = tid; v < V; v += kF32Threads) {
    const PhiloxOut o = sign_block(seed, 2u + 3u * L, 0u, static_cast<uint32_t>(v >> 7));
    const uint32_t bit = (pick_word(o, (v >> 5) & 3) >> sign_bit_pos(v)) & 1u;
    const float e = signed_eps(eps, bit);
    const float w = m.theta[m.off_bout + v];
    bout[v] = w + e;
    bout[V + v] = w - e;
  }
  __syncthreads();

  for (int t = 0; t < m.T; ++t) {
    // Layer-0 input: perturbed embedding rows of the current tokens.
    for (int i = tid; i < nb * E; i += kF32Threads) {
      const int b = i / E, e = i % E;
      int tok = tokens[static_cast<int64_t>(b0 + b) * (m.T + 1) + t];
      tok = min(max(tok, 0), V - 1);  // invalid tokens are reported through the loss (NaN)
      const PhiloxOut o = sign_block(seed, 0u, static_cast<uint32_t>(tok), static_cast<uint32_t>(e >> 7));
      const uint32_t bit = (pick_word(o, (e >> 5) & 3) >> sign_bit_pos(e)) & 1u;
      const float ee = signed_eps(eps, bit);
      const float w = m.theta[m.off_emb + static_cast<int64_t>(tok) * E + e];
      xin[(0 * S + b) * X + e] = w + ee;
      xin[(1 * S + b) * X + e] = w - ee;
    }
    __syncthreads();
    for (int l = 0; l < L; ++l) {
      const int in = (l == 0) ? E : H;
      const float* x = (l == 0) ? xin : (h + (l - 1) * 2 * S * H);
      const int xs = (l == 0) ? X : H;
      const float* hl = h + l * 2 * S * H;
      for (int r = tid; r < G; r += kF32Threads) {
        float acc[2][kF32MaxSeq];
#pragma unroll
        for (int b = 0; b < kF32MaxSeq; ++b) acc[0][b] = acc[1][b] = 0.f;
        f32_row_dot(m.theta + m.off_wih[l] + static_cast<int64_t>(r) * in, in, seed, 1u + 3u * l,
                    static_cast<uint32_t>(r), eps, x, xs, S * xs, nb, acc);
        f32_row_dot(m.theta + m.off_whh[l] + static_cast<int64_t>(r) * H, H, seed, 2u + 3u * l,
                    static_cast<uint32_t>(r), eps, hl, H, S * H, nb, acc);
        for (int b = 0; b < nb; ++b) {
          gates[(0 * S + b) * G + r] = acc[0][b] + bias[(l * 2 + 0) * G + r];
          gates[(1 * S + b) * G + r] = acc[1][b] + bias[(l * 2 + 1) * G + r];
        }
      }
      __syncthreads();
      float* cl = c + l * 2 * S * H;
      float* hw = h + l * 2 * S * H;
      for (int i = tid; i < 2 * nb * H; i += kF32Threads) {
        const int s = i / (nb * H), b = (i / H) % nb, j = i % H;
        const float* g = gates + (s * S + b) * G;
        const float ig = 1.f / (1.f + expf(-g[j]));
        const float fg = 1.f / (1.f + expf(-g[H + j]));
        const float gg = tanhf(g[2 * H + j]);
        const float og = 1.f / (1.f + expf(-g[3 * H + j]));
        const int sidx = (s * S + b) * H + j;
        const float cn = fg * cl[sidx] + ig * gg;
        cl[sidx] = cn;
        hw[sidx] = og * tanhf(cn);
      }
      __syncthreads();
    }
    // Logits of both models from the last layer.
    const float* hl = h + (L - 1) * 2 * S * H;
    for (int v = tid; v < V; v += kF32Threads) {
      float acc[2][kF32MaxSeq];
#pragma unroll
      for (int b = 0; b < kF32MaxSeq; ++b) acc[0][b] = acc[1][b] = 0.f;
      f32_row_dot(m.theta + m.off_wout + static_cast<int64_t>(v) * H, H, seed, 1u + 3u * L,
                  static_cast<uint32_t>(v), eps, hl, H, S * H, nb, acc);
      for (int b = 0; b < nb; ++b) {
        z[(0 * S + b) * V + v] = acc[0][b] + bout[v];
        z[(1 * S + b) * V + v] = acc[1][b] + bout[V + v];
      }
    }
    __syncthreads();
    if (tid < 2 * nb) {
      const int s = tid / nb, b = tid % nb;
      const float* zz = z + (s * S + b) * V;
      float zmax = zz[0];
      for (int v = 1; v < V; ++v) zmax = fmaxf(zmax, zz[v]);
      float sum = 0.f;
      for (int v = 0; v < V; ++v) sum += expf(zz[v] - zmax);
      int y = tokens[static_cast<int64_t>(b0 + b) * (m.T + 1) + t + 1];
      y = min(max(y, 0), V - 1);
      loss[s * S + b] += (zmax + logf(sum)) - zz[y];
    }
    __syncthreads();
  }
  if (tid < 2 * nb) {
    const int s = tid / nb, b = tid % nb;
    seq_out[static_cast<int64_t>(2 * q + s) * m.B + b0 + b] = loss[s * S + b];
  }
}

// Floats of dynamic LDS k_lstm_f32 needs.

inline int64_t f32_lds_floats(int L, int V, int E, int H, int B) {
  const int64_t S = B < kF32MaxSeq ? B : kF32MaxSeq;
  const int64_t G = 4 * int64_t(H), X = (E > H ? E : H);
  return 2 * int64_t(L) * 2 * S * H + 2 * S * G + 2 * S * X + int64_t(L) * 2 * G + 2 * V +
         2 * S * V + 2 * S;
}

}  // namespace cdrge

// CPU oracle — test infrastructure only. Nothing in the product path may include or link this.
//
// The model whose loss CD-RGE evaluates: a character-level LSTM language model.
// The pages fix only "large LSTMs" trained for next-character prediction (pith.science review,
// Figure 2 caption; alex-wiki "Evidence And Limits", Penn Treebank bullet). The architecture
// below is this project's reading, chosen so that torch.nn.LSTM (with its second bias set to
// zero) computes exactly the same function:
//
//   embedding Emb[V][E] -> L stacked LSTM layers (gate order i, f, g, o; one bias per layer)
//   -> linear W_out[V][H] + b_out[V] -> softmax cross-entropy against the next token.
//
//   gates  = W_ih x_t + W_hh h_{t-1} + b            (rows: [i; f; g; o], each H long)
//   i, f, o = sigmoid(.),  g = tanh(.)
//   c_t = f * c_{t-1} + i * g,   h_t = o * tanh(c_t),   h_0 = c_0 = 0
//   loss = (1 / (B T)) * sum_{b,t} [ logsumexp(z_{b,t}) - z_{b,t}[tok[b][t+1]] ]
//
// Inputs and targets. For language modelling the input at step t is tok[b][t] and the target is
// the next token tok[b][t+1]. The synthetic transduction tasks the pages also train on (copy,
// reverse, rolling sum; alex-wiki "Evidence And Limits") give inputs and targets separately, and
// only the output part of a sequence is scored: a target below zero marks a position that adds
// nothing to the loss, and the loss is the mean over the scored positions (torch's cross_entropy
// with an ignore index and mean reduction). With every position scored this is the formula above.
//
// Flat parameter layout (tensor ids are what the Rademacher sign generator is keyed on):
//   id 0: Emb [V][E];  for layer l: id 1+3l W_ih [4H][in_l] (in_0 = E, else H),
//   id 2+3l W_hh [4H][H], id 3+3l b [1][4H];  id 1+3L W_out [V][H];  id 2+3L b_out [1][V].
//   All row-major, concatenated in id order.
//
// Arithmetic: every sum, nonlinearity and the loss are evaluated in the scalar type S (double,
// or a forward-mode dual number for exact directional derivatives). Gate sums run over the W_ih
// terms in ascending column order, then the W_hh terms, then the bias. The only roundings are
// the ones the bf16 model defines: when `round_act_bf16` is set, every activation that enters a
// matrix product (h into W_hh, W_ih of the next layer and W_out) is rounded once to bf16.
#pragma once
#include <cmath>
#include <cstdint>
#include <vector>

#include "bf16.hpp"

namespace oracle {

struct ModelShape {
  int L, V, E, H, B, T;
};

struct TensorInfo {
  uint32_t id;
  int64_t offset, rows, cols;
};

inline std::vector<TensorInfo> lstm_layout(const ModelShape& m) {
  std::vector<TensorInfo> t;
  int64_t off = 0;
  auto add = [&](uint32_t id, int64_t rows, int64_t cols) {
    t.push_back(TensorInfo{id, off, rows, cols});
    off += rows * cols;
  };
  add(0, m.V, m.E);
  for (int l = 0; l < m.L; ++l) {
    const int64_t in = (l == 0) ? m.E : m.H;
    add(1 + 3 * l, 4 * int64_t(m.H), in);
    add(2 + 3 * l, 4 * int64_t(m.H), m.H);
    add(3 + 3 * l, 1, 4 * int64_t(m.H));
  }
  add(1 + 3 * m.L, m.V, m.H);
  add(2 + 3 * m.L, 1, m.V);
  return t;
}

inline int64_t layout_size(const std::vector<TensorInfo>& t) {
  return t.empty() ? 0 : t.back().offset + t.back().rows * t.back().cols;
}

// Forward-mode dual number: value and one directional derivative.
struct Dual {
  double v = 0.0, d = 0.0;
  Dual() = default;
  Dual(double value) : v(value), d(0.0) {}
  Dual(double value, double deriv) : v(value), d(deriv) {}
};
inline Dual operator+(Dual a, Dual b) { return {a.v + b.v, a.d + b.d}; }
inline Dual operator-(Dual a, Dual b) { return {a.v - b.v, a.d - b.d}; }
inline Dual operator-(Dual a) { return {-a.v, -a.d}; }
inline Dual operator*(Dual a, Dual b) { return {a.v * b.v, a.d * b.v + a.v * b.d}; }
inline Dual operator/(Dual a, Dual b) { return {a.v / b.v, (a.d * b.v - a.v * b.d) / (b.v * b.v)}; }
inline Dual& operator+=(Dual& a, Dual b) { return a = a + b; }
inline Dual exp(Dual a) {
  const double e = std::exp(a.v);
  return {e, e * a.d};
}
inline Dual log(Dual a) { return {std::log(a.v), a.d / a.v}; }
inline Dual tanh(Dual a) {
  const double t = std::tanh(a.v);
  return {t, (1.0 - t * t) * a.d};
}
inline double value_of(double x) { return x; }
inline double value_of(const Dual& x) { return x.v; }

template <class S>
inline S sigmoid(S x) {
  using std::exp;
  return S(1.0) / (S(1.0) + exp(-x));
}

// Rounds an activation to bf16 where the bf16 model feeds it to a matrix product. On a dual
// number only the value is rounded (used only with round_act_bf16 = false in practice).
inline double act_round(double x, bool bf) { return bf ? round_to_bf16(x) : x; }
inline Dual act_round(Dual x, bool bf) { return bf ? Dual(round_to_bf16(x.v), x.d) : x; }

// Where the input and the target of (sequence b, step t) are read: inputs[b * in_stride + t] and
// targets[b * tg_stride + t]; a target below zero is not scored.
struct TokenView {
  const int32_t* inputs;
  int64_t in_stride;
  const int32_t* targets;
  int64_t tg_stride;
};

// The language-model view of tokens [B][T+1]: input tok[b][t], target tok[b][t+1].
inline TokenView lm_tokens(const int32_t* tokens, int T) {
  return TokenView{tokens, T + 1, tokens + 1, T + 1};
}

// Number of scored positions of the listed sequences.
inline int64_t scored_positions(const TokenView& tv, int T, const int* seq_ids, int n_seq) {
  int64_t n = 0;
  for (int s = 0; s < n_seq; ++s)
    for (int t = 0; t < T; ++t) n += tv.targets[int64_t(seq_ids[s]) * tv.tg_stride + t] >= 0 ? 1 : 0;
  return n;
}

// Per-sequence loss sums sum_t l_{b,t} over the scored steps, for the requested sequences.
//   W : weights as the model uses them (already perturbed and rounded), flat layout, type P.
//   tv : inputs and targets (see TokenView).
// P is the weight element type (float, double or Dual); S the arithmetic type.
template <class S, class P>
void lstm_sequence_losses(const ModelShape& m, const P* W, const TokenView& tv,
                          const int* seq_ids, int n_seq, bool round_act_bf16, S* seq_loss_out) {
  using std::exp;
  using std::log;
  using std::tanh;
  const auto lay = lstm_layout(m);
  const int H = m.H, L = m.L, V = m.V, E = m.E, T = m.T;
  const P* emb = W + lay[0].offset;
  const P* w_out = W + lay[1 + 3 * L].offset;
  const P* b_out = W + lay[2 + 3 * L].offset;

  std::vector<std::vector<S>> h(L, std::vector<S>(H)), c(L, std::vector<S>(H));
  std::vector<S> xin, hin, gates(4 * int64_t(H)), z(V);
  for (int s = 0; s < n_seq; ++s) {
    const int b = seq_ids[s];
    const int32_t* in_tok = tv.inputs + int64_t(b) * tv.in_stride;
    const int32_t* tg_tok = tv.targets + int64_t(b) * tv.tg_stride;
    for (int l = 0; l < L; ++l) {
      for (int j = 0; j < H; ++j) {
        h[l][j] = S(0.0);
        c[l][j] = S(0.0);
      }
    }
    S total = S(0.0);
    for (int t = 0; t < T; ++t) {
      // Layer-0 input: the embedding row of the current token (already in the model's storage
      // precision, so it needs no activation rounding).
      xin.assign(E, S(0.0));
      for (int e = 0; e < E; ++e) xin[e] = S(emb[int64_t(in_tok[t]) * E + e]);
      for (int l = 0; l < L; ++l) {
        const int in = (l == 0) ? E : H;
        const P* w_ih = W + lay[1 + 3 * l].offset;
        const P* w_hh = W + lay[2 + 3 * l].offset;
        const P* bias = W + lay[3 + 3 * l].offset;
        hin.assign(H, S(0.0));
        for (int j = 0; j < H; ++j) hin[j] = act_round(h[l][j], round_act_bf16);
        for (int r = 0; r < 4 * H; ++r) {
          S acc = S(0.0);
          for (int k = 0; k < in; ++k) acc += S(w_ih[int64_t(r) * in + k]) * xin[k];
          for (int k = 0; k < H; ++k) acc += S(w_hh[int64_t(r) * H + k]) * hin[k];
          acc += S(bias[r]);
          gates[r] = acc;
        }
        for (int j = 0; j < H; ++j) {
          const S ig = sigmoid(gates[j]);
          const S fg = sigmoid(gates[H + j]);
          const S gg = tanh(gates[2 * H + j]);
          const S og = sigmoid(gates[3 * H + j]);
          c[l][j] = fg * c[l][j] + ig * gg;
          h[l][j] = og * tanh(c[l][j]);
        }
        // This layer's output at time t is the next layer's input.
        xin.assign(H, S(0.0));
        for (int j = 0; j < H; ++j) xin[j] = act_round(h[l][j], round_act_bf16);
      }
      // Logits from the last layer's (rounded) output, then cross-entropy with max subtraction.
      const int y = tg_tok[t];
      if (y < 0) continue;  // not scored
      for (int v = 0; v < V; ++v) {
        S acc = S(0.0);
        for (int k = 0; k < H; ++k) acc += S(w_out[int64_t(v) * H + k]) * xin[k];
        acc += S(b_out[v]);
        z[v] = acc;
      }
      int vmax = 0;
      for (int v = 1; v < V; ++v)
        if (value_of(z[v]) > value_of(z[vmax])) vmax = v;
      const S zmax = z[vmax];
      S sum = S(0.0);
      for (int v = 0; v < V; ++v) sum += exp(z[v] - zmax);
      total += (zmax + log(sum)) - z[y];
    }
    seq_loss_out[s] = total;
  }
}

}  // namespace oracle

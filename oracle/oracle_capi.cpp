// CPU oracle — test infrastructure only. Only tests/, the smoke check and the benchmark's CPU
// baseline may load the library built from this file; the HIP product path never does.
//
// A plain, slow, single-threaded implementation of one CD-RGE step on an LSTM language model
// (see cdrge.hpp and lstm.hpp for the method, its sources and the readings taken), exported with
// a C ABI so Python tests can call it through ctypes. Build: g++ -O2 -ffp-contract=off.
#include <cstdint>
#include <cstring>
#include <type_traits>
#include <vector>

#include "cdrge.hpp"

using namespace oracle;

extern "C" {

// Model and probe configuration. storage: 0 = fp32, 1 = bf16 (as uint16 bit patterns),
// 2 = exact (double), 3 = bf16 parameters with the probe added exactly (cdrge.hpp).
struct oracle_cfg {
  int32_t n_layers, vocab, embed, hidden, batch, seq_len, n_probes, storage;
  float eps, lr;
  uint64_t base_seed;
};

static ModelShape shape_of(const oracle_cfg* c) {
  return ModelShape{c->n_layers, c->vocab, c->embed, c->hidden, c->batch, c->seq_len};
}

int64_t oracle_param_count(const oracle_cfg* c) { return layout_size(lstm_layout(shape_of(c))); }

// Writes [id, offset, rows, cols] per tensor; returns the tensor count.
int oracle_layout(const oracle_cfg* c, int64_t* out, int cap) {
  const auto lay = lstm_layout(shape_of(c));
  const int n = static_cast<int>(lay.size());
  for (int i = 0; i < n && i < cap; ++i) {
    out[4 * i + 0] = lay[i].id;
    out[4 * i + 1] = lay[i].offset;
    out[4 * i + 2] = lay[i].rows;
    out[4 * i + 3] = lay[i].cols;
  }
  return n;
}

void oracle_philox(const uint32_t* ctr, uint64_t key, uint32_t* out) {
  const U32x4 x = philox_u64key(U32x4{{ctr[0], ctr[1], ctr[2], ctr[3]}}, key);
  std::memcpy(out, x.w, sizeof(x.w));
}

uint64_t oracle_probe_seed(uint64_t base_seed, uint64_t step, uint32_t i) {
  return probe_seed(base_seed, step, i);
}

int oracle_sign(uint64_t seed, uint32_t tensor, uint32_t row, uint32_t col) {
  return probe_sign(seed, tensor, row, col);
}

// Signs of probe `seed` over a rectangular block of one tensor: out[r][c] for rows
// [r0, r0+nr), columns [c0, c0+nc).
void oracle_sign_block(uint64_t seed, uint32_t tensor, uint32_t r0, uint32_t nr, uint32_t c0,
                       uint32_t nc, int8_t* out) {
  for (uint32_t r = 0; r < nr; ++r)
    for (uint32_t c = 0; c < nc; ++c)
      out[int64_t(r) * nc + c] = static_cast<int8_t>(probe_sign(seed, tensor, r0 + r, c0 + c));
}

// Signs of one probe over the whole LSTM layout (flat order).
void oracle_probe_vector(const oracle_cfg* c, uint64_t seed, int8_t* out) {
  const auto p = probe_vector(lstm_layout(shape_of(c)), seed);
  std::memcpy(out, p.data(), p.size());
}

// Signs of one probe at the listed flat indices of the LSTM layout, each evaluated on its own
// (one Philox call per element, no reuse between elements), for sampled checks of large models.
void oracle_signs_at(const oracle_cfg* c, uint64_t seed, const int64_t* elems, int64_t n,
                     int8_t* out) {
  const auto lay = lstm_layout(shape_of(c));
  LayoutIndexer index(lay);
  for (int64_t q = 0; q < n; ++q) {
    const ElementIndex e = index.at(elems[q]);
    out[q] = static_cast<int8_t>(probe_sign(seed, e.tensor, e.row, e.col));
  }
}

// Per-sequence loss sums of the unperturbed model. `weights` are in the storage given by
// `weight_storage` (0 fp32, 1 bf16 bits, 2 double).
void oracle_lstm_seq_losses(const oracle_cfg* c, const void* weights, int weight_storage,
                            const int32_t* tokens, const int* seq_ids, int n_seq,
                            int round_act_bf16, double* out) {
  const ModelShape m = shape_of(c);
  const int64_t d = layout_size(lstm_layout(m));
  std::vector<double> w(d);
  for (int64_t j = 0; j < d; ++j) w[j] = load_param(weights, static_cast<Storage>(weight_storage), j);
  lstm_sequence_losses<double, double>(m, w.data(), lm_tokens(tokens, m.T), seq_ids, n_seq,
                                       round_act_bf16 != 0, out);
}

// The same with inputs [B][T] and targets [B][T] given separately (a target below zero is not
// scored): the transduction form.
void oracle_lstm_seq_losses_io(const oracle_cfg* c, const void* weights, int weight_storage,
                               const int32_t* inputs, const int32_t* targets, const int* seq_ids,
                               int n_seq, int round_act_bf16, double* out) {
  const ModelShape m = shape_of(c);
  const int64_t d = layout_size(lstm_layout(m));
  std::vector<double> w(d);
  for (int64_t j = 0; j < d; ++j) w[j] = load_param(weights, static_cast<Storage>(weight_storage), j);
  lstm_sequence_losses<double, double>(m, w.data(), TokenView{inputs, m.T, targets, m.T}, seq_ids, n_seq,
                                       round_act_bf16 != 0, out);
}

// Probe losses of a subset of probes on a subset of sequences.
//   losses_out[2k], [2k+1]: mean loss over the scored positions of the selected sequences for
//     probe probe_ids[k] at +eps and -eps (this is the CD-RGE loss when all B sequences are
//     selected), as float.
//   seq_out[(2k+side)*n_seq + s]: the per-sequence sum over the scored steps of the cross-entropy.
// theta is in cfg->storage. Activations are rounded to bf16 for bf16 storage.
static void probe_losses_view(const oracle_cfg* c, const void* theta, const TokenView& tv,
                              uint64_t step, const int* probe_ids, int n_ids, const int* seq_ids,
                              int n_seq, float* losses_out, double* seq_out) {
  const ModelShape m = shape_of(c);
  const auto lay = lstm_layout(m);
  const Storage s = static_cast<Storage>(c->storage);
  const bool round_act = bf16_weights(s);
  const double scored = static_cast<double>(scored_positions(tv, m.T, seq_ids, n_seq));
  std::vector<double> seq(n_seq);
  int side_index = 0;
  auto loss = [&](const auto& w) {
    using P = typename std::decay_t<decltype(w)>::value_type;
    lstm_sequence_losses<double, P>(m, w.data(), tv, seq_ids, n_seq, round_act, seq.data());
    double total = 0.0;
    for (int q = 0; q < n_seq; ++q) {
      total += seq[q];
      if (seq_out) seq_out[int64_t(side_index) * n_seq + q] = seq[q];
    }
    ++side_index;
    return total / scored;
  };
  std::vector<double> out(2 * int64_t(n_ids));
  if (s == Storage::F64 || s == Storage::BF16_EXACTP) {
    probe_losses_generic<double>(lay, theta, s, c->base_seed, step, probe_ids, n_ids, c->eps, loss,
                                 out.data());
  } else {
    // fp32 and bf16 weights are exact in float, which halves the copy for the largest models.
    probe_losses_generic<float>(lay, theta, s, c->base_seed, step, probe_ids, n_ids, c->eps, loss,
                                out.data());
  }
  for (int64_t q = 0; q < 2 * int64_t(n_ids); ++q) losses_out[q] = static_cast<float>(out[q]);
}

// Language-model form: tokens [B][T+1], every position scored.
void oracle_probe_losses(const oracle_cfg* c, const void* theta, const int32_t* tokens,
                         uint64_t step, const int* probe_ids, int n_ids, const int* seq_ids,
                         int n_seq, float* losses_out, double* seq_out) {
  probe_losses_view(c, theta, lm_tokens(tokens, c->seq_len), step, probe_ids, n_ids, seq_ids, n_seq,
                    losses_out, seq_out);
}

// Transduction form: inputs [B][T], targets [B][T] (below zero: not scored).
void oracle_probe_losses_io(const oracle_cfg* c, const void* theta, const int32_t* inputs,
                            const int32_t* targets, uint64_t step, const int* probe_ids, int n_ids,
                            const int* seq_ids, int n_seq, float* losses_out, double* seq_out) {
  probe_losses_view(c, theta, TokenView{inputs, c->seq_len, targets, c->seq_len}, step, probe_ids,
                    n_ids, seq_ids, n_seq, losses_out, seq_out);
}

// The CD-RGE update in place over all elements (elems null) or the listed flat indices.
// Returns 0, or 1 when a loss is not finite.
int oracle_update(const oracle_cfg* c, void* theta, uint64_t step, const float* losses,
                  const int64_t* elems, int64_t n_elems) {
  const auto lay = lstm_layout(shape_of(c));
  return cdrge_update<float>(lay, theta, static_cast<Storage>(c->storage), c->base_seed, step,
                             c->n_probes, losses, c->eps, c->lr, elems, n_elems);
}

// Same update with double losses (estimator checks on exact storage).
int oracle_update_f64losses(const oracle_cfg* c, void* theta, uint64_t step, const double* losses) {
  const auto lay = lstm_layout(shape_of(c));
  return cdrge_update<double>(lay, theta, static_cast<Storage>(c->storage), c->base_seed, step,
                              c->n_probes, losses, c->eps, c->lr, nullptr, 0);
}

// Full CD-RGE step on all probes and sequences: losses_out[2K], theta updated in place.
int oracle_step(const oracle_cfg* c, void* theta, const int32_t* tokens, uint64_t step,
                float* losses_out) {
  std::vector<int> probes(c->n_probes), seqs(c->batch);
  for (int i = 0; i < c->n_probes; ++i) probes[i] = i;
  for (int b = 0; b < c->batch; ++b) seqs[b] = b;
  oracle_probe_losses(c, theta, tokens, step, probes.data(), c->n_probes, seqs.data(), c->batch,
                      losses_out, nullptr);
  return oracle_update(c, theta, step, losses_out, nullptr, 0);
}

// Full CD-RGE step in the transduction form.
int oracle_step_io(const oracle_cfg* c, void* theta, const int32_t* inputs, const int32_t* targets,
                   uint64_t step, float* losses_out) {
  std::vector<int> probes(c->n_probes), seqs(c->batch);
  for (int i = 0; i < c->n_probes; ++i) probes[i] = i;
  for (int b = 0; b < c->batch; ++b) seqs[b] = b;
  oracle_probe_losses_io(c, theta, inputs, targets, step, probes.data(), c->n_probes, seqs.data(),
                         c->batch, losses_out, nullptr);
  return oracle_update(c, theta, step, losses_out, nullptr, 0);
}

// Loss and its exact directional derivative along `direction` (forward-mode dual numbers) for
// exact (double) weights, over all sequences.
void oracle_lstm_dir_deriv(const oracle_cfg* c, const double* theta, const int32_t* tokens,
                           const double* direction, double* value, double* deriv) {
  const ModelShape m = shape_of(c);
  const int64_t d = layout_size(lstm_layout(m));
  std::vector<Dual> w(d);
  for (int64_t j = 0; j < d; ++j) w[j] = Dual(theta[j], direction[j]);
  std::vector<int> ids(m.B);
  for (int b = 0; b < m.B; ++b) ids[b] = b;
  std::vector<Dual> seq(m.B);
  lstm_sequence_losses<Dual, Dual>(m, w.data(), lm_tokens(tokens, m.T), ids.data(), m.B, false, seq.data());
  Dual total(0.0);
  for (int b = 0; b < m.B; ++b) total += seq[b];
  const double scale = 1.0 / (static_cast<double>(m.B) * m.T);
  *value = total.v * scale;
  *deriv = total.d * scale;
}

// Exact gradient by d forward-mode passes (tiny models only).
void oracle_lstm_grad(const oracle_cfg* c, const double* theta, const int32_t* tokens,
                      double* grad) {
  const int64_t d = oracle_param_count(c);
  std::vector<double> dir(d, 0.0);
  double value;
  for (int64_t j = 0; j < d; ++j) {
    dir[j] = 1.0;
    oracle_lstm_dir_deriv(c, theta, tokens, dir.data(), &value, &grad[j]);
    dir[j] = 0.0;
  }
}

// CD-RGE on the quadratic L(theta) = 0.5 * ||A theta - b||^2 (A is m x d, row-major), with
// theta in exact storage laid out as one tensor [1][d] with id 0. Writes the 2n double losses of
// probes 0..n-1 and, when theta_out is not null, the updated theta (eta = lr).
void oracle_quadratic_cdrge(int d, int m, const double* A, const double* b, const double* theta,
                            uint64_t base_seed, uint64_t step, int n, float eps, float lr,
                            double* losses, double* theta_out) {
  const std::vector<TensorInfo> lay{TensorInfo{0, 0, 1, d}};
  auto loss = [&](const std::vector<double>& w) {
    double total = 0.0;
    for (int r = 0; r < m; ++r) {
      double acc = 0.0;
      for (int k = 0; k < d; ++k) acc += A[int64_t(r) * d + k] * w[k];
      const double res = acc - b[r];
      total += 0.5 * res * res;
    }
    return total;
  };
  std::vector<int> ids(n);
  for (int i = 0; i < n; ++i) ids[i] = i;
  probe_losses_generic<double>(lay, theta, Storage::F64, base_seed, step, ids.data(), n, eps, loss,
                               losses);
  if (theta_out) {
    std::memcpy(theta_out, theta, sizeof(double) * d);
    cdrge_update<double>(lay, theta_out, Storage::F64, base_seed, step, n, losses, eps, lr, nullptr,
                         0);
  }
}

// Sign vector of one probe over a single tensor [1][d] with id 0 (the quadratic's layout).
void oracle_flat_probe(uint64_t seed, int d, int8_t* out) {
  const std::vector<TensorInfo> lay{TensorInfo{0, 0, 1, d}};
  const auto p = probe_vector(lay, seed);
  std::memcpy(out, p.data(), p.size());
}

// bf16 rounding entry points (pinned against independent conversions in the tests).
uint16_t oracle_f32_to_bf16(float x) { return f32_to_bf16(x); }
uint16_t oracle_f64_to_bf16(double x) { return f64_to_bf16(x); }
void oracle_f32_to_bf16_array(const float* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(x[i]);
}

}  // extern "C"

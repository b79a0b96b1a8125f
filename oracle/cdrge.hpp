// CPU oracle — test infrastructure only. Nothing in the product path may include or link this.
//
// Central-difference random-vector gradient estimation (CD-RGE), one update step at a time.
//
// The method (pith.science review of arXiv 2505.17852, "What carries the argument"; alex-wiki
// source note, "Method"):
//   g_hat  = (1/K) * sum_i [ L(theta + eps p_i) - L(theta - eps p_i) ] / (2 eps) * p_i
//   theta' = theta - eta * g_hat = theta - eta / (2 K eps) * sum_i d_i p_i,
//   d_i    = L(theta + eps p_i) - L(theta - eps p_i),
// with Rademacher p_i regenerated from per-probe seeds (philox.hpp) and, in the paper's runs,
// eta = eps (the review's version of the update, 1/(2 n_pert) * sum d_i p_i, is the eta = eps case).
//
// Readings taken where the pages are silent (each one is listed in the design notes):
//   * losses[2i] = L(theta + eps p_i), losses[2i+1] = L(theta - eps p_i).
//   * The perturbed model never overwrites theta: the "perturb in place, forward, restore" of the
//     alex-wiki note is taken to restore exactly, so a perturbed copy is built per forward.
//   * Perturbed weight in the model's storage precision: fp32 storage uses the float sum
//     float(w) + float(+-eps); bf16 storage rounds that float sum once more to bf16. Exact
//     storage (double, used only by the estimator checks) adds in double.
//   * coef = eta / (2 K eps) is evaluated in double and rounded once to float, d_i is the float
//     difference of the float losses, the sum over probes and the step are evaluated in double
//     and the result is rounded once to the storage precision.
//   * Any non-finite loss leaves theta unchanged and reports an error.
//   * Exact-perturbation bf16 (storage BF16_EXACTP): bf16 parameters, but the probe is added
//     without rounding the perturbed weight back to bf16, so that radii below the bf16 spacing of
//     a weight still reach the loss: a matrix or bias element becomes w + s * eps' exactly, with
//     eps' = bf16(eps), the radius a bf16 operand can carry (the alex-wiki "Method" section
//     perturbs the weights by eps u_i; the pages fix no precision). The embedding rows are the
//     first product's activations and are rounded to bf16 after the perturbation like every
//     activation. The update's coefficient is eta / (2 K eps'): the central difference of the
//     losses divided by twice the radius actually applied.
#pragma once
#include <cmath>
#include <cstdint>
#include <vector>

#include "bf16.hpp"
#include "lstm.hpp"
#include "philox.hpp"

namespace oracle {

enum class Storage { F32 = 0, BF16 = 1, F64 = 2, BF16_EXACTP = 3 };

inline bool bf16_weights(Storage s) { return s == Storage::BF16 || s == Storage::BF16_EXACTP; }

// The probe radius applied: eps, or bf16(eps) for the exact-perturbation bf16 model.
inline double probe_radius(Storage s, float eps) {
  return s == Storage::BF16_EXACTP ? static_cast<double>(bf16_to_f32(f32_to_bf16(eps))) : static_cast<double>(eps);
}

// Reads a stored parameter as a double.
inline double load_param(const void* theta, Storage s, int64_t j) {
  switch (s) {
    case Storage::F32: return static_cast<const float*>(theta)[j];
    case Storage::BF16:
    case Storage::BF16_EXACTP: return bf16_to_f32(static_cast<const uint16_t*>(theta)[j]);
    default: return static_cast<const double*>(theta)[j];
  }
}

// Writes x to a stored parameter, rounding once to the storage precision.
inline void store_param(void* theta, Storage s, int64_t j, double x) {
  switch (s) {
    case Storage::F32: static_cast<float*>(theta)[j] = static_cast<float>(x); break;
    case Storage::BF16:
    case Storage::BF16_EXACTP: static_cast<uint16_t*>(theta)[j] = f64_to_bf16(x); break;
    default: static_cast<double*>(theta)[j] = x; break;
  }
}

// The perturbed weight w + sigma * eps * p in the storage precision (see the header comment);
// `activation` marks an element that enters a product as an activation (the embedding rows).
inline double perturbed_param(double w, Storage s, int signed_unit, float eps, bool activation = false) {
  switch (s) {
    case Storage::BF16_EXACTP: {
      const double r = probe_radius(s, eps);
      if (activation) return round_to_bf16(static_cast<double>(static_cast<float>(w) + static_cast<float>(signed_unit * r)));
      return w + signed_unit * r;
    }
    case Storage::F32: {
      const float sum = static_cast<float>(w) + static_cast<float>(signed_unit) * eps;
      return sum;
    }
    case Storage::BF16: {
      const float sum = static_cast<float>(w) + static_cast<float>(signed_unit) * eps;
      return bf16_to_f32(f32_to_bf16(sum));
    }
    default: return w + static_cast<double>(signed_unit) * static_cast<double>(eps);
  }
}

// Locates flat element j in the layout: tensor id, row and column.
struct ElementIndex {
  uint32_t tensor, row, col;
};

class LayoutIndexer {
 public:
  explicit LayoutIndexer(const std::vector<TensorInfo>& lay) : lay_(lay) {}
  ElementIndex at(int64_t j) {
    while (!(j >= lay_[cur_].offset && j < lay_[cur_].offset + lay_[cur_].rows * lay_[cur_].cols)) {
      cur_ = (j < lay_[cur_].offset) ? cur_ - 1 : cur_ + 1;
    }
    const TensorInfo& t = lay_[cur_];
    const int64_t local = j - t.offset;
    return ElementIndex{t.id, static_cast<uint32_t>(local / t.cols), static_cast<uint32_t>(local % t.cols)};
  }

 private:
  const std::vector<TensorInfo>& lay_;
  size_t cur_ = 0;
};

// probe_sign with the Philox output of the last (seed, tensor, row, 128-column block) kept, so
// that walking a row costs one Philox evaluation per 128 columns. Same values as probe_sign.
class SignReader {
 public:
  int operator()(uint64_t seed, uint32_t tensor, uint32_t row, uint32_t col) {
    const uint32_t blk = col >> 7;
    if (!valid_ || seed != seed_ || tensor != tensor_ || row != row_ || blk != blk_) {
      words_ = philox_u64key(U32x4{{blk, row, tensor, 0u}}, seed);
      seed_ = seed;
      tensor_ = tensor;
      row_ = row;
      blk_ = blk;
      valid_ = true;
    }
    const uint32_t word = words_.w[(col >> 5) & 3u];
    return ((word >> sign_bit_position(col)) & 1u) ? -1 : +1;
  }

 private:
  U32x4 words_{};
  uint64_t seed_ = 0;
  uint32_t tensor_ = 0, row_ = 0, blk_ = 0;
  bool valid_ = false;
};

// The full Rademacher probe vector for one seed, as +-1 per flat element.
inline std::vector<int8_t> probe_vector(const std::vector<TensorInfo>& lay, uint64_t seed) {
  const int64_t d = layout_size(lay);
  std::vector<int8_t> p(d);
  SignReader sign;
  for (const TensorInfo& t : lay)
    for (int64_t r = 0; r < t.rows; ++r)
      for (int64_t c = 0; c < t.cols; ++c)
        p[t.offset + r * t.cols + c] =
            static_cast<int8_t>(sign(seed, t.id, static_cast<uint32_t>(r), static_cast<uint32_t>(c)));
  return p;
}

// Perturbed copy theta + sigma * eps * p (storage rounding applied), as element type P.
template <class P>
void perturbed_copy(const std::vector<TensorInfo>& lay, const void* theta, Storage s, uint64_t seed,
                    int sigma, float eps, std::vector<P>& out) {
  const int64_t d = layout_size(lay);
  out.resize(d);
  SignReader sign;
  for (const TensorInfo& t : lay)
    for (int64_t r = 0; r < t.rows; ++r)
      for (int64_t c = 0; c < t.cols; ++c) {
        const int64_t j = t.offset + r * t.cols + c;
        const int p = sign(seed, t.id, static_cast<uint32_t>(r), static_cast<uint32_t>(c));
        out[j] = static_cast<P>(perturbed_param(load_param(theta, s, j), s, sigma * p, eps, t.id == 0));
      }
}

// Losses of probes `probe_ids` for a generic loss functor: loss(perturbed weights) -> double.
// out[2k] = L(theta + eps p_{probe_ids[k]}), out[2k+1] = L(theta - eps p_{probe_ids[k]}).
template <class P, class LossFn>
void probe_losses_generic(const std::vector<TensorInfo>& lay, const void* theta, Storage s,
                          uint64_t base_seed, uint64_t step, const int* probe_ids, int n_ids,
                          float eps, LossFn loss, double* out) {
  std::vector<P> w;
  for (int k = 0; k < n_ids; ++k) {
    const uint64_t seed = probe_seed(base_seed, step, static_cast<uint32_t>(probe_ids[k]));
    for (int side = 0; side < 2; ++side) {
      const int sigma = (side == 0) ? +1 : -1;
      perturbed_copy(lay, theta, s, seed, sigma, eps, w);
      out[2 * k + side] = loss(w);
    }
  }
}

// The update coefficient eta / (2 K eps), rounded once to float.
inline float update_coef(int K, float eps, float lr) {
  return static_cast<float>(static_cast<double>(lr) / (2.0 * K * static_cast<double>(eps)));
}

// theta <- theta - coef * sum_i d_i p_i over the elements listed in `elems` (all when null).
// Returns 0, or 1 when a loss is not finite (theta then untouched).
// LossT is float for the model path (d_i is then a float difference, as the losses are floats)
// and double for the estimator checks on exact storage.
template <class LossT>
int cdrge_update(const std::vector<TensorInfo>& lay, void* theta, Storage s, uint64_t base_seed,
                 uint64_t step, int K, const LossT* losses, float eps, float lr,
                 const int64_t* elems, int64_t n_elems) {
  for (int i = 0; i < 2 * K; ++i)
    if (!std::isfinite(losses[i])) return 1;
  std::vector<LossT> dif(K);
  std::vector<uint64_t> seeds(K);
  for (int i = 0; i < K; ++i) {
    dif[i] = losses[2 * i] - losses[2 * i + 1];
    seeds[i] = probe_seed(base_seed, step, static_cast<uint32_t>(i));
  }
  const double coef = update_coef(K, static_cast<float>(probe_radius(s, eps)), lr);
  LayoutIndexer index(lay);
  std::vector<SignReader> sign(K);  // one per probe, so consecutive elements reuse their block
  const int64_t n = elems ? n_elems : layout_size(lay);
  for (int64_t q = 0; q < n; ++q) {
    const int64_t j = elems ? elems[q] : q;
    const ElementIndex e = index.at(j);
    double acc = 0.0;
    for (int i = 0; i < K; ++i) {
      const int p = sign[i](seeds[i], e.tensor, e.row, e.col);
      acc += (p > 0) ? static_cast<double>(dif[i]) : -static_cast<double>(dif[i]);
    }
    store_param(theta, s, j, load_param(theta, s, j) - coef * acc);
  }
  return 0;
}

// Mean LSTM loss over the scored positions of all B sequences (in double).
template <class P>
double lstm_mean_loss(const ModelShape& m, const std::vector<P>& w, const TokenView& tv,
                      bool round_act_bf16) {
  std::vector<int> ids(m.B);
  for (int b = 0; b < m.B; ++b) ids[b] = b;
  std::vector<double> seq(m.B);
  lstm_sequence_losses<double, P>(m, w.data(), tv, ids.data(), m.B, round_act_bf16, seq.data());
  double total = 0.0;
  for (int b = 0; b < m.B; ++b) total += seq[b];
  return total / static_cast<double>(scored_positions(tv, m.T, ids.data(), m.B));
}

}  // namespace oracle

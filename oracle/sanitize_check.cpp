// CPU oracle — test infrastructure only. A driver that runs every entry point of the oracle's C
// API (oracle_capi.cpp) on small configurations, so that the oracle can be built with the host
// sanitizers (AddressSanitizer, UndefinedBehaviorSanitizer) and exercised end to end:
//
//   g++ -std=c++17 -O1 -g -fsanitize=address,undefined -fno-sanitize-recover=all \
//       -ffp-contract=off oracle/oracle_capi.cpp oracle/sanitize_check.cpp -o sanitize_check
//
// It checks a few identities on the way (signs are +-1, the update with d = e_i writes -coef p_i,
// chunked and whole probe lists agree) and exits non-zero on the first failure; a sanitizer
// report also ends the run with a non-zero status.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <vector>

extern "C" {
struct oracle_cfg {
  int32_t n_layers, vocab, embed, hidden, batch, seq_len, n_probes, storage;
  float eps, lr;
  uint64_t base_seed;
};
int64_t oracle_param_count(const oracle_cfg* c);
int oracle_layout(const oracle_cfg* c, int64_t* out, int cap);
void oracle_philox(const uint32_t* ctr, uint64_t key, uint32_t* out);
uint64_t oracle_probe_seed(uint64_t base_seed, uint64_t step, uint32_t i);
int oracle_sign(uint64_t seed, uint32_t tensor, uint32_t row, uint32_t col);
void oracle_sign_block(uint64_t seed, uint32_t tensor, uint32_t r0, uint32_t nr, uint32_t c0, uint32_t nc,
                       int8_t* out);
void oracle_probe_vector(const oracle_cfg* c, uint64_t seed, int8_t* out);
void oracle_signs_at(const oracle_cfg* c, uint64_t seed, const int64_t* elems, int64_t n, int8_t* out);
void oracle_lstm_seq_losses(const oracle_cfg* c, const void* weights, int weight_storage, const int32_t* tokens,
                            const int* seq_ids, int n_seq, int round_act_bf16, double* out);
void oracle_probe_losses(const oracle_cfg* c, const void* theta, const int32_t* tokens, uint64_t step,
                         const int* probe_ids, int n_ids, const int* seq_ids, int n_seq, float* losses_out,
                         double* seq_out);
int oracle_update(const oracle_cfg* c, void* theta, uint64_t step, const float* losses, const int64_t* elems,
                  int64_t n_elems);
int oracle_update_f64losses(const oracle_cfg* c, void* theta, uint64_t step, const double* losses);
int oracle_step(const oracle_cfg* c, void* theta, const int32_t* tokens, uint64_t step, float* losses_out);
void oracle_lstm_dir_deriv(const oracle_cfg* c, const double* theta, const int32_t* tokens,
                           const double* direction, double* value, double* deriv);
void oracle_lstm_grad(const oracle_cfg* c, const double* theta, const int32_t* tokens, double* grad);
void oracle_quadratic_cdrge(int d, int m, const double* A, const double* b, const double* theta,
                            uint64_t base_seed, uint64_t step, int n, float eps, float lr, double* losses,
                            double* theta_out);
void oracle_flat_probe(uint64_t seed, int d, int8_t* out);
uint16_t oracle_f32_to_bf16(float x);
uint16_t oracle_f64_to_bf16(double x);
void oracle_f32_to_bf16_array(const float* x, int64_t n, uint16_t* out);
}

namespace {

int g_failures = 0;

void check(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s\n", what);
    ++g_failures;
  }
}

// A small linear congruential stream for inputs (no method arithmetic).
struct Lcg {
  uint64_t s;
  uint32_t next() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return static_cast<uint32_t>(s >> 33);
  }
  double uniform(double lo, double hi) { return lo + (hi - lo) * (next() / 2147483648.0); }
};

void run_model(int L, int V, int E, int H, int B, int T, int K, int storage) {
  oracle_cfg c{L, V, E, H, B, T, K, storage, 1e-2f, 1e-2f, 4242};
  const int64_t d = oracle_param_count(&c);
  std::vector<int64_t> lay(64 * 4);
  const int nt = oracle_layout(&c, lay.data(), 64);
  check(nt == 3 * L + 3, "tensor count");
  Lcg rng{static_cast<uint64_t>(d) * 7 + storage};
  std::vector<int32_t> tokens(int64_t(B) * (T + 1));
  for (auto& t : tokens) t = static_cast<int32_t>(rng.next() % V);
  std::vector<float> f32(d);
  for (auto& w : f32) w = static_cast<float>(rng.uniform(-0.3, 0.3));
  std::vector<uint16_t> b16(d);
  oracle_f32_to_bf16_array(f32.data(), d, b16.data());
  std::vector<double> f64(f32.begin(), f32.end());
  void* theta = storage == 0 ? static_cast<void*>(f32.data())
                             : storage == 1 ? static_cast<void*>(b16.data()) : static_cast<void*>(f64.data());

  std::vector<int> seqs(B), probes(K);
  for (int b = 0; b < B; ++b) seqs[b] = b;
  for (int i = 0; i < K; ++i) probes[i] = i;
  std::vector<double> seq(B);
  oracle_lstm_seq_losses(&c, theta, storage, tokens.data(), seqs.data(), B, storage == 1, seq.data());
  for (double v : seq) check(std::isfinite(v) && v > 0, "sequence loss finite and positive");

  // whole probe list against one probe at a time, and an empty sequence list
  std::vector<float> losses(2 * K), one(2);
  std::vector<double> seq_out(2 * int64_t(K) * B), seq_one(2 * int64_t(B));
  oracle_probe_losses(&c, theta, tokens.data(), 3, probes.data(), K, seqs.data(), B, losses.data(),
                      seq_out.data());
  for (int i = 0; i < K; ++i) {
    oracle_probe_losses(&c, theta, tokens.data(), 3, &probes[i], 1, seqs.data(), B, one.data(), seq_one.data());
    check(one[0] == losses[2 * i] && one[1] == losses[2 * i + 1], "probe losses independent of the list");
  }
  oracle_probe_losses(&c, theta, tokens.data(), 3, probes.data(), 1, seqs.data(), 0, one.data(), nullptr);

  // signs: vector, uncached element reads and blocks agree
  std::vector<int8_t> p(d), q(d);
  std::vector<int64_t> every(d);
  for (int64_t j = 0; j < d; ++j) every[j] = j;
  const uint64_t seed = oracle_probe_seed(c.base_seed, 3, 0);
  oracle_probe_vector(&c, seed, p.data());
  oracle_signs_at(&c, seed, every.data(), d, q.data());
  check(std::memcmp(p.data(), q.data(), d) == 0, "probe vector equals uncached signs");
  for (int8_t s : p) check(s == 1 || s == -1, "sign is +-1");
  const int64_t rows = lay[4 * 1 + 2], cols = lay[4 * 1 + 3];
  std::vector<int8_t> blk(rows * cols);
  oracle_sign_block(seed, 1, 0, static_cast<uint32_t>(rows), 0, static_cast<uint32_t>(cols), blk.data());
  check(std::memcmp(blk.data(), p.data() + lay[4 * 1 + 1], blk.size()) == 0, "sign block equals vector");
  check(oracle_sign(seed, 1, 0, 0) == p[lay[4 * 1 + 1]], "single sign");

  // update: d = e_0 on theta = 0 gives -coef p_0; a listed subset; a non-finite loss
  std::vector<float> zero(d, 0.f), unit(2 * K, 0.f);
  unit[0] = 1.f;
  oracle_cfg cf = c;
  cf.storage = 0;
  check(oracle_update(&cf, zero.data(), 3, unit.data(), nullptr, 0) == 0, "update status");
  const float coef = static_cast<float>(1.0 / (2.0 * K));
  for (int64_t j = 0; j < d; ++j) check(zero[j] == -coef * p[j], "update writes -coef p");
  std::vector<int64_t> sub;
  for (int64_t j = d - 1; j >= 0; j -= 3) sub.push_back(j);
  check(oracle_update(&c, theta, 3, losses.data(), sub.data(), static_cast<int64_t>(sub.size())) == 0,
        "subset update");
  std::vector<float> bad(losses);
  bad[1] = std::numeric_limits<float>::quiet_NaN();
  check(oracle_update(&c, theta, 3, bad.data(), nullptr, 0) == 1, "non-finite loss rejected");
  check(oracle_step(&c, theta, tokens.data(), 4, losses.data()) == 0, "step");
}

}  // namespace

int main() {
  // bf16 rounding of specials and of a spread of values
  check(oracle_f32_to_bf16(0.f) == 0, "bf16 zero");
  check(oracle_f32_to_bf16(-0.f) == 0x8000, "bf16 negative zero");
  check(oracle_f32_to_bf16(std::numeric_limits<float>::infinity()) == 0x7F80, "bf16 inf");
  check((oracle_f32_to_bf16(std::numeric_limits<float>::quiet_NaN()) & 0x7FFF) > 0x7F80, "bf16 nan");
  check(oracle_f32_to_bf16(std::numeric_limits<float>::denorm_min()) == 0, "bf16 denormal");
  check(oracle_f64_to_bf16(1.0) == 0x3F80, "bf16 one from double");
  uint32_t ctr[4] = {1, 2, 3, 4}, out[4];
  oracle_philox(ctr, 0x0123456789ABCDEFull, out);

  run_model(1, 16, 16, 32, 4, 10, 3, 0);   // the tiny workload's shape, fp32
  run_model(2, 7, 200, 40, 3, 4, 2, 1);    // rows across 128-column Philox blocks, bf16
  run_model(3, 50, 6, 5, 2, 3, 2, 2);      // exact storage
  run_model(1, 2, 1, 1, 1, 1, 1, 0);       // smallest shape

  // exact gradients and directional derivatives (forward-mode) on a tiny model
  {
    oracle_cfg c{1, 5, 3, 4, 2, 3, 1, 2, 1e-3f, 1e-3f, 9};
    const int64_t d = oracle_param_count(&c);
    Lcg rng{11};
    std::vector<double> theta(d), dir(d), grad(d);
    for (auto& w : theta) w = rng.uniform(-0.5, 0.5);
    for (auto& v : dir) v = rng.uniform(-1, 1);
    std::vector<int32_t> tokens(2 * 4);
    for (auto& t : tokens) t = static_cast<int32_t>(rng.next() % 5);
    double value = 0, deriv = 0;
    oracle_lstm_dir_deriv(&c, theta.data(), tokens.data(), dir.data(), &value, &deriv);
    oracle_lstm_grad(&c, theta.data(), tokens.data(), grad.data());
    double dot = 0;
    for (int64_t j = 0; j < d; ++j) dot += grad[j] * dir[j];
    check(std::fabs(dot - deriv) <= 1e-12 * (1 + std::fabs(deriv)), "gradient . direction = derivative");
    std::vector<double> l64(2);
    oracle_cfg ce = c;
    std::vector<double> upd(theta);
    l64[0] = 1.0;
    l64[1] = 0.5;
    check(oracle_update_f64losses(&ce, upd.data(), 0, l64.data()) == 0, "f64 update");
  }
  // the quadratic estimator check
  {
    const int d = 32, m = 64, n = 16;
    Lcg rng{12};
    std::vector<double> A(int64_t(m) * d), b(m), theta(d), losses(2 * n), out(d);
    for (auto& v : A) v = rng.uniform(-1, 1);
    for (auto& v : b) v = rng.uniform(-1, 1);
    for (auto& v : theta) v = rng.uniform(-1, 1);
    oracle_quadratic_cdrge(d, m, A.data(), b.data(), theta.data(), 1, 2, n, 1e-2f, 1e-2f, losses.data(), out.data());
    std::vector<int8_t> fp(d);
    oracle_flat_probe(oracle_probe_seed(1, 2, 0), d, fp.data());
    for (int8_t s : fp) check(s == 1 || s == -1, "flat probe sign");
  }
  if (g_failures) {
    std::fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("sanitized oracle run: all checks passed\n");
  return 0;
}

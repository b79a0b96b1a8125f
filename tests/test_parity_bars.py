"""Planted mistakes, on the oracle alone (no GPU): the probe-difference bar that the bf16 parity
tests apply (parity_bars.py) rejects the mistakes a perturbed forward could make.

Each mistake is planted in the oracle's own results or in a perturbed parameter copy built here
from the oracle's probe vector and its bf16 rounding (the same copy the oracle builds, which the
first test checks bit for bit):
  * the two signs swapped (the + model run with -eps p_i and the - model with +eps p_i);
  * another probe's seed, or the seeds of another update step;
  * one tensor left unperturbed in both models, or perturbed with the same sign in both.
The bar must reject each with a margin (error at least 1.5 times the bar, 1.25 at eps = 1e-4). One tensor's mistake
is required only in the cases where every tensor carries a good share of d_i (eps = 2^-3); with
a smaller eps or theta = 0 the output bias carries most of d_i and a layer-0 tensor can carry
less than the bar's 2%.
"""
import numpy as np
import pytest

from oracle import OracleConfig
from parity_bars import PER_TENSOR, PROBE_CASES, diff_errors, probe_case_inputs

MARGIN = 1.5
STEP = 2


def _cfg(case):
    L, V, E, H, B, T, K, eps, base, ppc, zero = case
    return OracleConfig(L, V, E, H, B, T, K, "bf16", eps, eps, base)


def _bits_to_f32(u):
    return (np.asarray(u, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _copy(oracle, cfg, w_bits, step, i, sigma):
    """bf16(float(w) + sigma[t] * eps * p_i) per tensor t; sigma[t] = 0 leaves tensor t as is."""
    p = oracle.probe_vector(cfg, oracle.probe_seed(cfg.base_seed, step, i)).astype(np.float32)
    w32 = _bits_to_f32(w_bits)
    out = np.array(w_bits, copy=True)
    for tid, off, rows, cols in oracle.layout(cfg):
        if sigma[tid] == 0:
            continue
        sl = slice(off, off + rows * cols)
        out[sl] = oracle.f32_to_bf16(w32[sl] + np.float32(sigma[tid]) * np.float32(cfg.eps) * p[sl])
    return out


def _pair(oracle, cfg, w_bits, tokens, seqs, step, i, sig_plus, sig_minus):
    rows = []
    for sigma in (sig_plus, sig_minus):
        w = _copy(oracle, cfg, w_bits, step, i, sigma)
        rows.append(oracle.seq_losses(cfg, w, tokens, seq_ids=seqs, round_act_bf16=True))
    return np.stack(rows)


@pytest.mark.parametrize("name", list(PROBE_CASES))
def test_bar_rejects_planted_mistakes_where_the_probe_dominates(oracle, name):
    case = PROBE_CASES[name]
    cfg = _cfg(case)
    theta, tokens = probe_case_inputs(case)
    w = oracle.f32_to_bf16(theta)
    seqs = list(range(0, cfg.batch, max(1, cfg.batch // 24)))[:24]
    lay = oracle.layout(cfg)
    n_t = len(lay)
    _, ref = oracle.probe_losses(cfg, w, tokens, STEP, probe_ids=[0], seq_ids=seqs)
    # the copy built here is the oracle's own perturbed copy
    both = _pair(oracle, cfg, w, tokens, seqs, STEP, 0, [1] * n_t, [-1] * n_t)
    np.testing.assert_array_equal(both, ref)
    assert max(diff_errors(ref, ref)) == 0.0

    def rejected(bad, what):
        e = max(diff_errors(bad, ref))
        assert e >= MARGIN, f"{name}: {what} gives only {e:.2f} x the bar"

    rejected(ref[::-1], "swapped signs")
    _, other = oracle.probe_losses(cfg, w, tokens, STEP, probe_ids=[1], seq_ids=seqs)
    rejected(other, "probe 1's seed")
    _, other = oracle.probe_losses(cfg, w, tokens, STEP + 1, probe_ids=[0], seq_ids=seqs)
    rejected(other, "the next step's seeds")
    if name not in PER_TENSOR:
        return
    for t in range(n_t):
        plus, minus = [1] * n_t, [-1] * n_t
        plus[t] = minus[t] = 0
        rejected(_pair(oracle, cfg, w, tokens, seqs, STEP, 0, plus, minus), f"tensor {t} unperturbed")
        minus[t] = 1
        plus[t] = 1
        rejected(_pair(oracle, cfg, w, tokens, seqs, STEP, 0, plus, minus), f"tensor {t} with one sign")


# The eps = 1e-4 and 1e-3 bf16 shapes of the GPU parity tests: the bar still rejects a swapped
# sign and another probe's or step's seeds there (margin 1.25: over 64 timesteps the rounding
# floor is a larger share of the bar).
SMALL_EPS = {
    "bf16_ragged": (2, 50, 64, 128, 160, 3, 3, 1e-4, 79),
    "bf16_ce_split": (1, 50, 32, 416, 40, 3, 2, 1e-4, 84),
    "bf16_long": (2, 50, 64, 128, 24, 64, 2, 1e-4, 87),
    "bf16_v64": (3, 64, 96, 192, 130, 2, 2, 1e-3, 81),
}


@pytest.mark.parametrize("name", list(SMALL_EPS))
def test_bar_rejects_wrong_sign_or_probe_at_small_eps(oracle, name):
    L, V, E, H, B, T, K, eps, base = SMALL_EPS[name]
    cfg = OracleConfig(L, V, E, H, B, T, K, "bf16", eps, eps, base)
    rng = np.random.default_rng(5)
    d = oracle.param_count(cfg)
    bound = 1.0 / np.sqrt(H)
    w = oracle.f32_to_bf16(rng.uniform(-bound, bound, d).astype(np.float32))
    tokens = rng.integers(0, V, size=(B, T + 1)).astype(np.int32)
    seqs = list(range(min(B, 24)))
    _, ref = oracle.probe_losses(cfg, w, tokens, STEP, probe_ids=[0], seq_ids=seqs)
    for what, bad in [("swapped signs", ref[::-1]),
                      ("probe 1's seed", oracle.probe_losses(cfg, w, tokens, STEP, probe_ids=[1], seq_ids=seqs)[1]),
                      ("the next step's seeds", oracle.probe_losses(cfg, w, tokens, STEP + 1, probe_ids=[0],
                                                                    seq_ids=seqs)[1])]:
        e = max(diff_errors(bad, ref))
        assert e >= 1.25, f"{name}: {what} gives only {e:.2f} x the bar"

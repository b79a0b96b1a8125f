"""Parity bars that see the probe.

A probe moves a bf16 loss by far less than the 2e-2 relative bar that the losses are held to, so
that bar alone cannot tell a forward that applies +eps p_i / -eps p_i from one that applies the
wrong sign, the wrong probe or no perturbation to some tensor. The quantity that carries the
probe is the difference d_i = L(theta + eps p_i) - L(theta - eps p_i) (pith.science review, "What
carries the argument": the update is a sum of these differences times p_i). These helpers compare
the differences themselves, per probe i, normwise over the sequences b compared:

    D_i[b] = s(theta + eps p_i)[b] - s(theta - eps p_i)[b]      (s: per-sequence CE sum)
    || D_gpu,i - D_ref,i ||_inf  <=  rtol * || D_ref,i ||_inf  +  floor * || s_ref,i ||_inf

and the same for the differences summed over the compared sequences (with the floor times the
summed |s|). rtol = 2e-2 is the relative bar bf16 results are held to. The floor stands for the
rounding noise a correct kernel leaves: activations are rounded to bf16 (2^-8 relative spacing)
where they enter a product, and where the GPU's and the oracle's fp32 sums (different order)
straddle a rounding boundary, single activations differ by one bf16 step. That noise does not
shrink with eps, so it is kept as an absolute term; at 1e-5 of the sequence loss it is about ten
times the per-sequence agreement such differences leave. The planted-mistake tests
(test_parity_bars.py) show, on the oracle alone, that the bar rejects a swapped sign, another
probe's or step's seeds and, where the probe dominates the loss, a tensor left unperturbed.

No oracle code and no GPU code lives here.
"""
from __future__ import annotations

import numpy as np

RTOL = 2e-2
FLOOR = 1e-5

# Cases where the probe dominates the loss difference (large eps; theta = 0 makes every weight
# +-bf16(eps) p). Shapes: two layers, ragged batches over several 256-column blocks, several
# 32-unit row tiles, probe chunks of unequal size. Values: (n_layers, vocab, embed, hidden,
# batch, seq_len, n_probes, eps, base_seed, probes_per_chunk, theta_zero).
PROBE_CASES = {
    "pd_e2m3": (2, 50, 64, 128, 160, 3, 3, 2.0 ** -3, 92, 0, False),
    "pd_e2m3_h256": (2, 50, 96, 256, 300, 4, 4, 2.0 ** -3, 94, 3, False),
    "pd_e2m5": (2, 50, 64, 128, 160, 3, 3, 2.0 ** -5, 91, 2, False),
    "pd_e2m5_theta0": (2, 50, 64, 128, 160, 3, 3, 2.0 ** -5, 91, 2, True),
    "pd_e2m7_h256_theta0": (2, 50, 96, 256, 300, 4, 4, 2.0 ** -7, 93, 0, True),
}
# Cases in which every tensor carries at least 8% of the differences, so that leaving any one
# of them unperturbed (or perturbed with one sign) breaks the bar.
PER_TENSOR = ("pd_e2m3", "pd_e2m3_h256")


def probe_case_inputs(case, seed: int = 5):
    """Seeded theta (float32 values; the caller rounds to bf16) and tokens of a probe case."""
    L, V, E, H, B, T, K, eps, base, ppc, zero = case
    d = V * E + V * H + V + sum(4 * H * (E if l == 0 else H) + 4 * H * H + 4 * H for l in range(L))
    rng = np.random.default_rng(seed)
    bound = 1.0 / np.sqrt(H)
    theta = rng.uniform(-bound, bound, d).astype(np.float32)
    if zero:
        theta[:] = 0.0
    tokens = rng.integers(0, V, size=(B, T + 1)).astype(np.int32)
    return theta, tokens


def probe_diffs(seq_rows) -> np.ndarray:
    """Rows [2i] (+eps) and [2i+1] (-eps) of per-sequence losses -> differences [i][b] (float64)."""
    a = np.asarray(seq_rows, np.float64)
    return a[0::2] - a[1::2]


def diff_errors(got_seq, ref_seq, rtol: float = RTOL, floor: float = FLOOR) -> tuple[float, float]:
    """Worst ratio of error to bar, (per-sequence differences, summed differences); <= 1 passes."""
    ref = np.asarray(ref_seq, np.float64)
    dg, dr = probe_diffs(got_seq), probe_diffs(ref)
    mag = np.maximum(np.abs(ref[0::2]), np.abs(ref[1::2]))          # |s| per probe and sequence
    bar = rtol * np.max(np.abs(dr), axis=1) + floor * np.max(mag, axis=1)
    per_seq = np.max(np.abs(dg - dr), axis=1) / bar
    sg, sr = dg.sum(axis=1), dr.sum(axis=1)
    bar_sum = rtol * np.max(np.abs(sr)) + floor * np.max(mag.sum(axis=1))
    summed = np.max(np.abs(sg - sr)) / bar_sum
    return float(per_seq.max()), float(summed)


def assert_diffs_close(got_seq, ref_seq, what: str = "probe differences", rtol: float = RTOL,
                       floor: float = FLOOR):
    e_seq, e_sum = diff_errors(got_seq, ref_seq, rtol, floor)
    assert e_seq <= 1.0, f"{what}: per-sequence differences at {e_seq:.2f} x the bar"
    assert e_sum <= 1.0, f"{what}: summed differences at {e_sum:.2f} x the bar"
    return e_seq, e_sum

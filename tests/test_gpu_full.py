"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

The oracle evaluates sampled (probe, sequence) pairs at full model shape one by one and they are
compared with the GPU's per-sequence losses; the per-probe reduction (loss = sum of per-sequence
losses / (B T)) is checked on the GPU's own outputs; the update is checked element by element on a
sample of parameters from every tensor, feeding the GPU's losses to the oracle's update.
"""
import numpy as np
import pytest

from gpu_util import HipRun, TOL, as_f64, assert_losses_close, ocfg, say
from parity_bars import assert_diffs_close
from zero_order_recurrent_amd import binding as b
from zero_order_recurrent_amd.inputs import PRESETS, make_theta, make_tokens

pytestmark = pytest.mark.gpu


def _sample_elements(oracle, c, per_tensor=20000, seed=0):
    rng = np.random.default_rng(seed)
    out = []
    for tid, off, rows, cols in oracle.layout(ocfg(c)):
        n = rows * cols
        k = min(n, per_tensor)
        out.append(off + np.sort(rng.choice(n, size=k, replace=False)))
        out.append(np.array([off, off + n - 1]))
    return np.unique(np.concatenate(out)).astype(np.int64)


def _check(oracle, name, probes, seqs):
    p = PRESETS[name]
    c = b.config_from_preset(p)
    tol = TOL[p.dtype]
    say(f"[gpu] full-size {name}: probes {probes} sequences {seqs}")
    d = b.cdrge_param_count(c)
    theta, tokens = make_theta(p, d), make_tokens(p)
    run = HipRun(c, theta, tokens)
    losses, seq, st = run.probe_losses(0)
    assert st == 0
    assert np.isfinite(losses).all()
    np.testing.assert_allclose(losses, seq.astype(np.float64).sum(1) / (c.batch * c.seq_len), rtol=2e-6)
    ref_l, ref_seq = oracle.probe_losses(ocfg(c), theta, tokens, 0, probe_ids=probes, seq_ids=seqs)
    rows = [2 * i + s for i in probes for s in (0, 1)]
    err = assert_losses_close(seq[np.ix_(rows, seqs)], ref_seq, tol, "seq_losses")
    say(f"    seq-loss max rel err {err:.2e}")
    if p.dtype != "f32":
        e = assert_diffs_close(seq[np.ix_(rows, seqs)], ref_seq)
        say(f"    probe differences at {max(e):.3f} x the bar")
    if len(seqs) == c.batch:
        assert_losses_close(losses[rows], ref_l, tol)
    # update: same losses on both sides, sampled elements of every tensor
    assert run.update(0) == 0
    got = run.theta()
    elems = _sample_elements(oracle, c)
    ref = theta.copy()
    assert oracle.update(ocfg(c), ref, 0, losses, elems=elems) == 0
    a, r, t0 = as_f64(got[elems]), as_f64(ref[elems]), as_f64(theta[elems])
    if p.dtype == "f32":
        np.testing.assert_allclose(a, r, rtol=1e-6, atol=1e-7 * np.abs(r).max())
    else:
        mismatch = np.mean(got[elems] != ref[elems])
        assert mismatch < 1e-3, mismatch
        assert np.abs(a - r).max() <= tol * np.abs(r).max()
    say(f"    update checked on {len(elems)} elements; changed {np.mean(a != t0):.3f} of them")
    run.close()


def test_full_overfit(oracle):
    _check(oracle, "overfit", probes=[0, 1, 255, 511], seqs=[0])


def test_full_tiny(oracle):
    _check(oracle, "tiny", probes=list(range(8)), seqs=[0, 1, 2, 3])


def test_full_charlm(oracle):
    _check(oracle, "charlm", probes=[0, 63], seqs=[0, 1, 2, 255, 256, 511, 1000, 1023])


@pytest.mark.timeout(400)
def test_full_lstm270m(oracle):
    _check(oracle, "lstm270m", probes=[0, 31], seqs=[0, 1023])


@pytest.mark.timeout(600)
def test_full_lstm1b(oracle):
    # probe 0 runs in the first chunk of 8 pairs, probe 15 in the second
    _check(oracle, "lstm1b", probes=[0, 15], seqs=[0, 255])


@pytest.mark.parametrize("name,probes", [("charlm", (0, 31, 63)), ("lstm270m", (0, 17, 31)),
                                         ("lstm1b", (0, 7, 8, 15))])
@pytest.mark.timeout(300)
def test_full_layout_signs(oracle, name, probes):
    # Signs at the workload's own layout, observed through the ABI: theta = 0 and losses with
    # d = e_i leave theta' = -coef * p_i exactly (coef = eta / (2 K eps) = 1 / (2K), a power of two,
    # exact in bf16). Compared with the oracle's uncached sign on up to 2^20 sampled elements of
    # every tensor (all elements of the smaller ones, always the first and last).
    import torch
    p = PRESETS[name]
    c = b.config_from_preset(p)
    say(f"[gpu] full-layout signs {name}: probes {probes}")
    d = b.cdrge_param_count(c)
    K = c.n_probes
    rng = np.random.default_rng(17)
    elems = []
    for tid, off, rows, cols in oracle.layout(ocfg(c)):
        n = rows * cols
        k = min(n, 1 << 20)
        pick = np.arange(n) if k == n else rng.choice(n, size=k, replace=False)
        elems.append(off + pick)
        elems.append(np.array([off, off + n - 1]))
    elems = np.unique(np.concatenate(elems)).astype(np.int64)
    idx = torch.from_numpy(elems).cuda()
    params = torch.zeros(d, dtype=torch.int16, device="cuda")
    ctx = b.Context(c, params)
    coef = np.float32(1.0 / (2 * K))
    for i in probes:
        params.zero_()
        losses = torch.zeros(2 * K, dtype=torch.float32, device="cuda")
        losses[2 * i] = 1.0
        ctx.update(0, losses)
        assert ctx.sync_status() == 0
        got = params[idx].cpu().numpy().view(np.uint16)
        vals = (got.astype(np.uint32) << 16).view(np.float32)
        sgn = oracle.signs_at(ocfg(c), oracle.probe_seed(c.base_seed, 0, i), elems)
        np.testing.assert_array_equal(vals, -coef * sgn.astype(np.float32))
    say(f"    {len(elems)} sampled elements per probe bit-exact")
    ctx.close()


def test_full_charlm_exact_perturbation(oracle):
    # the char-LM workload in the exact-perturbation bf16 dtype (same theta and tokens as charlm)
    _check(oracle, "charlm_x", probes=[0, 63], seqs=[0, 1, 511, 1023])

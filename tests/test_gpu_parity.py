"""GPU parity against the CPU oracle, through the C ABI, at sizes the oracle finishes in seconds.

Shapes span several tiles and ragged tails: bf16 batches that are not a multiple of the 128-column
tile, several 64-unit row tiles, two layers, probe chunks of unequal size; fp32 batches split over
two workgroups, two probe pairs per workgroup with an odd pair count, more gate rows than threads,
inputs that are not a multiple of 32 columns. Bars: probe seeds and signs bit-exact; losses and per-sequence losses within
1e-5 (fp32) or 2e-2 (bf16) relative; updated parameters within the same bars normwise per tensor.
For bf16, whose 2e-2 bar is far wider than what a probe moves a loss, the differences
L(theta + eps p_i) - L(theta - eps p_i) per sequence and per probe are held to the probe-difference
bar of parity_bars.py, and cases with a large eps (or theta = 0) make the probe dominate the loss.
"""
import numpy as np
import pytest

from gpu_util import HipRun, TOL, as_f64, assert_losses_close, assert_theta_close, dtype_name, ocfg, say
from parity_bars import PROBE_CASES, assert_diffs_close, probe_case_inputs
from zero_order_recurrent_amd import binding as b
from zero_order_recurrent_amd.inputs import PRESETS, make_theta, make_tokens, to_bf16_bits

pytestmark = pytest.mark.gpu

SMALL = {
    "f32_ragged": b.make_config(2, 13, 20, 24, 11, 5, 3, "f32", 1e-3, 1e-3, 77, probes_per_chunk=2),
    "f32_long": b.make_config(1, 32, 16, 40, 2, 40, 4, "f32", 1e-3, 1e-3, 78),
    # 515 pairs: two pairs per workgroup, the last workgroup with one; 3 sequences over two
    # workgroups of two slots
    "f32_pairs2": b.make_config(1, 7, 12, 8, 3, 4, 515, "f32", 1e-3, 1e-3, 82),
    # 4H = 1,280 rows over 1,024 threads: rows wrap; V = 70 logit rows over 14 column slices
    "f32_wide": b.make_config(1, 70, 40, 320, 1, 3, 2, "f32", 1e-3, 1e-3, 83),
    "bf16_ragged": b.make_config(2, 50, 64, 128, 160, 3, 3, "bf16", 1e-4, 1e-4, 79, probes_per_chunk=2),
    "bf16_e32_v5": b.make_config(1, 5, 32, 64, 40, 4, 2, "bf16", 1e-2, 1e-2, 80),
    "bf16_v64": b.make_config(3, 64, 96, 192, 130, 2, 2, "bf16", 1e-3, 1e-3, 81),
    # H = 416 (13 chunks of 32): the logits' reduction over H is split in two slices (8 + 5 chunks)
    "bf16_ce_split": b.make_config(1, 50, 32, 416, 40, 3, 2, "bf16", 1e-4, 1e-4, 84),
    # smallest shapes: one sequence, one step, one probe pair, a single 32-wide K chunk per layer
    "bf16_min": b.make_config(1, 2, 32, 32, 1, 1, 1, "bf16", 1e-2, 1e-2, 85),
    "f32_min": b.make_config(1, 2, 1, 1, 1, 1, 1, "f32", 1e-2, 1e-2, 86),
    # a long sequence: 64 steps through the same fixed-size state
    "bf16_long": b.make_config(2, 50, 64, 128, 24, 64, 2, "bf16", 1e-4, 1e-4, 87),
    # fp32 on the row-sliced kernels (E and H multiples of 32, V <= 64, B >= 8, >= 256 columns per
    # chunk): 320 columns (five whole 64-column blocks), two layers of four row slices
    "f32sl_b8": b.make_config(2, 11, 32, 64, 8, 4, 20, "f32", 1e-3, 1e-3, 88),
    # nine sequences per model (pairs straddle the 64-column blocks), chunks of 15 and 10 pairs
    # (270 and 180 columns, ragged blocks), two row slices
    "f32sl_b9_chunks": b.make_config(1, 40, 64, 32, 9, 3, 25, "f32", 1e-3, 1e-3, 89, probes_per_chunk=15),
    # three layers, six row slices, the largest vocabulary of the sliced path
    "f32sl_v64": b.make_config(3, 64, 32, 96, 10, 2, 15, "f32", 1e-3, 1e-3, 90),
    # char-LM widths in fp32 (E = 128, H = 1,024): per-model state beyond the persistent kernel's
    # LDS, so only the row-sliced kernels run it (64 row slices, four 64-column blocks)
    "f32sl_h1024": b.make_config(1, 50, 128, 1024, 16, 3, 8, "f32", 1e-3, 1e-3, 91),
    # one timestep: only the first (no W_hh, zero state) launch and one cross-entropy
    "f32sl_t1": b.make_config(2, 20, 64, 64, 8, 1, 16, "f32", 1e-3, 1e-3, 92),
    # B a multiple of 16: the direct variant (perturbed weights as the matrix-core operand), two
    # layers, chunks of 10 and 5 pairs (320 and 160 columns)
    "f32sl_direct_chunks": b.make_config(2, 11, 32, 64, 16, 4, 15, "f32", 1e-3, 1e-3, 93, probes_per_chunk=10),
    # the direct variant with 32 sequences per model (two models per 64-column block), V = 64
    "f32sl_direct_b32": b.make_config(1, 64, 64, 96, 32, 3, 5, "f32", 1e-3, 1e-3, 94),
    # B a multiple of 64 (every column block in one model: one perturbed A value per K step for
    # the block's four tiles), two layers, 128 sequences per model (two blocks each)
    "f32sl_direct_b128": b.make_config(2, 20, 32, 64, 128, 3, 3, "f32", 1e-3, 1e-3, 95),
    # the largest sizes the library accepts: K = 1,024 probe pairs (every pair its own perturbed
    # models) with the most fp32 layers (8) on the persistent kernel, 8 layers on the row-sliced
    # kernels, and K = 1,024 in bf16 (one sequence per model, 1,024 column blocks)
    "f32_max_k_layers": b.make_config(8, 7, 12, 8, 2, 2, 1024, "f32", 1e-3, 1e-3, 100),
    "f32sl_l8": b.make_config(8, 10, 32, 32, 8, 2, 16, "f32", 1e-3, 1e-3, 101),
    "bf16_max_k": b.make_config(1, 5, 32, 32, 1, 2, 1024, "bf16", 1e-2, 1e-2, 102),
}


def _inputs(c, seed):
    rng = np.random.default_rng(seed)
    d = b.cdrge_param_count(c)
    bound = 1.0 / np.sqrt(c.hidden)
    theta = rng.uniform(-bound, bound, d).astype(np.float32)
    if c.dtype != b.CDRGE_F32:
        theta = to_bf16_bits(theta)
    tokens = rng.integers(0, c.vocab, size=(c.batch, c.seq_len + 1)).astype(np.int32)
    return theta, tokens


@pytest.mark.parametrize("name", list(SMALL))
def test_small_step_parity(oracle, name):
    c = SMALL[name]
    say(f"[gpu] small parity {name}")
    theta, tokens = _inputs(c, 5)
    tol = TOL[dtype_name(c)]
    run = HipRun(c, theta, tokens)
    # the cases cover both fp32 kernels: the f32sl_ ones the row-sliced path, the others the
    # persistent one
    expect = ("k_lstm_f32_sliced" if name.startswith("f32sl") else "k_lstm_f32") if c.dtype == b.CDRGE_F32 \
        else "k_lstm_gates_bf16"
    assert b.cdrge_timed_kernel(run.ctx.ctx, 0) == expect
    losses, seq, st = run.probe_losses(step=2)
    assert st == 0
    oc = ocfg(c)
    ref_l, ref_seq = oracle.probe_losses(oc, theta, tokens, 2)
    assert_losses_close(losses, ref_l, tol)
    assert_losses_close(seq, ref_seq, tol, "seq_losses")
    if c.dtype != b.CDRGE_F32:
        e = assert_diffs_close(seq, ref_seq)
        assert_diffs_close(losses[:, None], ref_l[:, None], "per-probe d_i")
        say(f"    probe differences at {max(e):.3f} x the bar")
    # the per-probe reduction: loss = sum_b seq / (B T)
    np.testing.assert_allclose(losses, seq.astype(np.float64).sum(1) / (c.batch * c.seq_len), rtol=1e-6)
    assert run.update(2) == 0
    ref_theta = theta.copy()
    assert oracle.update(oc, ref_theta, 2, ref_l) == 0
    assert_theta_close(oracle, c, run.theta(), ref_theta, tol)
    run.close()


def test_tiny_three_steps(oracle):
    p = PRESETS["tiny"]
    c = b.config_from_preset(p)
    say("[gpu] tiny preset, 3 steps")
    d = b.cdrge_param_count(c)
    theta, tokens = make_theta(p, d), make_tokens(p)
    run = HipRun(c, theta, tokens)
    ref = theta.copy()
    oc = ocfg(c)
    for s in range(p.steps):
        losses, _, st = run.probe_losses(s)
        assert st == 0
        ref_l, _ = oracle.probe_losses(oc, ref, tokens, s)
        assert_losses_close(losses, ref_l, 1e-5)
        assert run.update(s) == 0
        assert oracle.update(oc, ref, s, ref_l) == 0
        assert_theta_close(oracle, c, run.theta(), ref, 1e-5)
    run.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_signs_bit_exact_through_update(oracle, dtype):
    # theta = 0 and losses with d = e_i: theta' = -coef * p_i exactly (coef = 1/(2K) = 2^-k).
    c = b.make_config(2, 50, 64, 128, 3, 2, 4, dtype, 1e-3, 1e-3, 4242)
    say(f"[gpu] sign observation {dtype}")
    d = b.cdrge_param_count(c)
    zero = np.zeros(d, np.float32 if dtype == "f32" else np.uint16)
    tokens = np.zeros((3, 3), np.int32)
    for step in (0, 5):
        for i in range(c.n_probes):
            run = HipRun(c, zero, tokens)
            losses = np.zeros(2 * c.n_probes, np.float32)
            losses[2 * i] = 1.0
            assert run.update(step, losses) == 0
            got = run.theta()
            vals = got if dtype == "f32" else (got.astype(np.uint32) << 16).view(np.float32)
            p = oracle.probe_vector(ocfg(c), oracle.probe_seed(c.base_seed, step, i))
            np.testing.assert_array_equal(vals, (-p / (2 * c.n_probes)).astype(np.float32))
            run.close()


# bf16 with K <= 64 runs the permute-addressed update: K = 8, 13, 24, 40, 57 and 64 give 1, 2, 3,
# 5, 8 and 8 probe groups (13 and 57 with unused probe slots) in 32, 32, 32, 16, 16 and 16 table
# copies (one or two 64 KB regions). Otherwise K = 24, 300 and 600 keep 4, 2 and 1 copies of the
# probe-group tables in LDS.
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_probes", [8, 13, 24, 40, 57, 64, 300, 600, 1024])
def test_update_parity_identical_losses(oracle, dtype, n_probes):
    c = b.make_config(2, 50, 64, 192, 3, 2, n_probes, dtype, 1e-3, 1e-3, 99)
    say(f"[gpu] update parity {dtype} K={n_probes}")
    theta, tokens = _inputs(c, 9)
    rng = np.random.default_rng(4)
    losses = (3.0 + 1e-3 * rng.standard_normal(2 * c.n_probes)).astype(np.float32)
    run = HipRun(c, theta, tokens)
    assert run.update(3, losses) == 0
    ref = theta.copy()
    assert oracle.update(ocfg(c), ref, 3, losses) == 0
    got = run.theta()
    if dtype == "f32":
        # identical inputs: only the order of the probe sum differs (K rounding steps at most)
        assert_theta_close(oracle, c, got, ref, 1e-6)
    else:
        assert_theta_close(oracle, c, got, ref, 2e-2)
        assert np.mean(got != ref) < 1e-3
    run.close()


# K = 512 (coef = 2^-10): one table copy per group. K = 64 (coef = 2^-7): for bf16, eight probe
# groups of the permute-addressed update in two 64 KB table regions. Sampled probes from the first,
# a middle and the last group.
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n_probes,probes", [(512, (0, 7, 8, 263, 511)), (64, (0, 9, 34, 56, 63))])
def test_signs_bit_exact_through_update_many_probes(oracle, dtype, n_probes, probes):
    c = b.make_config(1, 50, 64, 128, 3, 2, n_probes, dtype, 1e-3, 1e-3, 4343)
    say(f"[gpu] sign observation, K={n_probes}, {dtype}")
    d = b.cdrge_param_count(c)
    zero = np.zeros(d, np.float32 if dtype == "f32" else np.uint16)
    tokens = np.zeros((3, 3), np.int32)
    for i in probes:
        run = HipRun(c, zero, tokens)
        losses = np.zeros(2 * c.n_probes, np.float32)
        losses[2 * i] = 1.0
        assert run.update(1, losses) == 0
        got = run.theta()
        vals = got if dtype == "f32" else (got.astype(np.uint32) << 16).view(np.float32)
        p = oracle.probe_vector(ocfg(c), oracle.probe_seed(c.base_seed, 1, i))
        np.testing.assert_array_equal(vals, (-p / (2 * c.n_probes)).astype(np.float32))
        run.close()


def test_update_parity_many_tensors(oracle):
    # 10 bf16 layers: 33 tensors, more than one launch's tensor table holds, so the update runs
    # per tensor with per-probe sign-adds.
    c = b.make_config(10, 20, 32, 32, 2, 2, 12, "bf16", 1e-3, 1e-3, 98)
    say("[gpu] update parity, 33 tensors, bf16")
    theta, tokens = _inputs(c, 12)
    rng = np.random.default_rng(6)
    losses = (3.0 + 1e-3 * rng.standard_normal(2 * c.n_probes)).astype(np.float32)
    run = HipRun(c, theta, tokens)
    assert run.update(2, losses) == 0
    ref = theta.copy()
    assert oracle.update(ocfg(c), ref, 2, losses) == 0
    got = run.theta()
    assert_theta_close(oracle, c, got, ref, 2e-2)
    assert np.mean(got != ref) < 1e-3
    run.close()


# eta = 0 (allowed: the configuration only requires eta >= 0): the coefficient eta / (2 K eps) is
# zero, so every update kernel must leave theta bit-identical whatever the loss differences (theta
# holds no exact zeros, whose sign the subtraction of a zero may change).
@pytest.mark.parametrize("dtype,layers,n_probes,kernel", [("bf16", 2, 8, "k_update_perm"),
                                                          ("f32", 2, 8, "k_update_lut"),
                                                          ("bf16", 2, 96, "k_update_lut"),
                                                          ("bf16", 10, 12, "k_update")])
def test_zero_learning_rate_leaves_theta(oracle, dtype, layers, n_probes, kernel):
    if layers == 10:
        c = b.make_config(10, 20, 32, 32, 2, 2, n_probes, dtype, 1e-3, 0.0, 97)
    else:
        c = b.make_config(layers, 50, 64, 192, 3, 2, n_probes, dtype, 1e-3, 0.0, 96)
    say(f"[gpu] zero learning rate, {kernel}, {dtype}, K={n_probes}")
    theta, tokens = _inputs(c, 13)
    assert (as_f64(theta) != 0).all()
    rng = np.random.default_rng(7)
    losses = (3.0 + 1e-2 * rng.standard_normal(2 * c.n_probes)).astype(np.float32)
    run = HipRun(c, theta, tokens)
    assert b.cdrge_timed_kernel(run.ctx.ctx, 2) == kernel
    assert run.update(5, losses) == 0
    np.testing.assert_array_equal(run.theta(), theta)
    ref = theta.copy()
    assert oracle.update(ocfg(c), ref, 5, losses) == 0
    np.testing.assert_array_equal(ref, theta)
    run.close()


def test_update_many_segments(oracle):
    # bf16, K = 16, d = 16.1M: each update workgroup strides over the 128-column segments several
    # times (both parameter buffers in turn, and a partial last pass); W_ih has 1,056 columns, so
    # every row ends in a 32-column segment. Checked on sampled elements of every tensor.
    c = b.make_config(1, 50, 1056, 1536, 2, 2, 16, "bf16", 1e-4, 1e-4, 4444)
    say("[gpu] update over many segments, K=16, bf16")
    theta, tokens = _inputs(c, 11)
    rng = np.random.default_rng(5)
    losses = (3.0 + 1e-3 * rng.standard_normal(2 * c.n_probes)).astype(np.float32)
    run = HipRun(c, theta, tokens)
    assert run.update(7, losses) == 0
    got = run.theta()
    elems = []
    for tid, off, rows, cols in oracle.layout(ocfg(c)):
        n = rows * cols
        elems.append(off + rng.choice(n, size=min(n, 30000), replace=False))
        elems.append(np.array([off, off + cols - 1, off + n - cols, off + n - 1]))
    elems = np.unique(np.concatenate(elems)).astype(np.int64)
    ref = theta.copy()
    assert oracle.update(ocfg(c), ref, 7, losses, elems=elems) == 0
    a, r = as_f64(got[elems]), as_f64(ref[elems])
    assert np.mean(got[elems] != ref[elems]) < 1e-3
    assert np.abs(a - r).max() <= 2e-2 * np.abs(r).max()
    assert np.mean(a != as_f64(theta[elems])) > 0.01
    run.close()


def test_nonfinite_loss_leaves_theta(oracle):
    c = SMALL["bf16_ragged"]
    say("[gpu] non-finite losses")
    theta, tokens = _inputs(c, 6)
    bad = theta.copy()
    bad[100] = 0x7FC0  # NaN in the embedding
    run = HipRun(c, bad, tokens)
    losses, _, st = run.probe_losses(0)
    assert st == 0
    assert np.isnan(losses).any()
    assert run.update(0) == 5  # CDRGE_ERR_NONFINITE
    np.testing.assert_array_equal(run.theta(), bad)
    assert run.ctx.sync_status() == 0  # the flag was cleared
    run.close()


# a token at or above V, or below zero (in the language-model form every target is scored), on
# each forward kernel: the step's losses are NaN and the update leaves theta alone
@pytest.mark.parametrize("name", ["f32_ragged", "bf16_ragged", "f32sl_direct_chunks", "f32sl_b9_chunks"])
@pytest.mark.parametrize("bad", ["vocab", "negative"])
def test_invalid_tokens_give_nan_losses(name, bad):
    c = SMALL[name]
    say(f"[gpu] invalid tokens {name} {bad}")
    theta, tokens = _inputs(c, 7)
    tokens[3, 2] = c.vocab if bad == "vocab" else -1
    run = HipRun(c, theta, tokens)
    losses, _, st = run.probe_losses(0)
    assert np.isnan(losses).all()
    assert run.update(0) == 5
    np.testing.assert_array_equal(run.theta(), theta)
    run.close()


# (case, chunk sizes): every chunk size keeps the case on one forward kernel, whose per-column
# arithmetic does not depend on which other models share a launch; the row-sliced cases need
# 2 P B >= 256 columns per chunk (the table variant, the direct one, and the direct one with one
# model per column block)
@pytest.mark.parametrize("name,ppcs", [("bf16_ragged", (0, 1, 2, 0)), ("f32_ragged", (0, 1, 2, 0)),
                                       ("f32sl_b9_chunks", (0, 15, 20, 0)),
                                       ("f32sl_direct_chunks", (0, 8, 10, 0)),
                                       ("f32sl_direct_b128", (0, 1, 2, 0))])
def test_deterministic_and_chunk_invariant(name, ppcs):
    c = SMALL[name]
    say(f"[gpu] determinism {name}")
    theta, tokens = _inputs(c, 8)
    outs = []
    kernels = set()
    for ppc in ppcs:
        cc = b.make_config(c.n_layers, c.vocab, c.embed, c.hidden, c.batch, c.seq_len, c.n_probes,
                           dtype_name(c), c.eps, c.lr, c.base_seed, probes_per_chunk=ppc)
        run = HipRun(cc, theta, tokens)
        kernels.add(b.cdrge_timed_kernel(run.ctx.ctx, 0))
        losses, seq, st = run.probe_losses(1)
        assert st == 0
        outs.append((losses, seq))
        run.close()
    assert len(kernels) == 1, kernels
    for l, s in outs[1:]:
        np.testing.assert_array_equal(l, outs[0][0])
        np.testing.assert_array_equal(s, outs[0][1])


def test_resume_equals_uninterrupted():
    c = SMALL["bf16_ragged"]
    say("[gpu] resume")
    theta, tokens = _inputs(c, 10)
    run = HipRun(c, theta, tokens)
    for s in range(3):
        run.probe_losses(s)
        run.update(s)
    straight = run.theta()
    run.close()
    run = HipRun(c, theta, tokens)
    for s in range(2):
        run.probe_losses(s)
        run.update(s)
    saved = run.theta()
    run.close()
    run = HipRun(c, saved, tokens)
    run.probe_losses(2)
    run.update(2)
    np.testing.assert_array_equal(run.theta(), straight)
    run.close()


@pytest.mark.parametrize("hidden,pairs", [(256, 32), (512, 16), (256, 12), (768, 8), (1024, 6), (640, 10), (544, 8)])
def test_xcd_grouped_tile_order(oracle, hidden, pairs):
    # B = 256 (one column block per model). H = 256: 8 row tiles and 32 pairs, grouped 8 x 4 per
    # XCD; H = 512: 16 row tiles and 16 pairs, grouped 16 x 2; H = 256 with 12 pairs: 96
    # workgroups, three 8 x 4 groups over the 8 XCDs (12 workgroups each), so groups straddle XCDs;
    # H = 768: 24 row tiles, so each pair of column blocks has one 16 x 2 group and a short 8 x 2
    # one; H = 1024 with 6 pairs: 16 x 2 groups, 24 workgroups per XCD; H = 640 and 544: 20 and 17
    # row tiles, short groups of 4 x 2 and 1 x 2.
    c = b.make_config(1, 50, 64, hidden, 256, 2, pairs, "bf16", 1e-3, 1e-3, 82)
    say(f"[gpu] xcd-grouped tile order, H={hidden}")
    theta, tokens = _inputs(c, 12)
    run = HipRun(c, theta, tokens)
    losses, seq, st = run.probe_losses(0)
    assert st == 0
    probes, seqs = [0, min(13, pairs - 2), pairs - 1], [0, 1, 100, 255]
    ref_l, ref_seq = oracle.probe_losses(ocfg(c), theta, tokens, 0, probe_ids=probes, seq_ids=seqs)
    rows = [2 * i + s for i in probes for s in (0, 1)]
    assert_losses_close(seq[np.ix_(rows, seqs)], ref_seq, 2e-2, "seq_losses")
    assert_diffs_close(seq[np.ix_(rows, seqs)], ref_seq)
    np.testing.assert_allclose(losses, seq.astype(np.float64).sum(1) / (c.batch * c.seq_len), rtol=1e-6)
    run.close()


@pytest.mark.parametrize("layers,embed,hidden", [(2, 128, 128), (1, 128, 256), (2, 256, 256), (1, 1024, 1024),
                                                 (1, 1056, 1056), (1, 128, 1088)])
def test_k_loop_end_instances(oracle, layers, embed, hidden):
    # The gate kernel's phased instance (no requests past the last K chunk, the cell state loaded
    # early) serves reductions of 8-64 chunks that are a multiple of 4, the plain one all others.
    # K chunks per launch at the first timestep / later ones: 128 x 128, both layers: 4 / 8;
    # 128 x 256: 4 / 12; 256 x 256, both layers: 8 / 16; 1024 x 1024: 32 / 64; 1056 x 1056: 33 /
    # 66; 128 x 1088: 4 / 38. So the phased instance runs with 0, 1 and several full groups before
    # its last two, beside the plain one, which also serves 66 chunks and counts that are not a
    # multiple of 4.
    c = b.make_config(layers, 50, embed, hidden, 40, 3, 2, "bf16", 1e-3, 1e-3, 83)
    say(f"[gpu] K-loop end instances, L={layers} E={embed} H={hidden}")
    theta, tokens = _inputs(c, 14)
    run = HipRun(c, theta, tokens)
    losses, seq, st = run.probe_losses(0)
    assert st == 0
    probes, seqs = [0, 1], [0, 17, 39]
    ref_l, ref_seq = oracle.probe_losses(ocfg(c), theta, tokens, 0, probe_ids=probes, seq_ids=seqs)
    rows = [2 * i + s for i in probes for s in (0, 1)]
    assert_losses_close(seq[np.ix_(rows, seqs)], ref_seq, 2e-2, "seq_losses")
    assert_diffs_close(seq[np.ix_(rows, seqs)], ref_seq)
    run.close()


@pytest.mark.parametrize("name", list(PROBE_CASES))
def test_probe_dominant_bf16(oracle, name):
    # eps = 2^-3 .. 2^-7 against weights of 1/sqrt(H) (or theta = 0): the probe moves the losses by
    # 0.5-10%, and the differences d_i must match the oracle's within the probe-difference bar
    L, V, E, H, B, T, K, eps, base, ppc, zero = PROBE_CASES[name]
    c = b.make_config(L, V, E, H, B, T, K, "bf16", eps, eps, base, probes_per_chunk=ppc)
    say(f"[gpu] probe-dominant bf16 {name}")
    theta32, tokens = probe_case_inputs(PROBE_CASES[name])
    theta = to_bf16_bits(theta32)
    run = HipRun(c, theta, tokens)
    # the cases cover both fp32 kernels: the f32sl_ ones the row-sliced path, the others the
    # persistent one
    expect = ("k_lstm_f32_sliced" if name.startswith("f32sl") else "k_lstm_f32") if c.dtype == b.CDRGE_F32 \
        else "k_lstm_gates_bf16"
    assert b.cdrge_timed_kernel(run.ctx.ctx, 0) == expect
    losses, seq, st = run.probe_losses(step=2)
    assert st == 0
    oc = ocfg(c)
    ref_l, ref_seq = oracle.probe_losses(oc, theta, tokens, 2)
    assert_losses_close(losses, ref_l, 2e-2)
    assert_losses_close(seq, ref_seq, 2e-2, "seq_losses")
    e = assert_diffs_close(seq, ref_seq)
    assert_diffs_close(losses[:, None], ref_l[:, None], "per-probe d_i")
    say(f"    probe differences at {max(e):.3f} x the bar")
    assert run.update(2) == 0
    ref_theta = theta.copy()
    assert oracle.update(oc, ref_theta, 2, ref_l) == 0
    assert_theta_close(oracle, c, run.theta(), ref_theta, 2e-2)
    run.close()


def test_long_sequence_charlm_widths(oracle):
    # The char-LM widths (E = 128, H = 1024, two layers) over T = 200 steps: the forward streams
    # through the same fixed-size state (h ping-pong per layer, c per tile) however long the
    # sequence, and the losses and their probe differences still match the oracle.
    c = b.make_config(2, 50, 128, 1024, 5, 200, 2, "bf16", 1e-4, 1e-4, 3103)
    say("[gpu] long sequence, char-LM widths, T=200")
    theta, tokens = _inputs(c, 14)
    run = HipRun(c, theta, tokens)
    losses, seq, st = run.probe_losses(0)
    assert st == 0
    seqs = [0, 2, 4]
    ref_l, ref_seq = oracle.probe_losses(ocfg(c), theta, tokens, 0, seq_ids=seqs)
    got = seq[:, seqs]
    err = assert_losses_close(got, ref_seq, 2e-2, "seq_losses")
    e = assert_diffs_close(got, ref_seq)
    say(f"    seq-loss max rel err {err:.2e}; probe differences at {max(e):.3f} x the bar")
    np.testing.assert_allclose(losses, seq.astype(np.float64).sum(1) / (c.batch * c.seq_len), rtol=1e-6)
    run.close()


# The exact-perturbation bf16 dtype: bf16 parameters, (W +- eps' P) x = W x +- eps' P x with the
# probe never rounded into the weight. Shapes as the bf16 cases: ragged batch, several row tiles,
# chunks of unequal size, the split logits reduction, a probe-dominant eps and eps = 1e-4 where
# the plain bf16 model quantises the probe.
EXACT = {
    "x_ragged": b.make_config(2, 50, 64, 128, 160, 3, 3, "bf16x", 1e-4, 1e-4, 701, probes_per_chunk=2),
    "x_h256": b.make_config(2, 50, 96, 256, 300, 4, 4, "bf16x", 2.0 ** -7, 2.0 ** -7, 702),
    "x_ce_split": b.make_config(1, 50, 32, 416, 40, 3, 2, "bf16x", 1e-3, 1e-3, 703),
    "x_min": b.make_config(1, 2, 32, 32, 1, 1, 1, "bf16x", 1e-2, 1e-2, 704),
    "x_e2m3": b.make_config(2, 50, 64, 128, 160, 3, 3, "bf16x", 2.0 ** -3, 2.0 ** -3, 705),
}


@pytest.mark.parametrize("name", list(EXACT))
def test_exact_perturbation_bf16(oracle, name):
    c = EXACT[name]
    say(f"[gpu] exact-perturbation bf16 {name}")
    theta, tokens = _inputs(c, 15)
    run = HipRun(c, theta, tokens)
    losses, seq, st = run.probe_losses(step=1)
    assert st == 0
    oc = ocfg(c)
    ref_l, ref_seq = oracle.probe_losses(oc, theta, tokens, 1)
    assert_losses_close(losses, ref_l, 2e-2)
    assert_losses_close(seq, ref_seq, 2e-2, "seq_losses")
    e = assert_diffs_close(seq, ref_seq)
    assert_diffs_close(losses[:, None], ref_l[:, None], "per-probe d_i")
    say(f"    probe differences at {max(e):.3f} x the bar")
    assert run.update(1) == 0
    ref_theta = theta.copy()
    assert oracle.update(oc, ref_theta, 1, ref_l) == 0
    assert_theta_close(oracle, c, run.theta(), ref_theta, 2e-2)
    run.close()

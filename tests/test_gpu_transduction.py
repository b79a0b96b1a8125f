"""Transduction workloads (copy, reverse, rolling sum; alex-wiki note, "Evidence And Limits",
synthetic-transduction bullet) through the C ABI's separate-targets entry points, against the
oracle's transduction form: inputs and targets given separately, targets below zero not scored,
the loss the mean over the scored positions.

Bars as for the language-model workloads: fp32 losses and per-sequence losses within 1e-5
relative, the update within 1e-6 normwise per tensor on identical losses; bf16 losses within 2e-2
and their probe differences within the probe-difference bar.
"""
import numpy as np
import pytest

from gpu_util import HipRun, assert_losses_close, assert_theta_close, ocfg, say
from parity_bars import assert_diffs_close
from zero_order_recurrent_amd import binding as b
from zero_order_recurrent_amd.inputs import PRESETS, make_io, make_theta, make_transduction, to_bf16_bits

pytestmark = pytest.mark.gpu


class IoRun(HipRun):
    def __init__(self, cfg, theta, inputs, targets, tokens=None):
        import torch
        if tokens is None:  # the language-model entry points are not used then
            tokens = np.zeros((cfg.batch, cfg.seq_len + 1), np.int32)
        super().__init__(cfg, theta, tokens)
        self.inputs = torch.from_numpy(np.ascontiguousarray(inputs, np.int32)).cuda()
        self.targets = torch.from_numpy(np.ascontiguousarray(targets, np.int32)).cuda()

    def probe_losses_io(self, step: int):
        b.cdrge_probe_losses_io(self.ctx.ctx, self.inputs, self.targets, step, self.ctx.losses, self.seq)
        st = self.ctx.sync_status()
        return self.ctx.losses.cpu().numpy().copy(), self.seq.cpu().numpy().copy(), st


@pytest.mark.parametrize("task", ["copy", "reverse", "rollsum"])
def test_transduction_preset_parity(oracle, task):
    p = PRESETS[task]
    c = b.config_from_preset(p)
    say(f"[gpu] transduction preset {task}")
    d = b.cdrge_param_count(c)
    theta = make_theta(p, d)
    inputs, targets = make_io(p)
    run = IoRun(c, theta, inputs, targets)
    losses, seq, st = run.probe_losses_io(0)
    assert st == 0
    ref_l, ref_seq = oracle.probe_losses_io(ocfg(c), theta, inputs, targets, 0)
    assert_losses_close(losses, ref_l, 1e-5)
    assert_losses_close(seq, ref_seq, 1e-5, "seq_losses")
    scored = int((targets >= 0).sum())
    np.testing.assert_allclose(losses, seq.astype(np.float64).sum(1) / scored, rtol=1e-6)
    assert run.update(0) == 0
    ref = theta.copy()
    assert oracle.update(ocfg(c), ref, 0, losses) == 0
    assert_theta_close(oracle, c, run.theta(), ref, 1e-6)
    run.close()


def test_transduction_evaluation_lengths(oracle):
    # the copy model on source lengths 11-60 (T = 120): the lengths the pages evaluate on
    p = PRESETS["copy"]
    c = b.make_config(p.n_layers, p.vocab, p.embed, p.hidden, 16, 120, 4, "f32", p.eps, p.lr, p.base_seed)
    say("[gpu] transduction, evaluation lengths 11-60")
    theta = make_theta(p, b.cdrge_param_count(c))
    inputs, targets = make_transduction("copy", p.vocab - 2, 16, 11, 60, 77)
    run = IoRun(c, theta, inputs, targets)
    losses, seq, st = run.probe_losses_io(3)
    assert st == 0
    ref_l, ref_seq = oracle.probe_losses_io(ocfg(c), theta, inputs, targets, 3)
    assert_losses_close(losses, ref_l, 1e-5)
    assert_losses_close(seq, ref_seq, 1e-5, "seq_losses")
    run.close()


@pytest.mark.parametrize("task", ["reverse", "rollsum"])
def test_transduction_bf16(oracle, task):
    # the bf16 kernels (gather, gate GEMM, logits and the split logits reduction) with unscored
    # targets; eps = 2^-5 so that the probe differences are far above rounding noise
    c = b.make_config(2, 10, 32, 64, 40, 20, 3, "bf16", 2.0 ** -5, 2.0 ** -5, 610, probes_per_chunk=2)
    say(f"[gpu] transduction bf16 {task}")
    rng = np.random.default_rng(31)
    d = b.cdrge_param_count(c)
    theta = to_bf16_bits(rng.uniform(-0.125, 0.125, d).astype(np.float32))
    inputs, targets = make_transduction(task, 8, 40, 1, 10, 78)
    run = IoRun(c, theta, inputs, targets)
    losses, seq, st = run.probe_losses_io(1)
    assert st == 0
    ref_l, ref_seq = oracle.probe_losses_io(ocfg(c), theta, inputs, targets, 1)
    assert_losses_close(losses, ref_l, 2e-2)
    assert_losses_close(seq, ref_seq, 2e-2, "seq_losses")
    assert_diffs_close(seq, ref_seq)
    assert_diffs_close(losses[:, None], ref_l[:, None], "per-probe d_i")
    run.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_language_model_is_the_shifted_io_form(dtype):
    # cdrge_probe_losses(tokens) and cdrge_probe_losses_io(tokens[:, :T], tokens[:, 1:]) run the
    # same kernels on the same values: bit-identical losses
    shape = (2, 50, 64, 128, 37) if dtype == "bf16" else (2, 20, 16, 40, 11)
    c = b.make_config(*shape, 4, 3, dtype, 1e-3, 1e-3, 611)
    say(f"[gpu] language model through the io entry point, {dtype}")
    rng = np.random.default_rng(32)
    d = b.cdrge_param_count(c)
    theta = rng.uniform(-0.08, 0.08, d).astype(np.float32)
    if dtype == "bf16":
        theta = to_bf16_bits(theta)
    tokens = rng.integers(0, c.vocab, size=(c.batch, 5)).astype(np.int32)
    run = IoRun(c, theta, tokens[:, :-1], tokens[:, 1:], tokens=tokens)
    a_l, a_s, st = run.probe_losses(2)
    assert st == 0
    b_l, b_s, st = run.probe_losses_io(2)
    assert st == 0
    np.testing.assert_array_equal(a_l, b_l)
    np.testing.assert_array_equal(a_s, b_s)
    run.close()


# B = 6 runs on the persistent fp32 kernel; B = 16 with 8 pairs (256 columns) on the row-sliced
# one, whose logits and cross-entropy skip unscored targets
@pytest.mark.parametrize("batch,pairs,kernel", [(6, 2, "k_lstm_f32"), (16, 8, "k_lstm_f32_sliced")])
def test_io_invalid_and_unscored(batch, pairs, kernel):
    c = b.make_config(1, 10, 32, 64, batch, 8, pairs, "f32", 1e-3, 1e-3, 612)
    say(f"[gpu] io form: invalid inputs, invalid targets, nothing scored ({kernel})")
    rng = np.random.default_rng(33)
    theta = rng.uniform(-0.1, 0.1, b.cdrge_param_count(c)).astype(np.float32)
    inputs, targets = make_transduction("copy", 8, batch, 1, 4, 79)
    for what, inp, tg in [("input out of range", np.where(np.arange(8) == 3, 10, inputs), targets),
                          ("target out of range", inputs, np.where(targets >= 0, 10, targets)),
                          ("nothing scored", inputs, np.full_like(targets, -1))]:
        run = IoRun(c, theta, inp.astype(np.int32), tg.astype(np.int32))
        assert b.cdrge_timed_kernel(run.ctx.ctx, 0) == kernel
        losses, _, st = run.probe_losses_io(0)
        assert st == 0
        assert np.isnan(losses).all(), what
        assert run.update(0) == 5, what
        np.testing.assert_array_equal(run.theta(), theta)
        run.close()

"""cdrge_step_noalloc (the step for callers that cannot allocate device memory) against cdrge_step
(the context entry point with a caller workspace), through the C ABI, on two calls in a row, the
second with a smaller input: the library's static scratch keeps the first call's contents, and the
second call must not depend on them. Same kernels, same inputs: losses and updated parameters are
required to be bit-identical (stricter than the 1e-5 / 2e-2 parity bars)."""
import numpy as np
import pytest

from gpu_util import HipRun, say, to_device_params, from_device_params
from zero_order_recurrent_amd import binding as b
from zero_order_recurrent_amd.inputs import to_bf16_bits

pytestmark = pytest.mark.gpu

PAIRS = {
    # bf16: two layers, ragged batch, probe chunks of 2 + 1; then one layer, fewer columns
    "bf16": (b.make_config(2, 50, 64, 128, 160, 3, 3, "bf16", 1e-3, 1e-3, 501, probes_per_chunk=2),
             b.make_config(1, 20, 32, 64, 40, 2, 2, "bf16", 1e-3, 1e-3, 502)),
    # fp32: the tiny workload's shape, then a smaller model
    "f32": (b.make_config(1, 16, 16, 32, 4, 10, 8, "f32", 1e-3, 1e-3, 503),
            b.make_config(1, 7, 12, 8, 3, 4, 5, "f32", 1e-3, 1e-3, 504)),
    # fp32 on the row-sliced kernels: two layers over 320 columns, then one layer over 256
    "f32_sliced": (b.make_config(2, 10, 32, 64, 8, 5, 20, "f32", 1e-3, 1e-3, 505),
                   b.make_config(1, 10, 32, 32, 16, 3, 8, "f32", 1e-3, 1e-3, 506)),
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


def _with_context(c, theta, tokens, step, kernel=None):
    run = HipRun(c, theta, tokens)
    if kernel is not None:
        assert b.cdrge_timed_kernel(run.ctx.ctx, 0) == kernel
    losses = run.ctx.step(run.tokens, step).cpu().numpy().copy()
    assert run.ctx.sync_status() == 0
    out = run.theta()
    run.close()
    return losses, out


def _noalloc(c, theta, tokens, step):
    import torch
    params = to_device_params(theta)
    tok = torch.from_numpy(np.ascontiguousarray(tokens, np.int32)).cuda()
    losses = torch.full((2 * c.n_probes,), float("nan"), dtype=torch.float32, device="cuda")
    b.cdrge_step_noalloc(c, params, tok, step, losses)
    torch.cuda.synchronize()
    return losses.cpu().numpy(), from_device_params(params)


@pytest.mark.parametrize("dtype", list(PAIRS))
def test_noalloc_step_matches_context_step(dtype):
    for k, c in enumerate(PAIRS[dtype]):
        say(f"[gpu] no-alloc step {dtype}, call {k + 1}")
        theta, tokens = _inputs(c, 40 + k)
        ref_l, ref_t = _with_context(c, theta, tokens, step=3,
                                     kernel="k_lstm_f32_sliced" if dtype == "f32_sliced" else None)
        got_l, got_t = _noalloc(c, theta, tokens, step=3)
        assert np.isfinite(ref_l).all()
        np.testing.assert_array_equal(got_l, ref_l)
        np.testing.assert_array_equal(got_t, ref_t)
        assert (got_t != theta).any()


def test_noalloc_rejects_oversized_workspace():
    import torch
    c = b.make_config(2, 50, 128, 1024, 1024, 10, 64, "bf16", 1e-4, 1e-4, 3003)
    say("[gpu] no-alloc step, oversized configuration")
    x = torch.zeros(16, dtype=torch.int16, device="cuda")
    with pytest.raises(b.CdrgeError) as err:
        b.cdrge_step_noalloc(c, x, x, 0, x)
    assert err.value.status == 3

"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI and compare it with
the oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np

from oracle import OracleConfig
from zero_order_recurrent_amd import binding as b

TOL = {"f32": 1e-5, "bf16": 2e-2, "bf16x": 2e-2}
NAMES = {b.CDRGE_F32: "f32", b.CDRGE_BF16: "bf16", b.CDRGE_BF16_EXACT: "bf16x"}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def ocfg(c: b.cdrge_config) -> OracleConfig:
    return OracleConfig(c.n_layers, c.vocab, c.embed, c.hidden, c.batch, c.seq_len, c.n_probes,
                        NAMES[c.dtype], c.eps, c.lr, c.base_seed)


def dtype_name(c: b.cdrge_config) -> str:
    return NAMES[c.dtype]


def to_device_params(theta: np.ndarray):
    import torch
    if theta.dtype == np.uint16:
        return torch.from_numpy(theta.view(np.int16).copy()).cuda()
    return torch.from_numpy(theta.copy()).cuda()


def from_device_params(t) -> np.ndarray:
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def as_f64(theta: np.ndarray) -> np.ndarray:
    if theta.dtype == np.uint16:
        return (theta.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return theta.astype(np.float64)


class HipRun:
    def __init__(self, cfg: b.cdrge_config, theta: np.ndarray, tokens: np.ndarray):
        import torch
        self.cfg = cfg
        self.params = to_device_params(theta)
        self.tokens = torch.from_numpy(np.ascontiguousarray(tokens, np.int32)).cuda()
        self.ctx = b.Context(cfg, self.params)
        self.seq = torch.zeros((2 * cfg.n_probes, cfg.batch), dtype=torch.float32, device="cuda")

    def probe_losses(self, step: int):
        self.ctx.probe_losses(self.tokens, step, self.seq)
        st = self.ctx.sync_status()
        return self.ctx.losses.cpu().numpy().copy(), self.seq.cpu().numpy().copy(), st

    def update(self, step: int, losses: np.ndarray | None = None):
        import torch
        if losses is not None:
            self.ctx.losses.copy_(torch.from_numpy(np.ascontiguousarray(losses, np.float32)))
        self.ctx.update(step)
        return self.ctx.sync_status()

    def theta(self) -> np.ndarray:
        return from_device_params(self.params)

    def close(self):
        self.ctx.close()


def assert_losses_close(got, ref, tol, what="losses"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rel = np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)
    worst = int(np.argmax(rel))
    assert rel.max() <= tol, f"{what}: max rel err {rel.max():.3e} at {worst} (gpu {got.flat[worst]}, oracle {ref.flat[worst]})"
    return float(rel.max())


def assert_theta_close(oracle, c, got: np.ndarray, ref: np.ndarray, tol: float):
    """Normwise per tensor: ||a - b||_inf / ||b||_inf <= tol."""
    worst = 0.0
    for tid, off, rows, cols in oracle.layout(ocfg(c)):
        a = as_f64(got[off:off + rows * cols])
        r = as_f64(ref[off:off + rows * cols])
        den = max(np.abs(r).max(), 1e-30)
        err = np.abs(a - r).max() / den
        worst = max(worst, err)
        assert err <= tol, f"tensor {tid}: normwise error {err:.3e}"
    return worst

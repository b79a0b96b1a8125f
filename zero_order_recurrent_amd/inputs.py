"""Workload presets and seeded synthetic inputs (no CD-RGE arithmetic lives here).

Both the HIP path's tests and the CPU oracle read their inputs from this module, so that the two
sides see the same bytes. The workloads stand in for the pages' character-level Penn Treebank
runs (alex-wiki source note, "Evidence And Limits": batch 1,024, training length 10, character
vocabulary) and the fixed-batch overfitting runs (same section: batch one, length 100, up to 512
perturbations). The dataset itself is not used: tokens are drawn from a seeded generator.

Recipe per preset with index c:
  * tokens int32 [B][T+1] from numpy.random.default_rng(1000 + c): uniform on [0, V) or Zipf(s)
    truncated to the vocabulary, P(token = k - 1) proportional to k^-s for k = 1..V;
  * parameters from default_rng(2000 + c): every element uniform on (-1/sqrt(H), 1/sqrt(H)) in
    float32; bf16 presets round that to the nearest bf16 (ties to even) through torch;
  * probe base seed 3000 + c.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Preset:
    name: str
    index: int
    n_layers: int
    embed: int
    hidden: int
    vocab: int
    dtype: str          # "f32" or "bf16"
    batch: int
    seq_len: int
    n_probes: int       # K probe pairs -> 2K forwards per step
    eps: float
    lr: float
    tokens: str         # "uniform" or "zipf"
    zipf_s: float = 1.1
    probes_per_chunk: int = 0   # 0 = all probes in one chunk
    steps: int = 1

    @property
    def base_seed(self) -> int:
        return 3000 + self.index

    def with_(self, **kw) -> "Preset":
        return replace(self, **kw)


PRESETS = {
    "tiny": Preset("tiny", 1, 1, 16, 32, 16, "f32", 4, 10, 8, 1e-3, 1e-3, "uniform", steps=3),
    "overfit": Preset("overfit", 2, 1, 64, 256, 32, "f32", 1, 100, 512, 1e-3, 1e-3, "uniform"),
    "charlm": Preset("charlm", 3, 2, 128, 1024, 50, "bf16", 1024, 10, 64, 1e-4, 1e-4, "zipf"),
    "lstm270m": Preset("lstm270m", 4, 2, 4096, 4096, 50, "bf16", 1024, 10, 32, 1e-4, 1e-4, "zipf"),
    "lstm1b": Preset("lstm1b", 5, 4, 5888, 5888, 50, "bf16", 256, 10, 16, 1e-4, 1e-4, "zipf",
                     probes_per_chunk=8),
}


def make_tokens(p: Preset) -> np.ndarray:
    rng = np.random.default_rng(1000 + p.index)
    shape = (p.batch, p.seq_len + 1)
    if p.tokens == "uniform":
        return rng.integers(0, p.vocab, size=shape, dtype=np.int64).astype(np.int32)
    k = np.arange(1, p.vocab + 1, dtype=np.float64)
    prob = k ** (-p.zipf_s)
    prob /= prob.sum()
    return rng.choice(p.vocab, size=shape, p=prob).astype(np.int32)


def make_theta_f32(p: Preset, d: int) -> np.ndarray:
    # Drawn in slices (same stream as one draw of d values) to bound the float64 temporaries.
    rng = np.random.default_rng(2000 + p.index)
    bound = 1.0 / np.sqrt(p.hidden)
    out = np.empty(d, dtype=np.float32)
    step = 1 << 25
    for s in range(0, d, step):
        n = min(step, d - s)
        out[s:s + n] = rng.uniform(-bound, bound, size=n)
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even, via torch's conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    out = np.empty(x.shape, dtype=np.uint16)
    step = 1 << 26
    flat_out = out.reshape(-1)
    flat_in = t.reshape(-1)
    for s in range(0, flat_in.numel(), step):
        flat_out[s:s + step] = flat_in[s:s + step].to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_theta(p: Preset, d: int) -> np.ndarray:
    """Initial parameters in storage form: float32, or uint16 bf16 bit patterns."""
    x = make_theta_f32(p, d)
    return to_bf16_bits(x) if p.dtype == "bf16" else x

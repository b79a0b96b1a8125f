"""ctypes binding of the plain C++ CD-RGE oracle (test infrastructure only).

The oracle follows the method of arXiv 2505.17852 as the pith.science review ("What carries
the argument") and the alex-wiki source note ("Method") describe it; every reading taken where the
pages are silent is stated in the C++ headers next to this file. This module only marshals
arguments: all arithmetic happens in ``oracle_capi.cpp``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SOURCES = ["oracle_capi.cpp", "cdrge.hpp", "lstm.hpp", "philox.hpp", "bf16.hpp"]


def oracle_library_path() -> str:
    return os.path.join(_HERE, "liboracle.so")


def build_oracle() -> str:
    """Compile the oracle with g++ (-O2, no floating-point contraction) into liboracle.so."""
    out = oracle_library_path()
    tmp = out + ".tmp"
    cmd = ["g++", "-O2", "-ffp-contract=off", "-std=c++17", "-Wall", "-shared", "-fPIC",
           os.path.join(_HERE, "oracle_capi.cpp"), "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class _Cfg(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("vocab", ctypes.c_int32), ("embed", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("n_probes", ctypes.c_int32), ("storage", ctypes.c_int32), ("eps", ctypes.c_float),
                ("lr", ctypes.c_float), ("base_seed", ctypes.c_uint64)]


STORAGE = {"f32": 0, "bf16": 1, "f64": 2, "bf16x": 3}


@dataclass
class OracleConfig:
    n_layers: int
    vocab: int
    embed: int
    hidden: int
    batch: int
    seq_len: int
    n_probes: int
    storage: str  # "f32", "bf16" (uint16 bit patterns), "f64" (exact) or "bf16x" (bf16, probe added exactly)
    eps: float
    lr: float
    base_seed: int

    def c(self) -> _Cfg:
        return _Cfg(self.n_layers, self.vocab, self.embed, self.hidden, self.batch, self.seq_len,
                    self.n_probes, STORAGE[self.storage], self.eps, self.lr, self.base_seed)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """Thin wrapper; arrays must be C-contiguous numpy arrays of the documented dtypes."""

    def __init__(self, path: str | None = None):
        path = path or oracle_library_path()
        if not os.path.exists(path):
            build_oracle()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64, u32, u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64
        sig = {
            "oracle_param_count": (i64, [P]),
            "oracle_layout": (ctypes.c_int, [P, P, ctypes.c_int]),
            "oracle_philox": (None, [P, u64, P]),
            "oracle_probe_seed": (u64, [u64, u64, u32]),
            "oracle_sign": (ctypes.c_int, [u64, u32, u32, u32]),
            "oracle_sign_block": (None, [u64, u32, u32, u32, u32, u32, P]),
            "oracle_probe_vector": (None, [P, u64, P]),
            "oracle_signs_at": (None, [P, u64, P, i64, P]),
            "oracle_lstm_seq_losses": (None, [P, P, ctypes.c_int, P, P, ctypes.c_int, ctypes.c_int, P]),
            "oracle_lstm_seq_losses_io": (None, [P, P, ctypes.c_int, P, P, P, ctypes.c_int, ctypes.c_int, P]),
            "oracle_probe_losses_io": (None, [P, P, P, P, u64, P, ctypes.c_int, P, ctypes.c_int, P, P]),
            "oracle_step_io": (ctypes.c_int, [P, P, P, P, u64, P]),
            "oracle_probe_losses": (None, [P, P, P, u64, P, ctypes.c_int, P, ctypes.c_int, P, P]),
            "oracle_update": (ctypes.c_int, [P, P, u64, P, P, i64]),
            "oracle_update_f64losses": (ctypes.c_int, [P, P, u64, P]),
            "oracle_step": (ctypes.c_int, [P, P, P, u64, P]),
            "oracle_lstm_dir_deriv": (None, [P, P, P, P, P, P]),
            "oracle_lstm_grad": (None, [P, P, P, P]),
            "oracle_quadratic_cdrge": (None, [ctypes.c_int, ctypes.c_int, P, P, P, u64, u64,
                                              ctypes.c_int, ctypes.c_float, ctypes.c_float, P, P]),
            "oracle_flat_probe": (None, [u64, ctypes.c_int, P]),
            "oracle_f32_to_bf16": (ctypes.c_uint16, [ctypes.c_float]),
            "oracle_f64_to_bf16": (ctypes.c_uint16, [ctypes.c_double]),
            "oracle_f32_to_bf16_array": (None, [P, i64, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        self.lib = lib
        del i32

    # -- layout ---------------------------------------------------------------------------
    def param_count(self, cfg: OracleConfig) -> int:
        c = cfg.c()
        return int(self.lib.oracle_param_count(ctypes.byref(c)))

    def layout(self, cfg: OracleConfig) -> list[tuple[int, int, int, int]]:
        c = cfg.c()
        buf = np.zeros((64, 4), dtype=np.int64)
        n = self.lib.oracle_layout(ctypes.byref(c), _ptr(buf), 64)
        return [tuple(int(v) for v in buf[i]) for i in range(n)]

    # -- random streams -------------------------------------------------------------------
    def philox(self, ctr, key: int) -> np.ndarray:
        c = np.asarray(ctr, dtype=np.uint32)
        out = np.zeros(4, dtype=np.uint32)
        self.lib.oracle_philox(_ptr(c), key, _ptr(out))
        return out

    def probe_seed(self, base_seed: int, step: int, i: int) -> int:
        return int(self.lib.oracle_probe_seed(base_seed, step, i))

    def probe_seeds(self, base_seed: int, step: int, k: int) -> np.ndarray:
        return np.array([self.probe_seed(base_seed, step, i) for i in range(k)], dtype=np.uint64)

    def sign(self, seed: int, tensor: int, row: int, col: int) -> int:
        return int(self.lib.oracle_sign(seed, tensor, row, col))

    def sign_block(self, seed: int, tensor: int, r0: int, nr: int, c0: int, nc: int) -> np.ndarray:
        out = np.zeros((nr, nc), dtype=np.int8)
        self.lib.oracle_sign_block(seed, tensor, r0, nr, c0, nc, _ptr(out))
        return out

    def probe_vector(self, cfg: OracleConfig, seed: int) -> np.ndarray:
        c = cfg.c()
        out = np.zeros(self.param_count(cfg), dtype=np.int8)
        self.lib.oracle_probe_vector(ctypes.byref(c), seed, _ptr(out))
        return out

    def signs_at(self, cfg: OracleConfig, seed: int, elems: np.ndarray) -> np.ndarray:
        """Signs of probe ``seed`` at flat indices ``elems``, one Philox call per element."""
        elems = np.ascontiguousarray(elems, np.int64)
        out = np.zeros(len(elems), dtype=np.int8)
        c = cfg.c()
        self.lib.oracle_signs_at(ctypes.byref(c), seed, _ptr(elems), len(elems), _ptr(out))
        return out

    def flat_probe(self, seed: int, d: int) -> np.ndarray:
        out = np.zeros(d, dtype=np.int8)
        self.lib.oracle_flat_probe(seed, d, _ptr(out))
        return out

    # -- model ----------------------------------------------------------------------------
    def seq_losses(self, cfg: OracleConfig, weights: np.ndarray, tokens: np.ndarray, seq_ids=None,
                   round_act_bf16: bool = False) -> np.ndarray:
        storage = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.float64): 2}[weights.dtype]
        seq_ids = np.arange(cfg.batch, dtype=np.int32) if seq_ids is None else np.asarray(seq_ids, np.int32)
        out = np.zeros(len(seq_ids), dtype=np.float64)
        c = cfg.c()
        self.lib.oracle_lstm_seq_losses(ctypes.byref(c), _ptr(np.ascontiguousarray(weights)), storage,
                                        _ptr(np.ascontiguousarray(tokens, np.int32)), _ptr(seq_ids),
                                        len(seq_ids), int(round_act_bf16), _ptr(out))
        return out

    def seq_losses_io(self, cfg: OracleConfig, weights: np.ndarray, inputs: np.ndarray, targets: np.ndarray,
                      seq_ids=None, round_act_bf16: bool = False) -> np.ndarray:
        storage = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.float64): 2}[weights.dtype]
        seq_ids = np.arange(cfg.batch, dtype=np.int32) if seq_ids is None else np.asarray(seq_ids, np.int32)
        out = np.zeros(len(seq_ids), dtype=np.float64)
        c = cfg.c()
        self.lib.oracle_lstm_seq_losses_io(ctypes.byref(c), _ptr(np.ascontiguousarray(weights)), storage,
                                           _ptr(np.ascontiguousarray(inputs, np.int32)),
                                           _ptr(np.ascontiguousarray(targets, np.int32)), _ptr(seq_ids),
                                           len(seq_ids), int(round_act_bf16), _ptr(out))
        return out

    def probe_losses_io(self, cfg: OracleConfig, theta: np.ndarray, inputs: np.ndarray, targets: np.ndarray,
                        step: int, probe_ids=None, seq_ids=None):
        """Transduction form of probe_losses: inputs [B][T], targets [B][T] (negative: not scored)."""
        probe_ids = np.arange(cfg.n_probes, dtype=np.int32) if probe_ids is None else np.asarray(probe_ids, np.int32)
        seq_ids = np.arange(cfg.batch, dtype=np.int32) if seq_ids is None else np.asarray(seq_ids, np.int32)
        losses = np.zeros(2 * len(probe_ids), dtype=np.float32)
        seq = np.zeros((2 * len(probe_ids), len(seq_ids)), dtype=np.float64)
        c = cfg.c()
        self.lib.oracle_probe_losses_io(ctypes.byref(c), _ptr(np.ascontiguousarray(theta)),
                                        _ptr(np.ascontiguousarray(inputs, np.int32)),
                                        _ptr(np.ascontiguousarray(targets, np.int32)), step,
                                        _ptr(probe_ids), len(probe_ids), _ptr(seq_ids), len(seq_ids),
                                        _ptr(losses), _ptr(seq))
        return losses, seq

    def step_io(self, cfg: OracleConfig, theta: np.ndarray, inputs: np.ndarray, targets: np.ndarray, step: int):
        losses = np.zeros(2 * cfg.n_probes, dtype=np.float32)
        c = cfg.c()
        rc = self.lib.oracle_step_io(ctypes.byref(c), _ptr(theta), _ptr(np.ascontiguousarray(inputs, np.int32)),
                                     _ptr(np.ascontiguousarray(targets, np.int32)), step, _ptr(losses))
        return losses, int(rc)

    def probe_losses(self, cfg: OracleConfig, theta: np.ndarray, tokens: np.ndarray, step: int,
                     probe_ids=None, seq_ids=None):
        """Returns (losses [n_ids*2] float32, seq_losses [n_ids*2, n_seq] float64)."""
        probe_ids = np.arange(cfg.n_probes, dtype=np.int32) if probe_ids is None else np.asarray(probe_ids, np.int32)
        seq_ids = np.arange(cfg.batch, dtype=np.int32) if seq_ids is None else np.asarray(seq_ids, np.int32)
        losses = np.zeros(2 * len(probe_ids), dtype=np.float32)
        seq = np.zeros((2 * len(probe_ids), len(seq_ids)), dtype=np.float64)
        c = cfg.c()
        self.lib.oracle_probe_losses(ctypes.byref(c), _ptr(np.ascontiguousarray(theta)),
                                     _ptr(np.ascontiguousarray(tokens, np.int32)), step,
                                     _ptr(probe_ids), len(probe_ids), _ptr(seq_ids), len(seq_ids),
                                     _ptr(losses), _ptr(seq))
        return losses, seq

    def update(self, cfg: OracleConfig, theta: np.ndarray, step: int, losses: np.ndarray,
               elems: np.ndarray | None = None) -> int:
        """In-place update of ``theta`` (all elements, or the flat indices ``elems``)."""
        assert theta.flags.c_contiguous
        losses = np.ascontiguousarray(losses, np.float32)
        c = cfg.c()
        if elems is None:
            return int(self.lib.oracle_update(ctypes.byref(c), _ptr(theta), step, _ptr(losses), None, 0))
        elems = np.ascontiguousarray(elems, np.int64)
        return int(self.lib.oracle_update(ctypes.byref(c), _ptr(theta), step, _ptr(losses), _ptr(elems), len(elems)))

    def update_f64losses(self, cfg: OracleConfig, theta: np.ndarray, step: int, losses: np.ndarray) -> int:
        losses = np.ascontiguousarray(losses, np.float64)
        c = cfg.c()
        return int(self.lib.oracle_update_f64losses(ctypes.byref(c), _ptr(theta), step, _ptr(losses)))

    def step(self, cfg: OracleConfig, theta: np.ndarray, tokens: np.ndarray, step: int):
        losses = np.zeros(2 * cfg.n_probes, dtype=np.float32)
        c = cfg.c()
        rc = self.lib.oracle_step(ctypes.byref(c), _ptr(theta), _ptr(np.ascontiguousarray(tokens, np.int32)),
                                  step, _ptr(losses))
        return losses, int(rc)

    def dir_deriv(self, cfg: OracleConfig, theta: np.ndarray, tokens: np.ndarray, direction: np.ndarray):
        v = ctypes.c_double()
        dv = ctypes.c_double()
        c = cfg.c()
        self.lib.oracle_lstm_dir_deriv(ctypes.byref(c), _ptr(np.ascontiguousarray(theta, np.float64)),
                                       _ptr(np.ascontiguousarray(tokens, np.int32)),
                                       _ptr(np.ascontiguousarray(direction, np.float64)),
                                       ctypes.byref(v), ctypes.byref(dv))
        return v.value, dv.value

    def grad(self, cfg: OracleConfig, theta: np.ndarray, tokens: np.ndarray) -> np.ndarray:
        g = np.zeros(self.param_count(cfg), dtype=np.float64)
        c = cfg.c()
        self.lib.oracle_lstm_grad(ctypes.byref(c), _ptr(np.ascontiguousarray(theta, np.float64)),
                                  _ptr(np.ascontiguousarray(tokens, np.int32)), _ptr(g))
        return g

    def quadratic_cdrge(self, A: np.ndarray, b: np.ndarray, theta: np.ndarray, base_seed: int, step: int,
                        n: int, eps: float, lr: float, want_update: bool = True):
        m, d = A.shape
        losses = np.zeros(2 * n, dtype=np.float64)
        out = np.zeros(d, dtype=np.float64) if want_update else None
        self.lib.oracle_quadratic_cdrge(d, m, _ptr(np.ascontiguousarray(A, np.float64)),
                                        _ptr(np.ascontiguousarray(b, np.float64)),
                                        _ptr(np.ascontiguousarray(theta, np.float64)), base_seed, step, n,
                                        eps, lr, _ptr(losses), _ptr(out) if out is not None else None)
        return losses, out

    # -- bf16 -----------------------------------------------------------------------------
    def f32_to_bf16(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x, np.float32)
        out = np.zeros(x.shape, dtype=np.uint16)
        self.lib.oracle_f32_to_bf16_array(_ptr(x), x.size, _ptr(out))
        return out

    def f64_to_bf16(self, x: float) -> int:
        return int(self.lib.oracle_f64_to_bf16(float(x)))

"""ctypes binding of libcdrge.so (include/cdrge.h), argument marshalling only.

Every function mirrors the C entry point of the same name. Device buffers are torch tensors on
the GPU (only their data pointers cross the boundary); the stream is torch's current stream
unless one is given. There is no fallback: if libcdrge.so is missing or does not load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcdrge.so")

CDRGE_ABI_VERSION = 1
CDRGE_F32, CDRGE_BF16, CDRGE_BF16_EXACT = 0, 1, 2
STATUS = {0: "CDRGE_OK", 1: "CDRGE_ERR_INVALID_ARG", 2: "CDRGE_ERR_UNSUPPORTED", 3: "CDRGE_ERR_WORKSPACE",
          4: "CDRGE_ERR_DEVICE", 5: "CDRGE_ERR_NONFINITE"}
KIND_GATES, KIND_CE, KIND_UPDATE, KIND_PREP = 0, 1, 2, 3


class CdrgeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}")
        self.status = status


class cdrge_config(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("n_layers", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("embed", ctypes.c_int32), ("hidden", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("n_probes", ctypes.c_int32), ("probes_per_chunk", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("eps", ctypes.c_float), ("lr", ctypes.c_float),
                ("base_seed", ctypes.c_uint64)]


def make_config(n_layers, vocab, embed, hidden, batch, seq_len, n_probes, dtype, eps, lr, base_seed,
                probes_per_chunk=0) -> cdrge_config:
    dt = {"f32": CDRGE_F32, "bf16": CDRGE_BF16, "bf16x": CDRGE_BF16_EXACT}.get(dtype, dtype)
    return cdrge_config(CDRGE_ABI_VERSION, n_layers, vocab, embed, hidden, batch, seq_len, n_probes,
                        probes_per_chunk, dt, eps, lr, base_seed)


def config_from_preset(p) -> cdrge_config:
    return make_config(p.n_layers, p.vocab, p.embed, p.hidden, p.batch, p.seq_len, p.n_probes, p.dtype,
                       p.eps, p.lr, p.base_seed, p.probes_per_chunk)


_lib = None

EXPORTS = {
    "cdrge_param_count": (ctypes.c_int64, [ctypes.c_void_p]),
    "cdrge_check_config": (ctypes.c_int, [ctypes.c_void_p]),
    "cdrge_workspace_bytes": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]),
    "cdrge_probe_seeds": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]),
    "cdrge_init": (ctypes.c_int, [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "cdrge_probe_losses": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                          ctypes.c_void_p]),
    "cdrge_update": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]),
    "cdrge_step": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]),
    "cdrge_sync_status": (ctypes.c_int, [ctypes.c_void_p]),
    "cdrge_destroy": (None, [ctypes.c_void_p]),
    "cdrge_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "cdrge_last_error_detail": (ctypes.c_char_p, []),
    "cdrge_set_timing": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int]),
    "cdrge_get_timing": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_int64), ctypes.c_int]),
    "cdrge_get_work": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]),
    "cdrge_timed_kernel": (ctypes.c_char_p, [ctypes.c_void_p, ctypes.c_int]),
    "cdrge_probe_losses_io": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                             ctypes.c_void_p, ctypes.c_void_p]),
    "cdrge_step_io": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                     ctypes.c_void_p]),
    "cdrge_step_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                          ctypes.c_void_p, ctypes.c_void_p]),
    "cdrge_noalloc_max_workspace_bytes": (ctypes.c_size_t, []),
}


def lib():
    """Loads libcdrge.so (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        # The caller's device buffers and streams come from torch's HIP runtime; importing torch
        # first makes the loader bind libcdrge.so to that same runtime (same soname) instead of
        # starting a second one.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int, where: str):
    if status != 0:
        detail = lib().cdrge_last_error_detail().decode() if status in (3, 4) else ""
        raise CdrgeError(status, f"{where} {detail}".strip())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# ---- entry points, same names as the C ABI ------------------------------------------------------

def cdrge_param_count(cfg: cdrge_config) -> int:
    return int(lib().cdrge_param_count(ctypes.byref(cfg)))


def cdrge_check_config(cfg: cdrge_config) -> int:
    return int(lib().cdrge_check_config(ctypes.byref(cfg)))


def cdrge_workspace_bytes(cfg: cdrge_config) -> int:
    out = ctypes.c_size_t()
    _check(lib().cdrge_workspace_bytes(ctypes.byref(cfg), ctypes.byref(out)), "cdrge_workspace_bytes")
    return int(out.value)


def cdrge_probe_seeds(cfg: cdrge_config, step: int):
    import numpy as np
    out = np.zeros(cfg.n_probes, dtype=np.uint64)
    _check(lib().cdrge_probe_seeds(ctypes.byref(cfg), step, out.ctypes.data_as(ctypes.c_void_p)),
           "cdrge_probe_seeds")
    return out


def cdrge_init(cfg: cdrge_config, params, workspace, stream=None) -> ctypes.c_void_p:
    ctx = ctypes.c_void_p()
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().cdrge_init(ctypes.byref(ctx), ctypes.byref(cfg), _ptr(params), _ptr(workspace), nbytes,
                            _stream_handle(stream)), "cdrge_init")
    return ctx


def cdrge_probe_losses(ctx, tokens, step: int, losses, seq_losses=None):
    _check(lib().cdrge_probe_losses(ctx, _ptr(tokens), step, _ptr(losses), _ptr(seq_losses)), "cdrge_probe_losses")


def cdrge_update(ctx, step: int, losses):
    _check(lib().cdrge_update(ctx, step, _ptr(losses)), "cdrge_update")


def cdrge_step(ctx, tokens, step: int, losses):
    _check(lib().cdrge_step(ctx, _ptr(tokens), step, _ptr(losses)), "cdrge_step")


def cdrge_probe_losses_io(ctx, inputs, targets, step: int, losses, seq_losses=None):
    _check(lib().cdrge_probe_losses_io(ctx, _ptr(inputs), _ptr(targets), step, _ptr(losses), _ptr(seq_losses)),
           "cdrge_probe_losses_io")


def cdrge_step_io(ctx, inputs, targets, step: int, losses):
    _check(lib().cdrge_step_io(ctx, _ptr(inputs), _ptr(targets), step, _ptr(losses)), "cdrge_step_io")


def cdrge_sync_status(ctx) -> int:
    return int(lib().cdrge_sync_status(ctx))


def cdrge_destroy(ctx):
    lib().cdrge_destroy(ctx)


def cdrge_status_string(status: int) -> str:
    return lib().cdrge_status_string(status).decode()


def cdrge_last_error_detail() -> str:
    return lib().cdrge_last_error_detail().decode()


def cdrge_set_timing(ctx, enable: bool):
    _check(lib().cdrge_set_timing(ctx, int(enable)), "cdrge_set_timing")


def cdrge_get_timing(ctx, kind: int, reset: bool = False):
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().cdrge_get_timing(ctx, kind, ctypes.byref(ms), ctypes.byref(n), int(reset)), "cdrge_get_timing")
    return ms.value, n.value


def cdrge_get_work(ctx, kind: int) -> float:
    w = ctypes.c_double()
    _check(lib().cdrge_get_work(ctx, kind, ctypes.byref(w)), "cdrge_get_work")
    return w.value


def cdrge_timed_kernel(ctx, kind: int) -> str:
    return lib().cdrge_timed_kernel(ctx, kind).decode()


def cdrge_step_noalloc(cfg: cdrge_config, params, tokens, step: int, losses, stream=None):
    _check(lib().cdrge_step_noalloc(ctypes.byref(cfg), _ptr(params), _ptr(tokens), step, _ptr(losses),
                                    _stream_handle(stream)), "cdrge_step_noalloc")


def cdrge_noalloc_max_workspace_bytes() -> int:
    return int(lib().cdrge_noalloc_max_workspace_bytes())


class Context:
    """Owns a context plus its torch-allocated parameter and workspace buffers on the GPU."""

    def __init__(self, cfg: cdrge_config, params, device="cuda", stream=None):
        import torch
        self.cfg = cfg
        self.d = cdrge_param_count(cfg)
        if params.numel() != self.d:
            raise ValueError(f"params has {params.numel()} elements, the configuration needs {self.d}")
        want = torch.float32 if cfg.dtype == CDRGE_F32 else torch.int16
        if params.dtype != want or not params.is_cuda or not params.is_contiguous():
            raise ValueError("params must be a contiguous CUDA tensor of float32 (fp32) or int16 bf16 bits")
        self.params = params
        nbytes = cdrge_workspace_bytes(cfg)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=params.device)
        self.stream = stream
        self.ctx = cdrge_init(cfg, params, self.workspace, stream)
        self.losses = torch.empty(2 * cfg.n_probes, dtype=torch.float32, device=params.device)

    def probe_losses(self, tokens, step: int, seq_losses=None):
        cdrge_probe_losses(self.ctx, tokens, step, self.losses, seq_losses)
        return self.losses

    def update(self, step: int, losses=None):
        cdrge_update(self.ctx, step, self.losses if losses is None else losses)

    def step(self, tokens, step: int):
        cdrge_step(self.ctx, tokens, step, self.losses)
        return self.losses

    def probe_losses_io(self, inputs, targets, step: int, seq_losses=None):
        cdrge_probe_losses_io(self.ctx, inputs, targets, step, self.losses, seq_losses)
        return self.losses

    def step_io(self, inputs, targets, step: int):
        cdrge_step_io(self.ctx, inputs, targets, step, self.losses)
        return self.losses

    def sync_status(self) -> int:
        return cdrge_sync_status(self.ctx)

    def close(self):
        if self.ctx:
            cdrge_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

"""C-ABI checks that need no GPU: the library loads, exports every declared entry point, and its
host-side logic (parameter count, configuration checks, workspace plan, probe seeds) agrees with
the oracle where both define the same quantity."""
import os
import re

import numpy as np
import pytest

from oracle import OracleConfig
from zero_order_recurrent_amd import binding as b
from zero_order_recurrent_amd.inputs import PRESETS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(b.LIB_PATH):
        from zero_order_recurrent_amd.build import build
        build()
    return b.lib()


def test_exports_every_declared_symbol(lib):
    header = open(os.path.join(ROOT, "include", "cdrge.h")).read()
    declared = set(re.findall(r"\b(cdrge_[a-z_]+)\s*\(", header))
    assert len(declared) >= 12
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(b.EXPORTS), declared ^ set(b.EXPORTS)


def _ocfg(c):
    return OracleConfig(c.n_layers, c.vocab, c.embed, c.hidden, c.batch, c.seq_len, c.n_probes,
                        {0: "f32", 1: "bf16", 2: "bf16x"}[c.dtype], c.eps, c.lr, c.base_seed)


def test_param_count_matches_oracle(lib, oracle):
    shapes = [p for p in PRESETS.values()]
    for p in shapes:
        c = b.config_from_preset(p)
        assert b.cdrge_param_count(c) == oracle.param_count(_ocfg(c))
    c = b.make_config(3, 13, 20, 24, 11, 5, 3, "f32", 1e-3, 1e-3, 1)
    assert b.cdrge_param_count(c) == oracle.param_count(_ocfg(c))


def test_probe_seeds_match_oracle(lib, oracle):
    for p in PRESETS.values():
        c = b.config_from_preset(p)
        for step in (0, 1, 7, 2**33 + 5):
            got = b.cdrge_probe_seeds(c, step)
            ref = oracle.probe_seeds(c.base_seed, step, c.n_probes)
            np.testing.assert_array_equal(got, ref)


def test_config_validation(lib):
    ok = b.make_config(2, 50, 64, 128, 160, 3, 3, "bf16", 1e-4, 1e-4, 9)
    assert b.cdrge_check_config(ok) == 0
    bad = [dict(n_layers=0), dict(vocab=1), dict(batch=0), dict(n_probes=0), dict(eps=0.0),
           dict(eps=float("nan")), dict(lr=-1.0), dict(dtype=7), dict(abi_version=2),
           dict(probes_per_chunk=-1)]
    for kw in bad:
        c = b.make_config(2, 50, 64, 128, 160, 3, 3, "bf16", 1e-4, 1e-4, 9)
        for k, v in kw.items():
            setattr(c, k, v)
        assert b.cdrge_check_config(c) == 1, kw
        assert b.cdrge_param_count(c) == -1, kw
    unsupported = [dict(embed=48), dict(hidden=80), dict(vocab=65), dict(n_probes=2048)]
    for kw in unsupported:
        c = b.make_config(2, 50, 64, 128, 160, 3, 3, "bf16", 1e-4, 1e-4, 9)
        for k, v in kw.items():
            setattr(c, k, v)
        assert b.cdrge_check_config(c) == 2, kw
    # fp32 state that does not fit the persistent kernel's LDS: supported on the row-sliced
    # kernels when E and H are multiples of 32, unsupported otherwise
    big_f32 = b.make_config(1, 50, 128, 1024, 1024, 10, 4, "f32", 1e-3, 1e-3, 1)
    assert b.cdrge_check_config(big_f32) == 0
    big_f32_odd = b.make_config(1, 50, 100, 1024, 1024, 10, 4, "f32", 1e-3, 1e-3, 1)
    assert b.cdrge_check_config(big_f32_odd) == 2


def test_workspace_plan(lib):
    for p in PRESETS.values():
        c = b.config_from_preset(p)
        n = b.cdrge_workspace_bytes(c)
        assert n > 0 and n % 256 == 0
    c1 = b.config_from_preset(PRESETS["charlm"].with_(probes_per_chunk=4))
    c2 = b.config_from_preset(PRESETS["charlm"])
    assert b.cdrge_workspace_bytes(c1) < b.cdrge_workspace_bytes(c2)


def test_workspace_flat_in_sequence_length(lib):
    # The forward streams over t with a fixed recurrent state, so device memory does not grow
    # with the context length (the pages' point that CD-RGE memory is flat in sequence length,
    # unlike backpropagation through time).
    for name in ("charlm", "lstm270m", "tiny", "overfit"):
        p = PRESETS[name]
        sizes = {b.cdrge_workspace_bytes(b.config_from_preset(p.with_(seq_len=T))) for T in (1, 10, 100, 10000)}
        assert len(sizes) == 1, (name, sizes)


def test_status_strings(lib):
    for k, v in b.STATUS.items():
        assert b.cdrge_status_string(k) == v


def test_noalloc_entry_point_rejects_before_any_device_work(lib):
    # 64 MiB of static scratch per device; configurations that need more are refused with
    # CDRGE_ERR_WORKSPACE (and a message) before the library touches a device, as are null pointers.
    assert b.cdrge_noalloc_max_workspace_bytes() == 64 << 20
    big = b.config_from_preset(PRESETS["charlm"])
    assert b.cdrge_workspace_bytes(big) > 64 << 20
    fake = b.ctypes.c_void_p(1 << 20)  # never dereferenced: the call returns first
    st = lib.cdrge_step_noalloc(b.ctypes.byref(big), fake, fake, 0, fake, None)
    assert st == 3
    assert "static scratch holds 67108864" in b.cdrge_last_error_detail()
    small = b.config_from_preset(PRESETS["tiny"])
    assert b.cdrge_workspace_bytes(small) <= 64 << 20
    assert lib.cdrge_step_noalloc(b.ctypes.byref(small), None, fake, 0, fake, None) == 1
    # the char-LM model at 768 sequences, one probe pair per chunk, fits
    fits = b.make_config(2, 50, 128, 1024, 768, 10, 64, "bf16", 1e-4, 1e-4, 3003, probes_per_chunk=1)
    assert b.cdrge_workspace_bytes(fits) <= 64 << 20

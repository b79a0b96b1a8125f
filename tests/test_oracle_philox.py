"""Pins for the oracle's random streams.

Philox4x32-10 is checked against rocRAND's own host-callable implementation (a library routine
written independently of the oracle), driven to the same key and counter. The probe-seed and sign
streams are then checked against rocRAND outputs through the mapping the oracle documents
(philox.hpp): seed = x0 | x1 << 32 of Philox(base, (i, lo(s), hi(s), 1)); sign of (t, r, c) is bit
((j >> 1) | ((j & 1) << 4)), j = c & 31, of word (c >> 5) & 3 of Philox(seed, (c >> 7, r, t, 0)),
set -> -1. The pages only ask for Rademacher probes from reconstructible seeds (pith.science
review, "What carries the argument"; alex-wiki "Method"), so this mapping is the project's own.
"""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND helper")
    tmp = tempfile.mkdtemp()
    exe = os.path.join(tmp, "rocrand_philox")
    subprocess.run([hipcc, "-O1", "-o", exe, os.path.join(HERE, "pins", "rocrand_philox.cpp")],
                   check=True, capture_output=True)

    def query(rows):
        text = "".join(f"{k} {a} {b} {c} {d}\n" for k, a, b, c, d in rows)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return np.array([[int(v) for v in line.split()] for line in out.strip().splitlines()],
                        dtype=np.uint64).astype(np.uint32)

    yield query
    shutil.rmtree(tmp, ignore_errors=True)


def test_philox_matches_rocrand(oracle, rocrand):
    rng = np.random.default_rng(7)
    rows = []
    for _ in range(3000):
        key = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        rows.append((key, int(rng.integers(0, 2**32)), int(rng.integers(0, 2**30)),
                     int(rng.integers(0, 2**32)), int(rng.integers(0, 2**32))))
    rows += [(0, 0, 0, 0, 0), (2**64 - 1, 0, 0, 0, 0), (1, 1, 0, 0, 0), (0, 0, 0, 0, 1)]
    ref = rocrand(rows)
    got = np.array([oracle.philox(r[1:], r[0]) for r in rows], dtype=np.uint32)
    np.testing.assert_array_equal(got, ref)


def test_probe_seed_stream(oracle, rocrand):
    rows, expect_args = [], []
    for base in (3001, 3003, 2**40 + 17):
        for step in (0, 1, 2, 12345):
            for i in (0, 1, 7, 63, 511):
                rows.append((base, i, step & 0xFFFFFFFF, step >> 32, 1))
                expect_args.append((base, step, i))
    ref = rocrand(rows)
    for (base, step, i), w in zip(expect_args, ref):
        assert oracle.probe_seed(base, step, i) == int(w[0]) | (int(w[1]) << 32)


def test_sign_mapping(oracle, rocrand):
    rng = np.random.default_rng(11)
    cases = []
    for _ in range(400):
        seed = int(rng.integers(0, 2**63))
        cases.append((seed, int(rng.integers(0, 14)), int(rng.integers(0, 30000)), int(rng.integers(0, 12000))))
    ref = rocrand([(s, c >> 7, r, t, 0) for s, t, r, c in cases])
    for (seed, t, r, c), words in zip(cases, ref):
        j = c & 31
        bit = (int(words[(c >> 5) & 3]) >> ((j >> 1) | ((j & 1) << 4))) & 1
        assert oracle.sign(seed, t, r, c) == (-1 if bit else 1)


def test_sign_block_consistent(oracle):
    seed = oracle.probe_seed(3003, 0, 5)
    blk = oracle.sign_block(seed, 2, 3, 4, 120, 20)
    for r in range(4):
        for c in range(20):
            assert blk[r, c] == oracle.sign(seed, 2, 3 + r, 120 + c)
    assert set(np.unique(blk)) <= {-1, 1}

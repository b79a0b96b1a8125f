"""Pin (d): the probe signs are balanced Rademacher entries with E[p p^T] = I.

The review of arXiv 2505.17852 (pith.science, "assumptions": probes zero-mean and isotropic,
E[p]=0 and E[pp^T]=I) and its Rademacher choice ("What carries the argument") fix what the sign
stream must satisfy. Checked statistically over about 1e7 signs with 5-sigma bounds, including the
coordinate pairs a faulty bit mapping would correlate (neighbouring columns, the two half-words
of one Philox word, neighbouring rows, the four words of one call).
"""
import numpy as np

from oracle import OracleConfig


def _probes(oracle, k=32):
    cfg = OracleConfig(1, 32, 64, 256, 1, 100, k, "f32", 1e-3, 1e-3, 3002)
    P = np.stack([oracle.probe_vector(cfg, oracle.probe_seed(cfg.base_seed, 0, i)) for i in range(k)])
    return cfg, P.astype(np.int8)


def test_signs_balanced_and_isotropic(oracle):
    cfg, P = _probes(oracle)
    k, d = P.shape
    n = P.size
    assert n > 1e7
    assert set(np.unique(P)) == {-1, 1}
    assert abs(P.astype(np.float64).mean()) < 5 / np.sqrt(n)
    G = (P.astype(np.float64) @ P.T.astype(np.float64)) / d
    np.testing.assert_array_equal(np.diag(G), 1.0)
    off = G[~np.eye(k, dtype=bool)]
    assert np.abs(off).max() < 5 / np.sqrt(d)


def test_each_bit_position_balanced(oracle):
    cfg, P = _probes(oracle)
    lay = {t[0]: t for t in oracle.layout(cfg)}
    _, off, rows, cols = lay[2]                      # W_hh [1024][256]
    W = P[:, off:off + rows * cols].reshape(P.shape[0], rows, cols // 128, 128).astype(np.float64)
    per_pos = W.mean(axis=(0, 1, 2))
    m = W.shape[0] * W.shape[1] * W.shape[2]
    assert np.abs(per_pos).max() < 5 / np.sqrt(m)


def test_no_correlation_between_related_coordinates(oracle):
    cfg, P = _probes(oracle)
    lay = {t[0]: t for t in oracle.layout(cfg)}
    _, off, rows, cols = lay[2]
    W = P[:, off:off + rows * cols].reshape(P.shape[0], rows, cols).astype(np.float64)
    pairs = {
        "next column": (W[:, :, :-1], W[:, :, 1:]),
        "column + 16": (W[:, :, :-16], W[:, :, 16:]),
        "column + 32": (W[:, :, :-32], W[:, :, 32:]),
        "column + 128": (W[:, :, :-128], W[:, :, 128:]),
        "next row": (W[:, :-1, :], W[:, 1:, :]),
    }
    for name, (a, b) in pairs.items():
        prod = a * b
        assert abs(prod.mean()) < 5 / np.sqrt(prod.size), name
    # the same (row, column) under different tensors
    _, off1, r1, c1 = lay[1]                          # W_ih [1024][64]
    A = P[:, off1:off1 + r1 * c1].reshape(P.shape[0], r1, c1).astype(np.float64)
    prod = A * W[:, :, :64]
    assert abs(prod.mean()) < 5 / np.sqrt(prod.size)


def test_mapping_uses_every_bit_once(oracle):
    # Within one 128-column block every column reads a distinct (word, bit) of the Philox call.
    seen = set()
    for c in range(128):
        j = c & 31
        seen.add(((c >> 5) & 3, (j >> 1) | ((j & 1) << 4)))
    assert len(seen) == 128
    # and the oracle's signs follow the call: flipping to another block changes the stream
    seed = oracle.probe_seed(1, 0, 0)
    a = oracle.sign_block(seed, 5, 0, 64, 0, 128).astype(np.float64)
    b = oracle.sign_block(seed, 5, 0, 64, 128, 128).astype(np.float64)
    assert abs((a * b).mean()) < 5 / np.sqrt(a.size)


# A layout whose rows cross 128-column Philox blocks (W_ih of layer 0 has 200 columns) and whose
# tensors are of every kind (embedding, matrices, biases, output layer).
_LAYOUT_CFG = OracleConfig(2, 7, 200, 40, 1, 1, 5, "f32", 1e-3, 1e-3, 3117)


def test_probe_vector_matches_uncached_sign(oracle):
    """probe_vector walks rows through a reader that keeps the last Philox block; every element
    must equal the uncached probe_sign (pinned to rocRAND above), evaluated element by element."""
    cfg = _LAYOUT_CFG
    d = oracle.param_count(cfg)
    every = np.arange(d, dtype=np.int64)
    for step, i in [(0, 0), (0, 4), (9, 2)]:
        seed = oracle.probe_seed(cfg.base_seed, step, i)
        np.testing.assert_array_equal(oracle.probe_vector(cfg, seed), oracle.signs_at(cfg, seed, every))
    # and per tensor through the rectangular block reader, which is also uncached
    seed = oracle.probe_seed(cfg.base_seed, 3, 1)
    vec = oracle.probe_vector(cfg, seed)
    for tid, off, rows, cols in oracle.layout(cfg):
        blk = oracle.sign_block(seed, tid, 0, rows, 0, cols)
        np.testing.assert_array_equal(vec[off:off + rows * cols], blk.reshape(-1))


def test_update_reads_uncached_signs(oracle):
    """The update keeps one cached reader per probe; with theta = 0 and d = e_i the updated theta
    is -coef * p_i exactly (coef = 1/(2K) at eta = eps), for all elements in order and for a
    shuffled subset of elements (the reader and the layout walk then jump between tensors)."""
    cfg = _LAYOUT_CFG
    d = oracle.param_count(cfg)
    coef = 1.0 / (2 * cfg.n_probes)
    rng = np.random.default_rng(3)
    subset = rng.permutation(d)[: d // 3].astype(np.int64)
    for i in (0, 3):
        losses = np.zeros(2 * cfg.n_probes, np.float32)
        losses[2 * i] = 1.0
        seed = oracle.probe_seed(cfg.base_seed, 4, i)
        theta = np.zeros(d, np.float32)
        assert oracle.update(cfg, theta, 4, losses) == 0
        np.testing.assert_array_equal(theta, -coef * oracle.signs_at(cfg, seed, np.arange(d)).astype(np.float32))
        part = np.zeros(d, np.float32)
        assert oracle.update(cfg, part, 4, losses, elems=subset) == 0
        np.testing.assert_array_equal(part[subset], -coef * oracle.signs_at(cfg, seed, subset).astype(np.float32))
        rest = np.setdiff1d(np.arange(d), subset)
        assert not part[rest].any()

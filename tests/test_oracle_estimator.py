"""Pins for the oracle's CD-RGE estimator and update, against what the mathematics fixes.

Method (pith.science review of arXiv 2505.17852, "What carries the argument"; alex-wiki source
note, "Method"): theta' = theta - eta/(2K eps) * sum_i [L(theta+eps p_i) - L(theta-eps p_i)] p_i.
  (a) a central difference is exact for a quadratic, so (L+ - L-)/(2 eps) = grad(L).p;
  (b) the probe mean converges to the true gradient (brute force: forward-mode dual numbers,
      cross-checked by coordinate central differences), with relative MSE (d-1)/K for Rademacher
      probes (the review's major comment on Section 2, Eq. (6));
  (c) the bias of a single central difference shrinks as eps^2 (review: bias O(eps^2));
  plus the antithetic form of the paper's Appendix C and exact unit cases of the update.
"""
import numpy as np
import pytest

from oracle import OracleConfig

U = 2.0 ** -53


def _quad(seed=0, m=64, d=32):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((m, d))
    b = rng.standard_normal(m)
    theta = rng.standard_normal(d) * 0.5
    return A, b, theta


def test_quadratic_central_difference_is_exact(oracle):
    A, b, theta = _quad()
    g = A.T @ (A @ theta - b)
    for eps in (1e-1, 1e-2, 1e-3, 1e-4):
        losses, _ = oracle.quadratic_cdrge(A, b, theta, base_seed=99, step=3, n=8, eps=eps, lr=eps,
                                           want_update=False)
        for i in range(8):
            p = oracle.flat_probe(oracle.probe_seed(99, 3, i), 32).astype(np.float64)
            # the float eps the oracle used
            e = float(np.float32(eps))
            est = (losses[2 * i] - losses[2 * i + 1]) / (2 * e)
            bound = 64 * U * (abs(losses[2 * i]) + abs(losses[2 * i + 1])) / (2 * e) + 1e-13 * abs(g @ p)
            assert abs(est - g @ p) <= bound, (eps, i, est, g @ p)


def test_quadratic_update_is_minus_eta_g_hat(oracle):
    A, b, theta = _quad(1)
    g = A.T @ (A @ theta - b)
    K, eps = 16, 1e-3
    e = float(np.float32(eps))
    losses, new = oracle.quadratic_cdrge(A, b, theta, base_seed=5, step=0, n=K, eps=eps, lr=eps)
    P = np.stack([oracle.flat_probe(oracle.probe_seed(5, 0, i), 32) for i in range(K)]).astype(np.float64)
    g_hat = (P @ g) @ P / K        # exact central differences of a quadratic
    coef = float(np.float32(e / (2 * K * e)))
    expect = theta - coef * 2 * e * ((P @ g) @ P)
    np.testing.assert_allclose(new, expect, rtol=0, atol=1e-9 * np.abs(theta).max())
    # and in g-hat form (eta = eps): theta' = theta - eta g_hat
    np.testing.assert_allclose((theta - new) / e, g_hat, rtol=1e-6, atol=1e-9)


def test_quadratic_relative_mse_is_d_minus_1_over_k(oracle):
    # E ||g_hat_K - g||^2 / ||g||^2 = (d - 1) / K for Rademacher probes and exact differences.
    A, b, theta = _quad(2, d=32)
    g = A.T @ (A @ theta - b)
    K, eps, steps = 16, 1e-2, 300
    e = float(np.float32(eps))
    errs = []
    for s in range(steps):
        _, new = oracle.quadratic_cdrge(A, b, theta, base_seed=77, step=s, n=K, eps=eps, lr=eps)
        g_hat = (theta - new) / e
        errs.append(np.sum((g_hat - g) ** 2) / np.sum(g ** 2))
    mean = float(np.mean(errs))
    expect = (32 - 1) / K
    # the estimate of the mean has a few percent standard error at 300 steps
    assert abs(mean - expect) < 0.15 * expect, (mean, expect)


TINY = dict(n_layers=1, vocab=6, embed=4, hidden=8, batch=2, seq_len=4)


def _tiny(oracle, n_probes=1, eps=1e-3, lr=1e-3, seed=31):
    cfg = OracleConfig(n_probes=n_probes, storage="f64", eps=eps, lr=lr, base_seed=4242, **TINY)
    d = oracle.param_count(cfg)
    rng = np.random.default_rng(seed)
    theta = rng.uniform(-0.5, 0.5, d)
    tokens = rng.integers(0, cfg.vocab, size=(cfg.batch, cfg.seq_len + 1)).astype(np.int32)
    return cfg, theta, tokens


def _loss(oracle, cfg, theta, tokens):
    return oracle.seq_losses(cfg, theta, tokens).sum() / (cfg.batch * cfg.seq_len)


def test_dual_gradient_matches_coordinate_differences(oracle):
    cfg, theta, tokens = _tiny(oracle)
    g = oracle.grad(cfg, theta, tokens)
    h = 1e-6
    rng = np.random.default_rng(0)
    for j in rng.choice(len(theta), 60, replace=False):
        tp, tm = theta.copy(), theta.copy()
        tp[j] += h
        tm[j] -= h
        fd = (_loss(oracle, cfg, tp, tokens) - _loss(oracle, cfg, tm, tokens)) / (2 * h)
        assert abs(fd - g[j]) <= 1e-7 + 1e-6 * abs(g[j]), (j, fd, g[j])


def test_probe_mean_converges_to_gradient(oracle):
    # Brute force on a tiny LSTM: the CD-RGE update with eta = eps is -eps * g_hat, and g_hat
    # approaches the true gradient with relative error about sqrt((d - 1) / K).
    cfg0, theta, tokens = _tiny(oracle)
    g = oracle.grad(cfg0, theta, tokens)
    d = len(theta)
    errors, cosines = [], []
    for K in (256, 1024, 4096):
        cfg = OracleConfig(**{**cfg0.__dict__, "n_probes": K})
        losses, _ = oracle.probe_losses(cfg, theta, tokens, step=0)
        new = theta.copy()
        # double-precision losses are recomputed from the float ones the update consumes
        assert oracle.update(cfg, new, 0, losses) == 0
        g_hat = (theta - new) / float(np.float32(cfg.eps))
        rel = np.linalg.norm(g_hat - g) / np.linalg.norm(g)
        errors.append(rel)
        cosines.append(g_hat @ g / np.linalg.norm(g_hat) / np.linalg.norm(g))
        assert rel < 3 * np.sqrt((d - 1) / K), (K, rel)
        assert rel > np.sqrt((d - 1) / K) / 3, (K, rel)
    assert errors[0] > errors[1] > errors[2]
    slope = np.polyfit(np.log([256, 1024, 4096]), np.log(errors), 1)[0]
    assert -0.8 < slope < -0.3, slope
    assert cosines[-1] > 0.6 and cosines[0] < cosines[-1]


def test_central_difference_bias_is_order_eps_squared(oracle):
    cfg, theta, tokens = _tiny(oracle, eps=1e-2)
    seed = oracle.probe_seed(cfg.base_seed, 0, 0)
    p = oracle.probe_vector(cfg, seed).astype(np.float64)
    _, dl = oracle.dir_deriv(cfg, theta, tokens, p)
    errs = []
    for eps in (0.02, 0.01, 0.005):
        c = OracleConfig(**{**cfg.__dict__, "eps": eps})
        losses, _ = oracle.probe_losses(c, theta, tokens, 0, probe_ids=[0])
        # float losses lose the small bias; recompute in double through the exact loss
        e = float(np.float32(eps))
        lp = _loss(oracle, cfg, theta + e * p, tokens)
        lm = _loss(oracle, cfg, theta - e * p, tokens)
        np.testing.assert_allclose([lp, lm], losses, rtol=1e-6)
        errs.append((lp - lm) / (2 * e) - dl)
    r1, r2 = errs[0] / errs[1], errs[1] / errs[2]
    assert 3.6 < r1 < 4.4 and 3.6 < r2 < 4.4, (errs, r1, r2)


def test_antithetic_form_equals_central_difference(oracle):
    # Appendix C of the paper (per the pith.science review): the antithetic forward estimator
    # (L(θ+εp) - L(θ)) p - (L(θ-εp) - L(θ)) p equals the central difference; L(θ) cancels.
    cfg, theta, tokens = _tiny(oracle, n_probes=4)
    losses, _ = oracle.probe_losses(cfg, theta, tokens, 0)
    l0 = np.float32(_loss(oracle, cfg, theta, tokens))
    anti = [(losses[2 * i] - l0) - (losses[2 * i + 1] - l0) for i in range(4)]
    cd = [losses[2 * i] - losses[2 * i + 1] for i in range(4)]
    np.testing.assert_allclose(anti, cd, rtol=1e-5, atol=1e-9)


def test_update_single_probe_exact(oracle):
    # K = 1: theta' = theta - coef * d * p element by element (fp32 storage, exact arithmetic).
    cfg = OracleConfig(1, 5, 4, 8, 1, 1, 1, "f32", 2.0 ** -10, 2.0 ** -10, 9)
    d = oracle.param_count(cfg)
    rng = np.random.default_rng(1)
    theta = (rng.integers(-2**10, 2**10, d) * 2.0 ** -12).astype(np.float32)
    losses = np.array([1.75, 1.5], np.float32)       # d = 0.25, coef = 1/2
    p = oracle.probe_vector(cfg, oracle.probe_seed(9, 4, 0)).astype(np.float64)
    new = theta.copy()
    assert oracle.update(cfg, new, 4, losses) == 0
    np.testing.assert_array_equal(new, (theta.astype(np.float64) - 0.5 * 0.25 * p).astype(np.float32))


def test_update_observes_signs_through_unit_losses(oracle):
    # theta = 0 and d = e_i give theta' = -coef * p_i exactly, in fp32 and in bf16.
    for storage in ("f32", "bf16"):
        cfg = OracleConfig(2, 7, 8, 16, 1, 1, 4, storage, 1e-4, 1e-4, 123)
        d = oracle.param_count(cfg)
        for i in range(4):
            losses = np.zeros(8, np.float32)
            losses[2 * i] = 1.0
            theta = np.zeros(d, np.float32 if storage == "f32" else np.uint16)
            assert oracle.update(cfg, theta, 2, losses) == 0
            p = oracle.probe_vector(cfg, oracle.probe_seed(123, 2, i)).astype(np.float64)
            vals = theta if storage == "f32" else (theta.astype(np.uint32) << 16).view(np.float32)
            np.testing.assert_array_equal(vals.astype(np.float64), -p / 8)


def test_update_linear_in_loss_differences(oracle):
    cfg = OracleConfig(1, 5, 4, 8, 1, 1, 3, "f64", 1e-3, 1e-3, 17)
    d = oracle.param_count(cfg)
    theta = np.zeros(d)
    rng = np.random.default_rng(3)
    l1 = rng.standard_normal(6)
    l2 = rng.standard_normal(6)
    a, b, c = theta.copy(), theta.copy(), theta.copy()
    oracle.update_f64losses(cfg, a, 0, l1)
    oracle.update_f64losses(cfg, b, 0, l2)
    oracle.update_f64losses(cfg, c, 0, l1 + l2)
    np.testing.assert_allclose(c, a + b, rtol=1e-12, atol=1e-15)


def test_update_rejects_non_finite_losses(oracle):
    cfg = OracleConfig(1, 5, 4, 8, 1, 1, 2, "f32", 1e-3, 1e-3, 17)
    d = oracle.param_count(cfg)
    theta = np.ones(d, np.float32)
    for bad in (np.nan, np.inf):
        losses = np.array([1.0, 2.0, bad, 0.5], np.float32)
        assert oracle.update(cfg, theta, 0, losses) == 1
        np.testing.assert_array_equal(theta, 1.0)


def test_coefficient_is_eta_over_2k_eps(oracle):
    # eta != eps: the step is eta * g_hat (alex-wiki "Method" g-hat form).
    cfg = OracleConfig(1, 5, 4, 8, 1, 1, 2, "f64", 1e-3, 5e-3, 17)
    d = oracle.param_count(cfg)
    theta = np.zeros(d)
    losses = np.array([1.0, 0.0, 0.0, 0.0])
    oracle.update_f64losses(cfg, theta, 0, losses)
    p = oracle.probe_vector(cfg, oracle.probe_seed(17, 0, 0)).astype(np.float64)
    coef = float(np.float32(np.float64(np.float32(5e-3)) / (2 * 2 * np.float64(np.float32(1e-3)))))
    np.testing.assert_allclose(theta, -coef * p, rtol=1e-15)

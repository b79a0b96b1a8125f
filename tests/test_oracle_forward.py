"""Pins for the oracle's LSTM language-model loss against torch's own modules.

torch.nn.LSTM (gate order i, f, g, o), nn.Embedding-style lookup, nn.functional.linear and
nn.functional.cross_entropy compute, in float64 on the CPU, the model the oracle defines (one bias
per layer: torch's bias_hh is set to zero). A dropped term, a transposed weight, a wrong gate order
or a shifted target index in the oracle changes these losses far beyond the tolerance.
"""
import numpy as np
import pytest
import torch

from oracle import OracleConfig

SHAPES = [
    dict(n_layers=1, vocab=16, embed=16, hidden=32, batch=4, seq_len=10),   # the tiny workload
    dict(n_layers=2, vocab=7, embed=8, hidden=12, batch=3, seq_len=5),
    dict(n_layers=3, vocab=50, embed=6, hidden=5, batch=2, seq_len=4),
]


def _cfg(shape, storage="f64"):
    return OracleConfig(n_probes=1, storage=storage, eps=1e-3, lr=1e-3, base_seed=1, **shape)


def torch_seq_losses(oracle, cfg, theta64, tokens):
    lay = {tid: (off, rows, cols) for tid, off, rows, cols in oracle.layout(cfg)}

    def tensor(tid):
        off, rows, cols = lay[tid]
        return torch.from_numpy(theta64[off:off + rows * cols].reshape(rows, cols).copy())

    L, H = cfg.n_layers, cfg.hidden
    lstm = torch.nn.LSTM(cfg.embed, H, num_layers=L, batch_first=True, dtype=torch.float64)
    with torch.no_grad():
        for l in range(L):
            getattr(lstm, f"weight_ih_l{l}").copy_(tensor(1 + 3 * l))
            getattr(lstm, f"weight_hh_l{l}").copy_(tensor(2 + 3 * l))
            getattr(lstm, f"bias_ih_l{l}").copy_(tensor(3 + 3 * l).reshape(-1))
            getattr(lstm, f"bias_hh_l{l}").zero_()
        emb = tensor(0)
        tok = torch.from_numpy(tokens.astype(np.int64))
        x = emb[tok[:, :-1]]
        out, _ = lstm(x)
        logits = torch.nn.functional.linear(out, tensor(1 + 3 * L), tensor(2 + 3 * L).reshape(-1))
        ce = torch.nn.functional.cross_entropy(logits.reshape(-1, cfg.vocab), tok[:, 1:].reshape(-1),
                                               reduction="none")
        return ce.reshape(cfg.batch, cfg.seq_len).sum(dim=1).numpy()


@pytest.mark.parametrize("shape", SHAPES)
def test_forward_matches_torch_lstm(oracle, shape):
    cfg = _cfg(shape)
    d = oracle.param_count(cfg)
    rng = np.random.default_rng(21)
    theta = rng.uniform(-0.6, 0.6, d)
    tokens = rng.integers(0, cfg.vocab, size=(cfg.batch, cfg.seq_len + 1)).astype(np.int32)
    got = oracle.seq_losses(cfg, theta, tokens)
    ref = torch_seq_losses(oracle, cfg, theta, tokens)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=0)


def test_forward_fp32_storage_reads_weights_exactly(oracle):
    cfg = _cfg(SHAPES[0], storage="f32")
    d = oracle.param_count(cfg)
    rng = np.random.default_rng(22)
    theta32 = rng.uniform(-0.2, 0.2, d).astype(np.float32)
    tokens = rng.integers(0, cfg.vocab, size=(cfg.batch, cfg.seq_len + 1)).astype(np.int32)
    got = oracle.seq_losses(cfg, theta32, tokens)
    ref = torch_seq_losses(oracle, cfg, theta32.astype(np.float64), tokens)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=0)


def test_param_count_and_layout(oracle):
    # single-bias layout: V*E + sum_l (4H*in_l + 4H*H + 4H) + V*H + V
    for shape in SHAPES:
        cfg = _cfg(shape)
        V, E, H, L = cfg.vocab, cfg.embed, cfg.hidden, cfg.n_layers
        expect = V * E + sum(4 * H * (E if l == 0 else H) + 4 * H * H + 4 * H for l in range(L)) + V * H + V
        assert oracle.param_count(cfg) == expect
        lay = oracle.layout(cfg)
        assert [t[0] for t in lay] == list(range(3 * L + 3))
        assert all(lay[i + 1][1] == lay[i][1] + lay[i][2] * lay[i][3] for i in range(len(lay) - 1))
    big = [(1, 64, 256, 32, 338_976), (2, 128, 1024, 50, 13_173_042), (2, 4096, 4096, 50, 268_877_874),
           (4, 5888, 5888, 50, 1_110_076_466), (1, 16, 32, 16, 7_056)]
    for L, E, H, V, d in big:
        cfg = OracleConfig(L, V, E, H, 1, 1, 1, "f32", 1e-3, 1e-3, 1)
        assert oracle.param_count(cfg) == d


def _bf16_round(x: torch.Tensor) -> torch.Tensor:
    """float64 -> nearest bf16 (through float32, ties to even) -> float64, by torch's own casts."""
    return x.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def torch_bf16_seq_losses(oracle, cfg, weights64, tokens):
    """The bf16 model of the oracle rebuilt from torch's LSTMCell, F.linear and F.cross_entropy in
    float64: weights are the given (bf16-valued) numbers, and every activation is rounded to bf16
    where it enters a matrix product - h into W_hh, into the next layer's W_ih and into W_out."""
    lay = {tid: (off, rows, cols) for tid, off, rows, cols in oracle.layout(cfg)}

    def tensor(tid):
        off, rows, cols = lay[tid]
        return torch.from_numpy(weights64[off:off + rows * cols].reshape(rows, cols).copy())

    L, H, B = cfg.n_layers, cfg.hidden, cfg.batch
    cells = []
    with torch.no_grad():
        for l in range(L):
            cell = torch.nn.LSTMCell(cfg.embed if l == 0 else H, H, dtype=torch.float64)
            cell.weight_ih.copy_(tensor(1 + 3 * l))
            cell.weight_hh.copy_(tensor(2 + 3 * l))
            cell.bias_ih.copy_(tensor(3 + 3 * l).reshape(-1))
            cell.bias_hh.zero_()
            cells.append(cell)
        tok = torch.from_numpy(tokens.astype(np.int64))
        emb = tensor(0)
        h = [torch.zeros(B, H, dtype=torch.float64) for _ in range(L)]
        c = [torch.zeros(B, H, dtype=torch.float64) for _ in range(L)]
        total = torch.zeros(B, dtype=torch.float64)
        for t in range(cfg.seq_len):
            x = emb[tok[:, t]]
            for l in range(L):
                h[l], c[l] = cells[l](x, (_bf16_round(h[l]), c[l]))
                x = _bf16_round(h[l])
            logits = torch.nn.functional.linear(x, tensor(1 + 3 * L), tensor(2 + 3 * L).reshape(-1))
            total += torch.nn.functional.cross_entropy(logits, tok[:, t + 1], reduction="none")
        return total.numpy()


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bits_to_f64(u: np.ndarray) -> np.ndarray:
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("shape", SHAPES[:2])
def test_bf16_forward_matches_torch_cells_with_rounded_activations(oracle, shape):
    cfg = _cfg(shape, storage="bf16")
    d = oracle.param_count(cfg)
    rng = np.random.default_rng(23)
    w16 = _bf16_bits(rng.uniform(-0.6, 0.6, d))
    tokens = rng.integers(0, cfg.vocab, size=(cfg.batch, cfg.seq_len + 1)).astype(np.int32)
    got = oracle.seq_losses(cfg, w16, tokens, round_act_bf16=True)
    ref = torch_bf16_seq_losses(oracle, cfg, _bits_to_f64(w16), tokens)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=0)
    # the rounding points matter: without them the losses move far beyond the tolerance
    unrounded = oracle.seq_losses(cfg, w16, tokens, round_act_bf16=False)
    assert np.max(np.abs(unrounded - ref) / np.abs(ref)) > 1e-6


def test_bf16_probe_losses_match_torch(oracle):
    """Perturbed bf16 forwards: theta' = bf16(float(w) + float(s eps) p) formed with torch's
    rounding from the oracle's probe vector (itself pinned to rocRAND's Philox and the sign
    mapping), then the torch model above. Covers the oracle's perturbed copy and its bf16 forward."""
    shape = SHAPES[1]
    cfg = OracleConfig(n_probes=3, storage="bf16", eps=1e-2, lr=1e-2, base_seed=77, **shape)
    d = oracle.param_count(cfg)
    rng = np.random.default_rng(24)
    w16 = _bf16_bits(rng.uniform(-0.3, 0.3, d))
    tokens = rng.integers(0, cfg.vocab, size=(cfg.batch, cfg.seq_len + 1)).astype(np.int32)
    step = 5
    _, seq = oracle.probe_losses(cfg, w16, tokens, step)
    w32 = torch.from_numpy(_bits_to_f64(w16).astype(np.float32))
    for i in range(cfg.n_probes):
        p = torch.from_numpy(oracle.probe_vector(cfg, oracle.probe_seed(cfg.base_seed, step, i)).astype(np.float32))
        for side, sgn in enumerate((1.0, -1.0)):
            pert = (w32 + torch.tensor(sgn * cfg.eps, dtype=torch.float32) * p).to(torch.bfloat16)
            ref = torch_bf16_seq_losses(oracle, cfg, pert.to(torch.float64).numpy(), tokens)
            np.testing.assert_allclose(seq[2 * i + side], ref, rtol=1e-12, atol=0)


def test_fp32_probe_losses_match_torch(oracle):
    """Perturbed fp32 forwards: theta' = fl32(w + s eps p) formed by torch in float32 (one
    rounding of the sum; s eps p is exact) from the oracle's probe vector, then torch's LSTM in
    float64 on those float32 values. Covers the fp32 branch of the oracle's perturbed copy. eps is
    large enough that leaving any one tensor unperturbed moves the losses far beyond 1e-12."""
    shape = SHAPES[1]
    cfg = OracleConfig(n_probes=2, storage="f32", eps=3e-2, lr=3e-2, base_seed=78, **shape)
    d = oracle.param_count(cfg)
    rng = np.random.default_rng(25)
    w32 = rng.uniform(-0.3, 0.3, d).astype(np.float32)
    tokens = rng.integers(0, cfg.vocab, size=(cfg.batch, cfg.seq_len + 1)).astype(np.int32)
    step = 3
    _, seq = oracle.probe_losses(cfg, w32, tokens, step)
    w = torch.from_numpy(w32)
    lay = oracle.layout(cfg)
    for i in range(cfg.n_probes):
        p = torch.from_numpy(oracle.probe_vector(cfg, oracle.probe_seed(cfg.base_seed, step, i)).astype(np.float32))
        for side, sgn in enumerate((1.0, -1.0)):
            pert = w + torch.tensor(sgn * cfg.eps, dtype=torch.float32) * p
            assert pert.dtype == torch.float32
            ref = torch_seq_losses(oracle, cfg, pert.to(torch.float64).numpy(), tokens)
            np.testing.assert_allclose(seq[2 * i + side], ref, rtol=1e-12, atol=0)
            # every tensor's perturbation is visible at this bar
            for tid, off, rows, cols in lay:
                part = pert.clone()
                part[off:off + rows * cols] = w[off:off + rows * cols]
                moved = torch_seq_losses(oracle, cfg, part.to(torch.float64).numpy(), tokens)
                assert np.max(np.abs(moved - ref) / np.abs(ref)) > 1e-9, tid


def torch_io_seq_losses(oracle, cfg, theta64, inputs, targets):
    """torch's LSTM on separate inputs [B][T]; cross-entropy against targets [B][T] with
    ignore_index=-1 (ignored positions add nothing). Returns per-sequence sums and the mean over
    the scored positions (torch's own 'mean' reduction)."""
    lay = {tid: (off, rows, cols) for tid, off, rows, cols in oracle.layout(cfg)}

    def tensor(tid):
        off, rows, cols = lay[tid]
        return torch.from_numpy(theta64[off:off + rows * cols].reshape(rows, cols).copy())

    L, H = cfg.n_layers, cfg.hidden
    lstm = torch.nn.LSTM(cfg.embed, H, num_layers=L, batch_first=True, dtype=torch.float64)
    with torch.no_grad():
        for l in range(L):
            getattr(lstm, f"weight_ih_l{l}").copy_(tensor(1 + 3 * l))
            getattr(lstm, f"weight_hh_l{l}").copy_(tensor(2 + 3 * l))
            getattr(lstm, f"bias_ih_l{l}").copy_(tensor(3 + 3 * l).reshape(-1))
            getattr(lstm, f"bias_hh_l{l}").zero_()
        x = tensor(0)[torch.from_numpy(inputs.astype(np.int64))]
        out, _ = lstm(x)
        logits = torch.nn.functional.linear(out, tensor(1 + 3 * L), tensor(2 + 3 * L).reshape(-1))
        tg = torch.from_numpy(targets.astype(np.int64)).reshape(-1)
        flat = logits.reshape(-1, cfg.vocab)
        ce = torch.nn.functional.cross_entropy(flat, tg, ignore_index=-1, reduction="none")
        mean = torch.nn.functional.cross_entropy(flat, tg, ignore_index=-1, reduction="mean")
        return ce.reshape(cfg.batch, cfg.seq_len).sum(dim=1).numpy(), float(mean)


def test_io_form_matches_torch_with_ignored_targets(oracle):
    """The transduction form: inputs and targets given separately, targets of -1 not scored, the
    loss the mean over the scored positions. Pinned to torch's cross_entropy with ignore_index;
    the perturbed losses of probe_losses_io to the same torch model on a perturbed copy formed in
    torch from the oracle's probe vector (fp32 storage)."""
    shape = SHAPES[1]
    cfg = OracleConfig(n_probes=2, storage="f32", eps=3e-2, lr=3e-2, base_seed=79, **shape)
    d = oracle.param_count(cfg)
    rng = np.random.default_rng(26)
    w32 = rng.uniform(-0.4, 0.4, d).astype(np.float32)
    B, T, V = cfg.batch, cfg.seq_len, cfg.vocab
    inputs = rng.integers(0, V, size=(B, T)).astype(np.int32)
    targets = rng.integers(0, V, size=(B, T)).astype(np.int32)
    targets[rng.random((B, T)) < 0.4] = -1
    targets[0, :] = -1                                   # a sequence with nothing scored
    targets[1, :] = rng.integers(0, V, size=T)           # one with everything scored
    got = oracle.seq_losses_io(cfg, w32, inputs, targets)
    ref, _ = torch_io_seq_losses(oracle, cfg, w32.astype(np.float64), inputs, targets)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-300)
    assert got[0] == 0.0
    step = 4
    losses, seq = oracle.probe_losses_io(cfg, w32, inputs, targets, step)
    w = torch.from_numpy(w32)
    for i in range(cfg.n_probes):
        p = torch.from_numpy(oracle.probe_vector(cfg, oracle.probe_seed(cfg.base_seed, step, i)).astype(np.float32))
        for side, sgn in enumerate((1.0, -1.0)):
            pert = (w + torch.tensor(sgn * cfg.eps, dtype=torch.float32) * p).to(torch.float64).numpy()
            ref_seq, ref_mean = torch_io_seq_losses(oracle, cfg, pert, inputs, targets)
            np.testing.assert_allclose(seq[2 * i + side], ref_seq, rtol=1e-12, atol=1e-300)
            assert losses[2 * i + side] == np.float32(ref_mean)


def test_lm_form_is_the_io_form_with_shifted_targets(oracle):
    shape = SHAPES[0]
    cfg = OracleConfig(n_probes=2, storage="bf16", eps=1e-2, lr=1e-2, base_seed=80, **shape)
    d = oracle.param_count(cfg)
    rng = np.random.default_rng(27)
    w16 = _bf16_bits(rng.uniform(-0.3, 0.3, d))
    tokens = rng.integers(0, cfg.vocab, size=(cfg.batch, cfg.seq_len + 1)).astype(np.int32)
    a = oracle.probe_losses(cfg, w16, tokens, 1)
    b = oracle.probe_losses_io(cfg, w16, tokens[:, :-1].copy(), tokens[:, 1:].copy(), 1)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_exact_perturbation_bf16_matches_torch(oracle):
    """The exact-perturbation bf16 model (storage 'bf16x'): bf16 parameters, the probe added without
    rounding back to bf16 at radius eps' = bf16(eps): w + s eps' p for every matrix and bias
    element (formed here in float64, where it is exact), bf16(fl32(w + s eps' p)) for the
    embedding rows (activations of the first product). Then the bf16 torch model above
    (activations rounded where they enter a product). eps = 3e-3 sits below the bf16 spacing of
    most of these weights, so the plain bf16 model swallows most of the probe and this one does
    not."""
    shape = SHAPES[1]
    cfg = OracleConfig(n_probes=2, storage="bf16x", eps=3e-3, lr=3e-3, base_seed=81, **shape)
    d = oracle.param_count(cfg)
    rng = np.random.default_rng(28)
    w16 = _bf16_bits(rng.uniform(-0.6, 0.6, d))
    tokens = rng.integers(0, cfg.vocab, size=(cfg.batch, cfg.seq_len + 1)).astype(np.int32)
    step = 2
    _, seq = oracle.probe_losses(cfg, w16, tokens, step)
    r = float(torch.tensor(cfg.eps, dtype=torch.float32).to(torch.bfloat16).to(torch.float64))
    assert r != cfg.eps
    w64 = _bits_to_f64(w16)
    lay = {tid: (off, rows, cols) for tid, off, rows, cols in oracle.layout(cfg)}
    off0, rows0, cols0 = lay[0]
    emb = slice(off0, off0 + rows0 * cols0)
    plain = OracleConfig(n_probes=2, storage="bf16", eps=3e-3, lr=3e-3, base_seed=81, **shape)
    _, seq_plain = oracle.probe_losses(plain, w16, tokens, step)
    for i in range(cfg.n_probes):
        p = oracle.probe_vector(cfg, oracle.probe_seed(cfg.base_seed, step, i)).astype(np.float64)
        for side, sgn in enumerate((1.0, -1.0)):
            pert = w64 + sgn * r * p
            e32 = torch.from_numpy(w64[emb].astype(np.float32)) + torch.tensor(sgn * r, dtype=torch.float32) * \
                torch.from_numpy(p[emb].astype(np.float32))
            pert[emb] = e32.to(torch.bfloat16).to(torch.float64).numpy()
            ref = torch_bf16_seq_losses(oracle, cfg, pert, tokens)
            np.testing.assert_allclose(seq[2 * i + side], ref, rtol=1e-12, atol=0)
        # the probe differences of the two definitions differ well beyond rounding
        dx = seq[2 * i] - seq[2 * i + 1]
        dp = seq_plain[2 * i] - seq_plain[2 * i + 1]
        assert np.max(np.abs(dx - dp)) > 0.05 * np.max(np.abs(dx))


def test_exact_perturbation_update_uses_the_applied_radius(oracle):
    # theta = 0, d = e_0: theta' = bf16(-eta / (2 K eps') p_0), eps' = bf16(eps)
    shape = SHAPES[0]
    cfg = OracleConfig(n_probes=4, storage="bf16x", eps=1e-4, lr=1e-4, base_seed=82, **shape)
    d = oracle.param_count(cfg)
    theta = np.zeros(d, np.uint16)
    losses = np.zeros(8, np.float32)
    losses[0] = 1.0
    assert oracle.update(cfg, theta, 0, losses) == 0
    r = float(torch.tensor(1e-4, dtype=torch.float32).to(torch.bfloat16).to(torch.float64))
    coef = np.float32(float(np.float32(1e-4)) / (2.0 * 4 * float(np.float32(r))))  # double, rounded once
    p = oracle.probe_vector(cfg, oracle.probe_seed(cfg.base_seed, 0, 0)).astype(np.float32)
    want = torch.from_numpy(-coef * p).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(theta, want)

"""Host-side checks of the benchmark's output contract and of its traffic look-up (no GPU).

The recorded lines under profiles/ are what bench.py printed on one MI355X; these tests check
their shape and internal arithmetic, not their values.
"""
import glob
import json
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RECORDS = sorted(glob.glob(os.path.join(ROOT, "profiles", "bench_*.json")))

TOP_KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
            "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"}
ROOFLINE_KEYS = {"bound", "achieved", "peak", "unit", "frac", "traffic"}
CPU_KEYS = {"value", "unit", "cores", "kind", "sample"}


def _last_line(path):
    with open(path) as f:
        return json.loads(f.read().strip().splitlines()[-1])


def test_records_exist():
    names = {os.path.basename(p) for p in RECORDS}
    for w in ("tiny", "overfit", "charlm", "lstm270m", "lstm1b"):
        assert f"bench_{w}.json" in names


@pytest.mark.parametrize("path", RECORDS, ids=[os.path.basename(p) for p in RECORDS])
def test_record_contract(path):
    d = _last_line(path)
    assert TOP_KEYS <= set(d), TOP_KEYS - set(d)
    assert d["n_gpus"] == 1 and d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["data"] == "synthetic" and d["scaling"] in ("weak", "strong")
    name = os.path.basename(path)[len("bench_"):-len(".json")]
    if "_seqlen" in name:  # the same workload at another sequence length
        name, T = name.split("_seqlen")
        assert d["config"]["seq_len"] == int(T)
    assert d["config"]["workload"] == name
    # value is whole-step throughput: 2K * B * T perturbed-forward tokens per step over ms_per_step
    c = d["config"]
    tokens = 2 * c["n_probes"] * c["batch"] * c["seq_len"]
    assert d["value"] == pytest.approx(tokens / (d["ms_per_step"] / 1e3), rel=1e-9)
    r = d["roofline"]
    assert ROOFLINE_KEYS <= set(r)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], rel=1e-9)
    if d["dtype"] == "bf16":
        assert (r["bound"], r["unit"], r["peak"]) == ("mfma", "TFLOP/s", 2500.0)
        # algorithmic flops per launch / mean launch duration
        assert r["achieved"] == pytest.approx(r["flops_per_launch"] / (r["mean_launch_ms"] / 1e3) / 1e12, rel=1e-9)
    else:
        # fp32: the row-sliced kernel on the fp32 matrix cores, the persistent one on the vector ALUs
        bound = "mfma" if r["kernel"] == "k_lstm_f32_sliced" else "alu"
        assert r["kernel"] in ("k_lstm_f32", "k_lstm_f32_sliced")
        assert (r["bound"], r["unit"], r["peak"]) == (bound, "TFLOP/s", 157.3)
    assert r["traffic"] is None or r["traffic"] > 0
    cb = d["cpu_baseline"]
    assert CPU_KEYS <= set(cb) and cb["kind"] == "oracle" and cb["cores"] >= 1 and cb["value"] > 0


def test_traffic_lookup_follows_source_hash(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"kernel_source_hash": "abc123", "probes_per_chunk": 4, "hbm_bytes_per_launch": 12345.0}
    (prof / "gates_bf16_demo_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc123")
    assert bench.traffic_from_profiles("gates_bf16", "demo", 4) == 12345.0
    # another launch shape (pairs per launch) is not the launch the counters measured
    assert bench.traffic_from_profiles("gates_bf16", "demo", 8) is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "changed")
    assert bench.traffic_from_profiles("gates_bf16", "demo", 4) is None
    assert bench.traffic_from_profiles("gates_bf16", "missing", 4) is None


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "zero_order_recurrent_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "k.h").write_text("int a = 1;  // first\n/* block */ int b = 2;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h1 = bench.kernel_source_hash()
    (src / "k.h").write_text("int a = 1;  // reworded\n/* other words */ int b = 2;\n")
    assert bench.kernel_source_hash() == h1
    (src / "k.h").write_text("int a = 1;\nint b = 3;\n")
    assert bench.kernel_source_hash() != h1

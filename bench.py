#!/usr/bin/env python3
"""Benchmark of one CD-RGE step on one MI355X.

A step is the whole hot path on one batch: 2K perturbed LSTM forward passes with per-probe
cross-entropy losses (cdrge_probe_losses), then the seed-regenerating update (cdrge_update).
The default workload is the character-level LM of the pages' runtime table setting
(batch 1,024, training length 10, character vocabulary): 2-layer LSTM, E = 128, H = 1024, V = 50,
bf16 weights with fp32 accumulation, K = 64 probe pairs, eps = eta = 1e-4, Zipf(1.1) tokens.

Printed JSON line:
  value        perturbed-forward tokens per second over whole steps, 2K * B * T / step time
  roofline     the recurrent gate kernel (the dominant kernel): algorithmic matrix-core flops
               per launch / mean launch duration from HIP events on the launch stream, against
               the bf16 dense MFMA peak
  cpu_baseline the plain single-threaded CPU oracle on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16_mfma_tflops": 2500.0, "fp32_tflops": 157.3, "hbm_gbs": 8000.0}


def _code_tokens(text: str) -> bytes:
    """Source text without comments and whitespace runs, so that editing a comment does not
    make a profile of unchanged code look stale."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split()).encode()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "zero_order_recurrent_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(_code_tokens(f.read()))
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_tag: str, workload: str):
    """HBM bytes per launch of a kernel from the committed counter summary (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain copy of known size), if it was taken on the current kernel
    sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(preset, theta, tokens, budget_s: float):
    """Times the oracle on one probe pair over as many sequences as fit in about budget_s."""
    from oracle import Oracle, OracleConfig
    o = Oracle()
    oc = OracleConfig(preset.n_layers, preset.vocab, preset.embed, preset.hidden, preset.batch,
                      preset.seq_len, preset.n_probes, preset.dtype, preset.eps, preset.lr, preset.base_seed)
    # the call's cost is a fixed part (the perturbed parameter copies) plus a per-sequence part
    def timed(n):
        t0 = time.perf_counter()
        o.probe_losses(oc, theta, tokens, 0, probe_ids=[0], seq_ids=list(range(n)))
        return time.perf_counter() - t0
    n_probe = min(4, preset.batch)
    t1, tn = timed(1), timed(n_probe)
    per_seq = max((tn - t1) / max(n_probe - 1, 1), 1e-4)
    fixed = max(t1 - per_seq, 0.0)
    n_seq = int(max(1, min(preset.batch, (budget_s - fixed) / per_seq)))
    dt = timed(n_seq)
    toks = 2 * n_seq * preset.seq_len
    return {"value": toks / dt, "unit": "perturbed-forward tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"probe pair 0 (both signs) x {n_seq} sequences x T={preset.seq_len} at full model "
                      f"shape, including the perturbed parameter copies; {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="charlm")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = 1 << 28  # float32 elements: 1 GiB per direction
        a = torch.ones(n, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_direction": n * 4, "copies": 3}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (sharding the probes across GPUs "
              "is described, not built). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from zero_order_recurrent_amd import binding as b
    from zero_order_recurrent_amd.inputs import PRESETS, make_theta, make_tokens

    p = PRESETS[args.workload]
    cfg = b.config_from_preset(p)
    d = b.cdrge_param_count(cfg)
    theta_host = make_theta(p, d)
    tokens_host = make_tokens(p)
    if p.dtype == "bf16":
        params = torch.from_numpy(theta_host.view(np.int16).copy()).cuda()
    else:
        params = torch.from_numpy(theta_host.copy()).cuda()
    tokens = torch.from_numpy(tokens_host).cuda()
    ctx = b.Context(cfg, params)
    stream = torch.cuda.current_stream()

    for s in range(args.warmup):
        ctx.step(tokens, s)
    st = ctx.sync_status()
    if st not in (0, 5):
        raise RuntimeError(f"warmup failed: {b.STATUS[st]}")

    b.cdrge_get_timing(ctx.ctx, 0, reset=True)
    b.cdrge_set_timing(ctx.ctx, True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        ctx.step(tokens, args.warmup + s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    b.cdrge_set_timing(ctx.ctx, False)
    work = {k: b.cdrge_get_work(ctx.ctx, k) for k in range(4)}
    timing = {k: b.cdrge_get_timing(ctx.ctx, k) for k in range(4)}
    st = ctx.sync_status()

    # A separate forward-only pass (same inputs) for the perturbed-forward rate on its own.
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    n_fwd = max(1, args.steps // 2)
    for s in range(n_fwd):
        ctx.probe_losses(tokens, 1000 + s)
    torch.cuda.synchronize()
    fwd_s = (time.perf_counter() - t1) / n_fwd

    step_s = elapsed / args.steps
    tokens_per_step = 2 * p.n_probes * p.batch * p.seq_len
    gate_ms, gate_n = timing[0]
    gate_flops_per_launch = work[0] / max(gate_n, 1)
    gate_mean_s = gate_ms / 1e3 / max(gate_n, 1)
    achieved = gate_flops_per_launch / gate_mean_s / 1e12 if gate_n else 0.0
    peak = PEAK["bf16_mfma_tflops"] if p.dtype == "bf16" else PEAK["fp32_tflops"]
    traffic = traffic_from_profiles("gates_bf16" if p.dtype == "bf16" else "lstm_f32", args.workload)
    upd_traffic = traffic_from_profiles("update_bf16" if p.dtype == "bf16" else "update_f32", args.workload)
    upd_ms, upd_n = timing[2]
    upd_gbs = work[2] / (upd_ms / 1e3) / 1e9 if upd_n else 0.0
    ce_ms, ce_n = timing[1]

    line = {
        "metric": "perturbed-forward tokens/sec (2K*batch*seq) + CD-RGE steps/sec; % MFMA/HBM peak",
        "value": tokens_per_step / step_s,
        "unit": "perturbed-forward tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step_s * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if p.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": p.name, "n_layers": p.n_layers, "embed": p.embed, "hidden": p.hidden,
                   "vocab": p.vocab, "batch": p.batch, "seq_len": p.seq_len, "n_probes": p.n_probes,
                   "eps": p.eps, "lr": p.lr, "params": d, "tokens": p.tokens},
        "cdrge_steps_per_sec": 1.0 / step_s,
        "forward_only_tokens_per_sec": tokens_per_step / fwd_s,
        "roofline": {"bound": "mfma" if p.dtype == "bf16" else "alu", "kernel": "k_lstm_gates_bf16"
                     if p.dtype == "bf16" else "k_lstm_f32",
                     "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": traffic, "launches": gate_n, "mean_launch_ms": gate_mean_s * 1e3,
                     "flops_per_launch": gate_flops_per_launch},
        "update_roofline": {"bound": "hbm", "kernel": "k_update_perm" if p.dtype == "bf16" and p.n_probes <= 64
                            else "k_update_lut", "achieved": upd_gbs, "peak": PEAK["hbm_gbs"], "unit": "GB/s",
                            "frac": upd_gbs / PEAK["hbm_gbs"], "traffic": upd_traffic, "launches": upd_n,
                            "total_ms_per_step": upd_ms / args.steps},
        "time_split_ms_per_step": {"gates": gate_ms / args.steps, "logits_ce": ce_ms / args.steps,
                                   "update": upd_ms / args.steps, "prep": timing[3][0] / args.steps},
        "status": b.STATUS[st],
        "kernel_source_hash": kernel_source_hash(),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(p, theta_host, tokens_host, args.cpu_budget)
        line["cpu_baseline"]["gpu_over_cpu"] = line["value"] / line["cpu_baseline"]["value"]
    ctx.close()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

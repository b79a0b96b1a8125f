#!/usr/bin/env python3
"""Benchmark of one CD-RGE step on one MI355X.

A step is the whole hot path on one batch: 2K perturbed LSTM forward passes with per-probe
cross-entropy losses (cdrge_probe_losses), then the seed-regenerating update (cdrge_update).
The default workload is the largest one that fits one GPU, the ~1.1B-parameter model: 4-layer
LSTM, E = H = 5888, V = 50, bf16 weights with fp32 accumulation, batch 256, sequence length 10,
K = 16 probe pairs evaluated in chunks of 8, eps = eta = 1e-4, Zipf(1.1) tokens. --workload
selects the others (tiny, overfit, charlm, lstm270m, and the transduction tasks copy, reverse and
rollsum, which score only the output part of each sequence).

Printed JSON line:
  value        perturbed-forward tokens per second over whole steps, 2K * B * T / step time
  roofline     the recurrent gate kernel (the dominant kernel, named by the library): algorithmic
               flops per launch / mean launch duration from HIP events on the launch stream,
               against the bf16 dense MFMA peak, or the 157.3 TFLOP/s fp32 peak (matrix cores for
               k_lstm_f32_sliced, vector ALUs for k_lstm_f32)
  update_roofline  the update kernel against HBM (algorithmic bytes / launch time), with its
               ALU issue floor next to it
  cpu_baseline the plain single-threaded CPU oracle on a bounded sample of the same workload: on
               one core and as independent processes on the host's cores, with the CPU model
               and an extrapolated full-step time
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


def traffic_from_profiles(kernel_tag: str, workload: str, probes_per_chunk: int):
    """HBM bytes per launch of a kernel from the committed counter summary (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain copy of known size), if it was taken on the current kernel
    sources with the same probe pairs per launch; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash() or rec.get("probes_per_chunk") != probes_per_chunk:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_info() -> dict:
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count()}


def _mem_available() -> int:
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemAvailable:"):
                    return int(line.split()[1]) * 1024
    except OSError:
        pass
    return 0


def _oracle_config(preset):
    from oracle import OracleConfig
    return OracleConfig(preset.n_layers, preset.vocab, preset.embed, preset.hidden, preset.batch,
                        preset.seq_len, preset.n_probes, preset.dtype, preset.eps, preset.lr, preset.base_seed)


def cpu_worker(args) -> None:
    """Child process of the all-cores leg: its probe pairs (both signs) over its own sequences."""
    from oracle import Oracle
    from zero_order_recurrent_amd.inputs import PRESETS
    theta = np.load(os.path.join(args.cpu_worker, "theta.npy"), mmap_mode="r")
    inputs = np.load(os.path.join(args.cpu_worker, "inputs.npy"))
    targets = np.load(os.path.join(args.cpu_worker, "targets.npy"))
    p = PRESETS[args.workload].with_(seq_len=inputs.shape[1])
    o = Oracle()
    seqs = [int(v) for v in args.worker_seqs.split(",")]
    probes = [int(v) for v in args.worker_probe.split(",")]
    # everything is loaded: wait for the parent's start signal, so that all workers run together
    print("ready", flush=True)
    sys.stdin.readline()
    t0 = time.perf_counter()
    o.probe_losses_io(_oracle_config(p), theta, inputs, targets, 0, probe_ids=probes, seq_ids=seqs)
    dt = time.perf_counter() - t0
    print(json.dumps({"seconds": dt, "tokens": 2 * len(probes) * len(seqs) * p.seq_len}), flush=True)


def cpu_baseline(preset, theta, inputs, targets, budget_s: float) -> dict:
    """The oracle (plain single-threaded C++) on the host's cores, on a bounded sample of the
    workload: one probe pair, both signs, over full sequences, at full model shape, including the
    perturbed parameter copies the oracle builds for each sign. When the extrapolated whole step
    fits three times the budget (the small fp32 workloads), the whole step is run and measured
    instead. The reported value is the faster of the two legs (for tiny models the processes of the
    all-cores leg cost more than the work they share).

    1 core: the copies alone (0 sequences) and then with n sequences give the fixed cost per
    perturbed model and the cost per sequence; with the oracle's update timed on a slice of
    parameters, they extrapolate a whole CD-RGE step (2K perturbed models x B sequences + update).
    All cores: independent oracle processes over disjoint (probe pair, sequence) slices, as many
    as the host's cores (at most 16) and its free memory (one perturbed copy per process) allow.
    """
    import subprocess
    import tempfile
    from oracle import Oracle
    o = Oracle()
    oc = _oracle_config(preset)
    d = theta.size

    def timed(probe, seqs):
        t0 = time.perf_counter()
        o.probe_losses_io(oc, theta, inputs, targets, 0, probe_ids=[probe], seq_ids=list(seqs))
        return time.perf_counter() - t0

    t_copies = timed(0, [])                      # two perturbed copies, no forward
    t_one = timed(0, [0])                        # the copies and one sequence per sign
    per_seq = max((t_one - t_copies) / 2, 1e-6)  # one sequence through one perturbed model
    per_copy = t_copies / 2
    n_seq = int(max(1, min(preset.batch, (budget_s - t_copies) / (2 * per_seq))))
    dt = t_one if n_seq == 1 else timed(0, range(n_seq))
    single = {"value": 2 * n_seq * preset.seq_len / dt, "cores": 1, "seconds": dt,
              "sample": f"probe pair 0 (both signs) x {n_seq} sequence(s) x T={preset.seq_len} at full model "
                        f"shape, including the two perturbed parameter copies"}
    # the update on the first parameters (a full-length buffer of which only that slice is ever
    # touched, since the oracle updates listed elements in place), scaled to d
    n_upd = int(min(d, 1 << 21))
    work = np.empty(d, dtype=theta.dtype)
    work[:n_upd] = theta[:n_upd]
    losses = (3.0 + 1e-3 * np.random.default_rng(0).standard_normal(2 * preset.n_probes)).astype(np.float32)
    t0 = time.perf_counter()
    o.update(oc, work, 0, losses, elems=None if n_upd == d else np.arange(n_upd, dtype=np.int64))
    t_upd = (time.perf_counter() - t0) * d / n_upd
    del work
    models = 2 * preset.n_probes
    step_1core = models * per_copy + models * preset.batch * per_seq + t_upd
    single["extrapolated_full_step_s"] = step_1core
    single["extrapolation"] = (f"extrapolated, not measured: {models} perturbed copies x {per_copy:.3g} s + "
                               f"{models} x {preset.batch} sequences x {per_seq:.3g} s + update "
                               f"{t_upd:.3g} s (timed on {n_upd} of {d} parameters)")

    # When the whole step fits the budget (the small fp32 workloads), it is measured rather than
    # extrapolated: every probe pair over every sequence, then the full update.
    full = step_1core <= 3 * budget_s
    if full:
        t0 = time.perf_counter()
        full_l, _ = o.probe_losses_io(oc, theta, inputs, targets, 0)
        t_fwd = time.perf_counter() - t0
        work = theta.copy()
        t0 = time.perf_counter()
        o.update(oc, work, 0, full_l)
        t_up = time.perf_counter() - t0
        del work
        single = {"value": models * preset.batch * preset.seq_len / t_fwd, "cores": 1, "seconds": t_fwd,
                  "sample": f"the whole step: all {preset.n_probes} probe pairs (both signs) x {preset.batch} "
                            f"sequence(s) x T={preset.seq_len}, then the update",
                  "full_step_s": t_fwd + t_up, "extrapolated_full_step_s": t_fwd + t_up,
                  "extrapolation": "measured, not extrapolated"}
        step_1core = t_fwd + t_up

    # all cores: disjoint (probe pair, sequences) slices in child processes
    info = cpu_info()
    per_proc_bytes = 4 * d + (256 << 20)
    mem_cap = max(1, int(0.6 * _mem_available() // per_proc_bytes)) if _mem_available() else 1
    workers = max(1, min(info["nproc"], 16, mem_cap, preset.n_probes * preset.batch))
    n_each = max(1, min(n_seq, preset.batch * preset.n_probes // workers))
    if full:  # every worker: its share of the probe pairs over all sequences
        workers = max(1, min(workers, preset.n_probes))
    allcores = None
    if workers > 1:
        tmp = tempfile.mkdtemp(prefix="cdrge_cpu_")
        try:
            np.save(os.path.join(tmp, "theta.npy"), theta)
            np.save(os.path.join(tmp, "inputs.npy"), inputs)
            np.save(os.path.join(tmp, "targets.npy"), targets)
            procs = []
            for w in range(workers):
                if full:
                    probes = ",".join(str(q) for q in range(w, preset.n_probes, workers))
                    seqs = ",".join(str(q) for q in range(preset.batch))
                else:
                    probes = str(w % preset.n_probes)
                    first = (w // preset.n_probes) * n_each
                    seqs = ",".join(str((first + q) % preset.batch) for q in range(n_each))
                procs.append(subprocess.Popen(
                    [sys.executable, os.path.abspath(__file__), "--workload", preset.name, "--cpu-worker", tmp,
                     "--worker-probe", probes, "--worker-seqs", seqs],
                    stdin=subprocess.PIPE, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
            for pr in procs:  # every worker has its inputs loaded
                if pr.stdout.readline().strip() != "ready":
                    raise RuntimeError(f"oracle worker failed to start: {pr.stderr.read()[-400:]}")
            t0 = time.perf_counter()
            for pr in procs:
                pr.stdin.write("go\n")
                pr.stdin.flush()
            outs = []
            for pr in procs:
                out, err = pr.communicate()
                if pr.returncode != 0:
                    raise RuntimeError(f"oracle worker failed ({pr.returncode}): {err[-400:]}")
                outs.append(json.loads(out.strip().splitlines()[-1]))
            wall = time.perf_counter() - t0
        finally:
            for name in ("theta.npy", "inputs.npy", "targets.npy"):
                try:
                    os.remove(os.path.join(tmp, name))
                except OSError:
                    pass
            os.rmdir(tmp)
        toks = sum(r["tokens"] for r in outs)
        speedup = (toks / wall) / single["value"]
        if full:
            allcores = {"value": toks / wall, "cores": workers, "seconds": wall,
                        "sample": f"{workers} oracle processes sharing all {preset.n_probes} probe pairs (both "
                                  f"signs) x {preset.batch} sequence(s) x T={preset.seq_len}: the whole forward "
                                  f"of the step",
                        "extrapolated_full_step_s": wall + (step_1core - single["seconds"]),
                        "extrapolation": "the forward measured on all processes, plus the 1-core update"}
        else:
            allcores = {"value": toks / wall, "cores": workers, "seconds": wall,
                        "sample": f"{workers} oracle processes, each one probe pair (both signs) x {n_each} "
                                  f"sequence(s) x T={preset.seq_len} at full model shape with its own perturbed "
                                  f"copies; disjoint (probe, sequence) slices",
                        "extrapolated_full_step_s": step_1core / speedup,
                        "extrapolation": f"extrapolated, not measured: the 1-core step divided by the measured "
                                         f"speed-up of {speedup:.2f} on {workers} processes"}
    best = allcores if allcores is not None and allcores["value"] > single["value"] else single
    out = {"value": best["value"], "unit": "perturbed-forward tokens/s", "cores": best["cores"], "kind": "oracle",
           "sample": best["sample"] + f"; {best['seconds']:.1f} s",
           "extrapolated_full_step_s": best["extrapolated_full_step_s"],
           "single_core": single, **info}
    if allcores is not None:
        out["all_cores"] = allcores
    return out


def update_alu_floor(workload: str, kernel_ms: float):
    """The update's issue floor from its committed VALU instruction count (rocprofv3 --pmc
    SQ_INSTS_VALU, per launch): a wave64 VALU instruction occupies a 16-lane SIMD for 4 cycles, so
    the launch needs at least insts * 4 / (1,024 SIMDs * 2.4 GHz). None unless the counter summary
    was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"update_{workload}_valu.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    insts = rec["valu_insts_per_launch"]
    floor_ms = insts * 4 / (1024 * 2.4e9) * 1e3
    return {"bound": "alu", "valu_insts_per_launch": insts, "floor_ms": floor_ms, "measured_ms": kernel_ms,
            "frac": floor_ms / kernel_ms if kernel_ms > 0 else None,
            "peak": "1,024 SIMDs x 2.4 GHz, one wave64 VALU instruction per SIMD per 4 cycles"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="lstm1b")
    ap.add_argument("--seq-len", type=int, default=0,
                    help="override the workload's sequence length T (same model, batch and probes)")
    ap.add_argument("--probes-per-chunk", type=int, default=-1,
                    help="override the workload's probe pairs per chain of forward launches (0: all K "
                         "pairs at once); K / G is one GPU's share of a run over G GPUs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for the HBM byte counters)")
    ap.add_argument("--copy-rate", action="store_true",
                    help="only time plain device copies (torch's copy_) of 1 GiB and of an lstm1b theta "
                         "(2.22 GB): the read + write rate an update kernel is compared with")
    ap.add_argument("--cpu-worker", default=None, help=argparse.SUPPRESS)
    ap.add_argument("--worker-probe", default="0", help=argparse.SUPPRESS)
    ap.add_argument("--worker-seqs", default="0", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_worker:
        cpu_worker(args)
        return
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
    if args.copy_rate:
        import torch
        out = []
        for nbytes in (1 << 30, 2 * 1110076466):
            a = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
            b = torch.empty_like(a)
            for _ in range(3):
                b.copy_(a)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 20
            e0.record()
            for _ in range(reps):
                b.copy_(a)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            out.append({"bytes_per_direction": nbytes, "ms_per_copy": ms,
                        "read_plus_write_gbs": 2 * nbytes / (ms / 1e3) / 1e9})
            del a, b
        print(json.dumps({"copy": "torch copy_ (bf16), HIP events on the current stream", "runs": out}), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (sharding the probes across GPUs "
              "is described, not built). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    from zero_order_recurrent_amd.inputs import PRESETS, make_io, make_theta, make_tokens

    p = PRESETS[args.workload]
    if args.seq_len > 0:
        if p.task != "lm":
            print("--seq-len applies to the language-model workloads", file=sys.stderr)
            sys.exit(2)
        p = p.with_(seq_len=args.seq_len)
    if args.probes_per_chunk >= 0:
        p = p.with_(probes_per_chunk=args.probes_per_chunk)
    theta_host = make_theta(p, _param_count(p))
    lm = p.task == "lm"
    tokens_host = make_tokens(p) if lm else None
    inputs_host, targets_host = make_io(p)
    # The CPU legs run first, before this process touches the GPU: the all-cores leg starts
    # child processes, and the GPU then sits idle rather than sharing the host with them.
    cpu = None if args.no_cpu_baseline else cpu_baseline(p, theta_host, inputs_host, targets_host, args.cpu_budget)

    import torch
    from zero_order_recurrent_amd import binding as b

    cfg = b.config_from_preset(p)
    d = b.cdrge_param_count(cfg)
    assert d == theta_host.size
    bf16 = p.dtype != "f32"
    if bf16:
        params = torch.from_numpy(theta_host.view(np.int16).copy()).cuda()
    else:
        params = torch.from_numpy(theta_host.copy()).cuda()
    ctx = b.Context(cfg, params)
    if lm:
        tokens = torch.from_numpy(tokens_host).cuda()
        run_step = lambda s: ctx.step(tokens, s)  # noqa: E731
        run_fwd = lambda s: ctx.probe_losses(tokens, s)  # noqa: E731
    else:
        inputs = torch.from_numpy(inputs_host).cuda()
        targets = torch.from_numpy(targets_host).cuda()
        run_step = lambda s: ctx.step_io(inputs, targets, s)  # noqa: E731
        run_fwd = lambda s: ctx.probe_losses_io(inputs, targets, s)  # noqa: E731

    for s in range(args.warmup):
        run_step(s)
    st = ctx.sync_status()
    if st != 0:
        print(f"warmup steps ended with {b.STATUS[st]}", file=sys.stderr)
        sys.exit(1)

    b.cdrge_get_timing(ctx.ctx, 0, reset=True)
    b.cdrge_set_timing(ctx.ctx, True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        run_step(args.warmup + s)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    b.cdrge_set_timing(ctx.ctx, False)
    work = {k: b.cdrge_get_work(ctx.ctx, k) for k in range(4)}
    timing = {k: b.cdrge_get_timing(ctx.ctx, k) for k in range(4)}
    st = ctx.sync_status()
    if st != 0:
        # a non-finite loss turns every update into a no-op: the timings would not be of the path
        print(f"timed steps ended with {b.STATUS[st]}; no throughput is reported", file=sys.stderr)
        sys.exit(1)

    # A separate forward-only pass (same inputs) for the perturbed-forward rate on its own.
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    n_fwd = max(1, args.steps // 2)
    for s in range(n_fwd):
        run_fwd(1000 + s)
    torch.cuda.synchronize()
    fwd_s = (time.perf_counter() - t1) / n_fwd

    step_s = elapsed / args.steps
    tokens_per_step = 2 * p.n_probes * p.batch * p.seq_len
    gate_ms, gate_n = timing[0]
    gate_flops_per_launch = work[0] / max(gate_n, 1)
    gate_mean_s = gate_ms / 1e3 / max(gate_n, 1)
    achieved = gate_flops_per_launch / gate_mean_s / 1e12 if gate_n else 0.0
    gate_kernel = b.cdrge_timed_kernel(ctx.ctx, 0)
    upd_kernel = b.cdrge_timed_kernel(ctx.ctx, 2)
    peak = PEAK["bf16_mfma_tflops"] if bf16 else PEAK["fp32_tflops"]
    # the row-sliced fp32 kernel multiplies W on the fp32 matrix cores (157.3 TFLOP/s dense); the
    # persistent one on the vector ALUs (157.3 TFLOP/s with packed FMAs)
    gate_bound = "mfma" if bf16 or gate_kernel == "k_lstm_f32_sliced" else "alu"
    traffic = traffic_from_profiles({"k_lstm_gates_bf16": "gates_bf16", "k_lstm_f32": "lstm_f32",
                                     "k_lstm_f32_sliced": "lstm_f32_sliced"}.get(gate_kernel, gate_kernel),
                                    args.workload, p.probes_per_chunk)
    upd_traffic = traffic_from_profiles("update_bf16" if bf16 else "update_f32", args.workload, p.probes_per_chunk)
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
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic",
        "config": {"workload": p.name, "n_layers": p.n_layers, "embed": p.embed, "hidden": p.hidden,
                   "vocab": p.vocab, "batch": p.batch, "seq_len": p.seq_len, "n_probes": p.n_probes,
                   "probes_per_chunk": p.probes_per_chunk, "eps": p.eps, "lr": p.lr, "params": d,
                   **({"perturbation": "exact (W x +- eps' P x, eps' = bf16(eps); twice the matrix-core work)"}
                      if p.dtype == "bf16x" else {}),
                   **({"tokens": p.tokens} if lm else
                      {"task": p.task, "source_lengths": [p.min_len, p.max_len],
                       "scored_positions": int((targets_host >= 0).sum())})},
        "cdrge_steps_per_sec": 1.0 / step_s,
        "ms_per_timestep": step_s * 1e3 / p.seq_len,
        "workspace_bytes": b.cdrge_workspace_bytes(cfg),
        "forward_only_tokens_per_sec": tokens_per_step / fwd_s,
        "roofline": {"bound": gate_bound, "kernel": gate_kernel,
                     "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": traffic, "launches": gate_n, "mean_launch_ms": gate_mean_s * 1e3,
                     "flops_per_launch": gate_flops_per_launch},
        "update_roofline": {"bound": "hbm", "kernel": upd_kernel, "achieved": upd_gbs, "peak": PEAK["hbm_gbs"], "unit": "GB/s",
                            "frac": upd_gbs / PEAK["hbm_gbs"], "traffic": upd_traffic, "launches": upd_n,
                            "total_ms_per_step": upd_ms / args.steps,
                            "alu": update_alu_floor(args.workload, upd_ms / max(upd_n, 1))},
        "time_split_ms_per_step": {"gates": gate_ms / args.steps, "logits_ce": ce_ms / args.steps,
                                   "update": upd_ms / args.steps, "prep": timing[3][0] / args.steps},
        "status": b.STATUS[st],
        "kernel_source_hash": kernel_source_hash(),
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
        line["cpu_baseline"]["gpu_over_cpu"] = line["value"] / cpu["value"]
    ctx.close()
    print(json.dumps(line), flush=True)


def _param_count(p) -> int:
    """d of the flat layout (embedding, per layer W_ih, W_hh and one bias, output layer)."""
    d = p.vocab * p.embed + p.vocab * p.hidden + p.vocab
    for l in range(p.n_layers):
        d += 4 * p.hidden * (p.embed if l == 0 else p.hidden) + 4 * p.hidden * p.hidden + 4 * p.hidden
    return d


if __name__ == "__main__":
    main()

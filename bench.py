#!/usr/bin/env python3
"""Benchmark of the fused LM-head log-prob + entropy head on one MI355X.

One step = the whole hot path over one batch: the forward (logits tiles with
running max / exp-sum / exp-weighted sum and target select, split merge)
and the backward (logits recompute, cotangent blocks, dh and dW GEMMs) at
the batch-16 x 4096-token Qwen3-4B-shaped head: N = 65,536 tokens,
H = 2,560, V = 151,936, chunk_size = 512. Inputs are seeded synthetic data
(hidden ~ N(0,1) scaled to RMS 1, W ~ N(0, 0.02), uniform targets,
cotangents g_logp ~ N(0,1), g_ent ~ N(0,0.1)), resident in HBM before the
timed region starts.

Prints one JSON line: whole-job tokens/s, the credited MFMA throughput
(6 N H V flops per step) as a fraction of the bf16 dense peak, a roofline
entry for the dominant kernel (its average launch duration measured live
with HIP events through the library's tracing, on the stream the kernels run
on), and the fp64 CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 5] [--warmup 2]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused LM-head logp+entropy fwd+bwd tokens/s and % bf16 MFMA peak, H=2560 V=151936"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
WORKLOAD_INDEX = 3            # batch 16 x 4096 tokens


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    import hashlib
    path = os.path.join(ROOT, "cross_entropy_amd", "csrc", "lmhead_kernels.hip")
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def stored_counters():
    """The committed counter summary (FETCH_SIZE / WRITE_SIZE passes, each
    scaled by a plain copy of known size), or None when the counters were
    taken on another version of the kernels."""
    path = os.path.join(ROOT, "profiles", "lmhead_traffic_headline.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernels_source_sha256") != kernel_source_hash():
        return None
    return t


def stored_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None."""
    t = stored_counters()
    if t is None or t.get("kernel") != kernel:
        return None
    return t.get("hbm_bytes_per_launch")


def w_stream(fwd_ms: float):
    """The forward's W stream from the committed counter passes (bytes fetched
    from beyond L2 per forward: a counted bracket and the schedule's figure),
    as GB/s over this run's forward time and as re-reads of the table."""
    t = stored_counters()
    if t is None or "w_stream" not in t:
        return None
    w = t["w_stream"]
    sec = fwd_ms * 1e-3
    return {
        "unit": "GB/s",
        "bytes_per_forward": [w["w_bytes_lower"], w["w_bytes_upper"]],
        "bytes_per_forward_schedule": w["w_bytes_model"],
        "achieved": [round(w["w_bytes_lower"] / sec / 1e9, 1), round(w["w_bytes_upper"] / sec / 1e9, 1)],
        "peak": PEAK_HBM_GBS,
        "reuse_vs_table": [round(w["w_bytes_lower"] / w["w_table_bytes"], 1),
                           round(w["w_bytes_upper"] / w["w_table_bytes"], 1)],
        "forward_fetch_bytes": t.get("fwd_stats_kernel_bytes_per_launch"),
        "note": "L2-to-fabric fetch (FETCH_SIZE); Infinity Cache hits are included, so HBM reads are at most this",
    }


def cpu_baseline(h_bits, W_bits, targets, chunk, g_l, g_e, sample: int, N: int):
    """The fp64 oracle, as it stands, on `sample` tokens of the same inputs
    (forward + backward of those tokens; dW over them)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle.lmhead_oracle as O
    from synthetic import sample_tokens

    idx = sample_tokens(targets, sample, seed=11)
    gl = np.zeros_like(g_l)
    ge = np.zeros_like(g_e)
    gl[idx], ge[idx] = g_l[idx], g_e[idx]
    t0 = time.perf_counter()
    O.forward_backward(h_bits, W_bits, targets, chunk, gl, ge, tokens=idx)
    dt = time.perf_counter() - t0
    threads = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    return {
        "value": round(idx.size / dt, 3),
        "unit": "tokens/s",
        "cores": int(max(threads) if threads else 1),
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": f"{idx.size} sampled tokens of the N={N} workload, fp64 forward+backward "
                  f"(full logits row per token, dW over the sample; W widened to fp64 once), {dt:.1f} s",
    }


def smi_power():
    """Board power and per-XCD graphics clocks from one `amd-smi metric`
    reading (a child process), or None where the tool is unavailable."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "--power", "--clock", "--json"], capture_output=True, text=True,
                           timeout=30)
        d = json.loads(r.stdout)
        g = d["gpu_data"][0] if isinstance(d, dict) and "gpu_data" in d else d[0]
        clk = g["clock"]
        xcd = [clk[k]["clk"]["value"] for k in sorted(clk) if k.startswith("gfx_") and isinstance(clk[k].get("clk"), dict)]
        return {"socket_power_W": g["power"]["socket_power"]["value"], "gfx_clock_MHz": xcd}
    except Exception as e:  # the tool is absent or printed something else
        return {"error": repr(e)[:200]}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--cpu-sample", type=int, default=512, help="tokens the CPU oracle runs on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", type=int, default=WORKLOAD_INDEX, choices=(1, 2, 3, 4, 5),
                    help="synthetic workload (default 3, the batch-16 x 4096 headline; the others are "
                         "the one-sequence head, the context-rank share and the pad-first packed row)")
    ap.add_argument("--chunk", type=int, default=0, help="chunk_size override (workload 4 runs 1024 and 4096)")
    ap.add_argument("--grad-dtype", choices=("f32", "bf16"), default="f32",
                    help="gradient outputs: float32 (lmhead_logps_bwd, the default) or bf16 "
                         "(lmhead_logps_bwd_bf16: float32 sums in the workspace, rounded once)")
    ap.add_argument("--power", action="store_true",
                    help="also read board power and XCD clocks (amd-smi) while the forward alone, then the "
                         "backward alone, run back to back for a few seconds each")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 times), the known-size "
                         "reference for scaling FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this head runs on a single MI355X and has no "
              f"multi-GPU path (asked for --gpus {args.gpus})", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.copy_probe:
        n = args.copy_probe * (1 << 20)
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "copies": 5}), flush=True)
        return 0

    import cross_entropy_amd as lm
    from cross_entropy_amd import _native
    from synthetic import WORKLOADS, make_cotangents, make_inputs

    cfg = WORKLOADS[args.workload]
    N, H, V, C = cfg.N, cfg.H, cfg.V, (args.chunk or cfg.chunk_size)
    lm.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] generating workload {cfg.name}: N={N} H={H} V={V} chunk={C}")
    h_bits, W_bits, targets = make_inputs(cfg)
    g_l, g_e = make_cotangents(cfg)

    h = torch.from_numpy(h_bits.view(np.int16)).to(dev)
    W = torch.from_numpy(W_bits.view(np.int16)).to(dev)
    t = torch.from_numpy(targets).to(dev)
    gl = torch.from_numpy(g_l).to(dev)
    ge = torch.from_numpy(g_e).to(dev)
    logp = torch.empty(N, dtype=torch.float32, device=dev)
    ent = torch.empty(N, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    bf16_grads = args.grad_dtype == "bf16"
    gdt = torch.bfloat16 if bf16_grads else torch.float32
    dh = torch.empty((N, H), dtype=gdt, device=dev)
    dW = torch.empty((V, H), dtype=gdt, device=dev)
    ws = lm.workspace_for(h, W, C, with_backward="bf16" if bf16_grads else True)
    stream = torch.cuda.current_stream(dev)

    def backward():
        if bf16_grads:
            lm.lmhead_logps_bwd_bf16(h, W, t, C, 1.0, lse, ent, gl, ge, dh, dW, 0, ws, stream)
        else:
            lm.lmhead_logps_bwd(h, W, t, C, lse, ent, gl, ge, dh, dW, ws, stream)

    def step():
        lm.lmhead_logps_fwd(h, W, t, C, logp, ent, lse, ws, stream)
        backward()

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps")
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record(stream)
        lm.lmhead_logps_fwd(h, W, t, C, logp, ent, lse, ws, stream)
        e1.record(stream)
        backward()
        e2.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    fwd_ms = sum(a.elapsed_time(b) for a, b, _ in ev) / args.steps
    bwd_ms = sum(b.elapsed_time(c) for _, b, c in ev) / args.steps
    if not (np.all(np.isfinite(lse.cpu().numpy())) and bool(torch.isfinite(dW).all())):
        log("[bench] non-finite outputs")
        return 1

    # per-kernel launch times from a second pass of the same steps with the
    # library's HIP-event tracing on (its event records stay out of the
    # headline timing above)
    log(f"[bench] traced pass of {args.steps} steps")
    _native.trace_enable(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    traced_elapsed = time.perf_counter() - t1
    kernels = _native.trace_read()
    _native.trace_enable(False)

    ms_step = elapsed * 1e3 / args.steps
    credited = 6.0 * N * H * V
    executed = 8.0 * N * H * V
    tflops = credited / (ms_step * 1e-3) / 1e12

    dom_name, dom = max(kernels.items(), key=lambda kv: kv[1]["ms"])
    avg_ms = dom["ms"] / max(1, dom["launches"])
    if dom["flops"] > 0:
        # credited flops per launch (the backward's logits recompute is executed, not credited)
        achieved = dom["flops"] / max(1, dom["launches"]) / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None}
        recompute = 2.0 * N * H * V * args.steps if dom_name.startswith("bwd_step") else 0.0
        exe = (dom["flops"] + recompute) / (dom["ms"] * 1e-3) / 1e12
        roof["executed_achieved"] = round(exe, 1)
        roof["executed_frac"] = round(exe / PEAK_BF16_TFLOPS, 4)
    else:
        achieved = dom["bytes"] / max(1, dom["launches"]) / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    traffic = stored_traffic(dom_name)
    if traffic is not None:
        roof["traffic"] = traffic
    roof["kernel"] = dom_name
    roof["avg_launch_ms"] = round(avg_ms, 4)
    roof["launches_per_step"] = dom["launches"] / args.steps

    out = {
        "metric": METRIC,
        "value": round(N * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict({"workload": cfg.name, "N": N, "H": H, "V": V, "chunk_size": C,
                        "grad_dtype": args.grad_dtype},
                       **({"batch": 16, "seq_len": 4096} if args.workload == 3 else {}),
                       parallelism="none (one GPU)"),
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "tflops_credited": round(tflops, 1),
        "tflops_executed": round(executed / (ms_step * 1e-3) / 1e12, 1),
        "fwd_ms": round(fwd_ms, 3),
        "bwd_ms": round(bwd_ms, 3),
        "roofline": roof,
        "kernels": {k: {"launches": v["launches"] // args.steps, "ms_per_step": round(v["ms"] / args.steps, 3)}
                    for k, v in kernels.items() if v["launches"]},
        "traced_ms_per_step": round(traced_elapsed * 1e3 / args.steps, 3),
        "w_stream": w_stream(fwd_ms) if args.workload == WORKLOAD_INDEX else None,
    }
    if args.no_cpu_baseline:
        out["cpu_baseline"] = None
    else:
        log(f"[bench] CPU oracle on {args.cpu_sample} sampled tokens")
        out["cpu_baseline"] = cpu_baseline(h_bits, W_bits, targets, C, g_l, g_e, args.cpu_sample, N)
    if args.power:
        # enough queued calls of one kind to keep the GPU busy past the reading
        torch.cuda.synchronize()
        time.sleep(1.0)
        out["power"] = {"idle": smi_power()}
        for kind, reps in (("forward", 120), ("backward", 40)):
            for _ in range(reps):
                if kind == "forward":
                    lm.lmhead_logps_fwd(h, W, t, C, logp, ent, lse, ws, stream)
                else:
                    backward()
            time.sleep(2.0)
            out["power"][kind] = smi_power()
            torch.cuda.synchronize()
    real = int(np.count_nonzero((targets >= 0) & (targets < V)))
    if real != N:   # padded workloads: the rate of real (unmasked) tokens as well
        out["real_tokens_per_s"] = round(real * args.steps / elapsed, 1)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

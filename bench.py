#!/usr/bin/env python3
"""Benchmark of the batched multi-session decode step on one MI355X.

Workload: the 32-layer dense decoder (d=4096, 32 Q / 8 KV heads, hd=128, SwiGLU 14336, Q4_0
weights, final RMSNorm), every session at ctx 4096 -- the weight-stream-bound case on which
the metric "aggregate decode tok/s at B=1..16" is quoted.  A step is one kd_decode_step over
B rows (all 32 layers + final norm).  K timed steps run at positions 4096..4096+K-1 after W
warm-up steps (the same positions are re-written, so caches hold the same bytes each pass).

Prints ONE JSON line: aggregate decode tok/s at B=8 (``value``), the B=1..16 sweep, step HBM
GB/s, the roofline of the dominant kernel (mmvq on the gate/up shape 14336 x 4096 Q4_0 at
B=8, timed with HIP events on the launch stream) and of fa_decode at B=8, and the CPU oracle
timed on a bounded sample beside it.

``--summarize-trace CSV`` instead prints per-(kernel, grid) average durations from a
rocprofv3 kernel-trace CSV (the profiles/ summaries are made with it).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def summarize_trace(path: str) -> None:
    import csv
    from collections import defaultdict
    acc = defaultdict(lambda: [0, 0.0])
    with open(path) as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name") or row.get("KernelName") or "?"
            grid = "x".join(row.get(k, "") for k in ("Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z") if k in row)
            if not grid:
                grid = row.get("Grid_Size", "")
            dur = float(row["End_Timestamp"]) - float(row["Start_Timestamp"])
            a = acc[(name[:90], grid)]
            a[0] += 1
            a[1] += dur
    tot = sum(v[1] for v in acc.values())
    print(f"{'calls':>7} {'avg_us':>10} {'total_ms':>10} {'share':>6}  grid  kernel")
    for (name, grid), (n, t) in sorted(acc.items(), key=lambda kv: -kv[1][1]):
        print(f"{n:7d} {t / n / 1e3:10.2f} {t / 1e6:10.3f} {100 * t / tot:5.1f}%  {grid}  {name}")


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--sweep", default="1,2,4,8,16", help="batch widths to time")
    ap.add_argument("--headline-b", type=int, default=8, help="width whose aggregate tok/s is `value`")
    ap.add_argument("--kernel-iters", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=16, help="layers of one step the oracle is timed on")
    ap.add_argument("--summarize-trace", default=None)
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; the step shards by session across GPUs with no "
              "exchange (each GPU holds the weights and its own sessions), which is not measured here.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workload as W
    import session_decode_step_amd as kd
    from session_decode_step_amd.runner import GpuWorkload

    torch.cuda.set_device(0)
    widths = [int(b) for b in args.sweep.split(",")]
    Bmax = max(widths)
    Bh = args.headline_b if args.headline_b in widths else Bmax
    K, Wu = args.steps, args.warmup
    wl = W.workload("c4", B=Bmax, steps=max(K, Wu, 1))
    sp = wl.spec
    t0 = time.time()
    gw = GpuWorkload(wl, fill="device")   # seeded N(0,1) fp16 KV drawn on the device (speed)
    setup_s = time.time() - t0
    stream = torch.cuda.current_stream()

    # ---------------------------------------------------------------- whole steps
    sweep = {}
    for B in widths:
        rows = list(range(B))
        out = torch.empty((B, sp.out_dim), dtype=torch.float32, device="cuda")
        for s in range(Wu):
            gw.step(s, rows=rows, out=out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_host = time.perf_counter()
        e0.record(stream)
        for s in range(K):
            gw.step(s, rows=rows, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        host_s = time.perf_counter() - t_host
        ms = e0.elapsed_time(e1)
        sweep[B] = {"tok_s": B * K / (ms / 1e3), "ms_per_step": ms / K, "host_ms_per_step": 1e3 * host_s / K}

    # algorithmic bytes of one step at width B (weights once + KV read + KV write + acts)
    wbytes = W.algorithmic_bytes_weights(sp)
    G, hd, L = sp.n_head_kv, sp.head_dim, sp.n_layers

    def step_bytes(B, s):
        kv = sum((p + 1) * G * hd * 2 * 2 for p in wl.positions(s)[:B]) * L
        return wbytes + kv + B * G * hd * 4 * L

    mid = K // 2
    for B in widths:
        sweep[B]["step_GBs"] = step_bytes(B, mid) / (sweep[B]["ms_per_step"] / 1e3) / 1e9

    # ---------------------------------------------------------------- dominant kernel: mmvq
    # gate/up shape of the FFN (14336 x 4096 Q4_0) at the headline width: 64 of the step's
    # launches and 54% of its weight bytes.
    B = Bh
    lay = gw.model["layers"][0]
    pw = kd.kd_pack_weight(lay["w_gate"])
    xin = torch.randn((B, sp.d), device="cuda", generator=torch.Generator(device="cuda").manual_seed(0))
    act = kd.kd_quantize_act_q8(xin)
    y = torch.empty((B, pw.n_out), dtype=torch.float32, device="cuda")
    for _ in range(5):
        kd.kd_mmvq_q4_0(pw, act, B, y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.kernel_iters):
        kd.kd_mmvq_q4_0(pw, act, B, y)
    e1.record(stream)
    torch.cuda.synchronize()
    mm_us = e0.elapsed_time(e1) * 1e3 / args.kernel_iters
    n, k = pw.n_out, pw.k
    mm_bytes = n * k * 18 // 32 + B * k * (1 + 4 / 32) + B * n * 4
    mm_gbs = mm_bytes / (mm_us * 1e-6) / 1e9

    # ---------------------------------------------------------------- fa_decode at B = 8
    t_kv = [p + 1 for p in wl.positions(mid)[:B]]
    q = torch.randn((B, sp.n_head, hd), device="cuda", generator=torch.Generator(device="cuda").manual_seed(1))
    kb = [gw.caches.k_ptr(s, 0) for s in range(B)]
    vb = [gw.caches.v_ptr(s, 0) for s in range(B)]
    fa_ws = torch.empty(kd.kd_fa_decode_workspace(B, sp.n_head, hd, t_kv), dtype=torch.uint8, device="cuda")
    fa_out = torch.empty_like(q)
    for _ in range(5):
        kd.kd_fa_decode_ragged(q, G, kb, vb, t_kv, wl.capacity, hd ** -0.5, ws=fa_ws, out=fa_out)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.kernel_iters):
        kd.kd_fa_decode_ragged(q, G, kb, vb, t_kv, wl.capacity, hd ** -0.5, ws=fa_ws, out=fa_out)
    e1.record(stream)
    torch.cuda.synchronize()
    fa_us = e0.elapsed_time(e1) * 1e3 / args.kernel_iters
    fa_bytes = sum(t_kv) * G * hd * 2 * 2 + 2 * B * sp.n_head * hd * 4
    fa_gbs = fa_bytes / (fa_us * 1e-6) / 1e9

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        import dataclasses
        import oracle
        try:
            from threadpoolctl import threadpool_info
            info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
            threads = max([i.get("num_threads", 1) for i in info] or [1])
            blas = ",".join(sorted({i.get("internal_api", "?") for i in info}))
        except Exception:
            threads, blas = os.cpu_count(), "?"
        nl = min(args.cpu_layers, sp.n_layers)
        sub_spec = dataclasses.replace(sp, n_layers=nl)
        sub_model = {"spec": sub_spec, "layers": gw.model["layers"][:nl], "final_norm": gw.model["final_norm"],
                     "lm_head": None}
        sub_wl = dataclasses.replace(wl, spec=sub_spec)
        oc = oracle.OracleCaches(sub_wl, sessions=list(range(Bh)))
        t0 = time.perf_counter()
        oracle.decode_step(sub_model, oc, W.step_inputs(wl, 0)[:Bh], list(range(Bh)), wl.positions(0)[:Bh])
        cpu_s = (time.perf_counter() - t0) * sp.n_layers / nl
        cpu = {"value": round(Bh / cpu_s, 3), "unit": "tok/s", "cores": int(threads), "kind": "oracle",
               "sample": f"one decode step of B={Bh} rows through {nl} of the {sp.n_layers} layers (fp64 numpy, "
                         f"{blas} BLAS, oracle's own seeded KV), time scaled by {sp.n_layers}/{nl}: "
                         f"{cpu_s:.1f} s per full step"}

    top = sweep[Bh]
    res = {
        "metric": "aggregate decode tok/s at B=1..16; achieved HBM GB/s vs MI355X peak",
        "value": round(top["tok_s"], 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wu,
        "ms_per_step": round(top["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 x int8 -> int32 block dots, fp32 epilogue / attention",
        "data": "synthetic (seeded): Q4_0 weights, fp16 KV N(0,1) (device generator), N(0,1) input rows",
        "config": {"workload": "32-layer dense decoder d=4096, 32Q/8KV hd=128, SwiGLU 14336, Q4_0 weights, "
                               f"final RMSNorm; B={Bh} sessions at ctx 4096, decode positions 4096..{4096 + K - 1}",
                   "B": Bh, "ctx": 4096, "layers": L, "parallelism": "single GPU"},
        "sweep": {str(b): {kk: round(v, 3) for kk, v in sweep[b].items()} for b in widths},
        "step_GBs": round(top["step_GBs"], 1),
        "step_frac_of_peak": round(top["step_GBs"] / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": "mmvq_kernel<Q4_0> 14336x4096 (gate/up) at B=%d" % Bh,
                     "achieved": round(mm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(mm_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "avg_launch_us": round(mm_us, 3), "algorithmic_bytes": int(mm_bytes)},
        "fa_roofline": {"bound": "hbm", "kernel": "fa_split_kernel + fa_combine_kernel, B=%d, t_kv=%d" % (B, t_kv[0]),
                        "achieved": round(fa_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(fa_gbs / HBM_PEAK_GBS, 4), "avg_launch_us": round(fa_us, 3),
                        "algorithmic_bytes": int(fa_bytes)},
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()

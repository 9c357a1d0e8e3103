#!/usr/bin/env python3
"""Benchmark of the batched multi-session decode step on one MI355X.

Workload: the 32-layer dense decoder (d=4096, 32 Q / 8 KV heads, hd=128, SwiGLU 14336, Q4_0
weights, final RMSNorm), every session at ctx 4096 -- the weight-stream-bound case on which
the metric "aggregate decode tok/s at B=1..16" is quoted.  A step is one kd_decode_step over
B rows (all 32 layers + final norm).  K timed steps run at positions 4096..4096+K-1 after W
warm-up steps (the same positions are re-written, so caches hold the same bytes each pass).

Prints ONE JSON line: aggregate decode tok/s at B=8 (``value``), the B=1..16 sweep, step HBM
GB/s, the roofline of the dominant kernel (fa_decode at B=8) and of the largest product (the
gate/up mmvq, 28672 x 4096 Q4_0 at B=8), both timed with HIP events on the launch stream, the
other workloads of the path (``other_workloads``: the 8-layer Q8_0 stack with lm_head at
B=1..8, the ragged B=16 attention sublayer and its fa_decode, the MoE verify step, the
headline stack with FP8 E4M3 caches and its fa_decode, the gated delta-rule state step), and the
CPU oracle timed on a bounded sample beside it.

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
    """Per-(kernel, grid) call counts and average durations from a rocprofv3 kernel-trace
    CSV, then the longest run of back-to-back dispatches of one of this library's (kernel,
    grid): the bench's own timing loop of a kernel, whose average the bench reports."""
    import csv
    from collections import defaultdict
    acc = defaultdict(lambda: [0, 0.0, 0])
    seq = []
    with open(path) as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name") or row.get("KernelName") or "?"
            grid = "x".join(row.get(k, "") for k in ("Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z") if k in row)
            dur = float(row["End_Timestamp"]) - float(row["Start_Timestamp"])
            key = (name[:90], grid)
            a = acc[key]
            a[0] += 1
            a[1] += dur
            a[2] = int(row.get("VGPR_Count") or 0) + int(row.get("Accum_VGPR_Count") or 0)
            seq.append((int(row.get("Dispatch_Id") or len(seq)), key, dur))
    seq.sort()
    tot = sum(v[1] for v in acc.values())
    print(f"{'calls':>7} {'avg_us':>10} {'total_ms':>10} {'share':>6} {'vgpr':>4}  grid  kernel")
    for (name, grid), (n, t, vg) in sorted(acc.items(), key=lambda kv: -kv[1][1]):
        print(f"{n:7d} {t / n / 1e3:10.2f} {t / 1e6:10.3f} {100 * t / tot:5.1f}% {vg:4d}  {grid}  {name}")
    best, i = (0, 0, 0), 0
    while i < len(seq):
        j = i
        while j + 1 < len(seq) and seq[j + 1][1] == seq[i][1]:
            j += 1
        if j - i + 1 > best[0] and "kd::" in seq[i][1][0]:   # this library's kernels only
            best = (j - i + 1, i, j)
        i = j + 1
    n, i, j = best
    if n > 1:
        durs = [d for _, _, d in seq[i:j + 1]]
        print(f"\nlongest back-to-back run: {n} dispatches of {seq[i][1][0]} grid {seq[i][1][1]}: "
              f"avg {sum(durs) / n / 1e3:.2f} us (min {min(durs) / 1e3:.2f}, max {max(durs) / 1e3:.2f})")
    # the fa_decode timing loop: back-to-back (split, combine) pairs of one shape
    best, i = (0, 0), 0
    while i + 1 < len(seq):
        a, b = seq[i][1], seq[i + 1][1]
        if "fa_split_kernel" in a[0] and "fa_combine_kernel" in b[0]:
            j = i
            while j + 3 < len(seq) and seq[j + 2][1] == a and seq[j + 3][1] == b:
                j += 2
            if (j - i) // 2 + 1 > best[0]:
                best = ((j - i) // 2 + 1, i)
            i = j + 2
        else:
            i += 1
    n, i = best
    if n > 1:
        sp = [seq[i + 2 * m][2] for m in range(n)]
        cb = [seq[i + 2 * m + 1][2] for m in range(n)]
        pr = [x + y for x, y in zip(sp, cb)]
        print(f"longest back-to-back fa_decode run: {n} (split, combine) pairs, split grid {seq[i][1][1]}: "
              f"split avg {sum(sp) / n / 1e3:.2f} us + combine avg {sum(cb) / n / 1e3:.2f} us = "
              f"{sum(pr) / n / 1e3:.2f} us per call (min {min(pr) / 1e3:.2f}, max {max(pr) / 1e3:.2f})")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def mmvq_algorithmic_bytes(n: int, k: int, B: int) -> int:
    """The interleaved gate/up product with its SwiGLU epilogue: Q4_0 weights once (18 B per
    32), B int8 activation rows of k with fp32 block scales in, B quantised rows of F = n/2
    (int8 codes + fp32 block scales) out."""
    F = n // 2
    return n * k * 18 // 32 + B * k + B * (k // 32) * 4 + B * F + B * (F // 32) * 4


def time_rotating(launch, iters: int, stream) -> float:
    """Average launch duration (us) of ``launch(i)`` over ``iters`` launches, HIP events on
    ``stream`` (the stream the launches go to), after a few untimed ones."""
    import torch
    for i in range(4):
        launch(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(iters):
        launch(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / iters


# ---------------------------------------------------------------------- HBM traffic (PMC)
CALIB_BYTES = 512 << 20
FA_B, FA_T, FA_CAP = 8, 4113, 4128          # fa_decode traffic case: B rows of t keys
MM_N, MM_K, MM_B = 28672, 4096, 8           # gate/up product traffic case


def fa_algorithmic_bytes(t_kv, G: int, H: int, hd: int, kv_bytes: int = 2) -> int:
    """fa_decode: each row's K and V (fp16, or 1-byte E4M3 codes) once, q in and the output
    out (fp32)."""
    return sum(t_kv) * G * hd * kv_bytes * 2 + 2 * len(t_kv) * H * hd * 4


TRAFFIC = {
    "fa": {"file": os.path.join(ROOT, "profiles", "traffic_fa_decode_b8_t4113.txt"),
           "sources": ("session_decode_step_amd/csrc/attn.hip", "session_decode_step_amd/csrc/kd_internal.h"),
           "kernels": ("fa_split_kernel", "fa_combine_kernel"),
           "title": "fa_decode (fa_split_kernel + fa_combine_kernel), B=8 rows of t=4113 keys, H=32, G=8, hd=128",
           "algorithmic": lambda: fa_algorithmic_bytes([FA_T] * FA_B, 8, 32, 128)},
    "mmvq": {"file": os.path.join(ROOT, "profiles", "traffic_mmvq_q4_0_28672x4096_b8.txt"),
             "sources": ("session_decode_step_amd/csrc/mmvq.hip", "session_decode_step_amd/csrc/kd_internal.h"),
             "kernels": ("mmvq_kernel",),
             "title": "mmvq_kernel<Q4_0> with the SwiGLU epilogue, gate/up 28672 x 4096, B=8",
             "algorithmic": lambda: mmvq_algorithmic_bytes(MM_N, MM_K, MM_B)},
}


def kernel_source_hash(kind: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC[kind]["sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_probe() -> None:
    """Launches for the two ``rocprofv3 --pmc`` passes: a plain fp32 elementwise copy of
    512 MiB (the calibration kernel: reads and writes 512 MiB), then 8 launches of the gate/up
    mmvq with its SwiGLU epilogue at B=8 over four distinct matrices, then 8 fa_decode calls
    at B=8 over two distinct sets of caches."""
    import torch
    import workload as W
    import session_decode_step_amd as kd
    torch.cuda.set_device(0)
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst
    mats = [kd.kd_pack_weight(W.draw_weight("q4_0", 0, 4, 90, 91, i, MM_N, MM_K)) for i in range(4)]
    act = kd.kd_quantize_act_q8(torch.randn((MM_B, MM_K), device="cuda"))
    h_act = kd.alloc_act(MM_B, MM_N // 2)
    for i in range(8):
        kd.kd_mmvq_swiglu(mats[i % 4], act, MM_B, h_act)
    torch.cuda.synchronize()
    H, G, hd = 32, 8, 128
    sets = [torch.empty((FA_B, 2, G, FA_CAP, hd), dtype=torch.float16, device="cuda").fill_(0.01) for _ in range(2)]
    t_kv = [FA_T] * FA_B
    q = torch.randn((FA_B, H, hd), device="cuda")
    ws = torch.empty(kd.kd_fa_decode_workspace(FA_B, H, hd, t_kv), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    for i in range(8):
        c = sets[i % 2]
        kd.kd_fa_decode_ragged(q, G, [c[b, 0].data_ptr() for b in range(FA_B)], [c[b, 1].data_ptr() for b in range(FA_B)],
                               t_kv, FA_CAP, hd ** -0.5, ws=ws, out=out)
    torch.cuda.synchronize()
    log("traffic probe done")


def _read_counters(path: str):
    """[(dispatch, kernel_name, counter_value)] in dispatch order from a rocprofv3
    counter_collection CSV (or the directory holding it)."""
    import csv
    import glob
    if os.path.isdir(path):
        hits = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
        if len(hits) != 1:
            raise SystemExit(f"expected one counter_collection.csv under {path}, found {hits}")
        path = hits[0]
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            key = int(row.get("Dispatch_Id") or row.get("Correlation_Id"))
            name = row.get("Kernel_Name", "?")
            val = float(row["Counter_Value"])
            prev = out.get(key, (name, 0.0))
            out[key] = (name, prev[1] + val)
    return [(k, nm, v) for k, (nm, v) in sorted(out.items())]


def traffic_summarize(fetch: str, write: str, fetch_cmd: str, write_cmd: str) -> None:
    """HBM bytes per launch of the measured kernels from the FETCH_SIZE and WRITE_SIZE passes
    (KiB per dispatch), each scaled by what the counter reads for the 512 MiB calibration
    copy; writes one profile summary per kernel, which the bench reads back.  A call of
    several kernels (fa_decode: split + combine) counts the mean of each kernel once."""
    rows = {tag: _read_counters(path) for tag, path in (("fetch", fetch), ("write", write))}
    factor, calib_kib = {}, {}
    for tag, rr in rows.items():
        calib = max((v for _, nm, v in rr if "MulFunctor" in nm), default=0.0)
        if not calib:
            raise SystemExit(f"{tag}: calibration dispatch missing")
        calib_kib[tag], factor[tag] = calib, CALIB_BYTES / (calib * 1024.0)
    for kind, spec in TRAFFIC.items():
        per = {}
        for tag, rr in rows.items():
            per[tag] = {kn: [v for _, nm, v in rr if kn in nm] for kn in spec["kernels"]}
            if not all(per[tag].values()):
                raise SystemExit(f"{tag}: {kind} dispatches missing")
        byts = {tag: sum(sum(v) / len(v) for v in per[tag].values()) * 1024.0 * factor[tag] for tag in per}
        alg = spec["algorithmic"]()
        total = byts["fetch"] + byts["write"]
        rec = {"kernel": spec["title"], "source_hash": kernel_source_hash(kind),
               "fetch_bytes": round(byts["fetch"]), "write_bytes": round(byts["write"]),
               "traffic_bytes": round(total), "algorithmic_bytes": alg,
               "traffic_over_algorithmic": round(total / alg, 4),
               "fetch_factor": round(factor["fetch"], 5), "write_factor": round(factor["write"], 5)}
        lines = [
            f"HBM traffic of {spec['title']} (rocprofv3 PMC, MI355X)",
            "",
            f"FETCH_SIZE pass: {fetch_cmd}",
            f"WRITE_SIZE pass: {write_cmd}",
            "summary: python bench.py --traffic-summarize <fetch dir> <write dir>",
            "",
            f"calibration: torch.mul(x, 1.0, out=y) over {CALIB_BYTES >> 20} MiB fp32 (reads and writes {CALIB_BYTES} B)",
            f"  FETCH_SIZE {calib_kib['fetch']:.0f} KiB -> factor {factor['fetch']:.5f} B per counted B",
            f"  WRITE_SIZE {calib_kib['write']:.0f} KiB -> factor {factor['write']:.5f}",
        ]
        for tag in ("fetch", "write"):
            for kn, vals in per[tag].items():
                lines.append(f"{kn} dispatches {tag.upper()}_SIZE KiB: {', '.join(f'{v:.0f}' for v in vals)}")
        lines += [
            f"per launch: fetch {rec['fetch_bytes']} B + write {rec['write_bytes']} B = {rec['traffic_bytes']} B; "
            f"algorithmic {alg} B; ratio {rec['traffic_over_algorithmic']}",
            "",
            "TRAFFIC_JSON " + json.dumps(rec),
        ]
        os.makedirs(os.path.dirname(spec["file"]), exist_ok=True)
        with open(spec["file"], "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines) + "\n")


def load_traffic(kind: str):
    """Measured HBM bytes per launch of a kernel, or None when no measurement exists or the
    kernel source has changed since it was taken."""
    path = TRAFFIC[kind]["file"]
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("TRAFFIC_JSON "):
            rec = json.loads(line[len("TRAFFIC_JSON "):])
            if rec.get("source_hash") == kernel_source_hash(kind):
                return rec["traffic_bytes"]
    return None


def _time_steps(gw, stream, K: int, Wu: int, rows=None, repeat_first: bool = False) -> float:
    """Average ms per kd_decode_step of ``gw`` over K steps after Wu warm-up steps (HIP
    events on ``stream``); ``repeat_first``: re-run step 0 (its appends rewrite the same
    slots, so the caches hold the same bytes each time)."""
    import torch
    rows = list(range(gw.wl.B)) if rows is None else list(rows)
    out = torch.empty((len(rows), gw.wl.spec.out_dim), dtype=torch.float32, device="cuda")
    steps = [0] * max(K, Wu) if repeat_first else list(range(max(K, Wu)))
    gw.prefetch(sorted(set(steps)), rows)
    for s in steps[:Wu]:
        gw.step(s, rows=rows, out=out, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in steps[:K]:
        gw.step(s, rows=rows, out=out, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / K


def other_workloads(stream, iters: int) -> dict:
    """The other measured workloads of the path, beside the headline (same stream, inputs
    resident): the 8-layer Q8_0 stack with its 32000-row lm_head at B = 1, 2, 4, 8 (ctx 1238);
    the attention sublayer with B = 16 ragged rows (log-uniform lengths in [512, 32768]), its
    step and its fa_decode; the 8-layer MoE stack's verify step (4 streams x 4 draft rows,
    ctx 8192); the headline stack with FP8 E4M3 caches and its fa_decode; the gated
    delta-rule state step at B = 8 x 32 heads."""
    import torch
    import workload as W
    import session_decode_step_amd as kd
    from session_decode_step_amd.runner import GpuWorkload
    res = {}
    # dense Q8_0 stack with lm_head
    log("8-layer Q8_0 stack with lm_head")
    wl = W.workload("c2", B=8, steps=64)
    gw = GpuWorkload(wl, fill="device")
    dense = {}
    for B in (1, 2, 4, 8):
        ms = _time_steps(gw, stream, 16, 3, rows=list(range(B)))
        dense[str(B)] = {"tok_s": round(B / ms * 1e3, 1), "ms_per_step": round(ms, 4)}
    res["8-layer d=2048 Q8_0 decoder + lm_head 32000, ctx 1238"] = dense
    del gw
    # attention sublayer, ragged B = 16
    log("attention sublayer, ragged B=16")
    wl = W.workload("c3")
    gw = GpuWorkload(wl, fill="device")
    ms = _time_steps(gw, stream, iters, 3, repeat_first=True)
    sp = wl.spec
    t_kv = [p + 1 for p in wl.positions(0)]
    q = torch.randn((wl.B, sp.n_head, sp.head_dim), device="cuda",
                    generator=torch.Generator(device="cuda").manual_seed(2))
    kb = [gw.caches.k_ptr(s, 0) for s in range(wl.B)]
    vb = [gw.caches.v_ptr(s, 0) for s in range(wl.B)]
    ws = torch.zeros(kd.kd_fa_decode_workspace(wl.B, sp.n_head, sp.head_dim, t_kv), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    us = time_rotating(lambda i: kd.kd_fa_decode_ragged(q, sp.n_head_kv, kb, vb, t_kv, wl.capacity,
                                                       sp.head_dim ** -0.5, ws=ws, out=out, stream=stream),
                       iters, stream)
    fb = fa_algorithmic_bytes(t_kv, sp.n_head_kv, sp.n_head, sp.head_dim)
    res["attention sublayer d=4096 32Q/8KV hd=128 Q8_0, B=16 ragged ctx 512..32768"] = {
        "ms_per_step": round(ms, 4), "rows_s": round(wl.B / ms * 1e3, 1), "t_kv": t_kv,
        "fa_us": round(us, 3), "fa_algorithmic_bytes": int(fb), "fa_GBs": round(fb / (us * 1e-6) / 1e9, 1),
        "fa_frac": round(fb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del gw
    # MoE verify step
    log("8-layer MoE stack, verify rows")
    wl = W.workload("c5")
    gw = GpuWorkload(wl, fill="device")
    ms = _time_steps(gw, stream, iters, 3, repeat_first=True)
    res["8-layer MoE d=2816 128 experts top-8 + shared, Q4_0; 4 streams x 4 verify rows, ctx 8192"] = {
        "ms_per_step": round(ms, 4), "rows_s": round(wl.B / ms * 1e3, 1)}
    del gw
    # the headline stack with FP8 E4M3 caches, and its fa_decode
    log("32-layer Q4_0 stack, FP8 E4M3 KV caches")
    import dataclasses
    base = W.workload("c4", B=8, steps=iters + 8)
    wl = dataclasses.replace(base, spec=dataclasses.replace(base.spec, kv_fp8=True))
    gw = GpuWorkload(wl, fill="device")
    ms = _time_steps(gw, stream, iters, 3)
    sp = wl.spec
    t_kv = [p + 1 for p in wl.positions(0)]
    q = torch.randn((wl.B, sp.n_head, sp.head_dim), device="cuda",
                    generator=torch.Generator(device="cuda").manual_seed(3))
    kb = [gw.caches.k_ptr(wl.rows[b][0], 0) for b in range(wl.B)]
    vb = [gw.caches.v_ptr(wl.rows[b][0], 0) for b in range(wl.B)]
    ws = torch.zeros(kd.kd_fa_decode_workspace(wl.B, sp.n_head, sp.head_dim, t_kv), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    us = time_rotating(lambda i: kd.kd_fa_decode_ragged_fp8(q, sp.n_head_kv, kb, vb, t_kv, wl.capacity,
                                                           sp.head_dim ** -0.5, ws=ws, out=out, stream=stream),
                       iters, stream)
    fb = fa_algorithmic_bytes(t_kv, sp.n_head_kv, sp.n_head, sp.head_dim, kv_bytes=1)
    res["32-layer d=4096 32Q/8KV Q4_0, FP8 E4M3 KV caches, B=8 ctx 4096"] = {
        "tok_s": round(wl.B / ms * 1e3, 1), "ms_per_step": round(ms, 4), "t_kv": t_kv,
        "fa_us": round(us, 3), "fa_algorithmic_bytes": int(fb), "fa_GBs": round(fb / (us * 1e-6) / 1e9, 1),
        "fa_frac": round(fb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del gw
    # gated delta-rule state step of a linear-attention layer: B = 8 rows x 32 value heads
    log("gated delta-rule state step, B=8 x 32 heads")
    B, H, D, sets = 8, 32, 128, 8
    gen = torch.Generator(device="cuda").manual_seed(4)
    st_in = [[torch.randn((H, D, D), device="cuda", generator=gen) for _ in range(B)] for _ in range(sets)]
    st_out = [[torch.empty((H, D, D), device="cuda") for _ in range(B)] for _ in range(sets)]
    gq = torch.nn.functional.normalize(torch.randn((B, H, D), device="cuda", generator=gen), dim=2)
    gk = torch.nn.functional.normalize(torch.randn((B, H, D), device="cuda", generator=gen), dim=2)
    gv = torch.randn((B, H, D), device="cuda", generator=gen)
    gg = -torch.rand((B, H), device="cuda", generator=gen)
    gb = torch.rand((B, H), device="cuda", generator=gen)
    go = torch.empty_like(gv)
    us = time_rotating(lambda i: kd.kd_gdn_step(gq, gk, gv, gg, gb, [t.data_ptr() for t in st_in[i % sets]],
                                                [t.data_ptr() for t in st_out[i % sets]], D ** -0.5, o=go,
                                                stream=stream), iters, stream)
    gbytes = B * H * D * D * 4 * 2 + B * H * D * 4 * 4 + B * H * 8
    res["gated delta-rule state step (kd_gdn_step), B=8 rows x 32 value heads, d_state 128, fp32 state"] = {
        "us": round(us, 3), "algorithmic_bytes": int(gbytes), "GBs": round(gbytes / (us * 1e-6) / 1e9, 1),
        "frac": round(gbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del st_in, st_out
    torch.cuda.synchronize()
    return res


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--sweep", default="1,2,4,8,16", help="batch widths to time")
    ap.add_argument("--headline-b", type=int, default=8, help="width whose aggregate tok/s is `value`")
    ap.add_argument("--kernel-iters", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other", action="store_true", help="skip the other workloads (headline only)")
    ap.add_argument("--cpu-layers", type=int, default=16, help="layers of one step the oracle is timed on")
    ap.add_argument("--summarize-trace", default=None)
    ap.add_argument("--traffic-probe", action="store_true", help="launches for the PMC traffic passes only")
    ap.add_argument("--traffic-summarize", nargs=2, metavar=("FETCH", "WRITE"), default=None)
    ap.add_argument("--traffic-cmds", nargs=2, metavar=("FETCH_CMD", "WRITE_CMD"), default=("?", "?"))
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.traffic_summarize:
        traffic_summarize(*args.traffic_summarize, *args.traffic_cmds)
        return
    if args.traffic_probe:
        traffic_probe()
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
    log("packing weights and filling caches")
    gw = GpuWorkload(wl, fill="device")   # seeded N(0,1) fp16 KV drawn on the device (speed)
    setup_s = time.time() - t0
    # every launch goes to one dedicated stream (default priority), as a serving loop would
    # own one; the legacy null stream adds an implicit cross-stream barrier to each launch
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)

    # ---------------------------------------------------------------- whole steps
    sweep = {}
    for B in widths:
        log(f"whole steps at B={B}")
        rows = list(range(B))
        out = torch.empty((B, sp.out_dim), dtype=torch.float32, device="cuda")
        gw.prefetch(range(max(K, Wu)), rows)   # inputs resident in HBM before timing
        for s in range(Wu):
            gw.step(s, rows=rows, out=out, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_host = time.perf_counter()
        e0.record(stream)
        for s in range(K):
            gw.step(s, rows=rows, out=out, stream=stream)
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

    # ---------------------------------------------------------------- the largest product
    # the FFN's interleaved gate/up product (28672 x 4096 Q4_0) with its SwiGLU + quantiser
    # epilogue, at the headline width: 54% of the step's weight bytes.  Launches rotate over
    # the 32 layers' own matrices (2.1 GB, well above the 256 MB Infinity Cache), as inside
    # a step.
    B = Bh
    log(f"gate/up mmvq with SwiGLU epilogue at B={B}")
    mats = [gw.km.packed[il]["w_gateup"] for il in range(L)]
    xin = torch.randn((B, sp.d), device="cuda", generator=torch.Generator(device="cuda").manual_seed(0))
    act = kd.kd_quantize_act_q8(xin)
    h_act = kd.alloc_act(B, mats[0].n_out // 2)
    mm_us = time_rotating(lambda i: kd.kd_mmvq_swiglu(mats[i % L], act, B, h_act, stream=stream), args.kernel_iters,
                          stream)
    n, k = mats[0].n_out, mats[0].k
    mm_bytes = mmvq_algorithmic_bytes(n, k, B)
    mm_gbs = mm_bytes / (mm_us * 1e-6) / 1e9
    mm_traffic = load_traffic("mmvq") if (n, k, B) == (MM_N, MM_K, MM_B) else None

    # ---------------------------------------------------------------- dominant kernel: fa_decode
    # the split kernel and its combine: the largest share of the step's time (~40% at B = 8).
    # Calls rotate over the 32 layers' caches (135 MB of KV per call), as inside a step.
    log(f"fa_decode at B={B}")
    t_kv = [p + 1 for p in wl.positions(mid)[:B]]
    q = torch.randn((B, sp.n_head, hd), device="cuda", generator=torch.Generator(device="cuda").manual_seed(1))
    kbl = [[gw.caches.k_ptr(s, il) for s in range(B)] for il in range(L)]
    vbl = [[gw.caches.v_ptr(s, il) for s in range(B)] for il in range(L)]
    fa_ws = torch.empty(kd.kd_fa_decode_workspace(B, sp.n_head, hd, t_kv), dtype=torch.uint8, device="cuda")
    fa_out = torch.empty_like(q)
    fa_us = time_rotating(lambda i: kd.kd_fa_decode_ragged(q, G, kbl[i % L], vbl[i % L], t_kv, wl.capacity,
                                                           hd ** -0.5, ws=fa_ws, out=fa_out, stream=stream),
                          args.kernel_iters, stream)
    fa_bytes = fa_algorithmic_bytes(t_kv, G, sp.n_head, hd)
    fa_gbs = fa_bytes / (fa_us * 1e-6) / 1e9
    fa_traffic = load_traffic("fa") if t_kv == [FA_T] * FA_B else None

    other = None if args.no_other else other_workloads(stream, 20)

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
        log(f"cpu baseline: oracle over {nl} layers")
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
        "roofline": {"bound": "hbm", "achieved": round(fa_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(fa_gbs / HBM_PEAK_GBS, 4), "traffic": fa_traffic,
                     "kernel": "fa_decode: fa_split_kernel + fa_combine_kernel, B=%d, t_kv=%d" % (B, t_kv[0]),
                     "avg_launch_us": round(fa_us, 3), "algorithmic_bytes": int(fa_bytes)},
        "mmvq_roofline": {"bound": "hbm", "achieved": round(mm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(mm_gbs / HBM_PEAK_GBS, 4), "traffic": mm_traffic,
                          "kernel": "mmvq_kernel<Q4_0, SwiGLU epilogue> 28672x4096 (gate/up) at B=%d" % Bh,
                          "avg_launch_us": round(mm_us, 3), "algorithmic_bytes": int(mm_bytes)},
        "cpu_baseline": cpu,
        "other_workloads": other,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(res))


if __name__ == "__main__":
    main()

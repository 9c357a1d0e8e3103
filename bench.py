#!/usr/bin/env python3
"""Benchmark of the batched multi-session decode step on one MI355X.

Workload: the 32-layer dense decoder (d=4096, 32 Q / 8 KV heads, hd=128, SwiGLU 14336, Q4_0
weights, final RMSNorm), every session at ctx 4096 -- the weight-stream-bound case on which
the metric "aggregate decode tok/s at B=1..16" is quoted.  A step is one kd_decode_step over
B rows (all 32 layers + final norm).  K timed steps run at positions 4096..4096+K-1 after W
warm-up steps (the same positions are re-written, so caches hold the same bytes each pass).

Prints ONE JSON line with:
* ``value``: aggregate decode tok/s at B=8, and the B=1..16 sweep with step HBM GB/s;
* ``roofline``: fa_decode (the dominant kernel: split + combine) at B=8 rows of 4113 keys,
  timed with HIP events on the launch stream, its PMC traffic, and the plain read of the same
  bytes (kd_debug_read_stream) as the practical ceiling;
* ``products``: each product of the stack at B=8 with its fused epilogue (QKV + RoPE +
  append, O + residual + norm codes, gate/up + SwiGLU, down + residual + norm codes) and the
  8-layer Q8_0 stack's lm_head, each with algorithmic bytes, GB/s, PMC traffic and the plain
  read of its weight bytes (``mmvq_roofline`` repeats gate/up, the largest);
* ``other_workloads``: the 8-layer Q8_0 stack with lm_head at B=1..8, the ragged B=16
  attention sublayer and its fa_decode, the MoE verify step (with its bytes counted over the
  distinct experts its rows hit), the headline stack with FP8 E4M3 caches and with int8
  (Q8_0-row) caches and their fa_decode, the gated delta-rule state step;
* ``cpu_baseline`` (the 32-layer stack at B=8) and ``cpu_baseline_configs`` (all five
  workloads at their headline widths): the oracle on the host cores, bounded samples;
* ``platform``: GPU name, ROCm and HIP versions.

``--summarize-trace CSV`` prints per-(kernel, grid) average durations from a rocprofv3
kernel-trace CSV; ``--traffic-probe`` makes the launches of the two PMC passes and
``--traffic-summarize FETCH WRITE`` turns them into the profiles/traffic_*.txt records.
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


# ---------------------------------------------------------------------- algorithmic bytes
# The 32-layer Q4_0 stack's products at the headline width, with their fused epilogues, and
# the 8-layer Q8_0 stack's lm_head: what each launch must move (weights once, activations in,
# the epilogue's reads and writes), per launch.
FA_B, FA_T = 8, 4113      # fa_decode roofline case: B rows of t keys (ctx 4096 + 16 decode steps + 1)
PB = 8                    # product roofline width
D4, H4, G4, HD4, F4 = 4096, 32, 8, 128, 14336


def act_bytes(B: int, k: int) -> int:
    """B quantised activation rows of length k: int8 codes and fp32 block scales."""
    return B * k + B * (k // 32) * 4


def w_bytes(fmt: str, n: int, k: int) -> int:
    return n * k * (34 if fmt == "q8_0" else 18) // 32


PRODUCTS = {
    # kind: (title, fmt, n, k, epilogue bytes beyond the weights and the activation rows in)
    "qkv": ("QKV product + 1/rms + RoPE + fp16 K/V append (kd_mmvq_rope_normed), 6144x4096 Q4_0", "q4_0",
            (H4 + 2 * G4) * HD4, D4,
            lambda B: B * (D4 // 32) * 4 + B * H4 * HD4 * 4 + B * G4 * HD4 * 2 * 2),
    "o": ("O product + residual + FFN-norm codes and block sums (kd_mmvq_resnorm), 4096x4096 Q4_0", "q4_0",
          D4, H4 * HD4, lambda B: 3 * B * D4 * 4 + D4 * 4 + act_bytes(B, D4) + B * (D4 // 32) * 4),
    "gateup": ("gate/up product + 1/rms + SwiGLU + quantiser (kd_mmvq_swiglu_normed), 28672x4096 Q4_0", "q4_0",
               2 * F4, D4, lambda B: B * (D4 // 32) * 4 + act_bytes(B, F4)),
    "down": ("down product + residual + next attention-norm codes and block sums (kd_mmvq_resnorm), "
             "4096x14336 Q4_0", "q4_0", D4, F4,
             lambda B: 3 * B * D4 * 4 + D4 * 4 + act_bytes(B, D4) + B * (D4 // 32) * 4),
    "lm_head": ("lm_head product of the 8-layer stack (kd_mmvq_q8_0), 32000x2048 Q8_0", "q8_0", 32000, 2048,
                lambda B: B * 32000 * 4),
}


def product_bytes(kind: str, B: int) -> int:
    _, fmt, n, k, epi = PRODUCTS[kind]
    return w_bytes(fmt, n, k) + act_bytes(B, k) + epi(B)


def fa_algorithmic_bytes(t_kv, G: int, H: int, hd: int, kv_bytes: int = 2) -> int:
    """fa_decode: each row's K and V (fp16, or 1-byte E4M3 codes) once, q in and the output
    out (fp32)."""
    return sum(t_kv) * G * hd * kv_bytes * 2 + 2 * len(t_kv) * H * hd * 4


# ---------------------------------------------------------------------- HBM traffic (PMC)
CALIB_BYTES = 512 << 20
MM_SRC = ("session_decode_step_amd/csrc/mmvq.hip", "session_decode_step_amd/csrc/mmvq_impl.h",
          "session_decode_step_amd/csrc/kd_internal.h")
FA_SRC = ("session_decode_step_amd/csrc/attn.hip", "session_decode_step_amd/csrc/kd_internal.h")
# in the order the probe launches them: (kind, profile file stem, sources, kernels per call)
TRAFFIC_ORDER = [
    ("fa", "traffic_fa_decode_b8_t4113", FA_SRC, ("fa_split_kernel", "fa_combine_kernel")),
    ("qkv", "traffic_mmvq_qkv_rope_q4_0_6144x4096_b8", MM_SRC, ("mmvq_kernel",)),
    ("o", "traffic_mmvq_o_resnorm_q4_0_4096x4096_b8", MM_SRC, ("mmvq_kernel",)),
    ("gateup", "traffic_mmvq_gateup_swiglu_q4_0_28672x4096_b8", MM_SRC, ("mmvq_kernel",)),
    ("down", "traffic_mmvq_down_resnorm_q4_0_4096x14336_b8", MM_SRC, ("mmvq_kernel",)),
    ("lm_head", "traffic_mmvq_lm_head_q8_0_32000x2048_b8", MM_SRC, ("mmvq_kernel",)),
]
PROBE_CALLS = 8


def _traffic_spec(kind):
    for k, stem, src, kernels in TRAFFIC_ORDER:
        if k == kind:
            return stem, src, kernels
    raise KeyError(kind)


def _traffic_title_bytes(kind):
    if kind == "fa":
        return (f"fa_decode (fa_split_kernel + fa_combine_kernel), B={FA_B} rows of t={FA_T} keys, H=32, G=8, hd=128",
                fa_algorithmic_bytes([FA_T] * FA_B, G4, H4, HD4))
    return f"mmvq_kernel: {PRODUCTS[kind][0]}, B={PB}", product_bytes(kind, PB)


def kernel_source_hash(kind: str) -> str:
    """Hash of the code (comments and whitespace removed) of the files a kernel is built from:
    a measurement stays attached to its kernel until the code changes."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in _traffic_spec(kind)[1]:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


class ProductRig:
    """Device inputs of the measured products at width B: each product's activation rows,
    the split-RMSNorm sums, residual rows, gains and output buffers (everything a launch
    reads or writes besides its matrix)."""

    def __init__(self, B: int, caches_k, caches_v, pos: int, capacity: int):
        import torch
        import session_decode_step_amd as kd
        g = torch.Generator(device="cuda").manual_seed(7)
        self.B = B
        self.x_d = kd.kd_quantize_act_q8(torch.randn((B, D4), device="cuda", generator=g))
        self.x_f = kd.kd_quantize_act_q8(torch.randn((B, F4), device="cuda", generator=g))
        self.x_lm = kd.kd_quantize_act_q8(torch.randn((B, 2048), device="cuda", generator=g))
        self.res = torch.randn((B, D4), device="cuda", generator=g)
        self.gain = 1 + 0.1 * torch.randn(D4, device="cuda", generator=g)
        self.x1 = torch.empty_like(self.res)
        self.out_d = kd.alloc_act(B, D4)
        self.ss = (self.res * self.res).view(B, D4 // 32, 32).sum(2).contiguous()
        self.h = kd.alloc_act(B, F4)
        self.q = torch.empty((B, H4 * HD4), device="cuda")
        self.y_lm = torch.empty((B, 32000), device="cuda")
        self.kb, self.vb, self.pos, self.cap = caches_k, caches_v, [pos] * B, capacity

    def launch(self, kind: str, W, stream=None):
        import session_decode_step_amd as kd
        B = self.B
        if kind == "qkv":
            kd.kd_mmvq_rope_normed(W, self.x_d, B, self.ss, 1e-5, H4, G4, HD4, self.q, self.kb, self.vb, self.pos,
                                   self.cap, 10000.0, stream=stream)
        elif kind == "o":
            kd.kd_mmvq_resnorm(W, self.x_d, B, self.res, self.gain, self.x1, self.out_d, self.ss, stream=stream)
        elif kind == "gateup":
            kd.kd_mmvq_swiglu_normed(W, self.x_d, B, self.ss, 1e-5, self.h, stream=stream)
        elif kind == "down":
            kd.kd_mmvq_resnorm(W, self.x_f, B, self.res, self.gain, self.x1, self.out_d, self.ss, stream=stream)
        else:
            kd.kd_mmvq_q8_0(W, self.x_lm, B, self.y_lm, stream=stream)


def lm_head_copies(n: int = 4):
    """n independently drawn 32000x2048 Q8_0 matrices (more than the 256 MB Infinity Cache
    holds together), packed: the lm_head launches rotate over them."""
    import workload as W
    import session_decode_step_amd as kd
    return [kd.kd_pack_weight(W.draw_weight("q8_0", 0, 2, 27, 28, 100 + i, 32000, 2048)) for i in range(n)]


def stack_products(gw):
    """The 32-layer stack's own packed matrices per product kind (one per layer)."""
    L = gw.wl.spec.n_layers
    return {"qkv": [gw.km.packed[il]["wqkv"] for il in range(L)], "o": [gw.km.packed[il]["wo"] for il in range(L)],
            "gateup": [gw.km.packed[il]["w_gateup"] for il in range(L)],
            "down": [gw.km.packed[il]["w_down"] for il in range(L)]}


def traffic_probe() -> None:
    """Launches for the two ``rocprofv3 --pmc`` passes: every input is prepared first; then a
    plain fp32 elementwise copy of 512 MiB (the calibration kernel: reads and writes 512 MiB),
    then, in TRAFFIC_ORDER, 8 fa_decode calls at B=8 (t=4113) over four layers' caches and 8
    launches of each product at B=8 over four layers' matrices (the lm_head over four drawn
    matrices)."""
    import dataclasses
    import torch
    import workload as W
    import session_decode_step_amd as kd
    from session_decode_step_amd.runner import GpuWorkload
    torch.cuda.set_device(0)
    base = W.workload("c4", B=FA_B, steps=32)
    wl = dataclasses.replace(base, spec=dataclasses.replace(base.spec, n_layers=4))
    gw = GpuWorkload(wl, fill="device")
    mats = stack_products(gw)
    mats["lm_head"] = lm_head_copies(4)
    rig = ProductRig(PB, [gw.caches.k_ptr(s, 0) for s in range(PB)], [gw.caches.v_ptr(s, 0) for s in range(PB)],
                     wl.capacity - 1, wl.capacity)
    t_kv = [FA_T] * FA_B
    q = torch.randn((FA_B, H4, HD4), device="cuda")
    ws = torch.empty(kd.kd_fa_decode_workspace(FA_B, H4, HD4, t_kv), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    kbl = [[gw.caches.k_ptr(s, il) for s in range(FA_B)] for il in range(4)]
    vbl = [[gw.caches.v_ptr(s, il) for s in range(FA_B)] for il in range(4)]
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(2):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst
    for kind, _, _, _ in TRAFFIC_ORDER:
        for i in range(PROBE_CALLS):
            if kind == "fa":
                kd.kd_fa_decode_ragged(q, G4, kbl[i % 4], vbl[i % 4], t_kv, wl.capacity, HD4 ** -0.5, ws=ws, out=out)
            else:
                rig.launch(kind, mats[kind][i % 4])
        torch.cuda.synchronize()
    log("traffic probe done")


def _read_counters(path: str):
    """[(dispatch, kernel_name, counter_value)] in dispatch order from a rocprofv3
    counter_collection CSV (or the directory holding it)."""
    import csv
    import glob
    if os.path.isdir(path):
        hits = glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
        if not hits:
            raise SystemExit(f"no counter_collection.csv under {path}")
        path = max(hits, key=os.path.getmtime)   # the latest pass written there
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
    """HBM bytes per launch of each measured kernel from the FETCH_SIZE and WRITE_SIZE passes
    (KiB per dispatch), each scaled by what the counter reads for the 512 MiB calibration
    copy; writes one profile summary per kernel, which the bench reads back.  The dispatches
    after the calibration are taken in the probe's order, PROBE_CALLS calls per kind (a call
    of fa_decode is its split and its combine; each kernel's mean counts once)."""
    rows = {tag: _read_counters(path) for tag, path in (("fetch", fetch), ("write", write))}
    factor, calib_kib, seqs = {}, {}, {}
    for tag, rr in rows.items():
        idx = [i for i, (_, nm, _) in enumerate(rr) if "MulFunctor" in nm]
        if not idx:
            raise SystemExit(f"{tag}: calibration dispatch missing")
        calib = max(rr[i][2] for i in idx)
        calib_kib[tag], factor[tag] = calib, CALIB_BYTES / (calib * 1024.0)
        seqs[tag] = [(nm, v) for _, nm, v in rr[idx[-1] + 1:] if "kd::" in nm]
    per = {tag: {} for tag in rows}
    for tag, seq in seqs.items():
        pos = 0
        for kind, _, _, kernels in TRAFFIC_ORDER:
            vals = {kn: [] for kn in kernels}
            for _ in range(PROBE_CALLS):
                for kn in kernels:
                    nm, v = seq[pos]
                    if kn not in nm:
                        raise SystemExit(f"{tag}: dispatch {pos} is {nm[:60]}, expected {kn} ({kind})")
                    vals[kn].append(v)
                    pos += 1
            per[tag][kind] = vals
    for kind, stem, _, kernels in TRAFFIC_ORDER:
        title, alg = _traffic_title_bytes(kind)
        byts = {tag: sum(sum(v) / len(v) for v in per[tag][kind].values()) * 1024.0 * factor[tag] for tag in per}
        total = byts["fetch"] + byts["write"]
        rec = {"kernel": title, "source_hash": kernel_source_hash(kind),
               "fetch_bytes": round(byts["fetch"]), "write_bytes": round(byts["write"]),
               "traffic_bytes": round(total), "algorithmic_bytes": alg,
               "traffic_over_algorithmic": round(total / alg, 4),
               "fetch_factor": round(factor["fetch"], 5), "write_factor": round(factor["write"], 5)}
        lines = [
            f"HBM traffic of {title} (rocprofv3 PMC, MI355X)",
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
            for kn, vals in per[tag][kind].items():
                lines.append(f"{kn} dispatches {tag.upper()}_SIZE KiB: {', '.join(f'{v:.0f}' for v in vals)}")
        lines += [
            f"per launch: fetch {rec['fetch_bytes']} B + write {rec['write_bytes']} B = {rec['traffic_bytes']} B; "
            f"algorithmic {alg} B; ratio {rec['traffic_over_algorithmic']}",
            "",
            "TRAFFIC_JSON " + json.dumps(rec),
        ]
        path = os.path.join(ROOT, "profiles", stem + ".txt")
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        print("\n".join(lines) + "\n")


def load_traffic(kind: str):
    """Measured HBM bytes per launch of a kernel, or None when no measurement exists or the
    kernel source has changed since it was taken."""
    path = os.path.join(ROOT, "profiles", _traffic_spec(kind)[0] + ".txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("TRAFFIC_JSON "):
            rec = json.loads(line[len("TRAFFIC_JSON "):])
            if rec.get("source_hash") == kernel_source_hash(kind):
                return rec["traffic_bytes"]
    return None


def read_ceiling_us(tensors, nbytes: int, stream, iters: int) -> float:
    """The plain read of ``nbytes`` of each tensor in turn (rotating, as the measured kernel
    rotates over its matrices): average us per read."""
    import torch
    import session_decode_step_amd as kd
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    return time_rotating(lambda i: kd.kd_debug_read_stream(tensors[i % len(tensors)], sink, nbytes, stream=stream),
                         iters, stream)


def tp8_shard(gw, stream, iters: int) -> dict:
    """One GPU's share of a C4 layer under 8-way tensor parallelism, at B=8 (what one GPU can
    show of that layout; the two [B, d] all-reduces per layer are not run): QKV rows of 4 query
    heads and 1 KV head (768 x 4096, RoPE + append epilogue), 1792 gate/up outputs (3584 x 4096,
    SwiGLU epilogue), O over 512 input columns (4096 x 512) and down over 1792 (4096 x 1792) as
    plain products (their partial sums go to the all-reduce), and fa_decode over 1 KV head
    (H = 4, G = 1, t = 4113).  Row shards are views of each layer's packed matrix (its leading
    tiles); column shards are the leading quads of every row group, copied once."""
    import torch
    import session_decode_step_amd as kd
    from session_decode_step_amd import PackedWeight
    wl = gw.wl
    L = wl.spec.n_layers
    mats = stack_products(gw)

    def tiles(W):
        nr, nq = W.n_out // 16, W.k // 128
        return nr, nq, W.qs.numel() // (nr * nq), W.d.numel() // (nr * nq)

    def rows(W, n):
        _, nq, tq, td = tiles(W)
        return PackedWeight(W.fmt, n, W.k, W.qs[: (n // 16) * nq * tq], W.d[: (n // 16) * nq * td])

    def cols(W, k):
        nr, nq, tq, td = tiles(W)
        nqs = k // 128
        return PackedWeight(W.fmt, W.n_out, k, W.qs.view(nr, nq, tq)[:, :nqs].contiguous().view(-1),
                            W.d.view(nr, nq, td)[:, :nqs].contiguous().view(-1))

    qkv = [rows(m, 768) for m in mats["qkv"]]
    gu = [rows(m, 3584) for m in mats["gateup"]]
    o = [cols(m, 512) for m in mats["o"]]
    down = [cols(m, 1792) for m in mats["down"]]
    g = torch.Generator(device="cuda").manual_seed(11)
    B = PB
    x_d = kd.kd_quantize_act_q8(torch.randn((B, D4), device="cuda", generator=g))
    x_o = kd.kd_quantize_act_q8(torch.randn((B, 512), device="cuda", generator=g))
    x_dn = kd.kd_quantize_act_q8(torch.randn((B, 1792), device="cuda", generator=g))
    res = torch.randn((B, D4), device="cuda", generator=g)
    ss = (res * res).view(B, D4 // 32, 32).sum(2).contiguous()
    qo = torch.empty((B, 4 * HD4), device="cuda")
    h = kd.alloc_act(B, 1792)
    y = torch.empty((B, D4), device="cuda")
    pos = [wl.capacity - 1] * B
    kb = [[gw.caches.k_ptr(s, il) for s in range(B)] for il in range(L)]
    vb = [[gw.caches.v_ptr(s, il) for s in range(B)] for il in range(L)]
    t_kv = [FA_T] * B
    q = torch.randn((B, 4, HD4), device="cuda", generator=g)
    fa_out = torch.empty_like(q)
    fa_ws = torch.empty(kd.kd_fa_decode_workspace(B, 4, HD4, t_kv), dtype=torch.uint8, device="cuda")
    launches = {
        "qkv 768x4096 + RoPE + append": lambda i: kd.kd_mmvq_rope_normed(
            qkv[i % L], x_d, B, ss, 1e-5, 4, 1, HD4, qo, kb[i % L], vb[i % L], pos, wl.capacity, 10000.0, stream=stream),
        "fa_decode H=4 G=1 t=4113": lambda i: kd.kd_fa_decode_ragged(
            q, 1, kb[i % L], vb[i % L], t_kv, wl.capacity, HD4 ** -0.5, ws=fa_ws, out=fa_out, stream=stream),
        "o 4096x512": lambda i: kd.kd_mmvq_q4_0(o[i % L], x_o, B, y, stream=stream),
        "gate/up 3584x4096 + SwiGLU": lambda i: kd.kd_mmvq_swiglu_normed(gu[i % L], x_d, B, ss, 1e-5, h, stream=stream),
        "down 4096x1792": lambda i: kd.kd_mmvq_q4_0(down[i % L], x_dn, B, y, stream=stream),
    }
    out = {}
    for name, fn in launches.items():
        out[name] = round(time_rotating(fn, iters, stream), 3)
    out["sum_us"] = round(sum(v for v in out.values()), 3)
    out["note"] = "per-layer kernels of one TP8 shard at B=8 (us; the two all-reduces per layer not run)"
    return out


def measure_products(gw, stream, iters: int) -> dict:
    """Each product of the 32-layer stack at B=8 with its fused epilogue (HIP events on the
    launch stream, rotating over the 32 layers' matrices), the 8-layer stack's lm_head
    (rotating over four drawn matrices), and the plain read of the same weight bytes."""
    mats = stack_products(gw)
    mats["lm_head"] = lm_head_copies(4)
    wl = gw.wl
    rig = ProductRig(PB, [gw.caches.k_ptr(s, 0) for s in range(PB)], [gw.caches.v_ptr(s, 0) for s in range(PB)],
                     wl.capacity - 1, wl.capacity)
    res = {}
    for kind in PRODUCTS:
        log(f"product {kind} at B={PB}")
        Ms = mats[kind]
        us = time_rotating(lambda i: rig.launch(kind, Ms[i % len(Ms)], stream=stream), iters, stream)
        alg = product_bytes(kind, PB)
        wb = w_bytes(PRODUCTS[kind][1], PRODUCTS[kind][2], PRODUCTS[kind][3])
        rd = read_ceiling_us([m.qs for m in Ms], Ms[0].qs.numel(), stream, iters)
        gbs = alg / (us * 1e-6) / 1e9
        res[kind] = {"kernel": PRODUCTS[kind][0], "bound": "hbm", "avg_launch_us": round(us, 3),
                     "algorithmic_bytes": int(alg), "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": load_traffic(kind),
                     "read_ceiling_us": round(rd, 3), "read_ceiling_GBs": round(wb / (rd * 1e-6) / 1e9, 1),
                     "frac_of_read_ceiling": round(rd / us, 4)}
    return res


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
    ctx 8192); the headline stack with FP8 E4M3 caches and its fa_decode, and with int8
    caches; the gated delta-rule state step at B = 8 x 32 heads; the 8-layer stack with
    K-quant weights and plain K-quant products; the 8-layer stack with gated delta-rule
    layers."""
    import numpy as np
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
    wb2 = W.algorithmic_bytes_weights(wl.spec)
    for B in (1, 2, 4, 8):
        ms = _time_steps(gw, stream, 16, 3, rows=list(range(B)))
        # weights once, each row's keys (ctx 1238 + the 16 timed steps' mean position) once
        kvb = B * (1238 + 8 + 1) * wl.spec.n_layers * wl.spec.n_head_kv * wl.spec.head_dim * 2 * 2
        dense[str(B)] = {"tok_s": round(B / ms * 1e3, 1), "ms_per_step": round(ms, 4),
                         "step_GBs": round((wb2 + kvb) / (ms * 1e-3) / 1e9, 1)}
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
    sb = W.algorithmic_bytes_weights(sp) + fb
    res["attention sublayer d=4096 32Q/8KV hd=128 Q8_0, B=16 ragged ctx 512..32768"] = {
        "ms_per_step": round(ms, 4), "rows_s": round(wl.B / ms * 1e3, 1), "t_kv": t_kv,
        "step_GBs": round(sb / (ms * 1e-3) / 1e9, 1),
        "fa_us": round(us, 3), "fa_algorithmic_bytes": int(fb), "fa_GBs": round(fb / (us * 1e-6) / 1e9, 1),
        "fa_frac": round(fb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    del gw
    # MoE verify step
    log("8-layer MoE stack, verify rows")
    wl = W.workload("c5")
    gw = GpuWorkload(wl, fill="device")
    ms = _time_steps(gw, stream, iters, 3, repeat_first=True)
    # algorithmic bytes of the step with experts merged across rows: each layer's attention
    # weights, router and shared expert, the distinct experts its 16 rows are routed to (read
    # once however many rows share one), and each stream's keys once (its 4 rows share a pass)
    sp = wl.spec
    ids = gw.step_trace(0)["moe_ids"]                      # [layers, rows, top-k]
    distinct = [len(np.unique(ids[il])) for il in range(sp.n_layers)]
    e_bytes = w_bytes("q4_0", 2 * sp.expert_ffn, sp.d) + w_bytes("q4_0", sp.d, sp.expert_ffn)
    attn_w = w_bytes("q4_0", (2 * sp.n_head_kv + sp.n_head) * sp.head_dim, sp.d) + \
        w_bytes("q4_0", sp.d, sp.n_head * sp.head_dim)
    shared = w_bytes("q4_0", 2 * sp.shared_ffn, sp.d) + w_bytes("q4_0", sp.d, sp.shared_ffn)
    router = sp.n_experts * sp.d * 4
    t_stream = [max(p + 1 for (st, _), p in zip(wl.rows, wl.positions(0)) if st == s) for s in range(len(wl.prefill))]
    kv_merged = sum(t_stream) * sp.n_head_kv * sp.head_dim * 2 * 2
    kv_rows = sum(p + 1 for p in wl.positions(0)) * sp.n_head_kv * sp.head_dim * 2 * 2
    merged = sum(attn_w + router + shared + n * e_bytes + kv_merged for n in distinct)
    per_row = sp.n_layers * (attn_w + router + shared + wl.B * sp.n_expert_used * e_bytes + kv_rows)
    res["8-layer MoE d=2816 128 experts top-8 + shared, Q4_0; 4 streams x 4 verify rows, ctx 8192"] = {
        "ms_per_step": round(ms, 4), "rows_s": round(wl.B / ms * 1e3, 1),
        "distinct_experts_per_layer": distinct, "expert_bytes": int(e_bytes),
        "step_algorithmic_bytes_merged": int(merged), "step_GBs_merged": round(merged / (ms * 1e-3) / 1e9, 1),
        "step_frac_of_peak": round(merged / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_bytes_if_each_row_read_its_experts_and_keys": int(per_row)}
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
    # the headline stack with int8 caches (Q8_0 rows), and its fa_decode
    log("32-layer Q4_0 stack, int8 KV caches")
    wl = dataclasses.replace(base, spec=dataclasses.replace(base.spec, kv_q8=True))
    gw = GpuWorkload(wl, fill="device")
    ms = _time_steps(gw, stream, iters, 3)
    sp = wl.spec
    t_kv = [p + 1 for p in wl.positions(0)]
    kb = [gw.caches.k_ptr(wl.rows[b][0], 0) for b in range(wl.B)]
    vb = [gw.caches.v_ptr(wl.rows[b][0], 0) for b in range(wl.B)]
    ws = torch.zeros(kd.kd_fa_decode_workspace(wl.B, sp.n_head, sp.head_dim, t_kv), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    us = time_rotating(lambda i: kd.kd_fa_decode_ragged_q8(q, sp.n_head_kv, kb, vb, t_kv, wl.capacity,
                                                          sp.head_dim ** -0.5, ws=ws, out=out, stream=stream),
                       iters, stream)
    fb = sum(t_kv) * sp.n_head_kv * (sp.head_dim + 16) * 2 + 2 * wl.B * sp.n_head * sp.head_dim * 4
    res["32-layer d=4096 32Q/8KV Q4_0, int8 (Q8_0-row) KV caches, B=8 ctx 4096"] = {
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
    # the 8-layer stack with K-quant weights (Q5_K QKV, Q4_K O and gate/up, Q6_K down and
    # lm_head) at ctx 1238, and plain K-quant products at the 32-layer stack's shapes, B = 8
    log("8-layer K-quant stack with lm_head")
    wl = W.workload("kq", B=8, steps=64)
    gw = GpuWorkload(wl, fill="device")
    wb = W.algorithmic_bytes_weights(wl.spec)
    kq = {}
    for B in (1, 8):
        ms = _time_steps(gw, stream, 16, 3, rows=list(range(B)))
        kvb = B * (1238 + 8) * wl.spec.n_layers * wl.spec.n_head_kv * wl.spec.head_dim * 2 * 2
        kq[str(B)] = {"tok_s": round(B / ms * 1e3, 1), "ms_per_step": round(ms, 4),
                      "step_GBs": round((wb + kvb) / (ms * 1e-3) / 1e9, 1)}
    res["8-layer d=2048 decoder with Q4_K / Q5_K / Q6_K weights + lm_head 32000 (Q6_K), ctx 1238"] = kq
    del gw
    x8 = kd.kd_quantize_act_q8(torch.randn((8, 14336), device="cuda", generator=torch.Generator(device="cuda").manual_seed(5)))
    x4 = kd.kd_quantize_act_q8(torch.randn((8, 4096), device="cuda", generator=torch.Generator(device="cuda").manual_seed(6)))
    prods = {}
    for fmt, n, k, x in (("q4_k", 28672, 4096, x4), ("q5_k", 6144, 4096, x4), ("q6_k", 4096, 14336, x8),
                         ("q4_0", 28672, 4096, x4)):
        copies = 8 if n * k < 64 << 20 else 4
        Ms = [kd.kd_pack_weight(W.draw_weight(fmt, 0, 7, 50, 51, 200 + i, n, k)) for i in range(copies)]
        y = torch.empty((8, n), device="cuda")
        us = time_rotating(lambda i: kd.kd_mmvq(Ms[i % copies], x, 8, y, stream=stream), iters, stream)
        rec = W.KQ_RECORD.get(fmt)
        wbytes = n * (k // 256) * rec if rec else w_bytes(fmt, n, k)
        alg = wbytes + act_bytes(8, k) + 8 * n * 4
        prods[f"{fmt} {n}x{k}"] = {"us": round(us, 3), "algorithmic_bytes": int(alg),
                                   "GBs": round(alg / (us * 1e-6) / 1e9, 1),
                                   "frac": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        del Ms
    res["plain mmvq (kd_mmvq) at B=8, K-quant records against Q4_0, rotating over drawn matrices"] = prods
    # the 8-layer Q8_0 stack with gated delta-rule layers on layers 0-2 and 4-6, ctx 1238
    log("8-layer hybrid stack (gated delta-rule layers)")
    wl = W.workload("hybrid", B=8, steps=64)
    gw = GpuWorkload(wl, fill="device")
    hy = {}
    for B in (1, 8):
        ms = _time_steps(gw, stream, 16, 3, rows=list(range(B)))
        hy[str(B)] = {"tok_s": round(B / ms * 1e3, 1), "ms_per_step": round(ms, 4)}
    res["8-layer d=2048 Q8_0 decoder, gated delta-rule layers 0-2 and 4-6 (16 value heads of 128), "
        "attention layers 3 and 7, lm_head 32000, ctx 1238"] = hy
    del gw
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
    ap.add_argument("--cpu-layers", type=int, default=8,
                    help="layers of one step of the 32-layer stack the oracle is timed on")
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

    # ---------------------------------------------------------------- the step as a HIP graph
    # one step (positions of step 0, so every replay rewrites the same cache slots) captured
    # whole and replayed K times, against the same step enqueued K times
    log(f"step captured in a HIP graph at B={Bh}")
    rows = list(range(Bh))
    gw.prefetch([0], rows)
    out_g = torch.empty((Bh, sp.out_dim), dtype=torch.float32, device="cuda")
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        gw.step(0, rows=rows, out=out_g)
    torch.cuda.synchronize()

    def _timed(fn):
        for _ in range(Wu):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    graph_ms = _timed(graph.replay)
    eager_ms = _timed(lambda: gw.step(0, rows=rows, out=out_g, stream=stream))
    graph_rec = {"B": Bh, "ms_per_step_graph": round(graph_ms, 4), "ms_per_step_enqueued": round(eager_ms, 4)}
    del graph

    # algorithmic bytes of one step at width B (weights once + KV read + KV write + acts)
    wbytes = W.algorithmic_bytes_weights(sp)
    G, hd, L = sp.n_head_kv, sp.head_dim, sp.n_layers

    def step_bytes(B, s):
        kv = sum((p + 1) * G * hd * 2 * 2 for p in wl.positions(s)[:B]) * L
        return wbytes + kv + B * G * hd * 4 * L

    mid = K // 2
    for B in widths:
        sweep[B]["step_GBs"] = step_bytes(B, mid) / (sweep[B]["ms_per_step"] / 1e3) / 1e9

    # ---------------------------------------------------------------- the products
    # each product of the stack with its fused epilogue at B=8, rotating over the 32 layers'
    # own matrices (2.1 GB for gate/up, well above the 256 MB Infinity Cache), as inside a
    # step; the lm_head of the 8-layer Q8_0 stack; and the plain read of the same bytes
    products = measure_products(gw, stream, args.kernel_iters)
    log("one TP8 shard of a layer at B=8")
    shard = tp8_shard(gw, stream, args.kernel_iters)

    # ---------------------------------------------------------------- dominant kernel: fa_decode
    # the split kernel and its combine: the largest share of the step's time (~40% at B = 8).
    # B=8 rows of 4113 keys (ctx 4096 after 16 decode steps + this one), whatever --steps is;
    # calls rotate over the 32 layers' caches (135 MB of KV per call), as inside a step.
    log(f"fa_decode at B={FA_B}, t={FA_T}")
    t_kv = [FA_T] * FA_B
    q = torch.randn((FA_B, sp.n_head, hd), device="cuda", generator=torch.Generator(device="cuda").manual_seed(1))
    kbl = [[gw.caches.k_ptr(s, il) for s in range(FA_B)] for il in range(L)]
    vbl = [[gw.caches.v_ptr(s, il) for s in range(FA_B)] for il in range(L)]
    fa_ws = torch.empty(kd.kd_fa_decode_workspace(FA_B, sp.n_head, hd, t_kv), dtype=torch.uint8, device="cuda")
    fa_out = torch.empty_like(q)
    fa_us = time_rotating(lambda i: kd.kd_fa_decode_ragged(q, G, kbl[i % L], vbl[i % L], t_kv, wl.capacity,
                                                           hd ** -0.5, ws=fa_ws, out=fa_out, stream=stream),
                          args.kernel_iters, stream)
    fa_bytes = fa_algorithmic_bytes(t_kv, G, sp.n_head, hd)
    fa_gbs = fa_bytes / (fa_us * 1e-6) / 1e9
    # the plain read of as many bytes (one launch over a contiguous range of a session's cache
    # tensor, rotating over sessions): the practical ceiling of this call
    rd_bytes = sum(t_kv) * G * hd * 2 * 2
    rd_us = read_ceiling_us([gw.caches.t[s] for s in range(FA_B)], rd_bytes, stream, args.kernel_iters)
    other = None if args.no_other else other_workloads(stream, 20)

    # ---------------------------------------------------------------- CPU oracle baselines
    cpu, cpu_configs = None, None
    if not args.no_cpu_baseline:
        cpu, cpu_configs = cpu_baselines(gw, Bh, args.cpu_layers)

    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        rocm = "?"
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
        "platform": {"gpu": torch.cuda.get_device_name(0),
                     "arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", "?"),
                     "cus": torch.cuda.get_device_properties(0).multi_processor_count, "rocm": rocm, "hip": torch.version.hip,
                     "torch": torch.__version__, "seed": 0},
        "sweep": {str(b): {kk: round(v, 3) for kk, v in sweep[b].items()} for b in widths},
        "step_GBs": round(top["step_GBs"], 1),
        "step_frac_of_peak": round(top["step_GBs"] / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(fa_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(fa_gbs / HBM_PEAK_GBS, 4), "traffic": load_traffic("fa"),
                     "kernel": "fa_decode: fa_split_kernel + fa_combine_kernel, B=%d, t_kv=%d" % (FA_B, FA_T),
                     "avg_launch_us": round(fa_us, 3), "algorithmic_bytes": int(fa_bytes),
                     "read_ceiling_us": round(rd_us, 3), "read_ceiling_GBs": round(rd_bytes / (rd_us * 1e-6) / 1e9, 1),
                     "frac_of_read_ceiling": round(rd_us / fa_us, 4)},
        "mmvq_roofline": products["gateup"],
        "products": products,
        "cpu_baseline": cpu,
        "cpu_baseline_configs": cpu_configs,
        "other_workloads": other,
        "graph_replay": graph_rec,
        "tp8_shard": shard,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(res))


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        return (max([i.get("num_threads", 1) for i in info] or [1]),
                ",".join(sorted({i.get("internal_api", "?") for i in info})))
    except Exception:
        return os.cpu_count(), "?"


def oracle_sample(name: str, model, wl, B: int, nl: int) -> dict:
    """The oracle on the host cores: the first ``nl`` layers and the output head of one step
    of ``wl``'s first B rows (its own seeded KV), the layer time scaled to the whole stack."""
    import numpy as np
    import oracle
    import workload as W
    threads, blas = _blas_threads()
    sp = wl.spec
    nl = min(nl, sp.n_layers)
    rows = list(range(B))
    sess = [wl.rows[b][0] for b in rows]
    oc = oracle.OracleCaches(wl, sessions=sorted(set(sess)), layers=range(nl))
    x = W.step_inputs(wl, 0)[rows].astype(np.float64)
    pos = wl.positions(0)[:B]
    t0 = time.perf_counter()
    for il in range(nl):
        x = oracle.decode_layer(model, il, oc, x, sess, pos)
    t1 = time.perf_counter()
    oracle.output_head(model, x)
    t2 = time.perf_counter()
    step_s = (t1 - t0) * sp.n_layers / nl + (t2 - t1)
    return {"value": round(B / step_s, 4), "unit": "rows/s" if name == "c5" else "tok/s", "cores": int(threads),
            "kind": "oracle", "B": B,
            "sample": f"{nl} of {sp.n_layers} layers + output head of one step (fp64 numpy, {blas} BLAS), "
                      f"layer time scaled by {sp.n_layers}/{nl}: {step_s:.2f} s per full step"}


def cpu_baselines(gw, Bh: int, c4_layers: int):
    """The oracle timed on the host cores on a bounded sample of each workload at its
    headline width: the 32-layer Q4_0 stack at B=8 (``cpu_baseline``, the bench's own
    workload) and the five workloads (single layer B=2; 8-layer Q8_0 + lm_head B=8; ragged
    attention sublayer B=16; 32-layer Q4_0 B=8; MoE verify rows B=16)."""
    import workload as W
    out = {}
    c4 = oracle_sample("c4", gw.model, W.workload("c4", B=Bh, steps=1), Bh, c4_layers)
    log("cpu baseline: c4 done")
    for name, B, nl in (("c1", 2, 1), ("c2", 8, 2), ("c3", 16, 1), ("c5", 16, 1)):
        wl = W.workload(name, B=B) if name != "c1" else W.workload("c1")
        model = W.make_model(wl.spec, wl.code, wl.seed)
        out[name] = oracle_sample(name, model, wl, B, nl)
        del model
        log(f"cpu baseline: {name} done")
    out["c4"] = c4
    return c4, {k: out[k] for k in ("c1", "c2", "c3", "c4", "c5")}


if __name__ == "__main__":
    main()

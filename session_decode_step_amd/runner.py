"""Device-side set-up of a synthetic decode workload: packed weights, per-session fp16 KV
caches holding the seeded prefill, and a ``step()`` that calls ``kd_decode_step``.

Marshalling only (uploads, pointer tables, buffer sizes); the step itself runs in libkd.
The seeded inputs come from the ``workload`` module, which holds no arithmetic of the step.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import workload as W

from . import KdModel, SessionCaches


class GpuWorkload:
    def __init__(self, wl: W.Workload, model: Optional[Dict] = None, device: str = "cuda",
                 fill: str = "seeded", sessions: Optional[Sequence[int]] = None, fused: bool = True):
        """``fill="seeded"``: KV prefill from the workload generator; ``fill="device"``: a
        seeded torch device generator (for GPU-only comparisons at large shapes)."""
        self.wl = wl
        sp = wl.spec
        self.model = model if model is not None else W.make_model(sp, wl.code, wl.seed)
        self.km = KdModel(self.model, device, fused=fused)
        n_sess = len(wl.prefill)
        lin = tuple(sp.linear_layers)
        self.caches = SessionCaches(n_sess, sp.n_layers, sp.n_head_kv, wl.capacity, sp.head_dim, device,
                                    fp8=sp.kv_fp8, q8=sp.kv_q8, linear_layers=lin,
                                    rec_bytes=self.km.recurrent_state_bytes() if lin else 0)
        fill_sessions = range(n_sess) if sessions is None else sessions
        if lin:   # recurrent states before step 0, in the buffers the first step reads (pos % 2)
            C, dc = sp.ssm_conv_dim, sp.ssm_d_conv
            ring = ((dc - 1) * C + 3) // 4 * 4
            state = sp.ssm_n_v * sp.ssm_d_state ** 2
            assert 4 * 2 * (ring + state) == self.km.recurrent_state_bytes()
            self.rec_layout = (ring, state, dc, C)
            for s in fill_sessions:
                par = wl.prefill[s] % 2
                for il in lin:
                    rings, states = self.caches.recurrent_views(s, il, *self.rec_layout)
                    conv, S = W.recurrent_prefill(wl, s, il)
                    rings[par].copy_(torch.from_numpy(conv))
                    states[par].copy_(torch.from_numpy(S.reshape(-1)))
        if fill == "seeded":
            for s in fill_sessions:
                pairs = [(s, il) for il in range(sp.n_layers) if il not in lin]
                for (ss, il), (k, v) in zip(pairs, W.kv_prefill_many(wl, pairs)):
                    self.caches.fill_prefill(ss, il, k, v)
        else:
            gen = torch.Generator(device=device)
            for s in fill_sessions:
                gen.manual_seed(1000003 * (wl.seed + 1) + s)
                L = wl.prefill[s]
                t = self.caches.t[s]   # every layer's K/V (a linear layer's are never read)
                if sp.kv_fp8:   # random E4M3 bytes: sign, exponent field 4 .. 8, mantissa
                    c = torch.randint(0, 80, t[:, :, :, :L].shape, generator=gen, device=device)
                    t[:, :, :, :L] = (((c & 1) << 7) | ((4 + (c >> 4)) << 3) | ((c >> 1) & 7)).to(torch.uint8)
                elif sp.kv_q8:  # random int8 rows: codes in [-127, 127], fp16 block scales ~1.7/127
                    hd = sp.head_dim
                    codes = torch.randint(-127, 128, t[:, :, :, :L, :hd].shape, generator=gen, device=device)
                    t[:, :, :, :L, :hd] = codes.to(torch.int8).view(torch.uint8)
                    sc = (1.7 / 127.0) * (0.5 + torch.rand(t[:, :, :, :L, :hd // 32].shape, generator=gen, device=device))
                    t[:, :, :, :L, hd:hd + hd // 16] = sc.to(torch.float16).view(torch.uint8)
                else:
                    t[:, :, :, :L].normal_(generator=gen)
        self.device = device
        last = max(0, wl.steps - 1)
        self.ws = torch.empty(self.km.workspace_bytes(wl.B, wl.positions(last)) + 4096, dtype=torch.uint8,
                              device=device)
        self.out = torch.empty((wl.B, sp.out_dim), dtype=torch.float32, device=device)
        self._x_cache: Dict = {}

    def inputs(self, step: int) -> torch.Tensor:
        """Device input rows of one step (uploaded on first use: call ``prefetch`` before a
        timed loop, so that no host-to-device copy stalls the stream inside it)."""
        if step not in self._x_cache:
            self._x_cache[step] = torch.from_numpy(W.step_inputs(self.wl, step)).to(self.device)
        return self._x_cache[step]

    def prefetch(self, steps: Sequence[int], rows: Optional[Sequence[int]] = None) -> None:
        """Upload the inputs of these steps (and gather the row subset) ahead of time."""
        for s in steps:
            self._rows_input(s, rows)
        torch.cuda.synchronize()

    def _rows_input(self, s: int, rows: Optional[Sequence[int]]) -> torch.Tensor:
        x = self.inputs(s)
        if rows is None or list(rows) == list(range(self.wl.B)):
            return x
        rows = list(rows)
        if rows == list(range(rows[0], rows[0] + len(rows))):
            return x[rows[0]:rows[0] + len(rows)]           # a contiguous view: no copy
        key = (s, tuple(rows))
        if key not in self._x_cache:
            self._x_cache[key] = x[rows].contiguous()
        return self._x_cache[key]

    def step(self, s: int, rows: Optional[Sequence[int]] = None, out: Optional[torch.Tensor] = None,
             stream=None, x: Optional[torch.Tensor] = None, pos: Optional[Sequence[int]] = None) -> torch.Tensor:
        """Run decode step ``s`` for the given row indices (default: all rows).  ``x``: device
        input rows [len(rows), d] to use instead of the workload's (e.g. embedded tokens);
        ``pos``: the rows' positions instead of the workload's (e.g. after a verify commit)."""
        wl = self.wl
        rows = list(range(wl.B)) if rows is None else list(rows)
        x = self._rows_input(s, rows) if x is None else x
        if pos is None:
            pos_all = wl.positions(s)
            pos = [pos_all[b] for b in rows]
        sess = [wl.rows[b][0] for b in rows]
        kb, vb = self.caches.tables(sess)
        if out is None:
            out = self.out if len(rows) == wl.B else torch.empty((len(rows), wl.spec.out_dim), dtype=torch.float32,
                                                                 device=self.device)
        return self.km.kd_decode_step(x, pos, kb, vb, wl.capacity, out, self.ws, stream)

    def step_trace(self, s: int, rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
        """Decode step ``s`` through kd_debug_decode_step_trace: the output and the per-layer
        record (residual rows entering each layer and after the last; MoE routing), on the host."""
        wl = self.wl
        rows = list(range(wl.B)) if rows is None else list(rows)
        x = self._rows_input(s, rows)
        pos_all = wl.positions(s)
        pos = [pos_all[b] for b in rows]
        kb, vb = self.caches.tables([wl.rows[b][0] for b in rows])
        out = torch.empty((len(rows), wl.spec.out_dim), dtype=torch.float32, device=self.device)
        rec = self.km.kd_debug_decode_step_trace(x, pos, kb, vb, wl.capacity, out, self.ws)
        return {k: v.cpu().numpy() for k, v in rec.items()}

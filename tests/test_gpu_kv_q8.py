"""int8 KV caches (Q8_0 blocks along each cached head row): the append's rows against the
oracle's codec, attention over int8 caches against the oracle, and the whole step with int8
caches against the oracle.

Bars: the appended rows (codes and fp16 block scales) bit-exact (integer decisions taken
from the same fp32 values on both sides); attention within 1e-4 of the oracle per row
(scores on the exact codes with per-block fp32 sums, values d q formed exactly and carried as
fp16 hi + lo), rows bit-identical to their one-row calls; the step: every layer teacher-forced
in tests/test_gpu_layers.py, end to end within the deep bar, rows bit-identical to B = 1.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import ops
import workload as W
from gpu_util import assert_close_rows, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

kd = pytest.importorskip("session_decode_step_amd")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


@pytest.mark.parametrize("hd", [128, 64])
def test_kv_append_q8_rows_exact(hd):
    say(f"kv_append_q8 hd={hd}")
    r = np.random.default_rng(23 + hd)
    B, G, cap = 5, 8, 40
    RS = ops.q8_kv_row_bytes(hd)
    caches = [(torch.zeros((G, cap, RS), dtype=torch.uint8, device="cuda"),
               torch.zeros((G, cap, RS), dtype=torch.uint8, device="cuda")) for _ in range(B)]
    k = (r.standard_normal((B, G, hd)) * np.exp2(r.uniform(-12, 9, (B, G, 1)))).astype(np.float32)
    v = r.standard_normal((B, G, hd)).astype(np.float32)
    # row 0, head 0: a block with max 63.5 (scale 0.5 exactly) and exact ties; an all-zero block
    k[0, 0, :32] = 0.0
    k[0, 0, :6] = [63.5, -63.5, 0.75, -1.25, 0.25, -0.25]
    k[0, 0, 32:64] = 0.0
    pos = [int(p) for p in r.integers(0, cap, B)]
    kd.kd_kv_append_q8(dev(k), dev(v), [c[0].data_ptr() for c in caches], [c[1].data_ptr() for c in caches], pos, cap)
    torch.cuda.synchronize()
    for b in range(B):
        kc, vc = caches[b][0].cpu().numpy(), caches[b][1].cpu().numpy()
        np.testing.assert_array_equal(kc[:, pos[b]], ops.q8_kv_encode(k[b]))
        np.testing.assert_array_equal(vc[:, pos[b]], ops.q8_kv_encode(v[b]))
        others = np.ones(cap, dtype=bool)
        others[pos[b]] = False
        assert not kc[:, others].any() and not vc[:, others].any()
    assert caches[0][0][0, pos[0], :6].cpu().numpy().view(np.int8).tolist() == [127, -127, 2, -3, 1, -1]


def _q8_caches(r, n, G, cap, hd):
    return [(dev(W.q8_rows(r, (G, cap, hd))), dev(W.q8_rows(r, (G, cap, hd)))) for _ in range(n)]


@pytest.mark.parametrize("H,G,hd", [(32, 8, 128), (16, 4, 128), (8, 8, 64), (16, 2, 64)])
def test_fa_q8_vs_oracle(H, G, hd):
    say(f"fa_q8 H={H} G={G} hd={hd}")
    r = np.random.default_rng(H * 7 + G + hd)
    t_kv = [1, 17, 129, 1000, 4113]
    B, cap = len(t_kv), 4200
    caches = _q8_caches(r, B, G, cap, hd)
    q = r.standard_normal((B, H, hd)).astype(np.float32)
    kb = [c[0].data_ptr() for c in caches]
    vb = [c[1].data_ptr() for c in caches]
    scale = 1.0 / math.sqrt(hd)
    out = kd.kd_fa_decode_ragged_q8(dev(q), G, kb, vb, t_kv, cap, scale).cpu().numpy()
    for b in range(B):
        K = ops.q8_kv_decode(caches[b][0].cpu().numpy(), hd)
        V = ops.q8_kv_decode(caches[b][1].cpu().numpy(), hd)
        ref = ops.attention(q[b], K, V, t_kv[b])
        assert_close_rows(out[b], ref, 1e-4, f"fa_q8 row {b} t={t_kv[b]}")
        o1 = kd.kd_fa_decode_ragged_q8(dev(q[b:b + 1]), G, kb[b:b + 1], vb[b:b + 1], t_kv[b:b + 1], cap, scale)
        np.testing.assert_array_equal(o1.cpu().numpy()[0].view(np.uint32), out[b].view(np.uint32))


def test_fa_q8_long_rows_and_rows_sharing_a_cache():
    """Multi-tile chunks (rows past 16384 keys) and a stream's verify rows sharing one cache
    (one pass over its keys, each row masking its own tail), against the oracle and the rows'
    one-row calls."""
    say("fa_q8 long rows, shared cache")
    r = np.random.default_rng(31)
    H, G, hd, cap = 16, 8, 128, 20000
    caches = _q8_caches(r, 2, G, cap, hd)
    # rows 0..3 share cache 0 at consecutive lengths; row 4 reads cache 1 past 16384 keys
    t_kv = [8193, 8194, 8195, 8196, 19000]
    kb = [caches[0][0].data_ptr()] * 4 + [caches[1][0].data_ptr()]
    vb = [caches[0][1].data_ptr()] * 4 + [caches[1][1].data_ptr()]
    q = r.standard_normal((5, H, hd)).astype(np.float32)
    scale = 1.0 / math.sqrt(hd)
    out = kd.kd_fa_decode_ragged_q8(dev(q), G, kb, vb, t_kv, cap, scale).cpu().numpy()
    dec = [(ops.q8_kv_decode(c[0].cpu().numpy(), hd), ops.q8_kv_decode(c[1].cpu().numpy(), hd)) for c in caches]
    for b in range(5):
        K, V = dec[0] if b < 4 else dec[1]
        assert_close_rows(out[b], ops.attention(q[b], K, V, t_kv[b]), 1e-4, f"fa_q8 row {b}")
        o1 = kd.kd_fa_decode_ragged_q8(dev(q[b:b + 1]), G, kb[b:b + 1], vb[b:b + 1], t_kv[b:b + 1], cap, scale)
        np.testing.assert_array_equal(o1.cpu().numpy()[0].view(np.uint32), out[b].view(np.uint32))


def _q8_c2(B, steps, **extra):
    base = W.workload("c2", B=B, steps=steps)
    return dataclasses.replace(base, spec=dataclasses.replace(base.spec, kv_q8=True, **extra))


def test_c2_stack_with_q8_caches():
    """The 8-layer Q8_0 stack with int8 caches (canonical wqkv; the separate RoPE launch codes
    the rows): oracle on two rows for two steps at the deep bar, every row bit-identical
    (outputs and the cache bytes it wrote) to its B = 1 run."""
    from session_decode_step_amd.runner import GpuWorkload
    say("c2 q8 kv")
    wl = _q8_c2(4, 2)
    gw = GpuWorkload(wl)
    assert all(L.wqkv_pair_rows == 0 for L in gw.km.layers)
    rows = [0, 3]
    oc = oracle.OracleCaches(wl, sessions=sorted({wl.rows[b][0] for b in rows}))
    dense = oracle.DenseWeights(6 << 30)
    outs = []
    for s in range(2):
        y = gw.step(s).cpu().numpy()
        outs.append(y)
        x = W.step_inputs(wl, s)[rows]
        pos = [wl.positions(s)[b] for b in rows]
        ref = oracle.decode_step(gw.model, oc, x, [wl.rows[b][0] for b in rows], pos, dense=dense)
        assert_close_rows(y[rows], ref, 2e-2, f"c2 q8 step {s}", elem_rel=6e-2)
    s = 1
    for b in range(4):
        sess_b = wl.rows[b][0]
        p = wl.positions(s)[b]
        before = gw.caches.t[sess_b][:, :, :, p].cpu().numpy().copy()
        y1 = gw.step(s, rows=[b]).cpu().numpy()
        np.testing.assert_array_equal(y1[0].view(np.uint32), outs[-1][b].view(np.uint32))
        np.testing.assert_array_equal(gw.caches.t[sess_b][:, :, :, p].cpu().numpy(), before)


def test_c2_q8_caches_with_sliding_window_layers():
    """int8 caches under sliding-window layers (the window is a view of whole rows of hd + 16
    bytes): oracle on two rows, rows bit-identical to B = 1."""
    from session_decode_step_amd.runner import GpuWorkload
    say("c2 q8 kv + sliding window")
    wl = _q8_c2(4, 1, swa_window=512, swa_layers=(0, 2, 4, 6))
    gw = GpuWorkload(wl)
    y = gw.step(0).cpu().numpy().copy()
    rows = [0, 3]
    oc = oracle.OracleCaches(wl, sessions=sorted({wl.rows[b][0] for b in rows}))
    ref = oracle.decode_step(gw.model, oc, W.step_inputs(wl, 0)[rows], [wl.rows[b][0] for b in rows],
                             [wl.positions(0)[b] for b in rows], dense=oracle.DenseWeights(6 << 30))
    assert_close_rows(y[rows], ref, 2e-2, "c2 q8 swa step 0", elem_rel=6e-2)
    for r in range(4):
        y1 = gw.step(0, rows=[r]).cpu().numpy()
        np.testing.assert_array_equal(y1[0].view(np.uint32), y[r].view(np.uint32))

"""FP8 (E4M3) KV caches: the append's codes against the oracle's codec, attention over code
caches against the oracle and against the fp16 kernel on the same values, and the whole step
with FP8 caches against the oracle.

Bars: codes bit-exact (an integer decision taken from the same fp32 value on both sides);
attention within the fp16-cache bars (the widened operands are the codes' exact values), and
bit-identical to the fp16-cache call on caches holding those values; the step within the deep
bar of the fp16-cache stack, rows bit-identical to B = 1.
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


def _code_caches(r, n, G, cap, hd, lo=4, hi=9):
    """n pairs of uint8 code caches [G, cap, hd] with random sign, exponent field in [lo, hi)
    and mantissa (no NaN codes)."""
    out = []
    for _ in range(n):
        pair = []
        for _ in range(2):
            sign = r.integers(0, 2, (G, cap, hd), dtype=np.uint8) << 7
            ex = r.integers(lo, hi, (G, cap, hd), dtype=np.uint8) << 3
            m = r.integers(0, 8, (G, cap, hd), dtype=np.uint8)
            pair.append(dev((sign | ex | m).astype(np.uint8)))
        out.append(tuple(pair))
    return out


def _as_f16(c):
    """The same values in an fp16 cache (torch's float8_e4m3fn reading of the bytes)."""
    return c.view(torch.float8_e4m3fn).to(torch.float16)


def test_kv_append_fp8_codes_exact():
    say("kv_append_fp8")
    r = np.random.default_rng(19)
    B, G, hd, cap = 5, 8, 128, 40
    caches = [(torch.zeros((G, cap, hd), dtype=torch.uint8, device="cuda"),
               torch.zeros((G, cap, hd), dtype=torch.uint8, device="cuda")) for _ in range(B)]
    k = (r.standard_normal((B, G, hd)) * np.exp2(r.uniform(-12, 9, (B, G, hd)))).astype(np.float32)
    v = r.standard_normal((B, G, hd)).astype(np.float32)
    # special values in row 0: ties to even, saturation, subnormals, signed zero
    special = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 448.0, 449.0, 464.0, 1e6, -1e6, -0.0, 0.0,
                        -2.0 ** -9, 2.0 ** -6, 240.0, -447.9], dtype=np.float32)
    k[0, 0, :special.size] = special
    pos = [0, 39, 7, 8, 20]
    kd.kd_kv_append_fp8(dev(k), dev(v), [c[0].data_ptr() for c in caches], [c[1].data_ptr() for c in caches], pos,
                        cap)
    torch.cuda.synchronize()
    for b in range(B):
        K = caches[b][0].cpu().numpy()
        V = caches[b][1].cpu().numpy()
        np.testing.assert_array_equal(K[:, pos[b]], ops.e4m3_encode(k[b].astype(np.float64)))
        np.testing.assert_array_equal(V[:, pos[b]], ops.e4m3_encode(v[b].astype(np.float64)))
        mask = np.ones(cap, bool)
        mask[pos[b]] = False
        assert not K[:, mask].any() and not V[:, mask].any()


@pytest.mark.parametrize("H,G,hd", [(32, 8, 128), (4, 2, 64), (8, 8, 64), (16, 2, 64)])
def test_fa_fp8_vs_oracle_and_fp16_kernel(H, G, hd):
    say(f"fa fp8 H={H} G={G} hd={hd}")
    r = np.random.default_rng(H * 10 + G + hd)
    t_kv = [1, 2, 127, 129, 300, 1238, 5000]
    B, cap = len(t_kv), 5008
    caches = _code_caches(r, B, G, cap, hd)
    q = (r.standard_normal((B, H, hd)) * 0.5).astype(np.float32)
    kb = [c[0].data_ptr() for c in caches]
    vb = [c[1].data_ptr() for c in caches]
    scale = 1.0 / math.sqrt(hd)
    out = kd.kd_fa_decode_ragged_fp8(dev(q), G, kb, vb, t_kv, cap, scale).cpu().numpy()
    Kn = [ops.e4m3_decode(c[0].cpu().numpy()) for c in caches]
    Vn = [ops.e4m3_decode(c[1].cpu().numpy()) for c in caches]
    ref = np.stack([ops.attention(q[b], Kn[b], Vn[b], t_kv[b]) for b in range(B)])
    assert_close_rows(out.reshape(B, -1), ref.reshape(B, -1), 2e-3, "fa fp8")
    assert_close_rows(out.reshape(B, -1), ref.reshape(B, -1), 1e-4, "fa fp8 tight")
    # one key: exactly the code's value
    np.testing.assert_array_equal(out[0], np.stack([Vn[0][h // (H // G), 0] for h in range(H)]).astype(np.float32))
    # the same values in fp16 caches: the same bits
    f16 = [(_as_f16(c[0]), _as_f16(c[1])) for c in caches]
    o16 = kd.kd_fa_decode_ragged(dev(q), G, [c[0].data_ptr() for c in f16], [c[1].data_ptr() for c in f16], t_kv,
                                 cap, scale).cpu().numpy()
    np.testing.assert_array_equal(out.view(np.uint32), o16.view(np.uint32))
    # rows are B-invariant
    for b in (3, 6):
        o1 = kd.kd_fa_decode_ragged_fp8(dev(q[b:b + 1]), G, kb[b:b + 1], vb[b:b + 1], t_kv[b:b + 1], cap, scale)
        np.testing.assert_array_equal(o1.cpu().numpy()[0].view(np.uint32), out[b].view(np.uint32))


def test_fa_fp8_subnormal_codes_and_long_rows():
    """V holding only subnormal codes (values m 2^-9) must come out at that scale, not flushed;
    a row past 128 x 128 keys takes the multi-tile split kernel; rows of one cache at
    consecutive lengths take the shared pass -- each against the fp16 call on the same values."""
    say("fa fp8 subnormal V + multi-tile + shared rows")
    H, G, hd = 16, 8, 128
    r = np.random.default_rng(23)
    cap = 20008
    (kc, vc), = _code_caches(r, 1, G, cap, hd)
    vsub = dev(((r.integers(0, 2, (G, cap, hd), dtype=np.uint8) << 7) |
                r.integers(1, 8, (G, cap, hd), dtype=np.uint8)).astype(np.uint8))
    t_kv = [20000, 129, 130, 131, 4113]
    kb = [kc.data_ptr()] * 5
    vb = [vsub.data_ptr()] * 4 + [vc.data_ptr()]
    B = len(t_kv)
    q = (r.standard_normal((B, H, hd)) * 0.5).astype(np.float32)
    scale = 1.0 / math.sqrt(hd)
    out = kd.kd_fa_decode_ragged_fp8(dev(q), G, kb, vb, t_kv, cap, scale).cpu().numpy()
    k16, v16, s16 = _as_f16(kc), _as_f16(vc), _as_f16(vsub)
    kb16 = [k16.data_ptr()] * 5
    vb16 = [s16.data_ptr()] * 4 + [v16.data_ptr()]
    o16 = kd.kd_fa_decode_ragged(dev(q), G, kb16, vb16, t_kv, cap, scale).cpu().numpy()
    np.testing.assert_array_equal(out.view(np.uint32), o16.view(np.uint32))
    Kn = ops.e4m3_decode(kc.cpu().numpy())
    Sn = ops.e4m3_decode(vsub.cpu().numpy())
    for b in (0, 1, 3):
        ref = ops.attention(q[b], Kn, Sn, t_kv[b])
        assert np.abs(ref).max() < 2.0 ** -6
        assert_close_rows(out[b].reshape(1, -1), ref.reshape(1, -1), 2e-3, f"fa fp8 subnormal row {b}")


def _fp8_c2(B, steps):
    base = W.workload("c2", B=B, steps=steps)
    return dataclasses.replace(base, spec=dataclasses.replace(base.spec, kv_fp8=True))


def test_c2_stack_with_fp8_caches():
    """The 8-layer Q8_0 stack with E4M3 caches: oracle on two rows for two steps, the appended
    codes equal to the oracle's where the oracle's k and v sit away from a rounding boundary,
    every row bit-identical (outputs and the code bytes it wrote) to its B = 1 run, and the
    fused layout (codes stored by the QKV product's RoPE epilogue) equal to the separate
    RoPE + append launch: the same layer-0 code bytes, outputs within the deep bar."""
    from session_decode_step_amd.runner import GpuWorkload
    say("c2 fp8 kv")
    wl = _fp8_c2(4, 2)
    gw = GpuWorkload(wl)
    assert all(L.wqkv_pair_rows == 1 for L in gw.km.layers)   # the QKV product stores the codes
    rows = [0, 3]
    sess = sorted({wl.rows[b][0] for b in rows})
    oc = oracle.OracleCaches(wl, sessions=sess)
    dense = oracle.DenseWeights(6 << 30)
    outs = []
    for s in range(2):
        y = gw.step(s).cpu().numpy()
        outs.append(y)
        x = W.step_inputs(wl, s)[rows]
        pos = [wl.positions(s)[b] for b in rows]
        ref = oracle.decode_step(gw.model, oc, x, [wl.rows[b][0] for b in rows], pos, dense=dense)
        assert_close_rows(y[rows], ref, 2e-2, f"c2 fp8 step {s}", elem_rel=6e-2)
    # layer 0's appended codes (its input is the step input: the k/v differ from the oracle's
    # by fp32 rounding only, so all but a few codes agree)
    s = 1
    for b in rows:
        sess_b = wl.rows[b][0]
        p = wl.positions(s)[b]
        g = gw.caches.t[sess_b][0, 0, :, p].cpu().numpy()
        o = oc.K[sess_b][0][:, p]
        assert np.mean(g == o) > 0.99, np.mean(g == o)
    # B = 1 runs write the same bytes and return the same rows
    for b in range(4):
        sess_b = wl.rows[b][0]
        p = wl.positions(s)[b]
        before = gw.caches.t[sess_b][:, :, :, p].cpu().numpy().copy()
        y1 = gw.step(s, rows=[b]).cpu().numpy()
        np.testing.assert_array_equal(y1[0].view(np.uint32), outs[-1][b].view(np.uint32))
        np.testing.assert_array_equal(gw.caches.t[sess_b][:, :, :, p].cpu().numpy(), before)
    # the separate RoPE + append launch on the canonical layout
    gs = GpuWorkload(wl, model=gw.model, fused=False)
    assert all(L.wqkv_pair_rows == 0 for L in gs.km.layers)
    for s2 in range(2):
        ys = gs.step(s2).cpu().numpy()
        assert_close_rows(outs[s2], ys.astype(np.float64), 2e-2, f"fp8 step {s2} fused vs separate", elem_rel=6e-2)
    for sess_b in range(len(wl.prefill)):
        np.testing.assert_array_equal(gw.caches.t[sess_b][0].cpu().numpy(), gs.caches.t[sess_b][0].cpu().numpy())


def test_c4_stack_with_fp8_caches_b8():
    """The bench's FP8 configuration: the 32-layer d=4096 Q4_0 stack at B = 8, ctx 4096, with
    E4M3 caches; the oracle on one row, every row bit-identical to its B = 1 run."""
    from session_decode_step_amd.runner import GpuWorkload
    say("c4 fp8 kv B=8")
    base = W.workload("c4", B=8, steps=1)
    wl = dataclasses.replace(base, spec=dataclasses.replace(base.spec, kv_fp8=True))
    gw = GpuWorkload(wl)
    y = gw.step(0).cpu().numpy().copy()
    b = 5
    oc = oracle.OracleCaches(wl, sessions=[wl.rows[b][0]])
    ref = oracle.decode_step(gw.model, oc, W.step_inputs(wl, 0)[[b]], [wl.rows[b][0]], [wl.positions(0)[b]])
    assert_close_rows(y[[b]], ref, 2e-2, "c4 fp8 step 0", elem_rel=6e-2)
    for r in range(8):
        y1 = gw.step(0, rows=[r]).cpu().numpy()
        np.testing.assert_array_equal(y1[0].view(np.uint32), y[r].view(np.uint32))


def test_c2_fp8_caches_with_sliding_window_layers():
    """FP8 caches under sliding-window layers (the window is a view one byte per element into
    the code cache): oracle on two rows, rows bit-identical to B = 1."""
    from session_decode_step_amd.runner import GpuWorkload
    say("c2 fp8 kv + sliding window")
    base = W.workload("c2", B=4, steps=1)
    wl = dataclasses.replace(base, spec=dataclasses.replace(base.spec, kv_fp8=True, swa_window=512,
                                                            swa_layers=(0, 2, 4, 6)))
    gw = GpuWorkload(wl)
    y = gw.step(0).cpu().numpy().copy()
    rows = [0, 3]
    oc = oracle.OracleCaches(wl, sessions=sorted({wl.rows[b][0] for b in rows}))
    ref = oracle.decode_step(gw.model, oc, W.step_inputs(wl, 0)[rows], [wl.rows[b][0] for b in rows],
                             [wl.positions(0)[b] for b in rows], dense=oracle.DenseWeights(6 << 30))
    assert_close_rows(y[rows], ref, 2e-2, "c2 fp8 swa step 0", elem_rel=6e-2)
    for r in range(4):
        y1 = gw.step(0, rows=[r]).cpu().numpy()
        np.testing.assert_array_equal(y1[0].view(np.uint32), y[r].view(np.uint32))

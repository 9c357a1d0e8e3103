"""Pins of the CPU oracle against things other than itself (no GPU).

Hand-worked blocks (tests/golden), closed forms, brute force on tiny inputs and library
routines (torch CPU in fp64).  Each pin is chosen so a plausible slip in the oracle (a
dropped term, a swapped nibble, a transposed operand, a wrong sign or index) fails it.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import ops
import workload as wlmod

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------- codecs (O1, O2)
def test_q4_0_golden_block():
    g = _gold("q4_0_block.json")
    w = {"fmt": "q4_0", "n": 1, "k": 32, "qs": np.frombuffer(bytes.fromhex(g["bytes_hex"]), np.uint8).reshape(1, 16),
         "d": np.array([[g["d"]]], dtype=np.float16)}
    assert ops.dequantize(w)[0].tolist() == g["values"]


def test_q8_0_golden_block():
    g = _gold("q8_0_block.json")
    w = {"fmt": "q8_0", "n": 1, "k": 32, "qs": np.array([g["codes"]], dtype=np.int8),
         "d": np.array([[g["d"]]], dtype=np.float16)}
    assert ops.dequantize(w)[0].tolist() == g["values"]


def test_q4_0_codes_cover_range_and_rows():
    # Two rows x two blocks, every nibble value present: decoded codes span [-8, 7] and row /
    # block indexing keeps each block's own scale.
    qs = np.array([[(j | ((15 - j) << 4)) for j in range(16)] * 2,
                   [((j * 5) % 16) | (((j * 3) % 16) << 4) for j in range(16)] * 2], dtype=np.uint8)
    d = np.array([[1.0, 2.0], [0.5, 4.0]], dtype=np.float16)
    w = {"fmt": "q4_0", "n": 2, "k": 64, "qs": qs, "d": d}
    q, dd = ops.weight_codes(w)
    assert q.min() == -8 and q.max() == 7
    assert q[1, 0, 3] == ((3 * 5) % 16) - 8 and q[1, 0, 19] == ((3 * 3) % 16) - 8
    v = ops.dequantize(w)
    assert v[0, 32 + 5] == 2.0 * (5 - 8) and v[1, 32 + 16 + 2] == 4.0 * (((2 * 3) % 16) - 8)


def _kq_record(fmt, hexs):
    rec = np.frombuffer(bytes.fromhex(hexs), np.uint8)
    assert rec.size == ops.KQ_BYTES[fmt]
    return {"fmt": fmt, "n": 1, "k": 256, "qs": rec.reshape(1, -1), "d": np.zeros((1, 0), np.float16)}


def test_kquant_packed_scales_and_mins_by_hand():
    g = _gold("kquant_records.json")
    b = np.frombuffer(bytes.fromhex(g["scales_hex"]), np.uint8)
    got = [ops.kquant_scale_min(b, j) for j in range(8)]
    assert [int(s) for s, _ in got] == g["scale_min_by_hand"]["sc"]
    assert [int(m) for _, m in got] == g["scale_min_by_hand"]["m"]


@pytest.mark.parametrize("fmt", ["q4_k", "q5_k", "q6_k"])
def test_kquant_golden_records(fmt):
    """Hand-worked values of one record per format (codes in both nibbles and every code run,
    sub-block scales and mins of both packings, fifth and upper bits, signed Q6_K scales)."""
    g = _gold("kquant_records.json")[fmt]
    v = ops.dequantize(_kq_record(fmt, g["record_hex"]))[0]
    for e, want in g["values"].items():
        assert v[int(e)] == want, (fmt, e, v[int(e)], want)


def test_kquant_structure():
    """Rows and super-blocks keep their own fields; Q5_K with no fifth bits is Q4_K with the same
    fields; a Q4_K record of zero codes holds -dmin m_j in sub-block j; a Q6_K record of codes
    32 is zero."""
    rng = np.random.default_rng(5)
    rec4 = rng.integers(0, 256, size=(3, 2, 144), dtype=np.uint8)
    rec4[:, :, 0:2] = np.array([0x00, 0x3C], np.uint8)      # d = 1
    rec4[:, :, 2:4] = np.array([0x00, 0x40], np.uint8)      # dmin = 2
    w4 = {"fmt": "q4_k", "n": 3, "k": 512, "qs": rec4.reshape(3, -1), "d": np.zeros((3, 0), np.float16)}
    rec5 = np.zeros((3, 2, 176), np.uint8)
    rec5[:, :, :16] = rec4[:, :, :16]
    rec5[:, :, 48:] = rec4[:, :, 16:]
    w5 = {"fmt": "q5_k", "n": 3, "k": 512, "qs": rec5.reshape(3, -1), "d": np.zeros((3, 0), np.float16)}
    v4 = ops.dequantize(w4)
    np.testing.assert_array_equal(v4, ops.dequantize(w5))
    np.testing.assert_array_equal(ops.dequantize(w4, 1, 3), v4[1:3])
    # second super-block of row 2 decoded alone
    one = {"fmt": "q4_k", "n": 1, "k": 256, "qs": rec4[2, 1][None, :], "d": np.zeros((1, 0), np.float16)}
    np.testing.assert_array_equal(ops.dequantize(one)[0], v4[2, 256:])
    zero = rec4.copy()
    zero[:, :, 16:] = 0
    wz = {"fmt": "q4_k", "n": 3, "k": 512, "qs": zero.reshape(3, -1), "d": np.zeros((3, 0), np.float16)}
    vz = ops.dequantize(wz).reshape(3, 2, 8, 32)
    for j in range(8):
        _, m = ops.kquant_scale_min(zero[:, :, 4:16], j)
        np.testing.assert_array_equal(vz[:, :, j, :], np.broadcast_to(-2.0 * m[:, :, None], (3, 2, 32)))
    rec6 = np.zeros((1, 210), np.uint8)
    rec6[0, 128:192] = 0xAA                                  # upper bits 2 in every pair: q = 32
    rec6[0, 192:208] = 7
    rec6[0, 208:210] = [0x00, 0x3C]
    np.testing.assert_array_equal(ops.dequantize({"fmt": "q6_k", "n": 1, "k": 256, "qs": rec6,
                                                  "d": np.zeros((1, 0), np.float16)}), np.zeros((1, 256)))


# --------------------------------------------------------------------------- quantiser (O3)
def test_act_quant_golden_blocks():
    g = _gold("act_quant_blocks.json")
    x = np.array([np.concatenate([b["x"] for b in g["blocks"]])], dtype=np.float32)
    q, d = ops.quantize_act(x)
    assert d[0].tolist() == [b["d"] for b in g["blocks"]]
    assert q[0].tolist() == sum((b["q"] for b in g["blocks"]), [])


def test_act_quant_invariants_random():
    r = np.random.default_rng(1)
    x = (r.standard_normal((7, 32 * 40)) * np.exp(r.uniform(-6, 6, (7, 1)))).astype(np.float32)
    x[3, 64:96] = 0.0
    q, d = ops.quantize_act(x)
    blk = x.reshape(7, 40, 32).astype(np.float64)
    qb = q.reshape(7, 40, 32).astype(np.float64)
    dd = d.astype(np.float64)[:, :, None]
    # reconstruction error at most half a step (plus fp32 rounding of x/d)
    assert np.all(np.abs(blk - dd * qb) <= dd * (0.5 + 1e-6))
    # the amax element maps to +-127, codes within range
    amax_idx = np.argmax(np.abs(blk), axis=2)
    picked = np.take_along_axis(qb, amax_idx[:, :, None], 2)[:, :, 0]
    nz = d > 0
    assert np.all(np.abs(picked[nz]) == 127)
    assert np.all(np.abs(qb) <= 127)
    # zero block: zero scale and codes
    assert d[3, 2] == 0 and np.all(q[3, 64:96] == 0)
    # scale is the IEEE fp32 quotient amax/127
    assert np.array_equal(d, (np.max(np.abs(x.reshape(7, 40, 32)), 2) / np.float32(127)).astype(np.float32))


def test_act_quant_ties_round_away_from_zero():
    # d = 1 (amax 127): x/d = k + 0.5 must round away from zero, for both signs.
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 127.0
    x[0, 1:9] = [0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5]
    q, _ = ops.quantize_act(x)
    assert q[0, 1:9].tolist() == [1, 2, 3, 4, -1, -2, -3, -4]
    # the largest fp32 below 0.5 rounds to 0 (an fp32 "+0.5 then floor" would give 1)
    x[0, 9] = np.nextafter(np.float32(0.5), np.float32(0))
    q, _ = ops.quantize_act(x)
    assert q[0, 9] == 0


# --------------------------------------------------------------------------- mmvq (O4)
def test_mmvq_golden_block():
    g = _gold("mmvq_block.json")
    w = {"fmt": "q8_0", "n": 1, "k": 32, "qs": np.array([g["w_codes"]], np.int8), "d": np.array([[g["w_d"]]], np.float16)}
    xq, xd = ops.quantize_act(np.array([g["x"]], np.float32))
    assert xq[0].tolist() == g["x_codes"] and xd[0, 0] == g["x_d"]
    assert ops.block_dots(w, xq)[0, 0, 0] == g["S"]
    assert ops.mmvq_blocks(w, xq, xd)[0, 0] == g["y"]


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_block_dots_bruteforce(fmt):
    r = np.random.default_rng(2)
    w = (wlmod.draw_q8_0 if fmt == "q8_0" else wlmod.draw_q4_0)(r, r, 3, 64)
    xq = r.integers(-127, 128, (2, 64)).astype(np.int8)
    S = ops.block_dots(w, xq)
    # brute force via an independent decode of each element from the raw bytes
    for n in range(3):
        for blk in range(2):
            for b in range(2):
                s = 0
                for i in range(32):
                    if fmt == "q8_0":
                        c = int(w["qs"][n, 32 * blk + i])
                    else:
                        byte = int(w["qs"][n, 16 * blk + (i % 16)])
                        c = ((byte >> 4) if i >= 16 else (byte & 15)) - 8
                    s += c * int(xq[b, 32 * blk + i])
                assert S[b, n, blk] == s


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_mmvq_block_formula_equals_dense(fmt):
    r = np.random.default_rng(3)
    w = (wlmod.draw_q8_0 if fmt == "q8_0" else wlmod.draw_q4_0)(r, r, 40, 256)
    x = r.standard_normal((5, 256)).astype(np.float32)
    xq, xd = ops.quantize_act(x)
    yb = ops.mmvq_blocks(w, xq, xd)
    yd = ops.mmvq(w, xq, xd, chunk=16)
    np.testing.assert_allclose(yb, yd, rtol=1e-12, atol=1e-12 * np.abs(yd).max())


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_mmvq_vs_unquantised_closed_form_bound(fmt):
    r = np.random.default_rng(4)
    w = (wlmod.draw_q8_0 if fmt == "q8_0" else wlmod.draw_q4_0)(r, r, 64, 512)
    x = r.standard_normal((4, 512)).astype(np.float32)
    xq, xd = ops.quantize_act(x)
    y = ops.mmvq_blocks(w, xq, xd)
    exact = x.astype(np.float64) @ ops.dequantize(w).T
    qw, dw = ops.weight_codes(w)
    bound = np.einsum("nk,bk->bn", np.abs(dw) * np.abs(qw).sum(2), xd.astype(np.float64) / 2)
    assert np.all(np.abs(y - exact) <= bound * (1 + 1e-6) + 1e-12)
    assert np.any(np.abs(y - exact) > 0.05 * bound)  # the bound is not vacuous


# --------------------------------------------------------------------------- row ops (O5, O6, O9)
def test_rmsnorm_constant_and_torch():
    g = np.array([1.5, -2.0, 0.25, 3.0])
    y = ops.rmsnorm(np.full(4, -3.0), g, 1e-5)
    np.testing.assert_allclose(y, -g * 3.0 / math.sqrt(9.0 + 1e-5), rtol=1e-15)
    r = np.random.default_rng(5)
    x = r.standard_normal((3, 64))
    gg = r.standard_normal(64)
    ref = torch.nn.functional.rms_norm(torch.tensor(x), (64,), torch.tensor(gg), eps=1e-5).numpy()
    np.testing.assert_allclose(ops.rmsnorm(x, gg, 1e-5), ref, rtol=1e-13, atol=1e-14)


def test_rope_closed_forms():
    r = np.random.default_rng(6)
    x = r.standard_normal((3, 128))
    np.testing.assert_array_equal(ops.rope_neox(x, 0, 10000.0), x)            # pos 0: identity
    y = ops.rope_neox(x, 1234, 10000.0)
    pn = lambda a: a[:, :64] ** 2 + a[:, 64:] ** 2
    np.testing.assert_allclose(pn(y), pn(x), rtol=1e-12)                       # pair norms kept
    np.testing.assert_allclose(ops.rope_neox(ops.rope_neox(x, 17, 1e4), 40, 1e4),
                               ops.rope_neox(x, 57, 1e4), rtol=1e-9, atol=1e-12)  # R(a)R(b)=R(a+b)
    q, k = r.standard_normal(128), r.standard_normal(128)
    d1 = ops.rope_neox(q[None], 100, 1e4)[0] @ ops.rope_neox(k[None], 90, 1e4)[0]
    d2 = ops.rope_neox(q[None], 5010, 1e4)[0] @ ops.rope_neox(k[None], 5000, 1e4)[0]
    assert abs(d1 - d2) < 1e-9 * (1 + abs(d1))                                   # relative position
    # the pairing is (i, i + hd/2): a vector with only element 0 set rotates into element 64
    e0 = np.zeros(128); e0[0] = 1.0
    y0 = ops.rope_neox(e0[None], 1, 1e4)[0]
    assert abs(y0[0] - math.cos(1.0)) < 1e-15 and abs(y0[64] - math.sin(1.0)) < 1e-15
    # element 1 rotates with theta = base^(-2/hd)
    e1 = np.zeros(128); e1[1] = 1.0
    y1 = ops.rope_neox(e1[None], 3, 1e4)[0]
    th = 3 * 1e4 ** (-2.0 / 128)
    assert abs(y1[1] - math.cos(th)) < 1e-15 and abs(y1[65] - math.sin(th)) < 1e-15


def test_swiglu_special_cases_and_torch():
    assert ops.silu(np.array([0.0]))[0] == 0.0
    assert abs(ops.swiglu(np.array([40.0]), np.array([3.0]))[0] - 120.0) < 1e-12
    r = np.random.default_rng(7)
    g, u = r.standard_normal(100), r.standard_normal(100)
    ref = (torch.nn.functional.silu(torch.tensor(g)) * torch.tensor(u)).numpy()
    np.testing.assert_allclose(ops.swiglu(g, u), ref, rtol=1e-14, atol=1e-15)


# --------------------------------------------------------------------------- attention (O8)
def test_attention_special_cases():
    r = np.random.default_rng(8)
    H, G, hd = 4, 2, 64
    K = r.standard_normal((G, 10, hd)).astype(np.float16)
    V = r.standard_normal((G, 10, hd)).astype(np.float16)
    q = r.standard_normal((H, hd))
    out = ops.attention(q, K, V, 1)                       # t = 1: out = V[0]
    for h in range(H):
        np.testing.assert_array_equal(out[h], V[h // 2, 0].astype(np.float64))
    out0 = ops.attention(np.zeros((H, hd)), K, V, 7)       # q = 0: uniform weights
    for h in range(H):
        np.testing.assert_allclose(out0[h], V[h // 2, :7].astype(np.float64).mean(0), rtol=1e-12, atol=1e-14)
    K2 = K.copy(); K2[:, :] = K[:, :1]                     # identical keys: mean of V
    out2 = ops.attention(q, K2, V, 9)
    np.testing.assert_allclose(out2[3], V[1, :9].astype(np.float64).mean(0), rtol=1e-12, atol=1e-14)
    K3 = np.zeros_like(K); K3[1, 4] = 1.0                  # one dominant key for heads of group 1
    q3 = np.zeros((H, hd)); q3[2:, :] = 60.0
    out3 = ops.attention(q3, K3, V, 10)
    np.testing.assert_allclose(out3[2], V[1, 4].astype(np.float64), rtol=1e-9, atol=1e-9)


def test_attention_vs_torch_sdpa_gqa():
    r = np.random.default_rng(9)
    H, G, hd, t = 8, 2, 64, 37
    K = r.standard_normal((G, 50, hd)).astype(np.float16)
    V = r.standard_normal((G, 50, hd)).astype(np.float16)
    q = r.standard_normal((H, hd))
    ours = ops.attention(q, K, V, t)
    kk = torch.tensor(K[:, :t].astype(np.float64)).repeat_interleave(H // G, 0)   # head h -> group h // (H/G)
    vv = torch.tensor(V[:, :t].astype(np.float64)).repeat_interleave(H // G, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(torch.tensor(q)[:, None, :], kk, vv)[:, 0].numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- router
def test_router_topk_ties_and_torch():
    r = np.array([0.5, 2.0, 2.0, -1.0, 3.0, 2.0, 0.1, 3.0])
    ids, p = ops.router_topk(r, 4)
    assert ids.tolist() == [4, 7, 1, 2]               # ties to the lower id
    np.testing.assert_allclose(p.sum(), 1.0, rtol=1e-15)
    np.testing.assert_allclose(p, torch.softmax(torch.tensor(r[ids]), 0).numpy(), rtol=1e-14)
    rr = np.random.default_rng(10).standard_normal(128)
    ids2, _ = ops.router_topk(rr, 8)
    assert ids2.tolist() == torch.topk(torch.tensor(rr), 8).indices.tolist()


def test_sliding_window_is_a_positional_mask():
    """The window view (the last W keys of the cache) against the plain definition: softmax
    over every key with the keys before len - W masked out; a window at least len long is
    full attention."""
    from oracle.step import _attend
    r = np.random.default_rng(21)
    G, H, hd, cap = 2, 4, 64, 80
    K = r.standard_normal((G, cap, hd)).astype(np.float16)
    V = r.standard_normal((G, cap, hd)).astype(np.float16)
    q = r.standard_normal((H, hd))
    for length, win in ((50, 16), (50, 49), (17, 16), (16, 16), (10, 32)):
        got = _attend(q, K, V, length, win)
        lo = max(0, length - win)
        ref = np.empty((H, hd))
        for h in range(H):
            g = h // (H // G)
            sc = (K[g, :length].astype(np.float64) @ q[h]) / np.sqrt(hd)
            sc[:lo] = -np.inf
            p = np.exp(sc - sc.max())
            p /= p.sum()
            ref[h] = p @ V[g, :length].astype(np.float64)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
        if win >= length:
            np.testing.assert_array_equal(got, ops.attention(q, K, V, length))


def test_qk_norm_heads_have_unit_rms_after_rope():
    """QK-norm with unit gains: every query head that enters attention, and every key head
    written to the cache, has RMS 1 (RoPE preserves each pair's norm), whatever the raw
    projection's scale."""
    import dataclasses
    spec = dataclasses.replace(TINY, qk_norm=True, rms_eps=1e-12)
    wl = _tiny_wl(spec, 91, [(0, 0), (1, 0)], [9, 20])
    model = wlmod.make_model(spec, wl.code, wl.seed)
    for L in model["layers"]:
        L["q_norm"] = np.ones_like(L["q_norm"])
        L["k_norm"] = np.ones_like(L["k_norm"])
    oc = oracle.OracleCaches(wl)
    trace = []
    oracle.decode_step(model, oc, wlmod.step_inputs(wl, 0), [0, 1], wl.positions(0), trace=trace)
    for t in trace:
        np.testing.assert_allclose(np.sqrt(np.mean(t["q"] ** 2, axis=-1)), 1.0, rtol=1e-9)
        np.testing.assert_allclose(np.sqrt(np.mean(t["k"].astype(np.float64) ** 2, axis=-1)), 1.0, rtol=1e-9)
    for s, p in ((0, 9), (1, 20)):
        kc = oc.K[s][0][:, p].astype(np.float64)                 # the appended key, fp16
        np.testing.assert_allclose(np.sqrt(np.mean(kc ** 2, axis=-1)), 1.0, rtol=2e-3)


def test_sigmoid_special_cases_and_silu():
    x = np.linspace(-30, 30, 121)
    s = ops.sigmoid(x)
    assert ops.sigmoid(np.array([0.0]))[0] == 0.5
    np.testing.assert_allclose(s + ops.sigmoid(-x), 1.0, rtol=0, atol=1e-15)   # odd symmetry about 1/2
    np.testing.assert_allclose(x * s, ops.silu(x), rtol=1e-15, atol=1e-300)     # silu(x) = x sigmoid(x)
    assert np.all(np.diff(s) > 0) and s[0] > 0 and s[-1] < 1


# --------------------------------------------------------------------------- next token
def test_greedy_token_hand_cases():
    # first maximum wins on ties; a lone entry; all-equal and all -inf rows give index 0
    x = np.array([[1.0, 3.0, 3.0, 2.0],
                  [-5.0, -1.0, -2.0, -1.0],
                  [7.0, 7.0, 7.0, 7.0],
                  [-np.inf, -np.inf, -np.inf, -np.inf],
                  [0.0, -0.0, 0.0, 1e-45]], dtype=np.float32)
    assert ops.greedy_token(x).tolist() == [1, 1, 0, 0, 3]
    assert ops.greedy_token(np.array([[4.5]], dtype=np.float32)).tolist() == [0]


def test_greedy_token_scan_and_numpy():
    # many ties (small integers): a strict-greater left-to-right scan, and numpy's argmax
    # (documented to return the first occurrence of the maximum)
    r = np.random.default_rng(11)
    x = r.integers(-3, 4, size=(64, 257)).astype(np.float32)
    scan = []
    for row in x:
        best, bi = row[0], 0
        for j in range(1, row.shape[0]):
            if row[j] > best:
                best, bi = row[j], j
        scan.append(bi)
    assert ops.greedy_token(x).tolist() == scan
    y = r.standard_normal((16, 32000)).astype(np.float32)
    assert ops.greedy_token(y).tolist() == np.argmax(y, axis=1).tolist()


def test_embed_rows_picks_rows():
    table = np.arange(7 * 5, dtype=np.float32).reshape(7, 5)
    out = ops.embed_rows(table, np.array([6, 0, 6, 3]))
    assert out[:, 0].tolist() == [30.0, 0.0, 30.0, 15.0]
    assert (out - out[:, :1] == np.arange(5, dtype=np.float32)).all()


def test_accept_drafts_hand_cases():
    # two streams of k = 4 rows: (fed = last token + 3 drafts, greedy of each row)
    fed = np.array([5, 10, 11, 12,    5, 10, 99, 12])
    greedy = np.array([10, 11, 12, 13,   10, 11, 12, 13])
    n_acc, nxt = ops.accept_drafts(greedy, fed, 4)
    assert n_acc.tolist() == [3, 1]          # all drafts kept; the second draft rejected
    assert nxt.tolist() == [13, 11]          # the token after the kept prefix
    # a mismatch at the first draft keeps none, and later agreement does not count
    n_acc, nxt = ops.accept_drafts(np.array([7, 11, 12, 13]), np.array([5, 10, 11, 12]), 4)
    assert (n_acc.tolist(), nxt.tolist()) == ([0], [7])
    # one row per stream: plain greedy decoding
    n_acc, nxt = ops.accept_drafts(np.array([3, 4]), np.array([1, 2]), 1)
    assert (n_acc.tolist(), nxt.tolist()) == ([0, 0], [3, 4])


def test_accept_drafts_matches_sequential_greedy():
    # a toy deterministic target (next = f(token)): drafts that follow it are all kept, and
    # the result equals running the target one token at a time
    f = lambda t: (7 * t + 3) % 50                                     # noqa: E731
    r = np.random.default_rng(12)
    for _ in range(200):
        k = int(r.integers(1, 6))
        t0 = int(r.integers(0, 50))
        seq = [t0]
        for _j in range(k):
            seq.append(f(seq[-1]))
        drafts = [seq[j] if r.random() < 0.8 else int(r.integers(0, 50)) for j in range(1, k)]
        fed = np.array([t0] + drafts)
        greedy = np.array([f(int(t)) for t in fed])
        n_acc, nxt = ops.accept_drafts(greedy, fed, k)
        a = 0
        while a < k - 1 and drafts[a] == seq[a + 1]:
            a += 1
        assert n_acc[0] == a and nxt[0] == seq[a + 1]


# --------------------------------------------------------------------------- composition
TINY = wlmod.ModelSpec("tiny", 2, 128, 4, 2, 64, 256, "q8_0", vocab=96, final_norm=True)
TINY_MOE = wlmod.ModelSpec("tiny_moe", 2, 128, 4, 2, 64, 0, "q4_0", final_norm=True,
                           n_experts=8, n_expert_used=3, expert_ffn=64, shared_ffn=96)


def _tiny_wl(spec, code, rows, prefill, cap=48):
    return wlmod.Workload(code, spec, prefill, rows, 1, cap, 0)


@pytest.mark.parametrize("spec", [TINY, TINY_MOE], ids=["dense", "moe"])
def test_step_block_formula_equals_dense_formulation(spec):
    wl = _tiny_wl(spec, 91, [(0, 0), (1, 0), (1, 1)], [5, 20])
    model = wlmod.make_model(spec, 91)
    x = wlmod.step_inputs(wl, 0)
    ys = []
    for blocks in (True, False):
        c = oracle.OracleCaches(wl)
        ys.append(oracle.decode_step(model, c, x, [0, 1, 1], wl.positions(0), blocks=blocks))
    np.testing.assert_allclose(ys[0], ys[1], rtol=1e-10, atol=1e-10 * np.abs(ys[1]).max())


def test_moe_routed_sum_equals_dense_masked_sum():
    spec = TINY_MOE
    model = wlmod.make_model(spec, 92)
    L = model["layers"][0]
    r = np.random.default_rng(11)
    z = r.standard_normal((3, spec.d))
    zq, zd = ops.quantize_act(z.astype(np.float32))
    routed = oracle.moe_ffn(spec, L, z, zq, zd, None, blocks=False)
    # dense evaluation of every expert, weighted by p masked to the top-k
    logits = z @ L["router"].astype(np.float64).T
    dense = np.zeros_like(routed)
    Fe, d = spec.expert_ffn, spec.d
    for b in range(3):
        order = sorted(range(spec.n_experts), key=lambda e: (-logits[b, e], e))[: spec.n_expert_used]
        w = np.zeros(spec.n_experts)
        ex = np.exp(logits[b, order] - logits[b, order].max())
        w[order] = ex / ex.sum()
        for e in range(spec.n_experts):
            Wg = ops.dequantize(L["e_gate"], e * Fe, (e + 1) * Fe)
            Wu = ops.dequantize(L["e_up"], e * Fe, (e + 1) * Fe)
            Wd = ops.dequantize(L["e_down"], e * d, (e + 1) * d)
            xv = ops.dequantize_act(zq[b:b + 1], zd[b:b + 1])
            hq, hd = ops.quantize_act(ops.swiglu(xv @ Wg.T, xv @ Wu.T).astype(np.float32))
            dense[b] += w[e] * (ops.dequantize_act(hq, hd) @ Wd.T)[0]
        xv = ops.dequantize_act(zq[b:b + 1], zd[b:b + 1])
        hq, hd = ops.quantize_act(ops.swiglu(xv @ ops.dequantize(L["s_gate"]).T,
                                             xv @ ops.dequantize(L["s_up"]).T).astype(np.float32))
        dense[b] += (ops.dequantize_act(hq, hd) @ ops.dequantize(L["s_down"]).T)[0]
    np.testing.assert_allclose(routed, dense, rtol=1e-10, atol=1e-12)


def _gated_pair(seed):
    """A one-layer gated stack and the same stack without the gate (its wqkv without the H hd
    gate rows), one row, and that row's quantised attention-norm input."""
    import dataclasses
    spec_g = dataclasses.replace(TINY, n_layers=1, attn_gate=True, vocab=0, final_norm=False)
    spec_u = dataclasses.replace(spec_g, attn_gate=False)
    mg = wlmod.make_model(spec_g, seed)
    Lg = mg["layers"][0]
    n_qkv = spec_u.qkv_rows
    Lu = {**Lg, "attn_gate": False,
          "wqkv": {**Lg["wqkv"], "n": n_qkv, "qs": Lg["wqkv"]["qs"][:n_qkv].copy(), "d": Lg["wqkv"]["d"][:n_qkv].copy()}}
    mu = {**mg, "spec": spec_u, "layers": [Lu]}
    wl = _tiny_wl(spec_g, seed, [(0, 0)], [13])
    x = wlmod.step_inputs(wl, 0)
    xq, _ = ops.quantize_act(ops.rmsnorm(x.astype(np.float64), Lg["attn_norm"], spec_g.rms_eps).astype(np.float32))
    return spec_g, mg, mu, wl, x, xq


def _set_gate_rows(model, spec, xq, sign_per_head):
    """Gate rows of head h = sign_per_head[h] * 127 * sign(codes of the row's input), scale 1:
    the gate is then +-127 sum |x| (huge) for that input, or exactly 0 where the sign is 0."""
    L = model["layers"][0]
    H, G, hd = spec.n_head, spec.n_head_kv, spec.head_dim
    qs, d = L["wqkv"]["qs"].copy(), L["wqkv"]["d"].copy()
    base = (H + 2 * G) * hd
    for h in range(H):
        rows = slice(base + h * hd, base + (h + 1) * hd)
        qs[rows] = (sign_per_head[h] * 127 * np.sign(xq[0].astype(np.int64)))[None, :].astype(np.int8)
        d[rows] = np.float16(1.0)
    L["wqkv"] = {**L["wqkv"], "qs": qs, "d": d}


def test_output_gate_saturated_open_equals_ungated():
    """Gate rows that make every gate huge and positive: sigmoid = 1, so the gated layer equals
    the same layer without a gate (a wrong gate slice, or a gate through silu, fails)."""
    spec, mg, mu, wl, x, xq = _gated_pair(201)
    _set_gate_rows(mg, spec, xq, [1] * spec.n_head)
    yg = oracle.decode_step(mg, oracle.OracleCaches(wl), x, [0], wl.positions(0), blocks=True)
    yu = oracle.decode_step(mu, oracle.OracleCaches(wl), x, [0], wl.positions(0), blocks=True)
    np.testing.assert_array_equal(yg, yu)


def test_output_gate_zero_halves_the_attention_contribution():
    """Gate rows of zeros: every gate is 0, sigmoid = 1/2 exactly; halving the attention output
    halves its block scales and keeps its codes, so the o product's contribution to the
    residual is exactly half the ungated one."""
    spec, mg, mu, wl, x, xq = _gated_pair(202)
    _set_gate_rows(mg, spec, xq, [0] * spec.n_head)
    tg, tu = [], []
    oracle.decode_step(mg, oracle.OracleCaches(wl), x, [0], wl.positions(0), blocks=True, trace=tg)
    oracle.decode_step(mu, oracle.OracleCaches(wl), x, [0], wl.positions(0), blocks=True, trace=tu)
    x0 = x.astype(np.float64)
    og, ou = tg[0]["x1"] - x0, tu[0]["x1"] - x0
    assert np.abs(ou).max() > 1e-3
    np.testing.assert_allclose(og, 0.5 * ou, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(tg[0]["attn"], 0.5 * tu[0]["attn"], rtol=1e-15, atol=0)


def test_output_gate_closed_head_removes_that_head():
    """Head 0's gate huge and negative (sigmoid = 0), the others huge and positive: the gated
    layer equals the ungated layer whose o matrix has head 0's input columns zeroed (a gate
    applied to the wrong head, or after the o product, fails)."""
    spec, mg, mu, wl, x, xq = _gated_pair(203)
    _set_gate_rows(mg, spec, xq, [-1] + [1] * (spec.n_head - 1))
    hd = spec.head_dim
    wo = mu["layers"][0]["wo"]
    qs = wo["qs"].copy()
    qs[:, :hd] = 0
    mu["layers"][0] = {**mu["layers"][0], "wo": {**wo, "qs": qs}}
    yg = oracle.decode_step(mg, oracle.OracleCaches(wl), x, [0], wl.positions(0), blocks=True)
    yu = oracle.decode_step(mu, oracle.OracleCaches(wl), x, [0], wl.positions(0), blocks=True)
    np.testing.assert_allclose(yg, yu, rtol=1e-12, atol=1e-12 * np.abs(yu).max())
    # and it differs from the fully open gate by head 0's contribution
    _set_gate_rows(mg, spec, xq, [1] * spec.n_head)
    yo = oracle.decode_step(mg, oracle.OracleCaches(wl), x, [0], wl.positions(0), blocks=True)
    assert np.abs(yo - yg).max() > 1e-3


def test_forced_codes_accept_exactly_the_valid_roundings():
    """Teacher forcing of the quantiser: the oracle's own codes change nothing (no flip, no
    invalid code, the same step output); a code one step off where the value is far from a
    rounding boundary is counted invalid; at a value within the tolerance of a boundary both
    neighbouring codes are accepted, the other one counted as a flip."""
    from oracle.step import _q_forced
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 64))
    q0, d0 = ops.quantize_act(x.astype(np.float32))
    rec = []
    q, d = _q_forced(x, q0, rec, "own")
    assert np.array_equal(q, q0) and np.array_equal(d, d0)
    assert rec[-1]["flips"] == 0 and rec[-1]["invalid"] == 0
    # one code one step off, away from a boundary
    ratio = x.astype(np.float32)[0, :32] / d0[0, 0]
    i = int(np.argmin(np.abs(ratio - np.round(ratio))))          # closest to an integer: mid-cell
    bad = q0.astype(np.int64).copy()
    bad[0, i] += 1 if bad[0, i] < 127 else -1
    _q_forced(x, bad, rec, "bad")
    assert rec[-1]["invalid"] == 1
    # a value on a boundary: block amax 127 d, and an element at (k + 1/2) d exactly
    xb = np.zeros((1, 32))
    xb[0, 0] = 127.0
    xb[0, 1] = 10.5
    qb, _ = ops.quantize_act(xb.astype(np.float32))
    assert qb[0, 1] == 11                                        # half away from zero
    alt = qb.astype(np.int64).copy()
    alt[0, 1] = 10
    _q_forced(xb, alt, rec, "tie")
    assert rec[-1]["invalid"] == 0 and rec[-1]["flips"] == 1
    alt[0, 1] = 12
    _q_forced(xb, alt, rec, "two off")
    assert rec[-1]["invalid"] == 1
    # a whole layer forced with its own codes equals the unforced layer
    wl = _tiny_wl(TINY, 97, [(0, 0), (1, 0)], [9, 30])
    model = wlmod.make_model(TINY, 97)
    xin = wlmod.step_inputs(wl, 0).astype(np.float64)
    tr = []
    y = oracle.decode_layer(model, 0, oracle.OracleCaches(wl), xin, [0, 1], wl.positions(0), trace=tr)
    L = model["layers"][0]
    xn = ops.rmsnorm(xin, L["attn_norm"], TINY.rms_eps)
    attn = tr[0]["attn"].reshape(2, -1)
    z = ops.rmsnorm(tr[0]["x1"], L["ffn_norm"], TINY.rms_eps)
    zq, zd = ops.quantize_act(z.astype(np.float32))
    g = ops.mmvq(L["w_gate"], zq, zd)
    u = ops.mmvq(L["w_up"], zq, zd)
    forced = {"attn_in": ops.quantize_act(xn.astype(np.float32))[0],
              "attn_out": ops.quantize_act(attn.astype(np.float32))[0], "ffn_in": zq,
              "ffn_mid": ops.quantize_act(ops.swiglu(g, u).astype(np.float32))[0]}
    rec = []
    yf = oracle.decode_layer(model, 0, oracle.OracleCaches(wl), xin, [0, 1], wl.positions(0), forced=forced,
                             record=rec)
    np.testing.assert_array_equal(yf, y)
    assert [r["what"] for r in rec] == ["attn in", "attn out", "ffn in", "ffn mid"]
    assert all(r["flips"] == 0 and r["invalid"] == 0 for r in rec)


def test_verify_rows_equal_sequential_steps():
    # A stream's 4 draft rows in one step (append all, then attend) equal 4 sequential
    # single-row steps at positions L..L+3 (Strata #1524 "Fresh validation": solo and batch
    # tokens matched; memra-engine decode_batch.rs: phase A then phase B).
    spec = TINY
    wl = _tiny_wl(spec, 93, [(0, j) for j in range(4)], [11])
    model = wlmod.make_model(spec, 93)
    x = wlmod.step_inputs(wl, 0)
    cb = oracle.OracleCaches(wl)
    yb = oracle.decode_step(model, cb, x, [0] * 4, wl.positions(0), blocks=True)
    cs = oracle.OracleCaches(wl)
    ys = np.concatenate([oracle.decode_step(model, cs, x[j:j + 1], [0], [11 + j], blocks=True) for j in range(4)])
    np.testing.assert_allclose(yb, ys, rtol=1e-12, atol=1e-12 * np.abs(ys).max())
    for il in range(spec.n_layers):
        np.testing.assert_array_equal(cb.K[0][il], cs.K[0][il])
        np.testing.assert_array_equal(cb.V[0][il], cs.V[0][il])


def test_rows_are_isolated_in_the_oracle():
    spec = TINY
    wl = _tiny_wl(spec, 94, [(0, 0), (1, 0)], [9, 30])
    model = wlmod.make_model(spec, 94)
    x = wlmod.step_inputs(wl, 0)
    y2 = oracle.decode_step(model, oracle.OracleCaches(wl), x, [0, 1], wl.positions(0), blocks=True)
    y1 = oracle.decode_step(model, oracle.OracleCaches(wl), x[1:], [1], [30], blocks=True)
    np.testing.assert_allclose(y2[1], y1[0], rtol=1e-12, atol=1e-12 * np.abs(y1).max())


def test_append_writes_exactly_one_slot_per_row():
    spec = TINY
    wl = _tiny_wl(spec, 95, [(0, 0), (1, 0)], [9, 30])
    model = wlmod.make_model(spec, 95)
    c = oracle.OracleCaches(wl)
    before = [[k.copy() for k in c.K[s]] for s in (0, 1)]
    oracle.decode_step(model, c, wlmod.step_inputs(wl, 0), [0, 1], wl.positions(0))
    for s, p in ((0, 9), (1, 30)):
        for il in range(spec.n_layers):
            diff = np.any(c.K[s][il] != before[s][il], axis=(0, 2))
            assert diff.nonzero()[0].tolist() == [p]


def test_workload_determinism():
    a = wlmod.make_model(TINY, 7)
    b = wlmod.make_model(TINY, 7)
    assert np.array_equal(a["layers"][1]["w_down"]["qs"], b["layers"][1]["w_down"]["qs"])
    wl = wlmod.workload("c1")
    assert np.array_equal(wlmod.step_inputs(wl, 0), wlmod.step_inputs(wl, 0))
    assert wl.positions(0) == [17, 40]
    lens = wlmod.c3_lengths(0)
    assert all(512 <= t <= 32768 for t in lens) and len(set(lens)) > 8


def test_deep_step_is_discontinuous_at_rounding_level():
    """The step is discontinuous (int8 activation codes): a 3e-7 relative perturbation of the
    input rows -- the size of fp32 evaluation error -- changes some rows of a deep stack's
    output by over 1e-4 (a >300x amplification no continuous evaluation of this stack shows)
    once a code flips and later codes follow, and the spread stays at the quantisation-noise
    level.  This is the evidence behind the whole-step tolerance for deep stacks (fp32 GPU
    path vs fp64 oracle)."""
    spec = wlmod.ModelSpec("deep", 8, 256, 4, 2, 64, 512, "q8_0", vocab=512, final_norm=True)
    rows = 32
    wl = _tiny_wl(spec, 96, [(b, 0) for b in range(rows)], [40] * rows, cap=48)
    model = wlmod.make_model(spec, 96)
    x = wlmod.step_inputs(wl, 0).astype(np.float64)
    ya = oracle.decode_step(model, oracle.OracleCaches(wl), x, list(range(rows)), wl.positions(0))
    xp = (x * (1 + 3e-7 * np.random.default_rng(0).standard_normal(x.shape))).astype(np.float32)
    yb = oracle.decode_step(model, oracle.OracleCaches(wl), xp, list(range(rows)), wl.positions(0))
    nw = np.sqrt(((ya - yb) ** 2).sum(1) / (ya ** 2).sum(1))
    assert nw.max() > 1e-4          # some rows cascade far beyond the input perturbation
    assert np.median(nw) < 1e-5     # most rows see no flip at all
    assert nw.max() < 2e-2          # and the spread saturates at the quantisation-noise level


# ---------------------------------------------------------------------------------------
# FP8 E4M3 KV codec
# ---------------------------------------------------------------------------------------
def test_e4m3_values_hand_cases_and_order():
    """Worked codes of the OCP E4M3 layout (sign, 4-bit exponent with bias 7, 3-bit mantissa)."""
    v = oracle.e4m3_values()
    hand = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
            0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, x in hand.items():
        assert v[c] == x, hex(c)
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.all(np.diff(v[:0x7F]) > 0)                      # codes order like their values
    np.testing.assert_array_equal(v[0x80:0xFF], -v[:0x7F])    # sign bit mirrors (0x80 is -0)
    assert np.signbit(v[0x80])


def test_e4m3_matches_torch_float8():
    """Every code decodes as torch.float8_e4m3fn does; in-range values encode as torch rounds
    them (nearest, ties to even)."""
    torch = pytest.importorskip("torch")
    c = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    t = c.view(torch.float8_e4m3fn).double().numpy()
    v = oracle.e4m3_values()
    np.testing.assert_array_equal(np.isnan(t), np.isnan(v))
    np.testing.assert_array_equal(t[~np.isnan(t)], v[~np.isnan(v)])
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(50000) * np.exp2(rng.uniform(-12, 8, 50000))).astype(np.float32)
    x = x[np.abs(x) < 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_encode(x.astype(np.float64)), ref)


def test_e4m3_encode_ties_saturation_and_round_trip():
    enc = oracle.e4m3_encode
    # ties go to the even mantissa: 1.0625 between 1.0 (m 0) and 1.125 (m 1) -> 1.0;
    # 1.1875 between 1.125 and 1.25 -> 1.25; 2^-10 between 0 and 2^-9 -> 0; 3 2^-10 -> 2^-8
    assert enc(np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10])).tolist() == [0x38, 0x3A, 0x00, 0x02]
    # past 448: saturate (464 is the midpoint to the NaN code's slot)
    assert enc(np.array([448.0, 449.0, 464.0, 1e6, -1e6])).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert enc(np.array([-0.0, 0.0, np.nan])).tolist() == [0x80, 0x00, 0x7F]
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    np.testing.assert_array_equal(enc(oracle.e4m3_decode(finite)), finite)


def test_oracle_fp8_step_appends_nearest_codes_and_attends_their_values():
    """With FP8 caches the oracle's append writes, at each row's position, the E4M3 code
    nearest each traced k and v value, and nothing else; its attention output equals the
    fp16-cache step's when that step's caches hold the same values (a one-layer model)."""
    import dataclasses
    base = wlmod.workload("c1")
    wl = dataclasses.replace(base, spec=dataclasses.replace(base.spec, kv_fp8=True))
    model = wlmod.make_model(wl.spec, wl.code, wl.seed)
    oc = oracle.OracleCaches(wl)
    before = [oc.K[s][0].copy() for s in range(2)]
    trace = []
    x = wlmod.step_inputs(wl, 0)
    pos = wl.positions(0)
    oracle.decode_step(model, oc, x, [0, 1], pos, trace=trace)
    for b in range(2):
        K = oc.K[b][0]
        np.testing.assert_array_equal(K[:, pos[b]], oracle.e4m3_encode(trace[0]["k"][b]))
        np.testing.assert_array_equal(oracle.e4m3_encode(trace[0]["v"][b]), oc.V[b][0][:, pos[b]])
        mask = np.ones(K.shape[1], bool)
        mask[pos[b]] = False
        np.testing.assert_array_equal(K[:, mask], before[b][:, mask])
        # attention over the decoded codes, from the traced q
        ref = oracle.attention(trace[0]["q"][b], oracle.e4m3_decode(K), oracle.e4m3_decode(oc.V[b][0]), pos[b] + 1)
        np.testing.assert_allclose(trace[0]["attn"][b], ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------
# Gated delta rule
# ---------------------------------------------------------------------------------------
def _gdn_inputs(seed, H=3, dk=8, dv=6):
    r = np.random.default_rng(seed)
    S = r.standard_normal((H, dv, dk))
    q = r.standard_normal((H, dk))
    k = r.standard_normal((H, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = r.standard_normal((H, dv))
    g = -r.uniform(0.01, 1.0, H)
    beta = r.uniform(0.1, 0.9, H)
    return S, q, k, v, g, beta


def test_gdn_delta_rule_writes_v_at_k():
    """No decay and beta = 1 with a unit key: afterwards the state recalls exactly v at k,
    and leaves every direction orthogonal to k unchanged."""
    S, q, k, v, g, beta = _gdn_inputs(1)
    Sn, _ = oracle.gdn_step(S, q, k, v, np.zeros(3), np.ones(3), 1.0)
    np.testing.assert_allclose(np.einsum("hvk,hk->hv", Sn, k), v, rtol=0, atol=1e-12)
    r = np.random.default_rng(2).standard_normal((3, 8))
    r -= np.sum(r * k, axis=1, keepdims=True) * k                # orthogonal to k
    np.testing.assert_allclose(np.einsum("hvk,hk->hv", Sn, r), np.einsum("hvk,hk->hv", S, r), rtol=0, atol=1e-12)


def test_gdn_special_cases_and_matrix_form():
    S, q, k, v, g, beta = _gdn_inputs(3)
    # beta = 0: pure decay
    Sn, o = oracle.gdn_step(S, q, k, v, g, np.zeros(3), 0.5)
    np.testing.assert_allclose(Sn, np.exp(g)[:, None, None] * S, rtol=1e-15)
    np.testing.assert_allclose(o, 0.5 * np.einsum("hvk,hk->hv", Sn, q), rtol=1e-14)
    # the closed matrix form a S (I - beta k k^T) + beta v k^T, written per head with numpy
    Sn, o = oracle.gdn_step(S, q, k, v, g, beta, 0.25)
    for h in range(3):
        I = np.eye(8)
        ref = np.exp(g[h]) * S[h] @ (I - beta[h] * np.outer(k[h], k[h])) + beta[h] * np.outer(v[h], k[h])
        np.testing.assert_allclose(Sn[h], ref, rtol=0, atol=1e-13)
        np.testing.assert_allclose(o[h], 0.25 * ref @ q[h], rtol=0, atol=1e-13)
    # zero state: the state becomes beta v k^T
    Sn, _ = oracle.gdn_step(np.zeros_like(S), q, k, v, g, beta, 1.0)
    np.testing.assert_allclose(Sn, beta[:, None, None] * v[:, :, None] * k[:, None, :], rtol=1e-15)


# ---------------------------------------------------------------------------------------
# int8 (Q8_0-block) KV cache codec
# ---------------------------------------------------------------------------------------
def test_q8_kv_hand_worked_row():
    """One 64-value row by hand: block 0 has max |x| = 63.5, so d = 0.5 exactly and the codes
    are x / 0.5 with ties away from zero; block 1 is all zero (scale 0, codes 0); 16 bytes of
    padding follow the two fp16 scales."""
    x = np.zeros(64, dtype=np.float32)
    x[:6] = [63.5, -63.5, 0.75, -1.25, 0.2, 10.0]      # x / d = 127, -127, 1.5, -2.5, 0.4, 20
    row = ops.q8_kv_encode(x)
    assert row.shape == (80,) and ops.q8_kv_row_bytes(64) == 80
    codes = row[:64].view(np.int8)
    assert codes[:6].tolist() == [127, -127, 2, -3, 0, 20] and not codes[6:].any()
    d = row[64:68].view(np.float16)
    assert d[0] == np.float16(0.5) and d[1] == 0
    assert not row[68:].any()
    np.testing.assert_array_equal(ops.q8_kv_decode(row, 64)[:6], [63.5, -63.5, 1.0, -1.5, 0.0, 10.0])


def test_q8_kv_scale_is_rounded_to_fp16_before_coding():
    """The stored scale is fp16(max/127) and the codes divide by that stored value: for a block
    with max 1.0 the scale is fp16(1/127) = 0.0078735..., and 1.0 / it = 127.0078 -> 127."""
    x = np.linspace(-1.0, 1.0, 32, dtype=np.float32)
    row = ops.q8_kv_encode(x)
    d = row[32:34].view(np.float16)[0]
    assert d == np.float16(np.float32(1.0) / np.float32(127.0))
    q = row[:32].view(np.int8)
    assert q[0] == -127 and q[-1] == 127
    ref = np.clip(np.sign(x / np.float32(d)) * np.floor(np.abs(x / np.float32(d)) + 0.5), -127, 127)
    np.testing.assert_array_equal(q, ref.astype(np.int8))


def test_q8_kv_round_trip_bound_and_row_independence():
    """Decoded values are within half a step of the input (d/2 per block, plus the scale's
    fp16 rounding for the clamped maximum); rows code independently of one another."""
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((5, 3, 128)) * np.exp(rng.uniform(-3, 3, (5, 3, 1)))).astype(np.float32)
    rows = ops.q8_kv_encode(x)
    y = ops.q8_kv_decode(rows, 128)
    d = rows[..., 128:136].copy().view(np.float16).astype(np.float64)           # [5, 3, 4]
    err = np.abs(y - x).reshape(5, 3, 4, 32)
    amax = np.abs(x).reshape(5, 3, 4, 32).max(axis=3)
    bound = np.maximum(d / 2, np.abs(amax - 127 * d))[..., None] * (1 + 1e-6)
    assert np.all(err <= bound)
    np.testing.assert_array_equal(ops.q8_kv_encode(x[2, 1]), rows[2, 1])


def test_oracle_q8_step_appends_encoded_rows():
    """A step of a stack with int8 caches writes, at each row's position, exactly the Q8 rows of
    the k and v it computed (the trace's fp32 values), and leaves every other slot as it was."""
    import dataclasses
    spec = dataclasses.replace(TINY, kv_q8=True)
    wl = _tiny_wl(spec, 98, [(0, 0), (1, 0)], [9, 30])
    model = wlmod.make_model(spec, 98)
    c = oracle.OracleCaches(wl)
    assert c.K[0][0].shape == (spec.n_head_kv, wl.capacity, spec.head_dim + 16) and c.K[0][0].dtype == np.uint8
    before = [[k.copy() for k in c.K[s]] for s in (0, 1)]
    tr = []
    oracle.decode_step(model, c, wlmod.step_inputs(wl, 0), [0, 1], wl.positions(0), trace=tr)
    for s, p in ((0, 9), (1, 30)):
        for il in range(spec.n_layers):
            diff = np.any(c.K[s][il] != before[s][il], axis=(0, 2))
            assert diff.nonzero()[0].tolist() == [p]
            np.testing.assert_array_equal(c.K[s][il][:, p], ops.q8_kv_encode(tr[il]["k"][s].astype(np.float32)))
            np.testing.assert_array_equal(c.V[s][il][:, p], ops.q8_kv_encode(tr[il]["v"][s].astype(np.float32)))


# ---------------------------------------------------------------------------------------
# Linear-attention layer pieces (conv ring, prep, gated norm) and the hybrid stack
# ---------------------------------------------------------------------------------------
def test_ssm_conv_step_by_hand_and_ring_shift():
    """Two channels, width 4: channel 0 weights (1, 0, 0, 1) add the oldest held input and the
    new one, channel 1 weights 0.5 each average the window; the ring then holds the newest 3."""
    state = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    w = np.array([[1.0, 0.0, 0.0, 1.0], [0.5, 0.5, 0.5, 0.5]])
    y, st = ops.ssm_conv_step(state, np.array([7.0, 8.0]), w)
    pre = np.array([1.0 + 7.0, 0.5 * (2 + 4 + 6 + 8)])
    np.testing.assert_allclose(y, pre / (1 + np.exp(-pre)), rtol=1e-15)
    np.testing.assert_array_equal(st, [[3.0, 4.0], [5.0, 6.0], [7.0, 8.0]])
    # a kernel that takes only the newest input passes it through silu; the ring keeps shifting
    y2, st2 = ops.ssm_conv_step(st, np.array([-1.0, 0.0]), np.array([[0, 0, 0, 1.0], [0, 0, 0, 1.0]]))
    np.testing.assert_allclose(y2, [-1.0 / (1 + np.e), 0.0], rtol=1e-15)
    np.testing.assert_array_equal(st2, [[5.0, 6.0], [7.0, 8.0], [-1.0, 0.0]])


def test_gdn_prep_heads_norms_gate_and_decay():
    """Key heads serve consecutive value heads (h // (n_v / n_k)); q and k leave with unit norm
    (up to eps); beta = sigmoid(beta_raw); g = a softplus(alpha + dt): a ln 2 at 0, about a x
    for large x, and tends to 0 for very negative x."""
    rng = np.random.default_rng(12)
    ds, nk, nv = 8, 2, 4
    c = rng.standard_normal(2 * nk * ds + nv * ds)
    q, k, v, g, beta = ops.gdn_prep(c, np.array([0.0, 2.0, -3.0, 40.0]), np.array([0.0, 30.0, -50.0, 1.0]),
                                    np.array([0.0, 0.0, 0.0, -1.0]), np.array([-1.0, -0.5, -2.0, -1.0]), ds, nk, nv,
                                    1e-12)
    qh = c[:nk * ds].reshape(nk, ds)
    np.testing.assert_allclose(q[0], qh[0] / np.linalg.norm(qh[0]), rtol=1e-12)
    np.testing.assert_allclose(q[1], q[0], rtol=0)
    np.testing.assert_allclose(q[2], qh[1] / np.linalg.norm(qh[1]), rtol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(k, axis=1), 1.0, rtol=1e-12)
    np.testing.assert_array_equal(v, c[2 * nk * ds:].reshape(nv, ds))
    np.testing.assert_allclose(beta, [0.5, 1 / (1 + np.exp(-2.0)), 1 / (1 + np.exp(3.0)), 1.0], rtol=1e-15)
    np.testing.assert_allclose(g[0], -np.log(2.0), rtol=1e-15)
    np.testing.assert_allclose(g[1], -0.5 * 30.0, rtol=1e-12)
    assert -1e-20 < g[2] < 0
    np.testing.assert_allclose(g[3], -np.log(2.0), rtol=1e-15)    # alpha + dt = 0


def test_gated_rmsnorm_cases_and_torch():
    """z = 0 closes the gate; a constant head normalises to the gain times silu(z); random rows
    equal torch's rms_norm times silu in fp64."""
    w = np.array([1.0, 2.0, 0.5, 1.0])
    o = np.full((2, 4), 3.0)
    np.testing.assert_array_equal(ops.gated_rmsnorm(o, w, np.zeros((2, 4)), 0.0), np.zeros((2, 4)))
    z = np.array([[1.0, 1.0, 1.0, 1.0], [-2.0, 0.0, 2.0, 4.0]])
    np.testing.assert_allclose(ops.gated_rmsnorm(o, w, z, 0.0), w * z / (1 + np.exp(-z)), rtol=1e-14)
    rng = np.random.default_rng(13)
    o, z, w = rng.standard_normal((3, 5, 16)), rng.standard_normal((3, 5, 16)), rng.standard_normal(16)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(o), (16,), torch.from_numpy(w), eps=1e-5) * \
        torch.nn.functional.silu(torch.from_numpy(z))
    np.testing.assert_allclose(ops.gated_rmsnorm(o, w, z, 1e-5), ref.numpy(), rtol=1e-12)


def _tiny_hybrid():
    import dataclasses
    return dataclasses.replace(TINY, linear_layers=(0,), ssm_d_state=32, ssm_n_k=1, ssm_n_v=2, ssm_d_conv=4)


def test_hybrid_stack_rows_isolated_and_state_carried():
    """A two-layer stack whose first layer is a gated delta-rule layer: each row's output does
    not depend on the other rows; the recurrent state after two steps equals the state step
    applied twice to the same inputs, and it enters the second step (a restarted second step
    from the prefill state differs)."""
    spec = _tiny_hybrid()
    wl = _tiny_wl(spec, 99, [(0, 0), (1, 0)], [9, 30])
    model = wlmod.make_model(spec, 99)
    assert model["layers"][0]["mixer"] == "linear" and model["layers"][0]["wqkv"]["n"] == spec.ssm_in_rows
    x = wlmod.step_inputs(wl, 0)
    c2 = oracle.OracleCaches(wl)
    y2 = oracle.decode_step(model, c2, x, [0, 1], wl.positions(0), blocks=True)
    c1 = oracle.OracleCaches(wl, sessions=[1])
    y1 = oracle.decode_step(model, c1, x[1:], [1], [30], blocks=True)
    np.testing.assert_allclose(y2[1], y1[0], rtol=1e-12, atol=1e-12 * np.abs(y1).max())
    np.testing.assert_allclose(c2.R[1][0]["S"], c1.R[1][0]["S"], rtol=1e-13, atol=1e-15)
    # step 2 from the carried state vs from the prefill state
    x1 = wlmod.step_inputs(wl, 1)
    ya = oracle.decode_step(model, c2, x1, [0, 1], wl.positions(1), blocks=True)
    yb = oracle.decode_step(model, oracle.OracleCaches(wl), x1, [0, 1], wl.positions(1), blocks=True)
    assert np.abs(ya - yb).max() > 1e-6


def test_hybrid_block_formula_equals_dense_formulation():
    """The hybrid stack through the block formula of every product equals the dense fp64
    formulation (as for the attention stacks)."""
    spec = _tiny_hybrid()
    wl = _tiny_wl(spec, 100, [(0, 0), (1, 0)], [5, 20])
    model = wlmod.make_model(spec, 100)
    x = wlmod.step_inputs(wl, 0)
    ys = [oracle.decode_step(model, oracle.OracleCaches(wl), x, [0, 1], wl.positions(0), blocks=blk)
          for blk in (True, False)]
    np.testing.assert_allclose(ys[0], ys[1], rtol=1e-10, atol=1e-10 * np.abs(ys[1]).max())


def test_dense_step_against_a_torch_composition():
    """The whole two-layer step (with lm_head) against the same step composed from torch's own
    routines in fp64: F.rms_norm, matmul with the dequantised weights, the rotate-half form of
    NEOX RoPE, scaled_dot_product_attention with GQA over each row's cache (every append of
    the layer first), F.silu.  Only the block codecs (pinned above) are shared.  Three rows,
    two of them on one cache at consecutive positions (causal verify rows).  A slip in the
    step's wiring -- a residual in the wrong place, RoPE on v, a wrong head map, the wrong key
    count, an append after the attention -- fails it."""
    import torch.nn.functional as F
    spec = TINY
    wl = _tiny_wl(spec, 93, [(0, 0), (1, 0), (1, 1)], [5, 20])
    model = wlmod.make_model(spec, 93)
    x_np = wlmod.step_inputs(wl, 0)
    sess, pos = [0, 1, 1], wl.positions(0)
    ref = oracle.decode_step(model, oracle.OracleCaches(wl), x_np, sess, pos)

    H, G, hd, d, eps = spec.n_head, spec.n_head_kv, spec.head_dim, spec.d, spec.rms_eps
    T = torch.float64
    caches = {}
    for s in (0, 1):
        for il in range(spec.n_layers):
            k, v = wlmod.kv_prefill(wl, s, il)
            Kc = torch.zeros((G, wl.capacity, hd), dtype=T)
            Vc = torch.zeros((G, wl.capacity, hd), dtype=T)
            Kc[:, :k.shape[1]] = torch.from_numpy(k.astype(np.float64))
            Vc[:, :v.shape[1]] = torch.from_numpy(v.astype(np.float64))
            caches[s, il] = (Kc, Vc)

    def q8(t):   # the step's activation codec (pinned by the golden blocks): fp32 in, values out
        q, dd = ops.quantize_act(t.numpy().astype(np.float32))
        return torch.from_numpy(ops.dequantize_act(q, dd))

    def W(w):
        return torch.from_numpy(ops.dequantize(w))

    def rope(t, p):   # t [n, hd] at position p: rotate-half form
        inv = torch.pow(torch.tensor(10000.0, dtype=T), -torch.arange(0, hd, 2, dtype=T) / hd)
        ang = p * inv
        c, s_ = torch.cat([torch.cos(ang)] * 2), torch.cat([torch.sin(ang)] * 2)
        rot = torch.cat([-t[:, hd // 2:], t[:, :hd // 2]], dim=1)
        return t * c + rot * s_

    x = torch.from_numpy(x_np.astype(np.float32).astype(np.float64))
    for il, L in enumerate(model["layers"]):
        g = lambda name: torch.from_numpy(L[name].astype(np.float64))
        xv = q8(F.rms_norm(x, (d,), weight=g("attn_norm"), eps=eps))
        qkv = xv @ W(L["wqkv"]).T
        q = qkv[:, :H * hd].reshape(-1, H, hd)
        k = qkv[:, H * hd:(H + G) * hd].reshape(-1, G, hd)
        v = qkv[:, (H + G) * hd:(H + 2 * G) * hd].reshape(-1, G, hd)
        qs = [rope(q[b], pos[b]) for b in range(3)]
        for b in range(3):   # every row's append before any attention, fp16 cache values
            Kc, Vc = caches[sess[b], il]
            Kc[:, pos[b]] = rope(k[b], pos[b]).to(torch.float16).to(T)
            Vc[:, pos[b]] = v[b].to(torch.float16).to(T)
        att = []
        for b in range(3):
            Kc, Vc = caches[sess[b], il]
            t = pos[b] + 1
            o = F.scaled_dot_product_attention(qs[b][None, :, None, :], Kc[None, :, :t], Vc[None, :, :t],
                                               scale=hd ** -0.5, enable_gqa=True)
            att.append(o[0, :, 0].reshape(H * hd))
        x1 = x + q8(torch.stack(att)) @ W(L["wo"]).T
        zv = q8(F.rms_norm(x1, (d,), weight=g("ffn_norm"), eps=eps))
        h = F.silu(zv @ W(L["w_gate"]).T) * (zv @ W(L["w_up"]).T)
        x = x1 + q8(h) @ W(L["w_down"]).T
    fn = torch.from_numpy(model["final_norm"].astype(np.float64))
    logits = q8(F.rms_norm(x, (d,), weight=fn, eps=eps)) @ W(model["lm_head"]).T
    np.testing.assert_allclose(logits.numpy(), ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())

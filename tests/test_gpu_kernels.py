"""Per-kernel parity of the HIP path against the CPU oracle (MI355X only).

Integers (quantised codes, per-block int32 dot products) and fp16 KV bytes must match
exactly; fp32 results within 2e-3 of the oracle's fp64 value (per-row scaled); every
row of a B-row call must equal, bit for bit, the 1-row call on that row.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import ops
import workload as W
from gpu_util import assert_close_rows, requires_gpu, say, untile_act

pytestmark = [pytest.mark.gpu, requires_gpu]

kd = pytest.importorskip("session_decode_step_amd")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def sync():
    torch.cuda.synchronize()


def _drawer(fmt):
    """The seeded matrix draw of a weight format, as f(rq, rd, n, k)."""
    if fmt in W.KQ_RECORD:
        return lambda rq, rd, n, k: W.draw_kquant(fmt, rq, rd, n, k)
    return W.draw_q8_0 if fmt == "q8_0" else W.draw_q4_0


def product_fn(fmt):
    """The plain product entry point of a format (the K-quants go through kd_mmvq)."""
    return {"q8_0": kd.kd_mmvq_q8_0, "q4_0": kd.kd_mmvq_q4_0}.get(fmt, kd.kd_mmvq)


# ------------------------------------------------------------------ activation quantiser
@pytest.mark.parametrize("B,k", [(1, 256), (5, 704), (16, 2048), (3, 14336)])
def test_act_quant_codes_and_scales_exact(B, k):
    say(f"act_quant B={B} k={k}")
    r = np.random.default_rng(100 + k)
    x = (r.standard_normal((B, k)) * np.exp(r.uniform(-4, 4, (B, 1)))).astype(np.float32)
    x[0, 32:64] = 0.0                                           # a zero block
    x[0, 64] = 127.0
    x[0, 65:69] = [0.5, -0.5, 2.5, -2.5]                         # exact ties (scale 1)
    act = kd.kd_quantize_act_q8(dev(x))
    sync()
    codes, sc, pad_codes, pad_sc = untile_act(act.qs, act.d, B, k)
    q_ref, d_ref = ops.quantize_act(x)
    np.testing.assert_array_equal(sc, d_ref)
    np.testing.assert_array_equal(codes, q_ref)
    assert np.all(pad_codes == 0) and np.all(pad_sc == 0)


# ------------------------------------------------------------------ mmvq
# ragged shapes, the 32-layer stack's O (4096 x 4096) and down (4096 x 14336: 14 waves of 8
# quads) products, the 8-layer stack's lm_head (32000 x 2048 Q8_0) and the largest k (16384)
SHAPES = [("q8_0", 100, 704), ("q8_0", 512, 2048), ("q4_0", 100, 704), ("q4_0", 4096, 4096), ("q8_0", 48, 256),
          ("q4_0", 4096, 14336), ("q8_0", 32000, 2048), ("q4_0", 272, 16384)]
# K-quants (k a multiple of 256): ragged rows, one record per row, an odd number of records
# (a quad pair split across waves), the 8-layer mixed stack's shapes and the largest k
SHAPES_KQ = [("q4_k", 100, 768), ("q5_k", 48, 256), ("q6_k", 100, 768), ("q4_k", 4096, 4096), ("q5_k", 3072, 2048),
             ("q6_k", 2048, 5632), ("q6_k", 32000, 2048), ("q4_k", 272, 16384), ("q5_k", 2816, 2816)]


@pytest.mark.parametrize("fmt,n,k", SHAPES)
def test_block_dots_exact(fmt, n, k):
    say(f"block_dots {fmt} n={n} k={k}")
    r = np.random.default_rng(7 + n)
    w = _drawer(fmt)(r, r, n, k)
    x = r.standard_normal((16, k)).astype(np.float32)
    pw = kd.kd_pack_weight(w)
    act = kd.kd_quantize_act_q8(dev(x))
    S = kd.kd_debug_block_dots(pw, act, 16)
    sync()
    xq, _ = ops.quantize_act(x)
    np.testing.assert_array_equal(S.cpu().numpy(), ops.block_dots(w, xq))


@pytest.mark.parametrize("fmt,n,k", SHAPES + SHAPES_KQ)
def test_mmvq_matches_oracle_and_rows_are_b_invariant(fmt, n, k):
    say(f"mmvq {fmt} n={n} k={k}")
    r = np.random.default_rng(11 + n + k)
    w = _drawer(fmt)(r, r, n, k)
    x = r.standard_normal((16, k)).astype(np.float32)
    pw = kd.kd_pack_weight(w)
    act = kd.kd_quantize_act_q8(dev(x))
    fn = product_fn(fmt)
    y16 = fn(pw, act, 16)
    sync()
    xq, xd = ops.quantize_act(x)
    ref = ops.mmvq(w, xq, xd)
    assert_close_rows(y16.cpu().numpy(), ref, 2e-3, "mmvq")
    # fp32 epilogue error is far below the budget: one rounding per block
    assert_close_rows(y16.cpu().numpy(), ref, 1e-4, "mmvq tight")
    y16h = y16.cpu().numpy()
    for B in range(1, 16):
        yB = fn(pw, act, B).cpu().numpy()
        np.testing.assert_array_equal(yB, y16h[:B])
    # a row alone (its activation moved to row 0) gives the same bytes
    for b in (5, 15):
        act1 = kd.kd_quantize_act_q8(dev(x[b:b + 1]))
        y1 = fn(pw, act1, 1).cpu().numpy()
        np.testing.assert_array_equal(y1[0], y16h[b])


@pytest.mark.parametrize("fmt", ["q4_k", "q5_k", "q6_k"])
def test_kquant_tiles_hold_the_records(fmt):
    """Packed K-quant tiles against the layout kd.h states, byte by byte, decoded from the
    oracle's fields of the same records: low code nibbles, fifth / upper bits, per-block
    scale bytes and the super-block's fp16 scales (rows past n_out zero)."""
    say(f"kquant tiles {fmt}")
    r = np.random.default_rng(91)
    n, k = 20, 512
    w = W.draw_kquant(fmt, r, r, n, k)
    pw = kd.kd_pack_weight(w)
    sync()
    qs = pw.qs.cpu().numpy().view(np.uint8)
    dd = pw.d.cpu().numpy().view(np.uint8)
    f = ops.kquant_fields(w)
    TQ = {"q4_k": 1024, "q5_k": 1280, "q6_k": 1536}[fmt]
    NQ, NR = k // 128, 2
    assert qs.size == NR * NQ * TQ and dd.size == NR * NQ * 192
    codes = f["q"].reshape(n, k // 32, 32)                     # [row, block, element]
    raw = np.ascontiguousarray(w["qs"]).reshape(n, k // 256, -1)
    for row in range(NR * 16):
        rr, nn = row // 16, row % 16
        for q in range(NQ):
            t = rr * NQ + q
            for j in range(4):
                blk = 4 * q + j
                c = codes[row, blk] if row < n else np.zeros(32, np.int64)
                for g in range(4):
                    lane = 16 * g + nn
                    lo, hi = c[4 * g:4 * g + 4], c[4 * g + 16:4 * g + 20]
                    np.testing.assert_array_equal(qs[t * TQ + lane * 16 + 4 * j:t * TQ + lane * 16 + 4 * j + 4],
                                                  (lo & 15) | ((hi & 15) << 4))
                    if fmt == "q5_k":
                        want = sum(int((lo[i] >> 4) & 1) << i for i in range(4)) + \
                            sum(int((hi[i] >> 4) & 1) << (4 + i) for i in range(4))
                        assert qs[t * TQ + 1024 + lane * 4 + j] == want
                    if fmt == "q6_k":
                        assert qs[t * TQ + 1024 + lane * 8 + 2 * j] == sum(int((lo[i] >> 4) & 3) << (2 * i) for i in range(4))
                        assert qs[t * TQ + 1024 + lane * 8 + 2 * j + 1] == sum(int((hi[i] >> 4) & 3) << (2 * i)
                                                                               for i in range(4))
                sb, sub = blk // 8, blk % 8
                pair = dd[t * 192 + 8 * nn + 2 * j:t * 192 + 8 * nn + 2 * j + 2]
                if row >= n:
                    assert pair.tolist() == [0, 0]
                elif fmt == "q6_k":
                    assert pair.view(np.int8).tolist() == [int(f["sc"][row, sb, 2 * sub]), int(f["sc"][row, sb, 2 * sub + 1])]
                else:
                    assert pair.tolist() == [int(f["sc"][row, sb, sub]), int(f["m"][row, sb, sub])]
            sup = dd[t * 192 + 128 + 4 * nn:t * 192 + 128 + 4 * nn + 4]
            if row >= n:
                assert sup.tolist() == [0, 0, 0, 0]
            elif fmt == "q6_k":
                assert sup.tolist() == raw[row, q // 2, 208:210].tolist() + [0, 0]
            else:
                assert sup.tolist() == raw[row, q // 2, 0:4].tolist()


def test_mmvq_rejects_wrong_format():
    r = np.random.default_rng(3)
    w = W.draw_q8_0(r, r, 16, 64)
    pw = kd.kd_pack_weight(w)
    act = kd.kd_quantize_act_q8(dev(np.ones((1, 64), np.float32)))
    with pytest.raises(kd.KdError):
        kd.kd_mmvq_q4_0(pw, act, 1)


# ------------------------------------------------------------------ row ops
def test_rmsnorm_and_add_rmsnorm():
    say("rmsnorm")
    r = np.random.default_rng(5)
    x = r.standard_normal((7, 2816)).astype(np.float32)
    res = r.standard_normal((7, 2816)).astype(np.float32)
    g = (1 + 0.1 * r.standard_normal(2816)).astype(np.float32)
    y = kd.kd_rmsnorm_rows(dev(x), dev(g), 1e-5).cpu().numpy()
    assert_close_rows(y, ops.rmsnorm(x, g, 1e-5), 1e-5, "rmsnorm")
    x1, y2 = kd.kd_add_rmsnorm_rows(dev(x), dev(res), dev(g), 1e-5)
    np.testing.assert_array_equal(x1.cpu().numpy(), x + res)
    assert_close_rows(y2.cpu().numpy(), ops.rmsnorm((x + res).astype(np.float64), g, 1e-5), 1e-5, "add_rmsnorm")
    # row invariance
    y1 = kd.kd_rmsnorm_rows(dev(x[3:4]), dev(g), 1e-5).cpu().numpy()
    np.testing.assert_array_equal(y1[0], y[3])


def test_rope_per_row_positions():
    say("rope")
    r = np.random.default_rng(6)
    for hd in (64, 128):
        x = r.standard_normal((4, 6, hd)).astype(np.float32)
        pos = [0, 17, 4096, 32768]
        t = dev(x)
        kd.kd_rope_neox_rows(t, pos, 10000.0)
        got = t.cpu().numpy()
        ref = np.stack([ops.rope_neox(x[b], pos[b], 10000.0) for b in range(4)])
        np.testing.assert_array_equal(got[0], x[0])  # pos 0 is the identity
        assert_close_rows(got, ref, 1e-5, f"rope hd={hd}")


def test_swiglu_and_add():
    say("swiglu")
    r = np.random.default_rng(8)
    g = (3 * r.standard_normal((5, 704))).astype(np.float32)
    u = r.standard_normal((5, 704)).astype(np.float32)
    a = kd.kd_swiglu_rows(dev(g), dev(u)).cpu().numpy()
    assert_close_rows(a, ops.swiglu(g, u), 1e-5, "swiglu")
    z = kd.kd_add_rows(dev(g), dev(u)).cpu().numpy()
    np.testing.assert_array_equal(z, g + u)


# ------------------------------------------------------------------ KV append + attention
def _caches(n, G, cap, hd):
    return [(torch.zeros((G, cap, hd), dtype=torch.float16, device="cuda"),
             torch.zeros((G, cap, hd), dtype=torch.float16, device="cuda")) for _ in range(n)]


def test_kv_append_bytes_exact():
    say("kv_append")
    r = np.random.default_rng(9)
    B, G, hd, cap = 5, 8, 128, 40
    caches = _caches(B, G, cap, hd)
    k = (r.standard_normal((B, G, hd)) * 10).astype(np.float32)
    v = r.standard_normal((B, G, hd)).astype(np.float32)
    pos = [0, 39, 7, 8, 20]
    kd.kd_kv_append(dev(k), dev(v), [c[0].data_ptr() for c in caches], [c[1].data_ptr() for c in caches], pos, cap)
    sync()
    for b in range(B):
        K = caches[b][0].cpu().numpy()
        V = caches[b][1].cpu().numpy()
        np.testing.assert_array_equal(K[:, pos[b]].view(np.uint16), k[b].astype(np.float16).view(np.uint16))
        np.testing.assert_array_equal(V[:, pos[b]].view(np.uint16), v[b].astype(np.float16).view(np.uint16))
        mask = np.ones(cap, bool)
        mask[pos[b]] = False
        assert not K[:, mask].any() and not V[:, mask].any()


@pytest.mark.parametrize("H,G,hd", [(32, 8, 128), (16, 4, 128), (4, 2, 64), (16, 8, 128), (8, 8, 64), (8, 1, 128), (16, 2, 64)])
def test_fa_decode_ragged_vs_oracle(H, G, hd):
    say(f"fa H={H} G={G} hd={hd}")
    r = np.random.default_rng(H * 100 + G)
    t_kv = [1, 2, 127, 128, 129, 300, 1238, 5000]
    B, cap = len(t_kv), 5008
    caches = _caches(B, G, cap, hd)
    Ks, Vs = [], []
    for b in range(B):
        Kb = r.standard_normal((G, cap, hd)).astype(np.float16)
        Vb = r.standard_normal((G, cap, hd)).astype(np.float16)
        caches[b][0].copy_(torch.from_numpy(Kb))
        caches[b][1].copy_(torch.from_numpy(Vb))
        Ks.append(Kb)
        Vs.append(Vb)
    q = (r.standard_normal((B, H, hd)) * 0.5).astype(np.float32)
    kb = [c[0].data_ptr() for c in caches]
    vb = [c[1].data_ptr() for c in caches]
    scale = 1.0 / math.sqrt(hd)
    out = kd.kd_fa_decode_ragged(dev(q), G, kb, vb, t_kv, cap, scale).cpu().numpy()
    ref = np.stack([ops.attention(q[b], Ks[b], Vs[b], t_kv[b]) for b in range(B)])
    assert_close_rows(out.reshape(B, -1), ref.reshape(B, -1), 2e-3, "fa")
    assert_close_rows(out.reshape(B, -1), ref.reshape(B, -1), 1e-4, "fa tight")
    # t = 1: exactly V[0] (one key: p = 1)
    np.testing.assert_array_equal(out[0], np.stack([Vs[0][h // (H // G), 0].astype(np.float32) for h in range(H)]))
    # rows are B-invariant
    for b in (3, 7):
        o1 = kd.kd_fa_decode_ragged(dev(q[b:b + 1]), G, kb[b:b + 1], vb[b:b + 1], t_kv[b:b + 1], cap, scale)
        np.testing.assert_array_equal(o1.cpu().numpy()[0], out[b])
    # other split sizes agree within fp32 rounding; the merge adds one rounding per split,
    # so the bound grows with the split count (5000 single-key splits at chunk = 1)
    for chunk, tol in ((1, 2e-5), (37, 2e-6), (1000, 2e-6)):
        oc = kd.kd_fa_decode_ragged(dev(q), G, kb, vb, t_kv, cap, scale, chunk=chunk).cpu().numpy()
        assert_close_rows(oc.reshape(B, -1), out.reshape(B, -1), tol, f"fa chunk={chunk}")


def test_fa_row_bits_independent_of_the_split_kernel_variant():
    """A batch holding a row longer than 128 x 128 keys runs the multi-tile split kernel for
    every row; a short row stepped alone runs the single-tile one.  Its output bits agree."""
    say("fa single/multi-tile variants")
    H, G, hd = 32, 8, 128
    t_kv = [4113, 20000, 129]
    B, cap = len(t_kv), 20008
    r = np.random.default_rng(7)
    caches = _caches(B, G, cap, hd)
    for b in range(B):
        caches[b][0].copy_(torch.from_numpy(r.standard_normal((G, cap, hd)).astype(np.float16)))
        caches[b][1].copy_(torch.from_numpy(r.standard_normal((G, cap, hd)).astype(np.float16)))
    q = (r.standard_normal((B, H, hd)) * 0.5).astype(np.float32)
    kb = [c[0].data_ptr() for c in caches]
    vb = [c[1].data_ptr() for c in caches]
    scale = 1.0 / math.sqrt(hd)
    out = kd.kd_fa_decode_ragged(dev(q), G, kb, vb, t_kv, cap, scale).cpu().numpy()
    for b in (0, 2):
        o1 = kd.kd_fa_decode_ragged(dev(q[b:b + 1]), G, kb[b:b + 1], vb[b:b + 1], t_kv[b:b + 1], cap, scale)
        np.testing.assert_array_equal(o1.cpu().numpy()[0].view(np.uint32), out[b].view(np.uint32))


# ------------------------------------------------------------------ products with fused epilogues
@pytest.mark.parametrize("fmt,F,k,B", [("q4_0", 1024, 512, 8), ("q8_0", 704, 256, 5), ("q4_0", 2048, 4096, 16),
                                       ("q4_0", 352, 704, 1), ("q4_k", 1024, 512, 8), ("q6_k", 704, 2816, 3),
                                       ("q5_k", 512, 4096, 16)])
def test_mmvq_swiglu_equals_unfused_path(fmt, F, k, B):
    """The SwiGLU epilogue gives the bytes of product -> kd_swiglu_rows -> quantiser, and the
    dequantised rows match the oracle's silu(gate) * up."""
    say(f"mmvq_swiglu {fmt} F={F} k={k} B={B}")
    r = np.random.default_rng(F + k + B)
    draw = _drawer(fmt)
    gate, up = draw(r, r, F, k), draw(r, r, F, k)
    x = r.standard_normal((B, k)).astype(np.float32)
    act = kd.kd_quantize_act_q8(dev(x))
    fused = kd.kd_mmvq_swiglu(kd.kd_pack_weight(kd.interleave_gate_up(gate, up)), act, B)
    fn = product_fn(fmt)
    g = fn(kd.kd_pack_weight(gate), act, B)
    u = fn(kd.kd_pack_weight(up), act, B)
    ref_act = kd.kd_quantize_act_q8(kd.kd_swiglu_rows(g, u))
    sync()
    c1, s1, pc1, ps1 = untile_act(fused.qs, fused.d, B, F)
    c2, s2, _, _ = untile_act(ref_act.qs, ref_act.d, B, F)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s1, s2)
    assert np.all(pc1 == 0) and np.all(ps1 == 0)            # padding blocks past F
    # against the oracle (fp64 products of the same quantised input)
    q, d = ops.quantize_act(x)
    a_ref = ops.swiglu(ops.mmvq(gate, q, d), ops.mmvq(up, q, d))
    deq = (c1.reshape(B, -1, 32).astype(np.float64) * s1.reshape(B, -1, 1)).reshape(B, F)
    # one quantisation step (d/2 per element) is the only error beyond fp32 rounding
    assert np.all(np.abs(deq - a_ref) <= 0.5 * np.repeat(s1.reshape(B, -1), 32, axis=1) + 2e-3 * np.abs(a_ref) + 1e-6)


@pytest.mark.parametrize("fmt,H,G,hd,B", [("q8_0", 4, 2, 64, 2), ("q4_0", 32, 8, 128, 8), ("q4_0", 16, 8, 128, 16),
                                          ("q5_k", 32, 8, 128, 8), ("q6_k", 4, 2, 64, 2)])
def test_mmvq_rope_equals_unfused_path(fmt, H, G, hd, B):
    """The RoPE/append epilogue writes the q bits and the fp16 K/V bytes of product ->
    kd_rope_neox_rows -> kd_kv_append; rows are B-invariant."""
    say(f"mmvq_rope {fmt} H={H} G={G} hd={hd} B={B}")
    r = np.random.default_rng(H * hd + B)
    k = 512
    n = (H + 2 * G) * hd
    w = _drawer(fmt)(r, r, n, k)
    x = r.standard_normal((B, k)).astype(np.float32)
    act = kd.kd_quantize_act_q8(dev(x))
    cap = 64
    pos = [int(p) for p in r.integers(0, cap, B)]
    fused_c = _caches(B, G, cap, hd)
    plain_c = _caches(B, G, cap, hd)
    q_f = torch.zeros((B, H * hd), dtype=torch.float32, device="cuda")
    kd.kd_mmvq_rope(kd.kd_pack_weight(kd.rope_pair_rows(w, H + 2 * G, hd)), act, B, H, G, hd, q_f,
                    [c[0].data_ptr() for c in fused_c], [c[1].data_ptr() for c in fused_c], pos, cap, 10000.0)
    fn = product_fn(fmt)
    y = fn(kd.kd_pack_weight(w), act, B)
    qk = y[:, :(H + G) * hd].contiguous().view(B, H + G, hd)
    kd.kd_rope_neox_rows(qk, pos, 10000.0)
    kv_k = qk[:, H:].contiguous()
    kv_v = y[:, (H + G) * hd:].contiguous().view(B, G, hd)
    kd.kd_kv_append(kv_k, kv_v, [c[0].data_ptr() for c in plain_c], [c[1].data_ptr() for c in plain_c], pos, cap)
    sync()
    np.testing.assert_array_equal(q_f.cpu().numpy().view(np.uint32),
                                  qk[:, :H].reshape(B, H * hd).cpu().numpy().view(np.uint32))
    for b in range(B):
        for j in (0, 1):
            np.testing.assert_array_equal(fused_c[b][j].cpu().numpy().view(np.uint16),
                                          plain_c[b][j].cpu().numpy().view(np.uint16))
    # against the oracle: RoPE of the fp64 product
    q, d = ops.quantize_act(x)
    ref = ops.mmvq(w, q, d)
    qref = np.stack([ops.rope_neox(ref[b, :H * hd].reshape(H, hd), pos[b], 10000.0) for b in range(B)])
    assert_close_rows(q_f.cpu().numpy(), qref.reshape(B, -1), 2e-3, "mmvq_rope q")


# ------------------------------------------------------------------ next token
@pytest.mark.parametrize("B,n,ldx", [(1, 1, 1), (5, 33, 40), (16, 32000, 32000), (3, 100003, 100008)])
def test_argmax_rows_exact(B, n, ldx):
    """Greedy tokens equal the oracle's (first maximum) on rows with planted ties, -inf rows,
    denormals and larger values past n in the row stride (ignored); values are the maxima."""
    say(f"argmax B={B} n={n} ldx={ldx}")
    r = np.random.default_rng(n + B)
    x = r.standard_normal((B, ldx)).astype(np.float32)
    x[:, n:] = 1e30                                              # past the row: never read as logits
    for b in range(B):
        if n > 8 and b % 2 == 0:                                 # the maximum planted several times
            m = np.float32(x[b, :n].max() + 1.0)
            for j in sorted(r.choice(n, size=min(4, n), replace=False)):
                x[b, j] = m
    if B > 1 and n > 3:
        x[1, :n] = -np.inf
        x[1, n - 1] = -np.inf
    if B > 2 and n > 3:
        x[2, :n] = 0.0
        x[2, n - 2] = 1e-45                                      # a denormal maximum
    idx, val = kd.kd_argmax_rows(dev(x), n)
    ref = ops.greedy_token(x[:, :n])
    np.testing.assert_array_equal(idx.cpu().numpy(), ref)
    np.testing.assert_array_equal(val.cpu().numpy().view(np.uint32), x[np.arange(B), ref].view(np.uint32))
    # every row equals its 1-row call
    for b in range(B):
        i1, _ = kd.kd_argmax_rows(dev(x[b:b + 1]), n)
        assert int(i1.cpu()[0]) == int(ref[b])


def test_embed_rows_exact():
    """Rows of the table, bit for bit; tokens outside [0, vocab) give zero rows."""
    say("embed rows")
    r = np.random.default_rng(5)
    vocab, d = 1000, 2048
    table = r.standard_normal((vocab, d)).astype(np.float32)
    tok = np.array([0, 999, 17, 17, -1, 1000, 523], dtype=np.int32)
    out = kd.kd_embed_rows(dev(table), dev(tok)).cpu().numpy()
    ok = (tok >= 0) & (tok < vocab)
    np.testing.assert_array_equal(out[ok].view(np.uint32), ops.embed_rows(table, tok[ok]).view(np.uint32))
    assert not out[~ok].any()


def test_verify_accept_exact():
    """Accepted prefixes and next tokens equal the oracle's on random stream-major rows."""
    say("verify accept")
    r = np.random.default_rng(13)
    for n_streams, k in ((4, 4), (2, 8), (16, 1), (3, 5), (1, 16)):
        for _ in range(20):
            fed = r.integers(0, 4, size=n_streams * k).astype(np.int32)
            greedy = np.roll(fed, -1).astype(np.int32)              # agrees unless perturbed
            flip = r.random(n_streams * k) < 0.25
            greedy[flip] = r.integers(0, 4, size=int(flip.sum()))
            n_acc, nxt = kd.kd_verify_accept(dev(greedy), dev(fed), k)
            ra, rn = ops.accept_drafts(greedy, fed, k)
            np.testing.assert_array_equal(n_acc.cpu().numpy(), ra)
            np.testing.assert_array_equal(nxt.cpu().numpy(), rn)



@pytest.mark.parametrize("H,G,hd,tails", [(16, 8, 128, (8193, 4)), (32, 8, 128, (4113, 2)), (8, 8, 64, (129, 8)),
                                          (16, 8, 128, (20000, 4))])
def test_fa_rows_sharing_a_cache_match_their_solo_pass(H, G, hd, tails):
    """Rows of one cache at consecutive lengths (speculative-verify rows) take one pass over
    the keys together; every row equals its own 1-row call bit for bit, next to a row of
    another cache, also with a forced small chunk (many splits, some rows ending early)."""
    t0, n = tails
    say(f"fa shared cache H={H} G={G} hd={hd} t0={t0} rows={n}")
    r = np.random.default_rng(t0 + n)
    cap = t0 + n + 8
    shared, other = _caches(2, G, cap, hd)
    for c in (shared, other):
        c[0].copy_(torch.from_numpy(r.standard_normal((G, cap, hd)).astype(np.float16)))
        c[1].copy_(torch.from_numpy(r.standard_normal((G, cap, hd)).astype(np.float16)))
    t_kv = [t0 + j for j in range(n)] + [t0 // 2 + 3]
    kb = [shared[0].data_ptr()] * n + [other[0].data_ptr()]
    vb = [shared[1].data_ptr()] * n + [other[1].data_ptr()]
    B = len(t_kv)
    q = (r.standard_normal((B, H, hd)) * 0.5).astype(np.float32)
    scale = 1.0 / math.sqrt(hd)
    for chunk in (0, 96):
        out = kd.kd_fa_decode_ragged(dev(q), G, kb, vb, t_kv, cap, scale, chunk=chunk).cpu().numpy()
        for b in range(B):
            o1 = kd.kd_fa_decode_ragged(dev(q[b:b + 1]), G, kb[b:b + 1], vb[b:b + 1], t_kv[b:b + 1], cap, scale,
                                        chunk=chunk).cpu().numpy()
            np.testing.assert_array_equal(o1[0].view(np.uint32), out[b].view(np.uint32))
    # and the oracle on the first and last shared rows
    Kn, Vn = shared[0].cpu().numpy(), shared[1].cpu().numpy()
    for b in (0, n - 1):
        ref = ops.attention(q[b], Kn, Vn, t_kv[b])
        assert_close_rows(out[b].reshape(1, -1), ref.reshape(1, -1), 2e-3, f"fa shared row {b}")


def test_fa_decode_at_the_key_limit():
    """A row at the documented maximum of 131072 keys (multi-tile chunks of 1024 keys, 128
    splits) beside a short row: oracle within the bar, and bit-identical to its 1-row call."""
    H, G, hd = 8, 2, 128
    t_kv = [131072, 300]
    say(f"fa at the key limit t={t_kv}")
    r = np.random.default_rng(77)
    cap = 131072
    caches = _caches(2, G, cap, hd)
    gen = torch.Generator(device="cuda").manual_seed(77)
    for c in caches:
        c[0].normal_(generator=gen)
        c[1].normal_(generator=gen)
    q = (r.standard_normal((2, H, hd)) * 0.5).astype(np.float32)
    kb = [c[0].data_ptr() for c in caches]
    vb = [c[1].data_ptr() for c in caches]
    scale = 1.0 / math.sqrt(hd)
    out = kd.kd_fa_decode_ragged(dev(q), G, kb, vb, t_kv, cap, scale).cpu().numpy()
    for b in range(2):
        ref = ops.attention(q[b], caches[b][0].cpu().numpy(), caches[b][1].cpu().numpy(), t_kv[b])
        assert_close_rows(out[b].reshape(1, -1), ref.reshape(1, -1), 2e-3, f"fa key limit row {b}")
        o1 = kd.kd_fa_decode_ragged(dev(q[b:b + 1]), G, kb[b:b + 1], vb[b:b + 1], t_kv[b:b + 1], cap, scale)
        np.testing.assert_array_equal(o1.cpu().numpy()[0].view(np.uint32), out[b].view(np.uint32))



@pytest.mark.parametrize("fmt,n,k,B", [("q4_0", 4096, 4096, 2), ("q4_0", 4096, 14336, 4), ("q8_0", 2048, 2048, 9),
                                       ("q4_0", 4096, 4096, 16), ("q6_k", 2048, 5632, 7)])
def test_resnorm_rows_bit_identical_to_their_one_row_call(fmt, n, k, B):
    """kd_mmvq_resnorm splits two or more rows over grid slices (ceil(B/2) rows each up to
    B = 4, then 4 or 8 rows); every row's x1, block codes, block scales and block sums must
    equal that row's own B = 1 call bit for bit (B = 9: a last slice of one row)."""
    say(f"resnorm rows vs 1-row calls {fmt} n={n} k={k} B={B}")
    r = np.random.default_rng(7 * n + k + B)
    w = kd.kd_pack_weight(_drawer(fmt)(r, r, n, k))
    a = r.standard_normal((B, k)).astype(np.float32)
    res = r.standard_normal((B, n)).astype(np.float32)
    gain = dev((1 + 0.1 * r.standard_normal(n)).astype(np.float32))
    act = kd.kd_quantize_act_q8(dev(a))
    x1, zq, ss = kd.kd_mmvq_resnorm(w, act, B, dev(res), gain)
    sync()
    x1, qs, qd, ss = (t.cpu().numpy() for t in (x1, zq.qs, zq.d, ss))
    nq, nbp = qs.size // B, qd.size // B   # per-row extents of the tiled codes and scales
    for b in range(B):
        x1b, zb, ssb = kd.kd_mmvq_resnorm(w, kd.act_rows_view(act, b, 1), 1, dev(res[b:b + 1]), gain)
        sync()
        np.testing.assert_array_equal(x1b.cpu().numpy()[0].view(np.uint32), x1[b].view(np.uint32), err_msg=f"x1 row {b}")
        np.testing.assert_array_equal(zb.qs.cpu().numpy(), qs[b * nq:(b + 1) * nq], err_msg=f"codes row {b}")
        np.testing.assert_array_equal(zb.d.cpu().numpy().view(np.uint32), qd[b * nbp:(b + 1) * nbp].view(np.uint32))
        np.testing.assert_array_equal(ssb.cpu().numpy()[0].view(np.uint32), ss[b].view(np.uint32))
    say(f"  {B} rows equal their 1-row calls")


@pytest.mark.parametrize("fmt,n,k,B", [("q4_0", 4096, 4096, 8), ("q8_0", 2048, 2048, 3), ("q4_0", 4096, 14336, 16),
                                       ("q4_0", 2816, 2048, 5), ("q4_k", 4096, 4096, 8), ("q6_k", 2048, 5632, 5),
                                       ("q5_k", 2816, 2048, 3)])
def test_resnorm_pair_matches_oracle(fmt, n, k, B):
    """The split RMSNorm: kd_mmvq_resnorm (x1 = res + W Q(a), the block codes of x1 * gain,
    the block sums of x1^2) and its consumers kd_mmvq_swiglu_normed / kd_mmvq_rope_normed,
    against the oracle's add + RMSNorm + Q and the products after it.  Every GPU code must
    be a valid rounding of the oracle's value (|x/d - code| <= 1/2 + 1e-3); the consumers
    are compared given the GPU's codes of their input (the oracle's own scales)."""
    from oracle.step import _q_forced
    say(f"resnorm pair {fmt} n={n} k={k} B={B}")
    r = np.random.default_rng(n + k + B)
    draw = _drawer(fmt)
    w = draw(r, r, n, k)
    a = r.standard_normal((B, k)).astype(np.float32)
    res = r.standard_normal((B, n)).astype(np.float32)
    gain = (1 + 0.1 * r.standard_normal(n)).astype(np.float32)
    act = kd.kd_quantize_act_q8(dev(a))
    x1, zq, ss = kd.kd_mmvq_resnorm(kd.kd_pack_weight(w), act, B, dev(res), dev(gain))
    sync()
    q, d = ops.quantize_act(a)
    x1_ref = res.astype(np.float64) + ops.mmvq(w, q, d)
    assert_close_rows(x1.cpu().numpy(), x1_ref, 1e-5, "resnorm x1")
    ss_ref = (x1_ref.reshape(B, -1, 32) ** 2).sum(axis=2)
    np.testing.assert_allclose(ss.cpu().numpy(), ss_ref, rtol=1e-5)
    codes, _, pad_codes, _ = untile_act(zq.qs, zq.d, B, n)
    z = ops.rmsnorm(x1_ref, gain, 1e-5)
    rec = []
    zc, zd = _q_forced(z, codes, rec, "z")
    assert rec[0]["invalid"] == 0, rec
    assert np.all(pad_codes == 0)
    say(f"  {rec[0]['flips']} of {rec[0]['codes']} codes the other valid rounding")
    # consumer 1: the interleaved gate/up product with SwiGLU on the normed input
    F = 1024
    gate, up = draw(r, r, F, n), draw(r, r, F, n)
    h = kd.kd_mmvq_swiglu_normed(kd.kd_pack_weight(kd.interleave_gate_up(gate, up)), zq, B, ss, 1e-5)
    sync()
    hc, _, _, _ = untile_act(h.qs, h.d, B, F)
    h_ref = ops.swiglu(ops.mmvq(gate, zc, zd), ops.mmvq(up, zc, zd))
    rec = []
    _q_forced(h_ref, hc, rec, "h")
    assert rec[0]["invalid"] == 0, rec
    # consumer 2: the pair-ordered QKV product with RoPE and the fp16 append on the normed input
    H, G, hd, cap = 8, 4, 128, 32
    wq = draw(r, r, (H + 2 * G) * hd, n)
    pos = [int(p) for p in r.integers(0, cap, B)]
    cs = _caches(B, G, cap, hd)
    q_out = torch.zeros((B, H * hd), dtype=torch.float32, device="cuda")
    kd.kd_mmvq_rope_normed(kd.kd_pack_weight(kd.rope_pair_rows(wq, H + 2 * G, hd)), zq, B, ss, 1e-5, H, G, hd,
                           q_out, [c[0].data_ptr() for c in cs], [c[1].data_ptr() for c in cs], pos, cap, 10000.0)
    sync()
    y = ops.mmvq(wq, zc, zd)
    qref = np.stack([ops.rope_neox(y[b, :H * hd].reshape(H, hd), pos[b], 10000.0) for b in range(B)])
    assert_close_rows(q_out.cpu().numpy(), qref.reshape(B, -1), 1e-4, "rope normed q")
    for b in range(B):
        kref = ops.rope_neox(y[b, H * hd:(H + G) * hd].reshape(G, hd), pos[b], 10000.0)
        kg = cs[b][0].cpu().numpy()[:, pos[b]].astype(np.float64)
        assert np.max(np.abs(kg - kref)) <= np.max(np.abs(kref)) * 2 ** -10 + 1e-5 * np.sqrt(np.mean(kref ** 2))

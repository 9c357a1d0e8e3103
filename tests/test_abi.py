"""C ABI checks that need no GPU: libkd.so loads, exports every symbol kd.h declares, the
layout size queries are right, and argument errors are reported before anything is
enqueued (so these calls never reach the HIP runtime)."""
import ctypes as C
import os
import re

import pytest
import torch

import session_decode_step_amd as kd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "kd.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kd.LIB_PATH), reason="libkd.so not built")


def declared_functions():
    src = open(HDR).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(kd_[a-z0-9_]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert len(names) >= 25
    L = kd.lib()
    for n in names:
        assert hasattr(L, n), n
        assert n in kd.SIGNATURES, f"{n} has no binding signature"
    assert set(kd.SIGNATURES) == set(names)


def test_version_and_error_strings():
    assert "gfx950" in kd.kd_version()
    assert isinstance(kd.lib().kd_last_error(), bytes)


def test_layout_sizes():
    L = kd.lib()
    # 4096 x 4096 Q4_0: 256 row groups x 32 quads, 1024 B + 128 B of scales per tile
    assert L.kd_weight_qs_bytes(kd.KD_FMT_Q4_0, 4096, 4096) == 256 * 32 * 1024
    assert L.kd_weight_d_bytes(kd.KD_FMT_Q4_0, 4096, 4096) == 256 * 32 * 128
    assert L.kd_weight_qs_bytes(kd.KD_FMT_Q8_0, 4096, 4096) == 256 * 32 * 2048
    # ragged shapes pad to whole tiles: 704 rows -> 44 groups; k = 704 -> 6 quads
    assert L.kd_weight_qs_bytes(kd.KD_FMT_Q4_0, 700, 704) == 44 * 6 * 1024
    assert L.kd_weight_qs_bytes(kd.KD_FMT_Q8_0, 16, 48) == 0           # k % 32 != 0
    assert L.kd_act_qs_bytes(3, 704) == 3 * 6 * 128
    assert L.kd_act_d_bytes(3, 704) == 3 * 24 * 4
    t = (C.c_int32 * 3)(1, 129, 40000)
    # splits: 1 -> 1 (chunk 128), 129 -> 2, 40000 -> chunk 157, 255 splits
    assert L.kd_fa_decode_workspace(3, 8, 128, t) == (1 + 2 + 255) * 8 * (128 + 2) * 4


def _status(fn, *args):
    return fn(*args)


def test_mmvq_validation_before_launch():
    L = kd.lib()
    w = kd.KdWeight(kd.KD_FMT_Q8_0, 64, 256, 0x1000, 0x2000)
    act = kd.KdAct(0x3000, 0x4000)
    assert L.kd_mmvq_q8_0(C.byref(w), act, 17, 0x5000, 64, None) == kd.KD_ERR_UNSUPPORTED
    assert L.kd_mmvq_q8_0(C.byref(w), act, 0, 0x5000, 64, None) == kd.KD_ERR_UNSUPPORTED
    assert b"B=0" in L.kd_last_error()
    assert L.kd_mmvq_q4_0(C.byref(w), act, 2, 0x5000, 64, None) == kd.KD_ERR_UNSUPPORTED  # format mismatch
    assert L.kd_mmvq_q8_0(C.byref(w), act, 2, None, 64, None) == kd.KD_ERR_INVALID
    assert L.kd_mmvq_q8_0(C.byref(w), act, 2, 0x5000, 32, None) == kd.KD_ERR_INVALID       # ldy < n_out
    w2 = kd.KdWeight(kd.KD_FMT_Q8_0, 64, 250, 0x1000, 0x2000)
    assert L.kd_mmvq_q8_0(C.byref(w2), act, 2, 0x5000, 64, None) == kd.KD_ERR_UNSUPPORTED  # k % 32
    w3 = kd.KdWeight(kd.KD_FMT_Q8_0, 64, 256, 0x1001, 0x2000)
    assert L.kd_mmvq_q8_0(C.byref(w3), act, 2, 0x5000, 64, None) == kd.KD_ERR_INVALID      # unaligned
    # fused-epilogue products
    out = kd.KdAct(0x6000, 0x7000)
    wg = kd.KdWeight(kd.KD_FMT_Q4_0, 96, 256, 0x1000, 0x2000)                               # 2F = 96: F % 32 != 0
    assert L.kd_mmvq_swiglu(C.byref(wg), act, 2, out, None) == kd.KD_ERR_UNSUPPORTED
    wg = kd.KdWeight(kd.KD_FMT_Q4_0, 128, 256, 0x1000, 0x2000)
    assert L.kd_mmvq_swiglu(C.byref(wg), act, 2, kd.KdAct(0x6001, 0x7000), None) == kd.KD_ERR_INVALID
    assert L.kd_mmvq_swiglu(C.byref(wg), act, 17, out, None) == kd.KD_ERR_UNSUPPORTED
    kb = (C.c_void_p * 2)(0x10000, 0x20000)
    vb = (C.c_void_p * 2)(0x30000, 0x40000)
    pos = (C.c_int32 * 2)(3, 4)
    wq = kd.KdWeight(kd.KD_FMT_Q8_0, (4 + 2 * 2) * 64, 256, 0x1000, 0x2000)
    assert L.kd_mmvq_rope(C.byref(wq), act, 2, 4, 2, 128, 0x8000, 512, kb, vb, pos, 8, 1e4, None) == kd.KD_ERR_INVALID
    assert L.kd_mmvq_rope(C.byref(wq), act, 2, 4, 2, 96, 0x8000, 512, kb, vb, pos, 8, 1e4, None) == kd.KD_ERR_UNSUPPORTED
    assert L.kd_mmvq_rope(C.byref(wq), act, 2, 4, 2, 64, 0x8000, 128, kb, vb, pos, 8, 1e4, None) == kd.KD_ERR_INVALID
    assert L.kd_mmvq_rope(C.byref(wq), act, 2, 4, 2, 64, 0x8000, 256, kb, vb, pos, 4, 1e4, None) == kd.KD_ERR_CAPACITY
    kb_same = (C.c_void_p * 2)(0x10000, 0x10000)
    pos_same = (C.c_int32 * 2)(3, 3)
    assert L.kd_mmvq_rope(C.byref(wq), act, 2, 4, 2, 64, 0x8000, 256, kb_same, vb, pos_same, 8, 1e4, None) \
        == kd.KD_ERR_INVALID
    assert L.kd_quantize_act_q8(0x1000, 2, 100, 100, act, None) == kd.KD_ERR_UNSUPPORTED
    assert L.kd_pack_weight(7, 16, 32, 0x10, 0x20, 0x30, 0x40, None) == kd.KD_ERR_UNSUPPORTED


def test_attention_and_append_validation_before_launch():
    L = kd.lib()
    kb = (C.c_void_p * 2)(0x1000, 0x2000)
    vb = (C.c_void_p * 2)(0x3000, 0x4000)
    t = (C.c_int32 * 2)(10, 20)
    st = L.kd_fa_decode_ragged(0x100, 2, 8, 3, 128, kb, vb, t, 64, 0.1, 0x200, 0x300, 1 << 20, None)
    assert st == kd.KD_ERR_UNSUPPORTED                       # H % G != 0
    st = L.kd_fa_decode_ragged(0x100, 2, 8, 2, 96, kb, vb, t, 64, 0.1, 0x200, 0x300, 1 << 20, None)
    assert st == kd.KD_ERR_UNSUPPORTED                       # hd 96
    st = L.kd_fa_decode_ragged(0x100, 2, 8, 2, 128, kb, vb, t, 15, 0.1, 0x200, 0x300, 1 << 20, None)
    assert st == kd.KD_ERR_CAPACITY                          # t_kv > capacity
    st = L.kd_fa_decode_ragged(0x100, 2, 8, 2, 128, kb, vb, t, 64, 0.1, 0x200, 0x300, 16, None)
    assert st == kd.KD_ERR_WORKSPACE
    tmax = (C.c_int32 * 2)(131072 + 1, 20)                   # one key past the documented maximum
    st = L.kd_fa_decode_ragged(0x100, 2, 8, 2, 128, kb, vb, tmax, 1 << 18, 0.1, 0x200, 0x300, 1 << 30, None)
    assert st == kd.KD_ERR_UNSUPPORTED and b"131072" in L.kd_last_error()
    t0 = (C.c_int32 * 2)(0, 20)                              # a row with no key
    st = L.kd_fa_decode_ragged(0x100, 2, 8, 2, 128, kb, vb, t0, 64, 0.1, 0x200, 0x300, 1 << 20, None)
    assert st == kd.KD_ERR_UNSUPPORTED
    pos = (C.c_int32 * 2)(63, 5)
    assert L.kd_kv_append(0x10, 0x20, 2, 2, 128, kb, vb, pos, 63, None) == kd.KD_ERR_CAPACITY
    pos2 = (C.c_int32 * 2)(5, 5)
    same = (C.c_void_p * 2)(0x1000, 0x1000)
    assert L.kd_kv_append(0x10, 0x20, 2, 2, 128, same, vb, pos2, 64, None) == kd.KD_ERR_INVALID  # same slot twice
    assert L.kd_kv_append(0x10, 0x20, 17, 2, 128, kb, vb, pos, 64, None) == kd.KD_ERR_UNSUPPORTED


def _fake_weight(fmt, n, k, base):
    return kd.KdWeight(fmt, n, k, base, base + (1 << 24))


def _fake_model(n_layers=2, d=256, H=4, G=2, hd=64, F=512):
    layers = (kd.KdLayerDesc * n_layers)()
    for il in range(n_layers):
        b = 0x10000000 * (il + 1)
        D = layers[il]
        D.attn_norm = b
        D.wqkv = _fake_weight(kd.KD_FMT_Q8_0, (H + 2 * G) * hd, d, b + 0x100000)
        D.wo = _fake_weight(kd.KD_FMT_Q8_0, d, H * hd, b + 0x200000)
        D.ffn_norm = b + 0x300000
        D.w_gate = _fake_weight(kd.KD_FMT_Q8_0, F, d, b + 0x400000)
        D.w_up = _fake_weight(kd.KD_FMT_Q8_0, F, d, b + 0x500000)
        D.w_down = _fake_weight(kd.KD_FMT_Q8_0, d, F, b + 0x600000)
    desc = kd.KdModelDesc(n_layers, d, H, G, hd, F, 0, 0, 0, 0, 0, 10000.0, 1e-5, layers, 0, kd.KdWeight())
    return desc, layers


def test_token_validation_before_launch():
    L = kd.lib()
    assert L.kd_argmax_rows(0x100, 0, 10, 10, 0x200, None, None) == kd.KD_ERR_UNSUPPORTED
    assert L.kd_argmax_rows(0x100, 2, 0, 10, 0x200, None, None) == kd.KD_ERR_INVALID
    assert L.kd_argmax_rows(0x100, 2, 11, 10, 0x200, None, None) == kd.KD_ERR_INVALID    # ldx < n
    assert b"ldx" in L.kd_last_error()
    assert L.kd_argmax_rows(None, 2, 10, 10, 0x200, None, None) == kd.KD_ERR_INVALID
    assert L.kd_argmax_rows(0x100, 2, 10, 10, None, None, None) == kd.KD_ERR_INVALID
    assert L.kd_embed_rows(0x100, 0, 8, 0x200, 2, 0x300, 8, None) == kd.KD_ERR_INVALID    # vocab
    assert L.kd_embed_rows(0x100, 4, 8, 0x200, 2, 0x300, 7, None) == kd.KD_ERR_INVALID    # ldo < d
    assert L.kd_embed_rows(0x100, 4, 8, None, 2, 0x300, 8, None) == kd.KD_ERR_INVALID
    assert L.kd_embed_rows(0x100, 4, 8, 0x200, 70000, 0x300, 8, None) == kd.KD_ERR_UNSUPPORTED
    assert L.kd_verify_accept(0x100, 0x200, 0, 4, 0x300, 0x400, None) == kd.KD_ERR_UNSUPPORTED
    assert L.kd_verify_accept(0x100, 0x200, 5, 4, 0x300, 0x400, None) == kd.KD_ERR_UNSUPPORTED   # 20 rows
    assert L.kd_verify_accept(0x100, 0x200, 4, 0, 0x300, 0x400, None) == kd.KD_ERR_UNSUPPORTED
    assert L.kd_verify_accept(0x100, None, 4, 4, 0x300, 0x400, None) == kd.KD_ERR_INVALID


def test_model_create_validation_and_step_errors():
    L = kd.lib()
    desc, layers = _fake_model()
    h = C.c_void_p()
    assert L.kd_model_create(C.byref(desc), C.byref(h)) == kd.KD_OK
    try:
        pos = (C.c_int32 * 2)(10, 63)
        kb = (C.c_void_p * 4)(0x1000, 0x2000, 0x3000, 0x4000)
        vb = (C.c_void_p * 4)(0x5000, 0x6000, 0x7000, 0x8000)
        need = L.kd_decode_step_workspace(h, 2, pos)
        assert need > 0
        assert L.kd_decode_step(h, 2, 0x100, pos, kb, vb, 63, 0x200, 0x300, need, None) == kd.KD_ERR_CAPACITY
        assert L.kd_decode_step(h, 2, 0x100, pos, kb, vb, 64, 0x200, 0x300, need - 300, None) == kd.KD_ERR_WORKSPACE
        assert L.kd_decode_step(h, 17, 0x100, pos, kb, vb, 64, 0x200, 0x300, need, None) == kd.KD_ERR_UNSUPPORTED
        kb_same = (C.c_void_p * 4)(0x1000, 0x1000, 0x3000, 0x4000)
        pos_same = (C.c_int32 * 2)(10, 10)
        assert L.kd_decode_step(h, 2, 0x100, pos_same, kb_same, vb, 64, 0x200, 0x300, 1 << 30, None) == kd.KD_ERR_INVALID
    finally:
        L.kd_model_destroy(h)
    bad = kd.KdModelDesc(desc.n_layers, 256, 4, 3, 64, 512, 0, 0, 0, 0, 0, 10000.0, 1e-5, layers, 0, kd.KdWeight())
    assert L.kd_model_create(C.byref(bad), C.byref(h)) == kd.KD_ERR_UNSUPPORTED        # H % G
    layers[1].wo = _fake_weight(kd.KD_FMT_Q8_0, 255, 256, 0x900000)
    assert L.kd_model_create(C.byref(desc), C.byref(h)) == kd.KD_ERR_INVALID          # wrong shape
    assert b"wo" in L.kd_last_error()


def test_layer_variant_fields_are_validated():
    """Sliding window, QK-norm and output-gate fields of the layer descriptor are checked by
    kd_model_create before anything is kept."""
    L = kd.lib()
    h = C.c_void_p()

    def create(edit):
        desc, layers = _fake_model()
        edit(layers[1])
        return L.kd_model_create(C.byref(desc), C.byref(h))

    def ok(edit):
        st = create(edit)
        if st == kd.KD_OK:
            L.kd_model_destroy(h)
        return st

    assert ok(lambda l: setattr(l, "swa_window", 512)) == kd.KD_OK
    assert ok(lambda l: setattr(l, "swa_window", -1)) == kd.KD_ERR_INVALID
    assert ok(lambda l: setattr(l, "q_norm", 0x7000)) == kd.KD_ERR_INVALID            # k_norm missing
    assert b"q_norm" in L.kd_last_error()

    def qk(l, pair):
        l.q_norm, l.k_norm, l.wqkv_pair_rows = 0x7000, 0x7100, pair
    assert ok(lambda l: qk(l, 0)) == kd.KD_OK
    assert ok(lambda l: qk(l, 1)) == kd.KD_ERR_UNSUPPORTED                            # needs the canonical layout
    assert ok(lambda l: setattr(l, "attn_gate", 2)) == kd.KD_ERR_INVALID
    assert ok(lambda l: setattr(l, "attn_gate", 1)) == kd.KD_ERR_INVALID              # wqkv lacks the gate rows
    assert b"wqkv" in L.kd_last_error()

    def gated(l):
        l.attn_gate = 1
        l.wqkv = _fake_weight(kd.KD_FMT_Q8_0, (2 * 4 + 2 * 2) * 64, 256, 0xA00000)
    assert ok(gated) == kd.KD_OK


def test_kv_format_is_validated():
    """kd_model_create accepts fp16 and E4M3 caches with either wqkv layout, int8 caches with
    the canonical layout only, and no other format."""
    L = kd.lib()
    h = C.c_void_p()

    def create(fmt, pair):
        desc, layers = _fake_model()
        desc.kv_format = fmt
        for il in range(desc.n_layers):
            layers[il].wqkv_pair_rows = pair
        st = L.kd_model_create(C.byref(desc), C.byref(h))
        if st == kd.KD_OK:
            L.kd_model_destroy(h)
        return st

    assert create(kd.KD_KV_F16, 1) == kd.KD_OK
    assert create(kd.KD_KV_FP8_E4M3, 0) == kd.KD_OK
    assert create(kd.KD_KV_FP8_E4M3, 1) == kd.KD_OK
    assert create(kd.KD_KV_Q8_0, 0) == kd.KD_OK
    assert create(kd.KD_KV_Q8_0, 1) == kd.KD_ERR_UNSUPPORTED
    assert b"int8 KV" in L.kd_last_error()
    assert create(3, 0) == kd.KD_ERR_INVALID
    assert b"kv_format" in L.kd_last_error()


def test_fp8_kv_entry_points_validate_before_launch():
    L = kd.lib()
    kb = (C.c_void_p * 2)(0x1000, 0x2000)
    vb = (C.c_void_p * 2)(0x3000, 0x4000)
    pos = (C.c_int32 * 2)(3, 3)
    assert L.kd_kv_append_fp8(0x100, 0x200, 2, 2, 96, kb, vb, pos, 8, None) == kd.KD_ERR_UNSUPPORTED   # hd
    assert L.kd_kv_append_fp8(0x100, 0x200, 2, 2, 64, kb, vb, pos, 3, None) == kd.KD_ERR_CAPACITY
    kb_same = (C.c_void_p * 2)(0x1000, 0x1000)
    assert L.kd_kv_append_fp8(0x100, 0x200, 2, 2, 64, kb_same, vb, pos, 8, None) == kd.KD_ERR_INVALID
    t = (C.c_int32 * 2)(5, 9)
    ws = L.kd_fa_decode_workspace(2, 4, 64, t)
    assert L.kd_fa_decode_ragged_fp8(0x100, 2, 4, 2, 64, kb, vb, t, 8, 0.125, 0x200, 0x300, ws, None) == \
        kd.KD_ERR_CAPACITY
    assert L.kd_fa_decode_ragged_fp8(0x100, 2, 4, 2, 64, kb, vb, t, 16, 0.125, 0x200, 0x300, ws - 4, None) == \
        kd.KD_ERR_WORKSPACE
    assert L.kd_fa_decode_ragged_fp8(0x100, 2, 6, 2, 64, kb, vb, t, 16, 0.125, 0x200, 0x300, ws, None) == \
        kd.KD_ERR_UNSUPPORTED                                                                          # H/G = 3


def test_gdn_step_validates_before_launch():
    L = kd.lib()
    si = (C.c_void_p * 2)(0x1000, 0x2000)
    so = (C.c_void_p * 2)(0x3000, 0x4000)
    args = (0x100, 0x200, 0x300, 0x400, 0x500)
    assert L.kd_gdn_step(*args, 2, 4, 64, si, so, 0.1, 0x600, None) == kd.KD_ERR_UNSUPPORTED       # d_state
    assert L.kd_gdn_step(*args, 17, 4, 128, si, so, 0.1, 0x600, None) == kd.KD_ERR_UNSUPPORTED      # B
    same = (C.c_void_p * 2)(0x3000, 0x3000)
    assert L.kd_gdn_step(*args, 2, 4, 128, si, same, 0.1, 0x600, None) == kd.KD_ERR_INVALID
    cross = (C.c_void_p * 2)(0x2000, 0x4000)                 # row 0 writes what row 1 reads
    assert L.kd_gdn_step(*args, 2, 4, 128, si, cross, 0.1, 0x600, None) == kd.KD_ERR_INVALID
    assert L.kd_gdn_step(0, *args[1:], 2, 4, 128, si, so, 0.1, 0x600, None) == kd.KD_ERR_INVALID


def test_products_reject_shapes_past_their_limits():
    """k beyond 16384 (the widest wave partition) and matrices whose tiled codes would reach
    2 GiB (past the buffer offsets' masking value) are refused before any launch, by the
    product entry points and by kd_model_create."""
    L = kd.lib()
    act = kd.KdAct(0x3000, 0x4000)
    ok = kd.KdWeight(kd.KD_FMT_Q4_0, 64, 16384, 0x1000, 0x2000)
    wide = kd.KdWeight(kd.KD_FMT_Q4_0, 64, 16384 + 32, 0x1000, 0x2000)
    assert L.kd_mmvq_q4_0(C.byref(wide), act, 2, 0x5000, 64, None) == kd.KD_ERR_UNSUPPORTED
    assert b"16384" in L.kd_last_error()
    assert L.kd_mmvq_swiglu(C.byref(kd.KdWeight(kd.KD_FMT_Q4_0, 64, 28672, 0x1000, 0x2000)), act, 2,
                            kd.KdAct(0x6000, 0x7000), None) == kd.KD_ERR_UNSUPPORTED
    assert L.kd_debug_block_dots(C.byref(wide), act, 2, 0x5000, None) == kd.KD_ERR_UNSUPPORTED
    # 2^31 bytes of Q8_0 tiles: 2^20 tiles of 2048 B, e.g. 131072 rows x 16384 columns (8192 x 128 tiles)
    assert L.kd_weight_qs_bytes(kd.KD_FMT_Q8_0, 131072, 16384) == 1 << 31
    big = kd.KdWeight(kd.KD_FMT_Q8_0, 131072, 16384, 0x1000, 0x2000)
    assert L.kd_mmvq_q8_0(C.byref(big), act, 2, 0x5000, 131072, None) == kd.KD_ERR_UNSUPPORTED
    assert b"2 GiB" in L.kd_last_error()
    # one row group less fits (the call then proceeds to the output checks: ldy too small)
    just = kd.KdWeight(kd.KD_FMT_Q8_0, 131072 - 16, 16384, 0x1000, 0x2000)
    assert L.kd_weight_qs_bytes(kd.KD_FMT_Q8_0, 131072 - 16, 16384) < 1 << 31
    assert L.kd_mmvq_q8_0(C.byref(just), act, 2, 0x5000, 16, None) == kd.KD_ERR_INVALID
    assert b"ldy" in L.kd_last_error()
    # ... and the same shapes inside a model: an FFN of 28672 (down product k = 28672)
    desc, layers = _fake_model(F=28672)
    h = C.c_void_p()
    assert L.kd_model_create(C.byref(desc), C.byref(h)) == kd.KD_ERR_UNSUPPORTED
    assert b"w_down" in L.kd_last_error() or b"w_gate" in L.kd_last_error()
    desc, layers = _fake_model(F=16384)
    assert L.kd_model_create(C.byref(desc), C.byref(h)) == kd.KD_OK
    L.kd_model_destroy(h)
    del ok, just


def test_noalloc_attention_rejects_partials_beyond_its_scratch():
    """kd_fa_decode_ragged_noalloc refuses, before touching the device, a call whose split
    partials exceed its 16 MiB scratch array (16 rows of 131072 keys, 64 query heads: 136 MB)."""
    L = kd.lib()
    B, H, G, hd, cap = 16, 64, 8, 128, 131072
    t = (C.c_int32 * B)(*([cap] * B))
    assert L.kd_fa_decode_workspace(B, H, hd, t) > 16 << 20
    kb = (C.c_void_p * B)(*[0x100000 * (i + 1) for i in range(B)])
    vb = (C.c_void_p * B)(*[0x8000000 + 0x100000 * i for i in range(B)])
    assert L.kd_fa_decode_ragged_noalloc(0x1000, B, H, G, hd, kb, vb, t, cap, 0.088, 0x2000, None) \
        == kd.KD_ERR_WORKSPACE
    assert b"scratch" in L.kd_last_error()


def _fake_hybrid(n_layers=2, d=256, nk=2, nv=4, dc=4):
    """_fake_model with layer 0 a gated delta-rule layer (128-wide heads, nk key / nv value heads)."""
    desc, layers = _fake_model(n_layers, d)
    C_, vd = 2 * 128 * nk + 128 * nv, 128 * nv
    D = layers[0]
    D.mixer = 1
    D.wqkv = _fake_weight(kd.KD_FMT_Q8_0, C_ + vd + 2 * nv, d, 0x30000000)
    D.wo = _fake_weight(kd.KD_FMT_Q8_0, d, vd, 0x31000000)
    D.ssm_conv, D.ssm_dt, D.ssm_a, D.ssm_norm = 0x32000000, 0x32100000, 0x32200000, 0x32300000
    desc.ssm_d_state, desc.ssm_n_k, desc.ssm_n_v, desc.ssm_d_conv = 128, nk, nv, dc
    return desc, layers


def test_linear_layers_are_validated():
    """A gated delta-rule layer needs its conv, dt, a and norm arrays, an input projection of
    conv channels + z + beta + alpha rows, an out projection of n_v 128 columns, no attention
    options, 128-wide heads with n_v a multiple of n_k; its recurrent state is two conv rings
    [(d_conv - 1), C] (each padded to 4 floats) and two states [n_v, 128, 128], fp32."""
    L = kd.lib()
    h = C.c_void_p()

    def create(edit=lambda desc, l: None):
        desc, layers = _fake_hybrid()
        edit(desc, layers[0])
        st = L.kd_model_create(C.byref(desc), C.byref(h))
        if st == kd.KD_OK:
            L.kd_model_destroy(h)
        return st

    assert create() == kd.KD_OK
    desc, layers = _fake_hybrid()
    assert L.kd_model_create(C.byref(desc), C.byref(h)) == kd.KD_OK
    try:
        ring = (4 - 1) * (2 * 128 * 2 + 128 * 4)
        assert L.kd_recurrent_state_bytes(h) == 4 * 2 * (ring + 4 * 128 * 128)
    finally:
        L.kd_model_destroy(h)
    desc, layers = _fake_model()
    assert L.kd_model_create(C.byref(desc), C.byref(h)) == kd.KD_OK
    assert L.kd_recurrent_state_bytes(h) == 0           # no linear layer
    L.kd_model_destroy(h)
    assert create(lambda d, l: setattr(l, "ssm_norm", 0)) == kd.KD_ERR_INVALID
    assert b"conv, dt, a or norm" in L.kd_last_error()
    assert create(lambda d, l: setattr(l, "ssm_norm", 0x32300004)) == kd.KD_ERR_INVALID      # unaligned
    assert create(lambda d, l: setattr(l, "mixer", 2)) == kd.KD_ERR_INVALID
    assert create(lambda d, l: setattr(l, "swa_window", 64)) == kd.KD_ERR_INVALID
    assert create(lambda d, l: setattr(d, "ssm_d_state", 64)) == kd.KD_ERR_UNSUPPORTED
    assert create(lambda d, l: setattr(d, "ssm_n_v", 3)) == kd.KD_ERR_UNSUPPORTED             # not a multiple of n_k
    assert create(lambda d, l: setattr(d, "ssm_d_conv", 1)) == kd.KD_ERR_UNSUPPORTED
    assert create(lambda d, l: setattr(l, "wo", _fake_weight(kd.KD_FMT_Q8_0, 256, 4 * 64, 0x31000000))) \
        == kd.KD_ERR_INVALID
    assert b"out projection" in L.kd_last_error()
    assert create(lambda d, l: setattr(l, "wqkv", _fake_weight(kd.KD_FMT_Q8_0, 1536, 256, 0x30000000))) \
        == kd.KD_ERR_INVALID
    assert b"input projection" in L.kd_last_error()


def test_linear_layer_states_are_checked_per_step():
    """kd_decode_step refuses a null or unaligned recurrent state and two rows whose states
    overlap (each row owns its state for the step)."""
    L = kd.lib()
    desc, layers = _fake_hybrid()
    h = C.c_void_p()
    assert L.kd_model_create(C.byref(desc), C.byref(h)) == kd.KD_OK
    try:
        rb = L.kd_recurrent_state_bytes(h)
        pos = (C.c_int32 * 2)(10, 20)
        vb = (C.c_void_p * 4)(0x5000, 0x6000, 0x7000, 0x8000)
        need = L.kd_decode_step_workspace(h, 2, pos)

        def step(s0, s1):
            kb = (C.c_void_p * 4)(s0, s1, 0x3000, 0x4000)    # layer 0: states; layer 1: K caches
            return L.kd_decode_step(h, 2, 0x100, pos, kb, vb, 64, 0x200, 0x300, need - 1, None)

        assert step(0x40000000, 0x40000000 + rb) == kd.KD_ERR_WORKSPACE   # the states pass
        assert step(0x40000000, 0x40000000 + rb - 256) == kd.KD_ERR_INVALID
        assert b"share a recurrent state" in L.kd_last_error()
        assert step(0, 0x50000000) == kd.KD_ERR_INVALID
        assert step(0x40000008, 0x50000000) == kd.KD_ERR_INVALID
    finally:
        L.kd_model_destroy(h)


def test_kquant_layouts_and_validation():
    """K-quant tiles: 1024 / 1280 / 1536 code bytes and 192 scale bytes per tile; k must be a
    multiple of 256 (one record) for the pack, the products and kd_model_create; the block-dot
    test export takes Q8_0 / Q4_0 only; kd_mmvq refuses the fp32 router format."""
    L = kd.lib()
    for fmt, tile in ((kd.KD_FMT_Q4_K, 1024), (kd.KD_FMT_Q5_K, 1280), (kd.KD_FMT_Q6_K, 1536)):
        assert L.kd_weight_qs_bytes(fmt, 20, 512) == 2 * 4 * tile       # 2 row groups x 4 quads
        assert L.kd_weight_d_bytes(fmt, 20, 512) == 2 * 4 * 192
        assert L.kd_weight_qs_bytes(fmt, 20, 384) == 0                  # not a whole record
        assert L.kd_pack_weight(fmt, 20, 384, 0x1000, None, 0x2000, 0x3000, None) == kd.KD_ERR_UNSUPPORTED
        act = kd.KdAct(0x3000, 0x4000)
        bad = kd.KdWeight(fmt, 64, 384, 0x1000, 0x2000)
        assert L.kd_mmvq(C.byref(bad), act, 2, 0x5000, 64, None) == kd.KD_ERR_UNSUPPORTED
        ok = kd.KdWeight(fmt, 64, 512, 0x1000, 0x2000)
        assert L.kd_mmvq(C.byref(ok), act, 2, None, 64, None) == kd.KD_ERR_INVALID      # gets to the output check
        assert L.kd_mmvq_q4_0(C.byref(ok), act, 2, 0x5000, 64, None) == kd.KD_ERR_UNSUPPORTED   # format mismatch
        assert L.kd_debug_block_dots(C.byref(ok), act, 2, 0x5000, None) == kd.KD_ERR_UNSUPPORTED
    f32 = kd.KdWeight(kd.KD_FMT_F32, 64, 512, 0x1000, None)
    assert L.kd_mmvq(C.byref(f32), kd.KdAct(0x3000, 0x4000), 2, 0x5000, 64, None) == kd.KD_ERR_UNSUPPORTED
    # a model with K-quant matrices: accepted at d = 256, refused where a k is not a whole record
    h = C.c_void_p()
    desc, layers = _fake_model()
    for il in range(desc.n_layers):
        layers[il].wqkv = _fake_weight(kd.KD_FMT_Q5_K, (4 + 2 * 2) * 64, 256, 0x10000000 * (il + 1) + 0x100000)
        layers[il].w_down = _fake_weight(kd.KD_FMT_Q6_K, 256, 512, 0x10000000 * (il + 1) + 0x600000)
    assert L.kd_model_create(C.byref(desc), C.byref(h)) == kd.KD_OK
    L.kd_model_destroy(h)
    desc, layers = _fake_model(F=640)
    layers[0].w_down = _fake_weight(kd.KD_FMT_Q4_K, 256, 640, 0x10600000)
    assert L.kd_model_create(C.byref(desc), C.byref(h)) == kd.KD_ERR_UNSUPPORTED
    assert b"w_down" in L.kd_last_error()


def test_read_stream_binding_bounds_the_bytes():
    """The read-ceiling export reads raw bytes from a pointer: its binding refuses a byte count
    past the tensor (nothing is launched)."""
    t = torch.zeros(64, dtype=torch.float16)
    sink = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        kd.kd_debug_read_stream(t, sink, 129)
    with pytest.raises(ValueError):
        kd.kd_debug_read_stream(t[::2], sink, 16)

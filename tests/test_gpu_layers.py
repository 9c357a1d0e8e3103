"""Teacher-forced per-layer parity of kd_decode_step against the CPU oracle.

Each layer of the GPU step is checked against the oracle's same layer fed the GPU's own
input to that layer (the residual rows kd_debug_decode_step_trace records), so the
comparison covers one layer's arithmetic (memra-engine decode_batch.rs exactness contract:
each layer of the batched walk must match its reference).

The layer holds four activation quantisations (five with an lm_head), and an fp32 and an fp64
evaluation reaching a quantiser with values a rounding apart may pick the two neighbouring
codes of a value that lies on a rounding boundary; one such flip in the FFN input moves
about 1% of the next quantiser's codes by one step, which shows as up to ~2e-3 in a layer's
output.  Both codes are correct results, so the comparison is made in two parts:

* forced: the oracle takes the GPU's codes at every quantisation after checking that each is
  a valid rounding of the oracle's own value (|x/d - code| <= 1/2 + 1e-3; none may fail),
  and then the layer's output is held to the stated bar, every element within 2e-3 of the
  oracle scaled by max(|ref_i|, rms(row)), and the layer's own contribution (output minus
  input) normwise within 2e-3; the appended K/V are the oracle's values rounded either way
  to the cache format;
* free: the oracle quantises on its own; the layer's output is reported, and held to 1e-2
  (the size of a flip's effect).

MoE layers: each row's experts (ids, by rank) must equal the oracle's exactly, and their
weights agree within 1e-6; a row whose 8th and 9th router logits lie within 1e-6 (relative)
would be reported as a near tie (none is expected).

Later steps: the oracle's caches take the GPU's bytes for the slots earlier steps wrote, so
each step's layer sees exactly what the GPU's did.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workload as W
from gpu_util import assert_close_rows, requires_gpu, row_errors, say, untile_codes

pytestmark = [pytest.mark.gpu, requires_gpu]

LAYER_BAR = 2e-3       # elementwise, scaled by max(|ref_i|, rms(row)): the stated bar
DELTA_BAR = 2e-3       # normwise, on the layer's own contribution
FREE_BAR = 1e-2        # free-running layer (quantiser flips included)
P_BAR = 1e-6           # router weights
STATE_BAR = 1e-4       # a linear layer's new recurrent state, relative to its rms
TIE_REL = 1e-6         # router near-tie report threshold

kd = pytest.importorskip("session_decode_step_amd")
from session_decode_step_amd.runner import GpuWorkload  # noqa: E402


def _gpu_slots_into(oc, gw, step, layers):
    """Copy the K/V bytes the GPU wrote at ``step`` into the oracle's caches."""
    wl = gw.wl
    lin = set(wl.spec.linear_layers)
    for b, (sess, _) in enumerate(wl.rows):
        if sess not in oc.K:
            continue
        p = wl.positions(step)[b]
        for il in layers:
            if il in lin:
                continue
            oc.K[sess][il][:, p] = gw.caches.t[sess][il, 0, :, p].cpu().numpy()
            oc.V[sess][il][:, p] = gw.caches.t[sess][il, 1, :, p].cpu().numpy()


def _slot_excess(g, r):
    """How far the GPU's appended values g exceed one rounding of the cache format from the
    oracle's r, beyond the fp32 evaluation error (1e-5 of each head's rms): <= 0 when g is r
    rounded either way.  fp16: one unit <= 2^-10 |r|; E4M3 codes: <= 2^-3 |r|, 2^-9 below 2^-6;
    int8 rows: one code step d of the block plus one fp16 unit of its scale times the code."""
    if g.dtype == np.uint8 and g.shape[-1] % 32 == 16:          # int8 rows: codes and block scales
        hd = g.shape[-1] - 16
        gv, rv = oracle.q8_kv_decode(g, hd), oracle.q8_kv_decode(r, hd)
        d = np.repeat(r[..., hd:hd + hd // 16].copy().view(np.float16).astype(np.float64), 32, axis=-1)
        unit = d * (1 + 2.0 ** -10) + 2.0 ** -10 * np.abs(rv)      # one code step, or the scale's fp16 unit
    elif g.dtype == np.uint8:
        gv, rv = oracle.e4m3_decode(g), oracle.e4m3_decode(r)
        unit = np.maximum(np.abs(rv) * 2.0 ** -3, 2.0 ** -9)
    else:
        gv, rv = g.astype(np.float64), r.astype(np.float64)
        unit = np.maximum(np.abs(rv) * 2.0 ** -10, 2.0 ** -24)
    rms = np.sqrt(np.mean(rv * rv, axis=-1, keepdims=True))
    return np.abs(gv - rv) - unit - 1e-5 * rms


def _forced_codes(rec, il, rows, sp):
    """The GPU's codes of layer il's quantisations, untiled, for the followed rows."""
    K = sp.n_expert_used
    w_out = sp.ssm_value_dim if il in sp.linear_layers else sp.n_head * sp.head_dim
    f = {"attn_in": untile_codes(rec["q_attn_in"][il][rows], sp.d),
         "attn_out": untile_codes(rec["q_attn_out"][il][rows][:, :(w_out + 127) // 128 * 128], w_out)}
    if "q_ffn_in" in rec:
        f["ffn_in"] = untile_codes(rec["q_ffn_in"][il][rows], sp.d)
    if sp.ffn:
        f["ffn_mid"] = untile_codes(rec["q_ffn_mid"][il][rows], sp.ffn)
    if sp.n_experts:
        pr = [b * K + r for b in rows for r in range(K)]
        f["ffn_mid"] = untile_codes(rec["q_ffn_mid"][il][pr], sp.expert_ffn)
        f["shared_mid"] = untile_codes(rec["q_shared_mid"][il][rows], sp.shared_ffn)
    return f


def _check_layers(gw, steps, layers, rows=None, dense_budget=6 << 30, head=True, free=True):
    """Run ``steps`` of the GPU stack with the per-layer record; check ``layers`` of each and
    (``head``) the output head against the oracle fed the GPU's layer inputs."""
    wl = gw.wl
    sp = wl.spec
    rows = list(range(wl.B)) if rows is None else list(rows)
    sess = [wl.rows[b][0] for b in rows]
    oc = oracle.OracleCaches(wl, sessions=sorted(set(sess)), layers=layers)
    dense = oracle.DenseWeights(dense_budget)
    worst, worst_delta, worst_free, n_ids, near, flips, codes, worst_state = 0.0, 0.0, 0.0, 0, 0, 0, 0, 0.0
    lin = set(sp.linear_layers)
    for s in steps:
        say(f"  {sp.name} step {s}: gpu")
        rec = gw.step_trace(s)
        resid = rec["resid"].astype(np.float64)
        pos = [wl.positions(s)[b] for b in rows]
        for il in layers:
            x_in = resid[il][rows]
            gpu = resid[il + 1][rows]
            linear = il in lin
            if linear:   # the recurrent state each evaluation starts from
                snap = {ss: {k: v.copy() for k, v in oc.R[ss][il].items()} for ss in set(sess)}
            if free:
                say(f"  step {s} layer {il}: oracle (free)")
                ref = oracle.decode_layer(gw.model, il, oc, x_in, sess, pos, dense=dense)
                worst_free = max(worst_free, assert_close_rows(gpu, ref, FREE_BAR, f"step {s} layer {il} (free)"))
                if linear:
                    for ss in snap:
                        oc.R[ss][il] = {k: v.copy() for k, v in snap[ss].items()}
            info, qrec = {}, []
            say(f"  step {s} layer {il}: oracle (forced codes)")
            ref = oracle.decode_layer(gw.model, il, oc, x_in, sess, pos, dense=dense, info=info,
                                      forced=_forced_codes(rec, il, rows, sp), record=qrec)
            bad = [r for r in qrec if r["invalid"]]
            assert not bad, f"step {s} layer {il}: GPU codes that are no rounding of the value: {bad}"
            flips += sum(r["flips"] for r in qrec)
            codes += sum(r["codes"] for r in qrec)
            worst = max(worst, assert_close_rows(gpu, ref, LAYER_BAR, f"step {s} layer {il}"))
            dnorm, _ = row_errors(gpu - x_in, ref - x_in)
            worst_delta = max(worst_delta, float(dnorm.max()))
            assert dnorm.max() <= DELTA_BAR, f"step {s} layer {il}: contribution normwise error {dnorm.max():.3e}"
            if linear:   # the new recurrent state; then the GPU's becomes the oracle's (teacher forcing)
                for i, b in enumerate(rows):
                    rings, states = gw.caches.recurrent_views(sess[i], il, *gw.rec_layout)
                    new = (pos[i] + 1) % 2
                    g_ring = rings[new].cpu().numpy().astype(np.float64)
                    g_S = states[new].cpu().numpy().astype(np.float64).reshape(oc.R[sess[i]][il]["S"].shape)
                    o_ring, o_S = oc.R[sess[i]][il]["conv"], oc.R[sess[i]][il]["S"]
                    np.testing.assert_array_equal(g_ring[:-1], o_ring[:-1])      # shifted: copies
                    assert_close_rows(g_ring[-1:], o_ring[-1:], 1e-5, f"step {s} layer {il} row {b} ring")
                    srms = np.sqrt(np.mean(o_S ** 2))
                    worst_state = max(worst_state, float(np.abs(g_S - o_S).max() / srms))
                    assert np.abs(g_S - o_S).max() <= STATE_BAR * srms, (s, il, b)
                    oc.R[sess[i]][il] = {"conv": g_ring, "S": g_S}
                continue
            # the appended K/V: the oracle's values, each rounded either way to the cache format
            for i, b in enumerate(rows):
                p = pos[i]
                for kv, arr in ((0, oc.K), (1, oc.V)):
                    g = gw.caches.t[sess[i]][il, kv, :, p].cpu().numpy()
                    ex = _slot_excess(g, arr[sess[i]][il][:, p])
                    assert ex.max() <= 0, f"step {s} layer {il} row {b}: appended {'KV'[kv]} off by {ex.max():.3e}"
            if sp.n_experts:
                ids_g = rec["moe_ids"][il][rows]
                p_g = rec["moe_p"][il][rows]
                for i in range(len(rows)):
                    tie = info["gap"][i] < TIE_REL * info["kth"][i]
                    near += int(tie)
                    if tie:
                        say(f"  near tie: step {s} layer {il} row {rows[i]} gap {info['gap'][i]:.3e}")
                        continue
                    np.testing.assert_array_equal(ids_g[i], info["ids"][i], err_msg=f"layer {il} row {rows[i]}")
                    np.testing.assert_allclose(p_g[i], info["p"][i], rtol=0, atol=P_BAR)
                    n_ids += 1
        if head:
            qrec = []
            fh = untile_codes(rec["q_head_in"][rows], sp.d) if sp.vocab else None
            ref = oracle.output_head(gw.model, resid[sp.n_layers][rows], dense=dense, forced=fh, record=qrec)
            assert not [r for r in qrec if r["invalid"]]
            flips += sum(r["flips"] for r in qrec)
            codes += sum(r["codes"] for r in qrec)
            worst = max(worst, assert_close_rows(rec["out"][rows], ref, LAYER_BAR, f"step {s} output head"))
        # the bytes this step wrote become the oracle's for the next step
        _gpu_slots_into(oc, gw, s, layers)
    say(f"  worst forced layer error {worst:.3e}, contribution {worst_delta:.3e}; free-running {worst_free:.3e}; "
        f"{flips} of {codes} GPU codes are the other valid rounding"
        + (f"; {n_ids} routings equal, {near} near ties" if sp.n_experts else "")
        + (f"; recurrent states within {worst_state:.3e} of their rms" if lin else ""))
    assert near == 0 or n_ids > 0


@pytest.mark.parametrize("variant", ["plain", "swa", "qk_norm", "gate", "fp8", "q8"])
def test_c2_every_layer_and_lm_head(variant):
    """8-layer d=2048 Q8_0 stack with lm_head 32000, ctx 1238, B = 4 (and its block variants:
    512-key windows on alternate layers, QK-norm, output gate, FP8 E4M3 caches): every layer
    and the lm_head of two steps, teacher-forced."""
    say(f"c2 per layer: {variant}")
    base = W.workload("c2", B=4, steps=2)
    sp = base.spec
    extra = {"plain": {}, "swa": {"swa_window": 512, "swa_layers": (0, 2, 4, 6)}, "qk_norm": {"qk_norm": True},
             "gate": {"attn_gate": True}, "fp8": {"kv_fp8": True}, "q8": {"kv_q8": True}}[variant]
    wl = dataclasses.replace(base, spec=dataclasses.replace(sp, **extra))
    gw = GpuWorkload(wl)
    _check_layers(gw, [0, 1], list(range(sp.n_layers)))


def test_c4_layers_0_15_31_and_output_norm():
    """32-layer d=4096 Q4_0 stack, ctx 4096, B = 8: layers 0, 15 and 31 and the output norm,
    teacher-forced, all rows."""
    say("c4 per layer")
    wl = W.workload("c4", B=8, steps=1)
    gw = GpuWorkload(wl)
    _check_layers(gw, [0], [0, 15, 31], dense_budget=8 << 30)


def test_c5_every_moe_layer_with_exact_routing():
    """8-layer MoE stack (128 experts, top-8, shared expert), 4 streams x 4 verify rows at ctx
    8192: every layer of all 16 rows teacher-forced, with each row's experts equal to the
    oracle's and their weights within 1e-6."""
    say("c5 per layer")
    wl = W.workload("c5")
    gw = GpuWorkload(wl)
    _check_layers(gw, [0], list(range(wl.spec.n_layers)), dense_budget=2 << 30, free=False)


def test_hybrid_gdn_stack_every_layer_and_lm_head():
    """The 8-layer Q8_0 stack with gated delta-rule layers in place of attention on layers 0-2
    and 4-6 (8 key / 16 value heads of 128, conv width 4), B = 4, three steps: every layer and
    the lm_head teacher-forced, each linear layer's new recurrent state (conv ring and state)
    against the oracle's, then carried into the next step."""
    say("hybrid per layer")
    wl = W.workload("hybrid", B=4, steps=3)
    gw = GpuWorkload(wl)
    _check_layers(gw, [0, 1, 2], list(range(wl.spec.n_layers)))


def test_kquant_stack_every_layer_and_lm_head():
    """The 8-layer d=2048 stack with K-quant weights (Q5_K QKV, Q4_K O and gate/up, Q6_K down
    and lm_head), B = 8, two steps: every layer and the lm_head teacher-forced at the stated
    bar, on rows 0 and 7."""
    say("kquant per layer")
    wl = W.workload("kq", B=8, steps=2)
    gw = GpuWorkload(wl)
    _check_layers(gw, [0, 1], list(range(wl.spec.n_layers)), rows=[0, 7])

"""One batched decode step over a layer stack, composed from :mod:`oracle.ops` in fp64.

TEST INFRASTRUCTURE ONLY: nothing in the product path imports this module.

The op order is the Full-attention arm of the batched layer walk on the memra-engine
page (src/decode_batch.rs, ``decode_batch_layers``): attn_norm -> quantise -> q/k/v
products at m = B -> RoPE with per-row positions -> phase A, append every row's K/V ->
phase B, every row attends over its own cache -> o product -> residual add +
post-attention norm -> quantise -> gate/up -> silu_mul -> quantise -> down -> residual
add; then the output norm and lm_head (``decode_step_batch_lean_masked``).  The block
variants of the same walk are options of a layer: QK-norm (per-head RMSNorm of q and k
before RoPE), the attention output gate (sigmoid of extra projection rows times the
attention output, before the o product) and the sliding-window view.  The
MoE FFN follows hf2q ADR-040 §0.7 F4 (per-token top-k routing, each active expert's
matrices applied to the rows routed to it, weighted sum) and the shared expert of the
Strata pull request #1524 ("What changes").
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence

import numpy as np

from . import ops


class DenseWeights:
    """Optional cache of dequantised fp64 matrices (speed only; values equal ops.dequantize)."""

    def __init__(self, budget_bytes: int = 0):
        self.budget = budget_bytes
        self.used = 0
        self.mem: Dict[int, np.ndarray] = {}

    def get(self, w: Dict) -> Optional[np.ndarray]:
        key = id(w)
        if key in self.mem:
            return self.mem[key]
        need = w["n"] * w["k"] * 8
        if self.used + need > self.budget:
            return None
        dense = ops.dequantize(w)
        self.mem[key] = dense
        self.used += need
        return dense


class OracleCaches:
    """K/V of the sessions the oracle follows: ``K[s][il]`` is ``[G, capacity, hd]``, fp16, or
    uint8 E4M3 codes for a model with FP8 caches (``spec.kv_fp8``), or uint8 rows
    ``[G, capacity, hd + 16]`` for int8 caches (``spec.kv_q8``, see ``ops.q8_kv_encode``)."""

    def __init__(self, wl, sessions: Optional[Sequence[int]] = None, layers: Optional[Sequence[int]] = None):
        """``layers``: only these layers' caches are filled (the others stay None), for
        following single layers of a deep stack."""
        from workload import kv_prefill_many, recurrent_prefill  # seeded inputs only
        sp = wl.spec
        self.sessions = list(range(len(wl.prefill))) if sessions is None else list(sessions)
        keep = set(range(sp.n_layers) if layers is None else layers)
        lin = set(getattr(sp, "linear_layers", ()))
        self.K: Dict[int, List[np.ndarray]] = {}
        self.V: Dict[int, List[np.ndarray]] = {}
        # linear layers: the recurrent state {"conv": [d_conv - 1, conv_dim], "S": [n_v, d, d]}
        self.R: Dict[int, Dict[int, Dict[str, np.ndarray]]] = {
            s: {il: dict(zip(("conv", "S"), (a.astype(np.float64) for a in recurrent_prefill(wl, s, il))))
                for il in sorted(keep & lin)} for s in self.sessions}
        keep -= lin
        pairs = [(s, il) for s in self.sessions for il in range(sp.n_layers) if il in keep]
        pre = dict(zip(pairs, kv_prefill_many(wl, pairs)))
        for s in self.sessions:
            self.K[s], self.V[s] = [], []
            for il in range(sp.n_layers):
                if il not in keep:
                    self.K[s].append(None)
                    self.V[s].append(None)
                    continue
                k0, v0 = pre[(s, il)]
                dt = np.uint8 if getattr(sp, "kv_fp8", False) or getattr(sp, "kv_q8", False) else np.float16
                K = np.zeros((sp.n_head_kv, wl.capacity, k0.shape[2]), dtype=dt)
                V = np.zeros_like(K)
                K[:, : k0.shape[1]] = k0
                V[:, : v0.shape[1]] = v0
                self.K[s].append(K)
                self.V[s].append(V)


def _mm(w: Dict, xq, xd, dense: Optional[DenseWeights], blocks: bool) -> np.ndarray:
    if blocks:
        return ops.mmvq_blocks(w, xq, xd)
    return ops.mmvq(w, xq, xd, dense.get(w) if dense is not None else None)


def _q(x: np.ndarray):
    """Q(.) of the fp64 value rounded to fp32 (the quantiser's input precision)."""
    return ops.quantize_act(np.asarray(x, dtype=np.float64).astype(np.float32))


# Teacher forcing of the quantiser's integer decisions.  An fp32 evaluation of the step and
# this fp64 one reach each quantiser with values that differ by rounding, so a value lying
# within that difference of a rounding boundary (x / d = k + 1/2) may take either neighbouring
# code: both are correct results.  Given another evaluation's codes, ``_q_forced`` accepts
# each code that is such a rounding of the oracle's own value -- |x / d - code| <= 1/2 + TOL,
# the ratio computed as Q computes it -- records how many differ from the oracle's own choice
# and how many are not valid roundings at all, and continues with the given codes, so that
# what follows compares continuous arithmetic only.  The scales stay the oracle's own.
FORCE_TOL = 1e-3


def _q_forced(x: np.ndarray, codes: Optional[np.ndarray], record: Optional[List], what: str):
    xq, xd = _q(x)
    if codes is None:
        return xq, xd
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    B, K = x32.shape
    g = np.asarray(codes, dtype=np.int64).reshape(B, K)
    safe = np.where(xd == 0, np.float32(1.0), xd).astype(np.float32)
    ratio = (x32.reshape(B, K // ops.QK, ops.QK) / safe[:, :, None]).astype(np.float32).astype(np.float64)
    ratio = np.where((xd == 0)[:, :, None], 0.0, ratio).reshape(B, K)
    dist = np.abs(ratio - g)
    invalid = int(np.sum((dist > 0.5 + FORCE_TOL) | (np.abs(g) > 127)))
    differ = g != xq.astype(np.int64)
    if record is not None:
        record.append({"what": what, "codes": int(g.size), "flips": int(differ.sum()), "invalid": invalid,
                       "flip_margin": float(np.max(np.abs(dist[differ] - 0.5))) if differ.any() else 0.0})
    return g.astype(np.int8), xd


def moe_ffn(spec, L: Dict, z: np.ndarray, zq, zd, dense: Optional[DenseWeights], blocks: bool,
            info: Optional[Dict] = None, forced: Optional[Dict] = None, record: Optional[List] = None):
    """Routed experts + shared expert for rows ``z[B, d]`` (reading: rank-ordered sum, then + shared)."""
    B, d = z.shape
    E, k, Fe = spec.n_experts, spec.n_expert_used, spec.expert_ffn
    r = z @ L["router"].astype(np.float64).T            # fp32 router weights, unquantised input
    out = np.zeros((B, d), dtype=np.float64)

    def fmid(b, rank):   # forced codes of row b's rank-th expert input to its down product
        return None if forced is None or "ffn_mid" not in forced else forced["ffn_mid"][b * k + rank:b * k + rank + 1]
    for b in range(B):
        ids, p = ops.router_topk(r[b], k)
        if info is not None:   # the routing decision, and how close it came to another one
            srt = np.sort(r[b])[::-1]
            info.setdefault("gap", []).append(float(srt[k - 1] - srt[k]) if k < E else np.inf)
            info.setdefault("kth", []).append(float(abs(srt[k - 1])))
            info.setdefault("ids", []).append(ids.copy())
            info.setdefault("p", []).append(p.copy())
        acc = np.zeros(d, dtype=np.float64)
        for rank in range(k):
            e = int(ids[rank])
            if blocks:
                sub = lambda w, r0, r1: {**w, "n": r1 - r0, "qs": w["qs"][r0:r1], "d": w["d"][r0:r1]}
                g = ops.mmvq_blocks(sub(L["e_gate"], e * Fe, (e + 1) * Fe), zq[b:b + 1], zd[b:b + 1])
                u = ops.mmvq_blocks(sub(L["e_up"], e * Fe, (e + 1) * Fe), zq[b:b + 1], zd[b:b + 1])
                hq, hd = _q_forced(ops.swiglu(g, u), fmid(b, rank), record, "expert mid")
                y = ops.mmvq_blocks(sub(L["e_down"], e * d, (e + 1) * d), hq, hd)
            else:
                g = ops.mmvq(L["e_gate"], zq[b:b + 1], zd[b:b + 1], r0=e * Fe, r1=(e + 1) * Fe)
                u = ops.mmvq(L["e_up"], zq[b:b + 1], zd[b:b + 1], r0=e * Fe, r1=(e + 1) * Fe)
                hq, hd = _q_forced(ops.swiglu(g, u), fmid(b, rank), record, "expert mid")
                y = ops.mmvq(L["e_down"], hq, hd, r0=e * d, r1=(e + 1) * d)
            acc += p[rank] * y[0]
        out[b] = acc
    # Shared expert: always on, weight 1, added after the routed sum.
    g = _mm(L["s_gate"], zq, zd, dense, blocks)
    u = _mm(L["s_up"], zq, zd, dense, blocks)
    hq, hd = _q_forced(ops.swiglu(g, u), None if forced is None else forced.get("shared_mid"), record, "shared mid")
    return out + _mm(L["s_down"], hq, hd, dense, blocks)


def _attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, length: int, win: int) -> np.ndarray:
    """Attention of one row over the ``length`` keys its cache holds after its append; with a
    sliding window ``win`` > 0 and ``length > win``, over the last ``win`` of them only
    (memra-engine decode_batch.rs, the SWA view of the Full-attention walk: the view starts at
    ``length - win`` and holds ``win`` keys, which keep their absolute rotation)."""
    if win and length > win:
        off = length - win
        return ops.attention(q, K[:, off:length], V[:, off:length], win)
    return ops.attention(q, K, V, length)


def decode_layer(model: Dict, il: int, caches: OracleCaches, x: np.ndarray, sessions: Sequence[int],
                 pos: Sequence[int], dense: Optional[DenseWeights] = None, blocks: bool = False,
                 info: Optional[Dict] = None, trace: Optional[List] = None, forced: Optional[Dict] = None,
                 record: Optional[List] = None) -> np.ndarray:
    """Layer ``il`` of the stack on the residual rows ``x[B, d]`` (fp64): returns the residual
    rows after the layer.  Row b appends its K/V at ``pos[b]`` of cache ``sessions[b]`` (layer
    il) and attends the first ``pos[b] + 1`` keys; every append precedes every attention
    (phase A / phase B of the batched walk), so rows sharing a cache at consecutive positions
    attend causally.  ``info`` (MoE layers) receives the routing of each row.  ``forced``
    (optional) holds another evaluation's codes for the layer's quantisations ("attn_in",
    "attn_out", "ffn_in", "ffn_mid", "shared_mid"; int8 rows), taken as described at
    ``_q_forced`` with ``record`` receiving the counts."""
    fc = (lambda name: None) if forced is None else forced.get
    sp = model["spec"]
    L = model["layers"][il]
    H, G, hd, eps = sp.n_head, sp.n_head_kv, sp.head_dim, sp.rms_eps
    x = np.asarray(x, dtype=np.float64)
    B = x.shape[0]
    xn = ops.rmsnorm(x, L["attn_norm"], eps)
    xq, xd = _q_forced(xn, fc("attn_in"), record, "attn in")
    if L.get("mixer") == "linear":
        mixed = _linear_mixer(sp, L, caches, il, xq, xd, sessions, dense, blocks, fc, record, trace)
        return _after_mixer(sp, L, x, mixed, dense, blocks, info, forced, record, fc, trace, il, None)
    qkv = _mm(L["wqkv"], xq, xd, dense, blocks)
    q = qkv[:, : H * hd].reshape(B, H, hd)
    k = qkv[:, H * hd: (H + G) * hd].reshape(B, G, hd)
    v = qkv[:, (H + G) * hd: (H + 2 * G) * hd].reshape(B, G, hd)
    # output gate (gated layers): H hd more projection rows after v, one gate per attention
    # output element
    gate = qkv[:, (H + 2 * G) * hd:(2 * H + 2 * G) * hd].reshape(B, H, hd) if L.get("attn_gate") else None
    if "q_norm" in L:   # QK-norm: every head RMS-normalised over its hd values, before RoPE
        q = ops.rmsnorm(q, L["q_norm"], eps)
        k = ops.rmsnorm(k, L["k_norm"], eps)
    q = np.stack([ops.rope_neox(q[b], pos[b], sp.rope_base) for b in range(B)])
    k = np.stack([ops.rope_neox(k[b], pos[b], sp.rope_base) for b in range(B)])
    fp8 = getattr(sp, "kv_fp8", False)
    q8 = getattr(sp, "kv_q8", False)
    for b in range(B):                                   # phase A: append all rows
        s = sessions[b]
        if fp8:   # FP8 caches: the nearest E4M3 code of each value
            caches.K[s][il][:, pos[b]] = ops.e4m3_encode(k[b])
            caches.V[s][il][:, pos[b]] = ops.e4m3_encode(v[b])
        elif q8:  # int8 caches: Q8_0 blocks of the fp32 values
            caches.K[s][il][:, pos[b]] = ops.q8_kv_encode(k[b].astype(np.float32))
            caches.V[s][il][:, pos[b]] = ops.q8_kv_encode(v[b].astype(np.float32))
        else:
            caches.K[s][il][:, pos[b]] = k[b].astype(np.float16)
            caches.V[s][il][:, pos[b]] = v[b].astype(np.float16)
    win = int(L.get("swa_window", 0))

    def kv(s):   # the values a row attends (codes read as their values)
        K, V = caches.K[s][il], caches.V[s][il]
        if fp8:
            return ops.e4m3_decode(K), ops.e4m3_decode(V)
        if q8:
            return ops.q8_kv_decode(K, hd), ops.q8_kv_decode(V, hd)
        return K, V
    attn = np.stack([_attend(q[b], *kv(sessions[b]), pos[b] + 1, win)
                     for b in range(B)])                  # phase B: attend
    if gate is not None:   # every attention output element times sigmoid of its gate, before W_o
        attn = attn * ops.sigmoid(gate)
    aq, ad = _q_forced(attn.reshape(B, H * hd), fc("attn_out"), record, "attn out")
    return _after_mixer(sp, L, x, (aq, ad), dense, blocks, info, forced, record, fc, trace, il,
                        {"q": q, "k": k, "v": v, "attn": attn})


def _linear_mixer(sp, L: Dict, caches: OracleCaches, il: int, xq, xd, sessions, dense, blocks, fc, record, trace):
    """The gated delta-rule mixer of a linear layer (memra-engine decode_batch.rs, the Linear
    arm of ``decode_batch_layers``): one product of the normed input gives the conv channels,
    z, beta and alpha; per row, the conv ring step, the prep, the state step (scale
    1/sqrt(d_state)), the gated norm; returns Q() of the gated-norm rows (the out product's
    input).  Each row's recurrent state in ``caches.R`` is updated in place."""
    B = xq.shape[0]
    nk, nv, ds = sp.ssm_n_k, sp.ssm_n_v, sp.ssm_d_state
    C, Vd = sp.ssm_conv_dim, sp.ssm_value_dim
    proj = _mm(L["wqkv"], xq, xd, dense, blocks)
    y = np.empty((B, Vd), dtype=np.float64)
    for b in range(B):
        st = caches.R[sessions[b]][il]
        conv_out, st["conv"] = ops.ssm_conv_step(st["conv"], proj[b, :C], L["ssm_conv"])
        z = proj[b, C:C + Vd]
        beta_raw = proj[b, C + Vd:C + Vd + nv]
        alpha = proj[b, C + Vd + nv:C + Vd + 2 * nv]
        q, k, v, g, beta = ops.gdn_prep(conv_out, beta_raw, alpha, L["ssm_dt"], L["ssm_a"], ds, nk, nv, sp.rms_eps)
        st["S"], o = ops.gdn_step(st["S"], q, k, v, g, beta, 1.0 / np.sqrt(ds))
        y[b] = ops.gated_rmsnorm(o, L["ssm_norm"], z.reshape(nv, ds), sp.rms_eps).reshape(Vd)
        if trace is not None:
            trace.append({"layer": il, "row": b, "conv_out": conv_out, "q": q, "k": k, "v": v, "g": g,
                          "beta": beta, "o": o, "y": y[b].copy()})
    return _q_forced(y, fc("attn_out"), record, "mixer out")


def _after_mixer(sp, L: Dict, x, mixed, dense, blocks, info, forced, record, fc, trace, il, attn_trace):
    """The o (out) product of the mixer's quantised output, the residual add, and the FFN."""
    aq, ad = mixed
    x1 = x + _mm(L["wo"], aq, ad, dense, blocks)
    if trace is not None and attn_trace is not None:
        trace.append({"layer": il, **attn_trace, "x1": x1})
    eps = sp.rms_eps
    if not sp.has_ffn:
        return x1
    z = ops.rmsnorm(x1, L["ffn_norm"], eps)
    zq, zd = _q_forced(z, fc("ffn_in"), record, "ffn in")
    if sp.n_experts:
        f = moe_ffn(sp, L, z, zq, zd, dense, blocks, info, forced, record)
    else:
        g = _mm(L["w_gate"], zq, zd, dense, blocks)
        u = _mm(L["w_up"], zq, zd, dense, blocks)
        hq, hdd = _q_forced(ops.swiglu(g, u), fc("ffn_mid"), record, "ffn mid")
        f = _mm(L["w_down"], hq, hdd, dense, blocks)
    return x1 + f


def output_head(model: Dict, x: np.ndarray, dense: Optional[DenseWeights] = None, blocks: bool = False,
                forced: Optional[np.ndarray] = None, record: Optional[List] = None) -> np.ndarray:
    """The stack's output from the residual rows after its last layer: logits ``[B, vocab]``
    if the model has an lm_head (output norm, Q, lm_head), the output-normed rows if it has an
    output norm, else the residual rows themselves.  ``forced``: another evaluation's codes of
    the lm_head input (see ``_q_forced``)."""
    sp = model["spec"]
    x = np.asarray(x, dtype=np.float64)
    if model["final_norm"] is not None:
        x = ops.rmsnorm(x, model["final_norm"], sp.rms_eps)
    if model["lm_head"] is not None:
        oq, od = _q_forced(x, forced, record, "head in")
        x = _mm(model["lm_head"], oq, od, dense, blocks)
    return x


def decode_step(model: Dict, caches: OracleCaches, x_in: np.ndarray, sessions: Sequence[int],
                pos: Sequence[int], dense: Optional[DenseWeights] = None, blocks: bool = False,
                info: Optional[Dict] = None, trace: Optional[List] = None) -> np.ndarray:
    """One decode step for rows ``x_in[B, d]``; row b writes and reads cache ``sessions[b]``.

    Every layer in order (:func:`decode_layer`), then :func:`output_head`.  Returns logits
    ``[B, vocab]`` if the model has an lm_head, the output-normed rows if it has an output
    norm, else the residual stream.  Caches are updated in place.  ``info[il]`` receives the
    routing of MoE layer il.
    """
    x = np.asarray(x_in, dtype=np.float32).astype(np.float64)
    for il in range(len(model["layers"])):
        x = decode_layer(model, il, caches, x, sessions, pos, dense, blocks,
                         info.setdefault(il, {}) if info is not None else None, trace)
    return output_head(model, x, dense, blocks)

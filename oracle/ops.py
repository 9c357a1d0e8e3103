"""Per-operation definitions of the batched decode step, in plain fp64 numpy.

TEST INFRASTRUCTURE ONLY: nothing in the product path imports this module.

Each function restates the operation from its definition; the pages it follows
are cited by title and section.  fp32 appears only at the rounding points the
method defines as part of its result: the activation quantiser (its integers
are part of the output of the quantise step) and the fp16 KV store.
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np

QK = 32  # elements per quantisation block


# ---------------------------------------------------------------------------------------
# Weight codecs
# ---------------------------------------------------------------------------------------
def weight_codes(w: Dict, r0: int = 0, r1: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Integer codes ``q[n, nb, 32]`` (int64) and fp64 block scales ``d[n, nb]`` of rows [r0, r1).

    Q8_0 (memra-engine decode_batch.rs, the exact-16 admission list names QT_Q8_0 as a
    per-block int8 class): each 32-element block stores int8 codes q in [-127, 127] and one
    fp16 scale; the value is ``d * q``.

    Q4_0 (same list, QT_Q4_0; hf2q ADR-040 names Q4_0 among GGUF weight types): each block
    stores 16 bytes; byte j holds the code of element j in its low nibble and of element
    j + 16 in its high nibble; the signed value is ``nibble - 8`` (range [-8, 7]).
    """
    r1 = w["n"] if r1 is None else r1
    nb = w["k"] // QK
    d = w["d"][r0:r1].astype(np.float64)
    if w["fmt"] == "q8_0":
        q = w["qs"][r0:r1].astype(np.int64).reshape(r1 - r0, nb, QK)
    elif w["fmt"] == "q4_0":
        by = w["qs"][r0:r1].reshape(r1 - r0, nb, QK // 2).astype(np.int64)
        lo = by & 0x0F          # elements 0..15 of the block
        hi = by >> 4            # elements 16..31 of the block
        q = np.concatenate([lo, hi], axis=2) - 8
    else:
        raise ValueError(w["fmt"])
    return q, d


def dequantize(w: Dict, r0: int = 0, r1: Optional[int] = None) -> np.ndarray:
    """Dense fp64 values ``[r1 - r0, k]`` of a quantised matrix: ``w = d * q`` per block
    (Q8_0, Q4_0), or the super-block formulas of :func:`kquant_fields` (Q4_K, Q5_K, Q6_K)."""
    if w["fmt"] in KQ_BYTES:
        return kquant_dequantize(w, r0, r1)
    q, d = weight_codes(w, r0, r1)
    return (q.astype(np.float64) * d[:, :, None]).reshape(q.shape[0], -1)


# ---------------------------------------------------------------------------------------
# K-quant weight codecs (super-blocks of 256 values)
# ---------------------------------------------------------------------------------------
# The pages name Q4_K, Q5_K and Q6_K among the weight types a batched decode must cover
# (hf2q ADR-040, "Quant scope": the fused batch decode path covers every inference ftype,
# Q4_K, Q5_K and Q6_K among them; memra-engine decode_batch.rs, the exact-16 admission list
# admits QT_Q4_K, QT_Q5_K and QT_Q6_K) but do not spell out their bytes.  The reading used
# here is the GGUF k-quant block format those names denote, one super-block of 256 values
# per record, rows of k / 256 records:
#   Q4_K, 144 bytes: fp16 d, fp16 dmin, 12 bytes of 6-bit sub-block scales and mins, 128
#         bytes of 4-bit codes.  Value = d * sc_j * q - dmin * m_j in 32-value sub-block j.
#   Q5_K, 176 bytes: as Q4_K, then 32 bytes of fifth bits before the 4-bit codes; q has 5 bits.
#   Q6_K, 210 bytes: 128 bytes of low 4 bits, 64 bytes of upper 2 bits, 16 int8 scales (one
#         per 16 values), fp16 d.  Value = d * sc_(e // 16) * (q - 32), q of 6 bits.
KQ_BYTES = {"q4_k": 144, "q5_k": 176, "q6_k": 210}
QK_K = 256


def kquant_scale_min(sc12: np.ndarray, j: int) -> Tuple[np.ndarray, np.ndarray]:
    """6-bit scale and min of sub-block j (0..7) from the 12 packed bytes (``[..., 12]``).

    Sub-blocks 0..3 keep both in the low 6 bits of bytes j (scale) and j + 4 (min).
    Sub-blocks 4..7 keep their low 4 bits in byte j + 4 (scale in the low nibble, min in the
    high one) and their top 2 bits in the spare top bits of bytes j - 4 (scale) and j (min).
    """
    b = sc12.astype(np.int64)
    if j < 4:
        return b[..., j] & 63, b[..., j + 4] & 63
    sc = (b[..., j + 4] & 15) | ((b[..., j - 4] >> 6) << 4)
    mn = (b[..., j + 4] >> 4) | ((b[..., j] >> 6) << 4)
    return sc, mn


def _f16_at(blocks: np.ndarray, off: int) -> np.ndarray:
    return np.ascontiguousarray(blocks[..., off:off + 2]).view(np.float16)[..., 0].astype(np.float64)


def kquant_fields(w: Dict, r0: int = 0, r1: Optional[int] = None) -> Dict[str, np.ndarray]:
    """The fields of rows [r0, r1) of a K-quant matrix, per super-block s of each row:

    * ``q``: the codes ``[n, nsb, 256]`` in value order (int64; Q4_K 0..15, Q5_K 0..31,
      Q6_K 0..63 before its offset of 32);
    * Q4_K / Q5_K: ``d``, ``dmin`` ``[n, nsb]`` and the sub-block ``sc``, ``m`` ``[n, nsb, 8]``;
    * Q6_K: ``d`` ``[n, nsb]`` and the int8 ``sc`` ``[n, nsb, 16]``.

    Value order within a super-block: Q4_K/Q5_K code bytes come in 4 runs of 32; byte l of
    run c holds value 64c + l in its low nibble and value 64c + 32 + l in its high nibble;
    the fifth bit of value 64c + l is bit 2c of fifth-bit byte l, of value 64c + 32 + l bit
    2c + 1.  Q6_K: two halves of 128 values, half h with low bytes [64h, 64h + 64) and upper
    bytes [32h, 32h + 32); for l < 32, low byte 64h + l gives values 128h + l (low nibble)
    and 128h + 64 + l (high nibble), low byte 64h + 32 + l gives 128h + 32 + l and 128h + 96 + l,
    and upper byte 32h + l gives those four values' top two bits in bit pairs 0-1, 2-3, 4-5, 6-7
    (in the order 128h + l, 128h + 32 + l, 128h + 64 + l, 128h + 96 + l).
    """
    fmt, k = w["fmt"], w["k"]
    r1 = w["n"] if r1 is None else r1
    assert k % QK_K == 0
    nsb, BS = k // QK_K, KQ_BYTES[fmt]
    blk = np.ascontiguousarray(w["qs"][r0:r1]).view(np.uint8).reshape(r1 - r0, nsb, BS)
    n = r1 - r0
    if fmt in ("q4_k", "q5_k"):
        out = {"d": _f16_at(blk, 0), "dmin": _f16_at(blk, 2)}
        sc12 = blk[..., 4:16]
        pairs = [kquant_scale_min(sc12, j) for j in range(8)]
        out["sc"] = np.stack([p[0] for p in pairs], axis=-1)
        out["m"] = np.stack([p[1] for p in pairs], axis=-1)
        qs = blk[..., -128:].astype(np.int64).reshape(n, nsb, 4, 32)      # runs c, bytes l
        q = np.empty((n, nsb, 4, 2, 32), dtype=np.int64)                  # value 64c + 32h + l
        q[:, :, :, 0] = qs & 15
        q[:, :, :, 1] = qs >> 4
        if fmt == "q5_k":
            qh = blk[..., 16:48].astype(np.int64)                          # byte l
            for c in range(4):
                for h in range(2):
                    q[:, :, c, h] += 16 * ((qh >> (2 * c + h)) & 1)
        out["q"] = q.reshape(n, nsb, QK_K)
        return out
    if fmt == "q6_k":
        ql = blk[..., 0:128].astype(np.int64).reshape(n, nsb, 2, 2, 32)    # half h, run r, byte l
        qh = blk[..., 128:192].astype(np.int64).reshape(n, nsb, 2, 32)     # half h, byte l
        q = np.empty((n, nsb, 2, 4, 32), dtype=np.int64)                   # value 128h + 32i + l
        q[:, :, :, 0] = (ql[:, :, :, 0] & 15) | (((qh >> 0) & 3) << 4)
        q[:, :, :, 1] = (ql[:, :, :, 1] & 15) | (((qh >> 2) & 3) << 4)
        q[:, :, :, 2] = (ql[:, :, :, 0] >> 4) | (((qh >> 4) & 3) << 4)
        q[:, :, :, 3] = (ql[:, :, :, 1] >> 4) | (((qh >> 6) & 3) << 4)
        return {"q": q.reshape(n, nsb, QK_K), "sc": blk[..., 192:208].view(np.int8).astype(np.int64),
                "d": _f16_at(blk, 208)}
    raise ValueError(fmt)


def kquant_dequantize(w: Dict, r0: int = 0, r1: Optional[int] = None) -> np.ndarray:
    """Dense fp64 values ``[r1 - r0, k]`` of a K-quant matrix (formulas of the block format)."""
    f = kquant_fields(w, r0, r1)
    q = f["q"].astype(np.float64)
    n, nsb, _ = q.shape
    if w["fmt"] == "q6_k":
        scale = f["d"][:, :, None] * f["sc"].astype(np.float64)            # per 16 values
        v = (q - 32.0).reshape(n, nsb, 16, 16) * scale[:, :, :, None]
    else:
        scale = f["d"][:, :, None] * f["sc"].astype(np.float64)            # per 32 values
        mins = f["dmin"][:, :, None] * f["m"].astype(np.float64)
        v = q.reshape(n, nsb, 8, 32) * scale[:, :, :, None] - mins[:, :, :, None]
    return v.reshape(n, nsb * QK_K)


# ---------------------------------------------------------------------------------------
# Activation quantiser Q(.)
# ---------------------------------------------------------------------------------------
def quantize_act(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric per-32-block int8 quantisation of fp32 rows ``x[B, K]``.

    The pages name the step (memra-engine decode_batch.rs, ``decode_batch_layers``: one
    ``quantize_q8_1`` of the normed rows feeds the q/k/v products, one feeds gate/up, one
    the down product) and its consumer (int8 dot products, the dp4a / batched-mmvq classes
    in the exact-16 admission notes), but not its arithmetic.  The reading used here:
    per block, ``a = max |x_i|``; if ``a == 0`` the scale and codes are 0; otherwise
    ``d = fp32(a / 127)`` (IEEE fp32 division) and ``q_i = clamp(round_half_away(fp32(x_i / d)),
    -127, 127)``.  Returns int8 codes ``[B, K]`` and fp32 scales ``[B, K/32]``.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    B, K = x.shape
    assert K % QK == 0
    blk = x.reshape(B, K // QK, QK)
    a = np.max(np.abs(blk), axis=2)                                 # exact in fp32
    d = (a / np.float32(127.0)).astype(np.float32)                  # IEEE fp32 division
    safe = np.where(d == 0, np.float32(1.0), d).astype(np.float32)
    ratio = (blk / safe[:, :, None]).astype(np.float32)             # IEEE fp32 division
    r64 = ratio.astype(np.float64)                                  # exact widening
    rounded = np.sign(r64) * np.floor(np.abs(r64) + 0.5)            # half away from zero, exact in fp64
    q = np.clip(rounded, -127, 127).astype(np.int64)
    q[d == 0] = 0
    return q.reshape(B, K).astype(np.int8), d


# ---------------------------------------------------------------------------------------
# mmvq: block-quantised matrix times B quantised rows
# ---------------------------------------------------------------------------------------
def block_dots(w: Dict, xq: np.ndarray, r0: int = 0, r1: Optional[int] = None) -> np.ndarray:
    """Exact per-block integer dot products ``S[b, n, blk] = sum_i q_w[n, blk, i] * q_x[b, blk, i]``."""
    qw, _ = weight_codes(w, r0, r1)
    B = xq.shape[0]
    qx = xq.astype(np.int64).reshape(B, -1, QK)
    return np.einsum("nki,bki->bnk", qw, qx, optimize=True)


def mmvq_blocks(w: Dict, xq: np.ndarray, xd: np.ndarray) -> np.ndarray:
    """Block formula ``y[b, n] = sum_blk d_w[n, blk] * d_x[b, blk] * S[b, n, blk]`` in fp64.

    One weight read serves all B rows (memra-engine decode_batch.rs module header: every
    projection at m = B rows amortises one weight read; hf2q ADR-040 §0.7 F3, small-m
    quantised decode GEMM).
    """
    S = block_dots(w, xq).astype(np.float64)
    _, dw = weight_codes(w)
    return np.einsum("nk,bk,bnk->bn", dw, xd.astype(np.float64), S, optimize=True)


def dequantize_act(xq: np.ndarray, xd: np.ndarray) -> np.ndarray:
    B, K = xq.shape
    return (xq.astype(np.float64).reshape(B, K // QK, QK) * xd.astype(np.float64)[:, :, None]).reshape(B, K)


def mmvq(w: Dict, xq: np.ndarray, xd: np.ndarray, dense: Optional[np.ndarray] = None,
         r0: int = 0, r1: Optional[int] = None, chunk: int = 4096) -> np.ndarray:
    """Same value as :func:`mmvq_blocks` via a dense fp64 product (dequantise, then matmul).

    ``sum_k (d_w q_w)(d_x q_x)`` regroups the block formula's terms, so the two agree to
    fp64 rounding; the dense form lets BLAS do the work on large shapes.  Rows [r0, r1) of
    the matrix only; ``dense`` may hold a cached dequantised copy of those rows.
    """
    r1 = w["n"] if r1 is None else r1
    xv = dequantize_act(xq, xd)
    if dense is not None:
        return xv @ dense.T
    out = np.empty((xq.shape[0], r1 - r0), dtype=np.float64)
    for c0 in range(r0, r1, chunk):
        c1 = min(r1, c0 + chunk)
        out[:, c0 - r0:c1 - r0] = xv @ dequantize(w, c0, c1).T
    return out


# ---------------------------------------------------------------------------------------
# Row operations
# ---------------------------------------------------------------------------------------
def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """``y = x / sqrt(mean(x^2) + eps) * g`` per row (memra-engine decode_batch.rs, the
    attn_norm / post_attn_norm / output-norm calls of the batched layer walk)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def rope_neox(x: np.ndarray, pos: int, base: float) -> np.ndarray:
    """NEOX rotary embedding of heads ``x[n_heads, hd]`` at position ``pos``.

    Element i < hd/2 pairs with element i + hd/2 and both rotate by
    ``theta_i = pos * base^(-2i/hd)``; every dim is rotated (memra-engine decode_batch.rs,
    ``rope_neox`` on q and k with the per-row position buffer).
    """
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    theta = float(pos) * np.power(float(base), -2.0 * i / hd)
    c, s = np.cos(theta), np.sin(theta)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def silu(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def sigmoid(g: np.ndarray) -> np.ndarray:
    """``1 / (1 + e^-g)`` in fp64 (memra-engine decode_batch.rs, the attention output gate)."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):   # e^-g = inf for g << 0 gives the limit 0 exactly
        return 1.0 / (1.0 + np.exp(-g))


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """``silu(g) * u`` (memra-engine decode_batch.rs, ``silu_mul`` between gate/up and down)."""
    return silu(g) * np.asarray(u, dtype=np.float64)


# ---------------------------------------------------------------------------------------
# Attention over one row's own cache
# ---------------------------------------------------------------------------------------
def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, t: int) -> np.ndarray:
    """Decode attention of one row: ``q[H, hd]`` over keys ``[0, t)`` of ``K, V[G, >=t, hd]``.

    Query head h reads KV head ``h // (H / G)`` (consecutive query heads share a KV head);
    ``score_j = q_h . K_j / sqrt(hd)``; ``p = softmax(score)``; ``out_h = sum_j p_j V_j``.
    No split: the split-K partition is an evaluation order, not part of the definition.
    (memra-engine decode_batch.rs: scale ``1/sqrt(head_dim)``, ``t_kv = pos + 1``.)
    """
    q = np.asarray(q, dtype=np.float64)
    H, hd = q.shape
    G = K.shape[0]
    grp = H // G
    out = np.empty((H, hd), dtype=np.float64)
    scale = 1.0 / np.sqrt(hd)
    for h in range(H):
        g = h // grp
        k = K[g, :t].astype(np.float64)
        v = V[g, :t].astype(np.float64)
        s = (k @ q[h]) * scale
        p = np.exp(s - np.max(s))
        p /= np.sum(p)
        out[h] = p @ v
    return out


# ---------------------------------------------------------------------------------------
# Router
# ---------------------------------------------------------------------------------------
def router_topk(r: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k experts of router logits ``r[E]`` and their softmax weights.

    Ranked by descending logit, ties to the lower expert id; weights are the softmax over
    the k selected logits (hf2q ADR-040 §0.7 F4 per-token top-k routing; the reading of the
    top-8 softmax router in the MoE workload).
    """
    r = np.asarray(r, dtype=np.float64)
    order = np.lexsort((np.arange(r.shape[0]), -r))   # primary: -r ascending; ties: id ascending
    ids = order[:k]
    z = r[ids] - np.max(r[ids])
    p = np.exp(z)
    p /= np.sum(p)
    return ids, p


# ---------------------------------------------------------------------------------------
# Next token
# ---------------------------------------------------------------------------------------
def greedy_token(logits: np.ndarray) -> np.ndarray:
    """Greedy token of each row of ``logits[B, n]``: the lowest index among the row's maxima.

    memra-engine 0.72.0, src/decode_batch.rs, ``decode_step_batch_sampled``: a greedy row
    takes the argmax of its logits, and the device result equals a host argmax.  The pages
    give no tie rule; the reading here is the first maximum, which a left-to-right scan that
    replaces its candidate only on a strictly larger value finds.  Rows are finite.
    """
    x = np.asarray(logits)
    out = np.empty(x.shape[0], dtype=np.int64)
    for b in range(x.shape[0]):
        m = np.max(x[b])
        out[b] = np.flatnonzero(x[b] == m)[0]
    return out


def embed_rows(table: np.ndarray, tokens: np.ndarray) -> np.ndarray:
    """The next step's input rows: row ``tokens[b]`` of the embedding table ``[vocab, d]``.

    memra-engine 0.72.0, src/decode_batch.rs, phase 0 of ``decode_step_batch``: each row
    enters the stack as its token's embedding row.
    """
    return np.asarray(table)[np.asarray(tokens, dtype=np.int64)].copy()


def accept_drafts(greedy: np.ndarray, fed: np.ndarray, k: int):
    """Accepted prefix of speculative-verify rows, per stream (rows stream-major, k each).

    Strata PR #1524, "What changes" (target verification of concurrent streams' drafts with
    accepted-prefix state commits).  Row j of a stream took token ``fed[j]`` as input (j = 0:
    the last committed token, j >= 1: draft j) and its greedy token ``greedy[j]`` is the
    target's choice after it.  Reading (greedy verification): walk the drafts in order and keep
    draft j while the previous row's greedy token equals it; the token after the kept prefix is
    the greedy token of the last kept row.  Returns (n_accept, next_token) per stream.
    """
    g = np.asarray(greedy).reshape(-1, k)
    f = np.asarray(fed).reshape(-1, k)
    n_acc, nxt = [], []
    for s in range(g.shape[0]):
        a = 0
        for j in range(1, k):
            if g[s, j - 1] != f[s, j]:
                break
            a = j
        n_acc.append(a)
        nxt.append(int(g[s, a]))
    return np.array(n_acc, dtype=np.int64), np.array(nxt, dtype=np.int64)



# ---------------------------------------------------------------------------------------
# FP8 KV cache codec
# ---------------------------------------------------------------------------------------
def e4m3_values() -> np.ndarray:
    """fp64 value of each of the 256 FP8 E4M3 codes (NaN for the two NaN codes).

    memra-engine decode_batch.rs, phase A of ``decode_batch_layers``: the KV append stores
    quantised rows and an engine switch turns the store to fp8 (``kv_fp8_on``); the format is
    not spelled out there.  Reading: the OCP 8-bit E4M3 encoding -- bit 7 sign, bits 6..3 a
    biased exponent e (bias 7), bits 2..0 a mantissa m; e > 0: 2^(e-7) (1 + m/8); e = 0:
    2^-6 m/8; no infinities; e = 15 with m = 7 is NaN.  One value per element, no scale.
    """
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 0x7
        if e == 15 and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """uint8 E4M3 codes of x: the nearest finite code, ties to the even code (even mantissa);
    magnitudes past 448, the largest finite value, take 448 (saturation); the sign of x --
    including -0 -- is kept; NaN gives 0x7F (0xFF if its sign bit is set).

    Reading of the store's rounding (the pages fix none): round to nearest even, saturating,
    the usual fp8 KV-cache conversion.  Done by brute force over the 127 non-negative finite
    codes: the code minimising |value - |x||, the even one of two at equal distance.
    """
    xa = np.asarray(x, dtype=np.float64)
    vals = e4m3_values()[:0x7F]                       # codes 0x00 .. 0x7E, ascending values
    a = np.minimum(np.abs(xa), vals[-1]).reshape(-1)
    dist = np.abs(a[:, None] - vals[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best                              # one code, or two at a tie
    codes = np.arange(0x7F)
    even = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    out = pick.astype(np.uint8).reshape(xa.shape)
    out = np.where(np.isnan(xa), np.uint8(0x7F), out)
    return np.where(np.signbit(xa), out | np.uint8(0x80), out).astype(np.uint8)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """fp64 values of E4M3 codes (see ``e4m3_values``)."""
    return e4m3_values()[np.asarray(codes, dtype=np.uint8).astype(np.int64)]


# ---------------------------------------------------------------------------------------
# Gated delta-rule recurrent state (linear-attention layers)
# ---------------------------------------------------------------------------------------
def gdn_step(S: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray, g: np.ndarray, beta: np.ndarray,
             scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """One decode step of the gated delta rule for every value head of one row.

    memra-engine decode_batch.rs, the Linear mixer of ``decode_batch_layers``: after the
    batched projections and the prep launch (L2-normalised q and k, the gate beta and the
    log-decay g per value head), one batched scan launch reads each sequence's state and
    writes its other buffer, with the scale 1/sqrt(d_state); the update itself is not spelled
    out there.  Reading (the published gated delta rule): per head, with state S [d_v, d_k],
    decay a = exp(g), S' = a S, the delta-rule correction writes v at key k with strength beta:
    S_new = S' + beta (v - S' k) k^T, and the output is o = scale S_new q.
    S [H, d_v, d_k], q and k [H, d_k], v [H, d_v], g and beta [H]; returns (S_new, o), fp64.
    """
    S = np.asarray(S, dtype=np.float64)
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    a = np.exp(np.asarray(g, dtype=np.float64))[:, None, None]
    Sd = a * S
    u = np.einsum("hvk,hk->hv", Sd, k)                     # what the decayed state recalls at k
    b = np.asarray(beta, dtype=np.float64)[:, None, None]
    S_new = Sd + b * (v - u)[:, :, None] * k[:, None, :]
    o = scale * np.einsum("hvk,hk->hv", S_new, q)
    return S_new, o


# ---------------------------------------------------------------------------------------
# int8 (Q8_0-block) KV cache codec
# ---------------------------------------------------------------------------------------
def q8_kv_row_bytes(hd: int) -> int:
    """Bytes of one cached (position, KV head) row: hd int8 codes, hd/32 fp16 block scales,
    zero padding to a multiple of 16 bytes."""
    return hd + 16


def q8_kv_encode(x: np.ndarray) -> np.ndarray:
    """Cache rows (uint8 ``[..., hd + 16]``) of fp32 values ``x[..., hd]``.

    memra-engine decode_batch.rs, phase A of ``decode_batch_layers``: the append stores
    quantised K/V rows (``append_kv_quantized_seqs``, with per-token row bytes); Strata PR #1524
    "What changes" runs with resident int8 KV.  The byte format is not given.  Reading: Q8_0
    blocks along the head row -- per 32 consecutive elements a = max |x_i|, the stored scale
    d = fp16(a / 127) (fp32 division, then round to nearest even), and codes
    q_i = clamp(round_half_away(x_i / d), -127, 127) with the stored scale as an fp32 number
    (all zero when d is 0); the value of a code is d q_i.  A row is its hd codes, then its
    hd/32 scales, then zeros up to hd + 16 bytes.
    """
    x = np.asarray(x, dtype=np.float32)
    hd = x.shape[-1]
    assert hd % 32 == 0
    lead = x.shape[:-1]
    blk = x.reshape(-1, hd // 32, 32)
    a = np.max(np.abs(blk), axis=2)
    d16 = (a / np.float32(127.0)).astype(np.float32).astype(np.float16)      # RNE to fp16
    df = d16.astype(np.float32)
    safe = np.where(df == 0, np.float32(1.0), df)
    r = (blk / safe[:, :, None]).astype(np.float32).astype(np.float64)       # IEEE fp32 division
    q = np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), -127, 127)
    q = np.where((df == 0)[:, :, None], 0, q).astype(np.int8)
    out = np.zeros((blk.shape[0], q8_kv_row_bytes(hd)), dtype=np.uint8)
    out[:, :hd] = q.reshape(-1, hd).view(np.uint8)
    out[:, hd:hd + 2 * (hd // 32)] = d16.view(np.uint8).reshape(-1, 2 * (hd // 32))
    return out.reshape(*lead, q8_kv_row_bytes(hd))


def q8_kv_decode(rows: np.ndarray, hd: int) -> np.ndarray:
    """fp64 values ``[..., hd]`` of cache rows written by :func:`q8_kv_encode` (d q_i)."""
    rows = np.asarray(rows, dtype=np.uint8)
    lead = rows.shape[:-1]
    flat = rows.reshape(-1, rows.shape[-1])
    q = flat[:, :hd].view(np.int8).astype(np.float64).reshape(-1, hd // 32, 32)
    d = np.ascontiguousarray(flat[:, hd:hd + 2 * (hd // 32)]).view(np.float16).astype(np.float64)
    return (q * d[:, :, None]).reshape(*lead, hd)


# ---------------------------------------------------------------------------------------
# Linear-attention (gated delta rule) layer pieces around the state step
# ---------------------------------------------------------------------------------------
def softplus(x: np.ndarray) -> np.ndarray:
    """log(1 + e^x) in fp64 (written as logaddexp(0, x), which does not overflow)."""
    return np.logaddexp(0.0, np.asarray(x, dtype=np.float64))


def l2_normalize(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(sum(x^2) + eps) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def ssm_conv_step(state: np.ndarray, x: np.ndarray, w: np.ndarray):
    """One decode step of the causal depthwise convolution that feeds the linear mixer.

    memra-engine decode_batch.rs, the Linear mixer of ``decode_batch_layers``: the mixed
    projection passes through a fused conv ring per sequence (``ssm_conv1d_fused_decode_b``,
    kernel width d_conv) before the prep.  Reading: channel c's output is
    silu(sum_j w[c, j] window[j, c]) over the window of the last d_conv inputs, oldest first --
    the d_conv - 1 held in the ring (``state [d_conv - 1, C]``) and this step's input ``x [C]``;
    the ring then holds the newest d_conv - 1 of them.  Returns (y [C], new state), fp64.
    """
    state = np.asarray(state, dtype=np.float64)
    window = np.concatenate([state, np.asarray(x, dtype=np.float64)[None, :]], axis=0)   # [d_conv, C]
    pre = np.einsum("cj,jc->c", np.asarray(w, dtype=np.float64), window)
    return silu(pre), window[1:].copy()


def gdn_prep(conv_out: np.ndarray, beta_raw: np.ndarray, alpha: np.ndarray, dt_bias: np.ndarray, a: np.ndarray,
             d_state: int, n_k: int, n_v: int, eps: float):
    """The prep between the conv and the state step, for one row.

    memra-engine decode_batch.rs (``gdn_prep_decode_b``): from the conv outputs and the beta /
    alpha projections it leaves L2-normalised q and k, v, a gate beta and a log-decay g per
    value head.  Reading: the conv output is q (n_k heads of d_state), then k (n_k heads), then
    v (n_v heads); value head h uses key head h // (n_v / n_k) for q and k; q and k are
    L2-normalised per head (``l2_normalize`` with the model's eps); beta = sigmoid(beta_raw);
    g = a softplus(alpha + dt_bias), a being the layer's negative per-head decay rate.
    Returns q, k, v [n_v, d_state] and g, beta [n_v], fp64.
    """
    c = np.asarray(conv_out, dtype=np.float64)
    kd_ = d_state * n_k
    qh = c[:kd_].reshape(n_k, d_state)
    kh = c[kd_:2 * kd_].reshape(n_k, d_state)
    v = c[2 * kd_:2 * kd_ + d_state * n_v].reshape(n_v, d_state)
    rep = np.arange(n_v) // (n_v // n_k)
    q = l2_normalize(qh, eps)[rep]
    k = l2_normalize(kh, eps)[rep]
    beta = sigmoid(beta_raw)
    g = np.asarray(a, dtype=np.float64) * softplus(np.asarray(alpha, dtype=np.float64) +
                                                   np.asarray(dt_bias, dtype=np.float64))
    return q, k, v, g, beta


def gated_rmsnorm(o: np.ndarray, w: np.ndarray, z: np.ndarray, eps: float) -> np.ndarray:
    """The linear mixer's output norm (memra-engine decode_batch.rs ``gated_rmsnorm`` over
    d_state per value head, with the z projection): y = rmsnorm(o_h) w * silu(z_h) for every
    head's row of d_state values (``o``, ``z`` [..., d_state], ``w`` [d_state])."""
    return rmsnorm(o, w, eps) * silu(z)

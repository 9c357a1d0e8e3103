"""Seeded synthetic inputs for the batched multi-session decode step.

This module is shared by the CPU oracle and the GPU harness, so it holds *only*
shapes and random draws: no arithmetic of the decode step (no quantisation, no
nibble decoding, no norm, no attention) lives here.  Every array is produced by
an independent numpy stream keyed by (seed, config, tensor, layer, index), so a
single tensor can be regenerated without drawing the others.

Distributions follow the workload descriptions of the batched-decode pages:

* Q8_0 weights: 32-element blocks of int8 drawn uniformly from the closed range
  [-127, 127] plus one fp16 scale ``|N(0, 0.02)| / 127`` per block.
* Q4_0 weights: 32-element blocks of 4-bit codes drawn uniformly (a uniformly
  random byte holds two uniformly random 4-bit codes), plus one fp16 scale
  ``|N(0, 0.02)| / 8`` per block (same max-|w| scale as Q8_0).
* Norm gains ``1 + 0.1 N(0, 1)`` (fp32), router weights ``N(0, 0.02)`` (fp32),
  step inputs ``N(0, 1)`` fp32 rows, token embedding rows ``N(0, 1)`` fp32, KV prefill
  ``fp16(N(0, 1))``.

Storage conventions of the arrays produced here (both sides read them):

* Q8_0 ``qs``: int8 ``[n_out, k]`` row-major; ``d``: fp16 ``[n_out, k/32]``.
* Q4_0 ``qs``: uint8 ``[n_out, k/2]`` (16 bytes per 32-element block, the
  block's bytes contiguous); ``d``: fp16 ``[n_out, k/32]``.
* Q4_K / Q5_K / Q6_K ``qs``: uint8 ``[n_out, (k/256) * record]``, each row's 256-value
  records of 144 / 176 / 210 bytes back to back (their scales inside); ``d``: empty
  ``[n_out, 0]``.
* KV prefill for one (session, layer): fp16 ``[G, L, hd]`` for K and for V (uint8 E4M3
  codes of the same shape for FP8 caches; uint8 rows ``[G, L, hd + 16]`` for int8 caches).
"""
from __future__ import annotations

import math
import dataclasses
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

# Tensor codes for the per-tensor seed key (stable across versions).
T_ATTN_NORM, T_WQKV_Q, T_WQKV_D, T_WO_Q, T_WO_D, T_FFN_NORM = 1, 2, 3, 4, 5, 6
T_GATE_Q, T_GATE_D, T_UP_Q, T_UP_D, T_DOWN_Q, T_DOWN_D = 7, 8, 9, 10, 11, 12
T_ROUTER = 13
T_EGATE_Q, T_EGATE_D, T_EUP_Q, T_EUP_D, T_EDOWN_Q, T_EDOWN_D = 14, 15, 16, 17, 18, 19
T_SGATE_Q, T_SGATE_D, T_SUP_Q, T_SUP_D, T_SDOWN_Q, T_SDOWN_D = 20, 21, 22, 23, 24, 25
T_FINAL_NORM, T_LM_Q, T_LM_D = 26, 27, 28
T_X_IN, T_K_PRE, T_V_PRE, T_LENGTHS = 29, 30, 31, 32
T_EMBED = 33
T_Q_NORM, T_K_NORM = 34, 35
T_SSM_IN_Q, T_SSM_IN_D, T_SSM_OUT_Q, T_SSM_OUT_D, T_SSM_CONV, T_SSM_DT, T_SSM_A, T_SSM_NORM = 36, 37, 38, 39, 40, 41, 42, 43
T_REC_CONV, T_REC_S = 44, 45


def rng_for(seed: int, cfg_code: int, tensor: int, layer: int = 0, index: int = 0) -> np.random.Generator:
    """An independent numpy Generator for one tensor (SeedSequence keyed by the tuple)."""
    return np.random.default_rng([int(seed), int(cfg_code), int(tensor), int(layer), int(index)])


@dataclass(frozen=True)
class ModelSpec:
    """Shape of a decoder stack (plain pre-norm block; no biases, no QK-norm, no gate)."""
    name: str
    n_layers: int
    d: int
    n_head: int
    n_head_kv: int
    head_dim: int
    ffn: int                 # dense SwiGLU width; 0 = none (attention-only or MoE)
    fmt: str                 # "q8_0", "q4_0", "q4_k", "q5_k" or "q6_k": every quantised matrix not in fmts
    vocab: int = 0           # lm_head rows; 0 = no lm_head
    final_norm: bool = False
    n_experts: int = 0       # 0 = dense FFN
    n_expert_used: int = 0
    expert_ffn: int = 0
    shared_ffn: int = 0
    rope_base: float = 10000.0
    rms_eps: float = 1e-5
    swa_window: int = 0                  # sliding-window attention width (0: none)
    swa_layers: Tuple[int, ...] = ()     # the layers that use it
    qk_norm: bool = False                # per-head RMSNorm of q and k before RoPE
    attn_gate: bool = False              # attention output scaled by sigmoid of H hd more projection rows
    kv_fp8: bool = False                 # KV caches hold FP8 E4M3 codes (uint8) instead of fp16
    kv_q8: bool = False                  # KV caches hold int8 rows (Q8_0 blocks: codes + fp16 scales)
    linear_layers: Tuple[int, ...] = ()  # gated delta-rule linear-attention layers (the others: attention)
    ssm_d_state: int = 128               # linear layers: state size per head (d_k = d_v)
    ssm_n_k: int = 0                     # key heads (q and k)
    ssm_n_v: int = 0                     # value heads
    ssm_d_conv: int = 4                  # conv kernel width
    fmts: Tuple[Tuple[str, str], ...] = ()  # per-matrix format overrides: (role, fmt), role in
    #                                      wqkv, wo, w_gate, w_up, w_down, lm_head

    def fmt_of(self, role: str) -> str:
        return dict(self.fmts).get(role, self.fmt)

    @property
    def qkv_rows(self) -> int:
        return (self.n_head + 2 * self.n_head_kv + (self.n_head if self.attn_gate else 0)) * self.head_dim

    @property
    def ssm_key_dim(self) -> int:
        return self.ssm_d_state * self.ssm_n_k

    @property
    def ssm_value_dim(self) -> int:
        return self.ssm_d_state * self.ssm_n_v

    @property
    def ssm_conv_dim(self) -> int:
        return 2 * self.ssm_key_dim + self.ssm_value_dim

    @property
    def ssm_in_rows(self) -> int:
        """Rows of a linear layer's input projection: the conv's q, k, v channels, then z
        (value_dim), then beta and alpha (one per value head each)."""
        return self.ssm_conv_dim + self.ssm_value_dim + 2 * self.ssm_n_v

    @property
    def has_ffn(self) -> bool:
        return self.ffn > 0 or self.n_experts > 0

    @property
    def out_dim(self) -> int:
        return self.vocab if self.vocab else self.d


@dataclass
class Workload:
    """Sessions, rows and steps of one synthetic decode workload.

    ``rows[b] = (session, j)``: row b decodes in cache ``session`` at position
    ``prefill[session] + j + step``.  Several rows may share a session only at
    distinct positions (speculative-verify rows, causal within the stream).
    """
    code: int
    spec: ModelSpec
    prefill: List[int]                   # cache length of each session before step 0
    rows: List[Tuple[int, int]]          # (session, draft offset) per row
    steps: int
    capacity: int
    seed: int = 0
    note: str = ""

    @property
    def B(self) -> int:
        return len(self.rows)

    def positions(self, step: int) -> List[int]:
        """pos of each row at this step: the session's cache length before the row is written."""
        return [self.prefill[s] + j + step for (s, j) in self.rows]


# --------------------------------------------------------------------------------------
# The five workloads (shapes and session mixes) and their reduced variants for CPU tests.
# --------------------------------------------------------------------------------------
SPEC_C1 = ModelSpec("c1_1layer_d256_q8_0", 1, 256, 4, 2, 64, 1024, "q8_0")
SPEC_C2 = ModelSpec("c2_8layer_d2048_q8_0_lm32000", 8, 2048, 16, 4, 128, 5632, "q8_0",
                    vocab=32000, final_norm=True)
SPEC_C3 = ModelSpec("c3_attn_d4096_q8_0", 1, 4096, 32, 8, 128, 0, "q8_0")
SPEC_C4 = ModelSpec("c4_32layer_d4096_q4_0", 32, 4096, 32, 8, 128, 14336, "q4_0", final_norm=True)
SPEC_C5 = ModelSpec("c5_moe8layer_d2816_q4_0", 8, 2816, 16, 8, 128, 0, "q4_0", final_norm=True,
                    n_experts=128, n_expert_used=8, expert_ffn=704, shared_ffn=2816)
# the 8-layer Q8_0 decoder with gated delta-rule layers in place of attention on three of every
# four layers (attention on layers 3 and 7): 8 key heads and 16 value heads of 128, conv width 4
SPEC_HYBRID = dataclasses.replace(SPEC_C2, name="hybrid_8layer_d2048_q8_0_gdn_lm32000",
                                  linear_layers=(0, 1, 2, 4, 5, 6), ssm_n_k=8, ssm_n_v=16)
# the same 8-layer decoder with K-quant weights in a mix of the kind mixed k-quant files use:
# Q4_K for O and gate/up, Q5_K for QKV, Q6_K for down and the lm_head
SPEC_KQ = dataclasses.replace(SPEC_C2, name="kq_8layer_d2048_q4_k_q5_k_q6_k_lm32000", fmt="q4_k",
                              fmts=(("wqkv", "q5_k"), ("w_down", "q6_k"), ("lm_head", "q6_k")))


def c3_lengths(seed: int = 0, B: int = 16) -> List[int]:
    """Per-session KV lengths drawn log-uniform in [512, 32768] (floor, clamped)."""
    r = rng_for(seed, 3, T_LENGTHS)
    u = r.uniform(math.log(512.0), math.log(32768.0), size=B)
    return [int(min(32768, max(512, math.floor(math.exp(v))))) for v in u]


def workload(name: str, B: Optional[int] = None, seed: int = 0, steps: Optional[int] = None) -> Workload:
    """Build one of the five workloads ("c1".."c5"); ``B``/``steps`` override the defaults."""
    if name == "c1":
        assert B in (None, 2, 1)
        prefill = [17, 40]
        rows = [(0, 0), (1, 0)] if B in (None, 2) else [(0, 0)]
        return Workload(1, SPEC_C1, prefill[: len(rows)], rows, steps or 1, 64, seed)
    if name == "c2":
        B = B or 8
        return Workload(2, SPEC_C2, [1238] * B, [(b, 0) for b in range(B)], steps or 64,
                        1238 + 64, seed)
    if name == "c3":
        B = B or 16
        lens = c3_lengths(seed, 16)[:B]
        return Workload(3, SPEC_C3, lens, [(b, 0) for b in range(B)], steps or 1, 32768 + 1, seed)
    if name == "c4":
        B = B or 8
        return Workload(4, SPEC_C4, [4096] * B, [(b, 0) for b in range(B)], steps or 32,
                        4096 + 32, seed)
    if name == "kq":
        B = B or 8
        return Workload(7, SPEC_KQ, [1238] * B, [(b, 0) for b in range(B)], steps or 4, 1238 + 64, seed)
    if name == "hybrid":
        B = B or 4
        return Workload(6, SPEC_HYBRID, [1238] * B, [(b, 0) for b in range(B)], steps or 4, 1238 + 64, seed)
    if name == "c5":
        n_streams = (B or 16) // 4
        assert n_streams * 4 == (B or 16)
        rows = [(s, j) for s in range(n_streams) for j in range(4)]
        return Workload(5, SPEC_C5, [8192] * n_streams, rows, steps or 1, 8192 + 4, seed)
    raise ValueError(name)


# --------------------------------------------------------------------------------------
# Random draws
# --------------------------------------------------------------------------------------
def draw_q8_0(rq: np.random.Generator, rd: np.random.Generator, n: int, k: int) -> Dict:
    qs = rq.integers(-127, 128, size=(n, k), dtype=np.int8)
    d = (np.abs(rd.standard_normal((n, k // 32), dtype=np.float32)) * np.float32(0.02)
         / np.float32(127.0)).astype(np.float16)
    return {"fmt": "q8_0", "n": n, "k": k, "qs": qs, "d": d}


def draw_q4_0(rq: np.random.Generator, rd: np.random.Generator, n: int, k: int) -> Dict:
    qs = rq.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    d = (np.abs(rd.standard_normal((n, k // 32), dtype=np.float32)) * np.float32(0.02)
         / np.float32(8.0)).astype(np.float16)
    return {"fmt": "q4_0", "n": n, "k": k, "qs": qs, "d": d}


KQ_RECORD = {"q4_k": 144, "q5_k": 176, "q6_k": 210}   # bytes per 256-value super-block


def draw_kquant(fmt: str, rq: np.random.Generator, rd: np.random.Generator, n: int, k: int) -> Dict:
    """A K-quant matrix: every byte of each 256-value record uniformly random (codes, fifth
    or upper bits, packed 6-bit scales and mins, int8 scales), then its fp16 scale fields set
    to drawn values: Q4_K / Q5_K ``d = |N(0, 1)| 0.04 / (15 * 63)`` and
    ``dmin = |N(0, 1)| 0.02 / 63`` at bytes 0 and 2; Q6_K ``d = |N(0, 1)| 0.02 / (32 * 127)`` at
    byte 208 (weights of about the other formats' magnitude)."""
    BS, nsb = KQ_RECORD[fmt], k // 256
    rec = rq.integers(0, 256, size=(n, nsb, BS), dtype=np.uint8)
    if fmt == "q6_k":
        d = (np.abs(rd.standard_normal((n, nsb), dtype=np.float32)) * np.float32(0.02 / (32 * 127))).astype(np.float16)
        rec[:, :, 208:210] = d.view(np.uint8).reshape(n, nsb, 2)
    else:
        d = (np.abs(rd.standard_normal((n, nsb), dtype=np.float32)) * np.float32(0.04 / (15 * 63))).astype(np.float16)
        dm = (np.abs(rd.standard_normal((n, nsb), dtype=np.float32)) * np.float32(0.02 / 63)).astype(np.float16)
        rec[:, :, 0:2] = d.view(np.uint8).reshape(n, nsb, 2)
        rec[:, :, 2:4] = dm.view(np.uint8).reshape(n, nsb, 2)
    return {"fmt": fmt, "n": n, "k": k, "qs": rec.reshape(n, nsb * BS), "d": np.zeros((n, 0), dtype=np.float16)}


def draw_weight(fmt: str, seed: int, code: int, tq: int, td: int, layer: int, n: int, k: int) -> Dict:
    rq, rd = rng_for(seed, code, tq, layer), rng_for(seed, code, td, layer)
    if fmt in KQ_RECORD:
        return draw_kquant(fmt, rq, rd, n, k)
    return (draw_q8_0 if fmt == "q8_0" else draw_q4_0)(rq, rd, n, k)


def draw_gain(seed: int, code: int, tensor: int, layer: int, n: int) -> np.ndarray:
    r = rng_for(seed, code, tensor, layer)
    return (np.float32(1.0) + np.float32(0.1) * r.standard_normal(n, dtype=np.float32)).astype(np.float32)


def make_linear_layer(spec: ModelSpec, code: int, seed: int, il: int) -> Dict:
    """A gated delta-rule layer: its input projection (quantised, rows as ``ssm_in_rows``), the
    conv kernel fp32 [conv_dim, d_conv] ~ N(0, 0.5^2), dt bias fp32 [n_v] ~ N(0, 0.5^2), decay
    rate a = -exp(U(-1, 1)) fp32 [n_v], the output-norm gain 1 + 0.1 N(0, 1) [d_state] and the
    out projection [d, value_dim] (quantised)."""
    d, fmt, nv = spec.d, spec.fmt, spec.ssm_n_v
    r = lambda t: rng_for(seed, code, t, il)
    return {
        "mixer": "linear",
        "attn_norm": draw_gain(seed, code, T_ATTN_NORM, il, d),
        "wqkv": draw_weight(fmt, seed, code, T_SSM_IN_Q, T_SSM_IN_D, il, spec.ssm_in_rows, d),
        "wo": draw_weight(fmt, seed, code, T_SSM_OUT_Q, T_SSM_OUT_D, il, d, spec.ssm_value_dim),
        "ssm_conv": (np.float32(0.5) * r(T_SSM_CONV).standard_normal((spec.ssm_conv_dim, spec.ssm_d_conv),
                                                                      dtype=np.float32)).astype(np.float32),
        "ssm_dt": (np.float32(0.5) * r(T_SSM_DT).standard_normal(nv, dtype=np.float32)).astype(np.float32),
        "ssm_a": (-np.exp(r(T_SSM_A).uniform(-1.0, 1.0, nv))).astype(np.float32),
        "ssm_norm": draw_gain(seed, code, T_SSM_NORM, il, spec.ssm_d_state),
    }


def recurrent_prefill(wl: "Workload", session: int, layer: int) -> Tuple[np.ndarray, np.ndarray]:
    """A linear layer's recurrent state before step 0: the conv ring [d_conv - 1, conv_dim]
    ~ N(0, 1) (the last inputs of a prefix) and the state [n_v, d_state, d_state] ~ N(0, 0.05^2),
    fp32."""
    sp = wl.spec
    conv = rng_for(wl.seed, wl.code, T_REC_CONV, layer, session).standard_normal(
        (sp.ssm_d_conv - 1, sp.ssm_conv_dim), dtype=np.float32)
    S = (np.float32(0.05) * rng_for(wl.seed, wl.code, T_REC_S, layer, session).standard_normal(
        (sp.ssm_n_v, sp.ssm_d_state, sp.ssm_d_state), dtype=np.float32)).astype(np.float32)
    return conv, S


def make_layer(spec: ModelSpec, code: int, seed: int, il: int) -> Dict:
    d, fmt = spec.d, spec.fmt
    if il in spec.linear_layers:
        L = make_linear_layer(spec, code, seed, il)
        if spec.has_ffn:
            L["ffn_norm"] = draw_gain(seed, code, T_FFN_NORM, il, d)
        if spec.ffn:
            F = spec.ffn
            L["w_gate"] = draw_weight(fmt, seed, code, T_GATE_Q, T_GATE_D, il, F, d)
            L["w_up"] = draw_weight(fmt, seed, code, T_UP_Q, T_UP_D, il, F, d)
            L["w_down"] = draw_weight(fmt, seed, code, T_DOWN_Q, T_DOWN_D, il, d, F)
        return L
    L: Dict = {
        "swa_window": spec.swa_window if il in spec.swa_layers else 0,
        "attn_gate": bool(spec.attn_gate),
        "attn_norm": draw_gain(seed, code, T_ATTN_NORM, il, d),
        "wqkv": draw_weight(spec.fmt_of("wqkv"), seed, code, T_WQKV_Q, T_WQKV_D, il, spec.qkv_rows, d),
        "wo": draw_weight(spec.fmt_of("wo"), seed, code, T_WO_Q, T_WO_D, il, d, spec.n_head * spec.head_dim),
    }
    if spec.qk_norm:
        L["q_norm"] = draw_gain(seed, code, T_Q_NORM, il, spec.head_dim)
        L["k_norm"] = draw_gain(seed, code, T_K_NORM, il, spec.head_dim)
    if spec.has_ffn:
        L["ffn_norm"] = draw_gain(seed, code, T_FFN_NORM, il, d)
    if spec.ffn:
        F = spec.ffn
        L["w_gate"] = draw_weight(spec.fmt_of("w_gate"), seed, code, T_GATE_Q, T_GATE_D, il, F, d)
        L["w_up"] = draw_weight(spec.fmt_of("w_up"), seed, code, T_UP_Q, T_UP_D, il, F, d)
        L["w_down"] = draw_weight(spec.fmt_of("w_down"), seed, code, T_DOWN_Q, T_DOWN_D, il, d, F)
    if spec.n_experts:
        E, Fe, Fs = spec.n_experts, spec.expert_ffn, spec.shared_ffn
        r = rng_for(seed, code, T_ROUTER, il)
        L["router"] = (r.standard_normal((E, d), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
        # Experts stacked along the output rows: expert e = rows [e*Fe, (e+1)*Fe) of
        # e_gate/e_up and rows [e*d, (e+1)*d) of e_down.
        L["e_gate"] = draw_weight(fmt, seed, code, T_EGATE_Q, T_EGATE_D, il, E * Fe, d)
        L["e_up"] = draw_weight(fmt, seed, code, T_EUP_Q, T_EUP_D, il, E * Fe, d)
        L["e_down"] = draw_weight(fmt, seed, code, T_EDOWN_Q, T_EDOWN_D, il, E * d, Fe)
        L["s_gate"] = draw_weight(fmt, seed, code, T_SGATE_Q, T_SGATE_D, il, Fs, d)
        L["s_up"] = draw_weight(fmt, seed, code, T_SUP_Q, T_SUP_D, il, Fs, d)
        L["s_down"] = draw_weight(fmt, seed, code, T_SDOWN_Q, T_SDOWN_D, il, d, Fs)
    return L


def make_model(spec: ModelSpec, code: int, seed: int = 0, threads: int = 8) -> Dict:
    """All weights of a model: {"spec", "layers": [...], "final_norm", "lm_head"}.

    Layers are drawn on a thread pool; every tensor has its own seed key, so the arrays do
    not depend on the thread count or order."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max(1, threads)) as ex:
        layers = list(ex.map(lambda il: make_layer(spec, code, seed, il), range(spec.n_layers)))
    m: Dict = {"spec": spec, "layers": layers}
    m["final_norm"] = draw_gain(seed, code, T_FINAL_NORM, 0, spec.d) if spec.final_norm else None
    m["lm_head"] = (draw_weight(spec.fmt_of("lm_head"), seed, code, T_LM_Q, T_LM_D, 0, spec.vocab, spec.d)
                    if spec.vocab else None)
    return m


def step_inputs(wl: Workload, step: int) -> np.ndarray:
    """Fresh N(0,1) fp32 input rows ``[B, d]`` for one step (one stream per (step, row))."""
    d = wl.spec.d
    out = np.empty((wl.B, d), dtype=np.float32)
    for b, (s, j) in enumerate(wl.rows):
        out[b] = rng_for(wl.seed, wl.code, T_X_IN, step, 1000 * s + j).standard_normal(d, dtype=np.float32)
    return out


def embedding_table(wl: Workload) -> np.ndarray:
    """Token embedding rows ``[vocab, d]`` fp32, N(0, 1) like the step inputs (one stream per
    row), for decoding with the greedy token fed back as the next step's input."""
    sp = wl.spec
    out = np.empty((sp.vocab, sp.d), dtype=np.float32)
    for t in range(sp.vocab):
        out[t] = rng_for(wl.seed, wl.code, T_EMBED, 0, t).standard_normal(sp.d, dtype=np.float32)
    return out


def kv_prefill(wl: Workload, session: int, layer: int) -> Tuple[np.ndarray, np.ndarray]:
    """fp16 K and V ``[G, L, hd]`` already in the cache before step 0 (treated as post-RoPE)."""
    sp = wl.spec
    shape = (sp.n_head_kv, wl.prefill[session], sp.head_dim)
    rk = rng_for(wl.seed, wl.code, T_K_PRE, layer, session)
    rv = rng_for(wl.seed, wl.code, T_V_PRE, layer, session)
    if sp.kv_fp8:
        return fp8_codes(rk, shape), fp8_codes(rv, shape)
    if sp.kv_q8:
        return q8_rows(rk, shape), q8_rows(rv, shape)
    k = rk.standard_normal(shape, dtype=np.float32).astype(np.float16)
    v = rv.standard_normal(shape, dtype=np.float32).astype(np.float16)
    return k, v


def fp8_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Random E4M3 bytes drawn field by field: a random sign, an exponent field in 4 .. 8
    (magnitudes 2^-3 .. 2^2, about the spread of unit-variance cache values) and a random
    mantissa; never a NaN code.  No conversion: the bytes are the inputs."""
    sign = rng.integers(0, 2, size=shape, dtype=np.uint8) << 7
    expo = rng.integers(4, 9, size=shape, dtype=np.uint8) << 3
    mant = rng.integers(0, 8, size=shape, dtype=np.uint8)
    return (sign | expo | mant).astype(np.uint8)


def q8_rows(rng: np.random.Generator, shape) -> np.ndarray:
    """Random int8 cache rows ``[G, L, hd + 16]`` drawn field by field: int8 codes uniform in
    [-127, 127] and, per 32-element block, an fp16 scale 1.7 / 127 times U(0.5, 1.5) (values
    of about unit spread), then zero padding.  No conversion: the bytes are the inputs."""
    G, L, hd = shape
    codes = rng.integers(-127, 128, size=(G, L, hd), dtype=np.int8)
    d = (np.float32(1.7 / 127.0) * rng.uniform(0.5, 1.5, size=(G, L, hd // 32)).astype(np.float32)).astype(np.float16)
    out = np.zeros((G, L, hd + 16), dtype=np.uint8)
    out[:, :, :hd] = codes.view(np.uint8)
    out[:, :, hd:hd + 2 * (hd // 32)] = d.view(np.uint8).reshape(G, L, 2 * (hd // 32))
    return out


def kv_prefill_many(wl: Workload, pairs, threads: int = 8):
    """kv_prefill for many (session, layer) pairs on a thread pool; same arrays as one by one."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max(1, threads)) as ex:
        return list(ex.map(lambda p: kv_prefill(wl, p[0], p[1]), pairs))


def algorithmic_bytes_weights(spec: ModelSpec) -> int:
    """Bytes of every quantised matrix and fp32 router the step streams once (dense view)."""
    def mat(n, k, role=""):
        fmt = spec.fmt_of(role)
        if fmt in KQ_RECORD:
            return n * (k // 256) * KQ_RECORD[fmt]
        return n * (k // 32) * (34 if fmt == "q8_0" else 18)    # bytes per 32-element block

    tot = 0
    for _ in range(spec.n_layers):
        tot += mat(spec.qkv_rows, spec.d, "wqkv") + mat(spec.d, spec.n_head * spec.head_dim, "wo")
        if spec.ffn:
            tot += mat(spec.ffn, spec.d, "w_gate") + mat(spec.ffn, spec.d, "w_up") + mat(spec.d, spec.ffn, "w_down")
        if spec.n_experts:
            tot += spec.n_experts * spec.d * 4
            tot += 2 * mat(spec.shared_ffn, spec.d) + mat(spec.d, spec.shared_ffn)
    if spec.vocab:
        tot += mat(spec.vocab, spec.d, "lm_head")
    return tot

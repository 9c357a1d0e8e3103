"""Python binding of libkd.so — the batched multi-session decode step on MI355X.

Argument marshalling only: every step of the decode path runs in the HIP kernels behind
the C ABI declared in ``include/kd.h``.  PyTorch provides device memory and the current
stream.  There is no fallback: if the library is not built, importing the binding's
entry points raises.

The wrappers keep the C names (``kd_mmvq_q8_0`` ...) and take torch tensors.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkd.so")

KD_OK, KD_ERR_INVALID, KD_ERR_UNSUPPORTED, KD_ERR_CAPACITY, KD_ERR_WORKSPACE, KD_ERR_HIP = 0, -1, -2, -3, -4, -5
KD_FMT_Q8_0, KD_FMT_Q4_0, KD_FMT_F32, KD_FMT_Q4_K, KD_FMT_Q5_K, KD_FMT_Q6_K = 1, 2, 3, 4, 5, 6
FMT_CODE = {"q8_0": KD_FMT_Q8_0, "q4_0": KD_FMT_Q4_0, "q4_k": KD_FMT_Q4_K, "q5_k": KD_FMT_Q5_K, "q6_k": KD_FMT_Q6_K}
KQ_FORMATS = (KD_FMT_Q4_K, KD_FMT_Q5_K, KD_FMT_Q6_K)
KD_MAX_B = 16


class KdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


class KdWeight(C.Structure):
    _fields_ = [("fmt", C.c_int32), ("n_out", C.c_int32), ("k", C.c_int32), ("qs", C.c_void_p), ("d", C.c_void_p)]


class KdAct(C.Structure):
    _fields_ = [("qs", C.c_void_p), ("d", C.c_void_p)]


class KdLayerDesc(C.Structure):
    _fields_ = [("attn_norm", C.c_void_p), ("wqkv", KdWeight), ("wqkv_pair_rows", C.c_int32), ("wo", KdWeight),
                ("ffn_norm", C.c_void_p),
                ("w_gate", KdWeight), ("w_up", KdWeight), ("w_down", KdWeight), ("router", C.c_void_p),
                ("e_gate", KdWeight), ("e_up", KdWeight), ("e_down", KdWeight),
                ("s_gate", KdWeight), ("s_up", KdWeight), ("s_down", KdWeight), ("swa_window", C.c_int32),
                ("q_norm", C.c_void_p), ("k_norm", C.c_void_p), ("attn_gate", C.c_int32),
                ("mixer", C.c_int32), ("ssm_conv", C.c_void_p), ("ssm_dt", C.c_void_p), ("ssm_a", C.c_void_p),
                ("ssm_norm", C.c_void_p)]


class KdModelDesc(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d", C.c_int32), ("n_head", C.c_int32), ("n_head_kv", C.c_int32),
                ("head_dim", C.c_int32), ("ffn", C.c_int32), ("n_experts", C.c_int32), ("n_expert_used", C.c_int32),
                ("expert_ffn", C.c_int32), ("shared_ffn", C.c_int32), ("vocab", C.c_int32),
                ("rope_base", C.c_float), ("rms_eps", C.c_float), ("layers", C.POINTER(KdLayerDesc)),
                ("final_norm", C.c_void_p), ("lm_head", KdWeight), ("ssm_d_state", C.c_int32), ("ssm_n_k", C.c_int32),
                ("ssm_n_v", C.c_int32), ("ssm_d_conv", C.c_int32), ("kv_format", C.c_int32)]


KD_KV_F16, KD_KV_FP8_E4M3, KD_KV_Q8_0 = 0, 1, 2


class KdStepTrace(C.Structure):
    _fields_ = [("resid", C.c_void_p), ("moe_ids", C.c_void_p), ("moe_p", C.c_void_p), ("q_attn_in", C.c_void_p),
                ("q_attn_out", C.c_void_p), ("q_ffn_in", C.c_void_p), ("q_ffn_mid", C.c_void_p),
                ("q_shared_mid", C.c_void_p), ("q_head_in", C.c_void_p)]


_P, _I, _F, _S = C.c_void_p, C.c_int32, C.c_float, C.c_size_t
_PW = C.POINTER(KdWeight)
_PP = C.POINTER(C.c_void_p)
_PI = C.POINTER(C.c_int32)

# name -> (restype, argtypes); the ABI surface of include/kd.h
SIGNATURES = {
    "kd_version": (C.c_char_p, []),
    "kd_last_error": (C.c_char_p, []),
    "kd_weight_qs_bytes": (_S, [_I, _I, _I]),
    "kd_weight_d_bytes": (_S, [_I, _I, _I]),
    "kd_act_qs_bytes": (_S, [_I, _I]),
    "kd_act_d_bytes": (_S, [_I, _I]),
    "kd_pack_weight": (_I, [_I, _I, _I, _P, _P, _P, _P, _P]),
    "kd_quantize_act_q8": (_I, [_P, _I, _I, _I, KdAct, _P]),
    "kd_mmvq_q8_0": (_I, [_PW, KdAct, _I, _P, _I, _P]),
    "kd_mmvq_q4_0": (_I, [_PW, KdAct, _I, _P, _I, _P]),
    "kd_mmvq": (_I, [_PW, KdAct, _I, _P, _I, _P]),
    "kd_rmsnorm_rows": (_I, [_P, _P, _P, _I, _I, _F, _P]),
    "kd_add_rmsnorm_rows": (_I, [_P, _P, _P, _P, _P, _I, _I, _F, _P]),
    "kd_rope_neox_rows": (_I, [_P, _I, _I, _I, _PI, _F, _P]),
    "kd_swiglu_rows": (_I, [_P, _P, _P, _I, _I, _P]),
    "kd_add_rows": (_I, [_P, _P, _P, _I, _I, _P]),
    "kd_argmax_rows": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "kd_embed_rows": (_I, [_P, _I, _I, _P, _I, _P, _I, _P]),
    "kd_verify_accept": (_I, [_P, _P, _I, _I, _P, _P, _P]),
    "kd_kv_append": (_I, [_P, _P, _I, _I, _I, _PP, _PP, _PI, _I, _P]),
    "kd_kv_append_fp8": (_I, [_P, _P, _I, _I, _I, _PP, _PP, _PI, _I, _P]),
    "kd_kv_append_q8": (_I, [_P, _P, _I, _I, _I, _PP, _PP, _PI, _I, _P]),
    "kd_gdn_step": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _PP, _PP, _F, _P, _P]),
    "kd_fa_decode_workspace": (_S, [_I, _I, _I, _PI]),
    "kd_fa_decode_ragged": (_I, [_P, _I, _I, _I, _I, _PP, _PP, _PI, _I, _F, _P, _P, _S, _P]),
    "kd_fa_decode_ragged_noalloc": (_I, [_P, _I, _I, _I, _I, _PP, _PP, _PI, _I, _F, _P, _P]),
    "kd_fa_decode_ragged_fp8": (_I, [_P, _I, _I, _I, _I, _PP, _PP, _PI, _I, _F, _P, _P, _S, _P]),
    "kd_fa_decode_ragged_q8": (_I, [_P, _I, _I, _I, _I, _PP, _PP, _PI, _I, _F, _P, _P, _S, _P]),
    "kd_model_create": (_I, [C.POINTER(KdModelDesc), C.POINTER(_P)]),
    "kd_model_destroy": (None, [_P]),
    "kd_decode_step_workspace": (_S, [_P, _I, _PI]),
    "kd_recurrent_state_bytes": (_S, [_P]),
    "kd_decode_step": (_I, [_P, _I, _P, _PI, _PP, _PP, _I, _P, _P, _S, _P]),
    "kd_mmvq_swiglu": (_I, [_PW, KdAct, _I, KdAct, _P]),
    "kd_mmvq_rope": (_I, [_PW, KdAct, _I, _I, _I, _I, _P, _I, _PP, _PP, _PI, _I, _F, _P]),
    "kd_mmvq_resnorm": (_I, [_PW, KdAct, _I, _P, _P, _P, KdAct, _P, _P]),
    "kd_mmvq_swiglu_normed": (_I, [_PW, KdAct, _I, _P, _F, KdAct, _P]),
    "kd_mmvq_rope_normed": (_I, [_PW, KdAct, _I, _P, _F, _I, _I, _I, _P, _I, _PP, _PP, _PI, _I, _F, _P]),
    "kd_debug_block_dots": (_I, [_PW, KdAct, _I, _P, _P]),
    "kd_debug_fa_workspace": (_S, [_I, _I, _I, _PI, _I]),
    "kd_debug_fa_decode_chunked": (_I, [_P, _I, _I, _I, _I, _PP, _PP, _PI, _I, _F, _P, _I, _P, _S, _P]),
    "kd_debug_read_stream": (_I, [_P, _S, _P, _P]),
    "kd_debug_decode_step_trace": (_I, [_P, _I, _P, _PI, _PP, _PP, _I, _P, _P, _S, C.POINTER(KdStepTrace), _P]),
    "kd_debug_moe_route": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
    "kd_debug_mmvq_grouped": (_I, [_PW, _I, KdAct, _I, _P, _P, _P, _I, _P, _I, KdAct, _P]),
}

_lib: Optional[C.CDLL] = None


def lib() -> C.CDLL:
    """The loaded libkd.so (raises if it has not been built: there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m session_decode_step_amd.build`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int, name: str) -> None:
    if status != KD_OK:
        raise KdError(status, f"{name}: {lib().kd_last_error().decode()}")


def _stream(stream=None) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _i32(seq: Sequence[int]):
    arr = (C.c_int32 * len(seq))(*[int(v) for v in seq])
    return arr


def _ptrs(seq: Sequence[int]):
    return (C.c_void_p * len(seq))(*[int(v) for v in seq])


def kd_version() -> str:
    return lib().kd_version().decode()


# ------------------------------------------------------------------------------ weights
@dataclass
class PackedWeight:
    fmt: int
    n_out: int
    k: int
    qs: torch.Tensor
    d: Optional[torch.Tensor]

    def c(self) -> KdWeight:
        return KdWeight(self.fmt, self.n_out, self.k, self.qs.data_ptr(), self.d.data_ptr() if self.d is not None else None)

    @property
    def nbytes(self) -> int:
        return self.qs.numel() * self.qs.element_size() + (0 if self.d is None else self.d.numel() * 2)


def kd_pack_weight(w: Dict, device="cuda", stream=None) -> PackedWeight:
    """Upload a row-major block matrix (``{"fmt","n","k","qs","d"}`` numpy) and repack it on the GPU."""
    fmt, n, k = FMT_CODE[w["fmt"]], int(w["n"]), int(w["k"])
    src_qs = torch.from_numpy(np.ascontiguousarray(w["qs"]).view(np.uint8)).to(device)
    # K-quant records carry their own scales (no separate d)
    src_d = None if fmt in KQ_FORMATS else torch.from_numpy(np.ascontiguousarray(w["d"]).view(np.int16)).to(device)
    qs = torch.empty(lib().kd_weight_qs_bytes(fmt, n, k), dtype=torch.uint8, device=device)
    dd = torch.empty(lib().kd_weight_d_bytes(fmt, n, k) // 2, dtype=torch.int16, device=device)
    _check(lib().kd_pack_weight(fmt, n, k, src_qs.data_ptr(), None if src_d is None else src_d.data_ptr(),
                                qs.data_ptr(), dd.data_ptr(), _stream(stream)), "kd_pack_weight")
    torch.cuda.current_stream().synchronize()   # the sources are freed on return
    return PackedWeight(fmt, n, k, qs, dd)


def _take_rows(w: Dict, order: np.ndarray) -> Dict:
    return {"fmt": w["fmt"], "n": len(order), "k": w["k"], "qs": np.ascontiguousarray(w["qs"][order]),
            "d": np.ascontiguousarray(w["d"][order])}


def interleave_gate_up(gate: Dict, up: Dict) -> Dict:
    """gate and up [F, k] as one [2F, k] matrix in blocks of 32 rows (gate rows 32m..32m+31,
    then up rows 32m..32m+31): the layout of the stacked gate/up product in ``kd.h``."""
    assert gate["fmt"] == up["fmt"] and gate["k"] == up["k"] and gate["n"] == up["n"] and gate["n"] % 32 == 0
    F = gate["n"]
    both = {"fmt": gate["fmt"], "n": 2 * F, "k": gate["k"], "qs": np.concatenate([gate["qs"], up["qs"]]),
            "d": np.concatenate([gate["d"], up["d"]])}
    blk = np.arange(F // 32)[:, None]
    order = np.concatenate([blk * 32 + np.arange(32)[None, :], F + blk * 32 + np.arange(32)[None, :]], axis=1)
    return _take_rows(both, order.reshape(-1))


def interleave_experts(gate: Dict, up: Dict, n_experts: int) -> Dict:
    """Stacked expert gate and up [E*Fe, k] as [E*2Fe, k]: expert e's rows are its gate and up
    interleaved in blocks of 32 rows (``interleave_gate_up`` per expert)."""
    assert gate["fmt"] == up["fmt"] and gate["k"] == up["k"] and gate["n"] == up["n"]
    EF = gate["n"]
    Fe = EF // n_experts
    assert Fe * n_experts == EF and Fe % 32 == 0
    both = {"fmt": gate["fmt"], "n": 2 * EF, "k": gate["k"], "qs": np.concatenate([gate["qs"], up["qs"]]),
            "d": np.concatenate([gate["d"], up["d"]])}
    e = np.arange(n_experts)[:, None, None]
    blk = np.arange(Fe // 32)[None, :, None]
    i = np.arange(32)[None, None, :]
    order = np.concatenate([e * Fe + blk * 32 + i, EF + e * Fe + blk * 32 + i], axis=2)   # [E][blocks][64]
    return _take_rows(both, order.reshape(-1))


def rope_pair_rows(wqkv: Dict, n_heads: int, hd: int) -> Dict:
    """wqkv with each head's rows in RoPE pair order: packed row 2i = row i, 2i+1 = row i + hd/2."""
    half = hd // 2
    within = np.stack([np.arange(half), np.arange(half) + half], axis=1).reshape(-1)
    order = (np.arange(n_heads)[:, None] * hd + within[None, :]).reshape(-1)
    assert wqkv["n"] == n_heads * hd
    return _take_rows(wqkv, order)


def expert_view(w: PackedWeight, n_out: int) -> PackedWeight:
    return PackedWeight(w.fmt, n_out, w.k, w.qs, w.d)


# ------------------------------------------------------------------------------ activations
@dataclass
class Act:
    qs: torch.Tensor
    d: torch.Tensor
    B: int
    k: int

    def c(self) -> KdAct:
        return KdAct(self.qs.data_ptr(), self.d.data_ptr())


def alloc_act(B: int, k: int, device="cuda") -> Act:
    qs = torch.empty(lib().kd_act_qs_bytes(B, k), dtype=torch.int8, device=device)
    d = torch.empty(lib().kd_act_d_bytes(B, k) // 4, dtype=torch.float32, device=device)
    return Act(qs, d, B, k)


def kd_quantize_act_q8(x: torch.Tensor, out: Optional[Act] = None, stream=None) -> Act:
    B, k = x.shape
    out = out or alloc_act(B, k, x.device)
    _check(lib().kd_quantize_act_q8(x.data_ptr(), B, k, x.stride(0), out.c(), _stream(stream)), "kd_quantize_act_q8")
    return out


def _mmvq(name: str, W: PackedWeight, x: Act, B: int, y: Optional[torch.Tensor], stream) -> torch.Tensor:
    if y is None:
        y = torch.empty((B, W.n_out), dtype=torch.float32, device=x.qs.device)
    wc = W.c()
    _check(getattr(lib(), name)(C.byref(wc), x.c(), B, y.data_ptr(), y.stride(0), _stream(stream)), name)
    return y


def kd_mmvq_q8_0(W: PackedWeight, x: Act, B: int, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    return _mmvq("kd_mmvq_q8_0", W, x, B, y, stream)


def kd_mmvq_q4_0(W: PackedWeight, x: Act, B: int, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    return _mmvq("kd_mmvq_q4_0", W, x, B, y, stream)


def kd_mmvq(W: PackedWeight, x: Act, B: int, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The product for any quantised format (Q8_0, Q4_0, Q4_K, Q5_K, Q6_K)."""
    return _mmvq("kd_mmvq", W, x, B, y, stream)


def kd_mmvq_swiglu(W: PackedWeight, x: Act, B: int, out: Optional[Act] = None, stream=None) -> Act:
    """Interleaved gate/up product with SwiGLU and the quantiser in its epilogue."""
    F = W.n_out // 2
    out = out or alloc_act(B, F, x.qs.device)
    wc = W.c()
    _check(lib().kd_mmvq_swiglu(C.byref(wc), x.c(), B, out.c(), _stream(stream)), "kd_mmvq_swiglu")
    return out


def kd_mmvq_rope(W: PackedWeight, x: Act, B: int, H: int, G: int, hd: int, q_out: torch.Tensor, k_base, v_base,
                 pos: Sequence[int], capacity: int, rope_base: float, stream=None) -> torch.Tensor:
    """Pair-ordered wqkv product with RoPE and the fp16 KV append in its epilogue."""
    wc = W.c()
    _check(lib().kd_mmvq_rope(C.byref(wc), x.c(), B, H, G, hd, q_out.data_ptr(), q_out.stride(0), _ptrs(k_base),
                              _ptrs(v_base), _i32(pos), capacity, rope_base, _stream(stream)), "kd_mmvq_rope")
    return q_out


def kd_mmvq_resnorm(W: PackedWeight, x: Act, B: int, res: torch.Tensor, gain: torch.Tensor,
                    x1: Optional[torch.Tensor] = None, out: Optional[Act] = None, ss: Optional[torch.Tensor] = None,
                    stream=None):
    """x1 = res + W x, the block codes of x1 * gain and the block sums of x1^2 (the producing
    half of a split RMSNorm): returns (x1, out, ss)."""
    n = W.n_out
    dev = x.qs.device
    x1 = torch.empty((B, n), dtype=torch.float32, device=dev) if x1 is None else x1
    out = alloc_act(B, n, dev) if out is None else out
    ss = torch.empty((B, n // 32), dtype=torch.float32, device=dev) if ss is None else ss
    wc = W.c()
    _check(lib().kd_mmvq_resnorm(C.byref(wc), x.c(), B, res.data_ptr(), gain.data_ptr(), x1.data_ptr(), out.c(),
                                 ss.data_ptr(), _stream(stream)), "kd_mmvq_resnorm")
    return x1, out, ss


def kd_mmvq_swiglu_normed(W: PackedWeight, x: Act, B: int, norm_ss: torch.Tensor, eps: float,
                          out: Optional[Act] = None, stream=None) -> Act:
    """kd_mmvq_swiglu on a split-RMSNorm input (x and norm_ss from kd_mmvq_resnorm)."""
    out = out or alloc_act(B, W.n_out // 2, x.qs.device)
    wc = W.c()
    _check(lib().kd_mmvq_swiglu_normed(C.byref(wc), x.c(), B, norm_ss.data_ptr(), eps, out.c(), _stream(stream)),
           "kd_mmvq_swiglu_normed")
    return out


def kd_mmvq_rope_normed(W: PackedWeight, x: Act, B: int, norm_ss: torch.Tensor, eps: float, H: int, G: int, hd: int,
                        q_out: torch.Tensor, k_base, v_base, pos: Sequence[int], capacity: int, rope_base: float,
                        stream=None) -> torch.Tensor:
    """kd_mmvq_rope on a split-RMSNorm input (x and norm_ss from kd_mmvq_resnorm)."""
    wc = W.c()
    _check(lib().kd_mmvq_rope_normed(C.byref(wc), x.c(), B, norm_ss.data_ptr(), eps, H, G, hd, q_out.data_ptr(),
                                     q_out.stride(0), _ptrs(k_base), _ptrs(v_base), _i32(pos), capacity, rope_base,
                                     _stream(stream)), "kd_mmvq_rope_normed")
    return q_out


def kd_debug_block_dots(W: PackedWeight, x: Act, B: int, stream=None) -> torch.Tensor:
    S = torch.empty((B, W.n_out, W.k // 32), dtype=torch.int32, device=x.qs.device)
    wc = W.c()
    _check(lib().kd_debug_block_dots(C.byref(wc), x.c(), B, S.data_ptr(), _stream(stream)), "kd_debug_block_dots")
    return S


def kd_debug_moe_route(z: torch.Tensor, router: torch.Tensor, K: int, stream=None) -> Dict[str, torch.Tensor]:
    """Routing of rows z [B, d] by router [E, d] (fp32 device tensors): ids, p, logits and the
    expert buckets (count [E], rows / pairs [E, 16]) as the MoE layer computes them."""
    B, d = z.shape
    E = router.shape[0]
    dev = z.device
    out = {"ids": torch.empty((B, K), dtype=torch.int32, device=dev), "p": torch.empty((B, K), device=dev),
           "logits": torch.empty((B, E), device=dev), "count": torch.empty(E, dtype=torch.int32, device=dev),
           "rows": torch.full((E, 16), -1, dtype=torch.int32, device=dev),
           "pairs": torch.full((E, 16), -1, dtype=torch.int32, device=dev)}
    _check(lib().kd_debug_moe_route(z.data_ptr(), router.data_ptr(), B, d, E, K, out["ids"].data_ptr(),
                                    out["p"].data_ptr(), out["logits"].data_ptr(), out["count"].data_ptr(),
                                    out["rows"].data_ptr(), out["pairs"].data_ptr(), _stream(stream)),
           "kd_debug_moe_route")
    return out


def kd_debug_mmvq_grouped(W: PackedWeight, n_groups: int, x: Act, act_rows: int, count: torch.Tensor,
                          act_row: torch.Tensor, out_row: torch.Tensor, out_rows: int, swiglu: bool = False,
                          stream=None):
    """Grouped product over row buckets: W is group 0 of n_groups stacked groups of W.n_out
    rows.  Returns fp32 rows [out_rows, W.n_out] (plain) or the quantised SwiGLU rows
    (an Act of out_rows rows of F = W.n_out / 2)."""
    wc = W.c()
    dev = x.qs.device
    if swiglu:
        out = alloc_act(out_rows, W.n_out // 2, dev)
        y, ldy, oc = None, 0, out.c()
    else:
        out = torch.zeros((out_rows, W.n_out), dtype=torch.float32, device=dev)
        y, ldy, oc = out.data_ptr(), W.n_out, KdAct(None, None)
    _check(lib().kd_debug_mmvq_grouped(C.byref(wc), n_groups, x.c(), act_rows, count.data_ptr(), act_row.data_ptr(),
                                       out_row.data_ptr(), 1 if swiglu else 0, y, ldy, oc, _stream(stream)),
           "kd_debug_mmvq_grouped")
    return out


def weight_group(W: PackedWeight, group: int, rows: int) -> PackedWeight:
    """Rows [group * rows, (group + 1) * rows) of a packed matrix as a matrix of its own (rows
    a multiple of 16: the group's tiles are one contiguous range)."""
    assert rows % 16 == 0
    tiles = (rows // 16) * ((W.k + 127) // 128)
    all_tiles = W.n_out // 16 * ((W.k + 127) // 128)
    per_qs = W.qs.numel() * W.qs.element_size() // all_tiles
    per_d = W.d.numel() // all_tiles                        # int16 entries per tile
    qs = W.qs.view(torch.uint8)[group * tiles * per_qs:(group + 1) * tiles * per_qs]
    d = W.d[group * tiles * per_d:(group + 1) * tiles * per_d]
    return PackedWeight(W.fmt, rows, W.k, qs, d)


def act_rows_view(x: Act, r0: int, n: int) -> Act:
    """Rows [r0, r0 + n) of a quantised activation buffer (the layout is row-contiguous)."""
    NQ = (x.k + 127) // 128
    return Act(x.qs[r0 * NQ * 128:(r0 + n) * NQ * 128], x.d[r0 * NQ * 4:(r0 + n) * NQ * 4], n, x.k)


def kd_debug_read_stream(t: torch.Tensor, sink: torch.Tensor, nbytes: Optional[int] = None, stream=None) -> None:
    """A plain read of the tensor's bytes (the first nbytes of them): the HBM read ceiling."""
    size = t.numel() * t.element_size()
    n = size if nbytes is None else nbytes
    if not t.is_contiguous() or n < 0 or n > size:
        raise ValueError(f"kd_debug_read_stream: {n} bytes from a tensor of {size} bytes (contiguous: "
                         f"{t.is_contiguous()})")
    _check(lib().kd_debug_read_stream(t.data_ptr(), n, sink.data_ptr(), _stream(stream)), "kd_debug_read_stream")


# ------------------------------------------------------------------------------ row ops
def kd_rmsnorm_rows(x: torch.Tensor, g: torch.Tensor, eps: float, stream=None) -> torch.Tensor:
    y = torch.empty_like(x)
    _check(lib().kd_rmsnorm_rows(x.data_ptr(), g.data_ptr(), y.data_ptr(), x.shape[0], x.shape[1], eps,
                                 _stream(stream)), "kd_rmsnorm_rows")
    return y


def kd_add_rmsnorm_rows(x: torch.Tensor, r: torch.Tensor, g: torch.Tensor, eps: float, stream=None):
    x1, y = torch.empty_like(x), torch.empty_like(x)
    _check(lib().kd_add_rmsnorm_rows(x.data_ptr(), r.data_ptr(), g.data_ptr(), x1.data_ptr(), y.data_ptr(),
                                     x.shape[0], x.shape[1], eps, _stream(stream)), "kd_add_rmsnorm_rows")
    return x1, y


def kd_rope_neox_rows(x: torch.Tensor, pos: Sequence[int], base: float, stream=None) -> torch.Tensor:
    B, nh, hd = x.shape
    _check(lib().kd_rope_neox_rows(x.data_ptr(), B, nh, hd, _i32(pos), base, _stream(stream)), "kd_rope_neox_rows")
    return x


def kd_swiglu_rows(g: torch.Tensor, u: torch.Tensor, stream=None) -> torch.Tensor:
    a = torch.empty_like(g)
    _check(lib().kd_swiglu_rows(g.data_ptr(), u.data_ptr(), a.data_ptr(), g.shape[0], g.shape[1], _stream(stream)),
           "kd_swiglu_rows")
    return a


def kd_add_rows(x: torch.Tensor, y: torch.Tensor, stream=None) -> torch.Tensor:
    z = torch.empty_like(x)
    _check(lib().kd_add_rows(x.data_ptr(), y.data_ptr(), z.data_ptr(), x.shape[0], x.shape[1], _stream(stream)),
           "kd_add_rows")
    return z


# ------------------------------------------------------------------------------ next token
def kd_argmax_rows(x: torch.Tensor, n: Optional[int] = None, stream=None):
    """Greedy token of each row of x [B, ldx] over its first n entries: (idx int32 [B],
    val fp32 [B]) on x's device."""
    B, ldx = x.shape
    n = ldx if n is None else n
    idx = torch.empty(B, dtype=torch.int32, device=x.device)
    val = torch.empty(B, dtype=torch.float32, device=x.device)
    _check(lib().kd_argmax_rows(x.data_ptr(), B, n, ldx, idx.data_ptr(), val.data_ptr(), _stream(stream)),
           "kd_argmax_rows")
    return idx, val


def kd_embed_rows(table: torch.Tensor, tokens: torch.Tensor, out: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Rows table[tokens[b]] of the fp32 embedding table [vocab, d] (tokens: device int32 [B])."""
    vocab, d = table.shape
    B = tokens.shape[0]
    out = torch.empty((B, d), dtype=torch.float32, device=table.device) if out is None else out
    _check(lib().kd_embed_rows(table.data_ptr(), vocab, d, tokens.data_ptr(), B, out.data_ptr(), out.stride(0),
                               _stream(stream)), "kd_embed_rows")
    return out


def kd_verify_accept(greedy: torch.Tensor, fed: torch.Tensor, k: int, stream=None):
    """Accepted draft count and next token per stream of stream-major verify rows (device int32
    [n_streams * k] each): (n_accept, next_token), device int32 [n_streams]."""
    n = greedy.shape[0] // k
    n_accept = torch.empty(n, dtype=torch.int32, device=greedy.device)
    nxt = torch.empty(n, dtype=torch.int32, device=greedy.device)
    _check(lib().kd_verify_accept(greedy.data_ptr(), fed.data_ptr(), n, k, n_accept.data_ptr(), nxt.data_ptr(),
                                  _stream(stream)), "kd_verify_accept")
    return n_accept, nxt


# ------------------------------------------------------------------------------ KV + attention
def kd_kv_append(k: torch.Tensor, v: torch.Tensor, k_base: Sequence[int], v_base: Sequence[int], pos: Sequence[int],
                 capacity: int, stream=None) -> None:
    B, G, hd = k.shape
    _check(lib().kd_kv_append(k.data_ptr(), v.data_ptr(), B, G, hd, _ptrs(k_base), _ptrs(v_base), _i32(pos), capacity,
                              _stream(stream)), "kd_kv_append")


def kd_kv_append_fp8(k: torch.Tensor, v: torch.Tensor, k_base: Sequence[int], v_base: Sequence[int],
                     pos: Sequence[int], capacity: int, stream=None) -> None:
    B, G, hd = k.shape
    _check(lib().kd_kv_append_fp8(k.data_ptr(), v.data_ptr(), B, G, hd, _ptrs(k_base), _ptrs(v_base), _i32(pos),
                                  capacity, _stream(stream)), "kd_kv_append_fp8")


def kd_kv_append_q8(k: torch.Tensor, v: torch.Tensor, k_base: Sequence[int], v_base: Sequence[int],
                    pos: Sequence[int], capacity: int, stream=None) -> None:
    B, G, hd = k.shape
    _check(lib().kd_kv_append_q8(k.data_ptr(), v.data_ptr(), B, G, hd, _ptrs(k_base), _ptrs(v_base), _i32(pos),
                                 capacity, _stream(stream)), "kd_kv_append_q8")


def kd_fa_decode_ragged_q8(q: torch.Tensor, G: int, k_base, v_base, t_kv, capacity: int, scale: float,
                           ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    B, H, hd = q.shape
    out = torch.empty_like(q) if out is None else out
    if ws is None:
        ws = torch.empty(max(kd_fa_decode_workspace(B, H, hd, t_kv), 16), dtype=torch.uint8, device=q.device)
    _check(lib().kd_fa_decode_ragged_q8(q.data_ptr(), B, H, G, hd, _ptrs(k_base), _ptrs(v_base), _i32(t_kv),
                                        capacity, scale, out.data_ptr(), ws.data_ptr(), ws.numel(),
                                        _stream(stream)), "kd_fa_decode_ragged_q8")
    return out


def kd_gdn_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                state_in: Sequence[int], state_out: Sequence[int], scale: float,
                o: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    B, H, d = q.shape
    o = torch.empty_like(v) if o is None else o
    _check(lib().kd_gdn_step(q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(), beta.data_ptr(), B, H, d,
                             _ptrs(state_in), _ptrs(state_out), scale, o.data_ptr(), _stream(stream)),
           "kd_gdn_step")
    return o


def kd_fa_decode_workspace(B: int, H: int, hd: int, t_kv: Sequence[int]) -> int:
    return lib().kd_fa_decode_workspace(B, H, hd, _i32(t_kv))


def kd_fa_decode_ragged_fp8(q: torch.Tensor, G: int, k_base, v_base, t_kv, capacity: int, scale: float,
                            ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    B, H, hd = q.shape
    out = torch.empty_like(q) if out is None else out
    if ws is None:
        ws = torch.empty(max(kd_fa_decode_workspace(B, H, hd, t_kv), 16), dtype=torch.uint8, device=q.device)
    _check(lib().kd_fa_decode_ragged_fp8(q.data_ptr(), B, H, G, hd, _ptrs(k_base), _ptrs(v_base), _i32(t_kv),
                                         capacity, scale, out.data_ptr(), ws.data_ptr(), ws.numel(),
                                         _stream(stream)), "kd_fa_decode_ragged_fp8")
    return out


def kd_fa_decode_ragged_noalloc(q: torch.Tensor, G: int, k_base, v_base, t_kv, capacity: int, scale: float,
                                out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kd_fa_decode_ragged with the split partials in the library's per-GPU scratch array."""
    B, H, hd = q.shape
    out = torch.empty_like(q) if out is None else out
    _check(lib().kd_fa_decode_ragged_noalloc(q.data_ptr(), B, H, G, hd, _ptrs(k_base), _ptrs(v_base), _i32(t_kv),
                                             capacity, scale, out.data_ptr(), _stream(stream)),
           "kd_fa_decode_ragged_noalloc")
    return out


def kd_fa_decode_ragged(q: torch.Tensor, G: int, k_base, v_base, t_kv, capacity: int, scale: float,
                        ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None, chunk: int = 0,
                        stream=None) -> torch.Tensor:
    B, H, hd = q.shape
    out = torch.empty_like(q) if out is None else out
    if chunk:
        need = lib().kd_debug_fa_workspace(B, H, hd, _i32(t_kv), chunk)
    else:
        need = kd_fa_decode_workspace(B, H, hd, t_kv)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if chunk:
        st = lib().kd_debug_fa_decode_chunked(q.data_ptr(), B, H, G, hd, _ptrs(k_base), _ptrs(v_base), _i32(t_kv),
                                              capacity, scale, out.data_ptr(), chunk, ws.data_ptr(), ws.numel(),
                                              _stream(stream))
        _check(st, "kd_debug_fa_decode_chunked")
    else:
        st = lib().kd_fa_decode_ragged(q.data_ptr(), B, H, G, hd, _ptrs(k_base), _ptrs(v_base), _i32(t_kv), capacity,
                                       scale, out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream))
        _check(st, "kd_fa_decode_ragged")
    return out


# ------------------------------------------------------------------------------ model + step
class KdModel:
    """Packs a model's weights (row-major block arrays, numpy) into device tiles and creates
    the kd_model.  The tensors it holds back the borrowed device pointers."""

    def __init__(self, model: Dict, device="cuda", fused: bool = True):
        """``fused``: pack wqkv in RoPE pair order and gate/up interleaved, so the step runs
        the RoPE/append and SwiGLU/quantise work in the products' epilogues; False keeps the
        canonical layouts (separate launches; the same results bit for bit)."""
        sp = model["spec"]
        self.spec = sp
        self.keep: List[torch.Tensor] = []
        self.layers = (KdLayerDesc * sp.n_layers)()
        self.weight_bytes = 0
        self.packed: List[Dict[str, PackedWeight]] = [dict() for _ in range(sp.n_layers + 1)]
        empty = KdWeight(0, 0, 0, None, None)
        slot = [0]

        def W(w, name=None):
            pw = kd_pack_weight(w, device)
            self.keep += [pw.qs, pw.d]
            self.weight_bytes += pw.nbytes
            if name:
                self.packed[slot[0]][name] = pw
            return pw.c()

        def F(a):
            t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
            self.keep.append(t)
            return t.data_ptr()

        kv_fp8 = bool(getattr(sp, "kv_fp8", False))   # E4M3 caches (kd_model_desc.kv_format)
        kv_q8 = bool(getattr(sp, "kv_q8", False))     # int8 rows: the canonical wqkv layout
        for il, L in enumerate(model["layers"]):
            slot[0] = il
            D = self.layers[il]
            D.attn_norm = F(L["attn_norm"])
            if L.get("mixer") == "linear":   # gated delta-rule layer: input and out projections, fp32 params
                D.mixer = 1
                D.wqkv, D.wqkv_pair_rows, D.wo = W(L["wqkv"], "wqkv"), 0, W(L["wo"], "wo")
                D.ssm_conv, D.ssm_dt, D.ssm_a, D.ssm_norm = (F(L["ssm_conv"]), F(L["ssm_dt"]), F(L["ssm_a"]),
                                                             F(L["ssm_norm"]))
                D.ffn_norm = F(L["ffn_norm"]) if "ffn_norm" in L else None
                if "w_gate" in L and fused:
                    D.w_gate, D.w_up, D.w_down = (W(interleave_gate_up(L["w_gate"], L["w_up"]), "w_gateup"), empty,
                                                  W(L["w_down"], "w_down"))
                elif "w_gate" in L:
                    D.w_gate, D.w_up, D.w_down = W(L["w_gate"], "w_gate"), W(L["w_up"], "w_up"), W(L["w_down"], "w_down")
                else:
                    D.w_gate = D.w_up = D.w_down = empty
                D.router = None
                D.e_gate = D.e_up = D.e_down = D.s_gate = D.s_up = D.s_down = empty
                continue
            D.swa_window = int(L.get("swa_window", 0))
            qk_norm = "q_norm" in L
            D.q_norm = F(L["q_norm"]) if qk_norm else None
            D.k_norm = F(L["k_norm"]) if qk_norm else None
            D.attn_gate = 1 if L.get("attn_gate") else 0
            n_heads_qkv = sp.n_head + 2 * sp.n_head_kv + (sp.n_head if D.attn_gate else 0)
            if fused and not qk_norm and not kv_q8:   # QK-norm and int8 caches need whole heads: canonical
                D.wqkv = W(rope_pair_rows(L["wqkv"], n_heads_qkv, sp.head_dim), "wqkv")
                D.wqkv_pair_rows = 1
            else:
                D.wqkv = W(L["wqkv"], "wqkv")
                D.wqkv_pair_rows = 0
            D.wo = W(L["wo"], "wo")
            D.ffn_norm = F(L["ffn_norm"]) if "ffn_norm" in L else None
            if "w_gate" in L and fused:   # gate and up interleaved: one product streams both
                D.w_gate, D.w_up, D.w_down = (W(interleave_gate_up(L["w_gate"], L["w_up"]), "w_gateup"), empty,
                                              W(L["w_down"], "w_down"))
            elif "w_gate" in L:
                D.w_gate, D.w_up, D.w_down = W(L["w_gate"], "w_gate"), W(L["w_up"], "w_up"), W(L["w_down"], "w_down")
            else:
                D.w_gate, D.w_up, D.w_down = empty, empty, empty
            if "router" in L:
                D.router = F(L["router"])
                if fused:   # each expert's (and the shared expert's) gate/up interleaved: one product each
                    D.e_gate, D.e_up = W(interleave_experts(L["e_gate"], L["e_up"], sp.n_experts)), empty
                    D.s_gate, D.s_up = W(interleave_gate_up(L["s_gate"], L["s_up"])), empty
                else:
                    D.e_gate, D.e_up = W(L["e_gate"]), W(L["e_up"])
                    D.s_gate, D.s_up = W(L["s_gate"]), W(L["s_up"])
                D.e_down, D.s_down = W(L["e_down"]), W(L["s_down"])
            else:
                D.router = None
                D.e_gate = D.e_up = D.e_down = D.s_gate = D.s_up = D.s_down = empty
        self.desc = KdModelDesc(sp.n_layers, sp.d, sp.n_head, sp.n_head_kv, sp.head_dim, sp.ffn, sp.n_experts,
                                sp.n_expert_used, sp.expert_ffn, sp.shared_ffn, sp.vocab, sp.rope_base, sp.rms_eps,
                                self.layers, F(model["final_norm"]) if model["final_norm"] is not None else None,
                                empty, getattr(sp, "ssm_d_state", 0), getattr(sp, "ssm_n_k", 0),
                                getattr(sp, "ssm_n_v", 0), getattr(sp, "ssm_d_conv", 0),
                                KD_KV_FP8_E4M3 if kv_fp8 else KD_KV_Q8_0 if kv_q8 else KD_KV_F16)
        slot[0] = sp.n_layers   # packed[n_layers] holds the output head
        if model["lm_head"] is not None:
            self.desc.lm_head = W(model["lm_head"], "lm_head")
        h = C.c_void_p()
        _check(lib().kd_model_create(C.byref(self.desc), C.byref(h)), "kd_model_create")
        self.handle = h

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                lib().kd_model_destroy(self.handle)
                self.handle = None
        except Exception:
            pass

    def workspace_bytes(self, B: int, pos: Sequence[int]) -> int:
        return lib().kd_decode_step_workspace(self.handle, B, _i32(pos))

    def recurrent_state_bytes(self) -> int:
        return lib().kd_recurrent_state_bytes(self.handle)

    def kd_decode_step(self, x_in: torch.Tensor, pos: Sequence[int], k_base: Sequence[int], v_base: Sequence[int],
                       capacity: int, out: torch.Tensor, ws: torch.Tensor, stream=None) -> torch.Tensor:
        B = x_in.shape[0]
        st = lib().kd_decode_step(self.handle, B, x_in.data_ptr(), _i32(pos), _ptrs(k_base), _ptrs(v_base), capacity,
                                  out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream))
        _check(st, "kd_decode_step")
        return out

    def kd_debug_decode_step_trace(self, x_in: torch.Tensor, pos: Sequence[int], k_base: Sequence[int],
                                   v_base: Sequence[int], capacity: int, out: torch.Tensor, ws: torch.Tensor,
                                   stream=None) -> Dict[str, torch.Tensor]:
        """kd_decode_step that also returns the residual rows entering every layer and after
        the last ([n_layers + 1, B, d]), for MoE layers each row's experts and weights, and the
        int8 codes of every activation quantisation (tiled layout, rows of NQ(k) * 128 bytes)."""
        sp = self.spec
        B = x_in.shape[0]
        dev = x_in.device
        nq = lambda k: (k + 127) // 128 * 128
        Lyr = sp.n_layers
        rec = {"resid": torch.empty((Lyr + 1, B, sp.d), dtype=torch.float32, device=dev),
               "q_attn_in": torch.zeros((Lyr, B, nq(sp.d)), dtype=torch.int8, device=dev),
               "q_attn_out": torch.zeros((Lyr, B, nq(max(sp.n_head * sp.head_dim, sp.ssm_value_dim))),
                                         dtype=torch.int8, device=dev)}
        if sp.ffn or sp.n_experts:
            rec["q_ffn_in"] = torch.zeros((Lyr, B, nq(sp.d)), dtype=torch.int8, device=dev)
        if sp.ffn:
            rec["q_ffn_mid"] = torch.zeros((Lyr, B, nq(sp.ffn)), dtype=torch.int8, device=dev)
        if sp.n_experts:
            K = sp.n_expert_used
            rec["q_ffn_mid"] = torch.zeros((Lyr, B * K, nq(sp.expert_ffn)), dtype=torch.int8, device=dev)
            rec["q_shared_mid"] = torch.zeros((Lyr, B, nq(sp.shared_ffn)), dtype=torch.int8, device=dev)
        if sp.vocab:
            rec["q_head_in"] = torch.zeros((B, nq(sp.d)), dtype=torch.int8, device=dev)
        tr = KdStepTrace(*[rec[k].data_ptr() if k in rec else None for k, _ in KdStepTrace._fields_])
        if sp.n_experts:
            rec["moe_ids"] = torch.full((Lyr, B, sp.n_expert_used), -1, dtype=torch.int32, device=dev)
            rec["moe_p"] = torch.zeros((Lyr, B, sp.n_expert_used), dtype=torch.float32, device=dev)
            tr.moe_ids, tr.moe_p = rec["moe_ids"].data_ptr(), rec["moe_p"].data_ptr()
        st = lib().kd_debug_decode_step_trace(self.handle, B, x_in.data_ptr(), _i32(pos), _ptrs(k_base),
                                              _ptrs(v_base), capacity, out.data_ptr(), ws.data_ptr(), ws.numel(),
                                              C.byref(tr), _stream(stream))
        _check(st, "kd_debug_decode_step_trace")
        rec["out"] = out
        return rec


class SessionCaches:
    """K/V caches of several sessions: one tensor [n_layers, 2, G, capacity, hd] per session,
    fp16, or uint8 E4M3 codes with ``fp8=True``, or uint8 int8 rows [..., hd + 16] with
    ``q8=True``."""

    def __init__(self, n_sessions: int, n_layers: int, G: int, capacity: int, hd: int, device="cuda",
                 fp8: bool = False, q8: bool = False, linear_layers: Sequence[int] = (), rec_bytes: int = 0):
        """``linear_layers``: layers holding a recurrent state of ``rec_bytes`` per session
        instead of K/V (``rec[s][il]``, fp32; kd_recurrent_state_bytes)."""
        self.n_layers, self.G, self.capacity, self.hd = n_layers, G, capacity, hd
        dt = torch.uint8 if (fp8 or q8) else torch.float16
        row = hd + 16 if q8 else hd
        self.t = [torch.zeros((n_layers, 2, G, capacity, row), dtype=dt, device=device)
                  for _ in range(n_sessions)]
        self.linear = set(linear_layers)
        self.rec = [{il: torch.zeros(rec_bytes // 4, dtype=torch.float32, device=device) for il in sorted(self.linear)}
                    for _ in range(n_sessions)]

    def k_ptr(self, s: int, il: int) -> int:
        if il in self.linear:
            return self.rec[s][il].data_ptr()
        return self.t[s][il, 0].data_ptr()

    def v_ptr(self, s: int, il: int) -> int:
        if il in self.linear:
            return self.rec[s][il].data_ptr()
        return self.t[s][il, 1].data_ptr()

    def tables(self, sessions: Sequence[int]):
        """Host tables [n_layers][B] of K and V base addresses for rows reading these sessions."""
        kb = [self.k_ptr(s, il) for il in range(self.n_layers) for s in sessions]
        vb = [self.v_ptr(s, il) for il in range(self.n_layers) for s in sessions]
        return kb, vb

    def recurrent_views(self, s: int, il: int, ring: int, state: int, d_conv: int, C: int):
        """(ring[2] [d_conv - 1, C], state[2] [n_v, d, d]) views of a session's recurrent state
        (the layout kd_recurrent_state_bytes describes; ring buffers padded to ``ring`` floats)."""
        t = self.rec[s][il]
        rings = [t[i * ring:i * ring + (d_conv - 1) * C].view(d_conv - 1, C) for i in range(2)]
        states = [t[2 * ring + i * state:2 * ring + (i + 1) * state] for i in range(2)]
        return rings, states

    def fill_prefill(self, s: int, il: int, k: np.ndarray, v: np.ndarray) -> None:
        L = k.shape[1]
        self.t[s][il, 0, :, :L] = torch.from_numpy(k).to(self.t[s].device)
        self.t[s][il, 1, :, :L] = torch.from_numpy(v).to(self.t[s].device)

"""CPU oracle of the batched multi-session decode step (plain fp64 numpy).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product path
(``session_decode_step_amd`` and its HIP library) never does, and this package
imports nothing from it.  The two share no code: only the seeded input generator
(``workload``), which holds no arithmetic of the method, serves both.

What it computes is the plain definition of one decode step for B sessions
(memra-engine 0.72.0, src/decode_batch.rs: module header and the Full-attention arm
of ``decode_batch_layers``; hf2q ADR-040 §0.7 task blocks F2-F5), in fp64, with
fp32 only at the rounding points the method defines: the activation quantiser and
the fp16 KV store.  Each function cites the passage it follows.

Pins (tests marked ``not gpu``) check it against hand-worked blocks, closed forms,
brute force and library routines; the composition of a whole dense step (two layers and
the lm_head) is pinned against the same step built from torch's own routines, the MoE
routed sum against a dense masked sum over every expert, and the block variants and the
linear layer by their closed forms and special cases.
"""
from .ops import (QK, KQ_BYTES, kquant_dequantize, kquant_fields, kquant_scale_min, accept_drafts, gated_rmsnorm, gdn_prep, l2_normalize, softplus, ssm_conv_step, attention, block_dots, dequantize, dequantize_act, e4m3_decode,  # noqa: F401
                  e4m3_encode, e4m3_values, embed_rows, gdn_step, greedy_token, sigmoid,
                  mmvq, mmvq_blocks, q8_kv_decode, q8_kv_encode, q8_kv_row_bytes, quantize_act, rmsnorm, rope_neox, router_topk, silu, swiglu, weight_codes)
from .step import DenseWeights, OracleCaches, decode_layer, decode_step, moe_ffn, output_head  # noqa: F401

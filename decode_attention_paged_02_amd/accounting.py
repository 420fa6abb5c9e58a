"""KV-cache byte and FLOP accounting for decode attention.

Formulas (stated on "Attention Kernel Variants: MQA, GQA, and MLA", the
design-space table and "Numbers Worth Remembering"):
  MHA/GQA/MQA: bytes/token = 2 x layers x kv_heads x head_dim x dtype_bytes
  MLA:         bytes/token = layers x (kv_lora_rank + rope_dim) x dtype_bytes
A decode step reads every cached token of every sequence once: B x C x bytes/token
(same page, "Decode Is a Bandwidth Problem"; the drill page, sec. 1, counts
2 x B x ctx x Hkv x D x 2 bytes for one layer).
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "e4m3": 1}


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, dtype_bytes: float) -> float:
    """Whole-model K+V bytes cached per token (MHA/GQA/MQA)."""
    return 2 * layers * kv_heads * head_dim * dtype_bytes


def mla_bytes_per_token(layers: int, d_latent: int, d_rope: int, dtype_bytes: float) -> float:
    """Whole-model bytes cached per token for an MLA latent record."""
    return layers * (d_latent + d_rope) * dtype_bytes


def step_kv_bytes(context_lens: Sequence[int], *, num_kv_heads: int, head_dim: int,
                  head_dim_v: int, kv_dtype: str, mla: bool = False) -> int:
    """Algorithmic bytes one decode step must read from the cache (one layer).

    GQA family: every valid token's K row (head_dim) and V row (head_dim_v) of
    every KV head, once.  MLA: every valid token's record (head_dim wide) once;
    V is the first head_dim_v values of those same bytes."""
    n = int(np.asarray(context_lens, dtype=np.int64).sum())
    eb = ELEM_BYTES[kv_dtype]
    if mla:
        return n * head_dim * eb
    return n * num_kv_heads * (head_dim + head_dim_v) * eb


def step_flops(context_lens: Sequence[int], *, num_q_heads: int, head_dim: int,
               head_dim_v: int) -> int:
    """Multiply-add FLOPs of one step: 2*(dk + dv) per (query head, token)."""
    n = int(np.asarray(context_lens, dtype=np.int64).sum())
    return 2 * n * num_q_heads * (head_dim + head_dim_v)


def case_kv_bytes(case) -> int:
    return step_kv_bytes(case.context_lens, num_kv_heads=case.num_kv_heads,
                         head_dim=case.head_dim, head_dim_v=case.head_dim_v,
                         kv_dtype=case.kv_dtype, mla=case.mla)


def case_flops(case) -> int:
    return step_flops(case.context_lens, num_q_heads=case.num_q_heads,
                      head_dim=case.head_dim, head_dim_v=case.head_dim_v)


def case_overhead_bytes(case, max_splits: int) -> dict:
    """Bytes a step moves besides the algorithmic KV bytes: q read, out and
    LSE written, block-table entries and lengths read, and (with splits) the
    partial outputs (fp32; binary16 for MLA) and fp32 LSEs written and read
    back by the combine."""
    eb_q = ELEM_BYTES[case.q_dtype]
    rows = case.batch * case.q_len * case.num_q_heads
    pages = int(((np.asarray(case.context_lens, dtype=np.int64) + case.page_size - 1)
                 // case.page_size).sum())
    r = {"q": rows * case.head_dim * eb_q,
         "out_and_lse": rows * (case.head_dim_v * eb_q + 4),
         "tables_and_lengths": pages * 4 + case.batch * 4,
         "split_partials": 0}
    if max_splits > 1:
        eb_part = 2 if case.mla else 4
        r["split_partials"] = 2 * rows * max_splits * (case.head_dim_v * eb_part + 4)
    return r

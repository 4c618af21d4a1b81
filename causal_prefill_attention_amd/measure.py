"""Algorithmic work of one prefill-attention call, and MI355X peaks.

FLOPs count only visible (query, key) pairs: each pair costs one
``head_dim``-long dot product for the score and one ``head_dim``-long
multiply-add into the output, i.e. ``4 * d`` flops per pair per query head.
Masked work inside diagonal tiles, softmax arithmetic and the dense
``L x L`` product are not counted.

Bytes are the algorithmic minimum: Q, K and V read once in their storage
dtype, and the bf16 output written once.
"""
from __future__ import annotations

from typing import Sequence

#: MI355X dense bf16 MFMA peak: 256 CUs x 4096 flop/clk/CU x 2.4 GHz.
PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
#: MI355X HBM3E peak bandwidth.
PEAK_HBM_GBS = 8000.0

DTYPE_BYTES = {"bf16": 2, "fp16": 2, "fp32": 4}


def visible_pairs_one(n: int, window: int) -> int:
    """Visible (query, key) pairs of one causal sequence of length n."""
    if n <= 0:
        return 0
    if window <= 0 or window >= n:
        return n * (n + 1) // 2
    return window * (window + 1) // 2 + (n - window) * window


def visible_pairs(lengths: Sequence[int], window: int) -> int:
    return sum(visible_pairs_one(int(n), window) for n in lengths)


def causal_flops(lengths: Sequence[int], n_q_heads: int, head_dim: int,
                 window: int) -> int:
    return 4 * head_dim * n_q_heads * visible_pairs(lengths, window)


def algorithmic_bytes(lengths: Sequence[int], n_q_heads: int, n_kv_heads: int,
                      head_dim: int, q_dtype: str, kv_dtype: str) -> int:
    t = int(sum(lengths))
    q = t * n_q_heads * head_dim * DTYPE_BYTES[q_dtype]
    kv = 2 * t * n_kv_heads * head_dim * DTYPE_BYTES[kv_dtype]
    o = t * n_q_heads * head_dim * 2
    return q + kv + o

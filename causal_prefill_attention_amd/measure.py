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

from typing import Optional, Sequence

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


def _prefix_visible(p: int, window: int) -> int:
    """Visible keys summed over the queries at positions 0 .. p - 1."""
    if p <= 0:
        return 0
    if window <= 0 or window >= p:
        return p * (p + 1) // 2
    return window * (window + 1) // 2 + (p - window) * window


def visible_pairs_history(n_q: int, n_k: int, window: int) -> int:
    """Visible pairs when the n_q queries are the last positions of n_k."""
    if n_q <= 0 or n_k <= 0:
        return 0
    first = max(n_k - n_q, 0)  # positions below 0 see nothing
    return _prefix_visible(n_k, window) - _prefix_visible(first, window)


def visible_pairs(lengths: Sequence[int], window: int,
                  kv_lengths: Optional[Sequence[int]] = None) -> int:
    if kv_lengths is None:
        return sum(visible_pairs_one(int(n), window) for n in lengths)
    return sum(visible_pairs_history(int(n), int(m), window)
               for n, m in zip(lengths, kv_lengths))


def causal_flops(lengths: Sequence[int], n_q_heads: int, head_dim: int,
                 window: int, kv_lengths: Optional[Sequence[int]] = None,
                 head_dim_v: Optional[int] = None) -> int:
    """2 * (d_qk + d_v) flops per visible pair and query head (4 * d when
    the two head sizes agree)."""
    dv = head_dim if head_dim_v is None else head_dim_v
    return 2 * (head_dim + dv) * n_q_heads * visible_pairs(lengths, window, kv_lengths)


def algorithmic_bytes(lengths: Sequence[int], n_q_heads: int, n_kv_heads: int,
                      head_dim: int, q_dtype: str, kv_dtype: str,
                      kv_lengths: Optional[Sequence[int]] = None,
                      head_dim_v: Optional[int] = None, v_in_k: bool = False) -> int:
    """Q, K, V read once (V not at all when it is part of K's rows) and the
    bf16 output written once."""
    t = int(sum(lengths))
    tk = t if kv_lengths is None else int(sum(kv_lengths))
    dv = head_dim if head_dim_v is None else head_dim_v
    q = t * n_q_heads * head_dim * DTYPE_BYTES[q_dtype]
    kv = tk * n_kv_heads * (head_dim + (0 if v_in_k else dv)) * DTYPE_BYTES[kv_dtype]
    o = t * n_q_heads * dv * 2
    return q + kv + o

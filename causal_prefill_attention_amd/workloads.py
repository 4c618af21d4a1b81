"""Seeded synthetic inputs for causal prefill attention.

This module holds shapes and random draws only -- no attention arithmetic.
The HIP path's tests and benchmark and the oracle's tests both take their
inputs from here, so the two sides see bit-identical tensors.

Recipe (the same for every workload):

* ``numpy.random.default_rng(seed)`` (PCG64).
* Draw order: sequence lengths (only for a random-length batch, inclusive
  bounds, ``integers(lo, hi + 1, n_seqs)``), then Q, K and V from
  ``standard_normal`` in float64, each shaped ``[T, heads, head_dim]``, then
  the K outlier positions (``choice`` without replacement over the flat K,
  ``floor(frac * K.size)`` of them), which are multiplied by the outlier
  factor in float64; a workload with outlier *channels* instead draws, per
  KV head, ``k_outlier_channels`` distinct head-dim indices (``choice``
  without replacement over ``head_dim``) and multiplies that column of
  every token by the same factor.
* The float64 draws are narrowed to the storage dtype by torch's CPU cast
  (round to nearest even).

The packed layout is ``[T, heads, head_dim]`` with the sequences stored one
after another; ``cu_seqlens`` holds the ``n_seqs + 1`` cumulative offsets.
A chunked-prefill workload gives each sequence a KV history: its K/V hold
``history + length`` tokens (packed by ``cu_seqlens_k``) and its Q only the
``length`` new ones; K and V are then drawn with ``Tk`` rows instead of
``T``, in the same order.
This matches the per-layer KV addressing ``[sequence][position][kv_head]
[head_dim]`` and the packed offsets of the m40-llm AGENTS.md page ("Project
Snapshot" and the varlen-batch task), with one layer's slice taken.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

_TORCH_DTYPES = {
    "bf16": torch.bfloat16,
    "fp16": torch.float16,
    "fp32": torch.float32,
}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic prefill-attention problem."""

    name: str
    seed: int
    lengths: Optional[Tuple[int, ...]]  # fixed lengths, or None for random
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    window: int = 0  # 0 = no sliding window
    q_dtype: str = "bf16"
    kv_dtype: str = "bf16"
    random_lengths: Optional[Tuple[int, int, int]] = None  # (n_seqs, lo, hi)
    k_outlier_frac: float = 0.0
    k_outlier_mult: float = 30.0
    k_outlier_channels: int = 0  # whole K channels (per KV head) scaled, every token
    scale: Optional[float] = None  # None -> 1/sqrt(head_dim)
    history: Optional[Tuple[int, ...]] = None  # KV history per sequence (chunked)
    decode: bool = False  # one query per sequence, run through the decode kernel
    head_dim_v: Optional[int] = None  # v/out head size when it differs (absorbed MLA)

    @property
    def attn_scale(self) -> float:
        if self.scale is not None:
            return float(self.scale)
        return 1.0 / math.sqrt(self.head_dim)

    def describe(self) -> Dict[str, object]:
        return {
            "workload": self.name,
            "seed": self.seed,
            "n_q_heads": self.n_q_heads,
            "n_kv_heads": self.n_kv_heads,
            "head_dim": self.head_dim,
            "window": self.window,
            "q_dtype": self.q_dtype,
            "kv_dtype": self.kv_dtype,
            "k_outlier_frac": self.k_outlier_frac,
            **({"k_outlier_channels": self.k_outlier_channels}
               if self.k_outlier_channels else {}),
            "scale": self.attn_scale,
            **({"history": list(self.history)} if self.history else {}),
            **({"decode": True} if self.decode else {}),
            **({"head_dim_v": self.head_dim_v} if self.head_dim_v else {}),
        }


_D = 128
_SCALE = 1.0 / math.sqrt(_D)

#: The five problem shapes of this kernel, by what they are.
WORKLOADS: Dict[str, Workload] = {
    # one short sequence, MQA 4:1 -- small enough for the oracle in full
    "causal_128tok_4q1kv": Workload(
        "causal_128tok_4q1kv", 0, (128,), 4, 1, _D, scale=_SCALE),
    # MLA-shaped layer: 128-d head (64 "nope" + 64 "rope", both N(0,1))
    "mla_2048tok_32q1kv": Workload(
        "mla_2048tok_32q1kv", 1, (2048,), 32, 1, _D, scale=_SCALE),
    # the same head shape, 4096 tokens with a 1024-token sliding window
    "window1024_4096tok_32q1kv": Workload(
        "window1024_4096tok_32q1kv", 2, (4096,), 32, 1, _D, window=1024,
        scale=_SCALE),
    # packed varlen batch, GQA 4:1, fp32 Q and fp16 K/V in storage
    "varlen16_gqa32q8kv_fp32q_fp16kv": Workload(
        "varlen16_gqa32q8kv_fp32q_fp16kv", 3, None, 32, 8, _D,
        q_dtype="fp32", kv_dtype="fp16", random_lengths=(16, 64, 2048),
        scale=_SCALE),
    # long prefill, MQA, 1% of the K entries scaled by 30
    "long_8192tok_32q1kv_outliers": Workload(
        "long_8192tok_32q1kv_outliers", 4, (8192,), 32, 1, _D,
        k_outlier_frac=0.01, scale=_SCALE),
    # the long prefill with whole outlier channels: round(1% of 128) = 1 K
    # channel per KV head scaled by 30 for every token (the peakiest
    # softmax that "1% of K entries x30 (outlier channels)" admits)
    "long_8192tok_32q1kv_outlier_channel": Workload(
        "long_8192tok_32q1kv_outlier_channel", 4, (8192,), 32, 1, _D,
        k_outlier_channels=1, scale=_SCALE),
    # one GPU's share of the long prefill under 8-way head sharding
    "long_8192tok_4q1kv_outliers_share": Workload(
        "long_8192tok_4q1kv_outliers_share", 4, (8192,), 4, 1, _D,
        k_outlier_frac=0.01, scale=_SCALE),
    # chunked prefill: the last 2048 tokens of an 8192-token sequence against
    # its 6144-token KV history
    "chunk2048_hist6144_32q1kv_outliers": Workload(
        "chunk2048_hist6144_32q1kv_outliers", 5, (2048,), 32, 1, _D,
        k_outlier_frac=0.01, scale=_SCALE, history=(6144,)),
    # the long prefill with 64-d heads
    "d64_8192tok_32q1kv_outliers": Workload(
        "d64_8192tok_32q1kv_outliers", 7, (8192,), 32, 1, 64,
        k_outlier_frac=0.01, scale=1.0 / 8.0),
    # 256-d heads, GQA 8:1
    "d256_4096tok_16q2kv_outliers": Workload(
        "d256_4096tok_16q2kv_outliers", 10, (4096,), 16, 2, 256,
        k_outlier_frac=0.01, scale=1.0 / 16.0),
    # 512-d heads (the page's path for head sizes above 256), GQA 4:1
    "d512_4096tok_8q2kv_outliers": Workload(
        "d512_4096tok_8q2kv_outliers", 12, (4096,), 8, 2, 512,
        k_outlier_frac=0.01, scale=1.0 / math.sqrt(512)),
    # absorbed MLA prefill: q [q_absorbed | q_rope] (320) against one
    # compressed cache row [kv_latent | k_rope] (320) per token, v = the
    # kv_latent part (256), scale 1/sqrt(320)
    "mla_absorbed_4096tok_16q_320_256": Workload(
        "mla_absorbed_4096tok_16q_320_256", 11, (4096,), 16, 1, 320,
        scale=1.0 / math.sqrt(320), head_dim_v=256),
    # decode: 64 sequences of mixed length (512 .. 8191 keys), GQA 4:1
    "decode64_gqa32q8kv_mixed": Workload(
        "decode64_gqa32q8kv_mixed", 8, (1,) * 64, 32, 8, _D, scale=_SCALE,
        history=tuple(511 + (s * 977) % 7680 for s in range(64)), decode=True),
    # decode: 32 sequences of 8192 keys, MQA with 32 query heads
    "decode32_mqa32q1kv_8192": Workload(
        "decode32_mqa32q1kv_8192", 9, (1,) * 32, 32, 1, _D, scale=_SCALE,
        history=(8191,) * 32, decode=True),
    # a packed batch of chunks with ragged histories, GQA 4:1
    "chunks8_gqa32q8kv_history": Workload(
        "chunks8_gqa32q8kv_history", 6, (300, 1, 64, 1000, 129, 0, 77, 512),
        32, 8, _D, scale=_SCALE, history=(700, 4000, 0, 24, 2000, 50, 3, 1536)),
}

#: The workload the throughput metric is quoted on.
HEADLINE = "long_8192tok_32q1kv_outliers"


def custom(name: str, lengths: Sequence[int], n_q_heads: int, n_kv_heads: int,
           head_dim: int = _D, window: int = 0, q_dtype: str = "bf16",
           kv_dtype: str = "bf16", seed: int = 0, scale: Optional[float] = None,
           k_outlier_frac: float = 0.0,
           history: Optional[Sequence[int]] = None,
           k_outlier_channels: int = 0) -> Workload:
    """A test-sized workload with explicit lengths (and KV histories)."""
    return Workload(name, seed, tuple(int(x) for x in lengths), n_q_heads,
                    n_kv_heads, head_dim, window=window, q_dtype=q_dtype,
                    kv_dtype=kv_dtype, scale=scale,
                    k_outlier_frac=k_outlier_frac,
                    k_outlier_channels=k_outlier_channels,
                    history=None if history is None else tuple(int(x) for x in history))


def draw_lengths(w: Workload, rng: np.random.Generator) -> List[int]:
    if w.random_lengths is not None:
        n, lo, hi = w.random_lengths
        return [int(x) for x in rng.integers(lo, hi + 1, n)]
    assert w.lengths is not None
    return list(w.lengths)


def cu_seqlens_of(lengths: Sequence[int]) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu.astype(np.int32)


def sha256_of(t: torch.Tensor) -> str:
    return hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()
                          ).hexdigest()


def make_inputs(w: Workload) -> Dict[str, object]:
    """Draw the workload's tensors on the CPU in their storage dtypes.

    Returns ``q``, ``k``, ``v`` (torch CPU tensors, contiguous
    ``[T, heads, head_dim]``), ``cu_seqlens`` (torch int32 CPU), ``lengths``
    and a SHA-256 per tensor; with a KV history also ``cu_seqlens_k`` and
    ``kv_lengths`` (K and V then have ``Tk`` rows).
    """
    rng = np.random.default_rng(w.seed)
    lengths = draw_lengths(w, rng)
    total = int(sum(lengths))
    if w.history is not None:
        if len(w.history) != len(lengths):
            raise ValueError("history needs one entry per sequence")
        kv_lengths = [int(h) + int(n) for h, n in zip(w.history, lengths)]
    else:
        kv_lengths = list(lengths)
    total_k = int(sum(kv_lengths))
    d = w.head_dim
    q64 = rng.standard_normal((total, w.n_q_heads, d))
    k64 = rng.standard_normal((total_k, w.n_kv_heads, d))
    v64 = rng.standard_normal((total_k, w.n_kv_heads, d))
    if w.k_outlier_frac > 0.0 and k64.size > 0:
        n_out = int(math.floor(w.k_outlier_frac * k64.size))
        idx = rng.choice(k64.size, size=n_out, replace=False)
        flat = k64.reshape(-1)
        flat[idx] *= w.k_outlier_mult
    if w.k_outlier_channels > 0 and k64.size > 0:
        for g in range(w.n_kv_heads):
            ch = rng.choice(d, size=w.k_outlier_channels, replace=False)
            k64[:, g, ch] *= w.k_outlier_mult
    q = torch.from_numpy(q64).to(_TORCH_DTYPES[w.q_dtype])
    k = torch.from_numpy(k64).to(_TORCH_DTYPES[w.kv_dtype])
    v = torch.from_numpy(v64).to(_TORCH_DTYPES[w.kv_dtype])
    if w.head_dim_v is not None:
        # absorbed MLA: the values are the first head_dim_v columns of the
        # cache row (a view of k); the drawn v is not used
        v = k[:, :, :w.head_dim_v]
    cu = torch.from_numpy(cu_seqlens_of(lengths))
    out = {
        "q": q, "k": k, "v": v, "cu_seqlens": cu, "lengths": lengths,
        "sha256": {"q": sha256_of(q), "k": sha256_of(k), "v": sha256_of(v),
                   "cu_seqlens": sha256_of(cu)},
    }
    if w.history is not None:
        cuk = torch.from_numpy(cu_seqlens_of(kv_lengths))
        out["cu_seqlens_k"] = cuk
        out["kv_lengths"] = kv_lengths
        out["sha256"]["cu_seqlens_k"] = sha256_of(cuk)
    return out


def sample_rows(lengths: Sequence[int], n_q_heads: int, n: int, seed: int
                ) -> List[Tuple[int, int]]:
    """Seeded (token, head) sample for spot checks at full size.

    Always includes the first and last token of the first and last non-empty
    sequence (head 0 and the last head) so that the causal edge rows are
    covered, then uniform draws.
    """
    total = int(sum(lengths))
    rows: List[Tuple[int, int]] = []
    cu = cu_seqlens_of(lengths)
    nonempty = [s for s, L in enumerate(lengths) if L > 0]
    for s in (nonempty[:1] + nonempty[-1:]):
        for tok in (int(cu[s]), int(cu[s + 1]) - 1):
            for h in (0, n_q_heads - 1):
                rows.append((tok, h))
    rng = np.random.default_rng(10_000 + seed)
    for _ in range(max(0, n - len(rows))):
        rows.append((int(rng.integers(0, total)), int(rng.integers(0, n_q_heads))))
    seen = set()
    out = []
    for r in rows:
        if r not in seen:
            seen.add(r)
            out.append(r)
    return out

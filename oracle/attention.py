"""FP64 CPU oracle for causal prefill attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` import this module.  The library,
its C ABI and its Python binding never import, call or link it, and it
imports nothing from them.

What is computed (the plain definition, written out):

For each packed sequence ``s`` (tokens ``cu[s] .. cu[s+1]-1``, local indices
``i, j`` in ``[0, L_s)``), each query head ``h`` and its key/value head
``g = h // (n_q_heads / n_kv_heads)``:

1. Inputs are converted exactly as passed to float64 (bf16, fp16 and fp32
   all embed exactly).
2. ``S = scale * Q[s, h] @ K[s, g]^T``, an ``L x L`` float64 matrix.
3. Key ``j`` is visible to query ``i`` iff ``j <= i`` and (``W == 0`` or
   ``j >= i - W + 1``): the causal bound ``kv_end = min(q_pos + 1,
   seq_len)`` of the fused MLA prefill kernel on the atlas PR #69 page
   (its re-audit commits), with the sliding window passed as a width where
   0 means "off" (the cache-skip MLA fix commit on the same page, which
   forwards ``sliding_window.unwrap_or(0)``).  ``W > 0`` keeps the W most
   recent keys including the query's own position -- the "exact recent
   ring" of the m40-llm AGENTS.md page ("Current Progress").
4. ``P = rowsoftmax(S + mask)``: the row maximum over visible keys is
   subtracted, the row is exponentiated and divided by its sum.  Every row
   has at least one visible key (``j = i``).
5. ``O[s, h] = P @ V[s, g]``.
6. Sequences never see each other.

Chunked prefill against a KV history (``attention_chunked``): a later
prefill chunk attends to every earlier token of its sequence, not only to
the tokens of the chunk -- the multi-chunk fix on the atlas PR #69 page
(later chunks use ``kv_len = seq_len_start + n``).  Sequence ``s`` then has
``Lq`` new queries and ``Lk >= Lq`` keys/values (history followed by the
chunk itself); query ``i`` sits at absolute position ``Lk - Lq + i`` and the
visibility rule of step 3 is applied to that position.  With ``Lq == Lk``
this is exactly the definition above.  A query with no visible key (only
possible when ``Lq > Lk``, outside the contract) has an all-zero output row.

Paged KV (``attention_paged``): the keys and values live in page pools of
``page_size`` token slots per page (the paged MLA prefill of atlas PR #69
reads every key through a page-table lookup; the m40-llm AGENTS.md page
addresses the cache per [sequence][position][kv_head][head_dim]).  Key
position ``j`` of sequence ``s`` is slot ``j % page_size`` of page
``block_table[s][j // page_size]``; ``seqlens_k[s]`` gives ``Lk``.  The result
is ``attention_chunked`` on the keys and values gathered in position order.

Decode (``attention_decode``): one new query per sequence, the batched
last-token step of the m40-llm AGENTS.md page ("Current Progress"); it is
``attention_chunked`` with ``Lq = 1`` for every sequence.

The online-softmax recurrence that the GPU kernel uses (the fused MLA prefill
commit on the atlas PR #69 page) is a reordering of steps 4-5 and is not
used here.  The head grouping ``g = h // group`` is the consecutive GQA
mapping (the m40-llm page's Qwen-shaped 16 Q / 2 KV packed-prefill test
leaves the mapping unstated; this is the plain reading).
"""
from __future__ import annotations

import concurrent.futures
import os
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "kv_head_of",
    "visibility",
    "softmax_probs",
    "attention_head",
    "attention_varlen",
    "attention_chunked",
    "attention_paged",
    "attention_decode",
    "gather_pages",
    "attention_rows",
    "visible_pairs",
]


def _as_f64(x) -> np.ndarray:
    """Exact widening to float64 (torch tensors or numpy arrays)."""
    if hasattr(x, "detach"):  # torch tensor: widen in torch, bf16 has no numpy dtype
        import torch

        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _as_offsets(cu_seqlens) -> List[int]:
    if hasattr(cu_seqlens, "detach"):
        cu_seqlens = cu_seqlens.detach().cpu().numpy()
    return [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]


def kv_head_of(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    """Key/value head read by query head ``h`` (consecutive grouping)."""
    group = n_q_heads // n_kv_heads
    return h // group


def visibility(n_rows: int, n_cols: int, window: int,
               q_offset: int = 0) -> np.ndarray:
    """Boolean ``[n_rows, n_cols]``: may query ``i`` attend to key ``j``.

    Query ``i`` sits at absolute position ``q_offset + i`` (0 for a prefill
    without history).
    """
    pos = q_offset + np.arange(n_rows)[:, None]
    j = np.arange(n_cols)[None, :]
    vis = j <= pos
    if window > 0:
        vis &= j >= pos - window + 1
    return vis


def softmax_probs(q_h, k_g, scale: float, window: int,
                  q_offset: Optional[int] = None) -> np.ndarray:
    """Attention probabilities ``P`` for one sequence and one head.

    ``q_h``: ``[Lq, d]``, ``k_g``: ``[Lk, d]``; the queries are the last
    ``Lq`` positions unless ``q_offset`` says otherwise.  Returns float64
    ``[Lq, Lk]`` whose rows sum to one over the visible keys and are exactly
    0 elsewhere (all 0 for a row without a visible key).
    """
    q_h = _as_f64(q_h)
    k_g = _as_f64(k_g)
    n_q, n_k = q_h.shape[0], k_g.shape[0]
    if q_offset is None:
        q_offset = n_k - n_q
    s = float(scale) * (q_h @ k_g.T)
    vis = visibility(n_q, n_k, window, q_offset)
    p = np.zeros((n_q, n_k), dtype=np.float64)
    rows = vis.any(axis=1)
    if rows.any():
        sv = np.where(vis[rows], s[rows], -np.inf)
        m = sv.max(axis=1, keepdims=True)
        e = np.exp(sv - m)
        p[rows] = e / e.sum(axis=1, keepdims=True)
    return p


def attention_head(q_h, k_g, v_g, scale: float, window: int,
                   q_offset: Optional[int] = None) -> np.ndarray:
    """``O = softmax(scale * Q K^T + mask) V`` for one sequence, one head."""
    if np.shape(q_h)[0] == 0:
        return np.zeros((0, np.shape(v_g)[1]), dtype=np.float64)
    p = softmax_probs(q_h, k_g, scale, window, q_offset)
    return p @ _as_f64(v_g)


def attention_varlen(q, k, v, cu_seqlens, n_q_heads: int, n_kv_heads: int,
                     scale: float, window: int,
                     workers: Optional[int] = None) -> np.ndarray:
    """Packed varlen causal attention, float64 ``[T, n_q_heads, d_v]``.

    ``q``: ``[T, n_q_heads, d]``; ``k``, ``v``: ``[T, n_kv_heads, d]``;
    ``cu_seqlens``: ``n_seqs + 1`` offsets.  (sequence, head) pairs are
    independent and run on a thread pool of ``workers`` threads (default:
    all host cores), each with a single BLAS thread.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    cu = _as_offsets(cu_seqlens)
    if n_q_heads % n_kv_heads != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    out = np.zeros((q.shape[0], n_q_heads, v.shape[2]), dtype=np.float64)
    jobs = [(s, h) for s in range(len(cu) - 1) for h in range(n_q_heads)
            if cu[s + 1] > cu[s]]

    def run(job):
        s, h = job
        a, b = cu[s], cu[s + 1]
        g = kv_head_of(h, n_q_heads, n_kv_heads)
        out[a:b, h, :] = attention_head(q[a:b, h, :], k[a:b, g, :],
                                        v[a:b, g, :], scale, window)

    n_workers = workers if workers is not None else (os.cpu_count() or 1)
    if n_workers <= 1 or len(jobs) <= 1:
        for job in jobs:
            run(job)
        return out
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1):
        with concurrent.futures.ThreadPoolExecutor(n_workers) as pool:
            for f in [pool.submit(run, job) for job in jobs]:
                f.result()
    return out


def attention_chunked(q, k, v, cu_seqlens_q, cu_seqlens_k, n_q_heads: int,
                      n_kv_heads: int, scale: float, window: int,
                      workers: Optional[int] = None) -> np.ndarray:
    """Chunked prefill against a KV history, float64 ``[Tq, n_q_heads, d_v]``.

    ``q``: ``[Tq, n_q_heads, d]`` packed by ``cu_seqlens_q``; ``k``, ``v``:
    ``[Tk, n_kv_heads, d]`` packed by ``cu_seqlens_k`` (same number of
    sequences).  Sequence ``s``'s queries are the last ``Lq`` of its ``Lk``
    positions.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    cq = _as_offsets(cu_seqlens_q)
    ck = _as_offsets(cu_seqlens_k)
    if len(cq) != len(ck):
        raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
    if n_q_heads % n_kv_heads != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    out = np.zeros((q.shape[0], n_q_heads, v.shape[2]), dtype=np.float64)
    jobs = [(s, h) for s in range(len(cq) - 1) for h in range(n_q_heads)
            if cq[s + 1] > cq[s]]

    def run(job):
        s, h = job
        a, b = cq[s], cq[s + 1]
        ka, kb = ck[s], ck[s + 1]
        g = kv_head_of(h, n_q_heads, n_kv_heads)
        out[a:b, h, :] = attention_head(q[a:b, h, :], k[ka:kb, g, :],
                                        v[ka:kb, g, :], scale, window,
                                        (kb - ka) - (b - a))

    n_workers = workers if workers is not None else (os.cpu_count() or 1)
    if n_workers <= 1 or len(jobs) <= 1:
        for job in jobs:
            run(job)
        return out
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1):
        with concurrent.futures.ThreadPoolExecutor(n_workers) as pool:
            for f in [pool.submit(run, job) for job in jobs]:
                f.result()
    return out


def gather_pages(pool, block_table, seqlens_k, page_size: int):
    """Keys (or values) of every sequence in position order, packed.

    ``pool``: ``[n_pages * page_size, heads, d]`` token slots;
    ``block_table``: ``[n_seqs, table_width]`` physical page numbers;
    ``seqlens_k``: keys per sequence.  Returns the packed float64 tensor and
    its ``n_seqs + 1`` offsets.
    """
    pool = _as_f64(pool)
    table = np.asarray(_as_f64(block_table), dtype=np.int64)
    lens = [int(x) for x in np.asarray(_as_f64(seqlens_k)).reshape(-1)]
    parts, cu = [], [0]
    for s, n in enumerate(lens):
        pos = np.arange(n)
        slots = table[s, pos // page_size] * page_size + pos % page_size
        parts.append(pool[slots])
        cu.append(cu[-1] + n)
    packed = (np.concatenate(parts) if parts else
              np.zeros((0,) + pool.shape[1:], dtype=np.float64))
    return packed, cu


def attention_paged(q, k_pool, v_pool, cu_seqlens_q, block_table, seqlens_k,
                    page_size: int, n_q_heads: int, n_kv_heads: int,
                    scale: float, window: int,
                    workers: Optional[int] = None) -> np.ndarray:
    """Chunked prefill whose KV history is read through a block table."""
    k, cu_k = gather_pages(k_pool, block_table, seqlens_k, page_size)
    v, _ = gather_pages(v_pool, block_table, seqlens_k, page_size)
    return attention_chunked(q, k, v, cu_seqlens_q, cu_k, n_q_heads, n_kv_heads,
                             scale, window, workers=workers)


def attention_decode(q, k, v, cu_seqlens_k, n_q_heads: int, n_kv_heads: int,
                     scale: float, window: int,
                     workers: Optional[int] = None) -> np.ndarray:
    """One query per sequence (``q``: ``[n_seqs, n_q_heads, d]``) against
    the packed keys of ``cu_seqlens_k``."""
    n = np.shape(q)[0]
    return attention_chunked(q, k, v, list(range(n + 1)), cu_seqlens_k, n_q_heads,
                             n_kv_heads, scale, window, workers=workers)


def attention_rows(q, k, v, cu_seqlens, n_q_heads: int, n_kv_heads: int,
                   scale: float, window: int,
                   rows: Iterable[Tuple[int, int]],
                   cu_seqlens_k=None) -> np.ndarray:
    """The same definition evaluated one output row at a time.

    ``rows`` lists ``(token, q_head)`` pairs; returns float64
    ``[len(rows), d_v]``.  Used for spot checks at sizes where the full
    result is too slow to form.  With ``cu_seqlens_k`` the keys come from a
    KV history as in ``attention_chunked``.
    """
    cu = _as_offsets(cu_seqlens)
    ck = cu if cu_seqlens_k is None else _as_offsets(cu_seqlens_k)
    rows = list(rows)
    q_t = q
    res = np.zeros((len(rows), np.shape(v)[2]), dtype=np.float64)
    for r, (tok, h) in enumerate(rows):
        s = int(np.searchsorted(np.asarray(cu), tok, side="right")) - 1
        while cu[s + 1] <= tok:  # skip empty sequences sharing the offset
            s += 1
        pos = (ck[s + 1] - ck[s]) - (cu[s + 1] - cu[s]) + (tok - cu[s])
        lo = 0 if window == 0 else max(0, pos - window + 1)
        if pos < 0:
            continue  # no visible key: zero row
        g = kv_head_of(h, n_q_heads, n_kv_heads)
        qi = _as_f64(q_t[tok, h, :])
        kk = _as_f64(k[ck[s] + lo:ck[s] + pos + 1, g, :])
        vv = _as_f64(v[ck[s] + lo:ck[s] + pos + 1, g, :])
        sc = float(scale) * (kk @ qi)
        e = np.exp(sc - sc.max())
        res[r] = (e / e.sum()) @ vv
    return res


def visible_pairs(lengths: Sequence[int], window: int,
                  q_lengths: Optional[Sequence[int]] = None) -> int:
    """Number of visible (query, key) pairs, summed over sequences.

    ``lengths`` are the key counts; ``q_lengths`` (default: the same) the
    query counts, the queries being the last positions.
    """
    total = 0
    q_lengths = lengths if q_lengths is None else q_lengths
    for n, nq in zip(lengths, q_lengths):
        if n and nq:
            total += int(visibility(int(nq), int(n), window, int(n) - int(nq)).sum())
    return total

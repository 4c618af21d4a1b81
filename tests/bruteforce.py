"""Literal-loop attention for tiny inputs: the independent pin of the oracle.

Written without numpy arithmetic: Python floats, ``math.exp`` and explicit
loops over queries, keys and head dimensions, so that it shares no code path
with the vectorised oracle.  The definition it spells out is the one of
``softmax(scale * q.k + mask) . v`` per query, with the causal bound
``kv_end = min(q_pos + 1, seq_len)`` and a sliding window of width W
(0 = off) covering the W most recent positions.
"""
import math


def brute_attention(q, k, v, cu, n_q_heads, n_kv_heads, scale, window):
    """q[t][h][c], k[t][g][c], v[t][g][c] as nested Python lists of floats.

    Returns out[t][h][c] as nested lists.
    """
    total = len(q)
    d_v = len(v[0][0]) if total else 0
    out = [[[0.0] * d_v for _ in range(n_q_heads)] for _ in range(total)]
    for s in range(len(cu) - 1):
        start, end = cu[s], cu[s + 1]
        for t in range(start, end):
            i = t - start
            for h in range(n_q_heads):
                g = (h * n_kv_heads) // n_q_heads
                keys = []
                for j in range(0, end - start):
                    if j > i:
                        continue
                    if window and i - j >= window:
                        continue
                    keys.append(j)
                scores = []
                for j in keys:
                    acc = 0.0
                    for c in range(len(q[t][h])):
                        acc += q[t][h][c] * k[start + j][g][c]
                    scores.append(scale * acc)
                top = max(scores)
                weights = [math.exp(x - top) for x in scores]
                z = sum(weights)
                for c in range(d_v):
                    acc = 0.0
                    for w, j in zip(weights, keys):
                        acc += w * v[start + j][g][c]
                    out[t][h][c] = acc / z
    return out


def brute_attention_chunked(q, k, v, cu_q, cu_k, n_q_heads, n_kv_heads, scale,
                            window):
    """Chunked prefill against a KV history, literal loops.

    Sequence s has queries q[cu_q[s] .. cu_q[s+1]) and keys/values
    k[cu_k[s] .. cu_k[s+1]); the queries are the last positions of the
    sequence, so local query i is at position (Lk - Lq) + i.  A query with no
    visible key gets a zero row.
    """
    total = len(q)
    d_v = len(v[0][0]) if len(v) else 0
    out = [[[0.0] * d_v for _ in range(n_q_heads)] for _ in range(total)]
    for s in range(len(cu_q) - 1):
        qa, qb = cu_q[s], cu_q[s + 1]
        ka, kb = cu_k[s], cu_k[s + 1]
        for t in range(qa, qb):
            pos = (kb - ka) - (qb - qa) + (t - qa)
            for h in range(n_q_heads):
                g = (h * n_kv_heads) // n_q_heads
                keys = [j for j in range(kb - ka)
                        if j <= pos and not (window and pos - j >= window)]
                if not keys:
                    continue
                scores = []
                for j in keys:
                    acc = 0.0
                    for c in range(len(q[t][h])):
                        acc += q[t][h][c] * k[ka + j][g][c]
                    scores.append(scale * acc)
                top = max(scores)
                weights = [math.exp(x - top) for x in scores]
                z = sum(weights)
                for c in range(d_v):
                    acc = 0.0
                    for wgt, j in zip(weights, keys):
                        acc += wgt * v[ka + j][g][c]
                    out[t][h][c] = acc / z
    return out


def brute_attention_paged(q, k_pool, v_pool, cu_q, block_table, seqlens_k,
                          page_size, n_q_heads, n_kv_heads, scale, window):
    """Paged KV, literal loops: key position j of sequence s is read from
    slot j % page_size of page block_table[s][j // page_size]."""
    total = len(q)
    d_v = len(v_pool[0][0]) if len(v_pool) else 0
    out = [[[0.0] * d_v for _ in range(n_q_heads)] for _ in range(total)]
    for s in range(len(cu_q) - 1):
        qa, qb = cu_q[s], cu_q[s + 1]
        n_k = seqlens_k[s]

        def slot(j):
            return block_table[s][j // page_size] * page_size + j % page_size

        for t in range(qa, qb):
            pos = n_k - (qb - qa) + (t - qa)
            for h in range(n_q_heads):
                g = (h * n_kv_heads) // n_q_heads
                keys = [j for j in range(n_k)
                        if j <= pos and not (window and pos - j >= window)]
                if not keys:
                    continue
                scores = []
                for j in keys:
                    acc = 0.0
                    for c in range(len(q[t][h])):
                        acc += q[t][h][c] * k_pool[slot(j)][g][c]
                    scores.append(scale * acc)
                top = max(scores)
                weights = [math.exp(x - top) for x in scores]
                z = sum(weights)
                for c in range(d_v):
                    acc = 0.0
                    for wgt, j in zip(weights, keys):
                        acc += wgt * v_pool[slot(j)][g][c]
                    out[t][h][c] = acc / z
    return out

"""Pins of the FP64 oracle: checks against facts fixed outside the oracle.

Each ``pin_*`` takes the oracle module (or a deliberately broken copy of it,
see ``test_oracle_mutants.py``) and raises ``AssertionError`` when the module
disagrees with:

* hand-derived closed forms (``golden/worked_examples.json``),
* the literal-loop brute force of ``bruteforce.py`` on tiny random inputs,
* invariants of the definition (rows of P sum to one, W = 0 equals W >= L,
  a one-token sequence returns its own V, W = 1 returns V, scale 0 gives the
  mean of the visible V rows, constant V, convex hull, shift invariance in
  K, packing and GQA replication),
* torch's CPU float64 ``scaled_dot_product_attention`` as a second library
  rendering of the causal case,
* for chunked prefill against a KV history: the literal-loop brute force,
  and the fact that running a sequence chunk by chunk against its growing
  history reproduces the single-pass rows,
* for a paged KV cache: a literal-loop brute force that addresses every key
  through the block table itself, and invariance under a permutation of the
  physical pages.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from bruteforce import (brute_attention, brute_attention_chunked,
                        brute_attention_paged)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "worked_examples.json")


def _cu(lengths):
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + n)
    return cu


def _rand(rng, lengths, hq, hkv, d):
    t = sum(lengths)
    return (rng.standard_normal((t, hq, d)), rng.standard_normal((t, hkv, d)),
            rng.standard_normal((t, hkv, d)))


def pin_golden(mod):
    with open(GOLDEN) as f:
        examples = json.load(f)["examples"]
    for ex in examples:
        if "block_table" in ex:
            got = mod.attention_paged(np.array(ex["q"]), np.array(ex["k"]),
                                      np.array(ex["v"]), ex["cu_seqlens"],
                                      np.array(ex["block_table"]), ex["seqlens_k"],
                                      ex["page_size"], ex["n_q_heads"],
                                      ex["n_kv_heads"], ex["scale"], ex["window"],
                                      workers=1)
        elif "cu_seqlens_k" in ex:
            got = mod.attention_chunked(np.array(ex["q"]), np.array(ex["k"]),
                                        np.array(ex["v"]), ex["cu_seqlens"],
                                        ex["cu_seqlens_k"], ex["n_q_heads"],
                                        ex["n_kv_heads"], ex["scale"],
                                        ex["window"], workers=1)
        else:
            got = mod.attention_varlen(np.array(ex["q"]), np.array(ex["k"]),
                                       np.array(ex["v"]), ex["cu_seqlens"],
                                       ex["n_q_heads"], ex["n_kv_heads"],
                                       ex["scale"], ex["window"], workers=1)
        want = np.array(ex["out"])
        assert got.shape == want.shape, ex["name"]
        err = np.max(np.abs(got - want))
        assert err <= 1e-12, f"{ex['name']}: max err {err}"


BRUTE_CASES = [
    # lengths, hq, hkv, d, window, scale
    ([5], 1, 1, 1, 0, 1.0),
    ([7], 2, 1, 2, 0, 0.7),
    ([9], 4, 2, 4, 2, 0.5),
    ([6, 1, 0, 3], 4, 4, 8, 0, 0.35),
    ([0, 2, 7], 4, 1, 4, 5, 1.3),
    ([11], 2, 2, 3, 1, 0.9),
    ([33], 4, 2, 8, 7, 0.25),
    ([1, 1, 2], 2, 1, 2, 0, -0.8),
    ([12, 5], 4, 2, 2, 12, 0.6),
]


def pin_bruteforce(mod):
    for case_id, (lengths, hq, hkv, d, w, scale) in enumerate(BRUTE_CASES):
        rng = np.random.default_rng(100 + case_id)
        q, k, v = _rand(rng, lengths, hq, hkv, d)
        cu = _cu(lengths)
        want = np.array(brute_attention(q.tolist(), k.tolist(), v.tolist(), cu,
                                        hq, hkv, scale, w)).reshape(q.shape[0], hq, d)
        got = mod.attention_varlen(q, k, v, cu, hq, hkv, scale, w, workers=1)
        err = np.max(np.abs(got - want)) if got.size else 0.0
        assert err <= 1e-12, f"brute case {case_id}: max err {err}"
        rows = [(t, h) for t in range(q.shape[0]) for h in range(hq)]
        if rows:
            got_r = mod.attention_rows(q, k, v, cu, hq, hkv, scale, w, rows)
            want_r = np.array([want[t, h] for t, h in rows])
            err_r = np.max(np.abs(got_r - want_r))
            assert err_r <= 1e-12, f"brute case {case_id} rows: max err {err_r}"


# Separate q/k and v head sizes (the absorbed MLA prefill of the atlas PR #69
# page attends with 320-wide q/k rows and extracts 256-wide values): the
# scores use d_qk columns, the output has d_v columns.  Both d_v < d_qk and
# d_v > d_qk occur, so that neither width can stand in for the other.
BRUTE_CASES_DV = [
    # lengths, hq, hkv, d_qk, d_v, window, scale
    ([5], 1, 1, 5, 3, 0, 0.8),
    ([4, 0, 7], 4, 2, 3, 5, 2, 0.6),
    ([9, 1], 2, 1, 8, 2, 0, -0.4),
    ([6], 4, 1, 2, 7, 4, 1.1),
]

CHUNK_CASES_DV = [
    # (q lengths, kv lengths), hq, hkv, d_qk, d_v, window, scale
    (([2, 3], [6, 3]), 2, 1, 5, 3, 0, 0.7),
    (([1], [8]), 4, 2, 2, 6, 3, 0.5),
]


def pin_bruteforce_split_head_sizes(mod):
    for case_id, (lengths, hq, hkv, dq, dv, w, scale) in enumerate(BRUTE_CASES_DV):
        rng = np.random.default_rng(500 + case_id)
        t = sum(lengths)
        q = rng.standard_normal((t, hq, dq))
        k = rng.standard_normal((t, hkv, dq))
        v = rng.standard_normal((t, hkv, dv))
        cu = _cu(lengths)
        want = np.array(brute_attention(q.tolist(), k.tolist(), v.tolist(), cu,
                                        hq, hkv, scale, w)).reshape(t, hq, dv)
        got = mod.attention_varlen(q, k, v, cu, hq, hkv, scale, w, workers=1)
        assert got.shape == (t, hq, dv), f"dv case {case_id}: shape {got.shape}"
        err = np.max(np.abs(got - want)) if got.size else 0.0
        assert err <= 1e-12, f"dv case {case_id}: max err {err}"
        rows = [(tok, h) for tok in range(t) for h in range(hq)]
        if rows:
            got_r = mod.attention_rows(q, k, v, cu, hq, hkv, scale, w, rows)
            want_r = np.array([want[tok, h] for tok, h in rows])
            assert np.max(np.abs(got_r - want_r)) <= 1e-12, f"dv case {case_id} rows"
    for case_id, ((lq, lk), hq, hkv, dq, dv, w, scale) in enumerate(CHUNK_CASES_DV):
        rng = np.random.default_rng(550 + case_id)
        q = rng.standard_normal((sum(lq), hq, dq))
        k = rng.standard_normal((sum(lk), hkv, dq))
        v = rng.standard_normal((sum(lk), hkv, dv))
        cq, ck = _cu(lq), _cu(lk)
        want = np.array(brute_attention_chunked(
            q.tolist(), k.tolist(), v.tolist(), cq, ck, hq, hkv, scale, w)
        ).reshape(q.shape[0], hq, dv)
        got = mod.attention_chunked(q, k, v, cq, ck, hq, hkv, scale, w, workers=1)
        assert got.shape == want.shape, f"dv chunk case {case_id}: shape {got.shape}"
        assert np.max(np.abs(got - want)) <= 1e-12, f"dv chunk case {case_id}"


def pin_rows_sum_to_one(mod):
    rng = np.random.default_rng(7)
    for n, w in ((1, 0), (17, 0), (40, 3), (40, 40)):
        q = rng.standard_normal((n, 8))
        k = rng.standard_normal((n, 8)) * 3.0
        p = mod.softmax_probs(q, k, 0.9, w)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12
        i = np.arange(n)[:, None]
        j = np.arange(n)[None, :]
        masked = (j > i) | ((w > 0) & (j <= i - w))
        assert np.all(p[masked] == 0.0)
        assert np.all(p[~masked] > 0.0)


def pin_window_zero_equals_long_window(mod):
    rng = np.random.default_rng(8)
    lengths = [23, 9]
    q, k, v = _rand(rng, lengths, 4, 2, 8)
    cu = _cu(lengths)
    o0 = mod.attention_varlen(q, k, v, cu, 4, 2, 0.4, 0, workers=1)
    for w in (23, 24, 1000):
        ow = mod.attention_varlen(q, k, v, cu, 4, 2, 0.4, w, workers=1)
        assert np.array_equal(o0, ow), f"window {w} differs from window 0"


def pin_window_one_returns_v(mod):
    rng = np.random.default_rng(9)
    lengths = [13, 4]
    q, k, v = _rand(rng, lengths, 4, 2, 8)
    out = mod.attention_varlen(q, k, v, _cu(lengths), 4, 2, 1.1, 1, workers=1)
    for h in range(4):
        assert np.array_equal(out[:, h, :], v[:, h // 2, :])


def pin_first_token_returns_v(mod):
    rng = np.random.default_rng(10)
    lengths = [1, 5, 1, 8, 3]
    q, k, v = _rand(rng, lengths, 2, 1, 8)
    cu = _cu(lengths)
    out = mod.attention_varlen(q, k, v, cu, 2, 1, 0.8, 0, workers=1)
    for s in range(len(lengths)):
        for h in range(2):
            assert np.array_equal(out[cu[s], h, :], v[cu[s], 0, :])


def pin_scale_zero_mean(mod):
    rng = np.random.default_rng(11)
    lengths = [19]
    q, k, v = _rand(rng, lengths, 2, 1, 4)
    for w in (0, 4):
        out = mod.attention_varlen(q, k, v, [0, 19], 2, 1, 0.0, w, workers=1)
        for i in range(19):
            lo = 0 if w == 0 else max(0, i - w + 1)
            want = v[lo:i + 1, 0, :].mean(axis=0)
            assert np.max(np.abs(out[i, 0] - want)) <= 1e-12
            assert np.max(np.abs(out[i, 1] - want)) <= 1e-12


def pin_constant_v_and_hull(mod):
    rng = np.random.default_rng(12)
    q, k, _ = _rand(rng, [21], 2, 1, 4)
    row = np.array([0.5, -2.0, 3.25, 1e-3])
    v = np.broadcast_to(row, (21, 1, 4)).copy()
    out = mod.attention_varlen(q, k, v, [0, 21], 2, 1, 1.7, 0, workers=1)
    assert np.max(np.abs(out - row)) <= 1e-12
    v = rng.standard_normal((21, 1, 4))
    out = mod.attention_varlen(q, k, v, [0, 21], 2, 1, 1.7, 5, workers=1)
    for i in range(21):
        vis = v[max(0, i - 4):i + 1, 0, :]
        assert np.all(out[i, 0] <= vis.max(axis=0) + 1e-12)
        assert np.all(out[i, 0] >= vis.min(axis=0) - 1e-12)


def pin_k_shift_invariance(mod):
    rng = np.random.default_rng(13)
    q, k, v = _rand(rng, [25], 2, 1, 8)
    base = mod.attention_varlen(q, k, v, [0, 25], 2, 1, 0.6, 6, workers=1)
    shifted = mod.attention_varlen(q, k + rng.standard_normal(8), v, [0, 25],
                                   2, 1, 0.6, 6, workers=1)
    assert np.max(np.abs(base - shifted)) <= 1e-11


def pin_packing_equals_separate(mod):
    rng = np.random.default_rng(14)
    lengths = [7, 0, 12, 1, 5]
    q, k, v = _rand(rng, lengths, 4, 2, 8)
    cu = _cu(lengths)
    packed = mod.attention_varlen(q, k, v, cu, 4, 2, 0.45, 3, workers=1)
    for s, n in enumerate(lengths):
        a, b = cu[s], cu[s + 1]
        alone = mod.attention_varlen(q[a:b], k[a:b], v[a:b], [0, n], 4, 2,
                                     0.45, 3, workers=1)
        assert np.max(np.abs(packed[a:b] - alone), initial=0.0) <= 1e-12


def pin_gqa_equals_replicated(mod):
    rng = np.random.default_rng(15)
    lengths = [10, 6]
    q, k, v = _rand(rng, lengths, 6, 2, 4)
    cu = _cu(lengths)
    gqa = mod.attention_varlen(q, k, v, cu, 6, 2, 0.5, 0, workers=1)
    k_rep = np.repeat(k, 3, axis=1)  # head h reads kv head h // 3
    v_rep = np.repeat(v, 3, axis=1)
    mha = mod.attention_varlen(q, k_rep, v_rep, cu, 6, 6, 0.5, 0, workers=1)
    assert np.max(np.abs(gqa - mha)) <= 1e-12


def pin_sdpa_crosscheck(mod):
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(16)
    n, hq, hkv, d = 37, 4, 1, 16
    q, k, v = _rand(rng, [n], hq, hkv, d)
    scale = 1.0 / math.sqrt(d)
    qt = torch.from_numpy(q).permute(1, 0, 2)  # [H, L, d]
    kt = torch.from_numpy(np.repeat(k, hq, axis=1)).permute(1, 0, 2)
    vt = torch.from_numpy(np.repeat(v, hq, axis=1)).permute(1, 0, 2)
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                         scale=scale).permute(1, 0, 2).numpy()
    got = mod.attention_varlen(q, k, v, [0, n], hq, hkv, scale, 0, workers=1)
    assert np.max(np.abs(got - ref)) <= 1e-12
    w = 5
    i = torch.arange(n)[:, None]
    j = torch.arange(n)[None, :]
    mask = (j <= i) & (j >= i - w + 1)
    ref_w = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                           scale=scale).permute(1, 0, 2).numpy()
    got_w = mod.attention_varlen(q, k, v, [0, n], hq, hkv, scale, w, workers=1)
    assert np.max(np.abs(got_w - ref_w)) <= 1e-12


def pin_parallel_equals_serial(mod):
    rng = np.random.default_rng(17)
    lengths = [30, 17, 0, 41]
    q, k, v = _rand(rng, lengths, 4, 1, 8)
    cu = _cu(lengths)
    a = mod.attention_varlen(q, k, v, cu, 4, 1, 0.3, 0, workers=1)
    b = mod.attention_varlen(q, k, v, cu, 4, 1, 0.3, 0, workers=4)
    assert np.array_equal(a, b)


CHUNK_CASES = [
    # (q lengths, kv lengths), hq, hkv, d, window, scale
    (([1], [6]), 1, 1, 2, 0, 0.8),
    (([3], [8]), 2, 1, 3, 0, 0.6),
    (([4], [4]), 2, 2, 2, 0, 0.9),
    (([2, 0, 5], [7, 3, 5]), 4, 2, 4, 3, 0.5),
    (([5, 1], [12, 1]), 2, 1, 2, 4, -0.7),
    (([6], [15]), 4, 1, 8, 1, 0.3),
    (([1, 2, 3], [9, 2, 10]), 4, 4, 2, 0, 1.1),
]


def _rand_chunked(rng, q_lengths, kv_lengths, hq, hkv, d):
    return (rng.standard_normal((sum(q_lengths), hq, d)),
            rng.standard_normal((sum(kv_lengths), hkv, d)),
            rng.standard_normal((sum(kv_lengths), hkv, d)))


def pin_chunked_bruteforce(mod):
    for case_id, ((lq, lk), hq, hkv, d, w, scale) in enumerate(CHUNK_CASES):
        rng = np.random.default_rng(300 + case_id)
        q, k, v = _rand_chunked(rng, lq, lk, hq, hkv, d)
        cq, ck = _cu(lq), _cu(lk)
        want = np.array(brute_attention_chunked(
            q.tolist(), k.tolist(), v.tolist(), cq, ck, hq, hkv, scale, w)
        ).reshape(q.shape[0], hq, d)
        got = mod.attention_chunked(q, k, v, cq, ck, hq, hkv, scale, w, workers=1)
        err = np.max(np.abs(got - want)) if got.size else 0.0
        assert err <= 1e-12, f"chunk case {case_id}: max err {err}"
        rows = [(t, h) for t in range(q.shape[0]) for h in range(hq)]
        if rows:
            got_r = mod.attention_rows(q, k, v, cq, hq, hkv, scale, w, rows,
                                       cu_seqlens_k=ck)
            want_r = np.array([want[t, h] for t, h in rows])
            assert np.max(np.abs(got_r - want_r)) <= 1e-12, f"chunk case {case_id} rows"


def pin_chunks_reproduce_single_pass(mod):
    # A sequence prefilled chunk by chunk, each chunk attending to the whole
    # history before it, gives the rows of the single-pass prefill.
    rng = np.random.default_rng(31)
    n, hq, hkv, d = 57, 4, 2, 8
    q, k, v = _rand(rng, [n], hq, hkv, d)
    for w in (0, 5, 200):
        full = mod.attention_varlen(q, k, v, [0, n], hq, hkv, 0.45, w, workers=1)
        bounds = [0, 1, 9, 10, 33, 57]
        for a, b in zip(bounds[:-1], bounds[1:]):
            got = mod.attention_chunked(q[a:b], k[:b], v[:b], [0, b - a], [0, b],
                                        hq, hkv, 0.45, w, workers=1)
            assert np.max(np.abs(got - full[a:b])) <= 1e-12, (w, a, b)
        # the same chunks packed as one batch of three "sequences"
        cq = [0, 9, 33, 57]
        ck = [0, 9, 9 + 33, 9 + 33 + 57]
        kk = np.concatenate([k[:9], k[:33], k[:57]])
        vv = np.concatenate([v[:9], v[:33], v[:57]])
        qq = np.concatenate([q[0:9], q[9:33], q[33:57]])
        got = mod.attention_chunked(qq, kk, vv, cq, ck, hq, hkv, 0.45, w, workers=1)
        assert np.max(np.abs(got - full)) <= 1e-12, w


PAGED_CASES = [
    # q lengths, kv lengths, page_size, hq, hkv, d, window, scale
    ([1], [5], 2, 1, 1, 2, 0, 0.8),
    ([3, 2], [7, 2], 4, 2, 1, 3, 0, 0.6),
    ([4, 0, 6], [9, 3, 6], 3, 4, 2, 2, 2, -0.5),
    ([8], [8], 8, 2, 2, 2, 3, 1.2),
]


def _paged_case(rng, lq, lk, page, hq, hkv, d):
    n_pages = sum((n + page - 1) // page for n in lk) + 3  # spare pages
    width = max(1, max((n + page - 1) // page for n in lk))
    perm = rng.permutation(n_pages)
    table = np.zeros((len(lk), width), dtype=np.int64)
    used = 0
    for s, n in enumerate(lk):
        for b in range((n + page - 1) // page):
            table[s, b] = perm[used]
            used += 1
    q = rng.standard_normal((sum(lq), hq, d))
    kp = rng.standard_normal((n_pages * page, hkv, d))
    vp = rng.standard_normal((n_pages * page, hkv, d))
    return q, kp, vp, table


def pin_paged_bruteforce(mod):
    for case_id, (lq, lk, page, hq, hkv, d, w, scale) in enumerate(PAGED_CASES):
        rng = np.random.default_rng(400 + case_id)
        q, kp, vp, table = _paged_case(rng, lq, lk, page, hq, hkv, d)
        cq = _cu(lq)
        want = np.array(brute_attention_paged(
            q.tolist(), kp.tolist(), vp.tolist(), cq, table.tolist(), lk, page, hq,
            hkv, scale, w)).reshape(q.shape[0], hq, d)
        got = mod.attention_paged(q, kp, vp, cq, table, lk, page, hq, hkv, scale, w,
                                  workers=1)
        err = np.max(np.abs(got - want)) if got.size else 0.0
        assert err <= 1e-12, f"paged case {case_id}: max err {err}"


def pin_paged_page_permutation_invariance(mod):
    # moving the pages and rewriting the table to match changes nothing
    rng = np.random.default_rng(41)
    lq, lk, page, hq, hkv, d = [5, 9], [13, 9], 4, 4, 2, 8
    q, kp, vp, table = _paged_case(rng, lq, lk, page, hq, hkv, d)
    a = mod.attention_paged(q, kp, vp, _cu(lq), table, lk, page, hq, hkv, 0.4, 0,
                            workers=1)
    n_pages = kp.shape[0] // page
    perm = rng.permutation(n_pages)  # new page of old page p is perm[p]
    kp2 = np.zeros_like(kp)
    vp2 = np.zeros_like(vp)
    for old in range(n_pages):
        kp2[perm[old] * page:(perm[old] + 1) * page] = kp[old * page:(old + 1) * page]
        vp2[perm[old] * page:(perm[old] + 1) * page] = vp[old * page:(old + 1) * page]
    b = mod.attention_paged(q, kp2, vp2, _cu(lq), perm[table], lk, page, hq, hkv,
                            0.4, 0, workers=1)
    assert np.max(np.abs(a - b)) <= 1e-12


def pin_decode_is_the_last_prefill_row(mod):
    # decoding the token after a prefix gives the single-pass prefill row of
    # that token (query at the last position sees every earlier key)
    rng = np.random.default_rng(51)
    lengths, hq, hkv, d = [1, 6, 23, 40], 8, 2, 8
    q, k, v = _rand(rng, lengths, hq, hkv, d)
    cu = _cu(lengths)
    for w in (0, 1, 5):
        full = mod.attention_varlen(q, k, v, cu, hq, hkv, 0.6, w, workers=1)
        last = [cu[s + 1] - 1 for s in range(len(lengths))]
        got = mod.attention_decode(q[last], k, v, cu, hq, hkv, 0.6, w, workers=1)
        assert np.max(np.abs(got - full[last])) <= 1e-12, w


ALL_PINS = [
    pin_golden,
    pin_bruteforce,
    pin_bruteforce_split_head_sizes,
    pin_rows_sum_to_one,
    pin_window_zero_equals_long_window,
    pin_window_one_returns_v,
    pin_first_token_returns_v,
    pin_scale_zero_mean,
    pin_constant_v_and_hull,
    pin_k_shift_invariance,
    pin_packing_equals_separate,
    pin_gqa_equals_replicated,
    pin_sdpa_crosscheck,
    pin_parallel_equals_serial,
    pin_chunked_bruteforce,
    pin_chunks_reproduce_single_pass,
    pin_paged_bruteforce,
    pin_paged_page_permutation_invariance,
    pin_decode_is_the_last_prefill_row,
]

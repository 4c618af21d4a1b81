"""The pins are strong enough: planted mistakes in a copy of the oracle fail.

Each mutant is a private copy of ``oracle/attention.py`` with one plausible
mistake (a wrong mask index, a dropped term, a transposed operand, a wrong
head map...).  The real oracle passes every pin (``test_oracle.py``); each
mutant must fail at least one.  The pristine copy is run through the same
harness first so that a harness that catches nothing cannot score.
"""
import importlib.util
import os

import numpy as np
import pytest

from oracle_pins import ALL_PINS

ORACLE_PATH = os.path.join(os.path.dirname(os.path.dirname(
    os.path.abspath(__file__))), "oracle", "attention.py")


def fresh_copy(tag):
    spec = importlib.util.spec_from_file_location(f"_oracle_copy_{tag}", ORACLE_PATH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def failing_pins(mod):
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except AssertionError:
            failed.append(pin.__name__)
        except Exception as e:  # a crash also counts as caught
            failed.append(f"{pin.__name__}:{type(e).__name__}")
    return failed


def _vis(op):
    def visibility(n_rows, n_cols, window, q_offset=0):
        i = q_offset + np.arange(n_rows)[:, None]
        j = np.arange(n_cols)[None, :]
        return op(i, j, window)
    return visibility


def _probs(variant):
    def softmax_probs(q_h, k_g, scale, window, q_offset=None, *, _v=variant):
        q_h = np.asarray(q_h, dtype=np.float64)
        k_g = np.asarray(k_g, dtype=np.float64)
        n, nk = q_h.shape[0], k_g.shape[0]
        if q_offset is None:
            q_offset = nk - n
        if _v == "history_ignored":
            q_offset = 0
        elif _v == "history_offset_plus_one":
            q_offset = q_offset + 1 if nk > n else q_offset
        vis = MUT_VIS_BASE(n, nk, window, q_offset)
        if _v == "transposed":
            s = scale * (k_g @ q_h.T)
        elif _v == "no_scale":
            s = q_h @ k_g.T
        elif _v == "neg_scale":
            s = -scale * (q_h @ k_g.T)
        else:
            s = scale * (q_h @ k_g.T)
        if _v == "mask_as_zero":
            s = np.where(vis, s, 0.0)
        else:
            s = np.where(vis, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        m = np.where(np.isfinite(m), m, 0.0)
        e = np.exp(s - m)
        if _v == "no_normalise":
            return e
        if _v == "normalise_columns":
            return e / e.sum(axis=0, keepdims=True)
        z = e.sum(axis=1, keepdims=True)
        return e / np.where(z > 0, z, 1.0)
    return softmax_probs


def MUT_VIS_BASE(n_rows, n_cols, window, q_offset=0):
    i = q_offset + np.arange(n_rows)[:, None]
    j = np.arange(n_cols)[None, :]
    vis = j <= i
    if window > 0:
        vis &= j >= i - window + 1
    return vis


def _no_isolation(mod):
    base = mod.attention_varlen

    def attention_varlen(q, k, v, cu_seqlens, hq, hkv, scale, window, workers=None):
        cu = [int(x) for x in np.asarray(cu_seqlens).reshape(-1)]
        return base(q, k, v, [0, cu[-1]], hq, hkv, scale, window, workers=workers)
    return attention_varlen


def _chunk_keys_only(mod):
    base = mod.attention_chunked

    def attention_chunked(q, k, v, cu_q, cu_k, hq, hkv, scale, window, workers=None):
        # keeps only the chunk's own keys: the last Lq of each sequence
        cq = [int(x) for x in np.asarray(cu_q).reshape(-1)]
        ck = [int(x) for x in np.asarray(cu_k).reshape(-1)]
        idx = []
        for s in range(len(cq) - 1):
            lq = cq[s + 1] - cq[s]
            idx.extend(range(ck[s + 1] - lq, ck[s + 1]))
        k2 = np.asarray(k)[idx]
        v2 = np.asarray(v)[idx]
        return base(q, k2, v2, cq, cq, hq, hkv, scale, window, workers=workers)
    return attention_chunked


def _paged_wrong_slot(mod):
    # reads key j from the page of logical block j // page_size but ignores
    # the table (physical page = logical page of sequence 0)
    def gather_pages(pool, block_table, seqlens_k, page_size):
        pool = np.asarray(pool, dtype=np.float64)
        lens = [int(x) for x in np.asarray(seqlens_k).reshape(-1)]
        parts, cu = [], [0]
        for s, n in enumerate(lens):
            parts.append(pool[np.arange(n)])
            cu.append(cu[-1] + n)
        return np.concatenate(parts), cu
    return gather_pages


def _paged_slot_transposed(mod):
    # swaps the roles of page and slot: page j % page_size, slot j // page_size
    def gather_pages(pool, block_table, seqlens_k, page_size):
        pool = np.asarray(pool, dtype=np.float64)
        table = np.asarray(block_table, dtype=np.int64)
        lens = [int(x) for x in np.asarray(seqlens_k).reshape(-1)]
        parts, cu = [], [0]
        for s, n in enumerate(lens):
            pos = np.arange(n)
            blk = np.minimum(pos % page_size, table.shape[1] - 1)
            slots = table[s, blk] * page_size + np.minimum(pos // page_size, page_size - 1)
            parts.append(pool[slots])
            cu.append(cu[-1] + n)
        return np.concatenate(parts), cu
    return gather_pages


def _values_cut_to_qk_width(mod):
    # forms P . V with only as many value columns as q/k have (the head size
    # of q taken for v's as well), zero beyond
    base = mod.attention_head

    def attention_head(q_h, k_g, v_g, scale, window, q_offset=None):
        v = np.array(v_g, dtype=np.float64)
        dq = np.shape(q_h)[1]
        v[:, dq:] = 0.0
        return base(q_h, k_g, v, scale, window, q_offset)
    return attention_head


def _scores_over_value_width(mod):
    # forms the scores over the first d_v columns of q and k (the head size
    # of v taken for q/k's as well)
    base = mod.attention_head

    def attention_head(q_h, k_g, v_g, scale, window, q_offset=None):
        dv = np.shape(v_g)[1]
        q = np.asarray(q_h, dtype=np.float64)[:, :dv]
        k = np.asarray(k_g, dtype=np.float64)[:, :dv]
        return base(q, k, v_g, scale, window, q_offset)
    return attention_head


MUTANTS = {
    "causal_excludes_self": ("visibility", _vis(
        lambda i, j, w: (j < i) | ((i == 0) & (j == 0)) if w == 0 else
        (j < i) & (j >= i - w + 1) | ((i == 0) & (j == 0)))),
    "causal_lookahead_one": ("visibility", _vis(
        lambda i, j, w: (j <= i + 1) & ((w == 0) | (j >= i - w + 1)))),
    "window_one_too_wide": ("visibility", _vis(
        lambda i, j, w: (j <= i) & ((w == 0) | (j >= i - w)))),
    "window_one_too_narrow": ("visibility", _vis(
        lambda i, j, w: (j <= i) & ((w == 0) | (j >= i - w + 2) | (j == i)))),
    "no_mask": ("visibility", _vis(lambda i, j, w: np.ones_like(i + j, dtype=bool))),
    "kv_head_modulo": ("kv_head_of", lambda h, hq, hkv: h % hkv),
    "kv_head_zero": ("kv_head_of", lambda h, hq, hkv: 0),
    "scores_transposed": ("softmax_probs", _probs("transposed")),
    "scale_dropped": ("softmax_probs", _probs("no_scale")),
    "scale_sign_flipped": ("softmax_probs", _probs("neg_scale")),
    "masked_scores_zero_not_neg_inf": ("softmax_probs", _probs("mask_as_zero")),
    "softmax_not_normalised": ("softmax_probs", _probs("no_normalise")),
    "softmax_normalised_over_queries": ("softmax_probs", _probs("normalise_columns")),
    "sequences_not_isolated": ("attention_varlen", None),
    "history_ignored": ("softmax_probs", _probs("history_ignored")),
    "history_offset_plus_one": ("softmax_probs", _probs("history_offset_plus_one")),
    "chunk_sees_only_its_own_keys": ("attention_chunked", None),
    "paged_table_ignored": ("gather_pages", None),
    "paged_page_and_slot_swapped": ("gather_pages", None),
    "values_cut_to_qk_width": ("attention_head", None),
    "scores_over_value_width": ("attention_head", None),
}


def test_pristine_copy_passes_every_pin():
    assert failing_pins(fresh_copy("pristine")) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = fresh_copy(name)
    attr, repl = MUTANTS[name]
    if name == "sequences_not_isolated":
        repl = _no_isolation(mod)
    if name == "chunk_sees_only_its_own_keys":
        repl = _chunk_keys_only(mod)
    if name == "paged_table_ignored":
        repl = _paged_wrong_slot(mod)
    if name == "paged_page_and_slot_swapped":
        repl = _paged_slot_transposed(mod)
    if name == "values_cut_to_qk_width":
        repl = _values_cut_to_qk_width(mod)
    if name == "scores_over_value_width":
        repl = _scores_over_value_width(mod)
    setattr(mod, attr, repl)
    assert failing_pins(mod), f"mutant {name} passed every pin"

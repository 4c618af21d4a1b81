"""Seeded generators and the work counter (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle
from causal_prefill_attention_amd import measure, workloads

VARLEN = "varlen16_gqa32q8kv_fp32q_fp16kv"


def test_varlen_lengths_are_seeded_and_in_range():
    w = workloads.WORKLOADS[VARLEN]
    a = workloads.draw_lengths(w, np.random.default_rng(w.seed))
    b = workloads.draw_lengths(w, np.random.default_rng(w.seed))
    assert a == b and len(a) == 16
    assert all(64 <= n <= 2048 for n in a)
    assert a == [1674, 234, 420, 534, 424, 1654, 1789, 1219, 142, 250, 723,
                 923, 1297, 1014, 589, 381]


def test_make_inputs_deterministic_and_typed():
    w = workloads.custom("t", [5, 0, 9], 4, 2, head_dim=16, q_dtype="fp32",
                         kv_dtype="fp16", seed=3)
    a = workloads.make_inputs(w)
    b = workloads.make_inputs(w)
    assert a["sha256"] == b["sha256"]
    assert a["q"].dtype == torch.float32 and a["k"].dtype == torch.float16
    assert tuple(a["q"].shape) == (14, 4, 16)
    assert tuple(a["k"].shape) == (14, 2, 16)
    assert a["cu_seqlens"].tolist() == [0, 5, 5, 14]
    assert a["cu_seqlens"].dtype == torch.int32


def test_outlier_count():
    w = workloads.custom("o", [64], 4, 1, head_dim=128, seed=4,
                         k_outlier_frac=0.01)
    base = workloads.custom("b", [64], 4, 1, head_dim=128, seed=4)
    k1 = workloads.make_inputs(w)["k"].float()
    k0 = workloads.make_inputs(base)["k"].float()
    changed = (k1 != k0).sum().item()
    n = math.floor(0.01 * k0.numel())
    # scaling by 30 can leave a value unchanged only if it was zero
    assert changed == n


def test_outlier_channels_scale_whole_columns():
    w = workloads.custom("oc", [50], 4, 2, head_dim=128, seed=6, k_outlier_channels=1)
    base = workloads.custom("b", [50], 4, 2, head_dim=128, seed=6)
    k1 = workloads.make_inputs(w)["k"].double()
    k0 = workloads.make_inputs(base)["k"].double()
    assert torch.equal(workloads.make_inputs(w)["q"], workloads.make_inputs(base)["q"])
    for g in range(2):
        cols = [c for c in range(128) if not torch.equal(k1[:, g, c], k0[:, g, c])]
        assert len(cols) == 1, cols
        c = cols[0]
        # x30 in float64 before the bf16 cast: compare after the same cast
        want = (k0[:, g, c] * 30).to(torch.bfloat16).double()
        assert torch.allclose(k1[:, g, c], want, rtol=2 ** -7)
    full = workloads.WORKLOADS["long_8192tok_32q1kv_outlier_channel"]
    assert full.k_outlier_channels == round(0.01 * 128) == 1


@pytest.mark.parametrize("n,w", [(0, 0), (1, 0), (5, 0), (5, 1), (5, 3),
                                 (5, 5), (5, 9), (64, 17), (130, 64)])
def test_pair_count_closed_form_matches_brute_count(n, w):
    assert measure.visible_pairs_one(n, w) == oracle.visible_pairs([n], w)


def test_headline_flops():
    w = workloads.WORKLOADS[workloads.HEADLINE]
    f = measure.causal_flops(list(w.lengths), w.n_q_heads, w.head_dim, w.window)
    assert f == 4 * 128 * 32 * (8192 * 8193 // 2)
    assert abs(f - 5.498e11) / 5.498e11 < 1e-3


def test_sample_rows_cover_edges():
    rows = workloads.sample_rows([3, 0, 5], 4, 20, seed=1)
    for r in [(0, 0), (0, 3), (2, 0), (3, 0), (7, 0), (7, 3)]:
        assert r in rows
    assert all(0 <= t < 8 and 0 <= h < 4 for t, h in rows)


@pytest.mark.parametrize("nq,nk,w", [(0, 5, 0), (1, 1, 0), (1, 9, 0), (3, 9, 0),
                                     (9, 9, 3), (4, 20, 5), (20, 20, 0),
                                     (7, 100, 1), (64, 200, 64), (5, 3, 0)])
def test_history_pair_count_matches_brute_count(nq, nk, w):
    assert (measure.visible_pairs_history(nq, nk, w)
            == oracle.visible_pairs([nk], w, q_lengths=[nq]))


def test_chunked_workload_shapes_and_prefix_draws():
    w = workloads.WORKLOADS["chunks8_gqa32q8kv_history"]
    inp = workloads.make_inputs(w)
    tq = sum(w.lengths)
    tk = sum(h + n for h, n in zip(w.history, w.lengths))
    assert inp["q"].shape == (tq, 32, 128)
    assert inp["k"].shape == (tk, 8, 128) and inp["v"].shape == (tk, 8, 128)
    assert inp["cu_seqlens_k"].tolist()[-1] == tk
    assert inp["kv_lengths"] == [h + n for h, n in zip(w.history, w.lengths)]
    # without a history the draws are the plain workload's
    plain = workloads.custom("p", [5, 7], 4, 1, seed=9)
    hist0 = workloads.custom("p", [5, 7], 4, 1, seed=9, history=[0, 0])
    a, b = workloads.make_inputs(plain), workloads.make_inputs(hist0)
    assert torch.equal(a["q"], b["q"]) and torch.equal(a["k"], b["k"])
    assert b["cu_seqlens_k"].tolist() == a["cu_seqlens"].tolist()


def test_chunked_headline_shape_flops():
    w = workloads.WORKLOADS["chunk2048_hist6144_32q1kv_outliers"]
    f = measure.causal_flops(list(w.lengths), w.n_q_heads, w.head_dim, w.window,
                             kv_lengths=[8192])
    # positions 6144..8191 see p + 1 keys each
    assert f == 4 * 128 * 32 * sum(p + 1 for p in range(6144, 8192))

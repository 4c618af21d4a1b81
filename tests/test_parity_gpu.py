"""Parity of the HIP kernel (through the C ABI) with the FP64 oracle.

Bar (on the bf16 outputs, against the unrounded float64 oracle):
    max |gpu - oracle| <= 2e-2   and   mean |gpu - oracle| <= 2e-3
Every comparison prints the fraction of each bar it used.

Sizes: the five problem shapes (128 and 2048 tokens, the 4096-token window,
the packed fp32-Q / fp16-KV GQA batch, the 8192-token long prefill with K
outlier entries, and the same with a whole outlier channel) are compared
element by element on every output; so are smaller ragged and packed
cases.  Every full-size workload is also compared on a seeded sample of
(token, head) rows that the oracle evaluates one by one, from the same
launch configuration the benchmark times.
"""
import json
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from causal_prefill_attention_amd import binding, workloads

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
LOG = os.environ.get("ATTN_PARITY_LOG")


def _oracle_threads():
    """Oracle worker threads: the CPUs this process may use, at most 16
    (each full-size job holds a few GB of float64 temporaries)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _announce(msg):
    sys.stdout.write(f"\n[case] {msg}\n")
    sys.stdout.flush()


def _record(name, max_err, mean_err, n):
    line = {"case": name, "max_abs": max_err, "mean_abs": mean_err,
            "max_frac": max_err / MAX_ABS, "mean_frac": mean_err / MEAN_ABS,
            "elements": n}
    sys.stdout.write(f"[parity] {json.dumps(line)}\n")
    sys.stdout.flush()
    if LOG:
        with open(LOG, "a") as f:
            f.write(json.dumps(line) + "\n")


def check(name, got, want):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == want.shape
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = np.abs(got - want)
    max_err = float(err.max()) if err.size else 0.0
    mean_err = float(err.mean()) if err.size else 0.0
    _record(name, max_err, mean_err, int(err.size))
    assert max_err <= MAX_ABS, f"{name}: max abs {max_err}"
    assert mean_err <= MEAN_ABS, f"{name}: mean abs {mean_err}"


def run_gpu(inp, hq, hkv, d, scale, window, out=None):
    """One launch through the C ABI; inputs with a KV history go through
    attn_prefill_chunked."""
    dev = torch.device("cuda:0")
    q = inp["q"].to(dev)
    k = inp["k"].to(dev)
    v = inp["v"].to(dev)
    cu = inp["cu_seqlens"].to(dev)
    if out is None:
        out = torch.empty(q.shape[0], hq, d, dtype=torch.bfloat16, device=dev)
    if inp.get("head_dim_v"):
        out = torch.empty(q.shape[0], hq, inp["head_dim_v"], dtype=torch.bfloat16, device=dev)
        binding.attn_prefill_ex(q, k, v, out, cu, hq, hkv, d, inp["head_dim_v"], scale, window,
                                cu_seqlens_k=inp["cu_seqlens_k"].to(dev)
                                if "cu_seqlens_k" in inp else None)
    elif inp.get("decode"):
        binding.attn_decode(q, k, v, out, inp["cu_seqlens_k"].to(dev), hq, hkv, d, scale,
                            window)
    elif "cu_seqlens_k" in inp:
        binding.attn_prefill_chunked(q, k, v, out, cu, inp["cu_seqlens_k"].to(dev),
                                     hq, hkv, d, scale, window)
    else:
        binding.attn_prefill(q, k, v, out, cu, hq, hkv, d, scale, window)
    torch.cuda.synchronize()
    return out


def oracle_of(inp, hq, hkv, scale, window):
    if "cu_seqlens_k" in inp:
        return oracle.attention_chunked(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"],
                                        inp["cu_seqlens_k"], hq, hkv, scale, window)
    return oracle.attention_varlen(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"],
                                   hq, hkv, scale, window)


def to64(t):
    return t.detach().cpu().to(torch.float64).numpy()


# ------------------------------------------------------- full-oracle parity
FULL = [
    # name, lengths, hq, hkv, window, q dtype, kv dtype, scale
    ("causal_128tok_4q1kv", None, 0, 0, 0, None, None, None),
    ("mla_2048tok_32q1kv", None, 0, 0, 0, None, None, None),
    ("window1024_4096tok_32q1kv", None, 0, 0, 0, None, None, None),
    ("varlen16_gqa32q8kv_fp32q_fp16kv", None, 0, 0, 0, None, None, None),
    ("long_8192tok_32q1kv_outliers", None, 0, 0, 0, None, None, None),
    ("long_8192tok_32q1kv_outlier_channel", None, 0, 0, 0, None, None, None),
    ("window256_1100tok_32q1kv", [1100], 32, 1, 256, "bf16", "bf16", None),
    ("varlen_gqa_fp32q_fp16kv_small", [300, 64, 1, 0, 517, 129], 32, 8, 0,
     "fp32", "fp16", None),
    ("outliers_1500tok_8q1kv", [1500], 8, 1, 0, "bf16", "bf16", None),
]


@pytest.mark.parametrize("case", FULL, ids=[c[0] for c in FULL])
def test_full_parity(case):
    name, lengths, hq, hkv, window, qd, kvd, scale = case
    if lengths is None:
        w = workloads.WORKLOADS[name]
    else:
        w = workloads.custom(name, lengths, hq, hkv, window=window, q_dtype=qd,
                             kv_dtype=kvd, seed=21,
                             k_outlier_frac=0.01 if "outliers" in name else 0.0,
                             scale=scale)
    _announce(f"{name} lengths={w.lengths or w.random_lengths} hq={w.n_q_heads} "
              f"hkv={w.n_kv_heads} W={w.window} q={w.q_dtype} kv={w.kv_dtype}")
    inp = workloads.make_inputs(w)
    out = run_gpu(inp, w.n_q_heads, w.n_kv_heads, w.head_dim, w.attn_scale, w.window)
    want = oracle.attention_varlen(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"],
                                   w.n_q_heads, w.n_kv_heads, w.attn_scale, w.window,
                                   workers=_oracle_threads())
    check(name, to64(out), want)


# ---------------------------------------------- small-shape grid (packed)
GRID_LENGTHS = [1, 2, 63, 64, 65, 127, 128, 129, 257, 0, 1, 200]
GRID_WINDOWS = [0, 1, 2, 63, 64, 65, 127, 128, 129, 256, 257, 258]
# (query heads, KV heads): groups of 1, 2 and 6 run one head per workgroup;
# groups of 4, 8, 12 and 32 run four heads of a KV head per workgroup
GRID_HEADS = [(1, 1), (4, 1), (32, 1), (8, 8), (32, 8), (12, 1), (16, 2), (6, 3)]
GRID_SCALES = [1 / math.sqrt(128), 0.0, 1.0, -0.3]


@pytest.mark.parametrize("hq,hkv", GRID_HEADS)
@pytest.mark.parametrize("scale", GRID_SCALES)
def test_grid_windows_packed(hq, hkv, scale):
    """All windows over one packed batch of ragged lengths per launch."""
    w = workloads.custom("grid", GRID_LENGTHS, hq, hkv, seed=5 + hq + hkv)
    inp = workloads.make_inputs(w)
    for window in GRID_WINDOWS:
        name = f"grid_h{hq}x{hkv}_s{scale:.3f}_w{window}"
        _announce(name)
        out = run_gpu(inp, hq, hkv, 128, scale, window)
        want = oracle.attention_varlen(inp["q"], inp["k"], inp["v"],
                                       inp["cu_seqlens"], hq, hkv, scale, window)
        check(name, to64(out), want)


@pytest.mark.parametrize("qd,kvd", [("bf16", "fp16"), ("fp32", "bf16"), ("fp32", "fp16")])
def test_dtype_variants(qd, kvd):
    w = workloads.custom(f"dt_{qd}_{kvd}", [190, 33, 260], 8, 2, q_dtype=qd,
                         kv_dtype=kvd, seed=31)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    for window in (0, 70):
        out = run_gpu(inp, 8, 2, 128, w.attn_scale, window)
        want = oracle.attention_varlen(inp["q"], inp["k"], inp["v"],
                                       inp["cu_seqlens"], 8, 2, w.attn_scale, window)
        check(f"{w.name}_w{window}", to64(out), want)


@pytest.mark.parametrize("kvd", ["bf16", "fp16"])
@pytest.mark.parametrize("trend", ["rising", "falling"])
def test_score_trends_through_the_lazy_reference(kvd, trend):
    """Scores that rise by about 35 log2 units per 64-key tile make every
    tile's probabilities overflow the lazy reference's cap (2^32 for bf16,
    2^15 for fp16 operands), so the running max moves on every tile; scores
    that fall as steeply leave every later tile's probabilities far below
    the first tile's, down to exact zeros.  Both against the float64
    oracle, with random V and two query-head signs per KV head."""
    T, hq, hkv, d = 700, 4, 1, 128
    w = workloads.custom(f"trend_{trend}_{kvd}", [T], hq, hkv, kv_dtype=kvd, seed=66)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    # s[i, j] = q[i] . k[j] = sign * 4.1 * j (raw units; scale 1/sqrt(128)
    # makes that 0.52 log2 units per key)
    slope = 4.1 if trend == "rising" else -4.1
    j = torch.arange(T, dtype=torch.float64)
    k = (slope * j / d)[:, None, None].expand(T, hkv, d).clone()
    signs = torch.tensor([1.0, 1.0, -1.0, -1.0], dtype=torch.float64)
    q = signs[None, :, None].expand(T, hq, d).clone()
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[kvd]
    inp = dict(inp, q=q.to(torch.bfloat16), k=k.to(dt))
    out = run_gpu(inp, hq, hkv, d, w.attn_scale, 0)
    check(w.name, to64(out), oracle_of(inp, hq, hkv, w.attn_scale, 0))


@pytest.mark.parametrize("qd", ["bf16", "fp32"])
def test_fp16_kv_with_unit_scale(qd):
    """fp16 K/V at scale 1: scores of about ±11 raw units (±16 log2 units)
    move the fp16 operands' lazy reference (cap 2^15) on many tiles."""
    w = workloads.custom(f"fp16_scale1_{qd}", [300, 77, 1, 130], 8, 2, q_dtype=qd,
                         kv_dtype="fp16", seed=67, scale=1.0)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    for window in (0, 100):
        out = run_gpu(inp, 8, 2, 128, w.attn_scale, window)
        check(f"{w.name}_w{window}", to64(out), oracle_of(inp, 8, 2, w.attn_scale, window))


def test_window_one_returns_v_exactly_rounded():
    """W = 1: every query sees only itself, so out = bf16(v) exactly."""
    w = workloads.custom("w1", [300, 5], 4, 2, seed=41)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    out = run_gpu(inp, 4, 2, 128, w.attn_scale, 1).cpu()
    for h in range(4):
        assert torch.equal(out[:, h, :], inp["v"][:, h // 2, :])


def test_first_token_of_each_sequence_is_its_v():
    w = workloads.custom("first", [1, 130, 1, 64, 257], 4, 1, seed=42)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    out = run_gpu(inp, 4, 1, 128, w.attn_scale, 0).cpu()
    cu = inp["cu_seqlens"].tolist()
    for s in range(len(cu) - 1):
        for h in range(4):
            assert torch.equal(out[cu[s], h], inp["v"][cu[s], 0])


# ------------------------------------------------- layouts and memory safety
def test_strided_inputs_with_nan_gaps_and_output_canaries():
    """Q/K/V are views into larger buffers whose gaps hold NaN; out is a view
    into a buffer whose gaps hold a canary.  Any read across a head or token
    boundary turns the output into NaN; any stray write breaks a canary."""
    dev = torch.device("cuda:0")
    lengths, hq, hkv, d = [150, 77, 200], 8, 2, 128
    w = workloads.custom("strided", lengths, hq, hkv, seed=51)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    T = sum(lengths)

    def padded(x, heads, pad_head, pad_tok, fill):
        buf = torch.full((T + 2, heads * (d + pad_head) + pad_tok), fill,
                         dtype=x.dtype)
        view = buf[1:T + 1, :heads * (d + pad_head)].view(T, heads, d + pad_head)[:, :, :d]
        view.copy_(x)
        return buf.to(dev), (1, pad_head, pad_tok)

    qb, _ = padded(inp["q"], hq, 8, 16, float("nan"))
    kb, _ = padded(inp["k"], hkv, 64, 8, float("nan"))
    vb, _ = padded(inp["v"], hkv, 16, 24, float("nan"))

    def view_of(buf, heads, pad_head):
        return buf[1:T + 1, :heads * (d + pad_head)].view(T, heads, d + pad_head)[:, :, :d]

    q = view_of(qb, hq, 8)
    k = view_of(kb, hkv, 64)
    v = view_of(vb, hkv, 16)
    canary = -12352.0  # exactly representable in bf16
    ob = torch.full((T + 2, hq * (d + 8) + 8), canary, dtype=torch.bfloat16, device=dev)
    out = view_of(ob, hq, 8)
    binding.attn_prefill(q, k, v, out, inp["cu_seqlens"].to(dev), hq, hkv, d,
                         w.attn_scale, 0)
    torch.cuda.synchronize()
    want = oracle.attention_varlen(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"],
                                   hq, hkv, w.attn_scale, 0)
    check("strided_nan_gaps", to64(out), want)
    mask = torch.ones_like(ob, dtype=torch.bool)
    mask[1:T + 1, :hq * (d + 8)].view(T, hq, d + 8)[:, :, :d] = False
    assert torch.all(ob[mask].float() == canary), "write outside the output view"


def test_head_major_layout():
    dev = torch.device("cuda:0")
    w = workloads.custom("headmajor", [140, 260], 4, 1, seed=52)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    T = sum(w.lengths)
    q = inp["q"].permute(1, 0, 2).contiguous().to(dev).permute(1, 0, 2)  # [H,T,d] storage
    k = inp["k"].permute(1, 0, 2).contiguous().to(dev).permute(1, 0, 2)
    v = inp["v"].to(dev)
    out = torch.empty(4, T, 128, dtype=torch.bfloat16, device=dev).permute(1, 0, 2)
    binding.attn_prefill(q, k, v, out, inp["cu_seqlens"].to(dev), 4, 1, 128,
                         w.attn_scale, 0)
    torch.cuda.synchronize()
    want = oracle.attention_varlen(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"],
                                   4, 1, w.attn_scale, 0)
    check("head_major", to64(out), want)


def test_deterministic_bitwise():
    w = workloads.custom("det", [700, 300], 32, 1, seed=53)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    a = run_gpu(inp, 32, 1, 128, w.attn_scale, 0).clone()
    b = run_gpu(inp, 32, 1, 128, w.attn_scale, 0)
    assert torch.equal(a, b)


# Folded grids: a workgroup's two wave groups take 32-row query blocks r and
# nb - 1 - r of a sequence.  Every row still meets key tiles 0, 1, ... in
# order (the folded lighter block only drops trailing tiles it cannot see,
# which add exact zeros), so folded and unfolded outputs agree bit for bit.
FOLD_SHAPES = [([1], 4, 1), ([31], 4, 1), ([33], 8, 2), ([96], 4, 1), ([100], 32, 1),
               ([257], 8, 2), ([1000], 4, 1), ([2048], 32, 1),
               ([300, 64, 1, 191, 0, 33], 8, 2), ([65, 2, 129, 500], 16, 4)]


def _fold_pair(monkeypatch, run):
    monkeypatch.setenv("ATTN_PREFILL_FOLD", "1")
    folded = run().clone()
    monkeypatch.setenv("ATTN_PREFILL_FOLD", "0")
    plain = run().clone()
    monkeypatch.delenv("ATTN_PREFILL_FOLD")
    return folded, plain


@pytest.mark.parametrize("lengths,hq,hkv", FOLD_SHAPES)
def test_folded_grid_matches_oracle_and_unfolded_bitwise(lengths, hq, hkv, monkeypatch):
    name = f"fold_{'_'.join(map(str, lengths))}_h{hq}x{hkv}"
    w = workloads.custom(name, lengths, hq, hkv, seed=64 + len(lengths) + hq)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    folded, plain = _fold_pair(monkeypatch,
                               lambda: run_gpu(inp, hq, hkv, 128, w.attn_scale, 0))
    check(name, to64(folded), oracle_of(inp, hq, hkv, w.attn_scale, 0))
    assert torch.equal(folded, plain)


@pytest.mark.parametrize("variant", ["chunked", "paged", "d64", "fp32q_fp16kv", "scale_neg",
                                     "d512", "d512_chunked", "d512_paged"])
def test_folded_grid_variants(variant, monkeypatch):
    """Folding with a KV history, a paged cache, 64-d heads, fp32 Q with fp16
    K/V, a negative scale, and 512-d heads (64-row blocks of one head)."""
    hq, hkv, d, scale = 8, 2, 128, None
    kw = {}
    lengths = [190, 33, 400, 1]
    if variant in ("chunked", "paged", "d512_chunked", "d512_paged"):
        kw["history"] = [500, 0, 129, 64]
    if variant == "d64":
        d = 64
        kw["head_dim"] = 64
    if variant.startswith("d512"):
        d = 512
        kw["head_dim"] = 512
    if variant == "fp32q_fp16kv":
        kw.update(q_dtype="fp32", kv_dtype="fp16")
    if variant == "scale_neg":
        scale = -0.3
    w = workloads.custom(f"fold_{variant}", lengths, hq, hkv, seed=65, scale=scale, **kw)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    if variant.endswith("paged"):
        k_pool, v_pool, table = to_paged(inp, 128, seed=9)
        folded, plain = _fold_pair(monkeypatch, lambda: run_paged(
            inp, k_pool, v_pool, table, 128, hq, hkv, w.attn_scale, 0, d=d))
        want = oracle.attention_paged(inp["q"], k_pool, v_pool, inp["cu_seqlens"], table,
                                      inp["kv_lengths"], 128, hq, hkv, w.attn_scale, 0)
    else:
        folded, plain = _fold_pair(monkeypatch,
                                   lambda: run_gpu(inp, hq, hkv, d, w.attn_scale, 0))
        want = oracle_of(inp, hq, hkv, w.attn_scale, 0)
    check(w.name, to64(folded), want)
    assert torch.equal(folded, plain)


@pytest.mark.parametrize("window", [0, 70])
def test_head_packing_matches_single_heads_bitwise(window):
    """Four query heads of one KV head run in one workgroup (64 rows each);
    each head alone runs 256 rows of one head.  Every row meets the same
    key tiles in the same order, so the outputs agree bit for bit."""
    w = workloads.custom("pack", [300, 64, 1, 191], 8, 2, seed=61)
    _announce(f"{w.name}_w{window}")
    inp = workloads.make_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev)
    cu = inp["cu_seqlens"].to(dev)
    packed = torch.empty(q.shape[0], 8, 128, dtype=torch.bfloat16, device=dev)
    binding.attn_prefill(q, k, v, packed, cu, 8, 2, 128, w.attn_scale, window)
    single = torch.empty_like(packed)
    for h in range(8):
        g = h // 4
        binding.attn_prefill(q[:, h:h + 1], k[:, g:g + 1], v[:, g:g + 1], single[:, h:h + 1],
                             cu, 1, 1, 128, w.attn_scale, window)
    torch.cuda.synchronize()
    assert torch.equal(packed, single)


def test_malformed_offsets_stay_in_bounds():
    """Offsets past T, decreasing or negative are clamped in the kernel: the
    call completes and nothing outside `out` is written."""
    dev = torch.device("cuda:0")
    T, hq, d = 300, 4, 128
    w = workloads.custom("malformed", [T], hq, 1, seed=54)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    ob = torch.full((T + 4, hq, d), 7.0, dtype=torch.bfloat16, device=dev)
    out = ob[2:T + 2]
    for cu in ([0, 5000], [0, 200, 100, 300], [-50, 120, 99999], [0, 300, 0, 300]):
        cu_t = torch.tensor(cu, dtype=torch.int32, device=dev)
        binding.attn_prefill(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev),
                             out, cu_t, hq, 1, d, w.attn_scale, 0)
        torch.cuda.synchronize()
        assert torch.all(ob[:2].float() == 7.0) and torch.all(ob[T + 2:].float() == 7.0)
        assert torch.all(torch.isfinite(out[:120].float()))
    # well-formed offsets on the same buffers still give the right answer
    cu_t = torch.tensor([0, T], dtype=torch.int32, device=dev)
    binding.attn_prefill(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev), out,
                         cu_t, hq, 1, d, w.attn_scale, 0)
    torch.cuda.synchronize()
    want = oracle.attention_varlen(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"],
                                   hq, 1, w.attn_scale, 0)
    check("after_malformed", to64(out), want)


def test_validate_env_rejects_bad_offsets(monkeypatch):
    dev = torch.device("cuda:0")
    w = workloads.custom("validate", [64], 1, 1, seed=55)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    monkeypatch.setenv("ATTN_PREFILL_VALIDATE", "1")
    out = torch.empty(64, 1, 128, dtype=torch.bfloat16, device=dev)
    bad = torch.tensor([0, 65], dtype=torch.int32, device=dev)
    with pytest.raises(binding.AttnPrefillError) as e:
        binding.attn_prefill(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev),
                             out, bad, 1, 1, 128, w.attn_scale, 0)
    assert e.value.status == binding.ATTN_ERR_INVALID_ARG


def test_native_library_is_loaded():
    w = workloads.custom("native", [16], 1, 1, seed=56)
    run_gpu(workloads.make_inputs(w), 1, 1, 128, w.attn_scale, 0)
    maps = open("/proc/self/maps").read()
    assert os.path.realpath(binding.LIB_PATH) in maps


# ---------------------------------------- full-size workloads, sampled rows
@pytest.mark.parametrize("name", [n for n in workloads.WORKLOADS])
def test_full_size_sampled(name):
    w = workloads.WORKLOADS[name]
    _announce(f"full-size {name}")
    inp = workloads.make_inputs(w)
    inp["decode"] = w.decode
    inp["head_dim_v"] = w.head_dim_v
    out = run_gpu(inp, w.n_q_heads, w.n_kv_heads, w.head_dim, w.attn_scale, w.window)
    rows = workloads.sample_rows(inp["lengths"], w.n_q_heads, 256, seed=w.seed)
    want = oracle.attention_rows(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"],
                                 w.n_q_heads, w.n_kv_heads, w.attn_scale, w.window,
                                 rows, cu_seqlens_k=inp.get("cu_seqlens_k"))
    got = to64(out)
    got_rows = np.stack([got[t, h] for t, h in rows])
    check(f"{name}_sampled{len(rows)}", got_rows, want)
    assert np.all(np.isfinite(got)), "non-finite output somewhere"


# ------------------------------------- prefill keys split across workgroups
def run_ws(inp, hq, hkv, d, scale, window, workspace, paged=None):
    dev = torch.device("cuda:0")
    q = inp["q"].to(dev)
    out = torch.empty(q.shape[0], hq, d, dtype=torch.bfloat16, device=dev)
    if paged is None:
        k, v = inp["k"].to(dev), inp["v"].to(dev)
        cuk = inp["cu_seqlens_k"].to(dev) if "cu_seqlens_k" in inp else None
        pg = None
    else:
        k_pool, v_pool, table, page = paged
        k, v = k_pool.to(dev), v_pool.to(dev)
        cuk = None
        pg = (torch.from_numpy(table).to(dev),
              torch.tensor(inp["kv_lengths"], dtype=torch.int32, device=dev), page)
    binding.attn_prefill_ex(q, k, v, out, inp["cu_seqlens"].to(dev), hq, hkv, d, d, scale,
                            window, cu_seqlens_k=cuk, paged=pg, workspace=workspace)
    torch.cuda.synchronize()
    return out


def split_workspace(inp, hq, hkv, d, max_keys=None, windows=(0,)):
    """A workspace for every listed window (the plan, and so its size,
    depends on the window), filled with NaN bytes: nothing may read a
    partial before it is written."""
    T = inp["q"].shape[0]
    n_seqs = len(inp["lengths"])
    mk = max_keys if max_keys is not None else inp["k"].shape[0]
    sizes = [binding.prefill_workspace_size(T, mk, n_seqs, hq, hkv, d, d, win)
             for win in windows]
    assert min(sizes) > 0, f"this shape is split at every window: {sizes}"
    nbytes = max(sizes)
    # NaN bytes: nothing may read a partial before it is written
    return torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda:0")


@pytest.mark.parametrize("d", [128, 64])
def test_prefill_split_packed(d):
    """A long and a short sequence (query tiles of one and of several
    pieces in one launch), 2 query heads on 1 KV head: against the oracle and
    against the unsplit kernel, causal, with windows and scale signs."""
    w = workloads.custom(f"split_d{d}", [3000, 200, 1], 2, 1, head_dim=d, seed=151,
                         k_outlier_frac=0.01)
    inp = workloads.make_inputs(w)
    ws = split_workspace(inp, 2, 1, d, windows=(0, 1, 700))
    for win in (0, 1, 700):
        for scale in (1 / math.sqrt(d), -0.5):
            _announce(f"{w.name} W={win} s={scale:.3f}")
            out = run_ws(inp, 2, 1, d, scale, win, ws)
            check(f"split_d{d}_w{win}_s{scale:.3f}", to64(out), oracle_of(inp, 2, 1, scale, win))
            ref = run_gpu(inp, 2, 1, d, scale, win)
            diff = float((out.float() - ref.float()).abs().max())
            assert diff <= 2e-2, f"split vs unsplit: {diff}"


def test_prefill_split_chunked_paged_and_dtypes():
    w = workloads.custom("split_chunked", [900, 64], 4, 2, seed=152, q_dtype="fp32",
                         kv_dtype="fp16", history=[2500, 10])
    _announce(w.name)
    inp = workloads.make_inputs(w)
    ws = split_workspace(inp, 4, 2, 128, windows=(0, 500))
    for win in (0, 500):
        out = run_ws(inp, 4, 2, 128, w.attn_scale, win, ws)
        check(f"split_chunked_w{win}", to64(out), oracle_of(inp, 4, 2, w.attn_scale, win))
    k_pool, v_pool, table = to_paged(inp, 128, seed=15)
    wsp = split_workspace(inp, 4, 2, 128, max_keys=table.shape[1] * 128)
    out = run_ws(inp, 4, 2, 128, w.attn_scale, 0, wsp, paged=(k_pool, v_pool, table, 128))
    want = oracle.attention_paged(inp["q"], k_pool, v_pool, inp["cu_seqlens"], table,
                                  inp["kv_lengths"], 128, 4, 2, w.attn_scale, 0)
    check("split_paged", to64(out), want)


def test_prefill_split_small_workspace_is_the_unsplit_kernel():
    """A workspace smaller than the split needs runs the unsplit kernel:
    the same bits as attn_prefill."""
    w = workloads.custom("split_small_ws", [2000], 2, 1, seed=153)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    full = split_workspace(inp, 2, 1, 128)
    small = torch.empty(full.numel() // 2, dtype=torch.uint8, device="cuda:0")
    out = run_ws(inp, 2, 1, 128, w.attn_scale, 0, small)
    assert torch.equal(out, run_gpu(inp, 2, 1, 128, w.attn_scale, 0))


@pytest.mark.parametrize("name", ["long_8192tok_4q1kv_outliers_share"])
def test_prefill_split_full_size_sampled(name):
    """The benchmark workloads that split, with the workspace the benchmark
    passes, on sampled rows."""
    w = workloads.WORKLOADS[name]
    _announce(f"{name} split")
    inp = workloads.make_inputs(w)
    ws = split_workspace(inp, w.n_q_heads, w.n_kv_heads, w.head_dim, windows=(w.window,))
    out = to64(run_ws(inp, w.n_q_heads, w.n_kv_heads, w.head_dim, w.attn_scale, w.window, ws))
    rows = workloads.sample_rows(inp["lengths"], w.n_q_heads, 256, seed=w.seed)
    want = oracle.attention_rows(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"],
                                 w.n_q_heads, w.n_kv_heads, w.attn_scale, w.window, rows)
    check(f"{name}_split_sampled", np.stack([out[t, h] for t, h in rows]), want)
    assert np.all(np.isfinite(out))


# ------------------------------------------------------------ size limits
def test_many_short_sequences_every_kernel():
    """300 sequences (the work decode scans the offsets 64 at a time, so this
    takes five passes and carries the tile count across them), empty ones
    among them, through the 64-, 128-, 256- and 512-wide kernels."""
    lengths = [int(x) for x in np.random.default_rng(141).integers(0, 41, size=300)]
    assert 0 in lengths and len(lengths) > 4 * 64
    for d, hq, hkv in ((128, 4, 2), (64, 2, 1), (256, 2, 1), (512, 2, 1)):
        w = workloads.custom(f"many_seqs_d{d}", lengths, hq, hkv, head_dim=d, seed=141 + d)
        inp = workloads.make_inputs(w)
        for win in (0, 7):
            _announce(f"{w.name} W={win}")
            out = run_gpu(inp, hq, hkv, d, w.attn_scale, win)
            check(f"{w.name}_w{win}", to64(out), oracle_of(inp, hq, hkv, w.attn_scale, win))


def test_many_sequences_chunked_and_paged():
    """150 chunks with histories (the key offsets are scanned with the query
    offsets), then the same keys through a paged cache."""
    rng = np.random.default_rng(143)
    lq = [int(x) for x in rng.integers(0, 21, size=150)]
    hist = [int(x) for x in rng.integers(0, 101, size=150)]
    w = workloads.custom("many_chunks", lq, 4, 1, seed=143, history=hist)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    for win in (0, 30):
        out = run_gpu(inp, 4, 1, 128, w.attn_scale, win)
        check(f"many_chunks_w{win}", to64(out), oracle_of(inp, 4, 1, w.attn_scale, win))
    k_pool, v_pool, table = to_paged(inp, 64, seed=14)
    out = run_paged(inp, k_pool, v_pool, table, 64, 4, 1, w.attn_scale, 0)
    want = oracle.attention_paged(inp["q"], k_pool, v_pool, inp["cu_seqlens"], table,
                                  inp["kv_lengths"], 64, 4, 1, w.attn_scale, 0)
    check("many_chunks_paged", to64(out), want)


def test_long_sequence_sampled():
    """One 65,536-token sequence (1024 key tiles for its last query tile),
    causal and with a 4096-key window, on sampled rows."""
    w = workloads.custom("long_65536", [65536], 2, 1, seed=144, k_outlier_frac=0.01)
    inp = workloads.make_inputs(w)
    rows = workloads.sample_rows(inp["lengths"], 2, 96, seed=144)
    for win in (0, 4096):
        _announce(f"{w.name} W={win}")
        out = to64(run_gpu(inp, 2, 1, 128, w.attn_scale, win))
        want = oracle.attention_rows(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], 2, 1,
                                     w.attn_scale, win, rows)
        check(f"long_65536_w{win}_sampled", np.stack([out[t, h] for t, h in rows]), want)
        assert np.all(np.isfinite(out))


def test_largest_kv_token_stride():
    """K and V as views with the largest token stride the library accepts
    (64 strides just under 2 GiB: 16,777,208 bf16 elements per token), for
    prefill and decode; one element more is rejected on the host."""
    dev = torch.device("cuda:0")
    stride = ((1 << 31) - 1) // 64 // 2 // 8 * 8  # elements; a multiple of 16 bytes
    assert stride * 2 * 64 <= (1 << 31) - 1 < (stride + 8) * 2 * 64
    lengths = [150, 50]
    w = workloads.custom("big_stride", lengths, 2, 1, seed=145)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    T = sum(lengths)

    def spread(t):
        big = torch.empty((T - 1) * stride + 128, dtype=torch.bfloat16, device=dev)
        view = torch.as_strided(big, (T, 1, 128), (stride, 128, 1))
        view.copy_(t.to(dev))
        return big, view

    kb, kview = spread(inp["k"])
    vb, vview = spread(inp["v"])
    q = inp["q"].to(dev)
    cu = inp["cu_seqlens"].to(dev)
    out = torch.empty(T, 2, 128, dtype=torch.bfloat16, device=dev)
    binding.attn_prefill(q, kview, vview, out, cu, 2, 1, 128, w.attn_scale, 0)
    torch.cuda.synchronize()
    check("big_stride_prefill", to64(out), oracle_of(inp, 2, 1, w.attn_scale, 0))
    # decode: the last token of each sequence against all of its keys
    last = [149, 199]
    dout = torch.empty(2, 2, 128, dtype=torch.bfloat16, device=dev)
    binding.attn_decode(q[last].contiguous(), kview, vview, dout, cu, 2, 1, 128,
                        w.attn_scale, 0)
    torch.cuda.synchronize()
    check("big_stride_decode", to64(dout), oracle_of(inp, 2, 1, w.attn_scale, 0)[last])
    too_far = torch.as_strided(kb, (2, 1, 128), (stride + 8, 128, 1))
    with pytest.raises(binding.AttnPrefillError) as e:
        binding.attn_prefill(q[:2], too_far, too_far, out[:2],
                             torch.tensor([0, 2], dtype=torch.int32, device=dev), 2, 1, 128,
                             w.attn_scale, 0)
    assert e.value.status == binding.ATTN_ERR_UNSUPPORTED
    del kb, vb, kview, vview, too_far
    torch.cuda.empty_cache()


# ------------------------------------- chunked prefill against a KV history
CHUNK_PAIRS = [(1, 1), (1, 200), (2, 2), (63, 64), (64, 64), (65, 300), (128, 1000),
               (200, 200), (0, 50), (257, 258), (3, 700), (256, 256), (255, 1023),
               (129, 129)]
CHUNK_WINDOWS = [0, 1, 2, 63, 64, 65, 256, 1000]


@pytest.mark.parametrize("hq,hkv", [(4, 1), (8, 2)])
@pytest.mark.parametrize("scale", [1 / math.sqrt(128), 1.0, -0.3])
def test_chunked_grid_packed(hq, hkv, scale):
    lq = [a for a, _ in CHUNK_PAIRS]
    hist = [b - a for a, b in CHUNK_PAIRS]
    w = workloads.custom(f"chunk_grid_h{hq}x{hkv}", lq, hq, hkv, seed=71, scale=scale,
                         history=hist)
    inp = workloads.make_inputs(w)
    for win in CHUNK_WINDOWS:
        _announce(f"{w.name} s={scale:.3f} W={win}")
        out = run_gpu(inp, hq, hkv, 128, scale, win)
        check(f"chunk_grid_h{hq}x{hkv}_s{scale:.3f}_w{win}", to64(out),
              oracle_of(inp, hq, hkv, scale, win))


@pytest.mark.parametrize("qd,kvd", [("fp32", "fp16"), ("bf16", "fp16")])
def test_chunked_dtype_variants(qd, kvd):
    w = workloads.custom(f"chunk_dt_{qd}_{kvd}", [190, 33, 400], 8, 2, q_dtype=qd,
                         kv_dtype=kvd, seed=72, history=[500, 0, 129])
    inp = workloads.make_inputs(w)
    for win in (0, 100):
        _announce(f"{w.name} W={win}")
        out = run_gpu(inp, 8, 2, 128, w.attn_scale, win)
        check(f"{w.name}_w{win}", to64(out), oracle_of(inp, 8, 2, w.attn_scale, win))


def test_chunked_without_history_is_attn_prefill_bitwise():
    w = workloads.custom("chunk_nohist", [700, 1, 300], 32, 1, seed=73,
                         history=[0, 0, 0])
    _announce(w.name)
    inp = workloads.make_inputs(w)
    a = run_gpu(inp, 32, 1, 128, w.attn_scale, 0).clone()
    plain = {k: v for k, v in inp.items() if k != "cu_seqlens_k"}
    b = run_gpu(plain, 32, 1, 128, w.attn_scale, 0)
    assert torch.equal(a, b)


def test_chunk_by_chunk_matches_single_pass():
    """A sequence prefilled chunk by chunk against its growing KV history
    gives the single-pass rows (the multi-chunk contract)."""
    dev = torch.device("cuda:0")
    n, hq = 1000, 32
    w = workloads.custom("chunk_split", [n], hq, 1, seed=74)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    full = to64(run_gpu(inp, hq, 1, 128, w.attn_scale, 0))
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    for a, b in ((0, 300), (300, 301), (301, 777), (777, 1000)):
        out = torch.empty(b - a, hq, 128, dtype=torch.bfloat16, device=dev)
        cq = torch.tensor([0, b - a], dtype=torch.int32, device=dev)
        ck = torch.tensor([0, b], dtype=torch.int32, device=dev)
        binding.attn_prefill_chunked(q[a:b], k[:b], v[:b], out, cq, ck, hq, 1, 128,
                                     w.attn_scale, 0)
        torch.cuda.synchronize()
        got = to64(out)
        diff = float(np.max(np.abs(got - full[a:b])))
        sys.stdout.write(f"[chunk] rows {a}..{b}: max |chunked - single pass| = {diff}\n")
        assert diff <= 1e-2, (a, b, diff)
        want = oracle.attention_chunked(inp["q"][a:b], inp["k"][:b], inp["v"][:b],
                                        [0, b - a], [0, b], hq, 1, w.attn_scale, 0)
        check(f"chunk_split_{a}_{b}", got, want)


def test_chunked_more_queries_than_keys_is_memory_safe():
    """Lq > Lk is outside the contract: queries left without a visible key
    get zero rows, the others follow the definition, nothing outside `out`
    is written."""
    dev = torch.device("cuda:0")
    w = workloads.custom("chunk_short_kv", [10], 4, 1, seed=75, history=[0])
    _announce(w.name)
    inp = workloads.make_inputs(w)
    ob = torch.full((14, 4, 128), 7.0, dtype=torch.bfloat16, device=dev)
    out = ob[2:12]
    cq = torch.tensor([0, 10], dtype=torch.int32, device=dev)
    ck = torch.tensor([0, 4], dtype=torch.int32, device=dev)
    binding.attn_prefill_chunked(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev),
                                 out, cq, ck, 4, 1, 128, w.attn_scale, 0)
    torch.cuda.synchronize()
    assert torch.all(ob[:2].float() == 7.0) and torch.all(ob[12:].float() == 7.0)
    want = oracle.attention_chunked(inp["q"], inp["k"][:4], inp["v"][:4], [0, 10],
                                    [0, 4], 4, 1, w.attn_scale, 0)
    assert np.all(want[:6] == 0.0)
    check("chunk_short_kv", to64(out), want)


# ------------------------------------------------------------ paged K/V
def to_paged(inp, page, seed, spare=3):
    """Scatters a chunked input's packed K/V into page pools in a seeded
    random page order; slots no sequence owns hold NaN, so that a wrong
    page or slot read shows up in the output."""
    rng = np.random.default_rng(seed)
    kv_lengths = inp["kv_lengths"]
    cu_k = inp["cu_seqlens_k"].tolist()
    n_blocks = [(n + page - 1) // page for n in kv_lengths]
    n_pages = sum(n_blocks) + spare
    perm = rng.permutation(n_pages)
    width = max(1, max(n_blocks))
    table = np.full((len(kv_lengths), width), n_pages + 5, dtype=np.int32)
    k, v = inp["k"], inp["v"]
    k_pool = torch.full((n_pages * page,) + tuple(k.shape[1:]), float("nan"), dtype=k.dtype)
    v_pool = torch.full((n_pages * page,) + tuple(v.shape[1:]), float("nan"), dtype=v.dtype)
    used = 0
    for s, n in enumerate(kv_lengths):
        for b in range(n_blocks[s]):
            pg = int(perm[used])
            used += 1
            table[s, b] = pg
            lo, hi = cu_k[s] + b * page, min(cu_k[s] + n, cu_k[s] + (b + 1) * page)
            k_pool[pg * page:pg * page + (hi - lo)] = k[lo:hi]
            v_pool[pg * page:pg * page + (hi - lo)] = v[lo:hi]
    return k_pool, v_pool, table


def run_paged(inp, k_pool, v_pool, table, page, hq, hkv, scale, window, d=128):
    dev = torch.device("cuda:0")
    q = inp["q"].to(dev)
    out = torch.empty(q.shape[0], hq, d, dtype=torch.bfloat16, device=dev)
    binding.attn_prefill_paged(
        q, k_pool.to(dev), v_pool.to(dev), out, inp["cu_seqlens"].to(dev),
        torch.from_numpy(table).to(dev),
        torch.tensor(inp["kv_lengths"], dtype=torch.int32, device=dev), page, hq, hkv,
        d, scale, window)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("page", [64, 128, 256])
@pytest.mark.parametrize("hq,hkv", [(4, 1), (8, 2)])
def test_paged_grid_packed(page, hq, hkv):
    lq = [a for a, _ in CHUNK_PAIRS]
    hist = [b - a for a, b in CHUNK_PAIRS]
    w = workloads.custom(f"paged_grid_p{page}_h{hq}x{hkv}", lq, hq, hkv, seed=81,
                         history=hist)
    inp = workloads.make_inputs(w)
    k_pool, v_pool, table = to_paged(inp, page, seed=page + hq)
    for win in (0, 63, 256):
        _announce(f"{w.name} W={win}")
        out = run_paged(inp, k_pool, v_pool, table, page, hq, hkv, w.attn_scale, win)
        want = oracle.attention_paged(inp["q"], k_pool, v_pool, inp["cu_seqlens"], table,
                                      inp["kv_lengths"], page, hq, hkv, w.attn_scale, win)
        check(f"paged_grid_p{page}_h{hq}x{hkv}_w{win}", to64(out), want)


def test_paged_dtype_fp32q_fp16kv():
    w = workloads.custom("paged_fp32q_fp16kv", [190, 33, 400], 8, 2, q_dtype="fp32",
                         kv_dtype="fp16", seed=82, history=[500, 0, 129])
    _announce(w.name)
    inp = workloads.make_inputs(w)
    k_pool, v_pool, table = to_paged(inp, 128, seed=5)
    out = run_paged(inp, k_pool, v_pool, table, 128, 8, 2, w.attn_scale, 0)
    want = oracle.attention_paged(inp["q"], k_pool, v_pool, inp["cu_seqlens"], table,
                                  inp["kv_lengths"], 128, 8, 2, w.attn_scale, 0)
    check(w.name, to64(out), want)


def test_paged_in_page_order_equals_chunked_bitwise():
    """Pages laid out in position order give the packed chunked result bit
    for bit (same tiles, same arithmetic)."""
    w = workloads.custom("paged_identity", [256, 64], 8, 1, seed=83, history=[128, 0])
    _announce(w.name)
    inp = workloads.make_inputs(w)
    page = 64
    # one sequence's keys per run of pages, in order: a pool equal to the
    # packed K/V, since both lengths are multiples of the page size
    k_pool, v_pool = inp["k"], inp["v"]
    table = np.array([[0, 1, 2, 3, 4, 5], [6, 0, 0, 0, 0, 0]], dtype=np.int32)
    a = run_paged(inp, k_pool, v_pool, table, page, 8, 1, w.attn_scale, 0).clone()
    b = run_gpu(inp, 8, 1, 128, w.attn_scale, 0)
    assert torch.equal(a, b)


def test_paged_full_size_sampled():
    w = workloads.WORKLOADS["chunk2048_hist6144_32q1kv_outliers"]
    _announce(f"paged full-size {w.name}")
    inp = workloads.make_inputs(w)
    k_pool, v_pool, table = to_paged(inp, 256, seed=7)
    out = run_paged(inp, k_pool, v_pool, table, 256, w.n_q_heads, w.n_kv_heads,
                    w.attn_scale, 0)
    rows = workloads.sample_rows(inp["lengths"], w.n_q_heads, 256, seed=w.seed)
    want = oracle.attention_rows(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"],
                                 w.n_q_heads, w.n_kv_heads, w.attn_scale, 0, rows,
                                 cu_seqlens_k=inp["cu_seqlens_k"])
    got = to64(out)
    check(f"paged_{w.name}_sampled{len(rows)}", np.stack([got[t, h] for t, h in rows]), want)
    assert np.all(np.isfinite(got))


# ------------------------------------------------------------ head_dim 64
D64_LENGTHS = [1, 2, 63, 64, 65, 127, 128, 129, 257, 0, 1, 200, 600]


@pytest.mark.parametrize("hq,hkv", [(4, 1), (8, 2), (6, 6)])
def test_head_dim_64_packed(hq, hkv):
    w = workloads.custom(f"d64_h{hq}x{hkv}", D64_LENGTHS, hq, hkv, head_dim=64, seed=91)
    inp = workloads.make_inputs(w)
    for win in (0, 1, 64, 129):
        for scale in (1 / 8.0, -0.5):
            _announce(f"{w.name} W={win} s={scale}")
            out = run_gpu(inp, hq, hkv, 64, scale, win)
            check(f"d64_h{hq}x{hkv}_w{win}_s{scale}", to64(out),
                  oracle_of(inp, hq, hkv, scale, win))


@pytest.mark.parametrize("qd,kvd", [("fp32", "fp16"), ("bf16", "fp16"), ("fp32", "bf16")])
def test_head_dim_64_dtypes(qd, kvd):
    w = workloads.custom(f"d64_{qd}_{kvd}", [300, 1, 77], 8, 2, head_dim=64, q_dtype=qd,
                         kv_dtype=kvd, seed=92)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    out = run_gpu(inp, 8, 2, 64, w.attn_scale, 0)
    check(w.name, to64(out), oracle_of(inp, 8, 2, w.attn_scale, 0))


def test_head_dim_64_chunked_and_paged():
    w = workloads.custom("d64_chunked", [190, 33, 400, 1], 8, 1, head_dim=64, seed=93,
                         history=[500, 0, 129, 1000])
    _announce(w.name)
    inp = workloads.make_inputs(w)
    for win in (0, 100):
        out = run_gpu(inp, 8, 1, 64, w.attn_scale, win)
        check(f"d64_chunked_w{win}", to64(out), oracle_of(inp, 8, 1, w.attn_scale, win))
    k_pool, v_pool, table = to_paged(inp, 128, seed=11)
    out = run_paged(inp, k_pool, v_pool, table, 128, 8, 1, w.attn_scale, 0, d=64)
    want = oracle.attention_paged(inp["q"], k_pool, v_pool, inp["cu_seqlens"], table,
                                  inp["kv_lengths"], 128, 8, 1, w.attn_scale, 0)
    check("d64_paged", to64(out), want)


# ---------------------------------------------------------------- decode
DECODE_LENGTHS = [1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000, 4097]


def decode_inputs(name, lengths, hq, hkv, seed, qd="bf16", kvd="bf16"):
    w = workloads.custom(name, [1] * len(lengths), hq, hkv, seed=seed, q_dtype=qd,
                         kv_dtype=kvd, history=[n - 1 for n in lengths])
    inp = workloads.make_inputs(w)
    inp["decode"] = True
    return w, inp


@pytest.mark.parametrize("hq,hkv", [(32, 1), (8, 2), (4, 4), (64, 1), (40, 8)])
def test_decode_grid(hq, hkv):
    w, inp = decode_inputs(f"decode_grid_h{hq}x{hkv}", DECODE_LENGTHS, hq, hkv, seed=101)
    for win in (0, 1, 64, 300):
        for scale in (1 / math.sqrt(128), -0.7):
            _announce(f"{w.name} W={win} s={scale:.3f}")
            out = run_gpu(inp, hq, hkv, 128, scale, win)
            want = oracle.attention_decode(inp["q"], inp["k"], inp["v"], inp["cu_seqlens_k"],
                                           hq, hkv, scale, win)
            check(f"decode_grid_h{hq}x{hkv}_w{win}_s{scale:.3f}", to64(out), want)


@pytest.mark.parametrize("qd,kvd", [("fp32", "fp16"), ("bf16", "fp16"), ("fp32", "bf16")])
def test_decode_dtypes(qd, kvd):
    w, inp = decode_inputs(f"decode_{qd}_{kvd}", [5, 700, 2048, 33], 16, 2, seed=102,
                           qd=qd, kvd=kvd)
    _announce(w.name)
    out = run_gpu(inp, 16, 2, 128, w.attn_scale, 0)
    want = oracle.attention_decode(inp["q"], inp["k"], inp["v"], inp["cu_seqlens_k"], 16, 2,
                                   w.attn_scale, 0)
    check(w.name, to64(out), want)


def test_decode_matches_prefill_last_rows():
    """The decode step for the token after a prefix equals the prefill row
    of that token (both on the GPU)."""
    dev = torch.device("cuda:0")
    lengths = [300, 1, 1000, 65]
    w = workloads.custom("decode_vs_prefill", lengths, 32, 4, seed=103)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    full = to64(run_gpu(inp, 32, 4, 128, w.attn_scale, 0))
    cu = inp["cu_seqlens"].tolist()
    last = [cu[s + 1] - 1 for s in range(len(lengths))]
    q = inp["q"][last].contiguous().to(dev)
    out = torch.empty(len(lengths), 32, 128, dtype=torch.bfloat16, device=dev)
    binding.attn_decode(q, inp["k"].to(dev), inp["v"].to(dev), out, inp["cu_seqlens"].to(dev),
                        32, 4, 128, w.attn_scale, 0)
    torch.cuda.synchronize()
    diff = float(np.max(np.abs(to64(out) - full[last])))
    sys.stdout.write(f"[decode] max |decode - prefill last row| = {diff}\n")
    assert diff <= 2e-2


def test_decode_paged_nan_pools():
    w, inp = decode_inputs("decode_paged", DECODE_LENGTHS, 32, 2, seed=104)
    _announce(w.name)
    dev = torch.device("cuda:0")
    for page in (64, 256):
        k_pool, v_pool, table = to_paged(inp, page, seed=page)
        out = torch.empty(len(DECODE_LENGTHS), 32, 128, dtype=torch.bfloat16, device=dev)
        binding.attn_decode_paged(
            inp["q"].to(dev), k_pool.to(dev), v_pool.to(dev), out,
            torch.from_numpy(table).to(dev),
            torch.tensor(inp["kv_lengths"], dtype=torch.int32, device=dev), page, 32, 2, 128,
            w.attn_scale, 0)
        torch.cuda.synchronize()
        want = oracle.attention_paged(inp["q"], k_pool, v_pool, inp["cu_seqlens"], table,
                                      inp["kv_lengths"], page, 32, 2, w.attn_scale, 0)
        check(f"decode_paged_p{page}", to64(out), want)


def test_decode_strided_views_and_empty_sequence():
    """q and out as strided views (head-major q); a sequence without keys
    (outside the contract) gives a zero row; nothing outside out is written."""
    dev = torch.device("cuda:0")
    lengths = [40, 0, 300]
    w = workloads.custom("decode_strided", [1, 1, 1], 8, 1, seed=105,
                         history=[39, 0, 299])
    _announce(w.name)
    inp = workloads.make_inputs(w)
    # the middle sequence has one key in the draw; give it none
    cu_k = torch.tensor([0, 40, 40, 340], dtype=torch.int32)
    k = torch.cat([inp["k"][:40], inp["k"][41:]])
    v = torch.cat([inp["v"][:40], inp["v"][41:]])
    qh = inp["q"].permute(1, 0, 2).contiguous().permute(1, 0, 2)  # head-major storage
    ob = torch.full((5, 8, 128), 7.0, dtype=torch.bfloat16, device=dev)
    out = ob[1:4]
    binding.attn_decode(qh.to(dev), k.to(dev), v.to(dev), out, cu_k.to(dev), 8, 1, 128,
                        w.attn_scale, 0)
    torch.cuda.synchronize()
    assert torch.all(ob[0].float() == 7.0) and torch.all(ob[4].float() == 7.0)
    want = oracle.attention_decode(inp["q"], k, v, cu_k, 8, 1, w.attn_scale, 0)
    assert np.all(want[1] == 0.0)
    check("decode_strided", to64(out), want)


# ------------------------------------------------ decode, keys split across workgroups
def run_decode_ws(inp, hq, hkv, scale, window, workspace):
    dev = torch.device("cuda:0")
    out = torch.empty(inp["q"].shape[0], hq, 128, dtype=torch.bfloat16, device=dev)
    binding.attn_decode(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev), out,
                        inp["cu_seqlens_k"].to(dev), hq, hkv, 128, scale, window,
                        workspace=workspace)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("hq,hkv", [(32, 1), (8, 2), (40, 8)])
def test_decode_split_grid(hq, hkv):
    """A small batch with the preferred split (and with workspaces that fit
    only a few ranges) against the oracle and against the unsplit kernel."""
    w, inp = decode_inputs(f"decode_split_h{hq}x{hkv}", DECODE_LENGTHS, hq, hkv, seed=106)
    n = len(DECODE_LENGTHS)
    full = binding.decode_workspace_size(n, hq, hkv, 128)
    assert full > 0, "a batch this small is split"
    units = n * hkv * ((hq // hkv + 31) // 32)
    range_bytes = units * (64 + 32 * 128) * 4  # one key range of every unit
    assert full % range_bytes == 0 and full // range_bytes >= 2
    for nbytes in (full, 2 * range_bytes + 16, 3 * full):
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda:0")  # NaN floats
        for win in (0, 1, 64, 300):
            for scale in (1 / math.sqrt(128), -0.7):
                _announce(f"{w.name} ws={nbytes} W={win} s={scale:.3f}")
                out = run_decode_ws(inp, hq, hkv, scale, win, ws)
                want = oracle.attention_decode(inp["q"], inp["k"], inp["v"],
                                               inp["cu_seqlens_k"], hq, hkv, scale, win)
                check(f"decode_split_h{hq}x{hkv}_ws{nbytes}_w{win}_s{scale:.3f}", to64(out),
                      want)
                ref = run_gpu(inp, hq, hkv, 128, scale, win)
                diff = float((out.float() - ref.float()).abs().max())
                assert diff <= 2e-2, f"split vs unsplit: {diff}"


def test_decode_split_long_single_sequence():
    """One 32K-key sequence (MQA, 32 heads): the case the split exists for."""
    w, inp = decode_inputs("decode_split_32k", [32768], 32, 1, seed=107)
    ws = binding.decode_workspace(1, 32, 1, 128)
    for win in (0, 4096):
        _announce(f"{w.name} W={win}")
        out = run_decode_ws(inp, 32, 1, w.attn_scale, win, ws)
        want = oracle.attention_decode(inp["q"], inp["k"], inp["v"], inp["cu_seqlens_k"],
                                       32, 1, w.attn_scale, win)
        check(f"decode_split_32k_w{win}", to64(out), want)


def test_decode_split_paged_and_workspace_reuse():
    """Paged decode with a split, then a smaller batch on the same workspace
    (stale partials from the first call must not leak into the second)."""
    w, inp = decode_inputs("decode_split_paged", DECODE_LENGTHS, 32, 2, seed=108)
    dev = torch.device("cuda:0")
    ws = binding.decode_workspace(len(DECODE_LENGTHS), 32, 2, 128)
    k_pool, v_pool, table = to_paged(inp, 64, seed=5)
    out = torch.empty(len(DECODE_LENGTHS), 32, 128, dtype=torch.bfloat16, device=dev)
    _announce(w.name)
    binding.attn_decode_paged(
        inp["q"].to(dev), k_pool.to(dev), v_pool.to(dev), out, torch.from_numpy(table).to(dev),
        torch.tensor(inp["kv_lengths"], dtype=torch.int32, device=dev), 64, 32, 2, 128,
        w.attn_scale, 0, workspace=ws)
    torch.cuda.synchronize()
    want = oracle.attention_paged(inp["q"], k_pool, v_pool, inp["cu_seqlens"], table,
                                  inp["kv_lengths"], 64, 32, 2, w.attn_scale, 0)
    check("decode_split_paged", to64(out), want)
    w2, inp2 = decode_inputs("decode_split_reuse", [3000, 17], 32, 2, seed=109)
    _announce(w2.name)
    out2 = run_decode_ws(inp2, 32, 2, w2.attn_scale, 0, ws)
    want2 = oracle.attention_decode(inp2["q"], inp2["k"], inp2["v"], inp2["cu_seqlens_k"],
                                    32, 2, w2.attn_scale, 0)
    check("decode_split_reuse", to64(out2), want2)


def test_decode_split_full_size_sampled():
    """The decode benchmark batch (32 sequences of 8192 keys, MQA) with the
    workspace the benchmark passes, on sampled sequences."""
    w = workloads.WORKLOADS["decode32_mqa32q1kv_8192"]
    inp = workloads.make_inputs(w)
    ws = binding.decode_workspace(32, w.n_q_heads, w.n_kv_heads, 128)
    _announce(f"{w.name} split")
    out = to64(run_decode_ws(inp, w.n_q_heads, w.n_kv_heads, w.attn_scale, w.window, ws))
    cu = inp["cu_seqlens_k"].tolist()
    for s in (0, 13, 31):
        sl = slice(cu[s], cu[s + 1])
        want = oracle.attention_decode(inp["q"][s:s + 1], inp["k"][sl], inp["v"][sl],
                                       torch.tensor([0, cu[s + 1] - cu[s]], dtype=torch.int32),
                                       w.n_q_heads, w.n_kv_heads, w.attn_scale, w.window)
        check(f"{w.name}_split_seq{s}", out[s:s + 1], want)


# ----------------------------------------------------------- head_dim 256
@pytest.mark.parametrize("hq,hkv", [(4, 1), (8, 2)])
def test_head_dim_256_packed(hq, hkv):
    w = workloads.custom(f"d256_h{hq}x{hkv}", D64_LENGTHS, hq, hkv, head_dim=256, seed=111)
    inp = workloads.make_inputs(w)
    for win in (0, 1, 64, 129):
        for scale in (1 / 16.0, -0.4):
            _announce(f"{w.name} W={win} s={scale}")
            out = run_gpu(inp, hq, hkv, 256, scale, win)
            check(f"d256_h{hq}x{hkv}_w{win}_s{scale}", to64(out),
                  oracle_of(inp, hq, hkv, scale, win))


@pytest.mark.parametrize("qd,kvd", [("fp32", "fp16"), ("bf16", "fp16")])
def test_head_dim_256_dtypes(qd, kvd):
    w = workloads.custom(f"d256_{qd}_{kvd}", [300, 1, 77], 4, 2, head_dim=256, q_dtype=qd,
                         kv_dtype=kvd, seed=112)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    out = run_gpu(inp, 4, 2, 256, w.attn_scale, 0)
    check(w.name, to64(out), oracle_of(inp, 4, 2, w.attn_scale, 0))


def test_head_dim_256_chunked_and_paged():
    w = workloads.custom("d256_chunked", [190, 33, 400, 1], 4, 1, head_dim=256, seed=113,
                         history=[500, 0, 129, 1000])
    _announce(w.name)
    inp = workloads.make_inputs(w)
    for win in (0, 100):
        out = run_gpu(inp, 4, 1, 256, w.attn_scale, win)
        check(f"d256_chunked_w{win}", to64(out), oracle_of(inp, 4, 1, w.attn_scale, win))
    k_pool, v_pool, table = to_paged(inp, 128, seed=12)
    out = run_paged(inp, k_pool, v_pool, table, 128, 4, 1, w.attn_scale, 0, d=256)
    want = oracle.attention_paged(inp["q"], k_pool, v_pool, inp["cu_seqlens"], table,
                                  inp["kv_lengths"], 128, 4, 1, w.attn_scale, 0)
    check("d256_paged", to64(out), want)


# ----------------------------------------------------------- head_dim 512
D512_LENGTHS = [1, 31, 32, 33, 63, 64, 65, 0, 129, 300]


@pytest.mark.parametrize("hq,hkv", [(2, 1), (4, 2)])
def test_head_dim_512_packed(hq, hkv):
    w = workloads.custom(f"d512_h{hq}x{hkv}", D512_LENGTHS, hq, hkv, head_dim=512, seed=131)
    inp = workloads.make_inputs(w)
    for win in (0, 1, 64, 129):
        for scale in (1 / math.sqrt(512), -0.3):
            _announce(f"{w.name} W={win} s={scale:.3f}")
            out = run_gpu(inp, hq, hkv, 512, scale, win)
            check(f"d512_h{hq}x{hkv}_w{win}_s{scale:.3f}", to64(out),
                  oracle_of(inp, hq, hkv, scale, win))


@pytest.mark.parametrize("qd,kvd", [("fp32", "fp16"), ("bf16", "fp16"), ("fp32", "bf16")])
def test_head_dim_512_dtypes(qd, kvd):
    w = workloads.custom(f"d512_{qd}_{kvd}", [200, 1, 77], 4, 2, head_dim=512, q_dtype=qd,
                         kv_dtype=kvd, seed=132)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    out = run_gpu(inp, 4, 2, 512, w.attn_scale, 0)
    check(w.name, to64(out), oracle_of(inp, 4, 2, w.attn_scale, 0))


def test_head_dim_512_fp32_fp16_outliers():
    """fp32 q and fp16 k with x30 outliers against the exact oracle on the
    inputs as stored (the products run in fp16, K/V as stored)."""
    w = workloads.custom("d512_fp32_fp16_outliers", [200, 1, 77], 4, 2, head_dim=512,
                         q_dtype="fp32", kv_dtype="fp16", seed=132, k_outlier_frac=0.01)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    out = run_gpu(inp, 4, 2, 512, w.attn_scale, 0)
    check(w.name, to64(out), oracle_of(inp, 4, 2, w.attn_scale, 0))


@pytest.mark.parametrize("d", [64, 128, 256, 512])
def test_fp16_kv_with_outliers_against_exact_oracle(d):
    """fp32 q, fp16 k/v with 1% of the K entries x30, causal and windowed,
    through the kernel of every head size: fp16 K/V run the fp16 products,
    so the exact oracle on the stored inputs is the reference."""
    w = workloads.custom(f"fp16kv_outliers_d{d}", [200, 1, 77, 300], 4, 2, head_dim=d,
                         q_dtype="fp32", kv_dtype="fp16", seed=140 + d, k_outlier_frac=0.01)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    for window in (0, 50):
        out = run_gpu(inp, 4, 2, d, w.attn_scale, window)
        check(f"{w.name}_w{window}", to64(out), oracle_of(inp, 4, 2, w.attn_scale, window))


def test_mla_absorbed_fp16_cache_with_outliers():
    """The absorbed 320 / 256 MLA shape over an fp16 cache with x30 outliers
    in 1% of the rope columns (256..319) of the cache rows.  v is the first
    256 columns, so the outliers touch the keys only: outliers in v would
    make outputs of magnitude ~100, whose bf16 rounding alone exceeds the
    absolute bar."""
    w = workloads.custom("mla_fp16_outliers", [150, 1, 260], 8, 1, head_dim=320,
                         q_dtype="fp32", kv_dtype="fp16", seed=146,
                         scale=1.0 / math.sqrt(320))
    _announce(w.name)
    inp = workloads.make_inputs(w)
    rope = inp["k"][:, :, 256:].to(torch.float64).contiguous()
    rng = np.random.default_rng(1460)
    idx = rng.choice(rope.numel(), size=rope.numel() // 100, replace=False)
    flat = rope.reshape(-1)
    flat[torch.from_numpy(idx)] *= 30.0
    inp["k"] = torch.cat([inp["k"][:, :, :256], rope.to(torch.float16)], dim=2)
    inp["v"] = inp["k"][:, :, :256]
    inp["head_dim_v"] = 256
    out = run_gpu(inp, 8, 1, 320, w.attn_scale, 0)
    check(w.name, to64(out), oracle_of(inp, 8, 1, w.attn_scale, 0))


def test_decode_fp16_kv_with_outliers():
    w = workloads.custom("decode_fp16_outliers", [1] * 12, 8, 2, q_dtype="fp32",
                         kv_dtype="fp16", seed=147, k_outlier_frac=0.01,
                         history=[0, 1, 63, 64, 65, 500, 1000, 7, 2000, 129, 31, 300])
    _announce(w.name)
    inp = workloads.make_inputs(w)
    inp["decode"] = True
    for window in (0, 40):
        out = run_gpu(inp, 8, 2, 128, w.attn_scale, window)
        want = oracle.attention_decode(inp["q"], inp["k"], inp["v"], inp["cu_seqlens_k"], 8, 2,
                                       w.attn_scale, window)
        check(f"{w.name}_w{window}", to64(out), want)


def test_head_dim_512_chunked_and_paged():
    w = workloads.custom("d512_chunked", [90, 33, 200, 1], 2, 1, head_dim=512, seed=133,
                         history=[300, 0, 129, 700])
    _announce(w.name)
    inp = workloads.make_inputs(w)
    for win in (0, 100):
        out = run_gpu(inp, 2, 1, 512, w.attn_scale, win)
        check(f"d512_chunked_w{win}", to64(out), oracle_of(inp, 2, 1, w.attn_scale, win))
    k_pool, v_pool, table = to_paged(inp, 64, seed=13)
    out = run_paged(inp, k_pool, v_pool, table, 64, 2, 1, w.attn_scale, 0, d=512)
    want = oracle.attention_paged(inp["q"], k_pool, v_pool, inp["cu_seqlens"], table,
                                  inp["kv_lengths"], 64, 2, 1, w.attn_scale, 0)
    check("d512_paged", to64(out), want)


def test_head_dim_512_strided_views_and_ex():
    """Head-major q and an out view inside a larger buffer; attn_prefill_ex
    with (512, 512) gives the same bits as attn_prefill."""
    dev = torch.device("cuda:0")
    w = workloads.custom("d512_views", [130, 7], 2, 1, head_dim=512, seed=134)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    T = inp["q"].shape[0]
    qh = inp["q"].permute(1, 0, 2).contiguous().permute(1, 0, 2).to(dev)
    ob = torch.full((T + 2, 2, 512), 7.0, dtype=torch.bfloat16, device=dev)
    out = ob[1:T + 1]
    cu = inp["cu_seqlens"].to(dev)
    k, v = inp["k"].to(dev), inp["v"].to(dev)
    binding.attn_prefill(qh, k, v, out, cu, 2, 1, 512, w.attn_scale, 0)
    out2 = torch.empty(T, 2, 512, dtype=torch.bfloat16, device=dev)
    binding.attn_prefill_ex(qh, k, v, out2, cu, 2, 1, 512, 512, w.attn_scale, 0)
    torch.cuda.synchronize()
    assert torch.all(ob[0].float() == 7.0) and torch.all(ob[T + 1].float() == 7.0)
    check("d512_views", to64(out), oracle_of(inp, 2, 1, w.attn_scale, 0))
    assert torch.equal(out, out2)


# ------------------------------------- absorbed MLA: q/k 320, v/out 256
def mla_inputs(name, lengths, hq, seed, history=None):
    """q [T, hq, 320]; one compressed cache row [kv_latent(256) | k_rope(64)]
    per key; k = the row, v = its first 256 columns (a view)."""
    w = workloads.custom(name, lengths, hq, 1, head_dim=320, seed=seed,
                         scale=1 / math.sqrt(320), history=history)
    inp = workloads.make_inputs(w)
    inp["v"] = inp["k"][:, :, :256]
    return w, inp


def run_mla(inp, hq, window):
    dev = torch.device("cuda:0")
    q, c = inp["q"].to(dev), inp["k"].to(dev)
    out = torch.empty(q.shape[0], hq, 256, dtype=torch.bfloat16, device=dev)
    binding.attn_prefill_ex(q, c, c[:, :, :256], out, inp["cu_seqlens"].to(dev), hq, 1, 320,
                            256, 1 / math.sqrt(320), window,
                            cu_seqlens_k=inp["cu_seqlens_k"].to(dev)
                            if "cu_seqlens_k" in inp else None)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("win", [0, 1, 100])
def test_mla_absorbed_320_256_packed(win):
    w, inp = mla_inputs("mla320", [1000, 1, 129, 0, 300], 8, seed=121)
    _announce(f"{w.name} W={win}")
    out = run_mla(inp, 8, win)
    want = oracle.attention_varlen(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"], 8, 1,
                                   1 / math.sqrt(320), win)
    check(f"mla320_w{win}", to64(out), want)


def test_mla_absorbed_320_256_chunked():
    w, inp = mla_inputs("mla320_chunked", [200, 64, 1], 16, seed=122,
                        history=[900, 0, 333])
    _announce(w.name)
    out = run_mla(inp, 16, 0)
    want = oracle.attention_chunked(inp["q"], inp["k"], inp["v"], inp["cu_seqlens"],
                                    inp["cu_seqlens_k"], 16, 1, 1 / math.sqrt(320), 0)
    check("mla320_chunked", to64(out), want)


def test_ex_same_head_sizes_match_attn_prefill_bitwise():
    dev = torch.device("cuda:0")
    w = workloads.custom("ex_256", [500, 77], 8, 2, head_dim=256, seed=123)
    _announce(w.name)
    inp = workloads.make_inputs(w)
    a = run_gpu(inp, 8, 2, 256, w.attn_scale, 0).clone()
    b = torch.empty_like(a)
    binding.attn_prefill_ex(inp["q"].to(dev), inp["k"].to(dev), inp["v"].to(dev), b,
                            inp["cu_seqlens"].to(dev), 8, 2, 256, 256, w.attn_scale, 0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ------------------------------------------------------------ graph capture
def test_graph_capture_replays_match_eager():
    """Every call is launches only (no allocation, host sync or memset), so
    it can be captured in a HIP graph: a packed GQA prefill, a prefill whose
    keys are split through a workspace and a split decode in one graph,
    replayed three times on new inputs written eagerly between replays, each
    replay equal bit for bit to eager calls on the same inputs."""
    dev = torch.device("cuda:0")
    _announce("graph_capture")
    gen = torch.Generator(device="cpu").manual_seed(91)

    def randn(*shape, dtype=torch.bfloat16):
        return torch.randn(*shape, generator=gen).to(dtype).to(dev)

    # packed GQA prefill (four heads of a KV head per workgroup)
    lens_a = [300, 129, 64]
    cu_a = torch.tensor([0, 300, 429, 493], dtype=torch.int32, device=dev)
    qa, ka, va = randn(493, 8, 128), randn(493, 2, 128), randn(493, 2, 128)
    # one long sequence on 2 query heads: keys split across workgroups
    cu_b = torch.tensor([0, 3000], dtype=torch.int32, device=dev)
    qb, kb, vb = randn(3000, 2, 128), randn(3000, 1, 128), randn(3000, 1, 128)
    ws_b_bytes = binding.prefill_workspace_size(3000, 3000, 1, 2, 1, 128, 128, 0)
    assert ws_b_bytes > 0
    ws_b = torch.full((ws_b_bytes,), 0xFF, dtype=torch.uint8, device=dev)
    # decode: 4 sequences of 2000 keys, 32 query heads on 8 KV heads, split
    cu_c = torch.tensor([0, 2000, 4000, 6000, 8000], dtype=torch.int32, device=dev)
    qc, kc, vc = randn(4, 32, 128), randn(8000, 8, 128), randn(8000, 8, 128)
    ws_c = binding.decode_workspace(4, 32, 8, 128, device=dev)
    assert ws_c is not None and ws_c.numel() > 0
    scale = 1 / math.sqrt(128)

    outs = [torch.empty(493, 8, 128, dtype=torch.bfloat16, device=dev),
            torch.empty(3000, 2, 128, dtype=torch.bfloat16, device=dev),
            torch.empty(4, 32, 128, dtype=torch.bfloat16, device=dev)]

    def calls(o):
        binding.attn_prefill(qa, ka, va, o[0], cu_a, 8, 2, 128, scale, 0)
        binding.attn_prefill_ex(qb, kb, vb, o[1], cu_b, 2, 1, 128, 128, scale, 0,
                                workspace=ws_b)
        binding.attn_decode(qc, kc, vc, o[2], cu_c, 32, 8, 128, scale, 0, workspace=ws_c)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls(outs)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(outs)
    for rep in range(3):
        for t in (qa, ka, qb, vb, qc, vc):  # new inputs, written eagerly
            t.copy_(randn(*t.shape))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        want = [torch.empty_like(o) for o in outs]
        calls(want)
        torch.cuda.synchronize()
        for name, g, w in zip(("prefill", "prefill_split", "decode_split"), got, want):
            assert torch.equal(g, w), f"replay {rep}: {name} differs from the eager call"

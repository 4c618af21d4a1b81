"""The C ABI on the CPU: the library loads, exports what the header declares,
and rejects every bad argument on the host before any HIP call.

Descriptors here carry fake, never-dereferenced device addresses: each case
fails a host check, so no kernel is launched and no GPU is needed.
"""
import ctypes
import math
import os
import re

import pytest

from causal_prefill_attention_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_prefill.h")

FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(attn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = B.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_library_shares_one_hip_runtime_with_torch():
    """Loading the library before anything imports torch still leaves one
    HIP runtime in the process (two runtimes leave the library's without a
    device)."""
    import subprocess
    import sys
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from causal_prefill_attention_amd import binding\n"
        "binding.load_library()\n"
        "import torch\n"
        "maps = open('/proc/self/maps').read().splitlines()\n"
        "print(len({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=300, check=True).stdout
    assert out.strip().splitlines()[-1] == "1"


def test_status_strings_and_head_dims():
    lib = B.load_library()
    for code in (B.ATTN_OK, B.ATTN_ERR_INVALID_ARG, B.ATTN_ERR_UNSUPPORTED,
                 B.ATTN_ERR_HIP, 99):
        assert lib.attn_prefill_status_string(code)
    assert B.supported_head_dims() == [64, 128, 256, 512]
    assert lib.attn_prefill_version() >= 100


def tens(addr, dtype, n, heads, d=128, ts=None, hs=None):
    hs = d if hs is None else hs
    ts = heads * hs if ts is None else ts
    return B.AttnTensor(addr, dtype, 0, n, ts, hs)


def base_args(n=256, hq=32, hkv=1, d=128):
    q = tens(FAKE, B.ATTN_BF16, n, hq, d)
    k = tens(FAKE + (1 << 30), B.ATTN_BF16, n, hkv, d)
    v = tens(FAKE + (2 << 30), B.ATTN_BF16, n, hkv, d)
    o = tens(FAKE + (3 << 30), B.ATTN_BF16, n, hq, d)
    s = B.AttnSeqlens(FAKE + (4 << 30), 1, 0)
    return dict(q=q, k=k, v=v, out=o, seqlens=s, n_q_heads=hq, n_kv_heads=hkv,
                head_dim=d, scale=1 / math.sqrt(d), sliding_window=0)


def call(**kw):
    return B.call_raw(kw["q"], kw["k"], kw["v"], kw["out"], kw["seqlens"],
                      kw["n_q_heads"], kw["n_kv_heads"], kw["head_dim"],
                      kw["scale"], kw["sliding_window"], None)


def with_(a, **kw):
    b = dict(a)
    b.update(kw)
    return b


def mutate(t, **kw):
    c = B.AttnTensor.from_buffer_copy(t)
    for k, val in kw.items():
        setattr(c, k, val)
    return c


BAD = [
    # (name, mutation of base_args, expected status, message fragment)
    ("zero_q_heads", lambda a: with_(a, n_q_heads=0), B.ATTN_ERR_INVALID_ARG, "n_q_heads"),
    ("zero_kv_heads", lambda a: with_(a, n_kv_heads=0), B.ATTN_ERR_INVALID_ARG, "n_kv_heads"),
    ("heads_not_multiple", lambda a: with_(a, n_q_heads=6, n_kv_heads=4),
     B.ATTN_ERR_INVALID_ARG, "multiple"),
    ("head_dim_1024_unsupported", lambda a: with_(a, head_dim=1024),
     B.ATTN_ERR_UNSUPPORTED, "head_dim 1024"),
    ("head_dim_384_unsupported", lambda a: with_(a, head_dim=384),
     B.ATTN_ERR_UNSUPPORTED, "head_dim 384"),
    ("head_dim_96_unsupported", lambda a: with_(a, head_dim=96),
     B.ATTN_ERR_UNSUPPORTED, "head_dim 96"),
    ("head_dim_zero", lambda a: with_(a, head_dim=0), B.ATTN_ERR_INVALID_ARG, "head_dim"),
    ("scale_nan", lambda a: with_(a, scale=float("nan")), B.ATTN_ERR_INVALID_ARG, "scale"),
    ("scale_inf", lambda a: with_(a, scale=float("inf")), B.ATTN_ERR_INVALID_ARG, "scale"),
    ("window_negative", lambda a: with_(a, sliding_window=-1),
     B.ATTN_ERR_INVALID_ARG, "sliding_window"),
    ("q_null_data", lambda a: with_(a, q=mutate(a["q"], data=None)),
     B.ATTN_ERR_INVALID_ARG, "q: data"),
    ("k_bad_dtype", lambda a: with_(a, k=mutate(a["k"], dtype=7)),
     B.ATTN_ERR_INVALID_ARG, "dtype"),
    ("reserved_nonzero", lambda a: with_(a, v=mutate(a["v"], reserved=1)),
     B.ATTN_ERR_INVALID_ARG, "reserved"),
    ("q_fp16_unsupported", lambda a: with_(a, q=mutate(a["q"], dtype=B.ATTN_FP16)),
     B.ATTN_ERR_UNSUPPORTED, "q dtype"),
    ("kv_fp32_unsupported", lambda a: with_(a, k=mutate(a["k"], dtype=B.ATTN_FP32),
                                            v=mutate(a["v"], dtype=B.ATTN_FP32)),
     B.ATTN_ERR_UNSUPPORTED, "k/v dtype"),
    ("kv_dtype_mismatch", lambda a: with_(a, k=mutate(a["k"], dtype=B.ATTN_FP16)),
     B.ATTN_ERR_UNSUPPORTED, "differ"),
    ("out_fp32_unsupported", lambda a: with_(a, out=mutate(a["out"], dtype=B.ATTN_FP32)),
     B.ATTN_ERR_UNSUPPORTED, "out dtype"),
    ("token_count_mismatch", lambda a: with_(a, v=mutate(a["v"], n_tokens=255)),
     B.ATTN_ERR_INVALID_ARG, "n_tokens differ"),
    ("negative_tokens", lambda a: with_(a, q=mutate(a["q"], n_tokens=-1)),
     B.ATTN_ERR_INVALID_ARG, "n_tokens"),
    ("too_many_tokens", lambda a: with_(a, q=mutate(a["q"], n_tokens=1 << 31)),
     B.ATTN_ERR_INVALID_ARG, "int32"),
    ("negative_stride", lambda a: with_(a, k=mutate(a["k"], token_stride=-128)),
     B.ATTN_ERR_INVALID_ARG, "negative stride"),
    ("overlapping_heads", lambda a: with_(a, q=mutate(a["q"], head_stride=64)),
     B.ATTN_ERR_INVALID_ARG, "overlap head vectors"),
    ("overlapping_tokens", lambda a: with_(a, q=mutate(a["q"], token_stride=31 * 128)),
     B.ATTN_ERR_INVALID_ARG, "overlap head vectors"),
    ("misaligned_pointer", lambda a: with_(a, q=mutate(a["q"], data=FAKE + 2)),
     B.ATTN_ERR_UNSUPPORTED, "aligned"),
    ("k_stride_beyond_buffer_range", lambda a: with_(a, k=mutate(a["k"], token_stride=1 << 24)),
     B.ATTN_ERR_UNSUPPORTED, "k: token stride"),
    ("v_stride_beyond_buffer_range",
     lambda a: with_(a, v=mutate(a["v"], token_stride=(1 << 24) + 8)),
     B.ATTN_ERR_UNSUPPORTED, "v: token stride"),
    ("stride_not_16_bytes", lambda a: with_(a, k=mutate(a["k"], token_stride=132)),
     B.ATTN_ERR_UNSUPPORTED, "16 bytes"),
    ("seqlens_null_data", lambda a: with_(a, seqlens=B.AttnSeqlens(None, 1, 0)),
     B.ATTN_ERR_INVALID_ARG, "cu_seqlens data"),
    ("seqlens_zero_seqs", lambda a: with_(a, seqlens=B.AttnSeqlens(FAKE, 0, 0)),
     B.ATTN_ERR_INVALID_ARG, "n_seqs"),
    ("seqlens_negative_hint", lambda a: with_(a, seqlens=B.AttnSeqlens(FAKE, 1, -5)),
     B.ATTN_ERR_INVALID_ARG, "max_seqlen"),
    ("out_aliases_q", lambda a: with_(a, out=mutate(a["out"], data=a["q"].data + 256)),
     B.ATTN_ERR_INVALID_ARG, "overlaps"),
    ("out_aliases_k", lambda a: with_(a, out=mutate(a["out"], data=a["k"].data)),
     B.ATTN_ERR_INVALID_ARG, "overlaps"),
]


@pytest.mark.parametrize("name,mut,status,frag", BAD, ids=[b[0] for b in BAD])
def test_bad_argument_rejected_on_host(name, mut, status, frag):
    rc = call(**mut(base_args()))
    assert rc == status, (rc, B.last_error())
    assert frag in B.last_error(), B.last_error()


def test_null_descriptors_rejected():
    lib = B.load_library()
    a = base_args()
    rc = lib.attn_prefill(None, ctypes.byref(a["k"]), ctypes.byref(a["v"]),
                          ctypes.byref(a["out"]), ctypes.byref(a["seqlens"]),
                          32, 1, 128, 0.1, 0, None)
    assert rc == B.ATTN_ERR_INVALID_ARG and "q: descriptor" in B.last_error()
    rc = lib.attn_prefill(ctypes.byref(a["q"]), ctypes.byref(a["k"]),
                          ctypes.byref(a["v"]), ctypes.byref(a["out"]), None,
                          32, 1, 128, 0.1, 0, None)
    assert rc == B.ATTN_ERR_INVALID_ARG and "cu_seqlens" in B.last_error()


def test_empty_batch_is_a_no_op_without_hip():
    a = base_args(n=0)
    for key in ("q", "k", "v", "out"):
        a[key] = mutate(a[key], data=None)
    assert call(**a) == B.ATTN_OK
    assert B.last_error() == ""


def test_head_major_layout_accepted_by_checks():
    # [H, T, d] strides pass the overlap check; the call then fails on the
    # next check (a misaligned out pointer) before any HIP call.
    a = base_args(n=64, hq=4)
    a["q"] = mutate(a["q"], token_stride=128, head_stride=64 * 128)
    a["out"] = mutate(a["out"], data=a["out"].data + 2)
    rc = call(**a)
    assert rc == B.ATTN_ERR_UNSUPPORTED and "out: data pointer" in B.last_error()


def test_binding_refuses_cpu_tensors():
    import torch

    q = torch.zeros(4, 1, 128, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        B.attn_prefill(q, q, q, q.clone(), cu, 1, 1, 128, 0.1)


# ---- attn_prefill_chunked: the same checks plus the history arguments


def chunked_args(nq=64, nk=256, hq=32, hkv=1, d=128):
    a = base_args(n=nq, hq=hq, hkv=hkv, d=d)
    a["k"] = mutate(a["k"], n_tokens=nk)
    a["v"] = mutate(a["v"], n_tokens=nk)
    a["seqlens_k"] = B.AttnSeqlens(FAKE + (5 << 30), 1, 0)
    return a


def call_chunked(**kw):
    return B.call_raw_chunked(kw["q"], kw["k"], kw["v"], kw["out"], kw["seqlens"],
                              kw["seqlens_k"], kw["n_q_heads"], kw["n_kv_heads"],
                              kw["head_dim"], kw["scale"], kw["sliding_window"], None)


BAD_CHUNKED = [
    ("out_tokens_differ_from_q", lambda a: with_(a, out=mutate(a["out"], n_tokens=63)),
     B.ATTN_ERR_INVALID_ARG, "q 64 out 63"),
    ("v_tokens_differ_from_k", lambda a: with_(a, v=mutate(a["v"], n_tokens=255)),
     B.ATTN_ERR_INVALID_ARG, "k 256 v 255"),
    ("no_keys_for_queries", lambda a: with_(a, k=mutate(a["k"], n_tokens=0, data=None),
                                            v=mutate(a["v"], n_tokens=0, data=None)),
     B.ATTN_ERR_INVALID_ARG, "k and v have none"),
    ("seqlens_k_null_data", lambda a: with_(a, seqlens_k=B.AttnSeqlens(None, 1, 0)),
     B.ATTN_ERR_INVALID_ARG, "cu_seqlens_k data"),
    ("seqlens_k_count_differs", lambda a: with_(a, seqlens_k=B.AttnSeqlens(FAKE, 2, 0)),
     B.ATTN_ERR_INVALID_ARG, "cu_seqlens_k 2"),
    ("seqlens_k_negative_hint", lambda a: with_(a, seqlens_k=B.AttnSeqlens(FAKE, 1, -1)),
     B.ATTN_ERR_INVALID_ARG, "max_seqlen"),
    ("k_stride_beyond_buffer_range",
     lambda a: with_(a, k=mutate(a["k"], token_stride=1 << 24)),
     B.ATTN_ERR_UNSUPPORTED, "k: token stride"),
    ("head_dim_96_unsupported", lambda a: with_(a, head_dim=96),
     B.ATTN_ERR_UNSUPPORTED, "head_dim 96"),
    ("out_aliases_v", lambda a: with_(a, out=mutate(a["out"], data=a["v"].data + 4096)),
     B.ATTN_ERR_INVALID_ARG, "overlaps"),
]


@pytest.mark.parametrize("name,mut,status,frag", BAD_CHUNKED,
                         ids=[b[0] for b in BAD_CHUNKED])
def test_chunked_bad_argument_rejected_on_host(name, mut, status, frag):
    rc = call_chunked(**mut(chunked_args()))
    assert rc == status, (rc, B.last_error())
    assert frag in B.last_error(), B.last_error()


def test_chunked_null_key_offsets_rejected():
    lib = B.load_library()
    a = chunked_args()
    rc = lib.attn_prefill_chunked(ctypes.byref(a["q"]), ctypes.byref(a["k"]),
                                  ctypes.byref(a["v"]), ctypes.byref(a["out"]),
                                  ctypes.byref(a["seqlens"]), None,
                                  32, 1, 128, 0.1, 0, None)
    assert rc == B.ATTN_ERR_INVALID_ARG and "cu_seqlens_k is NULL" in B.last_error()


def test_chunked_empty_queries_are_a_no_op_without_hip():
    # no new tokens: nothing to write, even with a KV history present
    a = chunked_args(nq=0)
    for key in ("q", "out"):
        a[key] = mutate(a[key], data=None)
    assert call_chunked(**a) == B.ATTN_OK
    assert B.last_error() == ""


# ---- attn_prefill_paged: pools, block table and key counts


def paged_args(nq=64, n_pages=8, page=64, hq=32, hkv=1, d=128):
    a = base_args(n=nq, hq=hq, hkv=hkv, d=d)
    a["k"] = mutate(a["k"], n_tokens=n_pages * page)
    a["v"] = mutate(a["v"], n_tokens=n_pages * page)
    a["paged"] = B.AttnPagedKV(FAKE + (5 << 30), FAKE + (6 << 30), 4, page)
    return a


def call_paged(**kw):
    return B.call_raw_paged(kw["q"], kw["k"], kw["v"], kw["out"], kw["seqlens"],
                            kw["paged"], kw["n_q_heads"], kw["n_kv_heads"],
                            kw["head_dim"], kw["scale"], kw["sliding_window"], None)


def _pg(a, **kw):
    c = B.AttnPagedKV.from_buffer_copy(a["paged"])
    for key, val in kw.items():
        setattr(c, key, val)
    return with_(a, paged=c)


BAD_PAGED = [
    ("page_size_not_multiple_of_64", lambda a: _pg(a, page_size=48),
     B.ATTN_ERR_UNSUPPORTED, "page_size 48"),
    ("page_size_zero", lambda a: _pg(a, page_size=0), B.ATTN_ERR_INVALID_ARG, "page_size 0"),
    ("table_stride_zero", lambda a: _pg(a, table_stride=0), B.ATTN_ERR_INVALID_ARG,
     "table_stride 0"),
    ("null_block_table", lambda a: _pg(a, block_table=None), B.ATTN_ERR_INVALID_ARG,
     "block_table"),
    ("null_seqlens_k", lambda a: _pg(a, seqlens_k=None), B.ATTN_ERR_INVALID_ARG,
     "seqlens_k"),
    ("pool_not_whole_pages", lambda a: with_(a, k=mutate(a["k"], n_tokens=500),
                                             v=mutate(a["v"], n_tokens=500)),
     B.ATTN_ERR_INVALID_ARG, "not a multiple of page_size"),
    ("pools_differ", lambda a: with_(a, v=mutate(a["v"], n_tokens=448)),
     B.ATTN_ERR_INVALID_ARG, "k 512 v 448"),
    ("empty_pool", lambda a: with_(a, k=mutate(a["k"], n_tokens=0, data=None),
                                   v=mutate(a["v"], n_tokens=0, data=None)),
     B.ATTN_ERR_INVALID_ARG, "k and v have none"),
    ("table_capacity_beyond_int32", lambda a: _pg(a, table_stride=1 << 30),
     B.ATTN_ERR_UNSUPPORTED, "exceeds int32"),
]


@pytest.mark.parametrize("name,mut,status,frag", BAD_PAGED, ids=[b[0] for b in BAD_PAGED])
def test_paged_bad_argument_rejected_on_host(name, mut, status, frag):
    rc = call_paged(**mut(paged_args()))
    assert rc == status, (rc, B.last_error())
    assert frag in B.last_error(), B.last_error()


def test_paged_null_descriptor_rejected():
    lib = B.load_library()
    a = paged_args()
    rc = lib.attn_prefill_paged(ctypes.byref(a["q"]), ctypes.byref(a["k"]),
                                ctypes.byref(a["v"]), ctypes.byref(a["out"]),
                                ctypes.byref(a["seqlens"]), None, 32, 1, 128, 0.1, 0, None)
    assert rc == B.ATTN_ERR_INVALID_ARG and "paged is NULL" in B.last_error()


def test_paged_empty_queries_are_a_no_op_without_hip():
    a = paged_args(nq=0)
    for key in ("q", "out"):
        a[key] = mutate(a[key], data=None)
    assert call_paged(**a) == B.ATTN_OK
    assert B.last_error() == ""


# ---- attn_decode / attn_decode_paged


def decode_args(n_seqs=16, nk=4096, hq=32, hkv=8, d=128):
    a = base_args(n=n_seqs, hq=hq, hkv=hkv, d=d)
    a["k"] = mutate(a["k"], n_tokens=nk)
    a["v"] = mutate(a["v"], n_tokens=nk)
    a["seqlens_k"] = B.AttnSeqlens(FAKE + (5 << 30), n_seqs, 0)
    return a


def call_decode(**kw):
    return B.call_raw_decode(kw["q"], kw["k"], kw["v"], kw["out"], kw["seqlens_k"],
                             kw["n_q_heads"], kw["n_kv_heads"], kw["head_dim"],
                             kw["scale"], kw["sliding_window"], None)


BAD_DECODE = [
    ("seq_count_differs_from_q", lambda a: with_(a, seqlens_k=B.AttnSeqlens(FAKE, 15, 0)),
     B.ATTN_ERR_INVALID_ARG, "15 sequences"),
    ("out_rows_differ", lambda a: with_(a, out=mutate(a["out"], n_tokens=15)),
     B.ATTN_ERR_INVALID_ARG, "q 16 out 15"),
    ("v_tokens_differ", lambda a: with_(a, v=mutate(a["v"], n_tokens=4095)),
     B.ATTN_ERR_INVALID_ARG, "k 4096 v 4095"),
    ("no_keys", lambda a: with_(a, k=mutate(a["k"], n_tokens=0, data=None),
                                v=mutate(a["v"], n_tokens=0, data=None)),
     B.ATTN_ERR_INVALID_ARG, "k and v have none"),
    ("head_dim_64_has_no_decode_kernel", lambda a: with_(a, head_dim=64),
     B.ATTN_ERR_UNSUPPORTED, "no decode kernel for head_dim 64"),
    ("heads_not_multiple", lambda a: with_(a, n_q_heads=30),
     B.ATTN_ERR_INVALID_ARG, "multiple"),
    ("q_fp16_unsupported", lambda a: with_(a, q=mutate(a["q"], dtype=B.ATTN_FP16)),
     B.ATTN_ERR_UNSUPPORTED, "q dtype"),
    ("scale_nan", lambda a: with_(a, scale=float("nan")), B.ATTN_ERR_INVALID_ARG, "scale"),
    ("out_aliases_k", lambda a: with_(a, out=mutate(a["out"], data=a["k"].data)),
     B.ATTN_ERR_INVALID_ARG, "overlaps"),
]


@pytest.mark.parametrize("name,mut,status,frag", BAD_DECODE, ids=[b[0] for b in BAD_DECODE])
def test_decode_bad_argument_rejected_on_host(name, mut, status, frag):
    rc = call_decode(**mut(decode_args()))
    assert rc == status, (rc, B.last_error())
    assert frag in B.last_error(), B.last_error()


def test_decode_null_arguments_rejected():
    lib = B.load_library()
    a = decode_args()
    rc = lib.attn_decode(ctypes.byref(a["q"]), ctypes.byref(a["k"]), ctypes.byref(a["v"]),
                         ctypes.byref(a["out"]), None, 32, 8, 128, 0.1, 0, None)
    assert rc == B.ATTN_ERR_INVALID_ARG and "cu_seqlens_k is NULL" in B.last_error()
    rc = lib.attn_decode_paged(ctypes.byref(a["q"]), ctypes.byref(a["k"]),
                               ctypes.byref(a["v"]), ctypes.byref(a["out"]), None,
                               32, 8, 128, 0.1, 0, None)
    assert rc == B.ATTN_ERR_INVALID_ARG and "paged is NULL" in B.last_error()


def test_decode_paged_page_size_checked():
    a = decode_args()
    pg = B.AttnPagedKV(FAKE + (6 << 30), FAKE + (7 << 30), 8, 32)
    rc = B.call_raw_decode_paged(a["q"], a["k"], a["v"], a["out"], pg, 32, 8, 128, 0.1, 0,
                                 None)
    assert rc == B.ATTN_ERR_UNSUPPORTED and "page_size 32" in B.last_error()


def call_decode_ws(workspace, nbytes, **kw):
    return B.call_raw_decode_ws(kw["q"], kw["k"], kw["v"], kw["out"], kw["seqlens_k"],
                                kw["n_q_heads"], kw["n_kv_heads"], kw["head_dim"],
                                kw["scale"], kw["sliding_window"], workspace, nbytes, None)


@pytest.mark.parametrize("name,mut,status,frag", BAD_DECODE, ids=[b[0] for b in BAD_DECODE])
def test_decode_ws_checks_the_same_arguments(name, mut, status, frag):
    rc = call_decode_ws(FAKE + (8 << 30), 1 << 20, **mut(decode_args()))
    assert rc == status, (rc, B.last_error())
    assert frag in B.last_error(), B.last_error()


def test_decode_ws_workspace_checked():
    a = decode_args()
    rc = call_decode_ws(None, 4096, **a)
    assert rc == B.ATTN_ERR_INVALID_ARG and "workspace is NULL" in B.last_error()
    rc = call_decode_ws(FAKE + (8 << 30) + 8, 4096, **a)
    assert rc == B.ATTN_ERR_INVALID_ARG and "16-byte aligned" in B.last_error()
    lib = B.load_library()
    rc = lib.attn_decode_ws(ctypes.byref(a["q"]), ctypes.byref(a["k"]), ctypes.byref(a["v"]),
                            ctypes.byref(a["out"]), None, 32, 8, 128, 0.1, 0, None, 0, None)
    assert rc == B.ATTN_ERR_INVALID_ARG and "cu_seqlens_k is NULL" in B.last_error()
    rc = lib.attn_decode_paged_ws(ctypes.byref(a["q"]), ctypes.byref(a["k"]),
                                  ctypes.byref(a["v"]), ctypes.byref(a["out"]), None,
                                  32, 8, 128, 0.1, 0, None, 0, None)
    assert rc == B.ATTN_ERR_INVALID_ARG and "paged is NULL" in B.last_error()


def test_decode_ws_paged_page_size_checked():
    a = decode_args()
    pg = B.AttnPagedKV(FAKE + (6 << 30), FAKE + (7 << 30), 8, 32)
    rc = B.call_raw_decode_paged_ws(a["q"], a["k"], a["v"], a["out"], pg, 32, 8, 128, 0.1,
                                    0, FAKE + (8 << 30), 1 << 20, None)
    assert rc == B.ATTN_ERR_UNSUPPORTED and "page_size 32" in B.last_error()


def call_decode_noalloc(**kw):
    return B.call_raw_decode_noalloc(kw["q"], kw["k"], kw["v"], kw["out"], kw["seqlens_k"],
                                     kw["n_q_heads"], kw["n_kv_heads"], kw["head_dim"],
                                     kw["scale"], kw["sliding_window"], None)


@pytest.mark.parametrize("name,mut,status,frag", BAD_DECODE, ids=[b[0] for b in BAD_DECODE])
def test_decode_noalloc_checks_the_same_arguments(name, mut, status, frag):
    rc = call_decode_noalloc(**mut(decode_args()))
    assert rc == status, (rc, B.last_error())
    assert frag in B.last_error(), B.last_error()


def test_decode_noalloc_null_offsets_and_empty_batch():
    lib = B.load_library()
    a = decode_args()
    rc = lib.attn_decode_noalloc(ctypes.byref(a["q"]), ctypes.byref(a["k"]),
                                 ctypes.byref(a["v"]), ctypes.byref(a["out"]), None, 32, 8,
                                 128, 0.1, 0, None)
    assert rc == B.ATTN_ERR_INVALID_ARG and "cu_seqlens_k is NULL" in B.last_error()
    rc = lib.attn_decode_noalloc(None, ctypes.byref(a["k"]), ctypes.byref(a["v"]),
                                 ctypes.byref(a["out"]), ctypes.byref(a["seqlens_k"]), 32, 8,
                                 128, 0.1, 0, None)
    assert rc == B.ATTN_ERR_INVALID_ARG, B.last_error()
    e = decode_args(n_seqs=0)
    for key in ("q", "out"):
        e[key] = mutate(e[key], data=None)
    assert call_decode_noalloc(**e) == B.ATTN_OK
    assert B.last_error() == ""


@pytest.mark.parametrize("args", [(0, 32, 1, 128), (4, 32, 1, 64), (4, 30, 8, 128),
                                  (4, 0, 1, 128), (-1, 32, 1, 128),
                                  ((1 << 31), 32, 1, 128), ((1 << 63) - 1, 32, 8, 128)])
def test_decode_workspace_size_is_zero_outside_the_contract(args):
    assert B.decode_workspace_size(*args) == 0


def test_decode_empty_batch_is_a_no_op_without_hip():
    a = decode_args(n_seqs=0)
    for key in ("q", "out"):
        a[key] = mutate(a[key], data=None)
    assert call_decode(**a) == B.ATTN_OK
    assert B.last_error() == ""


# ---- attn_prefill_ex: separate head sizes, one key layout


def call_ex(a, dqk, dv, seqlens_k=None, paged=None):
    return B.call_raw_ex(a["q"], a["k"], a["v"], a["out"], a["seqlens"], seqlens_k, paged,
                         a["n_q_heads"], a["n_kv_heads"], dqk, dv, a["scale"],
                         a["sliding_window"], None)


def ex_args(n=256, hq=8, dqk=320, dv=256):
    q = tens(FAKE, B.ATTN_BF16, n, hq, dqk)
    k = tens(FAKE + (1 << 30), B.ATTN_BF16, n, 1, dqk)
    v = tens(FAKE + (1 << 30), B.ATTN_BF16, n, 1, dv, ts=dqk)  # view of k's first columns
    o = tens(FAKE + (3 << 30), B.ATTN_BF16, n, hq, dv)
    s = B.AttnSeqlens(FAKE + (4 << 30), 1, 0)
    return dict(q=q, k=k, v=v, out=o, seqlens=s, n_q_heads=hq, n_kv_heads=1, head_dim=dqk,
                scale=1 / math.sqrt(dqk), sliding_window=0)


def test_ex_rejects_unsupported_head_pairs():
    a = ex_args()
    assert call_ex(a, 320, 128) == B.ATTN_ERR_UNSUPPORTED
    assert "head_dim 320 / head_dim_v 128" in B.last_error()
    assert call_ex(a, 512, 256) == B.ATTN_ERR_UNSUPPORTED
    assert "head_dim 512 / head_dim_v 256" in B.last_error()
    assert call_ex(a, 1024, 1024) == B.ATTN_ERR_UNSUPPORTED
    assert call_ex(a, 320, 0) == B.ATTN_ERR_INVALID_ARG and "head_dim_v" in B.last_error()


def test_ex_checks_v_and_out_with_their_own_head_size():
    a = ex_args()
    # out described with 256-wide heads but a 200-element head stride overlaps
    bad = with_(a, out=mutate(a["out"], head_stride=200, token_stride=8 * 256))
    assert call_ex(bad, 320, 256) == B.ATTN_ERR_INVALID_ARG
    assert "out: strides" in B.last_error() or "overlap" in B.last_error()


def test_ex_rejects_history_and_pages_together():
    a = ex_args()
    pg = B.AttnPagedKV(FAKE + (6 << 30), FAKE + (7 << 30), 4, 64)
    rc = call_ex(a, 320, 256, seqlens_k=B.AttnSeqlens(FAKE, 1, 0), paged=pg)
    assert rc == B.ATTN_ERR_INVALID_ARG and "both set" in B.last_error()


def test_ex_empty_batch_is_a_no_op_without_hip():
    a = ex_args(n=0)
    for key in ("q", "k", "v", "out"):
        a[key] = mutate(a[key], data=None)
    assert call_ex(a, 320, 256) == B.ATTN_OK


# ---- attn_prefill_ex_ws: keys split across workgroups through a workspace


def call_ex_ws(a, dqk, dv, workspace, nbytes, seqlens_k=None, paged=None):
    return B.call_raw_ex_ws(a["q"], a["k"], a["v"], a["out"], a["seqlens"], seqlens_k, paged,
                            a["n_q_heads"], a["n_kv_heads"], dqk, dv, a["scale"],
                            a["sliding_window"], workspace, nbytes, None)


@pytest.mark.parametrize("name,mut,status,frag", BAD, ids=[b[0] for b in BAD])
def test_prefill_ws_checks_the_same_arguments(name, mut, status, frag):
    a = mut(base_args())
    rc = call_ex_ws(a, a["head_dim"], a["head_dim"], FAKE + (8 << 30), 1 << 20)
    assert rc == status, (rc, B.last_error())
    assert frag in B.last_error(), B.last_error()


def test_prefill_ws_workspace_checked():
    a = base_args()
    rc = call_ex_ws(a, 128, 128, None, 4096)
    assert rc == B.ATTN_ERR_INVALID_ARG and "workspace is NULL" in B.last_error()
    rc = call_ex_ws(a, 128, 128, FAKE + (8 << 30) + 4, 4096)
    assert rc == B.ATTN_ERR_INVALID_ARG and "16-byte aligned" in B.last_error()
    pg = B.AttnPagedKV(FAKE + (6 << 30), FAKE + (7 << 30), 8, 64)
    rc = call_ex_ws(a, 128, 128, None, 0, seqlens_k=B.AttnSeqlens(FAKE + (5 << 30), 1, 0),
                    paged=pg)
    assert rc == B.ATTN_ERR_INVALID_ARG and "both set" in B.last_error()


def test_prefill_ws_unsupported_pairs_rejected_like_ex():
    a = ex_args()
    assert call_ex_ws(a, 320, 128, None, 0) == B.ATTN_ERR_UNSUPPORTED
    assert "head_dim 320 / head_dim_v 128" in B.last_error()


@pytest.mark.parametrize("args", [(0, 100, 1, 4, 1, 128, 128, 0),
                                  (100, 100, 0, 4, 1, 128, 128, 0),
                                  (100, 100, 1, 6, 4, 128, 128, 0),
                                  (100, -1, 1, 4, 1, 128, 128, 0),
                                  (100, 100, 1, 4, 1, 128, 128, -1),
                                  (8192, 8192, 1, 4, 1, 320, 256, 0),
                                  (8192, 8192, 1, 4, 1, 256, 256, 0),
                                  ((1 << 31), 8192, 1, 4, 1, 128, 128, 0),
                                  (8192, (1 << 31), 1, 4, 1, 128, 128, 0),
                                  ((1 << 63) - 1, (1 << 63) - 1, 1, 4, 1, 128, 128, 0)])
def test_prefill_workspace_size_is_zero_outside_the_split(args):
    # bad shapes, and head sizes without a split (also zero with no GPU)
    assert B.prefill_workspace_size(*args) == 0

"""ctypes binding of libattn_prefill.so -- argument marshalling only.

Torch provides device memory and the stream; every step of the attention
runs in the library's HIP kernels.  There is no CPU path: if the library is
missing or a tensor is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "libattn_prefill.so")

ATTN_OK = 0
ATTN_ERR_INVALID_ARG = 1
ATTN_ERR_UNSUPPORTED = 2
ATTN_ERR_HIP = 3

ATTN_BF16 = 0
ATTN_FP16 = 1
ATTN_FP32 = 2

#: Every symbol include/attn_prefill.h declares.
EXPORTS = ("attn_prefill", "attn_prefill_chunked", "attn_prefill_paged", "attn_prefill_ex",
           "attn_decode", "attn_decode_paged", "attn_decode_ws", "attn_decode_paged_ws",
           "attn_decode_noalloc",
           "attn_decode_workspace_size", "attn_prefill_ex_ws", "attn_prefill_workspace_size",
           "attn_prefill_status_string",
           "attn_prefill_last_error", "attn_prefill_supported_head_dims",
           "attn_prefill_version")


class AttnTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("n_tokens", ctypes.c_int64),
                ("token_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64)]


class AttnSeqlens(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("n_seqs", ctypes.c_int32),
                ("max_seqlen", ctypes.c_int32)]


class AttnPagedKV(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("seqlens_k", ctypes.c_void_p),
                ("table_stride", ctypes.c_int32), ("page_size", ctypes.c_int32)]


class AttnPrefillError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"attn_prefill failed ({status}): {message}")
        self.status = status
        self.message = message


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads the HIP library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with "
            "`python -m causal_prefill_attention_amd.build_lib` "
            "(there is no CPU fallback)")
    # torch first: its bundled HIP runtime carries the soname the library
    # asks for, so the library then shares torch's runtime (devices, streams,
    # memory).  Loaded first, the library would pull in the system runtime
    # and torch a second one, and the library's would see no device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    lib.attn_prefill.restype = ctypes.c_int
    lib.attn_prefill.argtypes = [
        ctypes.POINTER(AttnTensor), ctypes.POINTER(AttnTensor),
        ctypes.POINTER(AttnTensor), ctypes.POINTER(AttnTensor),
        ctypes.POINTER(AttnSeqlens), ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p]
    lib.attn_prefill_chunked.restype = ctypes.c_int
    lib.attn_prefill_chunked.argtypes = [
        ctypes.POINTER(AttnTensor), ctypes.POINTER(AttnTensor),
        ctypes.POINTER(AttnTensor), ctypes.POINTER(AttnTensor),
        ctypes.POINTER(AttnSeqlens), ctypes.POINTER(AttnSeqlens), ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p]
    lib.attn_prefill_paged.restype = ctypes.c_int
    lib.attn_prefill_paged.argtypes = [
        ctypes.POINTER(AttnTensor), ctypes.POINTER(AttnTensor),
        ctypes.POINTER(AttnTensor), ctypes.POINTER(AttnTensor),
        ctypes.POINTER(AttnSeqlens), ctypes.POINTER(AttnPagedKV), ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p]
    lib.attn_prefill_ex.restype = ctypes.c_int
    lib.attn_prefill_ex.argtypes = [
        ctypes.POINTER(AttnTensor), ctypes.POINTER(AttnTensor),
        ctypes.POINTER(AttnTensor), ctypes.POINTER(AttnTensor),
        ctypes.POINTER(AttnSeqlens), ctypes.POINTER(AttnSeqlens),
        ctypes.POINTER(AttnPagedKV), ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p]
    lib.attn_prefill_ex_ws.restype = ctypes.c_int
    lib.attn_prefill_ex_ws.argtypes = lib.attn_prefill_ex.argtypes[:-1] + [
        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.attn_prefill_workspace_size.restype = ctypes.c_size_t
    lib.attn_prefill_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                ctypes.c_int32, ctypes.c_int32]
    lib.attn_decode.restype = ctypes.c_int
    lib.attn_decode.argtypes = [
        ctypes.POINTER(AttnTensor), ctypes.POINTER(AttnTensor),
        ctypes.POINTER(AttnTensor), ctypes.POINTER(AttnTensor),
        ctypes.POINTER(AttnSeqlens), ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p]
    lib.attn_decode_paged.restype = ctypes.c_int
    lib.attn_decode_paged.argtypes = [
        ctypes.POINTER(AttnTensor), ctypes.POINTER(AttnTensor),
        ctypes.POINTER(AttnTensor), ctypes.POINTER(AttnTensor),
        ctypes.POINTER(AttnPagedKV), ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_float, ctypes.c_int32, ctypes.c_void_p]
    lib.attn_decode_ws.restype = ctypes.c_int
    lib.attn_decode_ws.argtypes = lib.attn_decode.argtypes[:-1] + [
        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.attn_decode_paged_ws.restype = ctypes.c_int
    lib.attn_decode_paged_ws.argtypes = lib.attn_decode_paged.argtypes[:-1] + [
        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.attn_decode_noalloc.restype = ctypes.c_int
    lib.attn_decode_noalloc.argtypes = lib.attn_decode.argtypes
    lib.attn_decode_workspace_size.restype = ctypes.c_size_t
    lib.attn_decode_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_int32]
    lib.attn_prefill_status_string.restype = ctypes.c_char_p
    lib.attn_prefill_status_string.argtypes = [ctypes.c_int]
    lib.attn_prefill_last_error.restype = ctypes.c_char_p
    lib.attn_prefill_last_error.argtypes = []
    lib.attn_prefill_supported_head_dims.restype = ctypes.c_int
    lib.attn_prefill_supported_head_dims.argtypes = [
        ctypes.POINTER(ctypes.c_int32), ctypes.c_int32]
    lib.attn_prefill_version.restype = ctypes.c_int
    lib.attn_prefill_version.argtypes = []
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().attn_prefill_last_error().decode()


def supported_head_dims():
    lib = load_library()
    n = lib.attn_prefill_supported_head_dims(None, 0)
    arr = (ctypes.c_int32 * n)()
    lib.attn_prefill_supported_head_dims(arr, n)
    return list(arr)


def call_raw(q: AttnTensor, k: AttnTensor, v: AttnTensor, out: AttnTensor,
             seqlens: AttnSeqlens, n_q_heads: int, n_kv_heads: int,
             head_dim: int, scale: float, sliding_window: int,
             stream: Optional[int] = None) -> int:
    """Calls the C entry point with prepared descriptors; returns the status."""
    lib = load_library()
    return lib.attn_prefill(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                            ctypes.byref(out), ctypes.byref(seqlens),
                            int(n_q_heads), int(n_kv_heads), int(head_dim),
                            float(scale), int(sliding_window),
                            ctypes.c_void_p(stream))


def call_raw_chunked(q: AttnTensor, k: AttnTensor, v: AttnTensor, out: AttnTensor,
                     seqlens_q: AttnSeqlens, seqlens_k: AttnSeqlens, n_q_heads: int,
                     n_kv_heads: int, head_dim: int, scale: float,
                     sliding_window: int, stream: Optional[int] = None) -> int:
    """Calls ``attn_prefill_chunked`` with prepared descriptors; returns the status."""
    lib = load_library()
    return lib.attn_prefill_chunked(
        ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(out),
        ctypes.byref(seqlens_q), ctypes.byref(seqlens_k), int(n_q_heads),
        int(n_kv_heads), int(head_dim), float(scale), int(sliding_window),
        ctypes.c_void_p(stream))


def call_raw_paged(q: AttnTensor, k_pool: AttnTensor, v_pool: AttnTensor,
                   out: AttnTensor, seqlens_q: AttnSeqlens, paged: AttnPagedKV,
                   n_q_heads: int, n_kv_heads: int, head_dim: int, scale: float,
                   sliding_window: int, stream: Optional[int] = None) -> int:
    """Calls ``attn_prefill_paged`` with prepared descriptors; returns the status."""
    lib = load_library()
    return lib.attn_prefill_paged(
        ctypes.byref(q), ctypes.byref(k_pool), ctypes.byref(v_pool), ctypes.byref(out),
        ctypes.byref(seqlens_q), ctypes.byref(paged), int(n_q_heads), int(n_kv_heads),
        int(head_dim), float(scale), int(sliding_window), ctypes.c_void_p(stream))


def call_raw_ex(q: AttnTensor, k: AttnTensor, v: AttnTensor, out: AttnTensor,
                seqlens_q: AttnSeqlens, seqlens_k: Optional[AttnSeqlens],
                paged: Optional[AttnPagedKV], n_q_heads: int, n_kv_heads: int,
                head_dim_qk: int, head_dim_v: int, scale: float, sliding_window: int,
                stream: Optional[int] = None) -> int:
    """Calls ``attn_prefill_ex`` with prepared descriptors; returns the status."""
    lib = load_library()
    return lib.attn_prefill_ex(
        ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(out),
        ctypes.byref(seqlens_q), ctypes.byref(seqlens_k) if seqlens_k is not None else None,
        ctypes.byref(paged) if paged is not None else None, int(n_q_heads), int(n_kv_heads),
        int(head_dim_qk), int(head_dim_v), float(scale), int(sliding_window),
        ctypes.c_void_p(stream))


def call_raw_ex_ws(q: AttnTensor, k: AttnTensor, v: AttnTensor, out: AttnTensor,
                   seqlens_q: AttnSeqlens, seqlens_k: Optional[AttnSeqlens],
                   paged: Optional[AttnPagedKV], n_q_heads: int, n_kv_heads: int,
                   head_dim_qk: int, head_dim_v: int, scale: float, sliding_window: int,
                   workspace: Optional[int], workspace_bytes: int,
                   stream: Optional[int] = None) -> int:
    """Calls ``attn_prefill_ex_ws`` with prepared descriptors; returns the status."""
    lib = load_library()
    return lib.attn_prefill_ex_ws(
        ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(out),
        ctypes.byref(seqlens_q), ctypes.byref(seqlens_k) if seqlens_k is not None else None,
        ctypes.byref(paged) if paged is not None else None, int(n_q_heads), int(n_kv_heads),
        int(head_dim_qk), int(head_dim_v), float(scale), int(sliding_window),
        ctypes.c_void_p(workspace), int(workspace_bytes), ctypes.c_void_p(stream))


def prefill_workspace_size(n_tokens_q: int, max_keys: int, n_seqs: int, n_q_heads: int,
                           n_kv_heads: int, head_dim_qk: int, head_dim_v: int,
                           sliding_window: int = 0) -> int:
    """Bytes of workspace with which ``attn_prefill_ex_ws`` splits a call on
    the current device (0: it would not split)."""
    return int(load_library().attn_prefill_workspace_size(
        int(n_tokens_q), int(max_keys), int(n_seqs), int(n_q_heads), int(n_kv_heads),
        int(head_dim_qk), int(head_dim_v), int(sliding_window)))


def prefill_workspace(n_tokens_q: int, max_keys: int, n_seqs: int, n_q_heads: int,
                      n_kv_heads: int, head_dim_qk: int, head_dim_v: int,
                      sliding_window: int = 0, device="cuda"):
    """A workspace tensor (uint8) sized by ``prefill_workspace_size``."""
    import torch

    n = prefill_workspace_size(n_tokens_q, max_keys, n_seqs, n_q_heads, n_kv_heads,
                               head_dim_qk, head_dim_v, sliding_window)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def call_raw_decode(q: AttnTensor, k: AttnTensor, v: AttnTensor, out: AttnTensor,
                    seqlens_k: AttnSeqlens, n_q_heads: int, n_kv_heads: int,
                    head_dim: int, scale: float, sliding_window: int,
                    stream: Optional[int] = None) -> int:
    """Calls ``attn_decode`` with prepared descriptors; returns the status."""
    lib = load_library()
    return lib.attn_decode(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                           ctypes.byref(out), ctypes.byref(seqlens_k), int(n_q_heads),
                           int(n_kv_heads), int(head_dim), float(scale),
                           int(sliding_window), ctypes.c_void_p(stream))


def call_raw_decode_paged(q: AttnTensor, k_pool: AttnTensor, v_pool: AttnTensor,
                          out: AttnTensor, paged: AttnPagedKV, n_q_heads: int,
                          n_kv_heads: int, head_dim: int, scale: float,
                          sliding_window: int, stream: Optional[int] = None) -> int:
    """Calls ``attn_decode_paged`` with prepared descriptors; returns the status."""
    lib = load_library()
    return lib.attn_decode_paged(ctypes.byref(q), ctypes.byref(k_pool), ctypes.byref(v_pool),
                                 ctypes.byref(out), ctypes.byref(paged), int(n_q_heads),
                                 int(n_kv_heads), int(head_dim), float(scale),
                                 int(sliding_window), ctypes.c_void_p(stream))


def call_raw_decode_ws(q: AttnTensor, k: AttnTensor, v: AttnTensor, out: AttnTensor,
                       seqlens_k: AttnSeqlens, n_q_heads: int, n_kv_heads: int,
                       head_dim: int, scale: float, sliding_window: int,
                       workspace: Optional[int], workspace_bytes: int,
                       stream: Optional[int] = None) -> int:
    """Calls ``attn_decode_ws`` with prepared descriptors; returns the status."""
    lib = load_library()
    return lib.attn_decode_ws(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                              ctypes.byref(out), ctypes.byref(seqlens_k), int(n_q_heads),
                              int(n_kv_heads), int(head_dim), float(scale),
                              int(sliding_window), ctypes.c_void_p(workspace),
                              int(workspace_bytes), ctypes.c_void_p(stream))


def call_raw_decode_paged_ws(q: AttnTensor, k_pool: AttnTensor, v_pool: AttnTensor,
                             out: AttnTensor, paged: AttnPagedKV, n_q_heads: int,
                             n_kv_heads: int, head_dim: int, scale: float,
                             sliding_window: int, workspace: Optional[int],
                             workspace_bytes: int, stream: Optional[int] = None) -> int:
    """Calls ``attn_decode_paged_ws`` with prepared descriptors; returns the status."""
    lib = load_library()
    return lib.attn_decode_paged_ws(ctypes.byref(q), ctypes.byref(k_pool),
                                    ctypes.byref(v_pool), ctypes.byref(out),
                                    ctypes.byref(paged), int(n_q_heads), int(n_kv_heads),
                                    int(head_dim), float(scale), int(sliding_window),
                                    ctypes.c_void_p(workspace), int(workspace_bytes),
                                    ctypes.c_void_p(stream))


def call_raw_decode_noalloc(q: AttnTensor, k: AttnTensor, v: AttnTensor, out: AttnTensor,
                            seqlens_k: AttnSeqlens, n_q_heads: int, n_kv_heads: int,
                            head_dim: int, scale: float, sliding_window: int,
                            stream: Optional[int] = None) -> int:
    """Calls ``attn_decode_noalloc`` with prepared descriptors; returns the status."""
    lib = load_library()
    return lib.attn_decode_noalloc(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                   ctypes.byref(out), ctypes.byref(seqlens_k), int(n_q_heads),
                                   int(n_kv_heads), int(head_dim), float(scale),
                                   int(sliding_window), ctypes.c_void_p(stream))


def decode_workspace_size(n_seqs: int, n_q_heads: int, n_kv_heads: int,
                          head_dim: int) -> int:
    """Bytes of workspace with which a decode batch uses its preferred split
    of the keys across workgroups on the current device (0: no split)."""
    return int(load_library().attn_decode_workspace_size(int(n_seqs), int(n_q_heads),
                                                         int(n_kv_heads), int(head_dim)))


def decode_workspace(n_seqs: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                     device="cuda"):
    """A workspace tensor (uint8) sized by ``decode_workspace_size``."""
    import torch

    n = decode_workspace_size(n_seqs, n_q_heads, n_kv_heads, head_dim)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def _workspace_ptr(workspace):
    if workspace is None:
        return None, 0
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _dtype_code(t) -> int:
    import torch

    codes = {torch.bfloat16: ATTN_BF16, torch.float16: ATTN_FP16,
             torch.float32: ATTN_FP32}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def describe(t) -> AttnTensor:
    """Descriptor of a [T, H, d] device tensor with a contiguous last axis."""
    if not t.is_cuda:
        raise ValueError("tensor is not on the GPU (there is no CPU path)")
    if t.dim() != 3:
        raise ValueError(f"expected [tokens, heads, head_dim], got {tuple(t.shape)}")
    if t.shape[2] > 1 and t.stride(2) != 1:
        raise ValueError("the head_dim axis must be contiguous")
    return AttnTensor(t.data_ptr() if t.numel() else None, _dtype_code(t), 0,
                      t.shape[0], t.stride(0), t.stride(1))


def attn_prefill(q, k, v, out, cu_seqlens, n_q_heads: int, n_kv_heads: int,
                 head_dim: int, scale: float, sliding_window: int = 0,
                 stream=None) -> None:
    """Runs the HIP kernel; ``out`` is written in place.

    q: [T, n_q_heads, head_dim] bf16/fp32; k, v: [T, n_kv_heads, head_dim]
    bf16/fp16; out: [T, n_q_heads, head_dim] bf16; cu_seqlens: int32 device
    tensor of n_seqs + 1 offsets.  ``stream`` defaults to torch's current
    stream on q's device.
    """
    seq = _seqlens(cu_seqlens, "cu_seqlens")
    status = call_raw(describe(q), describe(k), describe(v), describe(out), seq,
                      n_q_heads, n_kv_heads, head_dim, scale, sliding_window,
                      _stream_handle(q, stream))
    if status != ATTN_OK:
        raise AttnPrefillError(status, last_error())


def attn_prefill_chunked(q, k, v, out, cu_seqlens_q, cu_seqlens_k, n_q_heads: int,
                         n_kv_heads: int, head_dim: int, scale: float,
                         sliding_window: int = 0, stream=None) -> None:
    """Chunked prefill against a KV history; ``out`` is written in place.

    q, out: [Tq, heads, head_dim] packed by ``cu_seqlens_q``; k, v:
    [Tk, n_kv_heads, head_dim] packed by ``cu_seqlens_k`` (same number of
    sequences, each sequence's keys being its history followed by its new
    tokens).
    """
    sq = _seqlens(cu_seqlens_q, "cu_seqlens_q")
    sk = _seqlens(cu_seqlens_k, "cu_seqlens_k")
    status = call_raw_chunked(describe(q), describe(k), describe(v), describe(out),
                              sq, sk, n_q_heads, n_kv_heads, head_dim, scale,
                              sliding_window, _stream_handle(q, stream))
    if status != ATTN_OK:
        raise AttnPrefillError(status, last_error())


def attn_prefill_paged(q, k_pool, v_pool, out, cu_seqlens_q, block_table, seqlens_k,
                       page_size: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                       scale: float, sliding_window: int = 0, stream=None) -> None:
    """Chunked prefill against a paged K/V cache; ``out`` is written in place.

    k_pool, v_pool: [n_pages * page_size, n_kv_heads, head_dim] token slots;
    block_table: int32 GPU tensor [n_seqs, table_stride] of page numbers;
    seqlens_k: int32 GPU tensor [n_seqs] of keys per sequence.
    """
    import torch

    sq = _seqlens(cu_seqlens_q, "cu_seqlens_q")
    pg = _paged(block_table, seqlens_k, page_size, sq.n_seqs)
    status = call_raw_paged(describe(q), describe(k_pool), describe(v_pool), describe(out),
                            sq, pg, n_q_heads, n_kv_heads, head_dim, scale,
                            sliding_window, _stream_handle(q, stream))
    if status != ATTN_OK:
        raise AttnPrefillError(status, last_error())


def attn_prefill_ex(q, k, v, out, cu_seqlens_q, n_q_heads: int, n_kv_heads: int,
                    head_dim_qk: int, head_dim_v: int, scale: float, sliding_window: int = 0,
                    cu_seqlens_k=None, stream=None, paged=None, workspace=None) -> None:
    """Prefill with separate q/k and v/out head sizes (e.g. 320 / 256, the
    absorbed MLA layout, where v may be a view of k's first 256 columns);
    with ``cu_seqlens_k`` the keys carry a history as in
    ``attn_prefill_chunked``; with ``paged = (block_table, seqlens_k,
    page_size)`` k and v are page pools as in ``attn_prefill_paged``.  With
    ``workspace`` (see ``prefill_workspace``) a call that would not fill the
    chip splits each query tile's keys across workgroups
    (``attn_prefill_ex_ws``)."""
    sq = _seqlens(cu_seqlens_q, "cu_seqlens_q")
    sk = _seqlens(cu_seqlens_k, "cu_seqlens_k") if cu_seqlens_k is not None else None
    pg = _paged(*paged, sq.n_seqs) if paged is not None else None
    if workspace is None:
        status = call_raw_ex(describe(q), describe(k), describe(v), describe(out), sq, sk, pg,
                             n_q_heads, n_kv_heads, head_dim_qk, head_dim_v, scale,
                             sliding_window, _stream_handle(q, stream))
    else:
        ptr, nbytes = _workspace_ptr(workspace)
        status = call_raw_ex_ws(describe(q), describe(k), describe(v), describe(out), sq, sk,
                                pg, n_q_heads, n_kv_heads, head_dim_qk, head_dim_v, scale,
                                sliding_window, ptr, nbytes, _stream_handle(q, stream))
    if status != ATTN_OK:
        raise AttnPrefillError(status, last_error())


def attn_decode(q, k, v, out, cu_seqlens_k, n_q_heads: int, n_kv_heads: int,
                head_dim: int, scale: float, sliding_window: int = 0, stream=None,
                workspace=None) -> None:
    """One decode step: q, out [n_seqs, heads, head_dim]; k, v packed by
    ``cu_seqlens_k`` (each sequence's query sits after its last key).  With
    ``workspace`` (see ``decode_workspace``) a small batch splits each
    sequence's keys across workgroups (``attn_decode_ws``)."""
    sk = _seqlens(cu_seqlens_k, "cu_seqlens_k")
    if workspace is None:
        status = call_raw_decode(describe(q), describe(k), describe(v), describe(out), sk,
                                 n_q_heads, n_kv_heads, head_dim, scale, sliding_window,
                                 _stream_handle(q, stream))
    else:
        ptr, nbytes = _workspace_ptr(workspace)
        status = call_raw_decode_ws(describe(q), describe(k), describe(v), describe(out), sk,
                                    n_q_heads, n_kv_heads, head_dim, scale, sliding_window,
                                    ptr, nbytes, _stream_handle(q, stream))
    if status != ATTN_OK:
        raise AttnPrefillError(status, last_error())


def attn_decode_noalloc(q, k, v, out, cu_seqlens_k, n_q_heads: int, n_kv_heads: int,
                        head_dim: int, scale: float, sliding_window: int = 0,
                        stream=None) -> None:
    """``attn_decode`` that allocates nothing: a small batch splits its keys
    through the library's static device scratch (``attn_decode_noalloc``)."""
    sk = _seqlens(cu_seqlens_k, "cu_seqlens_k")
    status = call_raw_decode_noalloc(describe(q), describe(k), describe(v), describe(out), sk,
                                     n_q_heads, n_kv_heads, head_dim, scale, sliding_window,
                                     _stream_handle(q, stream))
    if status != ATTN_OK:
        raise AttnPrefillError(status, last_error())


def attn_decode_paged(q, k_pool, v_pool, out, block_table, seqlens_k, page_size: int,
                      n_q_heads: int, n_kv_heads: int, head_dim: int, scale: float,
                      sliding_window: int = 0, stream=None, workspace=None) -> None:
    """One decode step against a paged K/V cache (see attn_prefill_paged);
    ``workspace`` as for ``attn_decode``."""
    import torch

    for t, name in ((block_table, "block_table"), (seqlens_k, "seqlens_k")):
        if not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 GPU tensor")
    if block_table.dim() != 2 or seqlens_k.dim() != 1:
        raise ValueError("block_table must be [n_seqs, width], seqlens_k [n_seqs]")
    if block_table.shape[0] != q.shape[0] or seqlens_k.shape[0] != q.shape[0]:
        raise ValueError("block_table / seqlens_k rows must match the sequences")
    pg = AttnPagedKV(block_table.data_ptr(), seqlens_k.data_ptr(), block_table.shape[1],
                     page_size)
    if workspace is None:
        status = call_raw_decode_paged(describe(q), describe(k_pool), describe(v_pool),
                                       describe(out), pg, n_q_heads, n_kv_heads, head_dim,
                                       scale, sliding_window, _stream_handle(q, stream))
    else:
        ptr, nbytes = _workspace_ptr(workspace)
        status = call_raw_decode_paged_ws(describe(q), describe(k_pool), describe(v_pool),
                                          describe(out), pg, n_q_heads, n_kv_heads, head_dim,
                                          scale, sliding_window, ptr, nbytes,
                                          _stream_handle(q, stream))
    if status != ATTN_OK:
        raise AttnPrefillError(status, last_error())


def _paged(block_table, seqlens_k, page_size: int, n_seqs: int) -> AttnPagedKV:
    import torch

    for t, name in ((block_table, "block_table"), (seqlens_k, "seqlens_k")):
        if not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 GPU tensor")
    if block_table.dim() != 2 or seqlens_k.dim() != 1:
        raise ValueError("block_table must be [n_seqs, width], seqlens_k [n_seqs]")
    if block_table.shape[0] != n_seqs or seqlens_k.shape[0] != n_seqs:
        raise ValueError("block_table / seqlens_k rows must match the sequences")
    return AttnPagedKV(block_table.data_ptr(), seqlens_k.data_ptr(), block_table.shape[1],
                       page_size)


def _seqlens(cu, name: str) -> AttnSeqlens:
    import torch

    if not cu.is_cuda or cu.dtype != torch.int32:
        raise ValueError(f"{name} must be an int32 GPU tensor")
    if cu.dim() != 1 or cu.numel() < 2 or cu.stride(0) != 1:
        raise ValueError(f"{name} must be a contiguous 1-D tensor of n_seqs + 1")
    return AttnSeqlens(cu.data_ptr(), cu.numel() - 1, 0)


def _stream_handle(q, stream):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream

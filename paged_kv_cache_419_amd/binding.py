"""ctypes binding of libpagedkv.so: argument marshalling only.

Every step of the data plane runs in the HIP library; this module turns torch
tensors into device pointers and sizes, passes torch's current HIP stream, and
raises on a non-OK status.  There is no fallback: without the built library
(or without a GPU) every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PKV_OK, PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_HIP = 0, 1, 2, 3
_STATUS = {1: "invalid argument", 2: "unsupported", 3: "HIP error"}

EXPORTS = (
    "pkv_store_kvcache",
    "pkv_decode_workspace_bytes",
    "pkv_decode_split_tokens",
    "pkv_paged_decode_attention",
    "pkv_store_and_decode",
    "pkv_topk_sample",
    "pkv_prefill_workspace_bytes",
    "pkv_varlen_prefill_attention",
    "pkv_varlen_prefill_attention_noalloc",
    "pkv_last_error",
    "pkv_version",
    "pkv_bm_create",
    "pkv_bm_destroy",
    "pkv_bm_num_free",
    "pkv_bm_allocate",
    "pkv_bm_append",
    "pkv_bm_free",
    "pkv_bm_seq_len",
    "pkv_bm_block_table",
    "pkv_bm_slots",
    "pkv_bm_ref_count",
)


class PagedKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def _declare_block_manager(lib: ctypes.CDLL) -> None:
    """Argument and result types of the block manager's entry points (pkv_bm_*)."""
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.pkv_bm_create.argtypes = [i32, i32]
    lib.pkv_bm_create.restype = vp
    lib.pkv_bm_destroy.argtypes = [vp]
    lib.pkv_bm_destroy.restype = None
    lib.pkv_bm_num_free.argtypes = [vp]
    lib.pkv_bm_num_free.restype = i32
    lib.pkv_bm_allocate.argtypes = [vp, i64, i32p, i32]
    lib.pkv_bm_allocate.restype = i32
    lib.pkv_bm_append.argtypes = [vp, i64, i32]
    lib.pkv_bm_append.restype = i32
    lib.pkv_bm_free.argtypes = [vp, i64]
    lib.pkv_bm_free.restype = i32
    lib.pkv_bm_seq_len.argtypes = [vp, i64]
    lib.pkv_bm_seq_len.restype = i32
    lib.pkv_bm_block_table.argtypes = [vp, i64, i32p, i32]
    lib.pkv_bm_block_table.restype = i32
    lib.pkv_bm_slots.argtypes = [vp, i64, i32, i32, i32p]
    lib.pkv_bm_slots.restype = i32
    lib.pkv_bm_ref_count.argtypes = [vp, i32]
    lib.pkv_bm_ref_count.restype = i32


def load_block_manager(path: str) -> ctypes.CDLL:
    """A host-only build of the block manager (its pkv_bm_* entry points alone),
    such as the sanitizer build the CPU tests make; the data-plane calls are not in it."""
    lib = ctypes.CDLL(path)
    _declare_block_manager(lib)
    return lib


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the library once (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -m paged_kv_cache_419_amd.build`")
    lib = ctypes.CDLL(p)
    i32, i64, f32, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    lib.pkv_store_kvcache.argtypes = [vp, vp, vp, vp, vp, i64, i32, i32, i64, vp]
    lib.pkv_store_kvcache.restype = ctypes.c_int
    lib.pkv_decode_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.pkv_decode_workspace_bytes.restype = sz
    lib.pkv_decode_split_tokens.argtypes = [i32, i32, i32, i32, i32]
    lib.pkv_decode_split_tokens.restype = i32
    lib.pkv_paged_decode_attention.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                               i32, i32, f32, i32, vp, sz, vp]
    lib.pkv_paged_decode_attention.restype = ctypes.c_int
    lib.pkv_store_and_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                         i32, i32, i32, i64, f32, i32, vp, sz, vp]
    lib.pkv_store_and_decode.restype = ctypes.c_int
    lib.pkv_topk_sample.argtypes = [vp, vp, vp, i64, i64, i32, f32, vp]
    lib.pkv_topk_sample.restype = ctypes.c_int
    lib.pkv_prefill_workspace_bytes.argtypes = [i32, i64, i32, i32]
    lib.pkv_prefill_workspace_bytes.restype = sz
    lib.pkv_varlen_prefill_attention.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32,
                                                 i32, i32, i32, i32, i32, f32, i32, vp, sz, vp]
    lib.pkv_varlen_prefill_attention.restype = ctypes.c_int
    lib.pkv_varlen_prefill_attention_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32,
                                                         i32, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.pkv_varlen_prefill_attention_noalloc.restype = ctypes.c_int
    _declare_block_manager(lib)
    lib.pkv_last_error.argtypes = []
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_version.argtypes = []
    lib.pkv_version.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(status: int) -> None:
    if status != PKV_OK:
        raise PagedKVError(status, load().pkv_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, dtype, name: str, dims: int):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != dims or not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous {dims}-d tensor, got {tuple(t.shape)}")


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def version() -> str:
    return load().pkv_version().decode()


def store_kvcache(k: torch.Tensor, v: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                  slot_mapping: torch.Tensor, stream=None) -> None:
    """k_cache[slot_mapping[i]] = k[i], v_cache[...] = v[i] for slot_mapping[i] >= 0."""
    for name, t in (("k", k), ("v", v), ("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, torch.bfloat16, name, 3)
    _need(slot_mapping, torch.int32, "slot_mapping", 1)
    n, hkv, d = k.shape
    if v.shape != k.shape or k_cache.shape[1:] != (hkv, d) or v_cache.shape != k_cache.shape \
            or slot_mapping.shape[0] != n:
        raise ValueError("store_kvcache: inconsistent shapes")
    _check(load().pkv_store_kvcache(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(slot_mapping), n, hkv, d, k_cache.shape[0],
                                    _stream(stream)))


def decode_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           max_context_len: int, split_tokens: int = 0) -> int:
    r = load().pkv_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                          max_context_len, split_tokens)
    if r == ctypes.c_size_t(-1).value:
        raise PagedKVError(PKV_ERR_INVALID_ARG, "invalid sizes for the decode workspace")
    return int(r)


def decode_split_tokens(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                        max_context_len: int) -> int:
    return int(load().pkv_decode_split_tokens(batch, num_q_heads, num_kv_heads, head_dim,
                                              max_context_len))


def paged_decode_attention(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                           v_cache: torch.Tensor, block_tables: torch.Tensor,
                           context_lens: torch.Tensor, block_size: int, max_context_len: int,
                           scale: float, split_tokens: int = 0,
                           workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """out[b, h] = softmax(scale * q[b, h] K_b^T) V_b over the cached keys of sequence b."""
    for name, t in (("out", out), ("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, torch.bfloat16, name, 3)
    _need(block_tables, torch.int32, "block_tables", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    b, hq, d = q.shape
    hkv = k_cache.shape[1]
    if out.shape != q.shape or k_cache.shape[2] != d or v_cache.shape != k_cache.shape \
            or block_tables.shape[0] != b or context_lens.shape[0] != b:
        raise ValueError("paged_decode_attention: inconsistent shapes")
    need = decode_workspace_bytes(b, hq, hkv, d, max_context_len, split_tokens)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().pkv_paged_decode_attention(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), b, hq, hkv, d, block_size, block_tables.shape[1], max_context_len,
        float(scale), split_tokens, _ptr(workspace), ws_bytes, _stream(stream)))


def store_and_decode(out: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                     k_cache: torch.Tensor, v_cache: torch.Tensor, slot_mapping: torch.Tensor,
                     block_tables: torch.Tensor, context_lens: torch.Tensor, block_size: int,
                     max_context_len: int, scale: float, split_tokens: int = 0,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """One decode step in one kernel: store each sequence's new K/V row, then attend."""
    for name, t in (("out", out), ("q", q), ("k_new", k_new), ("v_new", v_new),
                    ("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, torch.bfloat16, name, 3)
    for name, t in (("slot_mapping", slot_mapping), ("context_lens", context_lens)):
        _need(t, torch.int32, name, 1)
    _need(block_tables, torch.int32, "block_tables", 2)
    b, hq, d = q.shape
    hkv = k_cache.shape[1]
    if out.shape != q.shape or k_new.shape != (b, hkv, d) or v_new.shape != k_new.shape \
            or k_cache.shape[2] != d or v_cache.shape != k_cache.shape \
            or slot_mapping.shape[0] != b or block_tables.shape[0] != b or context_lens.shape[0] != b:
        raise ValueError("store_and_decode: inconsistent shapes")
    need = decode_workspace_bytes(b, hq, hkv, d, max_context_len, split_tokens)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().pkv_store_and_decode(
        _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(slot_mapping), _ptr(block_tables), _ptr(context_lens), b, hq, hkv, d, block_size,
        block_tables.shape[1], max_context_len, k_cache.shape[0], float(scale), split_tokens,
        _ptr(workspace), ws_bytes, _stream(stream)))


def topk_sample(tokens: torch.Tensor, logits: torch.Tensor, gumbel: Optional[torch.Tensor],
                top_k: int, temperature: float, stream=None) -> None:
    """One token per row of ``logits`` (fp32 [rows, vocab]) into ``tokens`` (int32 [rows])."""
    _need(logits, torch.float32, "logits", 2)
    _need(tokens, torch.int32, "tokens", 1)
    rows, vocab = logits.shape
    if tokens.shape[0] != rows:
        raise ValueError("topk_sample: tokens must have one entry per row")
    if gumbel is not None:
        _need(gumbel, torch.float32, "gumbel", 2)
        if gumbel.shape != logits.shape:
            raise ValueError("topk_sample: gumbel must have the shape of logits")
    _check(load().pkv_topk_sample(_ptr(tokens), _ptr(logits), _ptr(gumbel), rows, vocab, int(top_k),
                                  float(temperature), _stream(stream)))


def prefill_workspace_bytes(num_seqs: int, total_q: int, num_q_heads: int,
                            num_kv_heads: int) -> int:
    r = load().pkv_prefill_workspace_bytes(num_seqs, total_q, num_q_heads, num_kv_heads)
    if r == ctypes.c_size_t(-1).value:
        raise PagedKVError(PKV_ERR_INVALID_ARG, "invalid sizes for the prefill workspace")
    return int(r)


def varlen_prefill_attention(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                             v_cache: torch.Tensor, cu_seqlens_q: torch.Tensor,
                             cu_seqlens_k: torch.Tensor, block_tables: torch.Tensor,
                             max_seqlen_q: int, max_seqlen_k: int, block_size: int,
                             scale: float, causal: bool = True,
                             workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Causal (or full) attention of packed query rows over their cached keys.

    ``workspace`` (uint8, on the device) is allocated per call when not given."""
    for name, t in (("out", out), ("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, torch.bfloat16, name, 3)
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        _need(t, torch.int32, name, 1)
    _need(block_tables, torch.int32, "block_tables", 2)
    total_q, hq, d = q.shape
    hkv = k_cache.shape[1]
    ns = cu_seqlens_q.shape[0] - 1
    if out.shape != q.shape or k_cache.shape[2] != d or v_cache.shape != k_cache.shape \
            or cu_seqlens_k.shape[0] != ns + 1 or block_tables.shape[0] != ns:
        raise ValueError("varlen_prefill_attention: inconsistent shapes")
    need = prefill_workspace_bytes(ns, total_q, hq, hkv) if hkv > 0 and hq % hkv == 0 else 0
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().pkv_varlen_prefill_attention(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
        _ptr(block_tables), ns, total_q, max_seqlen_q, max_seqlen_k, hq, hkv, d, block_size,
        block_tables.shape[1], float(scale), 1 if causal else 0, _ptr(workspace), ws_bytes,
        _stream(stream)))


# PKV_PREFILL_NOALLOC_SCRATCH_BYTES of pagedkv.h: the fixed per-GPU scratch of the
# allocation-free prefill entry point
PREFILL_NOALLOC_SCRATCH_BYTES = 2 << 20


def varlen_prefill_attention_noalloc(out: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                                     v_cache: torch.Tensor, cu_seqlens_q: torch.Tensor,
                                     cu_seqlens_k: torch.Tensor, block_tables: torch.Tensor,
                                     max_seqlen_q: int, max_seqlen_k: int, block_size: int,
                                     scale: float, causal: bool = True, stream=None) -> None:
    """varlen_prefill_attention on the library's fixed per-GPU scratch (allocates nothing;
    overlapping calls on one GPU race)."""
    for name, t in (("out", out), ("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, torch.bfloat16, name, 3)
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        _need(t, torch.int32, name, 1)
    _need(block_tables, torch.int32, "block_tables", 2)
    total_q, hq, d = q.shape
    hkv = k_cache.shape[1]
    ns = cu_seqlens_q.shape[0] - 1
    if out.shape != q.shape or k_cache.shape[2] != d or v_cache.shape != k_cache.shape \
            or cu_seqlens_k.shape[0] != ns + 1 or block_tables.shape[0] != ns:
        raise ValueError("varlen_prefill_attention_noalloc: inconsistent shapes")
    _check(load().pkv_varlen_prefill_attention_noalloc(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
        _ptr(block_tables), ns, total_q, max_seqlen_q, max_seqlen_k, hq, hkv, d, block_size,
        block_tables.shape[1], float(scale), 1 if causal else 0, _stream(stream)))

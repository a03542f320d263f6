"""Python binding of libattn.so: FlashAttention-style attention for MI355X (gfx950).

The functions carry the C ABI's names and only marshal arguments: they check devices, dtypes and
shapes, allocate outputs (and the split-K workspace) with torch, and pass raw device pointers and
torch's current HIP stream to the library.  Every step of the computation runs in the HIP kernels;
if libattn.so is not built the first call raises ImportError.

Layouts (see include/attn.h): varlen tensors are THD ``[tokens, heads, D]`` with int32 cu_seqlens;
paged caches are ``[num_pages, Hkv, 16, D]`` bf16 with an int32 ``[B, max_pages]`` block table.
"""
from __future__ import annotations

import math

import torch

from . import _lib
from ._lib import NOALLOC_SCRATCH_BYTES, SKIP_TILE, AttnError  # noqa: F401

__all__ = ["attn_prefill_varlen", "attn_prefill_varlen_backward", "attn_prefill_varlen_backward_workspace_size",
           "attn_decode_paged", "attn_decode_paged_workspace_size", "attn_decode_paged_noalloc",
           "attn_decode_paged_qdq", "attn_decode_paged_multi",
           "attn_decode_paged_multi_workspace_size", "attn_smallseq_cross",
           "attn_smallseq_cross_backward", "AttnError", "SKIP_TILE"]


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _cuda_contig(name, t, dtype=None, device=None):
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.is_cuda, f"{name} must be on a GPU")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if dtype is not None:
        _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    if device is not None:
        _need(t.device == device, f"{name} must be on {device}")


def attn_decode_paged_workspace_size(B: int, Hq: int, D: int, num_splits: int) -> int:
    """Workspace bytes the split-K schedule needs (0 for the sequential one)."""
    return int(_lib.load().attn_decode_paged_workspace_size(B, Hq, D, num_splits))


def attn_prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *, scale=None,
                        causal=True, skip_threshold=0.0, out=None, return_lse=False, return_skip_map=False):
    """Varlen THD attention.  Returns (o, lse or None, skip_map or None)."""
    lib = _lib.load()
    _need(q.dtype in (torch.float32, torch.bfloat16), "q must be float32 or bfloat16")
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _cuda_contig(name, t, q.dtype, dev)
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        _cuda_contig(name, t, torch.int32, dev)
    _need(q.dim() == 3 and k.dim() == 3 and k.shape == v.shape, "q [tq,Hq,D], k/v [tk,Hkv,D]")
    tq, Hq, D = q.shape
    Hkv = k.shape[1]
    _need(k.shape[2] == D, "head dims differ")
    B = cu_seqlens_q.numel() - 1
    _need(B >= 0 and cu_seqlens_k.numel() == B + 1, "cu_seqlens must both have B + 1 entries")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _cuda_contig("out", out, q.dtype, dev)
    _need(out.shape == q.shape, "out must match q")
    lse = torch.empty((tq, Hq), dtype=torch.float32, device=dev) if return_lse else None
    stride = max(1, (int(max_seqlen_k) + SKIP_TILE - 1) // SKIP_TILE)
    smap = torch.empty((tq, Hq, stride), dtype=torch.uint8, device=dev) if return_skip_map else None
    dt = _lib.ATTN_BF16 if q.dtype == torch.bfloat16 else _lib.ATTN_F32
    _lib.check(lib.attn_prefill_varlen(dt, q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens_q.data_ptr(),
                                       cu_seqlens_k.data_ptr(), B, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv,
                                       D, float(scale), int(bool(causal)), float(skip_threshold),
                                       out.data_ptr(), _ptr(lse), _ptr(smap), stride, _stream(q)))
    return out, lse, smap


def attn_prefill_varlen_backward_workspace_size(B: int, max_seqlen_q: int, Hq: int) -> int:
    """Workspace bytes of the prefill backward (per row: rowsum(dO * O) and lse * log2(e))."""
    return int(_lib.load().attn_prefill_varlen_backward_workspace_size(B, max_seqlen_q, Hq))


def attn_prefill_varlen_backward(q, k, v, o, dout, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *,
                                 scale=None, causal=True, workspace=None, dq=None, dk=None, dv=None):
    """Gradients of the dense varlen prefill from its output o and LSE.  Returns (dq, dk, dv)."""
    lib = _lib.load()
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _cuda_contig(name, t, torch.bfloat16, dev)
    _cuda_contig("lse", lse, torch.float32, dev)
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        _cuda_contig(name, t, torch.int32, dev)
    _need(q.dim() == 3 and k.dim() == 3 and k.shape == v.shape, "q [tq,Hq,D], k/v [tk,Hkv,D]")
    _need(o.shape == q.shape and dout.shape == q.shape, "o and dout must match q")
    tq, Hq, D = q.shape
    Hkv = k.shape[1]
    _need(k.shape[2] == D, "head dims differ")
    _need(lse.shape == (tq, Hq), "lse must be [tq, Hq]")
    B = cu_seqlens_q.numel() - 1
    _need(B >= 0 and cu_seqlens_k.numel() == B + 1, "cu_seqlens must both have B + 1 entries")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = attn_prefill_varlen_backward_workspace_size(B, int(max_seqlen_q), Hq)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _cuda_contig(name, t, torch.bfloat16, dev)
        _need(t.shape == ref.shape, f"{name} must match its input's shape")
    _lib.check(lib.attn_prefill_varlen_backward(_lib.ATTN_BF16, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                                                cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B,
                                                int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, D, float(scale),
                                                int(bool(causal)), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                                _ptr(workspace), ws_bytes, _stream(q)))
    return dq, dk, dv


def attn_decode_paged(q, k_cache, v_cache, block_table, seq_lens, *, scale=None, skip_threshold=0.0, num_splits=0,
                      workspace=None, out=None, return_lse=False, return_skip_map=False):
    """One-token paged decode.  Returns (o, lse or None, skip_map or None)."""
    lib = _lib.load()
    dev = q.device
    _cuda_contig("q", q, torch.bfloat16)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _cuda_contig(name, t, torch.bfloat16, dev)
    _cuda_contig("block_table", block_table, torch.int32, dev)
    _cuda_contig("seq_lens", seq_lens, torch.int32, dev)
    _need(q.dim() == 3 and k_cache.dim() == 4 and k_cache.shape == v_cache.shape,
          "q [B,Hq,D], caches [pages,Hkv,page,D]")
    B, Hq, D = q.shape
    num_pages, Hkv, page, Dk = k_cache.shape
    _need(Dk == D, "head dims differ")
    _need(block_table.dim() == 2 and block_table.shape[0] == B and seq_lens.shape == (B,),
          "block_table [B, max_pages], seq_lens [B]")
    max_pages = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    splits = num_splits if num_splits else (32 if skip_threshold == 0 else 1)
    need = attn_decode_paged_workspace_size(B, Hq, D, splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    _cuda_contig("out", out, torch.bfloat16, dev)
    _need(out.shape == q.shape, "out must match q")
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if return_lse else None
    stride = max(1, (max_pages * page + SKIP_TILE - 1) // SKIP_TILE)
    smap = torch.empty((B, Hq, stride), dtype=torch.uint8, device=dev) if return_skip_map else None
    _lib.check(lib.attn_decode_paged(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
                                     seq_lens.data_ptr(), B, Hq, Hkv, D, page, num_pages, max_pages, float(scale),
                                     float(skip_threshold), int(splits), _ptr(workspace), ws_bytes, out.data_ptr(),
                                     _ptr(lse), _ptr(smap), stride, _stream(q)))
    return out, lse, smap


def attn_decode_paged_noalloc(q, k_cache, v_cache, block_table, seq_lens, *, scale=None, skip_threshold=0.0,
                              num_splits=0, out, lse=None, skip_map=None):
    """attn_decode_paged for callers that cannot allocate: the split-K partials go to the library's own
    per-GPU scratch (NOALLOC_SCRATCH_BYTES).  Every output is caller-allocated (``out`` [B, Hq, D] bf16,
    optional ``lse`` [B, Hq] fp32 and ``skip_map`` [B, Hq, stride] uint8); nothing is allocated here.
    Calls that overlap on one GPU share the scratch and race.  Returns (out, lse, skip_map)."""
    lib = _lib.load()
    dev = q.device
    _cuda_contig("q", q, torch.bfloat16)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _cuda_contig(name, t, torch.bfloat16, dev)
    _cuda_contig("block_table", block_table, torch.int32, dev)
    _cuda_contig("seq_lens", seq_lens, torch.int32, dev)
    _need(q.dim() == 3 and k_cache.dim() == 4 and k_cache.shape == v_cache.shape,
          "q [B,Hq,D], caches [pages,Hkv,page,D]")
    B, Hq, D = q.shape
    num_pages, Hkv, page, Dk = k_cache.shape
    _need(Dk == D, "head dims differ")
    _need(block_table.dim() == 2 and block_table.shape[0] == B and seq_lens.shape == (B,),
          "block_table [B, max_pages], seq_lens [B]")
    max_pages = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _cuda_contig("out", out, torch.bfloat16, dev)
    _need(out.shape == q.shape, "out must match q")
    if lse is not None:
        _cuda_contig("lse", lse, torch.float32, dev)
        _need(lse.shape == (B, Hq), "lse must be [B, Hq]")
    stride = 0
    if skip_map is not None:
        _cuda_contig("skip_map", skip_map, torch.uint8, dev)
        _need(skip_map.dim() == 3 and skip_map.shape[:2] == (B, Hq), "skip_map must be [B, Hq, stride]")
        stride = skip_map.shape[2]
    _lib.check(lib.attn_decode_paged_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                             block_table.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv, D, page,
                                             num_pages, max_pages, float(scale), float(skip_threshold),
                                             int(num_splits), out.data_ptr(), _ptr(lse), _ptr(skip_map), stride,
                                             _stream(q)))
    return out, lse, skip_map


def attn_decode_paged_qdq(q, k_cache, v_cache, block_table, seq_lens, *, scale=None, skip_threshold=0.0,
                          p_amax=0.0, v_amax=0.0, out=None, return_lse=False, return_skip_map=False):
    """One-token paged decode, sequential schedule, with NVFP4 fake quantization of P (``p_amax`` > 0) and
    V (``v_amax`` > 0).  Returns (o, lse or None, skip_map or None)."""
    lib = _lib.load()
    dev = q.device
    _cuda_contig("q", q, torch.bfloat16)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _cuda_contig(name, t, torch.bfloat16, dev)
    _cuda_contig("block_table", block_table, torch.int32, dev)
    _cuda_contig("seq_lens", seq_lens, torch.int32, dev)
    _need(q.dim() == 3 and k_cache.dim() == 4 and k_cache.shape == v_cache.shape,
          "q [B,Hq,D], caches [pages,Hkv,page,D]")
    B, Hq, D = q.shape
    num_pages, Hkv, page, Dk = k_cache.shape
    _need(Dk == D, "head dims differ")
    _need(block_table.dim() == 2 and block_table.shape[0] == B and seq_lens.shape == (B,),
          "block_table [B, max_pages], seq_lens [B]")
    max_pages = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _cuda_contig("out", out, torch.bfloat16, dev)
    _need(out.shape == q.shape, "out must match q")
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev) if return_lse else None
    stride = max(1, (max_pages * page + SKIP_TILE - 1) // SKIP_TILE)
    smap = torch.empty((B, Hq, stride), dtype=torch.uint8, device=dev) if return_skip_map else None
    _lib.check(lib.attn_decode_paged_qdq(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                         block_table.data_ptr(), seq_lens.data_ptr(), B, Hq, Hkv, D, page, num_pages,
                                         max_pages, float(scale), float(skip_threshold), float(p_amax),
                                         float(v_amax), out.data_ptr(), _ptr(lse), _ptr(smap), stride, _stream(q)))
    return out, lse, smap


def attn_decode_paged_multi_workspace_size(total_q: int, max_seqlen_q: int, Hq: int, Hkv: int, D: int,
                                           num_splits: int = 0) -> int:
    """Workspace bytes of the multi-token decode (the split-K partials; 0 for long query chunks)."""
    return int(_lib.load().attn_decode_paged_multi_workspace_size(total_q, max_seqlen_q, Hq, Hkv, D, num_splits))


def attn_decode_paged_multi(q, cu_seqlens_q, max_seqlen_q, k_cache, v_cache, block_table, seq_lens, *, scale=None,
                            skip_threshold=0.0, num_splits=0, workspace=None, out=None, return_lse=False,
                            return_skip_map=False):
    """Several new tokens per sequence over the paged cache (THD queries, bottom-right causal): split-K
    decode for short dense query chunks, the paged prefill kernel for long ones and for skip-softmax.
    Returns (o, lse or None, skip_map or None)."""
    lib = _lib.load()
    dev = q.device
    _cuda_contig("q", q, torch.bfloat16)
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _cuda_contig(name, t, torch.bfloat16, dev)
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("block_table", block_table), ("seq_lens", seq_lens)):
        _cuda_contig(name, t, torch.int32, dev)
    _need(q.dim() == 3 and k_cache.dim() == 4 and k_cache.shape == v_cache.shape,
          "q [total_q,Hq,D], caches [pages,Hkv,page,D]")
    total_q, Hq, D = q.shape
    num_pages, Hkv, page, Dk = k_cache.shape
    _need(Dk == D, "head dims differ")
    B = seq_lens.numel()
    _need(cu_seqlens_q.numel() == B + 1 and block_table.dim() == 2 and block_table.shape[0] == B,
          "cu_seqlens_q [B + 1], block_table [B, max_pages], seq_lens [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    skip = skip_threshold > 0 or return_skip_map
    need = 0 if skip else attn_decode_paged_multi_workspace_size(total_q, int(max_seqlen_q), Hq, Hkv, D, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    _cuda_contig("out", out, torch.bfloat16, dev)
    _need(out.shape == q.shape, "out must match q")
    lse = torch.empty((total_q, Hq), dtype=torch.float32, device=dev) if return_lse else None
    stride = max(1, (block_table.shape[1] * page + SKIP_TILE - 1) // SKIP_TILE)
    smap = torch.empty((total_q, Hq, stride), dtype=torch.uint8, device=dev) if return_skip_map else None
    _lib.check(lib.attn_decode_paged_multi(q.data_ptr(), cu_seqlens_q.data_ptr(), total_q, int(max_seqlen_q),
                                           k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
                                           seq_lens.data_ptr(), B, Hq, Hkv, D, page, num_pages, block_table.shape[1],
                                           float(scale), float(skip_threshold), int(num_splits), _ptr(workspace),
                                           ws_bytes, out.data_ptr(), _ptr(lse), _ptr(smap), stride, _stream(q)))
    return out, lse, smap


def attn_smallseq_cross(q, k, v, cu_seqlens_kv, max_seqlen_kv, *, scale=None, return_weights=True,
                        return_lse=False, out=None):
    """s_q = 1 cross-attention.  Returns (o, attn_weights [B,H,1,max_seqlen_kv] or None, lse or None)."""
    lib = _lib.load()
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _cuda_contig(name, t, torch.bfloat16, dev)
    _cuda_contig("cu_seqlens_kv", cu_seqlens_kv, torch.int32, dev)
    _need(q.dim() == 3 and k.dim() == 3 and k.shape == v.shape and k.shape[1:] == q.shape[1:],
          "q [B,H,D], k/v [T,H,D]")
    B, H, D = q.shape
    _need(cu_seqlens_kv.numel() == B + 1, "cu_seqlens_kv must have B + 1 entries")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _cuda_contig("out", out, torch.bfloat16, dev)
    _need(out.shape == q.shape, "out must match q")
    w = torch.empty((B, H, 1, int(max_seqlen_kv)), dtype=torch.bfloat16, device=dev) if return_weights else None
    lse = torch.empty((B, H), dtype=torch.float32, device=dev) if return_lse else None
    _lib.check(lib.attn_smallseq_cross(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens_kv.data_ptr(), B, H, D,
                                       int(max_seqlen_kv), float(scale), out.data_ptr(), _ptr(w), _ptr(lse),
                                       _stream(q)))
    return out, w, lse


def attn_smallseq_cross_backward(q, k, v, attn_weights, dout, cu_seqlens_kv, max_seqlen_kv, *, scale=None, dq=None,
                                 dk=None, dv=None):
    """Gradients of the s_q = 1 cross-attention from its stored weights.  Returns (dq, dk, dv)."""
    lib = _lib.load()
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("attn_weights", attn_weights), ("dout", dout)):
        _cuda_contig(name, t, torch.bfloat16, dev)
    _cuda_contig("cu_seqlens_kv", cu_seqlens_kv, torch.int32, dev)
    _need(q.dim() == 3 and k.dim() == 3 and k.shape == v.shape and k.shape[1:] == q.shape[1:],
          "q [B,H,D], k/v [T,H,D]")
    B, H, D = q.shape
    _need(dout.shape == q.shape, "dout must match q")
    _need(attn_weights.shape == (B, H, 1, int(max_seqlen_kv)), "attn_weights must be [B, H, 1, max_seqlen_kv]")
    _need(cu_seqlens_kv.numel() == B + 1, "cu_seqlens_kv must have B + 1 entries")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _cuda_contig(name, t, torch.bfloat16, dev)
        _need(t.shape == ref.shape, f"{name} must match its input's shape")
    _lib.check(lib.attn_smallseq_cross_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), attn_weights.data_ptr(),
                                                dout.data_ptr(), cu_seqlens_kv.data_ptr(), B, H, D,
                                                int(max_seqlen_kv), float(scale), dq.data_ptr(), dk.data_ptr(),
                                                dv.data_ptr(), _stream(q)))
    return dq, dk, dv

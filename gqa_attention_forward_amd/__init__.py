"""Grouped-query attention forward for AMD MI355X (gfx950) -- Python binding.

Thin wrappers over the C ABI in include/gqa.h (libgqa.so, loaded with
ctypes).  PyTorch supplies device memory and the current stream only; every
step of the attention runs in the library's HIP kernels.  There is no CPU or
eager fallback: without the built library every call raises.

    prefill(q, k, v, ...)          dense [B, H, S, d] tensors, one pass or split-KV
    decode_splitkv(q, k, v, ...)   Sq = 1, split-KV partials + merge kernel
    decode_splitkv_noalloc(...)    the same with the library's own scratch (allocates nothing)
    splitkv_partial / splitkv_merge  the two split-KV phases on their own
    paged(q, cu_seqlens_q, k_cache, v_cache, page_table, kv_len, ...)
    workspace_size(...)
"""

from __future__ import annotations

import ctypes
import functools
import math

import torch

from . import _lib
from ._lib import (GQAError, GQAInvalidArgument, GQAUnsupported,  # noqa: F401
                   GQAWorkspaceError)

__all__ = ["prefill", "decode_splitkv", "decode_splitkv_noalloc", "decode_tile", "splitkv_partial",
           "splitkv_merge", "paged",
           "paged_append", "workspace_size", "n_splits", "GQAError"]


def _ptr(t):
    # plain ints: the argtypes (c_void_p) convert them, None passes NULL
    return None if t is None else t.data_ptr()


# the current stream's raw handle: torch's own accessor where it has one
# (about 1.5 us less per call than building a Stream object), else the
# public call
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device) -> int:
    if _raw_stream is not None:
        return _raw_stream(device.index if device.index is not None else
                           torch.cuda.current_device())
    return torch.cuda.current_stream(device).cuda_stream


def _need_dev(name, t, dtype, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the query on {device}")


# Shape checks run before the device checks.  The library takes the sizes
# from q and k alone, so a v, out, kv_len or sink that disagrees with them
# would have the kernels read or write past its end.
def _shape_is(name, t, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _vec(name, t, n):
    """An optional contiguous 1-D tensor of n entries (kv_len, sink)."""
    if t is not None and (tuple(t.shape) != (n,) or (n > 1 and t.stride(0) != 1)):
        raise ValueError(f"{name} must be a contiguous [{n}] tensor, got shape {tuple(t.shape)}")


def _dense_shapes(q, k, v, out, kv_len, sink):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, S, d]")
    B, Hq, _, d = q.shape
    _shape_is("v", v, k.shape)
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError(f"k {tuple(k.shape)} does not match q {tuple(q.shape)} in B or d")
    if out is not None:
        _shape_is("out", out, q.shape)
    _vec("kv_len", kv_len, B)
    _vec("sink", sink, Hq)


def _bhsd(name, t, device=None):
    _need_dev(name, t, torch.bfloat16, device)
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, H, S, d]")
    if t.stride(3) != 1:
        raise ValueError(f"{name} must have a contiguous head dim")


@functools.lru_cache(maxsize=None)
def _default_scale(d: int) -> float:
    """1/sqrt(d) rounded to fp32 (the value the kernels and the oracle use)."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))


def _scale(scale, d):
    return _default_scale(int(d)) if scale is None else float(scale)


def n_splits(Skv: int, tile_s_kv: int) -> int:
    return max(1, -(-int(Skv) // int(tile_s_kv))) if tile_s_kv > 0 else 1


def decode_tile(B, Hkv, Skv) -> int:
    """The library's split size for a decode of B sequences, Hkv kv heads and
    Skv keys (about one work unit per compute unit of the current device)."""
    out = ctypes.c_int32(0)
    _lib.check(_lib.load().gqa_attention_decode_tile(int(B), int(Hkv), int(Skv),
                                                     ctypes.byref(out)))
    return int(out.value)


def workspace_size(B, Hq, Sq, Skv, d, tile_s_kv) -> int:
    if tile_s_kv == 0:
        return 0  # one pass needs no workspace (the library reports 0 too)
    out = ctypes.c_size_t(0)
    _lib.check(_lib.load().gqa_attention_workspace_size(B, Hq, Sq, Skv, d, tile_s_kv,
                                                        ctypes.byref(out)))
    return int(out.value)


def _workspace(device, nbytes, workspace):
    if workspace is not None and (workspace.device != device or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the query's device")
    if nbytes == 0:
        return workspace
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace


def _dense_devices(q, k, v, out, kv_len, sink):
    _bhsd("q", q), _bhsd("k", k, q.device), _bhsd("v", v, q.device)
    if out is not None:
        _bhsd("out", out, q.device)
    _need_dev("kv_len", kv_len, torch.int32, q.device)
    _need_dev("sink", sink, torch.float32, q.device)


def prefill(q, k, v, *, kv_len=None, scale=None, sink=None, causal=False, tile_s_kv=0,
            out=None, workspace=None):
    """O = softmax(scale Q K^T + mask [+ sink]) V for dense [B, H, S, d] bf16 tensors."""
    _dense_shapes(q, k, v, out, kv_len, sink)
    _dense_devices(q, k, v, out, kv_len, sink)
    B, Hq, Sq, d = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    nbytes = workspace_size(B, Hq, Sq, Skv, d, tile_s_kv)
    workspace = _workspace(q.device, nbytes, workspace)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = _lib.load()
    _lib.check(lib.gqa_attention_prefill(
        _ptr(q), _lib.strides3(q.stride()[:3]), _ptr(k), _lib.strides3(k.stride()[:3]),
        _ptr(v), _lib.strides3(v.stride()[:3]), _ptr(out), _lib.strides3(out.stride()[:3]),
        B, Hq, Hkv, Sq, Skv, d, _ptr(kv_len), _scale(scale, d), _ptr(sink), int(bool(causal)),
        int(tile_s_kv), _ptr(workspace), wsb, _stream(q.device)))
    return out


def decode_splitkv(q, k, v, *, kv_len=None, scale=None, sink=None, tile_s_kv=1024, out=None,
                   workspace=None, fused=False, tickets=None):
    """Single-token decode: q [B, Hq, 1, d]; split-KV partials then the merge kernel.

    fused=True merges the partials inside the partial kernel (one launch).
    It takes `tickets`, an int32 device tensor of at least B * Hq entries
    that is zero before its first use and is left zero by every call (a
    zeroed one is allocated per call when none is given).
    """
    if fused:
        return _decode_fused(q, k, v, kv_len=kv_len, scale=scale, sink=sink,
                             tile_s_kv=tile_s_kv, out=out, workspace=workspace, tickets=tickets)
    _dense_shapes(q, k, v, out, kv_len, sink)
    _dense_devices(q, k, v, out, kv_len, sink)
    B, Hq, Sq, d = q.shape
    if Sq != 1:
        raise ValueError("decode_splitkv takes one query row per (b, h)")
    Hkv, Skv = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    nbytes = workspace_size(B, Hq, 1, Skv, d, tile_s_kv)
    workspace = _workspace(q.device, nbytes, workspace)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = _lib.load()
    _lib.check(lib.gqa_attention_decode_splitkv(
        _ptr(q), _lib.strides3(q.stride()[:3]), _ptr(k), _lib.strides3(k.stride()[:3]),
        _ptr(v), _lib.strides3(v.stride()[:3]), _ptr(out), _lib.strides3(out.stride()[:3]),
        B, Hq, Hkv, Skv, d, _ptr(kv_len), _scale(scale, d), _ptr(sink), int(tile_s_kv),
        _ptr(workspace), wsb, _stream(q.device)))
    return out


def decode_splitkv_noalloc(q, k, v, *, kv_len=None, scale=None, sink=None, tile_s_kv=1024,
                           out):
    """decode_splitkv without a workspace: the library keeps the partial
    states in a fixed scratch buffer of its own (one per GPU), so the call
    allocates nothing; `out` is required.  Calls that overlap in time on one
    GPU share that buffer and race."""
    _dense_shapes(q, k, v, out, kv_len, sink)
    _dense_devices(q, k, v, out, kv_len, sink)
    B, Hq, Sq, d = q.shape
    if Sq != 1:
        raise ValueError("decode_splitkv_noalloc takes one query row per (b, h)")
    Hkv, Skv = k.shape[1], k.shape[2]
    lib = _lib.load()
    _lib.check(lib.gqa_attention_decode_splitkv_noalloc(
        _ptr(q), _lib.strides3(q.stride()[:3]), _ptr(k), _lib.strides3(k.stride()[:3]),
        _ptr(v), _lib.strides3(v.stride()[:3]), _ptr(out), _lib.strides3(out.stride()[:3]),
        B, Hq, Hkv, Skv, d, _ptr(kv_len), _scale(scale, d), _ptr(sink), int(tile_s_kv),
        _stream(q.device)))
    return out


def _decode_fused(q, k, v, *, kv_len, scale, sink, tile_s_kv, out, workspace, tickets):
    _dense_shapes(q, k, v, out, kv_len, sink)
    _dense_devices(q, k, v, out, kv_len, sink)
    _need_dev("tickets", tickets, torch.int32, q.device)
    B, Hq, Sq, d = q.shape
    if Sq != 1:
        raise ValueError("decode_splitkv takes one query row per (b, h)")
    Hkv, Skv = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if tickets is None:
        tickets = torch.zeros(B * Hq, dtype=torch.int32, device=q.device)
    if not tickets.is_contiguous():
        raise ValueError("tickets must be a contiguous int32 tensor")
    nbytes = workspace_size(B, Hq, 1, Skv, d, tile_s_kv)
    workspace = _workspace(q.device, nbytes, workspace)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = _lib.load()
    _lib.check(lib.gqa_attention_decode_splitkv_fused(
        _ptr(q), _lib.strides3(q.stride()[:3]), _ptr(k), _lib.strides3(k.stride()[:3]),
        _ptr(v), _lib.strides3(v.stride()[:3]), _ptr(out), _lib.strides3(out.stride()[:3]),
        B, Hq, Hkv, Skv, d, _ptr(kv_len), _scale(scale, d), _ptr(sink), int(tile_s_kv),
        _ptr(workspace), wsb, _ptr(tickets), tickets.numel(), _stream(q.device)))
    return out


def splitkv_partial(q, k, v, *, tile_s_kv, kv_len=None, scale=None, causal=False,
                    workspace=None):
    """Partial states only; returns (ml [rows, n_split, 2], ot [rows, n_split, d], workspace)."""
    _dense_shapes(q, k, v, None, kv_len, None)
    _dense_devices(q, k, v, None, kv_len, None)
    B, Hq, Sq, d = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    nbytes = workspace_size(B, Hq, Sq, Skv, d, tile_s_kv)
    workspace = _workspace(q.device, nbytes, workspace)
    wsb = workspace.numel() * workspace.element_size()
    lib = _lib.load()
    _lib.check(lib.gqa_attention_splitkv_partial(
        _ptr(q), _lib.strides3(q.stride()[:3]), _ptr(k), _lib.strides3(k.stride()[:3]),
        _ptr(v), _lib.strides3(v.stride()[:3]), B, Hq, Hkv, Sq, Skv, d, _ptr(kv_len),
        _scale(scale, d), int(bool(causal)), int(tile_s_kv), _ptr(workspace), wsb,
        _stream(q.device)))
    rows, ns = B * Hq * Sq, n_splits(Skv, tile_s_kv)
    flat = workspace.view(torch.float32)
    ml = flat[: rows * ns * 2].view(rows, ns, 2)
    ot = flat[rows * ns * 2: rows * ns * (2 + d)].view(rows, ns, d)
    return ml, ot, workspace


def splitkv_merge(workspace, *, B, Hq, Sq, d, n_split, sink=None, out=None, device=None):
    """Merge n_split partial states per row from `workspace` into bf16 O [B, Hq, Sq, d]."""
    if out is not None:
        _shape_is("out", out, (B, Hq, Sq, d))
    _vec("sink", sink, Hq)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _need_dev("sink", sink, torch.float32, workspace.device)
    if out is None:
        out = torch.empty((B, Hq, Sq, d), dtype=torch.bfloat16, device=workspace.device)
    _bhsd("out", out, workspace.device)
    if out.dim() != 4 or out.stride(3) != 1:
        raise ValueError("out must be [B, H, S, d] with a contiguous head dim")
    lib = _lib.load()
    _lib.check(lib.gqa_attention_splitkv_merge(
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
        _lib.strides3(out.stride()[:3]), B, Hq, Sq, d, n_split, _ptr(sink),
        _stream(workspace.device)))
    return out


def paged(q, cu_seqlens_q, k_cache, v_cache, page_table, kv_len, *, max_q_len, scale=None,
          sink=None, causal=False, page_size=64, tile_s_kv=0, out=None, workspace=None):
    """Ragged-Q paged-KV attention: q [total_q, Hq, d]; pools [n_pages, 64, Hkv, d].

    tile_s_kv > 0 splits each sequence's keys into tiles of that many keys
    (partial states + merge kernel), which spreads long sequences over more
    workgroups.
    """
    return _paged(q, cu_seqlens_q, k_cache, v_cache, page_table, kv_len, None, None,
                  max_q_len=max_q_len, scale=scale, sink=sink, causal=causal,
                  page_size=page_size, tile_s_kv=tile_s_kv, out=out, workspace=workspace)


def paged_append(q, cu_seqlens_q, k_cache, v_cache, page_table, kv_len, k_new, v_new, *,
                 max_q_len, scale=None, sink=None, causal=False, page_size=64, tile_s_kv=0,
                 out=None, workspace=None):
    """`paged` with the query tokens' own K/V appended in the same launch.

    k_new / v_new: [total_q, Hkv, d] bf16, packed like q.  Token i of
    sequence b holds key row kv_len[b] - q_len_b + i: the kernel attends it
    from k_new / v_new and writes it into that row of the cache pages (which
    must be allocated in page_table).  kv_len counts the new tokens.  Up to
    32 query rows per kv head (max_q_len * Hq / Hkv <= 32).
    """
    return _paged(q, cu_seqlens_q, k_cache, v_cache, page_table, kv_len, k_new, v_new,
                  max_q_len=max_q_len, scale=scale, sink=sink, causal=causal,
                  page_size=page_size, tile_s_kv=tile_s_kv, out=out, workspace=workspace)


def _paged(q, cu_seqlens_q, k_cache, v_cache, page_table, kv_len, k_new, v_new, *, max_q_len,
           scale, sink, causal, page_size, tile_s_kv, out, workspace):
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [total_q, Hq, d] and the caches [n_pages, page_size, Hkv, d]")
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if k_cache.shape[1] != page_size or k_cache.shape[3] != q.shape[2]:
        raise ValueError(f"caches {tuple(k_cache.shape)} do not match page_size {page_size} "
                         f"and q's head dim {q.shape[2]}")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.numel() < 1 or cu_seqlens_q.stride(0) != 1:
        raise ValueError("cu_seqlens_q must be a contiguous [B + 1] tensor")
    nseq = cu_seqlens_q.numel() - 1
    if page_table.dim() != 2 or page_table.shape[0] != nseq:
        raise ValueError(f"page_table has shape {tuple(page_table.shape)}, expected "
                         f"[{nseq}, max_pages]")
    _vec("kv_len", kv_len, nseq)
    _vec("sink", sink, q.shape[1])
    if out is not None:
        _shape_is("out", out, q.shape)
    dv = q.device
    _need_dev("q", q, torch.bfloat16)
    _need_dev("k_cache", k_cache, torch.bfloat16, dv)
    _need_dev("v_cache", v_cache, torch.bfloat16, dv)
    _need_dev("cu_seqlens_q", cu_seqlens_q, torch.int32, dv)
    _need_dev("page_table", page_table, torch.int32, dv)
    _need_dev("kv_len", kv_len, torch.int32, dv)
    _need_dev("sink", sink, torch.float32, dv)
    _need_dev("out", out, torch.bfloat16, dv)
    if out is not None and out.stride(2) != 1:
        raise ValueError("out must have a contiguous head dim")
    if q.stride(2) != 1:
        raise ValueError("q must be [total_q, Hq, d] with a contiguous head dim")
    if k_cache.dim() != 4 or k_cache.stride(3) != 1:
        raise ValueError("caches must be [n_pages, page_size, Hkv, d] with a contiguous head dim")
    if page_table.dim() != 2 or page_table.stride(1) != 1 or page_table.stride(0) != page_table.shape[1]:
        raise ValueError("page_table must be a contiguous [B, max_pages] int32 tensor")
    total_q, Hq, d = q.shape
    B = cu_seqlens_q.numel() - 1
    Hkv = k_cache.shape[2]
    max_pages = page_table.shape[1]
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    nbytes = workspace_size(1, Hq, total_q, max_pages * page_size, d, tile_s_kv)
    workspace = _workspace(q.device, nbytes, workspace)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    lib = _lib.load()
    if k_new is None and v_new is None:
        _lib.check(lib.gqa_attention_paged(
            _ptr(q), q.stride(0), q.stride(1), _ptr(cu_seqlens_q), _ptr(k_cache), _ptr(v_cache),
            k_cache.stride(0), k_cache.stride(1), k_cache.stride(2), _ptr(page_table),
            max_pages, _ptr(kv_len), _ptr(out), out.stride(0), out.stride(1), B, Hq, Hkv,
            d, int(page_size), total_q, int(max_q_len), _scale(scale, d), _ptr(sink),
            int(bool(causal)), int(tile_s_kv), _ptr(workspace), wsb, _stream(q.device)))
        return out
    _need_dev("k_new", k_new, torch.bfloat16, dv)
    _need_dev("v_new", v_new, torch.bfloat16, dv)
    if k_new is None or v_new is None or k_new.shape != (total_q, Hkv, d) or \
            v_new.shape != k_new.shape or k_new.stride() != v_new.stride() or k_new.stride(2) != 1:
        raise ValueError("k_new and v_new must both be [total_q, Hkv, d] with equal strides "
                         "and a contiguous head dim")
    _lib.check(lib.gqa_attention_paged_append(
        _ptr(q), q.stride(0), q.stride(1), _ptr(cu_seqlens_q), _ptr(k_cache), _ptr(v_cache),
        k_cache.stride(0), k_cache.stride(1), k_cache.stride(2), _ptr(page_table),
        max_pages, _ptr(kv_len), _ptr(k_new), _ptr(v_new), k_new.stride(0), k_new.stride(1),
        _ptr(out), out.stride(0), out.stride(1), B, Hq, Hkv, d, int(page_size), total_q,
        int(max_q_len), _scale(scale, d), _ptr(sink), int(bool(causal)), int(tile_s_kv),
        _ptr(workspace), wsb, _stream(q.device)))
    return out

"""ctypes binding of libmasked_attn.so, with the C ABI's names.

Argument marshalling only: each function checks that tensors are CUDA
(HIP) tensors of the right dtype, shape and contiguity, allocates missing
outputs with torch, and passes raw device pointers plus the current torch
stream to the C entry point.  Every step of the computation runs in the HIP
kernels; there is no fallback.  If the shared library has not been built, the
first call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; nothing can redirect the binding to another library.
LIB_PATH = os.path.join(_HERE, "libmasked_attn.so")

ATTN_F32 = 0
ATTN_BF16 = 1

STATUS = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_UNSUPPORTED",
    4: "ATTN_ERR_WORKSPACE", 5: "ATTN_ERR_LAUNCH", 6: "ATTN_ERR_VALUE", 7: "ATTN_ERR_ALIGN",
    8: "ATTN_ERR_ALIAS", 9: "ATTN_ERR_SCRATCH",
}

EXPORTS = ("attn_fwd_masked", "attn_fwd_lse", "attn_fwd_varlen", "attn_merge_lse", "kv_append",
           "attn_decode", "attn_decode_workspace_bytes", "kv_append_paged", "attn_decode_paged",
           "attn_prefill", "attn_prefill_varlen", "kv_append_fp8", "attn_decode_fp8kv", "attn_prefill_fp8",
           "kv_append_int8", "attn_decode_int8kv", "attn_prefill_varlen_fp8", "kv_append_fp8_paged",
           "kv_append_int8_paged", "attn_decode_fp8kv_paged", "attn_decode_int8kv_paged", "attn_status_string", "attn_decode_noalloc")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}: {msg}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the shared library (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is not built; run __graft_entry__.build() "
                           "(or python -m masked_attention_attn_amd.build)")
    lib = ctypes.CDLL(path)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd_masked.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P]
    lib.attn_fwd_lse.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, I, P]
    lib.attn_fwd_varlen.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, I, P]
    lib.attn_merge_lse.argtypes = [I, ctypes.POINTER(P), ctypes.POINTER(P), P, P, I, I, I, I, I, P]
    lib.kv_append.argtypes = [P, P, P, P, P, I, I, I, I, I, P]
    lib.attn_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, I, P, S, P]
    lib.attn_decode_noalloc.argtypes = [P, P, P, P, P, P, I, I, I, I, I, F, I, P]
    lib.attn_prefill.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P]
    lib.attn_prefill_varlen.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, I, P]
    lib.kv_append_paged.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, P]
    lib.kv_append_fp8.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P]
    lib.attn_decode_fp8kv.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, F, P, S, P]
    lib.kv_append_int8.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P]
    lib.attn_decode_int8kv.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, F, P, S, P]
    lib.attn_prefill_varlen_fp8.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, F, P]
    for name in ("kv_append_fp8_paged", "kv_append_int8_paged"):
        getattr(lib, name).argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, P]
    for name in ("attn_decode_fp8kv_paged", "attn_decode_int8kv_paged"):
        getattr(lib, name).argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P, S, P]
    lib.attn_prefill_fp8.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P]
    lib.attn_decode_paged.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, I, P, S, P]
    lib.attn_decode_workspace_bytes.argtypes = [I, I, I, I, I]
    lib.attn_decode_workspace_bytes.restype = S
    lib.attn_status_string.argtypes = [I]
    lib.attn_status_string.restype = ctypes.c_char_p
    for name in ("attn_fwd_masked", "attn_fwd_lse", "attn_fwd_varlen", "attn_merge_lse", "kv_append",
                 "attn_decode", "attn_decode_noalloc", "kv_append_paged", "attn_decode_paged", "attn_prefill", "attn_prefill_varlen",
                 "kv_append_fp8", "attn_decode_fp8kv", "attn_prefill_fp8", "kv_append_int8",
                 "attn_decode_int8kv", "attn_prefill_varlen_fp8", "kv_append_fp8_paged", "kv_append_int8_paged",
                 "attn_decode_fp8kv_paged", "attn_decode_int8kv_paged"):
        getattr(lib, name).restype = I
    _lib = lib
    return lib


def _check(fn, status):
    if status != 0:
        raise AttnError(fn, status, load().attn_status_string(status).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (cuda/HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _fwd(fn, q, k, v, key_padding_mask, scale, out, lse):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, T, D]")
    B, H, Tq, D = q.shape
    Tk = k.shape[2]
    if k.shape != (B, H, Tk, D) or v.shape != (B, H, Tk, D):
        raise ValueError(f"k/v shapes {tuple(k.shape)}/{tuple(v.shape)} do not match q {tuple(q.shape)}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    code = _dtype_code(q)
    if key_padding_mask is not None:
        _dev(key_padding_mask, "key_padding_mask")
        if key_padding_mask.shape != (B, Tk):
            raise ValueError(f"key_padding_mask must be [B, Tk] = {(B, Tk)}")
        if key_padding_mask.dtype == torch.bool:
            key_padding_mask = key_padding_mask.view(torch.uint8)
        if key_padding_mask.dtype != torch.uint8:
            raise TypeError("key_padding_mask must be uint8 or bool (nonzero/True = padded)")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, "out")
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q in shape and dtype")
    lib = load()
    st = _stream(q.device)
    if fn == "attn_fwd_masked":
        _check(fn, lib.attn_fwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(key_padding_mask), _ptr(out),
                                       B, H, Tq, Tk, D, float(scale), code, st))
        return out
    if lse is None:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=q.device)
    else:
        _dev(lse, "lse")
        if lse.shape != (B, H, Tq) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [B, H, Tq]")
    _check(fn, lib.attn_fwd_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(key_padding_mask), _ptr(out), _ptr(lse),
                                B, H, Tq, Tk, D, float(scale), code, st))
    return out, lse


def attn_fwd_masked(q, k, v, key_padding_mask=None, scale=None, out=None):
    """O = softmax(scale·Q·Kᵀ with padded keys at -inf)·V; q/k/v [B, H, T, D]."""
    return _fwd("attn_fwd_masked", q, k, v, key_padding_mask, scale, out, None)


def attn_fwd_lse(q, k, v, key_padding_mask=None, scale=None, out=None, lse=None):
    """As attn_fwd_masked, also returning the float32 natural-log LSE [B, H, Tq]."""
    return _fwd("attn_fwd_lse", q, k, v, key_padding_mask, scale, out, lse)


def attn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, scale=None, out=None, lse=None,
                    want_lse: bool = True):
    """Packed variable-length attention: q/o [total_q, H, D], k/v [total_k, H, D] (bf16),
    cu_seqlens_* int32 [B+1] on the device; returns O (and the LSE [H, total_q])."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_k, "cu_seqlens_k")):
        _dev(t, n)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [total, H, D]")
    total_q, H, D = q.shape
    total_k = k.shape[0]
    if k.shape != (total_k, H, D) or v.shape != (total_k, H, D):
        raise ValueError("k/v must be [total_k, H, D] with q's H and D")
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("attn_fwd_varlen takes bfloat16 q, k, v")
    if (cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32 or cu_seqlens_q.dim() != 1
            or cu_seqlens_q.shape != cu_seqlens_k.shape):
        raise ValueError("cu_seqlens_q / cu_seqlens_k must be int32 [B+1] of equal length")
    B = cu_seqlens_q.shape[0] - 1
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, "out")
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q in shape and dtype")
    if want_lse and lse is None:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    if want_lse:
        _dev(lse, "lse")
        if lse.shape != (H, total_q) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [H, total_q]")
    _check("attn_fwd_varlen", load().attn_fwd_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(out),
        _ptr(lse if want_lse else None), B, H, total_q, total_k, int(max_seqlen_q), D, float(scale),
        ATTN_BF16, _stream(q.device)))
    return (out, lse) if want_lse else out


def attn_merge_lse(outs: Sequence[torch.Tensor], lses: Sequence[torch.Tensor], out=None,
                   lse_out=None, want_lse: bool = True):
    """Merge per-chunk (O_i [B,H,T,D], LSE_i [B,H,T]) into (O, LSE)."""
    n = len(outs)
    if n == 0 or len(lses) != n:
        raise ValueError("need matching, non-empty lists of outputs and LSEs")
    o0 = outs[0]
    for i in range(n):
        _dev(outs[i], f"outs[{i}]")
        _dev(lses[i], f"lses[{i}]")
        if outs[i].shape != o0.shape or outs[i].dtype != o0.dtype:
            raise ValueError("all outs must share shape and dtype")
        if lses[i].shape != o0.shape[:3] or lses[i].dtype != torch.float32:
            raise ValueError("each lse must be float32 [B, H, T]")
    B, H, T, D = o0.shape
    code = _dtype_code(o0)
    if out is None:
        out = torch.empty_like(o0)
    if want_lse and lse_out is None:
        lse_out = torch.empty((B, H, T), dtype=torch.float32, device=o0.device)
    P = ctypes.c_void_p
    optrs = (P * n)(*[t.data_ptr() for t in outs])
    lptrs = (P * n)(*[t.data_ptr() for t in lses])
    lib = load()
    _check("attn_merge_lse", lib.attn_merge_lse(n, optrs, lptrs, _ptr(out), _ptr(lse_out if want_lse else None),
                                                B, H, T, D, code, _stream(o0.device)))
    return (out, lse_out) if want_lse else out


def kv_append(k_cache, v_cache, cache_seqlens, k_new, v_new):
    """Write k_new/v_new [B, H_kv, 1, D] at slot cache_seqlens[b], then increment it (in place)."""
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (cache_seqlens, "cache_seqlens"),
                 (k_new, "k_new"), (v_new, "v_new")):
        _dev(t, n)
    B, Hkv, Tmax, D = k_cache.shape
    if v_cache.shape != k_cache.shape or k_new.shape != (B, Hkv, 1, D) or v_new.shape != (B, Hkv, 1, D):
        raise ValueError("cache / new-token shapes are inconsistent")
    if cache_seqlens.shape != (B,) or cache_seqlens.dtype != torch.int32:
        raise ValueError("cache_seqlens must be int32 [B]")
    code = _dtype_code(k_cache)
    for t in (v_cache, k_new, v_new):
        if t.dtype != k_cache.dtype:
            raise TypeError("caches and new tokens must share a dtype")
    _check("kv_append", load().kv_append(_ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens), _ptr(k_new),
                                         _ptr(v_new), B, Hkv, Tmax, D, code, _stream(k_cache.device)))


def attn_decode_workspace_bytes(B, H_q, H_kv, T_max, D) -> int:
    return int(load().attn_decode_workspace_bytes(B, H_q, H_kv, T_max, D))


def attn_decode(q, k_cache, v_cache, cache_seqlens, scale=None, out=None, lse=None, workspace=None,
                want_lse: bool = False):
    """One query token per sequence (q [B, H_q, 1, D]) against the first
    cache_seqlens[b] positions of k_cache/v_cache [B, H_kv, T_max, D]."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (cache_seqlens, "cache_seqlens")):
        _dev(t, n)
    B, Hq, one, D = q.shape
    if one != 1:
        raise ValueError("q must be [B, H_q, 1, D]")
    _, Hkv, Tmax, Dk = k_cache.shape
    if k_cache.shape[0] != B or Dk != D or v_cache.shape != k_cache.shape:
        raise ValueError("cache shapes do not match q")
    if cache_seqlens.shape != (B,) or cache_seqlens.dtype != torch.int32:
        raise ValueError("cache_seqlens must be int32 [B]")
    code = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise TypeError("q and caches must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = attn_decode_workspace_bytes(B, Hq, Hkv, Tmax, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check("attn_decode", load().attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens),
                                             _ptr(out), _ptr(lse if want_lse else None), B, Hq, Hkv, Tmax, D,
                                             float(scale), code, _ptr(workspace), nbytes, _stream(q.device)))
    return (out, lse) if want_lse else out


# Capacity of the library's static scratch behind attn_decode_noalloc (ATTN_DECODE_NOALLOC_SCRATCH_BYTES).
DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20


def attn_decode_noalloc(q, k_cache, v_cache, cache_seqlens, out, lse=None, scale=None):
    """attn_decode without a workspace: the library's static device scratch holds the partial
    results, and the C call allocates nothing.  The caller passes the outputs (out [B, H_q, 1, D],
    lse [B, H_q] float32 or None).  Sizes whose workspace would exceed the static buffer raise
    AttnError (ATTN_ERR_SCRATCH)."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (cache_seqlens, "cache_seqlens"),
                 (out, "out")):
        _dev(t, n)
    B, Hq, one, D = q.shape
    if one != 1:
        raise ValueError("q must be [B, H_q, 1, D]")
    _, Hkv, Tmax, Dk = k_cache.shape
    if k_cache.shape[0] != B or Dk != D or v_cache.shape != k_cache.shape:
        raise ValueError("cache shapes do not match q")
    if cache_seqlens.shape != (B,) or cache_seqlens.dtype != torch.int32:
        raise ValueError("cache_seqlens must be int32 [B]")
    code = _dtype_code(q)
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype or out.dtype != q.dtype or out.shape != q.shape:
        raise TypeError("q, caches and out must share a dtype, out the shape of q")
    if lse is not None:
        _dev(lse, "lse")
        if lse.shape != (B, Hq) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [B, H_q]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check("attn_decode_noalloc", load().attn_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens), _ptr(out), _ptr(lse), B, Hq, Hkv, Tmax, D,
        float(scale), code, _stream(q.device)))
    return (out, lse) if lse is not None else out


def _paged_args(k_pages, v_pages, block_table, cache_seqlens, B):
    for t, n in ((k_pages, "k_pages"), (v_pages, "v_pages"), (block_table, "block_table"),
                 (cache_seqlens, "cache_seqlens")):
        _dev(t, n)
    if k_pages.dim() != 4 or v_pages.shape != k_pages.shape:
        raise ValueError("k_pages / v_pages must be [num_pages, H_kv, page_size, D] of one shape")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 [B, max_pages_per_seq]")
    if cache_seqlens.shape != (B,) or cache_seqlens.dtype != torch.int32:
        raise ValueError("cache_seqlens must be int32 [B]")
    num_pages, Hkv, page_size, D = k_pages.shape
    return num_pages, Hkv, page_size, D, block_table.shape[1]


def kv_append_paged(k_pages, v_pages, block_table, cache_seqlens, k_new, v_new):
    """kv_append into a paged pool [num_pages, H_kv, page_size, D] through block_table [B, max_pages]."""
    B = k_new.shape[0]
    _dev(k_new, "k_new")
    _dev(v_new, "v_new")
    num_pages, Hkv, ps, D, mp = _paged_args(k_pages, v_pages, block_table, cache_seqlens, B)
    if k_new.shape != (B, Hkv, 1, D) or v_new.shape != (B, Hkv, 1, D):
        raise ValueError("k_new / v_new must be [B, H_kv, 1, D]")
    code = _dtype_code(k_pages)
    for t in (v_pages, k_new, v_new):
        if t.dtype != k_pages.dtype:
            raise TypeError("pools and new tokens must share a dtype")
    _check("kv_append_paged", load().kv_append_paged(
        _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(cache_seqlens), _ptr(k_new), _ptr(v_new),
        B, Hkv, num_pages, ps, mp, D, code, _stream(k_pages.device)))


def attn_decode_paged(q, k_pages, v_pages, block_table, cache_seqlens, scale=None, out=None, lse=None,
                      workspace=None, want_lse: bool = False):
    """attn_decode over a paged pool: q [B, H_q, 1, D] (bf16), pools [num_pages, H_kv, page_size, D],
    block_table int32 [B, max_pages]."""
    _dev(q, "q")
    B, Hq, one, D = q.shape
    if one != 1:
        raise ValueError("q must be [B, H_q, 1, D]")
    num_pages, Hkv, ps, Dk, mp = _paged_args(k_pages, v_pages, block_table, cache_seqlens, B)
    if Dk != D:
        raise ValueError("pool head_dim does not match q")
    if q.dtype != torch.bfloat16 or k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise TypeError("attn_decode_paged takes bfloat16 q and pools")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = attn_decode_workspace_bytes(B, Hq, Hkv, mp * ps, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check("attn_decode_paged", load().attn_decode_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(cache_seqlens), _ptr(out),
        _ptr(lse if want_lse else None), B, Hq, Hkv, num_pages, ps, mp, D, float(scale), ATTN_BF16,
        _ptr(workspace), nbytes, _stream(q.device)))
    return (out, lse) if want_lse else out


def attn_prefill(q, k, v, key_padding_mask=None, causal=False, scale=None, out=None, lse=None,
                 want_lse: bool = True):
    """GQA / causal attention: q [B, H_q, Tq, D], k/v [B, H_kv, Tk, D]; query head h reads KV
    head h // (H_q / H_kv); causal lets query i see keys j <= i + Tk - Tq."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, T, D]")
    B, Hq, Tq, D = q.shape
    _, Hkv, Tk, _ = k.shape
    if k.shape != (B, Hkv, Tk, D) or v.shape != k.shape:
        raise ValueError("k/v must be [B, H_kv, Tk, D] with q's B and D")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    code = _dtype_code(q)
    if key_padding_mask is not None:
        _dev(key_padding_mask, "key_padding_mask")
        if key_padding_mask.shape != (B, Tk):
            raise ValueError(f"key_padding_mask must be [B, Tk] = {(B, Tk)}")
        if key_padding_mask.dtype == torch.bool:
            key_padding_mask = key_padding_mask.view(torch.uint8)
        if key_padding_mask.dtype != torch.uint8:
            raise TypeError("key_padding_mask must be uint8 or bool (nonzero/True = padded)")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, "out")
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q in shape and dtype")
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    if want_lse:
        _dev(lse, "lse")
        if lse.shape != (B, Hq, Tq) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [B, H_q, Tq]")
    _check("attn_prefill", load().attn_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(key_padding_mask), _ptr(out), _ptr(lse if want_lse else None),
        B, Hq, Hkv, Tq, Tk, D, 1 if causal else 0, float(scale), code, _stream(q.device)))
    return (out, lse) if want_lse else out


def attn_prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, causal=False, scale=None,
                        out=None, lse=None, want_lse: bool = True):
    """Packed GQA / causal attention: q/o [total_q, H_q, D], k/v [total_k, H_kv, D] (bf16),
    cu_seqlens_* int32 [B+1]; returns O (and the LSE [H_q, total_q])."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_k, "cu_seqlens_k")):
        _dev(t, n)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [total, H, D]")
    total_q, Hq, D = q.shape
    total_k, Hkv, Dk = k.shape
    if Dk != D or v.shape != k.shape:
        raise ValueError("k/v must be [total_k, H_kv, D] with q's D")
    if q.dtype != torch.bfloat16 or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("attn_prefill_varlen takes bfloat16 q, k, v")
    if (cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32 or cu_seqlens_q.dim() != 1
            or cu_seqlens_q.shape != cu_seqlens_k.shape):
        raise ValueError("cu_seqlens_q / cu_seqlens_k must be int32 [B+1] of equal length")
    B = cu_seqlens_q.shape[0] - 1
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, "out")
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("out must match q in shape and dtype")
    if want_lse and lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    if want_lse:
        _dev(lse, "lse")
        if lse.shape != (Hq, total_q) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [H_q, total_q]")
    _check("attn_prefill_varlen", load().attn_prefill_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(out),
        _ptr(lse if want_lse else None), B, Hq, Hkv, total_q, total_k, int(max_seqlen_q), D,
        1 if causal else 0, float(scale), ATTN_BF16, _stream(q.device)))
    return (out, lse) if want_lse else out


def _q8_cache_args(k_cache, v_cache, k_scale, v_scale, cache_seqlens, code_dtype, what):
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (k_scale, "k_scale"), (v_scale, "v_scale"),
                 (cache_seqlens, "cache_seqlens")):
        _dev(t, n)
    if k_cache.dtype != code_dtype or v_cache.dtype != code_dtype or k_cache.dim() != 4 \
            or v_cache.shape != k_cache.shape:
        raise ValueError(f"k_cache / v_cache must be {code_dtype} [B, H_kv, T_max, D] ({what}) of one shape")
    B, Hkv, Tmax, D = k_cache.shape
    if k_scale.shape != (B, Hkv) or v_scale.shape != (B, Hkv) or k_scale.dtype != torch.float32 \
            or v_scale.dtype != torch.float32:
        raise ValueError("k_scale / v_scale must be float32 [B, H_kv]")
    if cache_seqlens.shape != (B,) or cache_seqlens.dtype != torch.int32:
        raise ValueError("cache_seqlens must be int32 [B]")
    return B, Hkv, Tmax, D


def _q8_append(fn, code_dtype, what, k_cache, v_cache, k_scale, v_scale, cache_seqlens, k_new, v_new):
    B, Hkv, Tmax, D = _q8_cache_args(k_cache, v_cache, k_scale, v_scale, cache_seqlens, code_dtype, what)
    _dev(k_new, "k_new")
    _dev(v_new, "v_new")
    if k_new.shape != (B, Hkv, 1, D) or v_new.shape != (B, Hkv, 1, D) or v_new.dtype != k_new.dtype:
        raise ValueError("k_new / v_new must be [B, H_kv, 1, D] of one dtype")
    _check(fn, getattr(load(), fn)(
        _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(cache_seqlens), _ptr(k_new),
        _ptr(v_new), B, Hkv, Tmax, D, _dtype_code(k_new), _stream(k_cache.device)))


def _q8_decode(fn, code_dtype, what, q, k_cache, v_cache, k_scale, v_scale, cache_seqlens, scale, out, lse,
               workspace, want_lse):
    _dev(q, "q")
    B, Hkv, Tmax, D = _q8_cache_args(k_cache, v_cache, k_scale, v_scale, cache_seqlens, code_dtype, what)
    if q.dim() != 4 or q.shape[0] != B or q.shape[2] != 1 or q.shape[3] != D or q.dtype != torch.bfloat16:
        raise ValueError("q must be bfloat16 [B, H_q, 1, D]")
    Hq = q.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = attn_decode_workspace_bytes(B, Hq, Hkv, Tmax, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check(fn, getattr(load(), fn)(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(cache_seqlens), _ptr(out),
        _ptr(lse if want_lse else None), B, Hq, Hkv, Tmax, D, float(scale), _ptr(workspace), nbytes,
        _stream(q.device)))
    return (out, lse) if want_lse else out


def kv_append_fp8(k_cache, v_cache, k_scale, v_scale, cache_seqlens, k_new, v_new):
    """Quantise k_new/v_new [B, H_kv, 1, D] (bf16 or float32) into slot cache_seqlens[b] of the
    E4M3 caches (uint8 codes), then increment cache_seqlens (in place)."""
    _q8_append("kv_append_fp8", torch.uint8, "E4M3 codes", k_cache, v_cache, k_scale, v_scale, cache_seqlens,
               k_new, v_new)


def attn_decode_fp8kv(q, k_cache, v_cache, k_scale, v_scale, cache_seqlens, scale=None, out=None, lse=None,
                      workspace=None, want_lse: bool = False):
    """attn_decode against E4M3 caches with per-(sequence, KV head) scales; q [B, H_q, 1, D] bf16."""
    return _q8_decode("attn_decode_fp8kv", torch.uint8, "E4M3 codes", q, k_cache, v_cache, k_scale, v_scale,
                      cache_seqlens, scale, out, lse, workspace, want_lse)


def kv_append_int8(k_cache, v_cache, k_scale, v_scale, cache_seqlens, k_new, v_new):
    """Quantise k_new/v_new [B, H_kv, 1, D] (bf16 or float32) into slot cache_seqlens[b] of the
    symmetric INT8 caches (int8 codes), then increment cache_seqlens (in place)."""
    _q8_append("kv_append_int8", torch.int8, "INT8 codes", k_cache, v_cache, k_scale, v_scale, cache_seqlens,
               k_new, v_new)


def attn_decode_int8kv(q, k_cache, v_cache, k_scale, v_scale, cache_seqlens, scale=None, out=None, lse=None,
                       workspace=None, want_lse: bool = False):
    """attn_decode against INT8 caches with per-(sequence, KV head) scales; q [B, H_q, 1, D] bf16."""
    return _q8_decode("attn_decode_int8kv", torch.int8, "INT8 codes", q, k_cache, v_cache, k_scale, v_scale,
                      cache_seqlens, scale, out, lse, workspace, want_lse)


def attn_prefill_fp8(q, k, v, q_scale, k_scale, v_scale, key_padding_mask=None, causal=False, scale=None,
                     out=None, lse=None, want_lse: bool = True):
    """attn_prefill on E4M3 codes: q uint8 [B, H_q, Tq, D], k/v uint8 [B, H_kv, Tk, D] (or
    torch.float8_e4m3fn, passed as its bytes); q_scale [B, H_q], k_scale / v_scale [B, H_kv]
    float32.  Returns O bf16 [B, H_q, Tq, D] (and the LSE [B, H_q, Tq] float32)."""
    q, k, v = (t.view(torch.uint8) if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn else t
               for t in (q, k, v))
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale")):
        _dev(t, n)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, T, D]")
    if q.dtype != torch.uint8 or k.dtype != torch.uint8 or v.dtype != torch.uint8:
        raise TypeError("q, k, v must be E4M3 codes (uint8 or float8_e4m3fn)")
    B, Hq, Tq, D = q.shape
    _, Hkv, Tk, _ = k.shape
    if k.shape != (B, Hkv, Tk, D) or v.shape != k.shape:
        raise ValueError("k/v must be [B, H_kv, Tk, D] with q's B and D")
    for t, n, shp in ((q_scale, "q_scale", (B, Hq)), (k_scale, "k_scale", (B, Hkv)), (v_scale, "v_scale", (B, Hkv))):
        if t.shape != shp or t.dtype != torch.float32:
            raise ValueError(f"{n} must be float32 {list(shp)}")
    if key_padding_mask is not None:
        _dev(key_padding_mask, "key_padding_mask")
        if key_padding_mask.shape != (B, Tk):
            raise ValueError(f"key_padding_mask must be [B, Tk] = {(B, Tk)}")
        if key_padding_mask.dtype == torch.bool:
            key_padding_mask = key_padding_mask.view(torch.uint8)
        if key_padding_mask.dtype != torch.uint8:
            raise TypeError("key_padding_mask must be uint8 or bool (nonzero/True = padded)")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hq, Tq, D), dtype=torch.bfloat16, device=q.device)
    else:
        _dev(out, "out")
        if out.shape != (B, Hq, Tq, D) or out.dtype != torch.bfloat16:
            raise ValueError("out must be bfloat16 [B, H_q, Tq, D]")
    if want_lse and lse is None:
        lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    if want_lse:
        _dev(lse, "lse")
        if lse.shape != (B, Hq, Tq) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [B, H_q, Tq]")
    _check("attn_prefill_fp8", load().attn_prefill_fp8(
        _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), _ptr(key_padding_mask),
        _ptr(out), _ptr(lse if want_lse else None), B, Hq, Hkv, Tq, Tk, D, 1 if causal else 0, float(scale),
        _stream(q.device)))
    return (out, lse) if want_lse else out


def attn_prefill_varlen_fp8(q, k, v, q_scale, k_scale, v_scale, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                            causal=False, scale=None, out=None, lse=None, want_lse: bool = True):
    """attn_prefill_varlen on E4M3 codes: q uint8 [total_q, H_q, D], k/v uint8 [total_k, H_kv, D]
    (or torch.float8_e4m3fn), per-(sequence, head) float32 scales q_scale [B, H_q], k_scale /
    v_scale [B, H_kv].  Returns O bf16 [total_q, H_q, D] (and the LSE [H_q, total_q])."""
    q, k, v = (t.view(torch.uint8) if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn else t
               for t in (q, k, v))
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (q_scale, "q_scale"), (k_scale, "k_scale"), (v_scale, "v_scale"),
                 (cu_seqlens_q, "cu_seqlens_q"), (cu_seqlens_k, "cu_seqlens_k")):
        _dev(t, n)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3 or q.dtype != torch.uint8 or k.dtype != torch.uint8 \
            or v.dtype != torch.uint8:
        raise ValueError("q, k, v must be E4M3 codes [total, H, D]")
    total_q, Hq, D = q.shape
    total_k, Hkv, _ = k.shape
    if k.shape[2] != D or v.shape != k.shape:
        raise ValueError("k/v must be [total_k, H_kv, D] with q's D")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32 or cu_seqlens_q.dim() != 1 \
            or cu_seqlens_k.shape != cu_seqlens_q.shape:
        raise ValueError("cu_seqlens_q / cu_seqlens_k must be int32 [B + 1]")
    B = cu_seqlens_q.numel() - 1
    for t, n, shp in ((q_scale, "q_scale", (B, Hq)), (k_scale, "k_scale", (B, Hkv)), (v_scale, "v_scale", (B, Hkv))):
        if t.shape != shp or t.dtype != torch.float32:
            raise ValueError(f"{n} must be float32 {list(shp)}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((total_q, Hq, D), dtype=torch.bfloat16, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    _check("attn_prefill_varlen_fp8", load().attn_prefill_varlen_fp8(
        _ptr(q), _ptr(k), _ptr(v), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_k), _ptr(out), _ptr(lse if want_lse else None), B, Hq, Hkv, total_q, total_k,
        int(max_seqlen_q), D, 1 if causal else 0, float(scale), _stream(q.device)))
    return (out, lse) if want_lse else out


def _q8_paged_args(k_pages, v_pages, k_scale, v_scale, block_table, cache_seqlens, B, code_dtype):
    num_pages, Hkv, ps, D, mp = _paged_args(k_pages, v_pages, block_table, cache_seqlens, B)
    if k_pages.dtype != code_dtype or v_pages.dtype != code_dtype:
        raise ValueError(f"k_pages / v_pages must hold {code_dtype} codes")
    for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        _dev(t, n)
        if t.shape != (B, Hkv) or t.dtype != torch.float32:
            raise ValueError(f"{n} must be float32 [B, H_kv]")
    return num_pages, Hkv, ps, D, mp


def _q8_append_paged(fn, code_dtype, k_pages, v_pages, k_scale, v_scale, block_table, cache_seqlens, k_new, v_new):
    _dev(k_new, "k_new")
    _dev(v_new, "v_new")
    B = k_new.shape[0]
    num_pages, Hkv, ps, D, mp = _q8_paged_args(k_pages, v_pages, k_scale, v_scale, block_table, cache_seqlens, B,
                                               code_dtype)
    if k_new.shape != (B, Hkv, 1, D) or v_new.shape != (B, Hkv, 1, D) or v_new.dtype != k_new.dtype:
        raise ValueError("k_new / v_new must be [B, H_kv, 1, D] of one dtype")
    _check(fn, getattr(load(), fn)(
        _ptr(k_pages), _ptr(v_pages), _ptr(k_scale), _ptr(v_scale), _ptr(block_table), _ptr(cache_seqlens),
        _ptr(k_new), _ptr(v_new), B, Hkv, num_pages, ps, mp, D, _dtype_code(k_new), _stream(k_pages.device)))


def _q8_decode_paged(fn, code_dtype, q, k_pages, v_pages, k_scale, v_scale, block_table, cache_seqlens, scale, out,
                     lse, workspace, want_lse):
    _dev(q, "q")
    if q.dim() != 4 or q.shape[2] != 1 or q.dtype != torch.bfloat16:
        raise ValueError("q must be bfloat16 [B, H_q, 1, D]")
    B, Hq, _, D = q.shape
    num_pages, Hkv, ps, Dk, mp = _q8_paged_args(k_pages, v_pages, k_scale, v_scale, block_table, cache_seqlens, B,
                                                code_dtype)
    if Dk != D:
        raise ValueError("pool head_dim does not match q")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = attn_decode_workspace_bytes(B, Hq, Hkv, mp * ps, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check(fn, getattr(load(), fn)(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scale), _ptr(v_scale), _ptr(block_table), _ptr(cache_seqlens),
        _ptr(out), _ptr(lse if want_lse else None), B, Hq, Hkv, num_pages, ps, mp, D, float(scale), _ptr(workspace),
        nbytes, _stream(q.device)))
    return (out, lse) if want_lse else out


def kv_append_fp8_paged(k_pages, v_pages, k_scale, v_scale, block_table, cache_seqlens, k_new, v_new):
    """kv_append_fp8 into E4M3 page pools [num_pages, H_kv, page_size, D] (uint8) through block_table."""
    _q8_append_paged("kv_append_fp8_paged", torch.uint8, k_pages, v_pages, k_scale, v_scale, block_table,
                     cache_seqlens, k_new, v_new)


def kv_append_int8_paged(k_pages, v_pages, k_scale, v_scale, block_table, cache_seqlens, k_new, v_new):
    """kv_append_int8 into INT8 page pools [num_pages, H_kv, page_size, D] (int8) through block_table."""
    _q8_append_paged("kv_append_int8_paged", torch.int8, k_pages, v_pages, k_scale, v_scale, block_table,
                     cache_seqlens, k_new, v_new)


def attn_decode_fp8kv_paged(q, k_pages, v_pages, k_scale, v_scale, block_table, cache_seqlens, scale=None, out=None,
                            lse=None, workspace=None, want_lse: bool = False):
    """attn_decode_fp8kv over E4M3 page pools through block_table [B, max_pages]."""
    return _q8_decode_paged("attn_decode_fp8kv_paged", torch.uint8, q, k_pages, v_pages, k_scale, v_scale,
                            block_table, cache_seqlens, scale, out, lse, workspace, want_lse)


def attn_decode_int8kv_paged(q, k_pages, v_pages, k_scale, v_scale, block_table, cache_seqlens, scale=None, out=None,
                             lse=None, workspace=None, want_lse: bool = False):
    """attn_decode_int8kv over INT8 page pools through block_table [B, max_pages]."""
    return _q8_decode_paged("attn_decode_int8kv_paged", torch.int8, q, k_pages, v_pages, k_scale, v_scale,
                            block_table, cache_seqlens, scale, out, lse, workspace, want_lse)

"""CPU oracle for the INT8 key/value cache.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the library never
imports it and it shares no code with the HIP path.

KV-cache quantisation keeps each cached K/V element in fewer bytes plus scale
metadata and dequantises inside the attention kernel; INT8 is one of the
formats the page lists (LLM inference memory accounting 2/10, section
"18. KV Quantization은 Byte와 Kernel을 함께 바꾼다").  The page fixes neither the scale granularity
nor the rounding; the readings taken here:
  * symmetric INT8: code q stands for q * scale, with one float32 scale per
    (sequence, KV head) for K and one for V (the FP8 cache's granularity);
  * quantising x: y = x / scale in float32 (IEEE division), rounded to the
    nearest integer with ties to even, clamped to [-127, 127] (the symmetric
    range; -128 is never written, and decodes as -128 if present).
Decoding against the quantised cache is exactly ``decode`` applied to the
dequantised caches.
"""
from __future__ import annotations

import numpy as np

from .attention import decode, gather_pages, kv_append_paged, _f64

__all__ = ["INT8_MAX", "quantize_int8", "dequantize_int8", "kv_append_int8", "decode_int8kv",
           "kv_append_int8_paged", "decode_int8kv_paged"]

INT8_MAX = 127


def quantize_int8(x, scale):
    """int8 codes of x / scale (float32 division, nearest integer with ties to even, clamped
    to +-127).  x: any shape (taken as float32); scale broadcasts against x."""
    x32 = np.asarray(_f64(x), dtype=np.float32)
    s32 = np.asarray(_f64(scale), dtype=np.float32)
    y = (x32 / s32).astype(np.float64)                       # IEEE float32 division
    y = np.rint(y)                                           # round half to even
    return np.clip(y, -INT8_MAX, INT8_MAX).astype(np.int8)


def dequantize_int8(codes, scale):
    """float64 values code * scale."""
    codes = np.asarray(codes.detach().cpu().numpy() if hasattr(codes, "detach") else codes)
    return codes.astype(np.int8).astype(np.float64) * np.asarray(_f64(scale))


def kv_append_int8(k_cache, v_cache, k_scale, v_scale, lens, k_new, v_new):
    """Quantise one new token per sequence into slot lens[b] of the int8 caches.

    k_cache/v_cache int8 [B, H_kv, T_max, D]; k_scale/v_scale [B, H_kv];
    k_new/v_new [B, H_kv, 1, D] (any float dtype).  Returns copies of the caches
    and lens + 1.
    """
    kc = np.array(k_cache, dtype=np.int8, copy=True)
    vc = np.array(v_cache, dtype=np.int8, copy=True)
    lens = np.asarray(lens).astype(np.int64)
    ks, vs = _f64(k_scale), _f64(v_scale)
    kn, vn = _f64(k_new), _f64(v_new)
    for b in range(kc.shape[0]):
        t = int(lens[b])
        assert 0 <= t < kc.shape[2], "cache full"
        kc[b, :, t, :] = quantize_int8(kn[b, :, 0, :], ks[b][:, None])
        vc[b, :, t, :] = quantize_int8(vn[b, :, 0, :], vs[b][:, None])
    return kc, vc, lens + 1


def decode_int8kv(q, k_cache, v_cache, k_scale, v_scale, lens, scale=None, heads=None):
    """``decode`` against the dequantised caches (code x per-(b, KV head) scale)."""
    kd = dequantize_int8(k_cache, _f64(k_scale)[:, :, None, None])
    vd = dequantize_int8(v_cache, _f64(v_scale)[:, :, None, None])
    return decode(q, kd, vd, lens, scale, heads)


def kv_append_int8_paged(k_pages, v_pages, k_scale, v_scale, block_table, lens, k_new, v_new):
    """``kv_append_int8`` into page pools [num_pages, H_kv, page_size, D] of codes: the new token's
    codes (quantised with its (b, KV head) scales) are written at logical slot lens[b] through
    the block table, as ``kv_append_paged``.  Returns copies of the pools and lens + 1."""
    ks, vs = _f64(k_scale), _f64(v_scale)
    kn = quantize_int8(_f64(k_new), ks[:, :, None, None])
    vn = quantize_int8(_f64(v_new), vs[:, :, None, None])
    kp = np.asarray(k_pages.detach().cpu().numpy() if hasattr(k_pages, "detach") else k_pages)
    vp = np.asarray(v_pages.detach().cpu().numpy() if hasattr(v_pages, "detach") else v_pages)
    return kv_append_paged(kp.astype(np.int8), vp.astype(np.int8), block_table, lens, kn, vn)


def decode_int8kv_paged(q, k_pages, v_pages, k_scale, v_scale, block_table, lens, scale=None, heads=None):
    """``decode_int8kv`` over page pools of codes: each sequence's first lens[b] codes are gathered
    through its block-table row into a contiguous cache, which is then decoded as
    ``decode_int8kv`` (per-(sequence, KV head) scales)."""
    lens = np.asarray(lens).astype(np.int64)
    kp, vp = _f64(k_pages), _f64(v_pages)
    B, H_kv, D = lens.size, kp.shape[1], kp.shape[3]
    T = max(1, int(lens.max()) if lens.size else 1)
    kc = np.zeros((B, H_kv, T, D), dtype=np.int8)
    vc = np.zeros((B, H_kv, T, D), dtype=np.int8)
    for b in range(B):
        n = int(lens[b])
        kc[b, :, :n] = gather_pages(kp, block_table, b, n).astype(np.int8)
        vc[b, :, :n] = gather_pages(vp, block_table, b, n).astype(np.int8)
    return decode_int8kv(q, kc, vc, k_scale, v_scale, lens, scale, heads)

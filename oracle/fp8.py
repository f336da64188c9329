"""CPU oracle for the FP8 (E4M3) key/value cache.

TEST INFRASTRUCTURE ONLY, like the rest of this package: the library never
imports it and it shares no code with the HIP path.

KV-cache quantisation stores each cached K/V element in fewer bytes plus scale
metadata, and the attention kernel must dequantise on the fly (LLM inference
memory accounting 2/10, section "18. KV Quantization은 Byte와 Kernel을 함께 바꾼다": lower-precision
KV halves or quarters the bytes per token and brings scales and a dequant
step with it).  The pages fix neither the 8-bit format nor the scale
granularity; the readings taken here:
  * format: OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent bits with bias 7,
    3 mantissa bits, subnormals, no infinities, S.1111.111 = NaN, largest
    finite magnitude 448;
  * one float32 scale per (sequence, KV head) for K and one for V: the cached
    value of element x is q(x) * scale;
  * quantising x: y = x / scale in float32 (IEEE division), clamped to
    [-448, 448], rounded to the nearest E4M3 value, ties to the even mantissa.
Decoding against the quantised cache is exactly ``decode`` applied to the
dequantised caches.

FP8 prefill with LSE: the aiter ring-attention analysis (sglang PR 49078
analysis, section "1. aiter.py") notes that the FP8 prefill kernel there
returns no LSE, so a ring hop that needs the LSE falls back to BF16.  The
FP8 prefill here keeps the LSE.  Reading taken: Q, K and V all arrive as E4M3
codes, with one float32 scale per (sequence, query head) for Q and one per
(sequence, KV head) for K and for V; the result is exactly ``prefill`` (GQA,
optional key padding, optional causal limit) on the dequantised tensors.
"""
from __future__ import annotations

import numpy as np

from .attention import decode, prefill, prefill_varlen, gather_pages, kv_append_paged, _f64

__all__ = ["E4M3_MAX", "e4m3_values", "quantize_e4m3", "dequantize_e4m3", "kv_append_fp8", "decode_fp8kv",
           "prefill_fp8", "prefill_varlen_fp8",
           "kv_append_fp8_paged", "decode_fp8kv_paged"]

E4M3_MAX = 448.0


def e4m3_values():
    """float64 [256]: the value of every byte under E4M3 (NaN for the two NaN codes)."""
    out = np.empty(256)
    for byte in range(256):
        s = -1.0 if byte & 0x80 else 1.0
        e = (byte >> 3) & 0xF
        m = byte & 0x7
        if e == 0xF and m == 0x7:
            out[byte] = np.nan
        elif e == 0:
            out[byte] = s * (m / 8.0) * 2.0 ** (1 - 7)          # subnormal
        else:
            out[byte] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_VALS = e4m3_values()
# non-negative finite codes in increasing value order (0x00 .. 0x7E)
_POS_CODES = np.arange(0x7F)
_POS_VALS = _VALS[:0x7F]


def _round_e4m3_magnitude(a):
    """Codes (0..0x7E) of the nearest E4M3 magnitudes to a >= 0 (a <= 448), ties to even."""
    a = np.asarray(a, dtype=np.float64)
    hi = np.searchsorted(_POS_VALS, a, side="left")          # first value >= a
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    dlo = a - _POS_VALS[lo]
    dhi = _POS_VALS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0) & (hi != lo))
    return np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])


def quantize_e4m3(x, scale):
    """uint8 codes of x / scale (float32 division, clamped to +-448, nearest, ties to even).

    x: any shape (its values are taken as float32); scale broadcasts against x.
    """
    x32 = np.asarray(_f64(x), dtype=np.float32)
    s32 = np.asarray(_f64(scale), dtype=np.float32)
    y = (x32 / s32).astype(np.float64)                       # IEEE float32 division
    y = np.clip(y, -E4M3_MAX, E4M3_MAX)
    code = _round_e4m3_magnitude(np.abs(y))
    neg = (y < 0) | ((y == 0) & np.signbit(y))
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def dequantize_e4m3(codes, scale):
    """float64 values code_value * scale (exact: both factors are exact in float64)."""
    codes = np.asarray(codes.detach().cpu().numpy() if hasattr(codes, "detach") else codes, dtype=np.uint8)
    return _VALS[codes] * np.asarray(_f64(scale))


def kv_append_fp8(k_cache, v_cache, k_scale, v_scale, lens, k_new, v_new):
    """Quantise one new token per sequence into slot lens[b] of the uint8 caches.

    k_cache/v_cache uint8 [B, H_kv, T_max, D]; k_scale/v_scale [B, H_kv];
    k_new/v_new [B, H_kv, 1, D] (any float dtype).  Returns copies of the
    caches and lens + 1.
    """
    kc = np.array(k_cache, dtype=np.uint8, copy=True)
    vc = np.array(v_cache, dtype=np.uint8, copy=True)
    lens = np.asarray(lens).astype(np.int64)
    ks, vs = _f64(k_scale), _f64(v_scale)
    kn, vn = _f64(k_new), _f64(v_new)
    for b in range(kc.shape[0]):
        t = int(lens[b])
        assert 0 <= t < kc.shape[2], "cache full"
        kc[b, :, t, :] = quantize_e4m3(kn[b, :, 0, :], ks[b][:, None])
        vc[b, :, t, :] = quantize_e4m3(vn[b, :, 0, :], vs[b][:, None])
    return kc, vc, lens + 1


def decode_fp8kv(q, k_cache, v_cache, k_scale, v_scale, lens, scale=None, heads=None):
    """``decode`` against the dequantised caches (code value x per-(b, KV head) scale)."""
    ks = _f64(k_scale)[:, :, None, None]
    vs = _f64(v_scale)[:, :, None, None]
    kd = dequantize_e4m3(k_cache, ks)
    vd = dequantize_e4m3(v_cache, vs)
    return decode(q, kd, vd, lens, scale, heads)


def prefill_fp8(q, k, v, q_scale, k_scale, v_scale, key_padding_mask=None, causal=False, scale=None,
                rows=None):
    """``prefill`` on dequantised E4M3 inputs.

    q uint8 [B, H_q, Tq, D], k and v uint8 [B, H_kv, Tk, D]; q_scale [B, H_q],
    k_scale and v_scale [B, H_kv].  Element x of Q stands for value(x) * q_scale[b, h]
    (K and V likewise with their KV head's scale).  Returns O and LSE as ``prefill``.
    """
    qd = dequantize_e4m3(q, _f64(q_scale)[:, :, None, None])
    kd = dequantize_e4m3(k, _f64(k_scale)[:, :, None, None])
    vd = dequantize_e4m3(v, _f64(v_scale)[:, :, None, None])
    return prefill(qd, kd, vd, key_padding_mask, causal, scale, rows)


def prefill_varlen_fp8(q, k, v, q_scale, k_scale, v_scale, cu_seqlens_q, cu_seqlens_k, causal=False, scale=None):
    """``prefill_varlen`` on dequantised E4M3 inputs.

    q uint8 [total_q, H_q, D], k and v uint8 [total_k, H_kv, D] (packed sequences as in
    ``attention_varlen``); q_scale [B, H_q], k_scale and v_scale [B, H_kv], one per (sequence,
    head).  Returns O [total_q, H_q, D] and LSE [H_q, total_q] as ``prefill_varlen``.
    """
    cq = np.asarray(_f64(cu_seqlens_q), dtype=np.int64)
    ck = np.asarray(_f64(cu_seqlens_k), dtype=np.int64)
    qs, ks, vs = _f64(q_scale), _f64(k_scale), _f64(v_scale)
    B = cq.size - 1
    # per-row scales: row t of sequence b takes that sequence's (b, head) scale
    bq = np.repeat(np.arange(B), np.diff(cq))
    bk = np.repeat(np.arange(B), np.diff(ck))
    qd = dequantize_e4m3(q, qs[bq][:, :, None])
    kd = dequantize_e4m3(k, ks[bk][:, :, None])
    vd = dequantize_e4m3(v, vs[bk][:, :, None])
    return prefill_varlen(qd, kd, vd, cq, ck, causal, scale)


def kv_append_fp8_paged(k_pages, v_pages, k_scale, v_scale, block_table, lens, k_new, v_new):
    """``kv_append_fp8`` into page pools [num_pages, H_kv, page_size, D] of codes: the new token's
    codes (quantised with its (b, KV head) scales) are written at logical slot lens[b] through
    the block table, as ``kv_append_paged``.  Returns copies of the pools and lens + 1."""
    ks, vs = _f64(k_scale), _f64(v_scale)
    kn = quantize_e4m3(_f64(k_new), ks[:, :, None, None])
    vn = quantize_e4m3(_f64(v_new), vs[:, :, None, None])
    kp = np.asarray(k_pages.detach().cpu().numpy() if hasattr(k_pages, "detach") else k_pages)
    vp = np.asarray(v_pages.detach().cpu().numpy() if hasattr(v_pages, "detach") else v_pages)
    return kv_append_paged(kp.astype(np.uint8), vp.astype(np.uint8), block_table, lens, kn, vn)


def decode_fp8kv_paged(q, k_pages, v_pages, k_scale, v_scale, block_table, lens, scale=None, heads=None):
    """``decode_fp8kv`` over page pools of codes: each sequence's first lens[b] codes are gathered
    through its block-table row into a contiguous cache, which is then decoded as
    ``decode_fp8kv`` (per-(sequence, KV head) scales)."""
    lens = np.asarray(lens).astype(np.int64)
    kp, vp = _f64(k_pages), _f64(v_pages)
    B, H_kv, D = lens.size, kp.shape[1], kp.shape[3]
    T = max(1, int(lens.max()) if lens.size else 1)
    kc = np.zeros((B, H_kv, T, D), dtype=np.uint8)
    vc = np.zeros((B, H_kv, T, D), dtype=np.uint8)
    for b in range(B):
        n = int(lens[b])
        kc[b, :, :n] = gather_pages(kp, block_table, b, n).astype(np.uint8)
        vc[b, :, :n] = gather_pages(vp, block_table, b, n).astype(np.uint8)
    return decode_fp8kv(q, kc, vc, k_scale, v_scale, lens, scale, heads)

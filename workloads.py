"""Seeded synthetic inputs for the attention library and its CPU oracle.

This module holds no attention arithmetic: it draws random tensors, casts
them to the storage dtype, and builds key-padding masks and cache lengths.
Both the GPU path (tests, bench) and the oracle receive exactly the tensors
made here, so the oracle sees the same bits the kernels see (the bf16 cast
happens once, here).

Recipe (shared by every workload):
  * CPU ``torch.Generator().manual_seed(seed)``, seed 0 unless stated; the
    mask-polarity demonstration on the MultiheadAttention fast-path page
    (molayo1419.me, section "출력은 달라졌는가") seeds its RNG with 0 too.
  * ``torch.randn`` in the order Q, K, V (decode: lengths, K cache, V cache,
    k_new, v_new, Q), multiplied by ``amp`` (a power of two, so exact), then
    ``.to(dtype)`` (round-to-nearest-even for bf16).
  * Key-padding masks are uint8 ``[B, Tk]``, nonzero = padded = ignored (the
    nn.MultiheadAttention ``key_padding_mask`` polarity the same page warns
    about), built from per-sequence valid lengths or an explicit pattern.

The named workloads mirror the shapes the pages measure: 16-head patch
self-attention at P = 1,944 and 11,616 patches (0.5 MP and ~3 MP images cut
into 16x16-pixel patches; MultiheadAttention fast-path page, section
"무엇이 일어나고 있었는가"), a 512-token 16-head fp32 case matching the CPU
profiler run on that page ("프로파일러로 검증하기"), a two-chunk KV split as
one ring-attention hop sees it (sglang PR 49078 analysis, section "1. aiter.py"),
and GQA decode with 32 query / 8 KV heads at head_dim 128 (LLM inference
memory accounting 2/10, section "11. 계산 예시: GQA Decoder").
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

__all__ = [
    "Prefill", "Chunked", "Decode", "Varlen", "Paged", "to_paged",
    "make_prefill", "make_chunked", "make_decode", "make_varlen", "cu_from_lengths",
    "mask_from_valid_lengths", "round_up",
    "fp32_masked_t512", "patch_p1944", "patch_p11616",
    "chunked_kv_2x8192", "gqa_decode_b32", "varlen_p1944_packed", "varlen_ring_hop_8192",
    "gqa_decode_b32_paged", "DecodeFp8", "make_decode_fp8", "gqa_decode_b32_fp8", "make_gqa_prefill", "gqa_causal_prefill_8192", "gqa_causal_prompts_packed",
]


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


@dataclass
class Prefill:
    q: torch.Tensor            # [B, H, Tq, D]
    k: torch.Tensor            # [B, H, Tk, D]
    v: torch.Tensor            # [B, H, Tk, D]
    mask: Optional[torch.Tensor]  # uint8 [B, Tk], nonzero = padded; None = no padding
    scale: float
    name: str = ""

    @property
    def shape(self):
        B, H, Tq, D = self.q.shape
        return B, H, Tq, self.k.shape[2], D


@dataclass
class Chunked:
    q: torch.Tensor                    # [B, H, Tq, D]
    k_chunks: list                     # each [B, H, Tk_i, D]
    v_chunks: list
    scale: float
    name: str = ""


@dataclass
class Decode:
    q: torch.Tensor        # [B, H_q, 1, D]
    k_cache: torch.Tensor  # [B, H_kv, T_max, D]
    v_cache: torch.Tensor
    k_new: torch.Tensor    # [B, H_kv, 1, D]
    v_new: torch.Tensor
    lens: torch.Tensor     # int32 [B], cached length BEFORE the append
    scale: float
    name: str = ""


@dataclass
class Varlen:
    q: torch.Tensor        # [total_q, H, D]
    k: torch.Tensor        # [total_k, H, D]
    v: torch.Tensor
    cu_q: torch.Tensor     # int32 [B + 1], 0 .. total_q
    cu_k: torch.Tensor     # int32 [B + 1], 0 .. total_k
    max_q: int
    scale: float
    name: str = ""

    @property
    def lens_q(self):
        return (self.cu_q[1:] - self.cu_q[:-1]).tolist()

    @property
    def lens_k(self):
        return (self.cu_k[1:] - self.cu_k[:-1]).tolist()


@dataclass
class Paged:
    """A decode workload with its caches scattered into a pool of physical pages."""
    dec: Decode
    k_pages: torch.Tensor      # [num_pages, H_kv, page_size, D]
    v_pages: torch.Tensor
    block_table: torch.Tensor  # int32 [B, max_pages]: logical page i of b -> physical page
    page_size: int


@dataclass
class DecodeFp8:
    """Decode inputs with an E4M3 cache: codes (uint8) and float32 scales per (b, KV head)."""
    q: torch.Tensor        # [B, H_q, 1, D] bf16
    k_cache: torch.Tensor  # [B, H_kv, T_max, D] uint8 (E4M3 codes)
    v_cache: torch.Tensor
    k_scale: torch.Tensor  # [B, H_kv] float32
    v_scale: torch.Tensor
    k_new: torch.Tensor    # [B, H_kv, 1, D] bf16
    v_new: torch.Tensor
    lens: torch.Tensor     # int32 [B], cached length BEFORE the append
    scale: float
    name: str = ""


@dataclass
class PrefillFp8:
    """Prefill inputs as E4M3 codes with float32 scales per (b, head)."""
    q: torch.Tensor        # [B, H_q, Tq, D] uint8 (E4M3 codes)
    k: torch.Tensor        # [B, H_kv, Tk, D] uint8
    v: torch.Tensor
    q_scale: torch.Tensor  # [B, H_q] float32
    k_scale: torch.Tensor  # [B, H_kv] float32
    v_scale: torch.Tensor
    mask: Optional[torch.Tensor]  # uint8 [B, Tk], nonzero = padded; None = no padding
    scale: float
    name: str = ""


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(seed)
    return g


def _randn(g, shape, amp, dtype):
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if amp != 1.0:
        x.mul_(amp)
    return x.to(dtype).contiguous()


def randn_device(shape, seed: int, device, dtype=torch.bfloat16, amp=1.0) -> torch.Tensor:
    """Seeded N(0, amp^2) values drawn on `device` in float32, then cast (round to nearest even),
    for inputs of billions of elements that the host would take minutes to draw.  The same
    tensor serves both sides: the caller copies it to the host for the oracle."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if amp != 1.0:
        x.mul_(amp)
    return x.to(dtype)


def _uniform_scales(seed: int, shape, lo=0.01, hi=2.0) -> torch.Tensor:
    """Float32 scale factors U[lo, hi) from a generator of their own (seed + 7919), so that
    asking for them leaves every other draw of a workload unchanged.  Unlike powers of two,
    their products with the softmax scale and with each other round in float32."""
    g = _gen(seed + 7919)
    return (lo + (hi - lo) * torch.rand(*shape, generator=g)).float().contiguous()


def mask_from_valid_lengths(valid: Sequence[int], Tk: int) -> torch.Tensor:
    """uint8 [B, Tk]; keys at index >= valid[b] are marked padded (1)."""
    idx = torch.arange(Tk)
    return torch.stack([(idx >= int(n)).to(torch.uint8) for n in valid]).contiguous()


def make_prefill(B, H, Tq, Tk, D, dtype=torch.bfloat16, *, valid=None, mask=None,
                 amp=1.0, seed=0, scale=None, name="") -> Prefill:
    g = _gen(seed)
    q = _randn(g, (B, H, Tq, D), amp, dtype)
    k = _randn(g, (B, H, Tk, D), amp, dtype)
    v = _randn(g, (B, H, Tk, D), amp, dtype)
    if mask is None and valid is not None:
        mask = mask_from_valid_lengths(valid, Tk)
    if mask is not None:
        mask = mask.to(torch.uint8).contiguous()
        assert mask.shape == (B, Tk)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Prefill(q, k, v, mask, float(scale), name)


def make_chunked(B, H, Tq, chunk_lens, D, dtype=torch.bfloat16, *, amp=1.0, seed=0,
                 scale=None, name="") -> Chunked:
    """Q plus K/V drawn as one [B, H, sum(chunk_lens), D] tensor, then split."""
    g = _gen(seed)
    Tk = int(sum(chunk_lens))
    q = _randn(g, (B, H, Tq, D), amp, dtype)
    k = _randn(g, (B, H, Tk, D), amp, dtype)
    v = _randn(g, (B, H, Tk, D), amp, dtype)
    ks, vs, s = [], [], 0
    for n in chunk_lens:
        ks.append(k[:, :, s:s + n].contiguous())
        vs.append(v[:, :, s:s + n].contiguous())
        s += n
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Chunked(q, ks, vs, float(scale), name)


def make_decode(B, H_q, H_kv, D, len_lo, len_hi, dtype=torch.bfloat16, *, T_max=None,
                amp=1.0, seed=0, scale=None, lens=None, name="") -> Decode:
    """Cached lengths uniform in [len_lo, len_hi] (inclusive) unless given.

    T_max defaults to the smallest multiple of 64 that holds the longest
    sequence after one appended token.
    """
    g = _gen(seed)
    if lens is None:
        lens = torch.randint(len_lo, len_hi + 1, (B,), generator=g, dtype=torch.int64)
    lens = torch.as_tensor(lens, dtype=torch.int64)
    if T_max is None:
        T_max = round_up(len_hi + 1, 64)
    kc = _randn(g, (B, H_kv, T_max, D), amp, dtype)
    vc = _randn(g, (B, H_kv, T_max, D), amp, dtype)
    kn = _randn(g, (B, H_kv, 1, D), amp, dtype)
    vn = _randn(g, (B, H_kv, 1, D), amp, dtype)
    q = _randn(g, (B, H_q, 1, D), amp, dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Decode(q, kc, vc, kn, vn, lens.to(torch.int32), float(scale), name)


def cu_from_lengths(lens: Sequence[int]) -> torch.Tensor:
    """int32 [B + 1] running totals 0, l0, l0 + l1, ... of the sequence lengths."""
    c = [0]
    for n in lens:
        assert int(n) >= 0
        c.append(c[-1] + int(n))
    return torch.tensor(c, dtype=torch.int32)


def make_varlen(lens_q, lens_k, H, D, dtype=torch.bfloat16, *, H_kv=None, amp=1.0, seed=0, scale=None,
                name="") -> Varlen:
    """Packed [total, H, D] Q and [total, H_kv, D] K, V (H_kv defaults to H) for sequences of
    the given query / key lengths."""
    assert len(lens_q) == len(lens_k) >= 1
    H_kv = H if H_kv is None else H_kv
    g = _gen(seed)
    cq, ck = cu_from_lengths(lens_q), cu_from_lengths(lens_k)
    tq, tk = int(cq[-1]), int(ck[-1])
    q = _randn(g, (tq, H, D), amp, dtype)
    k = _randn(g, (tk, H_kv, D), amp, dtype)
    v = _randn(g, (tk, H_kv, D), amp, dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Varlen(q, k, v, cq, ck, max([int(n) for n in lens_q]), float(scale), name)


@dataclass
class VarlenFp8:
    """Packed prefill inputs as E4M3 codes with float32 scales per (sequence, head)."""
    q: torch.Tensor        # [total_q, H_q, D] uint8
    k: torch.Tensor        # [total_k, H_kv, D] uint8
    v: torch.Tensor
    q_scale: torch.Tensor  # [B, H_q] float32
    k_scale: torch.Tensor  # [B, H_kv] float32
    v_scale: torch.Tensor
    cu_q: torch.Tensor     # int32 [B + 1]
    cu_k: torch.Tensor
    max_q: int
    scale: float
    name: str = ""


def make_varlen_fp8(lens_q, lens_k, H, D, *, H_kv=None, amp=1.0, seed=0, scale=None, name="",
                    scales="pow2") -> VarlenFp8:
    """Packed E4M3 inputs whose dequantised values are about N(0, amp^2), with make_prefill_fp8's
    recipe per (sequence, head): scale amp * 2^-e, e ~ U{2..6}, codes N(0,1) * 2^e cast to
    float8_e4m3fn.  Draw order: Q, K, V scale exponents, then Q, K, V.  scales="uniform" as
    make_prefill_fp8."""
    H_kv = H if H_kv is None else H_kv
    g = _gen(seed)
    B = len(lens_q)
    cq, ck = cu_from_lengths(lens_q), cu_from_lengths(lens_k)
    tq, tk = int(cq[-1]), int(ck[-1])
    eq = torch.randint(2, 7, (B, H), generator=g)
    ek = torch.randint(2, 7, (B, H_kv), generator=g)
    ev = torch.randint(2, 7, (B, H_kv), generator=g)
    rq = torch.repeat_interleave(torch.arange(B), torch.as_tensor(lens_q, dtype=torch.int64))
    rk = torch.repeat_interleave(torch.arange(B), torch.as_tensor(lens_k, dtype=torch.int64))

    def codes(total, heads, e, rows):
        x = torch.randn(total, heads, D, generator=g) * torch.exp2(e.float())[rows][:, :, None]
        return x.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()

    q = codes(tq, H, eq, rq)
    k = codes(tk, H_kv, ek, rk)
    v = codes(tk, H_kv, ev, rk)
    sc = lambda e: (amp * torch.exp2(-e.float())).contiguous()
    qs, ks, vs = sc(eq), sc(ek), sc(ev)
    if scales == "uniform":
        uq = _uniform_scales(seed, (B, H))
        uk, uv = _uniform_scales(seed + 1, (2, B, H_kv))
        qs, ks, vs = (qs * uq).contiguous(), (ks * uk).contiguous(), (vs * uv).contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return VarlenFp8(q, k, v, qs, ks, vs, cq, ck, max([int(n) for n in lens_q]), float(scale), name)


def to_paged(dec: Decode, page_size: int, *, seed=1, spare_pages=3) -> Paged:
    """Scatter the contiguous caches of `dec` into shuffled physical pages.

    Logical page i of sequence b (tokens i*page_size .. +page_size-1 of its T_max slots)
    is copied to physical page block_table[b, i], a seeded random permutation of
    B*max_pages + spare_pages pages (the spares hold random data and are never mapped).
    A bit copy: the paged and contiguous caches hold the same values.
    """
    B, H_kv, T_max, D = dec.k_cache.shape
    assert T_max % page_size == 0
    mp = T_max // page_size
    n = B * mp + spare_pages
    g = _gen(seed)
    perm = torch.randperm(n, generator=g)
    bt = perm[:B * mp].reshape(B, mp).to(torch.int32).contiguous()
    kp = _randn(g, (n, H_kv, page_size, D), 1.0, dec.k_cache.dtype)
    vp = _randn(g, (n, H_kv, page_size, D), 1.0, dec.k_cache.dtype)
    kc = dec.k_cache.reshape(B, H_kv, mp, page_size, D).permute(0, 2, 1, 3, 4)   # [B, mp, H_kv, ps, D]
    vc = dec.v_cache.reshape(B, H_kv, mp, page_size, D).permute(0, 2, 1, 3, 4)
    kp[bt.reshape(-1).long()] = kc.reshape(B * mp, H_kv, page_size, D)
    vp[bt.reshape(-1).long()] = vc.reshape(B * mp, H_kv, page_size, D)
    return Paged(dec, kp.contiguous(), vp.contiguous(), bt, page_size)


def make_decode_fp8(B, H_q, H_kv, D, len_lo, len_hi, *, T_max=None, seed=0, scale=None, lens=None,
                    name="", scales="pow2") -> DecodeFp8:
    """E4M3 caches drawn as N(0,1) cast to float8_e4m3fn (round to nearest even), scales
    2^U{-6..-2} per (b, KV head) (scales="uniform": U[0.01, 2) instead, from their own
    generator), new tokens N(0,1) times their head's scale in bf16 (so they quantise into the
    bulk of the code range), Q N(0,1) bf16.  Draw order: lengths, K cache, V cache, K scale
    exponents, V scale exponents, k_new, v_new, Q."""
    g = _gen(seed)
    if lens is None:
        lens = torch.randint(len_lo, len_hi + 1, (B,), generator=g, dtype=torch.int64)
    lens = torch.as_tensor(lens, dtype=torch.int64)
    if T_max is None:
        T_max = round_up(len_hi + 1, 64)
    kc = torch.randn(B, H_kv, T_max, D, generator=g).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    vc = torch.randn(B, H_kv, T_max, D, generator=g).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    ks = torch.exp2(torch.randint(-6, -1, (B, H_kv), generator=g).float()).contiguous()
    vs = torch.exp2(torch.randint(-6, -1, (B, H_kv), generator=g).float()).contiguous()
    if scales == "uniform":
        ks, vs = _uniform_scales(seed, (2, B, H_kv))
    kn = (torch.randn(B, H_kv, 1, D, generator=g) * ks[:, :, None, None]).to(torch.bfloat16).contiguous()
    vn = (torch.randn(B, H_kv, 1, D, generator=g) * vs[:, :, None, None]).to(torch.bfloat16).contiguous()
    q = torch.randn(B, H_q, 1, D, generator=g).to(torch.bfloat16).contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return DecodeFp8(q, kc, vc, ks, vs, kn, vn, lens.to(torch.int32), float(scale), name)


def make_decode_int8(B, H_q, H_kv, D, len_lo, len_hi, *, T_max=None, seed=0, scale=None, lens=None,
                     name="", scales="pow2") -> DecodeFp8:
    """Symmetric INT8 caches: codes round(N(0,1) * 32) clamped to +-127 (int8), scales 2^U{-10..-6}
    per (b, KV head) (dequantised values about N(0,1) * 2^-5 .. 2^-1, the FP8 cache's range;
    scales="uniform": 2^-5 * U[0.01, 2) instead, from their own generator), new
    tokens N(0,1) * 32 * their head's scale in bf16 (so they quantise into the bulk of the code
    range), Q N(0,1) bf16.  Draw order as make_decode_fp8.  Returned in a DecodeFp8 record (the
    caches hold int8 codes)."""
    g = _gen(seed)
    if lens is None:
        lens = torch.randint(len_lo, len_hi + 1, (B,), generator=g, dtype=torch.int64)
    lens = torch.as_tensor(lens, dtype=torch.int64)
    if T_max is None:
        T_max = round_up(len_hi + 1, 64)
    codes = lambda: torch.round(torch.randn(B, H_kv, T_max, D, generator=g) * 32).clamp(-127, 127).to(torch.int8)
    kc = codes().contiguous()
    vc = codes().contiguous()
    ks = torch.exp2(torch.randint(-10, -5, (B, H_kv), generator=g).float()).contiguous()
    vs = torch.exp2(torch.randint(-10, -5, (B, H_kv), generator=g).float()).contiguous()
    if scales == "uniform":
        ks, vs = _uniform_scales(seed, (2, B, H_kv)) * 2.0 ** -5
    kn = (torch.randn(B, H_kv, 1, D, generator=g) * 32 * ks[:, :, None, None]).to(torch.bfloat16).contiguous()
    vn = (torch.randn(B, H_kv, 1, D, generator=g) * 32 * vs[:, :, None, None]).to(torch.bfloat16).contiguous()
    q = torch.randn(B, H_q, 1, D, generator=g).to(torch.bfloat16).contiguous()
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return DecodeFp8(q, kc, vc, ks, vs, kn, vn, lens.to(torch.int32), float(scale), name)


def make_gqa_prefill(B, H_q, H_kv, Tq, Tk, D, dtype=torch.bfloat16, *, valid=None, amp=1.0, seed=0,
                     scale=None, name="") -> Prefill:
    """Q [B, H_q, Tq, D] and K/V [B, H_kv, Tk, D] (grouped-query layout), drawn Q, K, V."""
    g = _gen(seed)
    q = _randn(g, (B, H_q, Tq, D), amp, dtype)
    k = _randn(g, (B, H_kv, Tk, D), amp, dtype)
    v = _randn(g, (B, H_kv, Tk, D), amp, dtype)
    mask = mask_from_valid_lengths(valid, Tk) if valid is not None else None
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Prefill(q, k, v, mask, float(scale), name)


def make_prefill_fp8(B, H_q, H_kv, Tq, Tk, D, *, valid=None, amp=1.0, seed=0, scale=None,
                     name="", scales="pow2") -> PrefillFp8:
    """E4M3 prefill inputs whose dequantised values are about N(0, amp^2): each (b, head) of Q, K
    and V gets a scale amp * 2^-e with e ~ U{2..6}, and its codes are N(0,1) * 2^e cast to
    float8_e4m3fn (round to nearest even; |N * 2^e| stays far below 448).  Draw order: Q, K, V
    scale exponents, then Q, K, V.  scales="uniform": each scale also carries a factor
    U[0.01, 2) from its own generator (values about N(0, (amp u)^2))."""
    g = _gen(seed)
    eq = torch.randint(2, 7, (B, H_q), generator=g)
    ek = torch.randint(2, 7, (B, H_kv), generator=g)
    ev = torch.randint(2, 7, (B, H_kv), generator=g)

    def codes(shape, e):
        x = torch.randn(*shape, generator=g) * torch.exp2(e.float())[:, :, None, None]
        return x.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()

    q = codes((B, H_q, Tq, D), eq)
    k = codes((B, H_kv, Tk, D), ek)
    v = codes((B, H_kv, Tk, D), ev)
    sc = lambda e: (amp * torch.exp2(-e.float())).contiguous()
    qs, ks, vs = sc(eq), sc(ek), sc(ev)
    if scales == "uniform":
        uq = _uniform_scales(seed, (B, H_q))
        uk, uv = _uniform_scales(seed + 1, (2, B, H_kv))
        qs, ks, vs = (qs * uq).contiguous(), (ks * uk).contiguous(), (vs * uv).contiguous()
    mask = mask_from_valid_lengths(valid, Tk) if valid is not None else None
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return PrefillFp8(q, k, v, qs, ks, vs, mask, float(scale), name)


# ---- the five named workloads -------------------------------------------------

def fp32_masked_t512(seed=0) -> Prefill:
    """fp32, B1 H16 T512 D64, last 48 keys padded, scale 1/sqrt(64)."""
    return make_prefill(1, 16, 512, 512, 64, torch.float32, valid=[512 - 48], seed=seed,
                        name="fp32 masked self-attention B1 H16 T512 D64, 48 padded keys")


def patch_p1944(seed=0) -> Prefill:
    """bf16, B2 H16 P1944 D64, valid lengths 1,944 and 1,700."""
    return make_prefill(2, 16, 1944, 1944, 64, torch.bfloat16, valid=[1944, 1700], seed=seed,
                        name="bf16 patch self-attention B2 H16 P1944 D64, valid 1944/1700")


def patch_p11616(seed=0) -> Prefill:
    """bf16, B1 H16 P11616 D64, last 16 keys padded, inputs N(0,1)*0.5."""
    return make_prefill(1, 16, 11616, 11616, 64, torch.bfloat16, valid=[11616 - 16], amp=0.5,
                        seed=seed, name="bf16 patch self-attention B1 H16 P11616 D64, 16 padded keys")


def chunked_kv_2x8192(seed=0) -> Chunked:
    """bf16, Q T8192 H24 D128 against 2 KV chunks of 8,192 keys, no mask."""
    return make_chunked(1, 24, 8192, [8192, 8192], 128, torch.bfloat16, seed=seed,
                        name="bf16 chunked KV B1 H24 Tq8192 D128, 2x8192 keys + LSE merge")


def gqa_decode_b32(seed=0) -> Decode:
    """bf16 GQA decode: B32, H_q 32 / H_kv 8, D128, cached len ~ U{512..8192}."""
    return make_decode(32, 32, 8, 128, 512, 8192, torch.bfloat16, seed=seed,
                       name="bf16 GQA decode B32 Hq32 Hkv8 D128, len U[512,8192] + 1 appended")


def varlen_p1944_packed(seed=0) -> Varlen:
    """bf16 packed patch self-attention: H16 D64, two sequences of 1,944 and 1,700 patches
    (the P = 1,944 batch with its padding removed instead of masked)."""
    return make_varlen([1944, 1700], [1944, 1700], 16, 64, seed=seed,
                       name="bf16 packed varlen H16 D64, sequences 1944 + 1700")


def varlen_ring_hop_8192(seed=0) -> Varlen:
    """bf16 packed ring hop: one sequence, 8,192 queries against an 8,192-key chunk, H24 D128."""
    return make_varlen([8192], [8192], 24, 128, seed=seed,
                       name="bf16 packed varlen ring hop H24 D128, 8192 queries x 8192-key chunk")


def gqa_decode_b32_paged(page_size=16, seed=0) -> Paged:
    """The GQA decode workload (B32, H_q 32 / H_kv 8, D128, len U[512, 8192]) in a paged cache."""
    return to_paged(gqa_decode_b32(seed), page_size)



def gqa_causal_prefill_8192(seed=0) -> Prefill:
    """bf16 causal GQA prompt pass: B1, H_q 32 / H_kv 8, D128, an 8,192-token prompt."""
    return make_gqa_prefill(1, 32, 8, 8192, 8192, 128, seed=seed,
                            name="bf16 causal GQA prefill B1 Hq32 Hkv8 D128, 8192-token prompt")


def gqa_causal_prompts_packed(seed=0) -> Varlen:
    """bf16 packed causal GQA prompts: 4 x 1,024 + 2 x 2,048 + 2 x 4,096 tokens, H_q 32 / H_kv 8,
    D128 (queries and keys of each prompt are the same positions)."""
    lens = [1024, 4096, 1024, 2048, 1024, 4096, 2048, 1024]
    g = _gen(seed)
    cq = cu_from_lengths(lens)
    n = int(cq[-1])
    q = _randn(g, (n, 32, 128), 1.0, torch.bfloat16)
    k = _randn(g, (n, 8, 128), 1.0, torch.bfloat16)
    v = _randn(g, (n, 8, 128), 1.0, torch.bfloat16)
    return Varlen(q, k, v, cq, cq.clone(), max(lens), 1.0 / math.sqrt(128),
                  "bf16 packed causal GQA prompts Hq32 Hkv8 D128, 4x1024 + 2x2048 + 2x4096")


def gqa_decode_b32_fp8(seed=0) -> DecodeFp8:
    """The GQA decode workload (B32, H_q 32 / H_kv 8, D128, len U[512, 8192]) with an E4M3 cache."""
    return make_decode_fp8(32, 32, 8, 128, 512, 8192, seed=seed,
                           name="E4M3-cache GQA decode B32 Hq32 Hkv8 D128, len U[512,8192] + 1 appended")


def patch_p11616_fp8(seed=0) -> PrefillFp8:
    """The P = 11,616 patch self-attention shape (B1 H16 D64, last 16 keys padded, values about
    N(0,1)*0.5) with E4M3 inputs."""
    return make_prefill_fp8(1, 16, 16, 11616, 11616, 64, valid=[11616 - 16], amp=0.5, seed=seed,
                            name="E4M3 patch self-attention B1 H16 P11616 D64, 16 padded keys")


def gqa_causal_prefill_8192_fp8(seed=0) -> PrefillFp8:
    """The causal GQA prompt pass (B1, H_q 32 / H_kv 8, D128, 8,192 tokens) with E4M3 inputs."""
    return make_prefill_fp8(1, 32, 8, 8192, 8192, 128, seed=seed,
                            name="E4M3 causal GQA prefill B1 Hq32 Hkv8 D128, 8192-token prompt")


def gqa_decode_b32_int8(seed=0) -> DecodeFp8:
    """The GQA decode workload (B32, H_q 32 / H_kv 8, D128, len U[512, 8192]) with an INT8 cache."""
    return make_decode_int8(32, 32, 8, 128, 512, 8192, seed=seed,
                            name="INT8-cache GQA decode B32 Hq32 Hkv8 D128, len U[512,8192] + 1 appended")


def varlen_ring_hop_8192_fp8(seed=0) -> VarlenFp8:
    """The packed ring hop (one sequence, 8,192 queries against an 8,192-key chunk, H24 D128) with
    E4M3 inputs."""
    return make_varlen_fp8([8192], [8192], 24, 128, seed=seed,
                           name="E4M3 packed varlen ring hop H24 D128, 8192 queries x 8192-key chunk")

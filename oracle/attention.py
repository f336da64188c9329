"""CPU oracle for masked / LSE / merge / append / decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this package; only
the test suite, the smoke check and the benchmark's CPU-baseline leg may.  It
shares no code with the HIP path.

Everything here is the plain definition written out in float64 NumPy, with
the full masked score matrix materialised one (batch, head) at a time, i.e.
exactly the computation the MultiheadAttention inference fast path performs
(molayo1419.me, "MultiheadAttention의 고속 경로가 VRAM을 18GB나 소모했던
이야기", section "소스의 현실": a score matrix of shape [B, heads, T, T] from
a batched Q·Kᵀ, a masked softmax, then a batched product with V).  The
library reaches the same real-number result without that matrix; this file
is the slow, obviously-correct yardstick.

Inputs are NumPy arrays (any float dtype; they are upcast to float64, which
holds every bf16 and fp32 value exactly) or anything ``numpy.asarray`` takes.

Readings of points the pages leave open:
  * mask polarity: nonzero = padded = ignored, the key_padding_mask sense;
    the same page, section "출력은 달라졌는가", warns that SDPA's boolean mask
    means the opposite.
  * padding becomes an additive -inf on the scores of padded keys (section
    "CPU에서 양을 측정하기" of that page describes the SDPA path that way).
  * a query row whose keys are all padded has O = 0 and LSE = -inf (the pages
    only require results free of NaN).
  * LSE is the natural log-sum-exp of the scaled, masked scores; the merge
    rule out = sum_i exp(lse_i - lse) out_i (sglang PR 49078 analysis,
    section "1. aiter.py") needs exactly that quantity.
  * GQA maps query head h to KV head h // (H_q / H_kv).
  * append writes the new token at slot len_b of a preallocated cache and
    then increments len_b, which equals concatenation (nanoVLM KV-cache page,
    section "1. 어텐션 블록 업데이트").
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "scores", "masked_softmax", "attention", "attention_varlen", "merge_lse", "kv_append", "decode",
    "allowed_keys", "prefill", "prefill_varlen",
    "gather_pages", "kv_append_paged", "decode_paged",
    "attention_flops", "score_matrix_bytes", "kv_bytes_per_token", "decode_kv_bytes",
]

NEG_INF = -np.inf


def _f64(x):
    if hasattr(x, "detach"):          # a torch tensor (bf16 / fp32): exact upcast on the CPU
        x = x.detach().cpu().double().numpy()
    return np.asarray(x, dtype=np.float64)


def _mask_bool(mask, B, Tk):
    if mask is None:
        return np.zeros((B, Tk), dtype=bool)
    if hasattr(mask, "detach"):
        mask = mask.detach().cpu().numpy()
    m = np.asarray(mask) != 0
    assert m.shape == (B, Tk), (m.shape, (B, Tk))
    return m


def scores(q_bh, k_bh, scale):
    """S = scale · Q Kᵀ for one (batch, head): [Tq, D] x [Tk, D] -> [Tq, Tk]."""
    return scale * (q_bh @ k_bh.T)


def masked_softmax(S, padded):
    """Row softmax of S with padded keys given -inf, plus per-row max and sum.

    Returns (weights, m, l) with weights[i, j] = exp(S_ij - m_i) / l_i,
    m_i = max_j S_ij over unpadded keys, l_i = sum_j exp(S_ij - m_i).  Rows
    with no unpadded key get weights 0, m = -inf, l = 0.
    """
    S = np.where(padded[None, :], NEG_INF, S)
    if S.shape[1] == 0:                             # no keys at all: as if all were padded
        z = np.zeros(S.shape[0])
        return np.zeros_like(S), np.full(S.shape[0], NEG_INF), z
    m = S.max(axis=1)
    live = np.isfinite(m)
    E = np.zeros_like(S)
    E[live] = np.exp(S[live] - m[live, None])       # exp(-inf) = 0 exactly at padded keys
    l = E.sum(axis=1)
    W = np.zeros_like(S)
    W[live] = E[live] / l[live, None]
    return W, m, l


def attention(q, k, v, key_padding_mask=None, scale=None, rows=None):
    """Masked scaled-dot-product attention and its per-row LSE.

    q [B, H, Tq, D], k and v [B, H, Tk, D], key_padding_mask [B, Tk] (nonzero
    = padded) or None, scale defaults to 1/sqrt(D).  ``rows`` optionally
    restricts the computation to a subset of query indices (each row's
    softmax depends on that row alone, so this is the same definition
    evaluated on fewer rows).

    Returns O [B, H, R, D] and LSE [B, H, R] in float64 (R = Tq or len(rows)).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Tq, D = q.shape
    Tk = k.shape[2]
    assert k.shape == (B, H, Tk, D) and v.shape == (B, H, Tk, D)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    padded = _mask_bool(key_padding_mask, B, Tk)
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        q = q[:, :, rows]
    R = q.shape[2]
    O = np.zeros((B, H, R, D))
    LSE = np.full((B, H, R), NEG_INF)
    for b in range(B):
        for h in range(H):
            S = scores(q[b, h], k[b, h], scale)
            W, m, l = masked_softmax(S, padded[b])
            O[b, h] = W @ v[b, h]
            live = np.isfinite(m)
            LSE[b, h, live] = m[live] + np.log(l[live])
    return O, LSE


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale=None):
    """Attention of packed variable-length sequences (no mask, non-causal).

    The packed layout a ring-attention hop passes to its varlen kernel
    (sglang PR 49078 analysis, section "1. aiter.py", forward_ring_kv_chunk):
    q [total_q, H, D], k and v [total_k, H, D], and cumulative lengths
    cu_seqlens_q / cu_seqlens_k of B + 1 entries from 0 to the totals.
    Sequence b is query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1 against
    key rows cu_seqlens_k[b] .. cu_seqlens_k[b+1] - 1; nothing else is
    attended, so each sequence is exactly ``attention`` on its own slice.

    Returns O [total_q, H, D] and LSE [H, total_q] (the page's LSE layout) in
    float64; a sequence with no keys has O = 0 and LSE = -inf.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    cq = np.asarray(_f64(cu_seqlens_q), dtype=np.int64)
    ck = np.asarray(_f64(cu_seqlens_k), dtype=np.int64)
    total_q, H, D = q.shape
    assert k.shape[1:] == (H, D) and v.shape == k.shape
    assert cq.shape == ck.shape and cq.ndim == 1 and cq.size >= 1
    assert cq[0] == 0 and ck[0] == 0 and cq[-1] == total_q and ck[-1] == k.shape[0]
    assert np.all(np.diff(cq) >= 0) and np.all(np.diff(ck) >= 0)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    O = np.zeros((total_q, H, D))
    LSE = np.full((H, total_q), NEG_INF)
    for b in range(cq.size - 1):
        q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        if q1 == q0:
            continue
        if k1 == k0:                    # no keys: the all-padded case
            continue
        # [T, H, D] -> [1, H, T, D]
        qs = q[q0:q1].transpose(1, 0, 2)[None]
        ks = k[k0:k1].transpose(1, 0, 2)[None]
        vs = v[k0:k1].transpose(1, 0, 2)[None]
        Ob, Lb = attention(qs, ks, vs, None, scale)
        O[q0:q1] = Ob[0].transpose(1, 0, 2)
        LSE[:, q0:q1] = Lb[0]
    return O, LSE


# ---- GQA and causal prefill ----------------------------------------------------------
# The prompt pass of a grouped-query-attention language model (nanoVLM-KV page, sections
# "1. 어텐션 블록 업데이트" (LanguageModelGroupedAttention) and "3. 생성 루프 분리" (the
# prefill phase encodes the whole prompt and fills the cache)): query head h reads KV head
# h // (H_q / H_kv), and an autoregressive model's position i sees positions <= i only.
# With Tk >= Tq the Tq queries are the LAST Tq positions of the Tk keys (a prompt chunk
# after a cached prefix), so query i sees keys j <= i + (Tk - Tq); with Tq = Tk that is
# j <= i, and a single query (Tq = 1) sees every key, which is the decode step.

def allowed_keys(Tq, Tk, causal, padded=None):
    """Boolean [Tq, Tk]: True where query i may attend key j (unpadded and, if causal,
    j <= i + Tk - Tq)."""
    ok = np.ones((Tq, Tk), dtype=bool)
    if causal:
        i = np.arange(Tq)[:, None]
        j = np.arange(Tk)[None, :]
        ok &= j <= i + (Tk - Tq)
    if padded is not None:
        ok &= ~np.asarray(padded, dtype=bool)[None, :]
    return ok


def _softmax_allowed(S, ok):
    """Row softmax of S over the allowed entries: (W, m, l) as masked_softmax, a row
    with no allowed entry giving W = 0, m = -inf, l = 0."""
    S = np.where(ok, S, NEG_INF)
    if S.shape[1] == 0:
        return np.zeros_like(S), np.full(S.shape[0], NEG_INF), np.zeros(S.shape[0])
    m = S.max(axis=1)
    live = np.isfinite(m)
    E = np.zeros_like(S)
    E[live] = np.exp(S[live] - m[live, None])
    l = E.sum(axis=1)
    W = np.zeros_like(S)
    W[live] = E[live] / l[live, None]
    return W, m, l


def prefill(q, k, v, key_padding_mask=None, causal=False, scale=None, rows=None):
    """GQA (optionally causal, optionally key-padded) attention and its LSE.

    q [B, H_q, Tq, D], k and v [B, H_kv, Tk, D] with H_q a multiple of H_kv; query head
    h uses KV head h // (H_q / H_kv).  ``rows`` restricts to a subset of query indices
    (the causal limit still uses each row's own index).  Returns O [B, H_q, R, D] and
    LSE [B, H_q, R] in float64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Tq, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    assert k.shape == (B, Hkv, Tk, D) and v.shape == k.shape and Hq % Hkv == 0
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    padded = _mask_bool(key_padding_mask, B, Tk)
    ridx = np.arange(Tq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = ridx.size
    O = np.zeros((B, Hq, R, D))
    LSE = np.full((B, Hq, R), NEG_INF)
    for b in range(B):
        ok = allowed_keys(Tq, Tk, causal, padded[b])[ridx]
        for h in range(Hq):
            S = scores(q[b, h, ridx], k[b, h // G], scale)
            W, m, l = _softmax_allowed(S, ok)
            O[b, h] = W @ v[b, h // G]
            live = np.isfinite(m)
            LSE[b, h, live] = m[live] + np.log(l[live])
    return O, LSE


def prefill_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, causal=False, scale=None):
    """``prefill`` on packed sequences: q [total_q, H_q, D], k and v [total_k, H_kv, D],
    sequences as in ``attention_varlen`` (the causal limit uses each sequence's own
    lengths).  Returns O [total_q, H_q, D] and LSE [H_q, total_q]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    cq = np.asarray(_f64(cu_seqlens_q), dtype=np.int64)
    ck = np.asarray(_f64(cu_seqlens_k), dtype=np.int64)
    total_q, Hq, D = q.shape
    Hkv = k.shape[1]
    assert k.shape[2] == D and v.shape == k.shape and Hq % Hkv == 0
    assert cq[0] == 0 and ck[0] == 0 and cq[-1] == total_q and ck[-1] == k.shape[0]
    O = np.zeros((total_q, Hq, D))
    LSE = np.full((Hq, total_q), NEG_INF)
    for b in range(cq.size - 1):
        q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        if q1 == q0:
            continue
        Ob, Lb = prefill(q[q0:q1].transpose(1, 0, 2)[None], k[k0:k1].transpose(1, 0, 2)[None],
                         v[k0:k1].transpose(1, 0, 2)[None], None, causal, scale)
        O[q0:q1] = Ob[0].transpose(1, 0, 2)
        LSE[:, q0:q1] = Lb[0]
    return O, LSE


def merge_lse(outs, lses):
    """Combine attention results over disjoint key chunks.

    outs: list of n arrays [..., D]; lses: list of n arrays [...].  With
    M = max_i lse_i, lse = M + log sum_i exp(lse_i - M) and
    out = sum_i exp(lse_i - lse) · out_i; where every lse_i is -inf the
    result is (0, -inf).
    """
    outs = [_f64(o) for o in outs]
    lses = [_f64(s) for s in lses]
    L = np.stack(lses)                      # [n, ...]
    M = L.max(axis=0)
    live = np.isfinite(M)
    Msafe = np.where(live, M, 0.0)
    w = np.exp(L - Msafe[None])             # exp(-inf) = 0 for empty chunks
    tot = w.sum(axis=0)
    lse = np.where(live, Msafe + np.log(np.where(live, tot, 1.0)), NEG_INF)
    out = np.zeros_like(outs[0])
    for i in range(len(outs)):
        coef = np.where(live, np.exp(L[i] - np.where(live, lse, 0.0)), 0.0)
        out += coef[..., None] * outs[i]
    return out, lse


def kv_append(k_cache, v_cache, lens, k_new, v_new):
    """Write one token per sequence at slot lens[b]; return (k, v, lens + 1).

    k_cache/v_cache [B, H_kv, T_max, D], k_new/v_new [B, H_kv, 1, D],
    lens int [B].  Inputs are not modified; copies are returned with the
    original dtype kept (the append is a bit copy).
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    lens = np.asarray(lens).astype(np.int64)
    T_max = kc.shape[2]
    for b in range(kc.shape[0]):
        t = int(lens[b])
        assert 0 <= t < T_max, "cache full"
        kc[b, :, t, :] = np.asarray(k_new)[b, :, 0, :]
        vc[b, :, t, :] = np.asarray(v_new)[b, :, 0, :]
    return kc, vc, lens + 1


def decode(q, k_cache, v_cache, lens, scale=None, heads=None):
    """One query token per sequence attending over the first lens[b] cache slots.

    q [B, H_q, 1, D]; caches [B, H_kv, T_max, D]; lens int [B] (the length
    after the append, so the new token is included).  Query head h reads KV
    head h // (H_q / H_kv).  No mask beyond the length.  ``heads`` optionally
    restricts to a list of (b, h) pairs, returned in that order as arrays
    O [n, D] and LSE [n]; otherwise O [B, H_q, 1, D] and LSE [B, H_q].
    """
    q = _f64(q)
    B, Hq, one, D = q.shape
    assert one == 1
    Hkv = k_cache.shape[1]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    lens = np.asarray(lens).astype(np.int64)

    def one_head(b, h):
        n = int(lens[b])
        kk = _f64(k_cache[b, h // G, :n])
        vv = _f64(v_cache[b, h // G, :n])
        S = scores(q[b, h], kk, scale)                  # [1, n]
        W, m, l = masked_softmax(S, np.zeros(n, dtype=bool))
        o = (W @ vv)[0]
        lse = m[0] + np.log(l[0]) if np.isfinite(m[0]) else NEG_INF
        return o, lse

    if heads is not None:
        res = [one_head(b, h) for (b, h) in heads]
        return np.stack([r[0] for r in res]), np.array([r[1] for r in res])
    O = np.zeros((B, Hq, 1, D))
    LSE = np.full((B, Hq), NEG_INF)
    for b in range(B):
        for h in range(Hq):
            O[b, h, 0], LSE[b, h] = one_head(b, h)
    return O, LSE


# ---- paged KV cache ---------------------------------------------------------------
# Paged layout (LLM inference memory accounting 2/10, section "15. Paged KV Cache가
# 해결하는 것"): a sequence's logical KV blocks 0, 1, 2, ... live in physical blocks
# block_table[b][0], block_table[b][1], ... of a shared pool, so token t of sequence b
# is row t % page_size of physical block block_table[b][t // page_size].  The pool is
# [num_pages, H_kv, page_size, D]: one physical block holds page_size tokens of every
# KV head, each head's rows contiguous, like a slice of the contiguous cache.

def gather_pages(pages, block_table, b, n):
    """Tokens 0..n-1 of sequence b from the pool, in logical order: [H_kv, n, D]."""
    pages = _f64(pages)
    bt = np.asarray(_f64(block_table), dtype=np.int64)
    ps = pages.shape[2]
    rows = [pages[bt[b, t // ps], :, t % ps, :] for t in range(n)]
    if not rows:
        return np.zeros((pages.shape[1], 0, pages.shape[3]))
    return np.stack(rows, axis=1)


def kv_append_paged(k_pages, v_pages, block_table, lens, k_new, v_new):
    """Write one token per sequence at logical position lens[b], i.e. row
    lens[b] % page_size of physical block block_table[b][lens[b] // page_size];
    return (k_pages, v_pages, lens + 1) as copies (bit copy, dtype kept)."""
    kp = np.array(k_pages, copy=True)
    vp = np.array(v_pages, copy=True)
    bt = np.asarray(block_table).astype(np.int64)
    lens = np.asarray(lens).astype(np.int64)
    ps = kp.shape[2]
    for b in range(bt.shape[0]):
        t = int(lens[b])
        assert 0 <= t < bt.shape[1] * ps, "cache full"
        p = int(bt[b, t // ps])
        kp[p, :, t % ps, :] = np.asarray(k_new)[b, :, 0, :]
        vp[p, :, t % ps, :] = np.asarray(v_new)[b, :, 0, :]
    return kp, vp, lens + 1


def decode_paged(q, k_pages, v_pages, block_table, lens, scale=None, heads=None):
    """``decode`` over a paged cache: each sequence's first lens[b] tokens are
    gathered from the pool through its block-table row, then attended exactly
    as in the contiguous cache.  Arguments and results as ``decode``."""
    q = _f64(q)
    B = q.shape[0]
    kp, vp = _f64(k_pages), _f64(v_pages)
    lens = np.asarray(lens).astype(np.int64)
    H_kv, D = kp.shape[1], kp.shape[3]
    T = max(1, int(lens.max()) if lens.size else 1)
    kc = np.zeros((B, H_kv, T, D))
    vc = np.zeros((B, H_kv, T, D))
    for b in range(B):
        n = int(lens[b])
        kc[b, :, :n] = gather_pages(kp, block_table, b, n)
        vc[b, :, :n] = gather_pages(vp, block_table, b, n)
    return decode(q, kc, vc, lens, scale, heads)


# ---- work and byte accounting --------------------------------------------------

def attention_flops(H, D, Tq, n_valid_per_batch):
    """Algorithmic FLOPs of masked attention: Q·Kᵀ and P·V each cost 2·D per
    (query, unpadded key) pair, so 4·D·H·Tq·sum_b n_valid_b."""
    return 4 * D * H * Tq * int(np.sum(n_valid_per_batch))


def score_matrix_bytes(heads, P, elem_bytes):
    """Bytes of one heads × P × P score matrix, the buffer the fast path builds
    (molayo1419.me page, section "무엇이 일어나고 있었는가": 16 heads at 3 MP in
    bf16 is about 4.32 GB)."""
    return heads * P * P * elem_bytes


def kv_bytes_per_token(layers, H_kv, D, elem_bytes):
    """KV bytes per token: layers × 2 (K and V) × KV heads × head_dim × bytes
    (LLM inference memory accounting 2/10, section "10. KV Cache Byte 공식")."""
    return layers * 2 * H_kv * D * elem_bytes


def decode_kv_bytes(lens, H_kv, D, elem_bytes):
    """K and V bytes one decode step must read for one layer: bytes per token
    times the total active tokens (same page, section "13. KV는 Token마다 자란다")."""
    return kv_bytes_per_token(1, H_kv, D, elem_bytes) * int(np.sum(np.asarray(lens, dtype=np.int64)))

"""GPU parity: every entry point through the C ABI against the CPU oracle.

Tolerances (max-abs over every element, fp64 comparison, NaN fails):
  fp32 inputs: O and LSE <= 1e-4
  bf16 inputs (fp32 accumulation): O <= 2e-2, LSE <= 1e-3
An oracle -inf LSE must be exactly -inf on the GPU with an O row of exactly 0.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL = {torch.float32: (1e-4, 1e-4), torch.bfloat16: (2e-2, 1e-3)}
DEV = "cuda"


def _np(t):
    return t.detach().float().cpu().double().numpy()


def check_attn(O, L, Oref, Lref, dtype, what="", o_tol=None):
    """Max-abs comparison of O and LSE with the oracle; o_tol overrides the O bar (LSE keeps
    its bar)."""
    to, tl = TOL[dtype]
    if o_tol is not None:
        to = o_tol
    O = _np(O)
    assert not np.isnan(O).any(), f"{what}: NaN in O"
    dead = np.isneginf(Lref)
    if L is not None:
        L = L.detach().cpu().double().numpy()
        assert not np.isnan(L).any(), f"{what}: NaN in LSE"
        assert np.array_equal(np.isneginf(L), dead), f"{what}: -inf LSE pattern differs"
        if (~dead).any():
            el = np.max(np.abs(L[~dead] - Lref[~dead]))
            assert el <= tl, f"{what}: max|dLSE| = {el:.3e} > {tl}"
    if dead.any():
        assert np.all(O[dead] == 0.0), f"{what}: rows with no unpadded key must be exactly 0"
    eo = np.max(np.abs(O - Oref)) if O.size else 0.0
    assert eo <= to, f"{what}: max|dO| = {eo:.3e} > {to}"
    return eo


def run_fwd(ma, w, lse=True):
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    m = w.mask.to(DEV) if w.mask is not None else None
    if lse:
        o, l = ma.attn_fwd_lse(q, k, v, m, w.scale)
    else:
        o, l = ma.attn_fwd_masked(q, k, v, m, w.scale), None
    torch.cuda.synchronize()
    return o, l


# ---- prefill, element by element ------------------------------------------------------

SHAPES = [
    # B, H, Tq, Tk, D, mask kind
    (1, 1, 1, 1, 64, None),
    (1, 2, 17, 5, 64, "suffix"),
    (2, 2, 64, 64, 64, "random"),
    (1, 3, 255, 257, 64, "suffix"),
    (2, 2, 256, 300, 64, "random"),
    (1, 2, 513, 129, 64, "none"),
    (2, 1, 300, 1000, 64, "holes"),
    (2, 2, 200, 700, 64, "prefix"),
    (2, 1, 150, 500, 64, "window"),
    (3, 1, 64, 300, 64, "single"),
    (1, 2, 90, 333, 128, "window"),
    (1, 2, 100, 77, 128, "suffix"),
    (2, 2, 130, 300, 128, "random"),
    (1, 1, 257, 33, 128, "none"),
    (3, 2, 100, 256, 64, "aligned"),
    (3, 1, 70, 256, 128, "aligned"),
]


def _mask(kind, B, Tk, seed):
    g = torch.Generator().manual_seed(seed)
    if kind in (None, "none"):
        return None
    if kind == "suffix":
        valid = torch.randint(1, Tk + 1, (B,), generator=g)
        return W.mask_from_valid_lengths(valid.tolist(), Tk)
    if kind == "random":
        m = (torch.rand(B, Tk, generator=g) < 0.3).to(torch.uint8)
        m[:, 0] = 0
        return m
    if kind in ("prefix", "window", "single"):
        # one contiguous run of valid keys [a, b]: leading (and trailing) padding only
        m = torch.ones(B, Tk, dtype=torch.uint8)
        for bi in range(B):
            a = int(torch.randint(1, Tk // 2, (1,), generator=g))
            if kind == "prefix":
                b = Tk - 1
            elif kind == "single":
                b = a
            else:
                b = int(torch.randint(a, Tk, (1,), generator=g))
            m[bi, a:b + 1] = 0
        return m
    if kind == "aligned":
        # valid runs that start and end on 32-key block edges ([32, 95], [64, 255]) and one
        # too short to hold a whole block ([3, 30]): the edges of the interior-block test
        m = torch.ones(B, Tk, dtype=torch.uint8)
        for bi, (a, b) in enumerate([(32, 95), (64, Tk - 1), (3, 30)][:B]):
            m[bi, a:b + 1] = 0
        return m
    if kind == "holes":   # whole 64-key tiles padded in the middle plus a ragged tail
        m = torch.zeros(B, Tk, dtype=torch.uint8)
        m[:, 64:192] = 1
        m[:, 500:533] = 1
        m[-1, Tk - 7:] = 1
        return m
    raise ValueError(kind)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", SHAPES)
def test_fwd_shapes(ma, shape, dtype):
    B, H, Tq, Tk, D, kind = shape
    w = W.make_prefill(B, H, Tq, Tk, D, dtype, mask=_mask(kind, B, Tk, Tq + Tk), seed=Tq * 7 + Tk)
    o, l = run_fwd(ma, w)
    Or, Lr = oracle.attention(w.q, w.k, w.v, w.mask, w.scale)
    check_attn(o, l, Or, Lr, dtype, f"{shape} {dtype}")
    o2, _ = run_fwd(ma, w, lse=False)
    assert torch.equal(o, o2), "attn_fwd_masked must equal attn_fwd_lse's O"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_fwd_fully_padded_sequence(ma, dtype):
    m = torch.zeros(3, 200, dtype=torch.uint8)
    m[1] = 1
    m[2, 5:] = 1
    w = W.make_prefill(3, 2, 70, 200, 64, dtype, mask=m, seed=3)
    o, l = run_fwd(ma, w)
    Or, Lr = oracle.attention(w.q, w.k, w.v, w.mask, w.scale)
    check_attn(o, l, Or, Lr, dtype, "fully padded sequence")
    assert torch.all(o[1] == 0) and torch.all(torch.isneginf(l[1]))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("holes", [False, True])
def test_fwd_visited_tile_counts(ma, D, holes):
    """The bf16 kernels keep K and V tiles of 64 keys in LDS rings filled several tiles ahead;
    the prologue and every tile end issue loads for tiles past the last visited one.  Visited
    ranges of 1 to 7 tiles, starting at tile 0, 1 or 2 and ending on, just past or inside a
    tile edge, with and without padded keys between the first and last unpadded ones."""
    g = torch.Generator().manual_seed(D + holes)
    for t0 in (0, 1, 2):
        for n in range(1, 8):
            for tail in (0, 1, 37):
                first = 64 * t0 + (5 if t0 else 0)
                last = max(first, 64 * (t0 + n - 1) + (63 if tail == 0 else tail - 1))
                Tk = last + 1 + int(torch.randint(0, 3, (1,), generator=g))
                m = torch.ones(1, Tk, dtype=torch.uint8)
                m[0, first:last + 1] = 0
                if holes and last - first > 4:
                    m[0, first + 1:last:3] = 1
                w = W.make_prefill(1, 2, 40, Tk, D, torch.bfloat16, mask=m, seed=1000 * t0 + 10 * n + tail)
                o, l = run_fwd(ma, w)
                Or, Lr = oracle.attention(w.q, w.k, w.v, w.mask, w.scale)
                check_attn(o, l, Or, Lr, torch.bfloat16, f"D={D} keys [{first}, {last}] of {Tk} holes={holes}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("amp", [4.0, 8.0])
def test_fwd_peaky_scores(ma, amp, D):
    """Large scores (Q, K, V ~ N(0, amp^2)): the reference rises often, exercising the lazy
    rescale.  LSE keeps its 1e-3 bar.  O is a convex combination of V rows, so its bf16
    roundings (of the weights before P·V and of the stored O) are relative to |V|: the O bar is
    the 2e-2 stated for N(0,1) values, in units of |V| = amp."""
    w = W.make_prefill(1, 2, 300, 700, D, torch.bfloat16, valid=[650], amp=amp, seed=int(amp) + D)
    o, l = run_fwd(ma, w)
    Or, Lr = oracle.attention(w.q, w.k, w.v, w.mask, w.scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, f"peaky amp={amp} D={D}", o_tol=2e-2 * amp)


def test_fp32_masked_t512(ma):
    w = W.fp32_masked_t512()
    o, l = run_fwd(ma, w)
    Or, Lr = oracle.attention(w.q, w.k, w.v, w.mask, w.scale)
    check_attn(o, l, Or, Lr, torch.float32, "fp32 T512")


@pytest.mark.parametrize("D", [64, 128])
def test_fp32_key_split_merge(ma, D):
    """The fp32 kernel splits a query block's keys over four wavefronts (key blocks w, w+4, ...)
    and merges their states: key ranges where some wavefronts see only padded blocks or no block
    at all, where the largest scores sit in one wavefront's blocks, and long ranges with several
    blocks per wavefront."""
    g = torch.Generator().manual_seed(D)
    cases = []
    for Tk in (31, 33, 97, 130, 1000):
        m = torch.zeros(3, Tk, dtype=torch.uint8)
        m[1, : Tk // 2] = 1                      # leading half padded
        if Tk > 64:
            m[2, 32:64] = 1                      # wavefront 1's first block wholly padded
            m[2, 96:] = 1                        # and everything past the third block
        cases.append(W.make_prefill(3, 2, 45, Tk, D, torch.float32, mask=m, seed=Tk + D))
    w = W.make_prefill(1, 2, 70, 900, D, torch.float32, seed=7 + D)
    w.k[0, :, 700:710] *= 8.0                    # peaky scores inside one wavefront's blocks
    cases.append(w)
    for w in cases:
        o, l = run_fwd(ma, w)
        Or, Lr = oracle.attention(w.q, w.k, w.v, w.mask, w.scale)
        check_attn(o, l, Or, Lr, torch.float32, f"fp32 D={D} Tk={w.k.shape[2]}")


def test_patch_p1944(ma):
    w = W.patch_p1944()
    o, l = run_fwd(ma, w)
    Or, Lr = oracle.attention(w.q, w.k, w.v, w.mask, w.scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, "bf16 P1944")


def tile_rows(T, tile=256, seed=0):
    """Rows that visit every q-tile of a T-row launch: one seeded row inside each tile of
    `tile` rows, plus the first and last row of every tile and the last row overall."""
    g = np.random.default_rng(seed)
    rows = set()
    for t0 in range(0, T, tile):
        t1 = min(T, t0 + tile)
        rows.update((t0, t1 - 1, int(g.integers(t0, t1))))
    return np.array(sorted(rows))


# ---- merge ---------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 32])
def test_merge_random_partials(ma, n, dtype):
    g = torch.Generator().manual_seed(n)
    B, H, T, D = 2, 3, 37, 128 if n % 2 else 64
    outs = [torch.randn(B, H, T, D, generator=g).to(dtype) for _ in range(n)]
    lses = [torch.randn(B, H, T, generator=g) * 3 for _ in range(n)]
    lses[0][0, 0, 3] = -math.inf
    for i in range(n):
        lses[i][1, 2, 5] = -math.inf     # a row empty in every chunk
    o, l = ma.attn_merge_lse([t.to(DEV) for t in outs], [t.to(DEV) for t in lses])
    torch.cuda.synchronize()
    Or, Lr = oracle.merge_lse(outs, lses)
    check_attn(o, l, Or, Lr, dtype, f"merge n={n}")


def test_chunked_kv_2x8192_merge_equals_single_pass(ma):
    """Two 8,192-key chunks via attn_fwd_lse + attn_merge_lse equal one call over 16,384 keys
    (an invariant of the GPU path; every row of both against the oracle is in test_fullsize)."""
    w = W.chunked_kv_2x8192()
    q = w.q.to(DEV)
    parts = [ma.attn_fwd_lse(q, kc.to(DEV), vc.to(DEV), None, w.scale) for kc, vc in zip(w.k_chunks, w.v_chunks)]
    om, lm = ma.attn_merge_lse([p[0] for p in parts], [p[1] for p in parts])
    k = torch.cat(w.k_chunks, dim=2).to(DEV)
    v = torch.cat(w.v_chunks, dim=2).to(DEV)
    of, lf = ma.attn_fwd_lse(q, k, v, None, w.scale)
    torch.cuda.synchronize()
    # merged vs single pass on the GPU (both bf16 outputs: two roundings apart)
    assert (om.float() - of.float()).abs().max().item() <= 2e-2
    assert (lm - lf).abs().max().item() <= 1e-3


# ---- append + decode -------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_kv_append_bit_exact(ma, dtype):
    w = W.make_decode(5, 4, 2, 64, 0, 30, dtype, T_max=32, seed=9,
                      lens=[0, 7, 31, 32, 40])          # 32 and 40: full / over capacity
    kc, vc = w.k_cache.to(DEV), w.v_cache.to(DEV)
    lens = w.lens.to(DEV)
    ma.kv_append(kc, vc, lens, w.k_new.to(DEV), w.v_new.to(DEV))
    torch.cuda.synchronize()
    ok = [0, 1, 2]
    ek, ev, el = oracle.kv_append(w.k_cache[ok].float().numpy(), w.v_cache[ok].float().numpy(),
                                  w.lens[ok].numpy(), w.k_new[ok].float().numpy(), w.v_new[ok].float().numpy())
    assert torch.equal(kc[ok].cpu(), torch.from_numpy(ek).to(dtype))
    assert torch.equal(vc[ok].cpu(), torch.from_numpy(ev).to(dtype))
    assert lens.cpu().tolist() == el.tolist() + [32, 40]
    # sequences at or past capacity are untouched
    assert torch.equal(kc[3:].cpu(), w.k_cache[3:]) and torch.equal(vc[3:].cpu(), w.v_cache[3:])


DEC_SHAPES = [
    # B, Hq, Hkv, D, len_lo, len_hi, T_max
    (3, 4, 4, 64, 1, 40, 64),
    (4, 8, 2, 128, 1, 1500, 1536),
    (2, 32, 8, 128, 500, 1100, 1152),
    (3, 6, 2, 64, 0, 600, 640),
    (2, 16, 2, 128, 1, 700, 768),
    (2, 3, 1, 128, 510, 514, 576),
    (2, 40, 1, 64, 100, 900, 960),       # 40 query heads per KV head: two column groups
    (70, 8, 4, 64, 1, 300, 320),         # more than 64 sequences; short items shared by two waves
    (4, 8, 8, 128, 1023, 1023, 1024),    # lengths after the append are whole splits
    (16, 64, 8, 128, 0, 3000, 3072),
    (1, 1, 1, 128, 0, 0, 64),            # a single token
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", DEC_SHAPES)
def test_append_then_decode(ma, shape, dtype):
    B, Hq, Hkv, D, lo, hi, Tm = shape
    w = W.make_decode(B, Hq, Hkv, D, lo, hi, dtype, T_max=Tm, seed=B * 100 + Hq)
    kc, vc, lens = w.k_cache.to(DEV), w.v_cache.to(DEV), w.lens.to(DEV)
    ma.kv_append(kc, vc, lens, w.k_new.to(DEV), w.v_new.to(DEV))
    o, l = ma.attn_decode(w.q.to(DEV), kc, vc, lens, w.scale, want_lse=True)
    torch.cuda.synchronize()
    ek, ev, el = oracle.kv_append(w.k_cache.float().numpy(), w.v_cache.float().numpy(), w.lens.numpy(),
                                  w.k_new.float().numpy(), w.v_new.float().numpy())
    Or, Lr = oracle.decode(w.q, ek, ev, el, w.scale)
    check_attn(o, l, Or, Lr, dtype, f"decode {shape}")


def test_decode_zero_length(ma):
    w = W.make_decode(2, 4, 2, 128, 0, 10, torch.bfloat16, T_max=64, lens=[0, 9], seed=1)
    o, l = ma.attn_decode(w.q.to(DEV), w.k_cache.to(DEV), w.v_cache.to(DEV), w.lens.to(DEV), w.scale,
                          want_lse=True)
    torch.cuda.synchronize()
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(l[0]))
    Or, Lr = oracle.decode(w.q[1:], w.k_cache[1:], w.v_cache[1:], w.lens[1:], w.scale)
    check_attn(o[1:], l[1:], Or, Lr, torch.bfloat16, "decode len 0 / 9")


def test_decode_zero_lengths_mixed(ma):
    """Empty sequences between non-empty ones (the work order skips them)."""
    w = W.make_decode(6, 8, 2, 128, 0, 10, torch.bfloat16, T_max=768, lens=[0, 5, 0, 700, 0, 513], seed=2)
    o, l = ma.attn_decode(w.q.to(DEV), w.k_cache.to(DEV), w.v_cache.to(DEV), w.lens.to(DEV), w.scale,
                          want_lse=True)
    torch.cuda.synchronize()
    for b in (0, 2, 4):
        assert torch.all(o[b] == 0) and torch.all(torch.isneginf(l[b]))
    keep = [1, 3, 5]
    Or, Lr = oracle.decode(w.q[keep], w.k_cache[keep], w.v_cache[keep], w.lens[keep], w.scale)
    check_attn(o[keep], l[keep], Or, Lr, torch.bfloat16, "decode mixed zero lengths")


# ---- packed variable-length sequences (cu_seqlens) -------------------------------------

VARLEN = [
    # lens_q, lens_k, H, D
    ([1], [1], 1, 64),
    ([300], [257], 2, 64),
    ([5, 0, 300, 64], [70, 33, 0, 129], 2, 64),
    ([256, 257, 1], [64, 65, 640], 3, 64),
    ([700, 100, 256], [700, 100, 513], 2, 64),
    ([77], [1000], 1, 128),
    ([130, 0, 31, 257], [300, 5, 64, 0], 2, 128),
    ([513, 200], [200, 513], 2, 128),
]


def run_varlen(ma, w, lse=True):
    q, k, v, cq, ck = (t.to(DEV) for t in (w.q, w.k, w.v, w.cu_q, w.cu_k))
    res = ma.attn_fwd_varlen(q, k, v, cq, ck, w.max_q, w.scale, want_lse=lse)
    torch.cuda.synchronize()
    return res if lse else (res, None)


@pytest.mark.parametrize("case", VARLEN)
def test_fwd_varlen(ma, case):
    lq, lk, H, D = case
    w = W.make_varlen(lq, lk, H, D, seed=len(lq) + H)
    o, l = run_varlen(ma, w)
    Oref, Lref = oracle.attention_varlen(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale)
    check_attn(o, l.t(), Oref, Lref.T, torch.bfloat16, f"varlen {case}")


@pytest.mark.parametrize("D", [64, 128])
def test_fwd_varlen_without_lse_matches_with(ma, D):
    w = W.make_varlen([200, 3, 333], [90, 400, 0], 2, D, seed=D)
    o1, _ = run_varlen(ma, w, lse=False)
    o2, _ = run_varlen(ma, w, lse=True)
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("D", [64, 128])
def test_fwd_varlen_bitwise_equals_padded_masked(ma, D):
    # The same sequences laid out [B, H, T, D] with trailing key padding go through the masked
    # entry point; each valid query row must match the packed result bit for bit.
    lq, lk = [300, 45, 129], [257, 511, 64]
    w = W.make_varlen(lq, lk, 2, D, seed=11)
    o, l = run_varlen(ma, w)
    B, H, Tq, Tk = 3, 2, max(lq), max(lk)
    cq, ck = w.cu_q.tolist(), w.cu_k.tolist()
    qd = torch.zeros(B, H, Tq, D, dtype=torch.bfloat16)
    kd = torch.zeros(B, H, Tk, D, dtype=torch.bfloat16)
    vd = torch.zeros(B, H, Tk, D, dtype=torch.bfloat16)
    for b in range(B):
        qd[b, :, :lq[b]] = w.q[cq[b]:cq[b + 1]].transpose(0, 1)
        kd[b, :, :lk[b]] = w.k[ck[b]:ck[b + 1]].transpose(0, 1)
        vd[b, :, :lk[b]] = w.v[ck[b]:ck[b + 1]].transpose(0, 1)
    m = W.mask_from_valid_lengths(lk, Tk)
    od, ld = ma.attn_fwd_lse(qd.to(DEV), kd.to(DEV), vd.to(DEV), m.to(DEV), w.scale)
    torch.cuda.synchronize()
    o, l, od, ld = o.cpu(), l.cpu(), od.cpu(), ld.cpu()
    for b in range(B):
        assert torch.equal(o[cq[b]:cq[b + 1]], od[b, :, :lq[b]].transpose(0, 1)), b
        assert torch.equal(l[:, cq[b]:cq[b + 1]], ld[b, :, :lq[b]]), b


def test_fwd_varlen_rows_past_max_seqlen_untouched(ma):
    # Rows of a sequence longer than max_seqlen_q are not written (the grid covers max_seqlen_q).
    w = W.make_varlen([40, 300], [50, 60], 2, 64, seed=2)
    q, k, v, cq, ck = (t.to(DEV) for t in (w.q, w.k, w.v, w.cu_q, w.cu_k))
    out = torch.full_like(q, 7.0)
    lse = torch.full((2, 340), 7.0, device=DEV)
    ma.attn_fwd_varlen(q, k, v, cq, ck, 256, w.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention_varlen(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale)
    rows = list(range(0, 40 + 256))
    check_attn(out[rows], lse[:, rows].t(), Oref[rows], Lref[:, rows].T, torch.bfloat16, "varlen truncated")
    assert torch.all(out[40 + 256:] == 7.0) and torch.all(lse[:, 40 + 256:] == 7.0)


def test_fwd_varlen_malformed_cu_stays_in_range(ma):
    # Decreasing and out-of-range entries are clamped to [0, total]: results are defined by
    # the clamped offsets and nothing outside the tensors is touched.
    w = W.make_varlen([100, 100], [80, 80], 2, 64, seed=9)
    q, k, v = (t.to(DEV) for t in (w.q, w.k, w.v))
    cq = torch.tensor([0, 150, 120], dtype=torch.int32, device=DEV)     # end < start for b = 1
    ck = torch.tensor([-5, 1000, 2000], dtype=torch.int32, device=DEV)
    out = torch.zeros_like(q)
    o, l = ma.attn_fwd_varlen(q, k, v, cq, ck, 200, w.scale, out=out)
    torch.cuda.synchronize()
    # clamped: sequence 0 = queries 0..149 vs keys 0..159; sequence 1 = no rows
    Oref, Lref = oracle.attention_varlen(w.q[:150], w.k, w.v, [0, 150], [0, 160], w.scale)
    check_attn(o[:150], l[:, :150].t(), Oref, Lref.T, torch.bfloat16, "varlen clamped")
    assert torch.all(o[150:] == 0)


def test_varlen_p1944_packed(ma):
    w = W.varlen_p1944_packed()
    o, l = run_varlen(ma, w)
    rows = list(range(0, 3644, 37)) + [1943, 1944, 3643]
    Oref, Lref = oracle.attention_varlen(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale)
    check_attn(o[rows], l[:, rows].t(), Oref[rows], Lref[:, rows].T, torch.bfloat16, "varlen p1944")


# ---- paged KV cache (block table) -------------------------------------------------------

PAGED_CASES = [(shape, ps) for shape in DEC_SHAPES for ps in (16, 64)] + [
    ((4, 8, 2, 128, 1, 1500, 1536), 512),
    ((4, 8, 8, 128, 1023, 1023, 1024), 1024),
    ((3, 16, 4, 64, 900, 4000, 4096), 2048),      # pages longer than a split
    ((2, 32, 8, 128, 10, 3000, 3072), 32),
]


def _paged_dev(pg):
    return (pg.k_pages.to(DEV), pg.v_pages.to(DEV), pg.block_table.to(DEV))


@pytest.mark.parametrize("case", PAGED_CASES)
def test_paged_append_then_decode(ma, case):
    (B, Hq, Hkv, D, lo, hi, Tm), ps = case
    w = W.make_decode(B, Hq, Hkv, D, lo, hi, torch.bfloat16, T_max=Tm, seed=B * 100 + Hq + ps)
    pg = W.to_paged(w, ps, seed=ps)
    kp, vp, bt = _paged_dev(pg)
    lens = w.lens.to(DEV)
    ma.kv_append_paged(kp, vp, bt, lens, w.k_new.to(DEV), w.v_new.to(DEV))
    o, l = ma.attn_decode_paged(w.q.to(DEV), kp, vp, bt, lens, w.scale, want_lse=True)
    torch.cuda.synchronize()
    ek, ev, el = oracle.kv_append_paged(pg.k_pages.float().numpy(), pg.v_pages.float().numpy(),
                                        pg.block_table.numpy(), w.lens.numpy(),
                                        w.k_new.float().numpy(), w.v_new.float().numpy())
    assert lens.cpu().tolist() == el.tolist()
    # the append is a bit copy into exactly the pages the oracle wrote
    assert np.array_equal(kp.cpu().float().numpy(), ek) and np.array_equal(vp.cpu().float().numpy(), ev)
    Or, Lr = oracle.decode_paged(w.q, ek, ev, pg.block_table, el, w.scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, f"paged decode {case}")


@pytest.mark.parametrize("ps", [16, 32, 128])
@pytest.mark.parametrize("D", [64, 128])
def test_paged_decode_bitwise_equals_contiguous(ma, ps, D):
    # Same values, same block order: the paged call must reproduce the contiguous call bit for bit.
    w = W.make_decode(5, 16, 4, D, 0, 2500, torch.bfloat16, T_max=2560, seed=ps + D)
    pg = W.to_paged(w, ps, seed=3)
    kp, vp, bt = _paged_dev(pg)
    lens = w.lens.to(DEV)
    o1, l1 = ma.attn_decode_paged(w.q.to(DEV), kp, vp, bt, lens, w.scale, want_lse=True)
    o2, l2 = ma.attn_decode(w.q.to(DEV), w.k_cache.to(DEV), w.v_cache.to(DEV), lens, w.scale, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_decode_shared_and_bad_entries(ma):
    # Two sequences share their first pages (a shared prefix); entries past a sequence's
    # length are garbage (never read); out-of-range entries inside the length are clamped.
    w = W.make_decode(3, 8, 2, 128, 10, 200, torch.bfloat16, T_max=256, lens=[100, 70, 40], seed=4)
    pg = W.to_paged(w, 16, seed=5)
    bt = pg.block_table.clone()
    n = pg.k_pages.shape[0]
    bt[1, :4] = bt[0, :4]                 # shared prefix pages
    bt[0, 7:] = 10 ** 6                   # past len 100 (pages 0..6 used): never read
    bt[2, 2] = -7                         # inside len 40: clamped to page 0
    bt[2, 1] = n + 5                      # clamped to the last page
    kp, vp, _ = _paged_dev(pg)
    o, l = ma.attn_decode_paged(w.q.to(DEV), kp, vp, bt.to(DEV), w.lens.to(DEV), w.scale, want_lse=True)
    torch.cuda.synchronize()
    eff = bt.clamp(0, n - 1)
    Or, Lr = oracle.decode_paged(w.q, pg.k_pages, pg.v_pages, eff, w.lens, w.scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, "paged shared / clamped")


def test_paged_decode_zero_lengths(ma):
    w = W.make_decode(5, 8, 2, 64, 0, 10, torch.bfloat16, T_max=1024, lens=[0, 513, 0, 0, 31], seed=6)
    pg = W.to_paged(w, 16, seed=7)
    kp, vp, bt = _paged_dev(pg)
    o, l = ma.attn_decode_paged(w.q.to(DEV), kp, vp, bt, w.lens.to(DEV), w.scale, want_lse=True)
    torch.cuda.synchronize()
    Or, Lr = oracle.decode_paged(w.q, pg.k_pages, pg.v_pages, pg.block_table, w.lens, w.scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, "paged zero lengths")


# ---- GQA + causal prefill ------------------------------------------------------------------

PREFILL = [
    # B, H_q, H_kv, Tq, Tk, D, causal, valid key lengths (None = no mask)
    (1, 1, 1, 1, 1, 64, True, None),
    (1, 2, 1, 31, 31, 128, True, None),
    (1, 4, 1, 300, 300, 64, True, None),
    (2, 8, 2, 257, 257, 128, True, None),
    (1, 2, 2, 100, 700, 64, True, None),          # a chunk after a cached prefix
    (1, 2, 1, 600, 200, 128, True, None),         # more queries than keys: early rows see nothing
    (2, 6, 3, 513, 513, 64, True, [513, 300]),    # causal and key padding together
    (1, 4, 2, 333, 333, 64, False, [333]),        # GQA, not causal
    (2, 4, 4, 1000, 1000, 64, True, None),
    (1, 8, 1, 600, 900, 128, False, [850]),
]


@pytest.mark.parametrize("case", PREFILL)
def test_prefill_gqa_causal(ma, case):
    B, Hq, Hkv, Tq, Tk, D, causal, valid = case
    w = W.make_gqa_prefill(B, Hq, Hkv, Tq, Tk, D, valid=valid, seed=Tq + Hq)
    m = w.mask.to(DEV) if w.mask is not None else None
    o, l = ma.attn_prefill(w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), m, causal, w.scale)
    torch.cuda.synchronize()
    Or, Lr = oracle.prefill(w.q, w.k, w.v, w.mask, causal, w.scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, f"prefill {case}")


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_gqa_bitwise_equals_mha_on_repeated_kv(ma, D):
    w = W.make_gqa_prefill(2, 8, 2, 300, 450, D, valid=[450, 200], seed=3)
    q, k, v, m = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), w.mask.to(DEV)
    o1, l1 = ma.attn_prefill(q, k, v, m, False, w.scale)
    o2, l2 = ma.attn_fwd_lse(q, k.repeat_interleave(4, dim=1).contiguous(),
                             v.repeat_interleave(4, dim=1).contiguous(), m, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_causal_single_query_bitwise_equals_noncausal(ma, D):
    # one query is the last position: it sees every key, exactly the non-causal call
    w = W.make_gqa_prefill(2, 4, 4, 1, 777, D, valid=[777, 500], seed=4)
    q, k, v, m = w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), w.mask.to(DEV)
    o1, l1 = ma.attn_prefill(q, k, v, m, True, w.scale)
    o2, l2 = ma.attn_fwd_lse(q, k, v, m, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


VARLEN_CAUSAL = [
    # lens_q, lens_k, H_q, H_kv, D, causal
    ([300, 0, 513, 64], [300, 10, 513, 100], 4, 2, 64, True),
    ([1, 257, 40], [1, 257, 600], 8, 2, 128, True),
    ([700, 129], [700, 129], 2, 1, 64, False),
    ([100, 300], [40, 300], 4, 4, 128, True),       # Tq > Tk in the first sequence
]


@pytest.mark.parametrize("case", VARLEN_CAUSAL)
def test_prefill_varlen_gqa_causal(ma, case):
    lq, lk, Hq, Hkv, D, causal = case
    w = W.make_varlen(lq, lk, Hq, D, H_kv=Hkv, seed=len(lq) * 10 + Hq)
    q, k, v, cq, ck = (t.to(DEV) for t in (w.q, w.k, w.v, w.cu_q, w.cu_k))
    o, l = ma.attn_prefill_varlen(q, k, v, cq, ck, w.max_q, causal, w.scale)
    torch.cuda.synchronize()
    Or, Lr = oracle.prefill_varlen(w.q, w.k, w.v, w.cu_q, w.cu_k, causal, w.scale)
    check_attn(o, l.t(), Or, Lr.T, torch.bfloat16, f"varlen prefill {case}")


def test_gqa_causal_prefill_8192_sampled_rows(ma):
    """The 8,192-token causal GQA prompt (H_q 32 / H_kv 8, D128): rows in every q-tile of every head."""
    w = W.gqa_causal_prefill_8192()
    o, l = ma.attn_prefill(w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), None, True, w.scale)
    torch.cuda.synchronize()
    rows = tile_rows(8192)
    Or, Lr = oracle.prefill(w.q, w.k, w.v, None, True, w.scale, rows=rows)
    check_attn(o[:, :, rows], l[:, :, rows], Or, Lr, torch.bfloat16, "causal 8192 sampled rows")


# ---- FP8 (E4M3) KV cache ----------------------------------------------------------------

FP8_DEC = [
    # B, Hq, Hkv, D, len_lo, len_hi, T_max
    (3, 4, 4, 64, 1, 40, 64),
    (4, 8, 2, 128, 1, 1500, 1536),
    (2, 32, 8, 128, 500, 1100, 1152),
    (3, 6, 2, 64, 0, 600, 640),
    (2, 40, 1, 64, 100, 900, 960),
    (70, 8, 4, 128, 1, 300, 320),
    (4, 8, 8, 128, 1023, 1023, 1024),
    (1, 1, 1, 128, 0, 0, 64),
]


def _fp8_dev(w):
    return (w.k_cache.to(DEV), w.v_cache.to(DEV), w.k_scale.to(DEV), w.v_scale.to(DEV), w.lens.to(DEV))


@pytest.mark.parametrize("shape", FP8_DEC)
def test_fp8_append_then_decode(ma, shape):
    B, Hq, Hkv, D, lo, hi, Tm = shape
    w = W.make_decode_fp8(B, Hq, Hkv, D, lo, hi, T_max=Tm, seed=B * 10 + Hq)
    kc, vc, ks, vs, lens = _fp8_dev(w)
    ma.kv_append_fp8(kc, vc, ks, vs, lens, w.k_new.to(DEV), w.v_new.to(DEV))
    o, l = ma.attn_decode_fp8kv(w.q.to(DEV), kc, vc, ks, vs, lens, w.scale, want_lse=True)
    torch.cuda.synchronize()
    ek, ev, el = oracle.kv_append_fp8(w.k_cache.numpy(), w.v_cache.numpy(), w.k_scale, w.v_scale, w.lens.numpy(),
                                      w.k_new, w.v_new)
    assert lens.cpu().tolist() == el.tolist()
    assert np.array_equal(kc.cpu().numpy(), ek) and np.array_equal(vc.cpu().numpy(), ev)   # bytes, exact
    Or, Lr = oracle.decode_fp8kv(w.q, ek, ev, w.k_scale, w.v_scale, el, w.scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, f"fp8 decode {shape}")


# Scales drawn U[0.01, 2) rather than powers of two: the kernels fold the softmax scale with the
# K scale, and the V scale into 1 / l, in float32, where only power-of-two scales are exact.
UNIFORM_DEC = [(3, 8, 2, 64, 1, 700, 768), (4, 32, 8, 128, 300, 2500, 2560), (70, 8, 4, 128, 1, 300, 320)]


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("shape", UNIFORM_DEC)
def test_8bit_decode_uniform_scales(ma, shape, fmt):
    B, Hq, Hkv, D, lo, hi, Tm = shape
    make = W.make_decode_fp8 if fmt == "fp8" else W.make_decode_int8
    w = make(B, Hq, Hkv, D, lo, hi, T_max=Tm, seed=B + Hq + D, scales="uniform")
    assert not torch.all(torch.log2(w.k_scale) == torch.round(torch.log2(w.k_scale)))
    append = ma.kv_append_fp8 if fmt == "fp8" else ma.kv_append_int8
    decode = ma.attn_decode_fp8kv if fmt == "fp8" else ma.attn_decode_int8kv
    kc, vc, ks, vs, lens = _fp8_dev(w)
    append(kc, vc, ks, vs, lens, w.k_new.to(DEV), w.v_new.to(DEV))
    o, l = decode(w.q.to(DEV), kc, vc, ks, vs, lens, w.scale, want_lse=True)
    torch.cuda.synchronize()
    oapp = oracle.kv_append_fp8 if fmt == "fp8" else oracle.kv_append_int8
    odec = oracle.decode_fp8kv if fmt == "fp8" else oracle.decode_int8kv
    ek, ev, el = oapp(w.k_cache.numpy(), w.v_cache.numpy(), w.k_scale, w.v_scale, w.lens.numpy(), w.k_new, w.v_new)
    assert np.array_equal(kc.cpu().numpy(), ek) and np.array_equal(vc.cpu().numpy(), ev)
    Or, Lr = odec(w.q, ek, ev, w.k_scale, w.v_scale, el, w.scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, f"{fmt} decode, uniform scales {shape}")


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_paged_8bit_decode_uniform_scales(ma, fmt):
    make, append, decode, o_append, o_decode, _, _ = _q8_calls(ma, fmt)
    w = make(4, 16, 4, 128, 1, 1500, T_max=1536, seed=77, scales="uniform")
    pg = W.to_paged(w, 32, seed=5)
    kp, vp, bt = _paged_dev(pg)
    ks, vs, lens = w.k_scale.to(DEV), w.v_scale.to(DEV), w.lens.to(DEV)
    append(kp, vp, ks, vs, bt, lens, w.k_new.to(DEV), w.v_new.to(DEV))
    o, l = decode(w.q.to(DEV), kp, vp, ks, vs, bt, lens, w.scale, want_lse=True)
    torch.cuda.synchronize()
    ek, ev, el = o_append(pg.k_pages, pg.v_pages, w.k_scale, w.v_scale, pg.block_table.numpy(), w.lens.numpy(),
                          w.k_new, w.v_new)
    assert np.array_equal(kp.cpu().numpy(), ek) and np.array_equal(vp.cpu().numpy(), ev)
    Or, Lr = o_decode(w.q, ek, ev, w.k_scale, w.v_scale, pg.block_table, el, w.scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, f"paged {fmt} decode, uniform scales")


@pytest.mark.parametrize("new_dtype", [torch.bfloat16, torch.float32])
def test_fp8_append_quantisation_edges(ma, new_dtype):
    # ties to even, saturation, the subnormal boundary, zeros and signs, in both input dtypes
    B, Hkv, D, Tm = 2, 2, 64, 64
    w = W.make_decode_fp8(B, 2, Hkv, D, 3, 10, T_max=Tm, seed=5)
    special = torch.tensor([1.0625, 1.1875, -1.0625, 1e6, -1e6, 2.0 ** -10, 3 * 2.0 ** -11, 0.0, -0.0,
                            448.0, 464.0, 0.0009765625, 240.0, 232.0, -3.5, 17.0])
    g = torch.Generator().manual_seed(9)
    kn = torch.randn(B, Hkv, 1, D, generator=g) * 40
    vn = torch.randn(B, Hkv, 1, D, generator=g) * 0.01
    kn[0, 0, 0, :16] = special
    vn[1, 1, 0, :16] = special
    kn, vn = kn.to(new_dtype).contiguous(), vn.to(new_dtype).contiguous()
    ks = torch.tensor([[1.0, 0.75], [0.3, 2.0]], dtype=torch.float32)
    vs = torch.tensor([[0.001, 0.25], [1.5, 1.0]], dtype=torch.float32)
    kc, vc = w.k_cache.to(DEV), w.v_cache.to(DEV)
    lens = w.lens.to(DEV)
    ma.kv_append_fp8(kc, vc, ks.to(DEV), vs.to(DEV), lens, kn.to(DEV), vn.to(DEV))
    torch.cuda.synchronize()
    ek, ev, el = oracle.kv_append_fp8(w.k_cache.numpy(), w.v_cache.numpy(), ks, vs, w.lens.numpy(), kn, vn)
    assert np.array_equal(kc.cpu().numpy(), ek) and np.array_equal(vc.cpu().numpy(), ev)
    assert lens.cpu().tolist() == el.tolist()


def test_fp8_decode_zero_lengths(ma):
    w = W.make_decode_fp8(5, 8, 2, 128, 0, 10, T_max=1024, lens=[0, 513, 0, 0, 31], seed=6)
    kc, vc, ks, vs, lens = _fp8_dev(w)
    o, l = ma.attn_decode_fp8kv(w.q.to(DEV), kc, vc, ks, vs, lens, w.scale, want_lse=True)
    torch.cuda.synchronize()
    Or, Lr = oracle.decode_fp8kv(w.q, w.k_cache, w.v_cache, w.k_scale, w.v_scale, w.lens, w.scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, "fp8 decode zero lengths")


# ---- FP8 (E4M3) prefill with LSE ------------------------------------------------------------

PREFILL_FP8 = [
    # B, H_q, H_kv, Tq, Tk, D, causal, valid key lengths (None = no mask)
    (1, 1, 1, 1, 1, 64, False, None),
    (1, 2, 1, 31, 31, 128, True, None),
    (2, 4, 2, 300, 333, 64, False, [333, 200]),
    (2, 8, 2, 257, 257, 128, True, None),
    (1, 2, 2, 100, 700, 64, True, None),          # a chunk after a cached prefix
    (1, 2, 1, 600, 200, 128, True, None),         # more queries than keys: early rows see nothing
    (2, 6, 3, 513, 513, 64, True, [513, 300]),    # causal and key padding together
    (1, 8, 1, 600, 900, 128, False, [850]),
    (2, 4, 4, 1000, 1000, 64, False, [1000, 0]),  # a fully padded sequence
    (1, 4, 2, 64, 4000, 128, False, [3990]),      # long key range, one q-tile
]


def _fp8_prefill(ma, w, causal, **kw):
    m = w.mask.to(DEV) if w.mask is not None else None
    r = ma.attn_prefill_fp8(w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), w.q_scale.to(DEV), w.k_scale.to(DEV),
                            w.v_scale.to(DEV), m, causal, w.scale, **kw)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("case", PREFILL_FP8)
def test_prefill_fp8(ma, case):
    B, Hq, Hkv, Tq, Tk, D, causal, valid = case
    w = W.make_prefill_fp8(B, Hq, Hkv, Tq, Tk, D, valid=valid, seed=Tq + Hq + D)
    o, l = _fp8_prefill(ma, w, causal)
    Or, Lr = oracle.prefill_fp8(w.q, w.k, w.v, w.q_scale, w.k_scale, w.v_scale, w.mask, causal, w.scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, f"fp8 prefill {case}")


def v_units(codes, v_scale, packed=False):
    """The largest per-(sequence, KV head) RMS of the dequantised V values (at least 1): the
    unit of the O bar for inputs spread wider than N(0, 1).  O is a convex combination of V
    rows, so its bf16 roundings scale with |V| (as in test_fwd_peaky_scores); LSE keeps its bar.
    codes: uint8 E4M3 [B, H_kv, T, D] (packed: [T, H_kv, D], one sequence)."""
    x = codes.view(torch.float8_e4m3fn).float()
    if packed:
        x = x.transpose(0, 1).unsqueeze(0)
    rms = x.pow(2).mean(dim=(2, 3)).sqrt() * v_scale[: x.shape[0]]
    return max(1.0, float(rms.max()))


@pytest.mark.parametrize("case", [PREFILL_FP8[i] for i in (2, 3, 6, 7, 9)])
def test_prefill_fp8_uniform_scales(ma, case):
    B, Hq, Hkv, Tq, Tk, D, causal, valid = case
    w = W.make_prefill_fp8(B, Hq, Hkv, Tq, Tk, D, valid=valid, seed=Tq + Hq + D + 1, scales="uniform")
    o, l = _fp8_prefill(ma, w, causal)
    Or, Lr = oracle.prefill_fp8(w.q, w.k, w.v, w.q_scale, w.k_scale, w.v_scale, w.mask, causal, w.scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, f"fp8 prefill, uniform scales {case}",
               o_tol=2e-2 * v_units(w.v, w.v_scale))


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_fp8_lse_flag_and_v_scale_bitwise(ma, D):
    # O does not depend on whether the LSE is written; doubling the V scale doubles O exactly
    # (a power-of-two factor on the final reciprocal) and leaves the LSE bit-identical
    w = W.make_prefill_fp8(2, 4, 2, 300, 450, D, valid=[450, 200], seed=3)
    o1, l1 = _fp8_prefill(ma, w, True)
    o2 = _fp8_prefill(ma, w, True, want_lse=False)
    w.v_scale = w.v_scale * 2
    o3, l3 = _fp8_prefill(ma, w, True)
    assert torch.equal(o1, o2)
    assert torch.equal(o3, o1 * 2) and torch.equal(l3, l1)


def test_prefill_fp8_p11616_sampled_rows(ma):
    """The P = 11,616 patch shape with E4M3 inputs: rows in every q-tile of every head."""
    w = W.patch_p11616_fp8()
    o, l = _fp8_prefill(ma, w, False)
    rows = tile_rows(11616)
    Or, Lr = oracle.prefill_fp8(w.q, w.k, w.v, w.q_scale, w.k_scale, w.v_scale, w.mask, False, w.scale,
                                rows=rows)
    check_attn(o[:, :, rows], l[:, :, rows], Or, Lr, torch.bfloat16, "fp8 P11616 sampled rows")


def test_gqa_causal_prefill_8192_fp8_sampled_rows(ma):
    """The causal GQA 8,192-token prompt with E4M3 inputs: rows in every q-tile of every head."""
    w = W.gqa_causal_prefill_8192_fp8()
    o, l = _fp8_prefill(ma, w, True)
    rows = tile_rows(8192)
    Or, Lr = oracle.prefill_fp8(w.q, w.k, w.v, w.q_scale, w.k_scale, w.v_scale, None, True, w.scale, rows=rows)
    check_attn(o[:, :, rows], l[:, :, rows], Or, Lr, torch.bfloat16, "fp8 causal 8192 sampled rows")


# ---- INT8 KV cache ----------------------------------------------------------------------------

@pytest.mark.parametrize("shape", FP8_DEC)
def test_int8_append_then_decode(ma, shape):
    B, Hq, Hkv, D, lo, hi, Tm = shape
    w = W.make_decode_int8(B, Hq, Hkv, D, lo, hi, T_max=Tm, seed=B * 10 + Hq + 1)
    kc, vc, ks, vs, lens = _fp8_dev(w)
    ma.kv_append_int8(kc, vc, ks, vs, lens, w.k_new.to(DEV), w.v_new.to(DEV))
    o, l = ma.attn_decode_int8kv(w.q.to(DEV), kc, vc, ks, vs, lens, w.scale, want_lse=True)
    torch.cuda.synchronize()
    ek, ev, el = oracle.kv_append_int8(w.k_cache.numpy(), w.v_cache.numpy(), w.k_scale, w.v_scale,
                                       w.lens.numpy(), w.k_new, w.v_new)
    assert lens.cpu().tolist() == el.tolist()
    assert np.array_equal(kc.cpu().numpy(), ek) and np.array_equal(vc.cpu().numpy(), ev)   # bytes, exact
    Or, Lr = oracle.decode_int8kv(w.q, ek, ev, w.k_scale, w.v_scale, el, w.scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, f"int8 decode {shape}")


@pytest.mark.parametrize("new_dtype", [torch.bfloat16, torch.float32])
def test_int8_append_quantisation_edges(ma, new_dtype):
    # ties to even, saturation at +-127, signed zero, and the full code range
    B, Hkv, D, Tm = 2, 2, 64, 64
    w = W.make_decode_int8(B, 2, Hkv, D, 3, 10, T_max=Tm, seed=5)
    special = torch.tensor([0.5, 1.5, 2.5, -0.5, -2.5, 126.5, 127.5, 1e6, -1e6, -0.0, 0.0, 3.25, -127.0,
                            100.5, -99.5, 127.49])
    g = torch.Generator().manual_seed(9)
    kn = torch.randn(B, Hkv, 1, D, generator=g) * 60
    vn = torch.randn(B, Hkv, 1, D, generator=g) * 0.05
    kn[0, 0, 0, :16] = special
    vn[1, 1, 0, :16] = special * 0.25
    kn, vn = kn.to(new_dtype).contiguous(), vn.to(new_dtype).contiguous()
    ks = torch.tensor([[1.0, 0.75], [0.3, 2.0]], dtype=torch.float32)
    vs = torch.tensor([[0.001, 0.25], [1.5, 0.25]], dtype=torch.float32)
    kc, vc = w.k_cache.to(DEV), w.v_cache.to(DEV)
    lens = w.lens.to(DEV)
    ma.kv_append_int8(kc, vc, ks.to(DEV), vs.to(DEV), lens, kn.to(DEV), vn.to(DEV))
    torch.cuda.synchronize()
    ek, ev, el = oracle.kv_append_int8(w.k_cache.numpy(), w.v_cache.numpy(), ks, vs, w.lens.numpy(), kn, vn)
    assert np.array_equal(kc.cpu().numpy(), ek) and np.array_equal(vc.cpu().numpy(), ev)
    assert lens.cpu().tolist() == el.tolist()


def test_int8_decode_v_scale_doubles_o_exactly(ma):
    # the V scale multiplies each partial O (a power-of-two factor is exact) and not the weights:
    # doubling it doubles O bit for bit and leaves the LSE unchanged.  Unit K scales (scores of
    # codes up to +-127: peaky rows, many raised references) against the oracle, with V at 1/64
    # (O of order one, the scale of the tolerance)
    w = W.make_decode_int8(4, 8, 2, 128, 1, 1500, T_max=1536, seed=12)
    kc, vc, lens = w.k_cache.to(DEV), w.v_cache.to(DEV), (w.lens + 1).to(DEV)
    ks = torch.ones(4, 2, dtype=torch.float32, device=DEV)
    vs = ks / 64
    q = w.q.to(DEV)
    o1, l1 = ma.attn_decode_int8kv(q, kc, vc, ks, vs, lens, w.scale, want_lse=True)
    o2, l2 = ma.attn_decode_int8kv(q, kc, vc, ks, vs * 2, lens, w.scale, want_lse=True)
    torch.cuda.synchronize()
    Or, Lr = oracle.decode_int8kv(w.q, w.k_cache, w.v_cache, np.ones((4, 2)), np.full((4, 2), 1 / 64),
                                  w.lens + 1, w.scale)
    check_attn(o1, l1, Or, Lr, torch.bfloat16, "int8 decode, unit K scales")
    assert torch.equal(o2, o1 * 2) and torch.equal(l2, l1)


# ---- lazy-rescale regression: the reference rises inside a 32-key block -------------------------

def _rising(B=2, Hq=8, Hkv=2, T=320, D=64, seed=31):
    """Q all ones; K rows constant per token.  Score steps of sqrt(D)·log2(e) log2 units sit in
    the second 16-key half of a 32-key block while its first half still carries the old
    reference's weights: 0 up to token 47, 1 for tokens 48..63 (block 1), 1 for 224..239 and 2
    for 240..255 (block 7; these last keys dominate the result, so a weight of the first half
    kept against the old reference shows in O).  V is N(0,1).  Returns float32 q, k, v and the
    scale."""
    g = torch.Generator().manual_seed(seed)
    q = torch.ones(B, Hq, 1, D)
    k = torch.zeros(B, Hkv, T, D)
    k[:, :, 48:64] = 1.0
    k[:, :, 224:240] = 1.0
    k[:, :, 240:256] = 2.0
    v = torch.randn(B, Hkv, T, D, generator=g)
    return q, k, v, 1.0 / math.sqrt(D)


def test_decode_rescale_inside_block_bf16_and_paged(ma):
    q, k, v, scale = _rising()
    B = q.shape[0]
    lens = torch.full((B,), 300, dtype=torch.int32)
    Or, Lr = oracle.decode(q, k, v, lens, scale)
    kb, vb, qb = k.to(torch.bfloat16), v.to(torch.bfloat16), q.to(torch.bfloat16)
    o, l = ma.attn_decode(qb.to(DEV), kb.to(DEV), vb.to(DEV), lens.to(DEV), scale, want_lse=True)
    torch.cuda.synchronize()
    check_attn(o, l, Or, Lr, torch.bfloat16, "bf16 decode, reference raised inside a block")
    d = W.Decode(qb, kb, vb, kb[:, :, :1].contiguous(), vb[:, :, :1].contiguous(), lens, scale)
    pg = W.to_paged(d, 16, seed=2)
    kp, vp, bt = _paged_dev(pg)
    o, l = ma.attn_decode_paged(qb.to(DEV), kp, vp, bt, lens.to(DEV), scale, want_lse=True)
    torch.cuda.synchronize()
    check_attn(o, l, Or, Lr, torch.bfloat16, "paged decode, reference raised inside a block")


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_decode_rescale_inside_block_8bit(ma, fmt):
    q, k, v, scale = _rising(D=128)
    B, Hkv, T, D = k.shape
    lens = torch.full((B,), 300, dtype=torch.int32)
    vs = torch.full((B, Hkv), 1.0 / 16)
    ks = torch.ones(B, Hkv)
    if fmt == "fp8":      # K values 0, 1, 2 and V / (1/16) are E4M3-exact after the cast
        kc = k.to(torch.float8_e4m3fn).view(torch.uint8)
        vc = (v * 16).to(torch.float8_e4m3fn).view(torch.uint8)
        kd, vd = oracle.dequantize_e4m3(kc, 1.0), oracle.dequantize_e4m3(vc, 1.0 / 16)
        fn = ma.attn_decode_fp8kv
    else:
        kc = k.to(torch.int8)
        vc = torch.round(v * 16).clamp(-127, 127).to(torch.int8)
        kd, vd = oracle.dequantize_int8(kc, 1.0), oracle.dequantize_int8(vc, 1.0 / 16)
        fn = ma.attn_decode_int8kv
    Or, Lr = oracle.decode(q, kd, vd, lens, scale)
    o, l = fn(q.to(torch.bfloat16).to(DEV), kc.contiguous().to(DEV), vc.contiguous().to(DEV), ks.to(DEV),
              vs.to(DEV), lens.to(DEV), scale, want_lse=True)
    torch.cuda.synchronize()
    check_attn(o, l, Or, Lr, torch.bfloat16, f"{fmt} decode, reference raised inside a block")


@pytest.mark.parametrize("half", [0, 1])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("fp8", [False, True])
def test_prefill_rescale_inside_step(ma, D, fp8, half):
    """The lazy reference rising at the second 16-key half of a 32-key block while the first half
    still carries the old reference's weights (the rescale then has to cover every PV product of
    the first half).  Q all ones; K rows constant per key: 0, except a for keys 48..63 (a = 0.5 at
    D = 64, 0.375 at D = 128: steps of 5.8 and 6.1 log2 units, a lane's chunk sum of ~440 and
    ~560, just past the 2^8 trigger, so the old-reference weights of the first half matter);
    V N(0,1).  half = 0 puts the step at keys 32..47 instead (the first half of block 1): the
    check of the first half then also redoes the second half's softmax stages already begun."""
    B, H, Tq, Tk = 1, 2, 64, 200
    g = torch.Generator().manual_seed(D)
    q = torch.ones(B, H, Tq, D)
    k = torch.zeros(B, H, Tk, D)
    lo = 48 if half else 32
    k[:, :, lo:64] = 0.5 if D == 64 else 0.375
    v = torch.randn(B, H, Tk, D, generator=g)
    scale = 1.0 / math.sqrt(D)
    Or, Lr = oracle.prefill(q, k, v, None, False, scale)
    if fp8:   # ones, the step and V·16 in E4M3 (V rounded, dequantised by the oracle)
        q8, k8 = q.to(torch.float8_e4m3fn).view(torch.uint8), k.to(torch.float8_e4m3fn).view(torch.uint8)
        v8 = (v * 16).to(torch.float8_e4m3fn).view(torch.uint8)
        qs, ks, vs = torch.ones(B, H), torch.ones(B, H), torch.full((B, H), 1.0 / 16)
        Or, Lr = oracle.prefill_fp8(q8, k8, v8, qs, ks, vs, None, False, scale)
        o, l = ma.attn_prefill_fp8(q8.to(DEV), k8.to(DEV), v8.to(DEV), qs.to(DEV), ks.to(DEV), vs.to(DEV), None,
                                   False, scale)
    else:
        o, l = ma.attn_prefill(q.to(torch.bfloat16).to(DEV), k.to(torch.bfloat16).to(DEV),
                               v.to(torch.bfloat16).to(DEV), None, False, scale)
    torch.cuda.synchronize()
    check_attn(o, l, Or, Lr, torch.bfloat16, f"prefill rescale inside a step D={D} fp8={fp8} half={half}")


# ---- packed (varlen) FP8 prefill ---------------------------------------------------------------

VARLEN_FP8 = [
    # lens_q, lens_k, H_q, H_kv, D, causal
    ([300, 0, 513, 64], [300, 10, 513, 100], 4, 2, 64, True),
    ([1, 257, 40], [1, 257, 600], 8, 2, 128, True),
    ([700, 129], [700, 129], 2, 1, 64, False),
    ([100, 300], [40, 300], 4, 4, 128, True),       # Tq > Tk in the first sequence
    ([333], [0], 2, 2, 64, False),                  # no keys at all
]


def _fp8v_dev(w):
    return tuple(t.to(DEV) for t in (w.q, w.k, w.v, w.q_scale, w.k_scale, w.v_scale, w.cu_q, w.cu_k))


@pytest.mark.parametrize("case", VARLEN_FP8)
def test_prefill_varlen_fp8(ma, case):
    lq, lk, Hq, Hkv, D, causal = case
    w = W.make_varlen_fp8(lq, lk, Hq, D, H_kv=Hkv, seed=len(lq) * 10 + Hq + D)
    q, k, v, qs, ks, vs, cq, ck = _fp8v_dev(w)
    o, l = ma.attn_prefill_varlen_fp8(q, k, v, qs, ks, vs, cq, ck, w.max_q, causal, w.scale)
    torch.cuda.synchronize()
    Or, Lr = oracle.prefill_varlen_fp8(w.q, w.k, w.v, w.q_scale, w.k_scale, w.v_scale, w.cu_q, w.cu_k,
                                       causal, w.scale)
    check_attn(o, l.t(), Or, Lr.T, torch.bfloat16, f"packed fp8 prefill {case}")


@pytest.mark.parametrize("case", [VARLEN_FP8[0], VARLEN_FP8[1]])
def test_prefill_varlen_fp8_uniform_scales(ma, case):
    lq, lk, Hq, Hkv, D, causal = case
    w = W.make_varlen_fp8(lq, lk, Hq, D, H_kv=Hkv, seed=len(lq) * 10 + Hq + D + 1, scales="uniform")
    q, k, v, qs, ks, vs, cq, ck = _fp8v_dev(w)
    o, l = ma.attn_prefill_varlen_fp8(q, k, v, qs, ks, vs, cq, ck, w.max_q, causal, w.scale)
    torch.cuda.synchronize()
    Or, Lr = oracle.prefill_varlen_fp8(w.q, w.k, w.v, w.q_scale, w.k_scale, w.v_scale, w.cu_q, w.cu_k,
                                       causal, w.scale)
    unit = max(v_units(w.v[int(w.cu_k[b]):int(w.cu_k[b + 1])], w.v_scale[b:b + 1], packed=True)
               for b in range(len(lk)) if lk[b] > 0)
    check_attn(o, l.t(), Or, Lr.T, torch.bfloat16, f"packed fp8 prefill, uniform scales {case}",
               o_tol=2e-2 * unit)


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_varlen_fp8_bitwise_equals_dense(ma, D):
    # one packed sequence is the dense [1, H, T, D] call on the same codes, bit for bit
    w = W.make_varlen_fp8([700], [900], 8, D, H_kv=2, seed=D + 1)
    q, k, v, qs, ks, vs, cq, ck = _fp8v_dev(w)
    o1, l1 = ma.attn_prefill_varlen_fp8(q, k, v, qs, ks, vs, cq, ck, w.max_q, True, w.scale)
    dense = lambda t: t.transpose(0, 1).unsqueeze(0).contiguous()
    o2, l2 = ma.attn_prefill_fp8(dense(q), dense(k), dense(v), qs, ks, vs, None, True, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2[0].transpose(0, 1)) and torch.equal(l1, l2[0])


def test_varlen_ring_hop_8192_fp8_sampled_rows(ma):
    """The E4M3 packed ring hop (8,192 queries x 8,192 keys, H24 D128): rows in every q-tile."""
    w = W.varlen_ring_hop_8192_fp8()
    q, k, v, qs, ks, vs, cq, ck = _fp8v_dev(w)
    o, l = ma.attn_prefill_varlen_fp8(q, k, v, qs, ks, vs, cq, ck, w.max_q, False, w.scale)
    torch.cuda.synchronize()
    rows = tile_rows(8192)
    dq = lambda t: t.transpose(0, 1).unsqueeze(0)
    Or, Lr = oracle.prefill_fp8(dq(w.q), dq(w.k), dq(w.v), w.q_scale, w.k_scale, w.v_scale, None, False, w.scale,
                                rows=rows)
    check_attn(o[rows].transpose(0, 1).unsqueeze(0), l[:, rows].unsqueeze(0), Or, Lr, torch.bfloat16,
               "packed fp8 ring hop sampled rows")


# ---- paged 8-bit caches ------------------------------------------------------------------------

PAGED8_CASES = [
    # (B, Hq, Hkv, D, len_lo, len_hi, T_max), page_size
    ((3, 8, 2, 128, 1, 700, 768), 16),
    ((4, 8, 8, 64, 0, 600, 640), 64),
    ((2, 32, 8, 128, 500, 1100, 1152), 32),
    ((5, 40, 1, 64, 1, 1500, 1536), 512),
]


def _q8_calls(ma, fmt):
    if fmt == "fp8":
        return (W.make_decode_fp8, ma.kv_append_fp8_paged, ma.attn_decode_fp8kv_paged, oracle.kv_append_fp8_paged,
                oracle.decode_fp8kv_paged, ma.kv_append_fp8, ma.attn_decode_fp8kv)
    return (W.make_decode_int8, ma.kv_append_int8_paged, ma.attn_decode_int8kv_paged, oracle.kv_append_int8_paged,
            oracle.decode_int8kv_paged, ma.kv_append_int8, ma.attn_decode_int8kv)


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("case", PAGED8_CASES)
def test_paged_8bit_append_then_decode(ma, case, fmt):
    (B, Hq, Hkv, D, lo, hi, Tm), ps = case
    make, append, decode, o_append, o_decode, _, _ = _q8_calls(ma, fmt)
    w = make(B, Hq, Hkv, D, lo, hi, T_max=Tm, seed=B * 100 + Hq + ps)
    pg = W.to_paged(w, ps, seed=ps)
    kp, vp, bt = _paged_dev(pg)
    ks, vs, lens = w.k_scale.to(DEV), w.v_scale.to(DEV), w.lens.to(DEV)
    append(kp, vp, ks, vs, bt, lens, w.k_new.to(DEV), w.v_new.to(DEV))
    o, l = decode(w.q.to(DEV), kp, vp, ks, vs, bt, lens, w.scale, want_lse=True)
    torch.cuda.synchronize()
    ek, ev, el = o_append(pg.k_pages, pg.v_pages, w.k_scale, w.v_scale, pg.block_table.numpy(), w.lens.numpy(),
                          w.k_new, w.v_new)
    assert lens.cpu().tolist() == el.tolist()
    assert np.array_equal(kp.cpu().numpy(), ek) and np.array_equal(vp.cpu().numpy(), ev)   # bytes, whole pools
    Or, Lr = o_decode(w.q, ek, ev, w.k_scale, w.v_scale, pg.block_table, el, w.scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, f"paged {fmt} decode {case}")


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
@pytest.mark.parametrize("ps", [16, 128])
def test_paged_8bit_bitwise_equals_contiguous(ma, ps, fmt):
    make, append, decode, _, _, c_append, c_decode = _q8_calls(ma, fmt)
    w = make(5, 16, 4, 128, 0, 2500, T_max=2560, seed=ps + 7)
    pg = W.to_paged(w, ps, seed=3)
    kp, vp, bt = _paged_dev(pg)
    kc, vc, ks, vs = w.k_cache.to(DEV), w.v_cache.to(DEV), w.k_scale.to(DEV), w.v_scale.to(DEV)
    l1, l2 = w.lens.to(DEV), w.lens.to(DEV)
    q, kn, vn = w.q.to(DEV), w.k_new.to(DEV), w.v_new.to(DEV)
    append(kp, vp, ks, vs, bt, l1, kn, vn)
    c_append(kc, vc, ks, vs, l2, kn, vn)
    o1, s1 = decode(q, kp, vp, ks, vs, bt, l1, w.scale, want_lse=True)
    o2, s2 = c_decode(q, kc, vc, ks, vs, l2, w.scale, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


# ---- repeated short-item decodes (the Q slot wait) ---------------------------------------------

@pytest.mark.parametrize("fmt", ["bf16", "fp8", "int8"])
def test_decode_short_items_repeated(ma, fmt):
    """Many short items (lengths 1..300, 2 query heads per KV head) start an item every few blocks,
    so an item's Q is read from its LDS slot soon after its buffer->LDS loads were issued.  Without a
    wait for those loads a read could see the slot's previous item (about 1% of such decodes went
    wrong); every one of 150 append + decode rounds must match the oracle."""
    B, Hq, Hkv, D = 32, 8, 4, 64
    if fmt == "bf16":
        w = W.make_decode(B, Hq, Hkv, D, 1, 300, torch.bfloat16, T_max=320, seed=41)
        ek, ev, el = oracle.kv_append(w.k_cache.float().numpy(), w.v_cache.float().numpy(), w.lens.numpy(),
                                      w.k_new.float().numpy(), w.v_new.float().numpy())
        Or, Lr = oracle.decode(w.q, ek, ev, el, w.scale)
    else:
        make = W.make_decode_fp8 if fmt == "fp8" else W.make_decode_int8
        w = make(B, Hq, Hkv, D, 1, 300, T_max=320, seed=41)
        oapp = oracle.kv_append_fp8 if fmt == "fp8" else oracle.kv_append_int8
        odec = oracle.decode_fp8kv if fmt == "fp8" else oracle.decode_int8kv
        ek, ev, el = oapp(w.k_cache.numpy(), w.v_cache.numpy(), w.k_scale, w.v_scale, w.lens.numpy(), w.k_new, w.v_new)
        Or, Lr = odec(w.q, ek, ev, w.k_scale, w.v_scale, el, w.scale)
    q, kn, vn = w.q.to(DEV), w.k_new.to(DEV), w.v_new.to(DEV)
    worst = 0.0
    for it in range(150):
        kc, vc, lens = w.k_cache.to(DEV), w.v_cache.to(DEV), w.lens.to(DEV)
        if fmt == "bf16":
            ma.kv_append(kc, vc, lens, kn, vn)
            o, l = ma.attn_decode(q, kc, vc, lens, w.scale, want_lse=True)
        else:
            ks, vs = w.k_scale.to(DEV), w.v_scale.to(DEV)
            (ma.kv_append_fp8 if fmt == "fp8" else ma.kv_append_int8)(kc, vc, ks, vs, lens, kn, vn)
            o, l = (ma.attn_decode_fp8kv if fmt == "fp8" else ma.attn_decode_int8kv)(q, kc, vc, ks, vs, lens, w.scale,
                                                                                     want_lse=True)
        torch.cuda.synchronize()
        worst = max(worst, float(np.max(np.abs(l.cpu().double().numpy() - Lr))))
        if it == 0 or worst > 1e-3:
            check_attn(o, l, Or, Lr, torch.bfloat16, f"{fmt} short-item decode, round {it}")
    assert worst <= 1e-3, f"{fmt}: max |dLSE| over the rounds {worst:.3e}"


# ---- partials held until a wavefront's range ends ----------------------------------------------

# (B, Hq, Hkv, len_lo, len_hi, T_max) at D = 128 with at most 4 query heads per KV head: the bf16
# and E4M3 decodes then have LDS left for two held partials per wavefront.  Lengths 1..80 make
# items of 1..3 blocks, so a 32-block range ends ~15 items inside it (two held, the rest stored
# at once); lengths 1,025..1,120 end one or two items inside most ranges (all held).
HELD_CASES = [(24, 4, 4, 1, 80, 128), (24, 16, 4, 1, 80, 128), (6, 32, 8, 1024, 1119, 1152), (9, 8, 8, 1024, 1119, 1152)]


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
@pytest.mark.parametrize("case", HELD_CASES)
def test_decode_held_partials(ma, case, fmt, paged):
    B, Hq, Hkv, lo, hi, Tm = case
    D = 128
    if fmt == "bf16":
        w = W.make_decode(B, Hq, Hkv, D, lo, hi, torch.bfloat16, T_max=Tm, seed=B + Hq + hi)
        ek, ev, el = oracle.kv_append(w.k_cache.float().numpy(), w.v_cache.float().numpy(), w.lens.numpy(),
                                      w.k_new.float().numpy(), w.v_new.float().numpy())
        Or, Lr = oracle.decode(w.q, ek, ev, el, w.scale)
    else:
        w = W.make_decode_fp8(B, Hq, Hkv, D, lo, hi, T_max=Tm, seed=B + Hq + hi)
        ek, ev, el = oracle.kv_append_fp8(w.k_cache.numpy(), w.v_cache.numpy(), w.k_scale, w.v_scale,
                                          w.lens.numpy(), w.k_new, w.v_new)
        Or, Lr = oracle.decode_fp8kv(w.q, ek, ev, w.k_scale, w.v_scale, el, w.scale)
    q, kn, vn, lens = w.q.to(DEV), w.k_new.to(DEV), w.v_new.to(DEV), w.lens.to(DEV)
    if paged:
        pg = W.to_paged(w, 16, seed=B)
        kp, vp, bt = _paged_dev(pg)
        if fmt == "bf16":
            ma.kv_append_paged(kp, vp, bt, lens, kn, vn)
            o, l = ma.attn_decode_paged(q, kp, vp, bt, lens, w.scale, want_lse=True)
        else:
            ks, vs = w.k_scale.to(DEV), w.v_scale.to(DEV)
            ma.kv_append_fp8_paged(kp, vp, ks, vs, bt, lens, kn, vn)
            o, l = ma.attn_decode_fp8kv_paged(q, kp, vp, ks, vs, bt, lens, w.scale, want_lse=True)
    else:
        kc, vc = w.k_cache.to(DEV), w.v_cache.to(DEV)
        if fmt == "bf16":
            ma.kv_append(kc, vc, lens, kn, vn)
            o, l = ma.attn_decode(q, kc, vc, lens, w.scale, want_lse=True)
        else:
            ks, vs = w.k_scale.to(DEV), w.v_scale.to(DEV)
            ma.kv_append_fp8(kc, vc, ks, vs, lens, kn, vn)
            o, l = ma.attn_decode_fp8kv(q, kc, vc, ks, vs, lens, w.scale, want_lse=True)
    torch.cuda.synchronize()
    assert lens.cpu().tolist() == el.tolist()
    check_attn(o, l, Or, Lr, torch.bfloat16, f"{fmt} decode with held partials {case} paged={paged}")

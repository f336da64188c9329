"""Pins for the CPU oracle: brute force, closed forms, invariants, a library
cross-check and the byte figures the pages print.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _tolist(a):
    return np.asarray(a, dtype=np.float64).tolist()


# ---- brute force ----------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_attention_matches_brute_force(seed):
    r = _rng(seed)
    B, H = int(r.integers(1, 3)), int(r.integers(1, 3))
    Tq, Tk, D = int(r.integers(1, 10)), int(r.integers(1, 10)), int(r.integers(1, 9))
    q = r.standard_normal((B, H, Tq, D)) * 1.5
    k = r.standard_normal((B, H, Tk, D))
    v = r.standard_normal((B, H, Tk, D))
    mask = (r.random((B, Tk)) < 0.35).astype(np.uint8)
    if seed == 3:
        mask[0, :] = 1                      # one sequence with every key padded
    scale = float(r.uniform(0.2, 1.5))
    O, L = oracle.attention(q, k, v, mask, scale)
    bO, bL = brute.attention(_tolist(q), _tolist(k), _tolist(v), mask.tolist(), scale)
    for b in range(B):
        for h in range(H):
            for i in range(Tq):
                if bL[b][h][i] == -math.inf:
                    assert L[b, h, i] == -np.inf
                    assert np.all(O[b, h, i] == 0.0)
                else:
                    assert abs(L[b, h, i] - bL[b][h][i]) <= 1e-12
                    assert np.max(np.abs(O[b, h, i] - np.array(bO[b][h][i]))) <= 1e-12


def test_attention_rows_subset_equals_full():
    w = workloads.make_prefill(2, 2, 11, 13, 8, torch.float32, valid=[13, 7], seed=5)
    O, L = oracle.attention(w.q, w.k, w.v, w.mask, w.scale)
    rows = [0, 4, 10, 3]
    Os, Ls = oracle.attention(w.q, w.k, w.v, w.mask, w.scale, rows=rows)
    assert np.array_equal(Os, O[:, :, rows]) and np.array_equal(Ls, L[:, :, rows])


@pytest.mark.parametrize("seed", range(4))
def test_merge_matches_brute_force(seed):
    r = _rng(100 + seed)
    n, R, D = int(r.integers(1, 5)), 6, 5
    outs = [r.standard_normal((R, D)) for _ in range(n)]
    lses = [r.standard_normal(R) * 3 for _ in range(n)]
    lses[0][2] = -np.inf                     # an empty chunk for one row
    if n > 1:
        for i in range(n):
            lses[i][4] = -np.inf             # a row empty in every chunk
    O, L = oracle.merge_lse(outs, lses)
    bO, bL = brute.merge([o.tolist() for o in outs], [l.tolist() for l in lses])
    for i in range(R):
        if bL[i] == -math.inf:
            assert L[i] == -np.inf and np.all(O[i] == 0)
        else:
            assert abs(L[i] - bL[i]) <= 1e-12
            assert np.max(np.abs(O[i] - np.array(bO[i]))) <= 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_decode_matches_brute_force(seed):
    r = _rng(200 + seed)
    B, Hkv, G, D, T = 2, 2, int(r.integers(1, 4)), 4, 9
    Hq = Hkv * G
    q = r.standard_normal((B, Hq, 1, D))
    kc = r.standard_normal((B, Hkv, T, D))
    vc = r.standard_normal((B, Hkv, T, D))
    lens = r.integers(1, T + 1, B)
    scale = 0.7
    O, L = oracle.decode(q, kc, vc, lens, scale)
    bO, bL = brute.decode(q[:, :, 0].tolist(), kc.tolist(), vc.tolist(), lens.tolist(), scale)
    for b in range(B):
        for h in range(Hq):
            assert abs(L[b, h] - bL[b][h]) <= 1e-12
            assert np.max(np.abs(O[b, h, 0] - np.array(bO[b][h]))) <= 1e-12


def test_decode_heads_subset():
    w = workloads.make_decode(3, 8, 2, 16, 3, 12, torch.float32, seed=2)
    O, L = oracle.decode(w.q, w.k_cache, w.v_cache, w.lens, w.scale)
    heads = [(0, 7), (2, 0), (1, 3)]
    Os, Ls = oracle.decode(w.q, w.k_cache, w.v_cache, w.lens, w.scale, heads=heads)
    for i, (b, h) in enumerate(heads):
        assert np.array_equal(Os[i], O[b, h, 0]) and Ls[i] == L[b, h]


# ---- closed forms -------------------------------------------------------------------

def test_zero_query_gives_uniform_weights():
    r = _rng(1)
    B, H, Tq, Tk, D = 2, 2, 3, 8, 5
    q = np.zeros((B, H, Tq, D))
    k = r.standard_normal((B, H, Tk, D))
    v = r.standard_normal((B, H, Tk, D))
    mask = np.zeros((B, Tk), np.uint8)
    mask[0, 5:] = 1
    mask[1, [0, 2, 3]] = 1
    O, L = oracle.attention(q, k, v, mask, 0.9)
    for b in range(B):
        valid = mask[b] == 0
        n = int(valid.sum())
        for h in range(H):
            expect = v[b, h, valid].mean(axis=0)
            assert np.allclose(O[b, h], expect[None, :], atol=1e-14, rtol=0)
            assert np.allclose(L[b, h], math.log(n), atol=1e-14, rtol=0)


def test_zero_keys_give_uniform_weights():
    r = _rng(2)
    q = r.standard_normal((1, 1, 4, 6))
    k = np.zeros((1, 1, 7, 6))
    v = r.standard_normal((1, 1, 7, 6))
    O, L = oracle.attention(q, k, v, None, 0.3)
    assert np.allclose(O[0, 0], v[0, 0].mean(axis=0)[None], atol=1e-14, rtol=0)
    assert np.allclose(L, math.log(7), atol=1e-14, rtol=0)


def test_single_valid_key():
    r = _rng(3)
    q = r.standard_normal((1, 2, 3, 4))
    k = r.standard_normal((1, 2, 6, 4))
    v = r.standard_normal((1, 2, 6, 4))
    mask = np.ones((1, 6), np.uint8)
    mask[0, 4] = 0
    s = 0.6
    O, L = oracle.attention(q, k, v, mask, s)
    for h in range(2):
        for i in range(3):
            assert np.array_equal(O[0, h, i], v[0, h, 4])
            assert abs(L[0, h, i] - s * float(q[0, h, i] @ k[0, h, 4])) <= 1e-14


def test_constant_values_pass_through():
    r = _rng(4)
    q = r.standard_normal((1, 1, 5, 3))
    k = r.standard_normal((1, 1, 9, 3))
    c = np.array([0.25, -1.5, 3.0])
    v = np.broadcast_to(c, (1, 1, 9, 3)).copy()
    O, _ = oracle.attention(q, k, v, (r.random((1, 9)) < 0.3).astype(np.uint8), 1.0)
    assert np.allclose(O[0, 0], c[None], atol=1e-14, rtol=0)


def test_single_key():
    r = _rng(5)
    q = r.standard_normal((1, 1, 4, 3))
    k = r.standard_normal((1, 1, 1, 3))
    v = r.standard_normal((1, 1, 1, 3))
    O, L = oracle.attention(q, k, v, None, 0.5)
    assert np.array_equal(O[0, 0], np.repeat(v[0, 0], 4, axis=0))
    assert np.allclose(L[0, 0], 0.5 * (q[0, 0] @ k[0, 0, 0]), atol=1e-15, rtol=0)


def test_two_keys_logistic():
    # Two keys with score gap d: the weight of key 0 is the logistic function of d.
    q = np.array([[[[1.0, 0.0]]]])
    k = np.array([[[[2.0, 0.0], [0.5, 0.0]]]])
    v = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    s = 0.8
    O, L = oracle.attention(q, k, v, None, s)
    d = s * (2.0 - 0.5)
    w0 = 1.0 / (1.0 + math.exp(-d))
    assert abs(O[0, 0, 0, 0] - w0) < 1e-15 and abs(O[0, 0, 0, 1] - (1 - w0)) < 1e-15
    assert abs(L[0, 0, 0] - math.log(math.exp(s * 2.0) + math.exp(s * 0.5))) < 1e-14


def test_fully_padded_sequence():
    r = _rng(6)
    q, k, v = (r.standard_normal((2, 1, 3, 4)) for _ in range(3))
    mask = np.zeros((2, 3), np.uint8)
    mask[1] = 1
    O, L = oracle.attention(q, k, v, mask, 1.0)
    assert np.all(O[1] == 0) and np.all(L[1] == -np.inf)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L[0]))


# ---- invariants ----------------------------------------------------------------------

def test_softmax_rows_sum_to_one_and_padded_weight_zero():
    r = _rng(7)
    S = r.standard_normal((6, 11)) * 4
    padded = r.random(11) < 0.4
    padded[0] = False
    W, m, l = oracle.masked_softmax(S, padded)
    assert np.all(W[:, padded] == 0.0)
    assert np.max(np.abs(W.sum(axis=1) - 1.0)) <= 1e-12
    assert np.all(W >= 0)
    assert np.array_equal(m, np.where(padded[None], -np.inf, S).max(axis=1))


def test_garbage_in_padded_keys_is_ignored():
    w = workloads.make_prefill(2, 3, 7, 10, 8, torch.float32, valid=[6, 10], seed=8)
    O, L = oracle.attention(w.q, w.k, w.v, w.mask, w.scale)
    k = w.k.clone()
    v = w.v.clone()
    k[0, :, 6:] = 1e4
    v[0, :, 6:] = -7e3
    O2, L2 = oracle.attention(w.q, k, v, w.mask, w.scale)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_masked_equals_truncated():
    w = workloads.make_prefill(1, 2, 9, 12, 6, torch.float32, valid=[8], seed=9)
    O, L = oracle.attention(w.q, w.k, w.v, w.mask, w.scale)
    Ot, Lt = oracle.attention(w.q, w.k[:, :, :8], w.v[:, :, :8], None, w.scale)
    assert np.max(np.abs(O - Ot)) <= 1e-14 and np.max(np.abs(L - Lt)) <= 1e-14


def test_key_permutation_invariance():
    r = _rng(10)
    w = workloads.make_prefill(1, 2, 5, 9, 4, torch.float32,
                               mask=torch.tensor([[0, 1, 0, 0, 1, 0, 0, 0, 1]]), seed=10)
    perm = r.permutation(9)
    O, L = oracle.attention(w.q, w.k, w.v, w.mask, w.scale)
    Op, Lp = oracle.attention(w.q, w.k[:, :, perm], w.v[:, :, perm], w.mask[:, perm], w.scale)
    assert np.max(np.abs(O - Op)) <= 1e-13 and np.max(np.abs(L - Lp)) <= 1e-13


def test_mask_polarity_matters():
    w = workloads.make_prefill(1, 2, 16, 16, 8, torch.float32, valid=[10], seed=11)
    O, _ = oracle.attention(w.q, w.k, w.v, w.mask, w.scale)
    Oinv, _ = oracle.attention(w.q, w.k, w.v, 1 - w.mask, w.scale)
    assert np.max(np.abs(O - Oinv)) > 0.1


@pytest.mark.parametrize("splits", [[13], [5, 8], [1, 6, 6], [3, 3, 3, 4]])
def test_chunked_merge_equals_single_pass(splits):
    w = workloads.make_chunked(2, 2, 7, splits, 8, torch.float32, seed=12)
    parts = [oracle.attention(w.q, kc, vc, None, w.scale) for kc, vc in zip(w.k_chunks, w.v_chunks)]
    O, L = oracle.merge_lse([p[0] for p in parts], [p[1] for p in parts])
    k = torch.cat(w.k_chunks, dim=2)
    v = torch.cat(w.v_chunks, dim=2)
    Of, Lf = oracle.attention(w.q, k, v, None, w.scale)
    assert np.max(np.abs(O - Of)) <= 1e-13 and np.max(np.abs(L - Lf)) <= 1e-13


def test_merge_single_chunk_is_identity():
    r = _rng(13)
    o, l = r.standard_normal((4, 3, 5)), r.standard_normal((4, 3))
    O, L = oracle.merge_lse([o], [l])
    assert np.max(np.abs(O - o)) <= 1e-15 and np.max(np.abs(L - l)) <= 1e-15


def test_append_touches_only_slot_len():
    w = workloads.make_decode(3, 4, 2, 8, 2, 10, torch.float32, T_max=16, seed=14)
    kc, vc, lens = oracle.kv_append(w.k_cache.numpy(), w.v_cache.numpy(), w.lens.numpy(),
                                    w.k_new.numpy(), w.v_new.numpy())
    for b in range(3):
        t = int(w.lens[b])
        assert lens[b] == t + 1
        assert np.array_equal(kc[b, :, t], w.k_new[b, :, 0].numpy())
        assert np.array_equal(vc[b, :, t], w.v_new[b, :, 0].numpy())
        keep = [i for i in range(16) if i != t]
        assert np.array_equal(kc[b][:, keep], w.k_cache.numpy()[b][:, keep])
        assert np.array_equal(vc[b][:, keep], w.v_cache.numpy()[b][:, keep])


def test_decode_equals_full_attention_over_cache_prefix():
    w = workloads.make_decode(3, 6, 2, 8, 4, 20, torch.float32, seed=15)
    kc, vc, lens = oracle.kv_append(w.k_cache.numpy(), w.v_cache.numpy(), w.lens.numpy(),
                                    w.k_new.numpy(), w.v_new.numpy())
    O, L = oracle.decode(w.q, kc, vc, lens, w.scale)
    G = 3
    for b in range(3):
        n = int(lens[b])
        k = np.repeat(kc[b:b + 1, :, :n], G, axis=1)      # expand KV heads to query heads
        v = np.repeat(vc[b:b + 1, :, :n], G, axis=1)
        Of, Lf = oracle.attention(w.q[b:b + 1].numpy(), k, v, None, w.scale)
        assert np.max(np.abs(O[b] - Of[0])) <= 1e-14 and np.max(np.abs(L[b] - Lf[0, :, 0])) <= 1e-14


# ---- library cross-check ---------------------------------------------------------------

def test_oracle_matches_torch_sdpa_on_fp32_t512():
    """The pages compare the materialising MHA path against SDPA on the CPU and see
    them agree to ~5e-8 in fp32; the oracle must agree with SDPA (additive -inf
    mask) the same way.  Passing the key-padding mask as SDPA's boolean mask
    unconverted must give a large error."""
    w = workloads.fp32_masked_t512()
    O, L = oracle.attention(w.q, w.k, w.v, w.mask, w.scale)
    add = torch.zeros(1, 1, 1, 512)
    add[..., w.mask[0].bool()] = float("-inf")
    ref = torch.nn.functional.scaled_dot_product_attention(w.q, w.k, w.v, attn_mask=add, scale=w.scale)
    assert np.max(np.abs(O - ref.double().numpy())) < 2e-6
    wrong = torch.nn.functional.scaled_dot_product_attention(
        w.q, w.k, w.v, attn_mask=w.mask.bool()[:, None, None, :], scale=w.scale)
    assert np.max(np.abs(O - wrong.double().numpy())) > 0.5
    # LSE against torch's logsumexp over the masked scores
    s = (w.q.double() @ w.k.double().transpose(-1, -2)) * w.scale + add.double()
    assert np.max(np.abs(L - torch.logsumexp(s, dim=-1).numpy())) < 1e-12


# ---- page-printed figures ---------------------------------------------------------------

def _golden():
    with open(os.path.join(GOLDEN, "page_numbers.json")) as f:
        return json.load(f)


def test_score_matrix_bytes_page_figures():
    g = _golden()
    e = g["score_matrix_3mp_bf16"]
    nbytes = oracle.score_matrix_bytes(e["heads"], e["P"], e["elem_bytes"])
    assert nbytes == 4_317_806_592
    assert round(nbytes / 1e9, 2) == e["approx_GB"]
    assert 4 * nbytes / 1e9 == pytest.approx(18.02, rel=0.05)   # "about four of them"
    e = g["score_matrix_8mp_bf16"]
    # 30.75 GiB for one matrix pins P to about 32.1 thousand, consistent with "about 32k"
    P = math.sqrt(e["GiB"] * 2**30 / (e["heads"] * e["elem_bytes"]))
    assert abs(P - e["P_approx"]) / e["P_approx"] < 0.01
    e = g["cpu_theory_p1024_fp32"]
    assert oracle.score_matrix_bytes(e["heads"], e["P"], e["elem_bytes"]) == e["MiB"] * 2**20


def test_kv_bytes_page_figures():
    g = _golden()
    e = g["gqa_kv_bytes_per_token"]
    bpt = oracle.kv_bytes_per_token(e["layers"], e["H_kv"], e["D"], e["elem_bytes"])
    assert bpt == e["bytes"]
    assert bpt * g["gqa_kv_8k_sequence"]["tokens"] == g["gqa_kv_8k_sequence"]["GiB"] * 2**30
    e32 = g["gqa_kv_32x8k"]
    assert bpt * e32["tokens"] * e32["sequences"] == e32["GiB"] * 2**30
    assert oracle.kv_bytes_per_token(32, g["mha_vs_gqa_factor"]["H_kv_mha"], 128, 2) == \
        g["mha_vs_gqa_factor"]["bytes_per_token"]
    assert oracle.kv_bytes_per_token(32, g["mqa_factor"]["H_kv_mqa"], 128, 2) == g["mqa_factor"]["bytes_per_token"]
    # one layer of the same shape reads 4 KiB per cached token
    assert oracle.decode_kv_bytes([1, 2, 3], 8, 128, 2) == 6 * 4096


def test_attention_flops_count():
    # 4·D·H·Tq·n_valid: at the 3 MP workload (16 heads, P 11,616, 16 padded keys)
    assert oracle.attention_flops(16, 64, 11616, [11600]) == 4 * 64 * 16 * 11616 * 11600
    # brute count of multiply-adds in Q·Kᵀ and P·V on a tiny case
    H, D, Tq, n = 2, 3, 4, [5, 2]
    macs = sum(H * Tq * nv * D * 2 for nv in n)
    assert oracle.attention_flops(H, D, Tq, n) == 2 * macs


# ---- packed variable-length sequences --------------------------------------------

def _varlen_brute(q, k, v, cq, ck, scale):
    """Row by row over the packed layout with the pure-Python attend_row."""
    total_q, H, D = q.shape
    O = np.zeros((total_q, H, D))
    L = np.full((H, total_q), -np.inf)
    for b in range(len(cq) - 1):
        keys = range(ck[b], ck[b + 1])
        for i in range(cq[b], cq[b + 1]):
            for h in range(H):
                kk = [k[j, h].tolist() for j in keys]
                vv = [v[j, h].tolist() for j in keys]
                o, l = brute.attend_row(q[i, h].tolist(), kk, vv, [False] * len(kk), scale)
                if l != -math.inf:
                    O[i, h] = o
                L[h, i] = l
    return O, L


@pytest.mark.parametrize("lens", [([3], [4]), ([2, 0, 5], [3, 4, 0]), ([1, 4, 2, 3], [6, 1, 2, 5]),
                                  ([0, 0], [2, 3])])
def test_varlen_matches_brute_force(lens):
    lq, lk = lens
    r = _rng(sum(lq) * 7 + sum(lk))
    H, D = 2, 5
    cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q = r.standard_normal((cq[-1], H, D)) * 1.3
    k = r.standard_normal((ck[-1], H, D))
    v = r.standard_normal((ck[-1], H, D))
    scale = 0.7
    O, L = oracle.attention_varlen(q, k, v, cq, ck, scale)
    bO, bL = _varlen_brute(q, k, v, cq, ck, scale)
    assert np.array_equal(np.isneginf(L), np.isneginf(bL))
    live = ~np.isneginf(bL)
    assert np.max(np.abs(L[live] - bL[live]), initial=0.0) <= 1e-12
    assert np.max(np.abs(O - bO), initial=0.0) <= 1e-12


def test_varlen_empty_key_sequence_gives_zero_and_neg_inf():
    w = workloads.make_varlen([3, 2], [0, 4], 2, 8, torch.float32, seed=3)
    O, L = oracle.attention_varlen(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale)
    assert np.all(O[:3] == 0.0) and np.all(np.isneginf(L[:, :3]))
    assert np.all(np.isfinite(L[:, 3:]))


def test_varlen_sequences_do_not_see_each_other():
    w = workloads.make_varlen([4, 5, 3], [6, 2, 7], 2, 8, torch.float32, seed=4)
    O, L = oracle.attention_varlen(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale)
    k2, v2 = w.k.clone(), w.v.clone()
    k2[6:8] += 3.0                       # only sequence 1's keys and values change
    v2[6:8] -= 2.0
    O2, L2 = oracle.attention_varlen(w.q, k2, v2, w.cu_q, w.cu_k, w.scale)
    for s, e in ((0, 4), (9, 12)):
        assert np.array_equal(O[s:e], O2[s:e]) and np.array_equal(L[:, s:e], L2[:, s:e])
    assert not np.allclose(O[4:9], O2[4:9])


def test_varlen_equals_padded_masked_dense():
    # Scattering the packed sequences into [B, H, T, D] with trailing key padding is the
    # masked definition; the valid query rows must agree (padded queries are not packed).
    lq, lk = [5, 1, 7], [3, 8, 6]
    w = workloads.make_varlen(lq, lk, 3, 8, torch.float32, seed=5)
    O, L = oracle.attention_varlen(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale)
    B, H, D, Tq, Tk = 3, 3, 8, max(lq), max(lk)
    qd = torch.zeros(B, H, Tq, D)
    kd = torch.zeros(B, H, Tk, D)
    vd = torch.zeros(B, H, Tk, D)
    cq, ck = w.cu_q.tolist(), w.cu_k.tolist()
    for b in range(B):
        qd[b, :, :lq[b]] = w.q[cq[b]:cq[b + 1]].transpose(0, 1)
        kd[b, :, :lk[b]] = w.k[ck[b]:ck[b + 1]].transpose(0, 1)
        vd[b, :, :lk[b]] = w.v[ck[b]:ck[b + 1]].transpose(0, 1)
    Od, Ld = oracle.attention(qd, kd, vd, workloads.mask_from_valid_lengths(lk, Tk), w.scale)
    for b in range(B):
        assert np.allclose(O[cq[b]:cq[b + 1]], Od[b, :, :lq[b]].transpose(1, 0, 2), atol=1e-13, rtol=0)
        assert np.allclose(L[:, cq[b]:cq[b + 1]], Ld[b, :, :lq[b]], atol=1e-13, rtol=0)


# ---- paged KV cache -----------------------------------------------------------------

@pytest.mark.parametrize("seed", range(3))
def test_decode_paged_matches_brute_force(seed):
    # Pure-Python walk of the page table: token t of sequence b is row t % ps of page bt[b][t // ps].
    r = _rng(100 + seed)
    B, Hkv, G, D, ps = 2, 2, 2, 4, 3
    mp = 4
    n_pages = B * mp + 2
    kp = r.standard_normal((n_pages, Hkv, ps, D))
    vp = r.standard_normal((n_pages, Hkv, ps, D))
    bt = r.permutation(n_pages)[:B * mp].reshape(B, mp)
    lens = [int(x) for x in r.integers(0, mp * ps + 1, B)]
    q = r.standard_normal((B, Hkv * G, 1, D))
    scale = 0.6
    O, L = oracle.decode_paged(q, kp, vp, bt, lens, scale)
    for b in range(B):
        for h in range(Hkv * G):
            g = h // G
            keys = [kp[bt[b][t // ps], g, t % ps].tolist() for t in range(lens[b])]
            vals = [vp[bt[b][t // ps], g, t % ps].tolist() for t in range(lens[b])]
            o, l = brute.attend_row(q[b, h, 0].tolist(), keys, vals, [False] * len(keys), scale)
            if l == -math.inf:
                assert L[b, h] == -np.inf and np.all(O[b, h, 0] == 0)
            else:
                assert abs(L[b, h] - l) <= 1e-12
                assert np.max(np.abs(O[b, h, 0] - np.array(o))) <= 1e-12


def test_decode_paged_identity_table_equals_contiguous():
    # With pages laid out in order (page b*mp + i = tokens i*ps.. of sequence b) the pool is a
    # reshape of the contiguous cache, so the two definitions must agree exactly.
    d = workloads.make_decode(3, 4, 2, 8, 0, 60, torch.float32, seed=6)
    B, Hkv, T, D = d.k_cache.shape
    ps = 16
    mp = T // ps
    kp = d.k_cache.reshape(B, Hkv, mp, ps, D).permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv, ps, D)
    vp = d.v_cache.reshape(B, Hkv, mp, ps, D).permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv, ps, D)
    bt = np.arange(B * mp).reshape(B, mp)
    O, L = oracle.decode_paged(d.q, kp, vp, bt, d.lens, d.scale)
    Oc, Lc = oracle.decode(d.q, d.k_cache, d.v_cache, d.lens, d.scale)
    assert np.array_equal(O, Oc) and np.array_equal(L, Lc)


def test_decode_paged_relabelling_pages_changes_nothing():
    pg = workloads.to_paged(workloads.make_decode(2, 4, 2, 8, 10, 60, torch.float32, seed=7), 16)
    O, L = oracle.decode_paged(pg.dec.q, pg.k_pages, pg.v_pages, pg.block_table, pg.dec.lens, pg.dec.scale)
    n = pg.k_pages.shape[0]
    pi = torch.randperm(n, generator=torch.Generator().manual_seed(3))
    kp2, vp2 = torch.empty_like(pg.k_pages), torch.empty_like(pg.v_pages)
    kp2[pi] = pg.k_pages
    vp2[pi] = pg.v_pages
    bt2 = pi[pg.block_table.long()]
    O2, L2 = oracle.decode_paged(pg.dec.q, kp2, vp2, bt2, pg.dec.lens, pg.dec.scale)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_paged_append_then_decode_equals_contiguous():
    d = workloads.make_decode(3, 4, 2, 8, 0, 47, torch.float32, seed=8)
    pg = workloads.to_paged(d, 16)
    kp, vp, lens = oracle.kv_append_paged(pg.k_pages, pg.v_pages, pg.block_table, d.lens, d.k_new, d.v_new)
    kc, vc, lens_c = oracle.kv_append(d.k_cache, d.v_cache, d.lens, d.k_new, d.v_new)
    assert np.array_equal(lens, lens_c)
    O, L = oracle.decode_paged(d.q, kp, vp, pg.block_table, lens, d.scale)
    Oc, Lc = oracle.decode(d.q, kc, vc, lens_c, d.scale)
    assert np.array_equal(O, Oc) and np.array_equal(L, Lc)
    # exactly one row of one page per sequence changed
    diff = np.argwhere(np.any(kp != pg.k_pages.numpy(), axis=(1, 3)))
    want = sorted((int(pg.block_table[b, int(d.lens[b]) // 16]), int(d.lens[b]) % 16) for b in range(3))
    got = sorted({(int(p), int(r)) for p, _, r in np.argwhere(np.any(kp != pg.k_pages.numpy(), axis=3))})
    assert got == want and len(diff) <= 3 * 2


def test_decode_zero_length_has_no_keys():
    # len 0: the empty key set, O = 0 and LSE = -inf like a fully padded row (brute force agrees)
    d = workloads.make_decode(3, 4, 2, 8, 0, 5, torch.float32, lens=[0, 3, 0], seed=9)
    O, L = oracle.decode(d.q, d.k_cache, d.v_cache, d.lens, d.scale)
    o, l = brute.attend_row(d.q[0, 0, 0].tolist(), [], [], [], d.scale)
    assert l == -math.inf
    for b in (0, 2):
        assert np.all(O[b] == 0) and np.all(np.isneginf(L[b]))
    assert np.all(np.isfinite(L[1]))
    pg = workloads.to_paged(d, 16)
    Op, Lp = oracle.decode_paged(d.q, pg.k_pages, pg.v_pages, pg.block_table, d.lens, d.scale)
    assert np.array_equal(Op, O) and np.array_equal(Lp, L)


# ---- GQA + causal prefill ------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_prefill_gqa_causal_matches_brute_force(seed):
    r = _rng(200 + seed)
    B, Hkv, G = int(r.integers(1, 3)), int(r.integers(1, 3)), int(r.integers(1, 4))
    Tq, Tk, D = int(r.integers(1, 9)), int(r.integers(1, 9)), int(r.integers(1, 7))
    q = r.standard_normal((B, Hkv * G, Tq, D)) * 1.4
    k = r.standard_normal((B, Hkv, Tk, D))
    v = r.standard_normal((B, Hkv, Tk, D))
    mask = (r.random((B, Tk)) < 0.25).astype(np.uint8) if seed % 2 else None
    causal = seed != 4
    scale = float(r.uniform(0.3, 1.2))
    O, L = oracle.prefill(q, k, v, mask, causal, scale)
    off = Tk - Tq
    for b in range(B):
        for h in range(Hkv * G):
            g = h // G
            for i in range(Tq):
                pad = [(mask is not None and mask[b, j] != 0) or (causal and j > i + off) for j in range(Tk)]
                o, l = brute.attend_row(q[b, h, i].tolist(), k[b, g].tolist(), v[b, g].tolist(), pad, scale)
                if l == -math.inf:
                    assert L[b, h, i] == -np.inf and np.all(O[b, h, i] == 0)
                else:
                    assert abs(L[b, h, i] - l) <= 1e-12
                    assert np.max(np.abs(O[b, h, i] - np.array(o))) <= 1e-12


def test_prefill_single_query_causal_is_decode():
    # the last position sees every key: Tq = 1 causal prefill = the decode step over the cache
    d = workloads.make_decode(3, 8, 2, 16, 5, 40, torch.float32, seed=10)
    n = int(d.lens.max())
    kc, vc = d.k_cache[:, :, :n], d.v_cache[:, :, :n]
    for b in range(3):
        lb = int(d.lens[b])
        Op, Lp = oracle.prefill(d.q[b:b + 1], kc[b:b + 1, :, :lb], vc[b:b + 1, :, :lb], None, True, d.scale)
        Od, Ld = oracle.decode(d.q[b:b + 1], kc[b:b + 1], vc[b:b + 1], d.lens[b:b + 1], d.scale)
        assert np.allclose(Op, Od, atol=1e-13, rtol=0) and np.allclose(Lp[..., 0], Ld, atol=1e-13, rtol=0)


def test_prefill_causal_row_is_attention_over_its_prefix():
    w = workloads.make_prefill(1, 2, 6, 9, 8, torch.float32, seed=11)
    O, L = oracle.prefill(w.q, w.k, w.v, None, True, w.scale)
    for i in range(6):
        n = i + 3 + 1                      # keys 0 .. i + (Tk - Tq)
        Oi, Li = oracle.attention(w.q[:, :, i:i + 1], w.k[:, :, :n], w.v[:, :, :n], None, w.scale)
        assert np.allclose(O[:, :, i:i + 1], Oi, atol=1e-13, rtol=0)
        assert np.allclose(L[:, :, i:i + 1], Li, atol=1e-13, rtol=0)


def test_prefill_gqa_equals_mha_on_repeated_kv_and_g1_is_attention():
    w = workloads.make_prefill(2, 2, 7, 11, 8, torch.float32, valid=[11, 6], seed=12)
    q6 = torch.cat([w.q, w.q * 0.5, -w.q], dim=1)          # 6 query heads over 2 KV heads
    O, L = oracle.prefill(q6, w.k, w.v, w.mask, False, w.scale)
    kr, vr = w.k.repeat_interleave(3, dim=1), w.v.repeat_interleave(3, dim=1)
    Om, Lm = oracle.attention(q6, kr, vr, w.mask, w.scale)
    assert np.allclose(O, Om, atol=1e-13, rtol=0) and np.allclose(L, Lm, atol=1e-13, rtol=0)
    O1, L1 = oracle.prefill(w.q, w.k, w.v, w.mask, False, w.scale)
    Oa, La = oracle.attention(w.q, w.k, w.v, w.mask, w.scale)
    assert np.array_equal(O1, Oa) and np.array_equal(L1, La)


def test_prefill_causal_rows_before_the_keys_are_empty():
    # Tq > Tk: queries i < Tq - Tk precede every key, so they attend nothing
    w = workloads.make_prefill(1, 1, 7, 4, 8, torch.float32, seed=13)
    O, L = oracle.prefill(w.q, w.k, w.v, None, True, w.scale)
    assert np.all(np.isneginf(L[0, 0, :3])) and np.all(O[0, 0, :3] == 0)
    assert np.all(np.isfinite(L[0, 0, 3:]))


def test_prefill_varlen_causal_gqa_matches_brute_force():
    r = _rng(14)
    lq, lk = [3, 0, 5, 2], [3, 4, 2, 6]
    Hkv, G, D = 2, 2, 4
    cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q = r.standard_normal((cq[-1], Hkv * G, D))
    k = r.standard_normal((ck[-1], Hkv, D))
    v = r.standard_normal((ck[-1], Hkv, D))
    O, L = oracle.prefill_varlen(q, k, v, cq, ck, True, 0.8)
    for b in range(4):
        off = lk[b] - lq[b]
        for i in range(lq[b]):
            for h in range(Hkv * G):
                keys = list(range(ck[b], ck[b + 1]))
                pad = [j - ck[b] > i + off for j in keys]
                o, l = brute.attend_row(q[cq[b] + i, h].tolist(), [k[j, h // G].tolist() for j in keys],
                                        [v[j, h // G].tolist() for j in keys], pad, 0.8)
                row = cq[b] + i
                if l == -math.inf:
                    assert L[h, row] == -np.inf and np.all(O[row, h] == 0)
                else:
                    assert abs(L[h, row] - l) <= 1e-12 and np.max(np.abs(O[row, h] - np.array(o))) <= 1e-12


# ---- FP8 (E4M3) key/value cache ---------------------------------------------------------

def test_e4m3_table_known_codes_and_library():
    v = oracle.e4m3_values()
    # format definition: 1.0 = 0 0111 000, 448 = 0 1111 110, smallest subnormal 2^-9, NaN codes
    assert v[0x38] == 1.0 and v[0x7E] == 448.0 and v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6
    assert v[0xBE] == -1.75 and v[0xC6] == -3.5 and np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert v[0x00] == 0.0 and v[0x80] == 0.0 and np.signbit(v[0x80])
    assert np.nanmax(np.abs(v)) == oracle.E4M3_MAX
    # library cross-check: torch's float8_e4m3fn decoding
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(v), np.isnan(t)) and np.array_equal(v[~np.isnan(v)], t[~np.isnan(t)])


def test_quantize_e4m3_rounding_saturation_and_library():
    q = oracle.quantize_e4m3
    one = np.float32(1.0)
    # ties to the even mantissa: 1 + 1/16 lies halfway between 1 and 1.125
    assert q(np.float32(1.0625), one) == 0x38 and q(np.float32(1.1875), one) == 0x3A
    assert q(np.float32(-1.0625), one) == 0xB8
    # saturation at 448 (never the NaN code); halfway to the subnormal step rounds to even (0)
    assert q(np.float32(1e6), one) == 0x7E and q(np.float32(-1e6), one) == 0xFE
    assert q(np.float32(2.0 ** -10), one) == 0x00 and q(np.float32(3 * 2.0 ** -11), one) == 0x01
    # the scale divides: x = 3.5 * s quantises to 3.5
    s = np.float32(0.0371)
    assert q(np.float32(3.5) * s, s) == 0x46 or oracle.e4m3_values()[q(np.float32(3.5) * s, s)] == 3.5
    # every finite code survives a round trip through its value times a power-of-two scale
    v = oracle.e4m3_values()
    codes = np.array([c for c in range(256) if not np.isnan(v[c]) and c != 0x80], dtype=np.uint8)
    assert np.array_equal(q(v[codes] * 4.0, np.float32(4.0)), codes)
    # library cross-check on random values: torch's float8 cast of the clamped quotient
    x = np.random.default_rng(3).standard_normal(50000).astype(np.float32) * 300
    s = np.float32(0.77)
    ref = torch.from_numpy(np.clip(x / s, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q(x, s), ref)


def test_decode_fp8kv_is_decode_of_dequantised_cache_and_brute_force():
    r = _rng(21)
    B, Hkv, G, D, T = 2, 2, 2, 4, 9
    k8 = r.integers(0, 256, (B, Hkv, T, D)).astype(np.uint8)
    v8 = r.integers(0, 256, (B, Hkv, T, D)).astype(np.uint8)
    vals = oracle.e4m3_values()
    k8[np.isnan(vals[k8])] = 0x38                       # no NaN codes in a cache
    v8[np.isnan(vals[v8])] = 0x30
    ks = r.uniform(0.01, 0.1, (B, Hkv))
    vs = r.uniform(0.5, 2.0, (B, Hkv))
    q = r.standard_normal((B, Hkv * G, 1, D))
    lens = [7, 0]
    O, L = oracle.decode_fp8kv(q, k8, v8, ks, vs, lens, 0.9)
    for b in range(B):
        for h in range(Hkv * G):
            g = h // G
            keys = [[vals[k8[b, g, t, d]] * ks[b, g] for d in range(D)] for t in range(lens[b])]
            vv = [[vals[v8[b, g, t, d]] * vs[b, g] for d in range(D)] for t in range(lens[b])]
            o, l = brute.attend_row(q[b, h, 0].tolist(), keys, vv, [False] * len(keys), 0.9)
            if l == -math.inf:
                assert L[b, h] == -np.inf and np.all(O[b, h, 0] == 0)
            else:
                assert abs(L[b, h] - l) <= 1e-12 and np.max(np.abs(O[b, h, 0] - np.array(o))) <= 1e-12


def test_kv_append_fp8_writes_only_the_quantised_slot():
    r = _rng(22)
    B, Hkv, T, D = 3, 2, 8, 8
    kc = r.integers(0, 0x70, (B, Hkv, T, D)).astype(np.uint8)
    vc = r.integers(0, 0x70, (B, Hkv, T, D)).astype(np.uint8)
    ks = r.uniform(0.05, 0.2, (B, Hkv)).astype(np.float32)
    vs = r.uniform(0.05, 0.2, (B, Hkv)).astype(np.float32)
    kn = r.standard_normal((B, Hkv, 1, D)).astype(np.float32)
    vn = r.standard_normal((B, Hkv, 1, D)).astype(np.float32)
    lens = np.array([0, 5, 7])
    kc2, vc2, l2 = oracle.kv_append_fp8(kc, vc, ks, vs, lens, kn, vn)
    assert l2.tolist() == [1, 6, 8]
    for b in range(B):
        t = lens[b]
        assert np.array_equal(kc2[b, :, t], oracle.quantize_e4m3(kn[b, :, 0], ks[b][:, None]))
        assert np.array_equal(vc2[b, :, t], oracle.quantize_e4m3(vn[b, :, 0], vs[b][:, None]))
        other = [i for i in range(T) if i != t]
        assert np.array_equal(kc2[b, :, other], kc[b, :, other]) and np.array_equal(vc2[b, :, other], vc[b, :, other])


# ---- FP8 prefill with LSE ---------------------------------------------------------------

def _e4m3_codes(r, shape):
    c = r.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C                         # no NaN codes in an input
    return c


def _torch_e4m3(c):
    """Values of E4M3 codes by torch's float8_e4m3fn decoding (independent of the oracle's table)."""
    return torch.from_numpy(np.ascontiguousarray(c)).view(torch.float8_e4m3fn).double().numpy()


@pytest.mark.parametrize("seed", range(4))
def test_prefill_fp8_matches_brute_force(seed):
    r = _rng(300 + seed)
    B, Hkv, G = int(r.integers(1, 3)), int(r.integers(1, 3)), int(r.integers(1, 3))
    Tq, Tk, D = int(r.integers(1, 7)), int(r.integers(1, 8)), int(r.integers(1, 6))
    q8 = _e4m3_codes(r, (B, Hkv * G, Tq, D))
    k8 = _e4m3_codes(r, (B, Hkv, Tk, D))
    v8 = _e4m3_codes(r, (B, Hkv, Tk, D))
    qs = r.uniform(2 ** -8, 2 ** -5, (B, Hkv * G))
    ks = r.uniform(2 ** -8, 2 ** -5, (B, Hkv))
    vs = r.uniform(0.5, 2.0, (B, Hkv))
    mask = (r.random((B, Tk)) < 0.3).astype(np.uint8) if seed % 2 else None
    causal = seed >= 2
    scale = float(r.uniform(0.3, 1.2))
    O, L = oracle.prefill_fp8(q8, k8, v8, qs, ks, vs, mask, causal, scale)
    qv, kv, vv = _torch_e4m3(q8), _torch_e4m3(k8), _torch_e4m3(v8)
    off = Tk - Tq
    for b in range(B):
        for h in range(Hkv * G):
            g = h // G
            keys = [[kv[b, g, t, d] * ks[b, g] for d in range(D)] for t in range(Tk)]
            vals = [[vv[b, g, t, d] * vs[b, g] for d in range(D)] for t in range(Tk)]
            for i in range(Tq):
                qrow = [qv[b, h, i, d] * qs[b, h] for d in range(D)]
                pad = [(mask is not None and mask[b, j] != 0) or (causal and j > i + off) for j in range(Tk)]
                o, l = brute.attend_row(qrow, keys, vals, pad, scale)
                if l == -math.inf:
                    assert L[b, h, i] == -np.inf and np.all(O[b, h, i] == 0)
                else:
                    assert abs(L[b, h, i] - l) <= 1e-12
                    assert np.max(np.abs(O[b, h, i] - np.array(o))) <= 1e-12


def test_prefill_fp8_scale_roles():
    # the Q and K scales only multiply the scores (a factor on `scale`); the V scale only
    # multiplies O (the LSE ignores it): a swapped or dropped scale fails one of these
    r = _rng(310)
    B, Hkv, G, T, D = 2, 2, 2, 9, 8
    q8, k8, v8 = _e4m3_codes(r, (B, Hkv * G, T, D)), _e4m3_codes(r, (B, Hkv, T, D)), _e4m3_codes(r, (B, Hkv, T, D))
    ones_q, ones_kv = np.ones((B, Hkv * G)), np.ones((B, Hkv))
    O1, L1 = oracle.prefill_fp8(q8, k8, v8, ones_q, ones_kv, ones_kv, None, False, 0.01)
    O2, L2 = oracle.prefill_fp8(q8, k8, v8, ones_q * 0.5, ones_kv * 0.25, ones_kv * 3.0, None, False, 0.08)
    np.testing.assert_allclose(L2, L1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(O2, 3.0 * O1, rtol=1e-12, atol=1e-12)
    # per-head scales act on their own head only
    qs = ones_q.copy()
    qs[1, 3] = 2.0
    O3, L3 = oracle.prefill_fp8(q8, k8, v8, qs, ones_kv, ones_kv, None, False, 0.01)
    O4, L4 = oracle.prefill_fp8(q8, k8, v8, ones_q, ones_kv, ones_kv, None, False, 0.02)
    np.testing.assert_allclose(O3[1, 3], O4[1, 3], atol=1e-12)
    np.testing.assert_allclose(L3[1, 3], L4[1, 3], atol=1e-12)
    keep = np.ones((B, Hkv * G), bool)
    keep[1, 3] = False
    assert np.array_equal(O3[keep], O1[keep]) and np.array_equal(L3[keep], L1[keep])


# ---- INT8 KV cache ------------------------------------------------------------------------

def test_quantize_int8_ties_saturation_and_library():
    q = oracle.quantize_int8
    s = np.float32(1.0)
    vals = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 127.4, 127.5, 300.0, -300.0, 0.49999997,
                     -0.0, 3.0, -126.5], dtype=np.float32)
    assert q(vals, s).tolist() == [0, 2, 2, 0, -2, -2, 126, 127, 127, 127, -127, 0, 0, 3, -126]
    # every code round-trips through a power-of-two scale (exact products)
    codes = np.arange(-127, 128).astype(np.int8)
    assert np.array_equal(q(oracle.dequantize_int8(codes, 0.125), np.float32(0.125)), codes)
    # library cross-check: torch.round rounds half to even, on the float32 quotient
    x = np.random.default_rng(4).standard_normal(50000).astype(np.float32) * 90
    sc = np.float32(0.61)
    ref = torch.round(torch.from_numpy(x) / torch.tensor(sc)).clamp(-127, 127).to(torch.int8).numpy()
    assert np.array_equal(q(x, sc), ref)


def test_decode_int8kv_is_decode_of_dequantised_cache_and_brute_force():
    r = _rng(23)
    B, Hkv, G, D, T = 2, 2, 3, 4, 10
    k8 = r.integers(-128, 128, (B, Hkv, T, D)).astype(np.int8)
    v8 = r.integers(-128, 128, (B, Hkv, T, D)).astype(np.int8)
    ks = r.uniform(0.002, 0.02, (B, Hkv))
    vs = r.uniform(0.005, 0.05, (B, Hkv))
    q = r.standard_normal((B, Hkv * G, 1, D))
    lens = [0, 9]
    O, L = oracle.decode_int8kv(q, k8, v8, ks, vs, lens, 0.7)
    for b in range(B):
        for h in range(Hkv * G):
            g = h // G
            keys = [[int(k8[b, g, t, d]) * ks[b, g] for d in range(D)] for t in range(lens[b])]
            vv = [[int(v8[b, g, t, d]) * vs[b, g] for d in range(D)] for t in range(lens[b])]
            o, l = brute.attend_row(q[b, h, 0].tolist(), keys, vv, [False] * len(keys), 0.7)
            if l == -math.inf:
                assert L[b, h] == -np.inf and np.all(O[b, h, 0] == 0)
            else:
                assert abs(L[b, h] - l) <= 1e-12 and np.max(np.abs(O[b, h, 0] - np.array(o))) <= 1e-12


def test_kv_append_int8_writes_only_the_quantised_slot():
    r = _rng(24)
    B, Hkv, T, D = 3, 2, 8, 8
    kc = r.integers(-128, 128, (B, Hkv, T, D)).astype(np.int8)
    vc = r.integers(-128, 128, (B, Hkv, T, D)).astype(np.int8)
    ks = r.uniform(0.01, 0.05, (B, Hkv)).astype(np.float32)
    vs = r.uniform(0.01, 0.05, (B, Hkv)).astype(np.float32)
    kn = r.standard_normal((B, Hkv, 1, D)).astype(np.float32)
    vn = r.standard_normal((B, Hkv, 1, D)).astype(np.float32)
    lens = np.array([0, 5, 7])
    kc2, vc2, l2 = oracle.kv_append_int8(kc, vc, ks, vs, lens, kn, vn)
    assert l2.tolist() == [1, 6, 8]
    for b in range(B):
        t = lens[b]
        # written codes: within half a step of x, x clamped to the +-127 steps
        for c2, xn, sc in ((kc2, kn, ks), (vc2, vn, vs)):
            lim = 127.0 * sc[b][:, None].astype(np.float64)
            err = np.abs(c2[b, :, t].astype(np.float64) * sc[b][:, None] - np.clip(xn[b, :, 0], -lim, lim))
            assert np.all(err <= sc[b][:, None] * 0.5 + 1e-7)
        other = [i for i in range(T) if i != t]
        assert np.array_equal(kc2[b, :, other], kc[b, :, other]) and np.array_equal(vc2[b, :, other], vc[b, :, other])


def test_prefill_varlen_fp8_equals_dense_per_sequence():
    # each packed sequence equals the dense FP8 prefill of that sequence alone (its own scales)
    r = _rng(320)
    lq, lk = [5, 0, 7, 3], [6, 4, 7, 0]
    Hkv, G, D = 2, 2, 8
    cq, ck = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q8 = _e4m3_codes(r, (cq[-1], Hkv * G, D))
    k8, v8 = _e4m3_codes(r, (ck[-1], Hkv, D)), _e4m3_codes(r, (ck[-1], Hkv, D))
    qs, ks, vs = r.uniform(0.01, 0.1, (4, Hkv * G)), r.uniform(0.01, 0.1, (4, Hkv)), r.uniform(0.5, 2, (4, Hkv))
    for causal in (False, True):
        O, L = oracle.prefill_varlen_fp8(q8, k8, v8, qs, ks, vs, cq, ck, causal, 0.6)
        for b in range(4):
            if lq[b] == 0:
                continue
            tq = q8[cq[b]:cq[b + 1]].transpose(1, 0, 2)[None]
            tk, tv = k8[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None], v8[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None]
            Od, Ld = oracle.prefill_fp8(tq, tk, tv, qs[b:b + 1], ks[b:b + 1], vs[b:b + 1], None, causal, 0.6)
            assert np.allclose(O[cq[b]:cq[b + 1]], Od[0].transpose(1, 0, 2), atol=1e-12, rtol=0)
            Lv = L[:, cq[b]:cq[b + 1]]
            assert np.array_equal(np.isneginf(Lv), np.isneginf(Ld[0]))
            assert np.allclose(Lv[np.isfinite(Lv)], Ld[0][np.isfinite(Ld[0])], atol=1e-12, rtol=0)
        # a sequence's scales touch that sequence only
        qs2 = qs.copy()
        qs2[2] *= 3
        O2, L2 = oracle.prefill_varlen_fp8(q8, k8, v8, qs2, ks, vs, cq, ck, causal, 0.6)
        other = np.r_[0:cq[2], cq[3]:cq[-1]]
        assert np.array_equal(O2[other], O[other]) and not np.allclose(O2[cq[2]:cq[3]], O[cq[2]:cq[3]])


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_paged_8bit_equals_contiguous(fmt):
    # the paged 8-bit append + decode equal the contiguous ones on the same codes, through an
    # identity table and through shuffled physical pages (a relabelling changes nothing)
    r = _rng(330)
    B, Hkv, G, D, ps, mp = 3, 2, 2, 8, 4, 5
    T = ps * mp
    if fmt == "fp8":
        codes = lambda shp: _e4m3_codes(r, shp)
        append, decode = oracle.kv_append_fp8, oracle.decode_fp8kv
        append_p, decode_p = oracle.kv_append_fp8_paged, oracle.decode_fp8kv_paged
    else:
        codes = lambda shp: r.integers(-128, 128, shp).astype(np.int8)
        append, decode = oracle.kv_append_int8, oracle.decode_int8kv
        append_p, decode_p = oracle.kv_append_int8_paged, oracle.decode_int8kv_paged
    kc, vc = codes((B, Hkv, T, D)), codes((B, Hkv, T, D))
    ks, vs = r.uniform(0.01, 0.1, (B, Hkv)).astype(np.float32), r.uniform(0.01, 0.1, (B, Hkv)).astype(np.float32)
    kn, vn = r.standard_normal((B, Hkv, 1, D)), r.standard_normal((B, Hkv, 1, D))
    lens = np.array([0, 7, T - 1])
    q = r.standard_normal((B, Hkv * G, 1, D))
    ek, ev, el = append(kc, vc, ks, vs, lens, kn, vn)
    O, L = decode(q, ek, ev, ks, vs, el, 0.5)
    for shuffle in (False, True):
        perm = r.permutation(B * mp + 2) if shuffle else np.arange(B * mp + 2)
        bt = perm[:B * mp].reshape(B, mp)
        kp, vp = codes((B * mp + 2, Hkv, ps, D)), codes((B * mp + 2, Hkv, ps, D))
        for b in range(B):
            for i in range(mp):
                kp[bt[b, i]] = kc[b, :, i * ps:(i + 1) * ps]
                vp[bt[b, i]] = vc[b, :, i * ps:(i + 1) * ps]
        kp2, vp2, el2 = append_p(kp, vp, ks, vs, bt, lens, kn, vn)
        assert el2.tolist() == el.tolist()
        for b in range(B):
            t = int(lens[b])
            assert np.array_equal(kp2[bt[b, t // ps], :, t % ps], ek[b, :, t])
            assert np.array_equal(vp2[bt[b, t // ps], :, t % ps], ev[b, :, t])
        Op, Lp = decode_p(q, kp2, vp2, ks, vs, bt, el2, 0.5)
        assert np.array_equal(Op, O) and np.array_equal(Lp, L)

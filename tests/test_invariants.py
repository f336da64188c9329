"""GPU invariants the pages fix, checked on the HIP path itself."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.test_parity import DEV, run_fwd

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_garbage_in_padded_keys_is_ignored_bitwise(ma, dtype):
    m = torch.zeros(2, 333, dtype=torch.uint8)
    m[0, 250:] = 1
    m[1, 10:70] = 1
    w = W.make_prefill(2, 2, 200, 333, 64, dtype, mask=m, seed=21)
    o, l = run_fwd(ma, w)
    k, v = w.k.clone(), w.v.clone()
    k[m.bool()[:, None, :, None].expand_as(k)] = 300.0
    v[m.bool()[:, None, :, None].expand_as(v)] = -1000.0
    w2 = W.Prefill(w.q, k, v, w.mask, w.scale)
    o2, l2 = run_fwd(ma, w2)
    assert torch.equal(o, o2) and torch.equal(l, l2)


def test_masked_equals_truncated(ma):
    w = W.make_prefill(1, 2, 150, 400, 64, torch.bfloat16, valid=[300], seed=22)
    o, l = run_fwd(ma, w)
    wt = W.Prefill(w.q, w.k[:, :, :300].contiguous(), w.v[:, :, :300].contiguous(), None, w.scale)
    ot, lt = run_fwd(ma, wt)
    assert (o.float() - ot.float()).abs().max().item() <= 2e-2
    assert (l - lt).abs().max().item() <= 1e-3


def test_mask_polarity_inverted_gives_large_difference(ma):
    w = W.make_prefill(1, 2, 128, 128, 64, torch.bfloat16, valid=[80], seed=23)
    o, _ = run_fwd(ma, w)
    winv = W.Prefill(w.q, w.k, w.v, (1 - w.mask).contiguous(), w.scale)
    oi, _ = run_fwd(ma, winv)
    assert (o.float() - oi.float()).abs().max().item() > 0.5


def test_bool_mask_equals_uint8_mask(ma):
    w = W.make_prefill(1, 2, 64, 100, 64, torch.bfloat16, valid=[77], seed=24)
    o, l = run_fwd(ma, w)
    ob, lb = ma.attn_fwd_lse(w.q.to(DEV), w.k.to(DEV), w.v.to(DEV), w.mask.bool().to(DEV), w.scale)
    assert torch.equal(o, ob) and torch.equal(l, lb)


def test_run_to_run_bitwise_determinism(ma):
    w = W.make_prefill(2, 3, 300, 500, 64, torch.bfloat16, valid=[500, 321], seed=25)
    a = run_fwd(ma, w)
    b = run_fwd(ma, w)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    d = W.make_decode(4, 8, 2, 128, 100, 2000, torch.bfloat16, seed=26)
    args = (d.q.to(DEV), d.k_cache.to(DEV), d.v_cache.to(DEV), d.lens.to(DEV), d.scale)
    r1 = ma.attn_decode(*args, want_lse=True)
    r2 = ma.attn_decode(*args, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1])


@pytest.mark.parametrize("G", [1, 4])
def test_decode_equals_prefill_over_cache_with_mask(ma, G):
    """Decode over len_b cached tokens equals the masked prefill kernel with Tq = 1
    and keys >= len_b padded (KV heads expanded to query heads for GQA)."""
    B, Hkv, D, Tm = 3, 2, 128, 640
    d = W.make_decode(B, Hkv * G, Hkv, D, 1, 600, torch.bfloat16, T_max=Tm, seed=27 + G)
    lens = d.lens.to(DEV)
    od, ld = ma.attn_decode(d.q.to(DEV), d.k_cache.to(DEV), d.v_cache.to(DEV), lens, d.scale, want_lse=True)
    k = d.k_cache.repeat_interleave(G, dim=1).contiguous().to(DEV)
    v = d.v_cache.repeat_interleave(G, dim=1).contiguous().to(DEV)
    mask = W.mask_from_valid_lengths(d.lens.tolist(), Tm).to(DEV)
    of, lf = ma.attn_fwd_lse(d.q.to(DEV), k, v, mask, d.scale)
    torch.cuda.synchronize()
    assert (od.float() - of.float()).abs().max().item() <= 2e-2
    assert (ld - lf[:, :, 0]).abs().max().item() <= 1e-3


def test_calls_allocate_no_device_memory(ma):
    """With outputs preallocated, a call leaves device free memory unchanged (the
    library has no allocation path; O(P) extra memory is exactly O + LSE)."""
    w = W.make_prefill(1, 16, 1944, 1944, 64, torch.bfloat16, valid=[1900], seed=28)
    q, k, v, m = (t.to(DEV) for t in (w.q, w.k, w.v, w.mask))
    o = torch.empty_like(q)
    l = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    ma.attn_fwd_lse(q, k, v, m, w.scale, out=o, lse=l)       # warm-up: code objects load
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    alloc0 = torch.cuda.memory_allocated()
    for _ in range(3):
        ma.attn_fwd_lse(q, k, v, m, w.scale, out=o, lse=l)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
    assert torch.cuda.memory_allocated() == alloc0

"""GPU parity at the full sizes of the measured workloads: every element of O and LSE
against the float64 oracle, in the launch configuration the benchmark times.

  * P = 11,616 patch self-attention (B1 H16 D64 bf16, last 16 keys padded): all 16 heads,
    all 11,616 rows each, in four groups of four heads (one GPU call shared by the groups).
  * Chunked KV (Q 8,192 x H24 x D128 against 2 x 8,192 keys): the merged result of two
    attn_fwd_lse calls and attn_merge_lse, and the single call over all 16,384 keys, both
    against the oracle over the concatenated keys, all 24 heads in six groups of four.
  * GQA decode (B32, 32 query / 8 KV heads, D128, len U[512, 8192] + 1): every (b, h) pair,
    after kv_append, for the bf16, E4M3, INT8 and 16-token paged caches.

The pages' own checks are whole-output ones: a max-abs difference over the full output,
free of NaN (molayo1419.me, "MultiheadAttention의 고속 경로가 VRAM을 18GB나 소모했던 이야기",
section "출력은 달라졌는가"), and the merged ring result against the single pass (sglang PR
49078 analysis, section "정확도").  Tolerances are the ones every parity test uses.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.test_parity import DEV, check_attn

pytestmark = pytest.mark.gpu

HEAD_GROUPS_16 = [(0, 4), (4, 8), (8, 12), (12, 16)]
HEAD_GROUPS_24 = [(0, 4), (4, 8), (8, 12), (12, 16), (16, 20), (20, 24)]


@pytest.fixture(scope="module")
def p11616(ma):
    w = W.patch_p11616()
    q, k, v, m = (t.to(DEV) for t in (w.q, w.k, w.v, w.mask))
    o, l = ma.attn_fwd_lse(q, k, v, m, w.scale)
    torch.cuda.synchronize()
    return w, o.cpu(), l.cpu()


@pytest.mark.parametrize("heads", HEAD_GROUPS_16)
def test_patch_p11616_every_row(p11616, heads):
    w, o, l = p11616
    h0, h1 = heads
    Or, Lr = oracle.attention(w.q[:, h0:h1], w.k[:, h0:h1], w.v[:, h0:h1], w.mask, w.scale)
    check_attn(o[:, h0:h1], l[:, h0:h1], Or, Lr, torch.bfloat16, f"P11616 heads {h0}..{h1 - 1}")


@pytest.fixture(scope="module")
def chunked(ma):
    w = W.chunked_kv_2x8192()
    q = w.q.to(DEV)
    parts = [ma.attn_fwd_lse(q, kc.to(DEV), vc.to(DEV), None, w.scale) for kc, vc in zip(w.k_chunks, w.v_chunks)]
    om, lm = ma.attn_merge_lse([p[0] for p in parts], [p[1] for p in parts])
    k = torch.cat(w.k_chunks, dim=2)
    v = torch.cat(w.v_chunks, dim=2)
    of, lf = ma.attn_fwd_lse(q, k.to(DEV), v.to(DEV), None, w.scale)
    torch.cuda.synchronize()
    return w, k, v, om.cpu(), lm.cpu(), of.cpu(), lf.cpu()


@pytest.mark.parametrize("heads", HEAD_GROUPS_24)
def test_chunked_kv_2x8192_every_row(chunked, heads):
    w, k, v, om, lm, of, lf = chunked
    h0, h1 = heads
    Or, Lr = oracle.attention(w.q[:, h0:h1], k[:, h0:h1], v[:, h0:h1], None, w.scale)
    check_attn(om[:, h0:h1], lm[:, h0:h1], Or, Lr, torch.bfloat16, f"chunked merged heads {h0}..{h1 - 1}")
    check_attn(of[:, h0:h1], lf[:, h0:h1], Or, Lr, torch.bfloat16, f"single pass heads {h0}..{h1 - 1}")


def test_gqa_decode_b32_every_head(ma):
    w = W.gqa_decode_b32()
    kc, vc, lens = w.k_cache.to(DEV), w.v_cache.to(DEV), w.lens.to(DEV)
    ma.kv_append(kc, vc, lens, w.k_new.to(DEV), w.v_new.to(DEV))
    o, l = ma.attn_decode(w.q.to(DEV), kc, vc, lens, w.scale, want_lse=True)
    torch.cuda.synchronize()
    ek, ev, el = oracle.kv_append(w.k_cache.float().numpy(), w.v_cache.float().numpy(), w.lens.numpy(),
                                  w.k_new.float().numpy(), w.v_new.float().numpy())
    assert lens.cpu().tolist() == el.tolist()
    assert torch.equal(kc.cpu(), torch.from_numpy(ek).to(torch.bfloat16))
    assert torch.equal(vc.cpu(), torch.from_numpy(ev).to(torch.bfloat16))
    Or, Lr = oracle.decode(w.q, ek, ev, el, w.scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, "B32 decode, every (b, h)")


def test_gqa_decode_b32_paged_every_head(ma):
    pg = W.gqa_decode_b32_paged(16)
    w = pg.dec
    kp, vp, bt = pg.k_pages.to(DEV), pg.v_pages.to(DEV), pg.block_table.to(DEV)
    lens = w.lens.to(DEV)
    ma.kv_append_paged(kp, vp, bt, lens, w.k_new.to(DEV), w.v_new.to(DEV))
    o, l = ma.attn_decode_paged(w.q.to(DEV), kp, vp, bt, lens, w.scale, want_lse=True)
    torch.cuda.synchronize()
    ek, ev, el = oracle.kv_append_paged(pg.k_pages.float().numpy(), pg.v_pages.float().numpy(),
                                        pg.block_table.numpy(), w.lens.numpy(), w.k_new.float().numpy(),
                                        w.v_new.float().numpy())
    assert lens.cpu().tolist() == el.tolist()
    Or, Lr = oracle.decode_paged(w.q, ek, ev, pg.block_table.numpy(), el, w.scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, "B32 paged decode, every (b, h)")


@pytest.mark.parametrize("fmt", ["fp8", "int8"])
def test_gqa_decode_b32_8bit_every_head(ma, fmt):
    w = W.gqa_decode_b32_fp8() if fmt == "fp8" else W.gqa_decode_b32_int8()
    append = ma.kv_append_fp8 if fmt == "fp8" else ma.kv_append_int8
    decode = ma.attn_decode_fp8kv if fmt == "fp8" else ma.attn_decode_int8kv
    kc, vc, ks, vs, lens = (t.to(DEV) for t in (w.k_cache, w.v_cache, w.k_scale, w.v_scale, w.lens))
    append(kc, vc, ks, vs, lens, w.k_new.to(DEV), w.v_new.to(DEV))
    o, l = decode(w.q.to(DEV), kc, vc, ks, vs, lens, w.scale, want_lse=True)
    torch.cuda.synchronize()
    oappend = oracle.kv_append_fp8 if fmt == "fp8" else oracle.kv_append_int8
    odecode = oracle.decode_fp8kv if fmt == "fp8" else oracle.decode_int8kv
    ek, ev, el = oappend(w.k_cache.numpy(), w.v_cache.numpy(), w.k_scale, w.v_scale, w.lens.numpy(),
                         w.k_new, w.v_new)
    assert lens.cpu().tolist() == el.tolist()
    assert np.array_equal(kc.cpu().numpy(), ek) and np.array_equal(vc.cpu().numpy(), ev)
    Or, Lr = odecode(w.q, ek, ev, w.k_scale, w.v_scale, el, w.scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, f"B32 {fmt} decode, every (b, h)")

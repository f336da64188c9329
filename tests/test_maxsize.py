"""GPU parity at the largest sizes the boundary accepts, where the 32-bit buffer ranges end.

The bf16 prefill addresses one (b, KV head)'s K and V through a 32-bit buffer range and the
boundary accepts Tk·D·2 bytes up to 2^31 - 1; the decode kernels do the same for one
(sequence, KV head) of the cache (T_max·D·2 bytes for bf16, T_max·D for the 8-bit caches).
The packed calls accept total_k·H_kv·D elements up to 2^30 - 1, with a sequence's rows strided
by H_kv·D.  At those sizes the kernels' per-lane tile offsets, look-ahead included, pass 2^31,
the last blocks sit at the very end of the range, and a sequence of the decode is cut into
~8,200 (bf16) or ~16,400 (E4M3) splits whose parts the combine merges over hundreds of rounds.

Inputs are seeded normal draws made on the GPU by the workload module (billions of values);
the same tensors are copied to the host for the oracle.  Every output row of the prefill and
the sampled query heads of the decodes are compared with the float64 oracle at the bars every
parity test uses.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.test_parity import DEV, check_attn

pytestmark = pytest.mark.gpu

D = 128
TK_MAX_BF16 = (2**31 - 1) // (D * 2)       # 8,388,607 keys or cached tokens
T_MAX_8BIT = (2**31 - 1) // D              # 16,777,215 cached tokens


def test_prefill_largest_key_range(ma):
    Tq, Tk = 40, TK_MAX_BF16
    q = W.randn_device((1, 1, Tq, D), 101, DEV)
    k = W.randn_device((1, 1, Tk, D), 102, DEV)
    v = W.randn_device((1, 1, Tk, D), 103, DEV)
    # padded: the first 100 keys, an interior hole a few tiles before the end (so the per-tile
    # flags are read at the largest offsets) and the last 37 keys
    mask = torch.zeros((1, Tk), dtype=torch.uint8)
    mask[0, :100] = 1
    mask[0, Tk - 5000:Tk - 4990] = 1
    mask[0, Tk - 37:] = 1
    scale = 1.0 / np.sqrt(D)
    o, l = ma.attn_fwd_lse(q, k, v, mask.to(DEV), scale)
    torch.cuda.synchronize()
    o, l = o.cpu(), l.cpu()
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    del q, k, v
    torch.cuda.empty_cache()
    Or, Lr = oracle.attention(qc, kc, vc, mask, scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, f"prefill Tq={Tq} Tk={Tk} D={D}")


def test_decode_largest_cache(ma):
    B, Hq, Hkv, T_max = 1, 4, 1, TK_MAX_BF16
    kc = W.randn_device((B, Hkv, T_max, D), 201, DEV)
    vc = W.randn_device((B, Hkv, T_max, D), 202, DEV)
    kn = W.randn_device((B, Hkv, 1, D), 203, DEV)
    vn = W.randn_device((B, Hkv, 1, D), 204, DEV)
    q = W.randn_device((B, Hq, 1, D), 205, DEV)
    lens0 = torch.tensor([T_max - 1], dtype=torch.int32)
    k_host, v_host = kc.cpu().float().numpy(), vc.cpu().float().numpy()     # the inputs, before the append
    lens = lens0.to(DEV)
    ma.kv_append(kc, vc, lens, kn, vn)
    scale = 1.0 / np.sqrt(D)
    o, l = ma.attn_decode(q, kc, vc, lens, scale, want_lse=True)
    torch.cuda.synchronize()
    assert lens.cpu().tolist() == [T_max]
    ek, ev, el = oracle.kv_append(k_host, v_host, lens0.numpy(), kn.cpu().float().numpy(),
                                  vn.cpu().float().numpy())
    del k_host, v_host
    # the append is a bit copy into the last slot: the whole cache must equal the oracle's
    assert torch.equal(kc[0, 0, -1].cpu(), torch.from_numpy(ek[0, 0, -1]).to(torch.bfloat16))
    assert torch.equal(vc[0, 0, -1].cpu(), torch.from_numpy(ev[0, 0, -1]).to(torch.bfloat16))
    assert torch.equal(kc.cpu(), torch.from_numpy(ek).to(torch.bfloat16))
    heads = [(0, 0), (0, 3)]
    Or, Lr = oracle.decode(q.cpu(), ek, ev, el, scale, heads=heads)
    o, l = o.cpu(), l.cpu()
    check_attn(torch.stack([o[b, h, 0] for b, h in heads]), torch.stack([l[b, h] for b, h in heads]),
               Or, Lr, torch.bfloat16, f"decode T_max={T_max} D={D}, heads {heads}")


def test_fp8_decode_largest_cache(ma):
    B, Hq, Hkv, T_max = 1, 4, 1, T_MAX_8BIT
    kc = W.randn_device((B, Hkv, T_max, D), 301, DEV, torch.float8_e4m3fn).view(torch.uint8)
    vc = W.randn_device((B, Hkv, T_max, D), 302, DEV, torch.float8_e4m3fn).view(torch.uint8)
    ks = torch.tensor([[0.75]], dtype=torch.float32)
    vs = torch.tensor([[1.5]], dtype=torch.float32)
    kn = W.randn_device((B, Hkv, 1, D), 303, DEV, amp=0.75)
    vn = W.randn_device((B, Hkv, 1, D), 304, DEV, amp=1.5)
    q = W.randn_device((B, Hq, 1, D), 305, DEV)
    lens0 = torch.tensor([T_max - 1], dtype=torch.int32)
    k_host, v_host = kc.cpu().numpy(), vc.cpu().numpy()
    lens = lens0.to(DEV)
    ma.kv_append_fp8(kc, vc, ks.to(DEV), vs.to(DEV), lens, kn, vn)
    scale = 1.0 / np.sqrt(D)
    o, l = ma.attn_decode_fp8kv(q, kc, vc, ks.to(DEV), vs.to(DEV), lens, scale, want_lse=True)
    torch.cuda.synchronize()
    assert lens.cpu().tolist() == [T_max]
    ek, ev, el = oracle.kv_append_fp8(k_host, v_host, ks, vs, lens0.numpy(), kn.cpu(), vn.cpu())
    del k_host, v_host
    assert np.array_equal(kc[0, 0, -1].cpu().numpy(), ek[0, 0, -1])
    assert np.array_equal(vc[0, 0, -1].cpu().numpy(), ev[0, 0, -1])
    heads = [(0, 1)]
    Or, Lr = oracle.decode_fp8kv(q.cpu(), ek, ev, ks, vs, el, scale, heads=heads)
    o, l = o.cpu(), l.cpu()
    check_attn(torch.stack([o[b, h, 0] for b, h in heads]), torch.stack([l[b, h] for b, h in heads]),
               Or, Lr, torch.bfloat16, f"E4M3 decode T_max={T_max} D={D}, heads {heads}")


def test_varlen_gqa_largest_packed_keys(ma):
    # packed K/V of total_k * H_kv * D elements, the largest the packed calls accept
    Hq, Hkv = 16, 8
    total_k = (2**30 - 1) // (Hkv * D)          # 1,048,575 rows of 8 KV heads
    lens_k = [total_k // 2, total_k - total_k // 2]
    lens_q = [24, 17]
    cu_q, cu_k = W.cu_from_lengths(lens_q), W.cu_from_lengths(lens_k)
    q = W.randn_device((sum(lens_q), Hq, D), 401, DEV)
    k = W.randn_device((total_k, Hkv, D), 402, DEV)
    v = W.randn_device((total_k, Hkv, D), 403, DEV)
    scale = 1.0 / np.sqrt(D)
    o, l = ma.attn_prefill_varlen(q, k, v, cu_q.to(DEV), cu_k.to(DEV), max(lens_q), True, scale)
    torch.cuda.synchronize()
    o, l = o.cpu(), l.cpu()
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    del q, k, v
    torch.cuda.empty_cache()
    Or, Lr = oracle.prefill_varlen(qc, kc, vc, cu_q, cu_k, True, scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, f"packed causal GQA prefill, total_k={total_k}")


def test_fp8_prefill_largest_key_range(ma):
    Hq, Hkv, Tq, Tk = 2, 1, 24, T_MAX_8BIT
    q = W.randn_device((1, Hq, Tq, D), 501, DEV, torch.float8_e4m3fn).view(torch.uint8)
    k = W.randn_device((1, Hkv, Tk, D), 502, DEV, torch.float8_e4m3fn).view(torch.uint8)
    v = W.randn_device((1, Hkv, Tk, D), 503, DEV, torch.float8_e4m3fn).view(torch.uint8)
    qs = torch.tensor([[0.5, 0.25]], dtype=torch.float32)
    ks = torch.tensor([[0.375]], dtype=torch.float32)
    vs = torch.tensor([[1.25]], dtype=torch.float32)
    mask = torch.zeros((1, Tk), dtype=torch.uint8)
    mask[0, :64] = 1
    mask[0, Tk - 100:] = 1
    scale = 1.0 / np.sqrt(D)
    o, l = ma.attn_prefill_fp8(q, k, v, qs.to(DEV), ks.to(DEV), vs.to(DEV), mask.to(DEV), False, scale)
    torch.cuda.synchronize()
    o, l = o.cpu(), l.cpu()
    qc, kc, vc = q.cpu().numpy(), k.cpu().numpy(), v.cpu().numpy()
    del q, k, v
    torch.cuda.empty_cache()
    Or, Lr = oracle.prefill_fp8(qc, kc, vc, qs, ks, vs, mask, False, scale)
    check_attn(o, l, Or, Lr, torch.bfloat16, f"E4M3 prefill Tk={Tk} D={D}")

"""attn_decode_noalloc (the decode for callers that cannot allocate: its partial results live
in the library's static device scratch) against attn_decode with a caller workspace: the same
kernels on the same inputs, so the outputs must be bit-identical.  Two calls in a row, the
second smaller than the first (the scratch keeps the first call's contents), each checked,
plus the oracle on the second."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.test_parity import DEV, check_attn

pytestmark = pytest.mark.gpu


def _decode_both(ma, w):
    kc, vc, lens = w.k_cache.to(DEV), w.v_cache.to(DEV), w.lens.to(DEV)
    ma.kv_append(kc, vc, lens, w.k_new.to(DEV), w.v_new.to(DEV))
    q = w.q.to(DEV)
    o_ref, l_ref = ma.attn_decode(q, kc, vc, lens, w.scale, want_lse=True)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[0], q.shape[1]), float("nan"), dtype=torch.float32, device=DEV)
    ma.attn_decode_noalloc(q, kc, vc, lens, o, lse, w.scale)
    torch.cuda.synchronize()
    return o_ref, l_ref, o, lse, kc, vc, lens


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_noalloc_equals_decode_twice(ma, dtype):
    big = W.make_decode(32, 32, 8, 128, 512, 8192, dtype, seed=11)          # the B32 decode workload shape
    small = W.make_decode(5, 8, 2, 64, 1, 700, dtype, T_max=768, seed=12)   # smaller: fewer, shorter items
    for w in (big, small):
        o_ref, l_ref, o, lse, kc, vc, lens = _decode_both(ma, w)
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), "noalloc differs from attn_decode"
    Or, Lr = oracle.decode(small.q, kc.cpu(), vc.cpu(), lens.cpu().numpy(), small.scale)
    check_attn(o, lse, Or, Lr, dtype, "noalloc decode, second call")


def test_decode_noalloc_rejects_oversize_before_enqueue(ma):
    # B·H_q·ceil(T_max/1024) beyond the static buffer: refused on the host, output untouched
    B, Hq, Hkv, D, Tm = 64, 64, 8, 128, 9216
    assert ma.attn_decode_workspace_bytes(B, Hq, Hkv, Tm, D) > ma.DECODE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(B, Hq, 1, D, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(B, Hkv, Tm, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    lens = torch.ones(B, dtype=torch.int32, device=DEV)
    o = torch.full_like(q, 7.0)
    with pytest.raises(ma.AttnError) as e:
        ma.attn_decode_noalloc(q, kc, vc, lens, o)
    assert e.value.status == 9
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)

"""Streams and HIP graphs: every call enqueues its kernels on the stream it is given and on
nothing else, and makes no allocation, copy or synchronisation, so the path can run on a
side stream and be captured into a graph (the allocation-free decode is the call meant for
that).  Results are compared bit for bit with eager calls on the default stream: every kernel
is deterministic.

A graph is replayed several times with eager work and device synchronisations between the
replays (its outputs are cleared by a fill kernel before each one), and every replay is
checked, since graph nodes of some kinds have misbehaved on replays after the first.
"""
import pytest
import torch

import workloads as W
from tests.test_parity import DEV

pytestmark = pytest.mark.gpu


def _inputs():
    pf = W.make_prefill(2, 4, 300, 700, 64, torch.bfloat16, valid=[700, 650], seed=5)
    ch = W.make_chunked(1, 3, 200, [256, 300], 128, seed=6)
    dc = W.make_decode(3, 8, 2, 128, 1, 2000, seed=7)
    dev = lambda t: t.to(DEV)
    d = {
        "q1": dev(pf.q), "k1": dev(pf.k), "v1": dev(pf.v), "m1": dev(pf.mask), "s1": pf.scale,
        "q2": dev(ch.q), "k2": [dev(t) for t in ch.k_chunks], "v2": [dev(t) for t in ch.v_chunks],
        "s2": ch.scale,
        "kc": dev(dc.k_cache), "vc": dev(dc.v_cache), "kn": dev(dc.k_new), "vn": dev(dc.v_new),
        "q3": dev(dc.q), "lens0": dev(dc.lens), "s3": dc.scale,
    }
    d["lens"] = d["lens0"].clone()
    return d


def _outputs(ma, d):
    q1, q2, q3 = d["q1"], d["q2"], d["q3"]
    B3, H3, _, D3 = q3.shape
    return {
        "o1": torch.empty_like(q1), "l1": torch.empty(q1.shape[:3], dtype=torch.float32, device=DEV),
        "o2": [torch.empty_like(q2) for _ in range(2)],
        "l2": [torch.empty(q2.shape[:3], dtype=torch.float32, device=DEV) for _ in range(2)],
        "om": torch.empty_like(q2), "lm": torch.empty(q2.shape[:3], dtype=torch.float32, device=DEV),
        "o3": torch.empty_like(q3), "l3": torch.empty((B3, H3), dtype=torch.float32, device=DEV),
        "o4": torch.empty_like(q3), "l4": torch.empty((B3, H3), dtype=torch.float32, device=DEV),
        "ws": torch.empty(ma.attn_decode_workspace_bytes(B3, H3, d["kc"].shape[1], d["kc"].shape[2], D3),
                          dtype=torch.uint8, device=DEV),
    }


def _path(ma, d, r):
    """The whole path on the current stream: prefill, chunked pair + merge, append + decode,
    and the allocation-free decode on the appended cache."""
    d["lens"].copy_(d["lens0"])
    ma.attn_fwd_lse(d["q1"], d["k1"], d["v1"], d["m1"], d["s1"], out=r["o1"], lse=r["l1"])
    for i in range(2):
        ma.attn_fwd_lse(d["q2"], d["k2"][i], d["v2"][i], None, d["s2"], out=r["o2"][i], lse=r["l2"][i])
    ma.attn_merge_lse(r["o2"], r["l2"], out=r["om"], lse_out=r["lm"])
    ma.kv_append(d["kc"], d["vc"], d["lens"], d["kn"], d["vn"])
    ma.attn_decode(d["q3"], d["kc"], d["vc"], d["lens"], d["s3"], out=r["o3"], lse=r["l3"],
                   workspace=r["ws"], want_lse=True)
    ma.attn_decode_noalloc(d["q3"], d["kc"], d["vc"], d["lens"], r["o4"], r["l4"], scale=d["s3"])


RESULTS = ("o1", "l1", "om", "lm", "o3", "l3", "o4", "l4")


def _snapshot(r):
    return {k: r[k].clone() for k in RESULTS}


def test_side_stream_matches_default_stream(ma):
    d = _inputs()
    ref = _outputs(ma, d)
    _path(ma, d, ref)
    torch.cuda.synchronize()
    want = _snapshot(ref)
    r = _outputs(ma, d)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _path(ma, d, r)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for k in RESULTS:
        assert torch.equal(r[k], want[k]), f"{k} differs on a side stream"
    # the allocation-free decode equals attn_decode bit for bit
    assert torch.equal(want["o3"], want["o4"]) and torch.equal(want["l3"], want["l4"])


def test_graph_capture_and_replays(ma):
    d = _inputs()
    r = _outputs(ma, d)
    _path(ma, d, r)                      # eager: one-time set-up of the library, and the reference
    torch.cuda.synchronize()
    want = _snapshot(r)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _path(ma, d, r)
    torch.cuda.synchronize()
    for rep in range(4):
        for k in RESULTS:
            r[k].fill_(float("nan") if r[k].is_floating_point() else 0)   # eager fill kernels
        ma.attn_fwd_lse(d["q1"], d["k1"], d["v1"], d["m1"], d["s1"])    # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in RESULTS:
            assert torch.equal(r[k], want[k]), f"replay {rep}: {k} differs from the eager call"
        assert torch.equal(d["lens"], d["lens0"] + 1)

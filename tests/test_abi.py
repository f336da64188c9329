"""The C ABI library loads, exports every symbol include/attn.h declares, and
rejects bad arguments on the host (before any HIP call, so these run without
a GPU: the pointers passed are never dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    import masked_attention_attn_amd as ma
    if not os.path.exists(ma.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return ma.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)))


def test_header_declares_the_five_calls():
    names = _declared()
    for n in ("attn_fwd_masked", "attn_fwd_lse", "attn_merge_lse", "kv_append", "attn_decode"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    import masked_attention_attn_amd as ma
    names = _declared()
    assert set(names) == set(ma.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


# Every HIP runtime routine the library may import: kernel registration and launch, error
# query, device and occupancy queries, the kernel LDS attribute, and the address of a
# file-scope device array.  No allocation, free, copy, memset or synchronisation.
ALLOWED_HIP_IMPORTS = {
    "__hipPopCallConfiguration", "__hipPushCallConfiguration", "__hipRegisterFatBinary",
    "__hipRegisterFunction", "__hipUnregisterFatBinary", "__hipRegisterVar", "hipDeviceGetAttribute",
    "hipFuncSetAttribute", "hipGetDevice", "hipGetLastError", "hipLaunchKernel",
    "hipOccupancyMaxActiveBlocksPerMultiprocessor", "hipGetSymbolAddress",
}


def test_library_imports_no_allocation_or_sync(lib):
    """The calls allocate no device memory and never synchronise: the shared library does not
    even import hipMalloc*, hipFree*, hipMemset*, hipMemcpy* or any synchronisation routine."""
    import shutil
    import subprocess
    import masked_attention_attn_amd as ma
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", ma.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    hip = {line.split()[-1].split("@")[0] for line in out.splitlines() if "hip" in line.lower()}
    assert hip, "expected HIP runtime imports"
    assert hip <= ALLOWED_HIP_IMPORTS, sorted(hip - ALLOWED_HIP_IMPORTS)
    assert not any(("alloc" in n.lower() or "free" in n.lower() or "sync" in n.lower()) for n in hip)


def test_status_strings(lib):
    for code in range(10):
        s = lib.attn_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.attn_status_string(99).decode() == "unknown status"


A = 0x10000      # fake, 16-byte aligned device addresses (never dereferenced)
B_ = 0x20000
C = 0x30000
O = 0x40000
L = 0x50000


def fwd(lib, q=A, k=B_, v=C, m=0, o=O, B=1, H=2, Tq=8, Tk=8, D=64, scale=0.125, dtype=1):
    return lib.attn_fwd_masked(q, k, v, m, o, B, H, Tq, Tk, D, scale, dtype, None)


def test_fwd_validation(lib):
    assert fwd(lib, q=0) == 1
    assert fwd(lib, o=0) == 1
    assert fwd(lib, D=96) == 3
    assert fwd(lib, D=32) == 3
    assert fwd(lib, dtype=7) == 3
    assert fwd(lib, B=0) == 2
    assert fwd(lib, Tq=0) == 2
    assert fwd(lib, Tk=-1) == 2
    assert fwd(lib, scale=0.0) == 6
    assert fwd(lib, scale=-1.0) == 6
    assert fwd(lib, scale=float("nan")) == 6
    assert fwd(lib, scale=float("inf")) == 6
    assert fwd(lib, q=A + 2) == 7
    assert fwd(lib, o=O + 8) == 7
    assert fwd(lib, o=B_) == 8
    assert fwd(lib, o=C) == 8
    # LSE variant: missing lse pointer, lse aliasing an input
    assert lib.attn_fwd_lse(A, B_, C, 0, O, 0, 1, 2, 8, 8, 64, 0.125, 1, None) == 1
    assert lib.attn_fwd_lse(A, B_, C, 0, O, A, 1, 2, 8, 8, 64, 0.125, 1, None) == 8


def test_alias_rule_covers_byte_ranges(lib):
    # an output that shares any byte with an input or with another output is refused:
    # in place (o == q), partial overlaps, LSE inside O, and a mask inside O
    n = 1 * 2 * 8 * 64 * 2            # bytes of q and o at B1 H2 T8 D64 bf16
    assert fwd(lib, o=A) == 8
    assert fwd(lib, o=A + n - 16) == 8
    assert fwd(lib, m=O + 64) == 8
    assert lib.attn_fwd_lse(A, B_, C, 0, O, O + n - 16, 1, 2, 8, 8, 64, 0.125, 1, None) == 8
    assert lib.attn_fwd_lse(A, B_, C, 0, O, B_ + 16, 1, 2, 8, 8, 64, 0.125, 1, None) == 8


def test_merge_validation(lib):
    P = ctypes.c_void_p
    outs = (P * 2)(A, B_)
    lses = (P * 2)(C, L)
    assert lib.attn_merge_lse(0, outs, lses, O, 0, 1, 2, 8, 64, 1, None) == 2
    assert lib.attn_merge_lse(33, outs, lses, O, 0, 1, 2, 8, 64, 1, None) == 3
    assert lib.attn_merge_lse(2, None, lses, O, 0, 1, 2, 8, 64, 1, None) == 1
    bad = (P * 2)(A, 0)
    assert lib.attn_merge_lse(2, bad, lses, O, 0, 1, 2, 8, 64, 1, None) == 1
    assert lib.attn_merge_lse(2, outs, lses, A, 0, 1, 2, 8, 64, 1, None) == 8
    assert lib.attn_merge_lse(2, outs, lses, O, L, 1, 2, 8, 64, 1, None) == 8
    assert lib.attn_merge_lse(2, outs, lses, A + 1024, 0, 1, 2, 8, 64, 1, None) == 8   # inside outs[0]
    assert lib.attn_merge_lse(2, outs, lses, O, O + 512, 1, 2, 8, 64, 1, None) == 8    # lse inside out
    assert lib.attn_merge_lse(2, outs, lses, O, 0, 1, 2, 8, 100, 1, None) == 3
    assert lib.attn_merge_lse(2, outs, lses, O + 4, 0, 1, 2, 8, 64, 1, None) == 7
    assert lib.attn_merge_lse(2, outs, lses, O, 0, 1, 0, 8, 64, 1, None) == 2


def test_append_validation(lib):
    assert lib.kv_append(A, B_, 0, C, L, 2, 2, 16, 64, 1, None) == 1
    assert lib.kv_append(A, B_, O, C, L, 2, 2, 16, 80, 1, None) == 3
    assert lib.kv_append(A, B_, O, C, L, 2, 2, 0, 64, 1, None) == 2
    assert lib.kv_append(A, A, O, C, L, 2, 2, 16, 64, 1, None) == 8
    assert lib.kv_append(A + 2, B_, O, C, L, 2, 2, 16, 64, 1, None) == 7
    assert lib.kv_append(A, B_, O, A + 4096, L, 2, 2, 16, 64, 1, None) == 8    # k_new inside k_cache
    assert lib.kv_append(A, B_, A + 64, C, L, 2, 2, 16, 64, 1, None) == 8      # lengths inside k_cache


def test_decode_validation(lib):
    ws = lib.attn_decode_workspace_bytes(4, 8, 2, 1000, 128)
    assert ws > 0
    W = 0x60000

    def dec(**kw):
        a = dict(q=A, k=B_, v=C, lens=L, o=O, lse=0, B=4, Hq=8, Hkv=2, Tmax=1000, D=128,
                 scale=0.088, dtype=1, ws=W, wsb=ws)
        a.update(kw)
        return lib.attn_decode(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"], a["B"], a["Hq"],
                               a["Hkv"], a["Tmax"], a["D"], a["scale"], a["dtype"], a["ws"], a["wsb"], None)
    assert dec(lens=0) == 1
    assert dec(Hq=6, Hkv=4) == 2
    assert dec(Hkv=0) == 2
    assert dec(D=256) == 3
    assert dec(scale=0.0) == 6
    assert dec(ws=0) == 4
    assert dec(wsb=ws - 1) == 4
    assert dec(o=A) == 8
    assert dec(ws=O + 256) == 8            # workspace overlapping the output
    assert dec(o=B_ + 4096) == 8           # output inside the K cache
    assert dec(q=A + 1) == 7
    assert lib.attn_decode_workspace_bytes(4, 6, 4, 1000, 128) == 0
    assert lib.attn_decode_workspace_bytes(0, 8, 2, 1000, 128) == 0


def test_workspace_grows_linearly_with_cache_capacity(lib):
    # O(T_max) scratch, never O(T_max^2): doubling capacity at most doubles it (+ one split)
    a = lib.attn_decode_workspace_bytes(32, 32, 8, 8256, 128)
    b = lib.attn_decode_workspace_bytes(32, 32, 8, 16512, 128)
    assert a > 0 and b <= 2 * a + 32 * 32 * (128 + 2) * 4


def test_varlen_validation(lib):
    CQ, CK = 0x70000, 0x80000

    def vl(**kw):
        a = dict(q=A, k=B_, v=C, cq=CQ, ck=CK, o=O, lse=L, B=2, H=4, tq=100, tk=90, mq=60, D=64,
                 scale=0.125, dtype=1)
        a.update(kw)
        return lib.attn_fwd_varlen(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["o"], a["lse"], a["B"],
                                   a["H"], a["tq"], a["tk"], a["mq"], a["D"], a["scale"], a["dtype"], None)
    assert vl(cq=0) == 1
    assert vl(ck=0) == 1
    assert vl(o=0) == 1
    assert vl(dtype=0) == 3             # bf16 only
    assert vl(D=96) == 3
    assert vl(B=0) == 2
    assert vl(mq=101) == 2              # longer than the packed total
    assert vl(tk=-1) == 2
    assert vl(H=1 << 16, D=128) == 2    # one packed row too wide for the 32-bit tile offsets
    assert vl(tk=(1 << 30) // 256) == 2
    assert vl(scale=0.0) == 6
    assert vl(k=B_ + 4) == 7
    assert vl(o=A) == 8
    assert vl(lse=C) == 8
    assert vl(tq=0, mq=0) == 0          # nothing to do: no launch, no pointer touched
    assert vl(mq=0) == 0


def test_paged_validation(lib):
    BT, W = 0x70000, 0x60000
    ws = lib.attn_decode_workspace_bytes(4, 8, 2, 64 * 16, 128)

    def dp(**kw):
        a = dict(q=A, k=B_, v=C, bt=BT, lens=L, o=O, lse=0, B=4, Hq=8, Hkv=2, npg=100, ps=16, mp=64, D=128,
                 scale=0.088, dtype=1, ws=W, wsb=ws)
        a.update(kw)
        return lib.attn_decode_paged(a["q"], a["k"], a["v"], a["bt"], a["lens"], a["o"], a["lse"], a["B"],
                                     a["Hq"], a["Hkv"], a["npg"], a["ps"], a["mp"], a["D"], a["scale"],
                                     a["dtype"], a["ws"], a["wsb"], None)
    assert dp(bt=0) == 1
    assert dp(lens=0) == 1
    assert dp(dtype=0) == 3           # bf16 only
    assert dp(D=96) == 3
    assert dp(ps=24) == 2             # not a power of two
    assert dp(ps=8) == 2              # below 16
    assert dp(npg=0) == 2
    assert dp(mp=0) == 2
    assert dp(mp=1 << 27) == 2        # capacity above 2^30 tokens
    assert dp(Hq=5) == 2
    assert dp(scale=-1.0) == 6
    assert dp(wsb=ws - 1) == 4
    assert dp(ws=0) == 4
    assert dp(k=B_ + 8) == 7
    assert dp(o=B_) == 8

    def ap(**kw):
        a = dict(k=A, v=B_, bt=BT, lens=L, kn=C, vn=O, B=4, Hkv=2, npg=100, ps=16, mp=64, D=128, dtype=1)
        a.update(kw)
        return lib.kv_append_paged(a["k"], a["v"], a["bt"], a["lens"], a["kn"], a["vn"], a["B"], a["Hkv"],
                                   a["npg"], a["ps"], a["mp"], a["D"], a["dtype"], None)
    assert ap(bt=0) == 1
    assert ap(kn=0) == 1
    assert ap(D=80) == 3
    assert ap(ps=48) == 2
    assert ap(B=0) == 2
    assert ap(v=A) == 8
    assert ap(kn=C + 4) == 7


def test_prefill_validation(lib):
    def pf(**kw):
        a = dict(q=A, k=B_, v=C, m=0, o=O, lse=0, B=1, Hq=8, Hkv=2, Tq=64, Tk=64, D=64, causal=1, scale=0.125,
                 dtype=1)
        a.update(kw)
        return lib.attn_prefill(a["q"], a["k"], a["v"], a["m"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                                a["Tq"], a["Tk"], a["D"], a["causal"], a["scale"], a["dtype"], None)
    assert pf(q=0) == 1
    assert pf(dtype=0) == 3                   # causal needs bf16
    assert pf(dtype=0, causal=0) == 3         # so does GQA
    assert pf(Hq=6, Hkv=4) == 2
    assert pf(Hkv=0) == 2
    assert pf(D=80) == 3
    assert pf(Tk=0) == 2
    assert pf(scale=0.0) == 6
    assert pf(v=C + 2) == 7
    assert pf(lse=O) == 8
    CQ, CK = 0x70000, 0x80000

    def pv(**kw):
        a = dict(q=A, k=B_, v=C, cq=CQ, ck=CK, o=O, lse=L, B=2, Hq=8, Hkv=2, tq=100, tk=90, mq=60, D=128,
                 causal=1, scale=0.088, dtype=1)
        a.update(kw)
        return lib.attn_prefill_varlen(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["o"], a["lse"], a["B"],
                                       a["Hq"], a["Hkv"], a["tq"], a["tk"], a["mq"], a["D"], a["causal"],
                                       a["scale"], a["dtype"], None)
    assert pv(cq=0) == 1
    assert pv(dtype=0) == 3
    assert pv(Hq=8, Hkv=3) == 2
    assert pv(mq=101) == 2
    assert pv(o=A) == 8
    assert pv(tq=0, mq=0) == 0
    assert pv(k=0) == 1


def test_fp8_validation(lib):
    KS, VS, W = 0x70000, 0x80000, 0x60000
    ws = lib.attn_decode_workspace_bytes(4, 8, 2, 1000, 128)

    def dec(**kw):
        a = dict(q=A, k=B_, v=C, ks=KS, vs=VS, lens=L, o=O, lse=0, B=4, Hq=8, Hkv=2, Tmax=1000, D=128,
                 scale=0.088, ws=W, wsb=ws)
        a.update(kw)
        return lib.attn_decode_fp8kv(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["lens"], a["o"], a["lse"], a["B"],
                                     a["Hq"], a["Hkv"], a["Tmax"], a["D"], a["scale"], a["ws"], a["wsb"], None)
    assert dec(ks=0) == 1
    assert dec(vs=0) == 1
    assert dec(D=96) == 3
    assert dec(Hq=6, Hkv=4) == 2
    assert dec(Tmax=(1 << 24) + 1) == 2          # T_max·D beyond the 32-bit range of one head
    assert dec(scale=0.0) == 6
    assert dec(wsb=ws - 1) == 4
    assert dec(k=B_ + 8) == 7
    assert dec(o=A) == 8
    assert dec(ws=O + 256) == 8            # workspace overlapping the output
    assert dec(o=B_ + 4096) == 8           # output inside the K cache
    assert lib.kv_append_fp8(A, B_, KS, 0, L, C, O, 2, 2, 16, 64, 1, None) == 1
    assert lib.kv_append_fp8(A, B_, KS, VS, L, C, O, 2, 2, 16, 64, 7, None) == 3
    assert lib.kv_append_fp8(A, B_, KS, VS, L, C, O, 2, 2, 0, 64, 1, None) == 2
    assert lib.kv_append_fp8(A, A, KS, VS, L, C, O, 2, 2, 16, 64, 1, None) == 8


def test_prefill_fp8_validation(lib):
    QS, KS, VS = 0x70000, 0x80000, 0x90000

    def pf(**kw):
        a = dict(q=A, k=B_, v=C, qs=QS, ks=KS, vs=VS, m=0, o=O, lse=L, B=2, Hq=8, Hkv=2, Tq=100, Tk=130, D=128,
                 causal=1, scale=0.088)
        a.update(kw)
        return lib.attn_prefill_fp8(a["q"], a["k"], a["v"], a["qs"], a["ks"], a["vs"], a["m"], a["o"], a["lse"],
                                    a["B"], a["Hq"], a["Hkv"], a["Tq"], a["Tk"], a["D"], a["causal"], a["scale"],
                                    None)
    assert pf(qs=0) == 1
    assert pf(ks=0) == 1
    assert pf(vs=0) == 1
    assert pf(o=0) == 1
    assert pf(D=96) == 3
    assert pf(Hq=6, Hkv=4) == 2
    assert pf(Hkv=0) == 2
    assert pf(Tq=0) == 2
    assert pf(Tk=(1 << 24) + 1) == 2           # Tk·D beyond the 32-bit range of one head
    assert pf(scale=float("nan")) == 6
    assert pf(k=B_ + 4) == 7
    assert pf(o=A) == 8
    assert pf(lse=C) == 8


def test_int8_validation(lib):
    KS, VS, W = 0x70000, 0x80000, 0x60000
    ws = lib.attn_decode_workspace_bytes(4, 8, 2, 1000, 128)

    def dec(**kw):
        a = dict(q=A, k=B_, v=C, ks=KS, vs=VS, lens=L, o=O, lse=0, B=4, Hq=8, Hkv=2, Tmax=1000, D=128,
                 scale=0.088, ws=W, wsb=ws)
        a.update(kw)
        return lib.attn_decode_int8kv(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["lens"], a["o"], a["lse"],
                                      a["B"], a["Hq"], a["Hkv"], a["Tmax"], a["D"], a["scale"], a["ws"], a["wsb"],
                                      None)
    assert dec(ks=0) == 1
    assert dec(D=96) == 3
    assert dec(Hq=6, Hkv=4) == 2
    assert dec(Tmax=(1 << 24) + 1) == 2
    assert dec(scale=-1.0) == 6
    assert dec(wsb=ws - 1) == 4
    assert dec(v=C + 8) == 7
    assert dec(o=B_) == 8
    assert lib.kv_append_int8(A, B_, 0, VS, L, C, O, 2, 2, 16, 64, 1, None) == 1
    assert lib.kv_append_int8(A, B_, KS, VS, L, C, O, 2, 2, 16, 64, 5, None) == 3
    assert lib.kv_append_int8(A, B_, KS, VS, L, C, O, 2, 0, 16, 64, 1, None) == 2
    assert lib.kv_append_int8(A, A, KS, VS, L, C, O, 2, 2, 16, 64, 1, None) == 8


def test_prefill_varlen_fp8_validation(lib):
    QS, KS, VS, CQ, CK = 0x70000, 0x80000, 0x90000, 0xA0000, 0xB0000

    def pv(**kw):
        a = dict(q=A, k=B_, v=C, qs=QS, ks=KS, vs=VS, cq=CQ, ck=CK, o=O, lse=L, B=2, Hq=8, Hkv=2, tq=100, tk=90,
                 mq=60, D=128, causal=1, scale=0.088)
        a.update(kw)
        return lib.attn_prefill_varlen_fp8(a["q"], a["k"], a["v"], a["qs"], a["ks"], a["vs"], a["cq"], a["ck"],
                                           a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["tq"], a["tk"], a["mq"],
                                           a["D"], a["causal"], a["scale"], None)
    assert pv(qs=0) == 1
    assert pv(cq=0) == 1
    assert pv(D=96) == 3
    assert pv(Hq=8, Hkv=3) == 2
    assert pv(mq=101) == 2
    assert pv(scale=0.0) == 6
    assert pv(q=A + 8) == 7
    assert pv(o=A) == 8
    assert pv(tq=0, mq=0) == 0

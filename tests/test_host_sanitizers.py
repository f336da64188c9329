"""Host-side checks of the C ABI on the CPU: a debug build of the library (ATTN_DEBUG: every
launcher asserts its grid, LDS bytes, 32-bit offsets and workspace layout against the buffer
extents) with AddressSanitizer and UndefinedBehaviorSanitizer on the host code, driven through
every entry point in a child process.

Valid calls pass the argument checks and the ATTN_DEBUG assertions, then fail to launch (there
is no GPU here), so they must return ATTN_ERR_LAUNCH; invalid calls must return their status
code.  Any sanitizer report or failed assertion aborts the child and fails the test.  The
pointers are fake device addresses, never dereferenced, so this test never runs where a GPU is
present (a valid call would then reach a real launch).
"""
import glob
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEBUG_LIB = os.path.join(ROOT, "_build", "host_san", "libmasked_attn_debug.so")


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm*/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:  # pragma: no cover
        return False


@pytest.fixture(scope="module")
def debug_lib():
    if _gpu_present():
        pytest.skip("host-sanitizer run is CPU-only (valid calls would reach a real launch)")
    if _asan_runtime() is None or shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc or the clang ASan runtime is not available")
    sys.path.insert(0, ROOT)
    from masked_attention_attn_amd import build as b
    san = ["-DATTN_DEBUG", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    b.build(verbose=False, out=DEBUG_LIB, build_dir=os.path.dirname(DEBUG_LIB), extra=san)
    return DEBUG_LIB


CHILD = r'''
import ctypes, json, sys
lib = ctypes.CDLL(sys.argv[1])
P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
G = 1 << 32                                   # fake device addresses, 4 GiB apart
Q, K, V, O, L, M, C1, C2, WS, BT, SC1, SC2, SC3 = (G * i for i in range(1, 14))
res = {}
def call(name, argtypes, *args):
    f = getattr(lib, name)
    f.argtypes = argtypes
    f.restype = I
    return f(*args)
fwd_t = [P, P, P, P, P, I, I, I, I, I, F, I, P]
lse_t = [P, P, P, P, P, P, I, I, I, I, I, F, I, P]
# masked / LSE forward: both dtypes and head dims, with and without a mask
for dt in (0, 1):
    for D in (64, 128):
        res[f"fwd_masked dt{dt} D{D}"] = call("attn_fwd_masked", fwd_t, Q, K, V, M, O, 2, 3, 300, 700, D, 0.1, dt, None)
        res[f"fwd_lse dt{dt} D{D}"] = call("attn_fwd_lse", lse_t, Q, K, V, 0, O, L, 1, 16, 11616, 11616, D, 0.125, dt, None)
res["fwd bad D"] = call("attn_fwd_masked", fwd_t, Q, K, V, 0, O, 1, 2, 8, 8, 96, 0.1, 1, None)
res["fwd alias"] = call("attn_fwd_lse", lse_t, Q, K, V, 0, O, O + 64, 1, 2, 8, 8, 64, 0.1, 1, None)
res["fwd zero B"] = call("attn_fwd_masked", fwd_t, Q, K, V, 0, O, 0, 2, 8, 8, 64, 0.1, 1, None)
# GQA / causal prefill, packed forms
res["prefill causal gqa"] = call("attn_prefill", [P] * 6 + [I] * 7 + [F, I, P],
                                 Q, K, V, 0, O, L, 1, 32, 8, 8192, 8192, 128, 1, 0.088, 1, None)
vl_t = [P, P, P, P, P, P, P] + [I] * 6 + [F, I, P]
res["varlen"] = call("attn_fwd_varlen", vl_t, Q, K, V, C1, C2, O, L, 4, 16, 3644, 3644, 1944, 64, 0.125, 1, None)
res["varlen causal gqa"] = call("attn_prefill_varlen", [P] * 7 + [I] * 8 + [F, I, P],
                                Q, K, V, C1, C2, O, L, 8, 32, 8, 16384, 16384, 4096, 128, 1, 0.088, 1, None)
res["varlen bad max"] = call("attn_fwd_varlen", vl_t, Q, K, V, C1, C2, O, L, 4, 16, 100, 100, 101, 64, 0.1, 1, None)
# merge
PA = P * 5
res["merge 2"] = call("attn_merge_lse", [I, ctypes.POINTER(P), ctypes.POINTER(P), P, P, I, I, I, I, I, P],
                      2, PA(Q, K), PA(V, M), O, L, 1, 24, 8192, 128, 1, None)
res["merge 5 f32"] = call("attn_merge_lse", [I, ctypes.POINTER(P), ctypes.POINTER(P), P, P, I, I, I, I, I, P],
                          5, PA(Q, K, V, M, C1), PA(C2, WS, BT, SC1, SC2), O, 0, 2, 3, 37, 64, 0, None)
# append + decode, contiguous and paged, both dtypes, and the allocation-free decode
ap_t = [P, P, P, P, P, I, I, I, I, I, P]
dec_t = [P, P, P, P, P, P, I, I, I, I, I, F, I, P, S, P]
for dt in (0, 1):
    res[f"append dt{dt}"] = call("kv_append", ap_t, K, V, C1, Q, M, 32, 8, 8256, 128, dt, None)
    res[f"decode dt{dt}"] = call("attn_decode", dec_t, Q, K, V, C1, O, L, 32, 32, 8, 8256, 128, 0.088, dt, WS,
                                 64 << 20, None)
res["decode small ws"] = call("attn_decode", dec_t, Q, K, V, C1, O, L, 32, 32, 8, 8256, 128, 0.088, 1, WS, 1024, None)
res["decode noalloc"] = call("attn_decode_noalloc", [P, P, P, P, P, P] + [I] * 5 + [F, I, P],
                             Q, K, V, C1, O, L, 32, 32, 8, 8256, 128, 0.088, 1, None)
res["decode noalloc oversize"] = call("attn_decode_noalloc", [P, P, P, P, P, P] + [I] * 5 + [F, I, P],
                                      Q, K, V, C1, O, L, 64, 64, 8, 9216, 128, 0.088, 1, None)
res["append paged"] = call("kv_append_paged", [P] * 6 + [I] * 7 + [P], K, V, BT, C1, Q, M, 32, 8, 9000, 16, 516,
                           128, 1, None)
res["decode paged"] = call("attn_decode_paged", [P] * 7 + [I] * 7 + [F, I, P, S, P], Q, K, V, BT, C1, O, L,
                           32, 32, 8, 9000, 16, 516, 128, 0.088, 1, WS, 64 << 20, None)
res["decode paged bad page"] = call("attn_decode_paged", [P] * 7 + [I] * 7 + [F, I, P, S, P], Q, K, V, BT, C1, O, L,
                                    32, 32, 8, 9000, 24, 516, 128, 0.088, 1, WS, 64 << 20, None)
# 8-bit caches and the E4M3 prefill
q8a_t = [P] * 7 + [I] * 5 + [P]
q8d_t = [P] * 8 + [I] * 5 + [F, P, S, P]
for fmt in ("fp8", "int8"):
    res[f"append {fmt}"] = call(f"kv_append_{fmt}", q8a_t, K, V, SC1, SC2, C1, Q, M, 32, 8, 8256, 128, 1, None)
    res[f"decode {fmt}"] = call(f"attn_decode_{fmt}kv", q8d_t, Q, K, V, SC1, SC2, C1, O, L, 32, 32, 8, 8256, 128,
                                0.088, WS, 64 << 20, None)
    res[f"append {fmt} paged"] = call(f"kv_append_{fmt}_paged", [P] * 8 + [I] * 7 + [P], K, V, SC1, SC2, BT, C1,
                                      Q, M, 32, 8, 9000, 16, 516, 128, 1, None)
    res[f"decode {fmt} paged"] = call(f"attn_decode_{fmt}kv_paged", [P] * 9 + [I] * 7 + [F, P, S, P], Q, K, V,
                                      SC1, SC2, BT, C1, O, L, 32, 32, 8, 9000, 16, 516, 128, 0.088, WS, 64 << 20,
                                      None)
res["prefill fp8"] = call("attn_prefill_fp8", [P] * 9 + [I] * 7 + [F, P], Q, K, V, SC1, SC2, SC3, M, O, L,
                          1, 16, 16, 11616, 11616, 64, 0, 0.125, None)
res["prefill varlen fp8"] = call("attn_prefill_varlen_fp8", [P] * 10 + [I] * 8 + [F, P], Q, K, V, SC1, SC2, SC3,
                                 C1, C2, O, L, 1, 24, 24, 8192, 8192, 8192, 128, 0, 0.088, None)
print(json.dumps(res))
'''

EXPECT = {
    "fwd bad D": 3, "fwd alias": 8, "fwd zero B": 2, "varlen bad max": 2, "decode small ws": 4,
    "decode noalloc oversize": 9, "decode paged bad page": 2,
}


def test_every_entry_point_under_host_sanitizers(debug_lib):
    env = dict(os.environ)
    env["LD_PRELOAD"] = _asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1:alloc_dealloc_mismatch=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env.pop("HIP_VISIBLE_DEVICES", None)
    r = subprocess.run([sys.executable, "-c", CHILD, debug_lib], capture_output=True, text=True, env=env,
                       timeout=600)
    assert r.returncode == 0, f"child failed ({r.returncode}):\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr, r.stderr[-4000:]
    res = json.loads(r.stdout.strip().splitlines()[-1])
    for name, status in res.items():
        want = EXPECT.get(name, 5)          # valid calls: checks pass, then no GPU to launch on
        assert status == want, f"{name}: status {status}, expected {want}"
    assert len(res) >= 35

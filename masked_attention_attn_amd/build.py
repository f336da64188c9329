"""Build the HIP shared library libmasked_attn.so for gfx950.

Compiles every csrc/*.hip file with hipcc into an object under _build/ and
links them into masked_attention_attn_amd/libmasked_attn.so (in-tree, so the
library travels with the source tree).  Always recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmasked_attn.so")
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# Per-source extras for the bf16 prefill kernels:
#  * -fno-honor-nans: the kernels produce no NaN (infinities are still honoured,
#    -inf marks padded keys), which lets fmaxf lower to v_max3_f32 on raw MFMA
#    results instead of canonicalise-then-max.
#  * VGPR-form MFMAs at D = 64 keep the score blocks in VGPRs for the vector
#    unit (no AGPR<->VGPR copies).
#  * the E4M3 kernels turn off machine sinking: it moves the E4M3 score MFMAs
#    of the next key block (used only by the next step) past the rescale
#    branches to the end of the step, where the next step's exponentials
#    would wait for them, instead of the slots the step gives them.
EXTRA = {
    "fwd_bf16_d64.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
    "fwd_bf16_d128.hip": ["-fno-honor-nans"],
    "fwd_fp8_d64.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans", "-mllvm", "-disable-machine-sink"],
    "fwd_fp8_d128.hip": ["-fno-honor-nans", "-mllvm", "-disable-machine-sink"],
    "decode_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
    "decode_q8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
}


def _compile(src: str, build_dir: str = BUILD, include_first=None, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src).replace(".hip", ".o"))
    inc = ["-I", include_first] if include_first else []
    cmd = [HIPCC, *inc, *FLAGS, *EXTRA.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True, out: str = LIB, build_dir: str = BUILD, csrc: str = CSRC, extra=(),
          link_extra=()) -> str:
    """Compile csrc/*.hip into `out` (default: the in-tree library).  `extra` flags go to every
    compile, `link_extra` to the link (the debug build with host sanitizers uses both)."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(csrc, "*.hip")))

    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, extra=extra), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} from {len(srcs)} sources")
    return out


if __name__ == "__main__":
    build()

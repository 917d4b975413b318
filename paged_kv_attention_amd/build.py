"""Compile the HIP sources into paged_kv_attention_amd/libfi.so for gfx950.

Every call recompiles (objects go to paged_kv_attention_amd/_build/). Usage:
    python -m paged_kv_attention_amd.build
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfi.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# Per-file extras. The MXFP4 decode kernel keeps its MFMA accumulators in
# ordinary VGPRs: in the AGPR form the compiler copies all 32 of them between
# the two register files on every step (the lazy rescale multiplies them on
# the VALU), which that ALU-bound kernel cannot afford.
EXTRA = {
    "fi_decode_fp4.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "fi_decode_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


# Host-sanitizer build (libfi_san.so, for the CPU tests): host code with
# AddressSanitizer and UBSan, device code unchanged.
SAN_LIB = os.path.join(HERE, "libfi_san.so")
SAN_BUILD = os.path.join(HERE, "_build_san")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_BUILD if sanitize else BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + COMMON + EXTRA.get(os.path.basename(src), []) + \
        (SAN_HOST if sanitize else []) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True, sanitize: bool = False) -> str:
    """Compile every source and link the library (``sanitize``: the
    host-sanitizer build, libfi_san.so, which needs the sanitizer runtime
    preloaded into the process that loads it)."""
    out_dir, lib = (SAN_BUILD, SAN_LIB) if sanitize else (BUILD, LIB)
    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, sanitize), srcs))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if sanitize:
        cmd += SAN_HOST + ["-shared-libsan"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} from {len(srcs)} sources")
    return lib


def sanitizer_runtime() -> str:
    """Path of the AddressSanitizer runtime the sanitizer build links."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("AddressSanitizer runtime not found next to hipcc's clang")
    return path


if __name__ == "__main__":
    build()
    sys.exit(0)

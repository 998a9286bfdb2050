"""Build libtri_attn.so for gfx950 with hipcc, in-tree.

    python -m triangular_pair_attention_amd.build

Objects go to _build/ at the repository root; the shared library to
triangular_pair_attention_amd/lib/libtri_attn.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "lib", "libtri_attn.so")
CALIB = os.path.join(PKG, "lib", "tri_attn_calib")
SOURCES = ("tri_attn.cpp", "pack_weights.hip", "k1_ln_proj.hip", "k1_split.hip", "k2_attention.hip",
           "k2_train.hip", "k3_out_proj.hip", "noalloc.hip", "bwd_train.hip", "onepass.hip")
# further compilation units: (source, object name, extra flags). The bf16
# head-size-16 attention kernel is built on its own with LLVM's
# max-memory-clause scheduler (its key loop measured 3% faster; the other
# attention shapes slower).
EXTRA_UNITS = (
    ("k2_attention.hip", "k2_attention_bf16_d16",
     ["-DTPA_K2_BF16_D16", "-mllvm", "-amdgpu-sched-strategy=max-memory-clause"]),
)


def units():
    """Every compilation unit: (source, object name, extra flags)."""
    return [(f, os.path.splitext(f)[0], []) for f in SOURCES] + [(f, o, list(x)) for f, o, x in EXTRA_UNITS]
ARCH = "gfx950"

FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    # no packed-fp32 VALU instructions in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: no v_accvgpr_read moves
    # before the VALU uses a result (float32 attention: -3% time)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _compile(src: str, extra, name=None) -> str:
    obj = os.path.join(OBJDIR, (name or os.path.splitext(src)[0]) + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    us = units()
    with ThreadPoolExecutor(max_workers=len(us)) as ex:
        objs = list(ex.map(lambda u: _compile(u[0], [*u[2], *extra], u[1]), us))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    # calibration microbenchmarks (a separate executable, not part of the library)
    cmd = [hipcc(), "-O3", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", os.path.join(PKG, "calib", "calib.hip"), "-o", CALIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the calibration tool failed:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {LIB} and {CALIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])

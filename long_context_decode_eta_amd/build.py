"""Build libeta.so (the HIP library) in-tree for gfx950.

Run ``python -m long_context_decode_eta_amd.build`` or call :func:`build`.
Every translation unit is compiled with hipcc for gfx950 only; packed FP32
instructions are disabled (``-packed-fp32-ops``) so the compiler never forms
v_pk_*_f32 from ordinary float code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libeta.so")
SOURCES = ["eta_api.hip", "kernels_meta.hip", "kernels_screen.hip", "kernels_decode.hip",
           "kernels_gqa.hip", "kernels_prefill.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# The matrix-core kernels keep their accumulators in ordinary VGPRs: with the
# AGPR form the compiler copied every accumulator out of and back into AGPRs on
# each tile (about 10% of the prefill loop's instructions).
FILE_FLAGS = {
    "kernels_gqa.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "kernels_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _compile(src: str, obj_dir: str = OBJ, defines: tuple = ()) -> str:
    out = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *defines, "-c", os.path.join(CSRC, src),
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose: bool = False, out: str = LIB, obj_dir: str = OBJ,
          defines: tuple = ()) -> str:
    """Compile every source and link `out`.  `defines` (-D flags) override the
    kernels' compile-time tuning constants (tile rows and the like)."""
    os.makedirs(obj_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, tuple(defines)), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

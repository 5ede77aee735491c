"""Build libparallax.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python -m parallax_local_linear_decode_amd.build
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
LIB = os.path.join(PKG, "libparallax.so")
SOURCES = ["api.hip", "decode.hip", "prefill.hip", "prefill_bwd.hip", "lla.hip", "proj.hip"]
# A plain read-stream kernel the benchmark times as the HBM reference; its
# own library, not part of libparallax.
PROBE_LIB = os.path.join(PKG, "libparallax_probe.so")
PROBE_SOURCES = ["read_probe.hip", "issue_probe.hip"]
ARCH = "gfx950"

# Packed fp32 VALU instructions are kept out of the generated code.  MFMA
# accumulators are allocated in the VGPR form: the kernels' accumulators are
# updated by VALU code too (rescaling), and with the AGPR form the compiler
# shuttles them between register files every loop iteration.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}",
]
# The projection's large-tile GEMM holds 256 fp32 accumulators per lane, which
# only fit in the accumulation registers, and no VALU code touches them, so
# its file keeps the compiler's default register form.
VGPR_FORM = ("-mllvm", "-amdgpu-mfma-vgpr-form=1")
AGPR_FORM = ("proj.hip",)


def flags_for(src: str) -> list:
    """hipcc flags of one source file (a name under csrc/)."""
    if src in AGPR_FORM:
        i = HIPCC_FLAGS.index(VGPR_FORM[1])
        return HIPCC_FLAGS[:i - 1] + HIPCC_FLAGS[i + 1:]
    return list(HIPCC_FLAGS)


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *flags_for(src), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES) + len(PROBE_SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES + PROBE_SOURCES))

    def link(target, target_objs):
        tmp = target + ".tmp"
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *target_objs, "-o", tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link of {os.path.basename(target)} failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp, target)

    link(LIB, objs[:len(SOURCES)])
    link(PROBE_LIB, objs[len(SOURCES):])
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

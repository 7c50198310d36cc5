"""Build libgqla.so (all HIP sources of the package) for gfx950 with hipcc.

Usage: python -m decode_attention_gqla_amd.build   (or call build()).
The library lands next to this file; nothing is installed elsewhere.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgqla.so")
SOURCES = ["gqla_api.hip", "gqa_decode.hip", "absorb_decode.hip", "absorb_wide.hip", "expand.hip", "combine.hip",
           "select.hip", "append.hip"]
# sources whose kernels keep MFMA accumulators in accumulation registers
ACC_FORM: set[str] = set()
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgqla)")


def flags(src: str = "") -> list[str]:
    f = [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 VALU forms are kept out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wno-unused-result",
    ]
    if src not in ACC_FORM:
        # MFMA accumulators in VGPRs: without it the GQA kernel copies its O
        # tiles between VGPRs and AGPRs around every MFMA
        f += ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    return f


def build(verbose: bool = False) -> str:
    """Compile every source and link libgqla.so; returns the library path."""
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [cc, *flags(src), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        text = out.decode(errors="replace")
        # the host pass of hipcc does not know the device-only feature flag
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if pr.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        msg = "\n".join(f"--- {s}\n{t}" for s, t in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

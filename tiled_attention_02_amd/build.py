"""Build libaule_attn.so in-tree with hipcc for gfx950.

Usage: ``python -m tiled_attention_02_amd.build`` (or ``build()`` from Python). Every call
recompiles. Objects go to ``_build/`` under the package; the shared library is written next
to this file, where the binding loads it.
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
LIB = os.path.join(PKG, "libaule_attn.so")
ARCH = "gfx950"

SOURCES = ["aule_attn_api.cpp", "attn_fwd_valu.hip", "attn_fwd_f32_mfma.hip", "attn_fwd_mfma.hip", "attn_fwd_short.hip", "attn_decode.hip", "attn_decode_mfma.hip", "attn_bwd.hip", "attn_bwd_f32_mfma.hip",
           "attn_bwd_mfma.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # no packed-fp32 VALU instructions in any device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libaule_attn.so")


def _compile(src: str, obj: str, extra: list[str]) -> None:
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc()] + COMMON_FLAGS + extra + lang + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stderr or "").splitlines() if ln.strip() and noise not in ln]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")


def build(verbose: bool = False, extra_flags: list[str] | None = None, out: str | None = None) -> str:
    """Compile every source and link the library (to `out`, default the in-tree path)."""
    extra = list(extra_flags or [])
    lib = out or LIB
    objdir = os.path.join(PKG, "_build" if out is None else "_build_" + os.path.basename(lib).replace(".", "_"))
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    for s in SOURCES:
        src = os.path.join(CSRC, s)
        obj = os.path.join(objdir, os.path.splitext(s)[0] + ".o")
        jobs.append((src, obj))
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        list(ex.map(lambda j: _compile(j[0], j[1], extra), jobs))
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for _, o in jobs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=None, help="library path (default: in-tree libaule_attn.so)")
    ap.add_argument("-D", "--define", action="append", default=[], help="extra preprocessor define")
    a = ap.parse_args()
    build(verbose=True, extra_flags=["-D" + d for d in a.define], out=a.out)

"""Build the HIP attention library (libfa.so) for gfx950 with hipcc.

    python -m exact_attention_84_amd.build [--jobs N] [--define NAME=VALUE ...]

Every source is compiled for gfx950 only, then linked into
``exact_attention_84_amd/libfa.so`` next to this file.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_fwd_wide.hip", "fa_fwd_fp8.hip", "fa_decode.hip", "fa_bwd.hip"]
# Per-source code-generation options.  The dK/dV kernel runs one wave per
# SIMD with its accumulators live across the whole loop; selecting the VGPR
# form of the MFMA instructions keeps them in place instead of copying them
# between AGPRs and VGPRs around every product.
# The 64-row forward keeps O in AGPRs that only its inline assembly names;
# its score products must therefore stay in VGPR form as well.
SOURCE_FLAGS = {"fa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "fa_fwd_wide.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def flags(defines=()):
    f = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # packed fp32 VALU ops are kept out of the generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]
    f += [f"-D{d}" for d in defines]
    return f


def _compile(src, out, defines):
    cmd = [hipcc(), *flags(defines), *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{err}")
    return err


def build(jobs: int = 4, defines=(), out_lib: str = LIB, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        futs = [ex.submit(_compile, s, o, defines) for s, o in zip(SOURCES, objs)]
        for f in futs:
            warn = f.result()
            if verbose and warn.strip():
                print(warn, file=sys.stderr)
    tmp = out_lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stderr}")
    _check_undefined(tmp)
    os.replace(tmp, out_lib)
    return out_lib


def _check_undefined(lib: str) -> None:
    """Refuse a library whose host side lacks a kernel launch stub (it would
    only fail when loaded)."""
    r = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True)
    missing = [l.split()[-1] for l in r.stdout.splitlines()
               if "__device_stub__" in l or "_ZN2fa" in l]
    if missing:
        os.remove(lib)
        raise RuntimeError("undefined symbols in the built library: " + ", ".join(missing))


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--define", action="append", default=[])
    ap.add_argument("--out", default=LIB)
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.define, a.out, a.verbose))


if __name__ == "__main__":
    main()

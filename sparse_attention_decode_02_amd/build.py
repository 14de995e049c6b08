"""Builds libdsa.so in-tree from csrc/*.hip for gfx950 only.

    python -m sparse_attention_decode_02_amd.build

Every HIP source is compiled with packed-fp32 instruction selection switched
off (plain fp32 VALU code only).
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libdsa.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources() -> list:
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compiles and links libdsa.so next to this file; returns its path."""
    srcs = sources()
    objs = []
    with tempfile.TemporaryDirectory(prefix="dsa_build_") as tmp:
        procs = []
        for s in srcs:
            o = os.path.join(tmp, os.path.basename(s) + ".o")
            cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
                   "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                   "-I", os.path.join(ROOT, "include"), *extra_flags, "-c", s, "-o", o]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                              text=True)))
            objs.append(o)
        failed = []
        for s, p in procs:
            out, _ = p.communicate()
            out = "\n".join(ln for ln in out.splitlines() if "packed-fp32-ops" not in ln)
            if p.returncode != 0:
                failed.append((s, out))
            elif verbose and out.strip():
                print(out)
        if failed:
            msg = "\n".join(f"--- {s}\n{o}" for s, o in failed)
            raise RuntimeError(f"HIP compile failed:\n{msg}")
        tmp_lib = LIB + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

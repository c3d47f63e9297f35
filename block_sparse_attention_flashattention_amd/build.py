"""Compile libvsa_attn.so for gfx950 with hipcc (ahead of time, in-tree).

Usage: python -m block_sparse_attention_flashattention_amd.build
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libvsa_attn.so")
SOURCES = ["attn_fwd.hip", "attn_fwd_pp.hip", "attn_fwd_iw.hip", "attn_fwd_2t.hip", "attn_fwd_2s.hip", "attn_fwd_4s.hip", "attn_bwd.hip", "frontend.hip",
           "measure.hip", "capi.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from emitting packed-fp32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source in parallel and link the shared library."""
    with tempfile.TemporaryDirectory(prefix="vsa_build_") as tmp:
        procs = []
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = []
        for src, proc in procs:
            out, _ = proc.communicate()
            if out and (verbose or proc.returncode):
                # the host pass does not know the packed-fp32 feature; that warning is expected
                lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
                if lines:
                    print("\n".join(lines), file=sys.stderr)
            if proc.returncode:
                failed.append(src)
        if failed:
            raise RuntimeError(f"hipcc failed for {failed}")
        tmp_lib = os.path.join(tmp, "libvsa_attn.so")
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, LIB) if os.path.dirname(tmp_lib) == os.path.dirname(LIB) else _copy(tmp_lib, LIB)
    return LIB


def _copy(src: str, dst: str) -> None:
    tmp = dst + ".tmp"
    with open(src, "rb") as f, open(tmp, "wb") as g:
        g.write(f.read())
    os.chmod(tmp, 0o755)
    os.replace(tmp, dst)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

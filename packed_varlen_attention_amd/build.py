"""Build the gfx950 HIP library (libmf.so) in-tree with hipcc.

Usage: python -m packed_varlen_attention_amd.build  (or build() from Python).
Objects go to packed_varlen_attention_amd/_build/; the library is written to
packed_varlen_attention_amd/libmf.so with an atomic rename.

  python -m packed_varlen_attention_amd.build --sanitize-host
builds a copy whose host code (argument checks, workspace layout, launches)
carries AddressSanitizer and UndefinedBehaviorSanitizer, for CPU checks of
the C ABI; device code is built as usual.  It goes to
packed_varlen_attention_amd/_build_san/libmf.so, never over the in-tree
library.  Load it with the sanitizer runtime preloaded, e.g.
  LD_PRELOAD=$(hipcc -print-file-name=libclang_rt.asan-x86_64.so) \
  MF_LIBRARY=packed_varlen_attention_amd/_build_san/libmf.so \
  ASAN_OPTIONS=detect_leaks=0 python -m pytest tests/test_abi.py
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmf.so")
SAN_BUILD = os.path.join(PKG, "_build_san")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
SOURCES = ["api.hip", "pack.hip", "rope.hip", "sched.hip", "attn_fwd.hip", "attn_bwd.hip", "flow.hip", "block.hip",
           "block_bwd.hip", "probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # keep the compiler from forming packed-fp32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


def _compile(src: str, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *common_flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize_host: bool = False) -> str:
    out_dir = SAN_BUILD if sanitize_host else BUILD
    lib = os.path.join(SAN_BUILD, "libmf.so") if sanitize_host else LIB
    extra = SAN_HOST if sanitize_host else []
    os.makedirs(out_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, out_dir, extra), SOURCES))
    tmp = lib + ".tmp"
    link_extra = ["-shared-libsan", *SAN_HOST[:4]] if sanitize_host else []
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(verbose=True, sanitize_host="--sanitize-host" in sys.argv[1:])
    sys.exit(0)

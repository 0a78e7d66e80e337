"""Builds libcsa2.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python sparse_attention_fp4_e2m1_amd/build.py [--sanitize]

(Run it as a script: importing the package loads the library it builds.)
--sanitize builds _build/libcsa2_sanitize.so instead: the same sources with
AddressSanitizer and UndefinedBehaviorSanitizer on the host code only (the
GPU code is built as usual), for the host-side validation and workspace
sizing tests; load it with the ASan runtime preloaded and CSA2_LIBRARY set to
its path (tests/test_sanitize_cpu.py does this).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcsa2.so")
SOURCES = ["csa2_api.hip", "csa2_append.hip", "csa2_index.hip", "csa2_index_gemm.hip",
           "csa2_attn.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Per-source extra flags.  The attention kernel keeps its matrix-core
# accumulators in ordinary VGPRs (gfx950 allows either file): with them in
# AGPRs the compiler copies the output tile between the files around every
# online-softmax update.
EXTRA_FLAGS = {"csa2_attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


# Host-only sanitizers: each -fsanitize= goes to the host pass alone.
SANITIZE_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                  "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZE_BUILD = os.path.join(BUILD, "sanitize")
SANITIZE_LIB = os.path.join(BUILD, "libcsa2_sanitize.so")


def _compile(src: str, sanitize: bool = False) -> str:
    out_dir = SANITIZE_BUILD if sanitize else BUILD
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    flags = HIPCC_FLAGS + (SANITIZE_FLAGS if sanitize else [])
    cmd = [_hipcc(), *flags, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if errs.strip():
        print(errs, file=sys.stderr)
    return obj


def build(verbose: bool = True, sanitize: bool = False) -> str:
    """Compiles every source and links the shared library; returns its path."""
    os.makedirs(SANITIZE_BUILD if sanitize else BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    lib = SANITIZE_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    link_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"] \
        if sanitize else []
    cmd = [_hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", *link_san, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])

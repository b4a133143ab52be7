"""Build libbsattn.so in-tree with hipcc for gfx950.

Every translation unit is compiled to an object file (in parallel) under
_build/ at the repository root, then linked into
block_sparse_attention_bsattn_amd/libbsattn.so.  HIP code is built with
packed-fp32 instructions disabled.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbsattn.so")

SOURCES = ["mask.hip", "compact.hip", "plan.hip", "fwd.hip", "fwd_bf16_t128.hip", "fwd_bf16_d64_t64.hip",
           "calib.hip", "energy_bf16_d128.hip", "reorder.hip", "repetition.hip", "rowcos_bf16_d128.hip", "mfma_ceiling.hip",
           "api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbsattn)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
            f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]


def hip_flags():
    return [f"--offload-arch={ARCH}", "-x", "hip",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-ffp-contract=fast", "-munsafe-fp-atomics"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags()
    if src.endswith(".hip"):
        cmd += hip_flags()
    else:
        cmd += ["-x", "c++"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the GPU-only target feature; that warning is
    # expected and harmless, anything else is shown
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libbsattn.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


CAPI_SRC = os.path.join(ROOT, "tests", "capi", "fwd_driver.c")
CAPI_EXE = os.path.join(ROOT, "tests", "capi", "fwd_driver")


def build_capi_driver(verbose: bool = False) -> str:
    """Compile the plain-C consumer of the library that the C-ABI test runs
    (C11, gcc, the HIP runtime's C API; no HIP device code)."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for tests/capi/fwd_driver.c")
    rocm_lib = "/opt/rocm/lib"
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           f"-I{INCLUDE}", CAPI_SRC, "-o", CAPI_EXE + ".tmp", f"-L{PKG}", "-lbsattn",
           f"-L{rocm_lib}", "-lamdhip64", f"-Wl,-rpath,{rocm_lib}",
           "-Wl,-rpath,$ORIGIN/../../block_sparse_attention_bsattn_amd"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("C driver build failed:\n" + r.stdout + r.stderr)
    os.replace(CAPI_EXE + ".tmp", CAPI_EXE)
    return CAPI_EXE


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

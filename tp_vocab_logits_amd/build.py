"""Build libhg.so (the HIP kernels and the C ABI) in-tree for gfx950, the
``_hgcall`` extension (fast-call Python wrappers of the per-call entry points)
and ``tests/c_client/hg_client`` (a plain C client of the ABI).

Usage: ``python -m tp_vocab_logits_amd.build`` (or ``__graft_entry__.build()``).
Always recompiles; each result replaces the previous file atomically.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import sysconfig
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhg.so")
SOURCES = ["hg_api.cpp", "hg_kernels.hip", "hg_lmhead.hip", "hg_static.hip"]
ARCH = "gfx950"
FASTCALL = os.path.join(PKG, "_hgcall" + sysconfig.get_config_var("EXT_SUFFIX"))
REF_LIB = os.path.join(PKG, "libhgref.so")  # the benchmark's reference streaming kernel
C_CLIENT_DIR = os.path.join(ROOT, "tests", "c_client")
C_CLIENT = os.path.join(C_CLIENT_DIR, "hg_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: cannot build libhg.so")


def compile_command(output: str) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
        # keep the compiler from forming packed-FP32 instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC, "-x", "hip",
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", output,
    ]


def build_fastcall(verbose: bool = False) -> str:
    """Compile the _hgcall extension (plain C, host only) and return its path."""
    fd, tmp = tempfile.mkstemp(prefix="_hgcall.", suffix=".so.tmp", dir=PKG)
    os.close(fd)
    try:
        cmd = [os.environ.get("CC", "gcc"), "-O2", "-shared", "-fPIC", "-Wall", "-Wextra",
               "-I", sysconfig.get_paths()["include"], os.path.join(CSRC, "hg_fastcall.c"),
               "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("_hgcall build failed:\n" + (res.stderr or res.stdout))
        os.chmod(tmp, 0o755)
        os.replace(tmp, FASTCALL)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return FASTCALL


def build_c_client(verbose: bool = False) -> str:
    """Compile the plain C client of the ABI (tests/c_client/hg_client.c, host
    code only, linked against libhg.so and the HIP runtime) and return its
    path. Needs libhg.so to exist."""
    fd, tmp = tempfile.mkstemp(prefix="hg_client.", suffix=".tmp", dir=C_CLIENT_DIR)
    os.close(fd)
    try:
        cmd = [os.environ.get("CC", "gcc"), "-O2", "-std=c11", "-Wall", "-Wextra",
               "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I", os.path.join(ROCM, "include"),
               os.path.join(C_CLIENT_DIR, "hg_client.c"), "-o", tmp,
               "-L", PKG, "-l:libhg.so", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
               "-Wl,-rpath,$ORIGIN/../../tp_vocab_logits_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hg_client build failed:\n" + (res.stderr or res.stdout))
        os.chmod(tmp, 0o755)
        os.replace(tmp, C_CLIENT)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return C_CLIENT


def build_ref(verbose: bool = False) -> str:
    """Compile libhgref.so: the reference streaming kernel bench.py times beside
    the gather (hg_stream_ref.hip; not part of libhg.so's ABI)."""
    fd, tmp = tempfile.mkstemp(prefix="libhgref.", suffix=".so.tmp", dir=PKG)
    os.close(fd)
    try:
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
               "-fvisibility=hidden", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-x", "hip", os.path.join(CSRC, "hg_stream_ref.hip"), "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("libhgref.so build failed:\n" + (res.stderr or res.stdout))
        os.replace(tmp, REF_LIB)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return REF_LIB


def build(verbose: bool = False) -> str:
    """Compile libhg.so, the _hgcall extension and the C client; return
    libhg.so's path. Raises on a compiler error."""
    build_fastcall(verbose)
    fd, tmp = tempfile.mkstemp(prefix="libhg.", suffix=".so.tmp", dir=PKG)
    os.close(fd)
    try:
        cmd = compile_command(tmp)
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        # hipcc's host pass does not know the packed-fp32 feature and says so
        noise = [ln for ln in (res.stderr or "").splitlines()
                 if ln.strip() and "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
        if res.returncode != 0:
            raise RuntimeError("libhg.so build failed:\n" + (res.stderr or res.stdout))
        if verbose and noise:
            print("\n".join(noise), file=sys.stderr)
        os.replace(tmp, LIB)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    build_c_client(verbose)
    build_ref(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

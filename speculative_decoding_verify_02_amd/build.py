"""Compile libverify_attn.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m speculative_decoding_verify_02_amd.build
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libverify_attn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["verify_attn.hip", "block_table.hip", "splitkv_fwd.hip", "splitkv_mla_fp8.hip", "splitkv_tile.hip",
           "combine.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # hipcc's own packed-fp32 code generation is switched off for every HIP source
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: with AGPR accumulators the online
    # softmax rescale copies every O register out and back each key block
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd: list, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")


# Host code under AddressSanitizer and UndefinedBehaviorSanitizer, for the CPU tests of
# the C ABI (which never reach a kernel launch).  Every sanitizer flag applies to the
# host side only; the device code is built as usual.
HOST_SANITIZER_FLAGS = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split() + [
    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> Optional[str]:
    """The compiler's shared AddressSanitizer runtime (it carries the UBSan handlers too),
    to preload into a process that loads the sanitized library; None if absent."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    hits = sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")) +
                  glob.glob(os.path.join(root, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def build_host_sanitized(out_path: str, extra_sources=(), verbose: bool = False) -> str:
    """Compile the library's host-side sources (argument checks, planning, workspace
    sizing, the block-table and combine launchers) with their host code under ASan +
    UBSan into out_path, together with `extra_sources` (the caller's stand-in for the
    split-KV launcher, whose kernels such a build leaves out).  Load it with
    sanitizer_runtime() preloaded."""
    sources = [os.path.join(CSRC, s) for s in ("verify_attn.hip", "block_table.hip", "combine.hip")]
    sources += list(extra_sources)
    flags = [f for f in HIPCC_FLAGS if f != "-shared"] + ["-Xarch_host", "-g"]
    objdir = tempfile.mkdtemp(prefix="va_hostsan_")
    try:
        objs = [os.path.join(objdir, f"{i}.o") for i in range(len(sources))]
        cmds = [[hipcc(), *flags, *HOST_SANITIZER_FLAGS, "-c", "-I", INCLUDE, "-I", CSRC, s, "-o", o]
                for s, o in zip(sources, objs)]
        workers = max(1, min(len(cmds), os.cpu_count() or 1, 8))
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
            for f in [pool.submit(_run, c, verbose) for c in cmds]:
                f.result()
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SANITIZER_FLAGS, *objs,
              "-o", out_path], verbose)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return out_path


C_CALLER_SRC = os.path.join(ROOT, "tests", "c_abi", "verify_c_caller.c")
C_CALLER_PATH = os.path.join(ROOT, "tests", "c_abi", "verify_c_caller")


def build_c_caller(out_path: str = C_CALLER_PATH, verbose: bool = False) -> str:
    """Compile the plain C caller of the library (tests/c_abi/verify_c_caller.c) with the
    host C compiler against include/verify_attn.h, the in-tree library and the HIP
    runtime's C API.  Returns the executable's path."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no host C compiler")
    _run([cc, "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
          "-I", INCLUDE, "-I", os.path.join(rocm, "include"), C_CALLER_SRC,
          "-L", PKG, "-lverify_attn", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
          f"-Wl,-rpath,{PKG}:{os.path.join(rocm, 'lib')}", "-o", out_path], verbose)
    return out_path


def build(verbose: bool = False) -> str:
    """Compile every HIP source into LIB_PATH (always recompiles).  Returns the path.

    Each source compiles to its own object in parallel (no source calls device code
    of another, so no relocatable device code is needed); one hipcc call links them."""
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    objdir = tempfile.mkdtemp(prefix="va_build_")
    try:
        objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[hipcc(), *compile_flags, "-c", "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        workers = max(1, min(len(cmds), os.cpu_count() or 1, 8))
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
            for f in [pool.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = LIB_PATH + ".tmp"
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, LIB_PATH)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

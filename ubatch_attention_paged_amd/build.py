"""Build libkvattn.so in-tree with hipcc for gfx950.

    python ubatch_attention_paged_amd/build.py              # libkvattn.so
    python ubatch_attention_paged_amd/build.py --sanitize   # libkvattn_san.so, host code under ASan/UBSan

(run by path: importing the package loads the library, which fails when an
older build lacks a newer symbol).

Compiles csrc/*.cpp and csrc/*.hip into one shared library next to this
file.  Packed-FP32 instructions are disabled for the device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libkvattn.so")
SOURCES = ["host_core.cpp", "api.cpp", "sched.cpp", "kernels_commit.hip", "kernels_state.hip", "attn_valu.hip", "attn_mfma.hip",
           "attn_both.hip", "attend_static.hip", "probes.hip"]
ARCH = os.environ.get("KVATTN_OFFLOAD_ARCH", "gfx950")


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


# Host-only sanitizer build (address + undefined behaviour) of the same
# sources: every -fsanitize flag is scoped to the host compilation, the GPU
# code is built as usual.  The result is a separate library for CPU test
# runs (the host half: batch intake, split, placement, planner, scheduler);
# see sanitize_env() for how to load it.
SAN_LIB = os.path.join(HERE, "libkvattn_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-shared-libsan"]


def sanitizer_runtime() -> str:
    """clang's shared address-sanitizer runtime (it must be preloaded into
    an uninstrumented interpreter)."""
    import glob
    cands = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(hipcc())), "llvm", "lib", "clang", "*",
                                          "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not cands:
        raise RuntimeError("clang's libclang_rt.asan-x86_64.so not found")
    return cands[-1]


def sanitize_env() -> dict:
    """Environment for running the CPU tests against SAN_LIB."""
    env = dict(os.environ)
    env["LD_PRELOAD"] = sanitizer_runtime()
    env["KVATTN_LIB"] = SAN_LIB
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"   # the interpreter itself is not instrumented
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source (always; a stale library is never reused here)."""
    out = SAN_LIB if sanitize else LIB
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O1" if sanitize else "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function", "-Wno-unused-result",
           "-I", INCLUDE, "-I", CSRC, "-o", tmp] + (SAN_FLAGS if sanitize else []) + \
          [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(errs))
    if verbose and errs:
        print("\n".join(errs), file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))

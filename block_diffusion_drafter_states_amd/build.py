"""Compile the HIP sources of the DFlash C-ABI library for gfx950.

    python -m block_diffusion_drafter_states_amd.build

produces ``block_diffusion_drafter_states_amd/libdflash.so`` in the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libdflash.so")
ARCH = os.environ.get("DFLASH_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


PROBE_OUT = os.path.join(HERE, "libdflash_probe.so")


def _compile(src: str, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-shared", "-fPIC",
           # packed fp32 VALU forms are kept out of the generated code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"), "-o", tmp, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    os.replace(tmp, out)


SANITIZED_OUT = os.path.join(ROOT, "_build", "libdflash_hostsan.so")


def build_host_sanitized(verbose: bool = False) -> str:
    """The C ABI with AddressSanitizer and UndefinedBehaviorSanitizer on its host code only
    (argument validation, launch planning, workspace carving); the device code is built as
    usual.  Loaded by the host-only tests with the sanitizer runtime preloaded.  Returns the
    path of the library (``_build/libdflash_hostsan.so``)."""
    os.makedirs(os.path.dirname(SANITIZED_OUT), exist_ok=True)
    tmp = SANITIZED_OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-shared", "-fPIC",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-Xarch_host", "-shared-libsan",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument",
           "-I", os.path.join(ROOT, "include"), "-o", tmp, os.path.join(CSRC, "dflash.hip")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building the host-sanitized library")
    os.replace(tmp, SANITIZED_OUT)
    return SANITIZED_OUT


def sanitizer_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (to preload)."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    llvm = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "lib", "clang")
    for ver in sorted(os.listdir(llvm)) if os.path.isdir(llvm) else []:
        cand = os.path.join(llvm, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(cand):
            return cand
    raise RuntimeError("AddressSanitizer runtime not found")


def build(verbose: bool = False) -> str:
    """libdflash.so (the C ABI) and libdflash_probe.so (the benchmark's bandwidth / MFMA probes)."""
    _compile(os.path.join(CSRC, "dflash.hip"), OUT, verbose)
    _compile(os.path.join(CSRC, "probe.hip"), PROBE_OUT, verbose)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))

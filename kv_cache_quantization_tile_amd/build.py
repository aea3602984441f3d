"""Build the KVarN HIP library in-tree: kv_cache_quantization_tile_amd/libkvarn.so, and the
benchmark's streaming-read probe beside it (libkvarn_probe.so, measurement only).

Runs hipcc for gfx950 on every call (the build is a few seconds). Usable as a script:
    python -m kv_cache_quantization_tile_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkvarn.so")
SOURCES = ["api.hip", "quantize.hip", "decode.hip", "mq.hip"]
PROBE_LIB = os.path.join(PKG, "libkvarn_probe.so")
PROBE_SOURCES = ["probe/stream_read.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed-FP32 VALU forms stay out of the generated code (hipcc emits them from plain
    # float code otherwise)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core results straight into VGPRs (no accumulation-register copies)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-result", "-fvisibility=hidden",
]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the KVarN library needs ROCm to build")
    return exe


def _compile(sources, out: str, verbose: bool, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, *extra, "-I", os.path.join(ROOT, "include"),
           *[os.path.join(CSRC, s) for s in sources], "-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    log = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + log)
    if verbose and log.strip():
        print(log, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libkvarn.so and the probe into libkvarn_probe.so (each
    atomically replaced). Returns the library's path."""
    _compile(SOURCES, LIB, verbose)
    _compile(PROBE_SOURCES, PROBE_LIB, verbose)
    return LIB


def build_variant(out: str, extra_flags, verbose: bool = False) -> str:
    """The same library built to `out` with extra hipcc flags (tests build instrumented
    variants this way); the in-tree libkvarn.so is untouched."""
    return _compile(SOURCES, out, verbose, extra=list(extra_flags))


if __name__ == "__main__":
    print(build(verbose=True))

"""The ABI validation layer under AddressSanitizer (host code only, no GPU): the library is
rebuilt with ASan instrumenting its host side (argument checks, sizing, launch set-up; the
device code is compiled as usual) and tests/test_abi_cpu.py runs against that build in a child
process with the clang ASan runtime loaded first. Any heap, stack or global out-of-bounds
access, use-after-free or double free in the host code aborts the child with a report."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from kv_cache_quantization_tile_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# each sanitizer flag applies to the host compilation only
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
             "-shared-libasan"]


def _asan_runtime():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(exe)))
    hits = sorted(glob.glob(os.path.join(rocm, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


@pytest.fixture(scope="module")
def asan_lib(tmp_path_factory):
    rt = _asan_runtime()
    if rt is None or not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc or the clang ASan runtime is not installed")
    out = str(tmp_path_factory.mktemp("asan") / "libkvarn_asan.so")
    B.build_variant(out, HOST_ASAN)
    return out, rt


def _child_env(lib, rt):
    env = dict(os.environ)
    # the ASan runtime must be the first preloaded library; anything already listed stays
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1"
    env["KVARN_LIBRARY"] = lib
    return env


def test_asan_build_is_instrumented(asan_lib):
    lib, rt = asan_lib
    code = ("import ctypes; ctypes.CDLL(None)['__asan_address_is_poisoned']; "
            "from kv_cache_quantization_tile_amd import kvarn as K; "
            f"assert K._LIB_PATH == {lib!r}; "
            "assert K.lib.kvarn_abi_version() == 2; print('asan-ok')")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_child_env(lib, rt),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "asan-ok" in r.stdout, r.stdout + r.stderr
    nm = shutil.which("nm")
    if nm:
        syms = subprocess.run([nm, "-D", lib], capture_output=True, text=True).stdout
        assert "__asan_report" in syms


def test_abi_cpu_suite_under_asan(asan_lib):
    lib, rt = asan_lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=_child_env(lib, rt), capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr
    assert " passed" in r.stdout

"""Host AddressSanitizer run of the C-ABI layer (CPU only).

The argument-validation, workspace-layout and split-heuristic code of the host layer (abi.hip)
is built with AddressSanitizer on its host side only (the device code is built as usual), linked
with the library's other objects, and the CPU ABI and binding tests are run against that build
in a child process with the sanitizer runtime preloaded. Any heap, stack or global overflow, or
use after free, in the host layer on those paths ends the child with a sanitizer report.
"""
import glob
import os
import subprocess
import sys

import pytest

from mla_varlen_prefill_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OBJ_DIR = os.path.join(_build.PKG_DIR, "_build")
ASAN_DIR = os.path.join(OBJ_DIR, "asan")
OTHER_OBJS = [os.path.join(OBJ_DIR, s.replace(".hip", ".o")) for s in _build.SOURCES if s != "abi.hip"]


def _asan_runtime():
    hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return hits[0] if hits else None


def _build_asan_library() -> str:
    cc = _build.hipcc()
    os.makedirs(ASAN_DIR, exist_ok=True)
    obj = os.path.join(ASAN_DIR, "abi_asan.o")
    lib = os.path.join(ASAN_DIR, "libmla_prefill_asan.so")
    flags = [f for f in _build.compile_flags() if f != "-O3"]
    # the sanitizer applies to the host compilation only; device code is unaffected
    cmd = [cc, *flags, "-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
           "-c", os.path.join(_build.CSRC, "abi.hip"), "-o", obj]
    subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    subprocess.run([cc, f"--offload-arch={_build.ARCH}", "-shared", "-fPIC", obj, *OTHER_OBJS, "-o", lib],
                   check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    return lib


@pytest.mark.skipif(not all(os.path.exists(o) for o in OTHER_OBJS), reason="library objects not built")
@pytest.mark.skipif(_asan_runtime() is None, reason="no clang AddressSanitizer runtime")
def test_abi_host_layer_under_address_sanitizer():
    lib = _build_asan_library()
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib], check=True, capture_output=True, text=True).stdout
    assert "__asan_report_load" in nm, "the host layer was not instrumented"
    env = dict(os.environ)
    env.update(MLA_PREFILL_LIBRARY=lib, LD_PRELOAD=_asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1:exitcode=86")
    tests = [os.path.join(ROOT, "tests", "test_abi_cpu.py"), os.path.join(ROOT, "tests", "test_binding_cpu.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert "AddressSanitizer" not in r.stderr, tail
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail

"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code.

Two CPU-only runs, each in a child process with the sanitizer runtime
preloaded (Python itself is not instrumented):
  * the fp64 oracle compiled by gcc with -fsanitize=address,undefined, running
    the oracle pins (tests/test_oracle_pins.py);
  * libfsa with its host code (argument checks, planning, workspace layout)
    compiled by hipcc with address and undefined-behaviour instrumentation on
    the host side only, running the ABI suite (tests/test_abi.py) -- which
    makes no GPU call.
Any sanitizer report aborts the child (halt_on_error), failing the test.
"""

import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_child(code, preload, tmp_path):
    env = dict(os.environ, LD_PRELOAD=preload, **SAN_ENV)
    res = subprocess.run([sys.executable, "-c", code], cwd=str(tmp_path), env=env,
                         capture_output=True, text=True, timeout=900)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "runtime error" not in res.stderr and "ERROR: AddressSanitizer" not in res.stderr, tail
    return res.stdout


def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = str(tmp_path / "liboracle_san.so")
    src = os.path.join(ROOT, "oracle", "fsa_oracle.c")
    cmd = ["gcc", "-O1", "-g", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", src, "-o", lib, "-lm"]
    subprocess.run(cmd, check=True)
    code = (f"import sys; sys.path.insert(0, {ROOT!r})\n"
            "import oracle, pytest\n"
            f"oracle._LIB_PATH = {lib!r}\n"
            f"rc = pytest.main(['-q', '-x', '-p', 'no:cacheprovider', "
            f"{os.path.join(ROOT, 'tests', 'test_oracle_pins.py')!r}])\n"
            f"assert oracle._lib._name == {lib!r}, oracle._lib._name\n"
            "sys.exit(rc)\n")
    out = _run_child(code, f"{asan}:{ubsan}", tmp_path)
    assert " passed" in out


def test_libfsa_host_code_under_asan_and_ubsan(tmp_path):
    rts = glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not rts:
        pytest.skip("clang sanitizer runtime not installed")
    from top_block_sparse_amd import build as B
    objs_dir = os.path.join(ROOT, "top_block_sparse_amd", "_build")
    others = [os.path.join(objs_dir, s.replace(".hip", ".o")) for s in B.SOURCES
              if s != "fsa_api.hip"]
    if not all(os.path.exists(o) for o in others):
        B.build_library()
    api_obj = str(tmp_path / "fsa_api_san.o")
    lib = str(tmp_path / "libfsa_san.so")
    src = os.path.join(B.CSRC, "fsa_api.hip")
    cmd = [B.hipcc(), f"--offload-arch={B.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"),
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-c", src, "-o", api_obj]
    subprocess.run(cmd, check=True, capture_output=True)
    link = [B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", api_obj, *others, "-o", lib,
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-shared-libsan"]
    subprocess.run(link, check=True, capture_output=True)
    code = (f"import sys; sys.path.insert(0, {ROOT!r})\n"
            "from top_block_sparse_amd import _lib\n"
            "import pytest\n"
            f"_lib.LIB_PATH = {lib!r}\n"
            f"rc = pytest.main(['-q', '-x', '-p', 'no:cacheprovider', "
            f"{os.path.join(ROOT, 'tests', 'test_abi.py')!r}])\n"
            f"assert _lib._lib._name == {lib!r}, _lib._lib._name\n"
            "sys.exit(rc)\n")
    out = _run_child(code, sorted(rts)[-1], tmp_path)
    assert " passed" in out

"""AddressSanitizer and UndefinedBehaviorSanitizer on the CPU side: the
oracle, with all its pins, and the library's host code (argument validation,
workspace sizing, the rejections of the C ABI), each built with the
sanitizers into a temporary directory and run in a child process.  Any
sanitizer report fails the test.  No GPU is used: the C ABI validates its
arguments before any HIP call, and the ABI tests only take those paths.
"""
import glob
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1", "OMP_NUM_THREADS": "2"}

_RUNNER = r"""
import sys
sys.path[:0] = [%r, %r]
import oracle, oracle_pins
orc = oracle.OracleLib(%r)
for pin in oracle_pins.ALL_PINS:
    pin(orc)
print("ALL_PINS_PASSED")
"""


def _instrumented(so):
    """The library calls into the ASan and UBSan runtimes."""
    syms = subprocess.run(["nm", "-D", so], capture_output=True, text=True, check=True).stdout
    return "__asan_report" in syms and "__ubsan_handle" in syms


def _reports(text):
    return [l for l in text.splitlines()
            if "AddressSanitizer" in l or "runtime error:" in l or "LeakSanitizer" in l]


def test_oracle_pins_under_asan_ubsan(tmp_path):
    so = oracle.build_variant(oracle.source_text(), str(tmp_path), "oracle_san",
                              ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                               "-fno-omit-frame-pointer", "-g"])
    assert _instrumented(so)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True, check=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan, **SAN_ENV)
    res = subprocess.run([sys.executable, "-c", _RUNNER % (ROOT, HERE, so)], capture_output=True,
                         text=True, timeout=600, env=env)
    out = res.stdout + res.stderr
    assert res.returncode == 0 and "ALL_PINS_PASSED" in res.stdout, out[-3000:]
    assert not _reports(out), _reports(out)[:5]


def _clang_asan_runtime():
    libs = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    return libs[0] if libs else None


def test_host_api_under_asan_ubsan(tmp_path):
    from block_sparse_long_index_amd import build as B
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("no clang ASan runtime in this ROCm install")
    # the C ABI's source with the host sanitizers (device code unchanged),
    # linked with the kernels' objects of the regular build
    B.build_library()
    api = os.path.join(B.CSRC, "msa_api.hip")
    obj = str(tmp_path / "msa_api_san.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    subprocess.check_call([B.HIPCC] + B.FLAGS + san + ["-g", "-c", api, "-o", obj])
    others = [o for o in glob.glob(os.path.join(B.BUILD_DIR, "*.hip.o"))
              if not os.path.basename(o).startswith("msa_api")]
    assert others, "the regular build's objects are missing"
    so = str(tmp_path / "libmsa_san.so")
    subprocess.check_call([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan",
                           "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                           "-fsanitize=undefined", "-o", so, obj] + others)
    assert _instrumented(so)
    env = dict(os.environ, LD_PRELOAD=rt, MSA_LIB_PATH=so, **SAN_ENV)
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(HERE, "test_abi.py")], capture_output=True, text=True,
                         timeout=600, env=env, cwd=ROOT)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-3000:]
    assert not _reports(out), _reports(out)[:5]

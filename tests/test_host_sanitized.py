"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

1. A sanitizer build of the oracle (oracle/qgemm_oracle.c, gcc) runs every
   oracle pin test in a child process.
2. A build of libqgemm.so with host-side instrumentation (hipcc, each
   -fsanitize behind -Xarch_host; the gfx950 device code is built as usual)
   runs the host ABI tests: symbol exports and every validation path.

An instrumented library needs its sanitizer runtime loaded first, hence
LD_PRELOAD in the child (gcc's libasan for the oracle, clang's shared ASan
runtime for hipcc's objects).  Any out-of-bounds access, use of freed memory,
signed overflow, invalid shift or misaligned access aborts the child.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PIN_FILES = ["test_oracle_pins.py", "test_oracle_fp8_pins.py", "test_oracle_w8a16_pins.py",
             "test_oracle_mha_pins.py"]


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


PRELOADED = bool(os.environ.get("LD_PRELOAD")) or os.path.exists("/etc/ld.so.preload")


@pytest.mark.skipif(PRELOADED, reason="a preload is already configured for this process tree; not overriding it")
def test_oracle_pins_under_asan_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no ASan runtime for gcc")
    sys.path.insert(0, ROOT)
    from oracle import build
    lib = build.build(out=str(tmp_path / "liboracle_san.so"), sanitize=True)
    env = dict(os.environ, QGEMM_ORACLE_LIB=lib, LD_PRELOAD=asan, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"]
    cmd += [os.path.join(HERE, f) for f in PIN_FILES]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail


def _clang_asan_runtime():
    import glob
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


@pytest.mark.skipif(PRELOADED, reason="a preload is already configured for this process tree; not overriding it")
def test_abi_host_under_asan_ubsan(tmp_path):
    rt = _clang_asan_runtime()
    if rt is None:
        pytest.skip("no shared ASan runtime in the ROCm toolchain")
    sys.path.insert(0, ROOT)
    from bit_quantized_gemm_qgemm_amd import build
    lib = build.build(out=str(tmp_path / "libqgemm_san.so"), host_sanitize=True)
    env = dict(os.environ, QGEMM_LIB=lib, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(HERE, "test_abi_host.py")]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in tail and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail

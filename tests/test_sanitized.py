"""The CPU suite again under AddressSanitizer and UndefinedBehaviorSanitizer.

Two runs, one per sanitizer runtime (gcc's and clang's cannot share a
process):
  * library: libqlora_san.so, whose host code (argument checks, plans,
    workspace carving in api.cpp and noalloc.hip) is built with clang's
    -fsanitize=address,undefined, loaded through QLORA_LIB with the clang ASan
    runtime preloaded;
  * oracle: libqlora_oracle_san.so, the oracle's C built with gcc's
    -fsanitize=address,undefined (QLORA_ORACLE_SANITIZE=1), with libasan and
    libubsan preloaded.
Each run is `pytest -m "not gpu"` in a child process; inside it,
test_runtime_is_sanitized checks that the runtime and the sanitized library
are the ones loaded.  UBSan findings abort (-fno-sanitize-recover).  Leak
checking is off: the interpreter and the HIP runtime keep allocations until
exit by design.
"""
import ctypes
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_LIB = os.path.join(ROOT, "bit_quantized_lora_quantize_amd", "libqlora_san.so")
INNER = os.environ.get("QLORA_SANITIZED_RUN")


def _clang_asan():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _gcc_runtime(name):
    try:
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                           check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _run_suite(env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-m", "not gpu", "-q",
           "-x", "-p", "no:cacheprovider"]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    tail = "\n".join((res.stdout + res.stderr).splitlines()[-40:])
    assert res.returncode == 0, f"sanitized run failed (exit {res.returncode}):\n{tail}"
    assert " passed" in res.stdout, tail


@pytest.mark.skipif(INNER is not None, reason="inside a sanitized run")
def test_suite_with_sanitized_library():
    rt = _clang_asan()
    if rt is None:
        pytest.skip("clang ASan runtime not found")
    if not os.path.exists(SAN_LIB):
        pytest.skip("libqlora_san.so not built (python -m bit_quantized_lora_quantize_amd.build_lib)")
    _run_suite({"LD_PRELOAD": rt, "QLORA_LIB": SAN_LIB, "QLORA_SANITIZED_RUN": "library"})


@pytest.mark.skipif(INNER is not None, reason="inside a sanitized run")
def test_suite_with_sanitized_oracle():
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc sanitizer runtimes not found")
    sys.path.insert(0, ROOT)
    from oracle import oracle as orc
    orc.build(sanitize=True)
    _run_suite({"LD_PRELOAD": f"{asan} {ubsan}", "QLORA_ORACLE_SANITIZE": "1",
                "QLORA_SANITIZED_RUN": "oracle"})


@pytest.mark.skipif(INNER is None, reason="only inside a sanitized run")
def test_runtime_is_sanitized():
    proc = ctypes.CDLL(None)
    assert hasattr(proc, "__asan_init"), "no ASan runtime in this process"
    if INNER == "library":
        from bit_quantized_lora_quantize_amd import _lib
        assert _lib.LIB_PATH == SAN_LIB
        assert hasattr(_lib.lib(), "qlora_abi_version")
        assert hasattr(proc, "__ubsan_handle_add_overflow")
    else:
        from oracle import oracle as orc
        assert orc._LIB.endswith("libqlora_oracle_san.so")
        orc._load()
        assert hasattr(proc, "__ubsan_handle_add_overflow")

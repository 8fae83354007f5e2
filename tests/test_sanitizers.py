"""CPU sanitizer runs (no GPU):

1. the oracle (oracle/qkvf_oracle.c) built with -fsanitize=address,undefined
   and every oracle and checker pin run against that build;
2. the C-ABI layer (kv_insert_amd/csrc/qkvf_api.cpp) built host-only with
   the same sanitizers, its device launches replaced by stubs
   (tests/sanitize/launch_stubs.cpp), driven through every entry point's
   refusal paths (tests/sanitize/refusals.cpp).

Any sanitizer report fails the run (-fno-sanitize-recover=all)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-O1", "-g"]
PINS = ["tests/test_oracle.py", "tests/test_oracle_attn2.py", "tests/test_oracle_layer_front.py",
        "tests/test_oracle_route.py", "tests/test_checker.py"]


def _asan_runtime() -> str:
    path = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("no ASan runtime for gcc here")
    return path


def _env(**extra):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:alloc_dealloc_mismatch=0:detect_odr_violation=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.update(extra)
    return env


@pytest.mark.slow
def test_oracle_pins_under_address_and_undefined_sanitizers(tmp_path):
    lib = tmp_path / "libqkvf_oracle_san.so"
    subprocess.check_call(["gcc", *SAN, "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
                           "-o", str(lib), os.path.join(ROOT, "oracle", "qkvf_oracle.c"), "-lm"])
    preload = _asan_runtime()
    if os.environ.get("LD_PRELOAD"):
        preload += ":" + os.environ["LD_PRELOAD"]
    env = _env(QKVF_ORACLE_LIB=str(lib), LD_PRELOAD=preload)
    # the sanitized build is the one the oracle loads, with ASan active
    probe = subprocess.run(
        [sys.executable, "-c",
         "import ctypes, oracle; L = oracle._load(); print(L._name); "
         "ctypes.CDLL(None).__asan_init; print(oracle.float_to_bf16(1.0))"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.splitlines()[0] == str(lib)
    run = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          *PINS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = run.stdout[-3000:] + run.stderr[-3000:]
    assert run.returncode == 0, out
    assert "runtime error" not in run.stderr and "ERROR: AddressSanitizer" not in run.stderr, out
    assert " passed" in run.stdout


@pytest.mark.slow
def test_c_abi_refusal_paths_under_address_and_undefined_sanitizers(tmp_path):
    exe = tmp_path / "refusals"
    csrc = os.path.join(ROOT, "kv_insert_amd", "csrc")
    subprocess.check_call(
        ["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
         "-I", csrc, "-I", "/opt/rocm/include", os.path.join(csrc, "qkvf_api.cpp"),
         os.path.join(ROOT, "tests", "sanitize", "launch_stubs.cpp"),
         os.path.join(ROOT, "tests", "sanitize", "refusals.cpp"),
         "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)])
    run = subprocess.run([str(exe)], env=_env(), capture_output=True, text=True, timeout=300)
    out = run.stdout[-3000:] + run.stderr[-3000:]
    assert run.returncode == 0, out
    assert "0 failures" in run.stdout, out
    assert "runtime error" not in run.stderr and "ERROR: AddressSanitizer" not in run.stderr, out

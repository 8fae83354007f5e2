"""The front from a C program that uses no PyTorch (tests/c_consumer/gpu_front.c):
its own device memory, stream and copies through the HIP runtime's C API,
qkvf_check, qkvf_prepare and two qkvf_run calls, compared with the oracle
like every other parity case.  Torch only writes the seeded inputs here."""
import os
import subprocess

import numpy as np
import pytest
import torch

import kv_insert_amd as qf
from kv_insert_amd import workloads as wl

from helpers import Case, check, say, to_bits

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def build_program(out: str) -> None:
    """gcc, on the host: the program is C11 against include/qkvf.h."""
    libdir = os.path.dirname(qf.LIB_PATH)
    res = subprocess.run(
        ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
         "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
         os.path.join(ROOT, "tests", "c_consumer", "gpu_front.c"),
         "-L", libdir, "-lqkvfront", "-Wl,-rpath," + libdir,
         "-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", out],
        capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]


def test_front_from_a_c_program_without_torch(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    qf.lib()  # raises if the library is not built
    exe = str(tmp_path / "gpu_front")
    build_program(exe)
    w = wl.C2   # 2 KV heads, 8 rows (4 K splits), consecutive slots across a page
    case = Case(w)
    to_bits(case.x).tofile(tmp_path / "x.bin")
    to_bits(case.W).tofile(tmp_path / "W.bin")
    case.positions.numpy().astype("<i8").tofile(tmp_path / "positions.bin")
    case.slots.numpy().astype("<i8").tofile(tmp_path / "slots.bin")
    case.cos_sin.numpy().astype("<f4").tofile(tmp_path / "cos_sin.bin")
    to_bits(case.cache).tofile(tmp_path / "cache.bin")
    say(f"C program {w.name} M={case.M} nkv={case.nkv} N={case.N}")
    run = subprocess.run(
        [exe, str(tmp_path), str(case.N), str(case.nkv), str(case.M),
         str(case.cos_sin.shape[0]), str(case.cache.shape[0])],
        capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-2000:]
    y = np.fromfile(tmp_path / "y.bin", dtype=np.uint16).reshape(case.M, case.N)
    cache = np.fromfile(tmp_path / "cache_out.bin", dtype=np.uint16).reshape(case.cache.shape)
    g = {"y": torch.from_numpy(y.view(np.int16)).view(torch.bfloat16),
         "kv_cache": torch.from_numpy(cache.view(np.int16)).view(torch.bfloat16)}
    print(check(case, g))

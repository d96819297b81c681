"""The C ABI used from C: tests/c/abi_check.c is compiled as C11 with gcc
against include/tp_mlp.h, linked to the in-tree libtpmlp.so, and run (host
calls only; no GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "megatron_tensor_transformer_rank_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_header_compiles_as_c_and_host_calls_answer(tmp_path):
    lib = os.path.join(PKG, "libtpmlp.so")
    assert os.path.exists(lib), "build the library first"
    exe = tmp_path / "abi_check"
    cmd = ["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{ROOT}/include", "-I/opt/rocm/include",
           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-o", str(exe), f"-L{PKG}", "-ltpmlp",
           f"-Wl,-rpath,{PKG}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "c abi ok" in r.stdout, r.stdout + r.stderr

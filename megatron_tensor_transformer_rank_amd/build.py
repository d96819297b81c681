"""Build libtpmlp.so (gfx950) in-tree with hipcc.

    python -m megatron_tensor_transformer_rank_amd.build
    python -m megatron_tensor_transformer_rank_amd.build --host-sanitize

Each ``csrc/*.hip`` file is compiled to an object under ``_build/`` (in
parallel) and the objects are linked into ``libtpmlp.so`` next to this file.
hipcc cross-compiles for gfx950, so this runs on a machine without a GPU.

``--host-sanitize`` builds ``_build/host_sanitize/libtpmlp.so`` instead: the
host code (argument validation, dispatch) instrumented with AddressSanitizer
and UndefinedBehaviorSanitizer, device code as usual.  It is for the host-only
ABI tests on a machine without a GPU, with clang's ASan runtime preloaded:

    LD_PRELOAD=$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so) \
    ASAN_OPTIONS=detect_leaks=0:verify_asan_link_order=0 UBSAN_OPTIONS=halt_on_error=1 \
    TPMLP_LIB=megatron_tensor_transformer_rank_amd/_build/host_sanitize/libtpmlp.so \
    python -m pytest -s tests/test_abi_host.py
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtpmlp.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 ops are disabled for device code (hipcc's host pass warns that it
# does not know the feature, which is harmless).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
CXXFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
            f"-I{INCLUDE}", f"-I{CSRC}"] + DEVICE_FLAGS


def sources():
    return sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


# host-side sanitizers only (each -fsanitize= right after -Xarch_host)
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, src[:-4] + ".o")
    cmd = [HIPCC, *CXXFLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", flush=True)
    return LIB


def build_host_sanitized(verbose: bool = True) -> str:
    out = os.path.join(BUILD, "host_sanitize")
    os.makedirs(out, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = list(ex.map(lambda f: _compile(f, out, SANITIZE + ["-O1", "-g"]), srcs))
    lib = os.path.join(out, "libtpmlp.so")
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libasan", "-o", lib, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {lib} (host code under ASan + UBSan)", flush=True)
    return lib


if __name__ == "__main__":
    if "--host-sanitize" in sys.argv[1:]:
        build_host_sanitized()
    else:
        build()
    sys.exit(0)

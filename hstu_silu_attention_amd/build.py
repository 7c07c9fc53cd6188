"""Build the HIP library libhstu.so in-tree with hipcc for gfx950.

Every HIP source is compiled with packed-FP32 instructions disabled (the
compiler would otherwise form v_pk_* float32 operations from ordinary float
code). The library exports the C ABI declared in include/hstu.h.

``python -m hstu_silu_attention_amd.build --sanitize`` builds libhstu_asan.so
instead: the same sources with AddressSanitizer and UndefinedBehaviorSanitizer on
the host code only (validation, the planner, the page pool; the GPU code is built
as usual), for running the CPU tests under the sanitizers:

    ASAN_OPTIONS=detect_leaks=0 HSTU_LIBRARY=$PWD/hstu_silu_attention_amd/libhstu_asan.so \
    LD_PRELOAD=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so) \
    python -m pytest tests -m "not gpu"
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libhstu.so")
LIB_SANITIZED = os.path.join(HERE, "libhstu_asan.so")
# host-side sanitizers only: each -fsanitize flag applies to the host compilation
SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SOURCES = ["hstu_abi.hip", "launch.hip", "gemm_bf16.hip", "attn_bf16.hip", "kernels_f32.hip", "pack.hip", "score.hip", "kv_pool.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    cc = hipcc()
    objdir = os.path.join(HERE, "_build_asan" if sanitize else "_build")
    os.makedirs(objdir, exist_ok=True)
    extra = SANITIZE if sanitize else []
    lib = LIB_SANITIZED if sanitize else LIB

    def compile_one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *common_flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = lib + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *(["-Xarch_host", "-shared-libsan"] if sanitize else []),
           *extra, "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))

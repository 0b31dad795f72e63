"""Build the DSA HIP library for gfx950 into long_context_sparse_fp8_amd/_lib/libdsa.so.

Every source is compiled with hipcc for gfx950 only, packed-fp32 VALU forms
disabled, and linked into one shared library exporting the C ABI of
include/dsa.h (all other symbols hidden).
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_lib")
OBJ_DIR = os.path.join(OUT_DIR, "obj")
LIB = os.path.join(OUT_DIR, "libdsa.so")
SOURCES = ["dsa_api.cpp", "cache_store.hip", "indexer.hip", "topk.hip", "sparse_mla.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]
# Sparse MLA: the compiler's MFMAs in their VGPR form (S^T is read by VALU
# code); the O^T accumulation is written as AGPR-form asm in the source.
SOURCE_FLAGS = {"sparse_mla.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in (r.stderr or "").splitlines()
                    if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if verbose and err.strip():
        print(err)
    return obj


def build(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    # the library must load with every symbol resolved: hipcc can drop a kernel's
    # host-side launch stub without an error (seen with an inline-asm operand of a
    # 256-bit vector type), which would only show when the library is loaded
    r = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({tmp!r}).dsa_abi_version()"],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{tmp} does not load:\n{r.stderr.strip()}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

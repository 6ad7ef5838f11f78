"""Build libtq.so in-tree with hipcc for gfx950.

    python -m kv_cache_vector_02_amd.build        # or __graft_entry__.build()

Every source is compiled to an object under _build/ (in parallel), then linked
into kv_cache_vector_02_amd/libtq.so.  It always rebuilds.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtq.so")

SOURCES = ["tq_api.cpp", "tq_codebook.cpp", "tq_encode.hip", "tq_encode2k.hip", "tq_decode.hip", "tq_retrieval.hip",
           "tq_polar.hip",
           "tq_testing.hip"]

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 VALU forms stay off (the compiler emits them from plain float code)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]
# decode kernels: matrix-core results straight into VGPRs (no AGPR read-back)
# encode: the epilogue loops must unroll fully (lane indices and plane bit
# positions are immediates); the default pragma threshold is below their size
EXTRA = {"tq_encode.hip": ["-mllvm", "-pragma-unroll-threshold=200000"],
         "tq_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "tq_retrieval.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        msg = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


SANITIZE_DIR = os.path.join(BUILD, "host_sanitized")
SANITIZED_LIB = os.path.join(SANITIZE_DIR, "libtq_host_sanitized.so")


def build_host_sanitized() -> str:
    """The library with its host code under AddressSanitizer and
    UndefinedBehaviorSanitizer (-Xarch_host: the device code is built as
    usual), for tests/test_host_sanitized.py.  Built outside the package
    directory; objects are rebuilt only when a source or header is newer."""
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    headers = [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".h")]
    headers += [os.path.join(ROOT, "include", h) for h in os.listdir(os.path.join(ROOT, "include"))]
    newest_header = max(os.path.getmtime(h) for h in headers)

    def one(src):
        obj = os.path.join(SANITIZE_DIR, os.path.basename(src) + ".o")
        path = os.path.join(CSRC, src)
        if os.path.exists(obj) and os.path.getmtime(obj) > max(os.path.getmtime(path), newest_header):
            return obj
        cmd = [hipcc(), *FLAGS, *EXTRA.get(src, []), *san, "-c", path, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            msg = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
            raise RuntimeError(f"sanitized build failed for {src}:\n{msg}")
        return obj

    jobs = min(len(SOURCES), int(os.environ.get("MAX_JOBS", "8")))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(one, SOURCES))
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-o", SANITIZED_LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    return SANITIZED_LIB


def asan_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (to preload into Python)."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime of the compiler was not found")
    return path


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

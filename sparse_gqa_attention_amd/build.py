"""Build libdsa.so (and the benchmark's libdsa_roofline.so) for gfx950 in-tree with hipcc.

Every HIP source is compiled with packed-FP32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); the C-ABI translation unit
is host code.  `python -m sparse_gqa_attention_amd.build` rebuilds.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
ROOFLINE_LIB = os.path.join(HERE, "libdsa_roofline.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["dsa_api.cpp", "indexer.hip", "topk.hip", "attention.hip", "cache_append.hip",
           "rmsnorm_rope.hip"]
ROOFLINE_SOURCES = ["roofline.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument"]


def _compile(src):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose=False):
    """Compile every source and link sparse_gqa_attention_amd/libdsa.so and libdsa_roofline.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + ROOFLINE_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        results = dict(zip(srcs, ex.map(_compile, srcs)))
    if verbose:
        for _, err in results.values():
            if err.strip():
                print(err, file=sys.stderr)
    _link([results[s][0] for s in SOURCES], LIB)
    _link([results[s][0] for s in ROOFLINE_SOURCES], ROOFLINE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

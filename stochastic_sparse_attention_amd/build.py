"""Build libsanta.so (gfx950) in-tree with hipcc.

    python -m stochastic_sparse_attention_amd.build
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsanta.so")
ARCH = os.environ.get("SANTA_OFFLOAD_ARCH", "gfx950")

# kernel sources, each compiled once per KV storage type (-DSANTA_KV=...)
KV_SOURCES = ["santa_prop.hip", "santa_prop_pass1.hip", "santa_prop_fused.hip", "santa_flash.hip", "santa_exact.hip"]
KV_TYPES = {"bf16": "uint16_t", "fp8": "uint8_t", "f32": "float"}
# sources built once: Bernoulli scoring (bf16 and e4m3 in one unit) and the
# allocation-free prop entry point (its static device workspace)
ONE_TYPE_SOURCES = ["santa_bernoulli.hip", "santa_static.hip"]
# host sources, compiled once
HOST_SOURCES = ["santa_api.cpp", "santa_dispatch.cpp"]
SOURCES = KV_SOURCES + ONE_TYPE_SOURCES + HOST_SOURCES
HEADERS = ["santa_device.h", "santa_score.h", "santa_launch.h", "santa_kernels.h", "santa_prop_body.h"]

COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed fp32 instructions are to be generated for the kernels
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose=False, jobs=None, out=None, defines=()):
    """Compile every source and link libsanta.so (or `out`).  `defines` adds
    preprocessor switches, e.g. ("SANTA_BF16_VALU",) builds the VALU scorer
    for bf16 instead of MFMA (used only for comparisons)."""
    lib = out or LIB
    objdir = os.path.join(HERE, "_build", "-".join(defines) or "default")
    os.makedirs(objdir, exist_ok=True)
    dflags = [f"-D{d}" for d in defines]

    def compile_one(job):
        src, kv = job
        stem = os.path.splitext(src)[0] + ("." + kv if kv else "")
        obj = os.path.join(objdir, stem + ".o")
        extra = [f"-DSANTA_KV={KV_TYPES[kv]}"] if kv else []
        cmd = [_hipcc(), *COMMON, *dflags, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src} ({kv or 'host'}):\n{r.stderr}")
        return obj

    jobs_list = ([(src, kv) for src in KV_SOURCES for kv in KV_TYPES] +
                 [(src, None) for src in ONE_TYPE_SOURCES + HOST_SOURCES])
    workers = jobs or min(len(jobs_list), os.cpu_count() or 4, 16)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(compile_one, jobs_list))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser()
    ap.add_argument("-v", action="store_true")
    ap.add_argument("--out", default=None)
    ap.add_argument("-D", action="append", default=[], dest="defines")
    a = ap.parse_args()
    print(build(verbose=a.v, out=a.out, defines=tuple(a.defines)))

"""Build libmoe_ffn.so (HIP, gfx950) in-tree with hipcc.

Every source is compiled for gfx950 only, with packed fp32 VALU instructions
disabled (the kernels never rely on them).
"""
import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_ffn.so")
SOURCES = ["api.hip", "repack.hip", "router.hip", "bucket.hip", "gemm.hip", "gemm_q4k.hip", "decode.hip", "combine.hip",
           "noalloc.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", f"--offload-arch={ARCH}", "-fno-gpu-rdc",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-mllvm", "-amdgpu-mfma-vgpr-form",
               "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
               "-I", INCLUDE, "-I", CSRC]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _compile(src, obj, verbose):
    cmd = [_hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


PROBE_LIB = os.path.join(PKG, "libmoe_probe.so")
PROBE_SOURCES = ["probe.hip"]


def _link(objs, out, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False, jobs: int = 6) -> str:
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    objs = [os.path.join(bdir, os.path.splitext(s)[0] + ".o") for s in srcs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda p: _compile(p[0], p[1], verbose), zip(srcs, objs)))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

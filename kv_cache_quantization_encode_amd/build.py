"""Build libtq.so (HIP kernels for gfx950 + host code + C ABI) in-tree with hipcc.

Usage: python kv_cache_quantization_encode_amd/build.py  (importing the package needs the built library,
so this file is run or loaded by path)
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtq.so")
SOURCES = ["tq_host.cpp", "tq_encode.hip", "tq_decode.hip", "tq_dequant.hip", "tq_stats.hip", "tq_probe.hip"]
ARCH = "gfx950"


def build(verbose: bool = False, extra=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
           # packed fp32 VALU ops stay off (host pass warns that it does not know the feature)
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp] + srcs + list(extra)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed (%d)" % r.returncode)
    if verbose and r.stderr:
        # print warnings other than the known packed-fp32 host-pass notice
        for line in r.stderr.splitlines():
            if "packed-fp32-ops" not in line:
                print(line)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

"""Build libuno.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc.

    python -m lossless_decoding_uno_amd.build      # or build() from Python

Every source is compiled for gfx950 only, with packed fp32 arithmetic switched
off; the sampler and tree files are additionally compiled without
floating-point contraction (their integer weights and scores come from
separately rounded fp32 ops).
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
OUT = os.path.join(HERE, "libuno.so")
PROBE_OUT = os.path.join(HERE, "libuno_probe.so")   # measurement probes (include/uno_probe.h)
BUILD_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["api.cpp", "sampler.hip", "elementwise.hip", "gemm.hip", "attention.hip", "tree.hip"]
PROBE_SOURCES = ["probes.hip"]
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]
PER_FILE = {"sampler.hip": ["-ffp-contract=off"], "tree.hip": ["-ffp-contract=off"]}


def _compile(src):
    obj = os.path.join(BUILD_DIR, src + ".o")
    cmd = [HIPCC] + COMMON + PER_FILE.get(src, []) + ["-x", "hip", "-c",
                                                     os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, out)


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], OUT)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_OUT)
    if verbose:
        print("built", OUT, "and", PROBE_OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

"""Build libddp.so (HIP, gfx950) in-tree with hipcc.

Flags: IEEE FP32 throughout (no FMA contraction, denormals kept, no fast
math) so every add and multiply is one correctly rounded binary32 operation;
packed-FP32 instructions disabled.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libddp.so")
SOURCES = ["plan.cpp", "common.hip", "reduce.hip", "accumulate.hip", "copy.hip", "params.hip",
           "noalloc.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wshadow",
          "-ffp-contract=off", "-fno-fast-math",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]
DEVICE = ["--offload-arch=" + ARCH, "-fno-gpu-flush-denormals-to-zero",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


PROBE_SRC = "probe.hip"
PROBE_LIB = os.path.join(HERE, "libddp_probe.so")


def _build_probe(verbose: bool) -> str:
    """The benchmark's access-pattern probe, a library of its own."""
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-x", "hip"] + DEVICE + COMMON + ["-shared", os.path.join(CSRC, PROBE_SRC),
                                                    "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def _compile(src: str, verbose: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(CSRC, src.rsplit(".", 1)[0] + ".o")
    # hidden visibility: only the DDP_API declarations of ddp.h are exported
    cmd = [HIPCC] + COMMON + ["-fvisibility=hidden", "-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"] + DEVICE
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel, one hipcc per source) and link
    libddp.so (and libddp_probe.so) next to this file."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = max(1, min(len(SOURCES), len(os.sched_getaffinity(0)), 16))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, verbose), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    _build_probe(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

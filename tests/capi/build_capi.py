"""Build tests/capi/capi_check (plain C against libddp.so's ABI, with the
oracle's C core linked as the reference; test infrastructure only)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "capi_check")


def build() -> str:
    lib_dir = os.path.join(ROOT, "gradient_allreduce_averaging_amd")
    ora_dir = os.path.join(ROOT, "oracle")
    tmp = BIN + ".tmp%d" % os.getpid()
    subprocess.check_call([
        "gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__",
        "-I" + os.path.join(ROOT, "include"), "-I/opt/rocm/include",
        os.path.join(HERE, "capi_check.c"), "-o", tmp,
        "-L" + lib_dir, "-lddp", "-L" + ora_dir, "-loracle_core",
        "-L/opt/rocm/lib", "-lamdhip64",
        "-Wl,-rpath,$ORIGIN/../../gradient_allreduce_averaging_amd:$ORIGIN/../../oracle:/opt/rocm/lib"])
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build())

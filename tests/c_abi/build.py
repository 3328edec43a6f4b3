"""Build tests/c_abi/_build/c_abi_check: a plain C program against
include/rar.h, librar.so and the HIP runtime (gcc, no hipcc, no torch)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIBDIR = os.path.join(ROOT, "ring_all_reduce_scatter_amd")
EXE = os.path.join(HERE, "_build", "c_abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "c_abi_check.c"), "-o", EXE,
           "-L", LIBDIR, "-lrar", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../../ring_all_reduce_scatter_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    return EXE


if __name__ == "__main__":
    print(build())

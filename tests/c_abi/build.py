"""Builds tests/c_abi/c_gpu_prepare (plain C99 + the HIP runtime + libwt.so)
in-tree. Called by the repository's build step, so that no test compiles."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
EXE = os.path.join(HERE, "c_gpu_prepare")


def build() -> str:
    libdir = os.path.join(ROOT, "bf16_fp8_weight_amd")
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "c_gpu_prepare.c"), "-o", EXE,
           f"-L{libdir}", "-l:libwt.so", f"-Wl,-rpath,{libdir}",
           f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    subprocess.run(cmd, check=True)
    return EXE


if __name__ == "__main__":
    print(build())

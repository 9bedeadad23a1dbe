"""Builds tests/helpers/abi_client (a plain C client of libdust.so) with gcc:
host code only, linked against the HIP runtime and the in-tree library."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_client.c")
EXE = os.path.join(HERE, "abi_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    lib_dir = os.path.join(ROOT, "token_activation_perturbation_amd")
    tmp = f"{EXE}.{os.getpid()}.tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-o", tmp, "-L", lib_dir, "-ldust", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{lib_dir}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build())

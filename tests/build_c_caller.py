"""Builds tests/c_abi_caller.c (a plain C program against include/ar.h and
the HIP runtime API) into tests/_build/ar_c_caller, linked to the in-tree
libtpdc_ar.so."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "tp_decode_comms_amd")
OUT = os.path.join(HERE, "_build", "ar_c_caller")


def build(verbose=False):
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I/opt/rocm/include",
           os.path.join(HERE, "c_abi_caller.c"), "-o", OUT,
           "-L" + PKG, "-ltpdc_ar", "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../tp_decode_comms_amd", "-Wl,-rpath,/opt/rocm/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))

"""Compile the plain C caller of the library (tests/c_driver/adq_c_driver.c)
against include/adq.h and the built libaddrmsnorm_dq.so.  Called by
__graft_entry__.build() after the library is built."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "adq_c_driver")


def build() -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(HERE, "adq_c_driver.c"), "-o", BIN,
           "-L", os.path.join(ROOT, "int4_dynamic_quantization_amd"), "-laddrmsnorm_dq",
           "-L", "/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../int4_dynamic_quantization_amd", "-Wl,-rpath,/opt/rocm/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"C driver build failed: {' '.join(cmd)}\n{res.stderr}")
    return BIN


if __name__ == "__main__":
    print(build())

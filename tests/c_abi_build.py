"""Build the plain host program tests/c_abi_driver.cpp (g++, no device code),
which calls libfa.so through include/fa.h with memory from hipMalloc."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_driver.cpp")
BIN = os.path.join(HERE, "_bin", "c_abi_driver")
PKG = os.path.join(ROOT, "exact_io_aware_44_amd")


def build(force: bool = False) -> str:
    if not force and os.path.exists(BIN) and os.path.getmtime(BIN) >= os.path.getmtime(SRC):
        return BIN
    os.makedirs(os.path.dirname(BIN), exist_ok=True)
    cmd = ["g++", "-std=c++17", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), SRC,
           "-L" + PKG, "-lfa", "-L/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../exact_io_aware_44_amd", "-Wl,-rpath,/opt/rocm/lib",
           "-o", BIN]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building the C-ABI driver failed:\n" + r.stderr)
    return BIN


if __name__ == "__main__":
    print(build(force=True))

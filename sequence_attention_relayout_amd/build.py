"""Build libulysses.so in-tree for gfx950.

kernels.hip goes through hipcc (device code for gfx950 only); the plan and
the C ABI are plain host C++ built with g++ against the HIP runtime headers.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libulysses.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
              "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include"]
# -ffp-contract=off: the fused path rounds every product on its own.
# -packed-fp32-ops off: no packed fp32 instructions in any kernel.
DEVICE_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
                "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang",
                "-packed-fp32-ops", "-Wall"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build(verbose=False, defines=(), out=LIB, build_dir=BUILD, kernel_src=None):
    """Compile and link; `defines` are extra preprocessor definitions and
    `kernel_src` replaces csrc/kernels.hip (for experiments built outside the
    package)."""
    os.makedirs(build_dir, exist_ok=True)
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    dflags = [f"-D{d}" for d in defines]
    objs = []
    for src in ("plan.cpp", "capi.cpp"):
        obj = os.path.join(build_dir, src.replace(".cpp", ".o"))
        _run(["g++", *HOST_FLAGS, *dflags, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    kobj = os.path.join(build_dir, "kernels.o")
    _run([hipcc, *DEVICE_FLAGS, *dflags, f"-I{CSRC}", "-c",
          kernel_src or os.path.join(CSRC, "kernels.hip"), "-o", kobj], verbose)
    objs.append(kobj)
    tmp = out + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


C_CHECK = os.path.join(ROOT, "tests", "native", "abi_c_check")


def build_c_check(verbose=False):
    """tests/native/abi_c_check.c: a plain C99 caller of the ABI, linked
    against libulysses.so (which must be built) and the HIP runtime."""
    exe = C_CHECK
    _run(["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-pedantic", "-Werror",
          "-D__HIP_PLATFORM_AMD__", f"-isystem{ROCM}/include", f"-I{os.path.join(ROOT, 'include')}",
          os.path.join(ROOT, "tests", "native", "abi_c_check.c"), "-o", exe, f"-L{PKG}",
          "-lulysses", f"-Wl,-rpath,{PKG}", f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{ROCM}/lib"], verbose)
    return exe


def build_plan_test(verbose=False, build_dir=BUILD, sanitize=False):
    """Host-only test driver of the plan (no HIP): tests/native/plan_test.cpp.
    sanitize=True builds it with AddressSanitizer and UBSan (g++, host code)."""
    os.makedirs(build_dir, exist_ok=True)
    exe = os.path.join(build_dir, "plan_test_san" if sanitize else "plan_test")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g",
           "-fno-omit-frame-pointer"] if sanitize else []
    _run(["g++", "-O1" if sanitize else "-O2", "-std=c++17", "-Wall", *san, f"-I{CSRC}",
          os.path.join(ROOT, "tests", "native", "plan_test.cpp"),
          os.path.join(CSRC, "plan.cpp"), "-o", exe], verbose)
    return exe


if __name__ == "__main__":
    build(verbose=True)
    if shutil.which("g++"):
        print("built", LIB)

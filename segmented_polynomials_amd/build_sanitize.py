"""Sanitizer build of the library's host code (CPU only, never for a GPU run).

Compiles the host sources (descriptor builder, C ABI, generated registry)
with AddressSanitizer and UndefinedBehaviorSanitizer (g++), reuses the HIP
kernel objects of the normal build (``build.py``; device code is not
instrumented), links ``_build_san/libsegpoly_san.so`` and, with
``--run-tests``, runs the host tests of the C ABI against it:

    python segmented_polynomials_amd/build_sanitize.py --run-tests

The test process preloads the gcc sanitizer runtimes and points the Python
binding at the sanitized library (environment variable SEGPOLY_LIB); leak
detection is off (the interpreter and PyTorch keep allocations alive at
exit).  Any sanitizer report aborts the run with a non-zero status.
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
NORMAL_OBJ = os.path.join(ROOT, "_build", "obj")
GEN = os.path.join(ROOT, "_build", "gen")
OUT = os.path.join(ROOT, "_build_san")
LIB = os.path.join(OUT, "libsegpoly_san.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

HOST_SOURCES = ["irreps.cpp", "cg.cpp", "tp_descriptor.cpp", "symcon_descriptor.cpp", "capi.cpp", "capi_linear.cpp",
                "capi_sh.cpp", "capi_fctp.cpp", "capi_edge.cpp"]
SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]


def _run(cmd, env=None):
    r = subprocess.run(cmd, env=env)
    if r.returncode != 0:
        raise SystemExit(f"failed ({r.returncode}): {' '.join(cmd)}")


def build():
    if not os.path.isdir(NORMAL_OBJ) or not os.path.exists(os.path.join(GEN, "registry.cpp")):
        raise SystemExit("run the normal build first (python segmented_polynomials_amd/build.py)")
    os.makedirs(OUT, exist_ok=True)
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
             f"-I{CSRC}", f"-I{INCLUDE}", *SAN]
    objs = []
    for src in [os.path.join(CSRC, s) for s in HOST_SOURCES] + [os.path.join(GEN, "registry.cpp")]:
        o = os.path.join(OUT, os.path.basename(src) + ".o")
        _run(["g++", *flags, "-c", src, "-o", o])
        objs.append(o)
    # device kernels and their launchers: the normal build's objects, unchanged
    objs += sorted(os.path.join(NORMAL_OBJ, f) for f in os.listdir(NORMAL_OBJ) if f.endswith(".hip.o"))
    _run(["g++", "-shared", *SAN, *objs, "-o", LIB, f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"])
    return LIB


def run_tests():
    rt = [subprocess.check_output(["gcc", f"-print-file-name={n}"], text=True).strip()
          for n in ("libasan.so", "libubsan.so")]
    env = dict(os.environ, SEGPOLY_LIB=LIB, LD_PRELOAD=":".join(rt),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    _run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
          os.path.join(ROOT, "tests", "test_capi_host.py")], env=env)


if __name__ == "__main__":
    print(build())
    if "--run-tests" in sys.argv:
        run_tests()

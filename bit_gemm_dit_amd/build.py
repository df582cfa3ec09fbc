"""Build libditq.so (gfx950) in-tree with hipcc.

Compiles every HIP source of the library to an object under ``_build/`` (in
parallel) and links the shared library next to this file.  Usage:
``python bit_gemm_dit_amd/build.py`` (run as a file: importing the package
would load the library it is about to rebuild).

``python bit_gemm_dit_amd/build.py --sanitize`` builds instead a CPU-only library
of the ABI layer (abi.cpp, with host_stubs.cpp standing in for the kernel
launchers) instrumented with AddressSanitizer and UndefinedBehaviorSanitizer, at
``_build/san/libditq_san.so``, and prints the command that runs the ABI's CPU
tests against it:

    DITQ_LIB=_build/san/libditq_san.so LD_PRELOAD=<clang asan runtime> \
        ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
        python -m pytest tests/test_abi_cpu.py
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libditq.so")
SOURCES = ["abi.cpp", "quant.hip", "pack.hip", "gemm.hip", "measure.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off: only scalar / vector fp32 code is emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    # A kernel whose host-side stub was dropped leaves an undefined symbol that only
    # shows up when the library is loaded; refuse such a library here instead.
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in nm.stdout.splitlines() if "ditq" in ln]
    if nm.returncode != 0 or missing:
        raise RuntimeError(f"libditq.so has undefined library symbols: {missing or nm.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


SAN_DIR = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_DIR, "libditq_san.so")


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime matching hipcc's compiler."""
    r = subprocess.run([os.path.join(os.path.dirname(HIPCC), "..", "llvm", "bin", "clang++"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        import glob
        hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        if not hits:
            raise RuntimeError("clang AddressSanitizer runtime not found")
        path = hits[0]
    return os.path.realpath(path)


def build_sanitized(verbose: bool = False) -> str:
    """abi.cpp + host_stubs.cpp, host code only (no kernel is compiled), with ASan and UBSan."""
    os.makedirs(SAN_DIR, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    flags = ["-x", "hip", "--offload-host-only", "-std=c++17", "-fPIC", "-O1", "-g", "-fno-omit-frame-pointer",
             f"-I{INCLUDE}", f"-I{CSRC}", *san]
    objs = []
    for src in ("abi.cpp", "host_stubs.cpp"):
        obj = os.path.join(SAN_DIR, os.path.splitext(src)[0] + ".o")
        r = subprocess.run([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitizer build of {src} failed:\n{r.stderr}")
        objs.append(obj)
    r = subprocess.run([HIPCC, "-shared", "-fPIC", "-shared-libsan", *san, *objs, "-o", SAN_LIB],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitizer link failed:\n{r.stderr}")
    if verbose:
        print(f"built {SAN_LIB}")
        print("run the ABI CPU tests under it with:")
        print(f"  DITQ_LIB={SAN_LIB} LD_PRELOAD={asan_runtime()} ASAN_OPTIONS=detect_leaks=0 "
              "UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 python -m pytest tests/test_abi_cpu.py")
    return SAN_LIB


if __name__ == "__main__":
    import sys
    if "--sanitize" in sys.argv[1:]:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)

"""Compile the HIP library (kernels + C ABI) in-tree with hipcc for gfx950."""
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkda.so")
SOURCES = [os.path.join(CSRC, "kda_kernels.hip"), os.path.join(CSRC, "kda_noalloc.hip"),
           os.path.join(CSRC, "kda_api.cpp")]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the KDA library)")


def build_library(verbose=False, out=None, extra_flags=()):
    """Always recompiles (the build check must compile), then atomically replaces libkda.so (or
    writes `out`, with `extra_flags` added to the hipcc line: the CPU sanitizer test builds a
    host-instrumented copy this way)."""
    target = out or LIB
    tmp = target + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           # packed fp32 instructions are kept out of every HIP object
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-o", tmp] + list(extra_flags) + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + res.stdout)
    os.replace(tmp, target)
    return target


def asan_runtime():
    """The ASan runtime of the compiler that hipcc drives (to preload for a sanitised build)."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    for pat in ("llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so",
                "lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"):
        hits = sorted(glob.glob(os.path.join(root, pat)))
        if hits:
            return hits[-1]
    hits = sorted(glob.glob("/opt/rocm*/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if hits:
        return hits[-1]
    raise RuntimeError("clang ASan runtime not found")


if __name__ == "__main__":
    print(build_library(verbose=True))

"""Build libdetred.so in-tree with hipcc for gfx950.

Flags:
  -ffp-contract=off   no FMA contraction: every add and multiply in the
                      combine and row kernels rounds exactly as written;
  -munsafe-fp-atomics hardware fp32 atomic add for the atomic control;
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      keep the compiler from emitting packed fp32 ops.
"""
import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdetred.so")
ARCH = os.environ.get("DETRED_OFFLOAD_ARCH", "gfx950")

SOURCES = ["gemm.hip", "gemm_lds.hip", "rows.hip", "attention.hip", "noalloc.hip", "api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall",
          "-I", INCLUDE, "-I", CSRC]
DEVICE = ["--offload-arch=" + ARCH, "-munsafe-fp-atomics",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src, verbose):
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJDIR, src + ".o")
    if src.endswith(".hip"):
        cmd = [HIPCC, "-x", "hip"] + COMMON + DEVICE + ["-c", path, "-o", obj]
    else:
        cmd = [HIPCC] + COMMON + ["-D__HIP_PLATFORM_AMD__", "-c", path, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose=False):
    """Compile every source and link libdetred.so (always rebuilds)."""
    os.makedirs(OBJDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = [HIPCC, "-shared", "--offload-arch=" + ARCH, "-o", LIB + ".tmp"] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (r.stdout, r.stderr))
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

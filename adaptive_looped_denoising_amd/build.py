"""Builds the gfx950 HIP library (libalodlm.so) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libalodlm.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["runtime.cpp", "kernels_misc.hip", "generic.hip", "gemm_mfma.hip", "attn_mfma.hip", "synth_fill.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "--offload-arch=" + ARCH, "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJDIR, src + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + FLAGS + lang + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compiles every source for gfx950 and links libalodlm.so (always rebuilds)."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


ASAN_LIB = os.path.join(HERE, "libalodlm_asan.so")
# host-side AddressSanitizer for the C ABI and the host runtime (argument checks, workspace planning,
# tile choice): only the host half of runtime.cpp is instrumented (-Xarch_host), device code is not
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """The compiler's shared AddressSanitizer runtime (preloaded by the process that loads the library)."""
    base = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang")
    for ver in sorted(os.listdir(base)) if os.path.isdir(base) else []:
        p = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(p):
            return p
    return ""


def build_asan(verbose: bool = False) -> str:
    """libalodlm_asan.so: runtime.cpp with host AddressSanitizer, the kernels' objects as built by build()."""
    objs = [os.path.join(OBJDIR, s + ".o") for s in SOURCES if s != "runtime.cpp"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError("build() first: missing %s" % ", ".join(missing))
    obj = os.path.join(OBJDIR, "runtime.asan.o")
    cmd = [HIPCC] + FLAGS + ASAN_FLAGS + ["-c", os.path.join(CSRC, "runtime.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on runtime.cpp (asan):\n%s\n%s" % (r.stdout, r.stderr))
    tmp = ASAN_LIB + ".tmp%d" % os.getpid()
    r = subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, obj] + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("asan link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, ASAN_LIB)
    if verbose:
        print("built", ASAN_LIB)
    return ASAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)

"""Build libxattn.so in-tree with hipcc for gfx950.

Usage: ``python -m shared_history_candidate_amd.build`` (or ``build()``).
Objects go to ``_build/`` at the repository root; the shared library is
written next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build", "xattn")
LIB = os.path.join(PKG, "libxattn.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: no accvgpr moves before the
    # softmax arithmetic reads the scores
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # NaN operands are not supported inputs; without this every fmaxf operand
    # is canonicalised first (infinities are still honoured)
    "-fno-honor-nans",
    "-I" + INCLUDE, "-I" + CSRC,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libxattn")


# Host-side AddressSanitizer build (build(asan=True)): the host code of every
# source is instrumented, the device code is not (-Xarch_host keeps the flag
# off the gfx950 pass).  For host checks of the C ABI on a machine without a
# GPU; the product library is the plain build.
ASAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                   "-shared-libasan"]


def _compile(src: str, obj: str, verbose: bool, asan: bool = False) -> None:
    extra = os.environ.get("XATTN_EXTRA_HIPCC_FLAGS", "").split()   # tuning experiments
    if asan:
        extra = extra + ASAN_HOST_FLAGS
    cmd = [_hipcc()] + HIPCC_FLAGS + extra + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [_hipcc(), "-O3", "-std=c++17", "-fPIC", "-Wall", "-I" + INCLUDE, "-I" + CSRC,
               "-c", src, "-o", obj] + (ASAN_HOST_FLAGS if asan else [])
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s" % (src, errs))
    if verbose and errs.strip():
        print(errs)


def build(verbose: bool = False, jobs: int = 8, out: str = LIB, asan: bool = False) -> str:
    """Compile every HIP/C++ source under csrc/ and link libxattn.so (or `out`);
    asan=True instruments the host code with AddressSanitizer (objects kept
    apart from the plain build's)."""
    objdir = OBJDIR + ("_asan" if asan else "")
    os.makedirs(objdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in srcs]
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        list(ex.map(lambda so: _compile(so[0], so[1], verbose, asan), zip(srcs, objs)))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if asan:
        cmd += ["-fsanitize=address", "-shared-libasan"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    import sys
    if "--asan" in sys.argv:
        # python -m shared_history_candidate_amd.build --asan OUT.so
        print(build(verbose="-v" in sys.argv, asan=True, out=sys.argv[sys.argv.index("--asan") + 1]))
    else:
        print(build(verbose="-v" in sys.argv))

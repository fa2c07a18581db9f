"""Build libpoetx.so in-tree for gfx950 with hipcc.

    python -m orthogonal_equivalence_amd.build [--sanitize]

Compiles every source under csrc/ (the .hip kernels and the C ABI layer) to
objects in _build/, links them into orthogonal_equivalence_amd/libpoetx.so
and returns its path. Always recompiles. With --sanitize, builds the
host-sanitized copy _build/san/libpoetx_san.so instead (for the CPU tests).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpoetx.so")
ARCH = "gfx950"

COMMON = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpoetx)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same
# sources (the C ABI's validation and planning run on the CPU; the GPU code is
# compiled as usual). Loaded by the CPU tests through POETX_LIBRARY with the
# sanitizer runtime preloaded.
SAN_LIB = os.path.join(BUILD, "san", "libpoetx_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-g"]


def build(verbose: bool = False, sanitize: bool = False) -> str:
    cc = hipcc()
    out_dir = os.path.dirname(SAN_LIB) if sanitize else BUILD
    lib = SAN_LIB if sanitize else LIB
    extra = SAN_FLAGS if sanitize else []
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(out_dir, os.path.basename(s) + ".o") for s in srcs]
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        for s, o in zip(srcs, objs):
            lang = ["-x", "hip"] if s.endswith(".hip") else []
            jobs.append(ex.submit(_run, [cc, *COMMON, *extra, *lang, "-c", s, "-o", o]))
        for j in jobs:
            out = j.result()
            if verbose and out.strip():
                print(out)
    tmp = lib + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, *objs, "-o", tmp])
    os.replace(tmp, lib)
    return lib


def sanitizer_runtime() -> str:
    """Path of the AddressSanitizer runtime of hipcc's clang (to preload into
    an uninstrumented Python)."""
    out = subprocess.run([os.path.join(os.path.dirname(hipcc()), "..", "llvm", "bin", "clang"),
                          "-print-file-name=libclang_rt.asan-x86_64.so"],
                         stdout=subprocess.PIPE, text=True, check=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        import glob
        cands = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        if not cands:
            raise RuntimeError("AddressSanitizer runtime not found")
        out = cands[0]
    return out


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv)
    print(path)

"""Build liblce.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m linear_cross_entropy_lse_amd.build [--verbose] [--asan] [--debug-checks]

hipcc cross-compiles for gfx950 without a GPU.  Packed fp32 instructions are
disabled for the device code (-packed-fp32-ops); hipcc's host pass warns that
it does not know the feature, which is harmless.

Two checking builds sit beside the product library and never replace it:
  --asan          liblce_asan.so: the host code (argument checks, workspace
                  plans, launch sequences) built with AddressSanitizer; the
                  device code is built as usual.  Load it with the sanitizer
                  runtime preloaded (asan_runtime() below) and LCE_LIB pointing
                  at it; tests/test_sanitize_host.py runs the host ABI tests
                  that way, on the CPU.
  --debug-checks  liblce_debug.so: the row kernels check the indices they take
                  from their inputs (labels, sorted keys) before using them,
                  print the failing check and skip the access.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "liblce.so")
SOURCES = ["lce_api.hip", "lce_gemm.hip", "lce_rows.hip", "lce_order.hip", "lce_exact.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build liblce)")


def compile_flags(extra=()):
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result", f"-I{os.path.join(ROOT, 'include')}", *extra]


ASAN_LIB_PATH = os.path.join(HERE, "liblce_asan.so")
DEBUG_LIB_PATH = os.path.join(HERE, "liblce_debug.so")
# Host-only sanitizer flags: each -fsanitize= goes to the host pass alone.
ASAN_COMPILE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_LINK = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-shared-libasan"]


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (for LD_PRELOAD)."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    hits = sorted(glob.glob(os.path.join(root, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")) +
                  glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("AddressSanitizer runtime not found next to hipcc")
    return hits[-1]


def build(verbose: bool = False, out: str = LIB_PATH, extra=(), asan: bool = False,
          debug_checks: bool = False, bdir: str = None) -> str:
    """Compile every HIP source and link liblce.so (or a checking build, see
    the module docstring).  Always rebuilds."""
    cc = hipcc()
    link_extra = []
    if asan:
        extra = (*extra, *ASAN_COMPILE)
        link_extra = ASAN_LINK
        if out == LIB_PATH:
            out = ASAN_LIB_PATH
    if debug_checks:
        extra = (*extra, "-DLCE_DEBUG_CHECKS")
        if out == LIB_PATH:
            out = DEBUG_LIB_PATH
    if bdir is None:
        tag = ("_asan" if asan else "") + ("_debug" if debug_checks else "")
        bdir = os.path.join(HERE, "_build" + tag)
    os.makedirs(bdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        cmd = [cc, *compile_flags(extra), "-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                         if "packed-fp32-ops" not in l)
        return src, obj, cmd, res.returncode, msgs

    # The sources are independent translation units: compile them side by side.
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    objs = []
    for src, obj, cmd, rc, msgs in results:
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs)
        objs.append(obj)
    tmp = out + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_extra, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv, asan="--asan" in sys.argv,
                debug_checks="--debug-checks" in sys.argv))

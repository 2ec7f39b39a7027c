"""Build ``libpl.so`` (the C-ABI library) from ``csrc/*.hip`` with hipcc for gfx950.

Run ``python -m streaming_diffusion_portrait_amd.build`` (or
``__graft_entry__.build()``).  Compiles every translation unit in parallel and
links one shared library next to this file; it always recompiles.

``python -m streaming_diffusion_portrait_amd.build --sanitize`` builds
``libpl_san.so`` instead: the same sources with AddressSanitizer and
UndefinedBehaviorSanitizer on the host code only (device code is built as
usual).  It is for CPU runs of the argument checks; load it with the ASan
runtime preloaded and ``PL_LIBRARY`` pointing at it.

``--debug-bounds`` builds ``libpl_dbg.so``: the attention kernels with a
bounds check before every global and LDS access (``pl_debug_bounds`` reads
which access sites failed); load it through ``PL_LIBRARY``.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpl.so")
SAN_LIB = os.path.join(HERE, "libpl_san.so")
DBG_LIB = os.path.join(HERE, "libpl_dbg.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wextra",
    "-Werror",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

# host pass only: each sanitizer flag goes behind its own -Xarch_host
SAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all",
    "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-shared-libsan",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpl.so)")


def _compile(hipcc, src, objdir, extra):
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device feature flag; that warning is noise
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    return obj, msgs


def build(verbose=False, sanitize=False, lib_path=None, obj_dir=None, debug_bounds=False):
    """Compile every csrc/*.hip for gfx950 and link libpl.so (libpl_san.so with
    ``sanitize``, libpl_dbg.so with ``debug_bounds``), or ``lib_path`` with
    objects under ``obj_dir``; returns the library's path."""
    hipcc = _hipcc()
    variant = "san" if sanitize else "dbg" if debug_bounds else None
    objdir = obj_dir or (os.path.join(OBJ, variant) if variant else OBJ)
    extra = (SAN_FLAGS if sanitize else []) + (["-DPL_DEBUG_BOUNDS"] if debug_bounds else [])
    lib = lib_path or (SAN_LIB if sanitize else DBG_LIB if debug_bounds else LIB)
    os.makedirs(objdir, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(hipcc, s, objdir, extra), srcs))
    for obj, msgs in results:
        if verbose and msgs.strip():
            print(msgs)
    tmp = lib + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *[o for o, _ in results],
           "-Wl,-rpath,/opt/rocm/lib"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv, sanitize="--sanitize" in sys.argv, debug_bounds="--debug-bounds" in sys.argv)

"""Build libmoda.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoda.so")
# Measurement kernels (include/moda_probe.h): a library of their own, not part of libmoda.so.
PROBE_LIB = os.path.join(PKG, "libmoda_probe.so")
PROBE_SOURCES = ["moda_probe.hip"]
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["moda_api.cpp", "moda_fwd_bf16.hip", "moda_fwd_f32.hip", "moda_pack.hip", "moda_decode.hip",
           "moda_bwd.hip", "moda_kvproj.hip"]

# Per-source extra flags.  The bf16 kernels never produce NaN from finite
# inputs, and without NaN semantics each fmaxf in their row-max chains needs no
# canonicalising v_max_f32 x, x before the v_max3_f32.  The forward, backward
# and KV projection are scheduled with the iterative ILP strategy (no spills,
# bit-identical forward results): forward 1.7% faster at the long-context L=48
# workload (16.05 vs 16.33 ms, 15 interleaved runs), backward about 1% faster,
# the KV projection 2-5%; the decode kernels gained nothing and keep the default.
_ILP = ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"]
SOURCE_FLAGS = {"moda_fwd_bf16.hip": ["-fno-honor-nans"] + _ILP, "moda_decode.hip": ["-fno-honor-nans"],
                "moda_bwd.hip": ["-fno-honor-nans"] + _ILP, "moda_kvproj.hip": _ILP}

# Packed-fp32 VALU forms are switched off for all device code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def device_listing(src: str) -> str:
    """Path of the gfx950 assembly that build() keeps for the .hip source `src`."""
    return os.path.join(BUILD_DIR, os.path.splitext(src)[0] + "-hip-amdgcn-amd-amdhsa-gfx950.s")


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile every source for gfx950 and link libmoda.so (and the measurement library
    libmoda_probe.so) next to this file.  The device assembly of each .hip source is kept
    (-save-temps) and checked for the inline-asm load hazard of asm_check before linking."""
    try:
        from . import asm_check
    except ImportError:  # run as a script
        import asm_check

    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip", "-save-temps=obj"] if src.endswith(".hip") else []
        cmd = ([hipcc] + HIPCC_FLAGS + SOURCE_FLAGS.get(src, []) + list(extra_flags) + lang +
               ["-c", os.path.join(CSRC, src), "-o", obj])
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed on %s:\n%s" % (src, err))
        if verbose and err.strip():
            print(err, file=sys.stderr)
        if src.endswith(".hip"):
            with open(device_listing(src)) as f:
                bad = asm_check.check_listing(f.read())
            if bad:
                raise RuntimeError("%s: direct-to-LDS load hazard in the compiled code:\n%s" %
                                   (src, "\n".join("%s: %s" % b for b in bad[:10])))
        return obj

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, SOURCES + PROBE_SOURCES))
    for lib, lib_objs in ((LIB, objs[:len(SOURCES)]), (PROBE_LIB, objs[len(SOURCES):])):
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + lib_objs
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True, capture_output=not verbose)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

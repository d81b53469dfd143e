"""ctypes loader for libmoda.so (the HIP kernels behind the C ABI in include/moda.h)."""
import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoda.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moda.h")
PROBE_LIB_PATH = os.path.join(PKG, "libmoda_probe.so")
PROBE_HEADER = os.path.join(os.path.dirname(PKG), "include", "moda_probe.h")

_lib = None
_probe = None


def declared_symbols(header=HEADER):
    """Names of the functions a header (include/moda.h by default) declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moda_[a-z0-9_]+)\s*\(", text)))


def load_probe():
    """Load libmoda_probe.so, the measurement kernels of include/moda_probe.h."""
    global _probe
    if _probe is not None:
        return _probe
    if not os.path.exists(PROBE_LIB_PATH):
        raise RuntimeError("libmoda_probe.so is not built (%s)" % PROBE_LIB_PATH)
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.moda_probe_mfma_bf16.argtypes = [vp, i32, i32, i32, vp]
    lib.moda_probe_copy.argtypes = [vp, vp, sz, i32, vp]
    lib.moda_probe_read.argtypes = [vp, sz, i32, vp, vp]
    for fn in (lib.moda_probe_mfma_bf16, lib.moda_probe_copy, lib.moda_probe_read):
        fn.restype = i32
    _probe = lib
    return lib


def load():
    """Load libmoda.so; raise if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libmoda.so is not built (%s); build it with depth_stream_attention_amd.build.build() "
                           "or __graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    fwd_args = [vp] * 5 + [i32] * 7 + [vp, vp, vp]
    for name in ("moda_attn_fwd", "moda_attn_fwd_f32"):
        fn = getattr(lib, name)
        fn.argtypes = fwd_args
        fn.restype = i32
    lib.moda_attn_fwd_ring.argtypes = [vp] * 5 + [i32] * 8 + [vp, vp, vp]
    lib.moda_attn_fwd_ring.restype = i32
    lib.moda_attn_decode_ring.argtypes = [vp] * 5 + [i32] * 7 + [vp, vp, vp, ctypes.c_size_t, vp]
    lib.moda_attn_decode_ring.restype = i32
    lib.moda_attn_decode.argtypes = [vp] * 5 + [i32] * 6 + [vp, vp, vp, ctypes.c_size_t, vp]
    lib.moda_attn_decode.restype = i32
    lib.moda_attn_decode_noalloc.argtypes = [vp] * 5 + [i32] * 6 + [vp, vp, vp]
    lib.moda_attn_decode_noalloc.restype = i32
    lib.moda_attn_bwd.argtypes = [vp] * 8 + [i32] * 7 + [vp] * 6 + [ctypes.c_size_t, vp]
    lib.moda_attn_bwd.restype = i32
    lib.moda_attn_bwd_workspace.argtypes = [i32] * 6
    lib.moda_attn_bwd_workspace.restype = ctypes.c_size_t
    lib.moda_attn_decode_workspace.argtypes = [i32] * 6
    lib.moda_attn_decode_workspace.restype = ctypes.c_size_t
    lib.moda_kv_project.argtypes = [vp, vp] + [i32] * 5 + [vp] * 4 + [i32, i32, vp]
    lib.moda_kv_project.restype = i32
    lib.moda_pack_depth.argtypes = [vp, vp] + [i32] * 6 + [vp]
    lib.moda_pack_depth.restype = i32
    lib.moda_append_depth_slot.argtypes = [vp, vp] + [i32] * 7 + [vp]
    lib.moda_append_depth_slot.restype = i32
    lib.moda_block_span.argtypes = [i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.moda_block_span.restype = i32
    lib.moda_error_string.argtypes = [i32]
    lib.moda_error_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def ensure_built():
    """Load the library, compiling it first only if no built copy exists."""
    if not os.path.exists(LIB_PATH) or not os.path.exists(PROBE_LIB_PATH):
        from . import build
        build.build()
    return load()

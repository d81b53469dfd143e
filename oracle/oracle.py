"""ctypes wrapper of the fp64 CPU oracle (moda_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
CPU-baseline leg call this module.  It shares no code with the HIP path.

Inputs are host arrays (numpy, or torch CPU tensors) of dtype float64,
float32 or bfloat16.  bf16 tensors are handed over as their raw 16-bit
patterns and widened exactly inside the oracle.  Outputs are float64.

Layouts (row-major): q [B,T,Hq,d]; k_seq, v_seq [B,T,Hk,d]; depth K/V in the
generation layout [B,T,L,Hk,d]; out [B,T,Hq,d]; lse [B,Hq,T] (natural log).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_KIND_F64, _KIND_F32, _KIND_BF16 = 0, 1, 2
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
        lib.moda_oracle_fwd.argtypes = [vp] * 5 + [i32] * 8 + [vp, vp, i32]
        lib.moda_oracle_fwd.restype = i32
        lib.moda_oracle_fwd_rows.argtypes = [vp] * 5 + [i32] * 8 + [vp, i64, vp, vp, i32]
        lib.moda_oracle_fwd_rows.restype = i32
        lib.moda_oracle_bwd.argtypes = [vp] * 6 + [i32] * 8 + [vp] * 5 + [i32]
        lib.moda_oracle_bwd.restype = i32
        lib.moda_oracle_bwd_sampled.argtypes = ([vp] * 6 + [i32] * 8 + [vp, i64, vp, vp, i64, vp, vp, vp, i64, vp, vp]
                                                + [i32])
        lib.moda_oracle_bwd_sampled.restype = i32
        lib.moda_oracle_kv_project.argtypes = [vp, vp] + [i32] * 6 + [vp, vp]
        lib.moda_oracle_kv_project.restype = i32
        lib.moda_oracle_pack_depth.argtypes = [vp, vp] + [i32] * 6
        lib.moda_oracle_pack_depth.restype = i32
        lib.moda_oracle_append_depth_slot.argtypes = [vp, vp] + [i32] * 7
        lib.moda_oracle_append_depth_slot.restype = i32
        _lib = lib
    return _lib


def default_threads() -> int:
    """Host threads the oracle uses: the CPUs this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _host(x):
    """Return (contiguous numpy array, kind code) for a numpy array or torch CPU tensor."""
    if x is None:
        return None, None
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach()
        if x.device.type != "cpu":
            raise ValueError("oracle inputs must be host tensors")
        name = str(x.dtype)
        x = x.contiguous()
        if name == "torch.bfloat16":
            import torch
            return x.view(torch.int16).numpy().view(np.uint16), _KIND_BF16
        if name == "torch.float32":
            return x.numpy(), _KIND_F32
        if name == "torch.float64":
            return x.numpy(), _KIND_F64
        raise TypeError("unsupported oracle input dtype %s" % name)
    a = np.ascontiguousarray(x)
    if a.dtype == np.float64:
        return a, _KIND_F64
    if a.dtype == np.float32:
        return a, _KIND_F32
    raise TypeError("unsupported oracle input dtype %s (pass bf16 as a torch tensor)" % a.dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _prepare(q, k_seq, v_seq, k_depth, v_depth):
    arrs = [_host(x) for x in (q, k_seq, v_seq, k_depth, v_depth)]
    kinds = {k for (_, k) in arrs if k is not None}
    if len(kinds) != 1:
        raise TypeError("all oracle inputs must share one dtype")
    qa, ka, va, kda, vda = (a for (a, _) in arrs)
    B, T, Hq, d = qa.shape
    if ka.shape[:2] != (B, T) or ka.shape[3] != d or va.shape != ka.shape:
        raise ValueError("k_seq/v_seq must be [B,T,Hk,d] matching q")
    Hk = ka.shape[2]
    if kda is None or kda.size == 0:
        L, kda, vda = 0, None, None
    else:
        if kda.ndim != 5 or kda.shape[:2] != (B, T) or kda.shape[3:] != (Hk, d) or vda.shape != kda.shape:
            raise ValueError("depth K/V must be [B,T,L,Hk,d]")
        L = kda.shape[2]
    return (qa, ka, va, kda, vda), kinds.pop(), (B, T, Hq, Hk, d, L)


def moda_fwd(q, k_seq, v_seq, k_depth, v_depth, causal=True, nthreads=None):
    """Every row of the MoDA forward in fp64.  Returns (out [B,T,Hq,d], lse [B,Hq,T])."""
    lib = _load()
    (qa, ka, va, kda, vda), kind, (B, T, Hq, Hk, d, L) = _prepare(q, k_seq, v_seq, k_depth, v_depth)
    out = np.empty((B, T, Hq, d), np.float64)
    lse = np.empty((B, Hq, T), np.float64)
    rc = lib.moda_oracle_fwd(_ptr(qa), _ptr(ka), _ptr(va), _ptr(kda), _ptr(vda), kind,
                             B, T, Hq, Hk, d, L, int(bool(causal)), _ptr(out), _ptr(lse),
                             nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("moda_oracle_fwd failed with code %d" % rc)
    return out, lse


def moda_fwd_rows(q, k_seq, v_seq, k_depth, v_depth, rows, causal=True, nthreads=None):
    """Selected rows (an [n,3] int array of (b, t, h)).  Returns (out [n,d], lse [n])."""
    lib = _load()
    (qa, ka, va, kda, vda), kind, (B, T, Hq, Hk, d, L) = _prepare(q, k_seq, v_seq, k_depth, v_depth)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    n = r.shape[0]
    out = np.empty((n, d), np.float64)
    lse = np.empty((n,), np.float64)
    rc = lib.moda_oracle_fwd_rows(_ptr(qa), _ptr(ka), _ptr(va), _ptr(kda), _ptr(vda), kind,
                                  B, T, Hq, Hk, d, L, int(bool(causal)), _ptr(r), n,
                                  _ptr(out), _ptr(lse), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("moda_oracle_fwd_rows failed with code %d" % rc)
    return out, lse


def moda_bwd(q, k_seq, v_seq, k_depth, v_depth, dout, causal=True, nthreads=None):
    """Gradients of every input for the output gradient dout [B,T,Hq,d], in fp64.

    Returns (dq [B,T,Hq,d], dk, dv [B,T,Hk,d], dkd, dvd [B,T,L,Hk,d]); the depth
    gradients are None when L == 0.  dout must share the inputs' dtype.
    """
    lib = _load()
    (qa, ka, va, kda, vda), kind, (B, T, Hq, Hk, d, L) = _prepare(q, k_seq, v_seq, k_depth, v_depth)
    da, dkind = _host(dout)
    if dkind != kind or da.shape != qa.shape:
        raise ValueError("dout must be [B,T,Hq,d] with the inputs' dtype")
    dq = np.empty((B, T, Hq, d), np.float64)
    dk = np.empty((B, T, Hk, d), np.float64)
    dv = np.empty((B, T, Hk, d), np.float64)
    dkd = np.empty((B, T, L, Hk, d), np.float64) if L else None
    dvd = np.empty((B, T, L, Hk, d), np.float64) if L else None
    rc = lib.moda_oracle_bwd(_ptr(qa), _ptr(ka), _ptr(va), _ptr(kda), _ptr(vda), _ptr(da), kind,
                             B, T, Hq, Hk, d, L, int(bool(causal)),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dkd), _ptr(dvd),
                             nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("moda_oracle_bwd failed with code %d" % rc)
    return dq, dk, dv, dkd, dvd


def moda_bwd_sampled(q, k_seq, v_seq, k_depth, v_depth, dout, rows=(), keys=(), toks=(), causal=True,
                     nthreads=None):
    """Selected gradients in fp64: rows [n,3] (b, t, h) -> dq [n,d]; keys [m,3] (b, j, hk) ->
    (dk, dv) [m,d] of sequence key j; toks [r,3] (b, t, hk) -> (dkd, dvd) [r,L,d] of token t's
    depth slots.  Returns (dq, dk, dv, dkd, dvd)."""
    lib = _load()
    (qa, ka, va, kda, vda), kind, (B, T, Hq, Hk, d, L) = _prepare(q, k_seq, v_seq, k_depth, v_depth)
    da, dkind = _host(dout)
    if dkind != kind or da.shape != qa.shape:
        raise ValueError("dout must be [B,T,Hq,d] with the inputs' dtype")
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    kk = np.ascontiguousarray(np.asarray(keys, dtype=np.int32).reshape(-1, 3))
    tt = np.ascontiguousarray(np.asarray(toks, dtype=np.int32).reshape(-1, 3))
    dq = np.zeros((r.shape[0], d))
    dk = np.zeros((kk.shape[0], d))
    dv = np.zeros((kk.shape[0], d))
    dkd = np.zeros((tt.shape[0], L, d))
    dvd = np.zeros((tt.shape[0], L, d))
    rc = lib.moda_oracle_bwd_sampled(_ptr(qa), _ptr(ka), _ptr(va), _ptr(kda), _ptr(vda), _ptr(da), kind,
                                     B, T, Hq, Hk, d, L, int(bool(causal)),
                                     _ptr(r), r.shape[0], _ptr(dq), _ptr(kk), kk.shape[0], _ptr(dk), _ptr(dv),
                                     _ptr(tt), tt.shape[0], _ptr(dkd), _ptr(dvd), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("moda_oracle_bwd_sampled failed with code %d" % rc)
    return dq, dk, dv, dkd, dvd


def kv_project(x, w_kv, Hk, d):
    """k, v = the KV projection of x [B,T,Dm] by w_kv [2*Hk*d, Dm] (K rows, then V rows), in
    fp64: returns (k, v) [B,T,Hk,d]."""
    lib = _load()
    xa, kind = _host(x)
    wa, wkind = _host(w_kv)
    if kind != wkind:
        raise TypeError("x and w_kv must share one dtype")
    B, T, Dm = xa.shape
    if wa.shape != (2 * Hk * d, Dm):
        raise ValueError("w_kv must be [2*Hk*d, Dm]")
    k = np.empty((B, T, Hk, d))
    v = np.empty((B, T, Hk, d))
    rc = lib.moda_oracle_kv_project(_ptr(xa), _ptr(wa), kind, B, T, Dm, Hk, d, _ptr(k), _ptr(v))
    if rc != 0:
        raise RuntimeError("moda_oracle_kv_project failed with code %d" % rc)
    return k, v


def _raw_bytes(x):
    """(uint8-viewable contiguous numpy array, elem_bytes) for a numpy array or torch tensor."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().contiguous().reshape(-1)
        return x.view(torch.uint8).numpy(), x.element_size()
    a = np.ascontiguousarray(x).reshape(-1)
    return a.view(np.uint8), a.dtype.itemsize


def pack_depth(src):
    """dst[b,t,hk,l,:] = src[b,t,l,hk,:], bit for bit.  Returns a numpy array of src's dtype
    (bf16 comes back as uint16 bit patterns)."""
    lib = _load()
    shape = tuple(src.shape)
    B, T, L, Hk, d = shape
    raw, eb = _raw_bytes(src)
    out = np.empty(raw.nbytes, np.uint8)
    rc = lib.moda_oracle_pack_depth(_ptr(raw), _ptr(out), B, T, L, Hk, d, eb)
    if rc != 0:
        raise RuntimeError("moda_oracle_pack_depth failed with code %d" % rc)
    dt = {2: np.uint16, 4: np.float32, 8: np.float64}.get(eb, np.uint8)
    return out.view(dt).reshape(B, T, Hk, L, d)


def append_depth_slot(kv, dst, slot):
    """Return a copy of packed dst [B,T,Hk,L,d] with slot `slot` set to kv [B,T,Hk,d]."""
    lib = _load()
    B, T, Hk, L, d = tuple(dst.shape)
    raw_kv, eb = _raw_bytes(kv)
    raw_dst, eb2 = _raw_bytes(dst)
    if eb != eb2:
        raise TypeError("kv and dst element sizes differ")
    out = np.array(raw_dst, copy=True)
    rc = lib.moda_oracle_append_depth_slot(_ptr(raw_kv), _ptr(out), int(slot), B, T, L, Hk, d, eb)
    if rc != 0:
        raise RuntimeError("moda_oracle_append_depth_slot failed with code %d" % rc)
    dt = {2: np.uint16, 4: np.float32, 8: np.float64}.get(eb, np.uint8)
    return out.view(dt).reshape(B, T, Hk, L, d)

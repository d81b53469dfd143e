"""Python binding of the C ABI (include/moda.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU, checks that
their dtypes and shapes match the C signature, passes raw device pointers and
the current HIP stream to libmoda.so, and raises MODAError on a non-zero
return code.  All computation happens in the HIP kernels; nothing here
computes on the host.  torch supplies device memory (out / lse when not given)
and the stream.
"""
import ctypes

import torch

from . import _lib

MODA_OK = 0
MODA_ERR_NULL = -1
MODA_ERR_SHAPE = -2
MODA_ERR_UNSUPPORTED = -3
MODA_ERR_ALIGN = -4
MODA_ERR_HIP = -5
MODA_ERR_TOO_LARGE = -6
MODA_DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20


class MODAError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__("%s failed: %s (code %d)" % (fn, moda_error_string(code), code))


def moda_error_string(code: int) -> str:
    return _lib.load().moda_error_string(int(code)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(t, name, dtype, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _fwd(fn_name, dtype, q, k_seq, v_seq, k_depth, v_depth, causal, out, lse, stream, ring_L=None):
    _check(q, "q", dtype, 4)
    _check(k_seq, "k_seq", dtype, 4)
    _check(v_seq, "v_seq", dtype, 4)
    B, T, Hq, d = q.shape
    Hk = k_seq.shape[2]
    if tuple(k_seq.shape) != (B, T, Hk, d) or tuple(v_seq.shape) != (B, T, Hk, d):
        raise ValueError("k_seq / v_seq must be [B,T,Hk,d] = %s" % ((B, T, Hk, d),))
    L = 0
    if k_depth is not None and k_depth.numel() > 0:
        _check(k_depth, "k_depth", dtype, 5)
        _check(v_depth, "v_depth", dtype, 5)
        L = k_depth.shape[3]
        if tuple(k_depth.shape) != (B, T, Hk, L, d) or tuple(v_depth.shape) != (B, T, Hk, L, d):
            raise ValueError("packed depth K/V must be [B,T,Hk,L,d] = %s" % ((B, T, Hk, L, d),))
    else:
        k_depth = v_depth = None
    S = L
    if ring_L is not None:
        if not 0 <= ring_L <= S:
            raise ValueError("ring: need 0 <= L <= S = %d, got L = %d" % (S, ring_L))
        L = int(ring_L)
    if out is None:
        out = torch.empty((B, T, Hq, d), dtype=dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _check(out, "out", dtype, 4)
    _check(lse, "lse", torch.float32, 3)
    if tuple(out.shape) != (B, T, Hq, d) or tuple(lse.shape) != (B, Hq, T):
        raise ValueError("out must be [B,T,Hq,d] and lse [B,Hq,T]")
    sizes = (B, T, Hq, Hk, d, S, L) if ring_L is not None else (B, T, Hq, Hk, d, L)
    rc = getattr(_lib.load(), fn_name)(_ptr(q), _ptr(k_seq), _ptr(v_seq), _ptr(k_depth), _ptr(v_depth),
                                       *sizes, int(bool(causal)), _ptr(out), _ptr(lse), _stream(stream))
    if rc != MODA_OK:
        raise MODAError(fn_name, rc)
    return out, lse


def moda_attn_fwd(q, k_seq, v_seq, k_depth=None, v_depth=None, causal=True, out=None, lse=None, stream=None):
    """MoDA forward, bf16.  q [B,T,Hq,d]; k_seq, v_seq [B,T,Hk,d]; k_depth, v_depth packed
    [B,T,Hk,L,d] (None for L = 0).  Returns (out [B,T,Hq,d] bf16, lse [B,Hq,T] fp32)."""
    return _fwd("moda_attn_fwd", torch.bfloat16, q, k_seq, v_seq, k_depth, v_depth, causal, out, lse, stream)


def moda_attn_fwd_ring(q, k_seq, v_seq, k_depth, v_depth, L, causal=True, out=None, lse=None, stream=None):
    """MoDA forward over a bounded depth cache: k_depth, v_depth are [B,T,Hk,S,d] ring slots, of which
    the first L <= S are attended.  Returns (out, lse) as moda_attn_fwd."""
    return _fwd("moda_attn_fwd_ring", torch.bfloat16, q, k_seq, v_seq, k_depth, v_depth, causal, out, lse,
                stream, ring_L=L)


def moda_attn_fwd_f32(q, k_seq, v_seq, k_depth=None, v_depth=None, causal=True, out=None, lse=None, stream=None):
    """MoDA forward, fp32 throughout.  Same layouts as moda_attn_fwd."""
    return _fwd("moda_attn_fwd_f32", torch.float32, q, k_seq, v_seq, k_depth, v_depth, causal, out, lse, stream)


def moda_attn_bwd_workspace(B, T, Hq, Hk, d, L):
    """Bytes of workspace moda_attn_bwd needs (0 for invalid sizes)."""
    return int(_lib.load().moda_attn_bwd_workspace(B, T, Hq, Hk, d, L))


def moda_attn_bwd(q, k_seq, v_seq, k_depth, v_depth, out, lse, dout, causal=True, grads=None, workspace=None,
                  stream=None):
    """MoDA backward, bf16.  Inputs as given to moda_attn_fwd (k_depth, v_depth packed [B,T,Hk,L,d] or None),
    that call's (out, lse), and dout [B,T,Hq,d].  grads: optional preallocated (dq, dk, dv, dkd, dvd);
    workspace: a uint8 GPU tensor of at least moda_attn_bwd_workspace(...) bytes (allocated here when None).
    Returns (dq [B,T,Hq,d], dk_seq, dv_seq [B,T,Hk,d], dk_depth, dv_depth [B,T,Hk,L,d] or None), all bf16."""
    dtype = torch.bfloat16
    for t, n in ((q, "q"), (k_seq, "k_seq"), (v_seq, "v_seq"), (out, "out"), (dout, "dout")):
        _check(t, n, dtype, 4)
    _check(lse, "lse", torch.float32, 3)
    B, T, Hq, d = q.shape
    Hk = k_seq.shape[2]
    if tuple(k_seq.shape) != (B, T, Hk, d) or tuple(v_seq.shape) != (B, T, Hk, d):
        raise ValueError("k_seq / v_seq must be [B,T,Hk,d] = %s" % ((B, T, Hk, d),))
    if tuple(out.shape) != (B, T, Hq, d) or tuple(dout.shape) != (B, T, Hq, d) or tuple(lse.shape) != (B, Hq, T):
        raise ValueError("out, dout must be [B,T,Hq,d] and lse [B,Hq,T]")
    L = 0
    if k_depth is not None and k_depth.numel() > 0:
        _check(k_depth, "k_depth", dtype, 5)
        _check(v_depth, "v_depth", dtype, 5)
        L = k_depth.shape[3]
        if tuple(k_depth.shape) != (B, T, Hk, L, d) or tuple(v_depth.shape) != (B, T, Hk, L, d):
            raise ValueError("packed depth K/V must be [B,T,Hk,L,d] = %s" % ((B, T, Hk, L, d),))
    else:
        k_depth = v_depth = None
    if grads is None:
        dev = q.device
        grads = (torch.empty_like(q), torch.empty_like(k_seq), torch.empty_like(v_seq),
                 torch.empty((B, T, Hk, L, d), dtype=dtype, device=dev) if L else None,
                 torch.empty((B, T, Hk, L, d), dtype=dtype, device=dev) if L else None)
    dq, dk, dv, dkd, dvd = grads
    _check(dq, "dq", dtype, 4)
    _check(dk, "dk_seq", dtype, 4)
    _check(dv, "dv_seq", dtype, 4)
    if tuple(dq.shape) != (B, T, Hq, d) or tuple(dk.shape) != (B, T, Hk, d) or tuple(dv.shape) != (B, T, Hk, d):
        raise ValueError("dq must be [B,T,Hq,d] and dk_seq, dv_seq [B,T,Hk,d]")
    if L:
        _check(dkd, "dk_depth", dtype, 5)
        _check(dvd, "dv_depth", dtype, 5)
        if tuple(dkd.shape) != (B, T, Hk, L, d) or tuple(dvd.shape) != (B, T, Hk, L, d):
            raise ValueError("dk_depth / dv_depth must be [B,T,Hk,L,d]")
    need = moda_attn_bwd_workspace(B, T, Hq, Hk, d, L)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(workspace, "workspace", torch.uint8, 1)
    rc = _lib.load().moda_attn_bwd(_ptr(q), _ptr(k_seq), _ptr(v_seq), _ptr(k_depth), _ptr(v_depth), _ptr(out),
                                   _ptr(lse), _ptr(dout), B, T, Hq, Hk, d, L, int(bool(causal)),
                                   _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dkd if L else None), _ptr(dvd if L else None),
                                   _ptr(workspace), workspace.numel(), _stream(stream))
    if rc != MODA_OK:
        raise MODAError("moda_attn_bwd", rc)
    return dq, dk, dv, (dkd if L else None), (dvd if L else None)


def moda_attn_decode_workspace(B, T, Hq, Hk, d, L):
    """Bytes of workspace moda_attn_decode needs (0 for invalid sizes)."""
    return int(_lib.load().moda_attn_decode_workspace(B, T, Hq, Hk, d, L))


def moda_attn_decode_ring(q, k_cache, v_cache, k_depth, v_depth, L, out=None, lse=None, workspace=None,
                          stream=None):
    """Decode step over a bounded depth cache: k_depth, v_depth are [B,Hk,S,d] ring slots, of which the
    first L <= S are attended.  Returns (out, lse) as moda_attn_decode."""
    return moda_attn_decode(q, k_cache, v_cache, k_depth, v_depth, out, lse, workspace, stream, ring_L=L)


def moda_attn_decode(q, k_cache, v_cache, k_depth=None, v_depth=None, out=None, lse=None, workspace=None,
                     stream=None, ring_L=None):
    """MoDA decode step, bf16.  q [B,Hq,d]; k_cache, v_cache [B,T,Hk,d]; k_depth, v_depth [B,Hk,L,d]
    (the decode token's depth slab; None for L = 0).  workspace: a uint8 GPU tensor of at least
    moda_attn_decode_workspace(...) bytes (allocated here when None).  Returns (out [B,Hq,d] bf16,
    lse [B,Hq] fp32)."""
    dtype = torch.bfloat16
    _check(q, "q", dtype, 3)
    _check(k_cache, "k_cache", dtype, 4)
    _check(v_cache, "v_cache", dtype, 4)
    B, Hq, d = q.shape
    T, Hk = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, T, Hk, d) or tuple(v_cache.shape) != (B, T, Hk, d):
        raise ValueError("k_cache / v_cache must be [B,T,Hk,d] = %s" % ((B, T, Hk, d),))
    L = 0
    if k_depth is not None and k_depth.numel() > 0:
        _check(k_depth, "k_depth", dtype, 4)
        _check(v_depth, "v_depth", dtype, 4)
        L = k_depth.shape[2]
        if tuple(k_depth.shape) != (B, Hk, L, d) or tuple(v_depth.shape) != (B, Hk, L, d):
            raise ValueError("depth K/V must be [B,Hk,L,d] = %s" % ((B, Hk, L, d),))
    else:
        k_depth = v_depth = None
    S = L
    if ring_L is not None:
        if not 0 <= ring_L <= S:
            raise ValueError("ring: need 0 <= L <= S = %d, got L = %d" % (S, ring_L))
        L = int(ring_L)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check(out, "out", dtype, 3)
    _check(lse, "lse", torch.float32, 2)
    if tuple(out.shape) != (B, Hq, d) or tuple(lse.shape) != (B, Hq):
        raise ValueError("out must be [B,Hq,d] and lse [B,Hq]")
    need = moda_attn_decode_workspace(B, T, Hq, Hk, d, L)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(workspace, "workspace", torch.uint8, 1)
    lib = _lib.load()
    if ring_L is not None:
        rc = lib.moda_attn_decode_ring(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_depth), _ptr(v_depth),
                                       B, T, Hq, Hk, d, S, L, _ptr(out), _ptr(lse), _ptr(workspace),
                                       workspace.numel(), _stream(stream))
    else:
        rc = lib.moda_attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_depth), _ptr(v_depth),
                                  B, T, Hq, Hk, d, L, _ptr(out), _ptr(lse), _ptr(workspace),
                                  workspace.numel(), _stream(stream))
    if rc != MODA_OK:
        raise MODAError("moda_attn_decode_ring" if ring_L is not None else "moda_attn_decode", rc)
    return out, lse


def moda_attn_decode_noalloc(q, k_cache, v_cache, k_depth, v_depth, out, lse, stream=None):
    """moda_attn_decode with no workspace: the library keeps the partial results in its fixed
    per-GPU scratch (MODA_DECODE_NOALLOC_SCRATCH_BYTES), so the call allocates nothing.  out
    [B,Hq,d] bf16 and lse [B,Hq] fp32 are the caller's; other arguments as moda_attn_decode
    (k_depth, v_depth None for L = 0).  Calls that overlap in time on one GPU race on the
    scratch.  Returns (out, lse)."""
    dtype = torch.bfloat16
    _check(q, "q", dtype, 3)
    _check(k_cache, "k_cache", dtype, 4)
    _check(v_cache, "v_cache", dtype, 4)
    B, Hq, d = q.shape
    T, Hk = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, T, Hk, d) or tuple(v_cache.shape) != (B, T, Hk, d):
        raise ValueError("k_cache / v_cache must be [B,T,Hk,d] = %s" % ((B, T, Hk, d),))
    L = 0
    if k_depth is not None and k_depth.numel() > 0:
        _check(k_depth, "k_depth", dtype, 4)
        _check(v_depth, "v_depth", dtype, 4)
        L = k_depth.shape[2]
        if tuple(k_depth.shape) != (B, Hk, L, d) or tuple(v_depth.shape) != (B, Hk, L, d):
            raise ValueError("depth K/V must be [B,Hk,L,d] = %s" % ((B, Hk, L, d),))
    else:
        k_depth = v_depth = None
    _check(out, "out", dtype, 3)
    _check(lse, "lse", torch.float32, 2)
    if tuple(out.shape) != (B, Hq, d) or tuple(lse.shape) != (B, Hq):
        raise ValueError("out must be [B,Hq,d] and lse [B,Hq]")
    rc = _lib.load().moda_attn_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_depth),
                                              _ptr(v_depth), B, T, Hq, Hk, d, L, _ptr(out), _ptr(lse),
                                              _stream(stream))
    if rc != MODA_OK:
        raise MODAError("moda_attn_decode_noalloc", rc)
    return out, lse


def moda_kv_project(x, w_kv, Hk, d, k_out=None, v_out=None, k_depth=None, v_depth=None, slot=0, stream=None):
    """KV projection of x [B,T,Dm] by w_kv [2*Hk*d, Dm] (K rows, then V rows), bf16.  Writes the
    result into k_out, v_out [B,T,Hk,d] and/or slot `slot` of the packed depth buffers k_depth,
    v_depth [B,T,Hk,S,d]; with neither given, allocates and returns (k_out, v_out).  Returns
    (k_out, v_out, k_depth, v_depth)."""
    dtype = torch.bfloat16
    _check(x, "x", dtype, 3)
    _check(w_kv, "w_kv", dtype, 2)
    B, T, Dm = x.shape
    if tuple(w_kv.shape) != (2 * Hk * d, Dm):
        raise ValueError("w_kv must be [2*Hk*d, Dm] = %s" % ((2 * Hk * d, Dm),))
    if k_out is None and k_depth is None:
        k_out = torch.empty((B, T, Hk, d), dtype=dtype, device=x.device)
        v_out = torch.empty_like(k_out)
    S = 0
    if k_out is not None:
        for t, n in ((k_out, "k_out"), (v_out, "v_out")):
            _check(t, n, dtype, 4)
            if tuple(t.shape) != (B, T, Hk, d):
                raise ValueError("%s must be [B,T,Hk,d]" % n)
    if k_depth is not None:
        for t, n in ((k_depth, "k_depth"), (v_depth, "v_depth")):
            _check(t, n, dtype, 5)
        S = k_depth.shape[3]
        if tuple(k_depth.shape) != (B, T, Hk, S, d) or tuple(v_depth.shape) != (B, T, Hk, S, d):
            raise ValueError("depth buffers must be [B,T,Hk,S,d]")
    rc = _lib.load().moda_kv_project(_ptr(x), _ptr(w_kv), B, T, Dm, Hk, d, _ptr(k_out), _ptr(v_out),
                                     _ptr(k_depth), _ptr(v_depth), S, int(slot), _stream(stream))
    if rc != MODA_OK:
        raise MODAError("moda_kv_project", rc)
    return k_out, v_out, k_depth, v_depth


def _layout_check(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous GPU tensor" % name)


def moda_pack_depth(src, dst=None, stream=None):
    """Depth-stream pack: src [B,T,L,Hk,d] -> dst [B,T,Hk,L,d] (bit copy).  Returns dst."""
    _layout_check(src, "src")
    if src.dim() != 5:
        raise ValueError("src must be [B,T,L,Hk,d]")
    B, T, L, Hk, d = src.shape
    if dst is None:
        dst = torch.empty((B, T, Hk, L, d), dtype=src.dtype, device=src.device)
    _layout_check(dst, "dst")
    if tuple(dst.shape) != (B, T, Hk, L, d) or dst.dtype != src.dtype:
        raise ValueError("dst must be [B,T,Hk,L,d] of src's dtype")
    rc = _lib.load().moda_pack_depth(_ptr(src), _ptr(dst), B, T, L, Hk, d, src.element_size(), _stream(stream))
    if rc != MODA_OK:
        raise MODAError("moda_pack_depth", rc)
    return dst


def moda_append_depth_slot(kv_l, dst, slot, stream=None):
    """Write kv_l [B,T,Hk,d] into slot `slot` of the packed depth tensor dst [B,T,Hk,L,d]."""
    _layout_check(kv_l, "kv_l")
    _layout_check(dst, "dst")
    if dst.dim() != 5 or kv_l.dim() != 4:
        raise ValueError("kv_l must be [B,T,Hk,d] and dst [B,T,Hk,L,d]")
    B, T, Hk, L, d = dst.shape
    if tuple(kv_l.shape) != (B, T, Hk, d) or kv_l.dtype != dst.dtype:
        raise ValueError("kv_l must be [B,T,Hk,d] of dst's dtype")
    rc = _lib.load().moda_append_depth_slot(_ptr(kv_l), _ptr(dst), int(slot), B, T, L, Hk, d,
                                            dst.element_size(), _stream(stream))
    if rc != MODA_OK:
        raise MODAError("moda_append_depth_slot", rc)
    return dst


def moda_block_span(row0, rows, G):
    """(t_start, t_end) of expanded query rows [row0, row0 + rows) under group size G."""
    a, b = ctypes.c_int(), ctypes.c_int()
    rc = _lib.load().moda_block_span(int(row0), int(rows), int(G), ctypes.byref(a), ctypes.byref(b))
    if rc != MODA_OK:
        raise MODAError("moda_block_span", rc)
    return a.value, b.value

"""The C ABI without a GPU: the library loads, exports every declared symbol, and every
validation error is produced on the host before any HIP call."""
import ctypes
import json
import os

import pytest

from depth_stream_attention_amd import _lib
from depth_stream_attention_amd import api

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
A = ctypes.c_void_p(0x10000)      # aligned fake device addresses: never dereferenced,
A2 = ctypes.c_void_p(0x20000)     # validation fails before any HIP call
MIS = ctypes.c_void_p(0x10008)    # 8-byte aligned only


@pytest.fixture(scope="module")
def lib():
    return _lib.ensure_built()


def test_exports_every_declared_symbol(lib):
    names = _lib.declared_symbols()
    assert {"moda_attn_fwd", "moda_attn_fwd_f32", "moda_pack_depth", "moda_append_depth_slot",
            "moda_error_string", "moda_block_span", "moda_attn_decode", "moda_attn_decode_workspace"} <= set(names)
    for n in names:
        assert hasattr(lib, n), "libmoda.so does not export %s" % n


def test_error_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = api.moda_error_string(code)
        assert s and s != "unknown error"
    assert api.moda_error_string(17) == "unknown error"


def fwd(lib, name="moda_attn_fwd", q=A, k=A, v=A, kd=A, vd=A, B=1, T=16, Hq=4, Hk=2, d=128, L=2,
        causal=1, out=A2, lse=A2):
    return getattr(lib, name)(q, k, v, kd, vd, B, T, Hq, Hk, d, L, causal, out, lse, None)


@pytest.mark.parametrize("name", ["moda_attn_fwd", "moda_attn_fwd_f32"])
def test_fwd_validation(lib, name):
    N, S, U, AL = api.MODA_ERR_NULL, api.MODA_ERR_SHAPE, api.MODA_ERR_UNSUPPORTED, api.MODA_ERR_ALIGN
    f = lambda **kw: fwd(lib, name, **kw)  # noqa: E731
    assert f(q=None) == N and f(k=None) == N and f(v=None) == N
    assert f(out=None) == N and f(lse=None) == N
    assert f(kd=None) == N and f(vd=None) == N
    assert f(kd=None, vd=None, L=0) != N              # depth may be NULL when L == 0
    for kw in ({"B": 0}, {"T": 0}, {"Hq": 0}, {"Hk": 0}, {"d": 0}, {"L": -1}, {"Hq": 6, "Hk": 4},
               {"causal": 2}, {"causal": -1}):
        assert f(**kw) == S, kw
    for kw in ({"d": 96}, {"d": 256}, {"Hq": 6, "Hk": 2}, {"Hq": 128, "Hk": 2}):
        assert f(**kw) == U, kw
    for kw in ({"q": MIS}, {"k": MIS}, {"v": MIS}, {"kd": MIS}, {"vd": MIS}, {"out": MIS}, {"lse": MIS}):
        assert f(**kw) == AL, kw
    assert f(kd=MIS, vd=MIS, L=0) != AL                # depth pointers are ignored when L == 0
    assert f(T=(1 << 30), Hq=32, Hk=1) == U            # expanded rows beyond int32 launch limits
    if name == "moda_attn_fwd":                        # 32-bit buffer offsets of the bf16 kernel
        assert f(T=(1 << 22), Hq=16, Hk=8) == U
        assert f(L=1024, Hq=64, Hk=64) == U
        # A workgroup's depth window spans (rows per workgroup + 1) * Hk * L * d * 2 bytes:
        # with d=128, 128 rows below 32768 tokens and 256 from there on; with d=64, 128
        # rows at every length.  Hk=8, d=128, L=4081 fits the 32-bit offsets with 128 rows
        # (1.08e9 bytes) but not with 256 (2.148e9 > 2^31); Hk=8, d=64, L=8162 is the same
        # byte count.  A misaligned lse makes the accepted shape stop at the (later)
        # alignment check, so nothing is launched with these placeholder pointers.
        assert f(T=32767, Hq=8, Hk=8, L=4081, lse=MIS) == AL
        assert f(T=32768, Hq=8, Hk=8, L=4081, lse=MIS) == U
        assert f(T=32768, Hq=8, Hk=8, d=64, L=8162, lse=MIS) == AL


def test_layout_validation(lib):
    N, S, AL = api.MODA_ERR_NULL, api.MODA_ERR_SHAPE, api.MODA_ERR_ALIGN
    p = lambda src=A, dst=A2, B=1, T=4, L=3, Hk=2, d=128, eb=2: lib.moda_pack_depth(  # noqa: E731
        src, dst, B, T, L, Hk, d, eb, None)
    assert p(src=None) == N and p(dst=None) == N
    for kw in ({"B": 0}, {"T": -1}, {"L": 0}, {"Hk": 0}, {"d": 0}, {"eb": 3}, {"eb": 0}):
        assert p(**kw) == S, kw
    assert p(src=MIS) == AL and p(dst=MIS) == AL
    a = lambda kv=A, dst=A2, slot=0, B=1, T=4, L=3, Hk=2, d=128, eb=2: lib.moda_append_depth_slot(  # noqa: E731
        kv, dst, slot, B, T, L, Hk, d, eb, None)
    assert a(kv=None) == N and a(dst=None) == N
    assert a(slot=-1) == S and a(slot=3) == S and a(L=0) == S and a(eb=16) == S
    assert a(kv=MIS) == AL


def test_block_span_matches_pages_example(lib):
    with open(os.path.join(GOLDEN, "group_rows_example.json")) as f:
        ex = json.load(f)
    rows = ex["rows_last"] - ex["rows_first"] + 1
    assert api.moda_block_span(ex["rows_first"], rows, ex["G"]) == (ex["t_start"], ex["t_end"])
    assert sorted({r // ex["G"] for r in range(ex["rows_first"], ex["rows_last"] + 1)}) == ex["base_times"]


def test_block_span_against_brute_force(lib):
    for G in (1, 2, 3, 4, 8, 32):
        for row0 in range(0, 70, 7):
            for rows in (1, 5, 32, 128):
                ts = [r // G for r in range(row0, row0 + rows)]
                assert api.moda_block_span(row0, rows, G) == (min(ts), max(ts) + 1)
    with pytest.raises(api.MODAError):
        api.moda_block_span(-1, 4, 2)
    with pytest.raises(api.MODAError):
        api.moda_block_span(0, 0, 2)


def decode(lib, q=A, kc=A, vc=A, kd=A, vd=A, B=2, T=300, Hq=8, Hk=2, d=128, L=5, out=A2, lse=A2, ws=A2,
           ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.moda_attn_decode_workspace(B, T, Hq, Hk, d, L)
    return lib.moda_attn_decode(q, kc, vc, kd, vd, B, T, Hq, Hk, d, L, out, lse, ws, ws_bytes, None)


def test_decode_workspace_size(lib):
    # (d + 2) fp32 per (b, h, chunk).  Chunks: the largest of 1024/512/256 keys giving at
    # least 512 workgroups over B*Hk, else 128; plus one chunk for the depth slots when L > 0.
    assert lib.moda_attn_decode_workspace(2, 300, 8, 2, 128, 5) == 2 * 8 * (3 + 1) * 130 * 4
    assert lib.moda_attn_decode_workspace(1, 256, 4, 4, 64, 0) == 1 * 4 * 2 * 66 * 4
    assert lib.moda_attn_decode_workspace(1, 257, 4, 4, 64, 0) == 1 * 4 * 3 * 66 * 4
    assert lib.moda_attn_decode_workspace(16, 65536, 16, 4, 128, 48) == 16 * 16 * (64 + 1) * 130 * 4
    assert lib.moda_attn_decode_workspace(1, 65536, 16, 4, 128, 48) == 16 * (128 + 1) * 130 * 4
    assert lib.moda_attn_decode_workspace(0, 256, 4, 4, 64, 0) == 0
    assert lib.moda_attn_decode_workspace(1, 256, 4, 4, 64, -1) == 0
    assert lib.moda_attn_decode_workspace(1, 256, 6, 4, 64, 0) == 0


def test_decode_validation(lib):
    null = ctypes.c_void_p(0)
    for kw in (dict(q=null), dict(kc=null), dict(vc=null), dict(out=null), dict(lse=null), dict(ws=null),
               dict(kd=null), dict(vd=null)):
        assert decode(lib, **kw) == api.MODA_ERR_NULL, kw
    for kw in (dict(B=0), dict(T=0), dict(Hq=0), dict(Hk=0), dict(d=0), dict(L=-1), dict(Hq=6, Hk=4)):
        assert decode(lib, **kw) == api.MODA_ERR_SHAPE, kw
    assert decode(lib, ws_bytes=lib.moda_attn_decode_workspace(2, 300, 8, 2, 128, 5) - 4) == api.MODA_ERR_SHAPE
    for kw in (dict(d=96), dict(Hq=6, Hk=2), dict(Hq=128, Hk=2)):
        assert decode(lib, **kw) == api.MODA_ERR_UNSUPPORTED, kw
    for kw in (dict(q=MIS), dict(kc=MIS), dict(vc=MIS), dict(kd=MIS), dict(vd=MIS), dict(out=MIS), dict(ws=MIS)):
        assert decode(lib, **kw) == api.MODA_ERR_ALIGN, kw


def test_decode_noalloc_validation(lib):
    # every error comes from the host checks, before the scratch lookup or any launch
    null = ctypes.c_void_p(0)

    def dec(q=A, kc=A, vc=A, kd=A, vd=A, B=2, T=300, Hq=8, Hk=2, d=128, L=5, out=A2, lse=A2):
        return lib.moda_attn_decode_noalloc(q, kc, vc, kd, vd, B, T, Hq, Hk, d, L, out, lse, None)

    for kw in (dict(q=null), dict(kc=null), dict(vc=null), dict(out=null), dict(lse=null), dict(kd=null),
               dict(vd=null)):
        assert dec(**kw) == api.MODA_ERR_NULL, kw
    for kw in (dict(B=0), dict(T=0), dict(Hq=0), dict(Hk=0), dict(d=0), dict(L=-1), dict(Hq=6, Hk=4)):
        assert dec(**kw) == api.MODA_ERR_SHAPE, kw
    for kw in (dict(d=96), dict(Hq=6, Hk=2), dict(Hq=128, Hk=2)):
        assert dec(**kw) == api.MODA_ERR_UNSUPPORTED, kw
    for kw in (dict(q=MIS), dict(kc=MIS), dict(vc=MIS), dict(kd=MIS), dict(vd=MIS), dict(out=MIS)):
        assert dec(**kw) == api.MODA_ERR_ALIGN, kw
    # the fixed scratch: the decode workspace of B=16 T=65536 Hq=16 Hk=4 d=128 L=48 fits, B=32 does not
    cap = api.MODA_DECODE_NOALLOC_SCRATCH_BYTES
    assert lib.moda_attn_decode_workspace(16, 65536, 16, 4, 128, 48) <= cap
    assert lib.moda_attn_decode_workspace(32, 65536, 16, 4, 128, 48) > cap
    assert dec(B=32, T=65536, Hq=16, Hk=4, L=48) == api.MODA_ERR_TOO_LARGE


def test_ring_validation(lib):
    null = ctypes.c_void_p(0)
    ring = lambda S, L, kd=A, vd=A: lib.moda_attn_fwd_ring(A, A, A, kd, vd, 1, 16, 4, 2, 128, S, L, 1, A2, A2,
                                                             None)
    assert ring(4, 5) == api.MODA_ERR_SHAPE            # more attended slots than the ring holds
    assert ring(4, -1) == api.MODA_ERR_SHAPE
    assert ring(4, 2, kd=null) == api.MODA_ERR_NULL
    assert ring(4, 2, vd=MIS) == api.MODA_ERR_ALIGN
    assert ring(1 << 20, 2) == api.MODA_ERR_UNSUPPORTED  # slot stride beyond the 32-bit offsets
    dec = lambda S, L: lib.moda_attn_decode_ring(A, A, A, A, A, 1, 300, 8, 2, 128, S, L, A2, A2, A2,
                                                 lib.moda_attn_decode_workspace(1, 300, 8, 2, 128, max(L, 0)), None)
    assert dec(4, 5) == api.MODA_ERR_SHAPE
    assert dec(4, -1) == api.MODA_ERR_SHAPE


def bwd(lib, q=A, k=A, v=A, kd=A, vd=A, out=A, lse=A, do=A, B=2, T=300, Hq=8, Hk=2, d=128, L=5, causal=1,
        dq=A, dk=A, dv=A, dkd=A, dvd=A, ws=A2, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.moda_attn_bwd_workspace(B, T, Hq, Hk, d, L)
    return lib.moda_attn_bwd(q, k, v, kd, vd, out, lse, do, B, T, Hq, Hk, d, L, causal, dq, dk, dv, dkd, dvd,
                             ws, ws_bytes, None)


def test_bwd_workspace_size(lib):
    # lse2 and Dsum (fp32 per query row), plus the fp32 depth share of dq when L > 0;
    # each region rounded up to 256 bytes.
    r = lambda n: (n + 255) // 256 * 256  # noqa: E731
    assert lib.moda_attn_bwd_workspace(2, 300, 8, 2, 128, 5) == 2 * r(2 * 300 * 8 * 4) + r(2 * 300 * 8 * 128 * 4)
    assert lib.moda_attn_bwd_workspace(2, 300, 8, 2, 128, 0) == 2 * r(2 * 300 * 8 * 4)
    assert lib.moda_attn_bwd_workspace(1, 65536, 16, 4, 128, 48) == 2 * 65536 * 16 * 4 + 65536 * 16 * 128 * 4
    assert lib.moda_attn_bwd_workspace(0, 256, 4, 4, 64, 0) == 0
    assert lib.moda_attn_bwd_workspace(1, 256, 4, 4, 64, -1) == 0
    assert lib.moda_attn_bwd_workspace(1, 256, 6, 4, 64, 0) == 0


def test_bwd_validation(lib):
    null = ctypes.c_void_p(0)
    for name in ("q", "k", "v", "out", "lse", "do", "dq", "dk", "dv", "ws", "kd", "vd", "dkd", "dvd"):
        assert bwd(lib, **{name: null}) == api.MODA_ERR_NULL, name
    # depth pointers may be NULL when L == 0
    assert bwd(lib, L=0, kd=null, vd=null, dkd=null, dvd=null, ws=MIS) == api.MODA_ERR_ALIGN
    for kw in (dict(B=0), dict(T=0), dict(Hq=0), dict(Hk=0), dict(d=0), dict(L=-1), dict(Hq=6, Hk=4),
               dict(causal=2)):
        assert bwd(lib, **kw) == api.MODA_ERR_SHAPE, kw
    assert bwd(lib, ws_bytes=lib.moda_attn_bwd_workspace(2, 300, 8, 2, 128, 5) - 4) == api.MODA_ERR_SHAPE
    # G = 64 has no kernel; sizes beyond the 32-bit offsets are refused
    for kw in (dict(d=96), dict(Hq=6, Hk=2), dict(Hq=128, Hk=2), dict(T=1 << 20, Hq=16, Hk=2)):
        assert bwd(lib, **kw) == api.MODA_ERR_UNSUPPORTED, kw
    for name in ("q", "k", "v", "kd", "vd", "out", "lse", "do", "dq", "dk", "dv", "dkd", "dvd", "ws"):
        assert bwd(lib, **{name: MIS}) == api.MODA_ERR_ALIGN, name


def kvp(lib, x=A, w=A, B=2, T=100, Dm=256, Hk=2, d=128, ko=A, vo=A, kd=A, vd=A, S=4, slot=1):
    return lib.moda_kv_project(x, w, B, T, Dm, Hk, d, ko, vo, kd, vd, S, slot, None)


def test_kv_project_validation(lib):
    null = ctypes.c_void_p(0)
    for kw in (dict(x=null), dict(w=null), dict(ko=null, vo=null, kd=null, vd=null), dict(ko=null),
               dict(vd=null)):
        assert kvp(lib, **kw) == api.MODA_ERR_NULL, kw
    for kw in (dict(B=0), dict(T=0), dict(Dm=0), dict(Hk=0), dict(d=0), dict(slot=4), dict(slot=-1), dict(S=0)):
        assert kvp(lib, **kw) == api.MODA_ERR_SHAPE, kw
    # without depth buffers S and slot are not looked at
    assert kvp(lib, kd=null, vd=null, slot=9, x=MIS) == api.MODA_ERR_ALIGN
    for kw in (dict(d=96), dict(Dm=96), dict(Dm=1 << 23)):
        assert kvp(lib, **kw) == api.MODA_ERR_UNSUPPORTED, kw
    for name in ("x", "w", "ko", "vo", "kd", "vd"):
        assert kvp(lib, **{name: MIS}) == api.MODA_ERR_ALIGN, name


def test_probe_library_exports_and_validates():
    # the measurement kernels' library: every declared symbol, and host-side argument checks
    probe = _lib.load_probe()
    names = _lib.declared_symbols(_lib.PROBE_HEADER)
    assert {"moda_probe_mfma_bf16", "moda_probe_copy", "moda_probe_read"} <= set(names)
    for n in names:
        assert hasattr(probe, n), "libmoda_probe.so does not export %s" % n
    null = ctypes.c_void_p(0)
    assert probe.moda_probe_mfma_bf16(null, 4, 4, 1, None) == api.MODA_ERR_NULL
    assert probe.moda_probe_mfma_bf16(A, 0, 4, 1, None) == api.MODA_ERR_SHAPE
    assert probe.moda_probe_mfma_bf16(A, 4, 0, 1, None) == api.MODA_ERR_SHAPE
    assert probe.moda_probe_mfma_bf16(A, 4, 4, 2, None) == api.MODA_ERR_SHAPE
    assert probe.moda_probe_mfma_bf16(MIS, 4, 4, 1, None) == api.MODA_ERR_ALIGN
    assert probe.moda_probe_copy(null, A2, 64, 4, None) == api.MODA_ERR_NULL
    assert probe.moda_probe_copy(A, A2, 63, 4, None) == api.MODA_ERR_SHAPE
    assert probe.moda_probe_copy(A, A2, 0, 4, None) == api.MODA_ERR_SHAPE
    assert probe.moda_probe_copy(A, A2, 64, 0, None) == api.MODA_ERR_SHAPE
    assert probe.moda_probe_copy(A, MIS, 64, 4, None) == api.MODA_ERR_ALIGN
    assert probe.moda_probe_read(A, 64, 4, null, None) == api.MODA_ERR_NULL
    assert probe.moda_probe_read(A, 40, 4, A2, None) == api.MODA_ERR_SHAPE
    assert probe.moda_probe_read(MIS, 64, 4, A2, None) == api.MODA_ERR_ALIGN

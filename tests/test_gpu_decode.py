"""GPU parity of the decode step (moda_attn_decode) against the fp64 oracle.

The decode of the token at position T-1 is, by definition, row t = T-1 of the
causal forward on the same inputs (every cached key is visible; the depth set
is that token's own slots), so the expected values are the oracle's rows
(b, T-1, h).  bf16 bounds as for the forward: max|err| <= 2e-2 and
mean|err| <= 2e-3 on out, |dlse| <= 1e-3."""
import numpy as np
import pytest
import torch

import oracle
from depth_stream_attention_amd import api
from depth_stream_attention_amd import inputs as I
from parity_util import check, say

pytestmark = pytest.mark.gpu
S = I.Shape


def decode_case(shape, seed, workspace=None):
    host = I.random_inputs(shape, seed)
    B, T, Hq, Hk, d, L = shape.B, shape.T, shape.Hq, shape.Hk, shape.d, shape.L
    q = host["q"][:, T - 1].contiguous().cuda()
    kc, vc = host["k_seq"].cuda(), host["v_seq"].cuda()
    kd = host["k_depth"][:, T - 1].permute(0, 2, 1, 3).contiguous().cuda() if L else None  # [B,Hk,L,d]
    vd = host["v_depth"][:, T - 1].permute(0, 2, 1, 3).contiguous().cuda() if L else None
    out, lse = api.moda_attn_decode(q, kc, vc, kd, vd, workspace=workspace)
    torch.cuda.synchronize()
    rows = np.array([(b, T - 1, h) for b in range(B) for h in range(Hq)], dtype=np.int32)
    ref_out, ref_lse = oracle.moda_fwd_rows(host["q"], host["k_seq"], host["v_seq"], host["k_depth"],
                                            host["v_depth"], rows, causal=True)
    got_out = out.float().cpu().numpy().reshape(B * Hq, d)
    got_lse = lse.cpu().numpy().reshape(B * Hq)
    return check(shape, got_out, got_lse, ref_out, ref_lse, "decode")


@pytest.mark.parametrize("T", [1, 2, 31, 32, 33, 127, 128, 129, 255, 256, 257, 1000])
def test_decode_cache_lengths(T):
    # B*Hk = 4 workgroups per chunk index: the smallest (128-key) chunks.
    decode_case(S(2, T, 8, 2, 128, 5), 500 + T)


@pytest.mark.parametrize("B,T,Hk", [(1, 33000, 4), (2, 33000, 4), (8, 16389, 4)])
def test_decode_chunk_sizes(B, T, Hk):
    """Shapes that select 256-, 512- and 1024-key chunks, each with a ragged last chunk."""
    decode_case(S(B, T, 4 * Hk, Hk, 128, 6), 550 + B)


@pytest.mark.parametrize("L", [0, 1, 16, 48, 65, 200])
def test_decode_depth_slots(L):
    decode_case(S(1, 700, 16, 4, 128, L), 600 + L)


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16, 32])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_group_sizes(G, d):
    decode_case(S(2, 333, 2 * G, 2, d, 7), 700 + 10 * G + d)


def test_decode_long_cache():
    decode_case(S(1, 20000, 16, 4, 128, 48), 800)


def test_decode_depth_dominant():
    """Depth keys aligned with the queries dominate the softmax: a decode that drops or
    mis-indexes the depth chunk fails here even though depth is a small share of keys."""
    shape = S(1, 3000, 8, 2, 128, 24)
    host = I.make_inputs(shape, {n: 900 + k for k, n in enumerate(I.TENSORS)}, depth_aligned=True)
    B, T, Hq, Hk, d, L = shape.B, shape.T, shape.Hq, shape.Hk, shape.d, shape.L
    q = host["q"][:, T - 1].contiguous().cuda()
    kd = host["k_depth"][:, T - 1].permute(0, 2, 1, 3).contiguous().cuda()
    vd = host["v_depth"][:, T - 1].permute(0, 2, 1, 3).contiguous().cuda()
    out, lse = api.moda_attn_decode(q, host["k_seq"].cuda(), host["v_seq"].cuda(), kd, vd)
    torch.cuda.synchronize()
    rows = np.array([(0, T - 1, h) for h in range(Hq)], dtype=np.int32)
    ref_out, ref_lse = oracle.moda_fwd_rows(host["q"], host["k_seq"], host["v_seq"], host["k_depth"],
                                            host["v_depth"], rows, causal=True)
    check(shape, out.float().cpu().numpy().reshape(Hq, d), lse.cpu().numpy().reshape(Hq), ref_out, ref_lse,
          "decode depth-aligned")


def test_decode_workspace_reuse_and_determinism():
    """One caller-owned workspace reused across calls of different sizes; a repeated call
    gives bit-identical results (fixed merge order, no atomics)."""
    big = api.moda_attn_decode_workspace(2, 1000, 8, 2, 128, 5)
    ws = torch.empty(big, dtype=torch.uint8, device="cuda")
    decode_case(S(2, 1000, 8, 2, 128, 5), 1001, workspace=ws)
    decode_case(S(1, 300, 8, 2, 128, 2), 1002, workspace=ws)
    shape = S(1, 777, 16, 4, 128, 9)
    host = I.random_inputs(shape, 1003)
    q = host["q"][:, -1].contiguous().cuda()
    kd = host["k_depth"][:, -1].permute(0, 2, 1, 3).contiguous().cuda()
    vd = host["v_depth"][:, -1].permute(0, 2, 1, 3).contiguous().cuda()
    a = api.moda_attn_decode(q, host["k_seq"].cuda(), host["v_seq"].cuda(), kd, vd, workspace=ws)
    b = api.moda_attn_decode(q, host["k_seq"].cuda(), host["v_seq"].cuda(), kd, vd, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    say("decode repeat: bit-identical")


def test_decode_rejects_small_workspace():
    shape = S(1, 300, 8, 2, 128, 3)
    host = I.random_inputs(shape, 1100)
    q = host["q"][:, -1].contiguous().cuda()
    need = api.moda_attn_decode_workspace(1, 300, 8, 2, 128, 3)
    ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    kd = host["k_depth"][:, -1].permute(0, 2, 1, 3).contiguous().cuda()
    vd = host["v_depth"][:, -1].permute(0, 2, 1, 3).contiguous().cuda()
    with pytest.raises(api.MODAError) as e:
        api.moda_attn_decode(q, host["k_seq"].cuda(), host["v_seq"].cuda(), kd, vd, workspace=ws)
    assert e.value.code == api.MODA_ERR_SHAPE

"""The allocation-free decode entry point (moda_attn_decode_noalloc) against
moda_attn_decode, the entry point with a caller-owned workspace whose kernels it
shares: same inputs, bit-identical out and lse.  Two calls in a row, the second on
a smaller problem, so that the second reuses scratch that still holds the first
call's (larger) partial results; a third call on the first problem after an
ordinary decode with a different workspace.  Both entry points are also checked
against the fp64 oracle's row T-1 of the causal forward at the bf16 bounds."""
import numpy as np
import pytest
import torch

import oracle
from depth_stream_attention_amd import api
from depth_stream_attention_amd import inputs as I
from parity_util import BF16_LSE, BF16_MAX, BF16_MEAN, say

pytestmark = pytest.mark.gpu


def _case(shape, seed):
    host = I.random_inputs(shape, seed)
    B, T, Hq, Hk, d, L = shape.B, shape.T, shape.Hq, shape.Hk, shape.d, shape.L
    q = host["q"][:, T - 1].contiguous()                                       # [B,Hq,d]
    kd = host["k_depth"][:, T - 1].permute(0, 2, 1, 3).contiguous() if L else None  # [B,Hk,L,d]
    vd = host["v_depth"][:, T - 1].permute(0, 2, 1, 3).contiguous() if L else None
    rows = np.array([(b, T - 1, h) for b in range(B) for h in range(Hq)], dtype=np.int32)
    ref_out, ref_lse = oracle.moda_fwd_rows(host["q"], host["k_seq"], host["v_seq"], host["k_depth"],
                                            host["v_depth"], rows, causal=True)
    dev = dict(q=q.cuda(), kc=host["k_seq"].cuda(), vc=host["v_seq"].cuda(),
               kd=None if kd is None else kd.cuda(), vd=None if vd is None else vd.cuda())
    return dev, ref_out.reshape(B, Hq, d), ref_lse.reshape(B, Hq)


def _both(dev, B, Hq, d):
    out_ws = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse_ws = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    out_na = torch.full((B, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_na = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    api.moda_attn_decode(dev["q"], dev["kc"], dev["vc"], dev["kd"], dev["vd"], out_ws, lse_ws)
    api.moda_attn_decode_noalloc(dev["q"], dev["kc"], dev["vc"], dev["kd"], dev["vd"], out_na, lse_na)
    torch.cuda.synchronize()
    return out_ws, lse_ws, out_na, lse_na


def _check(label, shape, dev, ref_out, ref_lse):
    out_ws, lse_ws, out_na, lse_na = _both(dev, shape.B, shape.Hq, shape.d)
    assert torch.equal(out_na, out_ws) and torch.equal(lse_na, lse_ws), "%s: differs from moda_attn_decode" % label
    err = np.abs(out_na.float().cpu().numpy() - ref_out)
    lerr = np.abs(lse_na.cpu().numpy() - ref_lse)
    say("%s %s: bit-identical to moda_attn_decode; vs oracle max|err| %.3g mean %.3g max|dlse| %.3g"
        % (label, shape.describe(), err.max(), err.mean(), lerr.max()))
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN and lerr.max() <= BF16_LSE


def test_noalloc_decode_matches_workspace_decode():
    big = I.Shape(3, 5000, 16, 4, 128, 24)   # 40 key chunks of 128 + the depth chunk per (b, hk)
    small = I.Shape(1, 700, 8, 2, 64, 5)     # 6 key chunks + depth, fewer heads, another head dim
    dev_b, ref_b, lse_b = _case(big, 910)
    dev_s, ref_s, lse_s = _case(small, 920)
    assert api.moda_attn_decode_workspace(big.B, big.T, big.Hq, big.Hk, big.d, big.L) > \
        api.moda_attn_decode_workspace(small.B, small.T, small.Hq, small.Hk, small.d, small.L)
    _check("call 1", big, dev_b, ref_b, lse_b)
    _check("call 2 (smaller)", small, dev_s, ref_s, lse_s)
    _check("call 3", big, dev_b, ref_b, lse_b)


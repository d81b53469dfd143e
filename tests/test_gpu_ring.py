"""GPU parity of the bounded depth cache (moda_attn_fwd_ring / moda_attn_decode_ring).

The packed stream holds S ring slots per (token, KV head); the first L are attended.
Expected values: the oracle on the L attended slots only.  The S - L unattended slots are
filled with keys aligned to the queries and large values, so reading any of them moves the
output far beyond the bf16 bounds (max|err| <= 2e-2, mean <= 2e-3, |dlse| <= 1e-3)."""
import numpy as np
import pytest
import torch

import oracle
from depth_stream_attention_amd import api
from depth_stream_attention_amd import inputs as I
from parity_util import check

pytestmark = pytest.mark.gpu
S_ = I.Shape


def poisoned(shape, S, L, seed):
    """Inputs with S depth slots whose slots L..S-1 would dominate every row if read."""
    host = I.random_inputs(I.with_(shape, L=S), seed)
    kd = host["k_depth"].float().clone()  # [B,T,S,Hk,d]
    vd = host["v_depth"].float().clone()
    if L < S:
        lead = host["q"].float()[:, :, :: shape.G, :]      # [B,T,Hk,d]
        kd[:, :, L:] = 4.0 * lead.unsqueeze(2)
        vd[:, :, L:] = 50.0
    host["k_depth"], host["v_depth"] = kd.bfloat16(), vd.bfloat16()
    return host


@pytest.mark.parametrize("S,L", [(8, 0), (8, 3), (8, 8), (48, 17), (16, 1)])
def test_fwd_ring(S, L):
    shape = S_(2, 190, 8, 2, 128, L)
    host = poisoned(shape, S, L, 1200 + 10 * S + L)
    dev = {k: v.cuda() for k, v in host.items()}
    kd = api.moda_pack_depth(dev["k_depth"])   # [B,T,Hk,S,d]
    vd = api.moda_pack_depth(dev["v_depth"])
    out, lse = api.moda_attn_fwd_ring(dev["q"], dev["k_seq"], dev["v_seq"], kd, vd, L)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.moda_fwd(host["q"], host["k_seq"], host["v_seq"],
                                       host["k_depth"][:, :, :L].contiguous(), host["v_depth"][:, :, :L].contiguous())
    check(shape, out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, "ring S=%d L=%d" % (S, L))


def test_fwd_ring_order_invariance():
    """A full ring attended in rotated slot order gives the same result (the softmax is a
    sum over the slot set)."""
    shape = S_(1, 150, 8, 2, 128, 12)
    host = I.random_inputs(shape, 1300)
    dev = {k: v.cuda() for k, v in host.items()}
    kd, vd = api.moda_pack_depth(dev["k_depth"]), api.moda_pack_depth(dev["v_depth"])
    a = api.moda_attn_fwd_ring(dev["q"], dev["k_seq"], dev["v_seq"], kd, vd, 12)
    kr, vr = torch.roll(kd, 5, dims=3).contiguous(), torch.roll(vd, 5, dims=3).contiguous()
    b = api.moda_attn_fwd_ring(dev["q"], dev["k_seq"], dev["v_seq"], kr, vr, 12)
    torch.cuda.synchronize()
    assert (a[0].float() - b[0].float()).abs().max().item() <= 1e-2
    assert (a[1] - b[1]).abs().max().item() <= 1e-4


@pytest.mark.parametrize("S,L", [(8, 0), (8, 5), (48, 48), (64, 33)])
def test_decode_ring(S, L):
    shape = S_(2, 600, 16, 4, 128, L)
    host = poisoned(shape, S, L, 1400 + S + L)
    T = shape.T
    q = host["q"][:, T - 1].contiguous().cuda()
    kd = host["k_depth"][:, T - 1].permute(0, 2, 1, 3).contiguous().cuda()   # [B,Hk,S,d]
    vd = host["v_depth"][:, T - 1].permute(0, 2, 1, 3).contiguous().cuda()
    out, lse = api.moda_attn_decode_ring(q, host["k_seq"].cuda(), host["v_seq"].cuda(), kd, vd, L)
    torch.cuda.synchronize()
    rows = np.array([(b, T - 1, h) for b in range(shape.B) for h in range(shape.Hq)], dtype=np.int32)
    ref_out, ref_lse = oracle.moda_fwd_rows(host["q"], host["k_seq"], host["v_seq"],
                                            host["k_depth"][:, :, :L].contiguous(),
                                            host["v_depth"][:, :, :L].contiguous(), rows, causal=True)
    check(shape, out.float().cpu().numpy().reshape(-1, shape.d), lse.cpu().numpy().reshape(-1), ref_out, ref_lse,
          "decode ring S=%d L=%d" % (S, L))

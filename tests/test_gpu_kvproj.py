"""GPU parity of the depth write path (moda_kv_project) against the fp64 oracle's projection.

The kernel multiplies bf16 inputs exactly, sums in fp32 and rounds once to bf16, so
per element |gpu - ref| <= 2^-8 |ref| + Dm * 2^-23 * sum_m |x_m w_m| (bf16 rounding
plus a worst-case fp32 summation bound).  Every requested destination must hold the
same bf16 values; depth slots other than `slot` must keep their previous bits."""
import numpy as np
import pytest
import torch

import oracle
from depth_stream_attention_amd import api
from parity_util import say

pytestmark = pytest.mark.gpu
POISON = 0x7F00  # bf16 bit pattern of a huge finite value, put in every untouched slot


def _inputs(B, T, Dm, Hk, d, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(B, T, Dm, generator=g).to(torch.bfloat16)
    w = (torch.randn(2 * Hk * d, Dm, generator=g) / 8).to(torch.bfloat16)
    return x, w


def _check(x, w, Hk, d, got_k, got_v, label):
    ref_k, ref_v = oracle.kv_project(x, w, Hk, d)
    B, T, Dm = x.shape
    absmag = (x.abs().double().reshape(-1, Dm) @ w.abs().double().T).numpy()  # sum_m |x_m w_m|
    bound_k = absmag[:, :Hk * d].reshape(B, T, Hk, d) * Dm * 2.0 ** -23 + 2.0 ** -8 * np.abs(ref_k)
    bound_v = absmag[:, Hk * d:].reshape(B, T, Hk, d) * Dm * 2.0 ** -23 + 2.0 ** -8 * np.abs(ref_v)
    ek = np.abs(got_k.float().cpu().numpy() - ref_k)
    ev = np.abs(got_v.float().cpu().numpy() - ref_v)
    say("%s: max|err| k %.3g v %.3g, max err/bound %.3f" % (label, ek.max(), ev.max(),
                                                            max((ek / bound_k).max(), (ev / bound_v).max())))
    assert (ek <= bound_k).all() and (ev <= bound_v).all(), label


@pytest.mark.parametrize("B,T", [(1, 1), (2, 100), (1, 129), (3, 300)])
@pytest.mark.parametrize("Hk,d", [(1, 64), (2, 128), (4, 64)])
def test_kv_project_sequence_and_depth(B, T, Hk, d):
    Dm = 256
    x, w = _inputs(B, T, Dm, Hk, d, 100 * B + T + Hk + d)
    S, slot = 5, 3
    xd, wd = x.cuda(), w.cuda()
    kd = torch.full((B, T, Hk, S, d), 0, dtype=torch.int16, device="cuda").fill_(POISON).view(torch.bfloat16)
    vd = kd.clone()
    k, v, _, _ = api.moda_kv_project(xd, wd, Hk, d, k_out=torch.empty(B, T, Hk, d, dtype=torch.bfloat16,
                                                                       device="cuda"),
                                     v_out=torch.empty(B, T, Hk, d, dtype=torch.bfloat16, device="cuda"),
                                     k_depth=kd, v_depth=vd, slot=slot)
    torch.cuda.synchronize()
    _check(x, w, Hk, d, k, v, "kvproj B%d T%d Hk%d d%d" % (B, T, Hk, d))
    # the slot holds the same bits; every other slot is untouched
    assert torch.equal(kd[:, :, :, slot].view(torch.int16), k.view(torch.int16))
    assert torch.equal(vd[:, :, :, slot].view(torch.int16), v.view(torch.int16))
    others = [s for s in range(S) if s != slot]
    assert (kd[:, :, :, others].view(torch.int16) == POISON).all()
    assert (vd[:, :, :, others].view(torch.int16) == POISON).all()


@pytest.mark.parametrize("Dm", [64, 192, 2048])
def test_kv_project_hidden_sizes(Dm):
    x, w = _inputs(2, 77, Dm, 2, 64, Dm)
    k, v, _, _ = api.moda_kv_project(x.cuda(), w.cuda(), 2, 64)
    torch.cuda.synchronize()
    _check(x, w, 2, 64, k, v, "kvproj Dm%d" % Dm)


def test_kv_project_depth_only_equals_append():
    """Depth only: the slot equals the projection written to [B,T,Hk,d] and then appended
    with moda_append_depth_slot (the unfused path)."""
    B, T, Dm, Hk, d, S = 2, 150, 128, 4, 128, 3
    x, w = _inputs(B, T, Dm, Hk, d, 9)
    xd, wd = x.cuda(), w.cuda()
    k, v, _, _ = api.moda_kv_project(xd, wd, Hk, d)
    ka = torch.zeros(B, T, Hk, S, d, dtype=torch.bfloat16, device="cuda")
    va = torch.zeros_like(ka)
    api.moda_append_depth_slot(k, ka, 2)
    api.moda_append_depth_slot(v, va, 2)
    kd = torch.zeros_like(ka)
    vd = torch.zeros_like(ka)
    api.moda_kv_project(xd, wd, Hk, d, k_depth=kd, v_depth=vd, slot=2)
    torch.cuda.synchronize()
    assert torch.equal(kd.view(torch.int16), ka.view(torch.int16))
    assert torch.equal(vd.view(torch.int16), va.view(torch.int16))


def test_kv_project_long_context_layer_sampled():
    """The long-context layer: 65536 tokens, hidden size Hq*d = 2048, Hk = 4, d = 128, into
    slot 47 of a 48-slot stream; sampled tokens against the oracle (tokens are independent)."""
    B, T, Dm, Hk, d, S = 1, 65536, 2048, 4, 128, 48
    g = torch.Generator(device="cuda").manual_seed(11)
    xd = torch.randn(B, T, Dm, device="cuda", generator=g).bfloat16()
    wd = (torch.randn(2 * Hk * d, Dm, device="cuda", generator=g) / 8).bfloat16()
    kd = torch.zeros(B, T, Hk, S, d, dtype=torch.bfloat16, device="cuda")
    vd = torch.zeros_like(kd)
    k, v, _, _ = api.moda_kv_project(xd, wd, Hk, d, k_out=torch.empty(B, T, Hk, d, dtype=torch.bfloat16,
                                                                       device="cuda"),
                                     v_out=torch.empty(B, T, Hk, d, dtype=torch.bfloat16, device="cuda"),
                                     k_depth=kd, v_depth=vd, slot=S - 1)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    toks = np.unique(np.concatenate([[0, 1, 127, 128, T - 1], rng.integers(0, T, 60)]))
    ti = torch.from_numpy(toks).cuda()
    xs = xd[0, ti].cpu().unsqueeze(0)
    _check(xs, wd.cpu(), Hk, d, k[0, ti].unsqueeze(0), v[0, ti].unsqueeze(0), "kvproj long-context sampled")
    assert torch.equal(kd[:, :, :, S - 1], k) and torch.equal(vd[:, :, :, S - 1], v)
    assert not kd[:, :, :, :S - 1].any()

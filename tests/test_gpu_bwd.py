"""GPU parity of the backward (moda_attn_bwd) against the fp64 oracle's gradients.

The HIP backward takes the HIP forward's (out, lse) for the same inputs, as a
training step would; the oracle recomputes everything from the inputs and the
output gradient alone.  Every gradient is compared element by element, scaled
by the size of that gradient: bf16 inputs, bf16 softmax weights and score
gradients inside the products and bf16 results give relative errors of a few
2^-9, so max|err| <= 2e-2 * max|ref| and mean|err| <= 1e-2 * mean|ref| per
tensor."""
import numpy as np
import pytest
import torch

import oracle
from depth_stream_attention_amd import api
from depth_stream_attention_amd import inputs as I
from parity_util import random_shapes, say

pytestmark = pytest.mark.gpu
S = I.Shape

REL_MAX, REL_MEAN = 2e-2, 1e-2
NAMES = ("dq", "dk_seq", "dv_seq", "dk_depth", "dv_depth")


def run_bwd(shape, host, dout_host, workspace=None):
    dev = {k: v.cuda() for k, v in host.items()}
    kd = vd = None
    if shape.L > 0:
        kd = api.moda_pack_depth(dev["k_depth"])
        vd = api.moda_pack_depth(dev["v_depth"])
    out, lse = api.moda_attn_fwd(dev["q"], dev["k_seq"], dev["v_seq"], kd, vd, causal=shape.causal)
    grads = api.moda_attn_bwd(dev["q"], dev["k_seq"], dev["v_seq"], kd, vd, out, lse, dout_host.cuda(),
                              causal=shape.causal, workspace=workspace)
    torch.cuda.synchronize()
    res = []
    for i, g in enumerate(grads):
        if g is None:
            res.append(None)
            continue
        a = g.float().cpu().numpy()
        if i >= 3:
            a = a.transpose(0, 1, 3, 2, 4)  # packed [B,T,Hk,L,d] -> generation layout [B,T,L,Hk,d]
        res.append(a)
    return res


def compare(shape, got, ref, label):
    worst = 0.0
    for name, g, r in zip(NAMES, got, ref):
        if r is None:
            assert g is None
            continue
        assert np.all(np.isfinite(g)), "%s %s: non-finite gradient" % (label, name)
        err = np.abs(g.astype(np.float64) - r)
        scale_max = max(np.abs(r).max(), 1e-30)
        scale_mean = max(np.abs(r).mean(), 1e-30)
        rmax, rmean = err.max() / scale_max, err.mean() / scale_mean
        say("%s %s %-8s max|ref| %.3g  max|err| %.3g (%.2e rel)  mean rel %.2e" % (
            label, shape.describe(), name, scale_max, err.max(), rmax, rmean))
        assert rmax <= REL_MAX and rmean <= REL_MEAN, "%s %s: rel max %.3g mean %.3g" % (label, name, rmax, rmean)
        worst = max(worst, rmax)
    return worst


def bwd_case(shape, seed, workspace=None):
    host = I.random_inputs(shape, seed)
    dout = I.random_dout(shape, seed + 9)
    say("case", shape.describe(), "seed", seed)
    got = run_bwd(shape, host, dout, workspace)
    ref = oracle.moda_bwd(host["q"], host["k_seq"], host["v_seq"], host["k_depth"], host["v_depth"], dout,
                          causal=shape.causal)
    return compare(shape, got, ref, "bwd")


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 129, 300])
def test_bwd_sequence_lengths(T):
    bwd_case(S(2, T, 8, 2, 128, 5), 800 + T)


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16, 32])
@pytest.mark.parametrize("d", [64, 128])
def test_bwd_group_sizes(G, d):
    bwd_case(S(1, 200, 2 * G, 2, d, 6), 850 + 10 * G + d)


@pytest.mark.parametrize("L", [1, 16, 40])
def test_bwd_32_heads_per_kv_head(L):
    # G = 32: a token's rows are two 16-row halves in the depth-gradient kernel, whose slot
    # gradients sum both halves; one, one whole and two and a half 16-slot steps
    bwd_case(S(2, 97, 64, 2, 128, L), 870 + L)


@pytest.mark.parametrize("L", [0, 1, 15, 16, 17, 48])
def test_bwd_depth_slots(L):
    bwd_case(S(1, 160, 8, 2, 128, L), 900 + L)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_bwd_full_attention(causal, d):
    bwd_case(S(2, 190, 4, 2, d, 3, causal=causal), 950 + d + int(causal))


def test_bwd_is_deterministic_and_reuses_workspace():
    shape = S(1, 257, 8, 2, 128, 17)
    host = I.random_inputs(shape, 990)
    dout = I.random_dout(shape, 999)
    need = api.moda_attn_bwd_workspace(1, 257, 8, 2, 128, 17)
    ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")  # stale contents must not matter
    a = run_bwd(shape, host, dout, workspace=ws)
    b = run_bwd(shape, host, dout, workspace=ws)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("i,case", list(enumerate(random_shapes(12, 2029, 4e8))))
def test_bwd_random_shapes(i, case):
    bwd_case(case[0], 1500 + i)

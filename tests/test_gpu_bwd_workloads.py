"""The backward at the full workload sizes, launched as the benchmark launches it,
checked three ways against what does not come from the HIP path:
  * sampled gradients against the fp64 oracle (moda_bwd_sampled): dq of stratified
    rows, dk/dv of sequence keys (the last keys of a head, whose visible rows are few
    enough for the oracle, plus keys 0 and 1, which every row of their head group
    sees, wherever that costs the oracle seconds: T=4096 and T=8192 at G=4, T=16384
    at G=1), and the depth
    gradients of sampled tokens -- each an exact check of that output;
  * two identities over every key of every (batch, KV head): the value gradients
    (sequence + depth) sum to the sum of dout over the head group's rows, and the key
    gradients sum to zero, because each row's softmax weights sum to one;
  * every gradient element finite.
Tolerances as in test_gpu_bwd: max|err| <= 2e-2 * max|ref|, mean|err| <= 1e-2 * mean|ref|
per tensor over the sampled elements."""
import numpy as np
import pytest
import torch

import oracle
from depth_stream_attention_amd import api
from depth_stream_attention_amd import inputs as I
from parity_util import say

pytestmark = pytest.mark.gpu
REL_MAX, REL_MEAN = 2e-2, 1e-2


def _compare(name, got, ref, label):
    err = np.abs(got.astype(np.float64) - ref)
    rmax = err.max() / max(np.abs(ref).max(), 1e-30)
    rmean = err.mean() / max(np.abs(ref).mean(), 1e-30)
    say("%s %-8s n=%d max|ref| %.3g max|err| %.3g rel %.2e mean rel %.2e" % (
        label, name, ref.size, np.abs(ref).max(), err.max(), rmax, rmean))
    assert rmax <= REL_MAX and rmean <= REL_MEAN, "%s %s: rel max %.3g mean %.3g" % (label, name, rmax, rmean)


def _samples(shape, seed, key_groups, early_key):
    rng = np.random.default_rng(seed)
    B, T, Hq, Hk = shape.B, shape.T, shape.Hq, shape.Hk
    rows = []
    for b in range(B):
        for t in sorted({0, 1, T // 2, T - 2, T - 1} | set(rng.integers(0, T, 3).tolist())):
            for h in sorted({0, Hq - 1, int(rng.integers(0, Hq))}):
                rows.append((b, t, h))
    keys = []
    for (b, hk) in key_groups:
        for j in sorted({T - 1, T - 2, T - 64, T - 65, max(T - 100, 0)}):
            if j >= 0:
                keys.append((b, j, hk))
    if early_key:
        keys.append((0, 0, 0))
        keys.append((0, 1, 0))
    toks = []
    if shape.L > 0:
        for b in range(B):
            for t in sorted({0, T - 1, int(rng.integers(0, T))}):
                toks.append((b, t, int(rng.integers(0, Hk))))
    return rows, keys, toks


def _bwd_workload(c, v, key_groups=None, early_key=False):
    shape = I.workload(c, v)
    label = "bwd workload %d.%d" % (c, v)
    say(label, shape.describe())
    dev = I.workload_inputs(c, v, device="cuda")
    dout = I.random_dout(shape, 7000 + 10 * c + v, device="cuda")
    kd = api.moda_pack_depth(dev["k_depth"]) if shape.L else None
    vd = api.moda_pack_depth(dev["v_depth"]) if shape.L else None
    out, lse = api.moda_attn_fwd(dev["q"], dev["k_seq"], dev["v_seq"], kd, vd, causal=shape.causal)
    dq, dk, dv, dkd, dvd = api.moda_attn_bwd(dev["q"], dev["k_seq"], dev["v_seq"], kd, vd, out, lse, dout,
                                             causal=shape.causal)
    torch.cuda.synchronize()
    del out, lse, kd, vd
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv), ("dkd", dkd), ("dvd", dvd)):
        if g is not None:
            assert torch.isfinite(g.float()).all(), "%s: non-finite %s" % (label, name)

    # Identities over every key of every (b, hk), in fp64 on the GPU.
    B, T, Hq, Hk, d, G = shape.B, shape.T, shape.Hq, shape.Hk, shape.d, shape.G
    sv = dv.double().sum(1)                                   # [B,Hk,d]
    sk = dk.double().sum(1)
    sq_v = (dv.double() ** 2).sum(1)
    sq_k = (dk.double() ** 2).sum(1)
    if dvd is not None:
        sv += dvd.double().sum((1, 3))
        sk += dkd.double().sum((1, 3))
        sq_v += (dvd.double() ** 2).sum((1, 3))
        sq_k += (dkd.double() ** 2).sum((1, 3))
    want = dout.double().view(B, T, Hk, G, d).sum((1, 3))
    # bf16 results carry relative errors of a few 2^-9 per element; independent errors
    # sum to about 2^-8 * sqrt(sum x^2).  Allow 8 times that.
    tol_v = 8 * 2.0 ** -8 * sq_v.sqrt() + 1e-6
    tol_k = 8 * 2.0 ** -8 * sq_k.sqrt() + 1e-6
    ev, ek = (sv - want).abs(), sk.abs()
    say("%s identities: max|sum dv - sum dout| %.3g (tol %.3g)  max|sum dk| %.3g (tol %.3g)" % (
        label, ev.max().item(), tol_v.min().item(), ek.max().item(), tol_k.min().item()))
    assert (ev <= tol_v).all(), "%s: value-gradient sum identity" % label
    assert (ek <= tol_k).all(), "%s: key-gradient sum identity" % label

    # Sampled exact checks against the oracle.
    if key_groups is None:
        key_groups = [(b, hk) for b in range(B) for hk in range(Hk)]
    rows, keys, toks = _samples(shape, 100 * c + v, key_groups, early_key)
    host = {k_: t.cpu() for k_, t in dev.items()}
    ref = oracle.moda_bwd_sampled(host["q"], host["k_seq"], host["v_seq"], host["k_depth"], host["v_depth"],
                                  dout.cpu(), rows, keys, toks, causal=shape.causal)
    r = np.array(rows)
    kk = np.array(keys)
    got_dq = dq[r[:, 0], r[:, 1], r[:, 2]].float().cpu().numpy()
    got_dk = dk[kk[:, 0], kk[:, 1], kk[:, 2]].float().cpu().numpy()
    got_dv = dv[kk[:, 0], kk[:, 1], kk[:, 2]].float().cpu().numpy()
    _compare("dq", got_dq, ref[0], label)
    _compare("dk_seq", got_dk, ref[1], label)
    _compare("dv_seq", got_dv, ref[2], label)
    if toks:
        tt = np.array(toks)
        got_dkd = dkd[tt[:, 0], tt[:, 1], tt[:, 2]].float().cpu().numpy()  # [n,L,d] from packed [B,T,Hk,L,d]
        got_dvd = dvd[tt[:, 0], tt[:, 1], tt[:, 2]].float().cpu().numpy()
        _compare("dk_depth", got_dkd, ref[3], label)
        _compare("dv_depth", got_dvd, ref[4], label)
    del dev, dout, dq, dk, dv, dkd, dvd, host
    torch.cuda.empty_cache()


def test_bwd_workload2():
    _bwd_workload(2, 0, key_groups=[(0, 0), (3, 3)], early_key=True)


@pytest.mark.parametrize("v", [0, 1, 2, 3])
def test_bwd_workload3(v):
    _bwd_workload(3, v, key_groups=[(0, 0), (1, 7)], early_key=True)


@pytest.mark.parametrize("v", [0, 3])
def test_bwd_workload4(v):
    # keys 0 and 1 collect from every row of their head group: G=1 keeps the oracle's cost in seconds
    _bwd_workload(4, v, key_groups=[(0, 0), (0, 3)], early_key=(v == 0))


@pytest.mark.parametrize("v", [0, 1])
def test_bwd_workload5(v):
    _bwd_workload(5, v, key_groups=[(0, 1), (0, 2)])

"""Checks that pin the fp64 oracle to things other than itself.

Each function raises AssertionError when the oracle disagrees with:
  * torch's scaled_dot_product_attention (a library routine) run on the
    explicitly concatenated [sequence | depth] key set of every row,
  * the reduction L=0 -> causal GQA attention (Eq. (2) of the papercache
    summary "Mixture-of-Depths Attention", section 2.1),
  * the pages' worked example (MoDA reading notes, section 二.2: position 3
    with 4 depth slots -> 7 candidates, depth mass 4/7 at equal logits),
  * closed forms (T=1, uniform logits), invariants (convex combination,
    depth-slot permutation) and the two-branch merge identity of the MiTA
    reading notes (section 2.3: o = (Z_c o_c + Z_r o_r) / (Z_c + Z_r)).

They are shared by tests/test_oracle.py and by the planted-mistake tests,
which rebuild the oracle with a deliberate error and require some pin to fail.
"""
import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rand_problem(B, T, Hq, Hk, d, L, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    mk = lambda *s: torch.randn(*s, generator=g, dtype=torch.float64)  # noqa: E731
    return (mk(B, T, Hq, d), mk(B, T, Hk, d), mk(B, T, Hk, d),
            mk(B, T, L, Hk, d), mk(B, T, L, Hk, d))


def sdpa_reference(q, k, v, kd, vd, causal):
    """MoDA through torch SDPA: each row attends to cat(k_seq, k_depth[t]) with a mask.

    Head h reads KV head h // G (torch.repeat_interleave).  Returns
    (out [B,T,Hq,d], lse [B,Hq,T]) in fp64; lse comes from torch.logsumexp of
    the masked logits.
    """
    B, T, Hq, d = q.shape
    Hk = k.shape[2]
    G = Hq // Hk
    L = kd.shape[2]
    ke = k.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)            # [B,Hq,T,d]
    ve = v.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    kde = kd.repeat_interleave(G, dim=3).permute(0, 3, 1, 2, 4)       # [B,Hq,T,L,d]
    vde = vd.repeat_interleave(G, dim=3).permute(0, 3, 1, 2, 4)
    kall = torch.cat([ke.unsqueeze(2).expand(B, Hq, T, T, d), kde], dim=3)  # [B,Hq,T,T+L,d]
    vall = torch.cat([ve.unsqueeze(2).expand(B, Hq, T, T, d), vde], dim=3)
    mask = torch.ones(T, T + L, dtype=torch.bool)
    if causal:
        mask[:, :T] = torch.ones(T, T, dtype=torch.bool).tril()
    qq = q.permute(0, 2, 1, 3).unsqueeze(3)                            # [B,Hq,T,1,d]
    m5 = mask.view(1, 1, T, 1, T + L)
    out = F.scaled_dot_product_attention(qq, kall, vall, attn_mask=m5)  # [B,Hq,T,1,d]
    logits = torch.matmul(qq, kall.transpose(-1, -2).contiguous()) / math.sqrt(d)
    logits = logits.masked_fill(~m5, float("-inf"))
    lse = torch.logsumexp(logits, dim=-1).squeeze(-1)                   # [B,Hq,T]
    return out.squeeze(3).permute(0, 2, 1, 3).numpy(), lse.numpy()


def pin_sdpa(B, T, Hq, Hk, d, L, causal, seed, tol=1e-12):
    q, k, v, kd, vd = rand_problem(B, T, Hq, Hk, d, L, seed)
    out, lse = oracle.moda_fwd(q, k, v, kd, vd, causal=causal, nthreads=2)
    ro, rl = sdpa_reference(q, k, v, kd, vd, causal)
    assert np.abs(out - ro).max() <= tol, "out differs from SDPA on [seq|depth] by %g" % np.abs(out - ro).max()
    assert np.abs(lse - rl).max() <= tol, "lse differs from logsumexp by %g" % np.abs(lse - rl).max()


def pin_l0_is_gqa(B, T, Hq, Hk, d, causal, seed, tol=1e-12):
    """L=0: the oracle is plain GQA attention, softmax(Q_h K_phi(h)^T/sqrt(d) + M) V_phi(h)."""
    q, k, v, _, _ = rand_problem(B, T, Hq, Hk, d, 0, seed)
    out, _ = oracle.moda_fwd(q, k, v, None, None, causal=causal, nthreads=2)
    G = Hq // Hk
    ref = F.scaled_dot_product_attention(
        q.permute(0, 2, 1, 3), k.repeat_interleave(G, dim=2).permute(0, 2, 1, 3),
        v.repeat_interleave(G, dim=2).permute(0, 2, 1, 3), is_causal=bool(causal))
    ref = ref.permute(0, 2, 1, 3).numpy()
    assert np.abs(out - ref).max() <= tol, "L=0 differs from causal GQA SDPA by %g" % np.abs(out - ref).max()


def pin_worked_example():
    """Pages' example: equal logits (q = 0), position 3 (1-indexed), 4 depth slots -> depth mass 4/7."""
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        ex = json.load(f)
    T = ex["position_1_indexed"]       # the last row, t = T-1 (0-indexed), sees T sequence keys
    L = ex["depth_slots"]
    d = 4
    q = torch.zeros(1, T, 1, d, dtype=torch.float64)
    g = torch.Generator("cpu").manual_seed(5)
    k = torch.randn(1, T, 1, d, generator=g, dtype=torch.float64)
    kd = torch.randn(1, T, L, 1, d, generator=g, dtype=torch.float64)
    v = torch.zeros(1, T, 1, d, dtype=torch.float64)     # sequence values 0
    vd = torch.ones(1, T, L, 1, d, dtype=torch.float64)  # depth values 1 -> out = depth mass
    out, lse = oracle.moda_fwd(q, k, v, kd, vd, causal=True, nthreads=1)
    want = ex["depth_mass_numerator"] / ex["depth_mass_denominator"]
    got = out[0, T - 1, 0, :]
    assert np.abs(got - want).max() <= 1e-15, "depth mass %r, pages give 4/7" % (got[0],)
    assert abs(lse[0, 0, T - 1] - math.log(ex["candidates"])) <= 1e-15, "lse must be log(7) at zero logits"
    # every row t (0-indexed) then has depth mass L / (t + 1 + L)
    for t in range(T):
        assert abs(out[0, t, 0, 0] - L / (t + 1 + L)) <= 1e-15


def pin_t1_closed_form(seed):
    """T=1, L=0: one candidate, so out = v_0 and lse = q.k_0/sqrt(d) exactly."""
    q, k, v, _, _ = rand_problem(2, 1, 4, 2, 16, 0, seed)
    out, lse = oracle.moda_fwd(q, k, v, None, None, causal=True, nthreads=1)
    G = 2
    for b in range(2):
        for h in range(4):
            assert np.array_equal(out[b, 0, h], v[b, 0, h // G].numpy()), "T=1 L=0: out must equal v_0"
            want = float((q[b, 0, h] * k[b, 0, h // G]).sum()) / 4.0
            assert abs(lse[b, h, 0] - want) <= 1e-14, "T=1 L=0: lse must equal the single logit"


def pin_t1_depth(seed):
    """T=1: softmax over the token's own key plus its L depth keys (scipy-free closed form via torch.softmax)."""
    L, d = 5, 8
    q, k, v, kd, vd = rand_problem(1, 1, 2, 1, d, L, seed)
    out, lse = oracle.moda_fwd(q, k, v, kd, vd, causal=True, nthreads=1)
    keys = torch.cat([k[0, 0], kd[0, 0, :, 0]], dim=0)        # [1+L, d]
    vals = torch.cat([v[0, 0], vd[0, 0, :, 0]], dim=0)
    for h in range(2):
        w = torch.softmax(keys @ q[0, 0, h] / math.sqrt(d), dim=0)
        assert np.abs(out[0, 0, h] - (w @ vals).numpy()).max() <= 1e-14
        assert abs(lse[0, h, 0] - float(torch.logsumexp(keys @ q[0, 0, h] / math.sqrt(d), 0))) <= 1e-14


def pin_head_expansion(seed):
    """GQA with Hk KV heads equals MHA on KV heads repeated G times (head h -> h // G)."""
    B, T, Hq, Hk, d, L = 1, 9, 6, 2, 8, 3
    q, k, v, kd, vd = rand_problem(B, T, Hq, Hk, d, L, seed)
    G = Hq // Hk
    o1, l1 = oracle.moda_fwd(q, k, v, kd, vd, nthreads=2)
    o2, l2 = oracle.moda_fwd(q, k.repeat_interleave(G, 2), v.repeat_interleave(G, 2),
                             kd.repeat_interleave(G, 3), vd.repeat_interleave(G, 3), nthreads=2)
    assert np.abs(o1 - o2).max() <= 1e-14 and np.abs(l1 - l2).max() <= 1e-14
    # G = 1: every head is an independent single-head problem
    for h in range(Hq):
        oh, lh = oracle.moda_fwd(q[:, :, h:h + 1], k.repeat_interleave(G, 2)[:, :, h:h + 1],
                                 v.repeat_interleave(G, 2)[:, :, h:h + 1],
                                 kd.repeat_interleave(G, 3)[:, :, :, h:h + 1],
                                 vd.repeat_interleave(G, 3)[:, :, :, h:h + 1], nthreads=1)
        assert np.abs(oh[:, :, 0] - o2[:, :, h]).max() <= 1e-14
        assert np.abs(lh[:, 0] - l2[:, h]).max() <= 1e-14


def pin_convex_and_permutation(seed):
    """out is a convex combination of the visible values; permuting depth slots changes nothing."""
    B, T, Hq, Hk, d, L = 2, 11, 4, 2, 8, 5
    q, k, v, kd, vd = rand_problem(B, T, Hq, Hk, d, L, seed)
    out, lse = oracle.moda_fwd(q, k, v, kd, vd, nthreads=2)
    G = Hq // Hk
    for b in range(B):
        for t in range(T):
            for h in range(Hq):
                cand = torch.cat([v[b, : t + 1, h // G], vd[b, t, :, h // G]], dim=0).numpy()
                lo, hi = cand.min(axis=0), cand.max(axis=0)
                o = out[b, t, h]
                assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12), "out outside the value hull"
    perm = torch.randperm(L, generator=torch.Generator("cpu").manual_seed(seed + 1))
    op, lp = oracle.moda_fwd(q, k, v, kd[:, :, perm], vd[:, :, perm], nthreads=2)
    assert np.abs(op - out).max() <= 1e-13 and np.abs(lp - lse).max() <= 1e-13
    # a permutation applied to the keys only must change the result
    oq, _ = oracle.moda_fwd(q, k, v, kd[:, :, perm], vd, nthreads=2)
    assert np.abs(oq - out).max() > 1e-6


def pin_merge_identity(seed):
    """MoDA = (Z_s o_s + Z_d o_d) / (Z_s + Z_d) with the sequence-only result from the L=0
    oracle and the depth-only softmax from torch SDPA; lse = logaddexp(lse_s, lse_d)."""
    B, T, Hq, Hk, d, L = 1, 10, 4, 2, 8, 3
    q, k, v, kd, vd = rand_problem(B, T, Hq, Hk, d, L, seed)
    out, lse = oracle.moda_fwd(q, k, v, kd, vd, nthreads=2)
    o_s, lse_s = oracle.moda_fwd(q, k, v, None, None, nthreads=2)
    G = Hq // Hk
    kde = kd.repeat_interleave(G, 3).permute(0, 3, 1, 2, 4)  # [B,Hq,T,L,d]
    vde = vd.repeat_interleave(G, 3).permute(0, 3, 1, 2, 4)
    qq = q.permute(0, 2, 1, 3).unsqueeze(3)                   # [B,Hq,T,1,d]
    o_d = F.scaled_dot_product_attention(qq, kde, vde).squeeze(3).permute(0, 2, 1, 3).numpy()
    lse_d = torch.logsumexp(torch.matmul(qq, kde.transpose(-1, -2).contiguous()).squeeze(3) / math.sqrt(d),
                            dim=-1).numpy()                   # [B,Hq,T]
    zs = np.exp(lse_s - lse).transpose(0, 2, 1)[..., None]    # Z_s / Z as [B,T,Hq,1]
    zd = np.exp(lse_d - lse).transpose(0, 2, 1)[..., None]
    merged = zs * o_s + zd * o_d
    assert np.abs(merged - out).max() <= 1e-12, "merge identity broken by %g" % np.abs(merged - out).max()
    assert np.abs(np.logaddexp(lse_s, lse_d) - lse).max() <= 1e-12


def pin_depth_aligned(seed):
    """Depth keys equal to head 0's query (plus small noise) of the SAME token must take
    most of head 0's mass at every position; reading another token's slots would not."""
    B, T, Hq, Hk, d, L = 1, 40, 2, 1, 32, 4
    q, k, v, kd, vd = rand_problem(B, T, Hq, Hk, d, L, seed)
    kd = 2.0 * q[:, :, 0:1, :].unsqueeze(2).expand(B, T, L, Hk, d) + 0.1 * kd
    vd = torch.full_like(vd, 1.0)
    v = torch.zeros_like(v)
    out, _ = oracle.moda_fwd(q, k, v, kd.contiguous(), vd, nthreads=2)
    mass = out[0, :, 0, 0]                                    # head 0, depth mass per position
    assert mass.min() > 0.9, "depth mass of the aligned head fell to %g" % mass.min()


# ---- gradients ----------------------------------------------------------------

def autograd_reference(q, k, v, kd, vd, dout, causal):
    """Gradients of sum(dout * MoDA(q, k, v, kd, vd)) by torch autograd in fp64.

    The forward is written with plain tensor ops on the explicitly concatenated
    [sequence | depth] key set of every row (head h reads KV head h // G), so
    the derivative comes from torch's own autograd, not from a hand-written rule.
    Returns numpy (dq, dk, dv, dkd, dvd) in the input layouts.
    """
    leaves = [x.detach().clone().requires_grad_(True) for x in (q, k, v, kd, vd)]
    q_, k_, v_, kd_, vd_ = leaves
    B, T, Hq, d = q.shape
    Hk = k.shape[2]
    G = Hq // Hk
    L = kd.shape[2]
    ke = k_.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)           # [B,Hq,T,d]
    ve = v_.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    kde = kd_.repeat_interleave(G, dim=3).permute(0, 3, 1, 2, 4)      # [B,Hq,T,L,d]
    vde = vd_.repeat_interleave(G, dim=3).permute(0, 3, 1, 2, 4)
    kall = torch.cat([ke.unsqueeze(2).expand(B, Hq, T, T, d), kde], dim=3)
    vall = torch.cat([ve.unsqueeze(2).expand(B, Hq, T, T, d), vde], dim=3)
    mask = torch.ones(T, T + L, dtype=torch.bool)
    if causal:
        mask[:, :T] = torch.ones(T, T, dtype=torch.bool).tril()
    qq = q_.permute(0, 2, 1, 3).unsqueeze(3)                           # [B,Hq,T,1,d]
    logits = torch.matmul(qq, kall.transpose(-1, -2).contiguous()) / math.sqrt(d)
    logits = logits.masked_fill(~mask.view(1, 1, T, 1, T + L), float("-inf"))
    out = torch.matmul(torch.softmax(logits, dim=-1), vall).squeeze(3).permute(0, 2, 1, 3)
    (out * dout).sum().backward()
    return tuple(x.grad.numpy() for x in leaves)


def pin_bwd_autograd(B, T, Hq, Hk, d, L, causal, seed, tol=1e-11):
    q, k, v, kd, vd = rand_problem(B, T, Hq, Hk, d, L, seed)
    dout = torch.randn(B, T, Hq, d, generator=torch.Generator("cpu").manual_seed(seed + 7), dtype=torch.float64)
    got = oracle.moda_bwd(q, k, v, kd, vd, dout, causal=causal, nthreads=2)
    want = autograd_reference(q, k, v, kd, vd, dout, causal)
    for name, g, w in zip(("dq", "dk", "dv", "dkd", "dvd"), got, want):
        if g is None:
            assert L == 0 and w.size == 0
            continue
        err = np.abs(g - w).max()
        assert err <= tol * max(1.0, np.abs(w).max()), "%s differs from torch autograd by %g" % (name, err)


def pin_bwd_l0_gqa(B, T, Hq, Hk, d, causal, seed, tol=1e-11):
    """L=0: gradients equal those of torch's GQA SDPA (heads expanded by repeat_interleave)."""
    q, k, v, _, _ = rand_problem(B, T, Hq, Hk, d, 0, seed)
    dout = torch.randn(B, T, Hq, d, generator=torch.Generator("cpu").manual_seed(seed + 3), dtype=torch.float64)
    dq, dk, dv, dkd, dvd = oracle.moda_bwd(q, k, v, None, None, dout, causal=causal, nthreads=2)
    assert dkd is None and dvd is None
    G = Hq // Hk
    leaves = [x.clone().requires_grad_(True) for x in (q, k, v)]
    ref = F.scaled_dot_product_attention(
        leaves[0].permute(0, 2, 1, 3), leaves[1].repeat_interleave(G, dim=2).permute(0, 2, 1, 3),
        leaves[2].repeat_interleave(G, dim=2).permute(0, 2, 1, 3), is_causal=bool(causal))
    (ref.permute(0, 2, 1, 3) * dout).sum().backward()
    for name, g, leaf in zip(("dq", "dk", "dv"), (dq, dk, dv), leaves):
        err = np.abs(g - leaf.grad.numpy()).max()
        assert err <= tol, "L=0 %s differs from GQA SDPA autograd by %g" % (name, err)


def pin_bwd_finite_difference(seed, h=1e-5):
    """Directional derivatives of F = sum(dout * out) by central differences of the
    fp64 forward oracle must equal <grad, delta> for a random direction per input."""
    B, T, Hq, Hk, d, L = 1, 7, 4, 2, 8, 3
    xs = list(rand_problem(B, T, Hq, Hk, d, L, seed))
    g = torch.Generator("cpu").manual_seed(seed + 11)
    dout = torch.randn(B, T, Hq, d, generator=g, dtype=torch.float64)
    grads = oracle.moda_bwd(*xs, dout, nthreads=1)

    def F_of(args):
        out, _ = oracle.moda_fwd(*args, nthreads=1)
        return float((out * dout.numpy()).sum())

    for i, name in enumerate(("q", "k_seq", "v_seq", "k_depth", "v_depth")):
        delta = torch.randn(xs[i].shape, generator=g, dtype=torch.float64)
        plus = list(xs)
        minus = list(xs)
        plus[i] = xs[i] + h * delta
        minus[i] = xs[i] - h * delta
        fd = (F_of(plus) - F_of(minus)) / (2 * h)
        an = float((grads[i] * delta.numpy()).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), \
            "d/d%s: finite difference %.12g vs gradient %.12g" % (name, fd, an)


def pin_bwd_invariants(seed):
    """Softmax weights sum to one in every row, so per (b, KV head):
    sum of all value gradients (sequence + depth) = sum of dout over the group's rows, and
    sum of all key gradients = 0.  Equal values everywhere make out constant, so then every
    query and key gradient vanishes and the value gradients stay those of the weights."""
    B, T, Hq, Hk, d, L = 2, 12, 6, 2, 8, 4
    q, k, v, kd, vd = rand_problem(B, T, Hq, Hk, d, L, seed)
    dout = torch.randn(B, T, Hq, d, generator=torch.Generator("cpu").manual_seed(seed + 5), dtype=torch.float64)
    dq, dk, dv, dkd, dvd = oracle.moda_bwd(q, k, v, kd, vd, dout, nthreads=2)
    G = Hq // Hk
    for b in range(B):
        for hk in range(Hk):
            sv = dv[b, :, hk].sum(0) + dvd[b, :, :, hk].sum((0, 1))
            want = dout[b, :, hk * G:(hk + 1) * G].sum((0, 1)).numpy()
            assert np.abs(sv - want).max() <= 1e-11, "value-gradient mass not conserved"
            sk = dk[b, :, hk].sum(0) + dkd[b, :, :, hk].sum((0, 1))
            assert np.abs(sk).max() <= 1e-11, "key gradients must sum to zero"
    vc = torch.full_like(v, 0.5)
    vdc = torch.full_like(vd, 0.5)
    dq2, dk2, dv2, dkd2, dvd2 = oracle.moda_bwd(q, k, vc, kd, vdc, dout, nthreads=2)
    assert np.abs(dq2).max() <= 1e-13 and np.abs(dk2).max() <= 1e-13 and np.abs(dkd2).max() <= 1e-13
    # value gradients do not depend on the values
    assert np.abs(dv2 - dv).max() <= 1e-13 and np.abs(dvd2 - dvd).max() <= 1e-13
    # zero output gradient -> every gradient zero
    z = oracle.moda_bwd(q, k, v, kd, vd, torch.zeros_like(dout), nthreads=2)
    assert all(np.abs(x).max() == 0.0 for x in z)


def pin_bwd_sampled(seed, causal=True, tol=1e-11):
    """Selected gradients (rows' dq, keys' dk/dv, tokens' depth gradients) equal torch autograd's."""
    B, T, Hq, Hk, d, L = 2, 11, 4, 2, 8, 3
    q, k, v, kd, vd = rand_problem(B, T, Hq, Hk, d, L, seed)
    dout = torch.randn(B, T, Hq, d, generator=torch.Generator("cpu").manual_seed(seed + 13), dtype=torch.float64)
    rows = [(0, 0, 0), (1, 5, 3), (0, T - 1, 2), (1, T - 1, 1)]
    keys = [(0, 0, 0), (1, 4, 1), (0, T - 1, 1), (1, T - 2, 0)]
    toks = [(0, 0, 1), (1, 7, 0), (1, T - 1, 1)]
    dq, dk, dv, dkd, dvd = oracle.moda_bwd_sampled(q, k, v, kd, vd, dout, rows, keys, toks, causal=causal,
                                                   nthreads=3)
    wq, wk, wv, wkd, wvd = autograd_reference(q, k, v, kd, vd, dout, causal)
    G = Hq // Hk
    for i, (b, t, h) in enumerate(rows):
        assert np.abs(dq[i] - wq[b, t, h]).max() <= tol, "sampled dq row differs from autograd"
    for i, (b, j, hk) in enumerate(keys):
        assert np.abs(dk[i] - wk[b, j, hk]).max() <= tol, "sampled dk differs from autograd"
        assert np.abs(dv[i] - wv[b, j, hk]).max() <= tol, "sampled dv differs from autograd"
    for i, (b, t, hk) in enumerate(toks):
        assert np.abs(dkd[i] - wkd[b, t, :, hk]).max() <= tol, "sampled depth dk differs from autograd"
        assert np.abs(dvd[i] - wvd[b, t, :, hk]).max() <= tol, "sampled depth dv differs from autograd"
    assert G == 2


# ---- depth write: KV projection ---------------------------------------------------

def pin_kv_project(seed):
    """The projection equals numpy's matmul x @ w.T (a library routine) split into K and V
    halves and heads; a one-hot weight selects input features; it is linear in x."""
    g = np.random.default_rng(seed)
    B, T, Dm, Hk, d = 2, 5, 24, 3, 4
    x = g.standard_normal((B, T, Dm))
    w = g.standard_normal((2 * Hk * d, Dm))
    k, v = oracle.kv_project(x, w, Hk, d)
    full = x @ w.T                                            # [B,T,2*Hk*d]
    assert np.abs(k - full[..., :Hk * d].reshape(B, T, Hk, d)).max() <= 1e-12, "K half differs from x @ w.T"
    assert np.abs(v - full[..., Hk * d:].reshape(B, T, Hk, d)).max() <= 1e-12, "V half differs from x @ w.T"
    sel = np.zeros_like(w)
    for n in range(2 * Hk * d):
        sel[n, (3 * n + 1) % Dm] = 1.0
    ks, vs = oracle.kv_project(x, sel, Hk, d)
    idx = [(3 * n + 1) % Dm for n in range(2 * Hk * d)]
    assert np.array_equal(ks.reshape(B, T, -1), x[..., idx[:Hk * d]]), "one-hot K weight must select features"
    assert np.array_equal(vs.reshape(B, T, -1), x[..., idx[Hk * d:]]), "one-hot V weight must select features"
    k2, v2 = oracle.kv_project(2.0 * x + 1.0, w, Hk, d)
    k1, v1 = oracle.kv_project(np.ones_like(x), w, Hk, d)
    assert np.abs(k2 - (2 * k + k1)).max() <= 1e-12 and np.abs(v2 - (2 * v + v1)).max() <= 1e-12

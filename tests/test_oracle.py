"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle_pins as pins
from oracle_pins import (pin_convex_and_permutation, pin_depth_aligned, pin_head_expansion,
                         pin_l0_is_gqa, pin_merge_identity, pin_sdpa, pin_t1_closed_form,
                         pin_t1_depth, pin_worked_example, rand_problem)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("G,Hk", [(1, 2), (2, 2), (4, 1), (3, 2)])
@pytest.mark.parametrize("L", [0, 1, 3])
def test_matches_sdpa_on_concatenated_keys(causal, G, Hk, L):
    pin_sdpa(B=2, T=13, Hq=G * Hk, Hk=Hk, d=8, L=L, causal=causal, seed=100 + 7 * G + L)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Hq,Hk", [(4, 2), (8, 2), (4, 4)])
def test_l0_reduces_to_gqa_attention(causal, Hq, Hk):
    pin_l0_is_gqa(B=2, T=17, Hq=Hq, Hk=Hk, d=16, causal=causal, seed=7 + Hq)


def test_worked_example_from_pages():
    pin_worked_example()


def test_t1_closed_forms():
    pin_t1_closed_form(3)
    pin_t1_depth(4)


def test_head_expansion_and_g1_per_head():
    pin_head_expansion(11)


def test_convex_combination_and_slot_permutation():
    pin_convex_and_permutation(12)


def test_merge_identity_of_two_branches():
    pin_merge_identity(13)


def test_depth_aligned_input_uses_same_token_depth():
    pin_depth_aligned(14)


def _brute_row(q, k, v, kd, vd, b, t, h, causal):
    """Explicit [sequence | depth] concatenation with math.exp and math.fsum, tiny inputs only."""
    B, T, Hq, d = q.shape
    G = Hq // k.shape[2]
    hk = h // G
    keys = [k[b, j, hk] for j in range(t + 1 if causal else T)] + [kd[b, t, i, hk] for i in range(kd.shape[2])]
    vals = [v[b, j, hk] for j in range(t + 1 if causal else T)] + [vd[b, t, i, hk] for i in range(kd.shape[2])]
    logits = [math.fsum(float(q[b, t, h, c]) * float(kk[c]) for c in range(d)) / math.sqrt(d) for kk in keys]
    mx = max(logits)
    w = [math.exp(a - mx) for a in logits]
    Z = math.fsum(w)
    out = [math.fsum(wi * float(vv[c]) for wi, vv in zip(w, vals)) / Z for c in range(d)]
    return out, mx + math.log(Z)


def test_pure_python_brute_force():
    q, k, v, kd, vd = rand_problem(1, 6, 4, 2, 4, 2, 21)
    for causal in (True, False):
        out, lse = oracle.moda_fwd(q, k, v, kd, vd, causal=causal, nthreads=1)
        for t in range(6):
            for h in range(4):
                o, l = _brute_row(q.numpy(), k.numpy(), v.numpy(), kd.numpy(), vd.numpy(), 0, t, h, causal)
                assert np.abs(out[0, t, h] - np.array(o)).max() <= 1e-13
                assert abs(lse[0, h, t] - l) <= 1e-13


def test_rows_api_equals_full_api():
    q, k, v, kd, vd = rand_problem(2, 9, 4, 2, 8, 3, 22)
    out, lse = oracle.moda_fwd(q, k, v, kd, vd, nthreads=3)
    rows = np.array([[0, 0, 0], [1, 8, 3], [0, 4, 1], [1, 0, 2]], dtype=np.int32)
    ro, rl = oracle.moda_fwd_rows(q, k, v, kd, vd, rows, nthreads=2)
    for n, (b, t, h) in enumerate(rows):
        assert np.array_equal(ro[n], out[b, t, h])
        assert rl[n] == lse[b, h, t]


def test_thread_count_does_not_change_results():
    q, k, v, kd, vd = rand_problem(1, 20, 4, 2, 8, 2, 23)
    o1, l1 = oracle.moda_fwd(q, k, v, kd, vd, nthreads=1)
    o7, l7 = oracle.moda_fwd(q, k, v, kd, vd, nthreads=7)
    assert np.array_equal(o1, o7) and np.array_equal(l1, l7)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_narrow_inputs_are_widened_exactly(dtype):
    q, k, v, kd, vd = (x.to(dtype) for x in rand_problem(1, 7, 2, 1, 8, 2, 24))
    o1, l1 = oracle.moda_fwd(q, k, v, kd, vd, nthreads=1)
    o2, l2 = oracle.moda_fwd(*(x.double() for x in (q, k, v, kd, vd)), nthreads=1)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("dtype", [np.float32, np.float64, np.uint16])
def test_pack_depth_matches_numpy_transpose(dtype):
    rng = np.random.default_rng(3)
    src = (rng.standard_normal((2, 5, 3, 4, 8)) * 100).astype(dtype)
    dst = oracle.pack_depth(src)
    assert dst.dtype == src.dtype or dtype == np.float64
    assert np.array_equal(dst.view(src.dtype), np.ascontiguousarray(src.transpose(0, 1, 3, 2, 4)))


def test_pack_depth_hand_example():
    # B=T=1, L=2, Hk=2, d=1: src[l][hk] = 10*l + hk  ->  dst[hk][l] = 10*l + hk
    src = np.array([0, 1, 10, 11], dtype=np.float32).reshape(1, 1, 2, 2, 1)
    dst = oracle.pack_depth(src)
    assert dst.reshape(-1).tolist() == [0, 10, 1, 11]


def test_append_depth_slot_matches_slice_assignment():
    rng = np.random.default_rng(4)
    dst = rng.standard_normal((2, 3, 2, 5, 4)).astype(np.float32)
    kv = rng.standard_normal((2, 3, 2, 4)).astype(np.float32)
    got = oracle.append_depth_slot(kv, dst, 3)
    want = dst.copy()
    want[:, :, :, 3, :] = kv
    assert np.array_equal(got, want)
    with pytest.raises(RuntimeError):
        oracle.append_depth_slot(kv, dst, 5)


# ---- gradients ----------------------------------------------------------------

@pytest.mark.parametrize("causal,G,Hk,L", [(True, 2, 2, 3), (False, 1, 2, 2), (True, 4, 1, 0), (True, 1, 1, 6)])
def test_bwd_matches_torch_autograd(causal, G, Hk, L):
    pins.pin_bwd_autograd(2, 11, G * Hk, Hk, 8, L, causal, 300 + 7 * G + L)


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_l0_matches_gqa_sdpa_autograd(causal):
    pins.pin_bwd_l0_gqa(2, 17, 4, 2, 16, causal, 310)


def test_bwd_finite_differences():
    pins.pin_bwd_finite_difference(320)


def test_bwd_invariants():
    pins.pin_bwd_invariants(330)


def test_bwd_thread_count_and_bf16_widening():
    q, k, v, kd, vd = pins.rand_problem(2, 10, 4, 2, 8, 3, 340)
    dout = torch.randn(2, 10, 4, 8, generator=torch.Generator("cpu").manual_seed(341), dtype=torch.float64)
    a = oracle.moda_bwd(q, k, v, kd, vd, dout, nthreads=1)
    b = oracle.moda_bwd(q, k, v, kd, vd, dout, nthreads=4)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    bf = [x.to(torch.bfloat16) for x in (q, k, v, kd, vd, dout)]
    c = oracle.moda_bwd(*bf, nthreads=2)
    d = oracle.moda_bwd(*[x.double() for x in bf], nthreads=2)
    for x, y in zip(c, d):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_sampled_matches_autograd(causal):
    pins.pin_bwd_sampled(350, causal=causal)


def test_bwd_sampled_equals_full_oracle():
    q, k, v, kd, vd = rand_problem(1, 40, 8, 2, 16, 5, 360)
    dout = torch.randn(1, 40, 8, 16, generator=torch.Generator("cpu").manual_seed(361), dtype=torch.float64)
    full = oracle.moda_bwd(q, k, v, kd, vd, dout, nthreads=2)
    rows = [(0, t, h) for t in (0, 17, 39) for h in (0, 5, 7)]
    keys = [(0, j, hk) for j in (0, 20, 38, 39) for hk in (0, 1)]
    toks = [(0, t, hk) for t in (0, 33) for hk in (0, 1)]
    dq, dk, dv, dkd, dvd = oracle.moda_bwd_sampled(q, k, v, kd, vd, dout, rows, keys, toks, nthreads=4)
    for i, (b, t, h) in enumerate(rows):
        assert np.abs(dq[i] - full[0][b, t, h]).max() <= 1e-13
    for i, (b, j, hk) in enumerate(keys):
        assert np.abs(dk[i] - full[1][b, j, hk]).max() <= 1e-13
        assert np.abs(dv[i] - full[2][b, j, hk]).max() <= 1e-13
    for i, (b, t, hk) in enumerate(toks):
        assert np.abs(dkd[i] - full[3][b, t, :, hk]).max() <= 1e-13
        assert np.abs(dvd[i] - full[4][b, t, :, hk]).max() <= 1e-13


def test_kv_project_pins():
    pins.pin_kv_project(370)


def test_kv_project_bf16_widened_exactly():
    g = torch.Generator("cpu").manual_seed(371)
    x = torch.randn(1, 3, 16, generator=g).to(torch.bfloat16)
    w = torch.randn(16, 16, generator=g).to(torch.bfloat16)
    a = oracle.kv_project(x, w, 2, 4)
    b = oracle.kv_project(x.double(), w.double(), 2, 4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])

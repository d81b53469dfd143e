"""The five workloads at full size, in the launch configuration the benchmark times,
checked on stratified sampled rows against the oracle (rows are independent, so each
sampled row is an exact check), plus finiteness of every output element."""
import numpy as np
import pytest
import torch

import oracle
from depth_stream_attention_amd import inputs as I
from parity_util import BF16_MAX, check, full_parity, run_path, sample_rows, sampled_parity, say, to_dev

pytestmark = pytest.mark.gpu


def _run(c, v, n_uniform=24):
    shape = I.workload(c, v)
    say("workload", c, "variant", v, shape.describe())
    dev = I.workload_inputs(c, v, device="cuda")
    out, lse = run_path(shape, dev)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    rows = sample_rows(shape, n_uniform=n_uniform, seed=c * 10 + v)
    res = sampled_parity(shape, dev, out, lse, rows, "workload %d.%d" % (c, v))
    del dev, out, lse
    torch.cuda.empty_cache()
    return res


def test_workload1_full():
    full_parity(I.workload(1), 1)


def test_workload2():
    _run(2, 0)


@pytest.mark.parametrize("v", [0, 1, 2, 3])
def test_workload3(v):
    _run(3, v, n_uniform=12)


@pytest.mark.parametrize("v", [0, 1, 2, 3])
def test_workload4(v):
    _run(4, v)


@pytest.mark.parametrize("v", [0, 1])
def test_workload5(v):
    _run(5, v, n_uniform=16)


# Sequences of 32768 tokens and more run the forward's 8-wave workgroups (256 rows,
# 128-row depth tiles); these shapes cover that kernel for both head dims, G from 1
# to 32, causal and full attention, a ragged length and depth counts that leave a
# partial 16-slot chunk.
LONG_SHAPES = [
    I.Shape(1, 32768, 2, 2, 64, 0),
    I.Shape(1, 32768, 4, 1, 128, 5),
    I.Shape(1, 32771, 8, 2, 128, 16),
    I.Shape(1, 32768, 32, 1, 64, 33, causal=False),
    I.Shape(2, 32768, 4, 2, 128, 48),
]


@pytest.mark.parametrize("i", range(len(LONG_SHAPES)))
def test_long_sequence_workgroups(i):
    shape = LONG_SHAPES[i]
    say("long-sequence shape", shape.describe())
    dev = to_dev(I.random_inputs(shape, 400 + i))
    out, lse = run_path(shape, dev)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    rows = sample_rows(shape, n_uniform=8, seed=400 + i)
    sampled_parity(shape, dev, out, lse, rows, "long %d" % i)


def test_long_sequence_depth_aligned():
    """The depth-aligned stress (every depth slot of a lead head near its query) on the
    8-wave kernel, sampled on late rows."""
    shape = I.Shape(1, 32768, 8, 2, 128, 40)
    dev = to_dev(I.random_inputs(shape, 420, depth_aligned=True))
    out, lse = run_path(shape, dev)
    rows = _late_rows(shape, 420, n_uniform=8)
    sampled_parity(shape, dev, out, lse, rows, "long depth-aligned")


def _late_rows(shape, seed, n_uniform=16):
    """Rows (b, t, h) weighted to the end of the sequence: t in {T-2, T-1}, both edges of
    each of the last eight 128-row query blocks, the first two tokens, and seeded-uniform
    tokens, for every (b, h)."""
    T, G = shape.T, shape.G
    tb = max(1, 128 // G)
    special = {0, 1, T - 2, T - 1}
    for i in range(8):
        special |= {T - (i + 1) * tb, T - i * tb - 1}
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(shape.B):
        for h in range(shape.Hq):
            ts = {t for t in special if 0 <= t < T} | set(rng.integers(0, T, n_uniform).tolist())
            rows += [(b, t, h) for t in sorted(ts)]
    return np.array(rows, dtype=np.int32)


@pytest.mark.parametrize("c,v", [(5, 0), (3, 3)])
def test_depth_aligned_full_size(c, v):
    """Depth-aligned stress at full size (the long-context workload, L=48, and the depth
    sweep's L=96).  Each depth key of (b, t, hk) is the query of head hk*G plus 0.5 times
    noise, so that head's depth logits sit near sqrt(d) and its depth slots carry most of
    its softmax mass at every position, including t = T-1; with N(0,1) inputs depth holds
    only about L/(t+1+L) of the mass there (equal-logit case of the joint softmax: MoDA
    reading notes, 二.2 worked example), which the tolerances alone would hide.  The test
    also shows that it can see a depth indexing mistake: the oracle's result for the same
    rows with every token given the previous token's depth slab must differ from the true
    result, on every lead-head row, by far more than the tolerance."""
    shape = I.workload(c, v)
    say("depth-aligned workload", c, "variant", v, shape.describe())
    dev = I.workload_inputs(c, v, depth_aligned=True, device="cuda")
    out, lse = run_path(shape, dev)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    rows = _late_rows(shape, seed=500 + 10 * c + v)
    host = {k: t.cpu() for k, t in dev.items()}
    del dev
    torch.cuda.empty_cache()
    ref_out, ref_lse = oracle.moda_fwd_rows(host["q"], host["k_seq"], host["v_seq"], host["k_depth"],
                                            host["v_depth"], rows, causal=shape.causal)
    b, t, h = (torch.from_numpy(rows[:, i].astype(np.int64)).cuda() for i in range(3))
    check(shape, out[b, t, h].float().cpu().numpy(), lse[b, h, t].cpu().numpy(), ref_out, ref_lse,
          "depth-aligned %d.%d" % (c, v))
    del out, lse
    torch.cuda.empty_cache()

    # Sensitivity: token t reads token t-1's depth slab (token 0 reads the last token's).
    lead = (rows[:, 2] % shape.G == 0) & (rows[:, 1] >= 1)
    kd_prev = torch.roll(host["k_depth"], 1, dims=1)
    vd_prev = torch.roll(host["v_depth"], 1, dims=1)
    bad_out, _ = oracle.moda_fwd_rows(host["q"], host["k_seq"], host["v_seq"], kd_prev, vd_prev, rows[lead],
                                      causal=shape.causal)
    gap = np.abs(bad_out - ref_out[lead]).max(axis=1)
    say("depth-aligned %d.%d: previous-slab mistake moves lead-head rows by %.3g .. %.3g (n=%d)"
        % (c, v, gap.min(), gap.max(), gap.size))
    assert gap.size > 0 and gap.min() > 10 * BF16_MAX, "the stress input does not expose a wrong depth slab"


def _random_long_shapes(n, seed):
    """n shapes of 32768 to 36000 tokens (the 8-wave kernel) drawn with a fixed seed:
    group sizes 1 to 32, both head dims, causal and full attention, L from 0 to 64."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        G = int(rng.choice([1, 2, 4, 8, 16, 32]))
        Hk = int(rng.choice([1, 2]))
        d = int(rng.choice([64, 128]))
        T = int(rng.integers(32768, 36001))
        L = int(rng.choice([0, int(rng.integers(1, 65))]))
        causal = bool(rng.random() < 0.75)
        out.append(I.Shape(1, T, Hk * G, Hk, d, L, causal=causal))
    return out


@pytest.mark.parametrize("i,shape", list(enumerate(_random_long_shapes(6, 2031))))
def test_random_long_shapes(i, shape):
    say("random long shape", shape.describe())
    aligned = shape.L > 0 and i % 2 == 0
    dev = to_dev(I.random_inputs(shape, 700 + i, depth_aligned=aligned))
    out, lse = run_path(shape, dev)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    rows = _late_rows(shape, 700 + i, n_uniform=6) if aligned else sample_rows(shape, n_uniform=6, seed=700 + i)
    sampled_parity(shape, dev, out, lse, rows, "random long %d" % i)

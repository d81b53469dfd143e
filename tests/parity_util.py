"""Helpers of the GPU parity tests: run the HIP path through the C ABI, run the oracle
on the same inputs, compare."""
import numpy as np
import torch

import oracle
from depth_stream_attention_amd import api
from depth_stream_attention_amd import inputs as I

# Tolerances on out (vs the fp64 oracle on the same rounded inputs).
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
F32_MAX = 1e-4
# lse tolerances (natural log).
BF16_LSE, F32_LSE = 1e-3, 1e-4


def random_shapes(n, seed, budget):
    """n forward shapes drawn with a fixed seed, each with a flag for depth-aligned inputs:
    every group size, both head dims, causal and full attention, ragged lengths, L from 0
    past a 16-slot chunk boundary; the oracle's work B*Hq*T*(T/2+L)*d stays under
    `budget` multiply-adds per case."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        G = int(rng.choice([1, 2, 4, 8, 16, 32]))
        Hk = int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 4))
        T = int(rng.integers(1, 700))
        L = int(rng.choice([0, int(rng.integers(1, 70))]))
        causal = bool(rng.random() < 0.75)
        aligned = bool(L > 0 and rng.random() < 0.3)
        if B * Hk * G * T * (T / 2 + L) * d > budget:
            continue
        out.append((I.Shape(B, T, Hk * G, Hk, d, L, causal=causal), aligned))
    return out


def say(*a):
    print(*a, flush=True)


def to_dev(inp):
    return {k: v.cuda() for k, v in inp.items()}


def run_path(shape, dev, out=None, lse=None):
    """Pack the depth stream on the GPU, then run the forward; returns (out, lse) on the GPU."""
    kd = vd = None
    if shape.L > 0:
        kd = api.moda_pack_depth(dev["k_depth"])
        vd = api.moda_pack_depth(dev["v_depth"])
    fn = api.moda_attn_fwd if shape.dtype == "bf16" else api.moda_attn_fwd_f32
    o, l = fn(dev["q"], dev["k_seq"], dev["v_seq"], kd, vd, causal=shape.causal, out=out, lse=lse)
    torch.cuda.synchronize()
    return o, l


def check(shape, got_out, got_lse, ref_out, ref_lse, label=""):
    """Compare float64 host arrays of equal shape; raise AssertionError with the figures."""
    err = np.abs(got_out.astype(np.float64) - ref_out)
    lerr = np.abs(got_lse.astype(np.float64) - ref_lse)
    assert np.all(np.isfinite(got_out)) and np.all(np.isfinite(got_lse)), "%s: non-finite output" % label
    if shape.dtype == "bf16":
        ok = err.max() <= BF16_MAX and err.mean() <= BF16_MEAN and lerr.max() <= BF16_LSE
    else:
        ok = err.max() <= F32_MAX and lerr.max() <= F32_LSE
    say("%s %s: max|err| %.3g mean|err| %.3g max|dlse| %.3g over %d rows" % (
        label, shape.describe(), err.max(), err.mean(), lerr.max(), got_lse.size))
    assert ok, "%s: out max %.3g mean %.3g, lse max %.3g" % (label, err.max(), err.mean(), lerr.max())
    return err.max(), err.mean(), lerr.max()


def full_parity(shape, seed, depth_aligned=False):
    """Every row of a problem small enough for the oracle to finish in seconds."""
    host = I.random_inputs(shape, seed, depth_aligned=depth_aligned)
    say("case", shape.describe(), "seed", seed, "aligned" if depth_aligned else "")
    out, lse = run_path(shape, to_dev(host))
    ref_out, ref_lse = oracle.moda_fwd(host["q"], host["k_seq"], host["v_seq"], host["k_depth"],
                                       host["v_depth"], causal=shape.causal)
    return check(shape, out.float().cpu().numpy(), lse.cpu().numpy(), ref_out, ref_lse, "full")


def sample_rows(shape, n_uniform=24, seed=0):
    """Stratified rows (b, t, h): sequence ends, both edges of the first and last four
    128-row and 256-row query blocks (128/G and 256/G tokens each: the forward's
    workgroup sizes), and seeded-uniform tokens, per (b, h)."""
    T, G = shape.T, shape.G
    special = {0, 1, 2, 3, T - 2, T - 1}
    for rows in (128, 256):
        tb = max(1, rows // G)
        for i in range(4):
            special |= {i * tb, i * tb + tb - 1, T - (i + 1) * tb, T - i * tb - 1}
    special = sorted(t for t in special if 0 <= t < T)
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(shape.B):
        for h in range(shape.Hq):
            ts = set(special) | set(rng.integers(0, T, n_uniform).tolist())
            rows += [(b, t, h) for t in sorted(ts)]
    return np.array(rows, dtype=np.int32)


def sampled_parity(shape, dev, out, lse, rows, label):
    host = {k: v.cpu() for k, v in dev.items()}
    ref_out, ref_lse = oracle.moda_fwd_rows(host["q"], host["k_seq"], host["v_seq"], host["k_depth"],
                                            host["v_depth"], rows, causal=shape.causal)
    b, t, h = (torch.from_numpy(rows[:, i].astype(np.int64)).cuda() for i in range(3))
    got_out = out[b, t, h].float().cpu().numpy()
    got_lse = lse[b, h, t].cpu().numpy()
    return check(shape, got_out, got_lse, ref_out, ref_lse, label)

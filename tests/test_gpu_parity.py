"""GPU parity: the HIP path, called through the C ABI, against the fp64 oracle.

bf16: max|err| <= 2e-2 and mean|err| <= 2e-3 on out (fp32 accumulation),
|dlse| <= 1e-3.  fp32: max|err| <= 1e-4, |dlse| <= 1e-4.  The oracle runs on
exact host copies of the same rounded inputs."""
import numpy as np
import pytest
import torch

import oracle
from depth_stream_attention_amd import api
from depth_stream_attention_amd import inputs as I
from parity_util import full_parity, random_shapes, run_path, say, to_dev

pytestmark = pytest.mark.gpu
S = I.Shape


# ---- small problems, every row -------------------------------------------------

def test_tiny_workload_f32():
    full_parity(I.workload(1), 1)


def test_tiny_workload_bf16():
    full_parity(I.with_(I.workload(1), dtype="bf16"), 2)


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16, 32])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_group_sizes(G, dtype):
    full_parity(S(2, 150, 2 * G, 2, 128, 7, dtype), 10 + G)


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 129, 333])
def test_ragged_lengths(T):
    full_parity(S(1, T, 8, 2, 128, 3), 20 + T)


@pytest.mark.parametrize("L", [0, 1, 31, 32, 33, 96, 257, 512])
def test_depth_slot_counts(L):
    full_parity(S(2, 97, 8, 2, 128, L), 30 + L)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_head_dims(d, dtype):
    full_parity(S(1, 200, 4, 1, d, 5, dtype), 40 + d)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L", [0, 6])
def test_full_attention(dtype, L):
    full_parity(S(2, 130, 8, 4, 128, L, dtype, causal=False), 50 + L)


def test_keys_scaled_by_half():
    full_parity(S(1, 300, 8, 4, 128, 32, key_scale=0.5), 60)


@pytest.mark.parametrize("G,L", [(1, 12), (4, 12), (1, 40), (2, 40), (8, 40), (16, 40)])
def test_depth_aligned_stress(G, L):
    # head hk*G's depth keys track its query, so depth carries most of its mass at every t;
    # L = 40 gives each token three 16-slot depth tiles (the last one partial), and with
    # G <= 16 a wave's tokens fill both 16-row halves of its rows
    full_parity(S(1, 700, 4 * G, 4, 128, L), 70 + G + L, depth_aligned=True)


def test_several_tiles_multi_batch():
    full_parity(S(3, 517, 16, 4, 128, 24), 80)


# ---- structural properties ------------------------------------------------------

def test_bitwise_deterministic():
    sh = S(1, 1000, 16, 4, 128, 24)
    dev = to_dev(I.random_inputs(sh, 90))
    o1, l1 = run_path(sh, dev)
    o2, l2 = run_path(sh, dev)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_no_writes_outside_outputs(dtype):
    sh = S(2, 77, 8, 2, 128, 5, dtype)
    dev = to_dev(I.random_inputs(sh, 91))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    pad = 4096
    n = sh.B * sh.T * sh.Hq * sh.d
    obuf = torch.full((n + 2 * pad,), 7.0, dtype=tdt, device="cuda")
    lbuf = torch.full((sh.B * sh.Hq * sh.T + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
    out = obuf[pad:pad + n].view(sh.B, sh.T, sh.Hq, sh.d)
    lse = lbuf[pad:pad + sh.B * sh.Hq * sh.T].view(sh.B, sh.Hq, sh.T)
    run_path(sh, dev, out=out, lse=lse)
    for buf in (obuf, lbuf):
        assert torch.all(buf[:pad] == 7.0) and torch.all(buf[-pad:] == 7.0), "write outside the output"
    assert not torch.any(out == 7.0)


def test_pack_and_append_are_bit_exact():
    for dt in (torch.bfloat16, torch.float32):
        src = torch.randn(2, 33, 5, 3, 128, dtype=torch.float32).to(dt)
        got = api.moda_pack_depth(src.cuda())
        torch.cuda.synchronize()
        want = oracle.pack_depth(src)
        assert np.array_equal(got.cpu().view(torch.int16 if dt == torch.bfloat16 else torch.int32).numpy()
                              .view(want.dtype), want)
    dst = torch.randn(2, 9, 3, 6, 64, dtype=torch.float32).to(torch.bfloat16)
    kv = torch.randn(2, 9, 3, 64, dtype=torch.float32).to(torch.bfloat16)
    ddev = dst.cuda()
    api.moda_append_depth_slot(kv.cuda(), ddev, 4)
    torch.cuda.synchronize()
    want = oracle.append_depth_slot(kv, dst, 4)
    assert np.array_equal(ddev.cpu().view(torch.int16).numpy().view(np.uint16), want)


def test_append_builds_the_packed_stream():
    """Writing slot l from layer l's KV gives the same packed tensor as the full pack."""
    B, T, L, Hk, d = 1, 40, 7, 2, 128
    src = torch.randn(B, T, L, Hk, d).to(torch.bfloat16).cuda()
    packed = api.moda_pack_depth(src)
    built = torch.zeros_like(packed)
    for l in range(L):
        api.moda_append_depth_slot(src[:, :, l].contiguous(), built, l)
    torch.cuda.synchronize()
    assert torch.equal(packed, built)


def test_binding_rejects_bad_tensors():
    sh = S(1, 16, 4, 2, 128, 2)
    dev = to_dev(I.random_inputs(sh, 92))
    with pytest.raises(TypeError):
        api.moda_attn_fwd(dev["q"].float(), dev["k_seq"], dev["v_seq"])
    with pytest.raises(ValueError):
        api.moda_attn_fwd(dev["q"], dev["k_seq"][:, :8], dev["v_seq"])
    with pytest.raises(api.MODAError) as e:
        q = torch.zeros(1, 16, 6, 96, dtype=torch.bfloat16, device="cuda")
        kv = torch.zeros(1, 16, 2, 96, dtype=torch.bfloat16, device="cuda")
        api.moda_attn_fwd(q, kv, kv)
    assert e.value.code == api.MODA_ERR_UNSUPPORTED
    say("binding errors ok")


# ---- seeded random shapes ---------------------------------------------------------

@pytest.mark.parametrize("i,case", list(enumerate(random_shapes(24, 2027, 1e9))))
def test_random_shapes(i, case):
    shape, aligned = case
    full_parity(shape, 500 + i, depth_aligned=aligned)

"""The seeded input recipe: deterministic, shaped as the workloads, shared sequence inputs."""
import numpy as np
import torch

from depth_stream_attention_amd import inputs as I


def test_seed_formula_and_sharing():
    assert I.seeds(2, 0) == {"q": 2000, "k_seq": 2001, "v_seq": 2002, "k_depth": 2003, "v_depth": 2004}
    assert I.seeds(4, 3)["k_seq"] == 4031
    s3 = I.seeds(3, 2)
    assert (s3["q"], s3["k_seq"], s3["v_seq"], s3["k_depth"]) == (3000, 3001, 3002, 3023)
    assert I.seeds(5, 1)["q"] == I.seeds(5, 0)["q"] == 5000


def test_workload_shapes():
    assert I.workload(1) == I.Shape(1, 128, 4, 2, 64, 4, "f32")
    assert [s.L for s in I.WORKLOADS[3]] == [0, 12, 48, 96]
    assert [s.G for s in I.WORKLOADS[4]] == [1, 2, 4, 8]
    assert all(s.key_scale == 0.5 for s in I.WORKLOADS[4])
    assert I.workload(5, 1).L == 0 and I.workload(5, 0).L == 48


def test_inputs_are_deterministic_and_typed():
    a = I.workload_inputs(1)
    b = I.workload_inputs(1)
    for n in I.TENSORS:
        assert torch.equal(a[n], b[n])
        assert a[n].dtype == torch.float32
    assert tuple(a["k_depth"].shape) == (1, 128, 4, 2, 64)
    sh = I.Shape(1, 16, 4, 2, 8, 3)
    x = I.random_inputs(sh, 9)
    assert x["q"].dtype == torch.bfloat16
    # bf16 values are the RNE rounding of the fp32 Philox draw with key = seed
    g = np.random.Generator(np.random.Philox(key=9, counter=[0, 0, 0, 0]))
    want = torch.from_numpy(g.standard_normal(16 * 4 * 8, dtype=np.float32)).view(1, 16, 4, 8)
    assert torch.equal(x["q"], want.to(torch.bfloat16))


def test_chunked_host_draw_is_thread_count_independent(monkeypatch):
    a = I._randn((3, 1 << 21), 5)              # spans two chunks
    monkeypatch.setattr(I.os, "cpu_count", lambda: 1)
    b = I._randn((3, 1 << 21), 5)
    assert torch.equal(a, b)
    g = np.random.Generator(np.random.Philox(key=5, counter=[0, 0, 0, 1]))
    assert torch.equal(a.reshape(-1)[1 << 22:], torch.from_numpy(g.standard_normal((3 << 21) - (1 << 22),
                                                                                  dtype=np.float32)))


def test_key_scale_and_empty_depth():
    sh = I.Shape(1, 8, 2, 1, 8, 2, key_scale=0.5)
    x = I.random_inputs(sh, 1)
    y = I.random_inputs(I.with_(sh, key_scale=1.0), 1)
    assert torch.equal(x["k_seq"].float(), (y["k_seq"].float() * 0.5))
    assert torch.equal(x["v_seq"], y["v_seq"])
    z = I.random_inputs(I.with_(sh, L=0), 1)
    assert z["k_depth"].shape == (1, 8, 0, 1, 8)


def test_depth_aligned_recipe():
    sh = I.Shape(1, 8, 4, 2, 8, 3)
    x = I.random_inputs(sh, 2, depth_aligned=True)
    lead = x["q"].float()[:, :, ::2].unsqueeze(2)
    # keys sit within 0.5*N(0,1) (plus bf16 rounding) of the lead query
    assert ((x["k_depth"].float() - lead).abs().max() < 4.0)

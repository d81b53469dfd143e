"""The five workloads at full size, in the launch configuration the benchmark times,
checked on stratified sampled rows against the oracle (rows are independent, so each
sampled row is an exact check), plus finiteness of every output element."""
import pytest
import torch

from depth_stream_attention_amd import inputs as I
from parity_util import full_parity, run_path, sample_rows, sampled_parity, say

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

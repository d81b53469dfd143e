"""Work accounting used in the benchmark report, checked against the pages' printed values."""
import json
import os

from depth_stream_attention_amd import accounting as acc
from depth_stream_attention_amd import inputs as I

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_depth_utilisation_matches_table2():
    with open(os.path.join(GOLDEN, "depth_utilisation_table2.json")) as f:
        ex = json.load(f)
    for row in ex["rows"]:
        eta = acc.depth_utilisation("group", C=ex["C"], G=row["G"])
        assert round(100 * eta, ex["printed_decimals"]) == row["printed_percent"] or \
            abs(100 * eta - row["printed_percent"]) < 0.01
    assert acc.depth_utilisation("flash", T=4096) == 1 / 4096
    assert acc.depth_utilisation("chunk", C=64) == 1 / 64


def test_flops_by_brute_force_count():
    s = I.Shape(2, 9, 4, 2, 16, 3)
    pairs = sum(t + 1 for t in range(9))
    assert acc.flops(s) == 4 * 16 * 2 * 4 * (pairs + 9 * 3)
    assert acc.flops(I.with_(s, causal=False)) == 4 * 16 * 2 * 4 * (81 + 27)


def test_long_context_figures():
    s = I.workload(5, 0)
    assert abs(acc.flops_seq(s.B, s.T, s.Hq, s.d) - 1.759e13) / 1.759e13 < 1e-3
    assert abs(acc.flops_depth(s.B, s.T, s.Hq, s.d, s.L) - 2.58e10) / 2.58e10 < 1e-2
    assert abs(acc.depth_bytes(s) - 6.44e9) / 6.44e9 < 1e-2


def test_decode_bytes_and_flops():
    # B=2, T=10, Hq=8, Hk=2, d=4, L=3, bf16: K and V caches 2*(2*10*2*4)*2 = 640, depth slots
    # 2*(2*2*3*4)*2 = 192, q and out 2*(2*8*4)*2 = 256, lse 4*(2*8) = 64.
    assert acc.decode_bytes(2, 10, 8, 2, 4, 3) == 640 + 192 + 256 + 64
    assert acc.decode_flops(2, 10, 8, 4, 3) == 4 * 4 * 2 * 8 * 13


def test_bwd_accounting():
    s = I.workload(5, 0)
    P = 65536 * 65537 // 2
    assert acc.bwd_flops(s) == 10 * 128 * 16 * (P + 65536 * 48)
    assert acc.bwd_flops(s) * 2 == 5 * acc.flops(s)  # 2.5 x the forward
    e = 2
    assert acc.bwd_bytes(s) == (4 * 65536 * 16 * 128 * e + 4 * 65536 * 4 * 128 * e
                                + 4 * 65536 * 4 * 48 * 128 * e + 4 * 16 * 65536)


def test_kv_project_accounting():
    assert acc.kv_project_flops(1, 65536, 2048, 4, 128) == 2 * 65536 * 2048 * 1024
    assert acc.kv_project_bytes(1, 65536, 2048, 4, 128) == (65536 * 2048 * 2 + 1024 * 2048 * 2
                                                            + 2 * 65536 * 1024 * 2)

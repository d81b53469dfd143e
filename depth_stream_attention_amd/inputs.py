"""Seeded synthetic inputs for the MoDA forward.

This module draws random tensors and nothing else: it holds none of the
attention arithmetic, so both the HIP path and the CPU oracle can be fed from
it.  Every tensor is i.i.d. N(0, 1) drawn in fp32 and then rounded once (RNE) to
the working dtype.  Two counter-based generators are used, chosen by where
the tensor is drawn:
  * device="cpu": numpy's Philox4x64 bit generator with key = seed, the
    tensor split into chunks of 2**22 elements, chunk c drawn from counter
    (0, 0, 0, c) by Generator.standard_normal(dtype=float32).  The result does
    not depend on how many host threads fill the chunks.
  * device="cuda...": torch.randn with a torch.Generator on that device seeded
    with seed (torch's Philox on the GPU).  The full-size workloads are drawn
    this way (billions of elements); the oracle is given exact host copies.

The pages benchmark their kernel on synthetic fixed shapes (MoDA reading
notes, 三.1 kernel-benchmark row), so no dataset is involved.

Layouts (row-major): q [B,T,Hq,d]; k_seq, v_seq [B,T,Hk,d]; depth K/V in the
generation layout [B,T,L,Hk,d] (a position's L slots stored together; the
library's packer turns this into [B,T,Hk,L,d]).

Seeds: tensor k (q=0, k_seq=1, v_seq=2, k_depth=3, v_depth=4) of workload c,
variant v uses seed 1000*c + 10*v + k.  In the depth sweep (3) and the
long-context workload (5), q / k_seq / v_seq always use v = 0, so every depth
variant, the L=0 one included, shares one set of sequence inputs.
"""
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np
import torch

TENSORS = ("q", "k_seq", "v_seq", "k_depth", "v_depth")


@dataclass(frozen=True)
class Shape:
    B: int
    T: int
    Hq: int
    Hk: int
    d: int
    L: int
    dtype: str = "bf16"  # "bf16" or "f32"
    causal: bool = True
    key_scale: float = 1.0  # multiplies k_seq and k_depth before rounding

    @property
    def G(self) -> int:
        return self.Hq // self.Hk

    def describe(self) -> str:
        return ("B%d T%d Hq%d Hk%d d%d L%d %s%s%s" % (
            self.B, self.T, self.Hq, self.Hk, self.d, self.L, self.dtype,
            "" if self.causal else " full", "" if self.key_scale == 1.0 else " kscale%g" % self.key_scale))


# The five workloads, by number, each as a list of variants.
WORKLOADS = {
    1: [Shape(1, 128, 4, 2, 64, 4, "f32")],                                   # tiny check
    2: [Shape(4, 4096, 16, 4, 128, 24)],                                      # 700M-class layer
    3: [Shape(2, 8192, 32, 8, 128, L) for L in (0, 12, 48, 96)],              # depth sweep
    4: [Shape(1, 16384, 4 * G, 4, 128, 32, key_scale=0.5) for G in (1, 2, 4, 8)],  # GQA sweep
    5: [Shape(1, 65536, 16, 4, 128, 48), Shape(1, 65536, 16, 4, 128, 0)],     # long context, L=48 and L=0
}
SHARED_SEQUENCE_INPUTS = (3, 5)


def workload(c: int, v: int = 0) -> Shape:
    return WORKLOADS[c][v]


def seeds(c: int, v: int = 0):
    """Seed of each tensor of workload c, variant v (see module docstring)."""
    out = {}
    for k, name in enumerate(TENSORS):
        vv = 0 if (c in SHARED_SEQUENCE_INPUTS and k < 3) else v
        out[name] = 1000 * c + 10 * vv + k
    return out


def _torch_dtype(name: str):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


_CHUNK = 1 << 22


def _randn(shape, seed: int, device="cpu") -> torch.Tensor:
    device = torch.device(device)
    if device.type != "cpu":
        g = torch.Generator(device=device)
        g.manual_seed(int(seed))
        return torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    n = 1
    for x in shape:
        n *= int(x)
    out = np.empty(n, np.float32)

    def fill(c):
        g = np.random.Generator(np.random.Philox(key=int(seed), counter=[0, 0, 0, c]))
        lo = c * _CHUNK
        g.standard_normal(min(n, lo + _CHUNK) - lo, dtype=np.float32, out=out[lo:lo + _CHUNK])

    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks <= 1:
        if n:
            fill(0)
    else:
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1, nchunks)) as ex:
            list(ex.map(fill, range(nchunks)))
    return torch.from_numpy(out).view(tuple(int(x) for x in shape))


def make_inputs(shape: Shape, seed_of: dict, depth_aligned: bool = False, device="cpu"):
    """Draw q, k_seq, v_seq, k_depth, v_depth on `device` for `shape`.

    seed_of maps each tensor name to its seed.  With L == 0 the depth tensors
    are empty ([B,T,0,Hk,d]).  depth_aligned=True builds the stress input in
    which each depth key of (b, t, hk) is the query of head hk*G plus 0.5 times
    noise, so that head's depth logits stay large at every position.
    """
    s = shape
    dt = _torch_dtype(s.dtype)
    q = _randn((s.B, s.T, s.Hq, s.d), seed_of["q"], device)
    k = _randn((s.B, s.T, s.Hk, s.d), seed_of["k_seq"], device)
    v = _randn((s.B, s.T, s.Hk, s.d), seed_of["v_seq"], device)
    if s.L > 0:
        kd = _randn((s.B, s.T, s.L, s.Hk, s.d), seed_of["k_depth"], device)
        vd = _randn((s.B, s.T, s.L, s.Hk, s.d), seed_of["v_depth"], device)
        if depth_aligned:
            lead = q[:, :, :: s.G, :]  # [B,T,Hk,d]: head hk*G of each KV group
            kd = lead.unsqueeze(2) + 0.5 * kd
    else:
        kd = torch.empty((s.B, s.T, 0, s.Hk, s.d), dtype=torch.float32, device=device)
        vd = torch.empty((s.B, s.T, 0, s.Hk, s.d), dtype=torch.float32, device=device)
    if s.key_scale != 1.0:
        k = k * s.key_scale
        kd = kd * s.key_scale
    return {"q": q.to(dt), "k_seq": k.to(dt), "v_seq": v.to(dt),
            "k_depth": kd.to(dt), "v_depth": vd.to(dt)}


def workload_inputs(c: int, v: int = 0, depth_aligned: bool = False, device="cpu"):
    return make_inputs(workload(c, v), seeds(c, v), depth_aligned=depth_aligned, device=device)


def random_inputs(shape: Shape, seed: int, depth_aligned: bool = False, device="cpu"):
    """Inputs for an ad-hoc shape: tensor k uses seed + k."""
    return make_inputs(shape, {n: seed + k for k, n in enumerate(TENSORS)}, depth_aligned, device)


def random_dout(shape: Shape, seed: int, device="cpu"):
    """An output gradient [B,T,Hq,d] for the backward: N(0, 1), rounded once to the working dtype."""
    s = shape
    return _randn((s.B, s.T, s.Hq, s.d), seed, device).to(_torch_dtype(s.dtype))


def with_(shape: Shape, **kw) -> Shape:
    return replace(shape, **kw)

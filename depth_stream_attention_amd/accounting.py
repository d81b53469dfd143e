"""Algorithmic work of the MoDA forward: flops, minimum HBM bytes, depth utilisation.

Flops count multiply-adds of the two products per candidate (QK and PV,
2*d flops each): F_seq = 4*d*B*Hq*P with P = T(T+1)/2 visible pairs under the
causal mask (T^2 without it), F_depth = 4*d*B*Hq*T*L.  Exponentials are not
counted.  Bytes are the minimum the operation must move: every input element
read once, out and lse written once (the packed depth K/V is 2*B*T*Hk*L*d
elements, which the group-aware layout reads exactly once).
"""


def visible_pairs(T: int, causal: bool) -> int:
    return T * (T + 1) // 2 if causal else T * T


def flops_seq(B, T, Hq, d, causal=True) -> int:
    return 4 * d * B * Hq * visible_pairs(T, causal)


def flops_depth(B, T, Hq, d, L) -> int:
    return 4 * d * B * Hq * T * L


def flops(shape) -> int:
    s = shape
    return flops_seq(s.B, s.T, s.Hq, s.d, s.causal) + flops_depth(s.B, s.T, s.Hq, s.d, s.L)


def depth_bytes(shape) -> int:
    s = shape
    return 2 * s.B * s.T * s.Hk * s.L * s.d * elem_bytes(s)


def elem_bytes(shape) -> int:
    return {"bf16": 2, "f32": 4}[shape.dtype]


def algorithmic_bytes(shape) -> int:
    s = shape
    e = elem_bytes(s)
    q_out = 2 * s.B * s.T * s.Hq * s.d * e
    kv = 2 * s.B * s.T * s.Hk * s.d * e
    return q_out + kv + depth_bytes(s) + 4 * s.B * s.Hq * s.T


def bwd_flops(shape) -> int:
    """Algorithmic flops of the backward: five products per visible (row, candidate) pair --
    the recomputed scores Q K^T, dP = dO V^T, dV += P^T dO, dK += dS^T Q, dQ += dS K --
    2*d flops each, i.e. 2.5 times the forward's."""
    s = shape
    return 10 * s.d * s.B * s.Hq * (visible_pairs(s.T, s.causal) + s.T * s.L)


def bwd_bytes(shape) -> int:
    """Minimum bytes of the backward: q, out, dout read and dq written ([B,T,Hq,d]); k, v read
    and dk, dv written ([B,T,Hk,d]); depth K/V read and their gradients written; lse read."""
    s = shape
    e = elem_bytes(s)
    return (4 * s.B * s.T * s.Hq * s.d * e + 4 * s.B * s.T * s.Hk * s.d * e + 2 * depth_bytes(s)
            + 4 * s.B * s.Hq * s.T)


def kv_project_flops(B, T, Dm, Hk, d) -> int:
    """The depth-write KV projection: tokens x (2*Hk*d) outputs, Dm multiply-adds each."""
    return 2 * B * T * Dm * 2 * Hk * d


def kv_project_bytes(B, T, Dm, Hk, d, e=2) -> int:
    """Minimum bytes of the fused KV projection writing both the sequence K/V and one depth
    slot: x and w read once, each output element written twice."""
    return B * T * Dm * e + 2 * Hk * d * Dm * e + 2 * (2 * B * T * Hk * d * e)


def decode_bytes(B, T, Hq, Hk, d, L, e=2) -> int:
    """Minimum bytes of one decode step: the K/V cache and the token's depth slots read
    once, q read, out written (e bytes per element), lse written (fp32)."""
    return 2 * B * T * Hk * d * e + 2 * B * Hk * L * d * e + 2 * B * Hq * d * e + 4 * B * Hq


def decode_flops(B, T, Hq, d, L) -> int:
    return 4 * d * B * Hq * (T + L)


def depth_utilisation(layout: str, T: int = 0, C: int = 0, G: int = 1) -> float:
    """Fraction of computed depth scores that are unmasked when the depth stage is
    computed densely per query block ("Mixture-of-Depths Attention" summary,
    papercache.org, 3.2): flash-compatible layout 1/T, chunk-aware 1/C,
    group-aware G/C (query blocks aligned to G)."""
    if layout == "flash":
        return 1.0 / T
    if layout == "chunk":
        return 1.0 / C
    if layout == "group":
        return G / C
    raise ValueError(layout)

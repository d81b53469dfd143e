"""Planted mistakes: each test rebuilds the oracle from its C source with one
deliberate error (on the CPU, in a temporary directory) and requires at least
one of the pins in oracle_pins.py to reject it.  This shows the pins are
strong enough to catch a dropped term, a wrong index, sign or scale, a
transposed operand or layout, and an off-by-one mask."""
import ctypes
import os
import shutil
import subprocess

import pytest

import oracle.oracle as orc
import oracle_pins as pins

SRC = os.path.join(os.path.dirname(orc.__file__), "moda_oracle.c")

MUTANTS = {
    "depth_dropped_from_denominator": ("    Z += logit[n];", "    if (n < nseq) Z += logit[n];"),
    "interleaved_head_map": ("const int hk = h / G;", "const int hk = h % p->Hk;"),
    "causal_sees_next_key": ("const int nseq = p->causal ? t + 1 : p->T;",
                             "const int nseq = p->causal ? (t + 1 < p->T ? t + 2 : p->T) : p->T;"),
    "scale_one_over_d": ("const double s = 1.0 / sqrt((double)d);", "const double s = 1.0 / (double)d;"),
    "depth_keys_of_previous_token": (
        "dot += qrow[c] * orc_load(p->k_depth, ix_depth(p, b, t, i, hk, c), p->kind);",
        "dot += qrow[c] * orc_load(p->k_depth, ix_depth(p, b, t > 0 ? t - 1 : t, i, hk, c), p->kind);"),
    "depth_read_in_packed_layout": (
        "return ((((size_t)b * p->T + t) * p->L + i) * p->Hk + hk) * p->d + c;",
        "return ((((size_t)b * p->T + t) * p->Hk + hk) * p->L + i) * p->d + c;"),
    "lse_without_max": ("*lse_out = m + log(Z);", "*lse_out = log(Z);"),
    "exponent_sign": ("logit[n] = exp(logit[n] - m);", "logit[n] = exp(m - logit[n]);"),
    "depth_values_are_keys": (
        "acc += logit[nseq + i] * orc_load(p->v_depth, ix_depth(p, b, t, i, hk, c), p->kind);",
        "acc += logit[nseq + i] * orc_load(p->k_depth, ix_depth(p, b, t, i, hk, c), p->kind);"),
    "depth_logits_unscaled": ("    logit[nseq + i] = s * dot;", "    logit[nseq + i] = dot;"),
    # gradients
    "bwd_drops_row_correction": ("dS[n] = logit[n] * (dP[n] - D);", "dS[n] = logit[n] * dP[n];"),
    "bwd_dk_unscaled": ("dkp[kix] += s * dS[n] * qrow[c];", "dkp[kix] += dS[n] * qrow[c];"),
    "bwd_dv_weighted_by_dP": ("dvp[kix] += logit[n] * dorow[c];", "dvp[kix] += dP[n] * dorow[c];"),
    "bwd_dq_sign": ("job->dq[ix_q(p, b, t, h, c)] = s * acc;", "job->dq[ix_q(p, b, t, h, c)] = -s * acc;"),
    "bwd_causal_sees_all": ("const int nseq = p->causal ? t + 1 : T;", "const int nseq = T;"),
    "bwd_interleaved_head_map": ("const int h = hk * G + g;", "const int h = g * p->Hk + hk;"),
    "bwd_unnormalised_weights": ("logit[n] /= Z; /* P_n */", "logit[n] /= Z * Z; /* P_n */"),
    "sampled_dk_unscaled": ("j->dk[i * d + c] += s * dS[kj] * qrow[c];", "j->dk[i * d + c] += dS[kj] * qrow[c];"),
    "sampled_depth_slot_shift": ("j->dvd[(i * L + l) * d + c] += P[nseq + l] * dorow[c];",
                                 "j->dvd[(i * L + l) * d + c] += P[nseq + l - (l > 0)] * dorow[c];"),
    "sampled_missing_row_correction": ("for (int n = 0; n < ncand; ++n) dS_out[n] = P_out[n] * (dS_out[n] - D);",
                                       "for (int n = 0; n < ncand; ++n) dS_out[n] = P_out[n] * dS_out[n];"),
    "kv_weight_transposed": ("orc_load(w, (size_t)n * Dm + m, kind)", "orc_load(w, (size_t)m * 2 * N + n, kind)"),
    "kv_halves_swapped": ("double* dst = n < N ? k_out : v_out;", "double* dst = n < N ? v_out : k_out;"),
}

ALL_PINS = [
    lambda: pins.pin_sdpa(2, 13, 4, 2, 8, 3, True, 101),
    lambda: pins.pin_sdpa(1, 9, 2, 1, 8, 2, False, 102),
    lambda: pins.pin_l0_is_gqa(2, 17, 4, 2, 16, True, 103),
    pins.pin_worked_example,
    lambda: pins.pin_t1_closed_form(104),
    lambda: pins.pin_t1_depth(105),
    lambda: pins.pin_head_expansion(106),
    lambda: pins.pin_convex_and_permutation(107),
    lambda: pins.pin_merge_identity(108),
    lambda: pins.pin_depth_aligned(109),
    lambda: pins.pin_bwd_autograd(2, 9, 4, 2, 8, 3, True, 110),
    lambda: pins.pin_bwd_l0_gqa(1, 11, 4, 2, 8, True, 111),
    lambda: pins.pin_bwd_finite_difference(112),
    lambda: pins.pin_bwd_invariants(113),
    lambda: pins.pin_bwd_sampled(114),
    lambda: pins.pin_bwd_sampled(115, causal=False),
    lambda: pins.pin_kv_project(116),
]


def _build_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site for %s not found exactly once" % name
    path = tmp_path / ("mutant_%s.c" % name)
    path.write_text(src.replace(old, new))
    lib = tmp_path / ("mutant_%s.so" % name)
    subprocess.run(["gcc", "-O1", "-shared", "-fPIC", "-o", str(lib), str(path), "-lm", "-lpthread"], check=True)
    return str(lib)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(tmp_path, monkeypatch, name):
    good = orc._load()
    mutant = ctypes.CDLL(_build_mutant(tmp_path, name))
    for fn in ("moda_oracle_fwd", "moda_oracle_fwd_rows", "moda_oracle_bwd", "moda_oracle_bwd_sampled",
               "moda_oracle_kv_project", "moda_oracle_pack_depth", "moda_oracle_append_depth_slot"):
        getattr(mutant, fn).argtypes = getattr(good, fn).argtypes
        getattr(mutant, fn).restype = getattr(good, fn).restype
    monkeypatch.setattr(orc, "_lib", mutant)
    failures = []
    for pin in ALL_PINS:
        try:
            pin()
        except AssertionError as e:
            failures.append(str(e))
    assert failures, "no pin caught the planted mistake %s" % name


def test_unmutated_source_passes_every_pin():
    for pin in ALL_PINS:
        pin()

"""Mutation tests of the oracle's pins: each test plants one plausible mistake in a
copy of the oracle's C source (on the CPU, in a temporary directory), builds it,
and checks that at least one pin rejects the planted mistake."""
import functools
import os
import subprocess
import tempfile

import pytest

import oracle
from oracle.oracle import load
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

DECAY = """            for (int64_t c = 0; c < dk; ++c) {
                const double d = exp(gt[c]);
                for (int64_t e = 0; e < dv; ++e) S[c * dv + e] *= d;
            }
"""
WRITE = """            for (int64_t c = 0; c < dk; ++c)
                for (int64_t e = 0; e < dv; ++e)
                    S[c * dv + e] += kt[c] * (bt * vt[e] - at * kS[e]);
"""

MUTANTS = {
    "erase_sign": [("(bt * vt[e] - at * kS[e])", "(bt * vt[e] + at * kS[e])")],
    "alpha_beta_swapped": [("(bt * vt[e] - at * kS[e])", "(at * vt[e] - bt * kS[e])")],
    "scale_dropped": [("ot[e] = scale * acc;", "ot[e] = acc;")],
    "decay_dropped": [("const double d = exp(gt[c]);", "const double d = 1.0;")],
    "decay_after_write": [(DECAY, ""), (WRITE, WRITE + DECAY)],
    "gva_interleaved": [("hq = hv / group;\n        double* S", "hq = hv % Hq;\n        double* S")],
    "gate_of_previous_token": [("const double* gt = g + (t * Hv + hv) * dk;",
                                "const double* gt = g + ((t > cu[n] ? t - 1 : t) * Hv + hv) * dk;")],
    "output_reads_key": [("acc += S[c * dv + e] * qt[c];", "acc += S[c * dv + e] * kt[c];")],
    "initial_state_ignored": [("        if (h0)\n            memcpy(S,", "        if (0)\n            memcpy(S,")],
    "last_token_dropped": [("for (int64_t t = cu[n]; t < cu[n + 1]; ++t)",
                            "for (int64_t t = cu[n]; t + 1 < cu[n + 1]; ++t)")],
    "chunk_inverse_sign": [("acc -= Akk[i * C + m] * T[m * C + j];", "acc += Akk[i * C + m] * T[m * C + j];")],
    "chunk_decay_anchor": [("const double glast = G[(L - 1) * dk + c];", "const double glast = G[c];")],
    "chunk_aqk_strict": [("Aqk[i * C + j] = (j <= i) ? scale * sq : 0.0;", "Aqk[i * C + j] = (j < i) ? scale * sq : 0.0;")],
    "chunk_akk_with_diag": [("Akk[i * C + j] = (j < i) ? BETA(i) * sk : 0.0;",
                             "Akk[i * C + j] = (j <= i) ? BETA(i) * sk : 0.0;")],
}

PINS = [
    (lambda r, c: pins.pin_p1a_beta_zero(r), 1e-13),
    (lambda r, c: pins.pin_p1b_erase_off(r), 1e-12),
    (lambda r, c: pins.pin_p2_unit_key_write(r, one_hot=True), 4e-15),
    (lambda r, c: pins.pin_p2_unit_key_write(r, one_hot=False), 1e-12),
    (lambda r, c: pins.pin_p3_chunked_vs_recurrence(r, c), 1e-10),
    (lambda r, c: pins.pin_p4_chunk_size_invariance(c), 1e-10),
    (lambda r, c: pins.pin_p5_single_step(r), 1e-14),
    (lambda r, c: pins.pin_p7_split_resume(r), 1e-12),
    (lambda r, c: pins.pin_p10_key_value_memory(r), 1e-14),
    (lambda r, c: pins.pin_chunk_intermediates(r, c), 1e-12),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    src = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert old in src, f"mutation anchor for {name} not found"
        src = src.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as d:
        c_path, so_path = os.path.join(d, "m.c"), os.path.join(d, "m.so")
        open(c_path, "w").write(src)
        subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", so_path, c_path, "-lm"],
                       check=True)
        lib = load(so_path)
        rec = functools.partial(oracle.recurrence, lib=lib)
        chk = functools.partial(oracle.chunked, lib=lib)
        caught = []
        for i, (pin, bound) in enumerate(PINS):
            try:
                err = pin(rec, chk)
            except Exception:  # a crash or a rejected input also counts as caught
                err = float("inf")
            if not err <= bound:
                caught.append(i)
        assert caught, f"no pin caught the planted mistake {name}"


# The optional QG output (kda_oracle_qg) against its own pins.
QG_MUTANTS = {
    "qg_no_chunk_restart": [("if ((t - cu[n]) % C == 0) G = 0.0;", "if (t == cu[n]) G = 0.0;")],
    "qg_chunks_on_the_packed_grid": [("if ((t - cu[n]) % C == 0) G = 0.0;", "if (t % C == 0 || t == cu[n]) G = 0.0;")],
    "qg_exclusive_cumsum": [("G += g[(t * Hv + hv) * dk + c];\n                    qg[(t * Hv + hv) * dk + c] = "
                             "q[(t * Hq + hq) * dk + c] * exp(G);",
                             "qg[(t * Hv + hv) * dk + c] = q[(t * Hq + hq) * dk + c] * exp(G);\n"
                             "                    G += g[(t * Hv + hv) * dk + c];")],
    "qg_gva_interleaved": [("const int64_t hq = hv / group;\n                double G", "const int64_t hq = hv % Hq;\n"
                            "                double G")],
    "qg_gate_dropped": [("* exp(G);\n", "* 1.0;\n")],
}

QG_PINS = [
    (lambda f, c: pins.pin_qg_zero_gate(f), 0.0),
    (lambda f, c: pins.pin_qg_constant_gate(f), 1e-14),
    (lambda f, c: pins.pin_qg_matches_chunked_G(f, c), 1e-13),
]


@pytest.mark.parametrize("name", sorted(QG_MUTANTS))
def test_planted_qg_mistake_is_caught(name):
    src = open(SRC).read()
    for old, new in QG_MUTANTS[name]:
        assert old in src, f"mutation anchor for {name} not found"
        src = src.replace(old, new, 1)
    with tempfile.TemporaryDirectory() as d:
        c_path, so_path = os.path.join(d, "m.c"), os.path.join(d, "m.so")
        open(c_path, "w").write(src)
        subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", so_path, c_path, "-lm"],
                       check=True)
        lib = load(so_path)
        qg_fn = functools.partial(oracle.qg, lib=lib)
        chk = functools.partial(oracle.chunked, lib=lib)
        caught = []
        for i, (pin, bound) in enumerate(QG_PINS):
            try:
                err = pin(qg_fn, chk)
            except Exception:  # a crash or a rejected input also counts as caught
                err = float("inf")
            if not err <= bound:
                caught.append(i)
        assert caught, f"no pin caught the planted QG mistake {name}"

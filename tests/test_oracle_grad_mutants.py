"""Mutation tests of the gradient oracle's pins: each test plants one plausible
mistake in a copy of oracle/grad.py (on the CPU, compiled from its text into a
fresh module) and checks that the pin covering that function rejects it:
chunked_grads against the autograd gradients, forward against the C oracle."""
import os
import types

import numpy as np
import pytest

import oracle
from oracle import grad as og
from tests.pins import rand_case

SRC = open(os.path.join(os.path.dirname(og.__file__), "grad.py")).read()

CHUNKED = {
    "dgam_dropped": ('+ dgam * ops["gam"]', ""),
    "inverse_gradient_sign": ("dA = np.tril(-T.T @", "dA = np.tril(T.T @"),
    "dZ_untransposed": ('dZ = ops["Tb"].T @ dvn', 'dZ = ops["Tb"] @ dvn'),
    "dh_misses_output_term": ('+ ops["qg"].T @ dOc', ""),
    "cumsum_forward": ("np.cumsum(dG[::-1], axis=0)[::-1]", "np.cumsum(dG, axis=0)"),
    "kh_term_sign": ('- dkh * ops["kh"]', '+ dkh * ops["kh"]'),
    "dAqk_unmasked": ("dAqk = np.tril(dOc @ vn.T)", "dAqk = dOc @ vn.T"),
    "dbeta_misses_inverse_term": ("dbeta = np.sum(dTb * T, axis=0)", "dbeta = 0.0 * np.sum(dTb * T, axis=0)"),
    "gva_gradient_not_summed": ('out["dq"][b, s:e, hq] += dq_c', 'out["dq"][b, s:e, hq] = dq_c'),
}
FORWARD = {
    "erase_sign": ("S = S - bt * torch.outer(kt, kt @ S)", "S = S + bt * torch.outer(kt, kt @ S)"),
    "output_reads_key": ("scale * (S.T @ q[b, t, hq])", "scale * (S.T @ k[b, t, hq])"),
    "decay_on_columns": ("torch.exp(g[b, t, hv])[:, None] * S", "S * torch.exp(g[b, t, hv])[None, :dv]"),
}


def _mutant(old, new):
    assert SRC.count(old) == 1, old
    mod = types.ModuleType("grad_mutant")
    exec(compile(SRC.replace(old, new), "grad_mutant", "exec"), mod.__dict__)
    return mod


def _case():
    x = rand_case(1, 21, 1, 2, 5, 5, seed=51)
    rng = np.random.default_rng(52)
    return x, rng.standard_normal((1, 21, 2, 5)), rng.standard_normal((1, 2, 5, 5))


@pytest.mark.parametrize("name", sorted(CHUNKED))
def test_chunked_pin_rejects(name):
    x, do, dhT = _case()
    ref = og.grads(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.4, x["h0"], do, dhT)
    got = _mutant(*CHUNKED[name]).chunked_grads(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.4, x["h0"], do, dhT,
                                                chunk=8)
    worst = max(np.max(np.abs(got[n] - ref[n])) / np.max(np.abs(ref[n])) for n in ref)
    assert worst > 1e-6, (name, worst)   # the pin's bar is 1e-12


def test_chunked_pin_rejects_gva_mistake():
    # the group-sum mistake needs grouped heads to show
    x = rand_case(1, 21, 1, 2, 5, 5, seed=53)
    rng = np.random.default_rng(54)
    do = rng.standard_normal((1, 21, 2, 5))
    ref = og.grads(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.4, x["h0"], do, None)
    got = _mutant(*CHUNKED["gva_gradient_not_summed"]).chunked_grads(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.4,
                                                                       x["h0"], do, None, chunk=8)
    assert np.max(np.abs(got["dq"] - ref["dq"])) > 1e-6


@pytest.mark.parametrize("name", sorted(FORWARD))
def test_forward_pin_rejects(name):
    x = rand_case(1, 9, 1, 1, 5, 5, seed=55)
    m = _mutant(*FORWARD[name])
    o, hT = m.forward(*(og._f64(x[n]) for n in ("q", "k", "v", "g", "beta")), 0.3, og._f64(x["h0"]))
    o_ref, h_ref = oracle.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.3, h0=x["h0"])
    assert max(np.max(np.abs(o.numpy() - o_ref)), np.max(np.abs(hT.numpy() - h_ref))) > 1e-6, name

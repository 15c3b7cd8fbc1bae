"""Pins of the fp64 gradient oracle (oracle/grad.py): its forward loop equals
the C oracle's recurrence, its gradients equal central finite differences for
every input, and two closed forms hold (beta = 0 leaves k and v without
gradient; the key-value memory case gives dq in closed form)."""
import numpy as np
import torch

import oracle
from oracle import grad as og
from tests.pins import rand_case


def _inputs(B, T, Hq, Hv, dk, dv, seed, h0=True):
    x = rand_case(B, T, Hq, Hv, dk, dv, seed, h0=h0)
    return {n: x[n] for n in ("q", "k", "v", "g", "beta", "h0")}


def test_forward_loop_equals_the_c_oracle():
    x = _inputs(2, 19, 1, 2, 6, 5, seed=41)
    o, hT = og.forward(*(og._f64(x[n]) for n in ("q", "k", "v", "g", "beta")), 0.3, og._f64(x["h0"]))
    o_ref, h_ref = oracle.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.3, h0=x["h0"])
    assert np.max(np.abs(o.numpy() - o_ref)) <= 1e-12 * max(1.0, np.max(np.abs(o_ref)))
    assert np.max(np.abs(hT.numpy() - h_ref)) <= 1e-12 * max(1.0, np.max(np.abs(h_ref)))


def test_gradients_equal_central_differences():
    B, T, Hq, Hv, dk, dv = 1, 4, 1, 2, 3, 2
    x = _inputs(B, T, Hq, Hv, dk, dv, seed=42)
    rng = np.random.default_rng(43)
    do = rng.standard_normal((B, T, Hv, dv))
    dhT = rng.standard_normal((B, Hv, dk, dv))
    scale = 0.7
    got = og.grads(x["q"], x["k"], x["v"], x["g"], x["beta"], scale, x["h0"], do, dhT)

    def loss(vals):
        o, hT = og.forward(*(og._f64(vals[n]) for n in ("q", "k", "v", "g", "beta")), scale, og._f64(vals["h0"]))
        return float((o.numpy() * do).sum() + (hT.numpy() * dhT).sum())

    eps = 1e-6
    for name in og.NAMES:
        base = np.array(x[name], dtype=np.float64)
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = dict(x), dict(x)
            a, b = base.copy(), base.copy()
            a[idx] += eps
            b[idx] -= eps
            plus[name], minus[name] = a, b
            fd[idx] = (loss(plus) - loss(minus)) / (2 * eps)
        err = np.max(np.abs(got["d" + name] - fd))
        assert err <= 1e-7, (name, err)


def test_beta_zero_leaves_k_and_v_without_gradient():
    # with beta = 0 the state only decays: k and v enter every term multiplied by beta
    x = _inputs(1, 7, 2, 4, 5, 3, seed=44)
    x["beta"] = np.zeros_like(np.asarray(x["beta"], dtype=np.float64))
    rng = np.random.default_rng(45)
    got = og.grads(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.5, x["h0"], rng.standard_normal((1, 7, 4, 3)),
                   rng.standard_normal((1, 4, 5, 3)))
    assert not np.any(got["dk"]) and not np.any(got["dv"])
    assert np.any(got["dq"]) and np.any(got["dbeta"]) and np.any(got["dg"])


def test_key_value_memory_gives_dq_in_closed_form():
    # g = 0, beta = 1, keys e_(t mod dk): every write replaces one key's row of S by v_t, so
    # dq_t[c] = scale * (v of the last write to key c) . do_t
    B, T, H, dk, dv = 1, 9, 1, 4, 3
    rng = np.random.default_rng(46)
    q = rng.standard_normal((B, T, H, dk))
    k = np.zeros((B, T, H, dk))
    for t in range(T):
        k[0, t, 0, t % dk] = 1.0
    v = rng.standard_normal((B, T, H, dv))
    do = rng.standard_normal((B, T, H, dv))
    got = og.grads(q, k, v, np.zeros((B, T, H, dk)), np.ones((B, T, H)), 0.8, None, do, None)
    expect = np.zeros((B, T, H, dk))
    mem = np.zeros((dk, dv))
    for t in range(T):
        mem[t % dk] = v[0, t, 0]
        expect[0, t, 0] = 0.8 * (mem @ do[0, t, 0])
    assert np.max(np.abs(got["dq"] - expect)) <= 1e-14


def test_no_initial_state_and_gradient_terms_may_be_absent():
    x = _inputs(1, 5, 1, 1, 3, 2, seed=47, h0=False)
    rng = np.random.default_rng(48)
    do = rng.standard_normal((1, 5, 1, 2))
    g1 = og.grads(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.6, None, do, None)
    assert g1["dh0"] is None
    g2 = og.grads(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.6, None, do, np.zeros((1, 1, 3, 2)))
    for n in ("dq", "dk", "dv", "dg", "dbeta"):              # a zero dhT adds only zero terms
        assert np.max(np.abs(g1[n] - g2[n])) <= 1e-14
    assert torch.is_grad_enabled()


def test_chunked_backward_equals_autograd():
    # several chunks, a ragged tail, grouped value heads (q/k gradients summed over the group)
    x = _inputs(2, 21, 2, 4, 5, 3, seed=49)
    rng = np.random.default_rng(50)
    do = rng.standard_normal((2, 21, 4, 3))
    dhT = rng.standard_normal((2, 4, 5, 3))
    ref = og.grads(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.45, x["h0"], do, dhT)
    for chunk in (1, 4, 8, 64):
        got = og.chunked_grads(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.45, x["h0"], do, dhT, chunk=chunk)
        for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
            err = np.max(np.abs(got[n] - ref[n])) / np.max(np.abs(ref[n]))
            assert err <= 1e-12, (chunk, n, err)

"""Pins of the CPU oracle: special cases, closed forms and invariants that fix what
the KDA recurrence computes independently of the oracle's own code.

Each pin returns the largest error it finds; the tests assert the bounds, and the
mutation tests check that planted mistakes in the oracle break at least one pin.
Every pin takes the oracle's `recurrence` (and, where used, `chunked`) so that
another build of the oracle can be checked with the same code.

Recurrence being pinned (per sequence and value head):
    S_t = (I - alpha_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T,
    o_t = scale * S_t^T q_t,   alpha = beta for KDA.
dk != dv in most cases so that a transposed state or operand cannot pass.
"""
import numpy as np


def log_sigmoid(x):
    return -np.logaddexp(0.0, -x)


def rand_case(B, T, Hq, Hv, dk, dv, seed, h0=True, N=None, g_shift=3.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, Hq, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, T, Hq, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, Hv, dv))
    g = log_sigmoid(rng.standard_normal((B, T, Hv, dk)) + g_shift)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, Hv))))
    n = B if N is None else N
    s0 = 0.1 * rng.standard_normal((n, Hv, dk, dv)) if h0 else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=s0)


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def pin_p1a_beta_zero(rec, seed=1):
    """beta = 0 (so alpha = 0 too): no write and no erase, the state only decays.
    Closed form: o_t = scale (q_t * exp(G_t))^T S_0, S_T = Diag(exp G_T) S_0, with
    G the inclusive cumsum of g from the sequence start."""
    B, T, Hq, Hv, dk, dv = 2, 37, 2, 4, 12, 10
    x = rand_case(B, T, Hq, Hv, dk, dv, seed)
    x["beta"] = np.zeros_like(x["beta"])
    scale = 0.3
    o, hT = rec(x["q"], x["k"], x["v"], x["g"], x["beta"], scale, h0=x["h0"])
    G = np.cumsum(x["g"], axis=1)                       # [B,T,Hv,dk]
    qr = np.repeat(x["q"], Hv // Hq, axis=2)            # value head hv reads q head hv // group
    o_ref = scale * np.einsum("btvc,bvce->btve", qr * np.exp(G), x["h0"])
    h_ref = np.exp(G[:, -1])[..., None] * x["h0"]
    return max(_rel(o, o_ref), _rel(hT, h_ref))


def pin_p1b_erase_off(rec, seed=2):
    """alpha = 0, beta != 0: the recurrence becomes gated linear attention with
    values beta_s v_s, evaluated here by brute force in O(T^2):
    o_t = scale [ (q_t e^{G_t})^T S_0 + sum_{s<=t} (sum_c q_t,c k_s,c e^{G_t,c - G_s,c}) beta_s v_s ]."""
    B, T, Hq, Hv, dk, dv = 1, 41, 1, 3, 9, 7
    x = rand_case(B, T, Hq, Hv, dk, dv, seed)
    scale = 0.7
    o, hT = rec(x["q"], x["k"], x["v"], x["g"], x["beta"], scale, h0=x["h0"], alpha=np.zeros_like(x["beta"]))
    err = 0.0
    for hv in range(Hv):
        q = x["q"][0, :, hv // (Hv // Hq)]
        k = x["k"][0, :, hv // (Hv // Hq)]
        G = np.cumsum(x["g"][0, :, hv], axis=0)         # [T,dk]
        bv = x["beta"][0, :, hv, None] * x["v"][0, :, hv]
        S0 = x["h0"][0, hv]
        o_ref = np.zeros((T, dv))
        for t in range(T):
            acc = (q[t] * np.exp(G[t])) @ S0
            for s in range(t + 1):
                acc = acc + np.sum(q[t] * k[s] * np.exp(G[t] - G[s])) * bv[s]
            o_ref[t] = scale * acc
        h_ref = np.exp(G[-1])[:, None] * S0
        for s in range(T):
            h_ref = h_ref + np.outer(k[s] * np.exp(G[-1] - G[s]), bv[s])
        err = max(err, _rel(o[0, :, hv], o_ref), _rel(hT[0, hv], h_ref))
    return err


def pin_p2_unit_key_write(rec, one_hot, seed=3):
    """g = 0, beta = 1, |k_t| = 1: after step t the state maps k_t to v_t
    (S_t^T k_t = v_t).  With q_t = k_t and scale 1 the output is o_t = v_t."""
    B, T, H, dk, dv = 1, 29, 2, 8, 6
    rng = np.random.default_rng(seed)
    if one_hot:
        k = np.zeros((B, T, H, dk))
        idx = rng.integers(0, dk, size=(B, T, H))
        for t in range(T):
            for h in range(H):
                k[0, t, h, idx[0, t, h]] = 1.0
    else:
        k = rng.standard_normal((B, T, H, dk))
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = np.zeros((B, T, H, dk))
    beta = np.ones((B, T, H))
    h0 = rng.standard_normal((B, H, dk, dv))
    o, _ = rec(k, k, v, g, beta, 1.0, h0=h0)
    return float(np.max(np.abs(o - v)))


def pin_p3_chunked_vs_recurrence(rec, chk, seed=4):
    """The chunked form (a different algorithm, derived from the recurrence) agrees
    with the token recurrence on tiny inputs with tails, GVA and a nonzero S_0."""
    err = 0.0
    for T in (1, 63, 64, 65, 192):
        x = rand_case(1, T, 2, 4, 16, 12, seed + T)
        a = rec(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.25, h0=x["h0"])
        b = chk(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.25, h0=x["h0"], chunk=64)
        err = max(err, float(np.max(np.abs(a[0] - b[0]))), float(np.max(np.abs(a[1] - b[1]))))
    return err


def pin_p4_chunk_size_invariance(chk, seed=5):
    """The chunked form gives the same result for chunk sizes 1, 7, 16 and 64."""
    x = rand_case(1, 100, 1, 2, 8, 8, seed)
    ref = chk(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.5, h0=x["h0"], chunk=1)
    err = 0.0
    for C in (7, 16, 64):
        o, h = chk(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.5, h0=x["h0"], chunk=C)
        err = max(err, float(np.max(np.abs(o - ref[0]))), float(np.max(np.abs(h - ref[1]))))
    return err


def pin_p5_single_step(rec, seed=6):
    """T = 1: S_1 = (I - beta k k^T) Diag(exp g) S_0 + beta k v^T, o = scale S_1^T q
    (decay before the delta-rule read)."""
    x = rand_case(1, 1, 1, 1, 10, 7, seed)
    q, k, v, g, b, S0 = (x["q"][0, 0, 0], x["k"][0, 0, 0], x["v"][0, 0, 0], x["g"][0, 0, 0],
                         x["beta"][0, 0, 0], x["h0"][0, 0])
    S1 = (np.eye(10) - b * np.outer(k, k)) @ (np.diag(np.exp(g)) @ S0) + b * np.outer(k, v)
    o_ref = 0.9 * S1.T @ q
    o, hT = rec(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.9, h0=x["h0"])
    return max(_rel(o[0, 0, 0], o_ref), _rel(hT[0, 0], S1))


def pin_p6_affine_in_state(rec, seed=7):
    """The outputs are affine in S_0: o(a + b) - o(0) = [o(a) - o(0)] + [o(b) - o(0)]."""
    x = rand_case(1, 33, 1, 2, 6, 5, seed)
    rng = np.random.default_rng(seed + 100)
    a = rng.standard_normal(x["h0"].shape)
    b = rng.standard_normal(x["h0"].shape)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], 0.4)
    o0, h0 = rec(*args, h0=np.zeros_like(a))
    oa, ha = rec(*args, h0=a)
    ob, hb = rec(*args, h0=b)
    oab, hab = rec(*args, h0=a + b)
    return max(float(np.max(np.abs((oab - o0) - (oa - o0) - (ob - o0)))),
               float(np.max(np.abs((hab - h0) - (ha - h0) - (hb - h0)))))


def pin_p7_split_resume(rec, seed=8):
    """Running [0, T1) and then [T1, T) from the first run's final state equals one run."""
    x = rand_case(1, 90, 2, 2, 8, 6, seed)
    full_o, full_h = rec(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.3, h0=x["h0"])
    T1 = 37
    sl = lambda a, s: a[:, s]  # noqa: E731
    o1, h1 = rec(*(sl(x[n], slice(0, T1)) for n in ("q", "k", "v", "g", "beta")), 0.3, h0=x["h0"])
    o2, h2 = rec(*(sl(x[n], slice(T1, None)) for n in ("q", "k", "v", "g", "beta")), 0.3, h0=h1)
    return max(float(np.max(np.abs(np.concatenate([o1, o2], axis=1) - full_o))),
               float(np.max(np.abs(h2 - full_h))))


def pin_p8_varlen_is_independent(rec, seed=9):
    """A packed batch equals separate runs of its sequences (bit for bit)."""
    lens = [5, 1, 17, 0, 9]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = rand_case(1, int(cu[-1]), 2, 4, 6, 5, seed, N=len(lens))
    o, hT = rec(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.6, cu_seqlens=cu, h0=x["h0"])
    err = 0.0
    for n, L in enumerate(lens):
        s = slice(int(cu[n]), int(cu[n + 1]))
        on, hn = rec(*(x[m][:, s] for m in ("q", "k", "v", "g", "beta")), 0.6, h0=x["h0"][n:n + 1])
        err = max(err, float(np.max(np.abs(hn - hT[n:n + 1]))))
        if L:
            err = max(err, float(np.max(np.abs(on - o[:, s]))))
    return err


def pin_p9_gva_is_repeated_mha(rec, seed=10):
    """Grouped values (Hq | Hv) equal MHA with q, k repeated over each group of
    Hv / Hq consecutive value heads (bit for bit)."""
    x = rand_case(2, 20, 2, 6, 7, 5, seed)
    o, hT = rec(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.5, h0=x["h0"])
    qr, kr = np.repeat(x["q"], 3, axis=2), np.repeat(x["k"], 3, axis=2)
    o2, h2 = rec(qr, kr, x["v"], x["g"], x["beta"], 0.5, h0=x["h0"])
    return max(float(np.max(np.abs(o - o2))), float(np.max(np.abs(hT - h2))))


def pin_p10_key_value_memory(rec, seed=11):
    """g = 0, beta = 1, k_t = e_{t mod dk}, S_0 = 0: the state is a key-value memory
    whose row c holds the last value written to key c, so
    o_t = scale * sum_c q_t,c * v_{last write to c at or before t}."""
    T, dk, dv = 23, 5, 4
    rng = np.random.default_rng(seed)
    k = np.zeros((1, T, 1, dk))
    for t in range(T):
        k[0, t, 0, t % dk] = 1.0
    q = rng.standard_normal((1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    o, _ = rec(q, k, v, np.zeros((1, T, 1, dk)), np.ones((1, T, 1)), 1.5)
    mem = np.zeros((dk, dv))
    err = 0.0
    for t in range(T):
        mem[t % dk] = v[0, t, 0]
        err = max(err, float(np.max(np.abs(o[0, t, 0] - 1.5 * q[0, t, 0] @ mem))))
    return err


def pin_chunk_intermediates(rec, chk, seed=12):
    """Properties of the chunked form's intermediates: G is the chunk-local cumsum
    of g; T (I + Akk) = I; the state entering each chunk equals the recurrence's
    state after the tokens before it."""
    C, T, dk, dv = 16, 40, 6, 5
    x = rand_case(1, T, 1, 1, dk, dv, seed)
    o, hT, im = chk(x["q"], x["k"], x["v"], x["g"], x["beta"], 0.5, h0=x["h0"], chunk=C, intermediates=True)
    err = 0.0
    g = x["g"][0, :, 0]
    for c0 in range(0, T, C):
        L = min(C, T - c0)
        err = max(err, float(np.max(np.abs(im["G"][c0:c0 + L, 0] - np.cumsum(g[c0:c0 + L], axis=0)))))
        Akk = im["Akk"][c0:c0 + L, 0, :L]
        Tm = im["T"][c0:c0 + L, 0, :L]
        err = max(err, float(np.max(np.abs(Tm @ (np.eye(L) + Akk) - np.eye(L)))))
        if c0:
            _, hpre = rec(*(x[m][:, :c0] for m in ("q", "k", "v", "g", "beta")), 0.5, h0=x["h0"])
            err = max(err, float(np.max(np.abs(im["h_c"][c0 // C, 0] - hpre[0, 0]))))
        else:
            err = max(err, float(np.max(np.abs(im["h_c"][0, 0] - x["h0"][0, 0]))))
    return err


# ---- the optional QG output (q exp(G), G the chunk-local inclusive cumsum) ----

def pin_qg_zero_gate(qg_fn, seed=21):
    """g = 0: nothing decays, so QG is q itself; with grouped values, value head hv
    takes q/k head hv // (Hv / Hq)."""
    c = rand_case(1, 150, 2, 4, 48, 8, seed, h0=False)
    out = qg_fn(c["q"], np.zeros_like(c["g"]))
    return _rel(out, np.repeat(c["q"], 2, axis=2))


def pin_qg_constant_gate(qg_fn, seed=22):
    """g constant per (value head, channel): token i of a chunk (counted from the
    chunk's first token) has G = (i + 1) g, so QG = q exp((i + 1) g), and chunks
    start every 64 tokens from each sequence's own first token (packed lengths
    that put sequence starts off the 64-token grid, an empty sequence, tails)."""
    lens = [0, 5, 64, 130, 1, 70]
    T = sum(lens)
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, T, 2, 48))
    gc = -rng.uniform(0.0, 0.3, size=(4, 48))
    g = np.broadcast_to(gc, (1, T, 4, 48)).copy()
    cu = np.cumsum([0] + lens)
    out = qg_fn(q, g, cu_seqlens=cu, chunk=64)
    want = np.zeros_like(out)
    for n in range(len(lens)):
        for t in range(cu[n], cu[n + 1]):
            i = (t - cu[n]) % 64
            want[0, t] = np.repeat(q[0, t], 2, axis=0) * np.exp((i + 1) * gc)
    return _rel(out, want)


def pin_qg_matches_chunked_G(qg_fn, chk, seed=23):
    """QG equals q exp(G) with the G that the chunked evaluation of the recurrence
    (pinned above against the token recurrence) reports as its intermediate."""
    c = rand_case(1, 200, 2, 4, 48, 8, seed, h0=False)
    cu = np.array([0, 70, 70, 200])
    _, _, inter = chk(c["q"], c["k"], c["v"], c["g"], c["beta"], 0.3, cu_seqlens=cu, chunk=64, intermediates=True)
    want = np.repeat(c["q"], 2, axis=2) * np.exp(inter["G"].reshape(c["g"].shape))
    return _rel(qg_fn(c["q"], c["g"], cu_seqlens=cu, chunk=64), want)

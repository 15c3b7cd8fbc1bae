"""fp64 gradients of the KDA recurrence (test infrastructure only).

Only the test suite may import this module.  The GPU library never imports it
and shares no code with it.

The pages list a backward pass among the library's KDA kernels ("cuLA
REPO_LAYOUT.md", the kda/ entries for chunk_bwd and the WY dq/dk/dg kernels) but
print no equation.  The gradients here are those of the token recurrence itself,

    S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
    o_t = scale * S_t^T q_t,

for a loss whose gradients with respect to o and to the final state are given
(do, dhT).  They come from reverse-mode automatic differentiation (torch.autograd,
a library primitive) through a plain fp64 loop over the tokens.  The loop's
forward is checked against the C oracle, and the gradients against central
finite differences and closed forms, in tests/test_oracle_grads.py.

Layout: fixed-length batches.  q, k [B, T, Hq, dk]; v [B, T, Hv, dv];
g [B, T, Hv, dk]; beta [B, T, Hv]; h0 [B, Hv, dk, dv] or None (zero state).
Value head hv reads q/k head hv // (Hv // Hq).
"""
import numpy as np
import torch

NAMES = ("q", "k", "v", "g", "beta", "h0")


def _f64(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).clone()
    return torch.from_numpy(np.array(x, dtype=np.float64))


def forward(q, k, v, g, beta, scale, h0=None):
    """The recurrence, token by token, on fp64 torch tensors (differentiable).
    Returns o [B, T, Hv, dv] and the final state [B, Hv, dk, dv]."""
    B, T, Hq, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    group = Hv // Hq
    o_rows, finals = [], []
    for b in range(B):
        o_heads, f_heads = [], []
        for hv in range(Hv):
            hq = hv // group
            S = h0[b, hv] if h0 is not None else torch.zeros(dk, dv, dtype=torch.float64)
            o_t = []
            for t in range(T):
                kt, bt = k[b, t, hq], beta[b, t, hv]
                S = torch.exp(g[b, t, hv])[:, None] * S                      # decay the rows (key channels)
                S = S - bt * torch.outer(kt, kt @ S) + bt * torch.outer(kt, v[b, t, hv])
                o_t.append(scale * (S.T @ q[b, t, hq]))
            o_heads.append(torch.stack(o_t) if T else torch.zeros(0, dv, dtype=torch.float64))
            f_heads.append(S)
        o_rows.append(torch.stack(o_heads, dim=1))
        finals.append(torch.stack(f_heads))
    return torch.stack(o_rows), torch.stack(finals)


def grads(q, k, v, g, beta, scale, h0=None, do=None, dhT=None):
    """Gradients of sum(o * do) + sum(hT * dhT) with respect to q, k, v, g, beta
    and h0 (None where h0 is None), as fp64 numpy arrays in the inputs' layouts.
    do or dhT may be None (that term is absent)."""
    x = {n: _f64(a) for n, a in zip(NAMES, (q, k, v, g, beta, h0))}
    for t in x.values():
        if t is not None:
            t.requires_grad_(True)
    o, hT = forward(x["q"], x["k"], x["v"], x["g"], x["beta"], float(scale), x["h0"])
    loss = torch.zeros((), dtype=torch.float64)
    if do is not None:
        loss = loss + (o * _f64(do)).sum()
    if dhT is not None:
        loss = loss + (hT * _f64(dhT)).sum()
    wrt = [x[n] for n in NAMES if x[n] is not None]
    got = torch.autograd.grad(loss, wrt, allow_unused=True)
    out, it = {}, iter(got)
    for n in NAMES:
        if x[n] is None:
            out["d" + n] = None
            continue
        gr = next(it)
        out["d" + n] = (gr if gr is not None else torch.zeros_like(x[n])).numpy()
    return out


def _chunk_operands(q, k, g, beta, scale):
    """The chunk's operands in the chunked form, for one (sequence, value head):
    q, k, g [C, dk] and beta [C].  G is the chunk-local inclusive cumsum of g."""
    G = np.cumsum(g, axis=0)
    D = np.exp(G[:, None, :] - G[None, :, :])              # D[i, j, c] = exp(G_i - G_j)
    Aqk = np.tril(scale * np.einsum("ic,jc,ijc->ij", q, k, D))
    Abar = np.tril(np.einsum("ic,jc,ijc->ij", k, k, D), -1)
    T = np.linalg.inv(np.eye(len(beta)) + beta[:, None] * Abar)
    return dict(G=G, D=D, Aqk=Aqk, Abar=Abar, T=T, Tb=T * beta[None, :], kg=k * np.exp(G),
                qg=scale * q * np.exp(G), kh=k * np.exp(G[-1] - G), gam=np.exp(G[-1]))


def chunked_grads(q, k, v, g, beta, scale, h0=None, do=None, dhT=None, chunk=64):
    """The same gradients as grads(), evaluated through the chunked form instead of
    autograd: a forward pass keeps each chunk's entering state h, then a reverse
    pass over the chunks applies, per chunk,

        Z = v - kg h,  v_new = Tb Z,  o = qg h + Aqk v_new,  h' = gam * h + kh^T v_new
        dv_new = Aqk^T do + kh dh'      dZ = Tb^T dv_new      dv = dZ
        dh = gam * dh' + qg^T do - kg^T dZ
        d(qg) = do h^T   d(kg) = -dZ h^T   d(kh) = v_new dh'^T
        dAqk = lower(do v_new^T)   dTb = dv_new Z^T   dgam = rowsum(dh' * h)

    and takes the operand gradients back to q, k, beta and g through their
    definitions (the inverse, dA = -T^T dT T^T on the strict lower triangle, and
    the cumsum, dg = reverse cumsum of dG).  Inputs and outputs as grads()."""
    q, k, v, g, beta = (np.asarray(a, np.float64) for a in (q, k, v, g, beta))
    B, Tn, Hq, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    group = Hv // Hq
    do = np.zeros((B, Tn, Hv, dv)) if do is None else np.asarray(do, np.float64)
    dhT = np.zeros((B, Hv, dk, dv)) if dhT is None else np.asarray(dhT, np.float64)
    out = {n: np.zeros_like(a) for n, a in (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta))}
    out["dh0"] = None if h0 is None else np.zeros((B, Hv, dk, dv))
    bounds = [(s, min(s + chunk, Tn)) for s in range(0, Tn, chunk)]
    for b in range(B):
        for hv in range(Hv):
            hq = hv // group
            h = np.zeros((dk, dv)) if h0 is None else np.array(h0[b, hv], np.float64)
            saved = []
            for s, e in bounds:                                  # forward: keep h entering each chunk
                ops = _chunk_operands(q[b, s:e, hq], k[b, s:e, hq], g[b, s:e, hv], beta[b, s:e, hv], scale)
                Z = v[b, s:e, hv] - ops["kg"] @ h
                vn = ops["Tb"] @ Z
                saved.append((s, e, ops, h, Z, vn))
                h = ops["gam"][:, None] * h + ops["kh"].T @ vn
            dh = dhT[b, hv].copy()
            for s, e, ops, h, Z, vn in reversed(saved):
                qc, kc, bc, dOc = q[b, s:e, hq], k[b, s:e, hq], beta[b, s:e, hv], do[b, s:e, hv]
                dvn = ops["Aqk"].T @ dOc + ops["kh"] @ dh
                dZ = ops["Tb"].T @ dvn
                out["dv"][b, s:e, hv] += dZ
                dqg, dkg, dkh = dOc @ h.T, -dZ @ h.T, vn @ dh.T
                dAqk = np.tril(dOc @ vn.T)
                dTb = dvn @ Z.T
                dgam = np.sum(dh * h, axis=1)
                dh = ops["gam"][:, None] * dh + ops["qg"].T @ dOc - ops["kg"].T @ dZ
                # Tb = T diag(beta), T = (I + diag(beta) Abar)^-1
                T, G, D = ops["T"], ops["G"], ops["D"]
                dbeta = np.sum(dTb * T, axis=0)
                dA = np.tril(-T.T @ (dTb * bc[None, :]) @ T.T, -1)          # gradient of diag(beta) Abar
                dbeta += np.sum(dA * ops["Abar"], axis=1)
                dAbar = bc[:, None] * dA
                # Aqk[i,j] = scale sum_c q_i k_j D_ijc;  Abar[i,j] = sum_c k_i k_j D_ijc
                Pq = scale * dAqk[:, :, None] * D                           # [i, j, c]
                Pk = dAbar[:, :, None] * D
                dq_c = np.einsum("ijc,jc->ic", Pq, kc)
                dk_c = np.einsum("ijc,ic->jc", Pq, qc) + np.einsum("ijc,jc->ic", Pk, kc) \
                    + np.einsum("ijc,ic->jc", Pk, kc)
                tq = Pq * qc[:, None, :] * kc[None, :, :]
                tk = Pk * kc[:, None, :] * kc[None, :, :]
                dG = tq.sum(1) - tq.sum(0) + tk.sum(1) - tk.sum(0)
                # kg = k e^G, qg = scale q e^G, kh = k e^(G_last - G), gam = e^G_last
                eG = np.exp(G)
                dq_c += scale * dqg * eG
                dk_c += dkg * eG + dkh * np.exp(G[-1] - G)
                dG += dkg * ops["kg"] + dqg * ops["qg"] - dkh * ops["kh"]
                dG[-1] += np.sum(dkh * ops["kh"], axis=0) + dgam * ops["gam"]
                out["dq"][b, s:e, hq] += dq_c
                out["dk"][b, s:e, hq] += dk_c
                out["dbeta"][b, s:e, hv] += dbeta
                out["dg"][b, s:e, hv] += np.cumsum(dG[::-1], axis=0)[::-1]
            if h0 is not None:
                out["dh0"][b, hv] = dh
    return out

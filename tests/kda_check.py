"""Shared helpers of the GPU parity tests: tolerance checks and oracle subsets.

Tolerances (stated for this library; the pages give none): output o per
(sequence, value head) relative Frobenius error <= 3e-3 and global max-abs
error <= 2e-2; final state per (sequence, value head) relative Frobenius error
<= 1e-3.  Both sides see the same bf16/fp32 input bits; the oracle computes in
fp64.
"""
import numpy as np
import torch

O_REL_F = 3e-3
O_MAX_ABS = 2e-2
STATE_REL_F = 1e-3


def rel_frob_per_head(got, ref, seq_slices=None):
    """Max over (sequence, head) of ||got - ref||_F / ||ref||_F.
    got/ref: o as [B, T, H, D] (per batch row and head) or, with `seq_slices`, a
    packed [1, Ttot, H, D] split into the given token slices."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    worst = 0.0
    blocks = []
    if seq_slices is None:
        for b in range(got.shape[0]):
            blocks.append((got[b], ref[b]))
    else:
        for s in seq_slices:
            if s.stop > s.start:
                blocks.append((got[0, s], ref[0, s]))
    for gb, rb in blocks:
        for h in range(gb.shape[1]):
            num = np.linalg.norm(gb[:, h] - rb[:, h])
            den = np.linalg.norm(rb[:, h])
            worst = max(worst, num / den if den > 0 else num)
    return worst


def state_rel_frob(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    worst = 0.0
    for n in range(got.shape[0]):
        for h in range(got.shape[1]):
            num = np.linalg.norm(got[n, h] - ref[n, h])
            den = np.linalg.norm(ref[n, h])
            worst = max(worst, num / den if den > 0 else num)
    return worst


def head_subset(x, heads, Hq, Hv):
    """Inputs restricted to value heads `heads` (and the q/k head each one reads),
    as an MHA problem with len(heads) heads."""
    group = Hv // Hq
    qk_idx = [h // group for h in heads]
    sub = dict(q=x["q"][:, :, qk_idx], k=x["k"][:, :, qk_idx], v=x["v"][:, :, heads],
               g=x["g"][:, :, heads], beta=x["beta"][:, :, heads])
    sub["h0"] = x["h0"][:, heads] if x.get("h0") is not None else None
    return sub


def to_device(x, device="cuda"):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def seq_slices(cu):
    cu = [int(c) for c in cu]
    return [slice(cu[i], cu[i + 1]) for i in range(len(cu) - 1)]

"""Seeded synthetic inputs for the KDA forward pass.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic, and both the GPU library's tests and the CPU oracle's tests
use it so that both sides see the same bits.

Workloads (the pages, "cuLA PR #131", section Performance, time B=2 H=64 at
T in {512, 1024, 4096, 8192} with bf16 or fp32 beta, and a grouped-value case
B=1 Hq=16 Hv=64 T=4096; the value distributions and the other shapes below are
this library's stated synthetic recipe, since the pages give none):

  q, k  ~ N(0, 1), L2-normalised over the head dimension, stored bf16
  v     ~ N(0, 1), stored bf16
  g     = logsigmoid(N(0, 1) + 3), fp32 log-decay (all <= 0)
  beta  = sigmoid(N(0, 1)), bf16 or fp32
  h0    = 0.1 * N(0, 1), fp32 (only where a workload has an initial state)

All tensors come from one CPU torch.Generator, drawn in the order q, k, v, g,
beta, h0.  Packed variable-length lengths come from their own generator.
"""
from dataclasses import dataclass
from typing import List, Optional

import torch
import torch.nn.functional as F

D = 128        # head dimension (dk = dv)
CHUNK = 64     # chunk length of the chunked method


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    Hq: int
    Hv: int
    beta_dtype: torch.dtype
    has_h0: bool
    varlen_total: int = 0        # >0: packed variable-length batch of this many tokens
    seed: int = 0
    length_seed: int = 7
    lengths: tuple = ()          # a packed batch of these sequence lengths (instead of drawn ones)

    @property
    def scale(self) -> float:
        return 1.0 / (D ** 0.5)


WORKLOADS = {
    "tiny_b1_h2_t192": Workload("tiny_b1_h2_t192", 1, 192, 2, 2, torch.float32, False),
    "mha_b2_h64_t4096": Workload("mha_b2_h64_t4096", 2, 4096, 64, 64, torch.bfloat16, False),
    "mha_b2_h64_t8192": Workload("mha_b2_h64_t8192", 2, 8192, 64, 64, torch.float32, True),
    "mha_b2_h64_t512": Workload("mha_b2_h64_t512", 2, 512, 64, 64, torch.float32, True),
    "mha_b2_h64_t1024": Workload("mha_b2_h64_t1024", 2, 1024, 64, 64, torch.float32, True),
    "mha_b2_h64_t4096_h0": Workload("mha_b2_h64_t4096_h0", 2, 4096, 64, 64, torch.float32, True),
    "gva_b1_hq16_hv64_t4096": Workload("gva_b1_hq16_hv64_t4096", 1, 4096, 16, 64, torch.bfloat16, False),
    "varlen_h64_16k": Workload("varlen_h64_16k", 1, 16384, 64, 64, torch.float32, False, varlen_total=16384),
    # few heads per GPU: one long sequence, and the headline batch's share of one GPU
    # under 8-way head sharding (the segmented forward's workloads)
    "mha_b1_h8_t65536": Workload("mha_b1_h8_t65536", 1, 65536, 8, 8, torch.float32, True),
    "mha_b2_h8_t8192": Workload("mha_b2_h8_t8192", 2, 8192, 8, 8, torch.float32, True),
    # a packed batch with one long sequence among short ones, few heads (the
    # segmented forward on packed sequences)
    "packed_h8_long": Workload("packed_h8_long", 1, 65536 + 3000 + 100 + 7, 8, 8, torch.float32, True,
                               lengths=(3000, 65536, 100, 7)),
}


def varlen_lengths(total: int, seed: int = 7, forced=(1, 63, 65), hi: int = 4096) -> List[int]:
    """Sequence lengths: the forced lengths first, then uniform draws in [1, hi]
    from their own generator until the sum reaches `total`; the last draw is cut
    so that the lengths sum to exactly `total`."""
    gen = torch.Generator("cpu").manual_seed(seed)
    lens = list(forced)
    while sum(lens) < total:
        lens.append(int(torch.randint(1, hi + 1, (1,), generator=gen).item()))
    lens[-1] -= sum(lens) - total
    return [x for x in lens if x > 0]


def cu_from_lengths(lens) -> torch.Tensor:
    cu = [0]
    for x in lens:
        cu.append(cu[-1] + int(x))
    return torch.tensor(cu, dtype=torch.int32)


def make_inputs(B: int, T: int, Hq: int, Hv: int, beta_dtype=torch.float32, h0: bool = False,
                N: Optional[int] = None, seed: int = 0, dk: int = D, dv: int = D,
                g_shift: float = 3.0, g_scale: float = 1.0):
    """Draws one input set.  N is the number of sequences (B unless packed)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    q = F.normalize(torch.randn(B, T, Hq, dk, generator=gen), dim=-1).to(torch.bfloat16)
    k = F.normalize(torch.randn(B, T, Hq, dk, generator=gen), dim=-1).to(torch.bfloat16)
    v = torch.randn(B, T, Hv, dv, generator=gen).to(torch.bfloat16)
    g = F.logsigmoid(g_scale * torch.randn(B, T, Hv, dk, generator=gen) + g_shift)
    beta = torch.sigmoid(torch.randn(B, T, Hv, generator=gen)).to(beta_dtype)
    n = B if N is None else N
    s0 = (torch.randn(n, Hv, dk, dv, generator=gen) * 0.1) if h0 else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, h0=s0)


def workload_inputs(w: Workload, T: Optional[int] = None):
    """Inputs for a named workload; returns (dict of tensors, cu_seqlens or None)."""
    if w.varlen_total or w.lengths:
        lens = list(w.lengths) if w.lengths else varlen_lengths(w.varlen_total, w.length_seed)
        cu = cu_from_lengths(lens)
        x = make_inputs(1, sum(lens), w.Hq, w.Hv, w.beta_dtype, w.has_h0, N=len(lens), seed=w.seed)
        return x, cu
    x = make_inputs(w.B, T or w.T, w.Hq, w.Hv, w.beta_dtype, w.has_h0, seed=w.seed)
    return x, None

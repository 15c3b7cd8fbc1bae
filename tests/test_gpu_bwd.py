"""GPU parity of the backward (kda_bwd, through the C ABI) against the fp64
chunk-form gradients of the oracle (oracle/grad.py), which are themselves pinned
to autograd and finite differences on the CPU.

Tolerance: the kernels work in fp32 throughout, so each gradient is a chain of a
few fp32 products of length at most 192 (128 channels plus 64 tokens); with unit
roundoff 6e-8 that bounds the relative error of each product near 1.2e-5, and a
chain of four of them near 5e-5.  The test asks for a relative Frobenius error of
at most 1e-4 per gradient and per value head.

Each test prints the case it is about to launch before touching the GPU.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_35_amd import kda_bwd, kda_bwd_workspace_size, load_library
from gated_delta_rule_35_amd.inputs import cu_from_lengths, make_inputs, varlen_lengths
from oracle import grad as og
from tests.kda_check import head_subset, seq_slices, to_device

pytestmark = pytest.mark.gpu

SCALE = 128 ** -0.5
TOL = 1e-4
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    load_library()  # fails loudly if the HIP library is not built
    yield


def _case(B, T, Hq, Hv, seed, h0=True, dhT=True, beta_dtype=torch.float32):
    x = make_inputs(B, T, Hq, Hv, beta_dtype, h0, seed=seed)
    gen = torch.Generator("cpu").manual_seed(seed + 1000)
    x["do"] = torch.randn(B, T, Hv, 128, generator=gen).to(torch.bfloat16)
    x["dhT"] = torch.randn(B, Hv, 128, 128, generator=gen) if dhT else None
    return x


def _gpu_grads(x, want_dh0=True, workspace=None):
    d = to_device(x)
    g = kda_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], SCALE, d["do"], initial_state=d["h0"],
                d_final_state=d["dhT"], d_initial_state=want_dh0, workspace=workspace)
    torch.cuda.synchronize()
    return {n: (None if t is None else t.cpu().numpy().astype(np.float64)) for n, t in g.items()}


def _f64(t):
    return None if t is None else t.float().numpy().astype(np.float64)


def _oracle(x):
    # with no initial state the gradient is still taken at the zero state
    B, Hv = x["v"].shape[0], x["v"].shape[2]
    h0 = _f64(x["h0"]) if x["h0"] is not None else np.zeros((B, Hv, 128, 128))
    return og.chunked_grads(_f64(x["q"]), _f64(x["k"]), _f64(x["v"]), _f64(x["g"]), _f64(x["beta"]), SCALE,
                            h0, _f64(x["do"]), _f64(x["dhT"]), chunk=64)


def _rel_per_head(a, b, head_axis):
    a, b = np.moveaxis(a, head_axis, 0), np.moveaxis(b, head_axis, 0)
    out = []
    for h in range(a.shape[0]):
        den = np.linalg.norm(b[h])
        out.append(np.linalg.norm(a[h] - b[h]) / den if den > 0 else np.linalg.norm(a[h]))
    return max(out) if out else 0.0


def _compare(got, ref, label):
    for n in NAMES:
        if ref[n] is None:
            assert got[n] is None, n
            continue
        axis = 1 if n == "dh0" else 2
        err = _rel_per_head(got[n], ref[n], axis)
        _say(f"{label} {n}: rel frob {err:.2e}")
        assert err <= TOL, (label, n, err)


@pytest.mark.parametrize("B,T,Hq,Hv,h0,dhT,beta_dtype", [
    (2, 150, 2, 4, True, True, torch.float32),      # several chunks, ragged tail, grouped value heads
    (1, 64, 1, 1, False, False, torch.bfloat16),    # one full chunk, zero state, bf16 beta
    (1, 1, 2, 2, True, True, torch.float32),        # a single token
    (3, 200, 4, 4, True, False, torch.float32),     # MHA, three rows
])
def test_bwd_matches_oracle(B, T, Hq, Hv, h0, dhT, beta_dtype):
    x = _case(B, T, Hq, Hv, seed=B * 1000 + T, h0=h0, dhT=dhT, beta_dtype=beta_dtype)
    _say(f"kda_bwd B={B} T={T} Hq={Hq} Hv={Hv} h0={h0} dhT={dhT} beta={beta_dtype}")
    got = _gpu_grads(x)
    _compare(got, _oracle(x), f"B{B} T{T}")
    # and against autograd through the token recurrence itself (no chunk structure)
    Bv, Hvv = x["v"].shape[0], x["v"].shape[2]
    h0 = x["h0"] if x["h0"] is not None else torch.zeros(Bv, Hvv, 128, 128)
    rec = og.grads(x["q"], x["k"], x["v"], x["g"], x["beta"], SCALE, h0, x["do"], x["dhT"])
    _compare(got, rec, f"B{B} T{T} vs recurrence")


def test_bwd_strong_decay():
    # g near -3 per token and channel: e^G underflows within a chunk, the regime where
    # the forward needs its exact diagonal path; a chunk decays by about e^-190, past
    # the e^-120 bound of the anchored MFMA products, so the decay-weighted sums are
    # taken element by element (every factor exp of a non-positive difference)
    x = make_inputs(2, 140, 2, 2, torch.float32, True, seed=9, g_shift=-3.0)
    gen = torch.Generator("cpu").manual_seed(1009)
    x["do"] = torch.randn(2, 140, 2, 128, generator=gen).to(torch.bfloat16)
    x["dhT"] = torch.randn(2, 2, 128, 128, generator=gen)
    _say("kda_bwd B=2 T=140 strong decay (g_shift -3)")
    got = _gpu_grads(x)
    for n in NAMES:
        assert np.isfinite(got[n]).all(), n
    _compare(got, _oracle(x), "strong decay")


def test_bwd_empty_sequence_passes_the_state_gradient_through():
    x = _case(2, 0, 1, 2, seed=5)
    _say("kda_bwd T=0")
    got = _gpu_grads(x)
    assert np.array_equal(got["dh0"], _f64(x["dhT"]))
    assert got["dq"].size == 0 and got["dbeta"].size == 0


def test_bwd_without_initial_state_gradient_and_with_caller_workspace():
    x = _case(1, 130, 2, 4, seed=6)
    need = kda_bwd_workspace_size(130, 1, 2, 4)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    _say("kda_bwd B=1 T=130 caller workspace, no dh0")
    a = _gpu_grads(x, want_dh0=False, workspace=ws)
    b = _gpu_grads(x, want_dh0=True)
    assert a["dh0"] is None
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        assert np.array_equal(a[n], b[n]), n          # same kernels, same order: bitwise equal


def test_bwd_is_reproducible():
    x = _case(2, 300, 2, 2, seed=7)
    _say("kda_bwd B=2 T=300 twice")
    a, b = _gpu_grads(x), _gpu_grads(x)
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), n


def test_bwd_full_size_sampled_heads():
    # the 2 x 8192 token, 64-head batch the forward is measured on, with its initial
    # state ~ 0.1 N(0, 1), a random final-state gradient and the initial-state
    # gradient: 128 chunks of carried state gradient; two heads checked
    B, T, H = 2, 8192, 64
    x = _case(B, T, H, H, seed=8, h0=True, dhT=True)
    _say(f"kda_bwd B={B} T={T} H={H} with h0, dhT and dh0")
    got = _gpu_grads(x, want_dh0=True)
    heads = [0, 37]
    sub = head_subset(x, heads, H, H)
    sub["do"] = x["do"][:, :, heads]
    sub["dhT"] = x["dhT"][:, heads]
    ref = _oracle(sub)
    for n in NAMES:
        axis = 1 if n == "dh0" else 2
        g = got[n][:, heads] if n == "dh0" else got[n][:, :, heads]
        err = _rel_per_head(g, ref[n], axis)
        _say(f"full size {n}: rel frob {err:.2e}")
        assert err <= TOL, (n, err)
        assert np.isfinite(got[n]).all(), n


def test_bwd_full_size_gva_group():
    # the 1 x 4096 token batch with 16 q/k heads and 64 value heads: the four value heads of
    # q/k head 5 checked; dq and dk of that head are the sums over its group
    from gated_delta_rule_35_amd.inputs import WORKLOADS, workload_inputs
    w = WORKLOADS["gva_b1_hq16_hv64_t4096"]
    x, _ = workload_inputs(w)
    gen = torch.Generator("cpu").manual_seed(1010)
    x["do"] = torch.randn(w.B, w.T, w.Hv, 128, generator=gen).to(torch.bfloat16)
    x["dhT"] = None
    _say(f"kda_bwd GVA B={w.B} T={w.T} Hq={w.Hq} Hv={w.Hv}")
    got = _gpu_grads(x, want_dh0=x["h0"] is not None)
    group = w.Hv // w.Hq
    hq = 5
    heads = list(range(hq * group, (hq + 1) * group))
    sub = head_subset(x, heads, w.Hq, w.Hv)
    sub["do"] = x["do"][:, :, heads]
    sub["dhT"] = None
    ref = _oracle(sub)
    for n in ("dv", "dg", "dbeta"):
        err = _rel_per_head(got[n][:, :, heads], ref[n], 2)
        _say(f"GVA {n}: rel frob {err:.2e}")
        assert err <= TOL, (n, err)
    for n in ("dq", "dk"):
        g = got[n][:, :, hq]
        r = ref[n].sum(axis=2)
        err = np.linalg.norm(g - r) / np.linalg.norm(r)
        _say(f"GVA {n} (group sum): rel frob {err:.2e}")
        assert err <= TOL, (n, err)


def test_bwd_padded_rows_equal_separate_sequences():
    # sequences of different lengths as equal-length rows: the tail of the shorter row is
    # padded with q = k = v = 0, g = 0, beta = 0 and zero output gradient, tokens that
    # neither decay nor write the state, so each row's gradients are its sequence's own
    T, lens = 100, (100, 37)
    x = _case(2, T, 2, 2, seed=11)
    for key in ("q", "k", "v", "g", "beta", "do"):
        x[key][1, lens[1]:] = 0
    _say("kda_bwd padded rows: lengths 100 and 37")
    got = _gpu_grads(x)
    for b, L in enumerate(lens):
        row = {k: (v[b:b + 1, :L] if k in ("q", "k", "v", "g", "beta", "do") else
                   (v[b:b + 1] if v is not None else None)) for k, v in x.items()}
        ref = _oracle(row)
        for n in NAMES:
            g = got[n][b:b + 1] if n == "dh0" else got[n][b:b + 1, :L]
            err = _rel_per_head(g, ref[n], 1 if n == "dh0" else 2)
            _say(f"row {b} (length {L}) {n}: rel frob {err:.2e}")
            assert err <= TOL, (b, n, err)
        if L < T:
            for n in ("dq", "dk", "dv", "dbeta"):
                assert not np.any(got[n][b, L:]), n   # pads get no gradient


@pytest.mark.parametrize("g_shift", [-1.25, -1.3, -1.65])
def test_bwd_decay_near_the_anchored_limit(g_shift):
    # chunk decays of e^-82 .. e^-119 per channel (g_shift -1.25: every chunk on the
    # anchored MFMA products, factors up to e^59), e^-87 .. e^-121 (-1.3: the first
    # chunk of a head past e^-120 on some channel, so element by element, the second
    # anchored) and e^-103 .. e^-140 (-1.65: element by element throughout)
    x = make_inputs(1, 140, 2, 2, torch.float32, True, seed=19, g_shift=g_shift)
    gen = torch.Generator("cpu").manual_seed(1019)
    x["do"] = torch.randn(1, 140, 2, 128, generator=gen).to(torch.bfloat16)
    x["dhT"] = torch.randn(1, 2, 128, 128, generator=gen)
    G_last = x["g"][0, :64].sum(0)
    _say(f"kda_bwd B=1 T=140 g_shift {g_shift}: first chunk's decay e^{G_last.min():.1f} .. e^{G_last.max():.1f}")
    got = _gpu_grads(x)
    for n in NAMES:
        assert np.isfinite(got[n]).all(), n
    _compare(got, _oracle(x), f"g_shift {g_shift}")


# ---- packed sequences (cu_seqlens) ----

def _packed_case(lens, Hq, Hv, seed, h0=True, dhT=True, beta_dtype=torch.float32, tail=0):
    """One row of sum(lens) + tail tokens holding len(lens) sequences back to back;
    the last `tail` tokens belong to no sequence."""
    N, T = len(lens), sum(lens) + tail
    x = make_inputs(1, T, Hq, Hv, beta_dtype, h0, N=N, seed=seed)
    gen = torch.Generator("cpu").manual_seed(seed + 1000)
    x["do"] = torch.randn(1, T, Hv, 128, generator=gen).to(torch.bfloat16)
    x["dhT"] = torch.randn(N, Hv, 128, 128, generator=gen) if dhT else None
    return x, cu_from_lengths(lens)


def _packed_grads(x, cu, want_dh0=True, fill=None):
    d = to_device(x)
    grads = None
    if fill is not None:   # prefilled outputs: rows the call must leave alone keep the fill
        f32 = dict(device="cuda", dtype=torch.float32)
        grads = {n: torch.full(tuple(d[src].shape), fill, **f32)
                 for n, src in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dg", "g"), ("dbeta", "beta"))}
    g = kda_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], SCALE, d["do"], initial_state=d["h0"],
                d_final_state=d["dhT"], d_initial_state=want_dh0, grads=grads, cu_seqlens=cu.cuda())
    torch.cuda.synchronize()
    return {n: (None if t is None else t.cpu().numpy().astype(np.float64)) for n, t in g.items()}


def _sequence(x, n, sl):
    """Sequence n of a packed batch as a one-row batch of its own."""
    sub = {key: x[key][:, sl] for key in ("q", "k", "v", "g", "beta", "do")}
    sub["h0"] = None if x["h0"] is None else x["h0"][n:n + 1]
    sub["dhT"] = None if x["dhT"] is None else x["dhT"][n:n + 1]
    return sub


def _compare_packed(got, x, cu, label, recurrence=False):
    """Each sequence's gradients against the oracle run on that sequence alone."""
    Hv = x["v"].shape[2]
    for n, sl in enumerate(seq_slices(cu)):
        sub = _sequence(x, n, sl)
        part = {key: (got[key][:, sl] if key != "dh0" else got["dh0"][n:n + 1]) for key in NAMES}
        if sl.stop == sl.start:   # an empty sequence passes the state gradient through
            want = np.zeros((1, Hv, 128, 128)) if sub["dhT"] is None else _f64(sub["dhT"])
            assert np.array_equal(part["dh0"], want), (label, n)
            continue
        _compare(part, _oracle(sub), f"{label} seq {n} ({sl.stop - sl.start} tokens)")
        if recurrence:
            h0 = sub["h0"] if sub["h0"] is not None else torch.zeros(1, Hv, 128, 128)
            rec = og.grads(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], SCALE, h0, sub["do"], sub["dhT"])
            _compare(part, rec, f"{label} seq {n} vs recurrence")


@pytest.mark.parametrize("lens,Hq,Hv,h0,dhT,beta_dtype", [
    ([1, 63, 64, 65, 130, 7], 2, 4, True, True, torch.float32),    # chunk starts off the 64-token grid, GVA
    ([0, 200, 0, 0, 33], 1, 1, True, True, torch.bfloat16),          # empty sequences, bf16 beta
    ([129], 2, 2, False, False, torch.float32),                       # one sequence, zero state
])
def test_bwd_packed_matches_oracle_per_sequence(lens, Hq, Hv, h0, dhT, beta_dtype):
    x, cu = _packed_case(lens, Hq, Hv, seed=sum(lens) + len(lens), h0=h0, dhT=dhT, beta_dtype=beta_dtype)
    _say(f"kda_bwd packed lens={lens} Hq={Hq} Hv={Hv} h0={h0} dhT={dhT} beta={beta_dtype}")
    got = _packed_grads(x, cu)
    _compare_packed(got, x, cu, f"packed {lens}", recurrence=sum(lens) <= 200)


def test_bwd_packed_leaves_tokens_of_no_sequence_alone():
    # 40 trailing tokens lie in no sequence: their gradient rows keep the NaN fill,
    # every other row is written (finite)
    lens, tail = [70, 5, 64], 40
    for Hq, Hv in ((2, 2), (1, 4)):   # dq, dk written directly, and summed over a group
        x, cu = _packed_case(lens, Hq, Hv, seed=31 + Hv, tail=tail)
        _say(f"kda_bwd packed lens={lens} + {tail} uncovered tokens, Hq={Hq} Hv={Hv}")
        got = _packed_grads(x, cu, fill=float("nan"))
        covered = sum(lens)
        for n in ("dq", "dk", "dv", "dg", "dbeta"):
            assert np.isfinite(got[n][:, :covered]).all(), n
            assert np.isnan(got[n][:, covered:]).all(), n
        _compare_packed(got, x, cu, f"packed + tail Hv={Hv}")


def test_bwd_packed_equal_lengths_is_the_fixed_batch_bit_for_bit():
    # three sequences of 130 tokens packed into one row take the same chunks, in the
    # same order of arithmetic, as a fixed-length batch of three rows
    B, T, Hq, Hv = 3, 130, 2, 4
    x = _case(B, T, Hq, Hv, seed=41)
    _say("kda_bwd fixed B=3 T=130 against the same rows packed")
    a = _gpu_grads(x)
    packed = {key: (x[key].reshape(1, B * T, *x[key].shape[2:]) if key in ("q", "k", "v", "g", "beta", "do")
                    else x[key]) for key in x}
    b = _packed_grads(packed, cu_from_lengths([T] * B))
    for n in NAMES:
        want = a[n] if n == "dh0" else a[n].reshape(b[n].shape)
        assert np.array_equal(b[n], want), n


def test_bwd_packed_is_reproducible_and_takes_a_caller_workspace():
    lens = [300, 1, 90]
    x, cu = _packed_case(lens, 2, 4, seed=43)
    need = kda_bwd_workspace_size(sum(lens), len(lens), 2, 4)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    _say(f"kda_bwd packed lens={lens} twice, library and caller workspace")
    a = _packed_grads(x, cu)
    d = to_device(x)
    g = kda_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], SCALE, d["do"], initial_state=d["h0"],
                d_final_state=d["dhT"], d_initial_state=True, workspace=ws, cu_seqlens=cu.cuda())
    torch.cuda.synchronize()
    for n in NAMES:
        assert np.array_equal(a[n], g[n].cpu().numpy().astype(np.float64)), n


def test_bwd_full_size_packed_sampled_heads():
    # the 14-sequence, 16,384-token packed batch the forward is measured on, with an
    # initial state, a random final-state gradient and dh0; two value heads checked
    # on every sequence
    from gated_delta_rule_35_amd.inputs import WORKLOADS
    w = WORKLOADS["varlen_h64_16k"]
    lens = varlen_lengths(w.varlen_total, w.length_seed)
    x, cu = _packed_case(lens, w.Hq, w.Hv, seed=45)
    _say(f"kda_bwd packed {len(lens)} sequences, {sum(lens)} tokens, H={w.Hv}")
    got = _packed_grads(x, cu)
    heads = [3, 60]
    sub = head_subset(x, heads, w.Hq, w.Hv)
    sub["do"] = x["do"][:, :, heads]
    sub["dhT"] = x["dhT"][:, heads]
    part = {n: (got[n][:, heads] if n == "dh0" else got[n][:, :, heads]) for n in NAMES}
    for n in NAMES:
        assert np.isfinite(got[n]).all(), n
    _compare_packed(part, sub, cu, "full-size packed")

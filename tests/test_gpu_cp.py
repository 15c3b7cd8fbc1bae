"""GPU parity of the segmented forward (kda_fwd_cp: each sequence cut into
segments whose state maps are composed, so the scan walks them side by side)
against the fp64 CPU oracle, through the C ABI.

The result is the recurrence itself, so the oracle is the same token recurrence
the other parity tests use; the tolerances are the same.  Each test prints the
case it is about to launch before touching the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_35_amd import kda_fwd, kda_fwd_cp, load_library
from gated_delta_rule_35_amd.inputs import make_inputs
from tests.kda_check import O_MAX_ABS, O_REL_F, STATE_REL_F, rel_frob_per_head, state_rel_frob, to_device

pytestmark = pytest.mark.gpu

SCALE = 128 ** -0.5


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    load_library()  # fails loudly if the HIP library is not built
    yield


def run_cp(x, seg_chunks, first_chunks=0, want_state=True):
    d = to_device(x)
    o, hT = kda_fwd_cp(d["q"], d["k"], d["v"], d["g"], d["beta"], SCALE, seg_chunks, first_chunks,
                       initial_state=d["h0"], final_state=True if want_state else None)
    torch.cuda.synchronize()
    return o, hT


def check_cp(x, seg_chunks, label, first_chunks=0):
    o, hT = run_cp(x, seg_chunks, first_chunks)
    o, hT = o.float().cpu().numpy(), hT.cpu().numpy()
    o_ref, h_ref = oracle.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], SCALE, h0=x["h0"])
    rel = rel_frob_per_head(o, o_ref)
    mx = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    srel = state_rel_frob(hT, h_ref)
    _say(f"{label}: o relF={rel:.3e} maxabs={mx:.3e} state relF={srel:.3e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(hT))
    assert rel <= O_REL_F, rel
    assert mx <= O_MAX_ABS, mx
    assert srel <= STATE_REL_F, srel


@pytest.mark.parametrize("B,T,Hq,Hv,seg,first,beta,h0", [
    (1, 1000, 2, 2, 3, 0, torch.float32, True),     # 6 segments, the last one a partial chunk
    (3, 640, 3, 3, 1, 0, torch.float32, True),      # one chunk per segment: 10 segments, 8 composed maps
    (2, 4096, 2, 8, 8, 0, torch.bfloat16, False),   # grouped values, 8 segments
    (1, 193, 2, 2, 1, 0, torch.float32, True),      # 4 segments of one chunk, 1-token tail
    (2, 1500, 2, 2, 3, 7, torch.float32, True),     # a 7-chunk first segment, then 3 each; a 28-token tail
    (1, 4096, 1, 4, 16, 32, torch.bfloat16, False), # grouped values, first segment of half the sequence
])
def test_segmented_matches_oracle(B, T, Hq, Hv, seg, first, beta, h0):
    _say(f"kda_fwd_cp B={B} T={T} Hq={Hq} Hv={Hv} segment_chunks={seg} first={first} h0={h0}")
    x = make_inputs(B, T, Hq, Hv, beta, h0=h0, seed=200 + T)
    check_cp(x, seg, f"cp B={B} T={T} seg={seg} first={first}", first)


def test_segmented_long_sequence():
    _say("kda_fwd_cp B=1 T=65536 H=2 segment_chunks=64 (16 segments) with h0")
    x = make_inputs(1, 65536, 2, 2, torch.float32, h0=True, seed=201)
    check_cp(x, 64, "cp T=65536")


def test_two_segments_or_fewer_is_kda_fwd_ws_bitwise():
    from gated_delta_rule_35_amd import kda_fwd_ws
    _say("kda_fwd_cp with 2 segments vs kda_fwd_ws, B=2 T=256 H=2")
    x = make_inputs(2, 256, 2, 2, torch.float32, h0=True, seed=202)
    d = to_device(x)
    o1, h1 = kda_fwd_ws(d["q"], d["k"], d["v"], d["g"], d["beta"], SCALE, initial_state=d["h0"], final_state=True)
    o2, h2 = kda_fwd_cp(d["q"], d["k"], d["v"], d["g"], d["beta"], SCALE, 2, initial_state=d["h0"],
                        final_state=True)
    o3, h3 = kda_fwd_cp(d["q"], d["k"], d["v"], d["g"], d["beta"], SCALE, 1, 3, initial_state=d["h0"],
                        final_state=True)   # 3 + 1 chunks: two segments
    torch.cuda.synchronize()
    for o, h in ((o2, h2), (o3, h3)):
        assert torch.equal(o1.view(torch.int16), o.view(torch.int16))
        assert torch.equal(h1.view(torch.int32), h.view(torch.int32))


def test_segmented_is_repeatable_and_may_update_the_state_in_place():
    _say("kda_fwd_cp repeat and in-place state, B=2 T=1024 H=4 segment_chunks=4")
    x = make_inputs(2, 1024, 4, 4, torch.float32, h0=True, seed=203)
    d = to_device(x)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], SCALE, 4)
    o1, h1 = kda_fwd_cp(*args, initial_state=d["h0"], final_state=True)
    o2, h2 = kda_fwd_cp(*args, initial_state=d["h0"], final_state=True)
    st = d["h0"].clone()
    o3, h3 = kda_fwd_cp(*args, initial_state=st, final_state=st)
    torch.cuda.synchronize()
    for o in (o2, o3):
        assert torch.equal(o1.view(torch.int16), o.view(torch.int16))
    for h in (h2, h3):
        assert torch.equal(h1.view(torch.int32), h.view(torch.int32))


@pytest.mark.parametrize("name,heads", [("mha_b1_h8_t65536", [0, 7]), ("mha_b2_h8_t8192", [2, 5])])
def test_bench_workloads_with_the_plan(name, heads):
    """The few-head workloads bench.py --cp times, with the segment lengths it
    takes from kda_fwd_cp_plan; the oracle checks the sampled heads."""
    from gated_delta_rule_35_amd import kda_fwd_cp_plan
    from gated_delta_rule_35_amd.inputs import WORKLOADS, workload_inputs
    from tests.kda_check import head_subset
    w = WORKLOADS[name]
    x, _ = workload_inputs(w)
    B, T = x["q"].shape[0], x["q"].shape[1]
    plan = kda_fwd_cp_plan(B, T, w.Hv)
    assert plan is not None
    L, L0 = plan
    _say(f"{name} with the plan ({L0} chunks, then {L}), oracle on heads {heads}")
    d = to_device(x)
    o, hT = kda_fwd_cp(d["q"], d["k"], d["v"], d["g"], d["beta"], w.scale, L, L0, initial_state=d["h0"],
                       final_state=True)
    torch.cuda.synchronize()
    o = o[:, :, heads].float().cpu().numpy()
    hT = hT[:, heads].cpu().numpy()
    sub = head_subset(x, heads, w.Hq, w.Hv)
    o_ref, h_ref = oracle.recurrence(sub["q"], sub["k"], sub["v"], sub["g"], sub["beta"], w.scale, h0=sub["h0"])
    rel = rel_frob_per_head(o, o_ref)
    mx = float(np.max(np.abs(o - o_ref)))
    srel = state_rel_frob(hT, h_ref)
    _say(f"{name}: o relF={rel:.3e} maxabs={mx:.3e} state relF={srel:.3e}")
    assert rel <= O_REL_F and mx <= O_MAX_ABS and srel <= STATE_REL_F, (rel, mx, srel)


# ---- packed sequences (cu_seqlens): the plan is made on the device ----

def _packed(lens, Hq, Hv, seed, h0=True, beta=torch.float32, tail=0):
    from gated_delta_rule_35_amd.inputs import cu_from_lengths
    cu = cu_from_lengths(lens)
    T = int(cu[-1]) + tail
    x = make_inputs(1, T, Hq, Hv, beta, h0=h0, N=len(lens), seed=seed)
    return x, cu


def _check_packed(x, cu, seg, first, label, fill=None):
    d = to_device(x)
    out = None
    if fill is not None:
        out = torch.full_like(d["v"], fill)
    o, hT = kda_fwd_cp(d["q"], d["k"], d["v"], d["g"], d["beta"], SCALE, seg, first, initial_state=d["h0"],
                       out=out, final_state=True, cu_seqlens=cu.cuda())
    torch.cuda.synchronize()
    o_np, h_np = o.float().cpu().numpy(), hT.cpu().numpy()
    o_ref, h_ref = oracle.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], SCALE, cu_seqlens=cu, h0=x["h0"])
    cuv = [int(c) for c in cu]
    worst, mx = 0.0, 0.0
    for n in range(len(cuv) - 1):
        a, e = cuv[n], cuv[n + 1]
        if e > a:
            worst = max(worst, rel_frob_per_head(o_np[:, a:e], o_ref[:, a:e]))
            mx = max(mx, float(np.max(np.abs(o_np[:, a:e] - o_ref[:, a:e]))))
    srel = state_rel_frob(h_np, h_ref)
    _say(f"{label}: o relF={worst:.3e} maxabs={mx:.3e} state relF={srel:.3e}")
    assert np.all(np.isfinite(h_np))
    assert worst <= O_REL_F, worst
    assert mx <= O_MAX_ABS, mx
    assert srel <= STATE_REL_F, srel
    return o, hT


@pytest.mark.parametrize("lens,Hq,Hv,seg,first", [
    ([1, 63, 65, 700, 0, 2000, 5], 2, 2, 3, 0),     # empty, one-token, tail and long sequences
    ([1300, 64, 1], 2, 4, 1, 4),                    # one-chunk segments after a 4-chunk first one
    ([4096, 3000, 129], 1, 4, 8, 16),               # grouped values, three long sequences
    ([640] * 5, 3, 3, 2, 0),                        # equal lengths, 5 segments each
])
def test_packed_segmented_matches_oracle(lens, Hq, Hv, seg, first):
    _say(f"kda_fwd_cp packed lens={lens} Hq={Hq} Hv={Hv} segment_chunks={seg} first={first}")
    x, cu = _packed(lens, Hq, Hv, seed=300 + sum(lens))
    _check_packed(x, cu, seg, first, f"cp packed {lens}")


def test_packed_segmented_leaves_other_rows_and_repeats():
    """Rows past cu[N] keep what the caller put there; repeated calls are bitwise
    equal; with at most two segments per sequence the call equals kda_fwd_ws bit
    for bit (no map is composed)."""
    from gated_delta_rule_35_amd import kda_fwd_ws
    lens = [200, 0, 1000, 65]
    _say(f"kda_fwd_cp packed lens={lens} with 37 trailing tokens, repeats and kda_fwd_ws comparison")
    x, cu = _packed(lens, 2, 2, seed=310, tail=37)
    o1, h1 = _check_packed(x, cu, 4, 0, "cp packed trailing rows", fill=3.0)
    assert torch.all(o1[:, int(cu[-1]):] == 3.0)
    o2, h2 = _check_packed(x, cu, 4, 0, "cp packed repeat", fill=3.0)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(h1, h2)
    d = to_device(x)
    # 16 chunks per segment: every sequence has one or two segments
    o3, h3 = kda_fwd_cp(d["q"], d["k"], d["v"], d["g"], d["beta"], SCALE, 16, initial_state=d["h0"],
                        final_state=True, cu_seqlens=cu.cuda())
    o4, h4 = kda_fwd_ws(d["q"], d["k"], d["v"], d["g"], d["beta"], SCALE, cu_seqlens=cu.cuda(),
                        initial_state=d["h0"], final_state=True)
    torch.cuda.synchronize()
    n = int(cu[-1])
    assert torch.equal(o3[:, :n].view(torch.int16), o4[:, :n].view(torch.int16)) and torch.equal(h3, h4)


def test_packed_segmented_long_sequence_among_short_ones():
    """One 32,768-token sequence among three short ones, 8 heads, 16-chunk segments
    after a 32-chunk first one (the case the segmented form is for)."""
    lens = [100, 32768, 1, 500]
    _say(f"kda_fwd_cp packed lens={lens} H=8 segment_chunks=16 first=32")
    x, cu = _packed(lens, 8, 8, seed=320)
    _check_packed(x, cu, 16, 32, "cp packed long")

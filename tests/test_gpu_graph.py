"""The library's launches under HIP graph capture (torch.cuda.graph): kda_fwd_fused,
kda_fwd_ws, kda_fwd_cp (fixed length and packed), kda_decode and kda_bwd are captured once with caller-owned outputs and
workspaces (nothing is allocated and no memset is recorded), then replayed
several times with eager work and synchronisation in between; every replay
must reproduce the eager result bit for bit."""
import pytest
import torch

from gated_delta_rule_35_amd import (kda_decode, kda_fwd, kda_fwd_cp, kda_fwd_cp_packed_workspace_size,
                                     kda_fwd_cp_workspace_size, kda_fwd_fused, kda_fwd_workspace_size, kda_fwd_ws,
                                     load_library)
from gated_delta_rule_35_amd.inputs import cu_from_lengths, make_inputs
from tests.kda_check import to_device

pytestmark = pytest.mark.gpu

SCALE = 128 ** -0.5
REPLAYS = 4


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    load_library()  # fails loudly if the HIP library is not built
    yield


def capture_and_replay(call, outputs, reference):
    """call() writes into `outputs`; `reference` holds the eager results."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # one eager run on the side stream before capture
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for t in outputs:
            t.fill_(float("nan") if t.dtype.is_floating_point else 0)   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, ref in zip(outputs, reference):
            bits = torch.int16 if t.element_size() == 2 else torch.int32
            assert torch.equal(t.view(bits), ref.view(bits)), f"replay {r}"


def test_kda_fwd_fused_in_a_graph():
    _say("graph: kda_fwd_fused (nothing allocated) B=2 T=300 Hq=2 Hv=4 with h0")
    x = make_inputs(2, 300, 2, 4, torch.float32, h0=True, seed=302)
    d = to_device(x)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], SCALE)
    o_ref, h_ref = kda_fwd_fused(*args, initial_state=d["h0"], final_state=True)
    out, hT = torch.empty_like(o_ref), torch.empty_like(h_ref)
    capture_and_replay(lambda: kda_fwd_fused(*args, initial_state=d["h0"], out=out, final_state=hT), (out, hT),
                       (o_ref, h_ref))


def test_kda_fwd_ws_in_a_graph():
    _say("graph: kda_fwd_ws B=2 T=300 Hq=2 Hv=4 with h0")
    x = make_inputs(2, 300, 2, 4, torch.float32, h0=True, seed=300)
    d = to_device(x)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], SCALE)
    ws = torch.empty(kda_fwd_workspace_size(600, 2, 4), dtype=torch.uint8, device="cuda")
    o_ref, h_ref = kda_fwd_ws(*args, initial_state=d["h0"], final_state=True, workspace=ws)
    out, hT = torch.empty_like(o_ref), torch.empty_like(h_ref)
    capture_and_replay(lambda: kda_fwd_ws(*args, initial_state=d["h0"], out=out, final_state=hT, workspace=ws),
                       (out, hT), (o_ref, h_ref))


def test_kda_fwd_cp_in_a_graph():
    _say("graph: kda_fwd_cp B=1 T=2048 H=2, first segment 8 chunks, then 4")
    x = make_inputs(1, 2048, 2, 2, torch.float32, h0=True, seed=301)
    d = to_device(x)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], SCALE, 4, 8)
    o_ref, h_ref = kda_fwd_cp(*args, initial_state=d["h0"], final_state=True)
    out, hT = torch.empty_like(o_ref), torch.empty_like(h_ref)
    ws = torch.empty(kda_fwd_cp_workspace_size(1, 2048, 2, 4, 8), dtype=torch.uint8, device="cuda")
    capture_and_replay(lambda: kda_fwd_cp(*args, initial_state=d["h0"], out=out, final_state=hT, workspace=ws),
                       (out, hT), (o_ref, h_ref))


def test_kda_fwd_cp_packed_in_a_graph():
    """The packed segmented call plans on the device (a kernel writes the segment
    tables into the workspace), so it too is launches only."""
    lens = [1500, 3, 700]
    _say(f"graph: kda_fwd_cp packed lens={lens} H=2, first segment 8 chunks, then 3")
    cu = cu_from_lengths(lens).cuda()
    x = make_inputs(1, sum(lens), 2, 2, torch.float32, h0=True, N=len(lens), seed=303)
    d = to_device(x)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], SCALE, 3, 8)
    o_ref, h_ref = kda_fwd_cp(*args, initial_state=d["h0"], final_state=True, cu_seqlens=cu)
    out, hT = torch.empty_like(o_ref), torch.empty_like(h_ref)
    ws = torch.empty(kda_fwd_cp_packed_workspace_size(sum(lens), len(lens), 2, 3, 8), dtype=torch.uint8,
                     device="cuda")
    capture_and_replay(lambda: kda_fwd_cp(*args, initial_state=d["h0"], out=out, final_state=hT, workspace=ws,
                                          cu_seqlens=cu),
                       (out, hT), (o_ref, h_ref))


def test_kda_decode_in_a_graph():
    _say("graph: kda_decode N=3 Hq=2 Hv=4, state written to a separate buffer")
    x = make_inputs(3, 1, 2, 4, torch.float32, h0=True, seed=302)
    s = {k: v[:, 0].contiguous().cuda() for k, v in x.items() if k != "h0"}
    state = x["h0"].cuda()
    args = (s["q"], s["k"], s["v"], s["g"], s["beta"], SCALE, state)
    o_ref, n_ref = kda_decode(*args, new_state=torch.empty_like(state))
    out, new = torch.empty_like(o_ref), torch.empty_like(n_ref)
    capture_and_replay(lambda: kda_decode(*args, out=out, new_state=new), (out, new), (o_ref, n_ref))


def test_kda_bwd_in_a_graph():
    _say("graph: kda_bwd B=2 T=150 Hq=2 Hv=4 with h0, dhT and dh0")
    from gated_delta_rule_35_amd import kda_bwd, kda_bwd_workspace_size
    x = make_inputs(2, 150, 2, 4, torch.float32, h0=True, seed=302)
    d = to_device(x)
    gen = torch.Generator("cpu").manual_seed(303)
    do = torch.randn(2, 150, 4, 128, generator=gen).to(torch.bfloat16).cuda()
    dhT = torch.randn(2, 4, 128, 128, generator=gen).cuda()
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], SCALE, do)
    ref = kda_bwd(*args, initial_state=d["h0"], d_final_state=dhT, d_initial_state=True)
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "dg", "dbeta", "dh0")
    outs = {n: torch.empty_like(ref[n]) for n in names}
    ws = torch.empty(kda_bwd_workspace_size(2 * 150, 2, 2, 4), dtype=torch.uint8, device="cuda")
    capture_and_replay(lambda: kda_bwd(*args, initial_state=d["h0"], d_final_state=dhT, grads=outs,
                                       d_initial_state=outs["dh0"], workspace=ws),
                       [outs[n] for n in names], [ref[n] for n in names])

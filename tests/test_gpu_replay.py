"""Determinism at scale: one forward call captured into a HIP graph and replayed
10,000 times on the full workloads (the headline batch and the packed
variable-length one), for both forms of the forward.  Every replay's output and
final state must equal the first eager call's bit for bit ("cuLA PR #131: SM100/SM103
KDA forward to pure CuTeDSL", Validation: repeated fixed-shape and packed-varlen
runs with zero mismatches).  Mismatches are counted on the device after each
replay and read back every 1,000 replays, so the test stops soon after the first."""
import pytest
import torch

from gated_delta_rule_35_amd import kda_fwd_fused, kda_fwd_workspace_size, kda_fwd_ws, load_library
from gated_delta_rule_35_amd.inputs import WORKLOADS, workload_inputs
from tests.kda_check import to_device

pytestmark = pytest.mark.gpu

REPLAYS = 10_000
CHECK_EVERY = 1_000


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    load_library()  # fails loudly if the HIP library is not built
    yield


@pytest.mark.parametrize("form", ["two_pass", "fused"])
@pytest.mark.parametrize("name", ["mha_b2_h64_t8192", "varlen_h64_16k"])
def test_graph_replays_are_bitwise_identical(name, form):
    w = WORKLOADS[name]
    x, cu = workload_inputs(w)
    d = to_device(x)
    cu_d = cu.to("cuda") if cu is not None else None
    B, T = x["q"].shape[:2]
    N = B if cu is None else cu.shape[0] - 1
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], w.scale)
    if form == "two_pass":
        ws = torch.empty(kda_fwd_workspace_size(B * T, N, w.Hv), dtype=torch.uint8, device="cuda")
        call = lambda o, h: kda_fwd_ws(*args, cu_seqlens=cu_d, initial_state=d["h0"], out=o, final_state=h,
                                       workspace=ws)
    else:
        call = lambda o, h: kda_fwd_fused(*args, cu_seqlens=cu_d, initial_state=d["h0"], out=o, final_state=h)
    _say(f"{name} {form}: eager reference, then {REPLAYS} graph replays")
    o_ref = torch.empty_like(d["v"])
    h_ref = torch.empty(N, w.Hv, 128, 128, dtype=torch.float32, device="cuda")
    call(o_ref, h_ref)
    out, hT = torch.full_like(o_ref, float("nan")), torch.full_like(h_ref, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out, hT)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out, hT)
    torch.cuda.synchronize()
    o_bits, h_bits = o_ref.view(torch.int16), h_ref.view(torch.int32)
    mism = torch.zeros((), dtype=torch.int64, device="cuda")
    for r in range(REPLAYS):
        graph.replay()
        mism += torch.ne(out.view(torch.int16), o_bits).any().to(torch.int64)
        mism += torch.ne(hT.view(torch.int32), h_bits).any().to(torch.int64)
        if (r + 1) % CHECK_EVERY == 0:
            bad = int(mism.item())
            _say(f"  {name} {form}: {r + 1} replays, {bad} mismatching")
            assert bad == 0, f"replay mismatch by replay {r + 1}"

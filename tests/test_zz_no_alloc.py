"""kda_fwd_noalloc (the forward entry point that allocates nothing: its records
live in the library's static device scratch) against kda_fwd_ws, the two-pass
forward it varies, called through the C ABI: two calls in a row, the second on
a smaller problem, each compared bit for bit with kda_fwd_ws on the same inputs
(the same kernels), and the first also against the fp64 oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_35_amd import binding, kda_fwd_ws, load_library
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


def _noalloc(d, out, hT, cu=None):
    """kda_fwd_noalloc through ctypes on the current stream."""
    lib = load_library()
    ds = [binding.describe(t) for t in (d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d.get("h0"), out, hT)]
    r = lambda x: None if x is None else ctypes.byref(x)  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.kda_fwd_noalloc(r(ds[0]), r(ds[1]), r(ds[2]), r(ds[3]), r(ds[4]), SCALE, r(ds[5]), r(ds[6]),
                             r(ds[7]), r(ds[8]), stream)
    assert st == 0, lib.kda_status_string(st).decode()


def _run_pair(x, cu=None):
    """kda_fwd_noalloc into NaN-filled outputs, then kda_fwd_ws; both must agree bitwise."""
    d = to_device(x)
    cu_d = cu.cuda() if cu is not None else None
    N = x["q"].shape[0] if cu is None else cu.shape[0] - 1
    out = torch.full_like(d["v"], float("nan"))
    hT = torch.full((N, x["v"].shape[2], 128, 128), float("nan"), dtype=torch.float32, device="cuda")
    _noalloc(d, out, hT, cu_d)
    o_ref, h_ref = kda_fwd_ws(d["q"], d["k"], d["v"], d["g"], d["beta"], SCALE, cu_seqlens=cu_d,
                              initial_state=d.get("h0"), final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(hT.view(torch.int32), h_ref.view(torch.int32))
    return out, hT


def test_noalloc_two_calls_second_smaller():
    _say("kda_fwd_noalloc call 1: B=2 T=700 Hq=2 Hv=4 with h0")
    x1 = make_inputs(2, 700, 2, 4, torch.float32, h0=True, seed=501)
    o1, h1 = _run_pair(x1)
    o_ref, h_ref = oracle.recurrence(x1["q"], x1["k"], x1["v"], x1["g"], x1["beta"], SCALE, h0=x1["h0"])
    o1 = o1.float().cpu().numpy()
    assert rel_frob_per_head(o1, o_ref) <= O_REL_F
    assert np.max(np.abs(o1 - o_ref)) <= O_MAX_ABS
    assert state_rel_frob(h1.cpu().numpy(), h_ref) <= STATE_REL_F

    _say("kda_fwd_noalloc call 2 (smaller): B=1 T=130 Hq=1 Hv=2, bf16 beta, no h0")
    x2 = make_inputs(1, 130, 1, 2, torch.bfloat16, h0=False, seed=502)
    _run_pair(x2)


def test_noalloc_packed_sequences():
    _say("kda_fwd_noalloc packed: lengths 65, 0, 1, 200")
    lens = [65, 0, 1, 200]
    x = make_inputs(1, sum(lens), 2, 2, torch.float32, h0=True, N=len(lens), seed=503)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    _run_pair(x, cu)

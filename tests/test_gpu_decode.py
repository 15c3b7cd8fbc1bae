"""GPU parity of kda_decode (one recurrent step per sequence, through the C ABI)
against the fp64 oracle's token recurrence.

The decode step runs in fp32 throughout, so beside the library-wide tolerances
(o: per-head relative Frobenius <= 3e-3, the bf16 rounding of o dominating) the
state is held to 1e-5 per head: the fp32 result of a few steps differs from the
fp64 one by rounding only.  Each test prints its case before touching the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_35_amd import kda_decode, kda_fwd, load_library
from gated_delta_rule_35_amd.inputs import make_inputs
from tests.kda_check import O_MAX_ABS, O_REL_F, STATE_REL_F, rel_frob_per_head, state_rel_frob, to_device

pytestmark = pytest.mark.gpu

SCALE = 128 ** -0.5
DECODE_STATE_REL_F = 1e-5


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    load_library()  # fails loudly if the HIP library is not built
    yield


def _step_inputs(x, t):
    """Token t of every sequence as decode inputs ([N, H, ...])."""
    return {k: x[k][:, t].contiguous() for k in ("q", "k", "v", "g", "beta")}


def _decode_steps(x, t0, t1, state):
    """Decode tokens t0 .. t1 - 1 on the GPU from `state` (updated in place);
    returns o as [N, t1 - t0, Hv, 128] fp32 and the state."""
    outs = []
    for t in range(t0, t1):
        s = to_device(_step_inputs(x, t))
        o, state = kda_decode(s["q"], s["k"], s["v"], s["g"], s["beta"], SCALE, state)
        outs.append(o.float())
    torch.cuda.synchronize()
    return torch.stack(outs, dim=1).cpu().numpy(), state


@pytest.mark.parametrize("N,Hq,Hv,beta_dtype,h0", [
    (3, 4, 4, torch.float32, True),
    (2, 2, 8, torch.bfloat16, True),
    (5, 4, 4, torch.float32, False),
])
def test_one_step_matches_oracle(N, Hq, Hv, beta_dtype, h0):
    _say(f"decode one step N={N} Hq={Hq} Hv={Hv} beta={beta_dtype} h0={h0}")
    x = make_inputs(N, 1, Hq, Hv, beta_dtype, h0=h0, seed=41 + N)
    state = x["h0"].cuda() if h0 else None
    o, st = _decode_steps(x, 0, 1, state)
    o_ref, h_ref = oracle.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], SCALE, h0=x["h0"])
    rel = rel_frob_per_head(o, o_ref)
    srel = state_rel_frob(st.cpu().numpy(), h_ref)
    _say(f"  o relF={rel:.3e} state relF={srel:.3e}")
    assert rel <= O_REL_F and float(np.max(np.abs(o - o_ref))) <= O_MAX_ABS
    assert srel <= DECODE_STATE_REL_F


def test_many_steps_follow_the_recurrence():
    _say("decode 40 steps N=2 Hq=2 Hv=4 from h0")
    x = make_inputs(2, 40, 2, 4, torch.float32, h0=True, seed=43)
    o, st = _decode_steps(x, 0, 40, x["h0"].cuda())
    o_ref, h_ref = oracle.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], SCALE, h0=x["h0"])
    rel = rel_frob_per_head(o, o_ref)
    srel = state_rel_frob(st.cpu().numpy(), h_ref)
    _say(f"  o relF={rel:.3e} state relF={srel:.3e}")
    assert rel <= O_REL_F
    assert srel <= DECODE_STATE_REL_F


def test_decode_continues_the_forward():
    """Prefill 300 tokens with kda_fwd, then decode 6 more from its final state:
    the whole run matches the oracle's recurrence over 306 tokens."""
    _say("prefill 300 + decode 6, B=2 Hq=2 Hv=4")
    x = make_inputs(2, 306, 2, 4, torch.float32, h0=True, seed=44)
    d = to_device(x)
    pre = {k: d[k][:, :300].contiguous() for k in ("q", "k", "v", "g", "beta")}
    o_pre, state = kda_fwd(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], SCALE, initial_state=d["h0"],
                           final_state=True)
    o_dec, state = _decode_steps(x, 300, 306, state)
    o_ref, h_ref = oracle.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], SCALE, h0=x["h0"])
    o_all = np.concatenate([o_pre.float().cpu().numpy(), o_dec], axis=1)
    rel = rel_frob_per_head(o_all, o_ref)
    rel_dec = rel_frob_per_head(o_dec, o_ref[:, 300:])
    srel = state_rel_frob(state.cpu().numpy(), h_ref)
    _say(f"  o relF={rel:.3e} (decode part {rel_dec:.3e}) state relF={srel:.3e}")
    assert rel <= O_REL_F and rel_dec <= O_REL_F
    assert srel <= STATE_REL_F


def test_full_batch_and_bitwise_properties():
    """A serving-size batch (64 sequences x 64 heads) against the oracle, then:
    repeat runs, in place vs separate output state, and a NULL state vs zeros are
    bitwise identical."""
    _say("decode N=64 Hq=Hv=64 one step")
    x = make_inputs(64, 1, 64, 64, torch.bfloat16, h0=True, seed=45)
    s = to_device(_step_inputs(x, 0))
    h0 = x["h0"].cuda()
    o1, s1 = kda_decode(s["q"], s["k"], s["v"], s["g"], s["beta"], SCALE, h0, new_state=torch.empty_like(h0))
    o2, s2 = kda_decode(s["q"], s["k"], s["v"], s["g"], s["beta"], SCALE, h0, new_state=torch.empty_like(h0))
    inplace = h0.clone()
    o3, s3 = kda_decode(s["q"], s["k"], s["v"], s["g"], s["beta"], SCALE, inplace)
    torch.cuda.synchronize()
    assert s3.data_ptr() == inplace.data_ptr()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert torch.equal(o1, o3) and torch.equal(s1, s3)
    o_ref, h_ref = oracle.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], SCALE, h0=x["h0"])
    rel = rel_frob_per_head(o1.float().cpu().numpy()[:, None], o_ref)
    srel = state_rel_frob(s1.cpu().numpy(), h_ref)
    _say(f"  o relF={rel:.3e} state relF={srel:.3e}")
    assert rel <= O_REL_F
    assert srel <= DECODE_STATE_REL_F

    _say("decode N=3 Hq=Hv=4: NULL state vs explicit zeros")
    y = make_inputs(3, 1, 4, 4, torch.float32, seed=46)
    t = to_device(_step_inputs(y, 0))
    oa, sa = kda_decode(t["q"], t["k"], t["v"], t["g"], t["beta"], SCALE, None)
    ob, sb = kda_decode(t["q"], t["k"], t["v"], t["g"], t["beta"], SCALE,
                        torch.zeros((3, 4, 128, 128), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(sa, sb)

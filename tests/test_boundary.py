"""Host-side checks of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before any HIP call (so these run without a GPU;
the data pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_35_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

FAKE = 0x7f0000000000  # 16-byte aligned, never dereferenced by the checks


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(kda_\w+)\s*\(", text, flags=re.M)))


def test_header_declarations_are_exported(lib):
    names = declared_functions()
    assert set(names) == set(binding.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def T(shape, dtype=binding.KDA_BF16, data=FAKE, strides=None):
    d = binding.KdaTensor()
    d.data = data
    d.dtype = dtype
    d.ndim = len(shape)
    st = strides
    if st is None:
        st, acc = [], 1
        for s in reversed(shape):
            st.insert(0, acc)
            acc *= s
    for i, s in enumerate(shape):
        d.shape[i] = s
        d.stride[i] = st[i]
    return d


def good(B=1, T_=64, Hq=2, Hv=2, beta_dtype=binding.KDA_F32):
    return dict(q=T([B, T_, Hq, 128]), k=T([B, T_, Hq, 128]), v=T([B, T_, Hv, 128]),
                g=T([B, T_, Hv, 128], binding.KDA_F32), beta=T([B, T_, Hv], beta_dtype),
                out=T([B, T_, Hv, 128]))


def call(lib, a, scale=0.088, cu=None, h0=None, hT=None, ws=None, ws_size=None, entry="kda_fwd"):
    """One forward call: the 11-argument kda_fwd (or kda_fwd_noalloc), or, when a
    workspace size is given, kda_fwd_ws."""
    r = lambda d: None if d is None else ctypes.byref(d)  # noqa: E731
    args = (r(a.get("q")), r(a.get("k")), r(a.get("v")), r(a.get("g")), r(a.get("beta")), scale, r(cu), r(h0),
            r(a.get("out")), r(hT))
    if ws_size is not None:
        return lib.kda_fwd_ws(*args, ws, ws_size, None)
    return getattr(lib, entry)(*args, None)


def expect(lib, a, name, **kw):
    st = call(lib, a, **kw)
    assert binding.STATUS_NAMES[st] == name, (binding.STATUS_NAMES[st], name)


def test_null_descriptor_and_null_data(lib):
    for key in ("q", "k", "v", "g", "beta", "out"):
        a = good()
        a[key] = None
        expect(lib, a, "KDA_ERR_NULL")
    a = good()
    a["q"] = T([1, 64, 2, 128], data=None)
    expect(lib, a, "KDA_ERR_NULL")


def test_dtypes(lib):
    a = good()
    a["q"] = T([1, 64, 2, 128], binding.KDA_F16)
    expect(lib, a, "KDA_ERR_DTYPE")
    a = good()
    a["g"] = T([1, 64, 2, 128], binding.KDA_BF16)
    expect(lib, a, "KDA_ERR_DTYPE")
    a = good()
    a["beta"] = T([1, 64, 2], binding.KDA_I32)
    expect(lib, a, "KDA_ERR_DTYPE")
    a = good()
    expect(lib, a, "KDA_ERR_DTYPE", cu=T([3], binding.KDA_F32))


def test_shapes(lib):
    a = good()
    a["k"] = T([1, 64, 3, 128])
    expect(lib, a, "KDA_ERR_SHAPE")
    a = good()
    a["v"] = T([1, 63, 2, 128])
    expect(lib, a, "KDA_ERR_SHAPE")
    a = good()
    a["beta"] = T([1, 64, 3], binding.KDA_F32)
    expect(lib, a, "KDA_ERR_SHAPE")
    a = good()
    a["out"] = T([1, 64, 2])
    expect(lib, a, "KDA_ERR_SHAPE")
    a = good(B=1)
    expect(lib, a, "KDA_ERR_SHAPE", cu=T([4], binding.KDA_I32), h0=T([2, 2, 128, 128], binding.KDA_F32))
    a = good(B=2)
    expect(lib, a, "KDA_ERR_SHAPE", hT=T([3, 2, 128, 128], binding.KDA_F32))


def test_unsupported(lib):
    a = good()
    a["q"] = T([1, 64, 2, 64])
    a["k"] = T([1, 64, 2, 64])
    expect(lib, a, "KDA_ERR_UNSUPPORTED")
    a = good(Hq=3, Hv=4)
    expect(lib, a, "KDA_ERR_UNSUPPORTED")
    a = good(B=2)
    expect(lib, a, "KDA_ERR_UNSUPPORTED", cu=T([3], binding.KDA_I32))


def test_layout(lib):
    a = good()
    a["q"] = T([1, 64, 2, 128], strides=[64 * 2 * 128, 128, 64 * 128, 1])  # transposed heads
    expect(lib, a, "KDA_ERR_LAYOUT")
    a = good()
    a["v"] = T([1, 64, 2, 128], data=FAKE + 2)
    expect(lib, a, "KDA_ERR_LAYOUT")
    a = good(beta_dtype=binding.KDA_BF16)
    a["beta"] = T([1, 64, 2], binding.KDA_BF16, data=FAKE + 1)
    expect(lib, a, "KDA_ERR_LAYOUT")


def test_partly_overlapping_states(lib):
    a = good(B=2)
    st = lambda off: T([2, 2, 128, 128], binding.KDA_F32, data=FAKE + off)  # noqa: E731
    expect(lib, a, "KDA_ERR_LAYOUT", h0=st(0), hT=st(64 * 1024), ws=FAKE, ws_size=0)
    expect(lib, a, "KDA_ERR_LAYOUT", h0=st(64 * 1024), hT=st(0), ws=FAKE, ws_size=0)
    # in place, or fully apart: the workspace check is the next one to fail
    expect(lib, a, "KDA_ERR_WORKSPACE", h0=st(0), hT=st(0), ws=FAKE, ws_size=0)
    expect(lib, a, "KDA_ERR_WORKSPACE", h0=st(0), hT=st(4 * 2 * 2 * 128 * 128), ws=FAKE, ws_size=0)


def test_scale_value(lib):
    for s in (0.0, -1.0, float("inf"), float("nan")):
        expect(lib, good(), "KDA_ERR_VALUE", scale=s)


def test_empty_problem_needs_no_launch(lib):
    a = good(B=1, T_=0)
    for key in ("q", "k", "v", "g", "beta", "out"):
        a[key].data = None
    expect(lib, a, "KDA_OK")
    expect(lib, good(), "KDA_OK", cu=T([1], binding.KDA_I32))  # zero sequences
    # torch gives an empty tensor the strides of a size-1 dimension in its place:
    # an empty tensor addresses no element, so its strides are not checked
    a = good(B=2, T_=0)
    for key in ("q", "k", "v", "g", "beta", "out"):
        sh = [a[key].shape[i] for i in range(a[key].ndim)]
        st, acc = [], 1
        for n in reversed(sh):
            st.insert(0, acc)
            acc *= max(n, 1)
        a[key] = T(sh, a[key].dtype, data=None, strides=st)
    expect(lib, a, "KDA_OK")


def test_status_strings(lib):
    for i, name in enumerate(binding.STATUS_NAMES):
        assert lib.kda_status_string(i).decode().startswith(name)


def test_dv_slices(lib):
    # one scan work-group per 64-wide dv slice, whatever the sizes
    for n, hv in ((2, 64), (1, 64), (14, 64), (1, 1)):
        assert lib.kda_dv_slices(n, hv) == 2


def test_kda_fwd_has_the_eleven_argument_signature(lib):
    # q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, stream
    assert len(lib.kda_fwd.argtypes) == 11
    assert len(lib.kda_fwd_noalloc.argtypes) == 11
    assert len(lib.kda_fwd_ws.argtypes) == 13
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    decl = re.search(r"kda_status_t\s+kda_fwd\s*\((.*?)\);", text, flags=re.S).group(1)
    names = [p.strip().split()[-1].lstrip("*") for p in decl.split(",")]
    assert names == ["q", "k", "v", "g", "beta", "scale", "cu_seqlens", "initial_state", "out", "final_state",
                     "stream"]


def test_noalloc_limit_checked_on_the_host(lib):
    # 64 MiB of static scratch: a call whose workspace would exceed it is refused
    # before any HIP call; the tensor checks come first
    cap = lib.kda_fwd_noalloc_max_bytes()
    assert cap == 64 << 20
    rec = 61952
    assert lib.kda_fwd_workspace_size(2 * 8192, 2, 64) > cap
    a = good(B=2, T_=8192, Hq=64, Hv=64)
    expect(lib, a, "KDA_ERR_WORKSPACE", entry="kda_fwd_noalloc")
    # largest fitting: (ceil(T / 64) + 1) * Hv records for one sequence
    hv = cap // (rec * (128 + 1))
    assert lib.kda_fwd_workspace_size(8192, 1, hv) <= cap < lib.kda_fwd_workspace_size(8192, 1, hv + 1)
    b = good(B=1, T_=8192, Hq=hv + 1, Hv=hv + 1)
    expect(lib, b, "KDA_ERR_WORKSPACE", entry="kda_fwd_noalloc")
    b["q"] = T([1, 8192, hv + 1, 64])
    expect(lib, b, "KDA_ERR_UNSUPPORTED", entry="kda_fwd_noalloc")
    expect(lib, good(), "KDA_ERR_VALUE", scale=-1.0, entry="kda_fwd_noalloc")
    # an empty problem needs no scratch and no launch
    c = good(B=1, T_=0)
    for key in ("q", "k", "v", "g", "beta", "out"):
        c[key].data = None
    expect(lib, c, "KDA_OK", entry="kda_fwd_noalloc")


def test_trace_requires_descriptor(lib):
    a = good()
    r = ctypes.byref
    st = lib.kda_fwd_trace(r(a["q"]), r(a["k"]), r(a["v"]), r(a["g"]), r(a["beta"]), 0.1, None, None,
                           r(a["out"]), None, None, 0, None, None)
    assert binding.STATUS_NAMES[st] == "KDA_ERR_NULL"


def test_workspace_size(lib):
    # one 61,952-byte record per (64-token slot, value head): 12 fp16 operand
    # fragments of 64 lanes x 16 bytes (Aqk, T diag beta), three fp16 64x128
    # operands, 128 fp32; N extra slots for the partial chunks of sequences that
    # start mid-slot
    rec = 12 * 64 * 16 + 3 * 64 * 128 * 2 + 128 * 4
    assert rec == 61952
    assert lib.kda_fwd_workspace_size(2 * 8192, 2, 64) == (256 + 2) * 64 * rec
    assert lib.kda_fwd_workspace_size(16384, 14, 64) == (256 + 14) * 64 * rec
    assert lib.kda_fwd_workspace_size(1, 1, 1) == 2 * rec
    assert lib.kda_fwd_workspace_size(0, 0, 64) == 0
    assert lib.kda_fwd_workspace_size(-1, 1, 1) == -1


def test_workspace_checked_before_launch(lib):
    a = good(B=2, T_=100, Hv=4)
    need = lib.kda_fwd_workspace_size(200, 2, 4)
    expect(lib, a, "KDA_ERR_WORKSPACE", ws=FAKE, ws_size=need - 1)
    expect(lib, a, "KDA_ERR_WORKSPACE", ws=FAKE + 8, ws_size=need)
    expect(lib, a, "KDA_ERR_WORKSPACE", ws=None, ws_size=need)   # kda_fwd_ws requires one
    # a lone stage needs the caller's workspace
    r = lambda d: None if d is None else ctypes.byref(d)  # noqa: E731
    for entry in (lib.kda_fwd_intra, lib.kda_fwd_scan):
        st = entry(r(a["q"]), r(a["k"]), r(a["v"]), r(a["g"]), r(a["beta"]), 0.088, None, None, r(a["out"]), None,
                   None, 0, None)
        assert binding.STATUS_NAMES[st] == "KDA_ERR_WORKSPACE"
    # the workspace is checked after the tensors
    b = good(B=2, T_=100, Hv=4)
    b["q"] = T([2, 100, 2, 64])
    expect(lib, b, "KDA_ERR_UNSUPPORTED", ws=FAKE, ws_size=0)


# ---- kda_decode ----

def good_decode(N=2, Hq=2, Hv=4, beta_dtype=binding.KDA_F32, state=True):
    return dict(q=T([N, Hq, 128]), k=T([N, Hq, 128]), v=T([N, Hv, 128]), g=T([N, Hv, 128], binding.KDA_F32),
                beta=T([N, Hv], beta_dtype), s_in=T([N, Hv, 128, 128], binding.KDA_F32) if state else None,
                s_out=T([N, Hv, 128, 128], binding.KDA_F32), out=T([N, Hv, 128]))


def call_decode(lib, a, scale=0.088):
    r = lambda d: None if d is None else ctypes.byref(d)  # noqa: E731
    return lib.kda_decode(r(a.get("q")), r(a.get("k")), r(a.get("v")), r(a.get("g")), r(a.get("beta")), scale,
                          r(a.get("s_in")), r(a.get("s_out")), r(a.get("out")), None)


def expect_decode(lib, a, name, **kw):
    st = call_decode(lib, a, **kw)
    assert binding.STATUS_NAMES[st] == name, (binding.STATUS_NAMES[st], name)


def test_decode_rejects_bad_arguments(lib):
    for key in ("q", "k", "v", "g", "beta", "s_out", "out"):
        a = good_decode()
        a[key] = None
        expect_decode(lib, a, "KDA_ERR_NULL")
    a = good_decode()
    a["g"] = T([2, 4, 128], binding.KDA_BF16)
    expect_decode(lib, a, "KDA_ERR_DTYPE")
    a = good_decode()
    a["s_in"] = T([2, 4, 128, 128], binding.KDA_BF16)
    expect_decode(lib, a, "KDA_ERR_DTYPE")
    a = good_decode()
    a["v"] = T([3, 4, 128])
    expect_decode(lib, a, "KDA_ERR_SHAPE")
    a = good_decode()
    a["beta"] = T([2, 3], binding.KDA_F32)
    expect_decode(lib, a, "KDA_ERR_SHAPE")
    a = good_decode()
    a["s_out"] = T([2, 4, 128, 64], binding.KDA_F32)
    expect_decode(lib, a, "KDA_ERR_SHAPE")
    a = good_decode(Hq=3, Hv=4)
    expect_decode(lib, a, "KDA_ERR_UNSUPPORTED")
    a = good_decode()
    a["q"] = T([2, 2, 64])
    a["k"] = T([2, 2, 64])
    expect_decode(lib, a, "KDA_ERR_UNSUPPORTED")
    a = good_decode()
    a["out"] = T([2, 4, 128], data=FAKE + 8)
    expect_decode(lib, a, "KDA_ERR_LAYOUT")
    for s in (0.0, -1.0, float("nan")):
        expect_decode(lib, good_decode(), "KDA_ERR_VALUE", scale=s)


def test_decode_rejects_partly_overlapping_states(lib):
    a = good_decode()
    a["s_out"] = T([2, 4, 128, 128], binding.KDA_F32, data=FAKE + 64 * 1024)
    expect_decode(lib, a, "KDA_ERR_LAYOUT")


def test_decode_empty_batch_needs_no_launch(lib):
    a = good_decode(N=0)
    for key in a:
        if a[key] is not None:
            a[key].data = None
    expect_decode(lib, a, "KDA_OK")


# ---- kda_fwd_cp ----

def call_cp(lib, a, seg, first=0, scale=0.088, h0=None, hT=None, ws=None, ws_size=0, cu=None):
    r = lambda d: None if d is None else ctypes.byref(d)  # noqa: E731
    return lib.kda_fwd_cp(r(a.get("q")), r(a.get("k")), r(a.get("v")), r(a.get("g")), r(a.get("beta")), scale,
                          r(cu), r(h0), r(a.get("out")), r(hT), seg, first, ws, ws_size, None)


def test_cp_workspace_size(lib):
    rec = 61952
    # fewer than three segments: kda_fwd's workspace
    assert lib.kda_fwd_cp_workspace_size(2, 1000, 4, 8, 0) == lib.kda_fwd_workspace_size(2000, 2, 4)
    assert lib.kda_fwd_cp_workspace_size(2, 8192, 4, 16, 120) == lib.kda_fwd_workspace_size(16384, 2, 4)
    # B=2, T=8192 (128 chunks), Hv=8, 16 chunks per segment: P = 8
    B, T, H, P = 2, 8192, 8, 8
    blk = B * H * 128 * 128 * 4

    def expect(P):
        recs = ((B * T + 63) // 64 + B * P) * H * rec
        return (recs + 255) // 256 * 256 + 2 * (P - 2) * blk + (P - 1) * blk
    assert lib.kda_fwd_cp_workspace_size(B, T, H, 16, 0) == expect(8)
    assert lib.kda_fwd_cp_workspace_size(B, T, H, 16, 16) == expect(8)
    # a first segment of 32 chunks, then 16 each: 1 + ceil(96 / 16) = 7 segments
    assert lib.kda_fwd_cp_workspace_size(B, T, H, 16, 32) == expect(7)
    # a partial last segment counts: 1000 tokens = 16 chunks, 5 per segment -> 4 segments
    assert lib.kda_fwd_cp_workspace_size(1, 1000, 2, 5, 0) > lib.kda_fwd_workspace_size(1000, 1, 2)
    for bad in ((-1, 10, 2, 1, 0), (1, -1, 2, 1, 0), (1, 10, -2, 1, 0), (1, 10, 2, 0, 0), (1, 10, 2, 1, -1)):
        assert lib.kda_fwd_cp_workspace_size(*bad) == -1


def test_cp_checked_before_launch(lib):
    a = good(B=2, T_=1024)   # 16 chunks
    st = lambda: T([2, 2, 128, 128], binding.KDA_F32)  # noqa: E731
    for seg, first in ((0, 0), (-3, 0), (4, -1)):
        assert binding.STATUS_NAMES[call_cp(lib, a, seg, first, ws=FAKE, ws_size=1 << 40)] == "KDA_ERR_VALUE"
    # segmented (4 segments): the workspace is required and sized by kda_fwd_cp_workspace_size
    need = lib.kda_fwd_cp_workspace_size(2, 1024, 2, 4, 0)
    assert binding.STATUS_NAMES[call_cp(lib, a, 4)] == "KDA_ERR_WORKSPACE"
    assert binding.STATUS_NAMES[call_cp(lib, a, 4, ws=FAKE, ws_size=need - 1)] == "KDA_ERR_WORKSPACE"
    assert binding.STATUS_NAMES[call_cp(lib, a, 4, ws=FAKE + 8, ws_size=need)] == "KDA_ERR_WORKSPACE"
    need2 = lib.kda_fwd_cp_workspace_size(2, 1024, 2, 3, 6)   # 6 + 3 + 3 + 3 + 1 chunks: 5 segments
    assert binding.STATUS_NAMES[call_cp(lib, a, 3, 6, ws=FAKE, ws_size=need2 - 1)] == "KDA_ERR_WORKSPACE"
    # the tensor checks of kda_fwd come first
    b = good(B=2, T_=1024)
    b["q"] = T([2, 1024, 2, 64])
    assert binding.STATUS_NAMES[call_cp(lib, b, 4, ws=FAKE, ws_size=need)] == "KDA_ERR_UNSUPPORTED"
    assert binding.STATUS_NAMES[call_cp(lib, a, 4, h0=st(), hT=T([2, 2, 128, 128], binding.KDA_F32,
                                                                  data=FAKE + 4096))] == "KDA_ERR_LAYOUT"
    for s in (0.0, float("nan")):
        assert binding.STATUS_NAMES[call_cp(lib, a, 4, scale=s, ws=FAKE, ws_size=need)] == "KDA_ERR_VALUE"


def plan(lib, B, T, H, cus=256):
    seg, first = ctypes.c_int64(-1), ctypes.c_int64(-1)
    ok = lib.kda_fwd_cp_plan(B, T, H, cus, ctypes.byref(seg), ctypes.byref(first))
    return ok, seg.value, first.value


def test_cp_plan(lib):
    # a batch that fills the GPU, or short sequences: the ordinary path, zeros written
    assert plan(lib, 2, 8192, 64) == (0, 0, 0)
    assert plan(lib, 1, 1024, 8) == (0, 0, 0)
    assert plan(lib, 1, 4096, 64) == (0, 0, 0)   # grouped values with 64 value heads: measured no gain
    # few heads, long sequences: at least three segments, the first no shorter than the others
    for B, T, H in ((1, 65536, 8), (2, 8192, 8), (1, 32768, 16)):
        ok, L, L0 = plan(lib, B, T, H)
        nch = T // 64
        assert ok == 1 and L >= 1 and L0 >= L, (B, T, H, L, L0)
        assert nch > L0 and 1 + -(-(nch - L0) // L) >= 3, (B, T, H, L, L0)
    for bad in ((0, 8192, 8, 256), (1, 0, 8, 256), (1, 8192, 0, 256), (1, 8192, 8, 0)):
        assert plan(lib, *bad) == (0, 0, 0)
    # NULL outputs are allowed
    assert lib.kda_fwd_cp_plan(1, 65536, 8, 256, None, None) == 1


# ---- kda_bwd ----

def good_bwd(B=2, T_=100, Hq=2, Hv=4, beta_dtype=binding.KDA_F32, h0=True, dh0=True):
    F = binding.KDA_F32
    return dict(q=T([B, T_, Hq, 128]), k=T([B, T_, Hq, 128]), v=T([B, T_, Hv, 128]), g=T([B, T_, Hv, 128], F),
                beta=T([B, T_, Hv], beta_dtype), h0=T([B, Hv, 128, 128], F) if h0 else None,
                do=T([B, T_, Hv, 128]), dhT=T([B, Hv, 128, 128], F), dq=T([B, T_, Hq, 128], F),
                dk=T([B, T_, Hq, 128], F), dv=T([B, T_, Hv, 128], F), dg=T([B, T_, Hv, 128], F),
                dbeta=T([B, T_, Hv], F), dh0=T([B, Hv, 128, 128], F) if dh0 else None)


BWD_ARGS = ("q", "k", "v", "g", "beta")
BWD_REST = ("cu", "h0", "do", "dhT", "dq", "dk", "dv", "dg", "dbeta", "dh0")


def call_bwd(lib, a, scale=0.088, ws=None, ws_size=0):
    r = lambda d: None if d is None else ctypes.byref(d)  # noqa: E731
    return lib.kda_bwd(*[r(a.get(n)) for n in BWD_ARGS], scale, *[r(a.get(n)) for n in BWD_REST], ws, ws_size,
                       None)


def expect_bwd(lib, a, name, **kw):
    st = call_bwd(lib, a, **kw)
    assert binding.STATUS_NAMES[st] == name, (binding.STATUS_NAMES[st], name)


def test_bwd_workspace_size(lib):
    unit = 20480 * 4 + 2 * 128 * 128 * 4
    # (total tokens, sequences, Hq, Hv): ceil(total / 64) + N chunk slots per value head
    assert lib.kda_bwd_workspace_size(2 * 8192, 2, 64, 64) == (256 + 2) * 64 * unit
    # grouped value heads add dq and dk per value head; partial chunks count whole
    assert lib.kda_bwd_workspace_size(100, 1, 2, 4) == (2 + 1) * 4 * unit + 2 * 100 * 4 * 512
    assert lib.kda_bwd_workspace_size(1000, 14, 4, 4) == (16 + 14) * 4 * unit
    assert lib.kda_bwd_workspace_size(0, 3, 1, 1) == 0
    assert lib.kda_bwd_workspace_size(-1, 10, 1, 1) == -1
    assert lib.kda_bwd_workspace_size(10, -1, 1, 1) == -1
    assert lib.kda_bwd_workspace_size(10, 1, 0, 1) == -1


def test_bwd_rejects_bad_arguments(lib):
    for key in BWD_ARGS + ("do", "dq", "dk", "dv", "dg", "dbeta"):
        a = good_bwd()
        a[key] = None
        expect_bwd(lib, a, "KDA_ERR_NULL")
    for key in ("dq", "dv", "dg", "dbeta", "dh0", "dhT", "h0"):   # fp32 only
        a = good_bwd()
        a[key].dtype = binding.KDA_BF16
        expect_bwd(lib, a, "KDA_ERR_DTYPE")
    a = good_bwd()
    a["do"].dtype = binding.KDA_F32
    expect_bwd(lib, a, "KDA_ERR_DTYPE")
    for key, shape in (("dq", [2, 100, 4, 128]), ("dv", [2, 100, 2, 128]), ("dg", [2, 99, 4, 128]),
                       ("dbeta", [2, 100, 2]), ("do", [2, 100, 4, 64]), ("dh0", [2, 4, 128, 64]),
                       ("dhT", [1, 4, 128, 128]), ("h0", [2, 2, 128, 128])):
        a = good_bwd()
        a[key] = T(shape, a[key].dtype)
        expect_bwd(lib, a, "KDA_ERR_SHAPE")
    expect_bwd(lib, good_bwd(Hq=3, Hv=4), "KDA_ERR_UNSUPPORTED")
    a = good_bwd()
    a["dv"] = T([2, 100, 4, 128], binding.KDA_F32, data=FAKE + 8)
    expect_bwd(lib, a, "KDA_ERR_LAYOUT")
    for s in (0.0, -1.0, float("inf")):
        expect_bwd(lib, good_bwd(), "KDA_ERR_VALUE", scale=s)
    need = lib.kda_bwd_workspace_size(2 * 100, 2, 2, 4)
    expect_bwd(lib, good_bwd(), "KDA_ERR_WORKSPACE", ws=FAKE, ws_size=need - 1)
    expect_bwd(lib, good_bwd(), "KDA_ERR_WORKSPACE", ws=FAKE + 16, ws_size=need)


def test_bwd_rejects_bad_packed_batches(lib):
    I32 = binding.KDA_I32
    a = good_bwd()                       # cu_seqlens needs a single packed row
    a["cu"] = T([3], I32, data=FAKE)
    expect_bwd(lib, a, "KDA_ERR_UNSUPPORTED")
    a = good_bwd(B=1, h0=False, dh0=False)
    a["dhT"] = None
    a["cu"] = T([4], binding.KDA_F32, data=FAKE)
    expect_bwd(lib, a, "KDA_ERR_DTYPE")
    a["cu"] = T([0], I32, data=FAKE)
    expect_bwd(lib, a, "KDA_ERR_SHAPE")
    # the states follow the number of sequences, N = len(cu) - 1, not B
    for key in ("h0", "dhT", "dh0"):
        a = good_bwd(B=1, h0=False, dh0=False)
        a["dhT"] = None
        a["cu"] = T([4], I32, data=FAKE)
        a[key] = T([1, 4, 128, 128], binding.KDA_F32)
        expect_bwd(lib, a, "KDA_ERR_SHAPE")
    # the workspace is sized by the slots of the packed sequences
    a = good_bwd(B=1, h0=False, dh0=False)
    a["dhT"] = None
    a["cu"] = T([4], I32, data=FAKE)
    need = lib.kda_bwd_workspace_size(100, 3, 2, 4)
    expect_bwd(lib, a, "KDA_ERR_WORKSPACE", ws=FAKE, ws_size=need - 1)
    # no sequences: nothing to compute, no launch
    a = good_bwd(B=1, h0=False, dh0=False)
    a["dhT"] = None
    a["cu"] = T([1], I32, data=FAKE)
    for key in ("h0", "dhT", "dh0"):
        a[key] = T([0, 4, 128, 128], binding.KDA_F32, data=None)
    expect_bwd(lib, a, "KDA_OK")


def test_bwd_empty_problem_needs_no_launch(lib):
    for a in (good_bwd(B=0), good_bwd(T_=0, dh0=False)):
        for key in a:
            if a[key] is not None and a[key].shape[0] * a[key].shape[1] == 0:
                a[key].data = None
        expect_bwd(lib, a, "KDA_OK")


def test_binding_refuses_host_tensors():
    # no CPU fallback: host tensors are rejected before the library is called
    import torch
    from gated_delta_rule_35_amd import kda_bwd, kda_decode
    q = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16)
    g = torch.zeros(1, 4, 1, 128)
    beta = torch.zeros(1, 4, 1)
    with pytest.raises(ValueError):
        kda_bwd(q, q, q, g, beta, 0.1, q)
    with pytest.raises(ValueError):
        kda_decode(q[:, 0], q[:, 0], q[:, 0], g[:, 0], beta[:, 0], 0.1, None)


def call_qg(lib, a, qg, scale=0.088):
    r = lambda d: None if d is None else ctypes.byref(d)  # noqa: E731
    return lib.kda_fwd_qg(r(a.get("q")), r(a.get("k")), r(a.get("v")), r(a.get("g")), r(a.get("beta")), scale,
                          None, None, r(a.get("out")), None, r(qg), None, 0, None)


def test_qg_output_is_checked_before_any_hip_call(lib):
    """kda_fwd_qg: a NULL qg, a qg of the wrong dtype or shape, a non-contiguous or
    misaligned one, or one that overlaps another tensor is refused on the host; the
    forward's own checks still apply."""
    name = lambda st: binding.STATUS_NAMES[st]  # noqa: E731
    qg_addr = FAKE + (1 << 30)
    assert name(call_qg(lib, good(), None)) == "KDA_ERR_NULL"
    assert name(call_qg(lib, good(), T([1, 64, 2, 128], binding.KDA_F32, data=qg_addr))) == "KDA_ERR_DTYPE"
    assert name(call_qg(lib, good(), T([1, 64, 4, 128], data=qg_addr))) == "KDA_ERR_SHAPE"
    assert name(call_qg(lib, good(), T([1, 64, 2], data=qg_addr))) == "KDA_ERR_SHAPE"
    assert name(call_qg(lib, good(), T([1, 64, 2, 128], data=qg_addr + 2))) == "KDA_ERR_LAYOUT"
    assert name(call_qg(lib, good(), T([1, 64, 2, 128], data=qg_addr,
                                       strides=[64 * 256, 128, 64 * 128, 1]))) == "KDA_ERR_LAYOUT"
    a = good()
    a["out"] = T([1, 64, 2, 128], data=qg_addr + 4096)   # out inside qg's bytes
    assert name(call_qg(lib, a, T([1, 64, 2, 128], data=qg_addr))) == "KDA_ERR_LAYOUT"
    a = good()
    a["v"] = None
    assert name(call_qg(lib, a, T([1, 64, 2, 128], data=qg_addr))) == "KDA_ERR_NULL"
    assert name(call_qg(lib, good(), T([1, 64, 2, 128], data=qg_addr), scale=-1.0)) == "KDA_ERR_VALUE"


def test_cp_packed_workspace_size_and_checks(lib):
    """Packed segmented calls: the workspace bound, and the checks before any HIP
    call (B must be 1 with cu_seqlens; the workspace is required, sized by
    kda_fwd_cp_packed_workspace_size and 256-byte aligned)."""
    rec, blk = 61952, 2 * 128 * 128 * 4
    # T = 2000 tokens, N = 3 sequences, Hv = 2, L = 4, L0 = 4: TC = 32 + 3 = 35 chunks at
    # most, 35 // 4 + min(3, 35 // 5) + 1 = 12 later segments, 15 segments, 48 slots
    size = lib.kda_fwd_cp_packed_workspace_size(2000, 3, 2, 4, 0)
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    lat, smax = 12, 15
    expect = al(48 * 2 * rec)
    expect = al(expect + 3 * lat * blk)
    expect = al(expect + (smax + 2) * 4)
    expect = al(expect + 3 * 24)
    expect = al(expect + lat * 24)
    expect = al(expect + lat * 24)
    expect = al(expect + lat * 24)
    expect = al(expect + 3 * 16)
    assert size == expect, (size, expect)
    for bad in ((-1, 3, 2, 4, 0), (10, -1, 2, 4, 0), (10, 3, -2, 4, 0), (10, 3, 2, 0, 0), (10, 3, 2, 4, -1)):
        assert lib.kda_fwd_cp_packed_workspace_size(*bad) == -1
    a = good(B=1, T_=2000)
    cu = T([4], binding.KDA_I32, data=FAKE + (1 << 28))
    assert binding.STATUS_NAMES[call_cp(lib, a, 4, cu=cu)] == "KDA_ERR_WORKSPACE"
    assert binding.STATUS_NAMES[call_cp(lib, a, 4, cu=cu, ws=FAKE, ws_size=size - 1)] == "KDA_ERR_WORKSPACE"
    assert binding.STATUS_NAMES[call_cp(lib, a, 4, cu=cu, ws=FAKE + 16, ws_size=size)] == "KDA_ERR_WORKSPACE"
    b = good(B=2, T_=1000)
    assert binding.STATUS_NAMES[call_cp(lib, b, 4, cu=cu, ws=FAKE, ws_size=1 << 40)] == "KDA_ERR_UNSUPPORTED"
    bad_cu = T([4], binding.KDA_F32, data=FAKE + (1 << 28))
    assert binding.STATUS_NAMES[call_cp(lib, a, 4, cu=bad_cu, ws=FAKE, ws_size=1 << 40)] == "KDA_ERR_DTYPE"
    st = T([2, 2, 128, 128], binding.KDA_F32)   # N = 3 sequences need [3, 2, 128, 128]
    assert binding.STATUS_NAMES[call_cp(lib, a, 4, cu=cu, h0=st, ws=FAKE, ws_size=1 << 40)] == "KDA_ERR_SHAPE"

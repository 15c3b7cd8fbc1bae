"""ctypes binding of libkda.so (argument marshalling only).

Names follow the C ABI in include/kda.h: kda_fwd, kda_fwd_ws, kda_fwd_noalloc,
kda_fwd_intra, kda_fwd_scan, kda_fwd_trace, kda_fwd_cp, kda_decode, kda_bwd and
their size queries, kda_status_string, kda_dv_slices.  Tensors are passed as
kda_tensor_t descriptors built from torch tensors (data pointer, dtype, shape,
strides); the stream is torch's current HIP stream unless one is given.  Where
an entry point takes a workspace, it is a uint8 device tensor the caller passes
or one taken here from torch's caching allocator.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda.so")
_lib = None

KDA_BF16, KDA_F16, KDA_F32, KDA_I32 = 0, 1, 2, 3
_DTYPES = {torch.bfloat16: KDA_BF16, torch.float16: KDA_F16, torch.float32: KDA_F32, torch.int32: KDA_I32}
STATUS_NAMES = ["KDA_OK", "KDA_ERR_NULL", "KDA_ERR_DTYPE", "KDA_ERR_SHAPE", "KDA_ERR_LAYOUT",
                "KDA_ERR_UNSUPPORTED", "KDA_ERR_VALUE", "KDA_ERR_HIP", "KDA_ERR_WORKSPACE"]
EXPORTED = ["kda_fwd", "kda_fwd_fused", "kda_fwd_ws", "kda_fwd_qg", "kda_fwd_noalloc", "kda_fwd_noalloc_max_bytes", "kda_fwd_intra",
            "kda_fwd_scan", "kda_fwd_trace", "kda_fwd_cp", "kda_decode", "kda_bwd", "kda_fwd_workspace_size",
            "kda_fwd_cp_workspace_size", "kda_fwd_cp_packed_workspace_size", "kda_fwd_cp_plan", "kda_bwd_workspace_size", "kda_status_string",
            "kda_dv_slices"]


class KdaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class KdaTrace(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("G", "Aqk", "Akk", "T", "W", "U", "v_new", "h")]


class KdaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status
        self.name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)


def library_path():
    return _LIB_PATH


def load_library(path=None):
    """Loads libkda.so; raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with gated_delta_rule_35_amd/build.py "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(p)
    tp = ctypes.POINTER(KdaTensor)
    lib.kda_fwd.argtypes = [tp, tp, tp, tp, tp, ctypes.c_float, tp, tp, tp, tp, ctypes.c_void_p]
    lib.kda_fwd.restype = ctypes.c_int
    lib.kda_fwd_fused.argtypes = lib.kda_fwd.argtypes
    lib.kda_fwd_fused.restype = ctypes.c_int
    lib.kda_fwd_noalloc.argtypes = lib.kda_fwd.argtypes
    lib.kda_fwd_noalloc.restype = ctypes.c_int
    lib.kda_fwd_noalloc_max_bytes.argtypes = []
    lib.kda_fwd_noalloc_max_bytes.restype = ctypes.c_int64
    lib.kda_fwd_ws.argtypes = [tp, tp, tp, tp, tp, ctypes.c_float, tp, tp, tp, tp, ctypes.c_void_p, ctypes.c_int64,
                               ctypes.c_void_p]
    lib.kda_fwd_ws.restype = ctypes.c_int
    for name in ("kda_fwd_intra", "kda_fwd_scan"):
        getattr(lib, name).argtypes = lib.kda_fwd_ws.argtypes
        getattr(lib, name).restype = ctypes.c_int
    lib.kda_fwd_qg.argtypes = [tp, tp, tp, tp, tp, ctypes.c_float, tp, tp, tp, tp, tp, ctypes.c_void_p,
                               ctypes.c_int64, ctypes.c_void_p]
    lib.kda_fwd_qg.restype = ctypes.c_int
    lib.kda_fwd_trace.argtypes = [tp, tp, tp, tp, tp, ctypes.c_float, tp, tp, tp, tp, ctypes.c_void_p,
                                  ctypes.c_int64, ctypes.POINTER(KdaTrace), ctypes.c_void_p]
    lib.kda_fwd_trace.restype = ctypes.c_int
    lib.kda_fwd_cp.argtypes = [tp, tp, tp, tp, tp, ctypes.c_float, tp, tp, tp, tp, ctypes.c_int64, ctypes.c_int64,
                               ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.kda_fwd_cp.restype = ctypes.c_int
    lib.kda_fwd_cp_workspace_size.argtypes = [ctypes.c_int64] * 5
    lib.kda_fwd_cp_workspace_size.restype = ctypes.c_int64
    lib.kda_fwd_cp_packed_workspace_size.argtypes = [ctypes.c_int64] * 5
    lib.kda_fwd_cp_packed_workspace_size.restype = ctypes.c_int64
    lib.kda_fwd_cp_plan.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                    ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    lib.kda_fwd_cp_plan.restype = ctypes.c_int32
    lib.kda_decode.argtypes = [tp, tp, tp, tp, tp, ctypes.c_float, tp, tp, tp, ctypes.c_void_p]
    lib.kda_decode.restype = ctypes.c_int
    lib.kda_bwd.argtypes = [tp, tp, tp, tp, tp, ctypes.c_float] + [tp] * 10 + [ctypes.c_void_p, ctypes.c_int64,
                                                                            ctypes.c_void_p]
    lib.kda_bwd.restype = ctypes.c_int
    lib.kda_bwd_workspace_size.argtypes = [ctypes.c_int64] * 4
    lib.kda_bwd_workspace_size.restype = ctypes.c_int64
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_dv_slices.argtypes = [ctypes.c_int64, ctypes.c_int64]
    lib.kda_dv_slices.restype = ctypes.c_int32
    lib.kda_fwd_workspace_size.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
    lib.kda_fwd_workspace_size.restype = ctypes.c_int64
    if path is None:
        _lib = lib
    return lib


def describe(t):
    """kda_tensor_t for a torch tensor (or None).  No copies and no checks: the C
    library validates dtype, shape, layout and alignment."""
    if t is None:
        return None
    d = KdaTensor()
    d.data = t.data_ptr() if t.numel() else None
    d.dtype = _DTYPES.get(t.dtype, 99)
    d.ndim = t.dim()
    if t.dim() > 4:
        raise ValueError("kda tensors have at most 4 dimensions")
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ref(d):
    return None if d is None else ctypes.byref(d)


def _stream_handle(stream, tensors):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    dev = next((t.device for t in tensors if t is not None and t.is_cuda), None)
    if dev is None:
        raise ValueError("kda_fwd needs its tensors on the GPU")
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check(lib, status):
    if status != 0:
        raise KdaError(status, lib.kda_status_string(status).decode())


def kda_dv_slices(num_sequences, num_value_heads):
    return int(load_library().kda_dv_slices(num_sequences, num_value_heads))


def kda_fwd_workspace_size(total_tokens, num_sequences, num_value_heads):
    return int(load_library().kda_fwd_workspace_size(total_tokens, num_sequences, num_value_heads))


def _workspace(workspace, q, v, cu_seqlens, stream):
    """(tensor, pointer, size) of a workspace argument: the given uint8 tensor, or
    a fresh one from torch's caching allocator of the size the library asks for.
    A fresh tensor is marked as used on an explicitly given stream, so the
    caching allocator does not hand it out again before that stream's work on it
    is done."""
    if workspace is None:
        if q.dim() != 4 or v.dim() != 4:
            return None, None, 0   # the C library rejects the shapes
        n = q.shape[0] if cu_seqlens is None else cu_seqlens.shape[0] - 1
        size = kda_fwd_workspace_size(q.shape[0] * q.shape[1], max(n, 0), v.shape[2])
        if size <= 0:
            return None, None, 0
        workspace = torch.empty(size, dtype=torch.uint8, device=v.device)
        if stream is not None and isinstance(stream, torch.cuda.Stream):
            workspace.record_stream(stream)
    return workspace, workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _call(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, stream, trace, workspace,
          entry):
    """One forward entry point.  Entries with a workspace argument (kda_fwd_ws,
    the stage calls, kda_fwd_trace) get `workspace` (None: allocated here);
    kda_fwd, kda_fwd_fused and kda_fwd_noalloc take none."""
    lib = load_library()
    tensors = (q, k, v, g, beta, cu_seqlens, initial_state, out, final_state)
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError(f"{entry} needs every tensor on the GPU")
    descs = [describe(t) for t in tensors]
    s = _stream_handle(stream, tensors)
    args = [_ref(descs[0]), _ref(descs[1]), _ref(descs[2]), _ref(descs[3]), _ref(descs[4]), float(scale),
            _ref(descs[5]), _ref(descs[6]), _ref(descs[7]), _ref(descs[8])]
    if entry in ("kda_fwd", "kda_fwd_fused", "kda_fwd_noalloc"):
        _check(lib, getattr(lib, entry)(*args, s))
        return
    _ws, ws_ptr, ws_size = _workspace(workspace, q, v, cu_seqlens, stream)
    args += [ws_ptr, ws_size]
    if trace is None:
        _check(lib, getattr(lib, entry)(*args, s))
    else:
        tr = KdaTrace(**{n: (t.data_ptr() if t is not None else None) for n, t in trace.items()})
        _check(lib, lib.kda_fwd_trace(*args, ctypes.byref(tr), s))


def _outputs(q, v, cu_seqlens, out, final_state):
    if out is None:
        out = torch.empty(v.shape, dtype=torch.bfloat16, device=v.device)
    if final_state is True:
        n = q.shape[0] if cu_seqlens is None else cu_seqlens.shape[0] - 1
        final_state = torch.empty((n, v.shape[2], q.shape[3], v.shape[3]), dtype=torch.float32, device=v.device)
    return out, final_state


def kda_fwd(q, k, v, g, beta, scale, cu_seqlens=None, initial_state=None, out=None, final_state=None,
            stream=None, workspace=None):
    """KDA forward.  Returns (out, final_state); allocates them when not given
    (final_state is allocated only when `final_state=True` is passed).
    Without `workspace` this is the C kda_fwd (the single-pass kernel on
    fixed-length batches that fill the device, else the two-pass kernels); with a
    uint8 device tensor of at least kda_fwd_workspace_size() bytes it is
    kda_fwd_ws (the two-pass kernels) on that workspace."""
    out, final_state = _outputs(q, v, cu_seqlens, out, final_state)
    entry = "kda_fwd" if workspace is None else "kda_fwd_ws"
    _call(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, stream, None, workspace, entry)
    return out, final_state


def kda_fwd_fused(q, k, v, g, beta, scale, cu_seqlens=None, initial_state=None, out=None, final_state=None,
                  stream=None):
    """The single-pass forward (C kda_fwd_fused).  Returns (out, final_state); out
    and final_state=True are allocated here when not given."""
    out, final_state = _outputs(q, v, cu_seqlens, out, final_state)
    _call(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, stream, None, None,
          "kda_fwd_fused")
    return out, final_state


def kda_fwd_ws(q, k, v, g, beta, scale, cu_seqlens=None, initial_state=None, out=None, final_state=None,
               stream=None, workspace=None):
    """The two-pass forward with a caller workspace (C kda_fwd_ws); `workspace`
    None takes one from torch's caching allocator.  Returns (out, final_state)."""
    out, final_state = _outputs(q, v, cu_seqlens, out, final_state)
    _call(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, stream, None, workspace,
          "kda_fwd_ws")
    return out, final_state


def kda_fwd_qg(q, k, v, g, beta, scale, cu_seqlens=None, initial_state=None, out=None, final_state=None,
               qg=None, stream=None, workspace=None):
    """The forward with its QG output (C kda_fwd_qg): q exp(G), G the chunk-local
    inclusive cumsum of g, bf16 of v's shape.  Returns (out, final_state, qg); out,
    qg and final_state=True are allocated here when not given.  Without
    `workspace` the C call allocates its records in stream order."""
    out, final_state = _outputs(q, v, cu_seqlens, out, final_state)
    if qg is None:
        qg = torch.empty(v.shape, dtype=torch.bfloat16, device=v.device)
    lib = load_library()
    tensors = (q, k, v, g, beta, cu_seqlens, initial_state, out, final_state, qg)
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("kda_fwd_qg needs every tensor on the GPU")
    descs = [describe(t) for t in tensors]
    s = _stream_handle(stream, tensors)
    ws_ptr, ws_size = None, 0
    if workspace is not None:
        _ws, ws_ptr, ws_size = _workspace(workspace, q, v, cu_seqlens, stream)
    _check(lib, lib.kda_fwd_qg(_ref(descs[0]), _ref(descs[1]), _ref(descs[2]), _ref(descs[3]), _ref(descs[4]),
                               float(scale), _ref(descs[5]), _ref(descs[6]), _ref(descs[7]), _ref(descs[8]),
                               _ref(descs[9]), ws_ptr, ws_size, s))
    return out, final_state, qg


def kda_fwd_noalloc(q, k, v, g, beta, scale, cu_seqlens=None, initial_state=None, out=None, final_state=None,
                    stream=None):
    """kda_fwd_ws on the library's static device scratch (C kda_fwd_noalloc):
    the C call allocates nothing.  Returns (out, final_state); out and
    final_state=True are allocated here when not given."""
    out, final_state = _outputs(q, v, cu_seqlens, out, final_state)
    _call(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, stream, None, None,
          "kda_fwd_noalloc")
    return out, final_state


def kda_fwd_noalloc_max_bytes():
    return int(load_library().kda_fwd_noalloc_max_bytes())


def kda_fwd_intra(q, k, v, g, beta, scale, workspace, cu_seqlens=None, initial_state=None, out=None,
                  final_state=None, stream=None):
    """First kernel of kda_fwd: fills `workspace` (a uint8 device tensor of at
    least kda_fwd_workspace_size() bytes)."""
    _call(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, stream, None, workspace,
          "kda_fwd_intra")


def kda_fwd_scan(q, k, v, g, beta, scale, workspace, cu_seqlens=None, initial_state=None, out=None,
                 final_state=None, stream=None):
    """Second kernel of kda_fwd: reads `workspace` (filled by kda_fwd_intra with
    the same arguments) and writes `out` and `final_state`."""
    _call(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, stream, None, workspace,
          "kda_fwd_scan")


def kda_fwd_trace(q, k, v, g, beta, scale, trace, cu_seqlens=None, initial_state=None, out=None,
                  final_state=None, stream=None, workspace=None):
    """kda_fwd that also fills the fp32 intermediate dumps in `trace`, a dict with
    any of the keys G, Aqk, Akk, T, W, U, v_new, h (see include/kda.h)."""
    out, final_state = _outputs(q, v, cu_seqlens, out, final_state)
    _call(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, stream, trace, workspace,
          "kda_fwd_trace")
    return out, final_state


def kda_fwd_cp_workspace_size(batch, seq_len, num_value_heads, segment_chunks, first_segment_chunks=0):
    return int(load_library().kda_fwd_cp_workspace_size(batch, seq_len, num_value_heads, segment_chunks,
                                                        first_segment_chunks))


def kda_fwd_cp_packed_workspace_size(total_tokens, num_sequences, num_value_heads, segment_chunks,
                                     first_segment_chunks=0):
    return int(load_library().kda_fwd_cp_packed_workspace_size(total_tokens, num_sequences, num_value_heads,
                                                               segment_chunks, first_segment_chunks))


def kda_fwd_cp_plan(batch, seq_len, num_value_heads, num_cus=None):
    """(segment_chunks, first_segment_chunks) for kda_fwd_cp, or None when kda_fwd
    is about as fast.  num_cus defaults to the current GPU's compute units."""
    if num_cus is None:
        num_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    seg, first = ctypes.c_int64(0), ctypes.c_int64(0)
    ok = load_library().kda_fwd_cp_plan(batch, seq_len, num_value_heads, num_cus, ctypes.byref(seg),
                                        ctypes.byref(first))
    return (int(seg.value), int(first.value)) if ok else None


def kda_fwd_cp(q, k, v, g, beta, scale, segment_chunks, first_segment_chunks=0, initial_state=None, out=None,
               final_state=None, stream=None, workspace=None, cu_seqlens=None):
    """kda_fwd with each sequence cut into segments (the first of
    `first_segment_chunks` chunks, 0: `segment_chunks`, the others of
    `segment_chunks`) that the scan walks side by side (see include/kda.h); a
    fixed-length batch, or packed sequences with `cu_seqlens`.  Returns (out,
    final_state); final_state=True allocates it.  `workspace`: a uint8 device
    tensor of at least kda_fwd_cp_workspace_size() (fixed length) or
    kda_fwd_cp_packed_workspace_size() bytes (packed), or None (allocated here
    from torch's caching allocator)."""
    lib = load_library()
    if out is None:
        out = torch.empty(v.shape, dtype=torch.bfloat16, device=v.device)
    n_seq = q.shape[0] if cu_seqlens is None else cu_seqlens.shape[0] - 1
    if final_state is True:
        final_state = torch.empty((n_seq, v.shape[2], q.shape[3], v.shape[3]), dtype=torch.float32,
                                  device=v.device)
    tensors = (q, k, v, g, beta, cu_seqlens, initial_state, out, final_state)
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("kda_fwd_cp needs every tensor on the GPU")
    descs = [describe(t) for t in tensors]
    s = _stream_handle(stream, tensors)
    if workspace is None and q.dim() == 4 and v.dim() == 4:
        L, L0 = max(int(segment_chunks), 1), max(int(first_segment_chunks), 0)
        if cu_seqlens is None:
            size = kda_fwd_cp_workspace_size(q.shape[0], q.shape[1], v.shape[2], L, L0)
        else:
            size = kda_fwd_cp_packed_workspace_size(q.shape[0] * q.shape[1], max(n_seq, 0), v.shape[2], L, L0)
        workspace = torch.empty(max(size, 0), dtype=torch.uint8, device=v.device)
        if stream is not None and isinstance(stream, torch.cuda.Stream):
            workspace.record_stream(stream)
    ws_ptr = workspace.data_ptr() if workspace is not None and workspace.numel() else None
    ws_size = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib, lib.kda_fwd_cp(_ref(descs[0]), _ref(descs[1]), _ref(descs[2]), _ref(descs[3]), _ref(descs[4]),
                               float(scale), _ref(descs[5]), _ref(descs[6]), _ref(descs[7]), _ref(descs[8]),
                               int(segment_chunks), int(first_segment_chunks), ws_ptr, ws_size, s))
    return out, final_state


def kda_decode(q, k, v, g, beta, scale, state, out=None, new_state=None, stream=None):
    """One recurrent step for a batch of single tokens (q, k [N, Hq, 128]; v, g
    [N, Hv, 128]; beta [N, Hv]).  `state` [N, Hv, 128, 128] fp32 or None (a zero
    state); the new state goes to `new_state`, by default `state` itself (updated
    in place; allocated when state is None).  Returns (out, new_state)."""
    lib = load_library()
    if out is None:
        out = torch.empty(v.shape, dtype=torch.bfloat16, device=v.device)
    if new_state is None:
        new_state = state if state is not None else torch.empty(
            (v.shape[0], v.shape[1], q.shape[2], v.shape[2]), dtype=torch.float32, device=v.device)
    tensors = (q, k, v, g, beta, state, new_state, out)
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("kda_decode needs every tensor on the GPU")
    descs = [describe(t) for t in tensors]
    s = _stream_handle(stream, tensors)
    _check(lib, lib.kda_decode(_ref(descs[0]), _ref(descs[1]), _ref(descs[2]), _ref(descs[3]), _ref(descs[4]),
                               float(scale), _ref(descs[5]), _ref(descs[6]), _ref(descs[7]), s))
    return out, new_state


def kda_bwd_workspace_size(total_tokens, num_sequences, num_qk_heads, num_value_heads):
    """Bytes of device workspace kda_bwd needs for total_tokens = B * T tokens in
    num_sequences sequences (B, or N with cu_seqlens); see include/kda.h."""
    return int(load_library().kda_bwd_workspace_size(total_tokens, num_sequences, num_qk_heads, num_value_heads))


def kda_bwd(q, k, v, g, beta, scale, d_out, initial_state=None, d_final_state=None, grads=None,
            d_initial_state=False, stream=None, workspace=None, cu_seqlens=None):
    """Gradients of the forward: q, k [B, T, Hq, 128] and v, d_out [B, T, Hv, 128]
    bf16; g [B, T, Hv, 128] fp32; beta [B, T, Hv]; cu_seqlens (int32 [N + 1], B = 1)
    packs N sequences into the row, else N = B.  Returns a dict with dq, dk, dv, dg,
    dbeta (fp32, the inputs' shapes) and dh0 ([N, Hv, 128, 128] fp32 when
    d_initial_state is True or a tensor, else None).  `grads` may hold preallocated
    outputs under those names."""
    lib = load_library()
    B, T, Hq, _ = q.shape
    Hv = v.shape[2]
    N = B if cu_seqlens is None else cu_seqlens.shape[0] - 1
    dev = v.device
    out = dict(grads or {})
    f32 = torch.float32
    for name, shape in (("dq", q.shape), ("dk", q.shape), ("dv", v.shape), ("dg", g.shape), ("dbeta", beta.shape)):
        if out.get(name) is None:
            out[name] = torch.empty(shape, dtype=f32, device=dev)
    if isinstance(d_initial_state, torch.Tensor):
        out["dh0"] = d_initial_state
    elif d_initial_state:
        out["dh0"] = torch.empty((N, Hv, q.shape[3], v.shape[3]), dtype=f32, device=dev)
    else:
        out["dh0"] = None
    tensors = (q, k, v, g, beta, cu_seqlens, initial_state, d_out, d_final_state, out["dq"], out["dk"], out["dv"],
               out["dg"], out["dbeta"], out["dh0"])
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("kda_bwd needs every tensor on the GPU")
    descs = [describe(t) for t in tensors]
    s = _stream_handle(stream, tensors)
    ws, ws_size = (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    _check(lib, lib.kda_bwd(_ref(descs[0]), _ref(descs[1]), _ref(descs[2]), _ref(descs[3]), _ref(descs[4]),
                            float(scale), *[_ref(d) for d in descs[5:]], ws, ws_size, s))
    return out

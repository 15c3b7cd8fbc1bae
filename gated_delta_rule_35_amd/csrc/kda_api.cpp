// C-ABI front end of the KDA forward library: argument checks and launch.
//
// Every check runs on the host before any HIP call, so a rejected call enqueues
// nothing.  The number of sequences comes from the shape of cu_seqlens; the host
// never reads device memory and never synchronises.  The checks restate the
// input contract the pages describe for the public forward path ("cuLA PR #135",
// review of the KDA index helpers: chunk size and sorted cu_seqlens; "cuLA PR
// #131", review of the public forward: inputs made contiguous after validation).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>

#include "../../include/kda.h"
#include "kda_kernel.h"

namespace {

constexpr int64_t kHeadDim = 128;
constexpr int kIntra = 1, kScan = 2, kBoth = 3;   // which kernels a call launches
constexpr int64_t kMaxBlocks = int64_t(1) << 22;  // 512 threads each: a grid stays below 2^31 work-items

int64_t numel(const kda_tensor_t* t) {
    int64_t n = 1;
    for (int i = 0; i < t->ndim; ++i) n *= t->shape[i];
    return n;
}

size_t elem_size(kda_dtype_t d) { return (d == KDA_BF16 || d == KDA_F16) ? 2 : 4; }

bool contiguous(const kda_tensor_t* t) {
    int64_t expect = 1;
    for (int i = t->ndim - 1; i >= 0; --i) {
        if (t->shape[i] != 1 && t->stride[i] != expect) return false;
        expect *= t->shape[i];
    }
    return true;
}

kda_status_t check_tensor(const kda_tensor_t* t, int ndim, kda_dtype_t d0, kda_dtype_t d1, size_t align) {
    if (!t) return KDA_ERR_NULL;
    if (t->dtype != d0 && t->dtype != d1) return KDA_ERR_DTYPE;
    if (t->ndim != ndim) return KDA_ERR_SHAPE;
    for (int i = 0; i < ndim; ++i)
        if (t->shape[i] < 0) return KDA_ERR_SHAPE;
    const int64_t n = numel(t);
    if (n == 0) return KDA_OK;   // addresses no element: data and strides are not used
    if (!t->data) return KDA_ERR_NULL;
    if (!contiguous(t)) return KDA_ERR_LAYOUT;
    if ((reinterpret_cast<uintptr_t>(t->data) % align) != 0) return KDA_ERR_LAYOUT;
    return KDA_OK;
}

// Two state arrays of `bytes` each that share memory without starting at the
// same address.  A state may be updated in place, or written elsewhere; with a
// partial overlap one work-group's writes would land in tiles another has not
// read yet.
bool partly_overlap(const void* in, const void* out, int64_t bytes) {
    if (in == out || bytes <= 0) return false;
    const char* a = static_cast<const char*>(in);
    const char* b = static_cast<const char*>(out);
    return a < b + bytes && b < a + bytes;
}

// Two byte ranges that share memory (empty ranges share none).
bool ranges_overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    if (abytes <= 0 || bbytes <= 0 || !a || !b) return false;
    const char* x = static_cast<const char*>(a);
    const char* y = static_cast<const char*>(b);
    return x < y + bbytes && y < x + abytes;
}

bool same_shape(const kda_tensor_t* a, const int64_t* s, int nd) {
    for (int i = 0; i < nd; ++i)
        if (a->shape[i] != s[i]) return false;
    return true;
}

// Every host-side check of a forward call (tensors, shapes, sizes), and the kernel
// parameters it implies; the workspace is checked by the caller.
kda_status_t prepare(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v, const kda_tensor_t* g,
                     const kda_tensor_t* beta, float scale, const kda_tensor_t* cu, const kda_tensor_t* h0,
                     const kda_tensor_t* out, const kda_tensor_t* hT, kda::KdaParams& p, int64_t& B, int64_t& T,
                     int64_t& N) {
    kda_status_t st;
    if ((st = check_tensor(q, 4, KDA_BF16, KDA_BF16, 16)) != KDA_OK) return st;
    if ((st = check_tensor(k, 4, KDA_BF16, KDA_BF16, 16)) != KDA_OK) return st;
    if ((st = check_tensor(v, 4, KDA_BF16, KDA_BF16, 16)) != KDA_OK) return st;
    if ((st = check_tensor(g, 4, KDA_F32, KDA_F32, 16)) != KDA_OK) return st;
    if (!beta) return KDA_ERR_NULL;
    if ((st = check_tensor(beta, 3, KDA_BF16, KDA_F32, elem_size(beta->dtype))) != KDA_OK) return st;
    if ((st = check_tensor(out, 4, KDA_BF16, KDA_BF16, 16)) != KDA_OK) return st;
    if (cu && (st = check_tensor(cu, 1, KDA_I32, KDA_I32, 4)) != KDA_OK) return st;
    if (h0 && (st = check_tensor(h0, 4, KDA_F32, KDA_F32, 16)) != KDA_OK) return st;
    if (hT && (st = check_tensor(hT, 4, KDA_F32, KDA_F32, 16)) != KDA_OK) return st;

    B = q->shape[0];
    T = q->shape[1];
    const int64_t Hq = q->shape[2], Hv = v->shape[2];
    if (q->shape[3] != kHeadDim || v->shape[3] != kHeadDim) return KDA_ERR_UNSUPPORTED;
    if (!same_shape(k, q->shape, 4)) return KDA_ERR_SHAPE;
    if (v->shape[0] != B || v->shape[1] != T) return KDA_ERR_SHAPE;
    const int64_t gs[4] = {B, T, Hv, kHeadDim};
    if (!same_shape(g, gs, 4) || !same_shape(out, gs, 4)) return KDA_ERR_SHAPE;
    const int64_t bs[3] = {B, T, Hv};
    if (!same_shape(beta, bs, 3)) return KDA_ERR_SHAPE;
    if (Hq <= 0 || Hv <= 0) return KDA_ERR_SHAPE;
    if (Hv % Hq != 0) return KDA_ERR_UNSUPPORTED;
    N = B;
    if (cu) {
        if (B != 1) return KDA_ERR_UNSUPPORTED;
        if (cu->shape[0] < 1) return KDA_ERR_SHAPE;
        N = cu->shape[0] - 1;
    }
    const int64_t ss[4] = {N, Hv, kHeadDim, kHeadDim};
    if (h0 && !same_shape(h0, ss, 4)) return KDA_ERR_SHAPE;
    if (hT && !same_shape(hT, ss, 4)) return KDA_ERR_SHAPE;
    if (!std::isfinite(scale) || !(scale > 0.f)) return KDA_ERR_VALUE;
    if (h0 && hT && partly_overlap(h0->data, hT->data, N * Hv * kHeadDim * kHeadDim * 4)) return KDA_ERR_LAYOUT;
    // Per-block byte offsets of the kernel's buffer loads are 32-bit.
    if (Hv > (int64_t(1) << 16) || N > (int64_t(1) << 24)) return KDA_ERR_UNSUPPORTED;

    p = kda::KdaParams{};
    p.q = static_cast<const uint16_t*>(q->data);
    p.k = static_cast<const uint16_t*>(k->data);
    p.v = static_cast<const uint16_t*>(v->data);
    p.g = static_cast<const float*>(g->data);
    p.beta = beta->data;
    p.beta_f32 = beta->dtype == KDA_F32 ? 1 : 0;
    p.cu = cu ? static_cast<const int32_t*>(cu->data) : nullptr;
    p.h0 = h0 ? static_cast<const float*>(h0->data) : nullptr;
    p.o = static_cast<uint16_t*>(out->data);
    p.hT = hT ? static_cast<float*>(hT->data) : nullptr;
    p.T = T;
    p.N = static_cast<int32_t>(N);
    p.Hq = static_cast<int32_t>(Hq);
    p.Hv = static_cast<int32_t>(Hv);
    p.scale = scale;
    return KDA_OK;
}

kda_status_t finish(hipError_t e, hipStream_t hs) {
    if (e != hipSuccess) return KDA_ERR_HIP;
    if (std::getenv("KDA_DEBUG_SYNC")) {
        if (hipStreamSynchronize(hs) != hipSuccess) return KDA_ERR_HIP;
        if (hipGetLastError() != hipSuccess) return KDA_ERR_HIP;
    }
    return KDA_OK;
}

kda_status_t run(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v, const kda_tensor_t* g,
                 const kda_tensor_t* beta, float scale, const kda_tensor_t* cu, const kda_tensor_t* h0,
                 const kda_tensor_t* out, const kda_tensor_t* hT, void* workspace, int64_t workspace_size,
                 const kda_trace_t* trace, int stages, void* stream, const kda_tensor_t* qg = nullptr) {
    kda::KdaParams p;
    int64_t B, T, N;
    kda_status_t st = prepare(q, k, v, g, beta, scale, cu, h0, out, hT, p, B, T, N);
    if (st != KDA_OK) return st;
    if (qg) {
        // The optional QG output: v's shape, bf16, overlapping no input or output.
        if ((st = check_tensor(qg, 4, KDA_BF16, KDA_BF16, 16)) != KDA_OK) return st;
        const int64_t qs[4] = {B, T, (int64_t)p.Hv, kHeadDim};
        if (!same_shape(qg, qs, 4)) return KDA_ERR_SHAPE;
        const int64_t qb = B * T * p.Hv * kHeadDim * 2;
        const kda_tensor_t* others[] = {q, k, v, g, beta, out, h0, hT};
        for (const kda_tensor_t* t : others)
            if (t && ranges_overlap(qg->data, qb, t->data, numel(t) * (int64_t)elem_size(t->dtype)))
                return KDA_ERR_LAYOUT;
        p.qg = static_cast<uint16_t*>(qg->data);
    }
    const int64_t Hv = p.Hv;
    const int S = kda::scan_slices();
    if (N * Hv * S > kMaxBlocks) return KDA_ERR_UNSUPPORTED;
    const int64_t nslots = (B * T + 63) / 64 + N;
    if (nslots * Hv > kMaxBlocks) return KDA_ERR_UNSUPPORTED;
    const int64_t ws_need = kda::workspace_bytes(B * T, N, Hv);
    if (workspace && (workspace_size < ws_need || reinterpret_cast<uintptr_t>(workspace) % 16 != 0))
        return KDA_ERR_WORKSPACE;
    if (!workspace && stages != kBoth) return KDA_ERR_WORKSPACE;   // a lone stage needs the caller's workspace

    if (trace) {
        p.tr_G = trace->G;
        p.tr_Aqk = trace->Aqk;
        p.tr_Akk = trace->Akk;
        p.tr_T = trace->T;
        p.tr_W = trace->W;
        p.tr_U = trace->U;
        p.tr_vnew = trace->v_new;
        p.tr_h = trace->h;
    }
    p.nslots = nslots;
    if (N == 0 || (T == 0 && !hT)) return KDA_OK;  // nothing to compute or write
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    // Without a caller workspace the record array is allocated and released in
    // stream order around the two launches.
    void* ws = workspace;
    if (!ws && T > 0 && hipMallocAsync(&ws, (size_t)ws_need, hs) != hipSuccess) return KDA_ERR_HIP;
    p.ws = static_cast<char*>(ws);
    hipError_t e = hipSuccess;
    if (T > 0 && (stages & kIntra)) e = kda::launch_kda_intra(p, trace != nullptr, hs);
    if (e == hipSuccess && (stages & kScan)) e = kda::launch_kda_scan(p, trace != nullptr, hs);
    if (!workspace && ws && hipFreeAsync(ws, hs) != hipSuccess && e == hipSuccess) e = hipErrorUnknown;
    return finish(e, hs);
}

// ---- segmented forward ----
// Workspace of a segmented call: the records of all segments, then the segments'
// state maps M and offsets b (segments 1 .. P-2) and the states entering segments
// 1 .. P-1, each [segment][row][Hv][128][128] fp32.  With fewer than three
// segments the call is an ordinary forward and needs kda_fwd's workspace.
struct SegLayout {
    int64_t P = 0, rec = 0, maps = 0, total = 0;
};

// Segments per row: the first of first_chunks chunks, then seg_chunks each.
int64_t segment_count(int64_t nch, int64_t seg_chunks, int64_t first_chunks) {
    if (nch <= 0 || seg_chunks <= 0 || first_chunks <= 0) return 0;
    return nch <= first_chunks ? 1 : 1 + (nch - first_chunks + seg_chunks - 1) / seg_chunks;
}

SegLayout seg_layout(int64_t B, int64_t T, int64_t Hv, int64_t seg_chunks, int64_t first_chunks) {
    SegLayout c;
    const int64_t nch = (T + 63) / 64;
    c.P = segment_count(nch, seg_chunks, first_chunks);
    if (c.P < 3) {
        c.total = kda::workspace_bytes(B * T, B, Hv);
        return c;
    }
    const int64_t blk = B * Hv * kHeadDim * kHeadDim * 4;   // one segment's states
    c.rec = (kda::workspace_bytes(B * T, B * c.P, Hv) + 255) & ~int64_t(255);
    c.maps = blk * (c.P - 2);
    c.total = c.rec + 2 * c.maps + blk * (c.P - 1);
    return c;
}

// Workspace of a segmented call over packed sequences (planned on the device):
// the records of every segment, the maps M and offsets b of the middle segments
// and the states entering the later segments (each [lat_max][Hv][128][128] fp32),
// then the plan's tables.  Sizes are bounds: with TC = ceil(T / 64) + N chunks at
// most, there are at most TC / L + min(N, TC / (L0 + 1)) + 1 later segments.
struct PackedLayout {
    int64_t S_max = 0, lat_max = 0, nslots = 0;
    int64_t rec = 0, maps = 0, cu_seg = 0, first = 0, mid_m = 0, mid_b = 0, later = 0, chains = 0, total = 0;
};

PackedLayout packed_layout(int64_t T, int64_t N, int64_t Hv, int64_t L, int64_t L0) {
    PackedLayout c;
    auto al = [](int64_t x) { return (x + 255) & ~int64_t(255); };
    const int64_t tc = (T + 63) / 64 + N;
    c.lat_max = tc / L + std::min<int64_t>(N, tc / (L0 + 1)) + 1;
    c.S_max = N + c.lat_max;
    c.nslots = (T + 63) / 64 + c.S_max + 1;
    const int64_t blk = Hv * kHeadDim * kHeadDim * 4;   // one state
    int64_t o = al(kda::workspace_bytes(0, c.nslots, Hv));   // records: one per slot and value head
    c.rec = 0;
    c.maps = o;                       // M, then b, then the entering states
    o = al(o + 3 * c.lat_max * blk);
    c.cu_seg = o;
    o = al(o + (c.S_max + 2) * 4);
    const int64_t es = (int64_t)sizeof(kda::ScanEntry);
    c.first = o;
    o = al(o + N * es);
    c.mid_m = o;
    o = al(o + c.lat_max * es);
    c.mid_b = o;
    o = al(o + c.lat_max * es);
    c.later = o;
    o = al(o + c.lat_max * es);
    c.chains = o;
    o = al(o + N * 4 * 4);
    c.total = o;
    return c;
}

// Compute units of the current device, read once per device (concurrent first
// reads store the same value).  0 if the runtime cannot tell.
int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    int n = dev < 64 ? cus[dev].load(std::memory_order_relaxed) : 0;
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    if (dev < 64) cus[dev].store(n, std::memory_order_relaxed);
    return n;
}

// kda_fwd's choice of form: the single-pass kernel for fixed-length batches of at
// least 1024 tokens per row whose (sequence, value head, dv slice) work-groups
// cover every CU; there it beats the two-pass kernels by 5-10% (B=2 H=64, T=1024
// .. 8192) and needs no workspace.  With fewer work-groups than CUs, or packed
// sequences of unequal length, CUs would idle, and below 1024 tokens the two forms
// are even.
bool fused_fills_device(bool packed, int64_t T, int64_t work_groups) {
    if (packed || T < 1024 || work_groups > kMaxBlocks) return false;
    const int cus = device_cus();
    return cus > 0 && work_groups >= cus;
}

}  // namespace

extern "C" {

int32_t kda_dv_slices(int64_t num_sequences, int64_t num_value_heads) {
    (void)num_sequences;
    (void)num_value_heads;
    return kda::scan_slices();   // 64-wide dv slices
}

int64_t kda_fwd_workspace_size(int64_t total_tokens, int64_t num_sequences, int64_t num_value_heads) {
    if (total_tokens < 0 || num_sequences < 0 || num_value_heads < 0) return -1;
    return kda::workspace_bytes(total_tokens, num_sequences, num_value_heads);
}

kda_status_t kda_fwd(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v, const kda_tensor_t* g,
                     const kda_tensor_t* beta, float scale, const kda_tensor_t* cu_seqlens,
                     const kda_tensor_t* initial_state, const kda_tensor_t* out, const kda_tensor_t* final_state,
                     void* stream) {
    kda::KdaParams p;
    int64_t B, T, N;
    const kda_status_t st = prepare(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, p, B, T, N);
    if (st != KDA_OK) return st;
    if (fused_fills_device(cu_seqlens != nullptr, T, N * p.Hv * 2)) {
        const hipStream_t hs = static_cast<hipStream_t>(stream);
        return finish(kda::launch_kda_fused(p, hs), hs);
    }
    return run(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, nullptr, 0, nullptr, kBoth,
               stream);
}

kda_status_t kda_fwd_fused(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v,
                           const kda_tensor_t* g, const kda_tensor_t* beta, float scale,
                           const kda_tensor_t* cu_seqlens, const kda_tensor_t* initial_state,
                           const kda_tensor_t* out, const kda_tensor_t* final_state, void* stream) {
    kda::KdaParams p;
    int64_t B, T, N;
    kda_status_t st = prepare(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, p, B, T, N);
    if (st != KDA_OK) return st;
    if (N * p.Hv * 2 > kMaxBlocks) return KDA_ERR_UNSUPPORTED;
    if (N == 0 || (T == 0 && !final_state)) return KDA_OK;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    return finish(kda::launch_kda_fused(p, hs), hs);
}

kda_status_t kda_fwd_ws(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v, const kda_tensor_t* g,
                        const kda_tensor_t* beta, float scale, const kda_tensor_t* cu_seqlens,
                        const kda_tensor_t* initial_state, const kda_tensor_t* out, const kda_tensor_t* final_state,
                        void* workspace, int64_t workspace_size, void* stream) {
    if (!workspace) return KDA_ERR_WORKSPACE;
    return run(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, workspace, workspace_size,
               nullptr, kBoth, stream);
}

kda_status_t kda_fwd_qg(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v, const kda_tensor_t* g,
                        const kda_tensor_t* beta, float scale, const kda_tensor_t* cu_seqlens,
                        const kda_tensor_t* initial_state, const kda_tensor_t* out, const kda_tensor_t* final_state,
                        const kda_tensor_t* qg, void* workspace, int64_t workspace_size, void* stream) {
    if (!qg) return KDA_ERR_NULL;
    return run(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, workspace, workspace_size,
               nullptr, kBoth, stream, qg);
}

int64_t kda_fwd_noalloc_max_bytes(void) { return kda::NOALLOC_SCRATCH_BYTES; }

kda_status_t kda_fwd_noalloc(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v,
                             const kda_tensor_t* g, const kda_tensor_t* beta, float scale,
                             const kda_tensor_t* cu_seqlens, const kda_tensor_t* initial_state,
                             const kda_tensor_t* out, const kda_tensor_t* final_state, void* stream) {
    // Every host check first (as kda_fwd_ws), then the size limit; only then is the
    // device touched, to look up the scratch address.
    kda::KdaParams p;
    int64_t B, T, N;
    kda_status_t st = prepare(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, p, B, T, N);
    if (st != KDA_OK) return st;
    const int64_t need = kda::workspace_bytes(B * T, N, p.Hv);
    if (need > kda::NOALLOC_SCRATCH_BYTES) return KDA_ERR_WORKSPACE;
    if (N == 0 || (T == 0 && !final_state)) return KDA_OK;
    void* ws = nullptr;
    if (kda::noalloc_scratch(&ws) != hipSuccess) return KDA_ERR_HIP;
    return run(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, ws,
               kda::NOALLOC_SCRATCH_BYTES, nullptr, kBoth, stream);
}

kda_status_t kda_fwd_intra(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v,
                           const kda_tensor_t* g, const kda_tensor_t* beta, float scale,
                           const kda_tensor_t* cu_seqlens, const kda_tensor_t* initial_state,
                           const kda_tensor_t* out, const kda_tensor_t* final_state, void* workspace,
                           int64_t workspace_size, void* stream) {
    return run(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, workspace, workspace_size,
               nullptr, kIntra, stream);
}

kda_status_t kda_fwd_scan(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v,
                          const kda_tensor_t* g, const kda_tensor_t* beta, float scale,
                          const kda_tensor_t* cu_seqlens, const kda_tensor_t* initial_state,
                          const kda_tensor_t* out, const kda_tensor_t* final_state, void* workspace,
                          int64_t workspace_size, void* stream) {
    return run(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, workspace, workspace_size,
               nullptr, kScan, stream);
}

kda_status_t kda_fwd_trace(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v,
                           const kda_tensor_t* g, const kda_tensor_t* beta, float scale,
                           const kda_tensor_t* cu_seqlens, const kda_tensor_t* initial_state,
                           const kda_tensor_t* out, const kda_tensor_t* final_state, void* workspace,
                           int64_t workspace_size, const kda_trace_t* trace, void* stream) {
    if (!trace) return KDA_ERR_NULL;
    return run(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, workspace, workspace_size,
               trace, kBoth, stream);
}

int64_t kda_fwd_cp_workspace_size(int64_t batch, int64_t seq_len, int64_t num_value_heads, int64_t segment_chunks,
                                  int64_t first_segment_chunks) {
    if (batch < 0 || seq_len < 0 || num_value_heads < 0 || segment_chunks < 1 || first_segment_chunks < 0) return -1;
    const int64_t first = first_segment_chunks ? first_segment_chunks : segment_chunks;
    return seg_layout(batch, seq_len, num_value_heads, segment_chunks, first).total;
}

int32_t kda_fwd_cp_plan(int64_t batch, int64_t seq_len, int64_t num_value_heads, int32_t num_cus,
                        int64_t* segment_chunks, int64_t* first_segment_chunks) {
    if (segment_chunks) *segment_chunks = 0;
    if (first_segment_chunks) *first_segment_chunks = 0;
    if (batch <= 0 || seq_len <= 0 || num_value_heads <= 0 || num_cus <= 0) return 0;
    const int64_t nch = (seq_len + 63) / 64, per_seg = batch * num_value_heads * kda::scan_slices();
    if (per_seg >= num_cus) return 0;   // the ordinary scan already fills the GPU
    auto waves = [&](int64_t wgs, int64_t slots) { return (wgs + slots - 1) / slots; };
    // Cost in chunk steps.  Step 2: segment 0's pass holds per_seg CUs for its L0
    // chunks while the maps of segments 1 .. P-2 pass through the other CUs in
    // waves of L chunks (and through all of them once segment 0 is done); step 4:
    // the remaining segments in waves of L; plus one step per composed map and
    // eight for the extra launches.  The ordinary scan walks every chunk once.
    const int64_t base = nch;
    int64_t best_cost = base, best_L = 0, best_L0 = 0;
    for (int64_t L = 1; L <= nch; ++L) {
        for (int64_t m = 1; m <= 4; ++m) {
            const int64_t L0 = m * L, P = segment_count(nch, L, L0);
            if (P < 3 || P > 64) continue;
            const int64_t maps = 2 * per_seg * (P - 2);
            const int64_t beside = (L0 / L) * (num_cus - per_seg);   // map work-groups done within L0
            const int64_t step2 = maps <= beside ? L0 : L0 + L * waves(maps - beside, num_cus);
            const int64_t cost = step2 + L * waves(per_seg * (P - 1), num_cus) + (P - 2) + 8;
            if (cost < best_cost) {
                best_cost = cost;
                best_L = L;
                best_L0 = L0;
            }
        }
    }
    // Only when it saves a fifth or more: the model is coarse (the time of a chunk
    // step grows with the number of work-groups running), and a smaller predicted
    // saving measured as none (grouped values, B = 1, Hv = 64, T = 4096).
    if (5 * best_cost > 4 * base) return 0;
    if (segment_chunks) *segment_chunks = best_L;
    if (first_segment_chunks) *first_segment_chunks = best_L0;
    return 1;
}

int64_t kda_fwd_cp_packed_workspace_size(int64_t total_tokens, int64_t num_sequences, int64_t num_value_heads,
                                         int64_t segment_chunks, int64_t first_segment_chunks) {
    if (total_tokens < 0 || num_sequences < 0 || num_value_heads < 0 || segment_chunks < 1 || first_segment_chunks < 0)
        return -1;
    const int64_t first_chunks = first_segment_chunks ? first_segment_chunks : segment_chunks;
    return packed_layout(total_tokens, num_sequences, num_value_heads, segment_chunks, first_chunks).total;
}

kda_status_t kda_fwd_cp(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v, const kda_tensor_t* g,
                        const kda_tensor_t* beta, float scale, const kda_tensor_t* cu_seqlens,
                        const kda_tensor_t* initial_state, const kda_tensor_t* out, const kda_tensor_t* final_state,
                        int64_t segment_chunks, int64_t first_segment_chunks, void* workspace, int64_t workspace_size,
                        void* stream) {
    kda::KdaParams p;
    int64_t B, T, N;
    kda_status_t st = prepare(q, k, v, g, beta, scale, cu_seqlens, initial_state, out, final_state, p, B, T, N);
    if (st != KDA_OK) return st;
    if (segment_chunks < 1 || first_segment_chunks < 0) return KDA_ERR_VALUE;
    const int64_t first_chunks = first_segment_chunks ? first_segment_chunks : segment_chunks;
    if (cu_seqlens) {
        // Packed sequences: the segment boundaries depend on cu_seqlens, which the
        // host does not read; a plan kernel derives them (and every job's list)
        // on the device, within bounds the host computes from the shapes.
        const int64_t Hv = p.Hv;
        const PackedLayout c = packed_layout(T, N, Hv, segment_chunks, first_chunks);
        if (!workspace || workspace_size < c.total || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
            return KDA_ERR_WORKSPACE;
        const int S = kda::scan_slices();
        if (c.nslots * Hv > kMaxBlocks || (N + 2 * c.lat_max) * Hv * S > kMaxBlocks || c.S_max > (int64_t(1) << 24))
            return KDA_ERR_UNSUPPORTED;
        if (N == 0 || (T == 0 && !final_state)) return KDA_OK;
        char* ws = static_cast<char*>(workspace);
        const int64_t blk_f = Hv * kHeadDim * kHeadDim;
        kda::CpPlan pl{};
        pl.cu = static_cast<const int32_t*>(cu_seqlens->data);
        pl.N = static_cast<int32_t>(N);
        pl.T = T;
        pl.L = segment_chunks;
        pl.L0 = first_chunks;
        pl.hv_dd = blk_f;
        pl.h0 = p.h0;
        pl.hT = p.hT;
        pl.Mb = reinterpret_cast<float*>(ws + c.maps);
        pl.Bb = pl.Mb + c.lat_max * blk_f;
        pl.Hin = pl.Bb + c.lat_max * blk_f;
        pl.cu_seg = reinterpret_cast<int32_t*>(ws + c.cu_seg);
        pl.S_max = static_cast<int32_t>(c.S_max);
        pl.lat_max = static_cast<int32_t>(c.lat_max);
        pl.first = reinterpret_cast<kda::ScanEntry*>(ws + c.first);
        pl.mid_m = reinterpret_cast<kda::ScanEntry*>(ws + c.mid_m);
        pl.mid_b = reinterpret_cast<kda::ScanEntry*>(ws + c.mid_b);
        pl.later = reinterpret_cast<kda::ScanEntry*>(ws + c.later);
        pl.chains = reinterpret_cast<int32_t*>(ws + c.chains);
        const hipStream_t hs = static_cast<hipStream_t>(stream);
        hipError_t e = kda::launch_kda_cp_plan(pl, hs);
        // 1. intra kernel over every segment (record sequence = segment)
        kda::KdaParams ps = p;
        ps.cu = pl.cu_seg;
        ps.N = static_cast<int32_t>(c.S_max + 1);
        ps.nslots = c.nslots;
        ps.ws = ws + c.rec;
        ps.h0 = nullptr;
        ps.hT = nullptr;
        if (e == hipSuccess && T > 0) e = kda::launch_kda_intra(ps, false, hs);
        // 2. segment 0 of every sequence, and the maps of the middle segments
        kda::ScanJobs J1{};
        J1.njobs = 3;
        J1.job[0] = ps;
        J1.job[0].N = static_cast<int32_t>(N);
        J1.job[0].entries = pl.first;
        J1.job[1] = ps;
        J1.job[1].N = static_cast<int32_t>(c.lat_max);
        J1.job[1].entries = pl.mid_m;
        J1.job[1].h0_identity = 1;
        J1.job[1].v_zero = 1;
        J1.job[1].o = nullptr;
        J1.job[2] = ps;
        J1.job[2].N = static_cast<int32_t>(c.lat_max);
        J1.job[2].entries = pl.mid_b;
        J1.job[2].o = nullptr;
        if (e == hipSuccess) e = kda::launch_kda_scan_jobs(J1, hs);
        // 3. the states entering the later segments, per sequence
        if (e == hipSuccess)
            e = kda::launch_kda_compose_chains(pl.Mb, pl.Bb, pl.Hin, pl.chains, static_cast<int>(N),
                                               static_cast<int>(Hv), hs);
        // 4. every later segment from its entering state (the last one of a sequence
        //    writes its final state)
        kda::ScanJobs J2{};
        J2.njobs = 1;
        J2.job[0] = ps;
        J2.job[0].N = static_cast<int32_t>(c.lat_max);
        J2.job[0].entries = pl.later;
        if (e == hipSuccess) e = kda::launch_kda_scan_jobs(J2, hs);
        return finish(e, hs);
    }
    const int64_t Hv = p.Hv;
    const SegLayout c = seg_layout(B, T, Hv, segment_chunks, first_chunks);
    if (c.P < 3)   // one or two segments: nothing runs side by side; the ordinary path
        return run(q, k, v, g, beta, scale, nullptr, initial_state, out, final_state, workspace, workspace_size,
                   nullptr, kBoth, stream);
    if (!workspace || workspace_size < c.total || reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
        return KDA_ERR_WORKSPACE;
    const int64_t P = c.P, nseg = B * P;
    const int S = kda::scan_slices();
    if (nseg > (int64_t(1) << 24)) return KDA_ERR_UNSUPPORTED;
    const int64_t nslots = (B * T + 63) / 64 + nseg;
    if (nslots * Hv > kMaxBlocks || (B + 2 * B * (P - 2)) * Hv * S > kMaxBlocks) return KDA_ERR_UNSUPPORTED;

    char* ws = static_cast<char*>(workspace);
    float* Mb = reinterpret_cast<float*>(ws + c.rec);
    float* Bb = reinterpret_cast<float*>(ws + c.rec + c.maps);
    float* Hin = reinterpret_cast<float*>(ws + c.rec + 2 * c.maps);
    const int64_t blk_f = B * Hv * kHeadDim * kHeadDim;   // floats per segment of states
    p.ws = ws;
    p.seg_tokens = segment_chunks * 64;
    p.seg0_tokens = first_chunks * 64;
    p.seg_rows = static_cast<int32_t>(B);
    p.seg_per_row = static_cast<int32_t>(P);
    p.nslots = nslots;
    const hipStream_t hs = static_cast<hipStream_t>(stream);

    // 1. intra kernel over every segment of every row
    kda::KdaParams pi = p;
    pi.N = static_cast<int32_t>(nseg);
    hipError_t e = kda::launch_kda_intra(pi, false, hs);
    // 2. side by side: segment 0 of each row from the initial state (output and its
    //    final state), and the maps of segments 1 .. P-2: M from the identity with
    //    v = 0, b from zero with v
    kda::ScanJobs J1{};
    J1.njobs = 3;
    kda::KdaParams& j0 = J1.job[0];
    j0 = p;
    j0.N = static_cast<int32_t>(B);
    j0.seg_first = 0;
    j0.hT = Hin;
    kda::KdaParams& jm = J1.job[1];
    jm = p;
    jm.N = static_cast<int32_t>(B * (P - 2));
    jm.seg_first = 1;
    jm.h0 = nullptr;
    jm.h0_identity = 1;
    jm.v_zero = 1;
    jm.o = nullptr;
    jm.hT = Mb;
    kda::KdaParams& jb = J1.job[2];
    jb = p;
    jb.N = static_cast<int32_t>(B * (P - 2));
    jb.seg_first = 1;
    jb.h0 = nullptr;
    jb.o = nullptr;
    jb.hT = Bb;
    if (e == hipSuccess) e = kda::launch_kda_scan_jobs(J1, hs);
    // 3. the states entering segments 2 .. P-1
    if (e == hipSuccess)
        e = kda::launch_kda_compose(Mb, Bb, Hin, static_cast<int>(B), static_cast<int>(Hv), static_cast<int>(P - 2), hs);
    // 4. side by side: segments 1 .. P-1 from their entering states; the last one
    //    writes the final state
    kda::ScanJobs J2{};
    J2.njobs = 2;
    kda::KdaParams& ja = J2.job[0];
    ja = p;
    ja.N = static_cast<int32_t>(B * (P - 2));
    ja.seg_first = 1;
    ja.h0 = Hin;
    ja.hT = nullptr;
    kda::KdaParams& jz = J2.job[1];
    jz = p;
    jz.N = static_cast<int32_t>(B);
    jz.seg_first = static_cast<int32_t>(P - 1);
    jz.h0 = Hin + (P - 2) * blk_f;
    if (e == hipSuccess) e = kda::launch_kda_scan_jobs(J2, hs);
    return finish(e, hs);
}

kda_status_t kda_decode(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v, const kda_tensor_t* g,
                        const kda_tensor_t* beta, float scale, const kda_tensor_t* state_in,
                        const kda_tensor_t* state_out, const kda_tensor_t* out, void* stream) {
    kda_status_t st;
    if ((st = check_tensor(q, 3, KDA_BF16, KDA_BF16, 16)) != KDA_OK) return st;
    if ((st = check_tensor(k, 3, KDA_BF16, KDA_BF16, 16)) != KDA_OK) return st;
    if ((st = check_tensor(v, 3, KDA_BF16, KDA_BF16, 16)) != KDA_OK) return st;
    if ((st = check_tensor(g, 3, KDA_F32, KDA_F32, 16)) != KDA_OK) return st;
    if (!beta) return KDA_ERR_NULL;
    if ((st = check_tensor(beta, 2, KDA_BF16, KDA_F32, elem_size(beta->dtype))) != KDA_OK) return st;
    if ((st = check_tensor(out, 3, KDA_BF16, KDA_BF16, 16)) != KDA_OK) return st;
    if (state_in && (st = check_tensor(state_in, 4, KDA_F32, KDA_F32, 16)) != KDA_OK) return st;
    if ((st = check_tensor(state_out, 4, KDA_F32, KDA_F32, 16)) != KDA_OK) return st;

    const int64_t N = q->shape[0], Hq = q->shape[1], Hv = v->shape[1];
    if (q->shape[2] != kHeadDim || v->shape[2] != kHeadDim) return KDA_ERR_UNSUPPORTED;
    if (!same_shape(k, q->shape, 3)) return KDA_ERR_SHAPE;
    if (v->shape[0] != N) return KDA_ERR_SHAPE;
    const int64_t vs[3] = {N, Hv, kHeadDim};
    if (!same_shape(g, vs, 3) || !same_shape(out, vs, 3)) return KDA_ERR_SHAPE;
    const int64_t bs[2] = {N, Hv};
    if (!same_shape(beta, bs, 2)) return KDA_ERR_SHAPE;
    const int64_t ss[4] = {N, Hv, kHeadDim, kHeadDim};
    if (state_in && !same_shape(state_in, ss, 4)) return KDA_ERR_SHAPE;
    if (!same_shape(state_out, ss, 4)) return KDA_ERR_SHAPE;
    if (Hq <= 0 || Hv <= 0) return KDA_ERR_SHAPE;
    if (Hv % Hq != 0) return KDA_ERR_UNSUPPORTED;
    if (!std::isfinite(scale) || !(scale > 0.f)) return KDA_ERR_VALUE;
    if (N * Hv > (int64_t(1) << 31) - 1) return KDA_ERR_UNSUPPORTED;
    if (state_in && partly_overlap(state_in->data, state_out->data, N * Hv * kHeadDim * kHeadDim * 4))
        return KDA_ERR_LAYOUT;

    kda::DecodeParams p{};
    p.q = static_cast<const uint16_t*>(q->data);
    p.k = static_cast<const uint16_t*>(k->data);
    p.v = static_cast<const uint16_t*>(v->data);
    p.g = static_cast<const float*>(g->data);
    p.beta = beta->data;
    p.beta_f32 = beta->dtype == KDA_F32 ? 1 : 0;
    p.s_in = state_in ? static_cast<const float*>(state_in->data) : nullptr;
    p.s_out = static_cast<float*>(state_out->data);
    p.o = static_cast<uint16_t*>(out->data);
    p.N = static_cast<int32_t>(N);
    p.Hq = static_cast<int32_t>(Hq);
    p.Hv = static_cast<int32_t>(Hv);
    p.scale = scale;
    if (N == 0) return KDA_OK;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    return finish(kda::launch_kda_decode(p, hs), hs);
}

}  // extern "C"

// ---- backward ----
namespace {
// Workspace of kda_bwd, in 256-byte aligned blocks: the chunk operands (G, Aqk, T,
// Abar), the states entering the chunks, the state gradients leaving them, then,
// when Hq < Hv, dq and dk per value head.  Sized for ceil(total / 64) + N chunk
// slots per value head, which covers both chunk numberings of the kernels: B rows
// of ceil(T / 64) chunks, or the slots of N packed sequences.
struct BwdLayout {
    int64_t prep, hs, dhs, dqv, dkv, total;
};

BwdLayout bwd_layout(int64_t total_tokens, int64_t N, int64_t Hq, int64_t Hv) {
    auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
    const int64_t units = total_tokens > 0 ? ((total_tokens + 63) / 64 + N) * Hv : 0;
    BwdLayout L{};
    L.prep = 0;
    L.hs = L.prep + up(units * kda::BWP_FLOATS * 4);
    L.dhs = L.hs + up(units * kHeadDim * kHeadDim * 4);
    L.dqv = L.dhs + up(units * kHeadDim * kHeadDim * 4);
    const int64_t per = Hq < Hv ? up(total_tokens * Hv * kHeadDim * 4) : 0;
    L.dkv = L.dqv + per;
    L.total = L.dkv + per;
    return L;
}
}  // namespace

extern "C" {

int64_t kda_bwd_workspace_size(int64_t total_tokens, int64_t num_sequences, int64_t num_qk_heads,
                               int64_t num_value_heads) {
    if (total_tokens < 0 || num_sequences < 0 || num_qk_heads <= 0 || num_value_heads <= 0) return -1;
    return bwd_layout(total_tokens, num_sequences, num_qk_heads, num_value_heads).total;
}

kda_status_t kda_bwd(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v, const kda_tensor_t* g,
                     const kda_tensor_t* beta, float scale, const kda_tensor_t* cu_seqlens,
                     const kda_tensor_t* initial_state,
                     const kda_tensor_t* d_out, const kda_tensor_t* d_final_state, const kda_tensor_t* dq,
                     const kda_tensor_t* dk, const kda_tensor_t* dv, const kda_tensor_t* dg,
                     const kda_tensor_t* dbeta, const kda_tensor_t* d_initial_state, void* workspace,
                     int64_t workspace_size, void* stream) {
    kda_status_t st;
    if ((st = check_tensor(q, 4, KDA_BF16, KDA_BF16, 16)) != KDA_OK) return st;
    if ((st = check_tensor(k, 4, KDA_BF16, KDA_BF16, 16)) != KDA_OK) return st;
    if ((st = check_tensor(v, 4, KDA_BF16, KDA_BF16, 16)) != KDA_OK) return st;
    if ((st = check_tensor(g, 4, KDA_F32, KDA_F32, 16)) != KDA_OK) return st;
    if (!beta) return KDA_ERR_NULL;
    if ((st = check_tensor(beta, 3, KDA_BF16, KDA_F32, elem_size(beta->dtype))) != KDA_OK) return st;
    if (cu_seqlens && (st = check_tensor(cu_seqlens, 1, KDA_I32, KDA_I32, 4)) != KDA_OK) return st;
    if (initial_state && (st = check_tensor(initial_state, 4, KDA_F32, KDA_F32, 16)) != KDA_OK) return st;
    if ((st = check_tensor(d_out, 4, KDA_BF16, KDA_BF16, 16)) != KDA_OK) return st;
    if (d_final_state && (st = check_tensor(d_final_state, 4, KDA_F32, KDA_F32, 16)) != KDA_OK) return st;
    if ((st = check_tensor(dq, 4, KDA_F32, KDA_F32, 16)) != KDA_OK) return st;
    if ((st = check_tensor(dk, 4, KDA_F32, KDA_F32, 16)) != KDA_OK) return st;
    if ((st = check_tensor(dv, 4, KDA_F32, KDA_F32, 16)) != KDA_OK) return st;
    if ((st = check_tensor(dg, 4, KDA_F32, KDA_F32, 16)) != KDA_OK) return st;
    if ((st = check_tensor(dbeta, 3, KDA_F32, KDA_F32, 4)) != KDA_OK) return st;
    if (d_initial_state && (st = check_tensor(d_initial_state, 4, KDA_F32, KDA_F32, 16)) != KDA_OK) return st;

    const int64_t B = q->shape[0], T = q->shape[1], Hq = q->shape[2], Hv = v->shape[2];
    if (q->shape[3] != kHeadDim || v->shape[3] != kHeadDim) return KDA_ERR_UNSUPPORTED;
    if (!same_shape(k, q->shape, 4) || !same_shape(dq, q->shape, 4) || !same_shape(dk, q->shape, 4))
        return KDA_ERR_SHAPE;
    if (v->shape[0] != B || v->shape[1] != T) return KDA_ERR_SHAPE;
    const int64_t gs[4] = {B, T, Hv, kHeadDim};
    if (!same_shape(g, gs, 4) || !same_shape(d_out, gs, 4) || !same_shape(dv, gs, 4) || !same_shape(dg, gs, 4))
        return KDA_ERR_SHAPE;
    const int64_t bs[3] = {B, T, Hv};
    if (!same_shape(beta, bs, 3) || !same_shape(dbeta, bs, 3)) return KDA_ERR_SHAPE;
    if (Hq <= 0 || Hv <= 0) return KDA_ERR_SHAPE;
    if (Hv % Hq != 0) return KDA_ERR_UNSUPPORTED;
    int64_t N = B;
    if (cu_seqlens) {
        if (B != 1) return KDA_ERR_UNSUPPORTED;
        if (cu_seqlens->shape[0] < 1) return KDA_ERR_SHAPE;
        N = cu_seqlens->shape[0] - 1;
    }
    const int64_t ss[4] = {N, Hv, kHeadDim, kHeadDim};
    if (initial_state && !same_shape(initial_state, ss, 4)) return KDA_ERR_SHAPE;
    if (d_final_state && !same_shape(d_final_state, ss, 4)) return KDA_ERR_SHAPE;
    if (d_initial_state && !same_shape(d_initial_state, ss, 4)) return KDA_ERR_SHAPE;
    if (!std::isfinite(scale) || !(scale > 0.f)) return KDA_ERR_VALUE;
    const int64_t nc = (T + 63) / 64;
    const int64_t nslots = cu_seqlens ? nc + N : B * nc;
    if (nslots * Hv > kMaxBlocks || N * Hv * 8 > kMaxBlocks || N > (int64_t(1) << 24) || Hv > (int64_t(1) << 16))
        return KDA_ERR_UNSUPPORTED;
    // the group kernel's grid, (B T Hq 128) / 256 work-groups, must fit 32 bits
    if (B * T * Hq * kHeadDim > (int64_t(1) << 39)) return KDA_ERR_UNSUPPORTED;
    const BwdLayout L = bwd_layout(B * T, N, Hq, Hv);
    if (workspace && (workspace_size < L.total || reinterpret_cast<uintptr_t>(workspace) % 256 != 0))
        return KDA_ERR_WORKSPACE;

    kda::BwdParams p{};
    p.q = static_cast<const uint16_t*>(q->data);
    p.k = static_cast<const uint16_t*>(k->data);
    p.v = static_cast<const uint16_t*>(v->data);
    p.dO = static_cast<const uint16_t*>(d_out->data);
    p.g = static_cast<const float*>(g->data);
    p.beta = beta->data;
    p.beta_f32 = beta->dtype == KDA_F32 ? 1 : 0;
    p.h0 = initial_state ? static_cast<const float*>(initial_state->data) : nullptr;
    p.dhT = d_final_state ? static_cast<const float*>(d_final_state->data) : nullptr;
    p.dq = static_cast<float*>(dq->data);
    p.dk = static_cast<float*>(dk->data);
    p.dv = static_cast<float*>(dv->data);
    p.dg = static_cast<float*>(dg->data);
    p.dbeta = static_cast<float*>(dbeta->data);
    p.dh0 = d_initial_state ? static_cast<float*>(d_initial_state->data) : nullptr;
    p.cu = cu_seqlens ? static_cast<const int32_t*>(cu_seqlens->data) : nullptr;
    p.T = T;
    p.nslots = nslots;
    p.B = static_cast<int32_t>(B);
    p.N = static_cast<int32_t>(N);
    p.Hq = static_cast<int32_t>(Hq);
    p.Hv = static_cast<int32_t>(Hv);
    p.nc = static_cast<int32_t>(nc);
    p.scale = scale;
    if (N == 0 || (T == 0 && !d_initial_state)) return KDA_OK;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    void* ws = workspace;
    if (!ws && T > 0 && hipMallocAsync(&ws, (size_t)L.total, hs) != hipSuccess) return KDA_ERR_HIP;
    char* base = static_cast<char*>(ws);
    if (base) {
        p.prep = reinterpret_cast<float*>(base + L.prep);
        p.hs = reinterpret_cast<float*>(base + L.hs);
        p.dhs = reinterpret_cast<float*>(base + L.dhs);
        p.dqv = Hq < Hv ? reinterpret_cast<float*>(base + L.dqv) : p.dq;
        p.dkv = Hq < Hv ? reinterpret_cast<float*>(base + L.dkv) : p.dk;
    }
    hipError_t e = kda::launch_kda_bwd(p, hs);
    if (!workspace && ws && hipFreeAsync(ws, hs) != hipSuccess && e == hipSuccess) e = hipErrorUnknown;
    return finish(e, hs);
}

const char* kda_status_string(kda_status_t s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_NULL: return "KDA_ERR_NULL: a required descriptor or data pointer is NULL";
        case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE: unsupported dtype";
        case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: ranks or sizes disagree";
        case KDA_ERR_LAYOUT: return "KDA_ERR_LAYOUT: tensor not contiguous or not aligned";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: unsupported configuration";
        case KDA_ERR_VALUE: return "KDA_ERR_VALUE: scale must be finite and positive";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: HIP runtime error";
        case KDA_ERR_WORKSPACE:
            return "KDA_ERR_WORKSPACE: workspace missing, smaller than the entry point's workspace size or misaligned "
                   "(kda_fwd_noalloc: the call needs more than its static scratch)";
    }
    return "KDA: unknown status";
}

}  // extern "C"

// State-dependent stages of the KDA chunked forward for gfx950 (MI355X, CDNA4).
//
// One work-group of 512 threads (8 wave64s) owns one (sequence, value head,
// dv slice) and walks that sequence's chunks of 64 tokens in order.  Per chunk
// it runs the stages that depend on the recurrent state ("cuLA PR #131:
// SM100/SM103 KDA forward to pure CuTeDSL", Summary: recompute W/U; "cuLA
// REPO_LAYOUT.md", ops/: chunk delta-H and forward output):
//
//   a1  gate cumsum     G = chunk-local inclusive cumsum of g (fp32)
//   a4  W/U recompute   W = T (beta k e^G), U = T (beta v)                 (MFMA)
//   a5  delta-H scan    v_new = U - W h;
//                       h <- Diag(e^{G_last}) h + (k e^{G_last - G})^T v_new
//   a6  output          o = (scale q e^G) h + Aqk v_new                     (MFMA)
//
// Aqk and T diag(beta) come from the intra kernel's workspace record of the
// chunk.  The state slice h (128 x DV, fp32) lives in MFMA accumulator
// registers for the whole sequence.  MFMA operands are fp16, accumulation is
// fp32; o is rounded to bf16 once.
//
// Software pipeline.  The gate cumsum and the decay factors of a chunk
// (q e^G, k e^G, k e^{G_last - G}: the kernel's main vector-ALU load) do not
// depend on the state, so they are computed one chunk ahead, inside the
// previous chunk's MFMA phases, and held in registers until their chunk
// starts.  q, k and g are loaded two chunks ahead into two register sets used
// in turn (the chunk loop is unrolled by two), one third per phase; v and the
// workspace record one chunk ahead.  Per chunk, four barrier-separated phases:
//   C  stage this chunk's operands in LDS; store the previous chunk's output;
//      load the next chunk's v and workspace record
//   D  W^T and U on MFMA                 | gate sums of the next chunk; g of chunk + 2
//   E  v_new on MFMA                     | factors of the next chunk, rows 0-3; q of chunk + 2
//   F  o and the state update on MFMA    | factors of the next chunk, rows 4-7; k of chunk + 2
// and the fp16 copy of the new state for the next chunk's MFMAs.
#include "kda_device.h"

namespace kda {

namespace {

constexpr int S136 = 136;    // fp16 rows of 128 (+8 pad)
constexpr int S72 = 72;      // fp16 rows of 64 (+8 pad)

template <int DV>
struct ScanLds {
    static constexpr int Qg = 0;                          // [64][136] fp16, q e^G
    static constexpr int KgT = Qg + 64 * S136 * 2;         // [128][72] fp16, (k e^G)^T
    static constexpr int KhT = KgT + 128 * S72 * 2;        // [128][72] fp16, (k e^{G_last - G})^T
    static constexpr int Vt = KhT + 128 * S72 * 2;         // [DV][72] fp16, v^T
    static constexpr int T16 = Vt + DV * S72 * 2;          // [64][72] fp16, T diag(beta)
    static constexpr int Aqk = T16 + 64 * S72 * 2;         // [64][72] fp16
    static constexpr int W = Aqk + 64 * S72 * 2;           // [64][136] fp16, -W
    static constexpr int VnT = W + 64 * S136 * 2;          // [DV][72] fp16, v_new^T
    static constexpr int HT = VnT + DV * S72 * 2;          // [DV][136] fp16, h^T
    static constexpr int Ost = HT + DV * S136 * 2;         // [64][DV+8] bf16 output of the previous chunk
    static constexpr int Xs = Ost + 64 * (DV + 8) * 2;     // [8][128] fp32 sums of g over each wave's 8 rows
    static constexpr int Gam = Xs + 8 * 128 * 4;           // [128] fp32 e^{G_last}
    static constexpr int BYTES = Gam + 128 * 4;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// One chunk's q, k and g in the factor layout: lane = channel pair (channels
// 2 lane, 2 lane + 1), wave = rows 8 wave .. 8 wave + 7.
struct InRegs {
    float g[8][2];
    uint32_t q[8], k[8];
};

// Decay factors of one chunk in the same layout, as fp16: q e^G for rows rr
// (two channels per word), and per channel the eight rows of k e^G and
// k e^{G_last - G}.
struct FacRegs {
    uint32_t qg[8];
    half8 kg[2], kh[2];
    f32x2 gam;   // e^{G_last} of the two channels
};

}  // namespace

template <int DV, bool TRACE>
__global__ void __launch_bounds__(NTHREADS, 1) kda_scan_kernel(const KdaParams p) {
    using L = ScanLds<DV>;
    constexpr int S = DK / DV;          // dv slices
    constexpr int NU = 2 * (DV / 32);   // 32x32 tiles of a 64 x DV matrix
    constexpr int NH = 4 * (DV / 32);   // 32x32 tiles of the 128 x DV state (at most one per wave)
    static_assert(NH <= 8, "one state tile per wave");
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

    // tid and lane are re-made opaque at the top of every chunk (see `chunk`), so
    // the compiler recomputes the LDS addresses derived from them per chunk
    // instead of hoisting hundreds of them out of the loop into registers.
    int tid = threadIdx.x;
    int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // wave-uniform, kept in an SGPR

    // Work-group -> (sequence, value head, slice).  Slices of one head go to the
    // same XCD (work-groups are dealt to the 8 XCDs round robin), so their
    // duplicate q/k/g reads meet in that XCD's L2.
    const int npairs = p.N * p.Hv;
    int pair, s;
    if ((npairs & 7) == 0) {
        const int x = blockIdx.x & 7, loc = blockIdx.x >> 3;
        pair = (loc / S) * 8 + x;
        s = loc % S;
    } else {
        pair = blockIdx.x / S;
        s = blockIdx.x % S;
    }
    const int n = pair / p.Hv, hv = pair % p.Hv, hq = hv / (p.Hv / p.Hq);
    int64_t bos, len;
    seq_bounds(p, n, bos, len);
    const int64_t nch = (len + CH - 1) / CH;
    const int64_t qk_tok = (int64_t)p.Hq * DK;   // token stride of q, k
    const int64_t v_tok = (int64_t)p.Hv * DK;    // token stride of v, g, o
    const int dv0 = s * DV;
    const int64_t slot0 = chunk_slot(bos, n, 0);

    int64_t trace_chunk = 0;   // index of this sequence's first chunk in the h dump
    if (TRACE && p.tr_h) {
        if (p.cu) {
            for (int m = 0; m < n; ++m) {
                int64_t a, l;
                seq_bounds(p, m, a, l);
                trace_chunk += (l + CH - 1) / CH;
            }
        } else {
            trace_chunk = (int64_t)n * ((p.T + CH - 1) / CH);
        }
    }

    // State tile of this wave: rows c = 32 ct .., columns d = 32 dt .. of h (128 x DV).
    const bool has_h = wave < NH;
    const int h_ct = wave / (DV / 32), h_dt = wave % (DV / 32);
    f32x16 hacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) hacc[r] = 0.f;
    if (has_h && p.h0) {
        const float* src = p.h0 + ((int64_t)n * p.Hv + hv) * DK * DK + dv0 + 32 * h_dt + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) hacc[r] = src[(int64_t)(32 * h_ct + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * DK];
    }
    // fp16 copy of h^T in LDS (the B / A operand of the state's MFMAs).
    auto write_ht = [&]() {
        if (has_h) {
            const int d = 32 * h_dt + (lane & 31);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                half4 h4;
#pragma unroll
                for (int e = 0; e < 4; ++e) h4[e] = (_Float16)hacc[4 * q4 + e];
                *reinterpret_cast<half4*>(smem + L::HT + (d * S136 + 32 * h_ct + 8 * q4 + 4 * (lane >> 5)) * 2) = h4;
            }
        }
    };
    write_ht();
    // Upper 16x16 tiles of T16 and Aqk are zero (the MFMAs read some of them);
    // the chunk loop writes only the lower tiles.
    for (int it = tid; it < 2 * 6 * 32; it += NTHREADS) {
        const int mtx = it / 192, tile = (it / 32) % 6, w32 = it & 31;
        const int I = tile < 3 ? 0 : (tile < 5 ? 1 : 2);
        const int J = tile < 3 ? tile + 1 : (tile < 5 ? tile - 1 : 3);
        const int m = w32 >> 1, h = w32 & 1;
        *reinterpret_cast<uint4*>(smem + (mtx ? L::Aqk : L::T16) + ((16 * I + m) * S72 + 16 * J + 8 * h) * 2) =
            make_uint4(0, 0, 0, 0);
    }

    // Loop-invariant per-lane offsets, computed once from threadIdx.x (the
    // opaque tid below would make the compiler recompute them every chunk).
    // Workspace record pieces: 16 bytes each, tid and tid + 512 (< 640).
    int ws_dst[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int it = (int)threadIdx.x + NTHREADS * u;
        const int t = it >> 5, r = (it >> 1) & 15, h = it & 1;
        const int tt = t % 10;
        const int I = tt >= 6 ? 3 : (tt >= 3 ? 2 : (tt >= 1 ? 1 : 0));
        const int J = tt - I * (I + 1) / 2;
        ws_dst[u] = (t < 10 ? L::Aqk : L::T16) + ((16 * I + r) * S72 + 16 * J + 8 * h) * 2;
    }
    // Output pieces: row i, 8 channels c8 of the slice.
    constexpr int OPT = (CH * DV / 8 + NTHREADS - 1) / NTHREADS;
    int o_row[OPT], o_lds[OPT], o_glb[OPT];
#pragma unroll
    for (int u = 0; u < OPT; ++u) {
        const int it = (int)threadIdx.x + NTHREADS * u;
        const int i = it / (DV / 8), c8 = it % (DV / 8);
        o_row[u] = it < CH * DV / 8 ? i : CH;   // CH: no piece
        o_lds[u] = L::Ost + (i * (DV + 8) + 8 * c8) * 2;
        o_glb[u] = (int)((i * v_tok + 8 * c8) * 2);
    }

    float* sXs = reinterpret_cast<float*>(smem + L::Xs);
    float* sGam = reinterpret_cast<float*>(smem + L::Gam);

    // ---- loads ----
    // Raw buffer loads: a wave-uniform descriptor (scalar base and byte range) and
    // per-lane 32-bit offsets.  Rows past the sequence end, and whole chunks past
    // it, fall outside the range and read as zero without touching memory, so the
    // loads of later chunks need no branches.
    auto chunk_rows = [&](int64_t c) -> int {   // valid rows of chunk c (0 past the end)
        const int64_t r = len - c * CH;
        return r <= 0 ? 0 : (r >= CH ? CH : (int)r);
    };
    // part 0: g rows, 1: q rows, 2: k rows.
    auto load_inputs = [&](InRegs& in, int64_t c, int part) {
        const int Lc = chunk_rows(c);
        const int nr = Lc - 8 * wave < 0 ? 0 : (Lc - 8 * wave > 8 ? 8 : Lc - 8 * wave);
        const int64_t t0 = bos + c * CH + 8 * wave;
        if (part == 0) {
            const __amdgpu_buffer_rsrc_t rg =
                make_rsrc(p.g + t0 * v_tok + (int64_t)hv * DK, nr ? ((nr - 1) * v_tok + DK) * 4 : 0);
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const i32x2 g2 = __builtin_amdgcn_raw_buffer_load_b64(rg, 8 * lane + (int)(rr * v_tok * 4), 0, 0);
                in.g[rr][0] = __int_as_float(g2[0]);
                in.g[rr][1] = __int_as_float(g2[1]);
            }
        } else {
            const uint16_t* base = part == 1 ? p.q : p.k;
            const __amdgpu_buffer_rsrc_t r =
                make_rsrc(base + t0 * qk_tok + (int64_t)hq * DK, nr ? ((nr - 1) * qk_tok + DK) * 2 : 0);
            uint32_t* dst = part == 1 ? in.q : in.k;
#pragma unroll
            for (int rr = 0; rr < 8; ++rr)
                dst[rr] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, 4 * lane + (int)(rr * qk_tok * 2), 0, 0);
        }
    };
    // v: thread (jp, cg) = (tid % 32, tid / 32) holds tokens 2 jp and 2 jp + 1 of
    // channels 4 cg .. 4 cg + 3.
    uint2 pf_v[2];
    uint4 pf_w[2];
    auto load_v_ws = [&](int64_t c) {
        const int v_jp = tid & 31, v_cg = tid >> 5;
        const bool v_act = v_cg < DV / 4;
        const int v_off = (int)((2 * v_jp * v_tok + 4 * v_cg) * 2);
        const int Lc = chunk_rows(c);
        const int64_t t0 = bos + c * CH;
        const __amdgpu_buffer_rsrc_t rv =
            make_rsrc(p.v + t0 * v_tok + (int64_t)hv * DK + dv0, Lc ? ((Lc - 1) * v_tok + DV) * 2 : 0);
        pf_v[0] = make_uint2(0, 0);
        pf_v[1] = make_uint2(0, 0);
        if (v_act) {
            const i32x2 a = __builtin_amdgcn_raw_buffer_load_b64(rv, v_off, 0, 0);
            const i32x2 b = __builtin_amdgcn_raw_buffer_load_b64(rv, v_off + (int)(v_tok * 2), 0, 0);
            pf_v[0] = make_uint2((uint32_t)a[0], (uint32_t)a[1]);
            pf_v[1] = make_uint2((uint32_t)b[0], (uint32_t)b[1]);
        }
        const __amdgpu_buffer_rsrc_t rw =
            make_rsrc(p.ws + ((slot0 + c) * p.Hv + hv) * WS_RECORD_BYTES, Lc ? WS_RECORD_BYTES : 0);
        const i32x4 w0 = __builtin_amdgcn_raw_buffer_load_b128(rw, 16 * tid, 0, 0);
        pf_w[0] = make_uint4((uint32_t)w0[0], (uint32_t)w0[1], (uint32_t)w0[2], (uint32_t)w0[3]);
        pf_w[1] = make_uint4(0, 0, 0, 0);
        if (tid < WS_RECORD_BYTES / 16 - NTHREADS) {
            const i32x4 w1 = __builtin_amdgcn_raw_buffer_load_b128(rw, 16 * (tid + NTHREADS), 0, 0);
            pf_w[1] = make_uint4((uint32_t)w1[0], (uint32_t)w1[1], (uint32_t)w1[2], (uint32_t)w1[3]);
        }
    };
    static_assert(WS_RECORD_BYTES / 16 > NTHREADS && WS_RECORD_BYTES / 16 <= 2 * NTHREADS, "two pieces per thread");

    // ---- decay factors (state independent) ----
    // Per token and channel E = e^{g} = 2^{g log2 e}; the factors are running
    // products of E (one exponential per element instead of two):
    //   e^{G_r}          = e^{G at the end of the earlier waves' rows} * prod_{s <= r} E_s
    //   e^{G_last - G_r} = e^{G_last - G at the end of this wave's rows} * prod_{r < s <= 7} E_s
    // The cross-wave parts come from the waves' sums of g log2 e, exchanged in Xs.
    float ex[8][2];
    auto gate_sums = [&](const InRegs& in) {
        f32x2 tot = {0.f, 0.f};
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float x = in.g[rr][e] * LOG2E;
                tot[e] += x;
                ex[rr][e] = fexp2(x);
            }
        }
        *reinterpret_cast<f32x2*>(sXs + wave * 128 + 2 * lane) = tot;
    };
    // Running products: pg = e^{G} of the last row done, ph = e^{G_last - G} of row 3
    // (rows 0-3) or row 7 (rows 4-7).
    f32x2 pg;
    auto gate_offsets = [&](FacRegs& f) {
        f32x2 x[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) x[w] = *reinterpret_cast<const f32x2*>(sXs + w * 128 + 2 * lane);
        // prefix over the earlier waves; wave is uniform, so this is one scalar branch
        f32x2 off = {0.f, 0.f}, mine;
        switch (wave) {
#define KDA_OFF_CASE(W)                                      \
            case W:                                          \
                _Pragma("unroll") for (int w = 0; w < W; ++w) off += x[w]; \
                mine = x[W];                                 \
                break;
            KDA_OFF_CASE(0) KDA_OFF_CASE(1) KDA_OFF_CASE(2) KDA_OFF_CASE(3)
            KDA_OFF_CASE(4) KDA_OFF_CASE(5) KDA_OFF_CASE(6)
            default:
#pragma unroll
                for (int w = 0; w < 7; ++w) off += x[w];
                mine = x[7];
                break;
#undef KDA_OFF_CASE
        }
        const f32x2 all = ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
        pg = f32x2{fexp2(off[0]), fexp2(off[1])};
        f.gam = f32x2{fexp2(all[0]), fexp2(all[1])};
        return f32x2{fexp2(all[0] - off[0] - mine[0]), fexp2(all[1] - off[1] - mine[1])};   // e^{G_last - G_7}
    };
    // Rows r0 .. r0+3 of the factors: Qg = q e^G (scale is applied to the o
    // accumulator), Kg = k e^G, Kh = k e^{G_last - G}.  ph enters as
    // e^{G_last - G_{r0+3}}.
    auto factors = [&](const InRegs& in, FacRegs& f, int r0, f32x2 ph) {
        f32x2 eh[4];
#pragma unroll
        for (int j = 3; j >= 0; --j) {
            eh[j] = ph;
            if (j > 0) ph *= f32x2{ex[r0 + j][0], ex[r0 + j][1]};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int rr = r0 + j;
            pg *= f32x2{ex[rr][0], ex[rr][1]};
            const float q0 = bf_lo(in.q[rr]), q1 = bf_hi(in.q[rr]);
            const float k0 = bf_lo(in.k[rr]), k1 = bf_hi(in.k[rr]);
            f.qg[rr] = pack_h2(q0 * pg[0], q1 * pg[1]);
            f.kg[0][rr] = (_Float16)(k0 * pg[0]);
            f.kg[1][rr] = (_Float16)(k1 * pg[1]);
            f.kh[0][rr] = (_Float16)(k0 * eh[j][0]);
            f.kh[1][rr] = (_Float16)(k1 * eh[j][1]);
        }
    };
    // e^{G_last - G_3} from e^{G_last - G_7}: times E of rows 4..7.
    auto ph_rows03 = [&](f32x2 ph7) {
#pragma unroll
        for (int rr = 4; rr < 8; ++rr) ph7 *= f32x2{ex[rr][0], ex[rr][1]};
        return ph7;
    };

    // Output rows staged in Ost: 16-byte pieces, whole row segments per lane group.
    auto store_output = [&](int64_t t0, int rows) {
        char* base = reinterpret_cast<char*>(p.o + t0 * v_tok + (int64_t)hv * DK + dv0);
#pragma unroll
        for (int u = 0; u < OPT; ++u) {
            if (o_row[u] < rows)
                *reinterpret_cast<uint4*>(base + o_glb[u]) = *reinterpret_cast<const uint4*>(smem + o_lds[u]);
        }
    };

    InRegs in0, in1;
    FacRegs fac;
    if (nch > 0) {
        // Prologue: chunk 0's factors; chunk 1's q, k, g in flight.
        for (int part = 0; part < 3; ++part) load_inputs(in0, 0, part);
        load_v_ws(0);
        for (int part = 0; part < 3; ++part) load_inputs(in1, 1, part);
        gate_sums(in0);
        lds_barrier();
        const f32x2 ph7 = gate_offsets(fac);
        factors(in0, fac, 0, ph_rows03(ph7));
        factors(in0, fac, 4, ph7);
    }

    // One chunk.  `fr` held this chunk's inputs (consumed: it receives chunk c + 2);
    // `nx` holds chunk c + 1's, whose factors are computed here.
    auto chunk = [&](int64_t c, InRegs& fr, InRegs& nx) __attribute__((always_inline)) {
        asm volatile("" : "+v"(tid), "+v"(lane));
        const int64_t tok0 = bos + c * CH;
        const int Lc = chunk_rows(c);
        const bool more = c + 1 < nch;

        if (TRACE && p.tr_h && has_h) {
            const int d = dv0 + 32 * h_dt + (lane & 31);
            float* dst = p.tr_h + ((trace_chunk + c) * p.Hv + hv) * DK * DK;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dst[(int64_t)(32 * h_ct + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * DK + d] = hacc[r];
        }

        // ================= C: stage this chunk's operands =================
#pragma unroll
        for (int rr = 0; rr < 8; ++rr)
            *reinterpret_cast<uint32_t*>(smem + L::Qg + ((8 * wave + rr) * S136 + 2 * lane) * 2) = fac.qg[rr];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            *reinterpret_cast<half8*>(smem + L::KgT + ((2 * lane + e) * S72 + 8 * wave) * 2) = fac.kg[e];
            *reinterpret_cast<half8*>(smem + L::KhT + ((2 * lane + e) * S72 + 8 * wave) * 2) = fac.kh[e];
        }
        if (wave == 0) *reinterpret_cast<f32x2*>(sGam + 2 * lane) = fac.gam;
        const int v_jp = tid & 31, v_cg = tid >> 5;
        if (v_cg < DV / 4) {
            // v^T: channel 4 cg + e, tokens 2 jp and 2 jp + 1 as one 32-bit word.
            const uint32_t a[2] = {pf_v[0].x, pf_v[0].y}, b[2] = {pf_v[1].x, pf_v[1].y};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x0 = (e & 1) ? bf_hi(a[e >> 1]) : bf_lo(a[e >> 1]);
                const float x1 = (e & 1) ? bf_hi(b[e >> 1]) : bf_lo(b[e >> 1]);
                *reinterpret_cast<uint32_t*>(smem + L::Vt + ((4 * v_cg + e) * S72 + 2 * v_jp) * 2) = pack_h2(x0, x1);
            }
        }
        // Aqk and T diag(beta): the 20 lower 16x16 tiles of the workspace record.
        *reinterpret_cast<uint4*>(smem + ws_dst[0]) = pf_w[0];
        if (tid < WS_RECORD_BYTES / 16 - NTHREADS) *reinterpret_cast<uint4*>(smem + ws_dst[1]) = pf_w[1];
        // The previous chunk's output goes out after this chunk's v and workspace
        // registers are consumed and before they are reloaded: global stores share
        // the vmcnt counter with loads, so every wait for loaded data stays clear of
        // pending stores.
        if (c > 0) store_output(tok0 - CH, CH);
        load_v_ws(c + 1);
        lds_barrier();

        // ================= D: W^T = (k e^G)^T (T diag beta)^T, U = T diag(beta) v =================
        {
            const int ct = wave >> 1, it = wave & 1;  // W^T tile: rows c (32ct..), cols i (32it..)
            f32x16 acc;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk < 2 || it == 1) {              // T is lower triangular
                    const int ko = 16 * kk + 8 * (lane >> 5);
                    const half8 a = lds_h8(smem, L::KgT + ((32 * ct + (lane & 31)) * S72 + ko) * 2);
                    const half8 b = lds_h8(smem, L::T16 + ((32 * it + (lane & 31)) * S72 + ko) * 2);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
                }
            }
            const int i = 32 * it + (lane & 31);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int cc = 32 * ct + 8 * q4 + 4 * (lane >> 5);
                half4 h4;
#pragma unroll
                for (int e = 0; e < 4; ++e) h4[e] = (_Float16)(-acc[4 * q4 + e]);
                *reinterpret_cast<half4*>(smem + L::W + (i * S136 + cc) * 2) = h4;
                if (TRACE && p.tr_W && s == 0 && i < Lc) {
                    float* dst = p.tr_W + ((tok0 + i) * p.Hv + hv) * DK + cc;
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[e] = acc[4 * q4 + e];
                }
            }
        }
        f32x16 uacc;
        const int tu_it = wave / (DV / 32), tu_dt = wave % (DV / 32);
        if (wave < NU) {
#pragma unroll
            for (int e = 0; e < 16; ++e) uacc[e] = 0.f;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk < 2 || tu_it == 1) {
                    const int ko = 16 * kk + 8 * (lane >> 5);
                    const half8 a = lds_h8(smem, L::T16 + ((32 * tu_it + (lane & 31)) * S72 + ko) * 2);
                    const half8 b = lds_h8(smem, L::Vt + ((32 * tu_dt + (lane & 31)) * S72 + ko) * 2);
                    uacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, uacc, 0, 0, 0);
                }
            }
            if (TRACE && p.tr_U) {
                const int d = dv0 + 32 * tu_dt + (lane & 31);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int i = 32 * tu_it + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                    if (i < Lc) p.tr_U[((tok0 + i) * p.Hv + hv) * DK + d] = uacc[e];
                }
            }
        }
        if (more) gate_sums(nx);
        load_inputs(fr, c + 2, 0);
        lds_barrier();

        // ================= E: v_new = U - W h;  (q e^G) h for o =================
        if (wave < NU) {
            // Two independent accumulation chains (even / odd k steps) halve the
            // dependent MFMA latency; they are summed once at the end.
            f32x16 acc = uacc, acc1;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc1[e] = 0.f;
#pragma unroll
            for (int kk = 0; kk < 8; kk += 2) {
                const int ko = 16 * kk + 8 * (lane >> 5);
                const half8 a0 = lds_h8(smem, L::W + ((32 * tu_it + (lane & 31)) * S136 + ko) * 2);
                const half8 b0 = lds_h8(smem, L::HT + ((32 * tu_dt + (lane & 31)) * S136 + ko) * 2);
                const half8 a1 = lds_h8(smem, L::W + ((32 * tu_it + (lane & 31)) * S136 + ko + 16) * 2);
                const half8 b1 = lds_h8(smem, L::HT + ((32 * tu_dt + (lane & 31)) * S136 + ko + 16) * 2);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, acc, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, acc1, 0, 0, 0);
            }
            acc += acc1;
            const int d = 32 * tu_dt + (lane & 31);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int i = 32 * tu_it + 8 * q4 + 4 * (lane >> 5);
                half4 h4;
#pragma unroll
                for (int e = 0; e < 4; ++e) h4[e] = (_Float16)acc[4 * q4 + e];
                *reinterpret_cast<half4*>(smem + L::VnT + (d * S72 + i) * 2) = h4;
                if (TRACE && p.tr_vnew) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (i + e < Lc) p.tr_vnew[((tok0 + i + e) * p.Hv + hv) * DK + dv0 + d] = acc[4 * q4 + e];
                }
            }
        }
        // o^T = h^T (q e^G)^T scale + v_new^T Aqk^T: the first term needs only the
        // state entering the chunk, so waves 8 - NU .. 7 (idle in the v_new MFMAs)
        // take it here; the second follows in F.
        const int wo = 7 - wave;
        const int o_it = wo / (DV / 32), o_dt = wo % (DV / 32);
        f32x16 oacc;
        if (wo < NU) {
            f32x16 acc1;
#pragma unroll
            for (int e = 0; e < 16; ++e) { oacc[e] = 0.f; acc1[e] = 0.f; }
#pragma unroll
            for (int kk = 0; kk < 8; kk += 2) {
                const int ko = 16 * kk + 8 * (lane >> 5);
                const half8 a0 = lds_h8(smem, L::HT + ((32 * o_dt + (lane & 31)) * S136 + ko) * 2);
                const half8 b0 = lds_h8(smem, L::Qg + ((32 * o_it + (lane & 31)) * S136 + ko) * 2);
                const half8 a1 = lds_h8(smem, L::HT + ((32 * o_dt + (lane & 31)) * S136 + ko + 16) * 2);
                const half8 b1 = lds_h8(smem, L::Qg + ((32 * o_it + (lane & 31)) * S136 + ko + 16) * 2);
                oacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, oacc, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, acc1, 0, 0, 0);
            }
            // scale here; Aqk already carries it
            oacc = (oacc + acc1) * p.scale;
        }
        f32x2 ph7 = {0.f, 0.f};
        if (more) {
            ph7 = gate_offsets(fac);
            factors(nx, fac, 0, ph_rows03(ph7));
        }
        load_inputs(fr, c + 2, 1);
        lds_barrier();

        // ================= F: o += v_new^T Aqk^T; state update =================
        // o goes to the staging tile Ost and out to HBM during the next chunk.
        if (wo < NU) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk < 2 || o_it == 1) {
                    const int ko = 16 * kk + 8 * (lane >> 5);
                    const half8 a = lds_h8(smem, L::VnT + ((32 * o_dt + (lane & 31)) * S72 + ko) * 2);
                    const half8 b = lds_h8(smem, L::Aqk + ((32 * o_it + (lane & 31)) * S72 + ko) * 2);
                    oacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, oacc, 0, 0, 0);
                }
            }
            const int i = 32 * o_it + (lane & 31);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d = 32 * o_dt + 8 * q4 + 4 * (lane >> 5);
                uint2 w;
                w.x = pack_bf2(oacc[4 * q4], oacc[4 * q4 + 1]);
                w.y = pack_bf2(oacc[4 * q4 + 2], oacc[4 * q4 + 3]);
                *reinterpret_cast<uint2*>(smem + L::Ost + (i * (DV + 8) + d) * 2) = w;
            }
        }
        // h <- Diag(e^{G_last}) h + Khat^T v_new
        if (has_h) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 gm = *reinterpret_cast<const f32x4*>(sGam + 32 * h_ct + 8 * q4 + 4 * (lane >> 5));
#pragma unroll
                for (int e = 0; e < 4; ++e) hacc[4 * q4 + e] *= gm[e];
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int ko = 16 * kk + 8 * (lane >> 5);
                const half8 a = lds_h8(smem, L::KhT + ((32 * h_ct + (lane & 31)) * S72 + ko) * 2);
                const half8 b = lds_h8(smem, L::VnT + ((32 * h_dt + (lane & 31)) * S72 + ko) * 2);
                hacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, hacc, 0, 0, 0);
            }
        }
        if (more) factors(nx, fac, 4, ph7);
        load_inputs(fr, c + 2, 2);
        lds_barrier();
        write_ht();
        // The next chunk's phase C writes Qg, KgT, KhT, Gam, Vt, Aqk and T16; every
        // read of them in this chunk happened before the barrier above, and none
        // aliases HT.  Ost is read (and then rewritten) only after later barriers.
    };

    for (int64_t c = 0; c < nch; c += 2) {
        chunk(c, in0, in1);
        if (c + 1 < nch) chunk(c + 1, in1, in0);
    }

    // ---- output of the last chunk (staged in Ost before the loop's last barrier) ----
    if (nch > 0) {
        const int64_t last = (nch - 1) * CH;
        store_output(bos + last, (int)(len - last));
    }

    // ---- final state ----
    if (p.hT && has_h) {
        const int d = 32 * h_dt + (lane & 31);
        float* dst = p.hT + ((int64_t)n * p.Hv + hv) * DK * DK + dv0 + d;
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2)
            dst[(int64_t)(32 * h_ct + 8 * (r2 >> 2) + 4 * (lane >> 5) + (r2 & 3)) * DK] = hacc[r2];
    }
}

template <int DV, bool TRACE>
static hipError_t launch_dv(const KdaParams& p, int nblocks, hipStream_t stream) {
    hipLaunchKernelGGL((kda_scan_kernel<DV, TRACE>), dim3(nblocks), dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_kda_scan(const KdaParams& p, int dv_slices, bool trace, hipStream_t stream) {
    const int64_t nblocks = (int64_t)p.N * p.Hv * dv_slices;
    if (nblocks == 0) return hipSuccess;
    if (dv_slices == 2) return trace ? launch_dv<64, true>(p, (int)nblocks, stream) : launch_dv<64, false>(p, (int)nblocks, stream);
    return trace ? launch_dv<32, true>(p, (int)nblocks, stream) : launch_dv<32, false>(p, (int)nblocks, stream);
}

}  // namespace kda

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
// registers for the whole sequence.  The next chunk's inputs are loaded into
// registers while the current chunk computes.  MFMA operands are fp16,
// accumulation is fp32; o is rounded to bf16 once.
#include "kda_device.h"

namespace kda {

namespace {

constexpr int S136 = 136;    // fp16 rows of 128 (+8 pad)
constexpr int S72 = 72;      // fp16 rows of 64 (+8 pad)

template <int DV>
struct ScanLds {
    static constexpr int Qg = 0;                          // [64][136] fp16, scale q e^G
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

}  // namespace

template <int DV, bool TRACE>
__global__ void __launch_bounds__(NTHREADS, 1) kda_scan_kernel(const KdaParams p) {
    using L = ScanLds<DV>;
    constexpr int S = DK / DV;          // dv slices
    constexpr int NU = 2 * (DV / 32);   // 32x32 tiles of a 64 x DV matrix
    constexpr int NH = 4 * (DV / 32);   // 32x32 tiles of the 128 x DV state
    constexpr int HPW = (NH + 7) / 8;   // state tiles per wave
    constexpr int VPT = (CH * DV / 8 + NTHREADS - 1) / NTHREADS;   // 16-byte pieces of v per thread
    constexpr int WPT = (WS_RECORD_BYTES / 16 + NTHREADS - 1) / NTHREADS;   // 16-byte workspace pieces per thread
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];

    const int tid_o = threadIdx.x;
    const int lane_o = tid_o & 63;
    const int wave_o = __builtin_amdgcn_readfirstlane(tid_o >> 6);  // wave-uniform, kept in an SGPR
    const int tid = tid_o, lane = lane_o, wave = wave_o;

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

    // ---- initial state into accumulators and into h^T (fp16) in LDS ----
    f32x16 hacc[HPW];
#pragma unroll
    for (int u = 0; u < HPW; ++u) {
        const int th = wave + 8 * u;
#pragma unroll
        for (int r = 0; r < 16; ++r) hacc[u][r] = 0.f;
        if (th < NH) {
            const int ct = th / (DV / 32), dt = th % (DV / 32);
            const int d = 32 * dt + (lane & 31);
            if (p.h0) {
                const float* src = p.h0 + ((int64_t)n * p.Hv + hv) * DK * DK + dv0 + d;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int c = 32 * ct + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    hacc[u][r] = src[(int64_t)c * DK];
                }
            }
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int c = 32 * ct + 8 * q4 + 4 * (lane >> 5);
                half4 hv4;
#pragma unroll
                for (int e = 0; e < 4; ++e) hv4[e] = (_Float16)hacc[u][4 * q4 + e];
                *reinterpret_cast<half4*>(smem + L::HT + (d * S136 + c) * 2) = hv4;
            }
        }
    }
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

    float* sXs = reinterpret_cast<float*>(smem + L::Xs);
    float* sGam = reinterpret_cast<float*>(smem + L::Gam);

    // Prefetch registers: one chunk's inputs, loaded one chunk ahead of their use.
    // q, k, g in the factor layout (lane = channel pair, wave = 8-row group): every
    // load instruction of a wave reads one contiguous row segment (q, k: 256 B;
    // g: 512 B).  v and the workspace record in 16-byte pieces.
    float pf_g[8][2];
    uint32_t pf_q[8], pf_k[8];
    uint4 pf_v[VPT];
    uint4 pf_w[WPT];
    // Loads of q, k, g, v use raw buffer instructions: a wave-uniform 128-bit
    // descriptor (scalar base and byte range) and 32-bit per-lane offsets.  Rows
    // past the sequence end fall outside the descriptor's range and read as zero.
    auto pf_rows = [&](int64_t cstart, int wave_) {
        const int Ln = (int)((len - cstart) < CH ? (len - cstart) : CH);
        const int row0 = 8 * wave_;
        return Ln - row0 < 0 ? 0 : (Ln - row0 > 8 ? 8 : Ln - row0);
    };
    auto prefetch_gvw = [&](int64_t cstart, int tid_, int lane_, int wave_) {
        const int64_t t0 = bos + cstart;
        const int nrows = pf_rows(cstart, wave_);
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.g + (t0 + 8 * wave_) * v_tok + (int64_t)hv * DK,
                                                    nrows ? ((nrows - 1) * v_tok + DK) * 4 : 0);
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const i32x2 g2 = __builtin_amdgcn_raw_buffer_load_b64(rg, 8 * lane_ + (int)(rr * v_tok * 4), 0, 0);
            pf_g[rr][0] = __int_as_float(g2[0]);
            pf_g[rr][1] = __int_as_float(g2[1]);
        }
        const int Ln = (int)((len - cstart) < CH ? (len - cstart) : CH);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + t0 * v_tok + (int64_t)hv * DK + dv0,
                                                    Ln ? ((Ln - 1) * v_tok + DV) * 2 : 0);
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int it = tid_ + NTHREADS * u;
            const int j = it / (DV / 8), c8 = it % (DV / 8);
            pf_v[u] = make_uint4(0, 0, 0, 0);
            if (it < CH * DV / 8) {
                const i32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)((j * v_tok + 8 * c8) * 2), 0, 0);
                pf_v[u] = make_uint4((uint32_t)w[0], (uint32_t)w[1], (uint32_t)w[2], (uint32_t)w[3]);
            }
        }
        const uint4* rec = reinterpret_cast<const uint4*>(p.ws + ((slot0 + cstart / CH) * p.Hv + hv) * WS_RECORD_BYTES);
#pragma unroll
        for (int u = 0; u < WPT; ++u) {
            const int it = tid_ + NTHREADS * u;
            pf_w[u] = make_uint4(0, 0, 0, 0);
            if (it < WS_RECORD_BYTES / 16) pf_w[u] = rec[it];
        }
    };
    auto prefetch_qk = [&](int64_t cstart, int lane_, int wave_) {
        const int64_t t0 = bos + cstart;
        const int nrows = pf_rows(cstart, wave_);
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + (t0 + 8 * wave_) * qk_tok + (int64_t)hq * DK,
                                                    nrows ? ((nrows - 1) * qk_tok + DK) * 2 : 0);
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + (t0 + 8 * wave_) * qk_tok + (int64_t)hq * DK,
                                                    nrows ? ((nrows - 1) * qk_tok + DK) * 2 : 0);
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            pf_q[rr] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rq, 4 * lane_ + (int)(rr * qk_tok * 2), 0, 0);
            pf_k[rr] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rk, 4 * lane_ + (int)(rr * qk_tok * 2), 0, 0);
        }
    };
    // Output rows staged in Ost: 16-byte pieces, whole row segments per lane group.
    auto store_output = [&](int64_t t0, int rows, int tid_) {
#pragma unroll
        for (int u = 0; u < (CH * DV / 8 + NTHREADS - 1) / NTHREADS; ++u) {
            const int it = tid_ + NTHREADS * u;
            const int i = it / (DV / 8), c8 = it % (DV / 8);
            if (it < CH * DV / 8 && i < rows) {
                const uint4 w = *reinterpret_cast<const uint4*>(smem + L::Ost + (i * (DV + 8) + 8 * c8) * 2);
                *reinterpret_cast<uint4*>(p.o + (t0 + i) * v_tok + (int64_t)hv * DK + dv0 + 8 * c8) = w;
            }
        }
    };
    if (len > 0) {
        prefetch_gvw(0, tid, lane, wave);
        prefetch_qk(0, lane, wave);
    }

    int64_t chunk_idx = 0;
    for (int64_t c0 = 0; c0 < len; c0 += CH, ++chunk_idx) {
        // Opaque per-iteration copies of the thread coordinates: they stop the
        // compiler from hoisting every LDS address of the loop body out of the
        // chunk loop (which would hold hundreds of addresses in VGPRs).
        int tid = tid_o, lane = lane_o, wave = wave_o;
        asm volatile("" : "+v"(tid), "+v"(lane), "+s"(wave));
        const int64_t tok0 = bos + c0;
        const bool has_next = c0 + CH < len;

        if (TRACE && p.tr_h) {
#pragma unroll
            for (int u = 0; u < HPW; ++u) {
                const int th = wave + 8 * u;
                if (th < NH) {
                    const int ct = th / (DV / 32), dt = th % (DV / 32);
                    const int d = dv0 + 32 * dt + (lane & 31);
                    float* dst = p.tr_h + ((trace_chunk + chunk_idx) * p.Hv + hv) * DK * DK;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int c = 32 * ct + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        dst[(int64_t)c * DK + d] = hacc[u][r];
                    }
                }
            }
        }

        // ================= a1: gate cumsum (local part) and staging =================
        // Layout: lane cp = channel pair (channels 2cp, 2cp + 1), wave = rows
        // 8 wave .. 8 wave + 7.  lp = inclusive prefix sums of g log2(e) over the
        // wave's rows; the wave's total goes to Xs.
        const int cp = lane;
        float lp[8][2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            float acc = 0.f;
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) { acc += pf_g[rr][e] * LOG2E; lp[rr][e] = acc; }
        }
        *reinterpret_cast<f32x2*>(sXs + wave * 128 + 2 * cp) = f32x2{lp[7][0], lp[7][1]};
        // v tile (64 tokens x DV channels of this slice), stored transposed as fp16.
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int it = tid + NTHREADS * u;
            if (it < CH * DV / 8) {
                const int j = it / (DV / 8), c8 = it % (DV / 8);
                const uint32_t ww[4] = {pf_v[u].x, pf_v[u].y, pf_v[u].z, pf_v[u].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float f = (e & 1) ? bf_hi(ww[e >> 1]) : bf_lo(ww[e >> 1]);
                    reinterpret_cast<_Float16*>(smem + L::Vt)[(8 * c8 + e) * S72 + j] = (_Float16)f;
                }
            }
        }
        // Aqk and T diag(beta): the 20 lower 16x16 tiles of the workspace record.
#pragma unroll
        for (int u = 0; u < WPT; ++u) {
            const int it = tid + NTHREADS * u;
            if (it < WS_RECORD_BYTES / 16) {
                const int t = it >> 5, r = (it >> 1) & 15, h = it & 1;
                const int tt = t % 10;
                const int I = tt >= 6 ? 3 : (tt >= 3 ? 2 : (tt >= 1 ? 1 : 0));
                const int J = tt - I * (I + 1) / 2;
                *reinterpret_cast<uint4*>(smem + (t < 10 ? L::Aqk : L::T16) + ((16 * I + r) * S72 + 16 * J + 8 * h) * 2) =
                    pf_w[u];
            }
        }
        // The previous chunk's output, staged in Ost, goes out now: after this
        // chunk's g, v and workspace registers have been consumed and before their
        // next prefetch is issued.  Global stores share the vmcnt counter with
        // loads, so this order keeps every wait for prefetched data clear of
        // pending stores.
        if (c0 > 0) store_output(tok0 - CH, CH, tid);
        if (has_next) prefetch_gvw(c0 + CH, tid, lane, wave);
        lds_barrier();

        // Factors: G_r = (sum of the earlier waves' totals) + lp[r] in log2 units;
        //   Qg = scale q e^{G},  Kg = k e^{G},  Kh = k e^{G_last - G}.
        {
            f32x2 off = {0.f, 0.f}, all = {0.f, 0.f};
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const f32x2 x = *reinterpret_cast<const f32x2*>(sXs + w * 128 + 2 * cp);
                if (w < wave) off += x;
                all += x;
            }
            half8 kg[2], kh[2];
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const int row = 8 * wave + rr;
                const float G0 = off[0] + lp[rr][0], G1 = off[1] + lp[rr][1];
                const float e0 = fexp2(G0), e1 = fexp2(G1);
                const float h0 = fexp2(all[0] - G0), h1 = fexp2(all[1] - G1);
                const float q0 = bf_lo(pf_q[rr]), q1 = bf_hi(pf_q[rr]);
                const float k0 = bf_lo(pf_k[rr]), k1 = bf_hi(pf_k[rr]);
                *reinterpret_cast<uint32_t*>(smem + L::Qg + (row * S136 + 2 * cp) * 2) =
                    pack_h2(p.scale * q0 * e0, p.scale * q1 * e1);
                kg[0][rr] = (_Float16)(k0 * e0);
                kg[1][rr] = (_Float16)(k1 * e1);
                kh[0][rr] = (_Float16)(k0 * h0);
                kh[1][rr] = (_Float16)(k1 * h1);
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int c = 2 * cp + e;
                *reinterpret_cast<half8*>(smem + L::KgT + (c * S72 + 8 * wave) * 2) = kg[e];
                *reinterpret_cast<half8*>(smem + L::KhT + (c * S72 + 8 * wave) * 2) = kh[e];
            }
            if (wave == 0) *reinterpret_cast<f32x2*>(sGam + 2 * cp) = f32x2{fexp2(all[0]), fexp2(all[1])};
        }
        if (has_next) prefetch_qk(c0 + CH, lane, wave);
        lds_barrier();

        // ================= a4: W^T = (k e^G)^T (T diag beta)^T, U = T diag(beta) v =================
        {
            const int ct = wave >> 1, it = wave & 1;  // W^T tile: rows c (32ct..), cols i (32it..)
            f32x16 acc;
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[e] = 0.f;
            const int kmax = it == 0 ? 2 : 4;         // T is lower triangular
            for (int kk = 0; kk < kmax; ++kk) {
                const int ko = 16 * kk + 8 * (lane >> 5);
                const half8 a = lds_h8(smem, L::KgT + ((32 * ct + (lane & 31)) * S72 + ko) * 2);
                const half8 b = lds_h8(smem, L::T16 + ((32 * it + (lane & 31)) * S72 + ko) * 2);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
            }
            const int i = 32 * it + (lane & 31);
            const int Lc = (int)((len - c0) < CH ? (len - c0) : CH);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int c = 32 * ct + 8 * q4 + 4 * (lane >> 5);
                half4 h4;
#pragma unroll
                for (int e = 0; e < 4; ++e) h4[e] = (_Float16)(-acc[4 * q4 + e]);
                *reinterpret_cast<half4*>(smem + L::W + (i * S136 + c) * 2) = h4;
                if (TRACE && p.tr_W && s == 0 && i < Lc) {
                    float* dst = p.tr_W + ((tok0 + i) * p.Hv + hv) * DK + c;
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
            const int kmax = tu_it == 0 ? 2 : 4;
            for (int kk = 0; kk < kmax; ++kk) {
                const int ko = 16 * kk + 8 * (lane >> 5);
                const half8 a = lds_h8(smem, L::T16 + ((32 * tu_it + (lane & 31)) * S72 + ko) * 2);
                const half8 b = lds_h8(smem, L::Vt + ((32 * tu_dt + (lane & 31)) * S72 + ko) * 2);
                uacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, uacc, 0, 0, 0);
            }
            if (TRACE && p.tr_U) {
                const int Lc = (int)((len - c0) < CH ? (len - c0) : CH);
                const int d = dv0 + 32 * tu_dt + (lane & 31);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int i = 32 * tu_it + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                    if (i < Lc) p.tr_U[((tok0 + i) * p.Hv + hv) * DK + d] = uacc[e];
                }
            }
        }
        lds_barrier();

        // ================= a5 (first half): v_new = U - W h =================
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
            const int Lc = (int)((len - c0) < CH ? (len - c0) : CH);
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
        lds_barrier();

        // ================= a6: o^T = h^T (scale q e^G)^T + v_new^T Aqk^T =================
        // Results go to the output staging tile Ost; they are written to HBM during
        // the next chunk (or after the loop).
        {
            const int wo = 7 - wave;
            if (wo < NU) {
                const int it = wo / (DV / 32), dt = wo % (DV / 32);
                f32x16 acc, acc1;   // two accumulation chains, summed at the end
#pragma unroll
                for (int e = 0; e < 16; ++e) { acc[e] = 0.f; acc1[e] = 0.f; }
#pragma unroll
                for (int kk = 0; kk < 8; kk += 2) {
                    const int ko = 16 * kk + 8 * (lane >> 5);
                    const half8 a0 = lds_h8(smem, L::HT + ((32 * dt + (lane & 31)) * S136 + ko) * 2);
                    const half8 b0 = lds_h8(smem, L::Qg + ((32 * it + (lane & 31)) * S136 + ko) * 2);
                    const half8 a1 = lds_h8(smem, L::HT + ((32 * dt + (lane & 31)) * S136 + ko + 16) * 2);
                    const half8 b1 = lds_h8(smem, L::Qg + ((32 * it + (lane & 31)) * S136 + ko + 16) * 2);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, acc, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, acc1, 0, 0, 0);
                }
                const int kmax = it == 0 ? 2 : 4;
                for (int kk = 0; kk < kmax; kk += 2) {
                    const int ko = 16 * kk + 8 * (lane >> 5);
                    const half8 a0 = lds_h8(smem, L::VnT + ((32 * dt + (lane & 31)) * S72 + ko) * 2);
                    const half8 b0 = lds_h8(smem, L::Aqk + ((32 * it + (lane & 31)) * S72 + ko) * 2);
                    const half8 a1 = lds_h8(smem, L::VnT + ((32 * dt + (lane & 31)) * S72 + ko + 16) * 2);
                    const half8 b1 = lds_h8(smem, L::Aqk + ((32 * it + (lane & 31)) * S72 + ko + 16) * 2);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, acc, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, acc1, 0, 0, 0);
                }
                acc += acc1;
                const int i = 32 * it + (lane & 31);
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int d = 32 * dt + 8 * q4 + 4 * (lane >> 5);
                    uint2 w;
                    w.x = pack_bf2(acc[4 * q4], acc[4 * q4 + 1]);
                    w.y = pack_bf2(acc[4 * q4 + 2], acc[4 * q4 + 3]);
                    *reinterpret_cast<uint2*>(smem + L::Ost + (i * (DV + 8) + d) * 2) = w;
                }
            }
        }
        // ================= a5 (second half): h <- Diag(e^{G_last}) h + Khat^T v_new =================
#pragma unroll
        for (int u = 0; u < HPW; ++u) {
            const int th = wave + 8 * u;
            if (th < NH) {
                const int ct = th / (DV / 32), dt = th % (DV / 32);
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x4 gm = *reinterpret_cast<const f32x4*>(sGam + 32 * ct + 8 * q4 + 4 * (lane >> 5));
#pragma unroll
                    for (int e = 0; e < 4; ++e) hacc[u][4 * q4 + e] *= gm[e];
                }
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int ko = 16 * kk + 8 * (lane >> 5);
                    const half8 a = lds_h8(smem, L::KhT + ((32 * ct + (lane & 31)) * S72 + ko) * 2);
                    const half8 b = lds_h8(smem, L::VnT + ((32 * dt + (lane & 31)) * S72 + ko) * 2);
                    hacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, hacc[u], 0, 0, 0);
                }
            }
        }
        lds_barrier();
#pragma unroll
        for (int u = 0; u < HPW; ++u) {
            const int th = wave + 8 * u;
            if (th < NH) {
                const int ct = th / (DV / 32), dt = th % (DV / 32);
                const int d = 32 * dt + (lane & 31);
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int c = 32 * ct + 8 * q4 + 4 * (lane >> 5);
                    half4 h4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) h4[e] = (_Float16)hacc[u][4 * q4 + e];
                    *reinterpret_cast<half4*>(smem + L::HT + (d * S136 + c) * 2) = h4;
                }
            }
        }
        // The next chunk writes Xs, Vt, Aqk and T16 before its first barrier; none of
        // them aliases HT, and every read of them in this chunk happened before the
        // barrier above.  Ost is read (and then rewritten) only after later barriers.
    }

    // ---- output of the last chunk (staged in Ost before the loop's last barrier) ----
    if (len > 0) {
        const int64_t last = (len - 1) / CH * CH;
        store_output(bos + last, (int)(len - last), tid);
    }

    // ---- final state ----
    if (p.hT) {
#pragma unroll
        for (int u = 0; u < HPW; ++u) {
            const int th = wave + 8 * u;
            if (th < NH) {
                const int ct = th / (DV / 32), dt = th % (DV / 32);
                const int d = 32 * dt + (lane & 31);
                float* dst = p.hT + ((int64_t)n * p.Hv + hv) * DK * DK + dv0 + d;
#pragma unroll
                for (int r2 = 0; r2 < 16; ++r2) {
                    const int c = 32 * ct + 8 * (r2 >> 2) + 4 * (lane >> 5) + (r2 & 3);
                    dst[(int64_t)c * DK] = hacc[u][r2];
                }
            }
        }
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

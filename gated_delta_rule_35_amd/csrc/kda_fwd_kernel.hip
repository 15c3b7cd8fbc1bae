// Fused KDA chunked forward for gfx950 (MI355X, CDNA4).
//
// One work-group of 512 threads (8 wave64s) owns one (sequence, value head,
// dv slice) and walks that sequence's chunks of 64 tokens in order.  Per chunk
// it runs the six stages of the chunked method that the pages list ("cuLA PR
// #131: SM100/SM103 KDA forward to pure CuTeDSL", Summary: chunk intra, FP32 Akk
// inversion, recompute W/U; "cuLA REPO_LAYOUT.md", ops/: chunk delta-H and
// forward output) entirely in LDS and registers:
//
//   a1  gate cumsum         G = chunk-local inclusive cumsum of g (fp32)
//   a2  intra               Aqk = scale (q e^{G_i - G_j} k^T), j <= i
//                           Akk = beta_i (k e^{G_i - G_j} k^T), j < i      (MFMA)
//   a3  FP32 inversion      T = (I + Akk)^{-1}, blocked forward substitution
//   a4  W/U recompute       W = T (beta k e^G), U = T (beta v)             (MFMA)
//   a5  delta-H scan        v_new = U - W h;
//                           h <- Diag(e^{G_last}) h + (k e^{G_last - G})^T v_new
//   a6  output              o = (scale q e^G) h + Aqk v_new                 (MFMA)
//
// The state slice h (128 x DV, fp32) lives in MFMA accumulator registers for
// the whole sequence; HBM sees q, k, v, g, beta once and o once, plus the states.
//
// MFMA operands are fp16 (bf16 inputs convert exactly when in range; the
// rounding of derived operands to fp16 keeps the result within tolerance where
// bf16 would not).  Accumulation is fp32.
//
// Per-channel decay inside MFMA products.  exp(G_i - G_j) is factored through
// an anchor row a: exp(G_i - G_a) * exp(G_a - G_j).  The 64 rows form four
// 16-row blocks.  For an off-diagonal block pair (row block I > column block J)
// the anchor is the first row of I, so both factors are <= 1.  For a diagonal
// block the anchor is the block's first row: the row factor is <= 1 and the
// column factor is <= exp(block decay).  When a 16-row block decays by more
// than exp(-8) on some channel (far outside the usual gate range), the
// diagonal blocks of that chunk are recomputed element by element in fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_kernel.h"

namespace kda {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int CH = 64;       // chunk length
constexpr int DK = 128;      // key head dim
constexpr int NTHREADS = 512;
constexpr float GUARD_DECAY = 8.0f;

// LDS strides in elements.
constexpr int S136 = 136;    // fp16 rows of 128 (+8 pad)
constexpr int S72 = 72;      // fp16 rows of 64 (+8 pad)
constexpr int S68 = 68;      // fp32 rows of 64 (+4 pad)
constexpr int TS = 20;       // fp32 columns of a 16x16 column-major block (+4 pad)

template <int DV>
struct Lds {
    // Region R1, phase A view (intra operands, fp16):
    static constexpr int Aq = 0;                         // [64][136] q * F
    static constexpr int Ak = Aq + 64 * S136 * 2;        // [64][136] k * F
    static constexpr int Bd = Ak + 64 * S136 * 2;        // [64][136] k * e^{G_b - G_j}
    static constexpr int Bo = Bd + 64 * S136 * 2;        // [96][136] k * e^{G_{b_I} - G_j}, 6 pairs
    static constexpr int R1_A_END = Bo + 96 * S136 * 2;
    // Region R1, phase B view:
    static constexpr int A32 = 0;                        // [64][68] fp32 Akk, then T
    static constexpr int Aqk = A32 + 64 * S68 * 4;       // [64][72] fp16
    static constexpr int T16 = Aqk + 64 * S72 * 2;       // [64][72] fp16 T diag(beta)
    static constexpr int W = T16 + 64 * S72 * 2;         // [64][136] fp16, -W
    // fp32 inversion scratch inside W's slot, column-major 16x16 blocks (stride TS):
    static constexpr int TtD = W;                        // 4 diagonal T blocks
    static constexpr int Yt = TtD + 4 * 16 * TS * 4;     // 2 products A_IJ T_JJ
    static constexpr int T1t = Yt + 2 * 16 * TS * 4;     // T_10, T_32
    static constexpr int Xt = T1t + 2 * 16 * TS * 4;     // 4 blocks of the 32x32 step
    static constexpr int VnT = W + 64 * S136 * 2;        // [DV][72] fp16, v_new^T
    static constexpr int Qg = VnT + DV * S72 * 2;        // [64][136] fp16, scale q e^G
    static constexpr int KgT = Qg + 64 * S136 * 2;       // [128][72] fp16, (k e^G)^T
    static constexpr int KhT = KgT + 128 * S72 * 2;      // [128][72] fp16, (k e^{G_last-G})^T
    static constexpr int R1_B_END = KhT + 128 * S72 * 2;
    static constexpr int R1_END = R1_A_END > R1_B_END ? R1_A_END : R1_B_END;
    // Persistent / small regions.
    static constexpr int Vt = R1_END;                    // [DV][72] fp16, v^T
    static constexpr int HT = Vt + DV * S72 * 2;         // [DV][136] fp16, h^T
    static constexpr int Blk = HT + DV * S136 * 2;       // 3 x [4][128] fp32: g_b, Q_b, tot
    static constexpr int Scal = Blk + 3 * 4 * 128 * 4;   // Eb[4], Khs[4], InvR[4], Lam[6], Gam[1] x 128
    static constexpr int Beta = Scal + 19 * 128 * 4;     // [64] fp32
    static constexpr int Flag = Beta + 64 * 4;           // int: some chunk block decays past the guard
    static constexpr int BYTES = Flag + 16;
    static_assert(Xt + 4 * 16 * TS * 4 <= VnT, "inversion scratch overflows W slot");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

__device__ __forceinline__ uint16_t f2bf(float f) {  // round to nearest even
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Row (16-lane) shifts through DPP; lanes whose source lies outside the row read 0.
__device__ __forceinline__ float row_shr(float x, int n) {
    int v = __float_as_int(x);
    int r;
    switch (n) {
        case 1: r = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true); break;
        case 2: r = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true); break;
        case 4: r = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true); break;
        default: r = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true); break;
    }
    return __int_as_float(r);
}
__device__ __forceinline__ float row_shl(float x, int n) {
    int v = __float_as_int(x);
    int r;
    switch (n) {
        case 1: r = __builtin_amdgcn_update_dpp(0, v, 0x101, 0xf, 0xf, true); break;
        case 2: r = __builtin_amdgcn_update_dpp(0, v, 0x102, 0xf, 0xf, true); break;
        case 4: r = __builtin_amdgcn_update_dpp(0, v, 0x104, 0xf, 0xf, true); break;
        default: r = __builtin_amdgcn_update_dpp(0, v, 0x108, 0xf, 0xf, true); break;
    }
    return __int_as_float(r);
}

__device__ __forceinline__ float fexp(float x) { return __expf(x); }

__device__ __forceinline__ half8 lds_h8(const char* smem, int byte_off) {
    return *reinterpret_cast<const half8*>(smem + byte_off);
}

// C += A B for 16x16 fp32 blocks on v_mfma_f32_16x16x4f32.  A is row-major (row
// stride sa), B column-major (Bt[n][k], stride sb).  Instruction s takes the k
// indices 4*(lane/16) + s, so every lane loads its four A and four B values with
// one 16-byte read each.  C: lane holds rows 4*(lane/16) .. +3 of column lane%16.
__device__ __forceinline__ f32x4 mm16(const float* A, int sa, const float* Bt, int sb, f32x4 c, int lane) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(A + (lane & 15) * sa + 4 * (lane >> 4));
    const f32x4 b = *reinterpret_cast<const f32x4*>(Bt + (lane & 15) * sb + 4 * (lane >> 4));
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
    return c;
}
__device__ __forceinline__ void store_colmajor(float* Ct, f32x4 c, int lane) {
    *reinterpret_cast<f32x4*>(Ct + (lane & 15) * TS + 4 * (lane >> 4)) = c;
}
__device__ __forceinline__ void store_rowmajor(float* C, int sc, f32x4 c, int lane) {
#pragma unroll
    for (int e = 0; e < 4; ++e) C[(4 * (lane >> 4) + e) * sc + (lane & 15)] = c[e];
}

// Index of an off-diagonal 16x16 block pair (I > J) in 0..5.
__device__ __forceinline__ int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

template <int DV, bool TRACE>
__global__ void __launch_bounds__(NTHREADS, 1) kda_fwd_kernel(const KdaParams p) {
    using L = Lds<DV>;
    constexpr int S = DK / DV;          // dv slices
    constexpr int NU = 2 * (DV / 32);   // 32x32 tiles of a 64 x DV matrix
    constexpr int NH = 4 * (DV / 32);   // 32x32 tiles of the 128 x DV state
    constexpr int HPW = (NH + 7) / 8;   // state tiles per wave
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
    if (p.cu) {
        int64_t a = p.cu[n], e = p.cu[n + 1];
        a = a < 0 ? 0 : (a > p.T ? p.T : a);
        e = e < a ? a : (e > p.T ? p.T : e);
        bos = a;
        len = e - a;
    } else {
        bos = (int64_t)n * p.T;
        len = p.T;
    }
    const int64_t qk_tok = (int64_t)p.Hq * DK;   // token stride of q, k
    const int64_t v_tok = (int64_t)p.Hv * DK;    // token stride of v, g, o
    const int dv0 = s * DV;

    int64_t trace_chunk = 0;   // index of this sequence's first chunk in the h dump
    if (TRACE && p.tr_h) {
        if (p.cu) {
            for (int m = 0; m < n; ++m) {
                int64_t a = p.cu[m], e = p.cu[m + 1];
                a = a < 0 ? 0 : (a > p.T ? p.T : a);
                e = e < a ? a : (e > p.T ? p.T : e);
                trace_chunk += (e - a + CH - 1) / CH;
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

    float* sBlkGb = reinterpret_cast<float*>(smem + L::Blk);
    float* sBlkQb = sBlkGb + 512;
    float* sBlkTot = sBlkQb + 512;
    float* sEb = reinterpret_cast<float*>(smem + L::Scal);
    float* sKhs = sEb + 512;
    float* sInvR = sKhs + 512;
    float* sLam = sInvR + 512;
    float* sGam = sLam + 768;
    float* sBeta = reinterpret_cast<float*>(smem + L::Beta);
    int* sFlag = reinterpret_cast<int*>(smem + L::Flag);
    float* sA32 = reinterpret_cast<float*>(smem + L::A32);

    // Prefetch registers: one chunk's inputs in the a1 thread layout (row = lane,
    // channels 16*wave ..), loaded one chunk ahead of their use.
    constexpr int VPT = (CH * DV / 8 + NTHREADS - 1) / NTHREADS;   // 16-byte pieces of v per thread
    float pf_g[16];
    uint32_t pf_q[8], pf_k[8];
    uint4 pf_v[VPT];
    float pf_b = 0.f;
    auto prefetch = [&](int64_t cstart, int tid_, int lane_, int wave_) {
        const int Ln = (int)((len - cstart) < CH ? (len - cstart) : CH);
        const int64_t t0 = bos + cstart;
        if (lane_ < Ln) {
            const int64_t tok = t0 + lane_;
            const float4* gp = reinterpret_cast<const float4*>(p.g + tok * v_tok + (int64_t)hv * DK + 16 * wave_);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 t4 = gp[i];
                pf_g[4 * i] = t4.x; pf_g[4 * i + 1] = t4.y; pf_g[4 * i + 2] = t4.z; pf_g[4 * i + 3] = t4.w;
            }
            const uint4* qp = reinterpret_cast<const uint4*>(p.q + tok * qk_tok + (int64_t)hq * DK + 16 * wave_);
            const uint4* kp = reinterpret_cast<const uint4*>(p.k + tok * qk_tok + (int64_t)hq * DK + 16 * wave_);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint4 a = qp[i], b = kp[i];
                pf_q[4 * i] = a.x; pf_q[4 * i + 1] = a.y; pf_q[4 * i + 2] = a.z; pf_q[4 * i + 3] = a.w;
                pf_k[4 * i] = b.x; pf_k[4 * i + 1] = b.y; pf_k[4 * i + 2] = b.z; pf_k[4 * i + 3] = b.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) pf_g[i] = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) { pf_q[i] = 0; pf_k[i] = 0; }
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int it = tid_ + NTHREADS * u;
            const int j = it / (DV / 8), c8 = it % (DV / 8);
            pf_v[u] = make_uint4(0, 0, 0, 0);
            if (it < CH * DV / 8 && j < Ln)
                pf_v[u] = *reinterpret_cast<const uint4*>(p.v + (t0 + j) * v_tok + (int64_t)hv * DK + dv0 + 8 * c8);
        }
        if (tid_ < CH) {
            float b = 0.f;
            if (tid_ < Ln) {
                const int64_t idx = (t0 + tid_) * p.Hv + hv;
                b = p.beta_f32 ? reinterpret_cast<const float*>(p.beta)[idx]
                               : bf2f(reinterpret_cast<const uint16_t*>(p.beta)[idx]);
            }
            pf_b = b;
        }
    };
    if (len > 0) prefetch(0, tid, lane, wave);

    int64_t chunk_idx = 0;
    for (int64_t c0 = 0; c0 < len; c0 += CH, ++chunk_idx) {
        // Opaque per-iteration copies of the thread coordinates: they stop the
        // compiler from hoisting every LDS address of the loop body out of the
        // chunk loop (which would hold hundreds of addresses in VGPRs).
        int tid = tid_o, lane = lane_o, wave = wave_o;
        asm volatile("" : "+v"(tid), "+v"(lane), "+s"(wave));
        const int Lc = (int)((len - c0) < CH ? (len - c0) : CH);
        const int64_t tok0 = bos + c0;

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

        // ================= a1: gate cumsum (inputs were prefetched) =================
        // Thread layout for this phase: row r = lane (token within the chunk),
        // channel group cg = wave (channels 16cg .. 16cg+15).
        const int r = lane, cg = wave;
        const bool rvalid = r < Lc;
        float gv[16];
        uint32_t qw[8], kw[8];   // 16 bf16 values each, two per word
#pragma unroll
        for (int i = 0; i < 16; ++i) gv[i] = pf_g[i];
#pragma unroll
        for (int i = 0; i < 8; ++i) { qw[i] = pf_q[i]; kw[i] = pf_k[i]; }
        const float beta_r = pf_b;
        uint4 vcur[VPT];
#pragma unroll
        for (int i = 0; i < VPT; ++i) vcur[i] = pf_v[i];
        // Start the next chunk's loads now; they land while this chunk computes.
        if (c0 + CH < len) prefetch(c0 + CH, tid, lane, wave);

        auto qf = [&](int ch) { return __uint_as_float((ch & 1) ? (qw[ch >> 1] & 0xffff0000u) : (qw[ch >> 1] << 16)); };
        auto kf = [&](int ch) { return __uint_as_float((ch & 1) ? (kw[ch >> 1] & 0xffff0000u) : (kw[ch >> 1] << 16)); };
        // Within each 16-row block: P_r = sum_{b < r' <= r} g (so exp(P) = e^{G_r - G_b}),
        // Q_r = sum_{r < r' <= e} g (so exp(Q) = e^{G_e - G_r}).
        // F = exp(P) and R = exp(Q) are the factors the intra operands need.
        float Fv[16], Rv[16];
        float Pt[TRACE ? 16 : 1];
        const bool first_row = (r & 15) == 0;
        float qb_first[16];
#pragma unroll
        for (int ch = 0; ch < 16; ++ch) {
            float x = first_row ? 0.f : gv[ch];
            x += row_shr(x, 1);
            x += row_shr(x, 2);
            x += row_shr(x, 4);
            x += row_shr(x, 8);
            if constexpr (TRACE) Pt[ch] = x;
            Fv[ch] = fexp(x);
            float y = row_shl(gv[ch], 1);
            y += row_shl(y, 1);
            y += row_shl(y, 2);
            y += row_shl(y, 4);
            y += row_shl(y, 8);
            Rv[ch] = fexp(y);
            qb_first[ch] = y;
        }
        if (first_row) {
            const int I = r >> 4;
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                f32x4 a, b, t;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a[e] = gv[4 * c4 + e];
                    b[e] = qb_first[4 * c4 + e];
                    t[e] = a[e] + b[e];
                }
                *reinterpret_cast<f32x4*>(sBlkGb + I * 128 + 16 * cg + 4 * c4) = a;
                *reinterpret_cast<f32x4*>(sBlkQb + I * 128 + 16 * cg + 4 * c4) = b;
                *reinterpret_cast<f32x4*>(sBlkTot + I * 128 + 16 * cg + 4 * c4) = t;
            }
        }
        if (tid < CH) sBeta[tid] = beta_r;
        if (tid == 0) *sFlag = 0;
        // v tile (64 tokens x DV channels of this slice), stored transposed as fp16.
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int it = tid + NTHREADS * u;
            if (it < CH * DV / 8) {
                const int j = it / (DV / 8), c8 = it % (DV / 8);
                const uint32_t ww[4] = {vcur[u].x, vcur[u].y, vcur[u].z, vcur[u].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint16_t bits = (uint16_t)((ww[e >> 1] >> (16 * (e & 1))) & 0xffff);
                    reinterpret_cast<_Float16*>(smem + L::Vt)[(8 * c8 + e) * S72 + j] = (_Float16)bf2f(bits);
                }
            }
        }
        __syncthreads();

        // Per (block I, channel c) factors.  Thread layout: I = tid / 128, c = tid % 128.
        {
            const int I = tid >> 7, c = tid & 127;
            float tot[4];
#pragma unroll
            for (int K = 0; K < 4; ++K) tot[K] = sBlkTot[K * 128 + c];
            const float gb = sBlkGb[I * 128 + c], qb = sBlkQb[I * 128 + c];
            float off = 0.f;
            for (int K = 0; K < I; ++K) off += tot[K];
            float tail = 0.f;
            for (int K = 3; K > I; --K) tail += tot[K];
            sEb[I * 128 + c] = fexp(off + gb);            // e^{G_{b_I}}
            sKhs[I * 128 + c] = fexp(tail);               // e^{G_last - G_{e_I}}
            sInvR[I * 128 + c] = fexp(-qb);               // e^{G_{b_I} - G_{e_I}}
            float acc = gb;                               // e^{G_{b_I} - G_{e_J}}, J = I-1, I-2, ...
            for (int J = I - 1; J >= 0; --J) {
                sLam[pair_index(I, J) * 128 + c] = fexp(acc);
                acc += tot[J];
            }
            if (I == 0) sGam[c] = fexp(((tot[0] + tot[1]) + tot[2]) + tot[3]);
            if (-qb > GUARD_DECAY) *sFlag = 1;
        }
        __syncthreads();
        const bool guard = *sFlag != 0;   // block-uniform

        // Intra operands (thread layout: row r, channel group cg).  All LDS reads first.
        {
            const int I = r >> 4;
            float invR[16];
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                const f32x4 t = *reinterpret_cast<const f32x4*>(sInvR + I * 128 + 16 * cg + 4 * c4);
#pragma unroll
                for (int e = 0; e < 4; ++e) invR[4 * c4 + e] = t[e];
            }
            half8 aq[2], ak[2], bd[2];
#pragma unroll
            for (int ch = 0; ch < 16; ++ch) {
                const float qx = qf(ch), kx = kf(ch);
                aq[ch >> 3][ch & 7] = (_Float16)(qx * Fv[ch]);
                ak[ch >> 3][ch & 7] = (_Float16)(kx * Fv[ch]);
                bd[ch >> 3][ch & 7] = (_Float16)(kx * Rv[ch] * invR[ch]);
            }
            const int off = (r * S136 + 16 * cg) * 2;
            *reinterpret_cast<half8*>(smem + L::Aq + off) = aq[0];
            *reinterpret_cast<half8*>(smem + L::Aq + off + 16) = aq[1];
            *reinterpret_cast<half8*>(smem + L::Ak + off) = ak[0];
            *reinterpret_cast<half8*>(smem + L::Ak + off + 16) = ak[1];
            *reinterpret_cast<half8*>(smem + L::Bd + off) = bd[0];
            *reinterpret_cast<half8*>(smem + L::Bd + off + 16) = bd[1];
            for (int I2 = I + 1; I2 < 4; ++I2) {
                const int pi = pair_index(I2, I);
                float lam[16];
#pragma unroll
                for (int c4 = 0; c4 < 4; ++c4) {
                    const f32x4 t = *reinterpret_cast<const f32x4*>(sLam + pi * 128 + 16 * cg + 4 * c4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) lam[4 * c4 + e] = t[e];
                }
                half8 bo[2];
#pragma unroll
                for (int ch = 0; ch < 16; ++ch) bo[ch >> 3][ch & 7] = (_Float16)(kf(ch) * Rv[ch] * lam[ch]);
                const int o2 = ((16 * pi + (r & 15)) * S136 + 16 * cg) * 2;
                *reinterpret_cast<half8*>(smem + L::Bo + o2) = bo[0];
                *reinterpret_cast<half8*>(smem + L::Bo + o2 + 16) = bo[1];
            }
            if constexpr (TRACE) {
                if (p.tr_G && s == 0 && rvalid) {
                    float* dst = p.tr_G + ((tok0 + r) * p.Hv + hv) * DK + 16 * cg;
#pragma unroll
                    for (int ch = 0; ch < 16; ++ch) {
                        const int c = 16 * cg + ch;
                        float offv = 0.f;
                        for (int K = 0; K < I; ++K) offv += sBlkTot[K * 128 + c];
                        dst[ch] = offv + sBlkGb[I * 128 + c] + Pt[ch];
                    }
                }
            }
        }
        __syncthreads();

        // ================= a2: intra-chunk Aqk / Akk on MFMA =================
        // 20 jobs of 16x16 output tiles: (matrix, I, J) with J <= I.  Each tile is
        // computed transposed (rows j, cols i) so that results store as rows of i.
        f32x4 iacc[3];
        int jobI[3], jobJ[3], jobM[3];
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int job = wave + 8 * u;
            jobM[u] = -1;
            if (job < 20) {
                const int m = job / 10, pidx = job % 10;
                // pidx -> (I, J) over the lower triangle, row by row
                const int I = pidx >= 6 ? 3 : (pidx >= 3 ? 2 : (pidx >= 1 ? 1 : 0));
                const int J = pidx - I * (I + 1) / 2;
                jobM[u] = m; jobI[u] = I; jobJ[u] = J;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                const int rowB = (I == J) ? (L::Bd + ((16 * J + (lane & 15)) * S136) * 2)
                                          : (L::Bo + ((16 * pair_index(I, J) + (lane & 15)) * S136) * 2);
                const int rowA = (m == 0 ? L::Aq : L::Ak) + ((16 * I + (lane & 15)) * S136) * 2;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int co = (32 * kk + 8 * (lane >> 4)) * 2;
                    const half8 a = lds_h8(smem, rowB + co);
                    const half8 b = lds_h8(smem, rowA + co);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
                }
                iacc[u] = acc;
            }
        }
        // LDS reads for the derived operands below, issued before the barrier.
        float ebv[16], khs[16];
        {
            const int I = r >> 4;
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(sEb + I * 128 + 16 * cg + 4 * c4);
                const f32x4 b = *reinterpret_cast<const f32x4*>(sKhs + I * 128 + 16 * cg + 4 * c4);
#pragma unroll
                for (int e = 0; e < 4; ++e) { ebv[4 * c4 + e] = a[e]; khs[4 * c4 + e] = b[e]; }
            }
        }
        __syncthreads();
        // Store the lower tiles (masked, scaled), zero the upper ones.
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            if (jobM[u] >= 0) {
                const int I = jobI[u], J = jobJ[u];
                const int i = 16 * I + (lane & 15);
                const int j0 = 16 * J + 4 * (lane >> 4);
                if (jobM[u] == 0) {
                    half4 h4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) h4[e] = (_Float16)((j0 + e <= i) ? p.scale * iacc[u][e] : 0.f);
                    *reinterpret_cast<half4*>(smem + L::Aqk + (i * S72 + j0) * 2) = h4;
                    if (TRACE && p.tr_Aqk && s == 0 && i < Lc) {
                        float* dst = p.tr_Aqk + ((tok0 + i) * p.Hv + hv) * CH + j0;
#pragma unroll
                        for (int e = 0; e < 4; ++e) dst[e] = (j0 + e <= i) ? p.scale * iacc[u][e] : 0.f;
                    }
                } else {
                    const float bi = sBeta[i];
                    f32x4 v4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v4[e] = (j0 + e < i) ? bi * iacc[u][e] : 0.f;
                    *reinterpret_cast<f32x4*>(smem + L::A32 + (i * S68 + j0) * 4) = v4;
                }
            }
        }
        {
            // Upper 16x16 tiles (I < J) of Akk (fp32) and Aqk (fp16) are zero.
            const int tile = tid >> 6, w64 = tid & 63;   // 8 slots, 6 used
            if (tile < 6) {
                const int I = tile < 3 ? 0 : (tile < 5 ? 1 : 2);
                const int J = tile < 3 ? tile + 1 : (tile < 5 ? tile - 1 : 3);
                const int m = w64 >> 2, q4 = w64 & 3;
                const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
                *reinterpret_cast<f32x4*>(smem + L::A32 + ((16 * I + m) * S68 + 16 * J + 4 * q4) * 4) = z4;
                half4 hz = {(_Float16)0.f, (_Float16)0.f, (_Float16)0.f, (_Float16)0.f};
                *reinterpret_cast<half4*>(smem + L::Aqk + ((16 * I + m) * S72 + 16 * J + 4 * q4) * 2) = hz;
                if (TRACE && p.tr_Aqk && s == 0 && 16 * I + m < Lc) {
                    float* dst = p.tr_Aqk + ((tok0 + 16 * I + m) * p.Hv + hv) * CH + 16 * J + 4 * q4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[e] = 0.f;
                }
            }
        }
        if (guard) {
            // Exact fp32 diagonal blocks for strongly decaying chunks.
            __syncthreads();
            for (int idx = tid; idx < 4 * 256; idx += NTHREADS) {
                const int B = idx >> 8, m = (idx >> 4) & 15, nn = idx & 15;
                if (nn > m) continue;
                const int i = 16 * B + m, j = 16 * B + nn;
                float sq = 0.f, sk = 0.f;
                if (i < Lc) {
                    const uint16_t* qi = p.q + (tok0 + i) * qk_tok + (int64_t)hq * DK;
                    const uint16_t* ki = p.k + (tok0 + i) * qk_tok + (int64_t)hq * DK;
                    const uint16_t* kj = p.k + (tok0 + j) * qk_tok + (int64_t)hq * DK;
                    for (int c = 0; c < DK; ++c) {
                        float dsum = 0.f;
                        for (int rr = j + 1; rr <= i; ++rr) dsum += p.g[(tok0 + rr) * v_tok + (int64_t)hv * DK + c];
                        const float e = fexp(dsum);
                        const float kjv = bf2f(kj[c]) * e;
                        sq += bf2f(qi[c]) * kjv;
                        sk += bf2f(ki[c]) * kjv;
                    }
                }
                reinterpret_cast<_Float16*>(smem + L::Aqk)[i * S72 + j] = (_Float16)(p.scale * sq);
                sA32[i * S68 + j] = (nn < m) ? sBeta[i] * sk : 0.f;
                if (TRACE && p.tr_Aqk && s == 0 && i < Lc) p.tr_Aqk[((tok0 + i) * p.Hv + hv) * CH + j] = p.scale * sq;
            }
        }
        // Derived operands for W, the output and the state update (row r, channels 16cg..).
        {
            half8 qg[2];
#pragma unroll
            for (int ch = 0; ch < 16; ++ch) {
                const int c = 16 * cg + ch;
                const float kx = kf(ch);
                qg[ch >> 3][ch & 7] = (_Float16)(p.scale * qf(ch) * Fv[ch] * ebv[ch]);
                reinterpret_cast<_Float16*>(smem + L::KgT)[c * S72 + r] = (_Float16)(kx * Fv[ch] * ebv[ch]);
                reinterpret_cast<_Float16*>(smem + L::KhT)[c * S72 + r] = (_Float16)(kx * Rv[ch] * khs[ch]);
            }
            const int off = (r * S136 + 16 * cg) * 2;
            *reinterpret_cast<half8*>(smem + L::Qg + off) = qg[0];
            *reinterpret_cast<half8*>(smem + L::Qg + off + 16) = qg[1];
        }
        __syncthreads();
        if (TRACE && p.tr_Akk && s == 0) {
            for (int idx = tid; idx < CH * CH; idx += NTHREADS) {
                const int i = idx >> 6, j = idx & 63;
                if (i < Lc) p.tr_Akk[((tok0 + i) * p.Hv + hv) * CH + j] = sA32[i * S68 + j];
            }
        }

        // ================= a3: T = (I + Akk)^{-1} in fp32 =================
        // Diagonal 16x16 blocks: wave 0, lane = (block, column); forward substitution.
        // Results go back row-major into the diagonal blocks of A32 and column-major
        // into the TtD scratch (the B-operand layout of the fp32 MFMA products below).
        float* sTtD = reinterpret_cast<float*>(smem + L::TtD);
        float* sYt = reinterpret_cast<float*>(smem + L::Yt);
        float* sT1t = reinterpret_cast<float*>(smem + L::T1t);
        float* sXt = reinterpret_cast<float*>(smem + L::Xt);
        if (wave == 0) {
            const int B = lane >> 4, j = lane & 15;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int kk = 0; kk < 15; ++kk) {
#pragma unroll
                for (int i = kk + 1; i < 16; ++i) x[i] -= sA32[(16 * B + i) * S68 + 16 * B + kk] * x[kk];
            }
            // Diagonal blocks are read only by this wave; write back after all reads.
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
            for (int i = 0; i < 16; ++i) sA32[(16 * B + i) * S68 + 16 * B + j] = x[i];
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                f32x4 v4 = {x[4 * i4], x[4 * i4 + 1], x[4 * i4 + 2], x[4 * i4 + 3]};
                *reinterpret_cast<f32x4*>(sTtD + (B * 16 + j) * TS + 4 * i4) = v4;
            }
        }
        __syncthreads();
        // Off-diagonal blocks on fp32 MFMA (16x16x4): T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ,
        // by doubling: first (1,0) and (3,2), then the lower-left 32x32 block.
        // mm16 multiplies a row-major A block by a column-major B block.
        if (wave < 2) {
            // wave 0: pair (1,0); wave 1: pair (3,2)
            const int I = wave == 0 ? 1 : 3, J = I - 1;
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
            y = mm16(sA32 + (16 * I) * S68 + 16 * J, S68, sTtD + J * 16 * TS, TS, y, lane);
            store_colmajor(sYt + wave * 16 * TS, y, lane);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
            t = mm16(sA32 + (16 * I) * S68 + 16 * I, S68, sYt + wave * 16 * TS, TS, t, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = -t[e];
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            store_rowmajor(sA32 + (16 * I) * S68 + 16 * J, S68, t, lane);   // replaces A_IJ, no longer read
            store_colmajor(sT1t + wave * 16 * TS, t, lane);
        }
        __syncthreads();
        if (wave < 4) {
            // X_IJ = sum_{K=J}^{1} A_IK T_KJ for I in {2,3}, J in {0,1}; wave = 2 (I-2) + J
            const int I = 2 + (wave >> 1), J = wave & 1;
            f32x4 x4 = {0.f, 0.f, 0.f, 0.f};
            if (J == 0) {
                x4 = mm16(sA32 + (16 * I) * S68 + 0, S68, sTtD + 0 * 16 * TS, TS, x4, lane);      // A_I0 T_00
                x4 = mm16(sA32 + (16 * I) * S68 + 16, S68, sT1t + 0 * 16 * TS, TS, x4, lane);     // A_I1 T_10
            } else {
                x4 = mm16(sA32 + (16 * I) * S68 + 16, S68, sTtD + 1 * 16 * TS, TS, x4, lane);     // A_I1 T_11
            }
            store_colmajor(sXt + wave * 16 * TS, x4, lane);
        }
        __syncthreads();
        if (wave < 4) {
            // T_2J = -T_22 X_2J ; T_3J = -(T_32 X_2J + T_33 X_3J)
            const int I = 2 + (wave >> 1), J = wave & 1;
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
            if (I == 2) {
                t = mm16(sA32 + 32 * S68 + 32, S68, sXt + J * 16 * TS, TS, t, lane);
            } else {
                t = mm16(sA32 + 48 * S68 + 32, S68, sXt + J * 16 * TS, TS, t, lane);
                t = mm16(sA32 + 48 * S68 + 48, S68, sXt + (2 + J) * 16 * TS, TS, t, lane);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = -t[e];
            store_rowmajor(sA32 + (16 * I) * S68 + 16 * J, S68, t, lane);     // A_IJ is no longer read
        }
        __syncthreads();
        // T diag(beta) as the fp16 MFMA operand; row i, columns 8*(tid%8) ...
        {
            const int i = tid >> 3, j0 = 8 * (tid & 7);
            const f32x4 t0 = *reinterpret_cast<const f32x4*>(sA32 + i * S68 + j0);
            const f32x4 t1 = *reinterpret_cast<const f32x4*>(sA32 + i * S68 + j0 + 4);
            const f32x4 b0 = *reinterpret_cast<const f32x4*>(sBeta + j0);
            const f32x4 b1 = *reinterpret_cast<const f32x4*>(sBeta + j0 + 4);
            half8 h;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h[e] = (_Float16)(t0[e] * b0[e]);
                h[4 + e] = (_Float16)(t1[e] * b1[e]);
            }
            *reinterpret_cast<half8*>(smem + L::T16 + (i * S72 + j0) * 2) = h;
            if (TRACE && p.tr_T && s == 0 && i < Lc) {
                float* dst = p.tr_T + ((tok0 + i) * p.Hv + hv) * CH + j0;
#pragma unroll
                for (int e = 0; e < 4; ++e) { dst[e] = t0[e]; dst[4 + e] = t1[e]; }
            }
        }
        __syncthreads();

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
                const int d = dv0 + 32 * tu_dt + (lane & 31);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int i = 32 * tu_it + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                    if (i < Lc) p.tr_U[((tok0 + i) * p.Hv + hv) * DK + d] = uacc[e];
                }
            }
        }
        __syncthreads();

        // ================= a5 (first half): v_new = U - W h =================
        if (wave < NU) {
            f32x16 acc = uacc;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int ko = 16 * kk + 8 * (lane >> 5);
                const half8 a = lds_h8(smem, L::W + ((32 * tu_it + (lane & 31)) * S136 + ko) * 2);
                const half8 b = lds_h8(smem, L::HT + ((32 * tu_dt + (lane & 31)) * S136 + ko) * 2);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
            }
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
        __syncthreads();

        // ================= a6: o^T = h^T (scale q e^G)^T + v_new^T Aqk^T =================
        {
            const int wo = 7 - wave;
            if (wo < NU) {
                const int it = wo / (DV / 32), dt = wo % (DV / 32);
                f32x16 acc;
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[e] = 0.f;
#pragma unroll
                for (int kk = 0; kk < 8; ++kk) {
                    const int ko = 16 * kk + 8 * (lane >> 5);
                    const half8 a = lds_h8(smem, L::HT + ((32 * dt + (lane & 31)) * S136 + ko) * 2);
                    const half8 b = lds_h8(smem, L::Qg + ((32 * it + (lane & 31)) * S136 + ko) * 2);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
                }
                const int kmax = it == 0 ? 2 : 4;
                for (int kk = 0; kk < kmax; ++kk) {
                    const int ko = 16 * kk + 8 * (lane >> 5);
                    const half8 a = lds_h8(smem, L::VnT + ((32 * dt + (lane & 31)) * S72 + ko) * 2);
                    const half8 b = lds_h8(smem, L::Aqk + ((32 * it + (lane & 31)) * S72 + ko) * 2);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
                }
                const int i = 32 * it + (lane & 31);
                if (i < Lc) {
                    uint16_t* dst = p.o + (tok0 + i) * v_tok + (int64_t)hv * DK + dv0 + 32 * dt;
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const int d = 8 * q4 + 4 * (lane >> 5);
                        uint2 w;
                        w.x = (uint32_t)f2bf(acc[4 * q4]) | ((uint32_t)f2bf(acc[4 * q4 + 1]) << 16);
                        w.y = (uint32_t)f2bf(acc[4 * q4 + 2]) | ((uint32_t)f2bf(acc[4 * q4 + 3]) << 16);
                        *reinterpret_cast<uint2*>(dst + d) = w;
                    }
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
                for (int e = 0; e < 16; ++e) {
                    const int c = 32 * ct + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                    hacc[u][e] *= sGam[c];
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
        __syncthreads();
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
        // The next chunk's first LDS writes (sBlk, sBeta, Vt) do not alias HT, and
        // its first barrier orders these stores before any read of HT.
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
    hipLaunchKernelGGL((kda_fwd_kernel<DV, TRACE>), dim3(nblocks), dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_kda_fwd(const KdaParams& p, int dv_slices, bool trace, hipStream_t stream) {
    const int64_t nblocks = (int64_t)p.N * p.Hv * dv_slices;
    if (nblocks == 0) return hipSuccess;
    if (dv_slices == 2) return trace ? launch_dv<64, true>(p, (int)nblocks, stream) : launch_dv<64, false>(p, (int)nblocks, stream);
    return trace ? launch_dv<32, true>(p, (int)nblocks, stream) : launch_dv<32, false>(p, (int)nblocks, stream);
}

}  // namespace kda

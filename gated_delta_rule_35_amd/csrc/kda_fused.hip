// Fused KDA chunked forward for gfx950 (MI355X, CDNA4): every stage of a chunk
// ("cuLA PR #131: SM100/SM103 KDA forward to pure CuTeDSL", Summary: chunk intra,
// FP32 Akk inversion, recompute W/U; "cuLA REPO_LAYOUT.md", ops/: chunk delta-H
// and forward output) in one persistent work-group per (sequence, value head,
// 64-wide dv slice).  The chunk's operands never leave the CU: they are built in
// LDS and consumed from there, so the kernel reads q, k, v, g, beta once and
// writes o and the final state once.
//
// Roles (eight wave64s).  Waves 0..3 (scan waves) each own 16 dv columns of the
// state h (128 keys x 16 columns, fp32) in MFMA accumulators for the whole
// sequence, and walk the chunks in order:
//   a4+a5  Z = v - (k e^{G-A}) (e^A h),  v_new = T diag(beta) Z,
//          h <- e^{G_last-A} (e^A h + (k e^{A-G})^T v_new)
//   a6     o = scale (q e^{G-A}) (e^A h) + Aqk v_new
// A is a per-channel anchor inside the chunk (half the chunk's total log-decay),
// so every decay factor lies within e^{+-D/2} for a chunk decay D.  All products
// are v_mfma_f32_16x16x32_f16; the B operands of the chained products (e^A h,
// Z, v_new) are taken straight from the accumulators of the product before: a
// 16x16 accumulator tile holds rows 4 (lane / 16) + r of column lane % 16, so two
// tiles give a lane the eight rows 16 (s / 4) + 4 (lane / 16) + s % 4 of a
// 32-row k step, and every operand stored in LDS lists its k index in that
// order (position p <-> index 32 (p / 32) + 16 ((p % 8) / 4) + 4 ((p % 32) / 8)
// + p % 4).
// Waves 4..7 (intra waves) build the next chunk while the scan waves walk the
// current one:
//   a1  G = chunk-local inclusive cumsum of g (fp32, in log2 units), the anchor
//       A = G_last / 2 and the operands q e^{G-A}, -(k e^{G-A}), k e^{A-G} (fp16)
//   a2  Aqk = scale (q e^{G-A}) (k e^{A-G})^T, j <= i; Akk = beta_i (k e^{G-A})
//       (k e^{A-G})^T, j < i (MFMA, all eight waves)
//   a3  T = (I + Akk)^{-1} in fp32: diagonal 16x16 blocks by forward
//       substitution, the rest on v_mfma_f32_16x16x4f32
// A chunk whose decay exceeds e^{-16} on some channel (the fp16 factors would
// leave their range) takes an exact path instead: Aqk and Akk element by
// element in fp32 from G, and operands anchored so that every factor is <= 1.
//
// One chunk per period, with work-group barriers: the scan waves walk chunk c
// while the intra waves compute chunk c + 1's elementwise operands in registers;
// then the operands are stored, the intra products and the inversion run, and
// the next period starts.
#include "kda_device.h"

namespace kda {

namespace {

constexpr int FT = 512;                              // eight waves
constexpr float GUARD_LOG2 = 16.0f * LOG2E;          // chunk decay beyond e^-16: exact path
constexpr int S68 = 68;                              // fp32 rows of 64 (+4)
constexpr int TS = 20;                               // fp32 16x16 column-major blocks (+4)

constexpr int RA = 272;                              // bytes per row of 128 halves (+16)
constexpr int RB = 144;                              // bytes per row of 64 halves (+16)

struct FL {
    // Operands of one chunk (fp16).  Rows of 128 halves are 272 bytes apart and
    // rows of 64 halves 144 bytes apart (a 16-byte pad), so the sixteen
    // consecutive rows an MFMA operand read touches start in distinct bank groups.
    static constexpr int QG = 0;                     // [64 token][128 channel] q e^{G-A}
    static constexpr int KG = QG + 64 * RA;          // [64][128] -(k e^{G-A})
    static constexpr int KI = KG + 64 * RA;          // [64][128] k e^{A-G}
    static constexpr int KT = KI + 64 * RA;          // [128 channel][64 token] (k e^{A-G})^T
    static constexpr int AQ = KT + 128 * RB;         // [64 i][64 j] Aqk (scale included)
    static constexpr int TB = AQ + 64 * RB;          // [64 i][64 j] T diag(beta)
    static constexpr int A32 = TB + 64 * RB;         // [64][68] fp32 Akk, then T's blocks
    static constexpr int TtD = A32 + 64 * S68 * 4;   // 4 diagonal T blocks, column-major
    static constexpr int T1t = TtD + 4 * 16 * TS * 4;
    static constexpr int Xt = T1t + 2 * 16 * TS * 4;
    static constexpr int SC = Xt + 4 * 16 * TS * 4;  // per channel: a [128], b [128], d [128] fp32
    static constexpr int BETA = SC + 3 * 128 * 4;    // [64] fp32
    static constexpr int DIAG = BETA + 64 * 4;       // [4][64] fp32: q_i . k_i over each intra wave's channels
    static constexpr int FLAG = DIAG + 4 * 64 * 4;   // two ints (chunk parity)
    static constexpr int BYTES = FLAG + 16;
    // Exact-path staging, over QG .. KT: G^T [128][64] fp32 (log2 units), then
    // q^T and k^T [128][64] bf16.
    static constexpr int SG = 0;
    static constexpr int SQ = 32768;
    static constexpr int SK = 49152;
    static_assert(SK + 16384 <= AQ, "staging");
    static_assert(BYTES <= 160 * 1024, "LDS");
};

// Storage position of index x (channel or token) in the accumulator-row order of
// its 32-wide k step.
__device__ __forceinline__ int pi_pos(int x) {
    return (x & ~31) | (((x & 15) >> 2) << 3) | (((x >> 4) & 1) << 2) | (x & 3);
}

__device__ __forceinline__ int OFA(int row, int pc) { return row * RA + pc * 16; }
__device__ __forceinline__ int OFB(int row, int pc) { return row * RB + pc * 16; }
__device__ __forceinline__ int ELA(int row, int p) { return row * RA + p * 2; }
__device__ __forceinline__ int ELB(int row, int p) { return row * RB + p * 2; }

__device__ __forceinline__ f32x4 mfma16(half8 a, half8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ half8 ld8(const char* smem, int off) { return *reinterpret_cast<const half8*>(smem + off); }

// C += A B for 16x16 fp32 blocks on v_mfma_f32_16x16x4f32 (A row-major with row
// stride sa, B column-major with stride sb); C: lane holds rows 4 (lane / 16) ..
// + 3 of column lane % 16.
__device__ __forceinline__ f32x4 mm16(const float* A, int sa, const float* Bt, int sb, f32x4 c, int lane) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(A + (lane & 15) * sa + 4 * (lane >> 4));
    const f32x4 b = *reinterpret_cast<const f32x4*>(Bt + (lane & 15) * sb + 4 * (lane >> 4));
    f32x4 c1 = {0.f, 0.f, 0.f, 0.f};
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c1, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c1, 0, 0, 0);
    return c + c1;
}
__device__ __forceinline__ void store_colmajor(float* Ct, f32x4 c, int lane) {
    *reinterpret_cast<f32x4*>(Ct + (lane & 15) * TS + 4 * (lane >> 4)) = c;
}
__device__ __forceinline__ void store_rowmajor(float* C, int sc, f32x4 c, int lane) {
#pragma unroll
    for (int e = 0; e < 4; ++e) C[(4 * (lane >> 4) + e) * sc + (lane & 15)] = c[e];
}
// Block (I, J) of T (mm16's layout) times beta of its columns, as fp16 into TB.
__device__ __forceinline__ void store_tb(char* smem, f32x4 t, int I, int J, const float* beta, int lane) {
    const int j = 16 * J + (lane & 15);
    const float bj = beta[j];
    const int pj = pi_pos(j);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        *reinterpret_cast<_Float16*>(smem + FL::TB + ELB(16 * I + 4 * (lane >> 4) + e, pj)) = (_Float16)(t[e] * bj);
}

// A copy of x that the compiler cannot see through: per-lane addresses derived
// from it are recomputed where they are used instead of being hoisted out of the
// chunk loop and kept live (or spilled) across it.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// x from lane (lane ^ m) within each group of 32 lanes (m < 32): ds_swizzle in
// bit-mask mode (and-mask 0x1f, xor-mask m).
template <int M>
__device__ __forceinline__ float xor_lane(float x) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1f | (M << 10)));
}

}  // namespace

template <bool BETA_F32>
__global__ void __launch_bounds__(FT, 1) kda_fused_kernel(const KdaParams p) {
    __shared__ __attribute__((aligned(16))) char smem[FL::BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool is_scan = wave < 4;
    float* const sBeta = reinterpret_cast<float*>(smem + FL::BETA);
    float* const sA32 = reinterpret_cast<float*>(smem + FL::A32);
    // Plain LDS accesses: the barriers' memory clobbers order them.  (A volatile
    // access through a cast pointer would become a flat access, whose completion
    // wait would also wait for every outstanding global load.)
    int* const sFlag = reinterpret_cast<int*>(smem + FL::FLAG);

    // Work-group -> (sequence, value head, slice).  Work-groups are dealt to the 8
    // XCDs round robin; each XCD gets a contiguous run of (sequence, head) pairs
    // with both slices, so the slices of a head and the value heads of a q/k head
    // meet in one L2.
    const int npairs = p.N * p.Hv;
    int pair, sl;
    {
        const int b = (int)blockIdx.x;
        if ((npairs & 7) == 0) {
            const int x = b & 7, loc = b >> 3;
            pair = x * (npairs >> 3) + (loc >> 1);
            sl = loc & 1;
        } else {
            pair = b >> 1;
            sl = b & 1;
        }
    }
    const int n = pair / p.Hv, hv = pair % p.Hv;
    const int hq = hv / (p.Hv / p.Hq);
    int64_t bos, len;
    seq_bounds(p, n, bos, len);
    const int64_t nch = (len + CH - 1) / CH;
    const int64_t v_tok = (int64_t)p.Hv * DK, qk_tok = (int64_t)p.Hq * DK;
    auto rows_of = [&](int64_t c) -> int {
        const int64_t r = len - c * CH;
        return r <= 0 ? 0 : (r >= CH ? CH : (int)r);
    };

    if (tid < 2) sFlag[tid] = 0;
    lds_barrier();   // flags initialised

    // ---- phases that several roles share (each called at the same point of both loops) ----
    // The exact path's products: row i = wave + 8 u of Aqk and Akk, column jj = lane,
    // element by element in fp32 from the staged G^T, q^T, k^T (log2 units).
    auto exact_products = [&]() {
        const float* sG = reinterpret_cast<const float*>(smem + FL::SG);
        const uint16_t* sQ = reinterpret_cast<const uint16_t*>(smem + FL::SQ);
        const uint16_t* sK = reinterpret_cast<const uint16_t*>(smem + FL::SK);
        const int jj = opaque(lane);
        float aq[8], ak[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = wave + 8 * u;
            float sq = 0.f, sk = 0.f;
            if (jj <= i) {
                for (int ch = 0; ch < DK; ++ch) {
                    const float ex = fexp2(sG[ch * 64 + i] - sG[ch * 64 + jj]);
                    const float kj = bf2f(sK[ch * 64 + jj]) * ex;
                    sq = fmaf(bf2f(sQ[ch * 64 + i]), kj, sq);
                    sk = fmaf(bf2f(sK[ch * 64 + i]), kj, sk);
                }
            }
            aq[u] = sq;
            ak[u] = sk;
        }
        lds_barrier();   // (exact path) staging read by everyone
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = wave + 8 * u;
            *reinterpret_cast<_Float16*>(smem + FL::AQ + ELB(i, pi_pos(jj))) = (_Float16)(jj <= i ? p.scale * aq[u] : 0.f);
            sA32[i * S68 + jj] = jj < i ? sBeta[i] * ak[u] : 0.f;
        }
    };
    // Zero 16x16 tiles (0,1) and (2,3) of T diag(beta) (and of Aqk on the fast path):
    // the scan's k steps cover them.
    auto zero_tiles = [&](bool exact) {
        const int t = opaque(tid);
        const int zt = t >> 8, e = t & 255;
        const int row = 32 * zt + (e >> 4), col = 32 * zt + 16 + (e & 15);
        const int o = ELB(row, pi_pos(col));
        *reinterpret_cast<_Float16*>(smem + FL::TB + o) = (_Float16)0.f;
        if (!exact) *reinterpret_cast<_Float16*>(smem + FL::AQ + o) = (_Float16)0.f;
    };
    // Intra products on MFMA: tiles t = wave + 8 u of Aqk^T (t < 10) and Akk^T.
    auto intra_products = [&]() {
        const int ln = opaque(lane);
        const int g = ln >> 4, jj = ln & 15;
        const int ab = jj * RA + g * 16;
        // all operand fragments of this wave's tiles first, then the MFMAs
        half8 fa[3][4], fb[3][4];
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int t = wave + 8 * u;
            if (t < 20) {
                const int m = t / 10, pidx = t % 10;
                const int I = pidx >= 6 ? 3 : (pidx >= 3 ? 2 : (pidx >= 1 ? 1 : 0));
                const int J = pidx - I * (I + 1) / 2;
                const int xb = m == 0 ? FL::QG : FL::KG;
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    fa[u][kk] = ld8(smem, FL::KI + ab + 16 * J * RA + 64 * kk);
                    fb[u][kk] = ld8(smem, xb + ab + 16 * I * RA + 64 * kk);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int t = wave + 8 * u;
            if (t < 20) {
                const int m = t / 10, pidx = t % 10;
                const int I = pidx >= 6 ? 3 : (pidx >= 3 ? 2 : (pidx >= 1 ? 1 : 0));
                const int J = pidx - I * (I + 1) / 2;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) acc = mfma16(fa[u][kk], fb[u][kk], acc);
                // lane: row i = 16 I + jj, columns 16 J + 4 g + r
                const int i = 16 * I + jj, jb = 16 * J + 4 * g;
                if (m == 0) {
                    if (I == J) {
                        // the diagonal q_i . k_i (decay factor exactly one) in fp32 from
                        // the bf16 inputs, not from the rounded fp16 factors
                        const float* dg = reinterpret_cast<const float*>(smem + FL::DIAG);
                        const float di = ((dg[i] + dg[64 + i]) + dg[128 + i]) + dg[192 + i];
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (jb + r == i) acc[r] = di;
                    }
                    half4 h4;
#pragma unroll
                    for (int r = 0; r < 4; ++r) h4[r] = (_Float16)((I == J && jb + r > i) ? 0.f : p.scale * acc[r]);
                    *reinterpret_cast<half4*>(smem + FL::AQ + ELB(i, pi_pos(jb))) = h4;
                } else {
                    const float bi = sBeta[i];
                    f32x4 v4;
#pragma unroll
                    for (int r = 0; r < 4; ++r) v4[r] = (I == J && jb + r >= i) ? 0.f : -(bi * acc[r]);
                    *reinterpret_cast<f32x4*>(sA32 + i * S68 + jb) = v4;
                }
            }
        }
    };
    // T = (I + Akk)^{-1} in fp32 by waves 0..3, T diag(beta) to TB; three barriers.
    auto inversion = [&]() {
        float* sTtD = reinterpret_cast<float*>(smem + FL::TtD);
        float* sT1t = reinterpret_cast<float*>(smem + FL::T1t);
        float* sXt = reinterpret_cast<float*>(smem + FL::Xt);
        const int ln = opaque(lane);
        if (wave < 2) {
            // diagonal blocks (lane: block B, column j; lanes 32..63 repeat 0..31)
            const int B = 2 * wave + ((ln >> 4) & 1), j = ln & 15;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int kk = 0; kk < 15; ++kk) {
#pragma unroll
                for (int i = kk + 1; i < 16; ++i) x[i] -= sA32[(16 * B + i) * S68 + 16 * B + kk] * x[kk];
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (ln < 32) {
                const float bj = sBeta[16 * B + j];
                const int pj = pi_pos(16 * B + j);
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    sA32[(16 * B + i) * S68 + 16 * B + j] = x[i];
                    *reinterpret_cast<_Float16*>(smem + FL::TB + ELB(16 * B + i, pj)) = (_Float16)(x[i] * bj);
                }
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    f32x4 v4 = {x[4 * i4], x[4 * i4 + 1], x[4 * i4 + 2], x[4 * i4 + 3]};
                    *reinterpret_cast<f32x4*>(sTtD + (B * 16 + j) * TS + 4 * i4) = v4;
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            // T_I,I-1 = -T_II (A_I,I-1 T_I-1,I-1), I = 2 wave + 1
            const int I = 2 * wave + 1, J = I - 1;
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
            y = mm16(sA32 + (16 * I) * S68 + 16 * J, S68, sTtD + J * 16 * TS, TS, y, ln);
            store_colmajor(sT1t + wave * 16 * TS, y, ln);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
            t = mm16(sA32 + (16 * I) * S68 + 16 * I, S68, sT1t + wave * 16 * TS, TS, t, ln);
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = -t[e];
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            store_rowmajor(sA32 + (16 * I) * S68 + 16 * J, S68, t, ln);
            store_colmajor(sT1t + wave * 16 * TS, t, ln);
            store_tb(smem, t, I, J, sBeta, ln);
        }
        lds_barrier();
        if (wave < 4) {
            // X_IJ = sum_{K=J}^{1} A_IK T_KJ for I in {2,3}, J in {0,1}
            const int I = 2 + (wave >> 1), J = wave & 1;
            f32x4 x4 = {0.f, 0.f, 0.f, 0.f};
            if (J == 0) {
                x4 = mm16(sA32 + (16 * I) * S68 + 0, S68, sTtD + 0 * 16 * TS, TS, x4, ln);
                x4 = mm16(sA32 + (16 * I) * S68 + 16, S68, sT1t + 0 * 16 * TS, TS, x4, ln);
            } else {
                x4 = mm16(sA32 + (16 * I) * S68 + 16, S68, sTtD + 1 * 16 * TS, TS, x4, ln);
            }
            store_colmajor(sXt + wave * 16 * TS, x4, ln);
        }
        lds_barrier();
        if (wave < 4) {
            // T_2J = -T_22 X_2J ; T_3J = -(T_32 X_2J + T_33 X_3J)
            const int I = 2 + (wave >> 1), J = wave & 1;
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
            if (I == 2) {
                t = mm16(sA32 + 32 * S68 + 32, S68, sXt + J * 16 * TS, TS, t, ln);
            } else {
                t = mm16(sA32 + 48 * S68 + 32, S68, sXt + J * 16 * TS, TS, t, ln);
                t = mm16(sA32 + 48 * S68 + 48, S68, sXt + (2 + J) * 16 * TS, TS, t, ln);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = -t[e];
            store_tb(smem, t, I, J, sBeta, ln);
        }
        lds_barrier();   // chunk's operands, Aqk and T diag(beta) complete
    };
    // Every period after phase A: B1, the exact path's two barriers when taken, B2,
    // B3 and the inversion's three, in the same order on both roles.

    if (is_scan) {
        // ================= scan waves =================
        // Lane (g, jj): state rows 16 kt + 4 g + r (keys) of column dv0 + jj.
        const int dv0 = 64 * sl + 16 * wave;
        f32x4 hacc[8];
        uint16_t vr[16];   // v of the chunk to scan next: token 16 mt + 4 g + r, column dv0 + jj (index 4 mt + r)
        auto load_v = [&](int64_t c) {
            const int ln = opaque(lane);
            const int vb = (int)((4 * (ln >> 4) * v_tok + (ln & 15)) * 2);
            const int Lc = rows_of(c);
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + (bos + c * CH) * v_tok + (int64_t)hv * DK + dv0,
                                                        Lc ? ((Lc - 1) * v_tok + 16) * 2 : 0);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    vr[4 * mt + r] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(
                        rv, vb + (int)((16 * mt + r) * v_tok * 2), 0, 0);
            }
        };
        {
            const int ln = opaque(lane);
#pragma unroll
            for (int kt = 0; kt < 8; ++kt) hacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (p.h0) {
                const float* src = p.h0 + ((int64_t)n * p.Hv + hv) * DK * DK + dv0 + (ln & 15) + 4 * (ln >> 4) * DK;
#pragma unroll
                for (int kt = 0; kt < 8; ++kt) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) hacc[kt][r] = src[(16 * kt + r) * DK];
                }
            }
        }
        for (int64_t c = 0; c <= nch; ++c) {
            if (c > 0) {
                // ---- phase A: chunk c - 1 ----
                const int64_t cs = c - 1;
                const int Lc = rows_of(cs);
                const int64_t tok0 = bos + cs * CH;
                const int ln = opaque(lane);
                const int g = ln >> 4, jj = ln & 15;
                const int qb = jj * RA + g * 16;   // row jj of a 16-row tile, piece g of a k step
                const int tb = jj * RB + g * 16;
                const char* scp = smem + FL::SC + g * 16;
                // h~ = a h (operand), then h <- b h
                half8 hb[4];
#pragma unroll
                for (int kt = 0; kt < 8; ++kt) {
                    const f32x4 a4 = *reinterpret_cast<const f32x4*>(scp + kt * 64);
                    const f32x4 b4 = *reinterpret_cast<const f32x4*>(scp + 512 + kt * 64);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        hb[kt >> 1][4 * (kt & 1) + r] = (_Float16)(a4[r] * hacc[kt][r]);
                        hacc[kt][r] *= b4[r];
                    }
                }
                f32x4 z[4], o[4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) z[mt][r] = bf2f(vr[4 * mt + r]);
                    o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
                // Z = v - (k e^{G-A}) h~ ; o^T = h~^T (q e^{G-A})^T.  The eight
                // fragments of k step kk + 1 are read while the MFMAs of step kk run
                // (scheduling barriers keep that order).
                half8 fa[2][8];
                auto load_kq = [&](int kk, half8 (&f)[8]) {
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        f[mt] = ld8(smem, FL::KG + qb + 16 * mt * RA + 64 * kk);
                        f[4 + mt] = ld8(smem, FL::QG + qb + 16 * mt * RA + 64 * kk);
                    }
                };
                half8 ftb[6];   // T diag(beta): tiles (mt, k step) (0,0) (1,0) (2,0) (3,0) (2,1) (3,1)
                load_kq(0, fa[0]);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    if (kk < 3) {
                        load_kq(kk + 1, fa[(kk + 1) & 1]);
                    } else {
#pragma unroll
                        for (int mt = 0; mt < 4; ++mt) ftb[mt] = ld8(smem, FL::TB + tb + 16 * mt * RB);
                        ftb[4] = ld8(smem, FL::TB + tb + 32 * RB + 64);
                        ftb[5] = ld8(smem, FL::TB + tb + 48 * RB + 64);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        z[mt] = mfma16(fa[kk & 1][mt], hb[kk], z[mt]);
                        o[mt] = mfma16(hb[kk], fa[kk & 1][4 + mt], o[mt]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) o[mt] *= p.scale;
                // k e^{A-G} fragments of key tiles 0..3 (both k steps) while v_new forms
                half8 fkt[2][8];
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    fkt[0][2 * kt] = ld8(smem, FL::KT + tb + 16 * kt * RB);
                    fkt[0][2 * kt + 1] = ld8(smem, FL::KT + tb + 16 * kt * RB + 64);
                }
                // v_new = T diag(beta) Z (T lower triangular: token tiles 0, 1 need k step 0 only)
                half8 zb[2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        zb[kk][r] = (_Float16)z[2 * kk][r];
                        zb[kk][4 + r] = (_Float16)z[2 * kk + 1][r];
                    }
                }
                f32x4 vn[4];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) vn[mt] = mfma16(ftb[mt], zb[0], f32x4{0.f, 0.f, 0.f, 0.f});
                vn[2] = mfma16(ftb[4], zb[1], vn[2]);
                vn[3] = mfma16(ftb[5], zb[1], vn[3]);
                __builtin_amdgcn_sched_barrier(0);
                // key tiles 4..7 and the Aqk fragments while the first state MFMAs run
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    fkt[1][2 * kt] = ld8(smem, FL::KT + tb + 16 * (4 + kt) * RB);
                    fkt[1][2 * kt + 1] = ld8(smem, FL::KT + tb + 16 * (4 + kt) * RB + 64);
                }
                half8 vb[2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        vb[kk][r] = (_Float16)vn[2 * kk][r];
                        vb[kk][4 + r] = (_Float16)vn[2 * kk + 1][r];
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                // h += (k e^{A-G})^T v_new ; o^T += v_new^T Aqk^T
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    hacc[kt] = mfma16(fkt[0][2 * kt], vb[0], hacc[kt]);
                    hacc[kt] = mfma16(fkt[0][2 * kt + 1], vb[1], hacc[kt]);
                }
                half8 faq[6];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) faq[mt] = ld8(smem, FL::AQ + tb + 16 * mt * RB);
                faq[4] = ld8(smem, FL::AQ + tb + 32 * RB + 64);
                faq[5] = ld8(smem, FL::AQ + tb + 48 * RB + 64);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    hacc[4 + kt] = mfma16(fkt[1][2 * kt], vb[0], hacc[4 + kt]);
                    hacc[4 + kt] = mfma16(fkt[1][2 * kt + 1], vb[1], hacc[4 + kt]);
                }
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) o[mt] = mfma16(vb[0], faq[mt], o[mt]);
                o[2] = mfma16(vb[1], faq[4], o[2]);
                o[3] = mfma16(vb[1], faq[5], o[3]);
                // h <- d h
#pragma unroll
                for (int kt = 0; kt < 8; ++kt) hacc[kt] *= *reinterpret_cast<const f32x4*>(scp + 1024 + kt * 64);
                // o tile mt: lane holds dv columns 4 g .. + 3 of token 16 mt + jj
                uint16_t* obase = p.o + tok0 * v_tok + (int64_t)hv * DK + dv0 + 4 * g;
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const int i = 16 * mt + jj;
                    if (i < Lc) {
                        uint2 w;
                        w.x = pack_bf2(o[mt][0], o[mt][1]);
                        w.y = pack_bf2(o[mt][2], o[mt][3]);
                        *reinterpret_cast<uint2*>(obase + i * v_tok) = w;
                    }
                }
            }
            if (c == nch) break;
            lds_barrier();   // B1
            const bool exact = sFlag[c & 1] != 0;
            if (tid == 0) sFlag[(c + 1) & 1] = 0;
            load_v(c);   // v of chunk c, consumed in the next period's phase A
            if (exact) {
                lds_barrier();   // staging complete
                exact_products();
            }
            zero_tiles(exact);
            lds_barrier();   // B2
            if (!exact) intra_products();
            lds_barrier();   // B3
            inversion();
        }
        // ---- final state ----
        if (p.hT) {
            const int ln = opaque(lane);
            float* dst = p.hT + ((int64_t)n * p.Hv + hv) * DK * DK + dv0 + (ln & 15) + 4 * (ln >> 4) * DK;
#pragma unroll
            for (int kt = 0; kt < 8; ++kt) {
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(16 * kt + r) * DK] = hacc[kt][r];
            }
        }
    } else {
        // ================= intra waves =================
        // Lane (o, u) = (lane / 16, lane % 16): channels cc .. cc + 7 (cc = 32 (wave - 4)
        // + 8 o) of rows 4 u .. 4 u + 3.  Every global load is 16 bytes per lane, and the
        // row groups of one channel octet sit in one 16-lane row, so the cumsum's prefix
        // over row groups runs on row-local lane shifts.
        // Kept as the loads' own 16-byte vectors, so each load writes its final
        // registers (a reshuffle would make the compiler wait for the load there).
        i32x4 qraw[4], kraw[4];   // [row t] element d: bf16 pair (channels cc + 2 d, + 1)
        i32x4 graw[4][2];         // [row t][half] element e: g of channel cc + 4 half + e
        uint32_t braw_bits = 0;
        auto load_raw = [&](int64_t c) {
            const int ln = opaque(lane);
            const int row0 = 4 * (ln & 15), cc = 32 * (wave & 3) + 8 * (ln >> 4);
            const int gb = (int)((row0 * v_tok + cc) * 4), qb = (int)((row0 * qk_tok + cc) * 2);
            const int Lc = rows_of(c);
            const int64_t t0 = bos + c * CH;
            const __amdgpu_buffer_rsrc_t rg =
                make_rsrc(p.g + t0 * v_tok + (int64_t)hv * DK, Lc ? ((Lc - 1) * v_tok + DK) * 4 : 0);
            const __amdgpu_buffer_rsrc_t rq =
                make_rsrc(p.q + t0 * qk_tok + (int64_t)hq * DK, Lc ? ((Lc - 1) * qk_tok + DK) * 2 : 0);
            const __amdgpu_buffer_rsrc_t rk =
                make_rsrc(p.k + t0 * qk_tok + (int64_t)hq * DK, Lc ? ((Lc - 1) * qk_tok + DK) * 2 : 0);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                qraw[t] = __builtin_amdgcn_raw_buffer_load_b128(rq, qb + (int)(t * qk_tok * 2), 0, 0);
                kraw[t] = __builtin_amdgcn_raw_buffer_load_b128(rk, qb + (int)(t * qk_tok * 2), 0, 0);
                graw[t][0] = __builtin_amdgcn_raw_buffer_load_b128(rg, gb + (int)(t * v_tok * 4), 0, 0);
                graw[t][1] = __builtin_amdgcn_raw_buffer_load_b128(rg, gb + (int)(t * v_tok * 4) + 16, 0, 0);
            }
            if (wave == 4) {
                // beta of token ln (the dtype is a template parameter: no branch around
                // the load, so no wait for it at a join)
                const int esz = BETA_F32 ? 4 : 2;
                const __amdgpu_buffer_rsrc_t rb = make_rsrc(
                    reinterpret_cast<const char*>(p.beta) + (t0 * p.Hv + hv) * esz, Lc ? ((Lc - 1) * (int64_t)p.Hv + 1) * esz : 0);
                if constexpr (BETA_F32)
                    braw_bits = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rb, ln * p.Hv * 4, 0, 0);
                else
                    braw_bits = (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rb, ln * p.Hv * 2, 0, 0) << 16;
            }
        };
        // Results kept in registers until the store: per row t, the fp16 pairs of
        // channels (cc + 2 d, + 1); per channel, the fp16 pairs of rows (4 u + 2 e, + 1);
        // the chunk total of g per channel (log2 units); q . k of rows 4 u .. 4 u + 3
        // over this wave's 32 channels.
        uint32_t oq[4][4], okg[4][4], oki[4][4], okt[8][2];
        float tot2[8], dsum_rows[4];
        // Local inclusive cumsum of g within the 4 rows (log2 units), the cumsum of the
        // earlier row groups (an inclusive prefix over u, on the lanes of one 16-lane
        // row) and the chunk total (from lane 15 of the row).  Returns whether some
        // channel decays past the fast path's range.
        auto cumsum = [&](float (&sl)[4][8], float (&off2)[8], float (&tot2)[8]) -> int {
            const int ln = opaque(lane);
            int guard = 0;
#pragma unroll
            for (int ch = 0; ch < 8; ++ch) {
                float acc = 0.f;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    acc = fmaf(__int_as_float(graw[t][ch >> 2][ch & 3]), LOG2E, acc);
                    sl[t][ch] = acc;
                }
                float x = acc;
                x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));  // row_shr:1
                x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));  // row_shr:2
                x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));  // row_shr:4
                x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));  // row_shr:8
                off2[ch] = x - acc;
                tot2[ch] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (ln | 15), __float_as_int(x)));
                if (tot2[ch] < -GUARD_LOG2) guard = 1;
            }
            return guard;
        };
        // The operands q e^{G-A}, -(k e^{G-A}) and k e^{A-G} of the 4 x 8 elements, with
        // G = sl + off2 and A = `anchor` (log2 units; per channel).
        auto operands = [&](const float (&sl)[4][8], const float (&off2)[8], const float (&anchor)[8],
                            uint32_t (&oq)[4][4], uint32_t (&okg)[4][4], uint32_t (&oki)[4][4], uint32_t (&okt)[8][2]) {
            // one channel pair at a time (few live temporaries)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                float qe[2][4], ke[2][4], ki[2][4];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int ch = 2 * d + h;
                    const float base = off2[ch] - anchor[ch];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float a = sl[t][ch] + base;
                        const float E = fexp2(a), Ei = fexp2(-a);
                        const uint32_t qw = (uint32_t)qraw[t][d], kw = (uint32_t)kraw[t][d];
                        const float qf = h ? bf_hi(qw) : bf_lo(qw);
                        const float kf = h ? bf_hi(kw) : bf_lo(kw);
                        qe[h][t] = qf * E;
                        ke[h][t] = -(kf * E);
                        ki[h][t] = kf * Ei;
                    }
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    oq[t][d] = pack_h2(qe[0][t], qe[1][t]);
                    okg[t][d] = pack_h2(ke[0][t], ke[1][t]);
                    oki[t][d] = pack_h2(ki[0][t], ki[1][t]);
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    okt[2 * d + h][0] = pack_h2(ki[h][0], ki[h][1]);
                    okt[2 * d + h][1] = pack_h2(ki[h][2], ki[h][3]);
                }
                // keep the scheduler from hoisting the next pair's exponentials (each
                // pair's temporaries die here)
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // The store of a chunk's operands; the per-channel scalars come from tot2:
        // fast path a = b = e^{G_last / 2}, d = e^{G_last - G_last / 2}; exact path
        // a = 1, b = e^{G_last}, d = 1.
        auto store_operands = [&](bool exact, const uint32_t (&oq)[4][4], const uint32_t (&okg)[4][4],
                                  const uint32_t (&oki)[4][4], const uint32_t (&okt)[8][2], const float (&tot2)[8],
                                  const float (&dsum_rows)[4]) {
            const int ln = opaque(lane);
            const int u = ln & 15, cc = 32 * (wave & 3) + 8 * (ln >> 4);
            // channels cc .. cc + 3 and cc + 4 .. cc + 7 are two runs of four positions
            const int ra0 = ELA(4 * u, pi_pos(cc)), ra1 = ELA(4 * u, pi_pos(cc + 4));
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                *reinterpret_cast<uint2*>(smem + FL::QG + ra0 + t * RA) = make_uint2(oq[t][0], oq[t][1]);
                *reinterpret_cast<uint2*>(smem + FL::QG + ra1 + t * RA) = make_uint2(oq[t][2], oq[t][3]);
                *reinterpret_cast<uint2*>(smem + FL::KG + ra0 + t * RA) = make_uint2(okg[t][0], okg[t][1]);
                *reinterpret_cast<uint2*>(smem + FL::KG + ra1 + t * RA) = make_uint2(okg[t][2], okg[t][3]);
                *reinterpret_cast<uint2*>(smem + FL::KI + ra0 + t * RA) = make_uint2(oki[t][0], oki[t][1]);
                *reinterpret_cast<uint2*>(smem + FL::KI + ra1 + t * RA) = make_uint2(oki[t][2], oki[t][3]);
            }
            // rows 4 u .. 4 u + 3 of channel cc + ch: one run of four positions
            const int rt = ELB(cc, pi_pos(4 * u));
#pragma unroll
            for (int ch = 0; ch < 8; ++ch)
                *reinterpret_cast<uint2*>(smem + FL::KT + rt + ch * RB) = make_uint2(okt[ch][0], okt[ch][1]);
            if (u == 0) {
                float sa[8], sb[8], sd[8];
#pragma unroll
                for (int ch = 0; ch < 8; ++ch) {
                    const float h = fexp2(0.5f * tot2[ch]);
                    sa[ch] = exact ? 1.f : h;
                    sb[ch] = exact ? fexp2(tot2[ch]) : h;
                    sd[ch] = exact ? 1.f : fexp2(tot2[ch] - 0.5f * tot2[ch]);
                }
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    *reinterpret_cast<f32x4*>(smem + FL::SC + (cc + 4 * hh) * 4) =
                        f32x4{sa[4 * hh], sa[4 * hh + 1], sa[4 * hh + 2], sa[4 * hh + 3]};
                    *reinterpret_cast<f32x4*>(smem + FL::SC + 512 + (cc + 4 * hh) * 4) =
                        f32x4{sb[4 * hh], sb[4 * hh + 1], sb[4 * hh + 2], sb[4 * hh + 3]};
                    *reinterpret_cast<f32x4*>(smem + FL::SC + 1024 + (cc + 4 * hh) * 4) =
                        f32x4{sd[4 * hh], sd[4 * hh + 1], sd[4 * hh + 2], sd[4 * hh + 3]};
                }
                // the diagonal q_i . k_i partial sums of this wave's channels (lanes with o = 0)
                if ((ln >> 4) == 0)
                    *reinterpret_cast<f32x4*>(smem + FL::DIAG + (64 * (wave & 3) + 4 * u) * 4) =
                        f32x4{dsum_rows[0], dsum_rows[1], dsum_rows[2], dsum_rows[3]};
            }
            if (wave == 4) sBeta[ln] = __uint_as_float(braw_bits);
        };
        if (nch > 0) load_raw(0);
        for (int64_t c = 0; c < nch; ++c) {
            // ---- phase A: elementwise operands of chunk c ----
            {
                const int ln = opaque(lane);
                float sl[4][8], off2[8], anchor[8];
                const int guard = cumsum(sl, off2, tot2);
#pragma unroll
                for (int ch = 0; ch < 8; ++ch) anchor[ch] = 0.5f * tot2[ch];
                operands(sl, off2, anchor, oq, okg, oki, okt);
                // q_r . k_r over this wave's 32 channels for the 4 rows: this lane's 8
                // channels, then the four octets (lanes u, u + 16, u + 32, u + 48)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    float d = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        d = fmaf(bf_lo((uint32_t)qraw[t][e]), bf_lo((uint32_t)kraw[t][e]),
                                 fmaf(bf_hi((uint32_t)qraw[t][e]), bf_hi((uint32_t)kraw[t][e]), d));
                    d += xor_lane<16>(d);
                    d += __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (ln ^ 32), __float_as_int(d)));
                    dsum_rows[t] = d;
                }
                if (guard) sFlag[c & 1] = 1;
                // Materialise the results here, beside the scan of the previous chunk:
                // otherwise the compiler sinks this arithmetic past the barrier into the
                // store below, the only place that reads it.
#pragma unroll
                for (int t = 0; t < 4; ++t) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) asm volatile("" : "+v"(oq[t][d]), "+v"(okg[t][d]), "+v"(oki[t][d]));
                    asm volatile("" : "+v"(dsum_rows[t]));
                }
#pragma unroll
                for (int ch = 0; ch < 8; ++ch) asm volatile("" : "+v"(okt[ch][0]), "+v"(okt[ch][1]), "+v"(tot2[ch]));
            }
            lds_barrier();   // B1
            const bool exact = sFlag[c & 1] != 0;
            if (!exact) {
                store_operands(false, oq, okg, oki, okt, tot2, dsum_rows);
            } else {
                // Exact path (rare: a chunk decaying past e^-16).  The inputs are loaded
                // again, so that the fast path keeps nothing of them across the barrier.
                load_raw(c);
                float sl[4][8], off2[8], zero[8], xt[8];
                cumsum(sl, off2, xt);
                {
                    const int ln = opaque(lane);
                    const int row0 = 4 * (ln & 15), cc = 32 * (wave & 3) + 8 * (ln >> 4);
                    float* sG = reinterpret_cast<float*>(smem + FL::SG);
                    uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + FL::SQ);
                    uint16_t* sK = reinterpret_cast<uint16_t*>(smem + FL::SK);
#pragma unroll
                    for (int ch = 0; ch < 8; ++ch) {
                        *reinterpret_cast<f32x4*>(sG + (cc + ch) * 64 + row0) =
                            f32x4{sl[0][ch] + off2[ch], sl[1][ch] + off2[ch], sl[2][ch] + off2[ch], sl[3][ch] + off2[ch]};
                        uint32_t q4[4], k4[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const uint32_t qw = (uint32_t)qraw[t][ch >> 1], kw = (uint32_t)kraw[t][ch >> 1];
                            q4[t] = (ch & 1) ? qw >> 16 : qw & 0xffffu;
                            k4[t] = (ch & 1) ? kw >> 16 : kw & 0xffffu;
                        }
                        *reinterpret_cast<uint2*>(sQ + (cc + ch) * 64 + row0) = make_uint2(q4[0] | (q4[1] << 16), q4[2] | (q4[3] << 16));
                        *reinterpret_cast<uint2*>(sK + (cc + ch) * 64 + row0) = make_uint2(k4[0] | (k4[1] << 16), k4[2] | (k4[3] << 16));
                    }
                    if (wave == 4) sBeta[ln] = __uint_as_float(braw_bits);
                }
                lds_barrier();   // staging complete
                exact_products();
                // operands anchored at A = 0 (q e^G, -(k e^G)); the transposed copy as
                // k e^{G_last - G} (a = 1, b = e^{G_last}, d = 1): every factor <= 1
                uint32_t xq[4][4], xkg[4][4], xki[4][4], xkt[8][2];
#pragma unroll
                for (int ch = 0; ch < 8; ++ch) zero[ch] = 0.f;
                operands(sl, off2, zero, xq, xkg, xki, xkt);
#pragma unroll
                for (int ch = 0; ch < 8; ++ch) {
#pragma unroll
                    for (int t = 0; t < 4; t += 2) {
                        float r[2];
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const uint32_t kw = (uint32_t)kraw[t + e][ch >> 1];
                            const float kf = (ch & 1) ? bf_hi(kw) : bf_lo(kw);
                            r[e] = kf * fexp2(xt[ch] - (sl[t + e][ch] + off2[ch]));
                        }
                        xkt[ch][t >> 1] = pack_h2(r[0], r[1]);
                    }
                }
                store_operands(true, xq, xkg, xki, xkt, xt, dsum_rows);
            }
            zero_tiles(exact);
            lds_barrier();   // B2
            if (!exact) intra_products();
            lds_barrier();   // B3
            // the next chunk's inputs, issued while waves 0..3 invert (these waves only
            // take the inversion's barriers)
            if (c + 1 < nch) load_raw(c + 1);
            lds_barrier();
            lds_barrier();
            lds_barrier();
        }
    }
}

hipError_t launch_kda_fused(const KdaParams& p, hipStream_t stream) {
    const int64_t nblocks = (int64_t)p.N * p.Hv * 2;
    if (nblocks == 0) return hipSuccess;
    if (nblocks > INT32_MAX) return hipErrorInvalidValue;
    if (p.beta_f32)
        hipLaunchKernelGGL(kda_fused_kernel<true>, dim3((unsigned)nblocks), dim3(FT), 0, stream, p);
    else
        hipLaunchKernelGGL(kda_fused_kernel<false>, dim3((unsigned)nblocks), dim3(FT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace kda

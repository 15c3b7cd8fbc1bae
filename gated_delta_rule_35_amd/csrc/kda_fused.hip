// Fused KDA chunked forward for gfx950 (MI355X, CDNA4): every stage of a chunk
// ("cuLA PR #131: SM100/SM103 KDA forward to pure CuTeDSL", Summary: chunk intra,
// FP32 Akk inversion, recompute W/U; "cuLA REPO_LAYOUT.md", ops/: chunk delta-H
// and forward output) in one persistent work-group per (sequence, value head,
// 64-wide dv slice).  The chunk's operands never leave the CU: they are built in
// LDS and consumed from there, so the kernel reads q, k, v, g, beta once and
// writes o and the final state once.
//
// Two roles of four wave64s each run as a pipeline, one chunk apart.
// Scan waves (0..3) each own 16 dv columns of the state h (128 keys x 16
// columns, fp32) in MFMA accumulators for the whole sequence:
//   S1  Z = v - (k e^{G-A}) (e^A h),  o = scale (q e^{G-A}) (e^A h)
//   S2  v_new = T diag(beta) Z,  h <- e^{G_last-A} (e^A h + (k e^{A-G})^T v_new),
//       o += Aqk v_new
// A is a per-channel anchor inside the chunk (half the chunk's total log-decay),
// so every decay factor lies within e^{+-D/2} for a chunk decay D.  All products
// are v_mfma_f32_16x16x32_f16; the B operands of the chained products (e^A h,
// Z, v_new) are taken straight from the accumulators of the product before: a
// 16x16 accumulator tile holds rows 4 (lane / 16) + r of column lane % 16, so two
// tiles give a lane the eight rows 16 (s / 4) + 4 (lane / 16) + s % 4 of a
// 32-row k step, and every operand stored in LDS lists its k index in that
// order (position p <-> index 32 (p / 32) + 16 ((p % 8) / 4) + 4 ((p % 32) / 8)
// + p % 4).
// Intra waves (4..7) prepare chunk c + 1 while the scan waves walk chunk c:
//   a1  G = chunk-local inclusive cumsum of g (fp32, in log2 units), the anchor
//       A = G_last / 2 and the operands q e^{G-A}, -(k e^{G-A}), k e^{A-G} (fp16)
//   a2  Aqk = scale (q e^{G-A}) (k e^{A-G})^T, j <= i; Akk = beta_i (k e^{G-A})
//       (k e^{A-G})^T, j < i (MFMA)
//   a3  T = (I + Akk)^{-1} in fp32: diagonal 16x16 blocks by forward
//       substitution, the rest on v_mfma_f32_16x16x4f32
// A chunk whose decay exceeds e^{-16} on some channel (the fp16 factors would
// leave their range) takes an exact path instead: Aqk and Akk element by
// element in fp32 from G, and operands anchored so that every factor is <= 1.
//
// Hand-off.  The roles meet through monotonic counters in LDS, not work-group
// barriers: the intra waves write chunk c + 1's q/k operands only after the scan
// waves have read chunk c's (S1), and the scan waves start S1 / S2 of a chunk
// once its operands / its T are complete.  What S2 reads (the transposed k
// operand, Aqk, T diag(beta), the per-channel scalars) has two slots, so the
// intra waves fill chunk c + 1's slot while S2 of chunk c reads the other.  Every
// wait is bounded: past its limit it raises an abort word that releases every
// other wait, so a work-group always drains.
#include <type_traits>

#include "kda_device.h"

namespace kda {

namespace {

constexpr int FT = 512;                              // eight waves
constexpr float GUARD_LOG2 = 16.0f * LOG2E;          // chunk decay beyond e^-16: exact path
constexpr int S68 = 68;                              // fp32 rows of 64 (+4)
constexpr int TS = 20;                               // fp32 16x16 column-major blocks (+4)

constexpr int RA = 256;                              // bytes per row of 128 halves (swizzled, no pad)
constexpr int RB = 144;                              // bytes per row of 64 halves (+16)
constexpr int RK = 128;                              // bytes per row of 64 halves (swizzled, no pad)

struct FL {
    // Operands of one chunk (fp16).  Rows of 128 halves are 256 bytes with the
    // sixteen 16-byte pieces of row r permuted by r ^ (r >> 4) (mod 16): the sixteen
    // consecutive rows an MFMA operand read touches, and the sixteen rows 4 u + t
    // one store instruction touches, each land on sixteen distinct pieces.  Rows of
    // 64 halves are 144 bytes apart (a 16-byte pad).
    static constexpr int QG = 0;                     // [64 token][128 channel] q e^{G-A}
    static constexpr int KG = QG + 64 * RA;          // [64][128] -(k e^{G-A})
    static constexpr int KI = KG + 64 * RA;          // [64][128] k e^{A-G}
    // Two slots each (chunk parity):
    static constexpr int KT_SZ = 128 * RK;
    static constexpr int KT = KI + 64 * RA;          // [128 channel][64 token] (k e^{A-G})^T, swizzled rows
    static constexpr int AB_SZ = 64 * RB;
    static constexpr int AQ = KT + 2 * KT_SZ;        // [64 i][64 j] Aqk (scale included)
    static constexpr int TB = AQ + 2 * AB_SZ;        // [64 i][64 j] T diag(beta)
    // Intra waves only:
    static constexpr int A32 = TB + 2 * AB_SZ;       // [64][68] fp32 Akk, then T's blocks
    static constexpr int TtD = A32 + 64 * S68 * 4;   // 4 diagonal T blocks, column-major
    static constexpr int T1t = TtD + 4 * 16 * TS * 4;   // T_10, column-major
    static constexpr int Xt = T1t + 16 * TS * 4;         // X_21, column-major
    static constexpr int SC_SZ = 3 * 128 * 4;
    static constexpr int SC = Xt + 16 * TS * 4;      // two slots: per channel a [128], b [128], d [128] fp32
    static constexpr int BETA = SC + 2 * SC_SZ;      // two slots: [64] fp32
    static constexpr int DIAG = BETA + 2 * 64 * 4;   // [64 row][4] fp32: q_i . k_i over each intra wave's channels
    static constexpr int VT = DIAG + 4 * 64 * 4;     // [64 dv][64 token] v^T of the chunk (bf16, swizzled rows)
    static constexpr int BYTES = VT + 64 * RK;
    // Exact-path staging: G^T [128][64] fp32 (log2 units) and q^T [128][64] bf16
    // over QG .. KI, k^T [128][64] bf16 over A32.
    static constexpr int SG = 0;
    static constexpr int SQ = 32768;
    static constexpr int SK = A32;
    static_assert(SQ + 16384 <= KT, "staging");
    static_assert(16384 <= 64 * S68 * 4, "staging");
    static_assert(BYTES <= 160 * 1024 - 64, "LDS");
};

// Pipeline counters (LDS, monotonic) and words.
enum : int {
    C_OPS = 0,     // +1 per intra wave when chunk c's operands are stored
    C_S1 = 1,      // +1 per scan wave when S1 of chunk c has read them
    C_T = 2,       // +1 per scan wave when chunk c's T diag(beta) is stored
    C_I = 3,       // intra waves' own rendezvous
    C_G = 4,       // [4], [5]: exact-path word of chunk parity 0, 1
    C_ABORT = 6,   // a wait ran past its limit
    C_P = 7,       // +1 per intra wave when chunk c's Aqk and Akk are stored
    C_V = 8,       // scan waves' own rendezvous (the inversion's levels)
    C_COUNT = 12
};
constexpr int SPIN_LIMIT = 1 << 22;                  // polls (about 0.3 s) before a wait gives up

// Storage position of index x (channel or token) in the accumulator-row order of
// its 32-wide k step.
__device__ __forceinline__ int pi_pos(int x) {
    return (x & ~31) | (((x & 15) >> 2) << 3) | (((x >> 4) & 1) << 2) | (x & 3);
}

__device__ __forceinline__ int OFB(int row, int pc) { return row * RB + pc * 16; }
// Byte offset of position p of row `row` in a swizzled [64][128] operand.
__device__ __forceinline__ int ELA(int row, int p) {
    return row * RA + 16 * ((p >> 3) ^ ((row ^ (row >> 4)) & 15)) + 2 * (p & 7);
}
// Byte offset of position p of row `row` in a swizzled 128-byte-row operand (the
// transposed k copy, v^T): the eight 16-byte pieces of row r are permuted by
// (r / 2) mod 8, so that sixteen consecutive rows read at one piece land on
// sixteen distinct bank groups.
__device__ __forceinline__ int ELK(int row, int p) {
    return row * RK + 16 * ((p >> 3) ^ ((row >> 1) & 7)) + 2 * (p & 7);
}
// Lane's channel octet in the intra waves: lane groups 0..3 (of 16) take octets 0, 2,
// 1, 3, so that a 32-lane half of a store instruction writes disjoint bank halves.
__device__ __forceinline__ int octet(int ln) { return ((ln >> 5) & 1) | (((ln >> 4) & 1) << 1); }
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
// The same in two steps, so that a level's operand reads can all be issued before
// its MFMAs: the operands of one 16x16 block product, then the product.
struct Mm16Ops {
    f32x4 a, b;
};
__device__ __forceinline__ Mm16Ops mm16_ops(const float* A, int sa, const float* Bt, int sb, int lane) {
    return {*reinterpret_cast<const f32x4*>(A + (lane & 15) * sa + 4 * (lane >> 4)),
            *reinterpret_cast<const f32x4*>(Bt + (lane & 15) * sb + 4 * (lane >> 4))};
}
__device__ __forceinline__ f32x4 mm16_mac(const Mm16Ops& o, f32x4 c) {
    f32x4 c1 = {0.f, 0.f, 0.f, 0.f};
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(o.a[0], o.b[0], c, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(o.a[1], o.b[1], c1, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(o.a[2], o.b[2], c, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(o.a[3], o.b[3], c1, 0, 0, 0);
    return c + c1;
}
__device__ __forceinline__ void store_colmajor(float* Ct, f32x4 c, int lane) {
    *reinterpret_cast<f32x4*>(Ct + (lane & 15) * TS + 4 * (lane >> 4)) = c;
}
__device__ __forceinline__ void store_rowmajor(float* C, int sc, f32x4 c, int lane) {
#pragma unroll
    for (int e = 0; e < 4; ++e) C[(4 * (lane >> 4) + e) * sc + (lane & 15)] = c[e];
}
// Block (I, J) of T (mm16's layout) times beta of its columns, as fp16 into the TB slot at tbo.
__device__ __forceinline__ void store_tb(char* smem, int tbo, f32x4 t, int I, int J, const float* beta, int lane) {
    const int j = 16 * J + (lane & 15);
    const float bj = beta[j];
    const int pj = pi_pos(j);
#pragma unroll
    for (int e = 0; e < 4; ++e)
        *reinterpret_cast<_Float16*>(smem + tbo + ELB(16 * I + 4 * (lane >> 4) + e, pj)) = (_Float16)(t[e] * bj);
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
    __shared__ int sync_ctr[C_COUNT];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool is_scan = wave < 4;
    auto beta_slot = [&](int s) { return reinterpret_cast<float*>(smem + FL::BETA + s * 256); };
    float* const sA32 = reinterpret_cast<float*>(smem + FL::A32);

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
    const int nch = (int)((len + CH - 1) / CH);
    const int64_t v_tok = (int64_t)p.Hv * DK, qk_tok = (int64_t)p.Hq * DK;
    auto rows_of = [&](int c) -> int {
        const int64_t r = len - (int64_t)c * CH;
        return r <= 0 ? 0 : (r >= CH ? CH : (int)r);
    };

    if (tid < C_COUNT) sync_ctr[tid] = 0;
    // Tiles (0,1) and (2,3) of Aqk and T diag(beta), both slots: the scan's k steps
    // cover them, and nothing writes them after this (the exact path writes Aqk's
    // zeros itself).
    for (int e = tid; e < 2048; e += FT) {
        const int buf = e >> 9, t = (e >> 8) & 1, x = e & 255;
        const int row = 32 * t + (x >> 4), col = 32 * t + 16 + (x & 15);
        const int base = (buf < 2 ? FL::AQ : FL::TB) + (buf & 1) * FL::AB_SZ;
        *reinterpret_cast<_Float16*>(smem + base + ELB(row, pi_pos(col))) = (_Float16)0.f;
    }
    lds_barrier();   // the only work-group barrier

    // ---- pipeline counters ----
    auto ctr_load = [&](int i) -> int {
        return __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(&sync_ctr[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    };
    // This wave's LDS accesses so far are complete; then count it in.
    auto signal = [&](int i) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (lane == 0) __hip_atomic_fetch_add(&sync_ctr[i], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    auto wait_ge = [&](int i, int target) {
        if (ctr_load(i) < target) {
            int it = 0;
            do {
                __builtin_amdgcn_s_sleep(1);
                if ((++it & 1023) == 0 && (it >= SPIN_LIMIT || ctr_load(C_ABORT) != 0)) {
                    __hip_atomic_store(&sync_ctr[C_ABORT], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    break;
                }
            } while (ctr_load(i) < target);
        }
        asm volatile("" ::: "memory");
    };

    if (is_scan) {
        // ================= scan waves =================
        // Lane (g, jj): state rows 16 kt + 4 g + r (keys) of column dv0 + jj.
        const int dv0 = 64 * sl + 16 * wave;
        f32x4 hacc[8];
        // v of the next chunk: wave w loads tokens 16 w + 2 (lane / 8) + k (k = 0, 1),
        // dv columns 8 (lane % 8) .. + 7 of the slice (eight lanes per token row: a
        // full 128-byte line) and writes them to v^T, where every scan wave reads its
        // columns in accumulator order
        i32x4 vraw[2];
        auto load_vs = [&](int c) {
            const int ln = opaque(lane);
            const int Lc = rows_of(c);
            const int64_t t0 = bos + (int64_t)c * CH;
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + t0 * v_tok + (int64_t)hv * DK + 64 * sl,
                                                        Lc ? ((Lc - 1) * v_tok + 64) * 2 : 0);
            const int vo = (int)(((16 * wave + 2 * (ln >> 3)) * v_tok + 8 * (ln & 7)) * 2);
            vraw[0] = __builtin_amdgcn_raw_buffer_load_b128(rv, vo, 0, 0);
            vraw[1] = __builtin_amdgcn_raw_buffer_load_b128(rv, vo + (int)(v_tok * 2), 0, 0);
        };
        // v^T row 8 (lane % 8) + e, token pair 16 w + 2 (lane / 8): one word each; the
        // row's piece permutation is 4 ((lane % 8) mod 2) + e / 2
        auto store_vt = [&]() {
            const int ln = opaque(lane);
            const int tv = 16 * wave + 2 * (ln >> 3);
            const int vb = FL::VT + 8 * (ln & 7) * RK + 2 * (tv & 7), vp = (tv >> 3) ^ (4 * (ln & 1));
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t x = (uint32_t)vraw[0][d], y = (uint32_t)vraw[1][d];
                const int o = vb + 16 * (vp ^ d);
                *reinterpret_cast<uint32_t*>(smem + o + 2 * d * RK) = (x & 0xffffu) | (y << 16);
                *reinterpret_cast<uint32_t*>(smem + o + (2 * d + 1) * RK) = (x >> 16) | (y & 0xffff0000u);
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
        // a3: T = (I + Akk)^{-1} in fp32 by the four scan waves, T diag(beta) into slot
        // s of TB.  Level 0: wave w inverts diagonal block w by forward substitution
        // (lane j % 16: column j).  Then, on v_mfma_f32_16x16x4f32, with X_IJ =
        // sum_{K=J}^{1} A_IK T_KJ:
        //   level 1  w0: T_10 = -T_11 (A_10 T_00)   w1: T_32 = -T_33 (A_32 T_22)
        //            w2: X_21 = A_21 T_11            w3: X_31 = A_31 T_11
        //   level 2  w0: X_20, T_20 = -T_22 X_20
        //            w1: X_20, X_30, T_30 = -(T_32 X_20 + T_33 X_30)
        //            w2: T_21 = -T_22 X_21           w3: T_31 = -(T_32 X_21 + T_33 X_31)
        // with a scan-wave rendezvous between levels (waves 0 and 1 each form X_20,
        // so the block row 3 needs no third level).  A product's accumulators serve as
        // the next product's B operand in registers; only T_10, T_32 and X_21, which
        // other waves read, go through LDS.
        int tv = 0;   // running target of the scan waves' rendezvous counter
        auto vsync = [&]() {
            signal(C_V);
            tv += 4;
            wait_ge(C_V, tv);
        };
        auto inversion = [&](int s) {
            float* sTtD = reinterpret_cast<float*>(smem + FL::TtD);
            const int tbo = FL::TB + s * FL::AB_SZ;
            const float* sb = beta_slot(s);
            const int ln = opaque(lane);
            auto A = [&](int I, int J) { return sA32 + (16 * I) * S68 + 16 * J; };   // row-major block
            {
                // level 0: block B = wave; lanes 16 .. 63 repeat lanes 0 .. 15
                const int B = wave, j = ln & 15;
                const float* arow = A(B, B);
                f32x4 a4[16][4];
#pragma unroll
                for (int i = 1; i < 16; ++i) {
#pragma unroll
                    for (int q = 0; 4 * q < i; ++q) a4[i][q] = *reinterpret_cast<const f32x4*>(arow + i * S68 + 4 * q);
                }
                float x[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
                // column kk eliminated from every later row at once (each x[i] still
                // accumulates in kk order)
#pragma unroll
                for (int kk = 0; kk < 15; ++kk) {
#pragma unroll
                    for (int i = kk + 1; i < 16; ++i) x[i] = fmaf(-a4[i][kk >> 2][kk & 3], x[kk], x[i]);
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the block's reads before its overwrite
                if (ln < 16) {
                    const float bj = sb[16 * B + j];
                    const int pj = pi_pos(16 * B + j);
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        sA32[(16 * B + i) * S68 + 16 * B + j] = x[i];   // row-major, over A_BB
                        *reinterpret_cast<_Float16*>(smem + tbo + ELB(16 * B + i, pj)) = (_Float16)(x[i] * bj);
                    }
#pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4)   // column-major
                        *reinterpret_cast<f32x4*>(sTtD + (B * 16 + j) * TS + 4 * i4) =
                            f32x4{x[4 * i4], x[4 * i4 + 1], x[4 * i4 + 2], x[4 * i4 + 3]};
                }
            }
            vsync();
        };
        auto inversion_rest = [&](int s) {
            float* sTtD = reinterpret_cast<float*>(smem + FL::TtD);
            float* sT1t = reinterpret_cast<float*>(smem + FL::T1t);
            float* sXt = reinterpret_cast<float*>(smem + FL::Xt);
            const int tbo = FL::TB + s * FL::AB_SZ;
            const float* sb = beta_slot(s);
            const int ln = opaque(lane);
            const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
            auto neg = [](f32x4 v) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = -v[e];
                return v;
            };
            auto A = [&](int I, int J) { return sA32 + (16 * I) * S68 + 16 * J; };   // row-major block
            // This lane's A operand rows of block (I, J) of A32 (row-major).
            auto arow = [&](int I, int J) {
                return *reinterpret_cast<const f32x4*>(A(I, J) + (ln & 15) * S68 + 4 * (ln >> 4));
            };
            // A product's accumulators as the B operand of the next product: mm16's B
            // operand of lane (g, j) is rows 4 g .. 4 g + 3 of column j, exactly the rows
            // the lane's accumulator registers hold, so a block stays in registers
            // unless another wave reads it.
            auto chained = [](f32x4 a, f32x4 b) { return Mm16Ops{a, b}; };
            f32x4 x31 = z4;   // wave 3's X_31, kept for the second level
            if (wave < 2) {
                // T_I,I-1 = -T_II (A_I,I-1 T_I-1,I-1), I = 1 (wave 0), 3 (wave 1)
                const int I = 2 * wave + 1;
                const f32x4 tii = arow(I, I);   // T_II, row-major over A_II
                const f32x4 x = mm16_mac(mm16_ops(A(I, I - 1), S68, sTtD + (I - 1) * 16 * TS, TS, ln), z4);
                const f32x4 t = neg(mm16_mac(chained(tii, x), z4));
                if (wave == 0)
                    store_colmajor(sT1t, t, ln);               // T_10, column-major
                else
                    store_rowmajor(A(3, 2), S68, t, ln);       // T_32 over A_32, row-major
                store_tb(smem, tbo, t, I, I - 1, sb, ln);
            } else {
                // X_21 (wave 2; waves 2 and 3 read it), X_31 (wave 3) = A_I1 T_11
                const f32x4 x = mm16_mac(mm16_ops(A(wave, 1), S68, sTtD + 16 * TS, TS, ln), z4);
                if (wave == 2)
                    store_colmajor(sXt, x, ln);
                else
                    x31 = x;
            }
            vsync();
            // the second level; X_20 is formed by both waves that need it
            if (wave < 2) {
                // X_20 = A_20 T_00 + A_21 T_10
                const Mm16Ops a = mm16_ops(A(2, 0), S68, sTtD, TS, ln);
                const Mm16Ops b = mm16_ops(A(2, 1), S68, sT1t, TS, ln);
                if (wave == 0) {
                    // T_20 = -T_22 X_20
                    const f32x4 t22 = arow(2, 2);
                    const f32x4 x20 = mm16_mac(b, mm16_mac(a, z4));
                    store_tb(smem, tbo, neg(mm16_mac(chained(t22, x20), z4)), 2, 0, sb, ln);
                } else {
                    // X_30 = A_30 T_00 + A_31 T_10 ; T_30 = -(T_32 X_20 + T_33 X_30)
                    const Mm16Ops a3 = mm16_ops(A(3, 0), S68, sTtD, TS, ln);
                    const Mm16Ops b3 = mm16_ops(A(3, 1), S68, sT1t, TS, ln);
                    const f32x4 t32 = arow(3, 2), t33 = arow(3, 3);
                    const f32x4 x20 = mm16_mac(b, mm16_mac(a, z4));
                    const f32x4 x30 = mm16_mac(b3, mm16_mac(a3, z4));
                    store_tb(smem, tbo, neg(mm16_mac(chained(t33, x30), mm16_mac(chained(t32, x20), z4))), 3, 0, sb,
                             ln);
                }
            } else if (wave == 2) {
                // T_21 = -T_22 X_21
                store_tb(smem, tbo, neg(mm16_mac(mm16_ops(A(2, 2), S68, sXt, TS, ln), z4)), 2, 1, sb, ln);
            } else {
                // T_31 = -(T_32 X_21 + T_33 X_31)
                const Mm16Ops a = mm16_ops(A(3, 2), S68, sXt, TS, ln);
                const f32x4 t33 = arow(3, 3);
                store_tb(smem, tbo, neg(mm16_mac(chained(t33, x31), mm16_mac(a, z4))), 3, 1, sb, ln);
            }
        };
        if (nch > 0) {
            load_vs(0);
            store_vt();
            vsync();
        }
        for (int c = 0; c < nch; ++c) {
            const int s = c & 1;
            const int Lc = rows_of(c);
            const int64_t tok0 = bos + (int64_t)c * CH;
            const int ln = opaque(lane);
            const int g = ln >> 4, jj = ln & 15;
            // row jj of a 16-row tile, piece g of a k step: piece (g + 4 kk) of row
            // 16 mt + jj sits at piece (g ^ jj) ^ (4 kk ^ mt)
            const int qa0 = jj * RA + 16 * (g ^ jj);
            const int tb = jj * RB + g * 16;
            // the transposed k copy: piece (g + 4 h) of row 16 kt + jj sits at piece
            // (g + 4 h) ^ ((jj / 2) mod 8)
            const int kb0 = jj * RK + 16 * (g ^ ((jj >> 1) & 7)), kb1 = jj * RK + 16 * ((g | 4) ^ ((jj >> 1) & 7));
            const char* scp = smem + FL::SC + s * FL::SC_SZ + g * 16;
            const int kto = FL::KT + s * FL::KT_SZ, aqo = FL::AQ + s * FL::AB_SZ, tbo = FL::TB + s * FL::AB_SZ;
            wait_ge(C_OPS, 4 * (c + 1));
            if (c > 0) vsync();   // every scan wave's part of this chunk's v^T is in
            // ---- S1 ----
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
            // v of the chunk from v^T: tokens 16 mt + 4 g .. + 3 of column 16 wave + jj
            f32x4 z[4], o[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const uint2 w = *reinterpret_cast<const uint2*>(smem + FL::VT + ELK(16 * wave + jj, 16 * mt + 4 * g));
                z[mt] = f32x4{bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y)};
                o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            // Z = v - (k e^{G-A}) h~ ; o^T = h~^T (q e^{G-A})^T.  The eight fragments
            // of k step kk + 1 are read while the MFMAs of step kk run (scheduling
            // barriers keep that order).
            half8 fa[2][8];
            auto load_kq = [&](int kk, half8 (&f)[8]) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    const int o = (qa0 ^ (16 * (4 * kk ^ mt))) + 16 * mt * RA;
                    f[mt] = ld8(smem, FL::KG + o);
                    f[4 + mt] = ld8(smem, FL::QG + o);
                }
            };
            load_kq(0, fa[0]);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk < 3) load_kq(kk + 1, fa[(kk + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    z[mt] = mfma16(fa[kk & 1][mt], hb[kk], z[mt]);
                    o[mt] = mfma16(hb[kk], fa[kk & 1][4 + mt], o[mt]);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            signal(C_S1);   // q/k operands of chunk c read: the intra waves may overwrite them

#pragma unroll
            for (int mt = 0; mt < 4; ++mt) o[mt] *= p.scale;
            half8 zb[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    zb[kk][r] = (_Float16)z[2 * kk][r];
                    zb[kk][4 + r] = (_Float16)z[2 * kk + 1][r];
                }
            }
            wait_ge(C_P, 4 * (c + 1));
            inversion(s);
            // v of the next chunk: issued here, where the inversion's largest register
            // set is dead; written to v^T at the end of S2 and read in the next S1
            load_vs(c + 1);   // (past the last chunk: a zero-length range)
            inversion_rest(s);
            signal(C_T);
            wait_ge(C_T, 4 * (c + 1));
            // ---- S2 ----
            // T diag(beta): tiles (mt, k step) (0,0) (1,0) (2,0) (3,0) (2,1) (3,1)
            half8 ftb[6];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) ftb[mt] = ld8(smem, tbo + tb + 16 * mt * RB);
            ftb[4] = ld8(smem, tbo + tb + 32 * RB + 64);
            ftb[5] = ld8(smem, tbo + tb + 48 * RB + 64);
            // k e^{A-G} fragments of key tiles 0..3 (both k steps) while v_new forms
            half8 fkt[2][8];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                fkt[0][2 * kt] = ld8(smem, kto + kb0 + 16 * kt * RK);
                fkt[0][2 * kt + 1] = ld8(smem, kto + kb1 + 16 * kt * RK);
            }
            __builtin_amdgcn_sched_barrier(0);
            // v_new = T diag(beta) Z (T lower triangular: token tiles 0, 1 need k step 0 only)
            f32x4 vn[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) vn[mt] = mfma16(ftb[mt], zb[0], f32x4{0.f, 0.f, 0.f, 0.f});
            vn[2] = mfma16(ftb[4], zb[1], vn[2]);
            vn[3] = mfma16(ftb[5], zb[1], vn[3]);
            __builtin_amdgcn_sched_barrier(0);
            // key tiles 4..7 and the Aqk fragments while the first state MFMAs run
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                fkt[1][2 * kt] = ld8(smem, kto + kb0 + 16 * (4 + kt) * RK);
                fkt[1][2 * kt + 1] = ld8(smem, kto + kb1 + 16 * (4 + kt) * RK);
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
            for (int mt = 0; mt < 4; ++mt) faq[mt] = ld8(smem, aqo + tb + 16 * mt * RB);
            faq[4] = ld8(smem, aqo + tb + 32 * RB + 64);
            faq[5] = ld8(smem, aqo + tb + 48 * RB + 64);
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
            // v^T of the next chunk (every scan wave has read this chunk's: they are all
            // past the inversion's rendezvous)
            store_vt();
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
        return;
    }

    // ================= intra waves =================
    const int wi = wave - 4;
    int ti = 0;   // running target of the intra rendezvous counter
    auto isync = [&]() {
        signal(C_I);
        ti += 4;
        wait_ge(C_I, ti);
    };
    // Lane (o, u) = (octet(lane), lane % 16): channels cc .. cc + 7 (cc = 32 wi + 8 o)
    // of rows 4 u .. 4 u + 3.  Every global load is 16 bytes per lane, and the row
    // groups of one channel octet sit in one 16-lane row, so the cumsum's prefix
    // over row groups runs on row-local lane shifts.
    // Kept as the loads' own 16-byte vectors, so each load writes its final
    // registers (a reshuffle would make the compiler wait for the load there).
    i32x4 qraw[4], kraw[4];   // [row t] element d: bf16 pair (channels cc + 2 d, + 1)
    i32x4 graw[4][2];         // [row t][half] element e: g of channel cc + 4 half + e
    uint32_t braw_bits = 0;
    auto load_into = [&](int c, i32x4 (&q)[4], i32x4 (&k)[4], i32x4 (&gg)[4][2], uint32_t& bb, int part = 3) {
        const int ln = opaque(lane);
        const int row0 = 4 * (ln & 15), cc = 32 * wi + 8 * octet(ln);
        const int gb = (int)((row0 * v_tok + cc) * 4), qb = (int)((row0 * qk_tok + cc) * 2);
        const int Lc = rows_of(c);
        const int64_t t0 = bos + (int64_t)c * CH;
        const __amdgpu_buffer_rsrc_t rg =
            make_rsrc(p.g + t0 * v_tok + (int64_t)hv * DK, Lc ? ((Lc - 1) * v_tok + DK) * 4 : 0);
        const __amdgpu_buffer_rsrc_t rq =
            make_rsrc(p.q + t0 * qk_tok + (int64_t)hq * DK, Lc ? ((Lc - 1) * qk_tok + DK) * 2 : 0);
        const __amdgpu_buffer_rsrc_t rk =
            make_rsrc(p.k + t0 * qk_tok + (int64_t)hq * DK, Lc ? ((Lc - 1) * qk_tok + DK) * 2 : 0);
        if (part & 1) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                q[t] = __builtin_amdgcn_raw_buffer_load_b128(rq, qb + (int)(t * qk_tok * 2), 0, 0);
                k[t] = __builtin_amdgcn_raw_buffer_load_b128(rk, qb + (int)(t * qk_tok * 2), 0, 0);
            }
        }
        if (part & 2) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                gg[t][0] = __builtin_amdgcn_raw_buffer_load_b128(rg, gb + (int)(t * v_tok * 4), 0, 0);
                gg[t][1] = __builtin_amdgcn_raw_buffer_load_b128(rg, gb + (int)(t * v_tok * 4) + 16, 0, 0);
            }
        }
        if (wi == 0 && (part & 2)) {
            // beta of token ln (the dtype is a template parameter: no branch around
            // the load, so no wait for it at a join; a bf16 value is kept as loaded
            // and widened to fp32 where it is stored, so nothing here waits for it)
            const int esz = BETA_F32 ? 4 : 2;
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(
                reinterpret_cast<const char*>(p.beta) + (t0 * p.Hv + hv) * esz, Lc ? ((Lc - 1) * (int64_t)p.Hv + 1) * esz : 0);
            if constexpr (BETA_F32)
                bb = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rb, ln * p.Hv * 4, 0, 0);
            else
                bb = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rb, ln * p.Hv * 2, 0, 0);
        }
    };
    // Chunk c's inputs (past the last chunk: a zero-length range, so no access and
    // zeros; issuing it anyway keeps the load out of a branch, whose join would
    // make the compiler wait for it).  part: 1 = q and k, 2 = g and beta, 3 = both;
    // the intra loop issues the two halves apart, q and k only once the current
    // chunk's q and k operands are out of their registers.
    auto load_raw = [&](int c, int part = 3) { load_into(c, qraw, kraw, graw, braw_bits, part); };
    // Local inclusive cumsum of g within the 4 rows (log2 units), the cumsum of the
    // earlier row groups (an inclusive prefix over u, on the lanes of one 16-lane
    // row) and the chunk total (from lane 15 of the row).  Returns whether some
    // channel decays past the fast path's range.
    auto cumsum = [&](const i32x4 (&gg)[4][2], float (&sl)[4][8], float (&off2)[8], float (&tot2)[8]) -> int {
        const int ln = opaque(lane);
        int guard = 0;
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) {
            float acc = 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                acc = fmaf(__int_as_float(gg[t][ch >> 2][ch & 3]), LOG2E, acc);
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
        // fp32 products a0 b0, a1 b1 rounded to the low and high fp16 halves of a word;
        // `neg` negates both
        auto mul_h2 = [](float a0, float b0, float a1, float b1, bool neg) -> uint32_t {
            typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
            const float s0 = neg ? -a0 : a0, s1 = neg ? -a1 : a1;
            const h2_t r = {(_Float16)(s0 * b0), (_Float16)(s1 * b1)};
            return __builtin_bit_cast(uint32_t, r);
        };
        // one channel pair at a time (few live temporaries)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            float E[2][4], Ei[2][4];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int ch = 2 * d + h;
                const float base = off2[ch] - anchor[ch];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float a = sl[t][ch] + base;
                    E[h][t] = fexp2(a);
                    Ei[h][t] = fexp2(-a);
                }
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t qw = (uint32_t)qraw[t][d], kw = (uint32_t)kraw[t][d];
                const float q0 = bf_lo(qw), q1 = bf_hi(qw), k0 = bf_lo(kw), k1 = bf_hi(kw);
                oq[t][d] = mul_h2(q0, E[0][t], q1, E[1][t], false);
                okg[t][d] = mul_h2(k0, E[0][t], k1, E[1][t], true);
                oki[t][d] = mul_h2(k0, Ei[0][t], k1, Ei[1][t], false);
            }
            // the transposed copy: the same halves regrouped by row pairs
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
                const uint32_t x = oki[2 * tp][d], y = oki[2 * tp + 1][d];
                okt[2 * d][tp] = (x & 0xffffu) | (y << 16);
                okt[2 * d + 1][tp] = (x >> 16) | (y & 0xffff0000u);
            }
            // keep the scheduler from hoisting the next pair's exponentials (each
            // pair's temporaries die here)
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Stores of a chunk's operands.  Rows 4 u .. 4 u + 3 of channels cc .. cc + 7
    // (two runs of four positions) into a [64][128] operand at `base`:
    // The lane's store offsets do not change from chunk to chunk: computed once and
    // kept in registers.
    int st_off[4][2], kt_off[4];
    {
        const int ln = lane;
        const int u = ln & 15, cc = 32 * wi + 8 * octet(ln);
        const int p0 = pi_pos(cc), p1 = pi_pos(cc + 4);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            st_off[t][0] = opaque(ELA(4 * u + t, p0));
            st_off[t][1] = opaque(ELA(4 * u + t, p1));
        }
        // the transposed copy: row cc + ch, position pi_pos(4 u), piece permuted by
        // ((cc + ch) / 2) mod 8 = 4 (octet mod 2) + ch / 2
        const int pk = pi_pos(4 * u);
#pragma unroll
        for (int m = 0; m < 4; ++m)
            kt_off[m] = opaque(FL::KT + cc * RK + 16 * ((pk >> 3) ^ (4 * (octet(ln) & 1)) ^ m) + 2 * (pk & 7));
    }
    auto store_rows = [&](int base, const uint32_t (&x)[4][4]) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            *reinterpret_cast<uint2*>(smem + base + st_off[t][0]) = make_uint2(x[t][0], x[t][1]);
            *reinterpret_cast<uint2*>(smem + base + st_off[t][1]) = make_uint2(x[t][2], x[t][3]);
        }
    };
    // ... the transposed copy into slot s (rows 4 u .. 4 u + 3 of channel cc + ch: one
    // run of four positions) ...
    auto store_kt = [&](int s, const uint32_t (&x)[8][2]) {
#pragma unroll
        for (int ch = 0; ch < 8; ++ch)
            *reinterpret_cast<uint2*>(smem + kt_off[ch >> 1] + s * FL::KT_SZ + ch * RK) = make_uint2(x[ch][0], x[ch][1]);
    };

    // ... and, on the fast path, the per-channel scalars a = b = e^{G_last / 2},
    // d = e^{G_last - G_last / 2} into slot s, the diagonal q_i . k_i partial sums
    // and beta.
    auto store_scalars = [&](int s, const float (&tot2)[8], const float (&dsum_rows)[4], uint32_t beta_bits) {
        const int ln = opaque(lane);
        const int u = ln & 15, cc = 32 * wi + 8 * octet(ln);
        if (u == 0) {
            float sa[8], sd[8];
#pragma unroll
            for (int ch = 0; ch < 8; ++ch) {
                sa[ch] = fexp2(0.5f * tot2[ch]);
                sd[ch] = sa[ch];   // e^{G_last - A} = e^A: tot2 - tot2 / 2 is tot2 / 2 exactly
            }
            char* scs = smem + FL::SC + s * FL::SC_SZ;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const f32x4 a4 = {sa[4 * hh], sa[4 * hh + 1], sa[4 * hh + 2], sa[4 * hh + 3]};
                *reinterpret_cast<f32x4*>(scs + (cc + 4 * hh) * 4) = a4;
                *reinterpret_cast<f32x4*>(scs + 512 + (cc + 4 * hh) * 4) = a4;
                *reinterpret_cast<f32x4*>(scs + 1024 + (cc + 4 * hh) * 4) =
                    f32x4{sd[4 * hh], sd[4 * hh + 1], sd[4 * hh + 2], sd[4 * hh + 3]};
            }
        }
        // lanes with o = 0 hold the sums over the wave's 32 channels
        if ((ln >> 4) == 0) {
            float* dg = reinterpret_cast<float*>(smem + FL::DIAG) + 16 * u + wi;
#pragma unroll
            for (int t = 0; t < 4; ++t) dg[4 * t] = dsum_rows[t];
        }
        if (wi == 0) beta_slot(s)[ln] = __uint_as_float(BETA_F32 ? beta_bits : beta_bits << 16);
    };
    // Intra products on MFMA: the ten lower-triangular 16x16 tiles of Aqk^T and of
    // Akk^T, five per wave: Aqk and Akk tile wi, Aqk and Akk tile wi + 4 (each pair
    // back to back, sharing its k e^{A-G} fragments), then Aqk tile wi + 8 (waves 0,
    // 1) or Akk tile wi + 6 (waves 2, 3); tile t is block (I, J) of the lower
    // triangle in row order.  Instantiated per wave, so tile
    // indices and masks are compile-time.  A tile's row scalar is read before the
    // next tile's fragments, so the epilogue waits only for its own data; the next
    // tile's fragments are read while this tile's MFMAs run.
    auto intra_products = [&](auto wi_c, int s) {
        constexpr int WI = decltype(wi_c)::value;
        auto tile_m = [](int k) { return k < 4 ? (k & 1) : (WI < 2 ? 0 : 1); };
        auto tile_t = [](int k) { return k < 4 ? WI + 4 * (k >> 1) : (WI < 2 ? WI + 8 : WI + 6); };
        auto tile_I = [](int t) { return t >= 6 ? 3 : (t >= 3 ? 2 : (t >= 1 ? 1 : 0)); };
        auto tile_J = [&](int t) { const int I = tile_I(t); return t - I * (I + 1) / 2; };
        const int ln = opaque(lane);
        const int g = ln >> 4, jj = ln & 15;
        const int a0 = jj * RA + 16 * (g ^ jj);   // piece (g + 4 kk) of row 16 T + jj: (g ^ jj) ^ (4 kk ^ T)
        const float* sb = beta_slot(s);
        half8 fa[2][4], fb[2][4];
        auto load_tile = [&](int k, half8 (&a)[4], half8 (&b)[4], const half8 (&prev_a)[4]) {
            const int t = tile_t(k), I = tile_I(t), J = tile_J(t);
            const int xb = tile_m(k) == 0 ? FL::QG : FL::KG;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                a[kk] = (k & 1) && k < 4 ? prev_a[kk] : ld8(smem, FL::KI + (a0 ^ (16 * (4 * kk ^ J))) + 16 * J * RA);
                b[kk] = ld8(smem, xb + (a0 ^ (16 * (4 * kk ^ I))) + 16 * I * RA);
            }
        };
        load_tile(0, fa[0], fb[0], fa[1]);
#pragma unroll
        for (int k = 0; k < 5; ++k) {
            const int m = tile_m(k), t = tile_t(k), I = tile_I(t), J = tile_J(t);
            const bool diag = I == J;
            const int i = 16 * I + jj, jb = 16 * J + 4 * g;
            // row scalar: the exact diagonal q_i . k_i (fp32, from the bf16 inputs) for a
            // diagonal Aqk tile, beta_i for Akk
            float rs = 0.f;
            if (m == 0 && diag) {
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(smem + FL::DIAG + 16 * i);
                rs = ((d4[0] + d4[1]) + d4[2]) + d4[3];
            } else if (m == 1) {
                rs = sb[i];
            }
            if (k < 4) load_tile(k + 1, fa[(k + 1) & 1], fb[(k + 1) & 1], fa[k & 1]);
            __builtin_amdgcn_sched_barrier(0);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = mfma16(fa[k & 1][kk], fb[k & 1][kk], acc);
            // lane: row i, columns jb .. jb + 3
            if (m == 0) {
                half4 h4;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = p.scale * acc[r];
                    if (diag) {
                        const int j = jb + r;
                        v = j > i ? 0.f : (j == i ? p.scale * rs : v);
                    }
                    h4[r] = (_Float16)v;
                }
                *reinterpret_cast<half4*>(smem + FL::AQ + s * FL::AB_SZ + ELB(i, pi_pos(jb))) = h4;
            } else {
                f32x4 v4;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    v4[r] = -(rs * acc[r]);
                    if (diag && jb + r >= i) v4[r] = 0.f;
                }
                *reinterpret_cast<f32x4*>(sA32 + i * S68 + jb) = v4;
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (nch > 0) load_raw(0);
    for (int c = 0; c < nch; ++c) {
        const int s = c & 1;
        // ---- a1: elementwise operands of chunk c, in registers ----
        uint32_t oq[4][4], okg[4][4], oki[4][4], okt[8][2];
        float tot2[8], dsum_rows[4];
        {
            const int ln = opaque(lane);
            float sl[4][8], off2[8], anchor[8];
            const int guard = cumsum(graw, sl, off2, tot2);
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
            if (guard) sync_ctr[C_G + s] = 1;
            // Materialise the results here: otherwise the compiler sinks this
            // arithmetic past the rendezvous into the stores, the only readers.
#pragma unroll
            for (int t = 0; t < 4; ++t) {
#pragma unroll
                for (int d = 0; d < 4; ++d) asm volatile("" : "+v"(oq[t][d]), "+v"(okg[t][d]), "+v"(oki[t][d]));
                asm volatile("" : "+v"(dsum_rows[t]));
            }
#pragma unroll
            for (int ch = 0; ch < 8; ++ch) asm volatile("" : "+v"(okt[ch][0]), "+v"(okt[ch][1]), "+v"(tot2[ch]));
        }
        isync();   // every intra wave's guard is in
        const bool exact = ctr_load(C_G + s) != 0;
        if (wi == 0) sync_ctr[C_G + (s ^ 1)] = 0;   // the next chunk's word (its readers are past the rendezvous)
        const uint32_t beta_bits = braw_bits;
        load_raw(c + 1, 2);   // the next chunk's g and beta, in flight until its a1
        wait_ge(C_S1, 4 * c);   // the scan waves are done with chunk c - 1's q/k operands
        // The fast path's operands are stored either way (the exact path then
        // overwrites them), so that nothing computed above stays live across the
        // branch.
        store_rows(FL::QG, oq);
        store_rows(FL::KG, okg);
        store_rows(FL::KI, oki);
        store_kt(s, okt);
        store_scalars(s, tot2, dsum_rows, beta_bits);
        load_raw(c + 1, 1);   // the next chunk's q and k (the operands of chunk c are out of their registers)
        if (!exact) {
            signal(C_OPS);
            wait_ge(C_OPS, 4 * (c + 1));   // every intra wave's operands are in
            wait_ge(C_T, 4 * c);           // chunk c - 1's inversion is done with Akk's space
            switch (wi) {
                case 0: intra_products(std::integral_constant<int, 0>{}, s); break;
                case 1: intra_products(std::integral_constant<int, 1>{}, s); break;
                case 2: intra_products(std::integral_constant<int, 2>{}, s); break;
                default: intra_products(std::integral_constant<int, 3>{}, s); break;
            }
        } else {
            isync();   // every intra wave's fast-path stores are done (staging overwrites them)
            wait_ge(C_T, 4 * c);           // chunk c - 1's inversion is done with Akk's space (k^T is staged there)
            // Exact path (rare: a chunk decaying past e^-16).  The chunk's inputs are
            // loaded again (the registers already hold the next chunk's) into a
            // staging area, and everything else is computed from there.
            float* sG = reinterpret_cast<float*>(smem + FL::SG);
            uint16_t* sQ = reinterpret_cast<uint16_t*>(smem + FL::SQ);
            uint16_t* sK = reinterpret_cast<uint16_t*>(smem + FL::SK);
            {
                i32x4 xqr[4], xkr[4], xgr[4][2];
                uint32_t xb;
                load_into(c, xqr, xkr, xgr, xb);
                float sl[4][8], off2[8], xt[8];
                cumsum(xgr, sl, off2, xt);
                const int ln = opaque(lane);
                const int row0 = 4 * (ln & 15), cc = 32 * wi + 8 * octet(ln);
#pragma unroll
                for (int ch = 0; ch < 8; ++ch) {
                    *reinterpret_cast<f32x4*>(sG + (cc + ch) * 64 + row0) =
                        f32x4{sl[0][ch] + off2[ch], sl[1][ch] + off2[ch], sl[2][ch] + off2[ch], sl[3][ch] + off2[ch]};
                    uint32_t q4[4], k4[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const uint32_t qw = (uint32_t)xqr[t][ch >> 1], kw = (uint32_t)xkr[t][ch >> 1];
                        q4[t] = (ch & 1) ? qw >> 16 : qw & 0xffffu;
                        k4[t] = (ch & 1) ? kw >> 16 : kw & 0xffffu;
                    }
                    *reinterpret_cast<uint2*>(sQ + (cc + ch) * 64 + row0) = make_uint2(q4[0] | (q4[1] << 16), q4[2] | (q4[3] << 16));
                    *reinterpret_cast<uint2*>(sK + (cc + ch) * 64 + row0) = make_uint2(k4[0] | (k4[1] << 16), k4[2] | (k4[3] << 16));
                }
                if (wi == 0) beta_slot(s)[ln] = __uint_as_float(BETA_F32 ? beta_bits : beta_bits << 16);
            }
            isync();   // staging complete
            // This lane's operands anchored at A = 0: q e^G, -(k e^G) and the transposed
            // copy k e^{G_last - G}, every factor <= 1 (k e^{-G} is not needed: the
            // products below do not use it); scalars a = 1, b = e^{G_last}, d = 1.
            uint32_t xq[4][4], xkg[4][4], xkt[8][2];
            {
                const int ln = opaque(lane);
                const int u = ln & 15, row0 = 4 * u, cc = 32 * wi + 8 * octet(ln);
                float gl[8];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    float qe[2][4], ke[2][4], kt[2][4];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int ch = cc + 2 * d + h;
                        const f32x4 G4 = *reinterpret_cast<const f32x4*>(sG + ch * 64 + row0);
                        gl[2 * d + h] = sG[ch * 64 + 63];   // rows past the end add g = 0
                        const uint2 q2 = *reinterpret_cast<const uint2*>(sQ + ch * 64 + row0);
                        const uint2 k2 = *reinterpret_cast<const uint2*>(sK + ch * 64 + row0);
                        const float qf[4] = {bf_lo(q2.x), bf_hi(q2.x), bf_lo(q2.y), bf_hi(q2.y)};
                        const float kf[4] = {bf_lo(k2.x), bf_hi(k2.x), bf_lo(k2.y), bf_hi(k2.y)};
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const float E = fexp2(G4[t]);
                            qe[h][t] = qf[t] * E;
                            ke[h][t] = -(kf[t] * E);
                            kt[h][t] = kf[t] * fexp2(gl[2 * d + h] - G4[t]);
                        }
                    }
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        xq[t][d] = pack_h2(qe[0][t], qe[1][t]);
                        xkg[t][d] = pack_h2(ke[0][t], ke[1][t]);
                    }
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        xkt[2 * d + h][0] = pack_h2(kt[h][0], kt[h][1]);
                        xkt[2 * d + h][1] = pack_h2(kt[h][2], kt[h][3]);
                    }
                }
                if (u == 0) {
                    char* scs = smem + FL::SC + s * FL::SC_SZ;
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        *reinterpret_cast<f32x4*>(scs + (cc + 4 * hh) * 4) = f32x4{1.f, 1.f, 1.f, 1.f};
                        *reinterpret_cast<f32x4*>(scs + 512 + (cc + 4 * hh) * 4) =
                            f32x4{fexp2(gl[4 * hh]), fexp2(gl[4 * hh + 1]), fexp2(gl[4 * hh + 2]), fexp2(gl[4 * hh + 3])};
                        *reinterpret_cast<f32x4*>(scs + 1024 + (cc + 4 * hh) * 4) = f32x4{1.f, 1.f, 1.f, 1.f};
                    }
                }
            }
            {
                // rows i = wi + 4 u of Aqk and Akk, column jj = lane, element by element
                // in fp32 from the staged G^T, q^T, k^T (log2 units)
                const int jj = opaque(lane);
                const int aqo = FL::AQ + s * FL::AB_SZ;
                float ak[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int i = wi + 4 * u;
                    float sq = 0.f, sk = 0.f;
                    if (jj <= i) {
                        for (int ch = 0; ch < DK; ++ch) {
                            const float ex = fexp2(sG[ch * 64 + i] - sG[ch * 64 + jj]);
                            const float kj = bf2f(sK[ch * 64 + jj]) * ex;
                            sq = fmaf(bf2f(sQ[ch * 64 + i]), kj, sq);
                            sk = fmaf(bf2f(sK[ch * 64 + i]), kj, sk);
                        }
                    }
                    // Aqk's slot is not staging: written at once
                    *reinterpret_cast<_Float16*>(smem + aqo + ELB(i, pi_pos(jj))) = (_Float16)(jj <= i ? p.scale * sq : 0.f);
                    ak[u] = sk;
                }
                isync();   // staging read by every intra wave
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int i = wi + 4 * u;
                    sA32[i * S68 + jj] = jj < i ? beta_slot(s)[i] * ak[u] : 0.f;
                }
            }
            store_rows(FL::QG, xq);
            store_rows(FL::KG, xkg);
            store_kt(s, xkt);
            signal(C_OPS);
        }
        signal(C_P);   // Aqk and Akk of chunk c are stored (the inversion is scan wave 0's)
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

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
//   a3  FP32 inversion      T = (I + Akk)^{-1}: diagonal 16x16 blocks by forward
//                           substitution, the rest on fp32 MFMA
//   a4  W/U recompute       W = T (beta k e^G), U = T (beta v)             (MFMA)
//   a5  delta-H scan        v_new = U - W h;
//                           h <- Diag(e^{G_last}) h + (k e^{G_last - G})^T v_new
//   a6  output              o = (scale q e^G) h + Aqk v_new                 (MFMA)
//
// The state slice h (128 x DV, fp32) lives in MFMA accumulator registers for
// the whole sequence; HBM sees q, k, v, g, beta once and o once, plus the states.
// The next chunk's inputs are loaded into registers while the current chunk
// computes.
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
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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
    // Region R1, prep view (written before the intra MFMAs):
    static constexpr int Aq = 0;                         // [64][136] q * F         (intra, rows i)
    static constexpr int Ak = Aq + 64 * S136 * 2;        // [64][136] k * F         (intra, rows i)
    static constexpr int Bd = Ak + 64 * S136 * 2;        // [64][136] k * e^{G_b - G_j} (diagonal, rows j)
    static constexpr int Bo = Bd + 64 * S136 * 2;        // [96][136] k * e^{G_{b_I} - G_j}, 6 block pairs
    static constexpr int PREP_END = Bo + 96 * S136 * 2;
    // Region R1, later view (overlaps Aq..Bo once the intra MFMAs are done):
    static constexpr int A32 = 0;                        // [64][68] fp32 Akk, then T
    static constexpr int Aqk = A32 + 64 * S68 * 4;       // [64][72] fp16
    static constexpr int T16 = Aqk + 64 * S72 * 2;       // [64][72] fp16 T diag(beta)
    static constexpr int W = T16 + 64 * S72 * 2;         // [64][136] fp16, -W
    // fp32 inversion scratch inside W's slot, column-major 16x16 blocks (stride TS):
    static constexpr int TtD = W;                        // 4 diagonal T blocks
    static constexpr int T1t = TtD + 4 * 16 * TS * 4;    // T_10, T_32 (and their A T products)
    static constexpr int Xt = T1t + 2 * 16 * TS * 4;     // 4 blocks of the 32x32 step
    static constexpr int VnT = W + 64 * S136 * 2;        // [DV][72] fp16, v_new^T
    static constexpr int Qg = VnT + DV * S72 * 2;        // [64][136] fp16, scale q e^G
    static constexpr int LATE_END = Qg + 64 * S136 * 2;
    // Transposed operands, written with the prep view and live until the state update:
    static constexpr int KgT = (PREP_END > LATE_END ? PREP_END : LATE_END);  // [128][72] (k e^G)^T
    static constexpr int KhT = KgT + 128 * S72 * 2;      // [128][72] fp16, (k e^{G_last - G})^T
    static constexpr int Vt = KhT + 128 * S72 * 2;       // [DV][72] fp16, v^T
    static constexpr int HT = Vt + DV * S72 * 2;         // [DV][136] fp16, h^T
    static constexpr int Xch = HT + DV * S136 * 2;       // 3 x [4][128] fp32 half-block sums
    static constexpr int Gam = Xch + 3 * 4 * 128 * 4;    // [128] fp32 e^{G_last}
    static constexpr int Beta = Gam + 128 * 4;           // [64] fp32
    static constexpr int Flag = Beta + 64 * 4;           // int: some block decays past the guard
    static constexpr int Ost = Flag + 16;                // [64][DV+8] bf16 output of the previous chunk
    static constexpr int BYTES = Ost + 64 * (DV + 8) * 2;
    static_assert(Xt + 4 * 16 * TS * 4 <= VnT, "inversion scratch overflows W slot");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }


__device__ __forceinline__ float fexp(float x) { return __expf(x); }
// 2^x on the hardware exp2 (v_exp_f32); arguments here are sums of g log2(e) <= 0.
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ half8 lds_h8(const char* smem, int byte_off) {
    return *reinterpret_cast<const half8*>(smem + byte_off);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over [base, base + bytes): stride 0, 32-bit dwords
// (word 3 = 0x00020000 for gfx9-family raw buffers).  Loads past `bytes` read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Two fp32 values as one 32-bit word of two bf16 (v_cvt_pk_bf16_f32, round to
// nearest even under the default rounding mode).
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2v));
}

// Two fp32 values as one 32-bit word of two fp16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    half2v h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// C += A B for 16x16 fp32 blocks on v_mfma_f32_16x16x4f32.  A is row-major (row
// stride sa), B column-major (Bt[n][k], stride sb).  Instruction s takes the k
// indices 4*(lane/16) + s, so every lane loads its four A and four B values with
// one 16-byte read each.  C: lane holds rows 4*(lane/16) .. +3 of column lane%16.
__device__ __forceinline__ f32x4 mm16(const float* A, int sa, const float* Bt, int sb, f32x4 c, int lane) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(A + (lane & 15) * sa + 4 * (lane >> 4));
    const f32x4 b = *reinterpret_cast<const f32x4*>(Bt + (lane & 15) * sb + 4 * (lane >> 4));
    f32x4 c1 = {0.f, 0.f, 0.f, 0.f};   // second accumulation chain: half the dependent latency
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
// Block (I, J) of T, in the C layout of mm16, scaled by beta of its columns into
// the fp16 operand T16 (row stride 72).
__device__ __forceinline__ void store_t16(_Float16* T16, f32x4 t, int I, int J, const float* beta, int lane) {
    const int j = 16 * J + (lane & 15);
    const float bj = beta[j];
#pragma unroll
    for (int e = 0; e < 4; ++e) T16[(16 * I + 4 * (lane >> 4) + e) * 72 + j] = (_Float16)(t[e] * bj);
}
// Trace dump of block (I, J) of T (rows past the chunk's length are skipped).
__device__ __forceinline__ void trace_tblock(float* dst, int64_t tok0, int Lc, int Hv, int hv, f32x4 t, int I, int J,
                                             int lane) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = 16 * I + 4 * (lane >> 4) + e;
        if (i < Lc) dst[((tok0 + i) * Hv + hv) * 64 + 16 * J + (lane & 15)] = t[e];
    }
}

// Work-group barrier for LDS hand-offs only.  The waves of a work-group share
// data through LDS alone (global memory is only read, or written once per
// element), so the barrier waits for this wave's LDS operations and not for its
// outstanding global loads: the prefetch of the next chunk stays in flight
// across barriers.  The asm is also a compiler memory barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Per-(block, channel) exponents, in log2 units, for the column block IB given
// the four block sums tot: off = sum_{K < IB} tot_K (ascending), tail =
// sum_{K > IB} tot_K (descending), lamarg[d] = sum_{IB < K < I2} tot_K + g_{b_I2}
// for I2 = IB + 1 + d (0 where I2 > 3).
template <int IB>
__device__ __forceinline__ void block_scalars(const f32x2 (&tot)[4], const f32x2 (&gI)[4], f32x2& off, f32x2& tail,
                                              f32x2 (&lamarg)[3]) {
    off = f32x2{0.f, 0.f};
#pragma unroll
    for (int K = 0; K < IB; ++K) off += tot[K];
    tail = f32x2{0.f, 0.f};
#pragma unroll
    for (int K = 3; K > IB; --K) tail += tot[K];
    f32x2 acc = {0.f, 0.f};
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        const int I2 = IB + 1 + d;
        if (I2 < 4) {
            lamarg[d] = acc + gI[I2 < 4 ? I2 : 3];
            acc += tot[I2 < 4 ? I2 : 3];
        } else {
            lamarg[d] = f32x2{-1000.f, -1000.f};   // unused; exp2 gives 0
        }
    }
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
    constexpr int VPT = (CH * DV / 8 + NTHREADS - 1) / NTHREADS;   // 16-byte pieces of v per thread
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

    float* sXa = reinterpret_cast<float*>(smem + L::Xch);   // [4][128] sum of rows b+1..b+7
    float* sXb = sXa + 512;                                  // [4][128] sum of rows b+8..b+15
    float* sXg = sXb + 512;                                  // [4][128] g at row b
    float* sGam = reinterpret_cast<float*>(smem + L::Gam);
    float* sBeta = reinterpret_cast<float*>(smem + L::Beta);
    int* sFlag = reinterpret_cast<int*>(smem + L::Flag);
    float* sA32 = reinterpret_cast<float*>(smem + L::A32);

    // Prefetch registers: one chunk's inputs in the prep layout (lane = channel
    // pair, wave = 8-row half block), loaded one chunk ahead of their use.  Every
    // load instruction of a wave reads one contiguous row segment (q, k: 256 B;
    // g: 512 B).
    float pf_g[8][2];
    uint32_t pf_q[8], pf_k[8];
    uint4 pf_v[VPT];
    uint32_t pf_b = 0;   // raw beta bits; converted when used
    // Loads use raw buffer instructions: a wave-uniform 128-bit descriptor per
    // row block (scalar base and byte range) and 32-bit per-lane offsets.  Rows
    // past the sequence end fall outside the descriptor's range, and the hardware
    // returns zeros for them.
    // The next chunk's loads are split into groups issued at several points of
    // the current chunk, each right after the last use of the registers it
    // refills, so that the CU's load path works in the background instead of
    // stalling every wave at one point.
    auto pf_rows = [&](int64_t cstart, int wave_) {
        const int Ln = (int)((len - cstart) < CH ? (len - cstart) : CH);
        const int row0 = 8 * wave_;
        return Ln - row0 < 0 ? 0 : (Ln - row0 > 8 ? 8 : Ln - row0);
    };
    auto prefetch_g = [&](int64_t cstart, int lane_, int wave_, int r0, int r1) {
        const int64_t t0 = bos + cstart;
        const int nrows = pf_rows(cstart, wave_);
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(p.g + (t0 + 8 * wave_) * v_tok + (int64_t)hv * DK,
                                                    nrows ? ((nrows - 1) * v_tok + DK) * 4 : 0);
#pragma unroll
        for (int rr = r0; rr < r1; ++rr) {
            // The whole offset goes in the VGPR operand: only that part is range-checked.
            const i32x2 g2 = __builtin_amdgcn_raw_buffer_load_b64(rg, 8 * lane_ + (int)(rr * v_tok * 4), 0, 0);
            pf_g[rr][0] = __int_as_float(g2[0]);
            pf_g[rr][1] = __int_as_float(g2[1]);
        }
    };
    auto prefetch_qk = [&](int64_t cstart, int lane_, int wave_, int r0, int r1) {
        const int64_t t0 = bos + cstart;
        const int nrows = pf_rows(cstart, wave_);
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + (t0 + 8 * wave_) * qk_tok + (int64_t)hq * DK,
                                                    nrows ? ((nrows - 1) * qk_tok + DK) * 2 : 0);
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + (t0 + 8 * wave_) * qk_tok + (int64_t)hq * DK,
                                                    nrows ? ((nrows - 1) * qk_tok + DK) * 2 : 0);
#pragma unroll
        for (int rr = r0; rr < r1; ++rr) {
            pf_q[rr] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rq, 4 * lane_ + (int)(rr * qk_tok * 2), 0, 0);
            pf_k[rr] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rk, 4 * lane_ + (int)(rr * qk_tok * 2), 0, 0);
        }
    };
    auto prefetch_vb = [&](int64_t cstart, int tid_) {
        const int Ln = (int)((len - cstart) < CH ? (len - cstart) : CH);
        const int64_t t0 = bos + cstart;
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
        if (tid_ < CH) {
            const int esz = p.beta_f32 ? 4 : 2;
            const __amdgpu_buffer_rsrc_t rb =
                make_rsrc(reinterpret_cast<const char*>(p.beta) + (t0 * p.Hv + hv) * esz, Ln ? ((Ln - 1) * p.Hv + 1) * esz : 0);
            pf_b = p.beta_f32 ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rb, tid_ * p.Hv * 4, 0, 0)
                              : (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rb, tid_ * p.Hv * 2, 0, 0);
        }
    };
    auto prefetch = [&](int64_t cstart, int tid_, int lane_, int wave_) {
        prefetch_g(cstart, lane_, wave_, 0, 8);
        prefetch_qk(cstart, lane_, wave_, 0, 8);
        prefetch_vb(cstart, tid_);
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

        // ================= a1: gate cumsum and decay factors =================
        // Prep layout: lane cp = channel pair (channels 2cp, 2cp + 1), wave hb =
        // half block (rows 8hb .. 8hb+7), block Ib = hb / 2, half hh = hb % 2.
        const int cp = lane, hb = wave, Ib = hb >> 1, hh = hb & 1;
        // The prefetched registers are consumed in place: g right here, v and beta
        // below, q and k up to the output operand; the next prefetch refills them
        // after their last use.
        uint32_t (&qw)[8] = pf_q;
        uint32_t (&kw)[8] = pf_k;

        // Local sums inside the half block, per channel e, in log2 units (g log2 e):
        //   lp[rr] = sum over rows (hh == 0 ? 1 : 0) .. rr   (prefix; the block's first
        //            row b is excluded because factors are anchored there)
        //   ls[rr] = sum over rows rr+1 .. 7                  (exclusive suffix)
        constexpr float LOG2E = 1.4426950408889634f;
        float lp[8][2], ls[8][2], gb2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            float g2[8];
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) g2[rr] = pf_g[rr][e] * LOG2E;
            gb2[e] = g2[0];
            float acc = hh ? g2[0] : 0.f;
            lp[0][e] = acc;
#pragma unroll
            for (int rr = 1; rr < 8; ++rr) { acc += g2[rr]; lp[rr][e] = acc; }
            float sacc = 0.f;
            ls[7][e] = 0.f;
#pragma unroll
            for (int rr = 6; rr >= 0; --rr) { sacc += g2[rr + 1]; ls[rr][e] = sacc; }
        }
        if (hh == 0) {
            *reinterpret_cast<f32x2*>(sXa + Ib * 128 + 2 * cp) = f32x2{lp[7][0], lp[7][1]};
            *reinterpret_cast<f32x2*>(sXg + Ib * 128 + 2 * cp) = f32x2{gb2[0], gb2[1]};
        } else {
            *reinterpret_cast<f32x2*>(sXb + Ib * 128 + 2 * cp) = f32x2{lp[7][0], lp[7][1]};
        }
        if (tid < CH) sBeta[tid] = __uint_as_float(p.beta_f32 ? pf_b : pf_b << 16);
        if (tid == 0) *sFlag = 0;
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
        // g, v and beta of this chunk are consumed: next chunk's g rows 0..3, v, beta.
        const bool has_next = c0 + CH < len;
        if (has_next) {
            prefetch_g(c0 + CH, lane, wave, 0, 4);
            prefetch_vb(c0 + CH, tid);
        }
        lds_barrier();

        // Block sums of both channels; then the factors of every row of this half block:
        //   F = e^{G_r - G_b}  (<= 1),  R = e^{G_e - G_r}  (<= 1)
        // and the per-(block, channel) scalars.
        float F[8][2], R[8][2];
        float eb[2], khs[2], invr[2], lam[3][2];
        int guard_local = 0;
        {
            // Block sums in log2 units; Ib and hh are wave-uniform, so every LDS
            // address below is uniform per wave except for the channel.
            const f32x2 xa = *reinterpret_cast<const f32x2*>(sXa + Ib * 128 + 2 * cp);
            const f32x2 xb = *reinterpret_cast<const f32x2*>(sXb + Ib * 128 + 2 * cp);
            const f32x2 xg = *reinterpret_cast<const f32x2*>(sXg + Ib * 128 + 2 * cp);
            f32x2 tot[4], gI[4];
#pragma unroll
            for (int K = 0; K < 4; ++K) {
                const f32x2 a = *reinterpret_cast<const f32x2*>(sXa + K * 128 + 2 * cp);
                const f32x2 b = *reinterpret_cast<const f32x2*>(sXb + K * 128 + 2 * cp);
                gI[K] = *reinterpret_cast<const f32x2*>(sXg + K * 128 + 2 * cp);
                tot[K] = (gI[K] + a) + b;
            }
            // off = sum of the blocks before Ib, tail = sum of the blocks after Ib,
            // lamarg[d] = exponent of e^{G_{b_I2} - G_{e_Ib}} for I2 = Ib + 1 + d.
            // Ib is wave-uniform: one branch per wave, no per-lane selects.
            f32x2 off, tail, lamarg[3];
            switch (Ib) {
                case 0: block_scalars<0>(tot, gI, off, tail, lamarg); break;
                case 1: block_scalars<1>(tot, gI, off, tail, lamarg); break;
                case 2: block_scalars<2>(tot, gI, off, tail, lamarg); break;
                default: block_scalars<3>(tot, gI, off, tail, lamarg); break;
            }
            const f32x2 all = ((tot[0] + tot[1]) + tot[2]) + tot[3];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float pre = hh ? xa[e] : 0.f;   // rows b+1..b+7 precede the second half
                const float suf = hh ? 0.f : xb[e];   // rows b+8..b+15 follow the first half
#pragma unroll
                for (int rr = 0; rr < 8; ++rr) {
                    F[rr][e] = fexp2(pre + lp[rr][e]);
                    R[rr][e] = fexp2(suf + ls[rr][e]);
                }
                const float qb = xa[e] + xb[e];       // (G_e - G_b) log2 e of this block
                eb[e] = fexp2(off[e] + xg[e]);        // e^{G_b}
                khs[e] = fexp2(tail[e]);              // e^{G_last - G_e}
                invr[e] = fexp2(-qb);                 // e^{G_b - G_e}
                if (-qb > GUARD_DECAY * LOG2E) guard_local = 1;
                if constexpr (TRACE) {
                    if (p.tr_G && s == 0) {
#pragma unroll
                        for (int rr = 0; rr < 8; ++rr) {
                            const int row = 8 * hb + rr;
                            if (row < Lc)
                                p.tr_G[((tok0 + row) * p.Hv + hv) * DK + 2 * cp + e] =
                                    (off[e] + xg[e] + pre + lp[rr][e]) * 0.6931471805599453f;
                        }
                    }
                }
            }
#pragma unroll
            for (int d = 0; d < 3; ++d) {
                lam[d][0] = fexp2(lamarg[d][0]);
                lam[d][1] = fexp2(lamarg[d][1]);
            }
            if (Ib == 0 && hh == 0)
                *reinterpret_cast<f32x2*>(sGam + 2 * cp) = f32x2{fexp2(all[0]), fexp2(all[1])};
        }
        if (guard_local) *sFlag = 1;
        // Intra operands (rows of this half block, two channels per 32-bit word).
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const int row = 8 * hb + rr;
            const float q0 = bf_lo(qw[rr]), q1 = bf_hi(qw[rr]);
            const float k0 = bf_lo(kw[rr]), k1 = bf_hi(kw[rr]);
            const int o = (row * S136 + 2 * cp) * 2;
            *reinterpret_cast<uint32_t*>(smem + L::Aq + o) = pack_h2(q0 * F[rr][0], q1 * F[rr][1]);
            *reinterpret_cast<uint32_t*>(smem + L::Ak + o) = pack_h2(k0 * F[rr][0], k1 * F[rr][1]);
            const float kr0 = k0 * R[rr][0], kr1 = k1 * R[rr][1];
            *reinterpret_cast<uint32_t*>(smem + L::Bd + o) = pack_h2(kr0 * invr[0], kr1 * invr[1]);
#pragma unroll
            for (int d = 0; d < 3; ++d) {
                const int I2 = Ib + 1 + d;
                if (I2 < 4) {
                    const int o2 = ((16 * pair_index(I2, Ib) + (row & 15)) * S136 + 2 * cp) * 2;
                    *reinterpret_cast<uint32_t*>(smem + L::Bo + o2) = pack_h2(kr0 * lam[d][0], kr1 * lam[d][1]);
                }
            }
        }
        // Transposed operands: (k e^G)^T for W and (k e^{G_last - G})^T for the state
        // update; eight consecutive rows of one channel are one 16-byte store.
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            half8 kg, kh;
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const float kx = e ? bf_hi(kw[rr]) : bf_lo(kw[rr]);
                kg[rr] = (_Float16)(kx * F[rr][e] * eb[e]);
                kh[rr] = (_Float16)(kx * R[rr][e] * khs[e]);
            }
            const int c = 2 * cp + e;
            *reinterpret_cast<half8*>(smem + L::KgT + (c * S72 + 8 * hb) * 2) = kg;
            *reinterpret_cast<half8*>(smem + L::KhT + (c * S72 + 8 * hb) * 2) = kh;
        }
        if (has_next) prefetch_g(c0 + CH, lane, wave, 4, 8);
        lds_barrier();
        const bool guard = *sFlag != 0;   // block-uniform

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
        lds_barrier();
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
            const int tile = wave, w64 = lane;   // 8 slots, 6 used
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
            lds_barrier();
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
                        const float ex = fexp(dsum);
                        const float kjv = bf2f(kj[c]) * ex;
                        sq += bf2f(qi[c]) * kjv;
                        sk += bf2f(ki[c]) * kjv;
                    }
                }
                reinterpret_cast<_Float16*>(smem + L::Aqk)[i * S72 + j] = (_Float16)(p.scale * sq);
                sA32[i * S68 + j] = (nn < m) ? sBeta[i] * sk : 0.f;
                if (TRACE && p.tr_Aqk && s == 0 && i < Lc) p.tr_Aqk[((tok0 + i) * p.Hv + hv) * CH + j] = p.scale * sq;
            }
        }
        // scale q e^G for the output (rows of this half block, prep layout).
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const int row = 8 * hb + rr;
            const int o = (row * S136 + 2 * cp) * 2;
            *reinterpret_cast<uint32_t*>(smem + L::Qg + o) =
                pack_h2(p.scale * bf_lo(qw[rr]) * F[rr][0] * eb[0], p.scale * bf_hi(qw[rr]) * F[rr][1] * eb[1]);
        }
        // The previous chunk's output, staged in Ost, goes out now: after this
        // chunk's prefetched registers have been consumed and before the next
        // prefetch is issued.  Global stores share the vmcnt counter with loads, so
        // this order keeps every wait for prefetched data clear of pending stores.
        if (c0 > 0) store_output(tok0 - CH, CH, tid);
        if (has_next) prefetch_qk(c0 + CH, lane, wave, 0, 4);
        lds_barrier();
        if (TRACE && p.tr_Akk && s == 0) {
            for (int idx = tid; idx < CH * CH; idx += NTHREADS) {
                const int i = idx >> 6, j = idx & 63;
                if (i < Lc) p.tr_Akk[((tok0 + i) * p.Hv + hv) * CH + j] = sA32[i * S68 + j];
            }
        }

        // ================= a3: T = (I + Akk)^{-1} in fp32 =================
        // Three barrier-separated steps.  T diag(beta), the fp16 MFMA operand T16,
        // is written by whichever wave produces each block.
        //  1. waves 0 / 1: diagonal blocks (0,1) / (2,3) by forward substitution
        //     (lane = (block, column)), then the pair T_10 / T_32 =
        //     -T_II A_I,I-1 T_I-1,I-1 on fp32 MFMA; waves 2..7 zero T16's upper blocks.
        //  2. waves 0..3: X_IJ = sum_{K=J}^{1} A_IK T_KJ  (I in {2,3}, J in {0,1}).
        //  3. waves 0..3: T_2J = -T_22 X_2J, T_3J = -(T_32 X_2J + T_33 X_3J).
        // Diagonal T blocks go back row-major into A32 (as MFMA A operands) and
        // column-major into TtD (as B operands).
        float* sTtD = reinterpret_cast<float*>(smem + L::TtD);
        float* sT1t = reinterpret_cast<float*>(smem + L::T1t);
        float* sXt = reinterpret_cast<float*>(smem + L::Xt);
        _Float16* sT16 = reinterpret_cast<_Float16*>(smem + L::T16);
        if (wave < 2) {
            const int B = 2 * wave + ((lane >> 4) & 1), j = lane & 15;   // lanes 32..63 repeat 0..31
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int kk = 0; kk < 15; ++kk) {
#pragma unroll
                for (int i = kk + 1; i < 16; ++i) x[i] -= sA32[(16 * B + i) * S68 + 16 * B + kk] * x[kk];
            }
            // The diagonal blocks of A are read only by this wave; write back after all reads.
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            if (lane < 32) {
                const float bj = sBeta[16 * B + j];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    sA32[(16 * B + i) * S68 + 16 * B + j] = x[i];
                    sT16[(16 * B + i) * S72 + 16 * B + j] = (_Float16)(x[i] * bj);
                    if (TRACE && p.tr_T && s == 0 && 16 * B + i < Lc)
                        p.tr_T[((tok0 + 16 * B + i) * p.Hv + hv) * CH + 16 * B + j] = x[i];
                }
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    f32x4 v4 = {x[4 * i4], x[4 * i4 + 1], x[4 * i4 + 2], x[4 * i4 + 3]};
                    *reinterpret_cast<f32x4*>(sTtD + (B * 16 + j) * TS + 4 * i4) = v4;
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            // pair (I, I-1) with I = 2 wave + 1: T_I,I-1 = -T_II (A_I,I-1 T_I-1,I-1)
            const int I = 2 * wave + 1, J = I - 1;
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
            y = mm16(sA32 + (16 * I) * S68 + 16 * J, S68, sTtD + J * 16 * TS, TS, y, lane);
            store_colmajor(sT1t + wave * 16 * TS, y, lane);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
            t = mm16(sA32 + (16 * I) * S68 + 16 * I, S68, sT1t + wave * 16 * TS, TS, t, lane);
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = -t[e];
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            store_rowmajor(sA32 + (16 * I) * S68 + 16 * J, S68, t, lane);   // replaces A_IJ, no longer read
            store_colmajor(sT1t + wave * 16 * TS, t, lane);
            store_t16(sT16, t, I, J, sBeta, lane);
            if (TRACE && p.tr_T && s == 0) trace_tblock(p.tr_T, tok0, Lc, p.Hv, hv, t, I, J, lane);
        } else {
            // zero upper blocks (I < J) of T16: six 16x16 blocks, 8 columns per item
            for (int it = tid - 128; it < 6 * 32; it += NTHREADS - 128) {
                const int tile = it >> 5, w32 = it & 31;
                const int I = tile < 3 ? 0 : (tile < 5 ? 1 : 2);
                const int J = tile < 3 ? tile + 1 : (tile < 5 ? tile - 1 : 3);
                const int m = w32 >> 1, h = w32 & 1;
                half8 z;
#pragma unroll
                for (int e = 0; e < 8; ++e) z[e] = (_Float16)0.f;
                *reinterpret_cast<half8*>(smem + L::T16 + ((16 * I + m) * S72 + 16 * J + 8 * h) * 2) = z;
                if (TRACE && p.tr_T && s == 0 && 16 * I + m < Lc) {
                    float* dst = p.tr_T + ((tok0 + 16 * I + m) * p.Hv + hv) * CH + 16 * J + 8 * h;
#pragma unroll
                    for (int e = 0; e < 8; ++e) dst[e] = 0.f;
                }
            }
        }
        lds_barrier();
        // Next chunk's q, k rows 4..7 (waves 0 and 1 load theirs after the diagonal work).
        if (has_next) prefetch_qk(c0 + CH, lane, wave, 4, 8);
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
        lds_barrier();
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
            store_t16(sT16, t, I, J, sBeta, lane);
            if (TRACE && p.tr_T && s == 0) trace_tblock(p.tr_T, tok0, Lc, p.Hv, hv, t, I, J, lane);
        }
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
        // The next chunk writes Xch, Beta, Flag and Vt before its first barrier; none
        // of them aliases HT.  Ost is read (and then rewritten) only after later barriers.
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

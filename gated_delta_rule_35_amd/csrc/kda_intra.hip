// Intra-chunk stages of the KDA chunked forward for gfx950 (MI355X, CDNA4).
//
// The stages of the chunked method that do not depend on the recurrent state
// ("cuLA PR #131: SM100/SM103 KDA forward to pure CuTeDSL", Summary: chunk
// intra and the FP32 Akk inversion) run here for every chunk of every
// sequence and value head at once, one work-group of 512 threads (8 wave64s)
// per (chunk, value head):
//
//   a1  gate cumsum      G = chunk-local inclusive cumsum of g (fp32, LDS only)
//   a2  intra            Aqk = scale (q e^{G_i - G_j} k^T), j <= i
//                        Akk = beta_i (k e^{G_i - G_j} k^T), j < i       (MFMA)
//   a3  FP32 inversion   T = (I + Akk)^{-1}: diagonal 16x16 blocks by forward
//                        substitution, the rest on fp32 MFMA
//
// Each work-group writes one workspace record, in fp16 (the precision in which
// the scan kernel's MFMAs consume it): the lower 16x16 tiles of Aqk and of
// T diag(beta) (staged in LDS, stored as 16-byte pieces at the end), and the
// decayed operands scale q e^G, (k e^G)^T, (k e^{G_last - G})^T with e^{G_last}
// (stored from registers as soon as the factors exist).  The scan kernel then
// needs nothing of q, k and g.  Two work-groups share a CU, so one's loads and inversion
// latency overlap the other's factor and MFMA work.
//
// Per-channel decay inside MFMA products.  exp(G_i - G_j) is factored through
// an anchor row a: exp(G_i - G_a) * exp(G_a - G_j).  The 64 rows form four
// 16-row blocks.  For an off-diagonal block pair (row block I > column block J)
// the anchor is the first row of I, so both factors are <= 1.  For a diagonal
// block the anchor is the block's first row: the row factor is <= 1 and the
// column factor is <= exp(block decay).  When a 16-row block decays by more
// than exp(-8) on some channel (far outside the usual gate range), the
// diagonal blocks of that chunk are recomputed element by element in fp32.
#include "kda_device.h"

namespace kda {

namespace {

constexpr float GUARD_DECAY = 8.0f;
constexpr int S68 = 68;   // fp32 rows of 64 (+4 pad)
constexpr int S72 = 72;   // fp16 rows of 64 (+8 pad)
constexpr int TS = 20;    // fp32 columns of a 16x16 column-major block (+4 pad)

struct IntraLds {
    // Prep view: MFMA operand rows of 128 fp16 channels (256 B), unpadded; the
    // sixteen 16-byte pieces of row r are permuted by XOR with r mod 16, so the
    // 16 rows an MFMA operand read touches fall in distinct banks.
    static constexpr int Aq = 0;                  // [64]  q_i e^{G_i - G_b}
    static constexpr int Ak = Aq + 64 * 256;      // [64]  k_i e^{G_i - G_b}
    static constexpr int Bd = Ak + 64 * 256;      // [64]  k_j e^{G_b - G_j}        (diagonal blocks)
    static constexpr int Bo = Bd + 64 * 256;      // [96]  k_j e^{G_{b_I} - G_j}     (6 block pairs)
    static constexpr int PREP_END = Bo + 96 * 256;
    // Late view (overlaps the prep view once the intra MFMAs are done):
    static constexpr int A32 = 0;                          // [64][68] fp32 Akk, then T
    static constexpr int T16 = A32 + 64 * S68 * 4;         // [64][72] fp16 T diag(beta)
    static constexpr int TtD = T16 + 64 * S72 * 2;         // 4 diagonal T blocks, column-major
    static constexpr int T1t = TtD + 4 * 16 * TS * 4;      // T_10, T_32 (and their A T products)
    static constexpr int Xt = T1t + 2 * 16 * TS * 4;       // 4 blocks of the 32x32 step
    static constexpr int Aqk16 = Xt + 4 * 16 * TS * 4;     // [64][72] fp16 Aqk
    static constexpr int LATE_END = Aqk16 + 64 * S72 * 2;
    static constexpr int Xch = PREP_END;                   // 3 x [4][128] fp32 half-block sums
    static constexpr int Beta = Xch + 3 * 4 * 128 * 4;     // [64] fp32
    static constexpr int Flag = Beta + 64 * 4;             // int: some block decays past the guard
    static constexpr int BYTES = Flag + 16;
    static_assert(LATE_END <= PREP_END, "late view overflows the prep view");
    static_assert(BYTES <= 80 * 1024, "two work-groups per CU");
};

// Byte offset of channel c (even) of row r in a swizzled operand array.
__device__ __forceinline__ int swz(int r, int c) { return r * 256 + ((((c >> 3) ^ r) & 15) << 4) + ((c & 7) << 1); }
// Byte offset of the 16-byte piece kc (channels 8kc .. 8kc+7) of row r.
__device__ __forceinline__ int swz_piece(int r, int kc) { return r * 256 + (((kc ^ r) & 15) << 4); }

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
// the fp16 tile array T16 (row stride 72).
__device__ __forceinline__ void store_t16(_Float16* T16, f32x4 t, int I, int J, const float* beta, int lane) {
    const int j = 16 * J + (lane & 15);
    const float bj = beta[j];
#pragma unroll
    for (int e = 0; e < 4; ++e) T16[(16 * I + 4 * (lane >> 4) + e) * S72 + j] = (_Float16)(t[e] * bj);
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

// Per-(block, channel) exponents, in log2 units, for the column block IB given
// the four block sums tot: off = sum_{K < IB} tot_K, tail = sum_{K > IB} tot_K,
// lamarg[d] = sum_{IB < K < I2} tot_K + g_{b_I2} for I2 = IB + 1 + d (unused
// where I2 > 3).
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

// The MFMA operands of the eight rows 16 IB + 8 hh + rr of a half block, lane cp
// holding channels 2 cp, 2 cp + 1: q e^{G - G_b} (Aq), k e^{G - G_b} (Ak),
// k e^{G_b - G} (Bd) and, for each later block I2 = IB + 1 + d, k e^{G_{b_I2} - G}
// (the rows of the block pair (I2, IB) in Bo), from F = e^{G - G_b},
// R = e^{G_e - G}, invr = e^{G_b - G_e} and lam[d] = e^{G_{b_I2} - G_e}.
template <int IB>
__device__ __forceinline__ void write_operands(char* smem, const uint32_t (&qw)[8], const uint32_t (&kw)[8],
                                               const float (&F)[8][2], const float (&R)[8][2], const float (&invr)[2],
                                               const float (&lam)[3][2], int hh, int cp) {
    using L = IntraLds;
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
        const int row = 16 * IB + 8 * hh + rr;
        const float q0 = bf_lo(qw[rr]), q1 = bf_hi(qw[rr]);
        const float k0 = bf_lo(kw[rr]), k1 = bf_hi(kw[rr]);
        const int o = swz(row, 2 * cp);
        *reinterpret_cast<uint32_t*>(smem + L::Aq + o) = pack_h2(q0 * F[rr][0], q1 * F[rr][1]);
        *reinterpret_cast<uint32_t*>(smem + L::Ak + o) = pack_h2(k0 * F[rr][0], k1 * F[rr][1]);
        const float kr0 = k0 * R[rr][0], kr1 = k1 * R[rr][1];
        *reinterpret_cast<uint32_t*>(smem + L::Bd + o) = pack_h2(kr0 * invr[0], kr1 * invr[1]);
#pragma unroll
        for (int d = 0; d < 3 - IB; ++d) {
            const int o2 = swz(16 * pair_index(IB + 1 + d, IB) + (row & 15), 2 * cp);
            *reinterpret_cast<uint32_t*>(smem + L::Bo + o2) = pack_h2(kr0 * lam[d][0], kr1 * lam[d][1]);
        }
    }
}

// 4x4 transpose of 32-bit words across each quad of lanes: on entry quad lane j
// holds x[0..3]; on exit it holds x[p] = (x[j] of quad lane p).  Two butterfly
// stages: lanes j and j ^ 2 swap the 2x2 blocks off the diagonal, then lanes j and
// j ^ 1 swap the off-diagonal elements of each 2x2 block (DPP quad_perm
// [2,3,0,1], then [1,0,3,2]).
__device__ __forceinline__ void quad_transpose(uint32_t (&x)[4], int j) {
    const bool b1 = (j & 2) != 0, b0 = (j & 1) != 0;
#pragma unroll
    for (int e = 0; e < 2; ++e) {   // element pairs (0, 2), (1, 3)
        const uint32_t send = b1 ? x[e] : x[e + 2];
        const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x4e, 0xf, 0xf, false);
        if (b1) x[e] = recv; else x[e + 2] = recv;
    }
#pragma unroll
    for (int e = 0; e < 4; e += 2) {   // element pairs (0, 1), (2, 3)
        const uint32_t send = b0 ? x[e] : x[e + 1];
        const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xb1, 0xf, 0xf, false);
        if (b0) x[e] = recv; else x[e + 1] = recv;
    }
}

}  // namespace

template <bool TRACE, bool QGO>
__global__ void __launch_bounds__(NTHREADS, 4) kda_intra_kernel(const KdaParams p) {
    using L = IntraLds;
    __shared__ __attribute__((aligned(16))) char smem[L::BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // Work-group -> (slot, value head): slots from the last to the first, value
    // heads fastest.  The records the scan kernel reads first are then the last
    // written, and the last-level cache (the 256 MB MALL) still holds them when the
    // scan starts: when all records fit in it (B=1, Hv=64, T=4096: 258 MB) the
    // forward takes 7% less time; elsewhere the order changes nothing measurable.
    // Work-groups are dealt to the 8 XCDs round robin; the value heads that share
    // one q/k head (grouped values) are taken Hq work-groups apart, so that (Hq a
    // multiple of 8) they run on one XCD, whose L2 then serves their q and k.
    const int64_t slot = (p.nslots - 1) - (int64_t)(blockIdx.x / p.Hv);
    const int r = (int)(blockIdx.x % p.Hv);
    const int grp = p.Hv / p.Hq;
    const int hv = grp == 1 ? r : (r % p.Hq) * grp + r / p.Hq;
    const int hq = hv / grp;

    // slot -> (sequence, chunk): the first slot of sequence n, floor(bos_n / 64) + n,
    // does not decrease with n; take the last sequence whose first slot is <= slot.
    int n;
    if (!p.cu && !p.seg_tokens && p.T % CH == 0) {
        n = (int)(slot / (p.T / CH + 1));   // sequence n has slots n (T/64 + 1) .. + T/64 - 1
    } else {
        int lo = 0, hi = p.N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            int64_t b, l;
            seq_bounds(p, mid, b, l);
            if (chunk_slot(b, mid, 0) <= slot) lo = mid; else hi = mid - 1;
        }
        n = lo;
    }
    int64_t bos, len;
    seq_bounds(p, n, bos, len);
    const int64_t cidx = slot - chunk_slot(bos, n, 0);
    if (cidx < 0 || cidx * CH >= len) return;   // no chunk maps to this slot (uniform per work-group)
    const int64_t tok0 = bos + cidx * CH;
    const int Lc = (int)((len - cidx * CH) < CH ? (len - cidx * CH) : CH);
    const int64_t qk_tok = (int64_t)p.Hq * DK;   // token stride of q, k
    const int64_t v_tok = (int64_t)p.Hv * DK;    // token stride of g
    char* rec = p.ws + (slot * p.Hv + hv) * WS_RECORD_BYTES;

    float* sXa = reinterpret_cast<float*>(smem + L::Xch);   // [4][128] sum of rows b+1..b+7
    float* sXb = sXa + 512;                                  // [4][128] sum of rows b+8..b+15
    float* sXg = sXb + 512;                                  // [4][128] g at row b
    float* sBeta = reinterpret_cast<float*>(smem + L::Beta);
    int* sFlag = reinterpret_cast<int*>(smem + L::Flag);
    float* sA32 = reinterpret_cast<float*>(smem + L::A32);

    // ================= loads =================
    // Wave priority: the other work-group on the CU is usually in a VALU phase, and
    // a raised priority lets this one's loads (and, at the end, its record stores)
    // issue ahead of that work (about 0.7% on the whole kernel; keeping the priority
    // up through the VALU phases instead costs 9%).
    __builtin_amdgcn_s_setprio(3);
    // Layout: lane cp = channel pair (channels 2cp, 2cp + 1), wave hb = half block
    // (rows 8hb .. 8hb+7), block Ib = hb / 2, half hh = hb % 2.  Each load
    // instruction of a wave reads one contiguous row segment; rows past the
    // chunk's end fall outside the buffer range and read as zero.
    const int cp = lane, hb = wave, Ib = hb >> 1, hh = hb & 1;
    float gl[8][2];
    uint32_t qw[8], kw[8];
    {
        const int nr = Lc - 8 * hb < 0 ? 0 : (Lc - 8 * hb > 8 ? 8 : Lc - 8 * hb);
        const int64_t t0 = tok0 + 8 * hb;
        const __amdgpu_buffer_rsrc_t rg =
            make_rsrc(p.g + t0 * v_tok + (int64_t)hv * DK, nr ? ((nr - 1) * v_tok + DK) * 4 : 0);
        const __amdgpu_buffer_rsrc_t rq =
            make_rsrc(p.q + t0 * qk_tok + (int64_t)hq * DK, nr ? ((nr - 1) * qk_tok + DK) * 2 : 0);
        const __amdgpu_buffer_rsrc_t rk =
            make_rsrc(p.k + t0 * qk_tok + (int64_t)hq * DK, nr ? ((nr - 1) * qk_tok + DK) * 2 : 0);
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const i32x2 g2 = __builtin_amdgcn_raw_buffer_load_b64(rg, 8 * lane + (int)(rr * v_tok * 4), 0, 0);
            gl[rr][0] = __int_as_float(g2[0]);
            gl[rr][1] = __int_as_float(g2[1]);
        }
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            qw[rr] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rq, 4 * lane + (int)(rr * qk_tok * 2), 0, 0);
            kw[rr] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rk, 4 * lane + (int)(rr * qk_tok * 2), 0, 0);
        }
        if (tid < CH) {
            const int esz = p.beta_f32 ? 4 : 2;
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(reinterpret_cast<const char*>(p.beta) + (tok0 * p.Hv + hv) * esz,
                                                        ((Lc - 1) * (int64_t)p.Hv + 1) * esz);
            const float b = p.beta_f32
                                ? __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, tid * p.Hv * 4, 0, 0))
                                : bf2f((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rb, tid * p.Hv * 2, 0, 0));
            sBeta[tid] = b;
        }
    }
    __builtin_amdgcn_s_setprio(0);
    if (tid == 0) *sFlag = 0;

    // ================= a1: gate cumsum =================
    // Local sums inside the half block, per channel e, in log2 units (g log2 e):
    //   lp[rr] = sum over rows (hh == 0 ? 1 : 0) .. rr   (prefix; the block's first
    //            row b is excluded because factors are anchored there)
    //   ls[rr] = sum over rows rr+1 .. 7                  (exclusive suffix)
    float lp[8][2], ls[8][2], gb2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        float g2[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) g2[rr] = gl[rr][e] * LOG2E;
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
    lds_barrier();

    // Factors of every row of this half block:
    //   F = e^{G_r - G_b}  (<= 1),  R = e^{G_e - G_r}  (<= 1)   (b, e: first, last row)
    // and the per-(block, channel) scalars invr = e^{G_b - G_e}, lam[d] = e^{G_{b_I2} - G_e},
    // eb = e^{G_b}, khs = e^{G_last - G_e}.
    float F[8][2], R[8][2];
    float invr[2], lam[3][2], eb[2], khs[2];
    int guard_local = 0;
    {
        const f32x2 xa = *reinterpret_cast<const f32x2*>(sXa + Ib * 128 + 2 * cp);
        const f32x2 xb = *reinterpret_cast<const f32x2*>(sXb + Ib * 128 + 2 * cp);
        f32x2 tot[4], gI[4];
#pragma unroll
        for (int K = 0; K < 4; ++K) {
            const f32x2 a = *reinterpret_cast<const f32x2*>(sXa + K * 128 + 2 * cp);
            const f32x2 b = *reinterpret_cast<const f32x2*>(sXb + K * 128 + 2 * cp);
            gI[K] = *reinterpret_cast<const f32x2*>(sXg + K * 128 + 2 * cp);
            tot[K] = (gI[K] + a) + b;
        }
        // Ib is wave-uniform: one branch per wave, no per-lane selects.
        f32x2 off, tail, lamarg[3];
        switch (Ib) {
            case 0: block_scalars<0>(tot, gI, off, tail, lamarg); break;
            case 1: block_scalars<1>(tot, gI, off, tail, lamarg); break;
            case 2: block_scalars<2>(tot, gI, off, tail, lamarg); break;
            default: block_scalars<3>(tot, gI, off, tail, lamarg); break;
        }
        if (Ib == 0 && hh == 0) {
            // e^{G_last} of the two channels
            const f32x2 all = ((tot[0] + tot[1]) + tot[2]) + tot[3];
            *reinterpret_cast<f32x2*>(rec + WS_GAM + 8 * cp) = f32x2{fexp2(all[0]), fexp2(all[1])};
        }
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
            invr[e] = fexp2(-qb);                 // e^{G_b - G_e}
            eb[e] = fexp2(off[e] + gI[Ib][e]);    // e^{G_b}
            khs[e] = fexp2(tail[e]);              // e^{G_last - G_e}
            if (-qb > GUARD_DECAY * LOG2E) guard_local = 1;
            if constexpr (TRACE) {
                if (p.tr_G) {
                    const float gb = off[e] + gI[Ib][e];
#pragma unroll
                    for (int rr = 0; rr < 8; ++rr) {
                        const int row = 8 * hb + rr;
                        if (row < Lc) p.tr_G[((tok0 + row) * p.Hv + hv) * DK + 2 * cp + e] = (gb + pre + lp[rr][e]) * LN2;
                    }
                }
            }
        }
#pragma unroll
        for (int d = 0; d < 3; ++d) {
            lam[d][0] = fexp2(lamarg[d][0]);
            lam[d][1] = fexp2(lamarg[d][1]);
        }
    }
    if (guard_local) *sFlag = 1;
    // Intra operands (rows of this half block, two channels per 32-bit word); one
    // copy of the loop per block, so that each wave writes its 3 - Ib off-diagonal
    // operands without a branch per row.
    switch (Ib) {
        case 0: write_operands<0>(smem, qw, kw, F, R, invr, lam, hh, cp); break;
        case 1: write_operands<1>(smem, qw, kw, F, R, invr, lam, hh, cp); break;
        case 2: write_operands<2>(smem, qw, kw, F, R, invr, lam, hh, cp); break;
        default: write_operands<3>(smem, qw, kw, F, R, invr, lam, hh, cp); break;
    }
    // The scan kernel's operands of this chunk, straight to the record.  scale q e^G
    // and -(k e^G) go out as 16-byte row pieces of 8 channels, gathered from the
    // four lanes of a quad; (k e^{G_last - G})^T per channel as its eight rows.
    {
        const float sq0 = p.scale * eb[0], sq1 = p.scale * eb[1];
        if constexpr (QGO) {
            // The QG output, q e^G = q F e^{G_b} (no scale), rounded once to bf16:
            // each row is one 256-byte run over the wave's 64 channel pairs.
            uint16_t* qgo = p.qg + (tok0 + 8 * hb) * v_tok + (int64_t)hv * DK + 2 * cp;
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                if (8 * hb + rr < Lc)
                    *reinterpret_cast<uint32_t*>(qgo + rr * v_tok) =
                        pack_bf2(bf_lo(qw[rr]) * F[rr][0] * eb[0], bf_hi(qw[rr]) * F[rr][1] * eb[1]);
            }
        }
        uint32_t qg[8], kg[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const float k0 = bf_lo(kw[rr]), k1 = bf_hi(kw[rr]);
            qg[rr] = pack_h2(bf_lo(qw[rr]) * F[rr][0] * sq0, bf_hi(qw[rr]) * F[rr][1] * sq1);
            kg[rr] = pack_h2(-(k0 * F[rr][0] * eb[0]), -(k1 * F[rr][1] * eb[1]));
        }
        const int qa = cp >> 2, qj = cp & 3;   // quad: channels 8 qa .. 8 qa + 7
#pragma unroll
        for (int b4 = 0; b4 < 2; ++b4) {
            uint32_t xq[4] = {qg[4 * b4], qg[4 * b4 + 1], qg[4 * b4 + 2], qg[4 * b4 + 3]};
            uint32_t xk[4] = {kg[4 * b4], kg[4 * b4 + 1], kg[4 * b4 + 2], kg[4 * b4 + 3]};
            quad_transpose(xq, qj);
            quad_transpose(xk, qj);
            // row 8 hb + 4 b4 + qj, channels 8 qa ..: fragment (row / 32, qa / 2), lane row % 32 + 32 (qa % 2)
            const int row = 8 * hb + 4 * b4 + qj;
            const int fo = ((row >> 5) * 8 + (qa >> 1)) * WS_FRAG + ((row & 31) + 32 * (qa & 1)) * 16;
            *reinterpret_cast<uint4*>(rec + WS_QG + fo) = make_uint4(xq[0], xq[1], xq[2], xq[3]);
            *reinterpret_cast<uint4*>(rec + WS_KG + fo) = make_uint4(xk[0], xk[1], xk[2], xk[3]);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            half8 kh;
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const float kx = e ? bf_hi(kw[rr]) : bf_lo(kw[rr]);
                kh[rr] = (_Float16)(kx * R[rr][e] * khs[e]);
            }
            // channel c, rows 8 hb ..: fragment (c / 32, hb / 2), lane c % 32 + 32 (hb % 2)
            const int c = 2 * cp + e;
            const int fo = ((c >> 5) * 4 + (hb >> 1)) * WS_FRAG + ((c & 31) + 32 * (hb & 1)) * 16;
            *reinterpret_cast<half8*>(rec + WS_KH + fo) = kh;
        }
    }
    lds_barrier();
    const bool guard = *sFlag != 0;   // work-group uniform

    // ================= a2: intra-chunk Aqk / Akk on MFMA =================
    // 20 jobs of 16x16 output tiles: (matrix, I, J) with J <= I.  Each tile is
    // computed transposed (rows j, cols i) so that a lane holds 4 consecutive j of
    // one row i.
    // Lane l reads, in k step kk, the 16-byte piece 4 kk + l / 16 of row l % 16 of
    // a 16-row operand block: the same swizzled offset within every block.
    int swo[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) swo[kk] = swz_piece(lane & 15, 4 * kk + (lane >> 4));
    f32x4 iacc[3];
    int jobI[3], jobJ[3], jobM[3];
#pragma unroll
    for (int u = 0; u < 3; ++u) {
        const int job = wave + 8 * u;
        jobM[u] = -1;
        if (job < 20) {
            const int m = job / 10, pidx = job % 10;
            const int I = pidx >= 6 ? 3 : (pidx >= 3 ? 2 : (pidx >= 1 ? 1 : 0));
            const int J = pidx - I * (I + 1) / 2;
            jobM[u] = m; jobI[u] = I; jobJ[u] = J;
            const int baseB = (I == J) ? L::Bd + 16 * J * 256 : L::Bo + 16 * pair_index(I, J) * 256;
            const int baseA = (m == 0 ? L::Aq : L::Ak) + 16 * I * 256;
            // all eight operand pieces first, then the four MFMAs
            half8 a[4], b[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                a[kk] = lds_h8(smem, baseB + swo[kk]);
                b[kk] = lds_h8(smem, baseA + swo[kk]);
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[kk], b[kk], acc, 0, 0, 0);
            iacc[u] = acc;
        }
    }
    lds_barrier();   // A32 overlaps the operand arrays
    // Aqk tiles go to the fp16 staging tile Aqk16 (the diagonal ones are rewritten
    // exactly below for a guarded chunk); Akk tiles go to A32.  Only diagonal
    // tiles need the causal masks (I and J are uniform per wave).
    _Float16* sAqk16 = reinterpret_cast<_Float16*>(smem + L::Aqk16);
#pragma unroll
    for (int u = 0; u < 3; ++u) {
        if (jobM[u] >= 0) {
            const int I = jobI[u], J = jobJ[u];
            const int i = 16 * I + (lane & 15);
            const int j0 = 16 * J + 4 * (lane >> 4);
            f32x4 v4 = iacc[u];
            if (jobM[u] == 0) {
                v4 *= p.scale;
                if (I == J) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v4[e] = (j0 + e <= i) ? v4[e] : 0.f;
                }
                half4 h4;
#pragma unroll
                for (int e = 0; e < 4; ++e) h4[e] = (_Float16)v4[e];
                *reinterpret_cast<half4*>(sAqk16 + i * S72 + j0) = h4;
                if (TRACE && p.tr_Aqk && i < Lc) {
                    float* dst = p.tr_Aqk + ((tok0 + i) * p.Hv + hv) * CH + j0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[e] = v4[e];
                }
            } else {
                v4 *= sBeta[i];
                if (I == J) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v4[e] = (j0 + e < i) ? v4[e] : 0.f;
                }
                *reinterpret_cast<f32x4*>(smem + L::A32 + (i * S68 + j0) * 4) = v4;
            }
        }
    }
    if constexpr (TRACE) {
        // Upper 16x16 tiles (I < J) of Akk and Aqk are zero (the dumps read them).
        const int tile = wave, w64 = lane;   // 8 slots, 6 used
        if (tile < 6) {
            const int I = tile < 3 ? 0 : (tile < 5 ? 1 : 2);
            const int J = tile < 3 ? tile + 1 : (tile < 5 ? tile - 1 : 3);
            const int m = w64 >> 2, q4 = w64 & 3;
            const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<f32x4*>(smem + L::A32 + ((16 * I + m) * S68 + 16 * J + 4 * q4) * 4) = z4;
            if (p.tr_Aqk && 16 * I + m < Lc) {
                float* dst = p.tr_Aqk + ((tok0 + 16 * I + m) * p.Hv + hv) * CH + 16 * J + 4 * q4;
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[e] = 0.f;
            }
        }
    }
    if (guard) {
        // Exact fp32 diagonal blocks for strongly decaying chunks.
        lds_barrier();
        const int64_t tq = (int64_t)hq * DK, tg = (int64_t)hv * DK;
        for (int idx = tid; idx < 4 * 256; idx += NTHREADS) {
            const int B = idx >> 8, m = (idx >> 4) & 15, nn = idx & 15;
            const int i = 16 * B + m, j = 16 * B + nn;
            float sq = 0.f, sk = 0.f;
            if (nn <= m && i < Lc) {
                const uint16_t* qi = p.q + (tok0 + i) * qk_tok + tq;
                const uint16_t* ki = p.k + (tok0 + i) * qk_tok + tq;
                const uint16_t* kj = p.k + (tok0 + j) * qk_tok + tq;
                for (int c = 0; c < DK; ++c) {
                    float dsum = 0.f;
                    for (int rr = j + 1; rr <= i; ++rr) dsum += p.g[(tok0 + rr) * v_tok + tg + c];
                    const float ex = fexp(dsum);
                    const float kjv = bf2f(kj[c]) * ex;
                    sq += bf2f(qi[c]) * kjv;
                    sk += bf2f(ki[c]) * kjv;
                }
            }
            sAqk16[i * S72 + j] = (_Float16)(p.scale * sq);
            if (nn <= m) sA32[i * S68 + j] = (nn < m) ? sBeta[i] * sk : 0.f;
            if (TRACE && p.tr_Aqk && nn <= m && i < Lc) p.tr_Aqk[((tok0 + i) * p.Hv + hv) * CH + j] = p.scale * sq;
        }
    }
    lds_barrier();
    if (TRACE && p.tr_Akk) {
        for (int idx = tid; idx < CH * CH; idx += NTHREADS) {
            const int i = idx >> 6, j = idx & 63;
            if (i < Lc) p.tr_Akk[((tok0 + i) * p.Hv + hv) * CH + j] = sA32[i * S68 + j];
        }
    }

    // The fragments include the upper 16x16 tiles (0,1) and (2,3) of Aqk and T:
    // zero them in the staging tiles (waves 2..7 are idle in the first inversion step).
    if (tid >= 128 && tid < 128 + 4 * 32) {
        const int it = tid - 128, w = it >> 5, r = (it >> 1) & 15, h = it & 1;
        const int blk = w & 1;   // tile (0,1) or (2,3)
        *reinterpret_cast<uint4*>(smem + ((w >> 1) ? L::T16 : L::Aqk16) +
                                  ((32 * blk + r) * S72 + 32 * blk + 16 + 8 * h) * 2) = make_uint4(0, 0, 0, 0);
    }

    // ================= a3: T = (I + Akk)^{-1} in fp32 =================
    // Three barrier-separated steps.  T diag(beta) goes into T16 (fp16), written
    // by whichever wave produces each block.
    //  1. waves 0 / 1: diagonal blocks (0,1) / (2,3) by forward substitution
    //     (lane = (block, column)), then the pair T_10 / T_32 =
    //     -T_II A_I,I-1 T_I-1,I-1 on fp32 MFMA.
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
                if (TRACE && p.tr_T && 16 * B + i < Lc) p.tr_T[((tok0 + 16 * B + i) * p.Hv + hv) * CH + 16 * B + j] = x[i];
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
        if (TRACE && p.tr_T) trace_tblock(p.tr_T, tok0, Lc, p.Hv, hv, t, I, J, lane);
    } else if (TRACE && p.tr_T) {
        // upper blocks (I < J) of T are zero
        for (int it = tid - 128; it < 6 * 32; it += NTHREADS - 128) {
            const int tile = it >> 5, w32 = it & 31;
            const int I = tile < 3 ? 0 : (tile < 5 ? 1 : 2);
            const int J = tile < 3 ? tile + 1 : (tile < 5 ? tile - 1 : 3);
            const int m = w32 >> 1, h = w32 & 1;
            if (16 * I + m < Lc) {
                float* dst = p.tr_T + ((tok0 + 16 * I + m) * p.Hv + hv) * CH + 16 * J + 8 * h;
#pragma unroll
                for (int e = 0; e < 8; ++e) dst[e] = 0.f;
            }
        }
    }
    lds_barrier();
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
        if (TRACE && p.tr_T) trace_tblock(p.tr_T, tok0, Lc, p.Hv, hv, t, I, J, lane);
    }
    lds_barrier();

    __builtin_amdgcn_s_setprio(2);
    // The record's Aqk and T diag(beta) fragments (six each, 768 16-byte pieces;
    // the T columns in accumulator row order, two 8-byte runs per piece).
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int it = tid + NTHREADS * u;
        if (it < 12 * 64) {
            const int f = it >> 6, l = it & 63, ff = f % 6;
            const int m = ff < 2 ? 0 : 1, kk = ff < 2 ? ff : ff - 2;
            const int rowo = (32 * m + (l & 31)) * S72 + 16 * kk;
            uint4 w;
            if (f < 6) {
                w = *reinterpret_cast<const uint4*>(smem + L::Aqk16 + (rowo + 8 * (l >> 5)) * 2);
            } else {
                const uint2 lo = *reinterpret_cast<const uint2*>(smem + L::T16 + (rowo + 4 * (l >> 5)) * 2);
                const uint2 hi = *reinterpret_cast<const uint2*>(smem + L::T16 + (rowo + 8 + 4 * (l >> 5)) * 2);
                w = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
            *reinterpret_cast<uint4*>(rec + it * 16) = w;
        }
    }
}

hipError_t launch_kda_intra(const KdaParams& p, bool trace, hipStream_t stream) {
    const int64_t nblocks = p.nslots * p.Hv;
    if (nblocks == 0) return hipSuccess;
    if (trace)
        hipLaunchKernelGGL((kda_intra_kernel<true, false>), dim3((unsigned)nblocks), dim3(NTHREADS), 0, stream, p);
    else if (p.qg)
        hipLaunchKernelGGL((kda_intra_kernel<false, true>), dim3((unsigned)nblocks), dim3(NTHREADS), 0, stream, p);
    else
        hipLaunchKernelGGL((kda_intra_kernel<false, false>), dim3((unsigned)nblocks), dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
}

int64_t workspace_bytes(int64_t total_tokens, int64_t N, int64_t Hv) {
    return ((total_tokens + CH - 1) / CH + N) * Hv * WS_RECORD_BYTES;
}

}  // namespace kda

// State-dependent stages of the KDA chunked forward for gfx950 (MI355X, CDNA4).
//
// One work-group of six wave64s owns one (sequence, value head, 64-wide dv
// slice) and walks that sequence's chunks of 64 tokens in order.  Per chunk it
// runs the stages that depend on the recurrent state ("cuLA PR #131:
// SM100/SM103 KDA forward to pure CuTeDSL", Summary: recompute W/U; "cuLA
// REPO_LAYOUT.md", ops/: chunk delta-H and forward output):
//
//   a4+a5  v_new = U - W h  with  W = T diag(beta) (k e^G),  U = T diag(beta) v,
//          evaluated as  v_new = T diag(beta) (v - (k e^G) h)
//          h <- Diag(e^{G_last}) h + (k e^{G_last - G})^T v_new
//   a6     o = (scale q e^G) h + Aqk v_new
//
// Everything state-independent comes from the intra kernel's workspace record of
// the chunk, stored as MFMA operand fragments.  Two loader waves copy each record
// once into LDS by DMA (buffer loads that write LDS directly), two chunks ahead,
// double-buffered, between the two barriers of each chunk; every compute wave then
// reads its fragments from there.  v comes the
// same way, one chunk ahead.  The kernel reads only v and the records from
// memory, and writes o and the final state; its loops hold no loads into
// registers, so every wait for memory is an explicit, counted one.
//
// Roles.  Two wave pairs, each owning 32 dv columns, and two loader waves.  A pair's state h (128 x 32,
// fp32) is split by rows between its two waves, which keep their 32 x 32 tiles
// in MFMA accumulators for the whole sequence; only fp16 copies of h and v_new
// cross between them, through LDS.  Per chunk:
//   chain wave:   Z = v - (k e^G) h  (MFMA, accumulators start from v);
//                 v_new = T diag(beta) Z, its B operand taken straight from Z's
//                 accumulator registers (the record's T columns are in
//                 accumulator row order); v_new^T -> LDS
//   output wave:  o^T = h^T (scale q e^G)^T, the state-only part of o
//   barrier
//   both:         own state rows h <- e^{G_last} h + Khat^T v_new; fp16 h^T -> LDS
//   barrier
//   output wave:  o^T += v_new^T Aqk^T; o stored (bf16) straight from the
//                 accumulators, four channels per lane store
//   loader waves: after the first barrier, the record DMA of chunk + 2 into the
//                 buffer this chunk was read from; before the second, wait for
//                 chunk + 1's
// All products run on v_mfma_f32_32x32x16_f16 (fp16 operands, fp32 accumulate).
//
// A grid may hold up to three jobs (ScanJobs), each a full set of parameters over
// its own sequences: the segmented forward runs a sequence's segments side by side
// this way (segment 0 from the initial state next to the later segments' state
// maps: from the identity with v read as zero, and from zero, neither with output).
// The ordinary forward launches the single-job instantiation, whose parameters sit
// at fixed kernel-argument offsets.
#include "kda_device.h"

namespace kda {

namespace {

constexpr int SCAN_THREADS = 384;   // two (chain, output) pairs and two record loaders
constexpr int DVW = 32;             // dv columns per pair
constexpr int PAIRS = 2;
constexpr int SLICES = DK / (DVW * PAIRS);                   // work-groups per (sequence, head)
constexpr int REC_PIECES = (WS_RECORD_BYTES + WS_FRAG - 1) / WS_FRAG;   // 1 KB DMA pieces of a record
constexpr int REC_LDS = REC_PIECES * WS_FRAG;
constexpr int S136 = 136;           // fp16 rows of 128 (+8 pad)
constexpr int S72 = 72;             // 16-bit rows of 64 (+8 pad)

struct ScanLds {
    static constexpr int Rec = 0;                          // [2][REC_LDS] records of two chunks
    static constexpr int Pair = 2 * REC_LDS;               // then, per pair:
    static constexpr int HT = 0;                           //   [32][136] fp16 h^T (dv column x key)
    static constexpr int VnT = HT + DVW * S136 * 2;        //   [32][72] fp16 v_new^T (dv column x token)
    static constexpr int Vs = VnT + DVW * S72 * 2;         //   [64][32] bf16 v of the next chunk (DMA)
    static constexpr int PAIR_BYTES = Vs + CH * DVW * 2;
    static constexpr int BYTES = Pair + PAIRS * PAIR_BYTES;
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x16 mfma32(half8 a, half8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Accumulator registers 8j .. 8j+7 of a 32x32 tile as an fp16 B operand: rows
// 16 j + 8 (s / 4) + 4 (lane / 32) + s % 4 of the tile, the column order of the
// record's T fragments.
__device__ __forceinline__ half8 acc_to_b(const f32x16& a, int j) {
    half8 h;
#pragma unroll
    for (int s = 0; s < 8; ++s) h[s] = (_Float16)a[8 * j + s];
    return h;
}

// fp16 element (row i, column j) of the record's T diag(beta) fragments (zero
// above the 32x32 diagonal blocks); trace dumps only.
__device__ __forceinline__ float rec_t(const char* rec, int i, int j) {
    const int m = i >> 5, kk = j >> 4, jj = j & 15;
    if (m == 0 && kk >= 2) return 0.f;
    const int hh = (jj >> 2) & 1, s = ((jj >> 3) << 2) | (jj & 3);
    const int off = WS_T + frag_lt(m, kk) * WS_FRAG + ((i & 31) + 32 * hh) * 16 + 2 * s;
    return (float)*reinterpret_cast<const _Float16*>(rec + off);
}
// fp16 element (row i, channel c) of the record's -(k e^G) fragments.
__device__ __forceinline__ float rec_kg(const char* rec, int i, int c) {
    const int off = WS_KG + ((i >> 5) * 8 + (c >> 4)) * WS_FRAG + ((i & 31) + 32 * ((c >> 3) & 1)) * 16 + 2 * (c & 7);
    return (float)*reinterpret_cast<const _Float16*>(rec + off);
}

}  // namespace

template <bool TRACE, bool MULTI>
__global__ void __launch_bounds__(SCAN_THREADS, 1) kda_scan_kernel(const ScanJobs J) {
    using L = ScanLds;
    // The job this work-group belongs to, and its index within the job (a single
    // job: job 0, whose parameters then sit at fixed kernel-argument offsets).
    const int jb = !MULTI ? 0 : (blockIdx.x < (unsigned)J.end[0] ? 0 : (blockIdx.x < (unsigned)J.end[1] ? 1 : 2));
    const KdaParams& p = J.job[jb];
    const int bid = (int)blockIdx.x - (jb == 0 ? 0 : J.end[jb - 1]);
    __shared__ __attribute__((aligned(1024))) char smem[L::BYTES];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int pr = (wave >> 1) & 1, role = wave & 1;   // pair; role 0: chain, 1: output (waves 0..3)
    const bool loader = wave >= 4;                   // waves 4, 5: record DMA
    const int hl = lane >> 5, cl = lane & 31;
    char* const ps = smem + L::Pair + pr * L::PAIR_BYTES;   // this pair's LDS

    // Work-group -> (sequence, value head, slice).  The slices of one head go to
    // the same XCD (work-groups are dealt to the 8 XCDs round robin), so their
    // duplicate record reads meet in that XCD's L2.
    const int npairs = p.N * p.Hv;
    int pair, s;
    if ((npairs & 7) == 0) {
        const int x = bid & 7, loc = bid >> 3;
        pair = (loc / SLICES) * 8 + x;
        s = loc % SLICES;
    } else {
        pair = bid / SLICES;
        s = bid % SLICES;
    }
    const int n = pair / p.Hv, hv = pair % p.Hv;
    int64_t bos, len;
    int n_rec;   // the record sequence (equal to n without segments)
    // this sequence's state blocks ([Hv][128][128]; NULL: zero or identity / not written)
    const float* h0b;
    float* hTb;
    if (p.entries) {
        const ScanEntry e = p.entries[n];
        n_rec = e.rec;
        h0b = e.h0;
        hTb = e.hT;
        seq_bounds(p, n_rec, bos, len);
    } else {
        job_seq(p, n, bos, len, n_rec);
        h0b = p.h0 ? p.h0 + (int64_t)n * p.Hv * DK * DK : nullptr;
        hTb = p.hT ? p.hT + (int64_t)n * p.Hv * DK * DK : nullptr;
    }
    const int64_t nch = (len + CH - 1) / CH;
    const int64_t v_tok = (int64_t)p.Hv * DK;   // token stride of v, o
    const int dv0 = (PAIRS * s + pr) * DVW;     // this pair's dv columns
    const int64_t slot0 = chunk_slot(bos, n_rec, 0);   // record slot of chunk c: slot0 + c

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

    auto chunk_rows = [&](int64_t c) -> int {   // valid rows of chunk c (0 past the end)
        const int64_t r = len - c * CH;
        return r <= 0 ? 0 : (r >= CH ? CH : (int)r);
    };

    // ---- record DMA ----
    // Chunk c's record into LDS buffer b, by the two loader waves: 1 KB pieces, lane
    // l's 16 bytes to byte 16 l of a piece; loader 0 takes pieces 0 .. 29, loader 1
    // pieces 30 .. 60.  The loads are issued as inline assembly, so the compiler
    // adds no waits for them; their completion is awaited explicitly (counted)
    // before the barrier that publishes them.  Four consecutive pieces share one write of M0 (the LDS
    // address; writing it stalls the DMA issue): the instruction offset 0, 1 K,
    // 2 K or 3 K moves both the global and the LDS address.  A write of M0 is
    // followed by one other instruction before the DMA that uses it.
    //   Pieces 0 .. 59 lie inside the record, so the scalar offset may carry their
    // position; piece 60 (the last 512 bytes) carries it in the per-lane offset, so
    // that the range check drops its lanes 32 .. 63.  For chunks past the sequence
    // end the range is empty and the DMA writes zeros.
    static_assert(REC_PIECES == 61 && WS_RECORD_BYTES == 60 * WS_FRAG + 512, "record pieces");
    const uint32_t lds_rec = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(smem + L::Rec);
    auto dma_record = [&](int64_t c, int b) {
        const __amdgpu_buffer_rsrc_t r = make_rsrc(p.ws + ((slot0 + c) * p.Hv + hv) * WS_RECORD_BYTES,
                                                   chunk_rows(c) ? WS_RECORD_BYTES : 0);
        const int lr = wave & 1;   // loader 0: pieces 0 .. 29, loader 1: 30 .. 60
        uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_rec + b * REC_LDS + lr * 30 * WS_FRAG);
        uint32_t soff = lr * 30 * WS_FRAG;
        const int vlane = lane * 16;
        // pieces 30 lr .. 30 lr + 29: seven groups of four, then two
        asm volatile(
            "s_mov_b32 m0, %0\n\t"
            "s_nop 0\n\t"
            ".rept 7\n\t"
            "buffer_load_dwordx4 %2, %3, %1 offen lds\n\t"
            "buffer_load_dwordx4 %2, %3, %1 offen offset:1024 lds\n\t"
            "buffer_load_dwordx4 %2, %3, %1 offen offset:2048 lds\n\t"
            "buffer_load_dwordx4 %2, %3, %1 offen offset:3072 lds\n\t"
            "s_add_u32 m0, m0, 4096\n\t"
            "s_add_u32 %1, %1, 4096\n\t"
            ".endr\n\t"
            "buffer_load_dwordx4 %2, %3, %1 offen lds\n\t"
            "buffer_load_dwordx4 %2, %3, %1 offen offset:1024 lds"
            : "+s"(m0), "+s"(soff)
            : "v"(vlane), "s"(r)
            : "memory", "scc");
        if (lr == 1) {   // piece 60
            const uint32_t m60 = __builtin_amdgcn_readfirstlane(lds_rec + b * REC_LDS + 60 * WS_FRAG);
            const int vlast = 60 * WS_FRAG + vlane;
            asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m60), "v"(vlast),
                         "s"(r)
                         : "memory");
        }
    };
    if (loader) {
        // Record loaders: chunk c + 2's record into buffer c % 2 once the first barrier
        // of chunk c has passed (the buffer's last reads came before it); before the
        // second barrier, the record of chunk c + 1 (the older DMA) is complete.
        if (nch > 0) {
            dma_record(0, 0);
            dma_record(1, 1);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        for (int64_t c = 0; c < nch; ++c) {
            lds_barrier();   // first barrier of chunk c
            dma_record(c + 2, (int)(c & 1));
            // all but the DMA just issued (30 loads on loader 0, 31 on loader 1)
            if (wave == 4) asm volatile("s_waitcnt vmcnt(30)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(31)" ::: "memory");
            lds_barrier();   // second barrier of chunk c: chunk c + 1's record complete
        }
        return;
    }
    auto frag = [&](int b, int off) -> half8 {
        return *reinterpret_cast<const half8*>(smem + L::Rec + b * REC_LDS + off + lane * 16);
    };

    // State tiles of this wave: rows (keys) 32 t .. 32 t + 31, t = 2 role + tt, of the
    // pair's slice h[:, dv0 .. dv0 + 31].  Accumulator register r of a tile holds key
    // 32 t + 8 (r / 4) + 4 hl + r % 4, column cl.
    f32x16 hacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) hacc[tt][r] = 0.f;
        if (p.h0_identity) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                hacc[tt][r] = (32 * (2 * role + tt) + 8 * (r >> 2) + 4 * hl + (r & 3) == dv0 + cl) ? 1.f : 0.f;
        } else if (h0b) {
            const float* src = h0b + (int64_t)hv * DK * DK + dv0;
            const int lo = cl + 4 * hl * DK;
#pragma unroll
            for (int r = 0; r < 16; ++r) hacc[tt][r] = src[lo + (32 * (2 * role + tt) + 8 * (r >> 2) + (r & 3)) * DK];
        }
    }
    // fp16 h^T in LDS: this wave's rows, four consecutive keys per 8-byte store.
    auto write_ht = [&]() {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                half4 h4;
#pragma unroll
                for (int e = 0; e < 4; ++e) h4[e] = (_Float16)hacc[tt][4 * q4 + e];
                *reinterpret_cast<half4*>(ps + L::HT + (cl * S136 + 32 * (2 * role + tt) + 8 * q4 + 4 * hl) * 2) = h4;
            }
        }
    };
    // h as MFMA operand, k step kk (keys 16 kk + 8 hl + 0..7 of column cl): the B
    // operand of (k e^G) h and, identically, the A operand of h^T (q e^G)^T.
    half8 hf[8];
    auto read_ht = [&]() {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) hf[kk] = lds_h8(ps, L::HT + (cl * S136 + 16 * kk + 8 * hl) * 2);
    };

    // Z's accumulator layout gathers four consecutive tokens of one column per lane
    // (register 4 q + e of tile m: token 32 m + 8 q + 4 hl + e, column cl).  One
    // transposing LDS read (ds_read_b64_tr_b16) per (m, q) delivers them: in each
    // group of 16 lanes, lane 4 a + b receives element b of the 8-byte pieces
    // addressed by lanes a, a + 4, a + 8, a + 12 of the group, so lane s addresses
    // token 32 m + 8 q + 4 (s / 32) + (s / 4) % 4, columns 16 ((s / 16) % 2) + 4 (s % 4) ..
    const int vs_lane = (4 * (lane >> 5) + ((lane >> 2) & 3)) * DVW + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // v of chunk c (the pair's 32 columns) into the pair's Vs by DMA (chain wave):
    // four 1 KB pieces, lane l of piece u taking token 16 u + l / 4, channels
    // 8 (l % 4) .. + 7, so Vs is row-major [token][32].  Rows past the sequence end
    // fall outside the range and arrive as zeros.
    const uint32_t lds_vs = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)(ps + L::Vs);
    auto dma_v = [&](int64_t c) {
        const int Lc = chunk_rows(c);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + (bos + c * CH) * v_tok + (int64_t)hv * DK + dv0,
                                                    Lc && !p.v_zero ? ((Lc - 1) * v_tok + DVW) * 2 : 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_vs + u * WS_FRAG);
            const int voff = (int)(((16 * u + (lane >> 2)) * v_tok + 8 * (lane & 3)) * 2);
            asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(dst), "v"(voff),
                         "s"(rv)
                         : "memory");
        }
    };

    write_ht();
    if (nch > 0 && role == 0) dma_v(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();   // h^T, the first two records and the first chunk's v complete
    read_ht();

    auto trace_chunk_start = [&](int64_t c, int64_t tok0, int Lc) {
        if (p.tr_h) {
            float* dst = p.tr_h + ((trace_chunk + c) * p.Hv + hv) * DK * DK + dv0 + cl;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    dst[(int64_t)(32 * (2 * role + tt) + 8 * (r >> 2) + 4 * hl + (r & 3)) * DK] = hacc[tt][r];
            }
        }
        // W = T diag(beta) (k e^G) and U = T diag(beta) v from the record's fp16
        // values, element by element (the kernel itself never forms them).
        const char* rec = p.ws + ((slot0 + c) * p.Hv + hv) * WS_RECORD_BYTES;
        if (p.tr_W && s == 0 && pr == 0) {
            for (int it = threadIdx.x & 127; it < CH * DK; it += 128) {
                const int i = it / DK, ch = it % DK;
                if (i >= Lc) continue;
                float acc = 0.f;
                for (int j = 0; j < CH; ++j) acc += rec_t(rec, i, j) * -rec_kg(rec, j, ch);
                p.tr_W[((tok0 + i) * p.Hv + hv) * DK + ch] = acc;
            }
        }
        if (p.tr_U) {
            for (int it = threadIdx.x & 127; it < CH * DVW; it += 128) {
                const int i = it / DVW, d = it % DVW;
                if (i >= Lc) continue;
                float acc = 0.f;
                for (int j = 0; j < Lc; ++j)
                    acc += rec_t(rec, i, j) *
                           (float)(_Float16)bf2f(p.v[(tok0 + j) * v_tok + (int64_t)hv * DK + dv0 + d]);
                p.tr_U[((tok0 + i) * p.Hv + hv) * DK + dv0 + d] = acc;
            }
        }
    };
    // Decay of this wave's state rows by e^{G_last} (from the record in LDS).
    auto decay_state = [&](int b) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 gm = *reinterpret_cast<const f32x4*>(smem + L::Rec + b * REC_LDS + WS_GAM +
                                                                 (32 * (2 * role + tt) + 8 * q4 + 4 * hl) * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) hacc[tt][4 * q4 + e] *= gm[e];
            }
        }
    };
    half8 fkh[8];   // Khat^T fragments of this wave's state rows: (tt, kk) at 4 tt + kk
    half8 vf[4];    // v_new operand, k step kk: tokens 16 kk + 8 hl + 0..7 of column cl
    // After the first barrier: the state update h <- e^{G_last} h + Khat^T v_new of
    // this wave's rows, the fp16 h^T copy, the second barrier.
    auto update_state = [&]() {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) vf[kk] = lds_h8(ps, L::VnT + (cl * S72 + 16 * kk + 8 * hl) * 2);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            hacc[0] = mfma32(fkh[kk], vf[kk], hacc[0]);
            hacc[1] = mfma32(fkh[4 + kk], vf[kk], hacc[1]);
        }
        write_ht();
        lds_barrier();   // h^T and chunk c + 1's record complete; reads of v_new^T and the old h^T done
        read_ht();
    };

    if (role == 0) {
        for (int64_t c = 0; c < nch; ++c) {
            const int64_t tok0 = bos + c * CH;
            const int Lc = chunk_rows(c);
            const int b = (int)(c & 1);
            if (TRACE) trace_chunk_start(c, tok0, Lc);
            decay_state(b);
            // Z = v - (k e^G) h: two token tiles, accumulators starting from v, read from
            // Vs in the accumulator layout (token 32 m + 8 (r / 4) + 4 hl + r % 4,
            // column cl).  This chunk's v (the wave's only memory operations in flight)
            // has landed; once read, Vs is free for the next chunk's v.
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            f32x16 z[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const v4i16 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4i16*)(ps + L::Vs + (vs_lane + (32 * m + 8 * q) * DVW) * 2));
#pragma unroll
                    for (int e = 0; e < 4; ++e) z[m][4 * q + e] = bf2f((uint16_t)t[e]);
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            dma_v(c + 1);
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                z[0] = mfma32(frag(b, WS_KG + kk * WS_FRAG), hf[kk], z[0]);
                z[1] = mfma32(frag(b, WS_KG + (8 + kk) * WS_FRAG), hf[kk], z[1]);
            }
            // v_new = T diag(beta) Z (T lower triangular by 32x32 blocks).
            half8 ft[6];
#pragma unroll
            for (int f = 0; f < 6; ++f) ft[f] = frag(b, WS_T + f * WS_FRAG);
            half8 zb[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) zb[kk] = acc_to_b(z[kk >> 1], kk & 1);
            f32x16 vn[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
                for (int r = 0; r < 16; ++r) vn[m][r] = 0.f;
            }
            vn[0] = mfma32(ft[frag_lt(0, 0)], zb[0], vn[0]);
            vn[1] = mfma32(ft[frag_lt(1, 0)], zb[0], vn[1]);
            vn[0] = mfma32(ft[frag_lt(0, 1)], zb[1], vn[0]);
            vn[1] = mfma32(ft[frag_lt(1, 1)], zb[1], vn[1]);
            vn[1] = mfma32(ft[frag_lt(1, 2)], zb[2], vn[1]);
            vn[1] = mfma32(ft[frag_lt(1, 3)], zb[3], vn[1]);
#pragma unroll
            for (int f = 0; f < 8; ++f) fkh[f] = frag(b, WS_KH + (8 * role + f) * WS_FRAG);
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int i = 32 * m + 8 * q4 + 4 * hl;
                    half4 h4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) h4[e] = (_Float16)vn[m][4 * q4 + e];
                    *reinterpret_cast<half4*>(ps + L::VnT + (cl * S72 + i) * 2) = h4;
                    if (TRACE && p.tr_vnew) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (i + e < Lc) p.tr_vnew[((tok0 + i + e) * p.Hv + hv) * DK + dv0 + cl] = vn[m][4 * q4 + e];
                    }
                }
            }
            lds_barrier();   // v_new^T complete; every read of record buffer b and of v^T done
            update_state();
        }
    } else if (!p.o) {
        // No output (the runs that only produce a segment's state map): this wave
        // keeps its half of the state rows, with the same two barriers per chunk.
        for (int64_t c = 0; c < nch; ++c) {
            const int b = (int)(c & 1);
            decay_state(b);
#pragma unroll
            for (int f = 0; f < 8; ++f) fkh[f] = frag(b, WS_KH + (8 * role + f) * WS_FRAG);
            lds_barrier();   // v_new^T complete; every read of record buffer b and of v^T done
            update_state();
        }
    } else {
        for (int64_t c = 0; c < nch; ++c) {
            const int64_t tok0 = bos + c * CH;
            const int Lc = chunk_rows(c);
            const int b = (int)(c & 1);
            if (TRACE) trace_chunk_start(c, tok0, Lc);
            decay_state(b);
            // o^T = h^T (scale q e^G)^T: needs only the state entering the chunk.
            f32x16 oacc[2];   // o^T tiles (dv column x token), token tiles 0 / 1
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[m][r] = 0.f;
            }
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                oacc[0] = mfma32(hf[kk], frag(b, WS_QG + kk * WS_FRAG), oacc[0]);
                oacc[1] = mfma32(hf[kk], frag(b, WS_QG + (8 + kk) * WS_FRAG), oacc[1]);
            }
            half8 fq[6];   // Aqk fragments, read before the buffer is released
#pragma unroll
            for (int f = 0; f < 6; ++f) fq[f] = frag(b, WS_AQK + f * WS_FRAG);
#pragma unroll
            for (int f = 0; f < 8; ++f) fkh[f] = frag(b, WS_KH + (8 * role + f) * WS_FRAG);
            lds_barrier();   // v_new^T complete; every read of record buffer b and of v^T done
            update_state();
            // o^T += v_new^T Aqk^T (Aqk lower triangular by 32x32 blocks)
            oacc[0] = mfma32(vf[0], fq[frag_lt(0, 0)], oacc[0]);
            oacc[1] = mfma32(vf[0], fq[frag_lt(1, 0)], oacc[1]);
            oacc[0] = mfma32(vf[1], fq[frag_lt(0, 1)], oacc[0]);
            oacc[1] = mfma32(vf[1], fq[frag_lt(1, 1)], oacc[1]);
            oacc[1] = mfma32(vf[2], fq[frag_lt(1, 2)], oacc[1]);
            oacc[1] = mfma32(vf[3], fq[frag_lt(1, 3)], oacc[1]);
            // o^T tile m: register r holds channel 8 (r / 4) + 4 hl + r % 4, token 32 m + cl.
            uint16_t* obase = p.o + tok0 * v_tok + (int64_t)hv * DK + dv0;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int i = 32 * m + cl;
                if (i < Lc) {
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        uint2 w;
                        w.x = pack_bf2(oacc[m][4 * q4], oacc[m][4 * q4 + 1]);
                        w.y = pack_bf2(oacc[m][4 * q4 + 2], oacc[m][4 * q4 + 3]);
                        *reinterpret_cast<uint2*>(obase + i * v_tok + 8 * q4 + 4 * hl) = w;
                    }
                }
            }
        }
    }

    // ---- final state ----
    if (hTb) {
        // The lane offset is recomputed here from an opaque copy of the lane index,
        // so that it is not kept live (with the h0 addresses) through the chunk loop.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        float* dst = hTb + (int64_t)hv * DK * DK + dv0;
        const int lo = (ln & 31) + 4 * (ln >> 5) * DK;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) dst[lo + (32 * (2 * role + tt) + 8 * (r >> 2) + (r & 3)) * DK] = hacc[tt][r];
        }
    }
}

// Fills the jobs' work-group ranges; returns the grid size (0: nothing to run, -1: too large).
static int64_t job_ranges(ScanJobs& J) {
    int64_t total = 0;
    for (int j = 0; j < MAX_SCAN_JOBS; ++j) {
        if (j < J.njobs) total += (int64_t)J.job[j].N * J.job[j].Hv * SLICES;
        if (total > INT32_MAX) return -1;
        J.end[j] = (int32_t)total;
    }
    return total;
}

template <bool TRACE, bool MULTI>
static hipError_t launch(const ScanJobs& J, int nblocks, hipStream_t stream) {
    hipLaunchKernelGGL((kda_scan_kernel<TRACE, MULTI>), dim3(nblocks), dim3(SCAN_THREADS), 0, stream, J);
    return hipGetLastError();
}

int scan_slices() { return SLICES; }

hipError_t launch_kda_scan(const KdaParams& p, bool trace, hipStream_t stream) {
    ScanJobs J{};
    J.job[0] = p;
    J.njobs = 1;
    const int64_t nblocks = job_ranges(J);
    if (nblocks <= 0) return nblocks == 0 ? hipSuccess : hipErrorInvalidValue;
    return trace ? launch<true, false>(J, (int)nblocks, stream) : launch<false, false>(J, (int)nblocks, stream);
}

hipError_t launch_kda_scan_jobs(ScanJobs J, hipStream_t stream) {
    if (J.njobs < 1 || J.njobs > MAX_SCAN_JOBS) return hipErrorInvalidValue;
    const int64_t nblocks = job_ranges(J);
    if (nblocks <= 0) return nblocks == 0 ? hipSuccess : hipErrorInvalidValue;
    return launch<false, true>(J, (int)nblocks, stream);
}

}  // namespace kda

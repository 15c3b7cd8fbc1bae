// Composition of per-segment affine state maps, for the segmented (context
// parallel) forward on gfx950.
//
// Over one segment of a sequence the chunked recurrence is affine in the state
// that enters it: h_out = M h_in + b, where M is the segment's state map (the
// product of its chunks' maps diag(e^{G_last}) - Khat^T W, taken from the
// identity with v = 0) and b the state the segment reaches from zero.  Once
// every segment's (M, b) is known, the true entering states follow in order,
// h_in[s + 1] = M[s] h_in[s] + b[s]: a short serial chain of 128 x 128 products
// per (row, value head), independent across the columns of h.  One work-group
// per (row, value head, 8 columns) runs the chain in fp32, with h's columns and
// the step's M in LDS and each thread accumulating one row of four columns over
// the 128 keys in a fixed order (results are bitwise repeatable).
#include "kda_device.h"

namespace kda {

namespace {

constexpr int CMP_THREADS = 256;   // 128 rows x 2 groups of 4 columns
constexpr int CMP_COLS = 8;        // columns per work-group
constexpr int CMP_GROUPS = DK / CMP_COLS;
constexpr int MS = DK + 4;         // padded LDS row of M (floats): rows 16 apart share banks
constexpr int M_LOADS = DK * DK / 4 / CMP_THREADS;   // 16-byte pieces of M per thread

}  // namespace

// One step's M moves into LDS in two halves of the step: each thread loads its 16
// pieces (consecutive threads, consecutive 16 bytes) while the previous step's
// products run, and writes them to the other LDS buffer afterwards.
// With `chains` (packed sequences), row n is chain n: its steps read M and b from
// index chains[4 n] on and its states from index chains[4 n + 1] on, each index
// one [Hv][128][128] block, for chains[4 n + 2] steps (`nsteps` is ignored).
__global__ void __launch_bounds__(CMP_THREADS) kda_compose_kernel(const float* M, const float* b, float* h, int rows,
                                                                 int Hv, int nsteps, const int32_t* chains) {
    __shared__ __attribute__((aligned(16))) float sM[2][DK * MS];   // M of two steps
    __shared__ f32x4 sh[DK][CMP_COLS / 4];                          // the current h columns
    const int item = (int)(blockIdx.x / CMP_GROUPS);   // row * Hv + value head
    const int col0 = (int)(blockIdx.x % CMP_GROUPS) * CMP_COLS;
    const int t = threadIdx.x, i = t >> 1, jq = t & 1;   // output row i, columns col0 + 4 jq .. + 3
    const int64_t head = (int64_t)DK * DK;
    int64_t seg = (int64_t)rows * Hv * head;
    int64_t me = (int64_t)item * head + (int64_t)i * DK + col0 + 4 * jq;
    if (chains) {
        const int n = item / Hv, hv = item % Hv;
        const int64_t ms = chains[4 * n], ls = chains[4 * n + 1];
        nsteps = chains[4 * n + 2];
        if (nsteps <= 0) return;   // (uniform per work-group)
        seg = (int64_t)Hv * head;
        M += ms * seg;
        b += ms * seg;
        h += ls * seg;
        me = (int64_t)hv * head + (int64_t)i * DK + col0 + 4 * jq;
    }

    f32x4 r[M_LOADS];
    auto load_m = [&](int s) {
        const float* src = M + s * seg + (me - (int64_t)i * DK - col0 - 4 * jq);
#pragma unroll
        for (int e = 0; e < M_LOADS; ++e) r[e] = *reinterpret_cast<const f32x4*>(src + 4 * (t + CMP_THREADS * e));
    };
    auto store_m = [&](int buf) {
#pragma unroll
        for (int e = 0; e < M_LOADS; ++e) {
            const int idx = t + CMP_THREADS * e;   // piece idx: row idx / 32, columns 4 (idx % 32) ..
            *reinterpret_cast<f32x4*>(&sM[buf][(idx >> 5) * MS + 4 * (idx & 31)]) = r[e];
        }
    };

    sh[i][jq] = *reinterpret_cast<const f32x4*>(h + me);
    if (nsteps > 0) {
        load_m(0);
        store_m(0);
    }
    __syncthreads();
    for (int s = 0; s < nsteps; ++s) {
        if (s + 1 < nsteps) load_m(s + 1);   // in flight during this step's products
        f32x4 acc = *reinterpret_cast<const f32x4*>(b + s * seg + me);
        const float* Mrow = &sM[s & 1][i * MS];
#pragma unroll 8
        for (int k4 = 0; k4 < DK / 4; ++k4) {
            const f32x4 m4 = *reinterpret_cast<const f32x4*>(Mrow + 4 * k4);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc += m4[e] * sh[4 * k4 + e][jq];
        }
        __syncthreads();   // every read of the old columns and of this step's M is done
        sh[i][jq] = acc;
        *reinterpret_cast<f32x4*>(h + (s + 1) * seg + me) = acc;
        if (s + 1 < nsteps) store_m((s + 1) & 1);
        __syncthreads();
    }
}

hipError_t launch_kda_compose(const float* M, const float* b, float* h_in, int rows, int Hv, int nsteps,
                              hipStream_t stream) {
    const int64_t nblocks = (int64_t)rows * Hv * CMP_GROUPS;
    if (nblocks == 0 || nsteps <= 0) return hipSuccess;
    if (nblocks > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kda_compose_kernel, dim3((unsigned)nblocks), dim3(CMP_THREADS), 0, stream, M, b, h_in, rows, Hv,
                       nsteps, (const int32_t*)nullptr);
    return hipGetLastError();
}

hipError_t launch_kda_compose_chains(const float* M, const float* b, float* h_in, const int32_t* chains, int nchains,
                                     int Hv, hipStream_t stream) {
    const int64_t nblocks = (int64_t)nchains * Hv * CMP_GROUPS;
    if (nblocks == 0) return hipSuccess;
    if (nblocks > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kda_compose_kernel, dim3((unsigned)nblocks), dim3(CMP_THREADS), 0, stream, M, b, h_in, nchains,
                       Hv, 0, chains);
    return hipGetLastError();
}

// Plan of the segmented forward over packed sequences (one work-group; the host
// never reads cu_seqlens).  Sequence n (tokens [a, e), clamped to [0, T)) has
// nch = ceil((e - a) / 64) chunks and P = 1 segment if nch <= L0, else
// 1 + ceil((nch - L0) / L): segment 0 of L0 chunks, the others of L (the last may
// be shorter).  Segments get global indices in token order; segment j of sequence
// n starts at a (j = 0) or a + 64 (L0 + (j - 1) L).  Later segments (j >= 1) and
// middle segments (1 <= j <= P - 2) are numbered by prefix sums over the
// sequences, so each sequence's are consecutive.
// Two phases: per sequence (rounds of 256, prefix sums across the round) the
// counts, segment 0's entry and the chain; then per segment (all threads, the
// owning sequence found by binary search over the first-segment indices) the
// boundary and the later / middle entries, so one long sequence does not leave
// the work to one thread.  List entries past the totals point at the empty
// segment S_max and write nothing.  Every index is checked against the sizes the
// host planned for: with well-formed cu_seqlens they always fit; with malformed
// ones (overlapping sequences) the results are undefined but every access stays
// in bounds.
__global__ void __launch_bounds__(256) kda_cp_plan_kernel(const CpPlan pl) {
    __shared__ int s_cnt[3][256];
    __shared__ int s_carry[3];
    const int t = threadIdx.x;
    if (t < 3) s_carry[t] = 0;
    __syncthreads();
    auto bounds = [&](int n, int64_t& a, int64_t& e) {
        a = pl.cu[n];
        e = pl.cu[n + 1];
        a = a < 0 ? 0 : (a > pl.T ? pl.T : a);
        e = e < a ? a : (e > pl.T ? pl.T : e);
    };
    const int64_t hd = pl.hv_dd;
    // ---- phase 1: per sequence ----
    for (int base = 0; base < pl.N; base += 256) {
        const int n = base + t;
        int P = 0;
        if (n < pl.N) {
            int64_t a, e;
            bounds(n, a, e);
            const int64_t nch = (e - a + CH - 1) / CH;
            P = nch <= pl.L0 ? 1 : (int)(1 + (nch - pl.L0 + pl.L - 1) / pl.L);
        }
        const int later = P > 0 ? P - 1 : 0, mid = P > 1 ? P - 2 : 0;
        s_cnt[0][t] = P;
        s_cnt[1][t] = later;
        s_cnt[2][t] = mid;
        __syncthreads();
        // inclusive prefix sums over the 256 sequences of this round (Hillis-Steele)
        for (int d = 1; d < 256; d <<= 1) {
            int v[3];
            for (int q = 0; q < 3; ++q) v[q] = t >= d ? s_cnt[q][t - d] : 0;
            __syncthreads();
            for (int q = 0; q < 3; ++q) s_cnt[q][t] += v[q];
            __syncthreads();
        }
        const int segb = s_carry[0] + s_cnt[0][t] - P;
        const int ls = s_carry[1] + s_cnt[1][t] - later;
        const int ms = s_carry[2] + s_cnt[2][t] - mid;
        if (n < pl.N) {
            ScanEntry f;
            f.rec = segb <= pl.S_max ? segb : pl.S_max;
            f.pad = 0;
            f.h0 = pl.h0 ? pl.h0 + (int64_t)n * hd : nullptr;
            f.hT = P >= 2 ? (ls < pl.lat_max ? pl.Hin + (int64_t)ls * hd : nullptr)
                          : (pl.hT ? pl.hT + (int64_t)n * hd : nullptr);
            pl.first[n] = f;
            int steps = mid;
            if (ms + steps > pl.lat_max) steps = pl.lat_max - ms;
            if (ls + steps + 1 > pl.lat_max) steps = pl.lat_max - ls - 1;
            pl.chains[4 * n] = ms;
            pl.chains[4 * n + 1] = ls;
            pl.chains[4 * n + 2] = steps > 0 ? steps : 0;
            pl.chains[4 * n + 3] = segb;   // first segment (for phase 2)
        }
        __syncthreads();
        if (t == 255) {
            s_carry[0] += s_cnt[0][255];
            s_carry[1] += s_cnt[1][255];
            s_carry[2] += s_cnt[2][255];
        }
        __syncthreads();
    }
    const int S_total = s_carry[0];
    // ---- phase 2: per segment ----
    const int S_lim = S_total < pl.S_max + 2 ? S_total : pl.S_max + 2;
    for (int sg = t; sg < S_lim; sg += 256) {
        int lo = 0, hi = pl.N - 1;   // the last sequence whose first segment is <= sg
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pl.chains[4 * mid + 3] <= sg) lo = mid; else hi = mid - 1;
        }
        const int n = lo, segb = pl.chains[4 * n + 3];
        const int P = (n + 1 < pl.N ? pl.chains[4 * (n + 1) + 3] : S_total) - segb;
        const int ms = pl.chains[4 * n], ls = pl.chains[4 * n + 1];
        const int j = sg - segb;
        int64_t a, e;
        bounds(n, a, e);
        const int64_t st = j == 0 ? a : a + (int64_t)CH * (pl.L0 + (int64_t)(j - 1) * pl.L);
        pl.cu_seg[sg] = (int32_t)(st < e ? st : e);
        const int rec = sg <= pl.S_max ? sg : pl.S_max;
        if (j >= 1 && ls + j - 1 < pl.lat_max) {
            ScanEntry l;
            l.rec = rec;
            l.pad = 0;
            l.h0 = pl.Hin + (int64_t)(ls + j - 1) * hd;
            l.hT = (j == P - 1 && pl.hT) ? pl.hT + (int64_t)n * hd : nullptr;
            pl.later[ls + j - 1] = l;
        }
        if (j >= 1 && j + 1 < P && ms + j - 1 < pl.lat_max) {
            ScanEntry m;
            m.rec = rec;
            m.pad = 0;
            m.h0 = nullptr;
            m.hT = pl.Mb + (int64_t)(ms + j - 1) * hd;
            pl.mid_m[ms + j - 1] = m;
            m.hT = pl.Bb + (int64_t)(ms + j - 1) * hd;
            pl.mid_b[ms + j - 1] = m;
        }
    }
    // The end of the last segment, the empty padding segments, and the padding
    // entries of the lists.
    const int S = S_total < pl.S_max ? S_total : pl.S_max;
    const int LT = s_carry[1] < pl.lat_max ? s_carry[1] : pl.lat_max;
    const int MD = s_carry[2] < pl.lat_max ? s_carry[2] : pl.lat_max;
    int64_t end = pl.N > 0 ? pl.cu[pl.N] : 0;
    end = end < 0 ? 0 : (end > pl.T ? pl.T : end);
    __syncthreads();   // (phase 2's boundary writes come first: S_total may exceed S)
    for (int x = S + t; x <= pl.S_max + 1; x += 256)
        if (x >= S_total) pl.cu_seg[x] = (int32_t)end;
    ScanEntry z;
    z.rec = pl.S_max;
    z.pad = 0;
    z.h0 = nullptr;
    z.hT = nullptr;
    for (int x = LT + t; x < pl.lat_max; x += 256) pl.later[x] = z;
    for (int x = MD + t; x < pl.lat_max; x += 256) {
        pl.mid_m[x] = z;
        pl.mid_b[x] = z;
    }
}

hipError_t launch_kda_cp_plan(const CpPlan& pl, hipStream_t stream) {
    hipLaunchKernelGGL(kda_cp_plan_kernel, dim3(1), dim3(256), 0, stream, pl);
    return hipGetLastError();
}

}  // namespace kda

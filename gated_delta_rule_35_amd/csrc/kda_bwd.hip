// KDA backward pass on gfx950 (MI355X): gradients of the chunked forward with
// respect to q, k, v, g, beta and the initial state, for fixed-length batches and
// for sequences packed into one row (cu_seqlens).
//
// The pages list chunk backward kernels beside the forward ("cuLA REPO_LAYOUT.md",
// the kda/ entries for chunk_bwd and the WY dq/dk/dg kernels) but give no
// equation; these are the forward's chunk equations differentiated.  Per
// 64-token chunk of one (sequence, value head), with h the state entering it,
// G the chunk-local inclusive cumsum of g, kg = k e^G, qg = scale q e^G,
// kh = k e^(G_last - G), gam = e^G_last, Aqk[i][j] = scale sum_c q_i k_j
// e^(G_i - G_j) (j <= i), Abar[i][j] = sum_c k_i k_j e^(G_i - G_j) (j < i),
// T = (I + diag(beta) Abar)^-1 and Tb = T diag(beta), the forward is
//
//   Z = v - kg h,  v_new = Tb Z,  o = qg h + Aqk v_new,  h' = gam * h + kh^T v_new
//
// and, for given do and dh' (the gradient of the state leaving the chunk),
//
//   dv_new = Aqk^T do + kh dh',  dZ = Tb^T dv_new,  dv = dZ,
//   dh     = gam * dh' + qg^T do - kg^T dZ,
//
// with the operand gradients d(qg) = do h^T, d(kg) = -dZ h^T, d(kh) = v_new dh'^T,
// dAqk = lower(do v_new^T), dTb = dv_new Z^T, dgam = rowsum(dh' * h), taken back to
// q, k, beta and g through their definitions (dA = -T^T dT T^T on the strict lower
// triangle, and dg the reverse cumsum of dG within the chunk).
//
// Five kernels, all in fp32: the contractions on v_mfma_f32_16x16x4f32 (fp32
// operands, fp32 accumulation), the rest on the vector ALUs, operands in LDS:
//   prep    one work-group per (chunk, value head): G, Aqk, Abar and T
//   states  one per (sequence, value head, 32 value columns): walks the chunks
//           forward and stores each chunk's entering state h
//   dstate  the same grid, walking the chunks backward: stores each chunk's dh'
//           and writes the initial state's gradient
//   grad    one per (chunk, value head): dv, dbeta, and dq, dk, dg per value head
//   group   sums dq and dk over the value heads that share a q/k head
// The decay factors e^{G_i - G_j} of Aqk, Abar and the pairwise gradient sums are
// split at a per-channel anchor A = G_last / 2 (e^{G_i - A} e^{A - G_j}), so those
// sums become MFMA products; a chunk that decays by more than e^-120 on some channel
// (factors beyond e^60) is summed element by element instead.  Every output element
// has one writer and a fixed summation order, so results are bitwise reproducible.
#include "kda_device.h"

namespace kda {

namespace {

constexpr int BW_C = 64;      // chunk length
constexpr int BW_D = 128;     // head dimension
constexpr int BW_LD = 129;    // row stride of [64][128] LDS tiles: odd, so a column read across rows spreads over banks
constexpr int BW_MD = 65;     // row stride of [64][64] LDS tiles
constexpr int GLD = 132;      // row stride of [64][128] tiles read along rows with 16-byte loads
constexpr int BW_SL = 32;     // value columns per scan work-group
constexpr int BW_SD = 36;     // row stride of [*][32] LDS tiles: a multiple of 4 for 16-byte reads
constexpr int BW_NSL = BW_D / BW_SL;
constexpr int BW_ST = 512;    // threads of a scan work-group: row c = t % 128, columns 8 (t / 128) .. + 7
constexpr int GSL = 16;       // value columns per step of the grad kernel's slice loop
constexpr int GSD = 17;       // row stride of [*][16] LDS tiles
constexpr int GNSL = BW_D / GSL;
constexpr int64_t BW_STATE = (int64_t)BW_D * BW_D;

__device__ __forceinline__ f32x4 lds4(const float* a) { return *reinterpret_cast<const f32x4*>(a); }

__device__ __forceinline__ float ld_beta(const BwdParams& p, int64_t idx) {
    return p.beta_f32 ? static_cast<const float*>(p.beta)[idx] : bf2f(static_cast<const uint16_t*>(p.beta)[idx]);
}

struct ChunkIdx {
    int b, ci, hv, hq, len;   // b: the chunk's token row (0 for packed sequences); len 0: no chunk
    int64_t t0, ch;   // first token of the chunk within its row; (chunk slot, value head) index
};

// Token range of packed sequence n, [cu[n], cu[n+1]) clamped to [0, T), so that
// malformed offsets can never send an access out of bounds.
__device__ __forceinline__ void packed_seq(const BwdParams& p, int n, int64_t& bos, int64_t& len) {
    int64_t a = p.cu[n], e = p.cu[n + 1];
    a = a < 0 ? 0 : (a > p.T ? p.T : a);
    e = e < a ? a : (e > p.T ? p.T : e);
    bos = a;
    len = e - a;
}

// Chunk ci of packed sequence n (first token bos, len tokens) in value head hv.  Its
// slot is floor(bos / 64) + n + ci: slots of different chunks differ whenever the
// sequences do not overlap, and all lie below ceil(T / 64) + N.
__device__ __forceinline__ ChunkIdx packed_chunk(const BwdParams& p, int n, int64_t bos, int64_t len, int64_t ci,
                                                 int hv) {
    ChunkIdx x;
    x.hv = hv;
    x.hq = hv / (p.Hv / p.Hq);
    x.b = 0;
    x.ci = (int)ci;
    x.t0 = bos + ci * BW_C;
    const int64_t rest = len - ci * BW_C;
    x.len = rest <= 0 ? 0 : (rest < BW_C ? (int)rest : BW_C);
    x.ch = (bos / BW_C + n + ci) * p.Hv + hv;
    return x;
}

// Work-group index of a (chunk, value head) grid.  Fixed-length rows:
// blk = (b * nc + ci) * Hv + hv.  Packed sequences: blk = slot * Hv + hv, the
// sequence found by bisection (the first slot of sequence n, floor(bos_n / 64) + n,
// grows with n); a slot that holds no chunk comes back with len = 0.
__device__ __forceinline__ ChunkIdx chunk_of(const BwdParams& p, int64_t blk) {
    const int hv = (int)(blk % p.Hv);
    const int64_t cid = blk / p.Hv;
    if (p.cu) {
        int lo = 0, hi = p.N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            int64_t b0, l0;
            packed_seq(p, mid, b0, l0);
            if (b0 / BW_C + mid <= cid) lo = mid; else hi = mid - 1;
        }
        int64_t bos, len;
        packed_seq(p, lo, bos, len);
        return packed_chunk(p, lo, bos, len, cid - (bos / BW_C + lo), hv);
    }
    ChunkIdx x;
    x.hv = hv;
    x.b = (int)(cid / p.nc);
    x.ci = (int)(cid % p.nc);
    x.hq = x.hv / (p.Hv / p.Hq);
    x.t0 = (int64_t)x.ci * BW_C;
    const int64_t rest = p.T - x.t0;
    x.len = rest < BW_C ? (int)rest : BW_C;
    x.ch = blk;
    return x;
}

// The state walks' view of sequence n: its chunk count, and chunk ci of it.
struct SeqWalk {
    int64_t bos, len;
    int nc;
};
__device__ __forceinline__ SeqWalk seq_walk(const BwdParams& p, int n) {
    SeqWalk w{0, 0, p.nc};
    if (p.cu) {
        packed_seq(p, n, w.bos, w.len);
        w.nc = (int)((w.len + BW_C - 1) / BW_C);
    }
    return w;
}
__device__ __forceinline__ ChunkIdx walk_chunk(const BwdParams& p, const SeqWalk& w, int n, int ci, int hv) {
    return p.cu ? packed_chunk(p, n, w.bos, w.len, ci, hv) : chunk_of(p, ((int64_t)n * p.nc + ci) * p.Hv + hv);
}

__device__ __forceinline__ int64_t qk_off(const BwdParams& p, int b, int64_t t, int hq) {
    return (((int64_t)b * p.T + t) * p.Hq + hq) * BW_D;
}
__device__ __forceinline__ int64_t vh_off(const BwdParams& p, int b, int64_t t, int hv) {
    return (((int64_t)b * p.T + t) * p.Hv + hv) * BW_D;
}

// ---------------------------------------------------------------- prep
// q and k stay bf16 in LDS (exact: they are bf16 inputs), and Abar and T reuse
// their space once the pairwise products are done, so that two work-groups fit
// on a CU.
constexpr int BW_PT = 512;   // threads of the prep work-group
constexpr int PQ_LD = 136;   // row stride (bf16 elements) of the q / k tiles: 8-byte aligned rows
struct PrepLds {
    union {
        struct {
            uint16_t q[BW_C * PQ_LD], k[BW_C * PQ_LD];
        } in;
        struct {
            float A[BW_C * BW_MD], T[BW_C * BW_MD];
        } out;
    } u;
    float G[BW_C * GLD];
    float beta[BW_C];
};

__device__ __forceinline__ f32x4 lds_bf4(const uint16_t* a) {
    const uint2 w = *reinterpret_cast<const uint2*>(a);
    return f32x4{bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y)};
}

__global__ void __launch_bounds__(BW_PT, 2) kda_bwd_prep_kernel(const BwdParams p) {
    __shared__ __attribute__((aligned(16))) PrepLds L;
    const int tid = threadIdx.x;
    const ChunkIdx x = chunk_of(p, blockIdx.x);
    if (x.len == 0) return;   // a slot that holds no chunk (uniform per work-group)
    {
        // thread t: channels 4 (t % 32) .. + 3 of rows t / 32 + 16 v; rows past the
        // sequence's end: q = k = 0, g = 0
        const int c4 = 4 * (tid & 31);
        for (int v = 0; v < 4; ++v) {
            const int i = (tid >> 5) + 16 * v;
            uint2 qw = make_uint2(0u, 0u), kw = make_uint2(0u, 0u);
            f32x4 gv = {0.f, 0.f, 0.f, 0.f};
            if (i < x.len) {
                const int64_t t = x.t0 + i;
                qw = *reinterpret_cast<const uint2*>(p.q + qk_off(p, x.b, t, x.hq) + c4);
                kw = *reinterpret_cast<const uint2*>(p.k + qk_off(p, x.b, t, x.hq) + c4);
                gv = *reinterpret_cast<const f32x4*>(p.g + vh_off(p, x.b, t, x.hv) + c4);
            }
            *reinterpret_cast<uint2*>(L.u.in.q + i * PQ_LD + c4) = qw;
            *reinterpret_cast<uint2*>(L.u.in.k + i * PQ_LD + c4) = kw;
            *reinterpret_cast<f32x4*>(L.G + i * GLD + c4) = gv;
        }
    }
    if (tid < BW_C) L.beta[tid] = tid < x.len ? ld_beta(p, ((int64_t)x.b * p.T + x.t0 + tid) * p.Hv + x.hv) : 0.f;
    __syncthreads();
    if (tid < BW_D) {   // chunk-local inclusive cumsum; padded rows repeat the last valid G
        float run = 0.f;
        for (int i = 0; i < BW_C; ++i) {
            run += L.G[i * GLD + tid];
            L.G[i * GLD + tid] = run;
        }
    }
    __syncthreads();
    float* pr = p.prep + x.ch * BWP_FLOATS;
    for (int e = tid; e < BW_C * BW_D; e += BW_PT) pr[BWP_G + e] = L.G[(e >> 7) * GLD + (e & 127)];
    // Aqk (j <= i) and Abar (j < i).  With the anchor A = G_last / 2 of each channel,
    // e^{G_i - G_j} = e^{G_i - A} e^{A - G_j} and every factor lies within
    // e^{+-|G_last| / 2}: Aqk = scale (q e^{G-A}) (k e^{A-G})^T and Abar = (k e^{G-A})
    // (k e^{A-G})^T on v_mfma_f32_16x16x4f32.  A chunk that decays by more than e^-120
    // on some channel (factors beyond e^60) takes the element-by-element sums.
    float abar[BW_C * BW_C / BW_PT];
    const bool far = __syncthreads_or(tid < BW_D && !(L.G[(BW_C - 1) * GLD + tid] >= -120.f)) != 0;
    if (!far) {
        // This thread's 16 elements (row e / 128, channel e % 128, e = tid + 512 u).
        float qa[16], ka[16], kb[16];
        for (int u = 0; u < 16; ++u) {
            const int e = tid + BW_PT * u, i = e >> 7, c = e & 127;
            const float G = L.G[i * GLD + c], A = 0.5f * L.G[(BW_C - 1) * GLD + c];
            const float eP = fexp(G - A), eM = fexp(A - G);
            const float kv = bf2f(L.u.in.k[i * PQ_LD + c]);
            qa[u] = bf2f(L.u.in.q[i * PQ_LD + c]) * eP;
            ka[u] = kv * eM;
            kb[u] = kv * eP;
        }
        __syncthreads();   // q, k and G are read: q e^{G-A} goes over G, k e^{A-G} over q and k
        float* X = L.G;
        float* Y = reinterpret_cast<float*>(&L.u);
        static_assert(BW_C * GLD * 4 <= sizeof(L.u), "anchored operand over q and k");
        for (int u = 0; u < 16; ++u) {
            const int e = tid + BW_PT * u, i = e >> 7, c = e & 127;
            X[i * GLD + c] = qa[u];
            Y[i * GLD + c] = ka[u];
        }
        // zeros of the tiles above the diagonal (the products below write the rest)
        for (int s = 0; s < BW_C * BW_C / BW_PT; ++s) {
            const int e = tid + BW_PT * s, i = e >> 6, j = e & 63;
            if ((j >> 4) > (i >> 4)) {
                pr[BWP_AQK + e] = 0.f;
                pr[BWP_ABAR + e] = 0.f;
            }
        }
        __syncthreads();
        // Wave w: the lower-triangle tiles w and w + 8 (row-major order over (it, jt),
        // jt <= it).  MFMA b of channel block u sums channel 16 u + 4 (lane / 16) + b.
        const int lane = tid & 63, wv = tid >> 6, m4 = 4 * (lane >> 4), rl = lane & 15;
        auto tile_of = [](int t, int& ti, int& tj) {
            ti = t >= 6 ? 3 : (t >= 3 ? 2 : (t >= 1 ? 1 : 0));
            tj = t - ti * (ti + 1) / 2;
        };
        auto product = [&](const float* Aop, int ti, int tj) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
            for (int u = 0; u < BW_D / 16; ++u) {
                const f32x4 a4 = lds4(Aop + (16 * ti + rl) * GLD + 16 * u + m4);
                const f32x4 b4 = lds4(Y + (16 * tj + rl) * GLD + 16 * u + m4);
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[bb], b4[bb], acc, 0, 0, 0);
            }
            return acc;
        };
        const int ntile = wv + 8 < 10 ? 2 : 1;
        for (int k = 0; k < ntile; ++k) {
            int ti, tj;
            tile_of(wv + 8 * k, ti, tj);
            const f32x4 acc = product(X, ti, tj);
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * ti + m4 + r, j = 16 * tj + rl;
                pr[BWP_AQK + i * BW_C + j] = j <= i ? p.scale * acc[r] : 0.f;
            }
        }
        __syncthreads();   // q e^{G-A} is read: k e^{G-A} replaces it
        for (int u = 0; u < 16; ++u) {
            const int e = tid + BW_PT * u;
            X[(e >> 7) * GLD + (e & 127)] = kb[u];
        }
        __syncthreads();
        f32x4 accb[2];
        for (int k = 0; k < ntile; ++k) {
            int ti, tj;
            tile_of(wv + 8 * k, ti, tj);
            accb[k] = product(X, ti, tj);
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * ti + m4 + r, j = 16 * tj + rl;
                if (j >= i) accb[k][r] = 0.f;
                pr[BWP_ABAR + i * BW_C + j] = accb[k][r];
            }
        }
        __syncthreads();   // the operands are read: Abar goes to L.u.out.A
        for (int s = 0; s < BW_C * BW_C / BW_PT; ++s) {   // zeros above the diagonal tiles
            const int e = tid + BW_PT * s, i = e >> 6, j = e & 63;
            if ((j >> 4) > (i >> 4)) L.u.out.A[i * BW_MD + j] = 0.f;
        }
        for (int k = 0; k < ntile; ++k) {
            int ti, tj;
            tile_of(wv + 8 * k, ti, tj);
            for (int r = 0; r < 4; ++r) L.u.out.A[(16 * ti + m4 + r) * BW_MD + 16 * tj + rl] = accb[k][r];
        }
        __syncthreads();
    } else {
        // one wave per row i, lane j, four channels per LDS read
        for (int s = 0; s < BW_C * BW_C / BW_PT; ++s) {
            const int e = tid + BW_PT * s, i = e >> 6, j = e & 63;
            float aq = 0.f, ak = 0.f;
            if (j <= i) {
#pragma unroll 4
                for (int c = 0; c < BW_D; c += 4) {
                    const f32x4 gi = lds4(L.G + i * GLD + c), gj = lds4(L.G + j * GLD + c);
                    const f32x4 kj = lds_bf4(L.u.in.k + j * PQ_LD + c);
                    const f32x4 qi = lds_bf4(L.u.in.q + i * PQ_LD + c), ki = lds_bf4(L.u.in.k + i * PQ_LD + c);
                    for (int u = 0; u < 4; ++u) {
                        const float d = fexp(gi[u] - gj[u]) * kj[u];
                        aq += qi[u] * d;
                        ak += ki[u] * d;
                    }
                }
                if (j == i) ak = 0.f;
            }
            pr[BWP_AQK + e] = p.scale * aq;
            pr[BWP_ABAR + e] = ak;
            abar[s] = ak;
        }
        __syncthreads();   // q and k are dead: Abar and T take their space
        for (int s = 0; s < BW_C * BW_C / BW_PT; ++s) {
            const int e = tid + BW_PT * s;
            L.u.out.A[(e >> 6) * BW_MD + (e & 63)] = abar[s];
        }
        __syncthreads();
    }
    // T = (I + diag(beta) Abar)^-1 by forward substitution: lane j owns column j,
    // T[i][j] = delta_ij - beta_i sum_{m < i} Abar[i][m] T[m][j] (T[m][j] = 0 for m < j).
    // Rows go in blocks of 16: the columns m of earlier blocks are summed into the
    // block's 16 running sums (independent chains), then each finished row of the
    // block is added into the later rows' sums; every sum runs over m in increasing
    // order.
    if (tid < BW_C) {
        const int j = tid;
        for (int I = 0; I < BW_C / 16; ++I) {
            float sacc[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
            for (int m = 0; m < 16 * I; ++m) {
                const float tm = L.u.out.T[m * BW_MD + j];
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[r] += L.u.out.A[(16 * I + r) * BW_MD + m] * tm;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 16 * I + r;
                const float tm = m == j ? 1.f : (m > j ? -L.beta[m] * sacc[r] : 0.f);
                L.u.out.T[m * BW_MD + j] = tm;
                pr[BWP_T + m * BW_C + j] = tm;
#pragma unroll
                for (int r2 = r + 1; r2 < 16; ++r2) sacc[r2] += L.u.out.A[(16 * I + r2) * BW_MD + m] * tm;
            }
        }
    }
}

// The chunk's decayed key operands k e^G and k e^{G_last - G} into LDS ([64][ld]):
// thread t takes channels 4 (t % 32) .. + 3 of rows t / 32 + 16 v (v < 4), with 8- and
// 16-byte loads.
__device__ __forceinline__ void load_key_ops(const BwdParams& p, const ChunkIdx& x, const float* pr, float* sKG,
                                             float* sKH, int tid, int ld) {
    const int c4 = 4 * (tid & 31);
    const f32x4 Gl = *reinterpret_cast<const f32x4*>(pr + BWP_G + (BW_C - 1) * BW_D + c4);
    for (int v = 0; v < 4; ++v) {
        const int i = (tid >> 5) + 16 * v;
        const uint2 kw = i < x.len ? *reinterpret_cast<const uint2*>(p.k + qk_off(p, x.b, x.t0 + i, x.hq) + c4)
                                   : make_uint2(0u, 0u);
        const f32x4 G = *reinterpret_cast<const f32x4*>(pr + BWP_G + i * BW_D + c4);
        const f32x4 kv = {bf_lo(kw.x), bf_hi(kw.x), bf_lo(kw.y), bf_hi(kw.y)};
        f32x4 kg, kh;
        for (int e = 0; e < 4; ++e) {
            kg[e] = kv[e] * fexp(G[e]);
            kh[e] = kv[e] * fexp(Gl[e] - G[e]);
        }
        *reinterpret_cast<f32x4*>(sKG + i * ld + c4) = kg;
        *reinterpret_cast<f32x4*>(sKH + i * ld + c4) = kh;
    }
}

// Work-group -> (row, value head, slice) of the state walks.  Work-groups are dealt
// to the 8 XCDs round robin; the BW_NSL slices of a head read the same chunk
// operands, so they are kept on one XCD (one L2) when the head count allows.
__device__ __forceinline__ void walk_item(const BwdParams& p, int& slice, int64_t& bh) {
    const int64_t idx = blockIdx.x, nbh = (int64_t)p.N * p.Hv;
    if ((nbh & 7) == 0 && BW_NSL == 4) {
        const int64_t k = idx >> 3;
        bh = (idx & 7) + 8 * (k >> 2);
        slice = (int)(k & 3);
    } else {
        bh = idx / BW_NSL;
        slice = (int)(idx % BW_NSL);
    }
}

// ---------------------------------------------------------------- states
// Work-group (sequence b, hv, slice of 32 value columns), 512 threads: eight waves that
// keep the state's 16x16 tiles in MFMA accumulators (tile layout at the kernel).
// Raw inputs of one chunk, fetched into registers with 8- and 16-byte loads while
// the chunk before computes.  Thread t takes, of the [64][128] tiles (k, q, G),
// channels 4 (t % 32) .. + 3 of rows t / 32 + 16 v (v < 4); of the [64][64] tiles (T,
// Aqk), elements 4 (t + 512 v) .. + 3 (v < 2), whose columns 4 (t % 16) .. + 3 are the
// same for both; of the [64][32] value slice (v, do), elements 4 t .. + 3.
struct StatesRaw {
    uint2 k[4];
    f32x4 G[4], Gl, T[2];
    float beta[4];
    uint2 v;
};
__device__ __forceinline__ uint2 ld_bf4(const uint16_t* a) { return *reinterpret_cast<const uint2*>(a); }
__device__ __forceinline__ f32x4 bf4_to_f32(uint2 w) { return f32x4{bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y)}; }

__device__ __forceinline__ void states_fetch(const BwdParams& p, const ChunkIdx& x, int tid, int n0, StatesRaw& r) {
    const float* pr = p.prep + x.ch * BWP_FLOATS;
    const int c4 = 4 * (tid & 31);
    for (int v = 0; v < 4; ++v) {
        const int i = (tid >> 5) + 16 * v;
        r.k[v] = i < x.len ? ld_bf4(p.k + qk_off(p, x.b, x.t0 + i, x.hq) + c4) : make_uint2(0u, 0u);
        r.G[v] = lds4(pr + BWP_G + i * BW_D + c4);
    }
    r.Gl = lds4(pr + BWP_G + (BW_C - 1) * BW_D + c4);
    for (int v = 0; v < 2; ++v) r.T[v] = lds4(pr + BWP_T + 4 * (tid + BW_ST * v));
    const int j4 = 4 * (tid & 15);
    for (int e = 0; e < 4; ++e)
        r.beta[e] = j4 + e < x.len ? ld_beta(p, ((int64_t)x.b * p.T + x.t0 + j4 + e) * p.Hv + x.hv) : 0.f;
    const int iv = tid >> 3, nv = 4 * (tid & 7);
    r.v = iv < x.len ? ld_bf4(p.v + vh_off(p, x.b, x.t0 + iv, x.hv) + n0 + nv) : make_uint2(0u, 0u);
}

__global__ void __launch_bounds__(BW_ST) kda_bwd_states_kernel(const BwdParams p) {
    __shared__ __attribute__((aligned(16))) float sKG[BW_C * GLD];
    __shared__ __attribute__((aligned(16))) float sKH[BW_C * GLD];
    __shared__ __attribute__((aligned(16))) float sTB[BW_C * BW_MD];
    __shared__ __attribute__((aligned(16))) float sS[BW_D * BW_SD];
    __shared__ __attribute__((aligned(16))) float sV[BW_C * BW_SD];
    __shared__ __attribute__((aligned(16))) float sZ[BW_C * BW_SD];
    __shared__ __attribute__((aligned(16))) float sVN[BW_C * BW_SD];
    __shared__ float sGam[BW_D];
    const int tid = threadIdx.x;
    int slice;
    int64_t bh;
    walk_item(p, slice, bh);
    const int hv = (int)(bh % p.Hv), b = (int)(bh / p.Hv);
    const int n0 = slice * BW_SL;
    // The chunk products on v_mfma_f32_16x16x4f32, with the tiles of the reverse walk:
    // wave (it, nt) = (w % 4, w / 4) takes value columns 16 nt .. + 15 of the slice,
    // token tile it of Z and v_new, and state tiles (channels) 2 it, 2 it + 1 of h,
    // kept in accumulators for the whole walk.
    const int lane = tid & 63, wv = tid >> 6, it = wv & 3, nt = wv >> 2;
    const int m4 = 4 * (lane >> 4), rl = lane & 15, col = 16 * nt + rl;
    f32x4 S[2];
    for (int t = 0; t < 2; ++t)
        for (int r = 0; r < 4; ++r)
            S[t][r] = p.h0 ? p.h0[((int64_t)b * p.Hv + hv) * BW_STATE + (32 * it + 16 * t + m4 + r) * BW_D + n0 + col]
                           : 0.f;
    const SeqWalk w = seq_walk(p, b);
    StatesRaw raw;
    if (w.nc > 1) states_fetch(p, walk_chunk(p, w, b, 0, hv), tid, n0, raw);
#pragma unroll 1
    for (int ci = 0; ci < w.nc; ++ci) {
        const ChunkIdx x = walk_chunk(p, w, b, ci, hv);
        float* hs = p.hs + x.ch * BW_STATE + n0 + col;
        for (int t = 0; t < 2; ++t)
            for (int r = 0; r < 4; ++r) {
                const int cc = 32 * it + 16 * t + m4 + r;
                hs[cc * BW_D] = S[t][r];
                sS[cc * BW_SD + col] = S[t][r];
            }
        if (ci == w.nc - 1) break;   // the state leaving the last chunk is not needed
        {
            const int c4 = 4 * (tid & 31);
            for (int v = 0; v < 4; ++v) {
                const int i = (tid >> 5) + 16 * v;
                const f32x4 kv = bf4_to_f32(raw.k[v]);
                f32x4 kg, kh;
                for (int e = 0; e < 4; ++e) {
                    kg[e] = kv[e] * fexp(raw.G[v][e]);
                    kh[e] = kv[e] * fexp(raw.Gl[e] - raw.G[v][e]);
                }
                *reinterpret_cast<f32x4*>(sKG + i * GLD + c4) = kg;
                *reinterpret_cast<f32x4*>(sKH + i * GLD + c4) = kh;
            }
            if (tid < 32)
                for (int e = 0; e < 4; ++e) sGam[c4 + e] = fexp(raw.Gl[e]);
            for (int v = 0; v < 2; ++v) {
                const int e0 = 4 * (tid + BW_ST * v), i = e0 >> 6, j = e0 & 63;
                for (int e = 0; e < 4; ++e) sTB[i * BW_MD + j + e] = raw.T[v][e] * raw.beta[e];
            }
            *reinterpret_cast<f32x4*>(sV + (tid >> 3) * BW_SD + 4 * (tid & 7)) = bf4_to_f32(raw.v);
        }
        if (ci + 1 < w.nc - 1) states_fetch(p, walk_chunk(p, w, b, ci + 1, hv), tid, n0, raw);
        __syncthreads();
        {   // Z = v - kg h
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const int ti = 16 * it + rl;
#pragma unroll 4
            for (int u = 0; u < BW_D / 16; ++u) {
                const f32x4 a4 = lds4(sKG + ti * GLD + 16 * u + m4);
#pragma unroll
                for (int bb = 0; bb < 4; ++bb)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[bb], sS[(16 * u + m4 + bb) * BW_SD + col], acc, 0, 0, 0);
            }
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * it + m4 + r;
                sZ[i * BW_SD + col] = sV[i * BW_SD + col] - acc[r];
            }
        }
        __syncthreads();
        {   // v_new = Tb Z (Tb[i][j] is zero for j > i)
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const int ti = 16 * it + rl;
            for (int u = 0; u <= it; ++u) {
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const int j = 16 * u + m4 + bb;
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sTB[ti * BW_MD + j], sZ[j * BW_SD + col], acc, 0, 0, 0);
                }
            }
            for (int r = 0; r < 4; ++r) sVN[(16 * it + m4 + r) * BW_SD + col] = acc[r];
        }
        __syncthreads();
        // h' = gam h + kh^T v_new
        for (int t = 0; t < 2; ++t) {
            const int cb = 32 * it + 16 * t;
            for (int r = 0; r < 4; ++r) S[t][r] *= sGam[cb + m4 + r];
#pragma unroll 2
            for (int u = 0; u < BW_C / 16; ++u) {
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const int i = 16 * u + m4 + bb;
                    S[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(sKH[i * GLD + cb + rl], sVN[i * BW_SD + col], S[t], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- dstate
// Same grid and layout as states.  kh is needed only for dv_new and qg only for
// the state update, so they share one LDS tile: qg is written once dv_new is
// done.  The raw inputs of the next chunk (k, q, G, T, beta, Aqk, do; element
// layout of StatesRaw) are fetched into registers while the current chunk
// computes dZ and the state update.
struct DstateRaw {
    uint2 k[4], q[4];
    f32x4 G[4], Gl, T[2], A[2];
    float beta[4];
    uint2 dO;
};

__device__ __forceinline__ void dstate_fetch(const BwdParams& p, const ChunkIdx& x, int tid, int n0, DstateRaw& r) {
    const float* pr = p.prep + x.ch * BWP_FLOATS;
    const int c4 = 4 * (tid & 31);
    for (int v = 0; v < 4; ++v) {
        const int i = (tid >> 5) + 16 * v;
        const bool in = i < x.len;
        r.k[v] = in ? ld_bf4(p.k + qk_off(p, x.b, x.t0 + i, x.hq) + c4) : make_uint2(0u, 0u);
        r.q[v] = in ? ld_bf4(p.q + qk_off(p, x.b, x.t0 + i, x.hq) + c4) : make_uint2(0u, 0u);
        r.G[v] = lds4(pr + BWP_G + i * BW_D + c4);
    }
    r.Gl = lds4(pr + BWP_G + (BW_C - 1) * BW_D + c4);
    for (int v = 0; v < 2; ++v) {
        r.T[v] = lds4(pr + BWP_T + 4 * (tid + BW_ST * v));
        r.A[v] = lds4(pr + BWP_AQK + 4 * (tid + BW_ST * v));
    }
    const int j4 = 4 * (tid & 15);
    for (int e = 0; e < 4; ++e)
        r.beta[e] = j4 + e < x.len ? ld_beta(p, ((int64_t)x.b * p.T + x.t0 + j4 + e) * p.Hv + x.hv) : 0.f;
    const int iv = tid >> 3, nv = 4 * (tid & 7);
    r.dO = iv < x.len ? ld_bf4(p.dO + vh_off(p, x.b, x.t0 + iv, x.hv) + n0 + nv) : make_uint2(0u, 0u);
}

__global__ void __launch_bounds__(BW_ST) kda_bwd_dstate_kernel(const BwdParams p) {
    __shared__ __attribute__((aligned(16))) float sKG[BW_C * GLD];
    __shared__ __attribute__((aligned(16))) float sKQ[BW_C * GLD];   // kh, then qg
    __shared__ __attribute__((aligned(16))) float sAQ[BW_C * BW_MD];
    __shared__ __attribute__((aligned(16))) float sTB[BW_C * BW_MD];
    __shared__ __attribute__((aligned(16))) float sDH[BW_D * BW_SD];
    __shared__ __attribute__((aligned(16))) float sDO[BW_C * BW_SD];
    __shared__ __attribute__((aligned(16))) float sDVN[BW_C * BW_SD];
    __shared__ __attribute__((aligned(16))) float sDZ[BW_C * BW_SD];
    __shared__ float sGam[BW_D];
    const int tid = threadIdx.x;
    int slice;
    int64_t bh;
    walk_item(p, slice, bh);
    const int hv = (int)(bh % p.Hv), b = (int)(bh / p.Hv);
    const int n0 = slice * BW_SL;
    // The chunk products on v_mfma_f32_16x16x4f32.  Wave (it, nt) = (w % 4, w / 4):
    // value columns 16 nt .. + 15 of the slice; token tile it of dv_new and dZ; state
    // tiles (channels) 2 it and 2 it + 1 of dh, kept in accumulators for the whole
    // walk.  A tile's lane l holds rows 4 (l / 16) + r of column l % 16, and MFMA b
    // of a 16-wide k block u sums the index 16 u + 4 (l / 16) + b.
    const int lane = tid & 63, wv = tid >> 6, it = wv & 3, nt = wv >> 2;
    const int m4 = 4 * (lane >> 4), rl = lane & 15, col = 16 * nt + rl;
    f32x4 dh[2];
    for (int t = 0; t < 2; ++t)
        for (int r = 0; r < 4; ++r)
            dh[t][r] = p.dhT ? p.dhT[((int64_t)b * p.Hv + hv) * BW_STATE + (32 * it + 16 * t + m4 + r) * BW_D + n0 + col]
                             : 0.f;
    const SeqWalk w = seq_walk(p, b);
    DstateRaw raw;
    if (w.nc > 0) dstate_fetch(p, walk_chunk(p, w, b, w.nc - 1, hv), tid, n0, raw);
#pragma unroll 1
    for (int ci = w.nc - 1; ci >= 0; --ci) {
        const ChunkIdx x = walk_chunk(p, w, b, ci, hv);
        float* ds = p.dhs + x.ch * BW_STATE + n0 + col;
        for (int t = 0; t < 2; ++t)
            for (int r = 0; r < 4; ++r) {
                const int cc = 32 * it + 16 * t + m4 + r;
                ds[cc * BW_D] = dh[t][r];
                sDH[cc * BW_SD + col] = dh[t][r];
            }
        // this chunk's operands, from the registers fetched during the previous step
        {
            const int c4 = 4 * (tid & 31);
            for (int v = 0; v < 4; ++v) {
                const int i = (tid >> 5) + 16 * v;
                const f32x4 kv = bf4_to_f32(raw.k[v]);
                f32x4 kg, kh;
                for (int e = 0; e < 4; ++e) {
                    kg[e] = kv[e] * fexp(raw.G[v][e]);
                    kh[e] = kv[e] * fexp(raw.Gl[e] - raw.G[v][e]);
                }
                *reinterpret_cast<f32x4*>(sKG + i * GLD + c4) = kg;
                *reinterpret_cast<f32x4*>(sKQ + i * GLD + c4) = kh;
            }
            if (tid < 32)
                for (int e = 0; e < 4; ++e) sGam[c4 + e] = fexp(raw.Gl[e]);
            for (int v = 0; v < 2; ++v) {
                const int e0 = 4 * (tid + BW_ST * v), i = e0 >> 6, j = e0 & 63;
                for (int e = 0; e < 4; ++e) {
                    sTB[i * BW_MD + j + e] = raw.T[v][e] * raw.beta[e];
                    sAQ[i * BW_MD + j + e] = raw.A[v][e];
                }
            }
            *reinterpret_cast<f32x4*>(sDO + (tid >> 3) * BW_SD + 4 * (tid & 7)) = bf4_to_f32(raw.dO);
        }
        __syncthreads();
        {   // dv_new = kh dh' + Aqk^T do (Aqk[m][i] is zero for m < i)
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const int ti = 16 * it + rl;
#pragma unroll 4
            for (int u = 0; u < BW_D / 16; ++u) {
                const f32x4 a4 = lds4(sKQ + ti * GLD + 16 * u + m4);
#pragma unroll
                for (int bb = 0; bb < 4; ++bb)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[bb], sDH[(16 * u + m4 + bb) * BW_SD + col], acc, 0, 0, 0);
            }
            for (int u = it; u < BW_C / 16; ++u) {
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const int m = 16 * u + m4 + bb;
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sAQ[m * BW_MD + ti], sDO[m * BW_SD + col], acc, 0, 0, 0);
                }
            }
            for (int r = 0; r < 4; ++r) sDVN[(16 * it + m4 + r) * BW_SD + col] = acc[r];
        }
        __syncthreads();
        for (int v = 0; v < 4; ++v) {   // kh is done with: qg replaces it
            const f32x4 qv = bf4_to_f32(raw.q[v]);
            f32x4 qg;
            for (int e = 0; e < 4; ++e) qg[e] = p.scale * qv[e] * fexp(raw.G[v][e]);
            *reinterpret_cast<f32x4*>(sKQ + ((tid >> 5) + 16 * v) * GLD + 4 * (tid & 31)) = qg;
        }
        if (ci > 0) dstate_fetch(p, walk_chunk(p, w, b, ci - 1, hv), tid, n0, raw);
        {   // dZ = Tb^T dv_new (Tb[i][j] is zero for i < j)
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const int tj = 16 * it + rl;
            for (int u = it; u < BW_C / 16; ++u) {
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const int i = 16 * u + m4 + bb;
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sTB[i * BW_MD + tj], sDVN[i * BW_SD + col], acc, 0, 0, 0);
                }
            }
            for (int r = 0; r < 4; ++r) sDZ[(16 * it + m4 + r) * BW_SD + col] = acc[r];
        }
        __syncthreads();
        // dh = gam dh' + qg^T do - kg^T dZ
        for (int t = 0; t < 2; ++t) {
            const int cb = 32 * it + 16 * t;
            for (int r = 0; r < 4; ++r) dh[t][r] *= sGam[cb + m4 + r];
#pragma unroll 2
            for (int u = 0; u < BW_C / 16; ++u) {
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const int m = 16 * u + m4 + bb;
                    dh[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(sKQ[m * GLD + cb + rl], sDO[m * BW_SD + col], dh[t], 0, 0, 0);
                    dh[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(-sKG[m * GLD + cb + rl], sDZ[m * BW_SD + col], dh[t], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }
    if (p.dh0)
        for (int t = 0; t < 2; ++t)
            for (int r = 0; r < 4; ++r)
                p.dh0[((int64_t)b * p.Hv + hv) * BW_STATE + (32 * it + 16 * t + m4 + r) * BW_D + n0 + col] = dh[t][r];
}

// ---------------------------------------------------------------- grad
// One 512-thread work-group per (chunk, value head).  The value columns are
// taken 16 at a time; the tiles of one such slice that are read along the
// token index (do, v, Z, v_new, dv_new, dZ) are stored transposed, [16][68], so
// that a thread reads four consecutive tokens with one 16-byte LDS load.
constexpr int GTS = 68;    // row stride of the transposed slice tiles
constexpr int GMD = 68;    // row stride of the grad kernel's Tb tile (16-byte rows)
// LDS of the grad kernel, in floats.  Phase A (the loop over value slices):
constexpr int GA_KG = 0, GA_KH = GA_KG + BW_C * GLD, GA_AQ = GA_KH + BW_C * GLD, GA_TB = GA_AQ + BW_C * BW_MD;
constexpr int GA_H = GA_TB + BW_C * GMD, GA_DH = GA_H + BW_D * GSD, GA_DO = GA_DH + BW_D * GSD;
constexpr int GA_V = GA_DO + GSL * GTS, GA_Z = GA_V + GSL * GTS, GA_VN = GA_Z + GSL * GTS;
constexpr int GA_DVN = GA_VN + GSL * GTS, GA_DZ = GA_DVN + GSL * GTS, GA_END = GA_DZ + GSL * GTS;
static_assert(GA_H % 4 == 0 && GA_DO % 4 == 0 && GA_V % 4 == 0 && GA_Z % 4 == 0 && GA_VN % 4 == 0 &&
              GA_DVN % 4 == 0 && GA_DZ % 4 == 0 && GA_KH % 4 == 0 && GA_TB % 4 == 0, "16-byte aligned tiles");
// Phase B (the inverse's gradient), then phase C (the pairwise terms):
constexpr int GC_Q = 0, GC_K = GC_Q + BW_C * BW_LD, GC_G = GC_K + BW_C * BW_LD, GC_DAQ = GC_G + BW_C * BW_LD;
constexpr int GC_DAB = GC_DAQ + BW_C * BW_MD, GC_END = GC_DAB + BW_C * BW_MD;
constexpr int GB_M1 = 0, GB_M2 = GB_M1 + BW_C * BW_MD, GB_DA = GB_M2 + BW_C * BW_MD, GB_BETA = GB_DA + BW_C * BW_MD;
constexpr int GB_T = GB_BETA + BW_C, GB_AB = GB_T + BW_C * BW_MD, GB_DTB = GC_END, GB_END = GB_DTB + BW_C * BW_MD;
static_assert(GB_AB + BW_C * BW_MD <= GC_DAQ, "phase B temporaries must not overlap dAqk / dAbar");
constexpr int G_LDS = GA_END > GB_END ? GA_END : GB_END;
static_assert(G_LDS * 4 <= 160 * 1024, "grad kernel LDS");

__global__ void __launch_bounds__(512) kda_bwd_grad_kernel(const BwdParams p) {
    __shared__ __attribute__((aligned(16))) float F[G_LDS];
    const int tid = threadIdx.x;
    const ChunkIdx x = chunk_of(p, blockIdx.x);
    if (x.len == 0) return;   // a slot that holds no chunk (uniform per work-group)
    const float* pr = p.prep + x.ch * BWP_FLOATS;
    const float* hs = p.hs + x.ch * BW_STATE;
    const float* ds = p.dhs + x.ch * BW_STATE;
    // element (i, c) accumulators: c = tid % 128, rows i = 16 rg + r
    const int c = tid & 127, rg = tid >> 7, i0 = 16 * rg;
    // 64 x 64 tiles in phase B: row ai = tid / 8, columns 8 aj .. + 7
    const int ai = tid >> 3, aj = (tid & 7) * 8;
    // The operand gradients summed over the value columns, on v_mfma_f32_16x16x4f32:
    // wave w holds the 16x16 tiles (it, ct) of d(qg), -d(kg) and d(kh) (64 x 128) for
    // token tile it = w % 4 and channel tiles ct = 4 (w / 4) .. + 3, and the tiles
    // (it, jt) of dAqk and dTb (64 x 64) for jt = 2 (w / 4), + 1.  A tile's lane l
    // holds rows 4 (l / 16) + r of column l % 16.
    const int lane = tid & 63, wv = tid >> 6, it = wv & 3, chh = wv >> 2;
    f32x4 accQ[4], accKG[4], accKH[4], accAQ[2], accTB[2];
    for (int t = 0; t < 4; ++t) accQ[t] = accKG[t] = accKH[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int t = 0; t < 2; ++t) accAQ[t] = accTB[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dgam = 0.f;

    load_key_ops(p, x, pr, F + GA_KG, F + GA_KH, tid, GLD);
    {
        // Aqk and Tb: elements 4 (t + 512 v) .. + 3, columns 4 (t % 16) .. + 3 for both v
        const int j4 = 4 * (tid & 15);
        float bj[4];
        for (int e = 0; e < 4; ++e)
            bj[e] = j4 + e < x.len ? ld_beta(p, ((int64_t)x.b * p.T + x.t0 + j4 + e) * p.Hv + x.hv) : 0.f;
        for (int v = 0; v < 2; ++v) {
            const int e0 = 4 * (tid + 512 * v), i = e0 >> 6;
            const f32x4 a4 = lds4(pr + BWP_AQK + e0), t4 = lds4(pr + BWP_T + e0);
            for (int e = 0; e < 4; ++e) {
                F[GA_AQ + i * BW_MD + j4 + e] = a4[e];
                F[GA_TB + i * GMD + j4 + e] = t4[e] * bj[e];
            }
        }
    }
    // a slice's inputs for thread t: h and dh' of row t / 4, columns 4 (t % 4) .. + 3 of
    // the [128][16] slice; do and v of token t / 8, columns 2 (t % 8), + 1 of the
    // [64][16] slice; the next slice's are fetched while this one computes
    f32x4 rH, rDH;
    uint32_t rDO, rV;
    auto fetch = [&](int n0) {
        const int cc = tid >> 2, n = 4 * (tid & 3);
        rH = *reinterpret_cast<const f32x4*>(hs + cc * BW_D + n0 + n);
        rDH = *reinterpret_cast<const f32x4*>(ds + cc * BW_D + n0 + n);
        const int i = tid >> 3, n2 = 2 * (tid & 7);
        const bool in = i < x.len;
        const int64_t o = vh_off(p, x.b, x.t0 + i, x.hv) + n0 + n2;
        rDO = in ? *reinterpret_cast<const uint32_t*>(p.dO + o) : 0u;
        rV = in ? *reinterpret_cast<const uint32_t*>(p.v + o) : 0u;
    };
    fetch(0);
#pragma unroll 1
    for (int sl = 0; sl < GNSL; ++sl) {
        const int n0 = sl * GSL;
        {
            const int cc = tid >> 2, n = 4 * (tid & 3);
            for (int e = 0; e < 4; ++e) {
                F[GA_H + cc * GSD + n + e] = rH[e];
                F[GA_DH + cc * GSD + n + e] = rDH[e];
            }
            const int i = tid >> 3, n2 = 2 * (tid & 7);
            F[GA_DO + n2 * GTS + i] = bf_lo(rDO);
            F[GA_DO + (n2 + 1) * GTS + i] = bf_hi(rDO);
            F[GA_V + n2 * GTS + i] = bf_lo(rV);
            F[GA_V + (n2 + 1) * GTS + i] = bf_hi(rV);
        }
        if (sl + 1 < GNSL) fetch(n0 + GSL);
        __syncthreads();
        {
            // Z = v - kg h (waves 0..3) and dv_new = kh dh' + Aqk^T do (waves 4..7), token
            // tile it of the slice each.  MFMA b of k block u sums the index
            // 16 u + 4 (lane / 16) + b, so a lane reads four consecutive channels (or
            // tokens) of its row with one 16-byte load.
            const int m4 = 4 * (lane >> 4), rl = lane & 15, ti = 16 * it + rl;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (chh == 0) {
#pragma unroll 4
                for (int u = 0; u < BW_D / 16; ++u) {
                    const int cc = 16 * u + m4;
                    const f32x4 a4 = lds4(F + GA_KG + ti * GLD + cc);
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[b], F[GA_H + (cc + b) * GSD + rl], acc, 0, 0, 0);
                }
                const f32x4 v4 = lds4(F + GA_V + rl * GTS + 16 * it + m4);
                *reinterpret_cast<f32x4*>(F + GA_Z + rl * GTS + 16 * it + m4) = v4 - acc;
            } else {
#pragma unroll 4
                for (int u = 0; u < BW_D / 16; ++u) {
                    const int cc = 16 * u + m4;
                    const f32x4 a4 = lds4(F + GA_KH + ti * GLD + cc);
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[b], F[GA_DH + (cc + b) * GSD + rl], acc, 0, 0, 0);
                }
                // Aqk[m][i] is zero for m < i: token blocks u >= it
                for (int u = it; u < BW_C / 16; ++u) {
                    const int mm = 16 * u + m4;
                    const f32x4 b4 = lds4(F + GA_DO + rl * GTS + mm);
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(F[GA_AQ + (mm + b) * BW_MD + ti], b4[b], acc, 0, 0, 0);
                }
                *reinterpret_cast<f32x4*>(F + GA_DVN + rl * GTS + 16 * it + m4) = acc;
            }
        }
        __syncthreads();
        {
            // v_new = Tb Z (waves 0..3, token tile it) and dZ = Tb^T dv_new = dv (waves
            // 4..7, token tile it); Tb is lower triangular.
            const int m4 = 4 * (lane >> 4), rl = lane & 15, ti = 16 * it + rl;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (chh == 0) {
                for (int u = 0; u <= it; ++u) {
                    const int jj = 16 * u + m4;
                    const f32x4 a4 = lds4(F + GA_TB + ti * GMD + jj);
                    const f32x4 b4 = lds4(F + GA_Z + rl * GTS + jj);
#pragma unroll
                    for (int b = 0; b < 4; ++b) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[b], b4[b], acc, 0, 0, 0);
                }
                *reinterpret_cast<f32x4*>(F + GA_VN + rl * GTS + 16 * it + m4) = acc;
            } else {
                for (int u = it; u < BW_C / 16; ++u) {
                    const int mm = 16 * u + m4;
                    const f32x4 b4 = lds4(F + GA_DVN + rl * GTS + mm);
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(F[GA_TB + (mm + b) * GMD + ti], b4[b], acc, 0, 0, 0);
                }
                *reinterpret_cast<f32x4*>(F + GA_DZ + rl * GTS + 16 * it + m4) = acc;
                for (int r = 0; r < 4; ++r) {
                    const int i = 16 * it + m4 + r;
                    if (i < x.len) p.dv[vh_off(p, x.b, x.t0 + i, x.hv) + n0 + rl] = acc[r];
                }
            }
        }
        __syncthreads();
        if (rg == 0) {
            for (int n = 0; n < GSL; ++n) dgam += F[GA_DH + c * GSD + n] * F[GA_H + c * GSD + n];
        }
        {
            // Rank-16 updates of the slice: MFMA b of a k step sums the columns n = 4 m + b
            // (m = lane / 16 supplies n); A rows are tokens 16 it + lane % 16, B columns
            // channels (or tokens) 16 ct + lane % 16.
            const int m4 = 4 * (lane >> 4), rl = lane & 15, ti = 16 * it + rl;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int n = m4 + b;
                const float ado = F[GA_DO + n * GTS + ti], adz = F[GA_DZ + n * GTS + ti];
                const float avn = F[GA_VN + n * GTS + ti], advn = F[GA_DVN + n * GTS + ti];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int cc = 16 * (4 * chh + t) + rl;
                    const float bh = F[GA_H + cc * GSD + n], bdh = F[GA_DH + cc * GSD + n];
                    accQ[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(ado, bh, accQ[t], 0, 0, 0);
                    accKG[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(adz, bh, accKG[t], 0, 0, 0);
                    accKH[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(avn, bdh, accKH[t], 0, 0, 0);
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int tj = 16 * (2 * chh + t) + rl;
                    accAQ[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(ado, F[GA_VN + n * GTS + tj], accAQ[t], 0, 0, 0);
                    accTB[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(advn, F[GA_Z + n * GTS + tj], accTB[t], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }

    // The accumulated tiles to LDS: dTb and the lower triangle of dAqk in their
    // phase B/C places, d(qg), d(kg), d(kh) ([64][129] each) below them, from where
    // each thread takes its own elements (rows i0 .. + 15 of channel c).
    {
        const int rb = 16 * it + 4 * (lane >> 4), cl = lane & 15;
        for (int t = 0; t < 4; ++t) {
            const int cc = 16 * (4 * chh + t) + cl;
            for (int r = 0; r < 4; ++r) {
                F[(rb + r) * BW_LD + cc] = accQ[t][r];
                F[BW_C * BW_LD + (rb + r) * BW_LD + cc] = -accKG[t][r];
                F[2 * BW_C * BW_LD + (rb + r) * BW_LD + cc] = accKH[t][r];
            }
        }
        for (int t = 0; t < 2; ++t) {
            const int j = 16 * (2 * chh + t) + cl;
            for (int r = 0; r < 4; ++r) {
                F[GB_DTB + (rb + r) * BW_MD + j] = accTB[t][r];
                F[GC_DAQ + (rb + r) * BW_MD + j] = j <= rb + r ? accAQ[t][r] : 0.f;
            }
        }
    }
    static_assert(3 * BW_C * BW_LD <= GC_DAQ && GC_DAQ + BW_C * BW_MD <= GB_DTB, "accumulator staging");
    __syncthreads();
    float aQ[16], aKG[16], aKH[16];
    for (int r = 0; r < 16; ++r) {
        aQ[r] = F[(i0 + r) * BW_LD + c];
        aKG[r] = F[BW_C * BW_LD + (i0 + r) * BW_LD + c];
        aKH[r] = F[2 * BW_C * BW_LD + (i0 + r) * BW_LD + c];
    }
    __syncthreads();

    // Phase B: dA = lower_strict(-T^T (dTb diag beta) T^T), dbeta, dAbar = diag(beta) dA.
    for (int v = 0; v < 2; ++v) {
        const int e0 = 4 * (tid + 512 * v), i = e0 >> 6, j = e0 & 63;
        const f32x4 t4 = lds4(pr + BWP_T + e0), a4 = lds4(pr + BWP_ABAR + e0);
        for (int e = 0; e < 4; ++e) {
            F[GB_T + i * BW_MD + j + e] = t4[e];
            F[GB_AB + i * BW_MD + j + e] = a4[e];
        }
    }
    if (tid < BW_C)
        F[GB_BETA + tid] = tid < x.len ? ld_beta(p, ((int64_t)x.b * p.T + x.t0 + tid) * p.Hv + x.hv) : 0.f;
    __syncthreads();
    for (int s = 0; s < 8; ++s) {
        const int j = aj + s;
        F[GB_M1 + ai * BW_MD + j] = F[GB_DTB + ai * BW_MD + j] * F[GB_BETA + j];
    }
    __syncthreads();
    {
        // M2 = T^T M1 on v_mfma_f32_16x16x4f32 (T[m][a] is zero for m < a): wave (it, chh)
        // takes tiles (it, 2 chh) and (it, 2 chh + 1); MFMA b of block u sums m = 16 u +
        // 4 (lane / 16) + b.  The zeros of dA above its diagonal tiles are written here.
        const int m4 = 4 * (lane >> 4), rl = lane & 15, ta = 16 * it + rl;
        for (int t = 0; t < 2; ++t) {
            const int jt = 2 * chh + t;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int u = it; u < BW_C / 16; ++u) {
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const int m = 16 * u + m4 + bb;
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(F[GB_T + m * BW_MD + ta], F[GB_M1 + m * BW_MD + 16 * jt + rl],
                                                               acc, 0, 0, 0);
                }
            }
            for (int r = 0; r < 4; ++r) {
                F[GB_M2 + (16 * it + m4 + r) * BW_MD + 16 * jt + rl] = acc[r];
                if (jt > it) F[GB_DA + (16 * it + m4 + r) * BW_MD + 16 * jt + rl] = 0.f;
            }
        }
    }
    __syncthreads();
    {
        // dA = -M2 T^T, strictly lower (T[j][m] is zero for m > j): wave w takes the
        // lower-triangle tiles w and w + 8 (row-major order over (at, jt), jt <= at)
        const int m4 = 4 * (lane >> 4), rl = lane & 15;
        for (int k = 0; k < (wv + 8 < 10 ? 2 : 1); ++k) {
            const int t = wv + 8 * k;
            const int at = t >= 6 ? 3 : (t >= 3 ? 2 : (t >= 1 ? 1 : 0)), jt = t - at * (at + 1) / 2;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int u = 0; u <= jt; ++u) {
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    const int m = 16 * u + m4 + bb;
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(F[GB_M2 + (16 * at + rl) * BW_MD + m],
                                                               F[GB_T + (16 * jt + rl) * BW_MD + m], acc, 0, 0, 0);
                }
            }
            for (int r = 0; r < 4; ++r) {
                const int a = 16 * at + m4 + r, j = 16 * jt + rl;
                F[GB_DA + a * BW_MD + j] = j < a ? -acc[r] : 0.f;
            }
        }
    }
    __syncthreads();
    if (tid < BW_C) {
        const int j = tid;
        float db = 0.f;
        for (int i = 0; i < BW_C; ++i) db += F[GB_DTB + i * BW_MD + j] * F[GB_T + i * BW_MD + j];
        for (int m = 0; m < BW_C; ++m) db += F[GB_DA + j * BW_MD + m] * F[GB_AB + j * BW_MD + m];
        if (j < x.len) p.dbeta[((int64_t)x.b * p.T + x.t0 + j) * p.Hv + x.hv] = db;
    }
    for (int s = 0; s < 8; ++s) {
        const int j = aj + s;
        F[GC_DAB + ai * BW_MD + j] = F[GB_BETA + ai] * F[GB_DA + ai * BW_MD + j];
    }
    __syncthreads();

    // Phase C: q, k and G of the chunk (thread t: channels 4 (t % 32) .. + 3 of rows
    // t / 32 + 16 v), then the pairwise terms per channel.
    {
        const int c4 = 4 * (tid & 31);
        for (int v = 0; v < 4; ++v) {
            const int i = (tid >> 5) + 16 * v;
            uint2 qw = make_uint2(0u, 0u), kw = make_uint2(0u, 0u);
            if (i < x.len) {
                qw = *reinterpret_cast<const uint2*>(p.q + qk_off(p, x.b, x.t0 + i, x.hq) + c4);
                kw = *reinterpret_cast<const uint2*>(p.k + qk_off(p, x.b, x.t0 + i, x.hq) + c4);
            }
            const f32x4 G = lds4(pr + BWP_G + i * BW_D + c4);
            const float qf[4] = {bf_lo(qw.x), bf_hi(qw.x), bf_lo(qw.y), bf_hi(qw.y)};
            const float kf[4] = {bf_lo(kw.x), bf_hi(kw.x), bf_lo(kw.y), bf_hi(kw.y)};
            for (int e = 0; e < 4; ++e) {
                F[GC_Q + i * BW_LD + c4 + e] = qf[e];
                F[GC_K + i * BW_LD + c4 + e] = kf[e];
                F[GC_G + i * BW_LD + c4 + e] = G[e];
            }
        }
    }
    __syncthreads();
    const float Gl = F[GC_G + (BW_C - 1) * BW_LD + c];
    float qi[16], ki[16], Gi[16];
    for (int r = 0; r < 16; ++r) {
        Gi[r] = F[GC_G + (i0 + r) * BW_LD + c];
        qi[r] = F[GC_Q + (i0 + r) * BW_LD + c];
        ki[r] = F[GC_K + (i0 + r) * BW_LD + c];
    }
    // The pairwise sums, per element (i, c):
    //   Rq = sum_{j<=i} dAqk[i][j] k_j e^{G_i - G_j},  Rk = the same with dAbar,
    //   Cq = sum_{m>=i} dAqk[m][i] q_m e^{G_m - G_i},  Ck = sum_{m>=i} dAbar[m][i] k_m e^{G_m - G_i}.
    float oG[16], oP[16];
    auto finish = [&](int r, float Rq, float Rk, float Cq, float Ck) {
        const int i = i0 + r;
        const float eG = fexp(Gi[r]), eH = fexp(Gl - Gi[r]);
        const float oq = p.scale * (aQ[r] * eG + Rq);
        const float ok = aKG[r] * eG + aKH[r] * eH + p.scale * Cq + Ck + Rk;
        oP[r] = aKH[r] * ki[r] * eH;
        oG[r] = p.scale * qi[r] * Rq + ki[r] * Rk - p.scale * ki[r] * Cq - ki[r] * Ck + aKG[r] * ki[r] * eG +
                p.scale * aQ[r] * qi[r] * eG - oP[r];
        if (i < x.len) {
            const int64_t o = vh_off(p, x.b, x.t0 + i, x.hv) + c;
            p.dqv[o] = oq;
            p.dkv[o] = ok;
        }
    };
    // With the anchor A = G_last / 2 of each channel, e^{G_i - G_j} = e^{G_i - A} e^{A - G_j}
    // and every factor lies within e^{+-|G_last| / 2}: the four sums become products
    // of dAqk, dAbar (64 x 64) with k e^{A-G}, q e^{G-A}, k e^{G-A} (64 x 128) on
    // v_mfma_f32_16x16x4f32, scaled per element.  A chunk that decays by more than
    // e^-120 on some channel (factors beyond e^60) takes the element-by-element sums.
    const bool far = __syncthreads_or(rg == 0 && !(Gl >= -120.f)) != 0;
    if (!far) {
        const float A = 0.5f * Gl;
        for (int r = 0; r < 16; ++r) {
            const float eP = fexp(Gi[r] - A), eM = fexp(A - Gi[r]);
            F[GC_Q + (i0 + r) * BW_LD + c] = qi[r] * eP;   // q e^{G-A}
            F[GC_K + (i0 + r) * BW_LD + c] = ki[r] * eM;   // k e^{A-G}
            F[GC_G + (i0 + r) * BW_LD + c] = ki[r] * eP;   // k e^{G-A}
        }
        __syncthreads();
        f32x4 P1[4], P2[4], P3[4], P4[4];
        for (int t = 0; t < 4; ++t) P1[t] = P2[t] = P3[t] = P4[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            // wave (it, chh): token tile it, channel tiles 4 chh .. + 3; MFMA b of block u
            // sums the index 16 u + 4 (lane / 16) + b
            const int m4 = 4 * (lane >> 4), rl = lane & 15, ti = 16 * it + rl;
            for (int u = 0; u <= it; ++u) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int j = 16 * u + m4 + b;
                    const float a1 = F[GC_DAQ + ti * BW_MD + j], a2 = F[GC_DAB + ti * BW_MD + j];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float kb = F[GC_K + j * BW_LD + 16 * (4 * chh + t) + rl];
                        P1[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, kb, P1[t], 0, 0, 0);
                        P2[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a2, kb, P2[t], 0, 0, 0);
                    }
                }
            }
            for (int u = it; u < BW_C / 16; ++u) {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int m = 16 * u + m4 + b;
                    const float a3 = F[GC_DAQ + m * BW_MD + ti], a4 = F[GC_DAB + m * BW_MD + ti];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int cq = 16 * (4 * chh + t) + rl;
                        P3[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a3, F[GC_Q + m * BW_LD + cq], P3[t], 0, 0, 0);
                        P4[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4, F[GC_G + m * BW_LD + cq], P4[t], 0, 0, 0);
                    }
                }
            }
        }
        __syncthreads();   // operands read: the four products go to LDS ([4][64][129])
        static_assert(4 * BW_C * BW_LD <= GC_END, "pairwise staging");
        {
            const int rb = 16 * it + 4 * (lane >> 4), cl = lane & 15;
            for (int t = 0; t < 4; ++t) {
                const int cc = 16 * (4 * chh + t) + cl;
                for (int r = 0; r < 4; ++r) {
                    const int o = (rb + r) * BW_LD + cc;
                    F[o] = P1[t][r];
                    F[BW_C * BW_LD + o] = P2[t][r];
                    F[2 * BW_C * BW_LD + o] = P3[t][r];
                    F[3 * BW_C * BW_LD + o] = P4[t][r];
                }
            }
        }
        __syncthreads();
        for (int r = 0; r < 16; ++r) {
            const int o = (i0 + r) * BW_LD + c;
            const float eP = fexp(Gi[r] - A), eM = fexp(A - Gi[r]);
            finish(r, F[o] * eP, F[BW_C * BW_LD + o] * eP, F[2 * BW_C * BW_LD + o] * eM, F[3 * BW_C * BW_LD + o] * eM);
        }
    } else {
        for (int r = 0; r < 16; ++r) {
            const int i = i0 + r;
            float Rq = 0.f, Rk = 0.f, Cq = 0.f, Ck = 0.f;
            for (int j = 0; j <= i; ++j) {
                const float kE = F[GC_K + j * BW_LD + c] * fexp(Gi[r] - F[GC_G + j * BW_LD + c]);
                Rq += F[GC_DAQ + i * BW_MD + j] * kE;
                Rk += F[GC_DAB + i * BW_MD + j] * kE;   // zero on the diagonal
            }
            for (int m = i; m < BW_C; ++m) {
                const float E = fexp(F[GC_G + m * BW_LD + c] - Gi[r]);
                Cq += F[GC_DAQ + m * BW_MD + i] * F[GC_Q + m * BW_LD + c] * E;
                Ck += F[GC_DAB + m * BW_MD + i] * F[GC_K + m * BW_LD + c] * E;
            }
            finish(r, Rq, Rk, Cq, Ck);
        }
    }
    __syncthreads();   // q and k are no longer read: reuse them for dG and the kh terms
    for (int r = 0; r < 16; ++r) {
        const int i = i0 + r;
        F[GC_Q + i * BW_LD + c] = oG[r];
        F[GC_K + i * BW_LD + c] = oP[r];
    }
    __syncthreads();
    if (rg == 0) {
        // G_last collects sum_t dkh * kh and dgam * gam; dg is the reverse cumsum of dG.
        float tot = dgam * fexp(Gl);
        for (int i = 0; i < BW_C; ++i) tot += F[GC_K + i * BW_LD + c];
        float run = tot;
        for (int i = BW_C - 1; i >= 0; --i) {
            run += F[GC_Q + i * BW_LD + c];
            if (i < x.len) p.dg[vh_off(p, x.b, x.t0 + i, x.hv) + c] = run;
        }
    }
}

// ---------------------------------------------------------------- group
__global__ void __launch_bounds__(256) kda_bwd_group_kernel(const BwdParams p, int64_t total) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;   // over [B * T, Hq, 128]
    if (e >= total) return;
    const int c = (int)(e & 127);
    const int64_t rest = e >> 7;
    const int hq = (int)(rest % p.Hq);
    const int64_t tok = rest / p.Hq;
    if (p.cu) {   // tokens of no packed sequence are not written
        const int64_t a = p.cu[0], z = p.cu[p.N];
        if (tok < a || tok >= z) return;
    }
    const int group = p.Hv / p.Hq;
    float sq = 0.f, sk = 0.f;
    for (int u = 0; u < group; ++u) {
        const int64_t o = (tok * p.Hv + (int64_t)hq * group + u) * BW_D + c;
        sq += p.dqv[o];
        sk += p.dkv[o];
    }
    p.dq[e] = sq;
    p.dk[e] = sk;
}

}  // namespace

hipError_t launch_kda_bwd(const BwdParams& p, hipStream_t stream) {
    const int64_t chunks = p.T > 0 ? p.nslots * p.Hv : 0;
    const int64_t scans = (int64_t)p.N * p.Hv * BW_NSL;
    if (chunks > 0) {
        hipLaunchKernelGGL(kda_bwd_prep_kernel, dim3((unsigned)chunks), dim3(BW_PT), 0, stream, p);
        hipLaunchKernelGGL(kda_bwd_states_kernel, dim3((unsigned)scans), dim3(BW_ST), 0, stream, p);
    }
    if (scans > 0) hipLaunchKernelGGL(kda_bwd_dstate_kernel, dim3((unsigned)scans), dim3(BW_ST), 0, stream, p);
    if (chunks > 0) {
        hipLaunchKernelGGL(kda_bwd_grad_kernel, dim3((unsigned)chunks), dim3(512), 0, stream, p);
        if (p.Hv != p.Hq) {
            const int64_t total = (int64_t)p.B * p.T * p.Hq * BW_D;
            hipLaunchKernelGGL(kda_bwd_group_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, p,
                               total);
        }
    }
    return hipGetLastError();
}

}  // namespace kda

// One recurrent step of KDA for a batch of single tokens, on gfx950 (MI355X).
//
// The recurrence itself, one token at a time: for sequence n and value head hv
// (the decode half of the inference path that consumes the forward's final
// state; "cuLA REPO_LAYOUT.md", entry decode/ for the KDA decode reference):
//
//   S~ = Diag(e^g) S                                  (decay rows by key channel)
//   w  = beta (v - S~^T k)                            (delta-rule correction)
//   S' = S~ + k w^T        = (I - beta k k^T) Diag(e^g) S + beta k v^T
//   o  = scale S'^T q      = scale (S~^T q + (q . k) w)
//
// The state is fp32 and so is all arithmetic; o is rounded to bf16 once.  The
// step is bound by the state's HBM traffic (64 KB read and 64 KB written per
// head against about 1.5 KB of vectors), so the kernel is laid out for that:
// one 512-thread work-group per (sequence, value head); thread t takes columns
// 4 (t % 32) .. + 3 of rows 8 (t / 32) .. + 7, so every load and store moves 16
// contiguous bytes per lane and each row is one 512-byte run across 32 lanes.
// The two column sums over rows (S~^T k, S~^T q) combine the 16 row groups'
// partial sums through LDS in a fixed order: repeated runs are bitwise equal.
// A thread writes only state elements it has read, so the new state may
// overwrite the old one in place.
#include "kda_device.h"

namespace kda {

namespace {

constexpr int DEC_THREADS = 512;
constexpr int DEC_RG = 16;   // row groups of 8 rows
constexpr int DEC_CG = 32;   // column groups of 4 columns

}  // namespace

__global__ void __launch_bounds__(DEC_THREADS) kda_decode_kernel(const DecodeParams p) {
    __shared__ float sU[DEC_RG][DK];     // partial (S~^T k) per row group
    __shared__ float sQ[DEC_RG][DK];     // partial (S~^T q) per row group
    __shared__ float sQK[DEC_RG];        // partial q . k per row group
    __shared__ float sW[DK];             // w

    const int item = blockIdx.x;
    const int n = item / p.Hv, hv = item % p.Hv;
    const int hq = hv / (p.Hv / p.Hq);
    const int tid = threadIdx.x;
    const int cg = tid % DEC_CG, rg = tid / DEC_CG;
    const int c0 = 8 * rg, j0 = 4 * cg;

    const uint16_t* q = p.q + ((int64_t)n * p.Hq + hq) * DK;
    const uint16_t* k = p.k + ((int64_t)n * p.Hq + hq) * DK;
    const uint16_t* v = p.v + ((int64_t)n * p.Hv + hv) * DK;
    const float* g = p.g + ((int64_t)n * p.Hv + hv) * DK;
    const float beta = p.beta_f32 ? reinterpret_cast<const float*>(p.beta)[(int64_t)n * p.Hv + hv]
                                  : bf2f(reinterpret_cast<const uint16_t*>(p.beta)[(int64_t)n * p.Hv + hv]);
    const int64_t soff = ((int64_t)n * p.Hv + hv) * DK * DK;

    float kk[8], qq[8];
    f32x4 s[8];
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
        const int c = c0 + rr;
        kk[rr] = bf2f(k[c]);
        qq[rr] = bf2f(q[c]);
        const float eg = fexp(g[c]);
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (p.s_in) x = *reinterpret_cast<const f32x4*>(p.s_in + soff + (int64_t)c * DK + j0);
        s[rr] = x * eg;
    }
    f32x4 u = {0.f, 0.f, 0.f, 0.f}, oq = {0.f, 0.f, 0.f, 0.f};
    float qk = 0.f;
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
        u += kk[rr] * s[rr];
        oq += qq[rr] * s[rr];
        qk += qq[rr] * kk[rr];
    }
    *reinterpret_cast<f32x4*>(&sU[rg][j0]) = u;
    *reinterpret_cast<f32x4*>(&sQ[rg][j0]) = oq;
    if (cg == 0) sQK[rg] = qk;
    __syncthreads();

    if (tid < DK) {
        const int j = tid;
        float uj = 0.f, oj = 0.f, qkt = 0.f;
#pragma unroll
        for (int r = 0; r < DEC_RG; ++r) {
            uj += sU[r][j];
            oj += sQ[r][j];
            qkt += sQK[r];
        }
        const float w = beta * (bf2f(v[j]) - uj);
        sW[j] = w;
        const float o = p.scale * (oj + qkt * w);
        p.o[((int64_t)n * p.Hv + hv) * DK + j] = (uint16_t)(pack_bf2(o, 0.f) & 0xffffu);
    }
    __syncthreads();

    const f32x4 w4 = *reinterpret_cast<const f32x4*>(&sW[j0]);
#pragma unroll
    for (int rr = 0; rr < 8; ++rr)
        *reinterpret_cast<f32x4*>(p.s_out + soff + (int64_t)(c0 + rr) * DK + j0) = s[rr] + kk[rr] * w4;
}

hipError_t launch_kda_decode(const DecodeParams& p, hipStream_t stream) {
    const int64_t nblocks = (int64_t)p.N * p.Hv;
    if (nblocks == 0) return hipSuccess;
    hipLaunchKernelGGL(kda_decode_kernel, dim3((unsigned)nblocks), dim3(DEC_THREADS), 0, stream, p);
    return hipGetLastError();
}

}  // namespace kda

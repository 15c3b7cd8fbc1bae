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
__global__ void __launch_bounds__(CMP_THREADS) kda_compose_kernel(const float* M, const float* b, float* h, int rows,
                                                                 int Hv, int nsteps) {
    __shared__ __attribute__((aligned(16))) float sM[2][DK * MS];   // M of two steps
    __shared__ f32x4 sh[DK][CMP_COLS / 4];                          // the current h columns
    const int item = (int)(blockIdx.x / CMP_GROUPS);   // row * Hv + value head
    const int col0 = (int)(blockIdx.x % CMP_GROUPS) * CMP_COLS;
    const int t = threadIdx.x, i = t >> 1, jq = t & 1;   // output row i, columns col0 + 4 jq .. + 3
    const int64_t head = (int64_t)DK * DK, seg = (int64_t)rows * Hv * head;
    const int64_t me = (int64_t)item * head + (int64_t)i * DK + col0 + 4 * jq;

    f32x4 r[M_LOADS];
    auto load_m = [&](int s) {
        const float* src = M + s * seg + (int64_t)item * head;
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
                       nsteps);
    return hipGetLastError();
}

}  // namespace kda

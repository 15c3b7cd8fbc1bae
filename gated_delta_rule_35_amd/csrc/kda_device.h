// Device helpers shared by the two KDA kernels (intra-chunk and scan).
#pragma once
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
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

constexpr int CH = 64;        // chunk length
constexpr int DK = 128;       // key head dim
constexpr int NTHREADS = 512;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float fexp(float x) { return __expf(x); }
// 2^x on the hardware exp2 (v_exp_f32).
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ half8 lds_h8(const char* smem, int byte_off) {
    return *reinterpret_cast<const half8*>(smem + byte_off);
}

// Raw buffer descriptor over [base, base + bytes): stride 0, 32-bit dwords
// (word 3 = 0x00020000 for gfx9-family raw buffers).  Loads past `bytes` read 0.
// Only the per-lane (VGPR) offset is range-checked, so callers put the whole
// offset there.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Two fp32 values as one 32-bit word of two bf16 (v_cvt_pk_bf16_f32, round to
// nearest even under the default rounding mode).
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2v));
}

// Two fp32 values as one 32-bit word of two fp16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
    half2v h = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

// Work-group barrier for LDS hand-offs only: waits for this wave's LDS
// operations, not for its outstanding global loads, so prefetches stay in
// flight across it.  The asm is also a compiler memory barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Token range of (record) sequence n, clamped to [0, T) so that malformed
// cu_seqlens can never send an access out of bounds.  With segments, sequence n
// is segment n % seg_per_row of batch row n / seg_per_row (segment 0 of
// seg0_tokens tokens, each later one of seg_tokens).
__device__ __forceinline__ void seq_bounds(const KdaParams& p, int n, int64_t& bos, int64_t& len) {
    if (p.cu) {
        int64_t a = p.cu[n], e = p.cu[n + 1];
        a = a < 0 ? 0 : (a > p.T ? p.T : a);
        e = e < a ? a : (e > p.T ? p.T : e);
        bos = a;
        len = e - a;
    } else if (p.seg_tokens) {
        const int b = n / p.seg_per_row, s = n % p.seg_per_row;
        const int64_t off = s == 0 ? 0 : p.seg0_tokens + (int64_t)(s - 1) * p.seg_tokens;
        const int64_t cap = s == 0 ? p.seg0_tokens : p.seg_tokens, rest = p.T - off;
        bos = (int64_t)b * p.T + off;
        len = rest < 0 ? 0 : (rest > cap ? cap : rest);
    } else {
        bos = (int64_t)n * p.T;
        len = p.T;
    }
}

// Sequence n of a scan job: its token range and its record sequence (the index
// the intra kernel's slots were laid out with).  Without segments the two
// indices agree.
__device__ __forceinline__ void job_seq(const KdaParams& p, int n, int64_t& bos, int64_t& len, int& n_rec) {
    n_rec = p.seg_tokens ? (n % p.seg_rows) * p.seg_per_row + p.seg_first + n / p.seg_rows : n;
    seq_bounds(p, n_rec, bos, len);
}

// Workspace slot of chunk c of sequence n (first token bos): floor(start / 64) + n.
// Slots of different chunks differ whenever the sequences do not overlap, and every
// slot is below ceil(total tokens / 64) + N.
__device__ __forceinline__ int64_t chunk_slot(int64_t bos, int n, int64_t c) { return bos / CH + n + c; }

// Index of a lower 16x16 tile (I >= J) of a 64x64 matrix in 0..9, row by row.
__device__ __forceinline__ int tri_index(int I, int J) { return I * (I + 1) / 2 + J; }
// Index of an off-diagonal 16x16 block pair (I > J) in 0..5.
__device__ __forceinline__ int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

// Workspace record of one (chunk, value head): everything the scan kernel needs
// of the chunk besides v, in the precision its MFMAs consume (fp16).  Apart from
// e^{G_last}, it is a list of 1 KB operand fragments of v_mfma_f32_32x32x16_f16:
// 64 lanes x 16 bytes, loaded by the scan kernel's waves straight into registers.
// Fragment (m, kk) of a matrix X holds in lane l the eight elements
// X[32 m + l % 32][16 kk + 8 (l / 32) + s], s = 0 .. 7, unless stated otherwise.
//   WS_AQK  Aqk (scale included), the six lower fragments (m, kk): m = 0, kk < 2
//           and m = 1, kk < 4; index frag_lt(m, kk)
//   WS_T    T diag(beta), the same six, with the columns of each 16-wide k step
//           taken in the order in which a 32x32 MFMA accumulator tile holds its
//           rows: lane l holds columns 16 kk + 8 (s / 4) + 4 (l / 32) + s % 4
//   WS_QG   scale q e^G (64 x 128), fragments (m, kk), m < 2, kk < 8; index 8 m + kk
//   WS_KG   -(k e^G), likewise
//   WS_KH   (k e^{G_last - G})^T (128 x 64), fragments (m, kk), m < 4, kk < 4;
//           index 4 m + kk
//   WS_GAM  e^{G_last}, [128] fp32
constexpr int WS_FRAG = 64 * 16;
__host__ __device__ constexpr int frag_lt(int m, int kk) { return m == 0 ? kk : 2 + kk; }
constexpr int WS_AQK = 0;
constexpr int WS_T = WS_AQK + 6 * WS_FRAG;
constexpr int WS_QG = WS_T + 6 * WS_FRAG;
constexpr int WS_KG = WS_QG + 16 * WS_FRAG;
constexpr int WS_KH = WS_KG + 16 * WS_FRAG;
constexpr int WS_GAM = WS_KH + 16 * WS_FRAG;
constexpr int WS_RECORD_BYTES = WS_GAM + 128 * 4;
static_assert(WS_RECORD_BYTES == 61952, "record size");

}  // namespace kda

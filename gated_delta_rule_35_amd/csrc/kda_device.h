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

// Token range of sequence n, clamped to [0, T) so that malformed cu_seqlens can
// never send an access out of bounds.
__device__ __forceinline__ void seq_bounds(const KdaParams& p, int n, int64_t& bos, int64_t& len) {
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
}

// Workspace slot of chunk c of sequence n (first token bos): floor(start / 64) + n.
// Slots of different chunks differ whenever the sequences do not overlap, and every
// slot is below ceil(total tokens / 64) + N.
__device__ __forceinline__ int64_t chunk_slot(int64_t bos, int n, int64_t c) { return bos / CH + n + c; }

// Index of a lower 16x16 tile (I >= J) of a 64x64 matrix in 0..9, row by row.
__device__ __forceinline__ int tri_index(int I, int J) { return I * (I + 1) / 2 + J; }
// Index of an off-diagonal 16x16 block pair (I > J) in 0..5.
__device__ __forceinline__ int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

// Workspace record of one (chunk, value head): 20 fp16 tiles of 16x16, row-major
// inside a tile: tiles 0..9 hold the lower tiles of Aqk, tiles 10..19 those of
// T diag(beta), both in tri_index order.
constexpr int WS_TILE_BYTES = 16 * 16 * 2;
constexpr int WS_TILES = 20;
constexpr int WS_RECORD_BYTES = WS_TILES * WS_TILE_BYTES;

}  // namespace kda

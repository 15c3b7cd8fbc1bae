// Internal interface between the C-ABI front end and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct KdaParams {
    const uint16_t* q;     // [tokens, Hq, 128] bf16 bits
    const uint16_t* k;     // [tokens, Hq, 128] bf16 bits
    const uint16_t* v;     // [tokens, Hv, 128] bf16 bits
    const float* g;        // [tokens, Hv, 128]
    const void* beta;      // [tokens, Hv] bf16 bits or fp32
    const int32_t* cu;     // [N+1] or nullptr (fixed length)
    const float* h0;       // [N, Hv, 128, 128] or nullptr
    uint16_t* o;           // [tokens, Hv, 128] bf16 bits
    float* hT;             // [N, Hv, 128, 128] or nullptr
    char* ws;              // [nslots, Hv] records of the intra kernel's results
    int64_t nslots;        // ceil(total tokens / 64) + N
    int64_t T;             // tokens per sequence (fixed length) or total tokens (packed)
    int32_t N, Hq, Hv;
    int32_t beta_f32;
    float scale;
    // Optional fp32 dumps of the intermediates (all nullptr in production launches).
    float* tr_G;
    float* tr_Aqk;
    float* tr_Akk;
    float* tr_T;
    float* tr_W;
    float* tr_U;
    float* tr_vnew;
    float* tr_h;
};

// One recurrent step for a batch of single tokens (decode).
struct DecodeParams {
    const uint16_t* q;     // [N, Hq, 128] bf16 bits
    const uint16_t* k;     // [N, Hq, 128] bf16 bits
    const uint16_t* v;     // [N, Hv, 128] bf16 bits
    const float* g;        // [N, Hv, 128]
    const void* beta;      // [N, Hv] bf16 bits or fp32
    const float* s_in;     // [N, Hv, 128, 128] or nullptr (zero state)
    float* s_out;          // [N, Hv, 128, 128]; may equal s_in
    uint16_t* o;           // [N, Hv, 128] bf16 bits
    int32_t N, Hq, Hv;
    int32_t beta_f32;
    float scale;
};

hipError_t launch_kda_decode(const DecodeParams& p, hipStream_t stream);

// Workspace bytes for the given sizes (one record per chunk slot and value head).
int64_t workspace_bytes(int64_t total_tokens, int64_t N, int64_t Hv);

// Intra-chunk kernel: one work-group per (chunk slot, value head), nslots * Hv in all.
hipError_t launch_kda_intra(const KdaParams& p, bool trace, hipStream_t stream);

// Scan kernel: N * Hv * scan_slices() work-groups, each walking one sequence's chunks
// for one slice of the value head's dv columns.
int scan_slices();
hipError_t launch_kda_scan(const KdaParams& p, bool trace, hipStream_t stream);

}  // namespace kda

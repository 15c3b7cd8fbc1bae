// Internal interface between the C-ABI front end and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// One sequence of a scan job given by a list: its record sequence (an index into
// cu), and the [Hv][128][128] blocks its state enters from and leaves to (NULL:
// zero, or the identity with h0_identity; not written).
struct ScanEntry {
    const float* h0;
    float* hT;
    int32_t rec;
    int32_t pad;
};

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
    // Segments (fixed length only; seg_tokens = 0: none).  Row b of the batch is cut
    // into seg_per_row segments: the first of seg0_tokens tokens, the others of
    // seg_tokens (both multiples of 64; the last one may be shorter), and segment s
    // of row b is record sequence b * seg_per_row + s:
    // the intra kernel runs over all of them (N = rows * seg_per_row).  A scan job
    // walks segments seg_first .. seg_first + N / seg_rows - 1 of every row, its
    // sequence n being segment seg_first + n / seg_rows of row n % seg_rows; h0, hT
    // and o are indexed by that n (segment-major).
    int64_t seg_tokens, seg0_tokens;
    int32_t seg_rows, seg_per_row, seg_first;
    // Scan job variants: the state enters as the identity (h0 ignored), and / or v
    // reads as zero.  o == nullptr: no output is written.
    int32_t h0_identity, v_zero;
    // Scan jobs only: sequence n of the job is entries[n] (its token range from cu,
    // its states from the entry), instead of sequence n with h0 / hT indexed by n.
    const ScanEntry* entries;
    // Optional fp32 dumps of the intermediates (all nullptr in production launches).
    float* tr_G;
    float* tr_Aqk;
    float* tr_Akk;
    float* tr_T;
    float* tr_W;
    float* tr_U;
    float* tr_vnew;
    float* tr_h;
    // Optional QG output: q e^G per token, value head and key channel, G the
    // chunk-local inclusive cumsum of g ([tokens, Hv, 128] bf16 bits; nullptr: not
    // written).  Only the intra kernel writes it.
    uint16_t* qg;
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

// Backward pass (kda_bwd.hip) over a fixed-length batch [B, T] or, with cu, N
// sequences packed into one row of T tokens.
struct BwdParams {
    const uint16_t* q;     // [B, T, Hq, 128] bf16 bits
    const uint16_t* k;     // [B, T, Hq, 128] bf16 bits
    const uint16_t* v;     // [B, T, Hv, 128] bf16 bits
    const uint16_t* dO;    // [B, T, Hv, 128] bf16 bits: gradient of the output
    const float* g;        // [B, T, Hv, 128]
    const void* beta;      // [B, T, Hv] bf16 bits or fp32
    const int32_t* cu;     // [N + 1] sequence offsets into the packed row (B = 1), or nullptr
    const float* h0;       // [N, Hv, 128, 128] or nullptr (zero state)
    const float* dhT;      // [N, Hv, 128, 128] gradient of the final state, or nullptr (zero)
    float* dq;             // [B, T, Hq, 128]
    float* dk;             // [B, T, Hq, 128]
    float* dv;             // [B, T, Hv, 128]
    float* dg;             // [B, T, Hv, 128]
    float* dbeta;          // [B, T, Hv]
    float* dh0;            // [N, Hv, 128, 128] or nullptr (not written)
    float* prep;           // [nslots * Hv][BWP_FLOATS]: G, Aqk, T, Abar of each chunk
    float* hs;             // [nslots * Hv][128 * 128]: state entering each chunk
    float* dhs;            // [nslots * Hv][128 * 128]: gradient of the state leaving each chunk
    float* dqv;            // [B, T, Hv, 128]: dq per value head (equals dq when Hq == Hv)
    float* dkv;            // [B, T, Hv, 128]: dk per value head (equals dk when Hq == Hv)
    int64_t T;
    int64_t nslots;         // chunk slots: B * nc, or with cu ceil(T / 64) + N
    int32_t B, N, Hq, Hv, nc;  // N sequences (B without cu); nc = ceil(T / 64) chunks per row
    int32_t beta_f32;
    float scale;
};
constexpr int BWP_G = 0, BWP_AQK = 64 * 128, BWP_T = BWP_AQK + 64 * 64, BWP_ABAR = BWP_T + 64 * 64;
constexpr int BWP_FLOATS = BWP_ABAR + 64 * 64;

hipError_t launch_kda_bwd(const BwdParams& p, hipStream_t stream);

// Size of the static device scratch behind kda_fwd_noalloc (64 MiB), and its
// device address on the current device (looked up once per device).
constexpr int64_t NOALLOC_SCRATCH_BYTES = int64_t(64) << 20;
hipError_t noalloc_scratch(void** out);

// Workspace bytes for the given sizes (one record per chunk slot and value head).
int64_t workspace_bytes(int64_t total_tokens, int64_t N, int64_t Hv);

// Fused forward: one work-group per (sequence, value head, 64-wide dv slice),
// N * Hv * 2 in all; no workspace.
hipError_t launch_kda_fused(const KdaParams& p, hipStream_t stream);

// Intra-chunk kernel: one work-group per (chunk slot, value head), nslots * Hv in all.
hipError_t launch_kda_intra(const KdaParams& p, bool trace, hipStream_t stream);

// Scan kernel: N * Hv * scan_slices() work-groups, each walking one sequence's chunks
// for one slice of the value head's dv columns.
int scan_slices();
hipError_t launch_kda_scan(const KdaParams& p, bool trace, hipStream_t stream);

// Up to three scan jobs in one grid (so that they run side by side): job j has
// job[j].N * job[j].Hv * scan_slices() work-groups; jobs with N = 0 are skipped.
constexpr int MAX_SCAN_JOBS = 3;
struct ScanJobs {
    KdaParams job[MAX_SCAN_JOBS];
    int32_t end[MAX_SCAN_JOBS];   // first work-group past job j (filled by launch_kda_scan_jobs)
    int32_t njobs;
};
hipError_t launch_kda_scan_jobs(ScanJobs jobs, hipStream_t stream);

// Affine maps of consecutive segments composed in order, per (row, value head):
// h_in[s + 1] = M[s] h_in[s] + b[s] for s = 0 .. nsteps - 1, where h_in[0] is given.
// All arrays segment-major: [segment][rows][Hv][128][128] fp32.
// Packed sequences: one chain per sequence, chains[4 n .. 4 n + 2] = (first map,
// first entering state, steps): h[ls + s + 1] = M[ms + s] h[ls + s] + b[ms + s] for
// s < steps, every array [index][Hv][128][128] (chains[4 n + 3]: the sequence's
// first segment, for the plan).
hipError_t launch_kda_compose_chains(const float* M, const float* b, float* h_in, const int32_t* chains, int nchains,
                                     int Hv, hipStream_t stream);

// The segmented forward over packed sequences, planned on the device from
// cu_seqlens: segment boundaries (cu_seg, S_max + 2 entries), the scan jobs'
// entry lists and the chains of the maps to compose (see kda_fwd_cp).
struct CpPlan {
    const int32_t* cu;
    int32_t N;
    int64_t T;                 // tokens of the packed row (clamp bound)
    int64_t L, L0;             // chunks per segment, of the first segment
    int64_t hv_dd;             // Hv * 128 * 128 floats per state
    const float* h0;           // [N][Hv][128][128] or NULL
    float* hT;                 // [N][Hv][128][128] or NULL
    float* Hin;                // [lat_max]: states entering the later segments
    float* Mb;                 // [lat_max]: maps of the middle segments
    float* Bb;                 // [lat_max]: offsets of the middle segments
    int32_t* cu_seg;           // [S_max + 2]
    int32_t S_max, lat_max;
    ScanEntry* first;          // [N]: segment 0 of every sequence
    ScanEntry* mid_m;          // [lat_max]: middle segments, maps
    ScanEntry* mid_b;          // [lat_max]: middle segments, offsets
    ScanEntry* later;          // [lat_max]: segments 1 .. P-1 of every sequence
    int32_t* chains;           // [N][4]
};
hipError_t launch_kda_cp_plan(const CpPlan& pl, hipStream_t stream);

hipError_t launch_kda_compose(const float* M, const float* b, float* h_in, int rows, int Hv, int nsteps,
                              hipStream_t stream);

}  // namespace kda

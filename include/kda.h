/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention forward library.
 *
 * The library computes the chunked forward pass of KDA, the gated delta rule
 * with a per-channel decay, whose GPU stages the pages name ("cuLA PR #131:
 * SM100/SM103 KDA forward to pure CuTeDSL", sections Summary and Numerical
 * behavior: chunk intra, FP32 Akk inversion, recompute W/U, causal masking, tail
 * clamping; "cuLA REPO_LAYOUT.md", ops/ entries for the chunk delta-H and
 * forward-output kernels).  For every sequence n and value head hv the
 * library returns the outputs of the recurrence
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp g_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * evaluated chunk by chunk (chunk length 64) by two HIP kernels: an
 * intra-chunk kernel that runs every chunk at once (gate cumsum, the Aqk and
 * Akk products, the fp32 inversion of I + Akk) and a scan kernel that walks
 * each sequence's chunks in order (W/U recompute, state update, output).  The
 * intra kernel hands its results to the scan kernel through a device
 * workspace of kda_fwd_workspace_size() bytes (61,952 bytes per 64-token chunk
 * slot and value head: Aqk, T diag(beta) and the decayed q and k operands in
 * fp16, laid out as the scan kernel's MFMA operand fragments).
 *
 * Tensors are described by kda_tensor_t: a device pointer, a dtype, a rank
 * and per-dimension sizes and strides counted in elements.  All tensors must
 * be dense row-major (contiguous) and their data 16-byte aligned (beta and
 * cu_seqlens: aligned to their element size); a tensor with no elements may
 * have any strides and a NULL pointer.  The caller owns all memory it
 * passes; the library keeps no pointer after a call returns.
 *
 * Shapes (B batch rows, T tokens per row, Hq query/key heads, Hv value heads,
 * head dimension 128):
 *   q, k           [B, T, Hq, 128]  bf16
 *   v              [B, T, Hv, 128]  bf16
 *   g              [B, T, Hv, 128]  fp32 log-decay (the activated gate, <= 0)
 *   beta           [B, T, Hv]       bf16 or fp32
 *   cu_seqlens     [N + 1]          int32, or NULL.  With cu_seqlens, B must be 1
 *                                   and row 0 packs N sequences back to back:
 *                                   sequence n covers tokens
 *                                   [cu_seqlens[n], cu_seqlens[n+1]).  Without it,
 *                                   N = B and batch row b is sequence b.
 *   initial_state  [N, Hv, 128, 128] fp32 (key channel, value channel), or NULL
 *                                   for a zero state
 *   out            [B, T, Hv, 128]  bf16
 *   final_state    [N, Hv, 128, 128] fp32, or NULL (not written)
 * Grouped-value attention: Hq must divide Hv; value head hv reads query/key
 * head hv / (Hv / Hq).  Every sequence is cut into chunks of 64 tokens from its
 * own start; the last chunk may be partial.  Output rows of tokens that lie in
 * no sequence (packed mode) are not written.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KDA_BF16 = 0, KDA_F16 = 1, KDA_F32 = 2, KDA_I32 = 3 } kda_dtype_t;

typedef struct {
    void* data;          /* device pointer; may be NULL only if the tensor has no elements */
    kda_dtype_t dtype;
    int32_t ndim;        /* 1..4 */
    int64_t shape[4];
    int64_t stride[4];   /* in elements */
} kda_tensor_t;

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,        /* a required descriptor or data pointer is NULL */
    KDA_ERR_DTYPE = 2,       /* a dtype outside the table above */
    KDA_ERR_SHAPE = 3,       /* ranks or sizes that disagree with each other */
    KDA_ERR_LAYOUT = 4,      /* non-contiguous strides or misaligned data */
    KDA_ERR_UNSUPPORTED = 5, /* head dim != 128, Hv % Hq != 0, B != 1 with cu_seqlens, grid too large */
    KDA_ERR_VALUE = 6,       /* scale not finite or not > 0 */
    KDA_ERR_HIP = 7,         /* the HIP runtime reported an error at launch or allocation */
    KDA_ERR_WORKSPACE = 8    /* entry points with a workspace: missing, too small or misaligned */
} kda_status_t;

/*
 * kda_fwd -- the KDA forward pass over a batch.
 *
 * Two forms compute it: the single-pass kernel of kda_fwd_fused, and two
 * kernels (chunk-parallel intra work, then the sequential scan) that hand each
 * chunk's operands over through a device workspace.  kda_fwd takes the
 * single-pass kernel for fixed-length batches (no cu_seqlens) of at least 1024
 * tokens per row whose B * Hv * 2 work-groups cover every compute unit of the
 * current device, and the two-pass kernels otherwise; the two forms round
 * differently in the last bits (see Precision), and for a given shape and
 * device the choice never changes.
 *
 * Enqueues the work on `stream` (a hipStream_t; NULL is the null stream) and
 * returns without waiting: the host never reads device memory, so the number of
 * sequences comes from the shape of cu_seqlens, not its values.  Every argument
 * is checked on the host before any HIP call; on an error nothing is enqueued.
 * Results are bitwise reproducible from call to call (no atomics; each output
 * element has exactly one writer and a fixed reduction order).
 * initial_state may alias final_state (each state tile is read before it is
 * written, by the same work-group); a partial overlap of the two returns
 * KDA_ERR_LAYOUT.
 * The two-pass form needs a workspace: kda_fwd allocates it with
 * hipMallocAsync on `stream` and releases it with hipFreeAsync on it, so calls
 * on different streams never share it (kda_fwd_ws takes the caller's instead);
 * the single-pass form allocates nothing.
 * cu_seqlens must be non-decreasing with cu_seqlens[0] = 0 and
 * cu_seqlens[N] <= T.  That is a precondition the host cannot check without a
 * device read; the kernel clamps every sequence to [0, T) so that malformed
 * values never cause an out-of-bounds access.
 * Precision: q, k, v are bf16; the MFMA operands derived from them are fp16
 * and all accumulation, the gate cumsum, the inversion and the state are
 * fp32.  In the two-pass form, a chunk whose decay within a 16-token block
 * exceeds exp(-8) on some channel takes an exact fp32 path for its diagonal
 * blocks; the single-pass form anchors per chunk (see kda_fwd_fused).  The fp16
 * operands bound the range: entries of the state and of v_new must stay
 * below 65504 in magnitude (L2-normalised q and k, values of order one and
 * g <= 0 keep them orders of magnitude below it).
 */
kda_status_t kda_fwd(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v,
                     const kda_tensor_t* g, const kda_tensor_t* beta, float scale,
                     const kda_tensor_t* cu_seqlens, const kda_tensor_t* initial_state,
                     const kda_tensor_t* out, const kda_tensor_t* final_state, void* stream);

/*
 * kda_fwd_fused -- the single-pass form of the forward ("cuLA PR #131: SM100/SM103
 * KDA forward to pure CuTeDSL", Summary: chunk intra, FP32 Akk inversion,
 * recompute W/U; "cuLA REPO_LAYOUT.md", ops/: chunk delta-H and forward output,
 * and the fused-forward entries): one persistent work-group per (sequence, value
 * head, 64-wide dv slice) builds each chunk's operands, Aqk and T in LDS while it
 * scans the previous chunk, so nothing but q, k, v, g, beta, the states and o
 * crosses HBM.  Same arguments, checks, results semantics and reproducibility as
 * kda_fwd, and it allocates nothing (it can be captured into a HIP graph).
 * Precision: as kda_fwd's, except that the decay anchor is per 64-token chunk:
 * a chunk whose total decay exceeds exp(-16) on some channel takes an exact fp32
 * path (Aqk and Akk element by element, operands with every factor <= 1).
 * It runs N * Hv * 2 work-groups of 512 threads with about 153 KB of LDS each,
 * one per CU: it is meant for batches with at least that many work-groups and
 * sequences of equal length; kda_fwd takes it by itself where that holds (see
 * kda_fwd), and with fewer work-groups or packed sequences of unequal length
 * the two-pass form is faster.  More than 2^31 - 1 work-groups return
 * KDA_ERR_UNSUPPORTED.
 */
kda_status_t kda_fwd_fused(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v,
                           const kda_tensor_t* g, const kda_tensor_t* beta, float scale,
                           const kda_tensor_t* cu_seqlens, const kda_tensor_t* initial_state,
                           const kda_tensor_t* out, const kda_tensor_t* final_state, void* stream);

/*
 * kda_fwd_workspace_size -- bytes of device workspace kda_fwd_ws needs for a
 * call with `total_tokens` = B * T tokens, N sequences and Hv value heads:
 * (ceil(total_tokens / 64) + N) * Hv * 61952.  Returns -1 for a negative size.
 */
int64_t kda_fwd_workspace_size(int64_t total_tokens, int64_t num_sequences, int64_t num_value_heads);

/*
 * kda_fwd_ws -- the two-pass form of the forward with a caller-owned workspace:
 * an intra-chunk kernel over every chunk at once writes one record per chunk
 * and value head to `workspace`, and a scan kernel walks each sequence's chunks
 * in order, reading them.  Same arguments, checks, results and semantics as
 * kda_fwd, plus:
 * workspace: device memory of at least kda_fwd_workspace_size() bytes,
 * 16-byte aligned, owned by the caller and not used by anything else until the
 * call's work on `stream` has finished; its contents need no initialisation.
 * NULL, a smaller size or a misaligned pointer return KDA_ERR_WORKSPACE.
 * The call allocates nothing and records no memset, so it can be captured into
 * a HIP graph.
 */
kda_status_t kda_fwd_ws(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v,
                        const kda_tensor_t* g, const kda_tensor_t* beta, float scale,
                        const kda_tensor_t* cu_seqlens, const kda_tensor_t* initial_state,
                        const kda_tensor_t* out, const kda_tensor_t* final_state,
                        void* workspace, int64_t workspace_size, void* stream);

/*
 * kda_fwd_qg -- the forward with its optional QG output ("cuLA PR #131: SM100/
 * SM103 KDA forward to pure CuTeDSL", Summary, lists an optional QG among the
 * forward's outputs and its Changes table the intra and recompute paths that
 * produce it; no page defines it).  Read here as the decayed query of the output
 * product, before the scale:
 *   qg[b, t, hv, c] = q[b, t, hv / (Hv / Hq), c] * exp(G[b, t, hv, c]),
 * G the chunk-local inclusive cumsum of g (chunks of 64 tokens from each
 * sequence's start), computed in fp32 and rounded once to bf16 (nearest even).
 * qg: [B, T, Hv, 128] bf16 (v's shape), contiguous, 16-byte aligned, device
 * memory owned by the caller, sharing no byte with any other tensor argument;
 * NULL returns KDA_ERR_NULL.  Rows of tokens outside every sequence (packed
 * batches whose last offset is below T) are not written.
 * workspace, workspace_size: as kda_fwd_ws; workspace NULL allocates the
 * records in stream order on `stream`, as kda_fwd does.
 * out and final_state are bitwise those of kda_fwd_ws on the same inputs.
 * Errors: as kda_fwd_ws, plus KDA_ERR_DTYPE / KDA_ERR_SHAPE / KDA_ERR_LAYOUT for
 * a qg of the wrong dtype, shape, layout or one that overlaps another tensor.
 */
kda_status_t kda_fwd_qg(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v,
                        const kda_tensor_t* g, const kda_tensor_t* beta, float scale,
                        const kda_tensor_t* cu_seqlens, const kda_tensor_t* initial_state,
                        const kda_tensor_t* out, const kda_tensor_t* final_state, const kda_tensor_t* qg,
                        void* workspace, int64_t workspace_size, void* stream);

/*
 * kda_fwd_noalloc --kda_fwd_ws without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * The records live in a static device array of kda_fwd_noalloc_max_bytes()
 * bytes (64 MiB) that each GPU the library runs on holds from module load
 * until the process ends.  A call whose kda_fwd_workspace_size() exceeds it
 * returns KDA_ERR_WORKSPACE before any HIP call.  Results are bitwise those of
 * kda_fwd_ws.  Every call on one GPU uses that GPU's array, which keeps the
 * last call's contents (no call relies on them: every record a call reads it
 * writes first): calls that overlap on one GPU (two streams or two host
 * threads) race and must not be made.  The first call on a device looks up the
 * array's device address (hipGetSymbolAddress) with that device current.
 */
kda_status_t kda_fwd_noalloc(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v,
                             const kda_tensor_t* g, const kda_tensor_t* beta, float scale,
                             const kda_tensor_t* cu_seqlens, const kda_tensor_t* initial_state,
                             const kda_tensor_t* out, const kda_tensor_t* final_state, void* stream);
/* Size of kda_fwd_noalloc's static scratch per GPU, in bytes. */
int64_t kda_fwd_noalloc_max_bytes(void);

/*
 * kda_fwd_cp -- kda_fwd with each sequence cut into segments that the scan walks
 * side by side (context parallelism inside one GPU), for batches whose number of
 * (sequence, value head) pairs is too small to fill the chip.
 *
 * The scan walks a sequence's chunks one after another, so B * Hv * 2
 * work-groups are all that can run at once: with few heads most of the GPU
 * idles through a long sequence.  Over one segment the chunked recurrence is
 * affine in the state that enters it, h_out = M h_in + b, and M and b do not
 * depend on h_in (the state maps of the chunked method, "cuLA REPO_LAYOUT.md",
 * the chunk delta-H entry; the recurrence is the one above).  Segment 0 covers
 * the first first_segment_chunks chunks of its row (0: segment_chunks), each
 * later segment the next segment_chunks (the last may be shorter); with P
 * segments per row the call runs
 *   1. the intra-chunk kernel over every segment;
 *   2. side by side: segment 0 of each row from initial_state, and, for segments
 *      1 .. P-2, M (from the identity with v = 0) and b (from zero with v);
 *   3. the entering states h_in[s + 1] = M[s] h_in[s] + b[s], in fp32;
 *   4. side by side: segments 1 .. P-1 from their entering states.
 * The sequential depth is segment 0's chunks plus one later segment's (steps 2
 * and 4) instead of the whole row, at the price of 2 (P - 2) + 1 times the scan
 * work-groups of an ordinary call in step 2; it pays when B * Hv * 2 is well
 * below the number of CUs and the sequences are long.  A first segment longer
 * than the others lets the maps run in several waves beside it.
 *
 * Arguments are kda_fwd's, plus segment_chunks >= 1 and first_segment_chunks >= 0
 * (KDA_ERR_VALUE otherwise).  workspace (required, caller-owned, no
 * initialisation) must hold kda_fwd_cp_workspace_size() bytes (16-byte aligned)
 * for a fixed-length batch, kda_fwd_cp_packed_workspace_size() bytes (256-byte
 * aligned) with cu_seqlens.
 * Fixed length (cu_seqlens NULL): the segment boundaries follow from the shapes;
 * with fewer than three segments per row the call is exactly kda_fwd.
 * Packed sequences (cu_seqlens given, B = 1): every sequence is cut the same way
 * from its own start (P = 1 segment when it has at most first_segment_chunks
 * chunks); since the host never reads cu_seqlens, a plan kernel derives the
 * segments, the steps' work lists and the composition chains on the device,
 * within bounds computed from the shapes (at most N + TC / L + min(N, TC / (L0 +
 * 1)) + 1 segments for TC = ceil(T / 64) + N chunks), and the steps run over the
 * bounds (work past the actual counts exits at once).  A sequence with one or two
 * segments gets kda_fwd's results bit for bit; with malformed cu_seqlens the
 * results are undefined but every access stays in bounds.  The call launches
 * kernels only and can be captured into a HIP graph.
 * Results are bitwise repeatable; they agree with kda_fwd to within the rounding
 * of the fp16 MFMA operands (the maps are formed with the same operand precision
 * as the state), not bit for bit.  initial_state may alias final_state.
 */
/*
 * kda_fwd_cp_plan -- segment lengths (in 64-token chunks) for kda_fwd_cp on a
 * GPU with num_cus compute units.  Returns 1 and fills segment_chunks and
 * first_segment_chunks (either pointer may be NULL) when the segmented call is
 * expected to save a fifth or more; returns 0 and writes zeros when the ordinary
 * kda_fwd is about as fast (B * Hv fills the GPU, or the sequences are short).
 * Host arithmetic only: it minimises the chunk steps of the scan's waves of
 * work-groups, plus the composition steps and the extra launches.
 */
int32_t kda_fwd_cp_plan(int64_t batch, int64_t seq_len, int64_t num_value_heads, int32_t num_cus,
                        int64_t* segment_chunks, int64_t* first_segment_chunks);
/* Workspace bytes of a kda_fwd_cp call; -1 for negative sizes or segment_chunks < 1. */
int64_t kda_fwd_cp_workspace_size(int64_t batch, int64_t seq_len, int64_t num_value_heads, int64_t segment_chunks,
                                  int64_t first_segment_chunks);
/* Workspace bytes of a kda_fwd_cp call on packed sequences: total_tokens = T of
 * the packed row, num_sequences = N; -1 for negative sizes or segment_chunks < 1. */
int64_t kda_fwd_cp_packed_workspace_size(int64_t total_tokens, int64_t num_sequences, int64_t num_value_heads,
                                         int64_t segment_chunks, int64_t first_segment_chunks);
kda_status_t kda_fwd_cp(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v,
                        const kda_tensor_t* g, const kda_tensor_t* beta, float scale,
                        const kda_tensor_t* cu_seqlens, const kda_tensor_t* initial_state,
                        const kda_tensor_t* out, const kda_tensor_t* final_state, int64_t segment_chunks,
                        int64_t first_segment_chunks, void* workspace, int64_t workspace_size, void* stream);

/*
 * kda_fwd_intra, kda_fwd_scan -- the two kernels of kda_fwd as separate calls,
 * for callers that schedule them apart (e.g. the next batch's intra kernel on
 * another stream) or time them one by one.  kda_fwd_intra fills the workspace
 * (gate cumsum, Aqk, Akk, the inversion); kda_fwd_scan reads it and writes out
 * and final_state.  Both take kda_fwd's arguments and checks; the workspace is
 * required (NULL gives KDA_ERR_WORKSPACE).  kda_fwd_intra followed by
 * kda_fwd_scan with the same arguments, in stream order, gives exactly
 * kda_fwd's results.
 */
kda_status_t kda_fwd_intra(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v,
                           const kda_tensor_t* g, const kda_tensor_t* beta, float scale,
                           const kda_tensor_t* cu_seqlens, const kda_tensor_t* initial_state,
                           const kda_tensor_t* out, const kda_tensor_t* final_state,
                           void* workspace, int64_t workspace_size, void* stream);
kda_status_t kda_fwd_scan(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v,
                          const kda_tensor_t* g, const kda_tensor_t* beta, float scale,
                          const kda_tensor_t* cu_seqlens, const kda_tensor_t* initial_state,
                          const kda_tensor_t* out, const kda_tensor_t* final_state,
                          void* workspace, int64_t workspace_size, void* stream);

/*
 * Optional fp32 dumps of the chunked method's intermediates, for stage-by-stage
 * checks of kda_fwd_trace.  Any pointer may be NULL.  Ttot = B * T.
 *   G     [Ttot, Hv, 128]  chunk-local inclusive cumsum of g
 *   Aqk   [Ttot, Hv, 64]   row of scale * sum_c q_i k_j exp(G_i - G_j), j <= i
 *   Akk   [Ttot, Hv, 64]   row of beta_i * sum_c k_i k_j exp(G_i - G_j), j < i
 *   T     [Ttot, Hv, 64]   row of (I + Akk)^{-1}
 *   W     [Ttot, Hv, 128]  T (beta k exp G)
 *   U     [Ttot, Hv, 128]  T (beta v)
 *   v_new [Ttot, Hv, 128]  U - W h
 *   h     [num_chunks, Hv, 128, 128]  state entering each chunk; chunks are
 *         numbered by sequence, then by position within the sequence
 * Row t of a per-token dump belongs to the token's own chunk; columns past the
 * chunk's length are zero.  Rows of tokens in no sequence are not written.
 */
typedef struct {
    float* G;
    float* Aqk;
    float* Akk;
    float* T;
    float* W;
    float* U;
    float* v_new;
    float* h;
} kda_trace_t;

/*
 * kda_fwd_trace -- kda_fwd plus the dumps above (a test and debugging entry; the
 * same kernels with the extra stores compiled in).  Same arguments, checks and
 * results as kda_fwd; `trace` may not be NULL.
 */
kda_status_t kda_fwd_trace(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v,
                           const kda_tensor_t* g, const kda_tensor_t* beta, float scale,
                           const kda_tensor_t* cu_seqlens, const kda_tensor_t* initial_state,
                           const kda_tensor_t* out, const kda_tensor_t* final_state,
                           void* workspace, int64_t workspace_size,
                           const kda_trace_t* trace, void* stream);

/*
 * kda_decode -- one recurrent step for a batch of N single tokens: the decode
 * half of inference, continuing from a state such as kda_fwd's final_state
 * ("cuLA REPO_LAYOUT.md", entry decode/: the KDA decode reference).  For every
 * sequence n and value head hv (q/k head hv / (Hv / Hq)):
 *
 *     S' = (I - beta k k^T) Diag(exp g) S + beta k v^T,   o = scale * S'^T q
 *
 * with S = state_in[n, hv] (a zero state when state_in is NULL) and S' written
 * to state_out[n, hv].  Shapes: q, k [N, Hq, 128] bf16; v [N, Hv, 128] bf16;
 * g [N, Hv, 128] fp32 log-decay; beta [N, Hv] bf16 or fp32; states
 * [N, Hv, 128 (key), 128 (value)] fp32; out [N, Hv, 128] bf16.  All arithmetic is
 * fp32; o is rounded to bf16 once.  state_out may be state_in itself (in-place
 * update) or a separate buffer; a partial overlap returns KDA_ERR_LAYOUT.
 * Memory is caller-owned; the call allocates nothing and is asynchronous on
 * `stream`; repeated calls give bitwise-identical results.  Errors as for kda_fwd.
 */
kda_status_t kda_decode(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v,
                        const kda_tensor_t* g, const kda_tensor_t* beta, float scale,
                        const kda_tensor_t* state_in, const kda_tensor_t* state_out,
                        const kda_tensor_t* out, void* stream);

/*
 * kda_bwd_workspace_size -- bytes of device workspace kda_bwd needs for
 * total_tokens = B * T tokens in num_sequences sequences (B for a fixed-length
 * batch, N with cu_seqlens) with Hq query/key heads and Hv value heads: per
 * value head and each of ceil(total_tokens / 64) + num_sequences chunk slots,
 * 80 KB of chunk operands and two 64 KB states; when Hq < Hv, also
 * 2 * total_tokens * Hv * 512 bytes for dq and dk per value head.  Returns -1
 * for negative sizes or non-positive head counts.
 */
int64_t kda_bwd_workspace_size(int64_t total_tokens, int64_t num_sequences, int64_t num_qk_heads,
                               int64_t num_value_heads);

/*
 * kda_bwd -- gradients of kda_fwd with respect to q, k, v, g, beta and the
 * initial state, given the gradients of the output (d_out) and of the final
 * state (d_final_state, NULL for zero).
 *
 * The pages list the chunk backward among the library's KDA kernels ("cuLA
 * REPO_LAYOUT.md", the kda/ entries for chunk_bwd and the WY dq/dk/dg kernels)
 * without equations, and the bot summary of "cuLA PR #131" (New Features) has
 * the forward and backward take packed variable-length inputs.  This is the
 * exact gradient of the recurrence above, evaluated through the chunk form of
 * the forward (64-token chunks from each sequence's start): a forward walk
 * over each sequence's chunks stores the state entering each, a backward walk
 * carries the state gradient, and a chunk-parallel pass forms the token
 * gradients.  All arithmetic is fp32; the contractions run on fp32 matrix
 * instructions.
 *
 * Shapes and dtypes (B, T, Hq, Hv, N as for kda_fwd, head dimension 128):
 *   q, k, v, g, beta, cu_seqlens, initial_state   as for kda_fwd (cu_seqlens
 *                    and initial_state may be NULL)
 *   d_out            [B, T, Hv, 128]      bf16
 *   d_final_state    [N, Hv, 128, 128]    fp32, or NULL
 *   dq, dk           [B, T, Hq, 128]      fp32 (summed over the value heads of a group)
 *   dv, dg           [B, T, Hv, 128]      fp32
 *   dbeta            [B, T, Hv]           fp32
 *   d_initial_state  [N, Hv, 128, 128]    fp32, or NULL (not computed)
 * With cu_seqlens, gradient rows of tokens that lie in no sequence are not
 * written, and an empty sequence passes d_final_state through to its
 * d_initial_state.  Outputs must not overlap inputs or each other.
 * workspace: device memory of at least kda_bwd_workspace_size(B * T, N, Hq, Hv)
 * bytes, 256-byte aligned, owned by the caller and not used by anything else
 * until the call's work on `stream` has finished; NULL makes the library
 * allocate it with hipMallocAsync on `stream` and release it with
 * hipFreeAsync.  Checks, error codes, the cu_seqlens precondition, stream
 * semantics and reproducibility are those of kda_fwd; the call does not
 * synchronise.
 */
kda_status_t kda_bwd(const kda_tensor_t* q, const kda_tensor_t* k, const kda_tensor_t* v,
                     const kda_tensor_t* g, const kda_tensor_t* beta, float scale,
                     const kda_tensor_t* cu_seqlens, const kda_tensor_t* initial_state,
                     const kda_tensor_t* d_out, const kda_tensor_t* d_final_state, const kda_tensor_t* dq,
                     const kda_tensor_t* dk, const kda_tensor_t* dv, const kda_tensor_t* dg,
                     const kda_tensor_t* dbeta, const kda_tensor_t* d_initial_state, void* workspace,
                     int64_t workspace_size, void* stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* kda_status_string(kda_status_t status);

/* Number of dv slices (scan work-groups per sequence and value head) that
 * kda_fwd launches for N sequences and Hv value heads: 2 (64 dv columns each). */
int32_t kda_dv_slices(int64_t num_sequences, int64_t num_value_heads);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */

/*
 * kda.h - C ABI of the MI355X (gfx950) KDA forward prefill library (libkda.so).
 *
 * Kimi Delta Attention forward, one chain = one sequence x one head,
 * K = V = 128, chunk C = 16 tokens:
 *   q^ = q / sqrt(|q|^2 + 1e-6), k^ likewise; b = sigmoid(beta);
 *   l  = lower_bound * sigmoid(exp(A_log[h]) * (g + dt_bias[h]))  (per key channel)
 *   S_t = (I - b_t k^_t k^_t^T) Diag(exp(l_t)) S_{t-1} + b_t k^_t v_t^T;  o_t = scale * S_t^T q^_t
 * The state tensors hold S^T: element [n][h][v][k] = S[k][v].
 *
 * Interface from the pages: "How to Use FlashKDA as a Backend for
 * flash-linear-attention", sections "Kernel API and Tensor Requirements" (dtypes,
 * shapes, lower_bound range) and "State Handling and Variable-Length Batches"
 * (state [B,H,V,K] or [N,H,V,K], cu_seqlens with B = 1); "How FlashKDA
 * Integrates with CUTLASS", sections "Workspace Allocation and Memory Alignment"
 * (caller-allocated uint8 workspace sized by get_workspace_size(B*T, H)) and
 * "State Management and Accumulator Types" (bf16 or fp32 states); cuLA PR #106,
 * commit list (K1 chunk prep / K2 recurrence, CHUNK = 16; segment split
 * K1 -> pre_scan -> merge -> segment K2, said to be bit-identical to serial)
 * and review thread (use_intracard_cp auto / True / False; no implicit
 * conversions).  Here the segmented result has the serial path's bits
 * whenever every segment's transition M underflows to exactly zero in fp32
 * and the zero-start state has converged to the serial one by the segment's
 * checkpoint (strong decay, e.g. lower_bound -5 over 256-chunk segments);
 * otherwise it equals the serial result within rounding (fp32 merge).
 *
 * Conventions for every call below:
 *  - All tensor pointers are DEVICE pointers, contiguous, in the layouts stated.
 *    The library never dereferences them on the host, never allocates, never
 *    frees, never synchronises and never copies device -> host.
 *  - kda_fwd is asynchronous on `stream` (a hipStream_t; NULL = default stream).
 *  - Validation happens before any launch.  On error the status is negative,
 *    nothing is launched, the outputs are untouched and kda_last_error() holds
 *    a message.  There are no implicit dtype or layout conversions.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_HEAD_DIM 128
#define KDA_CHUNK 16
#define KDA_WORKSPACE_ALIGN 256

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARG = -1,          /* bad pointer, size, range or combination */
  KDA_ERR_UNSUPPORTED = -2,          /* valid request this library does not implement (D != 128) */
  KDA_ERR_WORKSPACE_TOO_SMALL = -3,  /* workspace_bytes < kda_get_workspace_size(...) */
  KDA_ERR_HIP = -4                   /* a HIP launch failed */
} kda_status;

typedef enum { KDA_STATE_BF16 = 0, KDA_STATE_FP32 = 1 } kda_state_dtype;
/* Layout of the caller's state tensors: [N, H, V, K] (the transposed layout
 * the kernel API requires, "State Handling and Variable-Length Batches") or
 * [N, H, K, V] (the chunk_kda call with transpose_state_layout=False). */
typedef enum { KDA_STATE_VK = 0, KDA_STATE_KV = 1 } kda_state_layout;

/* Segment split of long sequences (the intracard context-parallel switch of
 * the cuLA PR #106 page, with its automatic, off and on settings). */
typedef enum { KDA_CP_AUTO = 0, KDA_CP_OFF = 1, KDA_CP_FORCE = 2 } kda_cp_mode;

/* Planned segment length, in chunks of 16 tokens, for these sizes: 0 means
 * serial (one segment per sequence).  Pure host arithmetic.
 *   total_tokens : B*T (all batch rows, or the packed varlen length)
 *   num_heads    : H >= 1;  num_seqs: N >= 1 (B for fixed length)
 *   cp_mode      : kda_cp_mode;  seg_chunks: > 0 forces that segment length in
 *                  AUTO and FORCE modes, 0 lets the library choose.
 * With seg_chunks > 0 the call uses exactly this length.  With seg_chunks 0
 * it is the shortest length the call may use, and the one the workspace is
 * sized for: once the sequence lengths are known (on the device, for a varlen
 * call; kda_fixed_seg_chunks, for a fixed-length one) the call may take a
 * longer one, by at most a quarter and 63 chunks, where a model of how the
 * hardware places the (segment, head) workgroups predicts a shorter run (a
 * varlen call may also dispatch its shorter segments longest first).  It
 * does so for at most 16 sequences, H a multiple of 8 and N*H <= 256, and, in
 * a varlen call, where the planned length is at least 128 chunks.  The
 * length in use is in the counters and in every unit_tab row of the
 * workspace (kda_ws_offset).  Every length gives the same results.
 * Returns a negative kda_status on invalid arguments. */
int32_t kda_plan_seg_chunks(int64_t total_tokens, int32_t num_heads, int32_t num_seqs,
                            int32_t cp_mode, int32_t seg_chunks);

/* Segment length a fixed-length kda_fwd call (B sequences of T tokens, no
 * cu_seqlens) uses, with the arguments of that call: kda_plan_seg_chunks(B*T,
 * num_heads, B, cp_mode, seg_chunks), possibly lengthened as described there.
 * Pure host arithmetic.  Returns a negative kda_status on invalid arguments. */
int32_t kda_fixed_seg_chunks(int32_t B, int64_t T, int32_t num_heads, int32_t cp_mode, int32_t seg_chunks);

/* The segment plan a varlen kda_fwd call (cu_seqlens, B = 1) takes for these
 * sequence lengths, as its index kernel chooses it on the device, with a
 * workspace of at least kda_get_workspace_size(..., KDA_CP_FORCE, 0) bytes
 * (see kda_fwd, cp_mode):
 * *seg_out = the segment length (0: serial), *order_out = 1 where units are
 * dispatched longest first (the workspace counters' order: the shorter
 * segments after the full ones, or for a serial plan of at most 256 sequences
 * every sequence), else 0.  seq_lens: host int32[num_seqs], each >= 0; the other arguments as for
 * kda_plan_seg_chunks.  Pure host arithmetic.  Returns KDA_OK or a negative
 * kda_status on invalid arguments. */
int32_t kda_varlen_seg_choice(const int32_t* seq_lens, int32_t num_seqs, int32_t num_heads, int32_t cp_mode,
                              int32_t seg_chunks, int32_t* seg_out, int32_t* order_out);

/* Workspace bytes kda_fwd needs for these sizes and this plan (the pages'
 * get_workspace_size(B*T, H), plus the sequence count and segment plan, since
 * per-chunk and per-segment buffers scale with them).  Pure host arithmetic,
 * no device calls.  Returns 0 on invalid arguments (see kda_last_error). */
size_t kda_get_workspace_size(int64_t total_tokens, int32_t num_heads, int32_t num_seqs,
                              int32_t cp_mode, int32_t seg_chunks);

/* KDA forward.
 *   q, k, v, g   : bf16 [B, T, H, 128], contiguous
 *   beta         : bf16 [B, T, H] (logits; the sigmoid is applied inside)
 *   scale        : output scale (finite)
 *   out          : bf16 [B, T, H, 128], written (RNE)
 *   A_log        : fp32 [H];  dt_bias: fp32 [H, 128]
 *   lower_bound  : in [-5, 0]
 *   initial_state: NULL or [N, H, 128(V), 128(K)] in state_dtype (read)
 *   final_state  : NULL or [N, H, 128(V), 128(K)] in state_dtype (written);
 *                  may alias initial_state.  Any of the four presence
 *                  combinations is valid.
 *   state_dtype  : kda_state_dtype, applies to whichever state is present
 *   state_layout : kda_state_layout of both states (KDA_STATE_KV: [N, H,
 *                  128(K), 128(V)] instead)
 *   cu_seqlens   : NULL (fixed length, N = B) or int32 [num_seqs + 1] device
 *                  offsets into the packed token axis (then B must be 1).
 *                  Offsets are clamped into a non-decreasing sequence within
 *                  [0, B*T] on the device, so malformed offsets cannot cause
 *                  out-of-bounds access; they are not otherwise diagnosed.
 *   num_seqs     : N; with cu_seqlens == NULL it must equal B (or be 0)
 *   B, T, H, D   : D must be 128; H heads for v, g, beta, out, A_log, dt_bias
 *                  and the states (one recurrence per sequence and head)
 *   H_qk         : heads of q and k (0 means H).  When H_qk < H it must divide
 *                  H, and head h uses q and k of head h / (H / H_qk) (grouped
 *                  value heads: q and k are [B, T, H_qk, 128]; the reading of
 *                  "HV > H" on the cuLA PR #106 page that this library takes)
 *   workspace    : device buffer, KDA_WORKSPACE_ALIGN-aligned, of at least
 *                  kda_get_workspace_size(B*T, H, N, cp_mode, seg_chunks) bytes;
 *                  owned by the caller, clobbered by the call, and must not be
 *                  shared by calls that may overlap.
 *   cp_mode, seg_chunks : segment plan, as for kda_plan_seg_chunks.  A varlen
 *                  call on the automatic plan (KDA_CP_AUTO, seg_chunks 0) with
 *                  N*H >= 256 chains, which that plan keeps serial, splits its
 *                  sequences after all when its workspace also holds the
 *                  segmented layout (kda_get_workspace_size with KDA_CP_FORCE)
 *                  and, seen on the device, its longest sequence has more than
 *                  5/4 of the planned segment length: a skewed batch (one long
 *                  prompt among short ones) then runs in segments instead of
 *                  leaving the long chains as the whole pass.  The tables then
 *                  follow kda_workspace_offsets with KDA_CP_FORCE.  The plan
 *                  in use is in the workspace counters.
 *   stream       : hipStream_t to launch on (NULL = default stream)
 * B*T == 0 with no final_state returns KDA_OK without a launch. */
int32_t kda_fwd(const void* q, const void* k, const void* v, const void* g, const void* beta,
                float scale, void* out, const float* A_log, const float* dt_bias, float lower_bound,
                const void* initial_state, void* final_state, int32_t state_dtype, int32_t state_layout,
                const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int64_t T, int32_t H, int32_t H_qk,
                int32_t D, void* workspace, size_t workspace_bytes, int32_t cp_mode, int32_t seg_chunks,
                void* stream);

/* kda_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, and harnesses that forbid hipMalloc.
 * Same arguments, meaning and errors as kda_fwd, minus the workspace.  Its
 * scratch is one array of KDA_NOALLOC_SCRATCH_BYTES bytes per GPU, built into
 * the library and held from the library's first use of that GPU until the
 * process ends.  The call itself allocates and frees nothing, and never
 * synchronises.
 *   - The call runs on the device of `stream` (the current device for NULL).
 *   - A call whose kda_get_workspace_size(B*T, H, N, cp_mode, seg_chunks)
 *     exceeds KDA_NOALLOC_SCRATCH_BYTES returns KDA_ERR_WORKSPACE_TOO_SMALL
 *     before any launch (a longer seg_chunks, or KDA_CP_OFF, needs less).
 *     A segmented plan needs about 320 KiB per (segment, head) unit plus the
 *     index tables: one sequence of 64K tokens at H = 16 on the automatic
 *     plan takes 85 MiB, a serial plan of it 30 KiB.
 *   - The array counts as the workspace room for kda_fwd's skewed-batch
 *     split: a varlen call on the automatic plan with N*H >= 256 chains may
 *     split wherever the segmented layout fits in it, so it matches a kda_fwd
 *     call given a workspace of at least the KDA_CP_FORCE size, not one of the
 *     automatic plan's size.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents; no part of it needs to start at zero.  Calls that may
 *     overlap on one GPU (other streams, other host threads) race on it and
 *     must be serialised by the caller.
 *   - kda_workspace_offsets describes the array's layout for a call, but the
 *     array is not exposed: its tables cannot be inspected from the host. */
#define KDA_NOALLOC_SCRATCH_BYTES (128ll << 20)

int32_t kda_fwd_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta,
                        float scale, void* out, const float* A_log, const float* dt_bias, float lower_bound,
                        const void* initial_state, void* final_state, int32_t state_dtype, int32_t state_layout,
                        const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int64_t T, int32_t H,
                        int32_t H_qk, int32_t D, int32_t cp_mode, int32_t seg_chunks, void* stream);

/* Byte offsets of the workspace regions for these sizes and plan, so a caller
 * can inspect the index tables and segment maps a kda_fwd call left in its
 * workspace (a varlen call stores its tables; a fixed-length call stores only
 * the counters, see kda_write_fixed_tables).  offs must hold KDA_WS_NUM_OFFSETS entries, filled in the
 * order of kda_ws_offset.  Returns KDA_OK or a negative kda_status. */
typedef enum {
  KDA_WS_COUNTERS = 0,      /* int32[6]: n_chunks, n_segs, flags, early_stops, seg_chunks, order;
                               flags bits 0x1..0x8 name repaired cu_seqlens faults (first != 0,
                               decreasing, last != total, out of range), 0x100 / 0x200 a
                               chunk-kernel wait that gave up; early_stops counts the (segment,
                               head) pairs whose second pass matched the checkpoint and stopped
                               there; seg_chunks is the segment length the call used (0: serial);
                               order is 1 where unit_tab has units longest first (see there) */
  KDA_WS_SEQ_START,         /* int32[N+1]   clamped sequence boundaries (last = end of the last sequence) */
  KDA_WS_SEQ_LEN,           /* int32[N]     clamped length */
  KDA_WS_SEQ_CHUNK_OFF,     /* int32[N+1]   prefix sums of ceil(len/16) */
  KDA_WS_SEQ_SEG_OFF,       /* int32[N+1]   prefix sums of max(1, ceil(chunks/seg)), seg the length in use */
  KDA_WS_CHUNK_TAB,         /* int32[max_chunks][2] (sequence, chunk in sequence) */
  KDA_WS_SEG_TAB,           /* int32[max_segs][4] (sequence, chunk begin, chunk end, segment in sequence) */
  KDA_WS_SEG_M,             /* fp32 [max_segs][H][128][128] segment transitions M^T (CP only) */
  KDA_WS_SEG_R,             /* fp32 [max_segs][H][128][128] zero-start segment states R^T (CP only) */
  KDA_WS_SEG_S,             /* fp32 [max_segs][H][128][128] state entering segment 1 of each sequence
                               (segment 0's end state), [v][k], in that segment's slot; the second
                               pass merges the later segments' start states itself (CP only) */
  KDA_WS_SEG_MNZ,           /* int32 [max_segs][H][8]: per 16-column block of a middle segment's M, 1 if
                               any entry is nonzero, 0 if the block underflowed to exactly zero (its M
                               entries are then not stored) (CP only) */
  KDA_WS_SEG_CHK,           /* fp32 [max_segs][H][128][128] zero-start state R^T of a segment >= 1 after
                               its first 4 chunks (segments longer than that; CP only) */
  KDA_WS_SEQ_FULL_OFF,      /* int32[N+1]   prefix sums of the full-length segments per sequence
                               (floor(chunks/seg); 1 per sequence when serial) */
  KDA_WS_UNIT_TAB,          /* int32[max_segs][8] the segments in dispatch order: (segment, sequence,
                               chunk begin, chunk end, segment in sequence, sequence start token,
                               sequence length, segment length in use (0: serial)); every
                               full-length segment first, in segment order, then the shorter ones
                               (a sequence's last segment, or a sequence shorter than a segment)
                               in segment order or, where the call chose it (counters' order), by
                               first-pass chunks, longest first, ties in segment order; a serial
                               varlen plan of at most 256 sequences has them longest first (all
                               -1 past the live count) */
  KDA_WS_SEG_FIX,           /* fp32 [max_segs][H][128][128] state after a segment's first 4 chunks as the
                               first pass's block of the previous segment reached it, stored only when
                               that block could not compare it with the checkpoint (CP only) */
  KDA_WS_SEG_SYNC,          /* uint32 [max_segs][H][16] per segment and 16-column block b of the state:
                               word b, the call's number once its first-pass block has stored those
                               checkpoint columns; word 8 + b, (call number << 2) | result of the
                               comparison made at the end of the previous segment's first-pass block
                               (1 equal, 2 differ, 3 not compared); cleared by the second pass (CP only) */
  KDA_WS_MAX_CHUNKS,        /* (count, not an offset) chunk-table capacity */
  KDA_WS_MAX_SEGS,          /* (count, not an offset) segment-table capacity */
  KDA_WS_TOTAL,             /* total bytes (= kda_get_workspace_size) */
  KDA_WS_NUM_OFFSETS
} kda_ws_offset;

int32_t kda_workspace_offsets(int64_t total_tokens, int32_t num_heads, int32_t num_seqs, int32_t cp_mode,
                              int32_t seg_chunks, int64_t* offs);

/* Index tables of a fixed-length call, for inspection and tests.  A kda_fwd
 * call without cu_seqlens launches no index kernel: its chunk-kernel blocks
 * compute their rows of these tables in closed form (B sequences of T tokens:
 * sequence i starts at token i*T and has ceil(T/16) chunks) and store only the
 * counters.  This call writes every table region and the counters of the
 * layout kda_workspace_offsets gives for (B*T, H, B, cp_mode, seg_chunks), with
 * the contents the varlen construction gives for B equal lengths ("How
 * FlashKDA Integrates with CUTLASS", "Variable-Length Sequence Support": a
 * fixed-length batch read as a varlen one).  It launches one kernel on stream,
 * asynchronously, and allocates nothing.  The workspace (caller-owned, device)
 * must hold at least kda_get_workspace_size bytes and be KDA_WORKSPACE_ALIGN
 * aligned; the segment buffers are untouched.  Errors: KDA_ERR_INVALID_ARG,
 * KDA_ERR_WORKSPACE_TOO_SMALL (nothing launched), KDA_ERR_HIP. */
int32_t kda_write_fixed_tables(int32_t B, int64_t T, int32_t H, int32_t cp_mode, int32_t seg_chunks,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Per-kernel timing for benchmarks.  While enabled on a host thread, every
 * kernel that kda_fwd launches on that thread is launched with a pair of HIP
 * events (hipExtLaunchKernelGGL) that take the kernel's own start and end
 * times, with no gap between kernels added.  The events are created by the
 * library on first use, without the system-scope fence (which would write
 * back and invalidate the L2 at the event and lengthen the kernel it times),
 * and kept for reuse.  Leave it disabled while a call is captured into a HIP
 * graph.  kda_profile_collect waits for the recorded events, adds the elapsed
 * milliseconds of each kernel into its stage's stage_ms[0..n_stages-1] entry
 * and the number of timed launches of the stage into stage_calls, and forgets
 * them.
 * Stages: KDA_STAGE_INDEX (index tables; varlen calls only), KDA_STAGE_RECUR0 (chunk prep +
 * recurrence of whole sequences / first segments, and the pre-scan of
 * segments >= 1), KDA_STAGE_MERGE (no kernel reports it: the merge runs at
 * the start of the second pass), KDA_STAGE_RECUR1 (merge + chunk prep +
 * recurrence of segments >= 1).  Returns KDA_OK or KDA_ERR_HIP. */
typedef enum {
  KDA_STAGE_INDEX = 0,
  KDA_STAGE_RECUR0,
  KDA_STAGE_MERGE,
  KDA_STAGE_RECUR1,
  KDA_NUM_STAGES
} kda_stage;

/* enable: KDA_PROFILE_KERNELS (the kernel events above), KDA_PROFILE_HOST
 * (host time of each kda_fwd / kda_fwd_noalloc call on this thread, from its
 * entry to its return: validation, planning and the launches, without the
 * caller's own marshalling), both, or 0. */
#define KDA_PROFILE_KERNELS 1
#define KDA_PROFILE_HOST 2
int32_t kda_profile_enable(int32_t enable);
int32_t kda_profile_collect(double* stage_ms, int64_t* stage_calls, int32_t n_stages);

/* The host microseconds summed over the forward calls timed since the last
 * kda_profile_host call on this thread, and their count; then resets both.
 * Either pointer may be NULL.  Returns KDA_OK. */
int32_t kda_profile_host(double* host_us, int64_t* calls);

/* Static description of a status code. */
const char* kda_strerror(int32_t status);

/* Message of the last failed call on this host thread ("" if none). */
const char* kda_last_error(void);

/* Library version string. */
const char* kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */

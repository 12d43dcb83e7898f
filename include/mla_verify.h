/*
 * mla_verify.h -- C ABI of libmla_verify.so: speculative-decoding verify
 * attention for Multi-head Latent Attention (MLA) over a page_size = 1 latent
 * KV cache, on AMD Instinct MI355X (gfx950).
 *
 * The operation (magik.net, "The Decisive A/B": section "The Context: A Custom
 * Kernel in Production"; "The Moment of Truth": opening section):
 *   verify attention is the speculative-decoding step in which the target
 *   model scores a block of drafted tokens in one pass.  MLA shares one latent
 *   row per cached token among all heads; with page_size = 1 every token is its
 *   own scattered slot of the pool, reached through a slot index.  For request
 *   b with L = seq_lens[b] cached rows (its Q = q_lens[b] draft tokens
 *   included, as the last Q of them), draft token t < Q and head h:
 *     k_j   = kv_pool[slot_idx[ko_b + j]]          (576 bf16: 512 latent, 64 rope)
 *     v_j   = k_j[0:512]
 *     n_t   = L - Q + t + 1                        (causal within the draft block:
 *                                                   draft t sees the prefix and
 *                                                   drafts 0..t)
 *     s_j   = sm_scale * dot(q[qo_b + t, h, :], k_j),   j < n_t
 *     lse   = log(sum_j exp(s_j))                  (natural log, scale included)
 *     out   = sum_j exp(s_j - lse) * v_j
 *   where ko_b = sum of seq_lens before b and qo_b = sum of q_lens before b.
 *   It is computed the way the pages' kernel does, as a KV split with a
 *   partial result per chunk of keys followed by a reduce of the partials
 *   ("The Decisive A/B": "The Context" and "What This Reveals About the
 *   Bottleneck"), with a fixed split count and preallocated workspace so that
 *   a call can be captured in a HIP graph (same page, "The Context").
 *
 * Conventions for every entry point:
 *   - Return value: MLA_OK (0) or a negative MLA_ERR_* status.  No exception
 *     or signal crosses the ABI.  mla_verify_error_string() names a status.
 *   - Pointers marked "device" must be device memory of the current HIP device;
 *     the caller owns them and keeps them alive until the stream has passed
 *     the call.  Host-visible arguments are validated before any HIP call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously; nothing is allocated, copied or
 *     synchronised by the run/merge calls, so they may be captured in a graph.
 *   - Values the library cannot see from the host (contents of seq_lens,
 *     q_lens, slot_idx) must satisfy the stated ranges; violations are
 *     undefined behaviour except where a clamp is stated.
 */
#ifndef MLA_VERIFY_H
#define MLA_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_OK 0
#define MLA_ERR_INVALID_ARGUMENT (-1) /* null pointer, bad size, misaligned pointer, nsplit out of range, unknown form */
#define MLA_ERR_UNSUPPORTED (-2)      /* d_qk != 576 or d_v != 512 */
#define MLA_ERR_OUT_OF_MEMORY (-3)    /* workspace allocation failed */
#define MLA_ERR_HIP (-4)              /* a HIP runtime call or a kernel launch failed, or no GPU */
#define MLA_ERR_SCRATCH_TOO_SMALL (-5) /* mla_verify_run_noalloc: the call's partials exceed its fixed scratch */

#define MLA_VERIFY_D_QK 576 /* 512 latent + 64 rope dims per cached row and per query */
#define MLA_VERIFY_D_V 512  /* v is the first 512 dims of each cached row */

typedef struct mla_verify_s* mla_verify_handle; /* opaque */

/* Shapes fixed for the life of a handle (a captured graph sees the same shapes). */
typedef struct {
  int32_t num_heads;  /* H >= 1 */
  int32_t d_qk;       /* must be 576 */
  int32_t d_v;        /* must be 512 */
  int32_t batch;      /* B >= 1: number of requests per call */
  int32_t max_q_len;  /* Q_max >= 1: upper bound on every q_lens[b] */
  int32_t max_nsplit; /* >= 1: the workspace holds this many partials per row */
  int64_t num_slots;  /* rows in kv_pool (>= 1) */
  float sm_scale;     /* score scale, > 0 (1/sqrt(192) in the reference workloads) */
  int32_t form;       /* kernel-1 layout: MLA_VERIFY_FORM_AUTO (0), _128ROW (1), _TWO_STREAM (2) or
                         _FOUR_STREAM (3) */
  int32_t flags;      /* OR of MLA_VERIFY_FLAG_* (0: none) */
} mla_verify_config;

/* Batch invariance: a request's out and lse are bit for bit the same whatever other requests
 * share its call (and whatever the batch size of the handle), as long as the handle's max_q_len,
 * num_heads, form and the call's nsplit are the same.  Without it, batches of 2..64 requests
 * (of more than 64 rows each) spread their keys over the CUs by the range plan described at
 * mla_verify_run, which moves split boundaries with the batch and so changes rounding; the flag
 * turns the range plan off (each request is split on its own), at some cost in speed for ragged
 * batches.  Any other bit is INVALID_ARGUMENT. */
#define MLA_VERIFY_FLAG_BATCH_INVARIANT 1

/* Kernel-1 layouts (the result is the same up to rounding; they differ in speed).
 * 128ROW: workgroups of 128 (draft token, head) rows, one 32-key tile per step.
 * TWO_STREAM: workgroups of 64 rows over two key streams (two tiles per step);
 *   each wave's P.V covers its own 32 rows over all 512 output columns.
 * FOUR_STREAM: workgroups of 32 rows over four key streams, one per wave, in
 *   16-key half tiles (Q.K on MFMA 16x16x32); no barrier in the step loop.
 * AUTO: TWO_STREAM for requests of at most 64 rows, and for calls whose 128-row
 * workgroups (B * nsplit * ceil(Q_max*H/128)) would occupy at most half of the
 * CUs; 128ROW otherwise; then FOUR_STREAM instead of TWO_STREAM for calls whose
 * 64-row workgroups (B * nsplit * ceil(Q_max*H/64)) would occupy at most half of
 * the CUs.  Batches of 2..64 requests in the 128-row form spread their keys over
 * the CUs by the range plan (see mla_verify_run).  Use a fixed form to compare or
 * test the layouts. */
#define MLA_VERIFY_FORM_AUTO 0
#define MLA_VERIFY_FORM_128ROW 1
#define MLA_VERIFY_FORM_TWO_STREAM 2
#define MLA_VERIFY_FORM_FOUR_STREAM 3

/*
 * Validate `cfg`, allocate the split workspace on the current device
 * (B * max_nsplit * ceil(Q_max*H/128)*128 rows of 512 fp16 partial outputs,
 * 64 rows per split instead when Q_max*H <= 64, each normalised within its
 * split, plus one fp32 log-sum-exp each) and
 * return a handle in *out.  Call outside graph capture.
 * Errors: INVALID_ARGUMENT (null, non-positive sizes, unknown form or flag), UNSUPPORTED (dims),
 * OUT_OF_MEMORY, HIP (no device).  On error *out is set to NULL.
 */
int mla_verify_create(const mla_verify_config* cfg, mla_verify_handle* out);

/*
 * One verify-attention call: split partials (kernel 1) then their merge
 * (kernel 2), both on `stream`.  The split partials are fp16 (each row a
 * convex combination of v rows, so every v entry must stay below 65504 in
 * magnitude, which latent caches do by far), their LSEs fp32.
 *   q        device bf16 [T_q, H, 576], T_q = sum(q_lens), requests in order,
 *            rows 16-byte aligned (base pointer 16-byte aligned).
 *   kv_pool  device bf16 [num_slots, 576], row stride 1152 bytes, 16-byte aligned.
 *   slot_idx device int32 [sum(seq_lens)]: request b's L_b slots in key order
 *            (its draft rows last); each 0 <= slot < num_slots.
 *   seq_lens device int32 [B], L_b >= 0.
 *   q_lens   device int32 [B], 0 <= Q_b <= min(L_b, max_q_len).  Q_b = 0 writes
 *            nothing for request b.  Q_b is clamped to that range on the device.
 *   out      device bf16 [T_q, H, 512], 16-byte aligned (written, round to nearest even).
 *   lse      device fp32 [T_q, H] (written; natural log; -inf only if no key is visible).
 *   nsplit   1 <= nsplit <= max_nsplit.  The keys of each request are divided
 *            into at most nsplit contiguous chunks; the result does not depend
 *            on nsplit beyond rounding.  Keep it constant across replays of a
 *            captured graph.  With 2..64 requests (and more than 64 rows per
 *            request) the chunks are cut from the whole batch's key sequence so
 *            that every CU gets the same share of work; a request's result then
 *            depends on the other requests' lengths through where its chunks
 *            fall, again only up to rounding.
 * The handle's workspace is reused by every call: calls on one handle must
 * not overlap (serialise them on one stream).  Distinct handles are independent.
 */
int mla_verify_run(mla_verify_handle h, const void* q, const void* kv_pool, const int32_t* slot_idx,
                   const int32_t* seq_lens, const int32_t* q_lens, void* out, float* lse, int32_t nsplit,
                   void* stream);

/*
 * mla_verify_run without a handle and without any allocation, for callers that cannot allocate
 * device memory at the time of the call (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The same kernels and the same result as mla_verify_run on a
 * handle created from *cfg (bit for bit), but the split partials live in a fixed device array
 * inside the library, MLA_VERIFY_NOALLOC_SCRATCH_BYTES (40 MiB) per GPU, which each GPU the
 * library runs on holds from the first use until the process ends.
 *   cfg      the shapes, as for mla_verify_create (read on every call; not kept).
 *   other arguments as in mla_verify_run; nsplit <= cfg->max_nsplit.
 * Size limit: B * nsplit * rows_pad * 512 fp16 partials (rows_pad = ceil(Q_max*H/128)*128, or 64
 * when Q_max*H <= 64), then B * nsplit * rows_pad fp32 LSEs from the next 256-B boundary, must fit
 * the array; otherwise MLA_ERR_SCRATCH_TOO_SMALL and nothing is enqueued.  (One request of 1,024
 * rows at nsplit 32 takes 32.1 MiB; a 64-row decode step at nsplit 256 takes 16.1 MiB.)
 * Every call on one GPU uses that GPU's one array: calls that overlap in time on one GPU (other
 * streams, other threads, other handles' noalloc calls) race on it and give wrong results;
 * serialise them.  Nothing in the array needs to start at zero (every partial read is written
 * by the same call).  The first call on each device looks up the array's device address
 * (hipGetSymbolAddress, no allocation); make that first call outside graph capture.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (as for create), SCRATCH_TOO_SMALL, HIP.
 */
#define MLA_VERIFY_NOALLOC_SCRATCH_BYTES (40u << 20)
int mla_verify_run_noalloc(const mla_verify_config* cfg, const void* q, const void* kv_pool,
                           const int32_t* slot_idx, const int32_t* seq_lens, const int32_t* q_lens, void* out,
                           float* lse, int32_t nsplit, void* stream);

/*
 * Kernel 1 alone: the split partials of one call, left in the handle's
 * workspace: the partial half of the KV-split partial + reduce scheme (magik.net,
 * "The Decisive A/B", sections "The Context: A Custom Kernel in Production" and
 * "What This Reveals About the Bottleneck").  Partial s of a row is that row's
 * softmax attention over the s-th chunk of its keys, normalised within the chunk,
 * with the chunk's natural-log LSE.  Arguments
 * as in mla_verify_run.  mla_verify_run is this call followed by the merge;
 * this entry exists to time and inspect the partial phase by itself.
 */
int mla_verify_partials(mla_verify_handle h, const void* q, const void* kv_pool, const int32_t* slot_idx,
                        const int32_t* seq_lens, const int32_t* q_lens, int32_t nsplit, void* stream);

/*
 * Kernel 2 alone: merge caller-provided split partials, the reduce half of the
 * KV-split partial + reduce scheme (magik.net, "The Decisive A/B", sections "The
 * Context: A Custom Kernel in Production" and "Input and Output Knowledge"):
 *     lse = log sum_s exp(lse_s),   out = sum_s exp(lse_s - lse) * o_s,
 * -inf partials skipped.  Every one of the nsplit partials of a row
 * takes part; a partial with lse = -inf carries no weight.
 *   o_part   device fp32 [batch, nsplit, max_q_len * H, 512]: partial outputs,
 *            each already normalised within its chunk; row r of request b is
 *            (token r / H, head r % H).  16-byte aligned.
 *   lse_part device fp32 [batch, nsplit, max_q_len * H]: natural-log LSE per chunk.
 *   q_lens   device int32 [batch] (same clamp as in mla_verify_run).
 *   out, lse as in mla_verify_run.
 * Errors: INVALID_ARGUMENT, HIP.
 */
int mla_verify_merge(const float* o_part, const float* lse_part, const int32_t* q_lens, int32_t batch,
                     int32_t num_heads, int32_t max_q_len, int32_t nsplit, void* out, float* lse, void* stream);

/*
 * KV compaction: the "KV defragmentation" that magik.net, "The Moment of Truth"
 * (sections "The Broader Context: From Kernel to System" and "Conclusion")
 * names as a next step.  Copies the page_size = 1 rows of one slot list into
 * a contiguous range of destination slots, in order:
 *     dst_pool[dst_first + j] = kv_pool[slot_idx[j]]   for 0 <= j < n_rows,
 * each row the whole 576-dim bf16 latent row (1152 bytes, copied bit for bit),
 * and, when new_slot_idx is not NULL, new_slot_idx[j] = dst_first + j, so that
 * a verify call over (dst_pool, new_slot_idx) sees the same rows in the same
 * order as one over (kv_pool, slot_idx) and returns the same result.
 *   kv_pool      device bf16 [*, 576], 16-byte aligned.
 *   slot_idx     device int32 [n_rows]; each slot must be a row of kv_pool
 *                (not checked: a slot past the pool is undefined behaviour).
 *   n_rows       >= 0; 0 enqueues nothing.
 *   dst_pool     device bf16 [dst_slots, 576], 16-byte aligned.  It may be
 *                kv_pool itself as long as the destination rows are none of
 *                the source rows.
 *   dst_first    first destination slot; dst_first + n_rows <= dst_slots.
 *   new_slot_idx device int32 [n_rows] or NULL; with it, dst_first + n_rows
 *                must fit in int32.
 *   stream       hipStream_t; one kernel launch, nothing else (capture-safe).
 * Errors: INVALID_ARGUMENT (null pointers when n_rows > 0, negative sizes, a
 * destination range outside [0, dst_slots), misalignment), HIP.
 */
int mla_verify_compact(const void* kv_pool, const int32_t* slot_idx, int64_t n_rows, void* dst_pool,
                       int64_t dst_slots, int64_t dst_first, int32_t* new_slot_idx, void* stream);

/*
 * Step metadata on the device: the verify call's index arrays built once per
 * step from the serving side's request-to-token table, into caller-owned
 * static buffers, so that a captured step replays with fresh metadata and no
 * host work (magik.net, "The Moment of Truth": building combined indices once
 * per step instead of per layer, "Interpreting the Crossover: The Marshaling
 * Tax"; overriding the metadata replay logic with pre-allocated static
 * buffers, "The Thinking Process"; a marshaling kernel on the GPU,
 * "Assumptions and Their Validity").  For b < batch:
 *     seq_lens[b] = prefix_lens[b] + draft_lens[b],   q_lens[b] = draft_lens[b],
 *     slot_idx    = entries 0 .. seq_lens[b]-1 of table row req_ids[b], b in order
 * (prefix_lens[b] tokens already cached, draft_lens[b] draft tokens whose rows
 * are written at the next positions).
 *   req_to_token device int32 [table_rows, table_stride]: row r lists the cache
 *                slot of every position of the request in row r; only the
 *                first table_width entries of a row may be used.
 *   req_ids, prefix_lens, draft_lens  device int32 [batch], 0 <= batch <= 1024.
 *   slot_idx     device int32 [slot_capacity] (slot_capacity <= INT32_MAX).
 *   seq_lens, q_lens  device int32 [batch]; status device int32 [1].
 *   With batch == 0 the table and the per-request pointers may be NULL (only
 *   *status is written); with slot_capacity == 0 slot_idx may be NULL.
 *   stream       hipStream_t; one kernel launch, no host synchronisation.
 * Device-side checks set *status (0 = ok) to the OR of: 1 a row id outside
 * [0, table_rows), 2 a negative length, 4 a sequence longer than table_width,
 * 8 more than slot_capacity slots in all; then every seq_lens and q_lens entry
 * is 0 (a verify call on them does nothing) and no slot is written.
 * Errors (host): INVALID_ARGUMENT (null, sizes, alignment), HIP.
 */
int mla_verify_build_metadata(const int32_t* req_to_token, int32_t table_rows, int32_t table_width,
                              int64_t table_stride, const int32_t* req_ids, const int32_t* prefix_lens,
                              const int32_t* draft_lens, int32_t batch, int32_t* slot_idx, int64_t slot_capacity,
                              int32_t* seq_lens, int32_t* q_lens, int32_t* status, void* stream);

/*
 * Where a handle's split workspace lives (the partials kernel 1 writes and the
 * merge reads in mla_verify_run), for inspection and tests:
 *   *o_part   device fp16 [batch, max_nsplit, rows_pad, 512], rows_pad =
 *             ceil(max_q_len * H / 128) * 128 (row r of request b is (token r / H,
 *             head r % H)); *o_part_bytes its size.
 *   *lse_part device fp32 [batch, max_nsplit, rows_pad]; *lse_part_bytes its size.
 * The library owns the memory (freed by mla_verify_destroy).  Every call
 * overwrites the partials it reads before reading them; what the workspace
 * holds between calls has no meaning, and writing into it between calls (for
 * instance filling it with NaN) does not change any later call's result.
 * Any output pointer may be NULL.  Errors: INVALID_ARGUMENT (null handle).
 */
int mla_verify_workspace(mla_verify_handle h, void** o_part, int64_t* o_part_bytes, void** lse_part,
                         int64_t* lse_part_bytes);

/*
 * Checks of device-visible arguments (slot_idx, seq_lens and q_lens are read only on the device,
 * so a release build cannot reject them).  libmla_verify_debug.so is
 * the same library built with MLA_VERIFY_DEBUG defined: its verify kernels replace a bad value
 * before it is used for any memory access and OR a bit into a device word of the handle:
 *   MLA_VERIFY_DEBUG_SLOT_OUT_OF_RANGE   a slot outside [0, num_slots): clamped into it;
 *   MLA_VERIFY_DEBUG_NEGATIVE_LENGTH     seq_lens[b] < 0: read as 0 (then request b has no
 *                                        keys and no rows, and takes no slots);
 *   MLA_VERIFY_DEBUG_Q_LEN_OUT_OF_RANGE  q_lens[b] outside [0, min(seq_lens[b], max_q_len)]:
 *                                        clamped (the release build clamps it silently).
 * The results of such a call are whatever the clamped arguments give; the point is that no
 * access leaves the caller's buffers (given a pool of num_slots rows) and that the caller can
 * find out.  mla_verify_debug_flags synchronises the device, stores the word in *flags (0: no
 * check fired since creation or the last clear) and, if `clear` is non-zero, resets it.  In the
 * release library it stores 0 and returns MLA_ERR_UNSUPPORTED.  (mla_verify_run_noalloc clamps
 * the same way in the debug build but has no handle to keep a word in.)
 * Errors: INVALID_ARGUMENT (null), UNSUPPORTED (release build), HIP.
 */
#define MLA_VERIFY_DEBUG_SLOT_OUT_OF_RANGE 1
#define MLA_VERIFY_DEBUG_NEGATIVE_LENGTH 2
#define MLA_VERIFY_DEBUG_Q_LEN_OUT_OF_RANGE 4
int mla_verify_debug_flags(mla_verify_handle h, int32_t* flags, int32_t clear);

/* Free the workspace and the handle.  NULL is a no-op.  The caller must make
 * sure no enqueued call still uses the handle (synchronise its stream first). */
int mla_verify_destroy(mla_verify_handle h);

/* Static, NUL-terminated name of a status code; never NULL. */
const char* mla_verify_error_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_VERIFY_H */

/*
 * ssm_stream.h -- C ABI of the MI355X (gfx950) Mamba-2 streaming-state library.
 *
 * The library advances the Mamba-2 selective-scan recurrence, per head h of a
 * layer with H heads, head dim P, state size N and G groups of B/C
 * (g = h / (H/G)):
 *
 *     h_t = exp(dt_t[h] * A[h]) * h_{t-1} + dt_t[h] * x_t[h,:] (outer) B_t[g,:]
 *     y_t[h,p] = sum_n h_t[p,n] * C_t[g,n] + D[h] * x_t[h,p]
 *
 * (each token shrinks the previous state by its decay factor and adds its own
 * outer-product term: "Why Speculative Decoding Slows Hybrid Mamba Models at
 * Large Batch Sizes", section "The Fix: Log the Inputs, Checkpoint the State";
 * the matrix and recurrent views of the same algebra: "Mamba Streaming State
 * That Survives Chunking", section "Separate Mamba-2 algebra from kernel
 * behavior").
 *
 * Three paths advance it, all on the caller's HIP stream:
 *   ssm_scan_chunk   a chunk of L tokens of one stream, with carry-in/out,
 *                    per-token reset flags and mid-chunk checkpoints;
 *   ssm_decode_step  one token for each of a batch of streams (slots);
 *   ssm_replay_step  speculative verify of n_in in-flight tokens per slot
 *                    from a checkpoint plus a log of per-token inputs; the
 *                    full state is written only when the log fills.
 * ssm_copy_step is the copy-state-per-draft verify used as the measurement
 * baseline of the replay path.
 *
 * Conventions (all entry points):
 *  - Ownership.  The caller allocates and frees every device buffer (state,
 *    inputs, outputs, replay log, copy buffer, workspace, checkpoints).  The
 *    library never frees them.  It owns its host metadata and, per handle, one
 *    small device buffer (checksum and finite-check flags, 4 KiB) taken on
 *    first use from a per-device pool the library keeps until the process
 *    ends; ssm_destroy returns it to the pool.
 *  - Pointers named d_* or documented "device" are device pointers; h_* are
 *    host pointers read before the call returns.  x, dt, B, C, y use the
 *    handle's io dtype; state, checkpoints, A and D are fp32.
 *  - Layouts are row-major, last index fastest:
 *      state[S,H,P,N]  x,y[L,H,P]  dt[L,H]  B,C[L,G,N]  A,D[H]
 *    (for batched calls the leading L is the batch, or batch*n_in).
 *  - Ordering.  Work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream).  Results are valid after the stream has synchronised.  Calls on
 *    one handle must not run concurrently from several host threads.
 *  - Errors.  Every error detectable on the host is returned before anything
 *    is enqueued, with state and metadata unchanged.  ssm_last_error() gives
 *    a message for the calling thread.
 *  - Metadata is exact.  Positions (tokens since the stream's start or last
 *    reset) and chunk sequence numbers are host integers the kernels never
 *    write.
 */
#ifndef SSM_STREAM_H
#define SSM_STREAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SSM_OK = 0,
  SSM_E_INVALID_ARG = -1,   /* bad size, pointer, slot id, dtype ... */
  SSM_E_INVALID_CHUNK = -2, /* non-finite input (with SSM_FLAG_CHECK_FINITE) */
  SSM_E_INVALID_STATE = -3, /* unknown or destroyed handle */
  SSM_E_SEQUENCE = -4,      /* chunk_seq reordered or duplicated */
  SSM_E_SCHEMA = -5,        /* restore receipt incompatible with the handle */
  SSM_E_LOG = -6,           /* replay/copy bookkeeping misuse */
  SSM_E_HIP = -7            /* the HIP runtime reported an error */
} ssm_status;

/* dtype codes, the same numbering as the pion state_blob format ("SSM.PREFIX.*
 * -- recurrent-state companion", state_blob section): 0 fp32, 1 fp16, 2 bf16. */
typedef enum { SSM_F32 = 0, SSM_F16 = 1, SSM_BF16 = 2 } ssm_dtype;

/* Handle creation flags. */
#define SSM_FLAG_CHECK_FINITE 1u /* scan/decode/replay/copy first check their
                                    inputs on the device and synchronise; a
                                    non-finite value returns SSM_E_INVALID_CHUNK
                                    with nothing changed (the runnable
                                    artifact's "invalid_chunk") */

/* The recurrence a handle's state follows.
 *   SSM_MAMBA2       the selective-scan recurrence above.
 *   SSM_GATED_DELTA  the gated delta rule of Gated DeltaNet, per value head h
 *                    with key group g:
 *                      S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *                      o_t = S_t q_t,   alpha_t = exp(dt_t[h] * A[h])
 *                    with S [P value rows, N key columns] in the same
 *                    state[S,H,P,N] layout; x carries v [.,H,P], B carries
 *                    k and C carries q [.,G,N], beta [.,H] is an extra
 *                    input, D is unused.  The pages name it among the
 *                    recurrences whose update unrolls into a decay plus a
 *                    sum, so that replay applies ("Why Speculative Decoding
 *                    Slows Hybrid Mamba Models at Large Batch Sizes", section
 *                    "When Replaying the Inputs Is the Wrong Tool"); the
 *                    update itself is the published gated delta rule.  Its
 *                    handles serve the verify paths (ssm_gdn_replay_step,
 *                    ssm_gdn_copy_step) and the state operations. */
typedef enum { SSM_MAMBA2 = 0, SSM_GATED_DELTA = 1 } ssm_recurrence;

/* Layer description.  Supported: H,P >= 1; N % 4 == 0 and 4 <= N <= 128;
 * G >= 1 with H % G == 0; io_dtype SSM_F32 or SSM_BF16; recurrence an
 * ssm_recurrence (0, the default of a zeroed struct, is Mamba-2). */
typedef struct {
  int32_t H, P, N, G;
  int32_t io_dtype;        /* ssm_dtype of x, dt, B, C and y */
  uint32_t schema_version; /* caller's state-schema version */
  uint64_t model_rev;      /* caller's model revision */
  int32_t recurrence;      /* ssm_recurrence */
  int32_t reserved;        /* 0 */
} ssm_layer_desc;

/* Checkpoint receipt: the fields a resume must match ("Mamba Streaming State
 * That Survives Chunking", section "Make reset, checkpoint, and cancellation
 * observable": stream id, model and code revision, schema version, dtype,
 * dimensions, absolute position, chunk sequence and checksum). */
typedef struct {
  uint64_t stream_id;      /* opaque id the library gave the slot's stream */
  uint64_t model_rev;
  uint64_t code_rev;       /* ssm_code_rev() of the library that wrote it */
  uint32_t schema_version;
  uint32_t state_dtype;    /* always SSM_F32 */
  int32_t H, P, N, G;
  int64_t position;        /* tokens since the stream's start or last reset */
  uint64_t chunk_seq;      /* next chunk sequence number the stream expects */
  uint64_t checksum;       /* sum over the state's 32-bit words w_i of
                              w_i * (2*i + 1), modulo 2^64, i in [H,P,N] order */
  uint32_t recurrence;     /* ssm_recurrence of the state (states of different
                              recurrences never resume into each other:
                              section "Version state semantics for Mamba-3") */
  uint32_t reserved;
} ssm_receipt;

/* Lifecycle counters (resets, rejected duplicate or reordered chunks,
 * checkpoints, rejected resumes: "Mamba Streaming State That Survives
 * Chunking", section "Make reset, checkpoint, and cancellation observable").
 * Byte counters follow the algorithmic model (state bytes each path must
 * move), not hardware counters. */
typedef struct {
  uint64_t chunks_admitted, chunks_rejected, tokens_scanned, decode_tokens;
  uint64_t resets, replay_steps, replay_flushes, replay_tokens_committed;
  uint64_t copy_steps, checkpoints, restores, restores_rejected;
  uint64_t state_bytes_read, state_bytes_written;
} ssm_counters;

/* Handles are positive integers; a destroyed handle's id is never reused, so
 * a call on it returns SSM_E_INVALID_STATE (cancellation is observable). */
typedef int64_t ssm_handle;

/* ---------------------------------------------------------------- lifecycle */

/* Create a handle over n_slots stream slots whose fp32 state lives in the
 * caller's d_state[n_slots,H,P,N]; d_A[H], d_D[H] are the layer's fp32
 * parameters (device, kept by pointer: they must outlive the handle).  Every
 * slot starts as a fresh stream at position 0 with chunk_seq 0; the caller
 * decides what d_state holds (ssm_state_reset / ssm_state_init write it).
 * A slot is the stream-owned record of one stream's state, position and
 * chunk sequence ("Mamba Streaming State That Survives Chunking", section
 * "Treat Mamba streaming state as a stream-owned record"); the state is one
 * fixed-size fp32 array per stream and layer ("Why Speculative Decoding Slows
 * Hybrid Mamba Models at Large Batch Sizes", section "The Problem").
 * flags: SSM_FLAG_*.  No device call is made.  Errors: SSM_E_INVALID_ARG for
 * a bad desc, n_slots < 1, a NULL or misaligned (16 bytes) state, NULL A (or
 * NULL D for Mamba-2; Gated DeltaNet takes D = NULL), or unknown flags. */
ssm_status ssm_create(const ssm_layer_desc *desc, int32_t n_slots, float *d_state,
                      const float *d_A, const float *d_D, uint32_t flags, ssm_handle *out);

/* Cancel: release the handle (cancellation must be observable: "Mamba
 * Streaming State That Survives Chunking", section "Make reset, checkpoint,
 * and cancellation observable").  Work already enqueued still completes.
 * Nothing is synchronised: every call that uses the handle's scratch buffer
 * has synchronised its stream before returning, so the buffer goes back to
 * the library's pool at once.  Any later call with this handle returns
 * SSM_E_INVALID_STATE. */
ssm_status ssm_destroy(ssm_handle h);

/* Reset h_slots[n] (distinct): state zeroed on `stream`, position 0, chunk_seq
 * 0, a new stream id, replay log emptied, any live copy dropped: after a reset
 * nothing of the earlier stream carries over (section "Make reset, checkpoint,
 * and cancellation observable"). */
ssm_status ssm_state_reset(ssm_handle h, int32_t n, const int32_t *h_slots, void *stream);

/* Initialise h_slots[n] from a learned initial state d_init[n,H,P,N] (fp32,
 * device): as ssm_state_reset but the state is copied from d_init. */
ssm_status ssm_state_init(ssm_handle h, int32_t n, const int32_t *h_slots, const float *d_init,
                          void *stream);

/* ----------------------------------------------------------- chunked scan */

/* Bytes of device workspace for ssm_scan_chunk on chunks of up to L tokens
 * (0 for an invalid desc or L < 0).  Two forms of the scan exist, with the same
 * results up to floating-point rounding order:
 *   - tile-parallel (fp32 io, or bf16 shapes other than P=64/N=128; P of 32 or
 *     64 and N a multiple of 32): chunks of 64 tokens or more run in parallel
 *     over 64-token tiles.  It needs this many bytes (per-tile states, at most
 *     64 tiles at a time: min(ceil(L/64), 64)*H*P*N*4 + 256*H bytes) and x
 *     aligned to 4 elements;
 *   - recurrent / SSD: needs H*P*N*4 bytes only when a chunk both carries state
 *     in (no reset on its first token) and holds a reset later; otherwise
 *     d_workspace may be NULL.
 * A workspace smaller than the tile-parallel form's need selects the other. */
size_t ssm_scan_workspace_bytes(const ssm_layer_desc *desc, int64_t L);

/* Advance stream `slot` by the L tokens of one chunk.
 *   chunk_seq   must equal the slot's next expected sequence number (0 after
 *               create/reset/init); a lower value is a duplicate, a higher one
 *               a reorder or gap: both return SSM_E_SEQUENCE with nothing
 *               changed (section "Let the full scan define legal chunking": a
 *               chunk applied out of order or twice is an error).  On success the expected
 *               number becomes chunk_seq + 1; a retry of a chunk whose result
 *               was lost must restore a pre-chunk checkpoint first.
 *   L >= 0      L == 0 (an empty chunk) only advances chunk_seq.
 *   x[L,H,P] dt[L,H] B,C[L,G,N]  device, io dtype;  y[L,H,P] device, io dtype
 *   h_reset     host u8[L] or NULL: a nonzero entry zeroes the state and the
 *               position before that token (a new sequence boundary)
 *   n_ckpt, h_ckpt_at[n_ckpt]  host, strictly increasing token indices in
 *               [0,L); the state right after token h_ckpt_at[i] is written to
 *               d_ckpt_out[i,H,P,N] (device fp32), e.g. each packed
 *               sequence's final state
 *   d_workspace, ws_bytes  see ssm_scan_workspace_bytes
 * The slot's state is the carry-in and receives the carry-out.  The slot must
 * have no pending replay log or live copy (SSM_E_LOG; see
 * ssm_state_materialize). */
ssm_status ssm_scan_chunk(ssm_handle h, int32_t slot, uint64_t chunk_seq, int64_t L,
                          const void *x, const void *dt, const void *B, const void *C,
                          const uint8_t *h_reset, void *y, int32_t n_ckpt,
                          const int64_t *h_ckpt_at, float *d_ckpt_out, void *d_workspace,
                          size_t ws_bytes, void *stream);

/* Scan a batch of packed sequences, each into its own slot: the prefill of
 * several streams in one call.  Sequence i holds tokens [h_cu_seqlens[i],
 * h_cu_seqlens[i+1]) of x[L,H,P] dt[L,H] B,C[L,G,N] (device, io dtype;
 * L = h_cu_seqlens[nseq]) and writes y[L,H,P].  Its final state becomes the
 * state of slot h_seq_slots[i] (host, distinct) together with its position,
 * so that decode continues each stream where its prefill ended (continuous
 * batching moves recurrent state and position together: "Mamba Streaming
 * State That Survives Chunking", section "Separate Mamba-2 algebra from
 * kernel behavior").
 *   h_cu_seqlens  host int32[nseq+1]: 0 first, non-decreasing (empty
 *                 sequences are legal)
 *   h_continue    host u8[nseq] or NULL.  0 (or NULL): the sequence starts a
 *                 new stream from a zero state (a reset on its first token);
 *                 the slot gets a new stream id, position = its length and
 *                 chunk_seq 1.  Nonzero: it continues the slot's stream from
 *                 the slot's state; h_chunk_seq[i] must equal the slot's next
 *                 chunk sequence number (else SSM_E_SEQUENCE, nothing
 *                 changed), and position and chunk_seq advance as for
 *                 ssm_scan_chunk.
 *   h_chunk_seq   host u64[nseq]; required when any h_continue is set
 *   d_final       device fp32 [nseq,H,P,N] or NULL: a copy of every
 *                 sequence's final state (the checkpoint of each sequence)
 *   h_receipts    host [nseq] or NULL: the receipt of each slot's new state
 *                 (section "Make reset, checkpoint, and cancellation
 *                 observable": stream id, position, chunk sequence,
 *                 checksum...); with d_final, d_final[i] and h_receipts[i]
 *                 restore the stream into any slot (ssm_state_restore).
 *                 Taking the checksums synchronises `stream`.
 * Every slot must have no pending replay log or live copy (SSM_E_LOG).  No
 * workspace is needed: distinct slots never share a state. */
ssm_status ssm_scan_packed(ssm_handle h, int32_t nseq, const int32_t *h_cu_seqlens,
                           const int32_t *h_seq_slots, const uint8_t *h_continue,
                           const uint64_t *h_chunk_seq, const void *x, const void *dt,
                           const void *B, const void *C, void *y, float *d_final,
                           ssm_receipt *h_receipts, void *stream);

/* Bytes of workspace ssm_scan_chunk_static has: the size of the library's
 * static device scratch (16 MiB per GPU). */
#define SSM_STATIC_WORKSPACE_BYTES ((size_t)16 << 20)

/* ssm_scan_chunk for callers that cannot allocate device memory (code under
 * stream capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same chunk scan, arguments and results, with no workspace argument.  Its
 * workspace is the library's static device scratch, SSM_STATIC_WORKSPACE_BYTES
 * per GPU, which each GPU holds from the library's load until the process
 * ends; the call allocates and frees nothing (with SSM_FLAG_CHECK_FINITE the
 * finite-check flag lives there too).  The form is chosen as ssm_scan_chunk
 * chooses it for a workspace of that size: the tile-parallel form when
 * ssm_scan_workspace_bytes(desc, L) fits, else the recurrent or SSD form.  A
 * chunk that carries state in and resets later needs H*P*N*4 bytes of it; a
 * layer whose state is larger is refused with SSM_E_INVALID_ARG (nothing
 * changed).  Every call on one GPU shares that GPU's scratch, and the scratch
 * keeps what the last call left in it: calls that overlap on one GPU (on
 * different streams, or from several host threads) race and must not be
 * issued; calls in order on one stream are safe. */
ssm_status ssm_scan_chunk_static(ssm_handle h, int32_t slot, uint64_t chunk_seq, int64_t L,
                                 const void *x, const void *dt, const void *B, const void *C,
                                 const uint8_t *h_reset, void *y, int32_t n_ckpt,
                                 const int64_t *h_ckpt_at, float *d_ckpt_out, void *stream);

/* ------------------------------------------------------------------ decode */

/* One token for each of `batch` distinct slots h_slot_ids[batch] (decode moves
 * many streams forward by a token each: section "Separate Mamba-2 algebra
 * from kernel behavior").  x[batch,H,P] dt[batch,H] B,C[batch,G,N] in, y[batch,H,P]
 * out (device, io dtype).  h_reset: host u8[batch] or NULL; a set flag starts
 * the slot from a zero state (its old state is not read) and position 0, so a
 * reused batch slot cannot seed its next occupant.  The state is updated in
 * place.  Slots must have no pending replay log or live copy (SSM_E_LOG). */
ssm_status ssm_decode_step(ssm_handle h, int32_t batch, const int32_t *h_slot_ids,
                           const void *x, const void *dt, const void *B, const void *C,
                           const uint8_t *h_reset, void *y, void *stream);

/* ------------------------------------------------------------------ replay */

/* Bytes of the replay log for n_slots slots and window W: per slot two halves
 * of W entries of dt[H], x[H,P] and B[G,N] (Gated DeltaNet: also beta[H]) in
 * the io dtype, plus scratch. */
size_t ssm_replay_log_bytes(const ssm_layer_desc *desc, int32_t n_slots, int32_t W);

/* Attach the caller's log buffer (device, ssm_replay_log_bytes bytes) with
 * window W (1 <= W <= 64).  Every slot's log starts empty; the slot's state
 * buffer is its checkpoint (the Glossary of "Why Speculative Decoding Slows
 * Hybrid Mamba Models at Large Batch Sizes": the checkpoint is a whole-state
 * copy refreshed once per log window). */
ssm_status ssm_replay_attach(ssm_handle h, int32_t W, void *d_log, size_t log_bytes);

/* Verify n_in (1 <= n_in <= W) in-flight tokens per slot (the real token plus
 * drafts).  For each slot, if the committed log length plus n_in exceeds W, the
 * log is first folded into the checkpoint (the only state write, fused into
 * this call).  Outputs of every in-flight token are computed from the
 * checkpoint and the log without writing the state (section "The Fix: Log the
 * Inputs, Checkpoint the State"), and the in-flight inputs are appended to the log.
 *   x[batch,n_in,H,P] dt[batch,n_in,H] B,C[batch,n_in,G,N]; y[batch,n_in,H,P]
 * Each slot must then be committed before its next replay step. */
ssm_status ssm_replay_step(ssm_handle h, int32_t batch, const int32_t *h_slot_ids, int32_t n_in,
                           const void *x, const void *dt, const void *B, const void *C, void *y,
                           void *stream);

/* ReplaySSM verify of a Gated DeltaNet handle (desc.recurrence =
 * SSM_GATED_DELTA): as ssm_replay_step, with v[batch,n_in,H,P],
 * dt[batch,n_in,H], beta[batch,n_in,H], k,q[batch,n_in,G,N] and
 * o[batch,n_in,H,P].  Outputs come from the checkpoint and the log: each
 * in-flight query is carried back through the logged entries' rank-1 factors
 * alpha_j (I - beta_j k_j k_j^T) and meets the checkpoint once; the state is
 * written only when the log is full and is folded in.  Commit with
 * ssm_replay_commit; ssm_state_materialize folds a log into the state. */
ssm_status ssm_gdn_replay_step(ssm_handle h, int32_t batch, const int32_t *h_slot_ids,
                               int32_t n_in, const void *v, const void *dt, const void *beta,
                               const void *k, const void *q, void *o, void *stream);

/* Commit the last replay step of each slot: h_accepted[i] (1..n_in) leading
 * in-flight tokens join the log and the position; the rest are dropped (they
 * never enter the committed log: "Why Speculative Decoding Slows Hybrid Mamba
 * Models at Large Batch Sizes", section "The Fix: Log the Inputs, Checkpoint
 * the State"; the accepted count is the real token plus the drafts before
 * the first miss, section "Implementing It").  Host only: SSM_E_LOG for a
 * slot with no replay step awaiting commit or a count outside [1, n_in]. */
ssm_status ssm_replay_commit(ssm_handle h, int32_t batch, const int32_t *h_slot_ids,
                             const int32_t *h_accepted);

/* -------------------------------------------------- copy-per-draft baseline */

/* Bytes of the copy buffer: n_slots * n_in_max full fp32 states. */
size_t ssm_copy_buffer_bytes(const ssm_layer_desc *desc, int32_t n_slots, int32_t n_in_max);

/* Attach the caller's copy buffer d_copies[n_slots,n_in_max,H,P,N] (device). */
ssm_status ssm_copy_attach(ssm_handle h, int32_t n_in_max, float *d_copies, size_t bytes);

/* Baseline verify (section "The Problem": the server keeps one full state copy
 * per draft token so a rejected guess can be undone): read each slot's live state once, and for each of the n_in
 * tokens update it, write a full copy and emit the output.  Same layouts as
 * ssm_replay_step. */
ssm_status ssm_copy_step(ssm_handle h, int32_t batch, const int32_t *h_slot_ids, int32_t n_in,
                         const void *x, const void *dt, const void *B, const void *C, void *y,
                         void *stream);

/* The copy-state-per-draft verify of a Gated DeltaNet handle (the baseline
 * of ssm_gdn_replay_step; same layouts), committed with ssm_copy_commit. */
ssm_status ssm_gdn_copy_step(ssm_handle h, int32_t batch, const int32_t *h_slot_ids, int32_t n_in,
                             const void *v, const void *dt, const void *beta, const void *k,
                             const void *q, void *o, void *stream);

/* Adopt copy h_accepted[i]-1 as the slot's live state (an index move, no data
 * copied) and advance the position.  Host only. */
ssm_status ssm_copy_commit(ssm_handle h, int32_t batch, const int32_t *h_slot_ids,
                           const int32_t *h_accepted);

/* ------------------------------------------------------ state ops, receipts */

/* Make the slot's state buffer hold its current state: fold a non-empty replay
 * log into it, or copy a live copy back.  SSM_E_LOG if a replay or copy step
 * is awaiting commit. */
ssm_status ssm_state_materialize(ssm_handle h, int32_t n, const int32_t *h_slots, void *stream);

/* Checkpoint `slot`: materialize it, copy its state to d_dst[H,P,N] (device
 * fp32) and fill *out with the receipt a resume needs ("Mamba Streaming State
 * That Survives Chunking", section "Make reset, checkpoint, and cancellation
 * observable": stream id, revisions, schema, dtype, dimensions, absolute
 * position, chunk sequence and checksum).  In a replay stream the checkpoint
 * is the whole state after folding the log ("Why Speculative Decoding Slows
 * Hybrid Mamba Models at Large Batch Sizes", Glossary).  Synchronises
 * `stream` (the checksum is computed on the device and read back).  Errors:
 * SSM_E_INVALID_ARG (bad slot, NULL or misaligned d_dst, NULL out), SSM_E_LOG
 * (a verify step awaits commit). */
ssm_status ssm_state_checkpoint(ssm_handle h, int32_t slot, float *d_dst, ssm_receipt *out,
                                void *stream);

/* Resume `slot` from d_src[H,P,N] and its receipt.  Any semantic mismatch
 * (schema version, dtype, H, P, N, G, model or code revision) or a checksum
 * that does not match d_src returns SSM_E_SCHEMA with nothing changed (an
 * incompatible resume is refused, never padded or truncated: "Mamba
 * Streaming State That Survives Chunking", sections "Make reset, checkpoint,
 * and cancellation observable" and "Version state semantics for Mamba-3").
 * The slot takes the receipt's stream id, position and chunk sequence.
 * Synchronises `stream`. */
ssm_status ssm_state_restore(ssm_handle h, int32_t slot, const float *d_src,
                             const ssm_receipt *r, void *stream);

/* ------------------------------------------------------------- state blobs */

/* Bytes of the blob ssm_state_serialize writes for this layer: 28 + 4*H*P*N,
 * or 0 for an invalid desc.  The format is the reference serialization of the
 * recurrent-state companion store ("SSM.PREFIX.* -- recurrent-state
 * companion"): u32 version = 1, u32 n_arrays, then per array u32 ndim, u32
 * shape[ndim], u32 dtype_code (0 fp32, 1 fp16, 2 bf16 carried as fp32) and the
 * raw element bytes, all little-endian. */
size_t ssm_blob_bytes(const ssm_layer_desc *desc);

/* Bytes of the blob ssm_state_serialize writes for a slot of this handle:
 * ssm_blob_bytes, plus 16 + 4*C*(K-1) when a conv of width K > 1 is attached
 * (ssm_conv_attach); 0 for a handle that is not live. */
size_t ssm_state_blob_bytes(ssm_handle h);

/* Checkpoint `slot` into a host blob: materialize it and write the slot's
 * state as fp32 arrays (dtype code 0) into h_blob (caller-owned host memory of
 * `cap` bytes; SSM_E_INVALID_ARG if cap < ssm_state_blob_bytes): the conv
 * state [C, K-1] first when a conv with K > 1 is attached, then the scan
 * state [H, P, N] (a Mamba layer's [conv_state, ssm_state]).  Sets *written
 * and fills *out as ssm_state_checkpoint does (its checksum covers the scan
 * state).  The receipt travels beside the blob.  Synchronises `stream`. */
ssm_status ssm_state_serialize(ssm_handle h, int32_t slot, void *h_blob, size_t cap,
                               size_t *written, ssm_receipt *out, void *stream);

/* Resume `slot` from a host blob of `len` bytes and its receipt (the
 * section "Make reset, checkpoint, and cancellation observable" of "Mamba
 * Streaming State That Survives Chunking": a resume that does not match is
 * refused).  The blob may hold several arrays; the scan state is the last one
 * (a Mamba blob is [conv_state, ssm_state]), of shape [H, P, N] after any
 * leading extents of 1; with a conv of K > 1 attached the array before it is
 * the conv state, [C, K-1] (required).  Dtype codes 0 or 2 (fp32 words; for
 * code 2 every word must be a bf16 value) or 1 (fp16, widened exactly).
 * SSM_E_SCHEMA,
 * with the slot unchanged, for a malformed blob (wrong version, truncated,
 * trailing bytes, unknown dtype code), a state array of the wrong shape, a
 * receipt that does not match the handle, or a checksum (taken over the
 * widened fp32 words) that does not match the receipt.  The slot takes the
 * receipt's stream id, position and chunk sequence.  Synchronises `stream`. */
ssm_status ssm_state_deserialize(ssm_handle h, int32_t slot, const void *h_blob, size_t len,
                                 const ssm_receipt *r, void *stream);

/* -------------------------------------------- conv1d and the gated output */
/* The steps on either side of the scan.  The pages name the conv state as half
 * of a Mamba layer's recurrent state (the state blob of "SSM.PREFIX.* --
 * recurrent-state companion" lists [conv_state, ssm_state]) but define
 * neither step; these are the Mamba-2 block's:
 *   conv:  y[t,c] = act(b[c] + sum_{k<K} w[c,k] * x[t-(K-1)+k, c]), tap K-1 on
 *          the current token, act = SiLU (v * sigmoid(v)) or the identity;
 *   state: per slot and channel, the K-1 inputs before the next token, oldest
 *          first, fp32 [S, C, K-1]; a reset on token t hides every input
 *          before t, as for the scan;
 *   gate:  g = y * SiLU(z), then optionally each group of channels divided
 *          by its root mean square and scaled by a weight. */

/* Bytes of the conv state for n_slots slots: n_slots * C * (K-1) * 4, or 0
 * for a bad shape. */
size_t ssm_conv_state_bytes(int32_t n_slots, int32_t C, int32_t K);

/* Attach a causal depthwise conv of C channels and width K (1 <= K <= 4) to
 * the handle: d_conv_state[S, C, K-1] (device fp32, caller-owned; NULL when
 * K = 1), d_w[C, K] and d_bias[C] or NULL (device fp32; they must outlive the
 * handle), act 1 for SiLU, 0 for none.  The state memory is not touched:
 * ssm_state_reset / ssm_state_init clear both the conv state and the scan
 * state of a slot from now on. */
ssm_status ssm_conv_attach(ssm_handle h, int32_t C, int32_t K, int32_t act, float *d_conv_state,
                           const float *d_w, const float *d_bias);

/* The conv over one chunk of `slot`'s stream: x[L, C] in, y[L, C] out
 * (device, the handle's io dtype; y must not overlap x), h_reset host u8[L]
 * or NULL.  The slot's conv state is the carry-in and receives the carry-out,
 * so a stream cut into chunks gives the outputs of the whole stream.  Call
 * it once per chunk, in order, with the chunk's reset flags (the conv keeps
 * no sequence numbers of its own). */
ssm_status ssm_conv_chunk(ssm_handle h, int32_t slot, int64_t L, const void *x,
                          const uint8_t *h_reset, void *y, void *stream);

/* One token for each of `batch` distinct slots: x[batch, C] in, y[batch, C]
 * out; h_reset host u8[batch] or NULL (a set flag starts the slot's conv
 * window empty). */
ssm_status ssm_conv_decode(ssm_handle h, int32_t batch, const int32_t *h_slot_ids, const void *x,
                           const uint8_t *h_reset, void *y, void *stream);

/* Gated output over rows x C (device, io_dtype SSM_F32 or SSM_BF16):
 * out = y * SiLU(z); with d_norm_w[C] (device fp32) non-NULL, each group of
 * `group` channels (group divides C) is then divided by
 * sqrt(mean(g^2) + eps) and multiplied by d_norm_w.  out may be y. */
ssm_status ssm_gate(int32_t io_dtype, int64_t rows, int32_t C, int32_t group, const void *y,
                    const void *z, const float *d_norm_w, float eps, void *out, void *stream);

/* Read a slot's position (tokens since the stream's start or last reset, the
 * counter of the runnable artifact in "Mamba Streaming State That Survives
 * Chunking") and next expected chunk sequence number (section "Let the full
 * scan define legal chunking").  Either pointer may be NULL.  SSM_E_INVALID_ARG
 * for a bad slot. */
ssm_status ssm_get_position(ssm_handle h, int32_t slot, int64_t *pos, uint64_t *chunk_seq);

/* Read the replay log length of a slot (committed entries) and whether a
 * replay/copy step awaits commit. */
ssm_status ssm_get_log_state(ssm_handle h, int32_t slot, int32_t *log_len, int32_t *pending);

/* Lifecycle counters of the handle. */
ssm_status ssm_get_counters(ssm_handle h, ssm_counters *out);

/* --------------------------------------------------------------------- misc */

const char *ssm_last_error(void); /* message of the calling thread's last error */
uint64_t ssm_code_rev(void);      /* revision of the state semantics and kernels */

#ifdef __cplusplus
}
#endif
#endif /* SSM_STREAM_H */

/*
 * gqa_attn.h -- C ABI of libgqa_attn.so: grouped-query attention forward on
 * AMD Instinct MI355X (gfx950).
 *
 * One operation in three regimes -- full prefill, chunked prefill and
 * single-token KV-cache decode:
 *
 *     O = softmax(Q K^T * scale [+ causal mask]) V
 *
 * MHA, GQA and MQA are one code path: query head h reads K/V head
 * h / (Hq / Hkv), so g = Hq / Hkv consecutive query heads share one K/V head
 * (BootstrapAI evolution log, entry "Kernel 9 -- GQA Flash Attention
 * (MHA/GQA/MQA Unified)": the one-line head mapping, its Q/KV stride split
 * and the MHA / GQA / MQA mode table).  Prefill and decode are the two
 * regimes of the kaispace.site note on Chunked Prefill (prefill is
 * compute-bound, decode is bound by KV-cache reads); chunked prefill is a
 * query chunk placed at an absolute position q_offset.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers on the current HIP device,
 *    contiguous row-major (innermost dimension last), owned by the caller.
 *    The library never frees or keeps them.  Outputs must not alias inputs.
 *  - dtype: GQA_DTYPE_BF16 (bf16 inputs and output, fp32 accumulation) or
 *    GQA_DTYPE_F32 (fp32 everywhere).  All tensors of one call share it.
 *  - stream: a hipStream_t (NULL = the legacy default stream).  Calls only
 *    enqueue work and return; results are valid once the stream has been
 *    synchronised.
 *  - Every argument is validated on the host before any HIP call; on any
 *    error nothing is launched and the output is not written.  There is no
 *    fallback path: an unsupported case returns GQA_ERR_UNSUPPORTED.
 *  - Library state: one small block of scheduler counters per (device,
 *    stream), allocated and cleared on the first call that needs it, and,
 *    for forwards with fewer units than resident workgroups, a per-stream
 *    buffer of partial records grown when a call needs more (a replaced
 *    buffer is kept, so launches already queued and graphs captured earlier
 *    stay valid); all of it is kept until the process ends.  Calls on one
 *    stream are ordered; calls on different streams use different state.
 *  - HIP graphs: a call may be captured once one eager call with the same
 *    sizes has run on the capturing stream -- it then allocates nothing and
 *    records no memset, and each persistent launch leaves its counters at
 *    zero for the next replay.  A call that would have to set that state up
 *    while its stream is capturing fails with GQA_ERR_UNSUPPORTED and
 *    launches nothing.  Replays use the capturing stream's state, so a
 *    replay must not overlap other calls on that stream's state (replay on
 *    the capturing stream, or order the streams).
 *  - Return value: a gqa_status_t.  gqa_last_error_string() gives the
 *    detail of the most recent failure on the calling thread.
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GQA_DTYPE_F32 = 0,
  GQA_DTYPE_BF16 = 1
} gqa_dtype_t;

typedef enum {
  GQA_OK = 0,
  GQA_ERR_NULL_POINTER = 1,  /* a required pointer is NULL                          */
  GQA_ERR_BAD_SHAPE = 2,     /* a size <= 0, q_offset < 0, or an index overflows   */
  GQA_ERR_HEAD_GROUPING = 3, /* Hq is not a multiple of Hkv                        */
  GQA_ERR_UNSUPPORTED = 4,   /* head dim not in {32,64,128}, unknown dtype,
                                non-finite scale                                    */
  GQA_ERR_WORKSPACE = 5,     /* decode workspace NULL or smaller than required      */
  GQA_ERR_NO_DEVICE = 6,     /* no HIP device, or the current device is not gfx950 */
  GQA_ERR_HIP = 7            /* a HIP runtime or launch error                       */
} gqa_status_t;

/*
 * Prefill / chunked-prefill forward.
 *
 *   q, o : [B, Hq,  Nq, d]      k, v : [B, Hkv, Nk, d]
 *
 * Query row i sits at absolute position q_offset + i.  With causal != 0 it
 * sees keys j <= q_offset + i (diagonal included); without, all Nk keys and
 * q_offset is ignored.  A chunk of Nq queries of a longer prompt at
 * q_offset attending to the Nk = q_offset + Nq keys before and including it
 * is the chunked-prefill case of the kaispace.site note.  scale multiplies
 * Q K^T before the softmax (1/sqrt(d) is the usual value; any finite value
 * is accepted).
 *
 * Requirements: B, Hq, Hkv, Nq, Nk >= 1; Hq % Hkv == 0; d in {32, 64, 128};
 * q_offset >= 0 when causal; Nq*d and Nk*d below 2^31.
 */
int gqa_attn_fwd(const void* q, const void* k, const void* v, void* o,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 int causal, int q_offset, float scale,
                 int dtype, void* stream);

/*
 * The same forward over strided tensors, e.g. token-major [B, N, H, d]
 * (BTHD) activations used in place, with no layout copy.
 *
 *   q_strides  : host pointer to 3 int64 element strides of Q and O, in the
 *                order {batch, head, token}
 *   kv_strides : host pointer to 3 int64 element strides of K and V, same order
 *
 * Element (b, h, i, c) of Q sits at q + b*q_strides[0] + h*q_strides[1] +
 * i*q_strides[2] + c, and likewise for O; K and V use kv_strides.  The head
 * dimension is always contiguous.  Contiguous [B, H, N, d] is {H*N*d, N*d,
 * d}; BTHD is {N*H*d, d, H*d}.  Two stride sets, one for the query side and
 * one for the KV side, as in the GQA launcher of the BootstrapAI evolution
 * log ("Kernel 9"); token-major attention that removes the layout copies
 * around the kernel follows the microLLM-rocm optimization log (experiments
 * 162-164 and 201-204).
 *
 * Additional requirements (else nothing is launched):
 *   strides >= 0 (GQA_ERR_BAD_SHAPE) and multiples of 16 bytes
 *   (GQA_ERR_UNSUPPORTED); the Q/O strides must describe non-overlapping
 *   output rows (GQA_ERR_BAD_SHAPE); the K/V token stride below 2^25 bytes
 *   (GQA_ERR_BAD_SHAPE).  K and V may overlap or repeat (a zero stride
 *   broadcasts); O must not overlap Q, K or V.  Everything else as
 *   gqa_attn_fwd, whose result this equals bit for bit for the same values
 *   on the pair, quad and persistent schedules.  Where the balanced schedule
 *   runs (few units), its key-tile chunks follow the resident workgroups of
 *   the kernel launched, which for a run-time K/V stride may be fewer, so
 *   the units can be cut differently and the result then equals
 *   gqa_attn_fwd's to within rounding order.
 */
int gqa_attn_fwd_strided(const void* q, const void* k, const void* v, void* o,
                         int B, int Hq, int Hkv, int Nq, int Nk, int d,
                         const int64_t* q_strides, const int64_t* kv_strides,
                         int causal, int q_offset, float scale,
                         int dtype, void* stream);

/*
 * Packed variable-length forward: nseq sequences of different lengths back
 * to back in token-major tensors, one launch, no padding.
 *
 *   q, o          : [total_q, Hq, d]   (token-major: token, head, d)
 *   k, v          : [total_k, Hkv, d]
 *   cu_seqlens_q  : int32[nseq + 1], device memory; sequence s owns query
 *                   rows [cu_seqlens_q[s], cu_seqlens_q[s+1])
 *   cu_seqlens_k  : int32[nseq + 1], device memory; its key rows
 *   max_seqlen_q  : host int >= every sequence's query count (the schedule
 *                   is sized from it; rows beyond it are not computed)
 *
 * Each sequence is the forward of its own rows, with the head mapping of
 * gqa_attn_fwd: prompts batched into one launch, as the microLLM-rocm
 * optimization log batches prompts of different lengths into one prefill
 * (experiment 101), over token-major tensors (its experiments 201-204).
 * Its Nq queries are its last Nq tokens -- the chunk of a longer prompt in
 * the kaispace.site note "Chunked Prefill", the whole prompt when Nq = Nk --
 * so with causal = 1 query i sees keys j <= Nk - Nq + i; a row that sees no
 * key (Nk = 0, or i < Nq - Nk) is all zero.  The offsets must be
 * non-decreasing and within the tensors; they are read on the device and
 * not checked.  Work units are (sequence, K/V head, query-position block)
 * taken heaviest first from the persistent schedule's queues; units past a
 * sequence's queries cost one take.
 *
 * Requirements (else nothing is launched): pointers non-NULL
 * (GQA_ERR_NULL_POINTER); nseq, max_seqlen_q, Hq, Hkv, d >= 1,
 * max_seqlen_q <= 2^30, 64 key rows (64 * Hkv * d elements) under 2 GiB, at most
 * 2^31 - 1 work units (GQA_ERR_BAD_SHAPE); Hq a multiple of Hkv (GQA_ERR_HEAD_GROUPING); d in
 * {32, 64, 128}, dtype known, scale finite, q/k/v/o 16-byte aligned and the
 * offset arrays 4-byte aligned (GQA_ERR_UNSUPPORTED).  O must not overlap
 * Q, K or V.  Same scale, dtype, stream and error behaviour as gqa_attn_fwd.
 */
int gqa_attn_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int nseq,
                        int max_seqlen_q, int Hq, int Hkv, int d, int causal, float scale,
                        int dtype, void* stream);

/*
 * Bytes of device workspace gqa_attn_decode needs for these sizes (an upper
 * bound that does not depend on seqlens).  Returns 0 for invalid sizes.
 */
size_t gqa_attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Smax, int d);

/*
 * Single-token KV-cache decode.
 *
 *   q, o            : [B, Hq, d]
 *   kcache, vcache  : [B, Hkv, Smax, d]   (capacity Smax per head)
 *   seqlens         : int32[B], device memory
 *
 * The single query of row b attends cache slots [0, n) with
 * n = clamp(seqlens[b], 0, Smax): the caller has already written the new
 * token's K/V into slot n-1.  Slots >= n are never read (they may hold
 * anything, NaN included).  A row with n == 0 gets an all-zero output.
 * Cache heads are addressed in place through the head mapping, with no
 * per-query-head copies (microLLM-rocm optimization log, experiment 004,
 * and the per-head capacity stride of experiment 062); the KV sequence is
 * cut into parts (bf16) or splits (fp32) whose partial softmax states are
 * merged by a second pass (the split-sequence cached attention of
 * experiments 283/284), in a fixed order, so results repeat bit for bit.
 *
 * workspace: device memory of at least gqa_attn_decode_workspace_bytes(...)
 * bytes, owned by the caller; its contents on entry do not matter.  One
 * workspace must not be used by two calls that may run concurrently.
 */
int gqa_attn_decode(const void* q, const void* kcache, const void* vcache,
                    const int32_t* seqlens, void* o,
                    int B, int Hq, int Hkv, int Smax, int d, float scale,
                    int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gqa_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP-graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It allocates nothing -- no hipMalloc, no
 * allocating library call -- and takes its split records from a static
 * device array of GQA_DECODE_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on each GPU it runs on until the process ends.
 *
 * Arguments, layouts, semantics, status codes and outputs are those of
 * gqa_attn_decode (the same kernels, the same splits: the results are
 * bit-identical to a gqa_attn_decode call on the same inputs).  A call
 * whose gqa_attn_decode_workspace_bytes(B, Hq, Hkv, Smax, d) exceeds
 * GQA_DECODE_NOALLOC_SCRATCH_BYTES returns GQA_ERR_WORKSPACE, before any
 * HIP call.
 *
 * Every call on one GPU shares that GPU's scratch array: calls that may
 * overlap in time on one GPU (on different streams, or a captured graph
 * replayed while another call runs) race on it and are not allowed.  Calls
 * ordered on one stream are fine; nothing in the array has to start zeroed.
 */
#define GQA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int gqa_attn_decode_noalloc(const void* q, const void* kcache, const void* vcache,
                            const int32_t* seqlens, void* o,
                            int B, int Hq, int Hkv, int Smax, int d, float scale,
                            int dtype, void* stream);

/*
 * Decode step that also appends the new token's K/V to the caches, in the
 * same launch.
 *
 *   q, o            : [B, Hq, d]
 *   k_new, v_new    : [B, Hkv, d]        the new token's key / value rows
 *   kcache, vcache  : [B, Hkv, Smax, d]  read, and written at the positions
 *   positions       : int32[B], device memory
 *
 * Row b with p = positions[b] in [0, Smax) stores k_new[b, hk, :] and
 * v_new[b, hk, :] into cache slot p of every K/V head hk, and its query
 * heads attend slots [0, p] -- the new token included.  Any other p marks
 * the row inactive: nothing is stored and its output rows are zero.  Slots
 * > p are never read.  The positions are neither checked on the host nor
 * advanced: the caller moves each active row to p + 1 for the next step.
 * This is the single-launch store of one position's K and V (microLLM-rocm
 * optimization log, experiment 025) with a per-row position table, so rows
 * at different positions decode in one batch (its experiments 083/084 and
 * 098; inactive rows skipped explicitly as in experiment 097).  The
 * attention itself is that of gqa_attn_decode with seqlens[b] = p + 1.
 *
 * k_new, v_new, kcache and vcache must not overlap.  Workspace, stream,
 * status codes and error behaviour are those of gqa_attn_decode (same
 * workspace size).  On an error return nothing has been launched and the
 * caches are unchanged.
 */
int gqa_attn_decode_append(const void* q, const void* k_new, const void* v_new,
                           void* kcache, void* vcache, const int32_t* positions, void* o,
                           int B, int Hq, int Hkv, int Smax, int d, float scale,
                           int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode over a pool of cache rows reached through a slot table: row b of
 * the batch reads -- and, appending, writes -- cache row slots[b], so a
 * serving loop can keep its sequences wherever the pool has room, reorder
 * or compact its batch, and leave finished or waiting rows out, without
 * moving any cache (the microLLM-rocm optimization log: positions through a
 * small per-row table, experiment 098, and compaction of the active rows,
 * experiment 097).
 *
 *   q, o           : [B, Hq, d]            (batch row b)
 *   kcache, vcache : [Ncache, Hkv, Smax, d]
 *   slots          : int32[B], device; slots[b] in [0, Ncache) names row b's
 *                    cache row, any other value makes row b inactive: its
 *                    output is all zero and nothing of the cache is read or
 *                    written for it
 *   lengths        : int32[B], device; without k_new / v_new, the number of
 *                    cached tokens row b attends (clamped to [0, Smax]);
 *                    with them, the position p of row b's new token, as
 *                    gqa_attn_decode_append's positions (p outside [0, Smax)
 *                    makes the row inactive)
 *   k_new, v_new   : both NULL (plain decode) or both [B, Hkv, d] (append:
 *                    row b's new K/V rows go to position p of cache row
 *                    slots[b], and the row attends positions 0 .. p)
 *
 * Rows may share a slot when nothing is appended; appending rows must have
 * different slots (two writes to one cache row race).  With slots[b] = b and
 * Ncache = B the results are those of gqa_attn_decode / _append bit for bit.
 * Workspace: gqa_attn_decode_workspace_bytes(B, Hq, Hkv, Smax, d).  Inactive
 * rows are found on the device; their parts end at once.  Errors as
 * gqa_attn_decode / _append; Ncache < 1 -> GQA_ERR_BAD_SHAPE; a NULL slots
 * or lengths, or only one of k_new / v_new -> GQA_ERR_NULL_POINTER.
 */
int gqa_attn_decode_slots(const void* q, const void* k_new, const void* v_new, void* kcache,
                          void* vcache, int Ncache, const int32_t* slots, const int32_t* lengths,
                          void* o, int B, int Hq, int Hkv, int Smax, int d, float scale,
                          int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Mixed batch of one layer in one persistent launch: the causal query chunk
 * of a chunked prefill and single-token decode rows.
 *
 *   chunk (B >= 0 sequences; B == 0: none, and q, k, v, o may be NULL):
 *     q, o            : [B, Hq, Nq, d]
 *     k, v            : [B, Hkv, Nk, d]
 *     query row i sits at position q_offset + i and sees keys
 *     j <= min(q_offset + i, Nk - 1) -- gqa_attn_fwd with causal = 1.
 *   decode rows (Bd >= 0; Bd == 0: none, and qd, kcache, vcache, seqlens,
 *   od, workspace may be NULL):
 *     qd, od          : [Bd, Hq, d]
 *     kcache, vcache  : [Bd, Hkv, Smax, d]
 *     seqlens         : int32[Bd], device memory
 *     row b attends cache slots [0, clamp(seqlens[b], 0, Smax)) --
 *     gqa_attn_decode.
 *   Hq, Hkv, d, scale and dtype are shared by both parts (one layer).
 *
 * The kaispace.site note "Chunked Prefill" describes the batch: prefill
 * chunks (compute-bound) beside decode tokens (memory-bound).  Both come
 * from one persistent launch whose workgroups take the chunk's units (the
 * GQA head mapping and heaviest-first unit queues of the persistent prefill
 * schedule) and then the decode work from the same counters -- the
 * "Kernel 10" of the BootstrapAI evolution log, persistent scheduling with
 * the GQA head mapping -- so decode work fills the CUs the chunk leaves
 * idle.  The chunk runs as gqa_attn_fwd would run it: quad units when that
 * call takes them (few, long units); else, with too few units to balance
 * whole ones, the balanced schedule's key-tile chunks, sized for half of
 * the resident workgroups so the decode work starts at once on the rest;
 * else the persistent schedule's units.  Merge launches follow: the
 * chunk's units cut by the balanced schedule, then the decode rows'
 * partial states.  The chunk's outputs equal gqa_attn_fwd's bit for bit
 * when both cut its keys the same way (the quad and persistent units), and
 * to within rounding order otherwise.  bf16
 * decode rows run gqa_attn_decode's parts and equal its outputs bit for
 * bit.  fp32 decode rows use gqa_attn_decode's splits, and equal its
 * outputs bit for bit, unless the chunk's units fill every resident
 * workgroup; then they are cut into about twice as many splits (eight
 * decode waves per CU, run in the chunk's tail) and equal its outputs to
 * within rounding order.
 *
 * workspace: at least gqa_attn_decode_workspace_bytes(Bd, Hq, Hkv, Smax, d)
 * bytes when Bd > 0, as for gqa_attn_decode.  Calls that may run
 * concurrently must use different streams (each stream has its own
 * scheduler counters) and different workspaces.  The first call on a
 * stream allocates and clears that stream's counters, and a call whose
 * chunk needs more partial-record space than the stream holds grows it;
 * later calls of the same sizes allocate nothing and record no memset, so
 * they may be captured in a HIP graph (see the conventions at the top).
 *
 * Errors: B < 0 or Bd < 0 -> GQA_ERR_BAD_SHAPE; a NULL pointer of a part
 * that is present -> GQA_ERR_NULL_POINTER; otherwise each present part is
 * checked as gqa_attn_fwd / gqa_attn_decode check it, with the same codes.
 * B == Bd == 0 returns GQA_OK with nothing launched.  On any error nothing
 * is launched.
 */
int gqa_attn_mixed(const void* q, const void* k, const void* v, void* o,
                   int B, int Nq, int Nk, int q_offset,
                   const void* qd, const void* kcache, const void* vcache,
                   const int32_t* seqlens, void* od, int Bd, int Smax,
                   int Hq, int Hkv, int d, float scale, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace gqa_attn_bwd needs for these sizes: two fp32
 * row statistics per query row (B * Hq * Nq rows, rounded up to 16 bytes),
 * then, when the K/V side is small (fewer than 1024 key blocks of 64 keys),
 * P = min(16, ceil(1024 / (ceil(Nk / 64) * Hkv * B))) fp32 partial copies
 * of dk and dv (P * 2 * B * Hkv * Nk * d floats).  Returns 0 for invalid
 * sizes.
 */
size_t gqa_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d);

/*
 * Backward of gqa_attn_fwd: the gradients dq, dk, dv of a loss L given
 * dout = dL/do, for the forward with the same q, k, v, causal, q_offset and
 * scale, whose output o the caller passes back in.
 *
 *   q, o, dout, dq     : [B, Hq, Nq, d]
 *   k, v, dk, dv       : [B, Hkv, Nk, d]   (same dtype for all; contiguous)
 *
 * With P the forward's softmax weights, dP = dout V^T, D = rowsum(dout o)
 * and dS = P (dP - D):  dq = scale dS K,  dk = scale dS^T Q,  dv = P^T dout,
 * where dk and dv of K/V head hk are summed over its g query heads
 * h = hk*g .. hk*g + g-1.  This is the backward boundary of the
 * microLLM-rocm optimization log: experiment 044 (QK, causal softmax, PV
 * and the GQA head mapping under one forward/backward boundary, no T x T
 * probabilities kept, no K/V head copies) and experiments 051-054 (each
 * row's probabilities recomputed; the K/V gradients reduced over the heads
 * that share a K/V head -- here in registers, without atomics, so the
 * result is run-to-run reproducible).
 *
 * workspace: device memory of at least gqa_attn_bwd_workspace_bytes(B, Hq,
 * Hkv, Nq, Nk, d) bytes, owned by the caller, contents on entry irrelevant;
 * it receives each row's log-sum-exp and D, and the fp32 dk, dv of the
 * parts (up to sixteen) each key block's query range is cut into, added in a
 * fixed order at the end.  scale must be finite and > 0
 * (GQA_ERR_UNSUPPORTED otherwise).  Outputs must not alias inputs.  Other
 * status codes and error behaviour as gqa_attn_fwd (plus GQA_ERR_WORKSPACE).
 * Launches on the stream: dq (with the row statistics), dk/dv, and, with
 * more than one query part, the merge of the parts.
 */
int gqa_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 void* dq, void* dk, void* dv,
                 int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 int causal, int q_offset, float scale,
                 int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Static English name of a status code (never NULL). */
const char* gqa_status_string(int status);

/* Detail of the most recent failing call on this thread ("" if none). */
const char* gqa_last_error_string(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */

/*
 * jfa.h -- C ABI of libjfa.so: jagged (variable-length) multi-head attention,
 * forward and backward, on one AMD Instinct MI355X (gfx950).
 *
 * What it computes.  Jagged Flash Attention as described on the web page
 * piletech.kr/articles/112134 (Meta's GEM ads-model training efficiency
 * write-up), section 상세 정리 (Detailed notes):
 *   - jagged-input item: every sequence of a batch has its own length;
 *     attention runs per sequence with no padding, for self attention and for
 *     cross attention with different query and key lengths;
 *   - Jagged Flash Attention item: exact attention computed directly on the
 *     packed variable-length tensors, masking by subtraction instead of a
 *     -inf fill, and a backward pass whose parallel split has no atomics;
 *   - GDPA item: a non-softmax activation in place of softmax.  This library
 *     implements it as silu(scale * q.k) / L_kv, L_kv being the sequence's key
 *     count (also under causal masking).
 * For one sequence b and head h, with S = scale * Q K^T over its Lq queries
 * and Lk keys, and query i seeing key j iff j < Lk and (not causal or
 * j <= i + Lk - Lq):
 *   softmax: out_i = sum_j P_ij V_j, P = softmax over the visible keys,
 *            lse_i = ln sum_j exp(S_ij) over visible j;
 *            a row with no visible key gives out_i = 0 and lse_i = -inf;
 *   silu:    out_i = sum_j silu(S_ij) / Lk * V_j over visible j.
 * The backward returns the gradients of sum(out * dout) w.r.t. q, k and v.
 *
 * Layout (all row-major, contiguous, device memory owned by the caller):
 *   q, out, dout, dq : [total_q, heads, head_dim]
 *   k, v, dk, dv     : [total_kv, heads, head_dim]
 *   lse              : float [heads, total_q] (natural log)
 *   q_offsets        : int32 [batch + 1], q_offsets[0] = 0,
 *                      q_offsets[batch] = total_q, non-decreasing
 *   kv_offsets       : int32 [batch + 1], likewise with total_kv
 * Sequence b owns rows q_offsets[b] .. q_offsets[b+1]-1 of q (and of out,
 * dout, dq) and rows kv_offsets[b] .. kv_offsets[b+1]-1 of k (and v, dk, dv).
 * Element type: dtype JFA_DTYPE_BF16 (bfloat16) or JFA_DTYPE_FP32 (float) for
 * q, k, v, out, dout, dq, dk, dv alike.  Arithmetic: bf16 operands with fp32
 * accumulation (fp32 operands for JFA_DTYPE_FP32); results are rounded to
 * the element type to nearest even.
 *
 * Ownership and side effects.  The library never allocates or frees device
 * memory: scratch space is the caller's `workspace` (size from
 * jfa_workspace_size).  Inputs, offsets included, are only read.  Every
 * (row, head) of out, lse, dq, dk and dv that belongs to a sequence is
 * written exactly once; nothing else is written, so outputs need no
 * clearing.  Calls are asynchronous: they enqueue kernels on `stream` and
 * return; no call synchronises with the host.  The library holds no mutable
 * global state, so calls from several threads are safe; calls that share a
 * workspace must be ordered on one stream.
 *
 * Errors.  Every function returns a jfa_status.  Arguments are validated on
 * the host before anything is enqueued:
 *   JFA_ERR_INVALID_ARGUMENT  a required pointer is NULL; batch < 0;
 *       heads < 1; a total or max length < 0; a scale that is not finite
 *       or is below 1e-20 (zero and negative scales included: masking
 *       needs a positive scale); a bad
 *       activation, dtype or causal flag; a value pointer not 16-byte
 *       aligned; total_* * heads * head_dim >= 2^31 elements;
 *   JFA_ERR_UNSUPPORTED  head_dim not in {32, 64, 128}; heads > 256; a
 *       maximum length whose tile count exceeds the scheduler's 1023 cost
 *       classes (max_kv_len > 65472, or max_q_len > 65472 in the backward);
 *   JFA_ERR_WORKSPACE_TOO_SMALL  workspace_bytes < jfa_workspace_size(...);
 *   JFA_ERR_HIP  a HIP launch failed; jfa_last_error() has HIP's message.
 * batch == 0 (or no rows at all) is a successful no-op.  The offsets live in
 * device memory and are not validated by default: offsets that break the
 * rules above, or lengths above max_q_len / max_kv_len, are undefined
 * behaviour.  With the offsets check on (JFA_OPT_CHECK_OFFSETS, or the
 * environment variable JFA_CHECK_OFFSETS=1) they are checked on the device
 * instead (see jfa_check_device_error).
 */
#ifndef JFA_H_
#define JFA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum jfa_status {
  JFA_OK = 0,
  JFA_ERR_INVALID_ARGUMENT = 1,
  JFA_ERR_UNSUPPORTED = 2,
  JFA_ERR_WORKSPACE_TOO_SMALL = 3,
  JFA_ERR_HIP = 4
};

enum jfa_activation { JFA_ACT_SOFTMAX = 0, JFA_ACT_SILU = 1 };
enum jfa_dtype { JFA_DTYPE_BF16 = 0, JFA_DTYPE_FP32 = 1 };
enum jfa_pass {
  JFA_PASS_QUERY_TILES = 0,
  JFA_PASS_KEY_TILES = 1,
  JFA_PASS_DQ_TILES = 2,
  JFA_PASS_DQ_STORED_TILES = 3
};

/* Bytes of device workspace jfa_forward (for_backward = 0) or jfa_backward
 * (for_backward = 1) needs for these sizes and element type (dtype is a
 * jfa_dtype).  Never fails; returns 0 for arguments the calls would reject.
 * The backward's workspace includes a store for the dS blocks (32 queries x
 * 32 keys each, in the element type) of every query block:
 * heads * (total_q / 32 + batch) * ceil(max_kv_len / 32) blocks.  When that
 * store would exceed 16 GiB it is left out, and the backward then recomputes
 * dS in its dQ pass (slower, same results up to rounding).
 * for_backward = 2 gives the smallest workspace jfa_backward accepts: the
 * same without the dS store.  jfa_backward given less than the full size but
 * at least that recomputes dS in its dQ pass. */
size_t jfa_workspace_size(int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q,
                          int32_t total_kv, int32_t max_kv_len, int32_t dtype, int32_t for_backward);

/* Forward pass (Jagged Flash Attention item; GDPA item for JFA_ACT_SILU).
 * scale: score scale, typically 1/sqrt(head_dim).  lse may be NULL only for
 * JFA_ACT_SILU (no log-sum-exp exists there); it is not written for SILU.
 * Enqueues: the work-list builder, then the attention kernel.  When every
 * sequence is short (max_q_len <= 64 and max_kv_len <= 64) the attention
 * kernel runs as a two-wave variant that fits twice the work items per
 * compute unit; its outputs equal the four-wave kernel's bit for bit, and
 * the option JFA_OPT_FWD_SHORT = 0 keeps the four-wave kernel.  That
 * variant takes one workgroup per (sequence, head) straight from the
 * offsets, and no work list is built, unless the offsets check is on. */
int jfa_forward(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                const int32_t* kv_offsets, int32_t batch, int32_t heads, int32_t head_dim,
                int32_t total_q, int32_t total_kv, int32_t max_q_len, int32_t max_kv_len, float scale,
                int32_t activation, int32_t causal, int32_t dtype, void* out, float* lse, void* workspace,
                size_t workspace_bytes, hipStream_t stream);

/* jfa_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The work list and the offsets-check
 * word that jfa_forward keeps in the caller's workspace live in an array of
 * the library's own device memory instead: 8 MiB on every GPU the library
 * runs on, held until the process ends.  Arguments, layout, results (bit
 * for bit) and errors are those of jfa_forward, plus JFA_ERR_UNSUPPORTED
 * when jfa_workspace_size(..., for_backward = 0) exceeds 8 MiB (8388608
 * bytes; e.g. batch 256, heads 4, total_q 97k needs about 140 KB) and
 * JFA_ERR_HIP if the array's device address cannot be looked up.  It calls
 * no allocating routine.  All calls on one GPU share its array: calls that
 * overlap on one GPU (several streams or threads) race and must be ordered
 * by the caller.  With the offsets check on the offsets are still checked
 * (rejected offsets write nothing), but the check word is not readable
 * through jfa_check_device_error. */
int jfa_forward_noalloc(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                        const int32_t* kv_offsets, int32_t batch, int32_t heads, int32_t head_dim,
                        int32_t total_q, int32_t total_kv, int32_t max_q_len, int32_t max_kv_len, float scale,
                        int32_t activation, int32_t causal, int32_t dtype, void* out, float* lse,
                        hipStream_t stream);

/* Backward pass (Jagged Flash Attention item: no atomics -- dK/dV are
 * formed by key-tile-major work items and dQ by query-tile-major ones, each
 * output row summed in registers and stored once).  out and lse are the
 * forward's outputs; both may be NULL only for JFA_ACT_SILU.  Results are
 * bitwise reproducible from run to run.  Enqueues: the work-list builder
 * (both lists), the row statistics kernel (softmax only: per row,
 * sum(dout * out) and lse in log2 units, into the workspace), the dK/dV
 * kernel (which also stores the dS blocks in the workspace), then the dQ
 * kernel (dQ = scale * dS K over the stored blocks).  The option
 * JFA_OPT_BWD_DS_STORE = 0, or a workspace sized without the dS store,
 * makes the dQ kernel recompute dS from Q, K, V and dout instead.  When every
 * sequence is short (max_q_len <= 64 and max_kv_len <= 64, bf16 with
 * head_dim 64 or 128), each (sequence, head) is one dK/dV work item that
 * sees all of its keys and queries; that item then also forms and writes
 * the sequence's dQ from dS kept on chip, and the dQ kernel only zeroes the
 * rows of sequences without keys.  The results equal the two-pass ones bit
 * for bit.  The option JFA_OPT_BWD_SHORT_DQ = 0 turns this off; = 1 applies
 * it to the short sequences of any batch (the dQ kernel then skips them). */
int jfa_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, const int32_t* q_offsets, const int32_t* kv_offsets, int32_t batch,
                 int32_t heads, int32_t head_dim, int32_t total_q, int32_t total_kv, int32_t max_q_len,
                 int32_t max_kv_len, float scale, int32_t activation, int32_t causal, int32_t dtype, void* dq,
                 void* dk, void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The same two calls, additionally recording caller-created HIP events on
 * `stream` between their kernel launches, for per-kernel timing (every
 * kernel still runs; with events == NULL they are jfa_forward and
 * jfa_backward).  Forward: 3 events -- [0] before the work-list builder,
 * [1] before the attention kernel, [2] after it.  Backward: 5 events --
 * [0] start, [1] after the work-list builder (both lists, one launch),
 * [2] after the row statistics kernel (right after [1] for SiLU),
 * [3] after the dK/dV kernel, [4] after the dQ kernel.  A NULL entry of
 * `events` skips that point (each recorded event can add a few microseconds
 * between launches).  Events are not recorded when the call is a no-op or
 * is rejected. */
int jfa_forward_profiled(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                         const int32_t* kv_offsets, int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q,
                         int32_t total_kv, int32_t max_q_len, int32_t max_kv_len, float scale, int32_t activation,
                         int32_t causal, int32_t dtype, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, hipStream_t stream, hipEvent_t* events);
int jfa_backward_profiled(const void* q, const void* k, const void* v, const void* out, const void* dout,
                          const float* lse, const int32_t* q_offsets, const int32_t* kv_offsets, int32_t batch,
                          int32_t heads, int32_t head_dim, int32_t total_q, int32_t total_kv, int32_t max_q_len,
                          int32_t max_kv_len, float scale, int32_t activation, int32_t causal, int32_t dtype,
                          void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                          hipStream_t stream, hipEvent_t* events);

/* Inspection of the tile scheduler (software tile scheduling for jagged
 * tensors, GDPA item; persistent-kernel scheduling, JFA item).
 * jfa_worklist_bytes: size of the buffer jfa_build_worklist writes.
 * jfa_tile_shape: for a pass, the rows per work-item tile (*tile_rows) and
 * the rows per inner block whose count is an item's cost (*block_rows).
 * jfa_build_worklist: enqueues the builder the attention calls use and
 * writes into `out` (device, >= jfa_worklist_bytes): int32 item count at byte
 * 0, then from byte 16 int32 pairs (sequence, tile << 8 | head), one per
 * item, ordered by cost descending then (sequence, head, tile) ascending,
 * then int32 tile_start[batch + 1], then (32-byte aligned) the per-item
 * records the attention kernels read, whose layout is internal.
 * The builder runs one workgroup per cost class: each counts the items of
 * higher cost (they come first) and places its own class's items, a run of
 * tiles per sequence, by one prefix sum over the sequences.
 * JFA_PASS_QUERY_TILES is the list of the
 * forward kernel, JFA_PASS_DQ_STORED_TILES that of the dQ kernel over the
 * stored dS (larger query tiles), JFA_PASS_DQ_TILES that of the dQ kernel
 * that recomputes dS (smaller query tiles) and JFA_PASS_KEY_TILES that of
 * the dK/dV kernel. */
size_t jfa_worklist_bytes(int32_t pass, int32_t batch, int32_t heads, int32_t total_q, int32_t total_kv);
int jfa_tile_shape(int32_t pass, int32_t* tile_rows, int32_t* block_rows);
int jfa_build_worklist(int32_t pass, const int32_t* q_offsets, const int32_t* kv_offsets, int32_t batch,
                       int32_t heads, int32_t total_q, int32_t total_kv, int32_t max_q_len, int32_t max_kv_len,
                       int32_t causal, void* out, size_t out_bytes, hipStream_t stream);

/* BlockAttention with fixed blocks (same page and section, BlockAttention
 * item: fixed blocks of 64 tokens make attention's cost linear in the
 * length).  Self attention restricted to each run of `block` consecutive
 * tokens of a sequence, counted from its first token, is jagged attention
 * over those runs taken as sequences (the SiLU normaliser is then the run's
 * key count).  jfa_block_offsets writes, into `out` (device int32, at least
 * jfa_block_offsets_count(batch, total, block) = total / block + batch + 1
 * entries), the offsets of those runs for the sequences of `offsets` (device
 * int32 [batch + 1], rows 0 .. total-1), in order, followed by empty
 * sequences up to that count.  Passing `out` as both q_offsets and
 * kv_offsets to jfa_forward / jfa_backward, with batch' = count - 1 and
 * max lengths min(block, longest sequence), computes block attention on the
 * unchanged q, k, v tensors.  Asynchronous on `stream`; writes only
 * out[0 .. count-1].  Errors: NULL pointers, batch or total < 0, block < 1,
 * out_len below the count: JFA_ERR_INVALID_ARGUMENT. */
int64_t jfa_block_offsets_count(int32_t batch, int32_t total, int32_t block);
int jfa_block_offsets(const int32_t* offsets, int32_t batch, int32_t total, int32_t block, int32_t* out,
                      int64_t out_len, hipStream_t stream);

/* Base Batch Shuffling (page piletech.kr/articles/112134, section 핵심
 * 포인트 / Key points, BBS bullet, and section 상세 정리 / Detailed notes,
 * Base Batch Shuffling item): the batch former ahead of this path.  The
 * samples, in input order, form base batches of `base_batch` consecutive
 * samples (the last may be shorter).  A base batch's load is the sum over
 * its samples of their length (cost JFA_BBS_COST_TOKENS) or of its square
 * (JFA_BBS_COST_PAIRS: the (query, key) pairs of self attention).  Base
 * batches are sorted by load, heaviest first (ties: lower index first), and
 * the k-th heaviest is merged with the k-th lightest into merged batch k
 * (the heavier one's samples first, each in input order); with an odd number
 * of base batches the median one is a merged batch of its own, last.  For
 * pairs this minimises the largest merged load.
 * Host arrays (the data loader knows the lengths before any copy):
 *   lengths      int32 [n_samples], >= 0
 *   perm         int64 [n_samples], out: input index of every output sample
 *   batch_start  int64 [jfa_bbs_batch_count(...) + 1], out: merged batch i
 *                is perm[batch_start[i] .. batch_start[i+1]-1]
 * jfa_bbs_batch_count returns ceil(ceil(n_samples / base_batch) / 2), 0 for
 * invalid arguments.  Errors (JFA_ERR_INVALID_ARGUMENT): n_samples < 0,
 * base_batch < 1, a bad cost, a negative length, NULL arrays (lengths and
 * perm may be NULL when n_samples is 0).  Synchronous, host only, no
 * device access. */
enum jfa_bbs_cost { JFA_BBS_COST_TOKENS = 0, JFA_BBS_COST_PAIRS = 1 };
int64_t jfa_bbs_batch_count(int64_t n_samples, int32_t base_batch);
int jfa_bbs_plan(const int32_t* lengths, int64_t n_samples, int32_t base_batch, int32_t cost, int64_t* perm,
                 int64_t* batch_start);

/* BlockAttention with its fused rotary position embedding (page
 * piletech.kr/articles/112134, section 상세 정리 / Detailed notes,
 * BlockAttention item: fixed blocks of 64 tokens, combined with a fused
 * rotary position embedding).  Self attention of every sequence of
 * `offsets` (device int32 [batch + 1], rows 0 .. total-1 of q, k, v, out,
 * dout, dq, dk, dv laid out as for jfa_forward) restricted to each run of
 * `block` consecutive tokens counted from the sequence's first token
 * (1 <= block <= 64).  rope_base = 0: no rotary embedding (the same as
 * jfa_block_offsets + jfa_forward / jfa_backward, bit for bit).  rope_base >
 * 1: Q and K are first turned by the rotary embedding of that base
 * (rotate-half pairing: element i < head_dim/2 pairs with i + head_dim/2 and
 * turns by angle p * base^(-2i/head_dim) at position p), and the gradients
 * of q and k are those of the unturned inputs.  Positions are counted from
 * each block's first token; attention within a block depends on positions
 * only through their differences, so this equals counting from the
 * sequence's first token.  The rotation is fused into the attention
 * kernels (each Q and K row is turned once, on chip): it needs bf16 and
 * head_dim 64 or 128 (JFA_ERR_UNSUPPORTED otherwise).  max_len: the longest
 * sequence (>= 0).  The workspace (jfa_block_workspace_size, for_backward 0
 * or 1) holds the blocks' offsets and the jagged calls' workspace.  events:
 * NULL, or as for jfa_forward_profiled / jfa_backward_profiled (the block
 * offsets kernel runs between events [0] and [1]).  Errors as for
 * jfa_forward / jfa_backward, plus JFA_ERR_INVALID_ARGUMENT for block
 * outside 1 .. 64, a rope_base that is neither 0 nor a finite value above
 * 1, or max_len < 0. */
size_t jfa_block_workspace_size(int32_t batch, int32_t heads, int32_t head_dim, int32_t total, int32_t block,
                                int32_t dtype, int32_t for_backward);
int jfa_block_forward(const void* q, const void* k, const void* v, const int32_t* offsets, int32_t batch,
                      int32_t heads, int32_t head_dim, int32_t total, int32_t max_len, int32_t block, float scale,
                      int32_t activation, int32_t causal, int32_t dtype, float rope_base, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events);
int jfa_block_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                       const float* lse, const int32_t* offsets, int32_t batch, int32_t heads, int32_t head_dim,
                       int32_t total, int32_t max_len, int32_t block, float scale, int32_t activation, int32_t causal,
                       int32_t dtype, float rope_base, void* dq, void* dk, void* dv, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, hipEvent_t* events);

/* Pooled multi-head attention (page piletech.kr/articles/112134, section
 * 상세 정리 / Detailed notes, jagged-input item, which names it among the
 * attention patterns with no definition; this library reads it as pooling by
 * attention): n_seeds query vectors `seeds` [n_seeds, heads, head_dim],
 * shared by every sequence, attend over each sequence's keys and values (no
 * causal mask), pooling sequence b into rows b*n_seeds .. b*n_seeds +
 * n_seeds - 1 of out [batch * n_seeds, heads, head_dim] (lse [heads, batch *
 * n_seeds] for softmax).  The backward writes the gradients of k and v and
 * dseeds [n_seeds, heads, head_dim], the sum over sequences of the seeds'
 * per-sequence gradients (in fp32: each of min(batch, 16) chunks of
 * consecutive sequences summed in order, then the chunks in order:
 * reproducible bit for bit; all zeros for batch 0).  Other arguments, layouts and errors as
 * for jfa_forward / jfa_backward with total_q = batch * n_seeds and the
 * library writing the query offsets, plus JFA_ERR_INVALID_ARGUMENT for
 * n_seeds outside 1 .. 256 or NULL / misaligned seeds or dseeds.  The
 * workspace (jfa_pooled_workspace_size) holds the query offsets, the seeds
 * repeated once per sequence (and the per-sequence seed gradients) and the
 * jagged calls' workspace.  events: NULL, or as for jfa_forward_profiled /
 * jfa_backward_profiled (the seeds' repetition runs between events [0] and
 * [1], the seeds' gradient sum before event [4]). */
size_t jfa_pooled_workspace_size(int32_t batch, int32_t n_seeds, int32_t heads, int32_t head_dim, int32_t total_kv,
                                 int32_t max_kv_len, int32_t dtype, int32_t for_backward);
int jfa_pooled_forward(const void* seeds, const void* k, const void* v, const int32_t* kv_offsets, int32_t batch,
                       int32_t n_seeds, int32_t heads, int32_t head_dim, int32_t total_kv, int32_t max_kv_len,
                       float scale, int32_t activation, int32_t dtype, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, hipEvent_t* events);
int jfa_pooled_backward(const void* seeds, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, const int32_t* kv_offsets, int32_t batch, int32_t n_seeds, int32_t heads,
                        int32_t head_dim, int32_t total_kv, int32_t max_kv_len, float scale, int32_t activation,
                        int32_t dtype, void* dseeds, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                        hipStream_t stream, hipEvent_t* events);

/* MXFP8 attention forward (page piletech.kr/articles/112134, section 핵심
 * 포인트 / Key points, MXFP8 bullet, and section 상세 정리 / Detailed
 * notes, MXFP8 item: training in a microscaled 8-bit format, with the
 * softmax output quantised online).  Number format: OCP Microscaling
 * Formats (MX) v1.0, MXFP8 E4M3: blocks of 32 elements share an E8M0 scale
 * 2^(floor(log2 max|x|) - 8) (at least 2^-127); each element is x / scale
 * rounded to the nearest E4M3 value, ties to even, magnitudes beyond 448
 * clamped to 448.  jfa_mx_forward computes softmax attention (layouts,
 * offsets, causal rule and outputs as for jfa_forward, bf16 only, head_dim
 * 64 or 128) from the MXFP8 quantisations of q and k (blocks of 32
 * head-dim elements) and of v (blocks of 32 consecutive keys of a
 * sequence, counted from its first key, per column), with the weights
 * quantised as well: a row's weights 2^(t_j - m) (t_j = scale log2(e)
 * q.k_j, m the row max) in blocks of 32 consecutive keys counted from the
 * sequence's first key, the block's scale taken from its largest visible
 * weight; invisible keys weigh 0.  The normaliser and lse use the exact
 * weights.  Arithmetic: the products of the 8-bit operands accumulate in
 * fp32; out is rounded to bf16.  When max_q_len <= 64 the attention kernel
 * runs two waves per work item (twice the items per compute unit); its
 * outputs equal the four-wave kernel's bit for bit, and the option
 * JFA_OPT_FWD_SHORT = 0 keeps the four-wave kernel.  Workspace: jfa_mx_workspace_size with
 * with_images = 1 (256-byte aligned; it holds the work list and the three
 * MX images); events: NULL, or 4 events recorded before the quantisation,
 * after it, after the work list and after the attention kernel.  Errors as
 * for jfa_forward with activation softmax and dtype bf16, plus
 * JFA_ERR_UNSUPPORTED for head_dim other than 64 and 128 and
 * JFA_ERR_INVALID_ARGUMENT for a workspace not 256-byte aligned.
 *
 * jfa_mx_attend is the same attention from operands already in MXFP8: the
 * images of q and k (JFA_MX_ROWS) and of v (JFA_MX_KEYS) that
 * jfa_mx_quantize writes, or that a producer fusing the quantisation into
 * its own epilogue writes in that layout (the pages fuse it into the norm
 * and projection kernels).  jfa_mx_forward(q, k, v) equals jfa_mx_quantize
 * of each followed by jfa_mx_attend, bit for bit.  Workspace:
 * jfa_mx_workspace_size with with_images = 0 (the work list); events:
 * NULL, or 3 events, as for jfa_forward_profiled.  Errors as for
 * jfa_mx_forward, plus JFA_ERR_INVALID_ARGUMENT for an image not 256-byte
 * aligned.
 *
 * jfa_mx_quantize writes the MX image of one bf16 tensor x [total, heads,
 * head_dim] (offsets as for jfa_forward) into `image` (jfa_mx_image_bytes,
 * 256-byte aligned): uint8 E4M3 codes at byte 0, uint8 E8M0 scale codes
 * (value 2^(code - 127)) at byte align256(heads * 32 N * head_dim), with N =
 * total / 32 + batch block rows; row i of sequence b is image row
 * 32 (offsets[b] / 32 + b) + i (block row offsets[b] / 32 + b + i / 32).
 *   JFA_MX_ROWS (q, k): codes [heads][32 N][head_dim], scales [heads][32 N]
 *     [head_dim / 32], blocks of 32 consecutive elements of a row.
 *   JFA_MX_KEYS = JFA_MX_COLUMNS (v; for the backward also q, k and
 *     dout): codes [heads][N][head_dim][32]: within a column, row
 *     i of the block at byte 16 ((i / 4) % 2) + 4 (i / 8) + i % 4 (the order
 *     the attention kernel's weights arrive in); scales [heads][N][32]
 *     [head_dim / 32], column 32 c + r at [r][c]; blocks of 32 consecutive
 *     rows of a sequence, per column.
 * Image rows past the end of a sequence's last block hold zero codes; rows
 * in no sequence's blocks are not written.  Errors: those of the sizes as
 * for jfa_forward, JFA_ERR_UNSUPPORTED for head_dim other than 64 and 128,
 * JFA_ERR_INVALID_ARGUMENT for a bad layout or NULL / misaligned pointers,
 * JFA_ERR_WORKSPACE_TOO_SMALL for image_bytes below jfa_mx_image_bytes. */
enum jfa_mx_layout { JFA_MX_ROWS = 0, JFA_MX_KEYS = 1, JFA_MX_COLUMNS = 1 };
size_t jfa_mx_image_bytes(int32_t batch, int32_t heads, int32_t head_dim, int32_t total);
int jfa_mx_quantize(const void* x, const int32_t* offsets, int32_t batch, int32_t heads, int32_t head_dim,
                    int32_t total, int32_t layout, void* image, size_t image_bytes, hipStream_t stream);
size_t jfa_mx_workspace_size(int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q, int32_t total_kv,
                             int32_t with_images);
int jfa_mx_forward(const void* q, const void* k, const void* v, const int32_t* q_offsets, const int32_t* kv_offsets,
                   int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q, int32_t total_kv,
                   int32_t max_q_len, int32_t max_kv_len, float scale, int32_t causal, void* out, float* lse,
                   void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events);
int jfa_mx_attend(const void* q_image, const void* k_image, const void* v_image, const int32_t* q_offsets,
                  const int32_t* kv_offsets, int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q,
                  int32_t total_kv, int32_t max_q_len, int32_t max_kv_len, float scale, int32_t causal, void* out,
                  float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events);

/* MXFP8 attention backward (same page and sections as the MXFP8 forward:
 * training in MXFP8 covers the backward as well).  Every product takes its
 * two operands in MXFP8 blocks of 32 along its own contraction axis:
 *   S = q k^T and dP = dout v^T over the head dimension: q, k, v and dout
 *     in JFA_MX_ROWS images;
 *   dV = P^T dout and dK = scale dS^T q over queries: P and dS quantised in
 *     the kernel in blocks of 32 consecutive queries of a key, counted from
 *     the sequence's first query; dout and q in JFA_MX_COLUMNS images (q
 *     offsets);
 *   dQ = scale dS k over keys: dS in blocks of 32 consecutive keys of a
 *     query, counted from the sequence's first key; k in a JFA_MX_COLUMNS
 *     image (kv offsets).
 * P = exp(scale q.k - lse) is recomputed in fp32 from the quantised scores
 * and the forward's lse; delta = rowsum(dout o out) from the bf16 out and
 * dout; dS = P o (dP - delta) is formed in fp32 before either of its
 * quantisations.  Products accumulate in fp32; dq, dk and dv are written
 * in bf16 [total, heads, head_dim], every row (zeros where no pair is
 * visible).  Each output row is written by one workgroup: no atomics, the
 * result is reproducible bit for bit.
 *
 * jfa_mx_backward takes bf16 q, k, v, out, dout and the forward's lse
 * (arguments, layouts and causal rule as for jfa_backward with activation
 * softmax and dtype bf16, head_dim 64 or 128) and quantises the seven
 * images itself.  Workspace: jfa_mx_backward_workspace_size with
 * with_images = 1 (256-byte aligned: work lists, row statistics and the
 * seven images); events: NULL, or 5 events recorded before the
 * quantisation, after it, after the work lists and row statistics, after
 * the dK/dV kernel and after the dQ kernel.
 *
 * jfa_mx_backward_images takes the seven images instead of q, k, v (and
 * dout for the products; dout and out still give delta): `images` is a
 * host array of 7 device pointers, in this order: q (JFA_MX_ROWS), q
 * (JFA_MX_COLUMNS), k (ROWS), k (COLUMNS), v (ROWS), dout (ROWS), dout
 * (COLUMNS), each as jfa_mx_quantize writes it (256-byte aligned; NULL
 * allowed only for a side whose total is 0).  jfa_mx_backward equals
 * jfa_mx_quantize of each followed by jfa_mx_backward_images, bit for bit.
 * Workspace: jfa_mx_backward_workspace_size with with_images = 0; events:
 * NULL, or 4 events (before the work lists, after them, after dK/dV, after
 * dQ).
 *
 * Errors: as for jfa_backward (softmax, bf16), plus JFA_ERR_UNSUPPORTED for
 * head_dim other than 64 and 128 and JFA_ERR_INVALID_ARGUMENT for a
 * workspace or image not 256-byte aligned or a NULL image array. */
size_t jfa_mx_backward_workspace_size(int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q,
                                      int32_t total_kv, int32_t with_images);
int jfa_mx_backward(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                    const int32_t* q_offsets, const int32_t* kv_offsets, int32_t batch, int32_t heads,
                    int32_t head_dim, int32_t total_q, int32_t total_kv, int32_t max_q_len, int32_t max_kv_len,
                    float scale, int32_t causal, void* dq, void* dk, void* dv, void* workspace,
                    size_t workspace_bytes, hipStream_t stream, hipEvent_t* events);
int jfa_mx_backward_images(const void* const* images, const void* out, const void* dout, const float* lse,
                           const int32_t* q_offsets, const int32_t* kv_offsets, int32_t batch, int32_t heads,
                           int32_t head_dim, int32_t total_q, int32_t total_kv, int32_t max_q_len,
                           int32_t max_kv_len, float scale, int32_t causal, void* dq, void* dk, void* dv,
                           void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events);

/* Device check of the offsets (debug; the jagged-input item's offsets
 * contract).  With the option JFA_OPT_CHECK_OFFSETS = 1 (by default: the
 * environment variable JFA_CHECK_OFFSETS=1, read once), the work-list
 * builder of jfa_forward and jfa_backward first checks on the device that
 * q_offsets[0] = kv_offsets[0] = 0, that neither array decreases, that
 * q_offsets[batch] = total_q and kv_offsets[batch] = total_kv, and that no
 * length exceeds max_q_len / max_kv_len.  If a rule fails, no attention
 * kernel does any work and no output, lse or gradient is written.
 * jfa_check_device_error synchronises `stream` and reports the check of the
 * last call that built a work list in `workspace`: JFA_OK (also when the
 * check was off), or JFA_ERR_INVALID_ARGUMENT with the failed rules in
 * jfa_last_error(); JFA_ERR_HIP if the word cannot be read. */
int jfa_check_device_error(const void* workspace, hipStream_t stream);

/* Process-wide path options, for tests, timing studies and debugging.  Each
 * holds -1 (the library's choice, the default), 0 (off) or 1 (on); a call
 * takes the values set when it is made.  They choose between paths whose
 * results are equal bit for bit (or, for the offsets check, add a device
 * check of the inputs).
 *   JFA_OPT_CHECK_OFFSETS   device check of the offsets (above); default:
 *                           on iff JFA_CHECK_OFFSETS=1 in the environment.
 *   JFA_OPT_BWD_DS_STORE    0: the dQ kernel recomputes dS even when the
 *                           workspace holds the dS blocks.
 *   JFA_OPT_BWD_SHORT_DQ    the dK/dV kernel forms the dQ of short
 *                           sequences: 0 never, 1 whenever it can; default
 *                           when every sequence is short.
 *   JFA_OPT_FWD_SHORT       0: the forward keeps the four-wave kernel for
 *                           batches of short sequences, and the MXFP8
 *                           forward for batches of short query sequences.
 * jfa_set_option returns JFA_ERR_INVALID_ARGUMENT for an unknown option or
 * a value outside -1 .. 1; jfa_get_option returns the value, or -2 for an
 * unknown option. */
enum jfa_option {
  JFA_OPT_CHECK_OFFSETS = 0,
  JFA_OPT_BWD_DS_STORE = 1,
  JFA_OPT_BWD_SHORT_DQ = 2,
  JFA_OPT_FWD_SHORT = 3,
  JFA_OPT_COUNT = 4
};
int jfa_set_option(int32_t option, int32_t value);
int32_t jfa_get_option(int32_t option);

/* Human-readable name of a status code (static storage). */
const char* jfa_status_string(int status);
/* Message of the last JFA_ERR_HIP or argument error on the calling thread. */
const char* jfa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* JFA_H_ */

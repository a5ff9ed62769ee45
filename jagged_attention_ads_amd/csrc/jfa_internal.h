// Internal interfaces between the C-ABI layer (api.cpp) and the kernel
// translation units.  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

namespace jfa {

// Records `msg` as the calling thread's jfa_last_error() and returns status.
int report(int status, const std::string& msg);
// jfa_forward's argument checks (everything but the workspace): JFA_OK, or
// the status it would return, with jfa_last_error() set.
int forward_args_status(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                        const int32_t* kv_offsets, int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q,
                        int32_t total_kv, int32_t max_q_len, int32_t max_kv_len, float scale, int32_t activation,
                        int32_t causal, int32_t dtype, const void* out, const float* lse);

// Tile geometry, shared by the launchers and the host-side sizing code.
constexpr int kFwdBM = 128;     // query rows per forward / dQ work item
constexpr int kFwdBN = 64;      // key rows per forward / dQ inner step
constexpr int kBwdBN = 64;      // key rows per dK/dV work item
constexpr int kBwdBM = 64;      // query rows per dK/dV cost block
constexpr int kDqBM = 64;       // query rows per dQ work item
constexpr int kDqBN = 64;       // key rows per dQ cost block
constexpr int kDqDsBM = 256;    // query rows per work item of the dQ pass over stored dS
constexpr int kMaxBuckets = 1024;   // distinct tile costs the scheduler can sort
constexpr int kMaxHeads = 256;      // head index is packed into 8 bits

enum Pass { kPassQ = 0, kPassKV = 1, kPassDQ = 2, kPassDQS = 3 };

// Per-item record the attention kernels read with one load: the sequence's
// first query and key rows and lengths, the item's head and tile, and the
// sequence index.  Records past the item count have lq = -1.
struct ItemMeta {
  int32_t qs, lq, ks, lk, head, tile, seq, unused;
};

// dS blocks of the backward: 32 queries x 32 keys, stored as the byte image
// of a [key][query] LDS tile.  Sequence b's query block i (rows 32i .. 32i+31
// of the sequence) is block row q_offsets[b] / 32 + b + i, which keeps the
// sequences' ranges disjoint without a prefix sum; a block row holds
// ceil(max_kv_len / 32) key blocks, and a head holds total_q / 32 + batch
// block rows.
constexpr int kDsBlock = 32;
inline int64_t ds_block_rows(int32_t batch, int32_t total_q) { return (int64_t)total_q / kDsBlock + batch; }
inline int64_t ds_key_blocks(int32_t max_kv_len) { return ((int64_t)max_kv_len + kDsBlock - 1) / kDsBlock; }

// Short sequences of the backward: at most kBwdBN queries and 1 .. kBwdBN
// keys.  Such a sequence is a single dK/dV item whose workgroup sees every
// key and every query, so (where the dK/dV kernel has the LDS for it) that
// workgroup also writes the sequence's dQ rows, and the dQ pass skips it.
constexpr bool short_sequence(int lq, int lk) { return lq <= kBwdBN && lk >= 1 && lk <= kBwdBN; }

// Device layout of a work list (all offsets in bytes from its base):
//   0                      int32   item count
//   16                     int2    items[capacity]   (x = sequence, y = tile << 8 | head)
//   16 + 8*cap             int32   tile_start[batch + 1]
//   meta_off (32-aligned)  ItemMeta meta[capacity]
struct WorklistLayout {
  int64_t capacity;
  size_t items_off, tile_start_off, meta_off, bytes;
};
WorklistLayout worklist_layout(int pass, int32_t batch, int32_t heads, int32_t total_rows);

// Optional device check of the offsets before a list is built: with `check`
// set, the builder validates them first; if a rule fails it writes the
// failed rules (kOffsetsBad* bits) to *status and an empty list whose records
// make every attention workgroup exit.  *status is always written when not
// null (0: valid, or not checked).
enum {
  kOffsetsBadFirst = 1,    // q_offsets[0] or kv_offsets[0] is not 0
  kOffsetsBadOrder = 2,    // an offset array decreases
  kOffsetsBadTotal = 4,    // q_offsets[batch] != total_q or kv_offsets[batch] != total_kv
  kOffsetsBadLength = 8,   // a length above max_q_len or max_kv_len
};
struct OffsetCheck {
  int* status;
  int32_t check;
  int32_t total_q, total_kv, max_q_len, max_kv_len;
};

hipError_t launch_sched(int pass, const int32_t* qo, const int32_t* ko, int32_t batch, int32_t heads,
                        int32_t causal, int32_t nbuckets, void* wl_base, const WorklistLayout& lay,
                        const OffsetCheck& chk, hipStream_t stream);
// Inputs and outputs of the softmax backward's row statistics.
struct StatsArgs {
  const void* out;
  const void* dout;
  const float* lse;
  float* lse2;    // [heads, total_q]
  float* delta;   // [heads, total_q]
  int32_t heads;
  int32_t total_q;
};

// The backward's two lists in one launch (two workgroups): the dQ pass's
// query tiles (qpass: kPassQ or kPassDQS over stored dS, kPassDQ recomputing) and the key tiles.  With `stats`,
// the launch's further workgroups form the row statistics meanwhile.
hipError_t launch_sched_pair(int qpass, const int32_t* qo, const int32_t* ko, int32_t batch, int32_t heads,
                             int32_t causal, int32_t nb_dq, void* wl_dq, const WorklistLayout& lay_dq, int32_t nb_kv,
                             void* wl_kv, const WorklistLayout& lay_kv, const StatsArgs* stats, int dtype,
                             int head_dim, const OffsetCheck& chk, hipStream_t stream);

// BlockAttention's fused rotary embedding (see rope_rotate): on = 1 turns Q
// and K (and back the gradients of Q and K); k2 = -2 log2(base) / head_dim,
// so that pair i turns by base^(-2i/d) = exp2(i * k2) per position.  Only for
// batches of short sequences (every query and key length at most 64), bf16,
// head_dim 64 or 128: the kernels that run them turn each row once, counting
// positions from the start of the sequence (for BlockAttention's blocks, of
// the block: attention then depends on positions only through their
// differences).
struct RopeArgs {
  int32_t on;
  float k2;
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* qo;
  const int32_t* ko;
  const ItemMeta* meta;     // query-tile records; null: one item per (sequence, head), block
                            // b * heads + h (batches of short sequences only, see launch_fwd)
  void* out;
  float* lse;
  int32_t heads;
  int32_t total_q;
  int32_t total_kv;
  int32_t causal;
  float scale;        // softmax / silu score scale
  float scale_log2;   // scale * log2(e)
  RopeArgs rope;
};

// short_batch: every sequence has at most 64 queries and 64 keys (the
// two-wave variant of the kernel).  With a.meta null (short_batch only) the
// grid is batch * heads, one block per (sequence, head), and no work list
// is read.
hipError_t launch_fwd(const FwdArgs& a, int head_dim, int dtype, int act, int64_t grid, bool short_batch,
                      hipStream_t stream);

// Pooled multi-head attention (see pooled.hip): query offsets b * n_seeds
// and the seeds repeated per sequence; the seeds' gradient as the sum over
// sequences (fp32, fixed order).
hipError_t launch_pooled_prep(const void* seeds, int64_t seed_bytes, int32_t batch, int32_t n_seeds, void* q,
                              int32_t* q_offsets, hipStream_t stream);
// The sum runs over min(batch, kPooledChunks) chunks of consecutive
// sequences, each summed in order into `partial` (fp32 [chunks, seed
// elements], workspace), then the partials in chunk order.
constexpr int32_t kPooledChunks = 16;
int32_t pooled_chunks(int32_t batch);
hipError_t launch_pooled_reduce(const void* dq, int64_t seed_elems, int32_t batch, int dtype, float* partial,
                                void* dseeds, hipStream_t stream);

// MXFP8 (see mx.hip).  Images index a sequence's rows from a 32-row
// boundary: row i of sequence b at image row 32 (off[b]/32 + b) + i, in
// mx_block_rows(batch, total) blocks of 32 rows.
inline int64_t mx_block_rows(int32_t batch, int32_t total) { return (int64_t)total / 32 + batch; }

// Up to kMxQuantMax bf16 [total, heads, D] tensors into MX images in one
// launch.
// Row image (keys = 0): codes [heads][32 nbr][D], E8M0 scale codes
// [heads][32 nbr][D/32], blocks of 32 elements along a row.  Column image
// (keys = 1): codes [heads][nbr][D][32] with key i of a block at byte
// mx_key_pos(i) of its column, scales [heads][nbr][32][D/32] (column
// 32 c + r at [r][c]), blocks of 32 rows of a sequence per column.
constexpr int kMxQuantMax = 8;
struct MxQuantArgs {
  const void* x[kMxQuantMax];
  const int32_t* off[kMxQuantMax];
  int32_t total[kMxQuantMax];
  int32_t nbr[kMxQuantMax];
  int32_t keys[kMxQuantMax];
  uint8_t* codes[kMxQuantMax];
  uint8_t* scales[kMxQuantMax];
  int32_t batch;
  int32_t heads;
};
hipError_t launch_mx_quant(const MxQuantArgs& a, int head_dim, int count, hipStream_t stream);

struct MxFwdArgs {
  const uint8_t* qx;   // Q row image: codes, scales
  const uint8_t* qs;
  const uint8_t* kx;   // K row image
  const uint8_t* ks;
  const uint8_t* vx;   // V column image
  const uint8_t* vs;
  int64_t rq;          // image rows (32 block rows) of Q and of K / V
  int64_t rk;
  const ItemMeta* meta;   // query-tile records (kPassQ)
  void* out;              // bf16 [total_q, heads, D]
  float* lse;             // [heads, total_q]
  int32_t heads;
  int32_t total_q;
  int32_t causal;
  float scale_log2;
};
hipError_t launch_mx_fwd(const MxFwdArgs& a, int head_dim, bool narrow, int64_t grid, hipStream_t stream);

// MXFP8 backward (see mx_bwd.hip): every product takes its operands in MX
// blocks along its own contraction axis.  Row images (blocks along the head
// dimension) of Q, K, V and dO for S and dP; column images (blocks of 32
// rows of a sequence) of dO and Q for dV and dK, and of K for dQ.
struct MxImage {
  const uint8_t* x;    // codes
  const uint8_t* s;    // E8M0 scale codes
};
struct MxBwdArgs {
  MxImage q, k, v, dout;      // row images
  MxImage qc, kc, doc;        // column images
  int64_t rq;                 // image rows (32 block rows) of the query-side and key-side images
  int64_t rk;
  const ItemMeta* meta_q;     // 128-query tiles (kPassQ): the dQ pass
  const ItemMeta* meta_kv;    // 64-key tiles (kPassKV): the dK/dV pass
  const float* lse2;          // [heads, total_q]: lse * log2(e) (0 for rows without keys)
  const float* delta;         // [heads, total_q]: rowsum(dO o O)
  void* dq;                   // bf16 [total, heads, D]
  void* dk;
  void* dv;
  int32_t heads;
  int32_t total_q;
  int32_t causal;
  float scale;
  float scale_log2;
};
hipError_t launch_mx_bwd_dkdv(const MxBwdArgs& a, int head_dim, int64_t grid, hipStream_t stream);
hipError_t launch_mx_bwd_dq(const MxBwdArgs& a, int head_dim, int64_t grid, hipStream_t stream);

// BlockAttention: the runs of `block` tokens of every sequence as offsets
// (see blocks.hip).
hipError_t launch_block_offsets(const int32_t* off, int32_t batch, int32_t total, int32_t block, int32_t* out,
                                int32_t out_len, hipStream_t stream);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  const int32_t* qo;
  const int32_t* ko;
  const ItemMeta* meta_q;   // query-tile records of the dQ pass (128-row tiles when it reads
                            // the stored dS, 64-row tiles when it recomputes dS)
  const ItemMeta* meta_kv;  // key-tile records (dK/dV pass)
  float* lse2;             // [heads, total_q] workspace: lse * log2(e) per row, and
  float* delta;            // [heads, total_q] delta per row; both written by the row
                           // statistics kernel (softmax), read by both gradient passes
  void* ds;                // dS blocks (see kDsBlock), written by the dK/dV pass and read by
                           // the dQ pass; null when the dQ pass recomputes dS
  int64_t ds_head_blocks;  // blocks per head: ds_block_rows * ds_kb
  int32_t ds_kb;           // key blocks per block row
  int32_t dq_rows;         // query rows per item of the dQ pass over stored dS (128 or kDqDsBM)
  int32_t fuse_short;      // 1: the dK/dV pass writes dQ of short sequences (see short_sequence)
  void* dq;
  void* dk;
  void* dv;
  int32_t heads;
  int32_t total_q;
  int32_t total_kv;
  int32_t causal;
  float scale;
  float scale_log2;
  RopeArgs rope;
};

// Row statistics (softmax): lse2 and delta for every (row, head).
hipError_t launch_bwd_stats(const StatsArgs& a, int head_dim, int dtype, hipStream_t stream);
// Whether the dK/dV kernel for this dtype (0 bf16, 1 fp32) and head_dim
// writes the dQ rows of short sequences when BwdArgs::fuse_short is set.
bool dkdv_fuses_short(int dtype, int head_dim);
// dK/dV pass; with a.ds set it also stores dS for the dQ pass.
hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, int dtype, int act, int64_t grid, hipStream_t stream);
// dQ pass when every sequence is short or has no keys (a.fuse_short set):
// zero rows for the sequences without keys, unless the offsets check word
// `status` (written by the list builder) reports rejected offsets.
hipError_t launch_bwd_dq_keyless(const BwdArgs& a, const int* status, int batch, int head_dim, int dtype,
                                 hipStream_t stream);
// dQ pass: from the stored dS when a.ds is set, else recomputing dS.
hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, int dtype, int act, int64_t grid, hipStream_t stream);

}  // namespace jfa

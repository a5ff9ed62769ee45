// Internal interfaces between the C-ABI layer (api.cpp) and the kernel
// translation units.  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace jfa {

// Tile geometry, shared by the launchers and the host-side sizing code.
constexpr int kFwdBM = 128;     // query rows per forward / dQ work item
constexpr int kFwdBN = 64;      // key rows per forward / dQ inner step
constexpr int kBwdBN = 64;      // key rows per dK/dV work item
constexpr int kBwdBM = 64;      // query rows per dK/dV cost block
constexpr int kDqBM = 64;       // query rows per dQ work item
constexpr int kDqBN = 64;       // key rows per dQ cost block
constexpr int kMaxBuckets = 1024;   // distinct tile costs the scheduler can sort
constexpr int kMaxHeads = 256;      // head index is packed into 8 bits

enum Pass { kPassQ = 0, kPassKV = 1, kPassDQ = 2 };

// Per-item record the attention kernels read with one load: the sequence's
// first query and key rows and lengths, and the item's head and tile.
// Records past the item count have lq = -1.
struct ItemMeta {
  int32_t qs, lq, ks, lk, head, tile, unused0, unused1;
};

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

hipError_t launch_sched(int pass, const int32_t* qo, const int32_t* ko, int32_t batch, int32_t heads,
                        int32_t causal, int32_t nbuckets, void* wl_base, const WorklistLayout& lay,
                        hipStream_t stream);
// The backward's two lists in one launch (two workgroups): dQ tiles and key tiles.
hipError_t launch_sched_pair(const int32_t* qo, const int32_t* ko, int32_t batch, int32_t heads, int32_t causal,
                             int32_t nb_dq, void* wl_dq, const WorklistLayout& lay_dq, int32_t nb_kv, void* wl_kv,
                             const WorklistLayout& lay_kv, hipStream_t stream);

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* qo;
  const int32_t* ko;
  const ItemMeta* meta;     // query-tile records
  void* out;
  float* lse;
  int32_t heads;
  int32_t total_q;
  int32_t causal;
  float scale;        // softmax / silu score scale
  float scale_log2;   // scale * log2(e)
};

hipError_t launch_fwd(const FwdArgs& a, int head_dim, int dtype, int act, int64_t grid, hipStream_t stream);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  const int32_t* qo;
  const int32_t* ko;
  const ItemMeta* meta_q;   // dQ-tile records (dQ pass)
  const ItemMeta* meta_kv;  // key-tile records (dK/dV pass)
  float* lse2;             // [heads, total_q] workspace: lse * log2(e) per row, and
  float* delta;            // [heads, total_q] delta per row; both written by the dQ pass
                           // (softmax), read by the dK/dV pass
  void* dq;
  void* dk;
  void* dv;
  int32_t heads;
  int32_t total_q;
  int32_t total_kv;
  int32_t causal;
  float scale;
  float scale_log2;
};

hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, int dtype, int act, int64_t grid, hipStream_t stream);
hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, int dtype, int act, int64_t grid, hipStream_t stream);

}  // namespace jfa

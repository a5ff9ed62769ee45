// C ABI of libjfa.so: argument validation, workspace carving and the launch
// sequence of the forward and backward passes.  See include/jfa.h for the
// contract.
#include "jfa.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <string>

#include "jfa_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(JFA_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Largest dS store the backward keeps in its workspace; beyond it the dQ
// pass recomputes dS instead (see jfa.h).
constexpr uint64_t kDsMaxBytes = uint64_t(16) << 30;

struct WsLayout {
  jfa::WorklistLayout wq{}, wkv{};
  jfa::WorklistLayout wq_fwd{}, wq_dqs{};   // backward: the 128- and 256-row query tiles of the dQ pass over stored dS
  size_t off_wq = 0, off_wkv = 0, off_stats = 0, off_ds = 0, bytes = 0;
  int64_t ds_rows = 0, ds_kb = 0;
  bool ds = false;   // the workspace holds the dS blocks
};

// Both: the offsets-check word at byte 0 (256 bytes reserved).  Forward:
// the query-tile list.  Backward: the dQ-tile list (in the same slot), the
// key-tile list, the per-row statistics and, when they fit the limit, the
// dS blocks.
constexpr size_t kStatusBytes = 256;
WsLayout ws_layout(int32_t batch, int32_t heads, int32_t total_q, int32_t total_kv, int32_t max_kv_len,
                   int32_t dtype, bool backward, bool with_ds = true) {
  WsLayout L;
  L.wq = jfa::worklist_layout(backward ? jfa::kPassDQ : jfa::kPassQ, batch, heads, total_q);
  L.off_wq = kStatusBytes;
  size_t off = L.off_wq + L.wq.bytes;
  if (backward) {   // the slot holds either query-tile list
    L.wq_fwd = jfa::worklist_layout(jfa::kPassQ, batch, heads, total_q);
    L.wq_dqs = jfa::worklist_layout(jfa::kPassDQS, batch, heads, total_q);
    off = std::max({off, L.off_wq + L.wq_fwd.bytes, L.off_wq + L.wq_dqs.bytes});
  }
  if (backward) {
    L.wkv = jfa::worklist_layout(jfa::kPassKV, batch, heads, total_kv);
    L.off_wkv = off;
    off += L.wkv.bytes;
    L.off_stats = off;
    off += align256(static_cast<size_t>(heads) * static_cast<size_t>(total_q) * 2 * sizeof(float));
    L.ds_rows = jfa::ds_block_rows(batch, total_q);
    L.ds_kb = jfa::ds_key_blocks(max_kv_len);
    const uint64_t block = uint64_t(jfa::kDsBlock) * jfa::kDsBlock * (dtype == JFA_DTYPE_FP32 ? 4 : 2);
    const uint64_t ds_bytes = uint64_t(heads) * uint64_t(L.ds_rows) * uint64_t(L.ds_kb) * block;
    if (with_ds && ds_bytes <= kDsMaxBytes) {
      L.ds = true;
      L.off_ds = off;
      off += align256(static_cast<size_t>(ds_bytes));
    }
  }
  L.bytes = off;
  return L;
}

// Process-wide path options (jfa_set_option); -1 = chosen by the library.
std::atomic<int32_t> g_options[JFA_OPT_COUNT] = {{-1}, {-1}, {-1}, {-1}};

int32_t option(int32_t which) { return g_options[which].load(std::memory_order_relaxed); }

// The work-list builder validates the offsets on the device first (see
// jfa_check_device_error): JFA_OPT_CHECK_OFFSETS = 1, or by default the
// environment variable JFA_CHECK_OFFSETS=1, read once.
bool check_offsets_enabled() {
  static const bool env = [] {
    const char* e = std::getenv("JFA_CHECK_OFFSETS");
    return e && e[0] == '1' && e[1] == 0;
  }();
  const int32_t o = option(JFA_OPT_CHECK_OFFSETS);
  return o < 0 ? env : o == 1;
}

jfa::OffsetCheck offset_check(void* ws, int32_t total_q, int32_t total_kv, int32_t max_q_len, int32_t max_kv_len) {
  return jfa::OffsetCheck{static_cast<int*>(ws), check_offsets_enabled() ? 1 : 0, total_q, total_kv, max_q_len,
                          max_kv_len};
}

// JFA_OPT_BWD_DS_STORE = 0 makes the backward recompute dS in the dQ pass
// even when the workspace holds the dS blocks.
bool ds_disabled() { return option(JFA_OPT_BWD_DS_STORE) == 0; }

// Whether the dK/dV pass writes the dQ of short sequences (at most 64
// queries and 1 .. 64 keys) itself.  By default only when every sequence is
// short (the maximum lengths say so): then the dQ pass has nothing left but
// the zero rows of sequences without keys.  In a batch that also holds long
// sequences, the long ones set the dQ pass's duration and the short ones
// fill its gaps at no cost, while fusing lengthens the dK/dV pass.
// JFA_OPT_BWD_SHORT_DQ = 0: never; 1: whenever the kernel can.
bool fuse_short_wanted(int32_t max_q_len, int32_t max_kv_len) {
  const int32_t o = option(JFA_OPT_BWD_SHORT_DQ);
  if (o >= 0) return o == 1;
  return max_q_len <= jfa::kBwdBN && max_kv_len <= jfa::kBwdBN;
}

// Records events[i] on the stream when the caller asked for stage events
// (a null entry skips that point).
hipError_t record(hipEvent_t* events, int i, hipStream_t stream) {
  if (!events || !events[i]) return hipSuccess;
  return hipEventRecord(events[i], stream);
}

// Finite test on the bit pattern (the library is built with NaN-free
// floating-point assumptions, which may fold std::isfinite).
bool finite_float(float x) {
  uint32_t u;
  std::memcpy(&u, &x, sizeof(u));
  return (u & 0x7f800000u) != 0x7f800000u;
}

// Smallest accepted score scale (see check_common).
constexpr float kMinScale = 1e-20f;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t buckets_for(int32_t max_len, int32_t block) { return (max_len + block - 1) / block + 1; }

// Checks shared by every entry point that takes sizes.
int check_sizes(int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q, int32_t total_kv,
                int32_t max_q_len, int32_t max_kv_len) {
  if (batch < 0) return fail(JFA_ERR_INVALID_ARGUMENT, "batch < 0");
  if (heads < 1) return fail(JFA_ERR_INVALID_ARGUMENT, "heads < 1");
  if (total_q < 0 || total_kv < 0) return fail(JFA_ERR_INVALID_ARGUMENT, "negative total length");
  if (max_q_len < 0 || max_kv_len < 0) return fail(JFA_ERR_INVALID_ARGUMENT, "negative max length");
  if (head_dim != 32 && head_dim != 64 && head_dim != 128)
    return fail(JFA_ERR_UNSUPPORTED, "head_dim must be 32, 64 or 128");
  if (heads > jfa::kMaxHeads) return fail(JFA_ERR_UNSUPPORTED, "heads > 256");
  const int64_t lim = int64_t(1) << 31;
  if (int64_t(total_q) * heads * head_dim >= lim || int64_t(total_kv) * heads * head_dim >= lim)
    return fail(JFA_ERR_INVALID_ARGUMENT, "tensor has 2^31 or more elements");
  return JFA_OK;
}

int check_common(const void* q, const void* k, const void* v, const int32_t* qo, const int32_t* ko,
                 int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q, int32_t total_kv,
                 int32_t max_q_len, int32_t max_kv_len, float scale, int32_t activation, int32_t causal,
                 int32_t dtype) {
  // value pointers may be NULL only when their tensor has no rows
  if (!qo || !ko) return fail(JFA_ERR_INVALID_ARGUMENT, "NULL offsets pointer");
  if ((total_q > 0 && !q) || (total_kv > 0 && (!k || !v))) return fail(JFA_ERR_INVALID_ARGUMENT, "NULL input pointer");
  if (!finite_float(scale)) return fail(JFA_ERR_INVALID_ARGUMENT, "scale is not finite");
  // The softmax kernels mask a score by subtracting kMaskShift = 1e30 before
  // scaling and take the row max of the raw scores: both need a positive
  // scale large enough that a masked weight, exp2(-1e30 * scale * log2 e),
  // is exactly 0 in fp32.  One rule for both activations.
  if (!(scale >= kMinScale)) return fail(JFA_ERR_INVALID_ARGUMENT, "scale below 1e-20 (it must be positive)");
  if (activation != JFA_ACT_SOFTMAX && activation != JFA_ACT_SILU)
    return fail(JFA_ERR_INVALID_ARGUMENT, "bad activation");
  if (causal != 0 && causal != 1) return fail(JFA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  if (dtype != JFA_DTYPE_BF16 && dtype != JFA_DTYPE_FP32) return fail(JFA_ERR_INVALID_ARGUMENT, "bad dtype");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(JFA_ERR_INVALID_ARGUMENT, "value pointer not 16-byte aligned");
  return check_sizes(batch, heads, head_dim, total_q, total_kv, max_q_len, max_kv_len);
}

}  // namespace

int jfa::report(int status, const std::string& msg) { return fail(status, msg); }

int jfa::forward_args_status(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                             const int32_t* kv_offsets, int32_t batch, int32_t heads, int32_t head_dim,
                             int32_t total_q, int32_t total_kv, int32_t max_q_len, int32_t max_kv_len, float scale,
                             int32_t activation, int32_t causal, int32_t dtype, const void* out, const float* lse) {
  int st = check_common(q, k, v, q_offsets, kv_offsets, batch, heads, head_dim, total_q, total_kv, max_q_len,
                        max_kv_len, scale, activation, causal, dtype);
  if (st != JFA_OK) return st;
  if (total_q > 0 && !out) return fail(JFA_ERR_INVALID_ARGUMENT, "NULL out");
  if (!aligned16(out)) return fail(JFA_ERR_INVALID_ARGUMENT, "out not 16-byte aligned");
  if (activation == JFA_ACT_SOFTMAX && total_q > 0 && !lse)
    return fail(JFA_ERR_INVALID_ARGUMENT, "NULL lse for softmax");
  if (buckets_for(max_kv_len, jfa::kFwdBN) > jfa::kMaxBuckets)
    return fail(JFA_ERR_UNSUPPORTED, "max_kv_len exceeds the scheduler's range");
  return JFA_OK;
}

extern "C" {

const char* jfa_status_string(int status) {
  switch (status) {
    case JFA_OK: return "JFA_OK";
    case JFA_ERR_INVALID_ARGUMENT: return "JFA_ERR_INVALID_ARGUMENT";
    case JFA_ERR_UNSUPPORTED: return "JFA_ERR_UNSUPPORTED";
    case JFA_ERR_WORKSPACE_TOO_SMALL: return "JFA_ERR_WORKSPACE_TOO_SMALL";
    case JFA_ERR_HIP: return "JFA_ERR_HIP";
  }
  return "unknown jfa status";
}

const char* jfa_last_error(void) { return g_last_error.c_str(); }

size_t jfa_workspace_size(int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q, int32_t total_kv,
                          int32_t max_kv_len, int32_t dtype, int32_t for_backward) {
  if (check_sizes(batch, heads, head_dim, total_q, total_kv, 0, max_kv_len) != JFA_OK) return 0;
  if (dtype != JFA_DTYPE_BF16 && dtype != JFA_DTYPE_FP32) return 0;
  if (for_backward < 0 || for_backward > 2) return 0;
  return ws_layout(batch, heads, total_q, total_kv, max_kv_len, dtype, for_backward != 0, for_backward != 2).bytes;
}

bool valid_pass(int32_t pass) {
  return pass == JFA_PASS_QUERY_TILES || pass == JFA_PASS_KEY_TILES || pass == JFA_PASS_DQ_TILES ||
         pass == JFA_PASS_DQ_STORED_TILES;
}

size_t jfa_worklist_bytes(int32_t pass, int32_t batch, int32_t heads, int32_t total_q, int32_t total_kv) {
  if (!valid_pass(pass)) return 0;
  if (check_sizes(batch, heads, 32, total_q, total_kv, 0, 0) != JFA_OK) return 0;
  return jfa::worklist_layout(pass, batch, heads, pass == JFA_PASS_KEY_TILES ? total_kv : total_q).bytes;
}

int jfa_tile_shape(int32_t pass, int32_t* tile_rows, int32_t* block_rows) {
  if (!tile_rows || !block_rows) return fail(JFA_ERR_INVALID_ARGUMENT, "NULL output pointer");
  if (pass == JFA_PASS_QUERY_TILES) {
    *tile_rows = jfa::kFwdBM;
    *block_rows = jfa::kFwdBN;
  } else if (pass == JFA_PASS_KEY_TILES) {
    *tile_rows = jfa::kBwdBN;
    *block_rows = jfa::kBwdBM;
  } else if (pass == JFA_PASS_DQ_TILES) {
    *tile_rows = jfa::kDqBM;
    *block_rows = jfa::kDqBN;
  } else if (pass == JFA_PASS_DQ_STORED_TILES) {
    *tile_rows = jfa::kDqDsBM;
    *block_rows = jfa::kDqBN;
  } else {
    return fail(JFA_ERR_INVALID_ARGUMENT, "bad pass");
  }
  return JFA_OK;
}

int jfa_build_worklist(int32_t pass, const int32_t* q_offsets, const int32_t* kv_offsets, int32_t batch,
                       int32_t heads, int32_t total_q, int32_t total_kv, int32_t max_q_len, int32_t max_kv_len,
                       int32_t causal, void* out, size_t out_bytes, hipStream_t stream) {
  if (!valid_pass(pass)) return fail(JFA_ERR_INVALID_ARGUMENT, "bad pass");
  if (!q_offsets || !kv_offsets) return fail(JFA_ERR_INVALID_ARGUMENT, "NULL offsets pointer");
  if (causal != 0 && causal != 1) return fail(JFA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  int st = check_sizes(batch, heads, 32, total_q, total_kv, max_q_len, max_kv_len);
  if (st != JFA_OK) return st;
  const int32_t nb = pass == JFA_PASS_QUERY_TILES ? buckets_for(max_kv_len, jfa::kFwdBN)
                     : pass == JFA_PASS_KEY_TILES   ? buckets_for(max_q_len, jfa::kBwdBM)
                                                    : buckets_for(max_kv_len, jfa::kDqBN);
  if (nb > jfa::kMaxBuckets) return fail(JFA_ERR_UNSUPPORTED, "maximum length exceeds the scheduler's range");
  const jfa::WorklistLayout lay =
      jfa::worklist_layout(pass, batch, heads, pass == JFA_PASS_KEY_TILES ? total_kv : total_q);
  if (batch == 0) return JFA_OK;
  if (!out) return fail(JFA_ERR_INVALID_ARGUMENT, "NULL output pointer");
  if (out_bytes < lay.bytes) return fail(JFA_ERR_WORKSPACE_TOO_SMALL, "worklist buffer too small");
  const jfa::OffsetCheck none{nullptr, 0, total_q, total_kv, max_q_len, max_kv_len};
  hipError_t e = jfa::launch_sched(pass, q_offsets, kv_offsets, batch, heads, causal, nb, out, lay, none, stream);
  if (e != hipSuccess) return hip_fail(e, "work-list builder launch");
  return JFA_OK;
}

// jfa_forward_profiled with BlockAttention's fused rotary embedding when
// rope.on (batches of short sequences, bf16, head_dim 64 or 128).
static int forward_impl(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                        const int32_t* kv_offsets, int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q,
                        int32_t total_kv, int32_t max_q_len, int32_t max_kv_len, float scale, int32_t activation,
                        int32_t causal, int32_t dtype, void* out, float* lse, void* workspace, size_t workspace_bytes,
                        hipStream_t stream, hipEvent_t* events, const jfa::RopeArgs& rope) {
  int st = jfa::forward_args_status(q, k, v, q_offsets, kv_offsets, batch, heads, head_dim, total_q, total_kv,
                                    max_q_len, max_kv_len, scale, activation, causal, dtype, out, lse);
  if (st != JFA_OK) return st;
  const int32_t nb = buckets_for(max_kv_len, jfa::kFwdBN);
  if (batch == 0 || total_q == 0) return JFA_OK;   // nothing to write
  const WsLayout L = ws_layout(batch, heads, total_q, total_kv, max_kv_len, dtype, false);
  if (!workspace || workspace_bytes < L.bytes) return fail(JFA_ERR_WORKSPACE_TOO_SMALL, "workspace too small");

  char* ws = static_cast<char*>(workspace);
  hipError_t e;
  // every sequence at most 64 queries and 64 keys: the two-wave variant
  // (JFA_OPT_FWD_SHORT = 0 keeps the four-wave kernel, for tests and
  // timing).  Its items all cost at most one key block, so without the
  // offsets check it takes one block per (sequence, head) and no work list
  // is built.
  const bool lengths_short = max_q_len <= jfa::kBwdBN && max_kv_len <= jfa::kFwdBN;
  if (rope.on && (!lengths_short || dtype != JFA_DTYPE_BF16 || (head_dim != 64 && head_dim != 128)))
    return fail(JFA_ERR_UNSUPPORTED, "the rotary embedding needs lengths <= 64, bf16 and head_dim 64 or 128");
  // the rotary embedding lives in the two-wave variant only
  const bool short_batch = lengths_short && (rope.on || option(JFA_OPT_FWD_SHORT) != 0);
  const bool direct = short_batch && !check_offsets_enabled() && (int64_t)batch * heads <= INT32_MAX;
  if ((e = record(events, 0, stream)) != hipSuccess) return hip_fail(e, "event record");
  if (!direct) {
    e = jfa::launch_sched(jfa::kPassQ, q_offsets, kv_offsets, batch, heads, causal, nb, ws + L.off_wq, L.wq,
                          offset_check(ws, total_q, total_kv, max_q_len, max_kv_len), stream);
    if (e != hipSuccess) return hip_fail(e, "work-list builder launch");
  }
  if ((e = record(events, 1, stream)) != hipSuccess) return hip_fail(e, "event record");
  jfa::FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.qo = q_offsets;
  a.ko = kv_offsets;
  a.meta = direct ? nullptr : reinterpret_cast<const jfa::ItemMeta*>(ws + L.off_wq + L.wq.meta_off);
  a.out = out;
  a.lse = lse;
  a.heads = heads;
  a.total_q = total_q;
  a.total_kv = total_kv;
  a.causal = causal;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.rope = rope;
  e = jfa::launch_fwd(a, head_dim, dtype, activation, direct ? (int64_t)batch * heads : L.wq.capacity, short_batch,
                      stream);
  if (e != hipSuccess) return hip_fail(e, "forward kernel launch");
  if ((e = record(events, 2, stream)) != hipSuccess) return hip_fail(e, "event record");
  return JFA_OK;
}

int jfa_forward_profiled(const void* q, const void* k, const void* v, const int32_t* q_offsets,
                         const int32_t* kv_offsets, int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q,
                         int32_t total_kv, int32_t max_q_len, int32_t max_kv_len, float scale, int32_t activation,
                         int32_t causal, int32_t dtype, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, hipStream_t stream, hipEvent_t* events) {
  return forward_impl(q, k, v, q_offsets, kv_offsets, batch, heads, head_dim, total_q, total_kv, max_q_len,
                      max_kv_len, scale, activation, causal, dtype, out, lse, workspace, workspace_bytes, stream,
                      events, jfa::RopeArgs{});
}

int jfa_forward(const void* q, const void* k, const void* v, const int32_t* q_offsets, const int32_t* kv_offsets,
                int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q, int32_t total_kv,
                int32_t max_q_len, int32_t max_kv_len, float scale, int32_t activation, int32_t causal,
                int32_t dtype, void* out, float* lse, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  return jfa_forward_profiled(q, k, v, q_offsets, kv_offsets, batch, heads, head_dim, total_q, total_kv, max_q_len,
                              max_kv_len, scale, activation, causal, dtype, out, lse, workspace, workspace_bytes,
                              stream, nullptr);
}

// jfa_backward_profiled with BlockAttention's fused rotary embedding when
// rope.on (every sequence short, bf16, head_dim 64 or 128: the dK/dV pass
// forms dQ itself).
static int backward_impl(const void* q, const void* k, const void* v, const void* out, const void* dout,
                         const float* lse, const int32_t* q_offsets, const int32_t* kv_offsets, int32_t batch,
                         int32_t heads, int32_t head_dim, int32_t total_q, int32_t total_kv, int32_t max_q_len,
                         int32_t max_kv_len, float scale, int32_t activation, int32_t causal, int32_t dtype, void* dq,
                         void* dk, void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream,
                         hipEvent_t* events, const jfa::RopeArgs& rope) {
  int st = check_common(q, k, v, q_offsets, kv_offsets, batch, heads, head_dim, total_q, total_kv, max_q_len,
                        max_kv_len, scale, activation, causal, dtype);
  if (st != JFA_OK) return st;
  if ((total_q > 0 && (!dout || !dq)) || (total_kv > 0 && (!dk || !dv)))
    return fail(JFA_ERR_INVALID_ARGUMENT, "NULL gradient pointer");
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(JFA_ERR_INVALID_ARGUMENT, "gradient pointer not 16-byte aligned");
  if (activation == JFA_ACT_SOFTMAX) {
    if (total_q > 0 && (!out || !lse)) return fail(JFA_ERR_INVALID_ARGUMENT, "NULL out or lse for softmax");
    if (!aligned16(out)) return fail(JFA_ERR_INVALID_ARGUMENT, "out not 16-byte aligned");
  }
  const int32_t nbq = buckets_for(max_kv_len, jfa::kDqBN);
  const int32_t nbk = buckets_for(max_q_len, jfa::kBwdBM);
  static_assert(jfa::kDqBN == jfa::kFwdBN, "every query-tile list counts 64-key blocks");
  if (nbq > jfa::kMaxBuckets || nbk > jfa::kMaxBuckets)
    return fail(JFA_ERR_UNSUPPORTED, "maximum length exceeds the scheduler's range");
  if (batch == 0 || (total_q == 0 && total_kv == 0)) return JFA_OK;   // nothing to write
  // a workspace without room for the dS store (the store is its last part)
  // runs the dQ pass that recomputes dS
  WsLayout L = ws_layout(batch, heads, total_q, total_kv, max_kv_len, dtype, true);
  if (workspace && workspace_bytes < L.bytes) L = ws_layout(batch, heads, total_q, total_kv, max_kv_len, dtype, true, false);
  if (!workspace || workspace_bytes < L.bytes) return fail(JFA_ERR_WORKSPACE_TOO_SMALL, "workspace too small");

  char* ws = static_cast<char*>(workspace);
  hipError_t e;
  jfa::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.dout = dout;
  a.lse = lse;
  a.qo = q_offsets;
  a.ko = kv_offsets;
  // the dQ pass over stored dS walks the forward's 128-row query tiles, the
  // recomputing one 64-row tiles
  const bool use_ds = L.ds && !ds_disabled();
  // 256-row items halve the K re-reads of the dQ pass over stored dS, but
  // its longest item doubles: they are used only when no sequence is much
  // longer than the average (max <= 4 x mean), where the longest items do
  // not set the pass's duration.
  const bool wide = max_q_len > 128 && (int64_t)max_q_len * batch <= 4 * ((int64_t)total_q + batch - 1);
  const int qpass = use_ds ? (wide ? jfa::kPassDQS : jfa::kPassQ) : jfa::kPassDQ;
  const jfa::WorklistLayout& lay_q = use_ds ? (wide ? L.wq_dqs : L.wq_fwd) : L.wq;
  a.dq_rows = wide ? jfa::kDqDsBM : 128;
  const bool lengths_short = max_q_len <= jfa::kBwdBN && max_kv_len <= jfa::kBwdBN;
  if (rope.on && (!lengths_short || !jfa::dkdv_fuses_short(dtype, head_dim)))
    return fail(JFA_ERR_UNSUPPORTED, "the rotary embedding needs lengths <= 64, bf16 and head_dim 64 or 128");
  // the rotary embedding lives in the fused short-sequence path only
  a.fuse_short =
      (rope.on || fuse_short_wanted(max_q_len, max_kv_len)) && jfa::dkdv_fuses_short(dtype, head_dim) ? 1 : 0;
  a.meta_q = reinterpret_cast<const jfa::ItemMeta*>(ws + L.off_wq + lay_q.meta_off);
  a.meta_kv = reinterpret_cast<const jfa::ItemMeta*>(ws + L.off_wkv + L.wkv.meta_off);
  a.lse2 = reinterpret_cast<float*>(ws + L.off_stats);
  a.delta = a.lse2 + static_cast<size_t>(heads) * static_cast<size_t>(total_q);
  if (use_ds) {
    a.ds = ws + L.off_ds;
    a.ds_head_blocks = L.ds_rows * L.ds_kb;
    a.ds_kb = static_cast<int32_t>(L.ds_kb);
  }
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.heads = heads;
  a.total_q = total_q;
  a.total_kv = total_kv;
  a.causal = causal;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.rope = rope;

  // per-row lse2 and delta, read by both gradient passes (softmax): formed
  // by the work-list launch's spare workgroups when it builds both lists,
  // else by a kernel of their own
  const bool stats = activation == JFA_ACT_SOFTMAX && total_q > 0;
  const jfa::StatsArgs sa{out, dout, lse, a.lse2, a.delta, heads, total_q};
  if ((e = record(events, 0, stream)) != hipSuccess) return hip_fail(e, "event record");
  const bool pair = total_q > 0 && total_kv > 0;
  const jfa::OffsetCheck chk = offset_check(ws, total_q, total_kv, max_q_len, max_kv_len);
  if (pair) {
    e = jfa::launch_sched_pair(qpass, q_offsets, kv_offsets, batch, heads, causal, nbq, ws + L.off_wq, lay_q, nbk,
                               ws + L.off_wkv, L.wkv, stats ? &sa : nullptr, dtype, head_dim, chk, stream);
  } else if (total_q > 0) {
    e = jfa::launch_sched(qpass, q_offsets, kv_offsets, batch, heads, causal, nbq, ws + L.off_wq, lay_q, chk, stream);
  } else {
    e = jfa::launch_sched(jfa::kPassKV, q_offsets, kv_offsets, batch, heads, causal, nbk, ws + L.off_wkv, L.wkv, chk,
                          stream);
  }
  if (e != hipSuccess) return hip_fail(e, "work-list builder launch");
  if ((e = record(events, 1, stream)) != hipSuccess) return hip_fail(e, "event record");
  if (stats && !pair) {
    e = jfa::launch_bwd_stats(sa, head_dim, dtype, stream);
    if (e != hipSuccess) return hip_fail(e, "row statistics kernel launch");
  }
  if ((e = record(events, 2, stream)) != hipSuccess) return hip_fail(e, "event record");
  // dK/dV first: it also stores the dS blocks the dQ pass reads
  if (total_kv > 0) {
    e = jfa::launch_bwd_dkdv(a, head_dim, dtype, activation, L.wkv.capacity, stream);
    if (e != hipSuccess) return hip_fail(e, "dK/dV kernel launch");
  }
  if ((e = record(events, 3, stream)) != hipSuccess) return hip_fail(e, "event record");
  if (total_q > 0) {
    // every sequence short (or without keys): the dK/dV pass wrote all dQ
    // rows that see a key, the rest are zeros
    if (a.fuse_short && max_q_len <= jfa::kBwdBN && max_kv_len <= jfa::kBwdBN)
      e = jfa::launch_bwd_dq_keyless(a, chk.status, batch, head_dim, dtype, stream);
    else
      e = jfa::launch_bwd_dq(a, head_dim, dtype, activation, lay_q.capacity, stream);
    if (e != hipSuccess) return hip_fail(e, "dQ kernel launch");
  }
  if ((e = record(events, 4, stream)) != hipSuccess) return hip_fail(e, "event record");
  return JFA_OK;
}

int jfa_backward_profiled(const void* q, const void* k, const void* v, const void* out, const void* dout,
                          const float* lse, const int32_t* q_offsets, const int32_t* kv_offsets, int32_t batch,
                          int32_t heads, int32_t head_dim, int32_t total_q, int32_t total_kv, int32_t max_q_len,
                          int32_t max_kv_len, float scale, int32_t activation, int32_t causal, int32_t dtype,
                          void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                          hipStream_t stream, hipEvent_t* events) {
  return backward_impl(q, k, v, out, dout, lse, q_offsets, kv_offsets, batch, heads, head_dim, total_q, total_kv,
                       max_q_len, max_kv_len, scale, activation, causal, dtype, dq, dk, dv, workspace, workspace_bytes,
                       stream, events, jfa::RopeArgs{});
}

int64_t jfa_block_offsets_count(int32_t batch, int32_t total, int32_t block) {
  if (batch < 0 || total < 0 || block < 1) return 0;
  return (int64_t)total / block + batch + 1;
}

int jfa_block_offsets(const int32_t* offsets, int32_t batch, int32_t total, int32_t block, int32_t* out,
                      int64_t out_len, hipStream_t stream) {
  if (!offsets || !out) return fail(JFA_ERR_INVALID_ARGUMENT, "NULL offsets pointer");
  if (batch < 0 || total < 0) return fail(JFA_ERR_INVALID_ARGUMENT, "negative batch or total");
  if (block < 1) return fail(JFA_ERR_INVALID_ARGUMENT, "block < 1");
  const int64_t need = jfa_block_offsets_count(batch, total, block);
  if (out_len < need) return fail(JFA_ERR_INVALID_ARGUMENT, "out has fewer than total / block + batch + 1 entries");
  if (need > INT32_MAX) return fail(JFA_ERR_UNSUPPORTED, "too many blocks");
  hipError_t e = jfa::launch_block_offsets(offsets, batch, total, block, out, (int32_t)need, stream);
  if (e != hipSuccess) return hip_fail(e, "block offsets kernel launch");
  return JFA_OK;
}

// BlockAttention's calls: the run offsets go to the start of the workspace
// (jfa_block_offsets), the jagged calls' workspace follows.
static size_t block_runs_bytes(int32_t batch, int32_t total, int32_t block) {
  return align256((size_t)jfa_block_offsets_count(batch, total, block) * sizeof(int32_t));
}

static int block_check(int32_t batch, int32_t total, int32_t max_len, int32_t block, float rope_base, int32_t dtype,
                       int32_t head_dim, const int32_t* offsets) {
  if (!offsets) return fail(JFA_ERR_INVALID_ARGUMENT, "NULL offsets pointer");
  if (batch < 0 || total < 0 || max_len < 0) return fail(JFA_ERR_INVALID_ARGUMENT, "negative batch, total or max_len");
  if (block < 1 || block > jfa::kBwdBN) return fail(JFA_ERR_INVALID_ARGUMENT, "block must be 1 .. 64");
  if (jfa_block_offsets_count(batch, total, block) > INT32_MAX) return fail(JFA_ERR_UNSUPPORTED, "too many blocks");
  if (!finite_float(rope_base) || (rope_base != 0.f && !(rope_base > 1.f)))
    return fail(JFA_ERR_INVALID_ARGUMENT, "rope_base must be 0 (none) or a finite base above 1");
  if (rope_base != 0.f && (dtype != JFA_DTYPE_BF16 || (head_dim != 64 && head_dim != 128)))
    return fail(JFA_ERR_UNSUPPORTED, "the rotary embedding needs bf16 and head_dim 64 or 128");
  return JFA_OK;
}

static jfa::RopeArgs rope_args(float rope_base, int32_t head_dim) {
  jfa::RopeArgs r{};
  if (rope_base != 0.f) {
    r.on = 1;
    r.k2 = (float)(-2.0 * std::log2((double)rope_base) / (double)head_dim);
  }
  return r;
}

size_t jfa_block_workspace_size(int32_t batch, int32_t heads, int32_t head_dim, int32_t total, int32_t block,
                                int32_t dtype, int32_t for_backward) {
  if (batch < 0 || total < 0 || block < 1 || block > jfa::kBwdBN || for_backward < 0 || for_backward > 1) return 0;
  const int64_t n = jfa_block_offsets_count(batch, total, block);
  if (n > INT32_MAX) return 0;
  // the backward over runs of at most 64 tokens forms dQ in its dK/dV pass
  // where it can and needs no dS store; elsewhere it recomputes dS
  const size_t inner = jfa_workspace_size((int32_t)(n - 1), heads, head_dim, total, total, block, dtype,
                                          for_backward ? 2 : 0);
  if (inner == 0) return 0;
  return block_runs_bytes(batch, total, block) + inner;
}

int jfa_block_forward(const void* q, const void* k, const void* v, const int32_t* offsets, int32_t batch,
                      int32_t heads, int32_t head_dim, int32_t total, int32_t max_len, int32_t block, float scale,
                      int32_t activation, int32_t causal, int32_t dtype, float rope_base, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events) {
  int st = block_check(batch, total, max_len, block, rope_base, dtype, head_dim, offsets);
  if (st != JFA_OK) return st;
  const int32_t m = std::min(block, max_len);
  const int64_t n = jfa_block_offsets_count(batch, total, block);
  // every argument the forward takes, checked before anything is enqueued
  st = jfa::forward_args_status(q, k, v, offsets, offsets, (int32_t)(n - 1), heads, head_dim, total, total, m, m,
                                scale, activation, causal, dtype, out, lse);
  if (st != JFA_OK) return st;
  if (batch == 0 || total == 0) return JFA_OK;
  const size_t need = jfa_block_workspace_size(batch, heads, head_dim, total, block, dtype, 0);
  if (!workspace || workspace_bytes < need) return fail(JFA_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  int32_t* runs = static_cast<int32_t*>(workspace);
  const size_t rb = block_runs_bytes(batch, total, block);
  hipError_t e = record(events, 0, stream);
  if (e != hipSuccess) return hip_fail(e, "event record");
  e = jfa::launch_block_offsets(offsets, batch, total, block, runs, (int32_t)n, stream);
  if (e != hipSuccess) return hip_fail(e, "block offsets kernel launch");
  hipEvent_t later[3] = {nullptr, events ? events[1] : nullptr, events ? events[2] : nullptr};
  return forward_impl(q, k, v, runs, runs, (int32_t)(n - 1), heads, head_dim, total, total, m, m, scale, activation,
                      causal, dtype, out, lse, static_cast<char*>(workspace) + rb, workspace_bytes - rb, stream,
                      later, rope_args(rope_base, head_dim));
}

int jfa_block_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                       const float* lse, const int32_t* offsets, int32_t batch, int32_t heads, int32_t head_dim,
                       int32_t total, int32_t max_len, int32_t block, float scale, int32_t activation, int32_t causal,
                       int32_t dtype, float rope_base, void* dq, void* dk, void* dv, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, hipEvent_t* events) {
  int st = block_check(batch, total, max_len, block, rope_base, dtype, head_dim, offsets);
  if (st != JFA_OK) return st;
  const int32_t m = std::min(block, max_len);
  const int64_t n = jfa_block_offsets_count(batch, total, block);
  st = check_common(q, k, v, offsets, offsets, (int32_t)(n - 1), heads, head_dim, total, total, m, m, scale,
                    activation, causal, dtype);
  if (st != JFA_OK) return st;
  if (batch == 0 || total == 0) return JFA_OK;
  const size_t need = jfa_block_workspace_size(batch, heads, head_dim, total, block, dtype, 1);
  if (!workspace || workspace_bytes < need) return fail(JFA_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  // the remaining pointer checks are the backward's own; the run offsets
  // are written only once it would proceed
  if (!dout || !dq || !dk || !dv || (activation == JFA_ACT_SOFTMAX && (!out || !lse)))
    return fail(JFA_ERR_INVALID_ARGUMENT, "NULL gradient, out or lse pointer");
  int32_t* runs = static_cast<int32_t*>(workspace);
  const size_t rb = block_runs_bytes(batch, total, block);
  hipError_t e = record(events, 0, stream);
  if (e != hipSuccess) return hip_fail(e, "event record");
  e = jfa::launch_block_offsets(offsets, batch, total, block, runs, (int32_t)n, stream);
  if (e != hipSuccess) return hip_fail(e, "block offsets kernel launch");
  hipEvent_t later[5] = {nullptr};
  for (int i = 1; i < 5 && events; ++i) later[i] = events[i];
  return backward_impl(q, k, v, out, dout, lse, runs, runs, (int32_t)(n - 1), heads, head_dim, total, total, m, m,
                       scale, activation, causal, dtype, dq, dk, dv, static_cast<char*>(workspace) + rb,
                       workspace_bytes - rb, stream, later, rope_args(rope_base, head_dim));
}

// Pooled multi-head attention: the workspace holds the per-sequence query
// offsets, the seeds repeated per sequence (and, backward, the per-sequence
// query gradients), then the jagged calls' workspace.
struct PooledLayout {
  size_t off_q = 0, off_dq = 0, off_part = 0, off_inner = 0, bytes = 0;
};

static PooledLayout pooled_layout(int32_t batch, int32_t n_seeds, int32_t heads, int32_t head_dim, int32_t dtype,
                                  bool backward) {
  PooledLayout L;
  const size_t rows = (size_t)batch * n_seeds * heads * head_dim * (dtype == JFA_DTYPE_FP32 ? 4 : 2);
  L.off_q = align256(((size_t)batch + 1) * sizeof(int32_t));
  L.off_dq = L.off_q + align256(rows);
  L.off_part = L.off_dq + (backward ? align256(rows) : 0);
  L.off_inner = L.off_part + (backward ? align256((size_t)jfa::kPooledChunks * n_seeds * heads * head_dim * 4) : 0);
  return L;
}

static int pooled_check(int32_t batch, int32_t n_seeds, int32_t heads, int32_t head_dim, const void* seeds,
                        int32_t activation) {
  if (n_seeds < 1 || n_seeds > 256) return fail(JFA_ERR_INVALID_ARGUMENT, "n_seeds must be 1 .. 256");
  if (batch < 0 || heads < 1) return fail(JFA_ERR_INVALID_ARGUMENT, "batch < 0 or heads < 1");
  if ((int64_t)batch * n_seeds > INT32_MAX || (int64_t)batch * n_seeds * heads * head_dim >= (int64_t(1) << 31))
    return fail(JFA_ERR_INVALID_ARGUMENT, "batch * n_seeds rows exceed the index range");
  if (!seeds) return fail(JFA_ERR_INVALID_ARGUMENT, "NULL seeds");
  if (!aligned16(seeds)) return fail(JFA_ERR_INVALID_ARGUMENT, "seeds not 16-byte aligned");
  (void)activation;
  return JFA_OK;
}

size_t jfa_pooled_workspace_size(int32_t batch, int32_t n_seeds, int32_t heads, int32_t head_dim, int32_t total_kv,
                                 int32_t max_kv_len, int32_t dtype, int32_t for_backward) {
  if (batch < 0 || n_seeds < 1 || n_seeds > 256 || for_backward < 0 || for_backward > 1) return 0;
  if ((int64_t)batch * n_seeds > INT32_MAX) return 0;
  const size_t inner = jfa_workspace_size(batch, heads, head_dim, batch * n_seeds, total_kv, max_kv_len, dtype,
                                          for_backward);
  if (inner == 0) return 0;
  return pooled_layout(batch, n_seeds, heads, head_dim, dtype, for_backward != 0).off_inner + inner;
}

int jfa_pooled_forward(const void* seeds, const void* k, const void* v, const int32_t* kv_offsets, int32_t batch,
                       int32_t n_seeds, int32_t heads, int32_t head_dim, int32_t total_kv, int32_t max_kv_len,
                       float scale, int32_t activation, int32_t dtype, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, hipStream_t stream, hipEvent_t* events) {
  int st = pooled_check(batch, n_seeds, heads, head_dim, seeds, activation);
  if (st != JFA_OK) return st;
  const int32_t total_q = batch * n_seeds;
  // every other argument as the forward checks it (kv_offsets standing in
  // for the query offsets, which the library writes)
  st = jfa::forward_args_status(seeds, k, v, kv_offsets, kv_offsets, batch, heads, head_dim, total_q, total_kv,
                                n_seeds, max_kv_len, scale, activation, 0, dtype, out, lse);
  if (st != JFA_OK) return st;
  if (batch == 0) return JFA_OK;
  const size_t need = jfa_pooled_workspace_size(batch, n_seeds, heads, head_dim, total_kv, max_kv_len, dtype, 0);
  if (!workspace || workspace_bytes < need) return fail(JFA_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  char* ws = static_cast<char*>(workspace);
  const PooledLayout L = pooled_layout(batch, n_seeds, heads, head_dim, dtype, false);
  const int64_t seed_bytes = (int64_t)n_seeds * heads * head_dim * (dtype == JFA_DTYPE_FP32 ? 4 : 2);
  int32_t* qo = reinterpret_cast<int32_t*>(ws);
  hipError_t e = record(events, 0, stream);
  if (e != hipSuccess) return hip_fail(e, "event record");
  e = jfa::launch_pooled_prep(seeds, seed_bytes, batch, n_seeds, ws + L.off_q, qo, stream);
  if (e != hipSuccess) return hip_fail(e, "pooled prep kernel launch");
  hipEvent_t later[3] = {nullptr, events ? events[1] : nullptr, events ? events[2] : nullptr};
  return forward_impl(ws + L.off_q, k, v, qo, kv_offsets, batch, heads, head_dim, total_q, total_kv, n_seeds,
                      max_kv_len, scale, activation, 0, dtype, out, lse, ws + L.off_inner,
                      workspace_bytes - L.off_inner, stream, later, jfa::RopeArgs{});
}

int jfa_pooled_backward(const void* seeds, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, const int32_t* kv_offsets, int32_t batch, int32_t n_seeds, int32_t heads,
                        int32_t head_dim, int32_t total_kv, int32_t max_kv_len, float scale, int32_t activation,
                        int32_t dtype, void* dseeds, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                        hipStream_t stream, hipEvent_t* events) {
  int st = pooled_check(batch, n_seeds, heads, head_dim, seeds, activation);
  if (st != JFA_OK) return st;
  const int32_t total_q = batch * n_seeds;
  st = check_common(seeds, k, v, kv_offsets, kv_offsets, batch, heads, head_dim, total_q, total_kv, n_seeds,
                    max_kv_len, scale, activation, 0, dtype);
  if (st != JFA_OK) return st;
  if (!dseeds || !aligned16(dseeds)) return fail(JFA_ERR_INVALID_ARGUMENT, "NULL or misaligned dseeds");
  if (total_q > 0 && (!dout || (activation == JFA_ACT_SOFTMAX && (!out || !lse))))
    return fail(JFA_ERR_INVALID_ARGUMENT, "NULL dout, out or lse");
  if (total_kv > 0 && (!dk || !dv)) return fail(JFA_ERR_INVALID_ARGUMENT, "NULL dk or dv");
  const size_t need = jfa_pooled_workspace_size(batch, n_seeds, heads, head_dim, total_kv, max_kv_len, dtype, 1);
  if (batch > 0 && (!workspace || workspace_bytes < need)) return fail(JFA_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  char* ws = static_cast<char*>(workspace);
  const PooledLayout L = pooled_layout(batch, n_seeds, heads, head_dim, dtype, true);
  const int64_t seed_elems = (int64_t)n_seeds * heads * head_dim;
  const int64_t seed_bytes = seed_elems * (dtype == JFA_DTYPE_FP32 ? 4 : 2);
  hipError_t e = record(events, 0, stream);
  if (e != hipSuccess) return hip_fail(e, "event record");
  if (batch > 0) {
    int32_t* qo = reinterpret_cast<int32_t*>(ws);
    e = jfa::launch_pooled_prep(seeds, seed_bytes, batch, n_seeds, ws + L.off_q, qo, stream);
    if (e != hipSuccess) return hip_fail(e, "pooled prep kernel launch");
    hipEvent_t later[5] = {nullptr};
    for (int i = 1; i < 4 && events; ++i) later[i] = events[i];
    st = backward_impl(ws + L.off_q, k, v, out, dout, lse, qo, kv_offsets, batch, heads, head_dim, total_q, total_kv,
                       n_seeds, max_kv_len, scale, activation, 0, dtype, ws + L.off_dq, dk, dv, ws + L.off_inner,
                       workspace_bytes - L.off_inner, stream, later, jfa::RopeArgs{});
    if (st != JFA_OK) return st;
  }
  // with no sequences the sum is over none: zeros (no workspace is read)
  e = jfa::launch_pooled_reduce(batch > 0 ? ws + L.off_dq : nullptr, seed_elems, batch, dtype,
                                batch > 0 ? reinterpret_cast<float*>(ws + L.off_part) : nullptr, dseeds, stream);
  if (e != hipSuccess) return hip_fail(e, "pooled reduce kernel launch");
  if ((e = record(events, 4, stream)) != hipSuccess) return hip_fail(e, "event record");
  return JFA_OK;
}

// ------------------------------------------------------------------ MXFP8

}  // extern "C"

namespace {

// An MX image: codes, then the E8M0 scale codes, each 256-byte aligned.
struct MxImageLayout {
  int64_t nbr = 0;
  size_t scales = 0, bytes = 0;
};
MxImageLayout mx_image_layout(int32_t batch, int32_t heads, int32_t head_dim, int32_t total) {
  MxImageLayout L;
  L.nbr = jfa::mx_block_rows(batch, total);
  const size_t rows = static_cast<size_t>(heads) * static_cast<size_t>(L.nbr) * 32;
  L.scales = align256(rows * static_cast<size_t>(head_dim));
  L.bytes = L.scales + align256(rows * static_cast<size_t>(head_dim / 32));
  return L;
}

int mx_check_sizes(int32_t batch, int32_t heads, int32_t head_dim, int32_t total) {
  int st = check_sizes(batch, heads, 64, total, 0, 0, 0);
  if (st != JFA_OK) return st;
  if (head_dim != 64 && head_dim != 128) return fail(JFA_ERR_UNSUPPORTED, "MXFP8 needs head_dim 64 or 128");
  if (int64_t(total) * heads * head_dim >= (int64_t(1) << 31))
    return fail(JFA_ERR_INVALID_ARGUMENT, "tensor has 2^31 or more elements");
  return JFA_OK;
}

struct MxWsLayout {
  jfa::WorklistLayout wq{};
  MxImageLayout iq{}, ik{};
  size_t off_wq = 0, off_q = 0, off_k = 0, off_v = 0, bytes = 0;
};
// the offsets-check word, the query-tile list, then the images of Q, K, V
MxWsLayout mx_ws_layout(int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q, int32_t total_kv) {
  MxWsLayout L;
  L.wq = jfa::worklist_layout(jfa::kPassQ, batch, heads, total_q);
  L.off_wq = kStatusBytes;
  L.iq = mx_image_layout(batch, heads, head_dim, total_q);
  L.ik = mx_image_layout(batch, heads, head_dim, total_kv);
  L.off_q = align256(L.off_wq + L.wq.bytes);
  L.off_k = L.off_q + L.iq.bytes;
  L.off_v = L.off_k + L.ik.bytes;
  L.bytes = L.off_v + L.ik.bytes;
  return L;
}

}  // namespace

extern "C" {

size_t jfa_mx_image_bytes(int32_t batch, int32_t heads, int32_t head_dim, int32_t total) {
  if (mx_check_sizes(batch, heads, head_dim, total) != JFA_OK) return 0;
  return mx_image_layout(batch, heads, head_dim, total).bytes;
}

int jfa_mx_quantize(const void* x, const int32_t* offsets, int32_t batch, int32_t heads, int32_t head_dim,
                    int32_t total, int32_t layout, void* image, size_t image_bytes, hipStream_t stream) {
  int st = mx_check_sizes(batch, heads, head_dim, total);
  if (st != JFA_OK) return st;
  if (layout != JFA_MX_ROWS && layout != JFA_MX_KEYS) return fail(JFA_ERR_INVALID_ARGUMENT, "bad MX layout");
  if (!offsets) return fail(JFA_ERR_INVALID_ARGUMENT, "NULL offsets pointer");
  if (total > 0 && !x) return fail(JFA_ERR_INVALID_ARGUMENT, "NULL input pointer");
  if (!aligned16(x)) return fail(JFA_ERR_INVALID_ARGUMENT, "input not 16-byte aligned");
  const MxImageLayout L = mx_image_layout(batch, heads, head_dim, total);
  if (!image || (reinterpret_cast<uintptr_t>(image) & 255u) != 0)
    return fail(JFA_ERR_INVALID_ARGUMENT, "NULL or not 256-byte aligned image");
  if (image_bytes < L.bytes) return fail(JFA_ERR_WORKSPACE_TOO_SMALL, "image buffer too small");
  if (batch == 0 || total == 0) return JFA_OK;
  jfa::MxQuantArgs a{};
  a.x[0] = x;
  a.off[0] = offsets;
  a.total[0] = total;
  a.nbr[0] = static_cast<int32_t>(L.nbr);
  a.keys[0] = layout == JFA_MX_KEYS ? 1 : 0;
  a.codes[0] = static_cast<uint8_t*>(image);
  a.scales[0] = static_cast<uint8_t*>(image) + L.scales;
  a.batch = batch;
  a.heads = heads;
  hipError_t e = jfa::launch_mx_quant(a, head_dim, 1, stream);
  if (e != hipSuccess) return hip_fail(e, "MX quantisation kernel launch");
  return JFA_OK;
}

size_t jfa_mx_workspace_size(int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q, int32_t total_kv,
                             int32_t with_images) {
  if (mx_check_sizes(batch, heads, head_dim, total_q) != JFA_OK) return 0;
  if (mx_check_sizes(batch, heads, head_dim, total_kv) != JFA_OK) return 0;
  if (with_images != 0 && with_images != 1) return 0;
  const MxWsLayout L = mx_ws_layout(batch, heads, head_dim, total_q, total_kv);
  return with_images ? L.bytes : L.off_q;
}

}  // extern "C"

namespace {

// The attention from MX images: the work list (events [0] before, [1]
// after) and the kernel ([2] after).  Arguments already checked.
int mx_attend_impl(const uint8_t* qimg, const uint8_t* kimg, const uint8_t* vimg, const int32_t* q_offsets,
                   const int32_t* kv_offsets, int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q,
                   int32_t total_kv, int32_t max_q_len, int32_t max_kv_len, float scale, int32_t causal, void* out,
                   float* lse, char* ws, hipStream_t stream, hipEvent_t e0, hipEvent_t e1, hipEvent_t e2) {
  const MxWsLayout L = mx_ws_layout(batch, heads, head_dim, total_q, total_kv);
  hipError_t e;
  if (e0 && (e = hipEventRecord(e0, stream)) != hipSuccess) return hip_fail(e, "event record");
  e = jfa::launch_sched(jfa::kPassQ, q_offsets, kv_offsets, batch, heads, causal, buckets_for(max_kv_len, jfa::kFwdBN),
                        ws + L.off_wq, L.wq, offset_check(ws, total_q, total_kv, max_q_len, max_kv_len), stream);
  if (e != hipSuccess) return hip_fail(e, "work-list builder launch");
  if (e1 && (e = hipEventRecord(e1, stream)) != hipSuccess) return hip_fail(e, "event record");
  jfa::MxFwdArgs a{};
  a.qx = qimg;
  a.qs = qimg + L.iq.scales;
  a.kx = kimg;
  a.ks = kimg + L.ik.scales;
  a.vx = vimg;
  a.vs = vimg + L.ik.scales;
  a.rq = 32 * L.iq.nbr;
  a.rk = 32 * L.ik.nbr;
  a.meta = reinterpret_cast<const jfa::ItemMeta*>(ws + L.off_wq + L.wq.meta_off);
  a.out = out;
  a.lse = lse;
  a.heads = heads;
  a.total_q = total_q;
  a.causal = causal;
  a.scale_log2 = scale * 1.4426950408889634f;
  // at most 64 queries per sequence: the two-wave kernel (JFA_OPT_FWD_SHORT =
  // 0 keeps the four-wave one; the outputs are equal bit for bit)
  const bool narrow = max_q_len <= 64 && option(JFA_OPT_FWD_SHORT) != 0;
  e = jfa::launch_mx_fwd(a, head_dim, narrow, L.wq.capacity, stream);
  if (e != hipSuccess) return hip_fail(e, "MXFP8 forward kernel launch");
  if (e2 && (e = hipEventRecord(e2, stream)) != hipSuccess) return hip_fail(e, "event record");
  return JFA_OK;
}

bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

}  // namespace

extern "C" {

int jfa_mx_forward(const void* q, const void* k, const void* v, const int32_t* q_offsets, const int32_t* kv_offsets,
                   int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q, int32_t total_kv,
                   int32_t max_q_len, int32_t max_kv_len, float scale, int32_t causal, void* out, float* lse,
                   void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events) {
  int st = jfa::forward_args_status(q, k, v, q_offsets, kv_offsets, batch, heads, head_dim, total_q, total_kv,
                                    max_q_len, max_kv_len, scale, JFA_ACT_SOFTMAX, causal, JFA_DTYPE_BF16, out, lse);
  if (st != JFA_OK) return st;
  if (head_dim != 64 && head_dim != 128) return fail(JFA_ERR_UNSUPPORTED, "MXFP8 needs head_dim 64 or 128");
  if (batch == 0 || total_q == 0) return JFA_OK;   // nothing to write
  const MxWsLayout L = mx_ws_layout(batch, heads, head_dim, total_q, total_kv);
  if (!workspace || workspace_bytes < L.bytes) return fail(JFA_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  if (!aligned256(workspace)) return fail(JFA_ERR_INVALID_ARGUMENT, "workspace not 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  hipError_t e;
  if ((e = record(events, 0, stream)) != hipSuccess) return hip_fail(e, "event record");
  jfa::MxQuantArgs qa{};
  const void* src[3] = {q, k, v};
  const int32_t* offs[3] = {q_offsets, kv_offsets, kv_offsets};
  const int32_t tot[3] = {total_q, total_kv, total_kv};
  const size_t base[3] = {L.off_q, L.off_k, L.off_v};
  const MxImageLayout* lay[3] = {&L.iq, &L.ik, &L.ik};
  for (int z = 0; z < 3; ++z) {
    qa.x[z] = src[z];
    qa.off[z] = offs[z];
    qa.total[z] = tot[z];
    qa.nbr[z] = tot[z] > 0 ? static_cast<int32_t>(lay[z]->nbr) : 0;
    qa.keys[z] = z == 2 ? 1 : 0;
    qa.codes[z] = reinterpret_cast<uint8_t*>(ws + base[z]);
    qa.scales[z] = reinterpret_cast<uint8_t*>(ws + base[z] + lay[z]->scales);
  }
  qa.batch = batch;
  qa.heads = heads;
  e = jfa::launch_mx_quant(qa, head_dim, 3, stream);
  if (e != hipSuccess) return hip_fail(e, "MX quantisation kernel launch");
  return mx_attend_impl(reinterpret_cast<const uint8_t*>(ws + L.off_q), reinterpret_cast<const uint8_t*>(ws + L.off_k),
                        reinterpret_cast<const uint8_t*>(ws + L.off_v), q_offsets, kv_offsets, batch, heads, head_dim,
                        total_q, total_kv, max_q_len, max_kv_len, scale, causal, out, lse, ws, stream,
                        events ? events[1] : nullptr, events ? events[2] : nullptr, events ? events[3] : nullptr);
}

int jfa_mx_attend(const void* q_image, const void* k_image, const void* v_image, const int32_t* q_offsets,
                  const int32_t* kv_offsets, int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q,
                  int32_t total_kv, int32_t max_q_len, int32_t max_kv_len, float scale, int32_t causal, void* out,
                  float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events) {
  // the images stand where the bf16 values would: same pointer and size rules
  int st = jfa::forward_args_status(q_image, k_image, v_image, q_offsets, kv_offsets, batch, heads, head_dim, total_q,
                                    total_kv, max_q_len, max_kv_len, scale, JFA_ACT_SOFTMAX, causal, JFA_DTYPE_BF16,
                                    out, lse);
  if (st != JFA_OK) return st;
  if (head_dim != 64 && head_dim != 128) return fail(JFA_ERR_UNSUPPORTED, "MXFP8 needs head_dim 64 or 128");
  if (!aligned256(q_image) || !aligned256(k_image) || !aligned256(v_image))
    return fail(JFA_ERR_INVALID_ARGUMENT, "image not 256-byte aligned");
  if (batch == 0 || total_q == 0) return JFA_OK;
  const MxWsLayout L = mx_ws_layout(batch, heads, head_dim, total_q, total_kv);
  if (!workspace || workspace_bytes < L.off_q) return fail(JFA_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  return mx_attend_impl(static_cast<const uint8_t*>(q_image), static_cast<const uint8_t*>(k_image),
                        static_cast<const uint8_t*>(v_image), q_offsets, kv_offsets, batch, heads, head_dim, total_q,
                        total_kv, max_q_len, max_kv_len, scale, causal, out, lse, static_cast<char*>(workspace), stream,
                        events ? events[0] : nullptr, events ? events[1] : nullptr, events ? events[2] : nullptr);
}

}  // extern "C"

namespace {

// MXFP8 backward workspace: the offsets-check word, the query-tile list
// (dQ pass), the key-tile list (dK/dV pass), the row statistics, then (when
// the library quantises) the seven images in the order of kMxBwdImages.
constexpr int kMxBwdImages = 7;   // Q rows, Q columns, K rows, K columns, V rows, dO rows, dO columns
struct MxBwdWsLayout {
  jfa::WorklistLayout wq{}, wkv{};
  MxImageLayout iq{}, ik{};
  size_t off_wq = 0, off_wkv = 0, off_stats = 0, off_img[kMxBwdImages] = {}, lists = 0, bytes = 0;
};
MxBwdWsLayout mx_bwd_ws_layout(int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q, int32_t total_kv) {
  MxBwdWsLayout L;
  L.wq = jfa::worklist_layout(jfa::kPassQ, batch, heads, total_q);
  L.wkv = jfa::worklist_layout(jfa::kPassKV, batch, heads, total_kv);
  L.off_wq = kStatusBytes;
  L.off_wkv = align256(L.off_wq + L.wq.bytes);
  L.off_stats = align256(L.off_wkv + L.wkv.bytes);
  L.lists = L.off_stats + align256(static_cast<size_t>(heads) * static_cast<size_t>(total_q) * 2 * sizeof(float));
  L.iq = mx_image_layout(batch, heads, head_dim, total_q);
  L.ik = mx_image_layout(batch, heads, head_dim, total_kv);
  size_t off = L.lists;
  for (int i = 0; i < kMxBwdImages; ++i) {
    L.off_img[i] = off;
    off += (i == 2 || i == 3 || i == 4) ? L.ik.bytes : L.iq.bytes;
  }
  L.bytes = off;
  return L;
}

int mx_bwd_check(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                 const int32_t* q_offsets, const int32_t* kv_offsets, int32_t batch, int32_t heads, int32_t head_dim,
                 int32_t total_q, int32_t total_kv, int32_t max_q_len, int32_t max_kv_len, float scale,
                 int32_t causal, void* dq, void* dk, void* dv) {
  int st = jfa::forward_args_status(q, k, v, q_offsets, kv_offsets, batch, heads, head_dim, total_q, total_kv,
                                    max_q_len, max_kv_len, scale, JFA_ACT_SOFTMAX, causal, JFA_DTYPE_BF16, out, lse);
  if (st != JFA_OK) return st;
  if (head_dim != 64 && head_dim != 128) return fail(JFA_ERR_UNSUPPORTED, "MXFP8 needs head_dim 64 or 128");
  if ((total_q > 0 && (!dout || !dq)) || (total_kv > 0 && (!dk || !dv)))
    return fail(JFA_ERR_INVALID_ARGUMENT, "NULL gradient pointer");
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return fail(JFA_ERR_INVALID_ARGUMENT, "gradient pointer not 16-byte aligned");
  if (buckets_for(max_q_len, jfa::kBwdBM) > jfa::kMaxBuckets)
    return fail(JFA_ERR_UNSUPPORTED, "max_q_len exceeds the scheduler's range");
  return JFA_OK;
}

// The backward from the seven images: work lists and row statistics
// (events [0] before, [1] after), dK/dV ([2] after), dQ ([3] after).
// Arguments already checked.
int mx_bwd_impl(const uint8_t* const* img, const void* out, const void* dout, const float* lse,
                const int32_t* q_offsets, const int32_t* kv_offsets, int32_t batch, int32_t heads, int32_t head_dim,
                int32_t total_q, int32_t total_kv, int32_t max_q_len, int32_t max_kv_len, float scale, int32_t causal,
                void* dq, void* dk, void* dv, char* ws, hipStream_t stream, hipEvent_t* ev) {
  const MxBwdWsLayout L = mx_bwd_ws_layout(batch, heads, head_dim, total_q, total_kv);
  auto rec = [&](int i) { return ev && ev[i] ? hipEventRecord(ev[i], stream) : hipSuccess; };
  hipError_t e;
  jfa::MxBwdArgs a{};
  auto image = [&](int i, const MxImageLayout& il) { return jfa::MxImage{img[i], img[i] + il.scales}; };
  a.q = image(0, L.iq);
  a.qc = image(1, L.iq);
  a.k = image(2, L.ik);
  a.kc = image(3, L.ik);
  a.v = image(4, L.ik);
  a.dout = image(5, L.iq);
  a.doc = image(6, L.iq);
  a.rq = 32 * L.iq.nbr;
  a.rk = 32 * L.ik.nbr;
  a.meta_q = reinterpret_cast<const jfa::ItemMeta*>(ws + L.off_wq + L.wq.meta_off);
  a.meta_kv = reinterpret_cast<const jfa::ItemMeta*>(ws + L.off_wkv + L.wkv.meta_off);
  float* lse2 = reinterpret_cast<float*>(ws + L.off_stats);
  float* delta = lse2 + static_cast<size_t>(heads) * static_cast<size_t>(total_q);
  a.lse2 = lse2;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.heads = heads;
  a.total_q = total_q;
  a.causal = causal;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  const jfa::StatsArgs sa{out, dout, lse, lse2, delta, heads, total_q};
  const jfa::OffsetCheck chk = offset_check(ws, total_q, total_kv, max_q_len, max_kv_len);
  const int32_t nbq = buckets_for(max_kv_len, jfa::kFwdBN), nbk = buckets_for(max_q_len, jfa::kBwdBM);
  if ((e = rec(0)) != hipSuccess) return hip_fail(e, "event record");
  const bool pair = total_q > 0 && total_kv > 0;
  if (pair)
    e = jfa::launch_sched_pair(jfa::kPassQ, q_offsets, kv_offsets, batch, heads, causal, nbq, ws + L.off_wq, L.wq, nbk,
                               ws + L.off_wkv, L.wkv, &sa, JFA_DTYPE_BF16, head_dim, chk, stream);
  else if (total_q > 0)
    e = jfa::launch_sched(jfa::kPassQ, q_offsets, kv_offsets, batch, heads, causal, nbq, ws + L.off_wq, L.wq, chk,
                          stream);
  else
    e = jfa::launch_sched(jfa::kPassKV, q_offsets, kv_offsets, batch, heads, causal, nbk, ws + L.off_wkv, L.wkv, chk,
                          stream);
  if (e != hipSuccess) return hip_fail(e, "work-list builder launch");
  if (!pair && total_q > 0 && (e = jfa::launch_bwd_stats(sa, head_dim, JFA_DTYPE_BF16, stream)) != hipSuccess)
    return hip_fail(e, "row statistics kernel launch");
  if ((e = rec(1)) != hipSuccess) return hip_fail(e, "event record");
  if (total_kv > 0 && (e = jfa::launch_mx_bwd_dkdv(a, head_dim, L.wkv.capacity, stream)) != hipSuccess)
    return hip_fail(e, "MXFP8 dK/dV kernel launch");
  if ((e = rec(2)) != hipSuccess) return hip_fail(e, "event record");
  if (total_q > 0 && (e = jfa::launch_mx_bwd_dq(a, head_dim, L.wq.capacity, stream)) != hipSuccess)
    return hip_fail(e, "MXFP8 dQ kernel launch");
  if ((e = rec(3)) != hipSuccess) return hip_fail(e, "event record");
  return JFA_OK;
}

}  // namespace

extern "C" {

size_t jfa_mx_backward_workspace_size(int32_t batch, int32_t heads, int32_t head_dim, int32_t total_q,
                                      int32_t total_kv, int32_t with_images) {
  if (mx_check_sizes(batch, heads, head_dim, total_q) != JFA_OK) return 0;
  if (mx_check_sizes(batch, heads, head_dim, total_kv) != JFA_OK) return 0;
  if (with_images != 0 && with_images != 1) return 0;
  const MxBwdWsLayout L = mx_bwd_ws_layout(batch, heads, head_dim, total_q, total_kv);
  return with_images ? L.bytes : L.lists;
}

int jfa_mx_backward(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                    const int32_t* q_offsets, const int32_t* kv_offsets, int32_t batch, int32_t heads,
                    int32_t head_dim, int32_t total_q, int32_t total_kv, int32_t max_q_len, int32_t max_kv_len,
                    float scale, int32_t causal, void* dq, void* dk, void* dv, void* workspace,
                    size_t workspace_bytes, hipStream_t stream, hipEvent_t* events) {
  int st = mx_bwd_check(q, k, v, out, dout, lse, q_offsets, kv_offsets, batch, heads, head_dim, total_q, total_kv,
                        max_q_len, max_kv_len, scale, causal, dq, dk, dv);
  if (st != JFA_OK) return st;
  if (batch == 0 || (total_q == 0 && total_kv == 0)) return JFA_OK;   // nothing to write
  if ((st = mx_check_sizes(batch, heads, head_dim, total_q)) != JFA_OK) return st;
  if ((st = mx_check_sizes(batch, heads, head_dim, total_kv)) != JFA_OK) return st;
  const MxBwdWsLayout L = mx_bwd_ws_layout(batch, heads, head_dim, total_q, total_kv);
  if (!workspace || workspace_bytes < L.bytes) return fail(JFA_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  if (!aligned256(workspace)) return fail(JFA_ERR_INVALID_ARGUMENT, "workspace not 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  hipError_t e;
  if (events && events[0] && (e = hipEventRecord(events[0], stream)) != hipSuccess) return hip_fail(e, "event record");
  // the seven images in one launch
  jfa::MxQuantArgs qa{};
  const void* src[kMxBwdImages] = {q, q, k, k, v, dout, dout};
  const bool qside[kMxBwdImages] = {true, true, false, false, false, true, true};
  const bool cols[kMxBwdImages] = {false, true, false, true, false, false, true};
  const uint8_t* img[kMxBwdImages];
  for (int z = 0; z < kMxBwdImages; ++z) {
    const MxImageLayout& il = qside[z] ? L.iq : L.ik;
    const int32_t tot = qside[z] ? total_q : total_kv;
    qa.x[z] = src[z];
    qa.off[z] = qside[z] ? q_offsets : kv_offsets;
    qa.total[z] = tot;
    qa.nbr[z] = tot > 0 ? static_cast<int32_t>(il.nbr) : 0;
    qa.keys[z] = cols[z] ? 1 : 0;
    qa.codes[z] = reinterpret_cast<uint8_t*>(ws + L.off_img[z]);
    qa.scales[z] = reinterpret_cast<uint8_t*>(ws + L.off_img[z] + il.scales);
    img[z] = qa.codes[z];
  }
  qa.batch = batch;
  qa.heads = heads;
  e = jfa::launch_mx_quant(qa, head_dim, kMxBwdImages, stream);
  if (e != hipSuccess) return hip_fail(e, "MX quantisation kernel launch");
  return mx_bwd_impl(img, out, dout, lse, q_offsets, kv_offsets, batch, heads, head_dim, total_q, total_kv, max_q_len,
                     max_kv_len, scale, causal, dq, dk, dv, ws, stream, events ? events + 1 : nullptr);
}

int jfa_mx_backward_images(const void* const* images, const void* out, const void* dout, const float* lse,
                           const int32_t* q_offsets, const int32_t* kv_offsets, int32_t batch, int32_t heads,
                           int32_t head_dim, int32_t total_q, int32_t total_kv, int32_t max_q_len,
                           int32_t max_kv_len, float scale, int32_t causal, void* dq, void* dk, void* dv,
                           void* workspace, size_t workspace_bytes, hipStream_t stream, hipEvent_t* events) {
  if (!images) return fail(JFA_ERR_INVALID_ARGUMENT, "NULL image array");
  const uint8_t* img[kMxBwdImages];
  for (int i = 0; i < kMxBwdImages; ++i) {
    const int32_t tot = (i == 2 || i == 3 || i == 4) ? total_kv : total_q;
    if (tot > 0 && !images[i]) return fail(JFA_ERR_INVALID_ARGUMENT, "NULL image");
    if (!aligned256(images[i])) return fail(JFA_ERR_INVALID_ARGUMENT, "image not 256-byte aligned");
    img[i] = static_cast<const uint8_t*>(images[i]);
  }
  // the images stand where the bf16 values would: same pointer and size rules
  int st = mx_bwd_check(images[0], images[2], images[4], out, dout, lse, q_offsets, kv_offsets, batch, heads,
                        head_dim, total_q, total_kv, max_q_len, max_kv_len, scale, causal, dq, dk, dv);
  if (st != JFA_OK) return st;
  if (batch == 0 || (total_q == 0 && total_kv == 0)) return JFA_OK;
  if ((st = mx_check_sizes(batch, heads, head_dim, total_q)) != JFA_OK) return st;
  if ((st = mx_check_sizes(batch, heads, head_dim, total_kv)) != JFA_OK) return st;
  const MxBwdWsLayout L = mx_bwd_ws_layout(batch, heads, head_dim, total_q, total_kv);
  if (!workspace || workspace_bytes < L.lists) return fail(JFA_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  return mx_bwd_impl(img, out, dout, lse, q_offsets, kv_offsets, batch, heads, head_dim, total_q, total_kv, max_q_len,
                     max_kv_len, scale, causal, dq, dk, dv, static_cast<char*>(workspace), stream, events);
}

int jfa_set_option(int32_t which, int32_t value) {
  if (which < 0 || which >= JFA_OPT_COUNT) return fail(JFA_ERR_INVALID_ARGUMENT, "unknown option");
  if (value < -1 || value > 1) return fail(JFA_ERR_INVALID_ARGUMENT, "option value must be -1, 0 or 1");
  g_options[which].store(value, std::memory_order_relaxed);
  return JFA_OK;
}

int32_t jfa_get_option(int32_t which) {
  if (which < 0 || which >= JFA_OPT_COUNT) return -2;
  return option(which);
}

int jfa_check_device_error(const void* workspace, hipStream_t stream) {
  if (!workspace) return fail(JFA_ERR_INVALID_ARGUMENT, "NULL workspace");
  int word = 0;
  hipError_t e = hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "reading the offsets-check word");
  if (word == 0) return JFA_OK;
  std::string msg = "offsets rejected on the device:";
  if (word & jfa::kOffsetsBadFirst) msg += " first offset not 0;";
  if (word & jfa::kOffsetsBadOrder) msg += " offsets decrease;";
  if (word & jfa::kOffsetsBadTotal) msg += " last offset differs from the total;";
  if (word & jfa::kOffsetsBadLength) msg += " a length exceeds the maximum;";
  return fail(JFA_ERR_INVALID_ARGUMENT, msg);
}

int jfa_backward(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                 const int32_t* q_offsets, const int32_t* kv_offsets, int32_t batch, int32_t heads,
                 int32_t head_dim, int32_t total_q, int32_t total_kv, int32_t max_q_len, int32_t max_kv_len,
                 float scale, int32_t activation, int32_t causal, int32_t dtype, void* dq, void* dk, void* dv,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return jfa_backward_profiled(q, k, v, out, dout, lse, q_offsets, kv_offsets, batch, heads, head_dim, total_q,
                               total_kv, max_q_len, max_kv_len, scale, activation, causal, dtype, dq, dk, dv,
                               workspace, workspace_bytes, stream, nullptr);
}

}  // extern "C"

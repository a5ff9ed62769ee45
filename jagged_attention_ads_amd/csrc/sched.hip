// Device-side work-list builder: the software tile scheduler for jagged
// tensors (piletech.kr/articles/112134, section 상세 정리 / Detailed notes,
// items on Jagged Flash Attention -- persistent-kernel scheduling -- and on
// GDPA -- software tile scheduling for jagged tensors).
//
// From the offsets alone it enumerates every work item (sequence b, head h,
// tile t), prices it by the number of inner blocks the attention kernel will
// visit for it, and writes the items longest first (cost descending), ties
// in (b, h, t) order, followed by one record per item for the attention
// kernels.
//
// A tile's cost is monotone in t within a sequence (query tiles: later rows
// see more keys; key tiles: later keys are seen by fewer rows), so the tiles
// of one sequence with a given cost form one run.  One workgroup per cost
// does its part alone: it counts the items of higher costs (they come
// first), scans the runs of its cost over the sequences in order (their
// place within the cost's range) and writes those items and their records.
// Every workgroup reads only the offsets; none waits for another.
#include <algorithm>
#include <cstdint>
#include <cstdlib>

#include "bwd_stats.hpp"
#include "jfa_common.hpp"
#include "jfa_internal.h"

namespace jfa {

constexpr int kListThreads = 1024;      // threads of a standalone list workgroup
constexpr int kPairThreads = 1024;      // threads of the backward's list + statistics launch
constexpr int kPairWorkgroups = 256;    // statistics workgroups of that launch, at most

// Exclusive scan of N values per thread over a workgroup of NT threads, one
// pair of barriers: ex[i] the thread's prefix of v[i], tot[i] the total.
// `tmp` holds N * NT / 64 ints.
template <int NT, int N>
__device__ void block_excl_scan_n(const int (&v)[N], int (&ex)[N], int (&tot)[N], int* tmp) {
  constexpr int W = NT / kWave;
  const int l = lane_id(), w = threadIdx.x / kWave;
  int x[N];
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = v[i];
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int y = __shfl_up(x[i], off, kWave);
      if (l >= off) x[i] += y;
    }
  }
  if (l == kWave - 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) tmp[i * W + w] = x[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    int before = 0, t = 0;
#pragma unroll
    for (int j = 0; j < W; ++j) {
      const int s = tmp[i * W + j];
      before += (j < w) ? s : 0;
      t += s;
    }
    ex[i] = before + x[i] - v[i];
    tot[i] = t;
  }
  __syncthreads();
}

template <int PASS>
struct TileRule {
  // Tiles split the query side (forward: kPassQ; dQ: kPassDQ recomputing dS,
  // kPassDQS over the stored dS) or the key side (dK/dV: kPassKV).
  static constexpr bool kQuery = PASS != kPassKV;
  static constexpr int kTile =
      PASS == kPassQ ? kFwdBM : PASS == kPassDQ ? kDqBM : PASS == kPassDQS ? kDqDsBM : kBwdBN;
  __device__ static int rows(int lq, int lk) { return kQuery ? lq : lk; }
  __device__ static int cost(int lq, int lk, int t, int causal) {
    if (PASS == kPassQ) return q_tile_kv_blocks(lq, lk, t, kFwdBM, kFwdBN, causal);
    if (PASS == kPassDQ) return q_tile_kv_blocks(lq, lk, t, kDqBM, kDqBN, causal);
    if (PASS == kPassDQS) return q_tile_kv_blocks(lq, lk, t, kDqDsBM, kDqBN, causal);
    return kv_tile_q_blocks(lq, lk, t, kBwdBM, kBwdBN, causal);
  }
  // One sequence's tiles for cost class c (costs at or above nb - 1 share
  // the class nb - 1): how many tiles it has, how many are in higher
  // classes, how many in c, and the first of those (a run, by monotonicity).
  __device__ static void run(int lq, int lk, int c, int nb, int causal, int& ntiles, int& n_gt, int& n_eq,
                             int& first) {
    ntiles = ceil_div(rows(lq, lk), kTile);
    auto cls = [&](int t) { return min(cost(lq, lk, t, causal), nb - 1); };
    // tiles in classes >= x: the last ones (query tiles) or the first ones (key tiles)
    auto count_ge = [&](int x) {
      int lo = 0, hi = ntiles;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (kQuery ? cls(mid) >= x : cls(mid) < x) hi = mid;
        else lo = mid + 1;
      }
      return kQuery ? ntiles - lo : lo;
    };
    const int ge = count_ge(c), gt = c + 1 < nb ? count_ge(c + 1) : 0;
    n_gt = gt;
    n_eq = ge - gt;
    first = kQuery ? ntiles - ge : gt;
  }
};

// One pass's work list: where it goes and how it is built.
struct SchedJob {
  int nbuckets;
  int slices;      // workgroups per cost class: each writes a share of the class's items
  int64_t capacity;
  int* count;
  int2* items;
  int* tile_start;
  ItemMeta* meta;
  OffsetCheck chk;
};

// The offsets' rules (kOffsetsBad* bits that fail), over the whole
// workgroup.  Reads q_offsets[0 .. B] and kv_offsets[0 .. B] only.
template <int NT>
__device__ int offsets_violations(const int* __restrict__ qo, const int* __restrict__ ko, int B,
                                  const OffsetCheck& c) {
  int bits = 0;
  for (int b = threadIdx.x; b <= B; b += NT) {
    const int q = qo[b], k = ko[b];
    if (b == 0 && (q != 0 || k != 0)) bits |= kOffsetsBadFirst;
    if (b == B && (q != c.total_q || k != c.total_kv)) bits |= kOffsetsBadTotal;
    if (b < B) {
      const int64_t lq = (int64_t)qo[b + 1] - q, lk = (int64_t)ko[b + 1] - k;
      if (lq < 0 || lk < 0) bits |= kOffsetsBadOrder;
      if (lq > c.max_q_len || lk > c.max_kv_len) bits |= kOffsetsBadLength;
    }
  }
  int all = 0;
  for (int bit = 1; bit <= kOffsetsBadLength; bit <<= 1)
    if (__syncthreads_or(bits & bit)) all |= bit;
  return all;
}

// Workgroup c of a list's nbuckets workgroups: the items of cost class
// c = nbuckets - 1 - (its index), so that the first workgroups take the
// longest items.  Workgroup 0 also writes the count and tile_start; every
// workgroup writes its share of the empty records past the count.
// Offsets staged in LDS (as many sequences as fit): the workgroup reads
// them twice.
constexpr int kStageSeqs = 8191;

template <int PASS, int NT>
__device__ void sched_class(const int* __restrict__ qo_g, const int* __restrict__ ko_g, int B, int H, int causal,
                            const SchedJob& job, int wg, int* tmp, int* stage, int* seq_pre, int* seq_n,
                            int* seq_first) {
  using R = TileRule<PASS>;
  const int nb = job.nbuckets, ns = job.slices, c = nb - 1 - wg / ns, slice = wg % ns, nwg = nb * ns;
  const int tid = threadIdx.x;
  const int64_t cap = job.capacity;
  const int* qo = qo_g;
  const int* ko = ko_g;
  if (B <= kStageSeqs) {
    // four loads in flight per thread before the LDS stores
    for (int base = 0; base <= B; base += 4 * NT) {
      int q[4], k[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = base + i * NT + tid;
        q[i] = b <= B ? qo_g[b] : 0;
        k[i] = b <= B ? ko_g[b] : 0;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = base + i * NT + tid;
        if (b <= B) {
          stage[b] = q[i];
          stage[kStageSeqs + 1 + b] = k[i];
        }
      }
    }
    __syncthreads();
    qo = stage;
    ko = stage + kStageSeqs + 1;
  }
  const int bad = job.chk.check ? offsets_violations<NT>(qo, ko, B, job.chk) : 0;
  if (wg == 0 && job.chk.status && tid == 0) *job.chk.status = bad;
  if (bad) {
    // nothing is enumerated from such offsets: an empty list whose records
    // send every attention workgroup home
    if (wg == 0) {
      if (tid == 0) *job.count = 0;
      for (int b = tid; b <= B; b += NT) job.tile_start[b] = 0;
    }
    for (int64_t p = (int64_t)wg * NT + tid; p < cap; p += (int64_t)nwg * NT) job.meta[p] = ItemMeta{0, -1, 0, 0, 0, 0, 0, 0};
    return;
  }
  // Every sequence's run of this class: its tiles, those in higher classes
  // (they come first), those in this class and the first of them.  With at
  // most NT sequences one pass and one fused scan do it all; beyond, a first
  // pass totals the higher classes and a second scans chunk by chunk.
  auto seq_run = [&](int b, int& ntiles, int& n_gt, int& n_eq, int& first) {
    ntiles = n_gt = n_eq = first = 0;
    if (b < B) R::run(qo[b + 1] - qo[b], ko[b + 1] - ko[b], c, nb, causal, ntiles, n_gt, n_eq, first);
  };
  int64_t start = 0, n_items = 0;
  int total_tiles = 0;
  if (B > NT) {
    int gt = 0, all = 0;
    for (int b = tid; b < B; b += NT) {
      int ntiles, n_gt, n_eq, first;
      seq_run(b, ntiles, n_gt, n_eq, first);
      gt += n_gt;
      all += ntiles;
    }
    const int v[2] = {gt, all};
    int ex[2], tot[2];
    block_excl_scan_n<NT, 2>(v, ex, tot, tmp);
    start = (int64_t)H * tot[0];
    total_tiles = tot[1];
    n_items = (int64_t)H * total_tiles;
  }
  // this class's runs in sequence order: sequence b's items are the H runs
  // of its class (head-major), after those of the earlier sequences
  int carry = 0, carry_tiles = 0;
  for (int base = 0; base < B; base += NT) {
    const int b = base + tid;
    int ntiles, n_gt, n_eq, first;
    seq_run(b, ntiles, n_gt, n_eq, first);
    const int v[3] = {n_eq, ntiles, n_gt};
    int ex[3], tot[3];
    block_excl_scan_n<NT, 3>(v, ex, tot, tmp);
    if (B <= NT) {   // the one chunk: its totals are the whole batch's
      start = (int64_t)H * tot[2];
      total_tiles = tot[1];
      n_items = (int64_t)H * total_tiles;
    }
    if (wg == 0 && b < B) job.tile_start[b] = carry_tiles + ex[1];
    // the chunk's items in list order, one per lane: item i of the chunk
    // belongs to the last sequence j whose first item is at or before it
    seq_pre[tid] = ex[0];
    seq_n[tid] = n_eq;
    seq_first[tid] = first;
    __syncthreads();
    const int n_chunk = H * tot[0];
    const int64_t p_chunk = start + (int64_t)H * carry;
    const int i_end = (int)((int64_t)n_chunk * (slice + 1) / ns);
    for (int i = (int)((int64_t)n_chunk * slice / ns) + tid; i < i_end; i += NT) {
      int lo = 0, hi = NT - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (H * seq_pre[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      const int n = seq_n[lo], local = i - H * seq_pre[lo], hh = local / n, t = seq_first[lo] + local - hh * n;
      const int bb = base + lo;
      const int64_t p = p_chunk + i;
      if (p >= 0 && p < cap) {   // true for valid offsets
        const int q0 = qo[bb], q1 = qo[bb + 1], k0 = ko[bb], k1 = ko[bb + 1];
        job.items[p] = make_int2(bb, (t << 8) | hh);
        u32x4* m = reinterpret_cast<u32x4*>(job.meta + p);
        m[0] = u32x4{(uint32_t)q0, (uint32_t)(q1 - q0), (uint32_t)k0, (uint32_t)(k1 - k0)};
        m[1] = u32x4{(uint32_t)hh, (uint32_t)t, (uint32_t)bb, 0u};
      }
    }
    __syncthreads();   // the next chunk rewrites seq_*
    carry += tot[0];
    carry_tiles += tot[1];
  }
  if (wg == 0 && tid == 0) {
    job.tile_start[B] = total_tiles;
    *job.count = (int)n_items;
  }
  // 3. records past the count: a share per workgroup
  for (int64_t p = std::max<int64_t>(n_items, 0) + (int64_t)wg * NT + tid; p < cap; p += (int64_t)nwg * NT)
    job.meta[p] = ItemMeta{0, -1, 0, 0, 0, 0, 0, 0};
}

template <int PASS>
__global__ __launch_bounds__(kListThreads) void sched_kernel(const int* __restrict__ qo, const int* __restrict__ ko,
                                                             int B, int H, int causal, SchedJob job) {
  __shared__ int tmp[3 * kListThreads / kWave];
  __shared__ int stage[2 * (kStageSeqs + 1)];
  __shared__ int seq[3 * kListThreads];
  sched_class<PASS, kListThreads>(qo, ko, B, H, causal, job, blockIdx.x, tmp, stage, seq, seq + kListThreads,
                                  seq + 2 * kListThreads);
}

// The backward's two lists in one launch: the first jdq.nbuckets workgroups
// build the query-tile list of the dQ pass (QPASS: 128- or 256-row tiles
// over the stored dS, or the 64-row tiles of the recomputing pass), the
// next jkv.nbuckets the key-tile list.  Further workgroups, when launched
// (softmax), form the row statistics of elements T and head dimension D
// meanwhile: with G of them, statistics workgroup i takes the units i,
// i + G, i + 2G, ... (unit u: row chunk u / heads of head u % heads), and
// has the next unit's reads in flight while it reduces the current one.
template <int QPASS, typename T, int D>
__global__ __launch_bounds__(kPairThreads) void sched_pair_kernel(const int* __restrict__ qo,
                                                                  const int* __restrict__ ko, int B, int H,
                                                                  int causal, SchedJob jdq, SchedJob jkv,
                                                                  StatsArgs sa) {
  __shared__ int tmp[3 * kPairThreads / kWave];
  __shared__ int stage[2 * (kStageSeqs + 1)];
  __shared__ int seq[3 * kPairThreads];
  const int nq = jdq.nbuckets * jdq.slices, nl = nq + jkv.nbuckets * jkv.slices;
  const int wg = (int)blockIdx.x;
  if (wg < nq) {
    sched_class<QPASS, kPairThreads>(qo, ko, B, H, causal, jdq, wg, tmp, stage, seq, seq + kPairThreads,
                                     seq + 2 * kPairThreads);
  } else if (wg < nl) {
    sched_class<kPassKV, kPairThreads>(qo, ko, B, H, causal, jkv, wg - nq, tmp, stage, seq,
                                       seq + kPairThreads, seq + 2 * kPairThreads);
  } else {
    using R = StatsRows<T, D, kPairThreads>;
    const int64_t units = (int64_t)((sa.total_q + R::C::ROWS - 1) / R::C::ROWS) * sa.heads;
    const int64_t g = (int64_t)gridDim.x - nl;
    const int tid = (int)threadIdx.x;
    int64_t u = (int64_t)wg - nl;
    R cur, nxt;
    cur.load(sa, (int)(u / sa.heads), (int)(u % sa.heads), tid);
    for (; u < units; u += g) {
      const int64_t v = u + g;
      if (v < units) nxt.load(sa, (int)(v / sa.heads), (int)(v % sa.heads), tid);
      cur.finish(sa, (int)(u / sa.heads), (int)(u % sa.heads), tid);
      cur = nxt;
    }
  }
}

WorklistLayout worklist_layout(int pass, int32_t batch, int32_t heads, int32_t total_rows) {
  const int64_t tile = pass == kPassQ ? kFwdBM : pass == kPassDQ ? kDqBM : pass == kPassDQS ? kDqDsBM : kBwdBN;
  // sum over sequences of ceil(L_b / tile) <= (total + batch * (tile - 1)) / tile
  const int64_t tiles = (static_cast<int64_t>(total_rows) + static_cast<int64_t>(batch) * (tile - 1)) / tile;
  WorklistLayout lay;
  lay.capacity = tiles * heads;
  lay.items_off = 16;
  lay.tile_start_off = lay.items_off + static_cast<size_t>(lay.capacity) * 8;
  lay.meta_off = (lay.tile_start_off + (static_cast<size_t>(batch) + 1) * 4 + 31) & ~static_cast<size_t>(31);
  lay.bytes = lay.meta_off + static_cast<size_t>(lay.capacity) * sizeof(ItemMeta);
  lay.bytes = (lay.bytes + 255) & ~static_cast<size_t>(255);
  return lay;
}

// Workgroups per cost class: enough that each writes at most about four
// items per thread even if one class held every item of the list (with few
// distinct costs one class can: pooled attention's key tiles all cost one).
static int sched_slices(const WorklistLayout& lay, int threads) {
  const int64_t per = 4 * (int64_t)threads;
  return (int)std::min<int64_t>(64, std::max<int64_t>(1, (lay.capacity + per - 1) / per));
}

// The job of one pass; `slices` workgroups per cost class.
static SchedJob make_job(int32_t nbuckets, int slices, void* wl_base, const WorklistLayout& lay,
                         const OffsetCheck& chk) {
  char* base = static_cast<char*>(wl_base);
  SchedJob j;
  j.chk = chk;
  j.nbuckets = nbuckets;
  j.slices = slices;
  j.capacity = lay.capacity;
  j.count = reinterpret_cast<int*>(base);
  j.items = reinterpret_cast<int2*>(base + lay.items_off);
  j.tile_start = reinterpret_cast<int*>(base + lay.tile_start_off);
  j.meta = reinterpret_cast<ItemMeta*>(base + lay.meta_off);
  return j;
}

hipError_t launch_sched(int pass, const int32_t* qo, const int32_t* ko, int32_t batch, int32_t heads,
                        int32_t causal, int32_t nbuckets, void* wl_base, const WorklistLayout& lay,
                        const OffsetCheck& chk, hipStream_t stream) {
  const SchedJob j = make_job(nbuckets, sched_slices(lay, kListThreads), wl_base, lay, chk);
  const dim3 grid((unsigned)(nbuckets * j.slices)), block(kListThreads);
  if (pass == kPassQ)
    hipLaunchKernelGGL(sched_kernel<kPassQ>, grid, block, 0, stream, qo, ko, batch, heads, causal, j);
  else if (pass == kPassDQS)
    hipLaunchKernelGGL(sched_kernel<kPassDQS>, grid, block, 0, stream, qo, ko, batch, heads, causal, j);
  else if (pass == kPassDQ)
    hipLaunchKernelGGL(sched_kernel<kPassDQ>, grid, block, 0, stream, qo, ko, batch, heads, causal, j);
  else
    hipLaunchKernelGGL(sched_kernel<kPassKV>, grid, block, 0, stream, qo, ko, batch, heads, causal, j);
  return hipGetLastError();
}

template <int QPASS, typename T, int D>
static hipError_t pair_launch(const int32_t* qo, const int32_t* ko, int32_t batch, int32_t heads, int32_t causal,
                              const SchedJob& jq, const SchedJob& jkv, const StatsArgs* stats, hipStream_t stream) {
  constexpr int rows = StatsCfg<T, D, kPairThreads>::ROWS;
  // the statistics take the rest of the launch's workgroups (each loops)
  const int nl = jq.nbuckets * jq.slices + jkv.nbuckets * jkv.slices;
  const int64_t units = stats ? (int64_t)((stats->total_q + rows - 1) / rows) * heads : 0;
  const int64_t extra = std::min<int64_t>(units, kPairWorkgroups);
  const StatsArgs sa = stats ? *stats : StatsArgs{};
  hipLaunchKernelGGL((sched_pair_kernel<QPASS, T, D>), dim3((unsigned)(nl + extra)), dim3(kPairThreads), 0, stream,
                     qo, ko, batch, heads, causal, jq, jkv, sa);
  return hipGetLastError();
}

template <int QPASS, typename T>
static hipError_t pair_launch_d(int head_dim, const int32_t* qo, const int32_t* ko, int32_t batch, int32_t heads,
                                int32_t causal, const SchedJob& jq, const SchedJob& jkv, const StatsArgs* stats,
                                hipStream_t stream) {
  switch (head_dim) {
    case 32: return pair_launch<QPASS, T, 32>(qo, ko, batch, heads, causal, jq, jkv, stats, stream);
    case 64: return pair_launch<QPASS, T, 64>(qo, ko, batch, heads, causal, jq, jkv, stats, stream);
    case 128: return pair_launch<QPASS, T, 128>(qo, ko, batch, heads, causal, jq, jkv, stats, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_sched_pair(int qpass, const int32_t* qo, const int32_t* ko, int32_t batch, int32_t heads,
                             int32_t causal, int32_t nb_dq, void* wl_dq, const WorklistLayout& lay_dq, int32_t nb_kv,
                             void* wl_kv, const WorklistLayout& lay_kv, const StatsArgs* stats, int dtype,
                             int head_dim, const OffsetCheck& chk, hipStream_t stream) {
  const SchedJob jq = make_job(nb_dq, sched_slices(lay_dq, kPairThreads), wl_dq, lay_dq, chk);
  const SchedJob jkv = make_job(nb_kv, sched_slices(lay_kv, kPairThreads), wl_kv, lay_kv, chk);
  if (qpass == kPassDQS)
    return dtype == 0 ? pair_launch_d<kPassDQS, __bf16>(head_dim, qo, ko, batch, heads, causal, jq, jkv, stats, stream)
                      : pair_launch_d<kPassDQS, float>(head_dim, qo, ko, batch, heads, causal, jq, jkv, stats, stream);
  if (qpass == kPassQ)
    return dtype == 0 ? pair_launch_d<kPassQ, __bf16>(head_dim, qo, ko, batch, heads, causal, jq, jkv, stats, stream)
                      : pair_launch_d<kPassQ, float>(head_dim, qo, ko, batch, heads, causal, jq, jkv, stats, stream);
  return dtype == 0 ? pair_launch_d<kPassDQ, __bf16>(head_dim, qo, ko, batch, heads, causal, jq, jkv, stats, stream)
                    : pair_launch_d<kPassDQ, float>(head_dim, qo, ko, batch, heads, causal, jq, jkv, stats, stream);
}

}  // namespace jfa

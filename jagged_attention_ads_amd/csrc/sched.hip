// Device-side work-list builder: the software tile scheduler for jagged
// tensors (piletech.kr/articles/112134, section 상세 정리 / Detailed notes,
// items on Jagged Flash Attention -- persistent-kernel scheduling -- and on
// GDPA -- software tile scheduling for jagged tensors).
//
// From the offsets alone it enumerates every work item (sequence b, head h,
// tile t), prices it by the number of inner blocks the attention kernel will
// visit for it, and writes the items longest first (cost descending), ties
// in (b, h, t) order -- a stable counting sort by cost -- followed by one
// record per item for the attention kernels.  One workgroup of 1024 threads
// does it all on the device, so the caller's stream never waits for the
// host.  When its working set fits in LDS (the common case: 160 KB on
// gfx950) it keeps everything there; otherwise a slower body works from
// global memory.
#include <algorithm>
#include <cstdint>
#include <cstdlib>

#include "bwd_stats.hpp"
#include "jfa_common.hpp"
#include "jfa_internal.h"

namespace jfa {

constexpr int kSchedThreads = 1024;
constexpr int kStatsWorkgroups = 254;   // 256 CUs less the two list builders
constexpr int kSchedWaves = kSchedThreads / kWave;

// Exclusive block scan of one value per thread.  `tmp` holds kSchedWaves ints.
__device__ int block_excl_scan(int v, int* tmp, int& total) {
  const int l = lane_id(), w = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int y = __shfl_up(x, off, kWave);
    if (l >= off) x += y;
  }
  if (l == kWave - 1) tmp[w] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kSchedWaves; ++i) {
    int s = tmp[i];
    before += (i < w) ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + x - v;
}

// Last sequence b in [0, B) with tile_start[b] <= u.
__device__ int find_seq(const int* ts, int B, int u) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (ts[mid] <= u) lo = mid; else hi = mid;
  }
  return lo;
}

// LDS bytes of the cost-bucket arrays (both bodies).
__host__ __device__ constexpr size_t sched_lds_fixed(int nbuckets) {
  return (((size_t)nbuckets * (3 * 4 + 2 + 2 * kSchedWaves) + 32 * 4) + 15) & ~(size_t)15;
}
// LDS bytes of the all-LDS body beyond them: tile starts and q/kv offsets
// per sequence, a two-word record per tile (sequence << 10 | cost bucket,
// index in its run of equal-cost tiles | run length << 16) and the item list
// as (tile | head << 16) words.  Tile and head counts below 2^16 keep every
// field in range.
__host__ __device__ constexpr size_t sched_lds_all(int batch, int64_t max_tiles, int64_t capacity) {
  return (((size_t)3 * batch + 3) * 4 + 7) / 8 * 8 + (size_t)max_tiles * 8 + (size_t)capacity * 4;
}
constexpr int kTileInfoBits = 10;   // cost bucket bits: nbuckets <= 1024
constexpr int kMaxTileInfoBatch = 1 << (32 - kTileInfoBits);
constexpr size_t kSchedMinLds = 64 * 1024;   // budget when the device does not report one

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
  // Costs are monotone in t within a sequence: non-decreasing for query
  // tiles (later rows see more keys), non-increasing for key tiles (later
  // keys are seen by fewer rows).  before_or_eq(x, c): a tile of cost x may
  // come before (or is in) the run of cost c; after_or_eq: after or in it.
  __device__ static bool before_or_eq(int x, int c) { return kQuery ? x <= c : x >= c; }
  __device__ static bool after_or_eq(int x, int c) { return kQuery ? x >= c : x <= c; }
  // The run [first, first + len) of tiles of one sequence (ntiles tiles)
  // whose bucketed cost equals c, the cost of tile t.
  __device__ static void run_of(int lq, int lk, int t, int ntiles, int c, int nbuckets, int causal, int& first,
                                int& len) {
    int lo = 0, hi = t;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (after_or_eq(min(cost(lq, lk, mid, causal), nbuckets - 1), c)) hi = mid; else lo = mid + 1;
    }
    first = lo;
    lo = t;
    hi = ntiles - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (before_or_eq(min(cost(lq, lk, mid, causal), nbuckets - 1), c)) lo = mid; else hi = mid - 1;
    }
    len = lo - first + 1;
  }
};

// One pass's work list: where it goes and how it is built.
struct SchedJob {
  int nbuckets;
  int in_lds;      // the all-LDS body (else the global-memory one)
  int max_tiles;   // tile bound: capacity / heads
  int64_t capacity;
  int* count;
  int2* items;
  int* tile_start;
  ItemMeta* meta;
  OffsetCheck chk;
};

// Cost-bucket arrays in LDS, shared by both bodies.
struct Buckets {
  int* hist;                  // tiles per cost
  int* start;                 // first item slot of each cost
  int* carry;                 // tiles of each cost in earlier chunks
  int* tmp;                   // block-scan scratch
  unsigned short* chunk_tot;  // tiles of each cost in this chunk
  unsigned short* wave_cnt;   // [kSchedWaves][nbuckets]: per wave, then exclusive prefix
  __device__ Buckets(char* smem, int nbuckets) {
    hist = reinterpret_cast<int*>(smem);
    start = hist + nbuckets;
    carry = start + nbuckets;
    tmp = carry + nbuckets;
    chunk_tot = reinterpret_cast<unsigned short*>(tmp + 32);
    wave_cnt = chunk_tot + nbuckets;
  }
};

// Step 3: first item slot of each cost bucket, largest cost first.
__device__ void bucket_starts(const Buckets& k, int nbuckets, int H) {
  int run = 0;
  for (int base = 0; base < nbuckets; base += kSchedThreads) {
    const int o = base + threadIdx.x;
    const int c = nbuckets - 1 - o;
    const int n = (o < nbuckets) ? k.hist[c] : 0;
    int tot;
    const int ex = block_excl_scan(n, k.tmp, tot);
    if (o < nbuckets) k.start[c] = H * (run + ex);
    run += tot;
  }
  __syncthreads();
}

// Step 4's rank of a chunk's tile (cost c, or valid == false) among the
// chunk's tiles of equal cost before it.  In the wave: its peers are the
// live lanes that agree with it on every bit of the cost (one ballot per
// bit), and the first lane of each cost writes the wave's count of it.
// Across waves: an exclusive prefix of those counts per cost.  Returns the
// rank inside the chunk; the caller adds carry[c] and, after a barrier,
// folds chunk_tot into carry.
__device__ int chunk_rank(const Buckets& k, int nbuckets, bool valid, int c) {
  const int tid = threadIdx.x, l = lane_id(), w = tid / kWave;
  for (int i = tid; i < kSchedWaves * nbuckets; i += kSchedThreads) k.wave_cnt[i] = 0;
  __syncthreads();
  unsigned long long same = __ballot(valid);
  for (int bit = 0; (1 << bit) < nbuckets; ++bit) {
    const unsigned long long m = __ballot((c >> bit) & 1);
    same &= ((c >> bit) & 1) ? m : ~m;
  }
  const int local = __popcll(same & ((1ull << l) - 1ull));
  if (valid && local == 0) k.wave_cnt[w * nbuckets + c] = (unsigned short)__popcll(same);
  __syncthreads();
  for (int cc = tid; cc < nbuckets; cc += kSchedThreads) {
    int r = 0;
    for (int ww = 0; ww < kSchedWaves; ++ww) {
      const int x = k.wave_cnt[ww * nbuckets + cc];
      k.wave_cnt[ww * nbuckets + cc] = (unsigned short)r;
      r += x;
    }
    k.chunk_tot[cc] = (unsigned short)r;
  }
  __syncthreads();
  return valid ? k.wave_cnt[w * nbuckets + c] + local : 0;
}

// First item slot of a tile: items of bucket c are ordered (b, h, t), so
// all earlier sequences' tiles of this cost (rank - k of them) times H come
// first, then the H runs of length len; head hh's item is p0 + hh * len.
__device__ __forceinline__ int item_slot(const Buckets& k, int c, int rank, int k_in_run, int H) {
  return k.start[c] + H * (rank - k_in_run) + k_in_run;
}

// The body for working sets that fit in LDS.  Everything it reads after
// step 1 is in LDS, through pointers the compiler sees to be LDS.
template <int PASS>
__device__ void sched_body_lds(const int* __restrict__ qo, const int* __restrict__ ko, int B, int H, int causal,
                               const SchedJob& job, char* smem) {
  using R = TileRule<PASS>;
  const int nbuckets = job.nbuckets, capacity = (int)job.capacity;
  const Buckets k(smem, nbuckets);
  int* ts = reinterpret_cast<int*>(smem + sched_lds_fixed(nbuckets));   // [B + 1]
  int* qof = ts + (B + 1);                                              // [B + 1]
  int* kof = qof + (B + 1);                                             // [B + 1]
  uint2* tile_info = reinterpret_cast<uint2*>(smem + sched_lds_fixed(nbuckets) + (((size_t)3 * B + 3) * 4 + 7) / 8 * 8);
  unsigned* item_lds = reinterpret_cast<unsigned*>(tile_info + job.max_tiles);
  int* owner = reinterpret_cast<int*>(item_lds);   // step 2's tile -> sequence map (capacity >= tiles)
  const int tid = threadIdx.x;

  // 1. sequence offsets into LDS; tiles per sequence -> exclusive prefix
  int run = 0;
  for (int base = 0; base < B; base += kSchedThreads) {
    const int b = base + tid;
    int n = 0;
    if (b < B) {
      const int q0 = qo[b], q1 = qo[b + 1], k0 = ko[b], k1 = ko[b + 1];
      n = ceil_div(R::rows(q1 - q0, k1 - k0), R::kTile);
      qof[b] = q0;
      kof[b] = k0;
      if (b == B - 1) {
        qof[B] = q1;
        kof[B] = k1;
      }
    }
    int tot;
    const int ex = block_excl_scan(n, k.tmp, tot);
    if (b < B) {
      ts[b] = run + ex;
      job.tile_start[b] = run + ex;
    }
    run += tot;
  }
  const int total_tiles = run;
  if (tid == 0) {
    ts[B] = total_tiles;
    job.tile_start[B] = total_tiles;
  }
  for (int c = tid; c < nbuckets; c += kSchedThreads) {
    k.hist[c] = 0;
    k.carry[c] = 0;
  }
  __syncthreads();

  // 2. the sequence of every tile (a thread per sequence fills its tiles),
  // then per tile its cost, its run of equal-cost tiles and the histogram
  for (int b = tid; b < B; b += kSchedThreads)
    for (int u = ts[b]; u < ts[b + 1]; ++u) owner[u] = b;
  __syncthreads();
  for (int u = tid; u < total_tiles; u += kSchedThreads) {
    const int b = owner[u];
    const int t = u - ts[b], ntiles = ts[b + 1] - ts[b];
    const int lq = qof[b + 1] - qof[b], lk = kof[b + 1] - kof[b];
    const int c = min(R::cost(lq, lk, t, causal), nbuckets - 1);
    int first, len;
    R::run_of(lq, lk, t, ntiles, c, nbuckets, causal, first, len);
    tile_info[u] = make_uint2(((unsigned)b << kTileInfoBits) | (unsigned)c, (unsigned)(t - first) | ((unsigned)len << 16));
    atomicAdd(&k.hist[c], 1);
  }
  __syncthreads();

  // 3. bucket starts
  bucket_starts(k, nbuckets, H);

  // 4. stable rank of every tile among the tiles of equal cost; its H items
  // go to the list in LDS (this overwrites step 2's owner map)
  for (int base = 0; base < total_tiles; base += kSchedThreads) {
    const int u = base + tid;
    const bool valid = u < total_tiles;
    int c = 0, kr = 0, len = 0;
    if (valid) {
      const uint2 info = tile_info[u];
      c = (int)(info.x & ((1u << kTileInfoBits) - 1));
      kr = (int)(info.y & 0xffff);
      len = (int)(info.y >> 16);
    }
    const int r = chunk_rank(k, nbuckets, valid, c);
    if (valid) {
      const int p0 = item_slot(k, c, k.carry[c] + r, kr, H);
      for (int hh = 0; hh < H; ++hh) item_lds[p0 + hh * len] = (unsigned)u | ((unsigned)hh << 16);
    }
    __syncthreads();
    for (int cc = tid; cc < nbuckets; cc += kSchedThreads) k.carry[cc] += k.chunk_tot[cc];
    __syncthreads();
  }
  const int n_items = H * total_tiles;
  if (tid == 0) *job.count = n_items;

  // 5. items and records in list order; records past the count (lq = -1)
  // tell the attention kernels' surplus workgroups to exit
  for (int p = tid; p < capacity; p += kSchedThreads) {
    ItemMeta m{0, -1, 0, 0, 0, 0, 0, 0};
    if (p < n_items) {
      const unsigned w = item_lds[p];
      const int u = (int)(w & 0xffff), hh = (int)(w >> 16);
      const int b = (int)(tile_info[u].x >> kTileInfoBits), t = u - ts[b];
      job.items[p] = make_int2(b, (t << 8) | hh);
      m = ItemMeta{qof[b], qof[b + 1] - qof[b], kof[b], kof[b + 1] - kof[b], hh, t, b, 0};
    }
    job.meta[p] = m;
  }
}

// The body for working sets beyond the LDS: per-sequence arrays are read
// from global memory, tiles find their sequence by binary search, and the
// items are scattered to the global list and read back for the records.
template <int PASS>
__device__ void sched_body_global(const int* __restrict__ qo, const int* __restrict__ ko, int B, int H, int causal,
                                  const SchedJob& job, char* smem) {
  using R = TileRule<PASS>;
  const int nbuckets = job.nbuckets;
  const int64_t capacity = job.capacity;
  const Buckets k(smem, nbuckets);
  int* const ts = job.tile_start;
  int2* const items = job.items;
  const int tid = threadIdx.x;
  auto lengths = [&](int b, int& lq, int& lk) {
    lq = qo[b + 1] - qo[b];
    lk = ko[b + 1] - ko[b];
  };

  // 1. tiles per sequence -> exclusive prefix tile_start[b]
  int run = 0;
  for (int base = 0; base < B; base += kSchedThreads) {
    const int b = base + tid;
    int n = 0;
    if (b < B) {
      int lq, lk;
      lengths(b, lq, lk);
      n = ceil_div(R::rows(lq, lk), R::kTile);
    }
    int tot;
    const int ex = block_excl_scan(n, k.tmp, tot);
    if (b < B) ts[b] = run + ex;
    run += tot;
  }
  const int total_tiles = run;
  if (tid == 0) ts[B] = total_tiles;
  for (int c = tid; c < nbuckets; c += kSchedThreads) {
    k.hist[c] = 0;
    k.carry[c] = 0;
  }
  __syncthreads();

  // 2. histogram of tile costs
  for (int u = tid; u < total_tiles; u += kSchedThreads) {
    const int b = find_seq(ts, B, u);
    int lq, lk;
    lengths(b, lq, lk);
    atomicAdd(&k.hist[min(R::cost(lq, lk, u - ts[b], causal), nbuckets - 1)], 1);
  }
  __syncthreads();

  // 3. bucket starts
  bucket_starts(k, nbuckets, H);

  // 4. stable rank of each tile among the tiles of equal cost, then its H items
  for (int base = 0; base < total_tiles; base += kSchedThreads) {
    const int u = base + tid;
    const bool valid = u < total_tiles;
    int b = 0, t = 0, c = 0, lq = 0, lk = 0;
    if (valid) {
      b = find_seq(ts, B, u);
      t = u - ts[b];
      lengths(b, lq, lk);
      c = min(R::cost(lq, lk, t, causal), nbuckets - 1);
    }
    const int r = chunk_rank(k, nbuckets, valid, c);
    if (valid) {
      int first, len;
      R::run_of(lq, lk, t, ts[b + 1] - ts[b], c, nbuckets, causal, first, len);
      const int p0 = item_slot(k, c, k.carry[c] + r, t - first, H);
      for (int hh = 0; hh < H; ++hh) {
        const int64_t p = (int64_t)p0 + (int64_t)hh * len;
        if (p >= 0 && p < capacity) items[p] = make_int2(b, (t << 8) | hh);   // true for valid offsets
      }
    }
    __syncthreads();
    for (int cc = tid; cc < nbuckets; cc += kSchedThreads) k.carry[cc] += k.chunk_tot[cc];
    __syncthreads();
  }
  const int64_t n_items = (int64_t)H * total_tiles;
  if (tid == 0) *job.count = (int)n_items;

  // 5. records in list order, from the global list (the barrier that ends
  // step 4 makes its item stores visible).  Buffer accesses bounded to the
  // list keep the loop free of branches: loads past the item count read
  // zeros, stores past the capacity are dropped.
  constexpr int kUnroll = 4, kPer = kUnroll * kSchedThreads;
  for (int64_t base = 0; base < capacity; base += kPer) {
    const int n_in = (int)max((int64_t)0, min(n_items - base, (int64_t)kPer));
    const int n_cap = (int)min(capacity - base, (int64_t)kPer);
    const __amdgpu_buffer_rsrc_t irs =
        __builtin_amdgcn_make_buffer_rsrc(items + base, 0, n_in * (int)sizeof(int2), kBufferWord3);
    const __amdgpu_buffer_rsrc_t mrs =
        __builtin_amdgcn_make_buffer_rsrc(job.meta + base, 0, n_cap * (int)sizeof(ItemMeta), kBufferWord3);
    int2 it[kUnroll];
#pragma unroll
    for (int r = 0; r < kUnroll; ++r) {
      const int i = r * kSchedThreads + tid;
      it[r] = __builtin_bit_cast(int2, __builtin_amdgcn_raw_buffer_load_b64(irs, i * (int)sizeof(int2), 0, 0));
    }
#pragma unroll
    for (int r = 0; r < kUnroll; ++r) {
      const int i = r * kSchedThreads + tid;
      const int b = it[r].x;   // 0 past the count: a valid sequence to read
      const int q0 = qo[b], q1 = qo[b + 1], k0 = ko[b], k1 = ko[b + 1];
      const int lq = i < n_in ? q1 - q0 : -1;
      const u32x4 lo = {(uint32_t)q0, (uint32_t)lq, (uint32_t)k0, (uint32_t)(k1 - k0)};
      const u32x4 hi = {(uint32_t)(it[r].y & 255), (uint32_t)(it[r].y >> 8), (uint32_t)b, 0u};
      const int off = i * (int)sizeof(ItemMeta);
      __builtin_amdgcn_raw_buffer_store_b128(lo, mrs, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(hi, mrs, off + 16, 0, 0);
    }
  }
}

// The offsets' rules (kOffsetsBad* bits that fail), over the whole
// workgroup.  Reads q_offsets[0 .. B] and kv_offsets[0 .. B] only.
__device__ int offsets_violations(const int* __restrict__ qo, const int* __restrict__ ko, int B,
                                  const OffsetCheck& c) {
  int bits = 0;
  for (int b = threadIdx.x; b <= B; b += kSchedThreads) {
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

template <int PASS>
__device__ void sched_body(const int* __restrict__ qo, const int* __restrict__ ko, int B, int H, int causal,
                           const SchedJob& job, char* smem) {
  const int bad = job.chk.check ? offsets_violations(qo, ko, B, job.chk) : 0;
  if (job.chk.status && threadIdx.x == 0) *job.chk.status = bad;
  if (bad) {
    // nothing is enumerated from such offsets: an empty list whose records
    // send every attention workgroup home
    if (threadIdx.x == 0) *job.count = 0;
    for (int64_t p = threadIdx.x; p < job.capacity; p += kSchedThreads) job.meta[p] = ItemMeta{0, -1, 0, 0, 0, 0, 0, 0};
    for (int b = threadIdx.x; b <= B; b += kSchedThreads) job.tile_start[b] = 0;
    return;
  }
  if (job.in_lds) sched_body_lds<PASS>(qo, ko, B, H, causal, job, smem);
  else sched_body_global<PASS>(qo, ko, B, H, causal, job, smem);
}

template <int PASS>
__global__ __launch_bounds__(kSchedThreads) void sched_kernel(const int* __restrict__ qo, const int* __restrict__ ko,
                                                              int B, int H, int causal, SchedJob job) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  sched_body<PASS>(qo, ko, B, H, causal, job, smem);
}

// The backward's two lists in one launch: workgroup 0 builds the
// query-tile list of the dQ pass (QPASS: 128- or 256-row tiles over the
// stored dS, or the 64-row tiles of the recomputing pass), workgroup 1 the
// key-tile list.  Further workgroups, when
// launched (softmax), form the row statistics of elements T and head
// dimension D meanwhile: with G of them, workgroup 2 + i takes the units
// i, i + G, i + 2G, ... (unit u: row chunk u / heads of head u % heads), and
// has the next unit's reads in flight while it reduces the current one.
// The two builders run alone on their compute units for most of their
// time; the statistics fill the rest of the chip, one workgroup per CU.
template <int QPASS, typename T, int D>
__global__ __launch_bounds__(kSchedThreads) void sched_pair_kernel(const int* __restrict__ qo,
                                                                   const int* __restrict__ ko, int B, int H,
                                                                   int causal, SchedJob jdq, SchedJob jkv,
                                                                   StatsArgs sa) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  if (blockIdx.x == 0) {
    sched_body<QPASS>(qo, ko, B, H, causal, jdq, smem);
  } else if (blockIdx.x == 1) {
    sched_body<kPassKV>(qo, ko, B, H, causal, jkv, smem);
  } else {
    using R = StatsRows<T, D, kSchedThreads>;
    const int64_t units = (int64_t)((sa.total_q + R::C::ROWS - 1) / R::C::ROWS) * sa.heads;
    const int64_t g = (int64_t)gridDim.x - 2;
    const int tid = (int)threadIdx.x;
    int64_t u = (int64_t)blockIdx.x - 2;
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

// LDS a workgroup of the builder may take on the current device (the whole
// LDS of a compute unit on gfx950: the builder runs alone).
static size_t sched_lds_budget() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0)
    return kSchedMinLds;
  return (size_t)v;
}

// Whether the all-LDS body may be used where it fits (default): the
// environment variable JFA_SCHED_STAGE=0 forbids it, so that tests reach
// the global-memory body too.
static bool sched_lds_allowed() {
  const char* e = std::getenv("JFA_SCHED_STAGE");
  return !(e && e[0] == '0' && e[1] == '\0');
}

// The job of one pass and the dynamic LDS it needs.
static SchedJob make_job(int32_t batch, int32_t heads, int32_t nbuckets, void* wl_base, const WorklistLayout& lay,
                         const OffsetCheck& chk, size_t& lds) {
  char* base = static_cast<char*>(wl_base);
  SchedJob j;
  j.chk = chk;
  j.nbuckets = nbuckets;
  j.capacity = lay.capacity;
  // heads >= 1 items per tile: capacity / heads bounds the tile count
  const int64_t max_tiles = lay.capacity / heads;
  j.max_tiles = (int)std::min<int64_t>(max_tiles, INT32_MAX);
  const size_t all = sched_lds_fixed(nbuckets) + sched_lds_all(batch, max_tiles, lay.capacity);
  j.in_lds = sched_lds_allowed() && batch <= kMaxTileInfoBatch && nbuckets <= (1 << kTileInfoBits) &&
             max_tiles <= 0xffff && heads <= 0xffff && all <= sched_lds_budget();
  lds = j.in_lds ? all : sched_lds_fixed(nbuckets);
  j.count = reinterpret_cast<int*>(base);
  j.items = reinterpret_cast<int2*>(base + lay.items_off);
  j.tile_start = reinterpret_cast<int*>(base + lay.tile_start_off);
  j.meta = reinterpret_cast<ItemMeta*>(base + lay.meta_off);
  return j;
}

hipError_t launch_sched(int pass, const int32_t* qo, const int32_t* ko, int32_t batch, int32_t heads,
                        int32_t causal, int32_t nbuckets, void* wl_base, const WorklistLayout& lay,
                        const OffsetCheck& chk, hipStream_t stream) {
  size_t lds;
  const SchedJob j = make_job(batch, heads, nbuckets, wl_base, lay, chk, lds);
  if (pass == kPassQ)
    hipLaunchKernelGGL(sched_kernel<kPassQ>, dim3(1), dim3(kSchedThreads), lds, stream, qo, ko, batch, heads,
                       causal, j);
  else if (pass == kPassDQS)
    hipLaunchKernelGGL(sched_kernel<kPassDQS>, dim3(1), dim3(kSchedThreads), lds, stream, qo, ko, batch, heads,
                       causal, j);
  else if (pass == kPassDQ)
    hipLaunchKernelGGL(sched_kernel<kPassDQ>, dim3(1), dim3(kSchedThreads), lds, stream, qo, ko, batch, heads,
                       causal, j);
  else
    hipLaunchKernelGGL(sched_kernel<kPassKV>, dim3(1), dim3(kSchedThreads), lds, stream, qo, ko, batch, heads,
                       causal, j);
  return hipGetLastError();
}

template <int QPASS, typename T, int D>
static hipError_t pair_launch(const int32_t* qo, const int32_t* ko, int32_t batch, int32_t heads, int32_t causal,
                              const SchedJob& jq, const SchedJob& jkv, const StatsArgs* stats, size_t lds,
                              hipStream_t stream) {
  constexpr int rows = StatsCfg<T, D, kSchedThreads>::ROWS;
  // one statistics workgroup per remaining CU at most (the builders' LDS
  // may leave room for only one 1024-thread workgroup per CU), each looping
  const int64_t units = stats ? (int64_t)((stats->total_q + rows - 1) / rows) * heads : 0;
  const int64_t extra = std::min<int64_t>(units, kStatsWorkgroups);
  const StatsArgs sa = stats ? *stats : StatsArgs{};
  hipLaunchKernelGGL((sched_pair_kernel<QPASS, T, D>), dim3((unsigned)(2 + extra)), dim3(kSchedThreads), lds, stream,
                     qo, ko, batch, heads, causal, jq, jkv, sa);
  return hipGetLastError();
}

template <int QPASS, typename T>
static hipError_t pair_launch_d(int head_dim, const int32_t* qo, const int32_t* ko, int32_t batch, int32_t heads,
                                int32_t causal, const SchedJob& jq, const SchedJob& jkv, const StatsArgs* stats,
                                size_t lds, hipStream_t stream) {
  switch (head_dim) {
    case 32: return pair_launch<QPASS, T, 32>(qo, ko, batch, heads, causal, jq, jkv, stats, lds, stream);
    case 64: return pair_launch<QPASS, T, 64>(qo, ko, batch, heads, causal, jq, jkv, stats, lds, stream);
    case 128: return pair_launch<QPASS, T, 128>(qo, ko, batch, heads, causal, jq, jkv, stats, lds, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_sched_pair(int qpass, const int32_t* qo, const int32_t* ko, int32_t batch, int32_t heads,
                             int32_t causal, int32_t nb_dq, void* wl_dq, const WorklistLayout& lay_dq, int32_t nb_kv,
                             void* wl_kv, const WorklistLayout& lay_kv, const StatsArgs* stats, int dtype,
                             int head_dim, const OffsetCheck& chk, hipStream_t stream) {
  size_t lds_q, lds_kv;
  const SchedJob jq = make_job(batch, heads, nb_dq, wl_dq, lay_dq, chk, lds_q);
  const SchedJob jkv = make_job(batch, heads, nb_kv, wl_kv, lay_kv, chk, lds_kv);
  const size_t lds = lds_q > lds_kv ? lds_q : lds_kv;
  if (qpass == kPassDQS)
    return dtype == 0 ? pair_launch_d<kPassDQS, __bf16>(head_dim, qo, ko, batch, heads, causal, jq, jkv, stats, lds, stream)
                      : pair_launch_d<kPassDQS, float>(head_dim, qo, ko, batch, heads, causal, jq, jkv, stats, lds, stream);
  if (qpass == kPassQ)
    return dtype == 0 ? pair_launch_d<kPassQ, __bf16>(head_dim, qo, ko, batch, heads, causal, jq, jkv, stats, lds, stream)
                      : pair_launch_d<kPassQ, float>(head_dim, qo, ko, batch, heads, causal, jq, jkv, stats, lds, stream);
  return dtype == 0 ? pair_launch_d<kPassDQ, __bf16>(head_dim, qo, ko, batch, heads, causal, jq, jkv, stats, lds, stream)
                    : pair_launch_d<kPassDQ, float>(head_dim, qo, ko, batch, heads, causal, jq, jkv, stats, lds, stream);
}

}  // namespace jfa

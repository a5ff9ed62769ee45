// Device-side work-list builder: the software tile scheduler for jagged
// tensors (piletech.kr/articles/112134, section 상세 정리 / Detailed notes,
// items on Jagged Flash Attention -- persistent-kernel scheduling -- and on
// GDPA -- software tile scheduling for jagged tensors).
//
// From the offsets alone it enumerates every work item (sequence b, head h,
// tile t), prices it by the number of inner blocks the attention kernel will
// visit for it, and writes the items longest first (cost descending), ties
// in (b, h, t) order -- a stable counting sort by cost.  One workgroup of
// 1024 threads does it all on the device, so the caller's stream never waits
// for the host.
#include "jfa_common.hpp"
#include "jfa_internal.h"

namespace jfa {

constexpr int kSchedThreads = 1024;
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

// LDS bytes of the builder's cost-bucket arrays, and of the optional copy of
// the per-sequence tile starts and lengths.
__host__ __device__ constexpr size_t sched_lds_fixed(int nbuckets) {
  return (((size_t)nbuckets * (3 * 4 + 2 + 2 * kSchedWaves) + 32 * 4) + 15) & ~(size_t)15;
}
__host__ __device__ constexpr size_t sched_lds_seqs(int batch) { return ((size_t)3 * batch + 3) * 4; }
constexpr size_t kSchedMaxLds = 64 * 1024;

template <int PASS>
struct TileRule {
  // Tiles split the query side (forward: kPassQ, dQ: kPassDQ) or the key
  // side (dK/dV: kPassKV).
  static constexpr bool kQuery = PASS != kPassKV;
  static constexpr int kTile = PASS == kPassQ ? kFwdBM : PASS == kPassDQ ? kDqBM : kBwdBN;
  __device__ static int rows(int lq, int lk) { return kQuery ? lq : lk; }
  __device__ static int cost(int lq, int lk, int t, int causal) {
    if (PASS == kPassQ) return q_tile_kv_blocks(lq, lk, t, kFwdBM, kFwdBN, causal);
    if (PASS == kPassDQ) return q_tile_kv_blocks(lq, lk, t, kDqBM, kDqBN, causal);
    return kv_tile_q_blocks(lq, lk, t, kBwdBM, kBwdBN, causal);
  }
  // Costs are monotone in t within a sequence: non-decreasing for query
  // tiles (later rows see more keys), non-increasing for key tiles (later
  // keys are seen by fewer rows).  before_or_eq(x, c): a tile of cost x may
  // come before (or is in) the run of cost c; after_or_eq: after or in it.
  __device__ static bool before_or_eq(int x, int c) { return kQuery ? x <= c : x >= c; }
  __device__ static bool after_or_eq(int x, int c) { return kQuery ? x >= c : x <= c; }
};

// One pass's work list: where it goes and how it is built.
struct SchedJob {
  int nbuckets;
  int64_t capacity;
  int stage_seqs;
  int* count;
  int2* items;
  int* tile_start;
  ItemMeta* meta;
};

template <int PASS>
__device__ void sched_body(const int* __restrict__ qo, const int* __restrict__ ko, int B, int H, int causal,
                           const SchedJob& job, char* smem) {
  using R = TileRule<PASS>;
  const int nbuckets = job.nbuckets, stage_seqs = job.stage_seqs;
  const int64_t capacity = job.capacity;
  int* const count = job.count;
  int2* const items = job.items;
  int* const tile_start = job.tile_start;
  ItemMeta* const meta = job.meta;
  int* hist = reinterpret_cast<int*>(smem);
  int* start = hist + nbuckets;
  int* carry = start + nbuckets;
  int* tmp = carry + nbuckets;                       // kSchedWaves ints (+pad)
  unsigned short* chunk_tot = reinterpret_cast<unsigned short*>(tmp + 32);
  unsigned short* wave_cnt = chunk_tot + nbuckets;   // [kSchedWaves][nbuckets]
  // Per-sequence tile starts and lengths, read by every tile's binary
  // search: staged in LDS when the launch provided room (stage_seqs), else
  // read from global memory.
  int* seq_lds = reinterpret_cast<int*>(smem + sched_lds_fixed(nbuckets));
  int* ts = stage_seqs ? seq_lds : tile_start;
  const int* q_off = stage_seqs ? seq_lds + (B + 1) : qo;
  const int* k_off = stage_seqs ? seq_lds + (2 * B + 2) : ko;
  auto lengths = [&](int b, int& lq, int& lk) {
    lq = q_off[b + 1] - q_off[b];
    lk = k_off[b + 1] - k_off[b];
  };

  const int tid = threadIdx.x, l = lane_id(), w = tid / kWave;

  // 1. tiles per sequence -> exclusive prefix tile_start[b]
  int run = 0;
  for (int base = 0; base < B; base += kSchedThreads) {
    const int b = base + tid;
    int n = 0;
    if (b < B) {
      const int q0 = qo[b], q1 = qo[b + 1], k0 = ko[b], k1 = ko[b + 1];
      n = ceil_div(R::rows(q1 - q0, k1 - k0), R::kTile);
      if (stage_seqs) {
        seq_lds[B + 1 + b] = q0;
        seq_lds[2 * B + 2 + b] = k0;
        if (b == B - 1) {
          seq_lds[2 * B + 1] = q1;
          seq_lds[3 * B + 2] = k1;
        }
      }
    }
    int tot;
    const int ex = block_excl_scan(n, tmp, tot);
    if (b < B) {
      tile_start[b] = run + ex;
      if (stage_seqs) ts[b] = run + ex;
    }
    run += tot;
  }
  const int total_tiles = run;
  if (tid == 0) {
    tile_start[B] = total_tiles;
    if (stage_seqs) ts[B] = total_tiles;
  }
  for (int c = tid; c < nbuckets; c += kSchedThreads) {
    hist[c] = 0;
    carry[c] = 0;
  }
  __syncthreads();

  // 2. histogram of tile costs
  for (int u = tid; u < total_tiles; u += kSchedThreads) {
    const int b = find_seq(ts, B, u);
    const int t = u - ts[b];
    int lq, lk;
    lengths(b, lq, lk);
    const int c = min(R::cost(lq, lk, t, causal), nbuckets - 1);
    atomicAdd(&hist[c], 1);
  }
  __syncthreads();

  // 3. first output slot of each cost bucket, largest cost first
  run = 0;
  for (int base = 0; base < nbuckets; base += kSchedThreads) {
    const int o = base + tid;
    const int c = nbuckets - 1 - o;
    const int n = (o < nbuckets) ? hist[c] : 0;
    int tot;
    const int ex = block_excl_scan(n, tmp, tot);
    if (o < nbuckets) start[c] = H * (run + ex);
    run += tot;
  }
  __syncthreads();

  // 4. stable rank of each tile among the tiles of equal cost, then its H items
  for (int base = 0; base < total_tiles; base += kSchedThreads) {
    for (int i = tid; i < kSchedWaves * nbuckets; i += kSchedThreads) wave_cnt[i] = 0;
    __syncthreads();
    const int u = base + tid;
    const bool valid = u < total_tiles;
    int b = 0, t = 0, c = -1, lq = 0, lk = 0;
    if (valid) {
      b = find_seq(ts, B, u);
      t = u - ts[b];
      lengths(b, lq, lk);
      c = min(R::cost(lq, lk, t, causal), nbuckets - 1);
    }
    // rank inside the wave: one ballot per distinct cost present
    unsigned long long pending = __ballot(valid);
    int local = 0;
    while (pending) {
      const int leader = __ffsll((unsigned long long)pending) - 1;
      const int lc = __shfl(c, leader, kWave);
      const unsigned long long m = __ballot(c == lc);
      if (c == lc) local = __popcll(m & ((1ull << l) - 1ull));
      if (l == leader) wave_cnt[w * nbuckets + lc] = (unsigned short)__popcll(m);
      pending &= ~m;
    }
    __syncthreads();
    // rank offset of each wave inside this chunk, per cost
    for (int cc = tid; cc < nbuckets; cc += kSchedThreads) {
      int r = 0;
      for (int ww = 0; ww < kSchedWaves; ++ww) {
        const int x = wave_cnt[ww * nbuckets + cc];
        wave_cnt[ww * nbuckets + cc] = (unsigned short)r;
        r += x;
      }
      chunk_tot[cc] = (unsigned short)r;
    }
    __syncthreads();
    if (valid) {
      const int rank = carry[c] + wave_cnt[w * nbuckets + c] + local;
      // the run of tiles of sequence b with this same cost: [first, last]
      const int ntiles = ts[b + 1] - ts[b];
      int lo = 0, hi = t;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (R::after_or_eq(min(R::cost(lq, lk, mid, causal), nbuckets - 1), c)) hi = mid; else lo = mid + 1;
      }
      const int first = lo;
      lo = t;
      hi = ntiles - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (R::before_or_eq(min(R::cost(lq, lk, mid, causal), nbuckets - 1), c)) lo = mid; else hi = mid - 1;
      }
      const int len = lo - first + 1;
      const int k = t - first;
      // items of bucket c are ordered (b, h, t): all earlier sequences' tiles
      // of this cost (rank - k of them) times H, then h runs of length len
      const int p0 = start[c] + H * (rank - k) + k;
      for (int hh = 0; hh < H; ++hh) {
        const int64_t p = (int64_t)p0 + (int64_t)hh * len;
        if (p >= 0 && p < capacity) items[p] = make_int2(b, (t << 8) | hh);   // true for valid offsets
      }
    }
    __syncthreads();
    for (int cc = tid; cc < nbuckets; cc += kSchedThreads) carry[cc] += chunk_tot[cc];
    __syncthreads();
  }
  if (tid == 0) *count = H * total_tiles;

  // 5. the kernels' records, in list order.  Written from the (now final)
  // item list rather than where step 4 places each item: step 4 scatters,
  // and scattered 32-byte records cost far more than contiguous ones.
  // Records past the count (lq = -1) tell surplus workgroups to exit.  The
  // barrier at the end of step 4 makes the item stores visible here.
  // The offsets are read from LDS when staged (a separate copy of the loop,
  // so that its waits cover LDS reads only).  Buffer accesses bounded to the
  // list keep the loop free of branches: loads past the item count read
  // zeros, stores past the capacity are dropped.
  const int64_t n_items = (int64_t)H * total_tiles;
  auto records = [&](const int* qof, const int* kof) {
    constexpr int kUnroll = 4, kPer = kUnroll * kSchedThreads;
    for (int64_t base = 0; base < capacity; base += kPer) {
      const int n_in = (int)max((int64_t)0, min(n_items - base, (int64_t)kPer));
      const int n_cap = (int)min(capacity - base, (int64_t)kPer);
      const __amdgpu_buffer_rsrc_t irs =
          __builtin_amdgcn_make_buffer_rsrc(items + base, 0, n_in * (int)sizeof(int2), kBufferWord3);
      const __amdgpu_buffer_rsrc_t mrs =
          __builtin_amdgcn_make_buffer_rsrc(meta + base, 0, n_cap * (int)sizeof(ItemMeta), kBufferWord3);
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
        const int q0 = qof[b], q1 = qof[b + 1], k0 = kof[b], k1 = kof[b + 1];
        const int lq = i < n_in ? q1 - q0 : -1;
        const u32x4 lo = {(uint32_t)q0, (uint32_t)lq, (uint32_t)k0, (uint32_t)(k1 - k0)};
        const u32x4 hi = {(uint32_t)(it[r].y & 255), (uint32_t)(it[r].y >> 8), 0u, 0u};
        const int off = i * (int)sizeof(ItemMeta);
        __builtin_amdgcn_raw_buffer_store_b128(lo, mrs, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(hi, mrs, off + 16, 0, 0);
      }
    }
  };
  if (stage_seqs) records(q_off, k_off);
  else records(qo, ko);
}

template <int PASS>
__global__ __launch_bounds__(kSchedThreads) void sched_kernel(const int* __restrict__ qo, const int* __restrict__ ko,
                                                              int B, int H, int causal, SchedJob job) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  sched_body<PASS>(qo, ko, B, H, causal, job, smem);
}

// The backward's two lists in one launch: workgroup 0 builds the dQ-tile
// list, workgroup 1 the key-tile list.
__global__ __launch_bounds__(kSchedThreads) void sched_pair_kernel(const int* __restrict__ qo,
                                                                   const int* __restrict__ ko, int B, int H,
                                                                   int causal, SchedJob jdq, SchedJob jkv) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  if (blockIdx.x == 0) sched_body<kPassDQ>(qo, ko, B, H, causal, jdq, smem);
  else sched_body<kPassKV>(qo, ko, B, H, causal, jkv, smem);
}

WorklistLayout worklist_layout(int pass, int32_t batch, int32_t heads, int32_t total_rows) {
  const int64_t tile = pass == kPassQ ? kFwdBM : pass == kPassDQ ? kDqBM : kBwdBN;
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

// The job of one pass and the dynamic LDS it needs.
static SchedJob make_job(int32_t batch, int32_t nbuckets, void* wl_base, const WorklistLayout& lay, size_t& lds) {
  char* base = static_cast<char*>(wl_base);
  SchedJob j;
  j.nbuckets = nbuckets;
  j.capacity = lay.capacity;
  lds = sched_lds_fixed(nbuckets);
  j.stage_seqs = lds + sched_lds_seqs(batch) <= kSchedMaxLds ? 1 : 0;
  if (j.stage_seqs) lds += sched_lds_seqs(batch);
  j.count = reinterpret_cast<int*>(base);
  j.items = reinterpret_cast<int2*>(base + lay.items_off);
  j.tile_start = reinterpret_cast<int*>(base + lay.tile_start_off);
  j.meta = reinterpret_cast<ItemMeta*>(base + lay.meta_off);
  return j;
}

hipError_t launch_sched(int pass, const int32_t* qo, const int32_t* ko, int32_t batch, int32_t heads,
                        int32_t causal, int32_t nbuckets, void* wl_base, const WorklistLayout& lay,
                        hipStream_t stream) {
  size_t lds;
  const SchedJob j = make_job(batch, nbuckets, wl_base, lay, lds);
  if (pass == kPassQ)
    hipLaunchKernelGGL(sched_kernel<kPassQ>, dim3(1), dim3(kSchedThreads), lds, stream, qo, ko, batch, heads,
                       causal, j);
  else if (pass == kPassDQ)
    hipLaunchKernelGGL(sched_kernel<kPassDQ>, dim3(1), dim3(kSchedThreads), lds, stream, qo, ko, batch, heads,
                       causal, j);
  else
    hipLaunchKernelGGL(sched_kernel<kPassKV>, dim3(1), dim3(kSchedThreads), lds, stream, qo, ko, batch, heads,
                       causal, j);
  return hipGetLastError();
}

hipError_t launch_sched_pair(const int32_t* qo, const int32_t* ko, int32_t batch, int32_t heads, int32_t causal,
                             int32_t nb_dq, void* wl_dq, const WorklistLayout& lay_dq, int32_t nb_kv, void* wl_kv,
                             const WorklistLayout& lay_kv, hipStream_t stream) {
  size_t lds_q, lds_kv;
  const SchedJob jq = make_job(batch, nb_dq, wl_dq, lay_dq, lds_q);
  const SchedJob jkv = make_job(batch, nb_kv, wl_kv, lay_kv, lds_kv);
  hipLaunchKernelGGL(sched_pair_kernel, dim3(2), dim3(kSchedThreads), lds_q > lds_kv ? lds_q : lds_kv, stream, qo,
                     ko, batch, heads, causal, jq, jkv);
  return hipGetLastError();
}

}  // namespace jfa

// BlockAttention's fixed blocks as jagged sequences (piletech.kr/articles/
// 112134, section 상세 정리 / Detailed notes, BlockAttention item: fixed
// blocks of 64 tokens turn attention's cost from quadratic to linear in the
// sequence length).
//
// Attention restricted to each run of `block` consecutive tokens of a
// sequence (counted from its first token) is plain jagged attention over
// those runs taken as sequences of their own.  The block form therefore
// needs only new offsets, built here on the device: every sequence b (rows
// offsets[b] .. offsets[b+1]-1) is split into ceil(L_b / block) runs, in
// order, and the list is padded with empty sequences up to
// total / block + batch runs -- a size the host knows without reading the
// offsets, since sum_b ceil(L_b / block) <= total / block + batch.
#include "jfa_common.hpp"
#include "jfa_internal.h"

namespace jfa {

constexpr int kBlkThreads = 1024;

// One workgroup: sequences in chunks of 1024, a block-wide exclusive scan of
// the run counts gives each sequence's first run, and a running carry joins
// the chunks.  out[i] for i < runs is a run's first row; out[runs .. out_len-1]
// = total (the last run's end, then empty runs).  Writes stay inside
// out[0 .. out_len-1] whatever the offsets hold.
__global__ __launch_bounds__(kBlkThreads) void block_offsets_kernel(const int* __restrict__ off, int B, int total,
                                                                    int block, int* __restrict__ out, int out_len) {
  __shared__ int wsum[kBlkThreads / kWave];
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
  int carry = 0;
  for (int base = 0; base < B; base += kBlkThreads) {
    const int b = base + tid;
    int start = 0, n = 0;
    if (b < B) {
      start = off[b];
      const int len = max(off[b + 1] - start, 0);
      n = (int)(((int64_t)len + block - 1) / block);
    }
    int x = n;   // inclusive scan within the wave
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(x, o, kWave);
      if (lane >= o) x += y;
    }
    if (lane == kWave - 1) wsum[w] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kBlkThreads / kWave; ++i) {
      const int s = wsum[i];
      before += i < w ? s : 0;
      tot += s;
    }
    __syncthreads();
    const int64_t pos = (int64_t)carry + before + x - n;   // this sequence's first run
    for (int c = 0; c < n; ++c)
      if (pos + c < out_len) out[pos + c] = start + c * block;
    carry = (int)min((int64_t)carry + tot, (int64_t)out_len);
  }
  for (int i = carry + tid; i < out_len; i += kBlkThreads) out[i] = total;
}

hipError_t launch_block_offsets(const int32_t* off, int32_t batch, int32_t total, int32_t block, int32_t* out,
                                int32_t out_len, hipStream_t stream) {
  hipLaunchKernelGGL(block_offsets_kernel, dim3(1), dim3(kBlkThreads), 0, stream, off, batch, total, block, out,
                     out_len);
  return hipGetLastError();
}

}  // namespace jfa

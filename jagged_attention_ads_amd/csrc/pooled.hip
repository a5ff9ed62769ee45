// Pooled multi-head attention's two small kernels (the attention itself is
// the jagged cross attention of fwd.hip / bwd.hip).  Reading of the page
// piletech.kr/articles/112134, section 상세 정리 (Detailed notes), jagged-input
// item, which names pooled multi-head attention among the ads models'
// attention patterns: n_seeds query vectors shared by every sequence attend
// over each sequence's keys, pooling it into n_seeds rows.
//   pooled_prep_kernel:   the per-sequence query offsets b * n_seeds and the
//                         seeds repeated once per sequence (the queries of
//                         the cross attention);
//   pooled_partial_kernel, pooled_final_kernel: the seeds' gradient, the sum
//                         over sequences of their per-sequence query
//                         gradients, in fp32 and in a fixed order (no
//                         atomics: bitwise reproducible).
#include <algorithm>

#include "jfa_common.hpp"
#include "jfa_internal.h"

namespace jfa {

// Grid-stride over the 16-byte chunks of the repeated seeds, and the offsets.
__global__ __launch_bounds__(256) void pooled_prep_kernel(const u32x4* seeds, int64_t seed_chunks, int32_t batch,
                                                           int32_t n_seeds, u32x4* q, int32_t* q_offsets) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int64_t i = i0; i <= batch; i += stride) q_offsets[i] = (int32_t)(i * n_seeds);
  const int64_t total = seed_chunks * batch;
  for (int64_t i = i0; i < total; i += stride) q[i] = seeds[i % seed_chunks];
}

// The seeds' gradient in two passes, each element summed in a fixed order:
// pass 1 sums the sequences of chunk c (sequences c*per .. c*per+per-1, in
// order) into an fp32 partial, one thread per (element, chunk); pass 2 sums
// the partials in chunk order and rounds once.
template <typename T>
__global__ __launch_bounds__(256) void pooled_partial_kernel(const T* dq, int64_t seed_elems, int32_t batch,
                                                             int32_t per, float* partial) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int32_t c = blockIdx.y;
  if (e >= seed_elems) return;
  const int32_t b0 = c * per, b1 = min(batch, b0 + per);
  float acc = 0.f;
  for (int32_t b = b0; b < b1; ++b) acc += (float)dq[(int64_t)b * seed_elems + e];
  partial[(int64_t)c * seed_elems + e] = acc;
}

template <typename T>
__global__ __launch_bounds__(256) void pooled_final_kernel(const float* partial, int64_t seed_elems, int32_t chunks,
                                                           T* dseeds) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= seed_elems) return;
  float acc = 0.f;
  for (int32_t c = 0; c < chunks; ++c) acc += partial[(int64_t)c * seed_elems + e];
  dseeds[e] = (T)acc;
}

hipError_t launch_pooled_prep(const void* seeds, int64_t seed_bytes, int32_t batch, int32_t n_seeds, void* q,
                              int32_t* q_offsets, hipStream_t stream) {
  if (seed_bytes % 16 != 0) return hipErrorInvalidValue;
  const int64_t chunks = seed_bytes / 16;
  const int64_t work = std::max<int64_t>(chunks * batch, (int64_t)batch + 1);
  const unsigned grid = (unsigned)std::min<int64_t>((work + 255) / 256, 4096);
  hipLaunchKernelGGL(pooled_prep_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const u32x4*>(seeds), chunks,
                     batch, n_seeds, static_cast<u32x4*>(q), q_offsets);
  return hipGetLastError();
}

int32_t pooled_chunks(int32_t batch) { return std::max(1, std::min<int32_t>(kPooledChunks, batch)); }

hipError_t launch_pooled_reduce(const void* dq, int64_t seed_elems, int32_t batch, int dtype, float* partial,
                                void* dseeds, hipStream_t stream) {
  const unsigned gx = (unsigned)((seed_elems + 255) / 256);
  if (gx == 0) return hipSuccess;
  // no sequences: pass 2 alone, over no partials, writes zeros
  const int32_t chunks = batch > 0 ? pooled_chunks(batch) : 0;
  const int32_t per = chunks > 0 ? (batch + chunks - 1) / chunks : 0;
  if (dtype == 0) {
    if (chunks > 0)
      hipLaunchKernelGGL(pooled_partial_kernel<__bf16>, dim3(gx, (unsigned)chunks), dim3(256), 0, stream,
                         static_cast<const __bf16*>(dq), seed_elems, batch, per, partial);
    hipLaunchKernelGGL(pooled_final_kernel<__bf16>, dim3(gx), dim3(256), 0, stream, partial, seed_elems, chunks,
                       static_cast<__bf16*>(dseeds));
  } else {
    if (chunks > 0)
      hipLaunchKernelGGL(pooled_partial_kernel<float>, dim3(gx, (unsigned)chunks), dim3(256), 0, stream,
                         static_cast<const float*>(dq), seed_elems, batch, per, partial);
    hipLaunchKernelGGL(pooled_final_kernel<float>, dim3(gx), dim3(256), 0, stream, partial, seed_elems, chunks,
                       static_cast<float*>(dseeds));
  }
  return hipGetLastError();
}

}  // namespace jfa

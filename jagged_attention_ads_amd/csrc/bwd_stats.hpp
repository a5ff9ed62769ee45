// Row statistics of the softmax backward, shared by the standalone kernel
// (bwd.hip) and the backward's work-list launch (sched.hip), whose spare
// workgroups form them while two workgroups build the lists.
//
// Per (row i, head): delta_i = sum_c dO_ic O_ic -- the row sum of P o dP
// that the softmax Jacobian needs (the plain FlashAttention backward
// identity) -- as an fp32 sum of the stored values' products, and
// lse_i * log2(e), with rows that see no key (lse = -inf) mapped to 0: those
// rows are fully masked, and a finite value keeps every product finite.
#pragma once

#include "jfa_common.hpp"
#include "jfa_internal.h"

namespace jfa {

__device__ __forceinline__ float lse_log2(float lse) { return lse > -INFINITY ? lse * kLog2e : 0.f; }

// NT threads per workgroup: LPR lanes share one row's D values (16 bytes
// each) and reduce with cross-lane swaps; a workgroup covers ROWS
// consecutive rows of one head, loads first.
template <typename T, int D, int NT>
struct StatsCfg {
  static constexpr int LPR = D * (int)sizeof(T) / 16;   // lanes per row
  static constexpr int PPB = NT / LPR;                  // rows per pass of the workgroup
  static constexpr int kIter = 4;                       // passes per workgroup
  static constexpr int ROWS = PPB * kIter;              // rows per workgroup
};

// Rows chunk * ROWS .. +ROWS-1 of head h.  Memory-bound: every O and dO byte
// is read once, and the per-head outputs are written contiguously.  load()
// issues a thread's reads, finish() reduces and writes, so that a caller
// can have the next chunk's reads in flight while it reduces this one.
template <typename T, int D, int NT>
struct StatsRows {
  using C = StatsCfg<T, D, NT>;
  static constexpr int EPL = 16 / (int)sizeof(T);   // elements per lane
  u32x4 o[C::kIter], d[C::kIter];

  __device__ __forceinline__ void load(const StatsArgs& a, int chunk, int h, int tid) {
    const int sub = tid % C::LPR;
    const int r0 = chunk * C::ROWS + tid / C::LPR;
    const size_t rs = (size_t)a.heads * D;
#pragma unroll
    for (int i = 0; i < C::kIter; ++i) {
      const int r = r0 + i * C::PPB;
      o[i] = u32x4{0u, 0u, 0u, 0u};
      d[i] = o[i];
      if (r < a.total_q) {
        const size_t e = (size_t)r * rs + (size_t)h * D + (size_t)sub * EPL;
        o[i] = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.out) + e);
        d[i] = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.dout) + e);
      }
    }
  }

  __device__ __forceinline__ void finish(const StatsArgs& a, int chunk, int h, int tid) const {
    const int sub = tid % C::LPR;
    const int r0 = chunk * C::ROWS + tid / C::LPR;
#pragma unroll
    for (int i = 0; i < C::kIter; ++i) {
      float part = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if constexpr (sizeof(T) == 2) {
          part = fmaf(__uint_as_float(o[i][w] << 16), __uint_as_float(d[i][w] << 16), part);
          part = fmaf(__uint_as_float(o[i][w] & 0xffff0000u), __uint_as_float(d[i][w] & 0xffff0000u), part);
        } else {
          part = fmaf(__uint_as_float(o[i][w]), __uint_as_float(d[i][w]), part);
        }
      }
#pragma unroll
      for (int m = C::LPR / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m);
      const int r = r0 + i * C::PPB;
      if (sub == 0 && r < a.total_q) {
        const size_t si = (size_t)h * a.total_q + r;
        a.delta[si] = part;
        a.lse2[si] = lse_log2(a.lse[si]);
      }
    }
  }
};

template <typename T, int D, int NT>
__device__ __forceinline__ void stats_block(const StatsArgs& a, int chunk, int h, int tid) {
  StatsRows<T, D, NT> r;
  r.load(a, chunk, h, tid);
  r.finish(a, chunk, h, tid);
}

}  // namespace jfa

// Jagged attention backward (softmax and GDPA/SiLU) for gfx950, without
// atomics (piletech.kr/articles/112134, section 상세 정리 / Detailed notes,
// Jagged Flash Attention item: the backward's parallel split uses no atomic
// operations).
//
// The gradient sums over queries (dK, dV) and over keys (dQ) are split into
// two passes so that every output row is owned by exactly one workgroup and
// stored once:
//   dK/dV pass -- one work item per (sequence, head, 128-key tile); each wave
//     owns 32 keys (its K and V rows live in registers) and walks the
//     64-query blocks that see them, staged in swizzled LDS tiles.  P and dS are recomputed
//     from lse (softmax) or from the scores (SiLU).
//   dQ pass -- one work item per (sequence, head, 128-query tile); each wave
//     owns 32 queries and walks the 64-key blocks that they see.
// A preprocess kernel first forms delta_i = sum_c dO_ic O_ic (softmax only),
// the row sum of P o dP that the softmax Jacobian needs.
//
// Per (query i, key j) pair, with x = scale * q_i.k_j:
//   softmax: P = exp(x - lse_i);        dS = P (dP - delta_i)
//   silu:    P = silu(x) / Lk;          dS = dP silu'(x) / Lk,
//            silu'(x) = sig(x) (1 + x (1 - sig(x)))
//   dV_j += P dO_i,  dP = dO_i . V_j,  dK_j += scale dS q_i,  dQ_i += scale dS k_j
#include "jfa_common.hpp"
#include "jfa_internal.h"

namespace jfa {

// ---------------------------------------------------------------- delta

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ out, const T* __restrict__ dout,
                                                      float* __restrict__ delta, int heads, int total_q) {
  constexpr int LPR = D * (int)sizeof(T) / 16;   // lanes per (row, head)
  constexpr int RPB = 256 / LPR;                 // (row, head) pairs per block
  const int sub = threadIdx.x % LPR;
  const int64_t pair = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;   // = row * heads + head
  const int64_t npairs = (int64_t)total_q * heads;
  float acc = 0.f;
  if (pair < npairs) {
    const char* po = reinterpret_cast<const char*>(out + pair * D) + sub * 16;
    const char* pd = reinterpret_cast<const char*>(dout + pair * D) + sub * 16;
    const u32x4 a = *reinterpret_cast<const u32x4*>(po);
    const u32x4 b = *reinterpret_cast<const u32x4*>(pd);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (sizeof(T) == 2) {
        acc += __uint_as_float(a[e] << 16) * __uint_as_float(b[e] << 16);
        acc += __uint_as_float(a[e] & 0xffff0000u) * __uint_as_float(b[e] & 0xffff0000u);
      } else {
        acc += __uint_as_float(a[e]) * __uint_as_float(b[e]);
      }
    }
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m, kWave);
  if (pair < npairs && sub == 0) {
    const int64_t row = pair / heads, head = pair % heads;
    delta[head * total_q + row] = acc;
  }
}

// ---------------------------------------------------------------- shared math

// lse in log2 units, with rows that see no key (lse = -inf) mapped to 0:
// those rows are fully masked, and a finite value keeps exp2 at exactly 0.
__device__ __forceinline__ float lse_log2(float lse) { return lse > -INFINITY ? lse * kLog2e : 0.f; }

// P and dS of one score, softmax (ACT 0) or silu (ACT 1).
template <int ACT>
__device__ __forceinline__ void p_ds(float raw, float dp, float lse2, float delta, float scale, float scale_log2,
                                     float inv_lk, bool masked, float& p, float& ds) {
  if constexpr (ACT == 0) {
    const float x = raw * scale_log2 - lse2 - (masked ? kMaskShift : 0.f);
    p = fast_exp2(x);
    ds = p * (dp - delta);
  } else {
    const float x = raw * scale;
    const float sig = fast_rcp(1.0f + fast_exp2(-raw * scale_log2));
    const float keep = masked ? 0.f : inv_lk;
    p = x * sig * keep;
    ds = dp * sig * (1.0f + x * (1.0f - sig)) * keep;
  }
}

// ---------------------------------------------------------------- dK / dV

template <typename T, int D>
struct DkdvCfg {
  static constexpr int BN = kBwdBN, BM = kBwdBM, NT = 256;
  static constexpr int ES = sizeof(T);
  static constexpr int QT = Swz<T, D>::tile_bytes(BM);   // Q / dO tile
  static constexpr int STAGE = 2 * QT + 2 * BM * 4;   // Q, dO, lse2, delta
  static constexpr int LDS = 2 * STAGE;
  static constexpr int ND = D / 32, NK = D / 16;
};

template <typename T, int D, int ACT>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(BwdArgs a) {
  using C = DkdvCfg<T, D>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  if ((int)blockIdx.x >= *a.n_items_kv) return;
  int b, h, t;
  unpack_item(a.items_kv[blockIdx.x], b, h, t);
  const int qs = a.qo[b], lq = a.qo[b + 1] - qs;
  const int ks = a.ko[b], lk = a.ko[b + 1] - ks;
  const int off = lk - lq;

  const int tid = threadIdx.x, l = lane_id(), w = tid >> 6, g = l >> 5, c32 = l & 31;
  const int kw0 = t * C::BN + 32 * w;    // first key of this wave
  const int my_key = kw0 + c32;          // the key this lane owns (its column of S)
  const bool wave_live = kw0 < lk;
  const int nqb = kv_tile_q_blocks(lq, lk, t, C::BM, C::BN, a.causal);
  const int qb_first = kv_tile_first_q_block(lq, lk, t, C::BM, C::BN, a.causal);
  const size_t rs = (size_t)a.heads * D;
  const float inv_lk = lk > 0 ? 1.0f / (float)lk : 0.f;

  // this lane's key and value rows as B-operand fragments (d-slots 16*kk + 8*g + e)
  frag_t<T> kf[C::NK], vf[C::NK];
  {
    const int j = min(my_key, lk - 1);
    const T* kp = static_cast<const T*>(a.k) + (size_t)(ks + j) * rs + (size_t)h * D + 8 * g;
    const T* vp = static_cast<const T*>(a.v) + (size_t)(ks + j) * rs + (size_t)h * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < C::NK; ++kk) {
      kf[kk] = global_frag<T>(kp + 16 * kk);
      vf[kk] = global_frag<T>(vp + 16 * kk);
    }
  }
  f32x16 dk[C::ND], dv[C::ND];
#pragma unroll
  for (int i = 0; i < C::ND; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  const T* qb = static_cast<const T*>(a.q) + (size_t)qs * rs + (size_t)h * D;
  const T* db = static_cast<const T*>(a.dout) + (size_t)qs * rs + (size_t)h * D;
  const float* lse_h = ACT == 0 ? a.lse + (size_t)h * a.total_q + qs : nullptr;
  const float* del_h = ACT == 0 ? a.delta + (size_t)h * a.total_q + qs : nullptr;

  TileStage<T, D, C::BM, true> qst, dst;   // query rows stored swap23-permuted
  float st_lse = 0.f, st_del = 0.f;
  auto gload = [&](int qblk) {
    const int r0 = qblk * C::BM;
    qst.load(qb, (int)rs, r0, lq, tid);
    dst.load(db, (int)rs, r0, lq, tid);
    if (ACT == 0 && tid < C::BM) {
      const int r = min(r0 + tid, lq - 1);
      st_lse = lse_log2(lse_h[r]);
      st_del = del_h[r];
    }
  };
  auto lstore = [&](int buf) {
    char* st = smem + buf * C::STAGE;
    qst.store(st, tid);
    dst.store(st + C::QT, tid);
    if (ACT == 0 && tid < C::BM) {
      reinterpret_cast<float*>(st + 2 * C::QT)[tid] = st_lse;
      reinterpret_cast<float*>(st + 2 * C::QT + C::BM * 4)[tid] = st_del;
    }
  };

  if (nqb > 0) {
    gload(qb_first);
    lstore(0);
  }
  __syncthreads();

  for (int it = 0; it < nqb; ++it) {
    const int qblk = qb_first + it;
    if (it + 1 < nqb) gload(qblk + 1);
    const char* st = smem + (it & 1) * C::STAGE;
    const char* qt = st;
    const char* dt_ = st + C::QT;
    const float* lse2 = reinterpret_cast<const float*>(st + 2 * C::QT);
    const float* dlt = lse2 + C::BM;
    if (wave_live) {
#pragma unroll
      for (int sb = 0; sb < C::BM / 32; ++sb) {
        const int qa = qblk * C::BM + 32 * sb;   // first query row of the sub-block
        if (qa >= lq) break;
        if (a.causal && qa + 31 + off < kw0) continue;   // no row here sees this wave's keys
        // S and dP (32 queries x 32 keys); register r holds query qa + 16*(r/8) + 8*g + r%8
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int kk = 0; kk < C::NK; ++kk) {
          const frag_t<T> qfr = lds_row_frag<T, D>(qt, 32 * sb + c32, 16 * kk + 8 * g);
          mma(s, qfr, kf[kk]);
          const frag_t<T> dfr = lds_row_frag<T, D>(dt_, 32 * sb + c32, 16 * kk + 8 * g);
          mma(dp, dfr, vf[kk]);
        }
        const bool need_mask = (qa + 32 > lq) || (kw0 + 32 > lk) || (a.causal && kw0 + 31 > qa + off);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = 16 * (r >> 3) + 8 * g + (r & 7);   // row within the sub-block
          const int i = qa + qi;
          bool masked = false;
          if (need_mask) masked = (i >= lq) || (my_key >= lk) || (a.causal && my_key > i + off);
          float p, ds;
          const float l2 = ACT == 0 ? lse2[32 * sb + qi] : 0.f;
          const float de = ACT == 0 ? dlt[32 * sb + qi] : 0.f;
          p_ds<ACT>(s[r], dp[r], l2, de, a.scale, a.scale_log2, inv_lk, masked, p, ds);
          s[r] = p;
          dp[r] = ds;
        }
        // dV^T += dO^T P and dK^T += Q^T dS; k-step ss covers rows 16*ss .. +15 of the sub-block
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
          const frag_t<T> pf = pack_frag<T>(s, ss);
          const frag_t<T> sf = pack_frag<T>(dp, ss);
#pragma unroll
          for (int d2 = 0; d2 < C::ND; ++d2) {
            const frag_t<T> dof = lds_col_frag<T, D, true>(dt_, 32 * sb + 16 * ss, 32 * d2);
            mma(dv[d2], dof, pf);
            const frag_t<T> qtf = lds_col_frag<T, D, true>(qt, 32 * sb + 16 * ss, 32 * d2);
            mma(dk[d2], qtf, sf);
          }
        }
      }
    }
    if (it + 1 < nqb) lstore((it + 1) & 1);
    __syncthreads();
  }

  if (!wave_live || my_key >= lk) return;
  T* dkp = static_cast<T*>(a.dk) + (size_t)(ks + my_key) * rs + (size_t)h * D;
  T* dvp = static_cast<T*>(a.dv) + (size_t)(ks + my_key) * rs + (size_t)h * D;
  store_row<T, C::ND>(dkp, dk, a.scale);
  store_row<T, C::ND>(dvp, dv, 1.0f);
}

// ---------------------------------------------------------------- dQ

template <typename T, int D>
struct DqCfg {
  static constexpr int BM = kFwdBM, BN = kFwdBN, NT = 256;
  static constexpr int ES = sizeof(T);
  static constexpr int KT = Swz<T, D>::tile_bytes(BN);   // K / V tile
  static constexpr int STAGE = 2 * KT;
  static constexpr int LDS = 2 * STAGE;
  static constexpr int ND = D / 32, NK = D / 16;
};

template <typename T, int D, int ACT>
__global__ __launch_bounds__(256, (D >= 128 || sizeof(T) == 4) ? 1 : 2) void dq_kernel(BwdArgs a) {
  using C = DqCfg<T, D>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  if ((int)blockIdx.x >= *a.n_items_q) return;
  int b, h, t;
  unpack_item(a.items_q[blockIdx.x], b, h, t);
  const int qs = a.qo[b], lq = a.qo[b + 1] - qs;
  const int ks = a.ko[b], lk = a.ko[b + 1] - ks;
  const int off = lk - lq;

  const int tid = threadIdx.x, l = lane_id(), w = tid >> 6, g = l >> 5, c32 = l & 31;
  const int row0 = t * C::BM + 32 * w;
  const int my_row = row0 + c32;
  const bool wave_live = row0 < lq;
  const int n_kv = q_tile_kv_blocks(lq, lk, t, C::BM, C::BN, a.causal);
  const size_t rs = (size_t)a.heads * D;
  const float inv_lk = lk > 0 ? 1.0f / (float)lk : 0.f;

  frag_t<T> qf[C::NK], df[C::NK];
  float lse2 = 0.f, dlt = 0.f;
  {
    const int r = min(my_row, lq - 1);
    const T* qp = static_cast<const T*>(a.q) + (size_t)(qs + r) * rs + (size_t)h * D + 8 * g;
    const T* dp = static_cast<const T*>(a.dout) + (size_t)(qs + r) * rs + (size_t)h * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < C::NK; ++kk) {
      qf[kk] = global_frag<T>(qp + 16 * kk);
      df[kk] = global_frag<T>(dp + 16 * kk);
    }
    if (ACT == 0) {
      lse2 = lse_log2(a.lse[(size_t)h * a.total_q + qs + r]);
      dlt = a.delta[(size_t)h * a.total_q + qs + r];
    }
  }
  f32x16 dq[C::ND];
#pragma unroll
  for (int i = 0; i < C::ND; ++i) dq[i] = f32x16{};

  const T* kb = static_cast<const T*>(a.k) + (size_t)ks * rs + (size_t)h * D;
  const T* vb = static_cast<const T*>(a.v) + (size_t)ks * rs + (size_t)h * D;
  TileStage<T, D, C::BN, true> kst, vst;   // key rows stored swap23-permuted
  auto gload = [&](int kvt) {
    kst.load(kb, (int)rs, kvt * C::BN, lk, tid);
    vst.load(vb, (int)rs, kvt * C::BN, lk, tid);
  };
  auto lstore = [&](int buf) {
    char* st = smem + buf * C::STAGE;
    kst.store(st, tid);
    vst.store(st + C::KT, tid);
  };

  if (n_kv > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int it = 0; it < n_kv; ++it) {
    if (it + 1 < n_kv) gload(it + 1);
    const int kv0 = it * C::BN;
    const char* kt = smem + (it & 1) * C::STAGE;
    const char* vt = kt + C::KT;
    const bool active = wave_live && (!a.causal || kv0 <= row0 + 31 + off);
    if (active) {
      // S^T and dP^T (64 keys x 32 queries) as two 32-key tiles
      f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kk = 0; kk < C::NK; ++kk) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const frag_t<T> kfr = lds_row_frag<T, D>(kt, 32 * mt + c32, 16 * kk + 8 * g);
          mma(s[mt], kfr, qf[kk]);
          const frag_t<T> vfr = lds_row_frag<T, D>(vt, 32 * mt + c32, 16 * kk + 8 * g);
          mma(dp[mt], vfr, df[kk]);
        }
      }
      const bool need_mask = (kv0 + C::BN > lk) || (a.causal && kv0 + C::BN - 1 > row0 + off) || (row0 + 32 > lq);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kv0 + 32 * mt + 16 * (r >> 3) + 8 * g + (r & 7);
          bool masked = false;
          if (need_mask) masked = (j >= lk) || (my_row >= lq) || (a.causal && j > my_row + off);
          float p, ds;
          p_ds<ACT>(s[mt][r], dp[mt][r], lse2, dlt, a.scale, a.scale_log2, inv_lk, masked, p, ds);
          dp[mt][r] = ds;
        }
      }
      // dQ^T (D x 32 queries) += K^T dS^T
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
          const frag_t<T> sf = pack_frag<T>(dp[mt], ss);
#pragma unroll
          for (int d2 = 0; d2 < C::ND; ++d2) {
            const frag_t<T> ktf = lds_col_frag<T, D, true>(kt, 32 * mt + 16 * ss, 32 * d2);
            mma(dq[d2], ktf, sf);
          }
        }
      }
    }
    if (it + 1 < n_kv) lstore((it + 1) & 1);
    __syncthreads();
  }

  if (!wave_live || my_row >= lq) return;
  T* dqp = static_cast<T*>(a.dq) + (size_t)(qs + my_row) * rs + (size_t)h * D;
  store_row<T, C::ND>(dqp, dq, a.scale);
}

// ---------------------------------------------------------------- launchers

template <typename T>
static hipError_t pre_d(const BwdArgs& a, int head_dim, hipStream_t stream) {
  const int64_t pairs = (int64_t)a.total_q * a.heads;
  // (row, head) pairs per 256-thread block: 256 / (16-byte chunks per row)
  auto grid = [&](int D) {
    const int64_t per_block = 256 / (D * (int64_t)sizeof(T) / 16);
    return (unsigned)((pairs + per_block - 1) / per_block);
  };
  const T* o = static_cast<const T*>(a.out);
  const T* d = static_cast<const T*>(a.dout);
  switch (head_dim) {
    case 32: hipLaunchKernelGGL((bwd_pre_kernel<T, 32>), dim3(grid(32)), dim3(256), 0, stream, o, d, a.delta, a.heads, a.total_q); break;
    case 64: hipLaunchKernelGGL((bwd_pre_kernel<T, 64>), dim3(grid(64)), dim3(256), 0, stream, o, d, a.delta, a.heads, a.total_q); break;
    case 128: hipLaunchKernelGGL((bwd_pre_kernel<T, 128>), dim3(grid(128)), dim3(256), 0, stream, o, d, a.delta, a.heads, a.total_q); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bwd_pre(const BwdArgs& a, int head_dim, int dtype, hipStream_t stream) {
  if ((int64_t)a.total_q * a.heads == 0) return hipSuccess;
  return dtype == 0 ? pre_d<__bf16>(a, head_dim, stream) : pre_d<float>(a, head_dim, stream);
}

#define JFA_BWD_LAUNCHER(NAME, KERNEL)                                                                   \
  template <typename T, int ACT>                                                                         \
  static hipError_t NAME##_d(const BwdArgs& a, int head_dim, int64_t grid, hipStream_t stream) {         \
    switch (head_dim) {                                                                                  \
      case 32: hipLaunchKernelGGL((KERNEL<T, 32, ACT>), dim3((unsigned)grid), dim3(256), 0, stream, a); break;  \
      case 64: hipLaunchKernelGGL((KERNEL<T, 64, ACT>), dim3((unsigned)grid), dim3(256), 0, stream, a); break;  \
      case 128: hipLaunchKernelGGL((KERNEL<T, 128, ACT>), dim3((unsigned)grid), dim3(256), 0, stream, a); break; \
      default: return hipErrorInvalidValue;                                                              \
    }                                                                                                    \
    return hipGetLastError();                                                                            \
  }                                                                                                      \
  hipError_t launch_bwd_##NAME(const BwdArgs& a, int head_dim, int dtype, int act, int64_t grid,         \
                               hipStream_t stream) {                                                     \
    if (grid <= 0) return hipSuccess;                                                                    \
    if (dtype == 0) return act == 0 ? NAME##_d<__bf16, 0>(a, head_dim, grid, stream)                     \
                                    : NAME##_d<__bf16, 1>(a, head_dim, grid, stream);                    \
    return act == 0 ? NAME##_d<float, 0>(a, head_dim, grid, stream)                                      \
                    : NAME##_d<float, 1>(a, head_dim, grid, stream);                                     \
  }

JFA_BWD_LAUNCHER(dkdv, dkdv_kernel)
JFA_BWD_LAUNCHER(dq, dq_kernel)

}  // namespace jfa

// Jagged attention forward (softmax and GDPA/SiLU) for gfx950.
//
// Method: piletech.kr/articles/112134, section 상세 정리 (Detailed notes) --
// Jagged Flash Attention item (attention computed directly on the packed
// variable-length tensors, masking by subtraction instead of a -inf fill)
// and GDPA item (a non-softmax activation; here silu(s*q.k)/L_kv).
//
// One workgroup (4 waves) per work item = (sequence, head, 128-query tile),
// taken from the longest-first list the scheduler built.  Each wave owns 32
// query rows and keeps them in registers as the B operand of S^T = K Q^T, so
// that every lane ends up owning one query row (its column of S^T): the
// online-softmax statistics are per-lane scalars, reduced with a single
// permlane32 swap.  K and V tiles of 64 keys are copied from HBM straight
// into swizzled LDS tiles (buffer loads that write LDS, two slots each), and
// the loop is software-pipelined: the scores of the next key tile are
// computed on the matrix cores while the softmax of the current one runs on
// the vector ALUs.  V^T fragments come straight from the row-major V tile
// through ds_read_b64_tr_b16.  Ragged tails and the causal diagonal are
// masked arithmetically, only on the tiles that need it.
#include <type_traits>

#include "jfa_common.hpp"
#include "jfa_internal.h"

namespace jfa {

// SHORT: the variant for batches whose sequences all have at most 64
// queries and 64 keys (BlockAttention's runs).  Such an item has one key
// tile and fills only the first two waves' rows of its 128-row tile, so
// the variant runs those two waves with one K and one V slot: half the LDS
// and registers per item, twice the items in flight per CU, the same
// arithmetic per row.
template <typename T, int D, bool SHORT = false>
struct FwdCfg {
  static constexpr int BM = kFwdBM, BN = kFwdBN;
  static constexpr int NT = SHORT ? 128 : 256;
  static constexpr int KT = Swz<T, D>::tile_bytes(BN);   // one K or V tile
  static constexpr int SLOTS = SHORT ? 1 : 2;            // K slots, and as many V slots
  static constexpr int LDS = 2 * SLOTS * KT;
  static constexpr int ND = D / 32;                      // 32-wide d blocks of O^T
  static constexpr int NK = D / 16;                      // k-steps of S^T
  // waves per SIMD to fit (the second launch bound): two, i.e. two
  // workgroups per CU, or four of the two-wave SHORT variant
  static constexpr int WPS = (D >= 128 && sizeof(T) == 4) ? 1 : 2;
};

// ROPE (SHORT, bf16 only): BlockAttention's fused rotary embedding.  The
// lane's Q row is turned in its registers after the load, and the item's one
// K tile in LDS after it lands (one more barrier), positions counted from the
// sequence's first row.
template <typename T, int D, int ACT, bool SHORT, bool ROPE = false>
__global__ __launch_bounds__((FwdCfg<T, D, SHORT>::NT), (FwdCfg<T, D, SHORT>::WPS)) void fwd_kernel(FwdArgs a) {
  static_assert(!ROPE || (SHORT && sizeof(T) == 2), "the rotary embedding runs in the short-sequence bf16 variant");
  using C = FwdCfg<T, D, SHORT>;
  static_assert(C::NT / kWave * store_scratch_bytes<T, D>() <= C::LDS, "output staging must fit the LDS");
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  char* const kslot0 = smem;
  char* const vslot0 = smem + C::SLOTS * C::KT;

  ItemMeta m;
  if (SHORT && a.meta == nullptr) {
    // no work list: every item costs at most one key block, so the order
    // hardly matters; block b * heads + h takes sequence b, head h (offsets
    // outside the tensors, possible only when the offsets break their
    // contract, are left alone)
    const int b = (int)blockIdx.x / a.heads, hh = (int)blockIdx.x % a.heads;
    const int q0 = a.qo[b], q1 = a.qo[b + 1], k0 = a.ko[b], k1 = a.ko[b + 1];
    if (q0 < 0 || q1 <= q0 || q1 > a.total_q || k0 < 0 || k1 < k0 || k1 > a.total_kv) return;
    m = ItemMeta{q0, q1 - q0, k0, k1 - k0, hh, 0, b, 0};
  } else {
    m = a.meta[blockIdx.x];   // one load: offsets, lengths, head, tile
    if (m.lq < 0) return;     // past the item count
  }
  const int qs = m.qs, lq = m.lq, ks = m.ks, lk = m.lk, h = m.head, t = m.tile;
  const int off = lk - lq;   // causal: query i sees keys j <= i + off

  const int tid = threadIdx.x, l = lane_id(), w = tid >> 6, g = l >> 5, c32 = l & 31;
  const int row0 = t * C::BM + 32 * w;   // first query row of this wave
  const int my_row = row0 + c32;         // the query row this lane owns
  const bool wave_live = row0 < lq;
  const int n_kv = q_tile_kv_blocks(lq, lk, t, C::BM, C::BN, a.causal);
  const int rs = a.heads * D;            // elements between consecutive tokens
  // SHORT runs only where the host knows every length is at most 64; an
  // item that breaks that (lengths beyond the stated maxima) is left alone
  // rather than read past the one K and V slot
  if constexpr (SHORT)
    if (n_kv > 1 || lq > 2 * 32) return;

  const T* kb = static_cast<const T*>(a.k) + (size_t)ks * rs + (size_t)h * D;
  const T* vb = static_cast<const T*>(a.v) + (size_t)ks * rs + (size_t)h * D;

  // K rows are stored swap23-permuted, V rows in order (see the header note)
  TileDma<T, D, C::BN, true, C::NT> kdma;
  TileDma<T, D, C::BN, false, C::NT> vdma;
  kdma.init(rs, tid);
  vdma.init(rs, tid);

  // Prologue: K(0), V(0), K(1) into LDS while the Q fragments arrive.
  if (n_kv > 0) {
    kdma.issue(kslot0, kb, rs, 0, lk, tid);
    vdma.issue(vslot0, vb, rs, 0, lk, tid);
  }
  if (n_kv > 1) kdma.issue(kslot0 + C::KT, kb, rs, C::BN, lk, tid);

  frag_t<T> qf[C::NK];
  {
    const int r = min(my_row, lq - 1);
    const T* qp = static_cast<const T*>(a.q) + (size_t)(qs + r) * rs + (size_t)h * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < C::NK; ++kk) qf[kk] = global_frag<T>(qp + 16 * kk);
#pragma unroll
    for (int kk = 0; kk < C::NK; ++kk) settle(qf[kk]);
    if constexpr (ROPE) rope_frags<C::NK>(qf, my_row, a.rope.k2);
  }

  f32x16 o[C::ND];
#pragma unroll
  for (int i = 0; i < C::ND; ++i) o[i] = f32x16{};
  // running max, running sum of the exact weights (for lse) and of the
  // weights as rounded into the P operand (for normalising O)
  float m_run = -INFINITY, l_run = 0.f, l_used = 0.f;
  // silu weights: y = s * scale / L_kv * sigmoid(s * scale) for raw score s
  const float silu_out = lk > 0 ? a.scale / (float)lk : 0.f;
  const float silu_neg_l2 = -a.scale_log2;

  // lane address bases of the K row and V column fragment reads (bf16)
  [[maybe_unused]] const int k_addr = sizeof(T) == 2 ? RowFragAddr<T, D>::base() : 0;
  [[maybe_unused]] const int v_addr = sizeof(T) == 2 ? ColFragAddr<T, D, false>::base() : 0;

  // a wave takes part in key tile j iff some of its rows see a key of it
  auto wave_active = [&](int j) { return wave_live && (!a.causal || j * C::BN <= row0 + 31 + off); };

  // S^T (64 keys x 32 queries) = K Q^T for the key tile in K slot PAR
  // (the slot of key tile j is j & 1; a compile-time slot keeps the slot
  // offset in the reads' immediate field), as two 32-key tiles
  auto scores = [&](auto PAR, f32x16* s) {
    const char* kt = kslot0 + decltype(PAR)::value * C::KT;
    s[0] = f32x16{};
    s[1] = f32x16{};
    if constexpr (sizeof(T) == 2) {
      const int kx = refresh(k_addr);
#pragma unroll
      for (int kk = 0; kk < C::NK; ++kk) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) mma(s[mt], lds_row_frag_x<T, D>(kt, 32 * mt, kk, kx), qf[kk]);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < C::NK; ++kk) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) mma(s[mt], lds_row_frag<T, D>(kt, 32 * mt, c32, 16 * kk + 8 * g), qf[kk]);
      }
    }
  };

  // Keys of key tile j at or beyond `limit - kv0` are masked for this lane's
  // row (ragged tail and causal diagonal).  Register r of 32-key tile mt
  // holds key kv0 + 32*mt + 16*(r/8) + 8*g + r%8.
  const int row_limit = a.causal ? min(lk, my_row + off + 1) : lk;
  auto needs_mask = [&](int j) {
    const int kv0 = j * C::BN;
    return (kv0 + C::BN > lk) || (a.causal && kv0 + C::BN - 1 > row0 + off);
  };

  // Softmax weights of tile j in s (in place), with the S^T MFMAs of tile
  // j+1 (into s_nxt, when NEXT) interleaved with them, then
  // O^T += V^T P^T for tile j.  MASK: tile j needs masking.  Both flags are
  // compile-time so that the interleaved region has no branch.
  auto tile_step = [&](auto MASK, auto NEXT, auto PAR, f32x16* s, f32x16* s_nxt, int j) {
    constexpr bool kMask = decltype(MASK)::value;
    constexpr bool kNext = decltype(NEXT)::value;
    constexpr int kPar = decltype(PAR)::value;   // == j & 1
    const int lim = row_limit - j * C::BN - 8 * g;   // masked iff key offset >= lim
    if constexpr (ACT == 0) {
      if constexpr (kMask) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ko = 32 * mt + 16 * (r >> 3) + (r & 7);
            s[mt][r] -= (ko >= lim) ? kMaskShift : 0.f;
          }
        }
      }
      // row max of the raw scores (the scale is positive)
      float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s[0][r], s[1][r]));
      mx = xor32_max(mx) * a.scale_log2;
      // Rescale O and the sums only when the max grows by more than
      // kLazyRescale (log2 units); otherwise keep the stale max, so the
      // weights stay below 2^kLazyRescale.  Wave-uniform branch.
      const bool grow = mx > m_run + kLazyRescale;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        // a row whose keys are all masked so far takes a max near -1.3e29;
        // flooring it keeps its weights at exactly 0 (a live row's max is
        // a real score, far above the floor)
        const float m_use = grow ? fmaxf(mx, kMaxFloor) : m_run;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_use;
        l_run *= alpha;
        l_used *= alpha;
#pragma unroll
        for (int i = 0; i < C::ND; ++i) o[i] *= alpha;
      }
    }
    // --- straight-line region: next scores (MFMA) + weights (VALU) ---
    if constexpr (kNext) scores(std::integral_constant<int, 1 - kPar>{}, s_nxt);
    if constexpr (ACT == 0) {
      const float neg_m = -m_run;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s[mt][r], a.scale_log2, neg_m));
          l_run += p;
          s[mt][r] = p;
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float raw = s[mt][r];
          const float sig = fast_rcp(1.0f + fast_exp2(raw * silu_neg_l2));
          float y = raw * silu_out * sig;
          if constexpr (kMask) {
            const int ko = 32 * mt + 16 * (r >> 3) + (r & 7);
            y = (ko >= lim) ? 0.f : y;
          }
          s[mt][r] = y;
        }
      }
    }
    frag_t<T> pf[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) pf[mt][ss] = pack_frag<T>(s[mt], ss);
    }
    // --- P V for tile j ---
    if constexpr (ACT == 0) {
      // normalise by the sum of the weights the product really uses, so
      // that O stays a convex combination of V rows after P is rounded
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) frag_sum_into(l_used, pf[mt][ss]);
      }
    }
    const char* vt = vslot0 + kPar * C::KT;
    [[maybe_unused]] const int vx = refresh(v_addr);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
#pragma unroll
        for (int dt = 0; dt < C::ND; ++dt) {
          frag_t<T> vf;
          if constexpr (sizeof(T) == 2) vf = lds_col_frag_x<T, D, false>(vt, 32 * mt + 16 * ss, dt, vx);
          else vf = lds_col_frag<T, D, false>(vt, 32 * mt + 16 * ss, 32 * dt);
          mma(o[dt], vf, pf[mt][ss]);
        }
      }
    }
  };

  // One pipelined step for key tile j: start the copies of K(j+2) and
  // V(j+1), compute the scores of tile j+1 (MFMA) while the weights of tile
  // j are formed (VALU), accumulate P V for tile j, then wait and barrier.
  // Slot reuse: K(j+2) overwrites K(j), whose scores were formed in the
  // previous step; V(j+1) overwrites V(j-1), consumed in the previous step.
  auto step = [&](auto PAR, int j, f32x16* s_cur, f32x16* s_nxt) {
    constexpr int kPar = decltype(PAR)::value;   // == j & 1
    if (j + 2 < n_kv) kdma.issue(kslot0 + kPar * C::KT, kb, rs, (j + 2) * C::BN, lk, tid);
    if (j + 1 < n_kv) vdma.issue(vslot0 + (1 - kPar) * C::KT, vb, rs, (j + 1) * C::BN, lk, tid);
    const bool nxt = j + 1 < n_kv && wave_active(j + 1);
    if (wave_active(j)) {
      const bool msk = needs_mask(j);
      if (nxt) {
        if (msk) tile_step(std::true_type{}, std::true_type{}, PAR, s_cur, s_nxt, j);
        else tile_step(std::false_type{}, std::true_type{}, PAR, s_cur, s_nxt, j);
      } else {
        if (msk) tile_step(std::true_type{}, std::false_type{}, PAR, s_cur, s_nxt, j);
        else tile_step(std::false_type{}, std::false_type{}, PAR, s_cur, s_nxt, j);
      }
    } else if (nxt) {
      scores(std::integral_constant<int, 1 - kPar>{}, s_nxt);
    }
    dma_wait();
    __syncthreads();
  };

  dma_wait();
  __syncthreads();
  if constexpr (ROPE) {
    // the one K tile of a short item, turned in place (rows past the
    // sequence read as zeros and stay zeros)
    rope_lds_tile<D, true>(kslot0, C::BN, 0, a.rope.k2, tid, C::NT);
    __syncthreads();
  }
  f32x16 sa[2], sb[2];
  if (n_kv > 0 && wave_active(0)) scores(std::integral_constant<int, 0>{}, sa);
  // the first step copies K(2) over K(0): every wave must be done reading it
  __syncthreads();
  for (int j = 0; j < n_kv; j += 2) {
    step(std::integral_constant<int, 0>{}, j, sa, sb);
    if (j + 1 < n_kv) step(std::integral_constant<int, 1>{}, j + 1, sb, sa);
  }

  if (!wave_live) return;
  const float l_tot = ACT == 0 ? xor32_sum(l_run) : 1.f;
  const float l_out = ACT == 0 ? xor32_sum(l_used) : 1.f;
  const bool row_live = my_row < lq && lk > 0 && (!a.causal || my_row + off >= 0);
  float f = 0.f;
  if (row_live) f = ACT == 0 ? 1.0f / l_out : 1.0f;
  // every step ends with a barrier after its last LDS read: stage the rows there
  T* op = static_cast<T*>(a.out) + (size_t)(qs + row0) * rs + (size_t)h * D;
  store_rows_lds<T, D>(op, rs, min(32, lq - row0), o, f, smem + w * store_scratch_bytes<T, D>());
  if (ACT == 0 && g == 0 && my_row < lq) {
    a.lse[(size_t)h * a.total_q + qs + my_row] = row_live ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// Explicit instantiation of every variant (the host pass otherwise left some
// kernel stubs undefined).
#define JFA_FWD_INST(T, D, ACT)                                 \
  template __global__ void fwd_kernel<T, D, ACT, false>(FwdArgs); \
  template __global__ void fwd_kernel<T, D, ACT, true>(FwdArgs);
JFA_FWD_INST(__bf16, 32, 0) JFA_FWD_INST(__bf16, 64, 0) JFA_FWD_INST(__bf16, 128, 0)
JFA_FWD_INST(__bf16, 32, 1) JFA_FWD_INST(__bf16, 64, 1) JFA_FWD_INST(__bf16, 128, 1)
JFA_FWD_INST(float, 32, 0) JFA_FWD_INST(float, 64, 0) JFA_FWD_INST(float, 128, 0)
JFA_FWD_INST(float, 32, 1) JFA_FWD_INST(float, 64, 1) JFA_FWD_INST(float, 128, 1)
#undef JFA_FWD_INST
#define JFA_FWD_ROPE_INST(D, ACT) template __global__ void fwd_kernel<__bf16, D, ACT, true, true>(FwdArgs);
JFA_FWD_ROPE_INST(64, 0) JFA_FWD_ROPE_INST(128, 0) JFA_FWD_ROPE_INST(64, 1) JFA_FWD_ROPE_INST(128, 1)
#undef JFA_FWD_ROPE_INST

template <typename T, int D, int ACT>
static hipError_t launch_one(const FwdArgs& a, int64_t grid, bool short_batch, hipStream_t stream) {
  if (a.rope.on) {
    if constexpr (sizeof(T) == 2 && D >= 64) {
      if (!short_batch) return hipErrorInvalidValue;
      hipLaunchKernelGGL((fwd_kernel<T, D, ACT, true, true>), dim3((unsigned)grid), dim3(FwdCfg<T, D, true>::NT), 0,
                         stream, a);
      return hipGetLastError();
    }
    return hipErrorInvalidValue;
  }
  if (short_batch)
    hipLaunchKernelGGL((fwd_kernel<T, D, ACT, true>), dim3((unsigned)grid), dim3(FwdCfg<T, D, true>::NT), 0, stream,
                       a);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, ACT, false>), dim3((unsigned)grid), dim3(FwdCfg<T, D, false>::NT), 0,
                       stream, a);
  return hipGetLastError();
}

template <typename T, int ACT>
static hipError_t launch_d(const FwdArgs& a, int head_dim, int64_t grid, bool short_batch, hipStream_t stream) {
  switch (head_dim) {
    case 32: return launch_one<T, 32, ACT>(a, grid, short_batch, stream);
    case 64: return launch_one<T, 64, ACT>(a, grid, short_batch, stream);
    case 128: return launch_one<T, 128, ACT>(a, grid, short_batch, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdArgs& a, int head_dim, int dtype, int act, int64_t grid, bool short_batch,
                      hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (dtype == 0) return act == 0 ? launch_d<__bf16, 0>(a, head_dim, grid, short_batch, stream)
                                  : launch_d<__bf16, 1>(a, head_dim, grid, short_batch, stream);
  return act == 0 ? launch_d<float, 0>(a, head_dim, grid, short_batch, stream)
                  : launch_d<float, 1>(a, head_dim, grid, short_batch, stream);
}

}  // namespace jfa

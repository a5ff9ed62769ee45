// Jagged attention backward (softmax and GDPA/SiLU) for gfx950, without
// atomics (piletech.kr/articles/112134, section 상세 정리 / Detailed notes,
// Jagged Flash Attention item: the backward's parallel split uses no atomic
// operations).
//
// The gradient sums over queries (dK, dV) and over keys (dQ) are split into
// two passes so that every output row is owned by exactly one workgroup and
// stored once.  Launch order:
//   row statistics (softmax only) -- per (row, head): delta_i =
//     sum_c dO_ic O_ic, the row sum of P o dP that the softmax Jacobian
//     needs, and lse_i * log2(e) (bwd_stats.hpp; normally formed in the
//     spare workgroups of the work-list launch);
//   dK/dV pass -- one work item per (sequence, head, 64-key tile); each
//     pair of waves owns 32 keys and walks the query rows that see them in
//     32-row sub-blocks.  P and dS are recomputed from lse (softmax) or from
//     the scores (SiLU).  It also stores every dS block it forms (bf16 or
//     fp32, 32 queries x 32 keys), so that
//   dQ pass -- one work item per (sequence, head, 128-query tile) -- is the
//     single product dQ = scale * dS K over the stored blocks.  When the dS
//     blocks are not in the workspace, the dQ pass instead walks 64-query
//     tiles and recomputes S, P, dP and dS itself (three products instead
//     of one).
//
// Every pass streams the operand it walks (Q and dO, K and V, or K and dS)
// from HBM straight into a ring of swizzled LDS stages, two or more stages
// ahead of use (buffer loads that write LDS).
//
// Per (query i, key j) pair, with x = scale * q_i.k_j:
//   softmax: P = exp(x - lse_i);        dS = P (dP - delta_i)
//   silu:    P = silu(x) / Lk;          dS = dP silu'(x) / Lk,
//            silu'(x) = sig(x) (1 + x (1 - sig(x)))
//   dV_j += P dO_i,  dP = dO_i . V_j,  dK_j += scale dS q_i,  dQ_i += scale dS k_j
#include <type_traits>

#include "bwd_stats.hpp"
#include "jfa_common.hpp"
#include "jfa_internal.h"

namespace jfa {

// ---------------------------------------------------------------- shared math


// The 8 values of a fragment as floats (element e of the fragment -> v[e]).
__device__ __forceinline__ void frag_unpack(const bf16x8& f, float* v) {
  const u32x4 u = __builtin_bit_cast(u32x4, f);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(u[e] << 16);
    v[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
  }
}
__device__ __forceinline__ void frag_unpack(const f32x8& f, float* v) {
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = f[e];
}

// P and dS of one score, softmax (ACT 0) or silu (ACT 1); masked pairs give 0.
template <int ACT>
__device__ __forceinline__ void p_ds(float raw, float dp, float lse2, float delta, float scale, float scale_log2,
                                     float inv_lk, bool masked, float& p, float& ds) {
  if constexpr (ACT == 0) {
    const float e = fast_exp2(fmaf(raw, scale_log2, -lse2));
    p = masked ? 0.f : e;
    ds = p * (dp - delta);
  } else {
    const float x = raw * scale;
    const float sig = fast_rcp(1.0f + fast_exp2(-raw * scale_log2));
    const float keep = masked ? 0.f : inv_lk;
    p = x * sig * keep;
    ds = dp * sig * (1.0f + x * (1.0f - sig)) * keep;
  }
}

// Calls f(std::integral_constant<bool, A>, std::integral_constant<bool, B>):
// two runtime flags turned into compile-time ones, so that the code region
// they select is straight-line.
template <typename F>
__device__ __forceinline__ void with_flags(bool a, bool b, F&& f) {
  if (a) {
    if (b) f(std::true_type{}, std::true_type{});
    else f(std::true_type{}, std::false_type{});
  } else {
    if (b) f(std::false_type{}, std::true_type{});
    else f(std::false_type{}, std::false_type{});
  }
}

// Ring of LDS stages fed two stages ahead.  Stage s lives in slot s % 4.
// When stage s is opened (wait + barrier), every wave has finished with
// stage s-2 (the pipeline reads at most stages s-1 and s from then on), so
// its slot is refilled with stage s+2 right after the barrier.
constexpr int kStages = 4;

// Waits until stage s has landed while `ahead` (0..2) later stages, of
// N copies each per thread, may still be in flight.
template <int N>
__device__ __forceinline__ void wait_stage(int ahead) {
  if (ahead >= 2) dma_wait_all_but<2 * N>();
  else if (ahead == 1) dma_wait_all_but<N>();
  else dma_wait_all_but<0>();
}

// ---------------------------------------------------------------- row statistics

// Row statistics (softmax) as a kernel of its own: workgroup (x, y) covers
// head y of the rows of chunk x (the backward's work-list launch forms them
// in its spare workgroups instead whenever it builds both lists).
template <typename T, int D>
__global__ __launch_bounds__(256) void stats_kernel(StatsArgs a) {
  stats_block<T, D, 256>(a, blockIdx.x, blockIdx.y, threadIdx.x);
}

// One stored dS block: 32 x 32 values of a [key][query] tile in the LDS
// layout of 32-element rows (Swz<T, 32>), so that the dQ pass copies it into
// LDS unchanged and reads dS^T fragments with transposed LDS reads.
template <typename T>
struct DsTile {
  using S = Swz<T, kDsBlock>;
  static constexpr int BYTES = S::tile_bytes(kDsBlock);
};

// The 8 values of a fragment -- row r, columns c0 .. c0+7 (c0 a multiple
// of 8) -- stored into a dS block image, in HBM (GLOBAL) or in LDS.  The
// HBM stores are non-temporal: each block is read once, by the dQ pass, and
// should not displace the Q and dO rows that the dK/dV pass re-reads
// through the cache.
template <typename T, bool GLOBAL = true>
__device__ __forceinline__ void ds_store(char* blk, int r, int c0, const frag_t<T>& f) {
  using S = typename DsTile<T>::S;
  auto put = [](char* p, const u32x4& v) {
    if constexpr (GLOBAL) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
    else *reinterpret_cast<u32x4*>(p) = v;
  };
  if constexpr (sizeof(T) == 2) {
    put(blk + S::off(r, c0 >> 3), __builtin_bit_cast(u32x4, f));
  } else {
    put(blk + S::off(r, c0 >> 2), __builtin_bit_cast(u32x4, f32x4{f[0], f[1], f[2], f[3]}));
    put(blk + S::off(r, (c0 >> 2) + 1), __builtin_bit_cast(u32x4, f32x4{f[4], f[5], f[6], f[7]}));
  }
}

// ---------------------------------------------------------------- dK / dV

// Four waves per 64-key item: two pairs, each pair owning 32 keys.  Wave A of
// a pair forms S = Q K^T and P (masks applied) and accumulates dV^T += dO^T P;
// wave B forms dP = dO V^T, takes P from wave A through LDS, forms dS and
// accumulates dK^T += Q^T dS.  The matrix work splits evenly, nothing is
// computed twice, and a wave's registers (one of K or V, one accumulator
// set) and the item's LDS fit two workgroups per CU: one's vector work, LDS
// waits and prologue overlap the other's products.
//
// Per 32-row sub-block n there is one barrier.  Before it, A turns S(n) into
// P(n) and hands P over (the packed P fragments its own dV product uses, or
// for SiLU the derivative factor packed the same way) while B accumulates
// dK(n-1) and forms dP(n); after it, A accumulates dV(n) and already forms
// S(n+1), and B forms dS(n).  B's dK runs one sub-block behind so that both
// sides of the barrier carry MFMA work for both waves.
//
// A short sequence (short_sequence: at most 64 queries and 64 keys) is one
// item that sees all of the sequence's keys and queries, so with fuse_short
// set the item also forms dQ = scale dS K: wave B keeps its dS blocks in
// LDS instead of HBM, wave A puts the K rows it loaded there too, and after
// the loop the four waves take the (at most two) 32-query blocks of dQ, one
// half of d each, while they stage dK and dV.  The ring's slots 2 and 3 hold
// K and dS; a short sequence has at most two sub-blocks and never reaches
// them.
template <typename T, int D>
struct DkdvCfg {
  static constexpr int BN = kBwdBN;
  static constexpr int NPAIRS = BN / 32;                 // 32-key slices per item
  static constexpr int NT = NPAIRS * 2 * kWave;          // an A and a B wave per slice
  static constexpr int SR = 32;                          // query rows per stage = one sub-block
  static constexpr int QT = Swz<T, D>::tile_bytes(SR);   // Q or dO tile
  static constexpr int STATS = NT / kWave * 256;         // per wave: its 64 rows of lse2 or delta
  static constexpr int STAGE = 2 * QT + STATS;
  static constexpr int XSLOT = kWave * 2 * (int)sizeof(frag_t<T>);   // one hand-over: 2 fragments per lane
  static constexpr int XCH = NPAIRS * 2 * XSLOT;         // per pair, two slots
  // The B waves issue every copy of the ring (query rows stored
  // swap23-permuted): A's path is the longer one, and a burst of copies
  // right after the barrier stalls the waves that issue it.
  using Dma = TileDma<T, D, SR, true, NT / 2>;
  static constexpr int SINK = Dma::N * (NT / 2) > Dma::CHUNKS ? NT / 2 / kWave * 1024 : 0;
  static constexpr int NS = (4 * STAGE + XCH + SINK <= 80 * 1024) ? 4 : 3;   // stages in the ring
  static constexpr int LDS = NS * STAGE + XCH + SINK;
  static constexpr int ND = D / 32, NK = D / 16;
  static constexpr int DT = DsTile<T>::BYTES;            // one 32 x 32 dS block
  // short sequences: K rows (two query-tile images) and [query block][pair]
  // dS blocks in the slots past the first two
  static constexpr bool FUSE = sizeof(T) == 2 && NS >= 4 && (NS - 2) * STAGE >= 2 * QT + 2 * NPAIRS * DT;
};

// ROPE (short sequences, bf16, with the fused dQ): BlockAttention's fused
// rotary embedding.  Wave A turns its key row in registers, the item's Q
// stages (all of a short sequence's queries, landed in the prologue) are
// turned in LDS, dK is turned back in registers before its store, and the
// fused dQ is turned back through an fp32 exchange in LDS (the two halves
// of d that a rotation pairs belong to different waves).
template <typename T, int D, int ACT, bool DS, bool ROPE = false>
__global__ __launch_bounds__(256, 2) void dkdv_kernel(BwdArgs a) {
  using C = DkdvCfg<T, D>;
  static_assert(!ROPE || C::FUSE, "the rotary embedding runs with the fused dQ of short sequences");
  static_assert(C::NT / kWave * store_scratch_bytes<T, D>() <= C::LDS, "output staging must fit the LDS");
  using Dma = typename C::Dma;
  constexpr int NPS = 2 * Dma::N + (ACT == 0 ? 2 : 0);   // copies per B thread per stage
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  char* const xch = smem + C::NS * C::STAGE;
  char* const sink = xch + C::XCH;

  const ItemMeta m = a.meta_kv[blockIdx.x];   // one load: offsets, lengths, head, tile
  if (m.lq < 0) return;                       // past the item count
  const int qs = m.qs, lq = m.lq, ks = m.ks, lk = m.lk, h = m.head, t = m.tile;
  const int off = lk - lq;

  const int tid = threadIdx.x, l = lane_id(), w = tid >> 6, g = l >> 5, c32 = l & 31;
  // SiLU: roles alternate with the wave index (A: even waves, B: odd
  // ones).  The hardware places a workgroup's waves on the CU's four SIMDs
  // in a fixed order that starts one SIMD further for each new workgroup
  // on the CU (read from the waves' hardware ids on gfx950: 88 % of the
  // workgroup pairs resident together differ by one step), so the two
  // resident workgroups then put an A and a B wave on each SIMD; with A =
  // waves 0, 1 half the SIMDs hold two waves of one role.  SiLU's longer
  // weights phase (A) gains from the mix (dK/dV 990 -> 955 us on the
  // long-sequence batch); the softmax pass does not (equal or 1 % slower),
  // and keeps the halves.
  constexpr bool kAltRoles = ACT == 1;
  const int pair = kAltRoles ? w >> 1 : w % C::NPAIRS;
  const bool role_a = kAltRoles ? (w & 1) == 0 : w < C::NPAIRS;   // A: S, P, dV;  B: dP, dS, dK (and the dS store)
  const int kw0 = t * C::BN + 32 * pair;   // first key of this pair
  const int my_key = kw0 + c32;            // the key this lane owns (its column of S)
  const bool wave_live = kw0 < lk;
  const int nst = kv_tile_q_blocks(lq, lk, t, C::SR, C::BN, a.causal);
  const int q_first = kv_tile_first_q_block(lq, lk, t, C::SR, C::BN, a.causal) * C::SR;
  const int rs = a.heads * D;
  const float inv_lk = lk > 0 ? 1.0f / (float)lk : 0.f;
  bool fuse = false;   // uniform: this item also forms the sequence's dQ
  if constexpr (C::FUSE) fuse = a.fuse_short && short_sequence(lq, lk);
  char* const kq = smem + 2 * C::STAGE;   // fused: K rows 0-31, then 32-63
  char* const dsl = kq + 2 * C::QT;       // fused: dS blocks [query block][pair]
  // DS: this pair's dS block of sub-block 0; sub-block n is n block rows on
  [[maybe_unused]] char* ds_blk = nullptr;
  [[maybe_unused]] const int ds_row_bytes = a.ds_kb * DsTile<T>::BYTES;
  if constexpr (DS)
    ds_blk = static_cast<char*>(a.ds) +
             ((int64_t)h * a.ds_head_blocks + (int64_t)(qs / kDsBlock + m.seq + q_first / kDsBlock) * a.ds_kb +
              kw0 / kDsBlock) * DsTile<T>::BYTES;

  const T* qb = static_cast<const T*>(a.q) + (size_t)qs * rs + (size_t)h * D;
  const T* db = static_cast<const T*>(a.dout) + (size_t)qs * rs + (size_t)h * D;
  // A needs lse2 of the rows, B needs delta: B copies both, each into its
  // wave's private area of the stage
  const float* lse2_h = ACT == 0 ? a.lse2 + (size_t)h * a.total_q + qs : nullptr;
  const float* delta_h = ACT == 0 ? a.delta + (size_t)h * a.total_q + qs : nullptr;
  const int tid_b = kAltRoles ? pair * kWave + l : tid - C::NT / 2;   // B waves: 0 .. NT/2-1
  Dma dma;   // Q and dO tiles share the geometry, hence the offsets
  if (!role_a) dma.init(rs, tid_b);
  auto slot = [&](int s) { return smem + (s % C::NS) * C::STAGE; };
  auto issue_stage = [&](int s) {   // B waves only
    char* st = slot(s);
    const int r0 = q_first + s * C::SR;
    dma.issue(st, qb, rs, r0, lq, tid_b, sink);
    dma.issue(st + C::QT, db, rs, r0, lq, tid_b, sink);
    if constexpr (ACT == 0) {
      rows_dma(st + 2 * C::QT + w * 256, delta_h, r0, lq);         // this B wave's area
      rows_dma(st + 2 * C::QT + (kAltRoles ? w ^ 1 : w - C::NPAIRS) * 256, lse2_h, r0, lq);   // its pair's A wave's area
    }
  };

  // Prologue: stages 0 and 1, then this lane's key (A) or value (B) row as
  // B-operand fragments (d-slots 16*kk + 8*g + e); all of it lands before
  // the loop, and the rest of the ring is issued after the barrier.
  if (!role_a)
    for (int s = 0; s < min(2, nst); ++s) issue_stage(s);
  frag_t<T> xf[C::NK];
  {
    const int j = min(my_key, lk - 1);
    const T* xp = static_cast<const T*>(role_a ? a.k : a.v) + (size_t)(ks + j) * rs + (size_t)h * D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < C::NK; ++kk) xf[kk] = global_frag<T>(xp + 16 * kk);
#pragma unroll
    for (int kk = 0; kk < C::NK; ++kk) settle(xf[kk]);
    if constexpr (ROPE)
      if (role_a) rope_frags<C::NK>(xf, my_key, a.rope.k2);
  }
  if constexpr (C::FUSE) {
    // fused dQ: wave A's key row into LDS, at row swap23(key) of its pair's
    // 32-row image as the query-tile copies place rows (rows past lk repeat
    // row lk - 1; their dS is zero)
    if (fuse && role_a) {
      char* kt = kq + pair * C::QT;
#pragma unroll
      for (int kk = 0; kk < C::NK; ++kk)
        *reinterpret_cast<frag_t<T>*>(kt + Swz<T, D>::off(swap23(c32), 2 * kk + g)) = xf[kk];
    }
  }
  dma_wait();
  __syncthreads();
  if constexpr (ROPE) {
    // a short sequence's query rows are all in stages 0 and 1 by now: turn
    // them in place, stage s holding rows q_first + 32 s + swap23(r)
    for (int s = 0; s < min(2, nst); ++s) rope_lds_tile<D, true>(slot(s), C::SR, q_first + s * C::SR, a.rope.k2, tid, C::NT);
    __syncthreads();
  }
  if (!role_a)
    for (int s = 2; s <= C::NS - 2; ++s)
      if (s < nst) issue_stage(s);

  f32x16 acc[C::ND];   // dV^T (A) or dK^T (B): lane = key, registers = d
#pragma unroll
  for (int i = 0; i < C::ND; ++i) acc[i] = f32x16{};

  // S (A) or dP (B) of sub-block n: 32 queries x 32 keys; register r holds
  // query q_first + 32*n + 16*(r/8) + 8*g + r%8 of this lane's key
  auto products = [&](f32x16& x, const char* tile) {
    x = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::NK; ++kk) mma(x, lds_row_frag<T, D>(tile, 0, c32, 16 * kk + 8 * g), xf[kk]);
  };
  // hand-over slot of sub-block n: [fragment ss][lane]
  auto xslot = [&](int n) { return xch + (pair * 2 + (n & 1)) * C::XSLOT; };
  auto row_stats = [&](const char* st, float* v) {   // this wave's 16 rows of lse2 or delta
    const char* sp = st + 2 * C::QT + w * 256 + 8 * g * (int)sizeof(float);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 x4 = *reinterpret_cast<const f32x4*>(sp + (16 * (q4 >> 1) + 4 * (q4 & 1)) * (int)sizeof(float));
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * q4 + e] = x4[e];
    }
  };

  // Wave A, before the barrier of sub-block n: P(n) from S(n) in x (in place)
  // and its packed fragments pf; writes what B needs to the hand-over slot.
  frag_t<T> pf[2];
  auto a_weights = [&](auto MASK, f32x16& x, int n, const char* st) {
    constexpr bool kMask = decltype(MASK)::value;
    const int qa = q_first + 32 * n;
    const int lo = (a.causal ? my_key - off : 0) - qa - 8 * g;
    const int span = max((my_key < lk) ? (lq - qa - 8 * g) - lo : 0, 0);
    float l2[16];
    if constexpr (ACT == 0) row_stats(st, l2);
    f32x16 gfac;   // SiLU: silu'(x)/Lk
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 16 * (r >> 3) + (r & 7);
      bool masked = false;
      if constexpr (kMask) masked = (unsigned)(c - lo) >= (unsigned)span;
      if constexpr (ACT == 0) {
        const float p = fast_exp2(fmaf(x[r], a.scale_log2, -l2[r]));
        x[r] = masked ? 0.f : p;
      } else {
        const float xs = x[r] * a.scale;
        const float sig = fast_rcp(1.0f + fast_exp2(-x[r] * a.scale_log2));
        const float keep = masked ? 0.f : inv_lk;
        x[r] = xs * sig * keep;
        gfac[r] = sig * (1.0f + xs * (1.0f - sig)) * keep;
      }
    }
    char* xo = xslot(n) + l * (int)sizeof(frag_t<T>);
#pragma unroll
    for (int ss = 0; ss < 2; ++ss) {
      pf[ss] = pack_frag<T>(x, ss);
      *reinterpret_cast<frag_t<T>*>(xo + ss * kWave * (int)sizeof(frag_t<T>)) =
          ACT == 0 ? pf[ss] : pack_frag<T>(gfac, ss);
    }
  };

  // sub-blocks in which the keys kw .. kw+31 are seen by some row
  auto visible_of = [&](int n, int kw) {
    const int qa = q_first + 32 * n;
    return kw < lk && qa < lq && !(a.causal && qa + 31 + off < kw);
  };
  auto visible = [&](int n) { return visible_of(n, kw0); };
  auto needs_mask = [&](int n) {
    const int qa = q_first + 32 * n;
    return (qa + 32 > lq) || (kw0 + 32 > lk) || (a.causal && kw0 + 31 > qa + off);
  };

  // B, one sub-block behind: dK^T += Q^T dS(n) from the packed dS in sf and
  // stage n's Q rows (k-step ss covers rows 16*ss .. +15 of the sub-block)
  frag_t<T> sf[2];
  auto b_dk = [&](int n) {
    const char* qt = slot(n);
#pragma unroll
    for (int ss = 0; ss < 2; ++ss)
#pragma unroll
      for (int d2 = 0; d2 < C::ND; ++d2) mma(acc[d2], lds_col_frag<T, D, true>(qt, 16 * ss, 32 * d2), sf[ss]);
  };

  f32x16 x;   // A: S(n), then P(n);  B: dP(n), then dS(n)
  if (role_a && nst > 0 && visible(0)) products(x, slot(0));
  for (int n = 0; n < nst; ++n) {
    const char* st = slot(n);
    const char* dt = st + C::QT;
    const bool vis = visible(n);
    if (role_a) {
      if (vis) {
        if (needs_mask(n)) a_weights(std::true_type{}, x, n, st);
        else a_weights(std::false_type{}, x, n, st);
      }
    } else {
      // stage n-1 is refilled only after this sub-block's barrier
      if (n > 0 && visible(n - 1)) b_dk(n - 1);
      if (vis) products(x, dt);
    }
    // stage n+1 must have landed before the barrier (B issued it; A has no
    // copies in flight); later ones may be in flight
    if (!role_a && n + 1 < nst) wait_stage<NPS>(min(C::NS - 3, nst - 2 - n));
    // LDS only: a full barrier would also wait for every copy still meant to
    // be in flight and for B's dS stores (one counter covers them all)
    lds_barrier();
    // every wave is done with stage n-1: refill its slot
    if (!role_a && n + C::NS - 1 < nst) issue_stage(n + C::NS - 1);
    if (role_a) {
      // dV^T += dO^T P(n); k-step ss covers rows 16*ss .. +15 of the sub-block
      if (vis) {
#pragma unroll
        for (int ss = 0; ss < 2; ++ss)
#pragma unroll
          for (int d2 = 0; d2 < C::ND; ++d2) mma(acc[d2], lds_col_frag<T, D, true>(dt, 16 * ss, 32 * d2), pf[ss]);
      }
      // S(n+1), whose stage has landed (waited for before the barrier)
      if (n + 1 < nst && visible(n + 1)) products(x, slot(n + 1));
    } else if (vis) {
      float dl[16];
      if constexpr (ACT == 0) row_stats(st, dl);
      const char* xi = xslot(n) + l * (int)sizeof(frag_t<T>);
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const frag_t<T> ef = *reinterpret_cast<const frag_t<T>*>(xi + ss * kWave * (int)sizeof(frag_t<T>));
        float e8[8];
        frag_unpack(ef, e8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * ss + e;
          x[r] = ACT == 0 ? e8[e] * (x[r] - dl[r]) : x[r] * e8[e];   // dS
        }
      }
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) sf[ss] = pack_frag<T>(x, ss);
      // the dS the dK product uses, for dQ: this lane's key row, queries
      // 16*ss + 8*g .. +7 of the sub-block; in HBM for the dQ pass, or
      // (short sequence) in LDS for this workgroup's own dQ
      if (fuse) {
        char* blk = dsl + ((q_first / 32 + n) * C::NPAIRS + pair) * C::DT;
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) ds_store<T, false>(blk, c32, 16 * ss + 8 * g, sf[ss]);
      } else if constexpr (DS) {
        char* blk = ds_blk + (int64_t)n * ds_row_bytes;
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) ds_store<T>(blk, c32, 16 * ss + 8 * g, sf[ss]);
      }
    }
  }
  // the last sub-block's dK (its stage is never refilled)
  if (!role_a && nst > 0 && visible(nst - 1)) b_dk(nst - 1);

  // the ring is free once every wave is past the loop: stage the rows there
  __syncthreads();
  auto store_dkdv = [&]() {
    if constexpr (ROPE)
      if (!role_a) rope_acc_inverse<C::ND>(acc, my_key, a.rope.k2);   // dK of the turned keys, turned back
    T* op = static_cast<T*>(role_a ? a.dv : a.dk) + (size_t)(ks + kw0) * rs + (size_t)h * D;
    store_rows_lds<T, D>(op, rs, min(32, lk - kw0), acc, role_a ? 1.0f : a.scale,
                         smem + w * store_scratch_bytes<T, D>());
  };
  if constexpr (C::FUSE) {
    if (fuse) {
      // dQ^T = K^T dS^T, one wave per (query block qb, half of d); a short
      // sequence has at most two query blocks.  The sum runs over the key
      // blocks whose dS block wave B wrote (the pairs that saw sub-block
      // qb - q_first/32); rows that see no key get zeros.
      constexpr int NDH = C::ND / 2;
      const int qb = w & 1, half = w >> 1, qa = 32 * qb, n = qb - q_first / 32;
      const bool q_live = qa < lq;
      f32x16 accq[NDH];
#pragma unroll
      for (int i = 0; i < NDH; ++i) accq[i] = f32x16{};
      if (q_live && n >= 0) {
#pragma unroll
        for (int p = 0; p < C::NPAIRS; ++p) {
          if (!visible_of(n, 32 * p)) continue;
          const char* dt = dsl + (qb * C::NPAIRS + p) * C::DT;
          const char* kt = kq + p * C::QT;
#pragma unroll
          for (int ss = 0; ss < 2; ++ss) {
            const frag_t<T> sq = lds_col_frag<T, kDsBlock, false>(dt, 16 * ss, 0);
#pragma unroll
            for (int j = 0; j < NDH; ++j)
              mma(accq[j], lds_col_frag<T, D, true>(kt, 16 * ss, 32 * (half * NDH + j)), sq);
          }
        }
      }
      // dK and dV are staged in slots 0 and 1 while other waves may still
      // read slots 2 and 3
      static_assert(C::NT / kWave * store_scratch_bytes<T, D>() <= 2 * C::STAGE, "dK/dV staging must fit slots 0-1");
      static_assert(C::NT / kWave * store_scratch_bytes<T, D / 2>() <= (C::NS - 2) * C::STAGE,
                    "dQ staging must fit the slots past the first two");
      if (wave_live) store_dkdv();
      __syncthreads();   // K rows and dS blocks read: their LDS stages dQ
      char* dq_scratch = kq + w * store_scratch_bytes<T, D / 2>();
      if constexpr (ROPE) {
        // dQ of the turned queries, turned back: each wave puts its half of d
        // of its query block into an fp32 exchange over the K rows and dS
        // blocks (read by now), then takes its partner's half.  The dK/dV
        // staging in slots 0 and 1 is free after the barrier above, and
        // stages dQ instead.
        static_assert(2 * 32 * D * (int)sizeof(float) <= (C::NS - 2) * C::STAGE, "dQ exchange must fit");
        static_assert(C::NT / kWave * store_scratch_bytes<T, D / 2>() <= 2 * C::STAGE, "dQ staging must fit");
        float* x = reinterpret_cast<float*>(kq) + qb * 32 * D;
        auto col = [&](int j, int r) { return 32 * (half * NDH + j) + 8 * (r / 4) + 4 * g + r % 4; };
        if (q_live) {
#pragma unroll
          for (int j = 0; j < NDH; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) x[c32 * D + col(j, r)] = accq[j][r];
        }
        __syncthreads();
        if (q_live) {
#pragma unroll
          for (int j = 0; j < NDH; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int d = col(j, r), i = d % (D / 2);
              const float other = x[c32 * D + (half ? d - D / 2 : d + D / 2)];
              float lo = half ? other : accq[j][r], hi = half ? accq[j][r] : other;
              const float rev = __builtin_amdgcn_exp2f((float)i * a.rope.k2) * 0.15915494309189535f;
              rope_rotate(lo, hi, (float)(qa + c32) * rev, true);
              accq[j][r] = half ? hi : lo;
            }
        }
        dq_scratch = smem + w * store_scratch_bytes<T, D / 2>();
      }
      if (q_live)
        store_rows_lds<T, D / 2>(static_cast<T*>(a.dq) + (size_t)(qs + qa) * rs + (size_t)h * D + half * (D / 2), rs,
                                 min(32, lq - qa), accq, a.scale, dq_scratch);
      return;
    }
  }
  if (wave_live) store_dkdv();
}

// ---------------------------------------------------------------- dQ

// Four waves per 64-query item: two pairs, each owning 32 queries.  Wave A
// of a pair forms S^T = K Q^T for 32-key sub-block n and from it P (softmax)
// or silu'(x)/Lk (SiLU), which it hands over through LDS; wave B runs one
// sub-block behind: it forms dS^T of sub-block n-1 from its own
// dP^T = V dO^T and the handed-over values, accumulates dQ^T += K^T dS^T,
// then forms dP^T of sub-block n.  A's exponentials overlap B's products on
// the same SIMD; one barrier per sub-block.  Every lane owns one query, so
// lse and delta (from the row statistics kernel) are per-lane scalars.
// This is the dQ pass used when the dS blocks are not stored.
template <typename T, int D>
struct DqCfg {
  static constexpr int BM = kDqBM;
  static constexpr int NPAIRS = BM / 32;
  static constexpr int NT = NPAIRS * 2 * kWave;
  static constexpr int SR = 32;                          // key rows per stage = one sub-block
  static constexpr int KT = Swz<T, D>::tile_bytes(SR);   // K or V tile
  static constexpr int STAGE = 2 * KT;
  static constexpr int XCH = NPAIRS * 2 * 4096;          // per pair: two 32 x 32 fp32 hand-over slots
  using Dma = TileDma<T, D, SR, true, NT>;               // key rows stored swap23-permuted
  static constexpr int SINK = Dma::N * NT > Dma::CHUNKS ? NT / kWave * 1024 : 0;
  static constexpr int NS = (4 * STAGE + XCH + SINK <= 80 * 1024) ? 4 : 3;   // two workgroups per CU
  static constexpr int LDS = NS * STAGE + XCH + SINK;
  static constexpr int ND = D / 32, NK = D / 16;
};

template <typename T, int D, int ACT>
__global__ __launch_bounds__(256, 2) void dq_kernel(BwdArgs a) {
  using C = DqCfg<T, D>;
  static_assert(C::NT / kWave * store_scratch_bytes<T, D>() <= C::LDS, "output staging must fit the LDS");
  using Dma = typename C::Dma;
  constexpr int NPS = 2 * Dma::N;   // copies per thread per stage
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  char* const xch = smem + C::NS * C::STAGE;
  char* const sink = xch + C::XCH;

  const ItemMeta m = a.meta_q[blockIdx.x];   // one load: offsets, lengths, head, tile
  if (m.lq < 0) return;                       // past the item count
  if (a.fuse_short && short_sequence(m.lq, m.lk)) return;   // dQ written by the dK/dV pass
  const int qs = m.qs, lq = m.lq, ks = m.ks, lk = m.lk, h = m.head, t = m.tile;
  const int off = lk - lq;

  const int tid = threadIdx.x, l = lane_id(), w = tid >> 6, g = l >> 5, c32 = l & 31;
  const int pair = w % C::NPAIRS;
  const bool role_a = w < C::NPAIRS;         // A: S, P;  B: dP, dS, dQ
  const int row0 = t * C::BM + 32 * pair;    // first query of this pair
  const int my_row = row0 + c32;             // the query this lane owns
  const bool wave_live = row0 < lq;
  const int nst = q_tile_kv_blocks(lq, lk, t, C::BM, C::SR, a.causal);
  const int rs = a.heads * D;
  const float inv_lk = lk > 0 ? 1.0f / (float)lk : 0.f;

  const T* kb = static_cast<const T*>(a.k) + (size_t)ks * rs + (size_t)h * D;
  const T* vb = static_cast<const T*>(a.v) + (size_t)ks * rs + (size_t)h * D;
  Dma dma;   // K and V tiles share the geometry
  dma.init(rs, tid);
  auto slot = [&](int s) { return smem + (s % C::NS) * C::STAGE; };
  auto issue_stage = [&](int s) {
    char* st = slot(s);
    dma.issue(st, kb, rs, s * C::SR, lk, tid, sink);
    dma.issue(st + C::KT, vb, rs, s * C::SR, lk, tid, sink);
  };

  // Prologue: stages 0 and 1, then this lane's query (A) or output-gradient
  // (B) row and its statistic; all of it lands before the loop.
  for (int s = 0; s < min(2, nst); ++s) issue_stage(s);
  frag_t<T> xf[C::NK];
  float stat = 0.f;   // A: lse2;  B: delta
  {
    const int r = min(my_row, lq - 1);
    const size_t ro = (size_t)(qs + r) * rs + (size_t)h * D + 8 * g;
    const T* xp = static_cast<const T*>(role_a ? a.q : a.dout) + ro;
#pragma unroll
    for (int kk = 0; kk < C::NK; ++kk) xf[kk] = global_frag<T>(xp + 16 * kk);
    if (ACT == 0) stat = (role_a ? a.lse2 : a.delta)[(size_t)h * a.total_q + qs + r];
#pragma unroll
    for (int kk = 0; kk < C::NK; ++kk) settle(xf[kk]);
    settle(stat);
  }
  dma_wait();
  __syncthreads();
  for (int s = 2; s <= C::NS - 2; ++s)
    if (s < nst) issue_stage(s);

  f32x16 dq[C::ND];   // B: dQ^T (d x queries), lane = query
#pragma unroll
  for (int i = 0; i < C::ND; ++i) dq[i] = f32x16{};

  // S^T (A) or dP^T (B) of sub-block n: 32 keys x 32 queries; register r
  // holds key 32*n + 16*(r/8) + 8*g + r%8 of this lane's query
  auto products = [&](f32x16& x, const char* tile) {
    x = f32x16{};
#pragma unroll
    for (int kk = 0; kk < C::NK; ++kk) mma(x, lds_row_frag<T, D>(tile, 0, c32, 16 * kk + 8 * g), xf[kk]);
  };
  // hand-over slot of sub-block n: [r/4][lane][4] floats
  auto xslot = [&](int n) { return xch + (pair * 2 + (n & 1)) * 4096; };
  auto visible = [&](int n) { return wave_live && (!a.causal || 32 * n <= row0 + 31 + off); };
  auto needs_mask = [&](int n) {
    return (32 * n + 32 > lk) || (a.causal && 32 * n + 31 > row0 + off) || (row0 + 32 > lq);
  };
  // keys at offset >= this (relative to the sub-block's first key + 8*g) are masked
  const int key_end = my_row < lq ? min(lk, a.causal ? my_row + off + 1 : lk) - 8 * g : -(1 << 30);

  // Wave A: the value B needs for sub-block n, written to its hand-over slot
  auto a_weights = [&](auto MASK, f32x16& x, int n) {
    constexpr bool kMask = decltype(MASK)::value;
    const int lim = key_end - 32 * n;
    f32x16 e_out;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 16 * (r >> 3) + (r & 7);
      bool masked = false;
      if constexpr (kMask) masked = c >= lim;
      if constexpr (ACT == 0) {
        const float p = fast_exp2(fmaf(x[r], a.scale_log2, -stat));
        e_out[r] = masked ? 0.f : p;
      } else {
        const float xs = x[r] * a.scale;
        const float sig = fast_rcp(1.0f + fast_exp2(-x[r] * a.scale_log2));
        const float keep = masked ? 0.f : inv_lk;
        e_out[r] = sig * (1.0f + xs * (1.0f - sig)) * keep;
      }
    }
    char* xo = xslot(n) + l * 16;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 v = {e_out[4 * q4], e_out[4 * q4 + 1], e_out[4 * q4 + 2], e_out[4 * q4 + 3]};
      *reinterpret_cast<f32x4*>(xo + q4 * 1024) = v;
    }
  };

  f32x16 dp_prev;             // B: dP^T of the previous sub-block
  bool prev_visible = false;
  for (int n = 0; n <= nst; ++n) {
    const bool cur = n < nst && visible(n);
    if (role_a) {
      if (cur) {
        f32x16 x;
        products(x, slot(n));   // K rows of stage n
        if (needs_mask(n)) a_weights(std::true_type{}, x, n);
        else a_weights(std::false_type{}, x, n);
      }
    } else {
      if (prev_visible) {
        // dS^T of sub-block n-1, then dQ^T += K^T dS^T; k-step ss covers keys 16*ss .. +15
        const char* xi = xslot(n - 1) + l * 16;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 e4 = *reinterpret_cast<const f32x4*>(xi + q4 * 1024);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * q4 + e;
            dp_prev[r] = ACT == 0 ? e4[e] * (dp_prev[r] - stat) : dp_prev[r] * e4[e];
          }
        }
        const char* kt = slot(n - 1);
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
          const frag_t<T> sf = pack_frag<T>(dp_prev, ss);
#pragma unroll
          for (int d2 = 0; d2 < C::ND; ++d2) mma(dq[d2], lds_col_frag<T, D, true>(kt, 16 * ss, 32 * d2), sf);
        }
      }
      if (cur) products(dp_prev, slot(n) + C::KT);   // V rows of stage n
    }
    prev_visible = cur;
    // stage n+1 must have landed before the barrier; later ones may be in flight
    if (n + 1 < nst) wait_stage<NPS>(min(C::NS - 3, nst - 2 - n));
    __syncthreads();
    // every wave is done with stage n-1: refill its slot
    if (n + C::NS - 1 < nst) issue_stage(n + C::NS - 1);
  }

  // the loop's last barrier follows every wave's last LDS read: stage the rows there
  if (role_a || !wave_live) return;
  T* dqp = static_cast<T*>(a.dq) + (size_t)(qs + row0) * rs + (size_t)h * D;
  store_rows_lds<T, D>(dqp, rs, min(32, lq - row0), dq, a.scale, smem + w * store_scratch_bytes<T, D>());
}


// dQ from the stored dS blocks: dQ^T = scale * K^T dS^T, one product per
// (query, key) pair instead of three.  One workgroup per BM-query item
// (BM = 128: the forward's tiles; BM = 256 when no sequence is much longer
// than the average, so that each K row is fetched once per 256 queries):
// wave w owns query block w (32 queries) and every d-block.  Each stage of
// the LDS ring holds 32 key rows and the item's BM / 32 dS blocks of those
// keys, copied unchanged from HBM; K^T and dS^T fragments both come from
// transposed LDS reads (rows = keys).  A dS block is read only where the
// dK/dV pass wrote it: query blocks that see some key of the key block.
template <typename T, int D, int BM_>
struct DqDsCfg {
  static constexpr int BM = BM_;                         // queries per item
  static constexpr int NQB = BM / kDsBlock;              // dS blocks per stage = waves
  static constexpr int SR = kDsBlock;                    // key rows per stage
  static constexpr int NT = NQB * kWave;
  static constexpr int KT = Swz<T, D>::tile_bytes(SR);   // K tile
  static constexpr int DT = DsTile<T>::BYTES;            // one dS block
  static constexpr int STAGE = KT + NQB * DT;
  using Dma = TileDma<T, D, SR, false, NT>;              // key rows in order
  static constexpr int NDS = NQB * DT / 16 / NT;         // dS copies per thread per stage
  static_assert(NQB * DT % (16 * NT) == 0 && (DT / 16) % kWave == 0, "dS copies must split by whole waves");
  static constexpr int SINK = Dma::N * NT > Dma::CHUNKS ? NT / kWave * 1024 : 0;
  static constexpr int NS = 4 * STAGE + SINK <= 80 * 1024 ? 4 : 3;   // two stages in flight where it fits
  static constexpr int LDS = NS * STAGE + SINK;
  static constexpr int ND = D / 32;
  static constexpr int WGS = LDS <= 52 * 1024 ? 3 : LDS <= 80 * 1024 ? 2 : 1;   // workgroups per CU
};

// Waits until stage s has landed in a ring of NS stages whose later stages
// (up to NS - 2 of them, N copies each per thread) may still be in flight.
template <int N, int NS>
__device__ __forceinline__ void wait_ring(int ahead) {
  if constexpr (NS >= 4) {
    wait_stage<N>(ahead);
  } else {
    if (ahead >= 1) dma_wait_all_but<N>();
    else dma_wait_all_but<0>();
  }
}

template <typename T, int D, int BM>
__global__ __launch_bounds__((DqDsCfg<T, D, BM>::NT), (DqDsCfg<T, D, BM>::WGS)) void dq_ds_kernel(BwdArgs a) {
  using C = DqDsCfg<T, D, BM>;
  static_assert(C::NQB * store_scratch_bytes<T, D>() <= C::LDS, "output staging must fit the LDS");
  using Dma = typename C::Dma;
  constexpr int NPS = Dma::N + C::NDS;   // copies per thread per stage
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  char* const sink = smem + C::NS * C::STAGE;

  const ItemMeta m = a.meta_q[blockIdx.x];   // one load: offsets, lengths, head, tile, sequence
  if (m.lq < 0) return;                       // past the item count
  if (a.fuse_short && short_sequence(m.lq, m.lk)) return;   // dQ written by the dK/dV pass
  const int qs = m.qs, lq = m.lq, ks = m.ks, lk = m.lk, h = m.head, t = m.tile;
  const int off = lk - lq;

  const int tid = threadIdx.x, w = tid >> 6;
  const int row0 = t * C::BM + kDsBlock * w;   // first query of this wave
  const bool wave_live = row0 < lq;
  const int nst = q_tile_kv_blocks(lq, lk, t, C::BM, C::SR, a.causal);
  const int rs = a.heads * D;

  // query block qb of the item sees key block n (so its dS block exists)
  auto sees = [&](int qb, int n) {
    const int r0 = t * C::BM + kDsBlock * qb;
    return r0 < lq && (!a.causal || kDsBlock * n <= r0 + kDsBlock - 1 + off);
  };
  const T* kb = static_cast<const T*>(a.k) + (size_t)ks * rs + (size_t)h * D;
  // dS block row of the item's first query block; a block row is ds_kb blocks
  const char* ds0 = static_cast<const char*>(a.ds) +
                    ((int64_t)h * a.ds_head_blocks + (int64_t)(qs / kDsBlock + m.seq + t * C::NQB) * a.ds_kb) * C::DT;
  Dma dma;
  dma.init(rs, tid);
  auto slot = [&](int s) { return smem + (s % C::NS) * C::STAGE; };
  auto issue_stage = [&](int s) {
    char* st = slot(s);
    dma.issue(st, kb, rs, s * C::SR, lk, tid, sink);
#pragma unroll
    for (int i = 0; i < C::NDS; ++i) {
      const int pw = i * C::NT + kWave * w;    // this wave's first chunk of the stage's dS blocks
      const int qb = pw / (C::DT / 16), ch = pw % (C::DT / 16);
      const char* blk = ds0 + ((int64_t)qb * a.ds_kb + s) * C::DT;
      // blocks the dK/dV pass did not write are never read: zeros instead.
      // Non-temporal copies: every dS block is read exactly once
      buffer_load_lds16<true>(uniform_rsrc(blk, sees(qb, s) ? C::DT : 0), (ch + lane_id()) * 16, st + C::KT + pw * 16);
    }
  };

  for (int s = 0; s < min(2, nst); ++s) issue_stage(s);
  dma_wait();
  __syncthreads();
  for (int s = 2; s <= C::NS - 2; ++s)
    if (s < nst) issue_stage(s);

  f32x16 acc[C::ND];   // dQ^T (d x queries) of this wave's queries, lane = query
#pragma unroll
  for (int i = 0; i < C::ND; ++i) acc[i] = f32x16{};

  for (int n = 0; n < nst; ++n) {
    if (sees(w, n)) {
      const char* kt = slot(n);
      const char* dt = kt + C::KT + w * C::DT;
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
        const frag_t<T> sf = lds_col_frag<T, kDsBlock, false>(dt, 16 * ss, 0);
#pragma unroll
        for (int j = 0; j < C::ND; ++j) mma(acc[j], lds_col_frag<T, D, false>(kt, 16 * ss, 32 * j), sf);
      }
    }
    // stage n+1 must have landed before the barrier; later ones may be in flight
    if (n + 1 < nst) wait_ring<NPS, C::NS>(min(C::NS - 3, nst - 2 - n));
    __syncthreads();
    // every wave is done with stage n-1: refill its slot
    if (n + C::NS - 1 < nst) issue_stage(n + C::NS - 1);
  }

  // the loop's last barrier follows every wave's last LDS read (and with no
  // stage at all, the prologue's barrier): stage the rows there
  if (!wave_live) return;
  T* dqp = static_cast<T*>(a.dq) + (size_t)(qs + row0) * rs + (size_t)h * D;
  store_rows_lds<T, D>(dqp, rs, min(32, lq - row0), acc, a.scale, smem + w * store_scratch_bytes<T, D>());
}

#define JFA_BWD_INST(T, D, ACT)                                      \
  template __global__ void dkdv_kernel<T, D, ACT, false>(BwdArgs);   \
  template __global__ void dkdv_kernel<T, D, ACT, true>(BwdArgs);    \
  template __global__ void dq_kernel<T, D, ACT>(BwdArgs);
JFA_BWD_INST(__bf16, 32, 0) JFA_BWD_INST(__bf16, 64, 0) JFA_BWD_INST(__bf16, 128, 0)
JFA_BWD_INST(__bf16, 32, 1) JFA_BWD_INST(__bf16, 64, 1) JFA_BWD_INST(__bf16, 128, 1)
JFA_BWD_INST(float, 32, 0) JFA_BWD_INST(float, 64, 0) JFA_BWD_INST(float, 128, 0)
JFA_BWD_INST(float, 32, 1) JFA_BWD_INST(float, 64, 1) JFA_BWD_INST(float, 128, 1)
#undef JFA_BWD_INST
#define JFA_BWD_INST2(T, D)                                          \
  template __global__ void stats_kernel<T, D>(StatsArgs);            \
  template __global__ void dq_ds_kernel<T, D, 128>(BwdArgs);         \
  template __global__ void dq_ds_kernel<T, D, kDqDsBM>(BwdArgs);
JFA_BWD_INST2(__bf16, 32) JFA_BWD_INST2(__bf16, 64) JFA_BWD_INST2(__bf16, 128)
JFA_BWD_INST2(float, 32) JFA_BWD_INST2(float, 64) JFA_BWD_INST2(float, 128)
#undef JFA_BWD_INST2
#define JFA_BWD_ROPE_INST(D, ACT) template __global__ void dkdv_kernel<__bf16, D, ACT, false, true>(BwdArgs);
JFA_BWD_ROPE_INST(64, 0) JFA_BWD_ROPE_INST(128, 0) JFA_BWD_ROPE_INST(64, 1) JFA_BWD_ROPE_INST(128, 1)
#undef JFA_BWD_ROPE_INST

// ---------------------------------------------------------------- launchers

template <typename K>
static hipError_t launch_k(K kernel, const BwdArgs& a, int64_t grid, hipStream_t stream, int threads = 256) {
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

// kernel variant for (dtype, head_dim): pick(dtype 0 = bf16 / 1 = fp32, D)
#define JFA_PICK_D(EXPR_T_D)                                      \
  switch (head_dim) {                                             \
    case 32: { constexpr int D = 32; EXPR_T_D; }                  \
    case 64: { constexpr int D = 64; EXPR_T_D; }                  \
    case 128: { constexpr int D = 128; EXPR_T_D; }                \
  }                                                               \
  return hipErrorInvalidValue;

bool dkdv_fuses_short(int dtype, int head_dim) {
  auto pick = [&](auto tag) -> bool {
    using T = decltype(tag);
    switch (head_dim) {
      case 32: return DkdvCfg<T, 32>::FUSE;
      case 64: return DkdvCfg<T, 64>::FUSE;
      case 128: return DkdvCfg<T, 128>::FUSE;
    }
    return false;
  };
  return dtype == 0 ? pick(__bf16{}) : pick(float{});
}

template <typename T, int ACT>
static hipError_t dkdv_d(const BwdArgs& a, int head_dim, int64_t grid, hipStream_t stream) {
  if (a.rope.on) {   // short sequences with the fused dQ only (bf16, d 64 or 128)
    if (!a.fuse_short || sizeof(T) != 2) return hipErrorInvalidValue;
    if (head_dim == 64) return launch_k(dkdv_kernel<__bf16, 64, ACT, false, true>, a, grid, stream);
    if (head_dim == 128) return launch_k(dkdv_kernel<__bf16, 128, ACT, false, true>, a, grid, stream);
    return hipErrorInvalidValue;
  }
  const bool ds = a.ds != nullptr;
  JFA_PICK_D(return launch_k(ds ? dkdv_kernel<T, D, ACT, true> : dkdv_kernel<T, D, ACT, false>, a, grid, stream))
}
template <typename T, int ACT>
static hipError_t dq_d(const BwdArgs& a, int head_dim, int64_t grid, hipStream_t stream) {
  if (a.ds != nullptr) {
    if (a.dq_rows == kDqDsBM) {
      JFA_PICK_D(return launch_k(dq_ds_kernel<T, D, kDqDsBM>, a, grid, stream, DqDsCfg<T, D, kDqDsBM>::NT))
    }
    JFA_PICK_D(return launch_k(dq_ds_kernel<T, D, 128>, a, grid, stream, DqDsCfg<T, D, 128>::NT))
  }
  JFA_PICK_D(return launch_k(dq_kernel<T, D, ACT>, a, grid, stream))
}
template <typename T>
static hipError_t stats_d(const StatsArgs& a, int head_dim, hipStream_t stream) {
  JFA_PICK_D({
    const int gx = (a.total_q + (StatsCfg<T, D, 256>::ROWS) - 1) / (StatsCfg<T, D, 256>::ROWS);
    if (gx <= 0) return hipSuccess;
    hipLaunchKernelGGL((stats_kernel<T, D>), dim3((unsigned)gx, (unsigned)a.heads), dim3(256), 0, stream, a);
    return hipGetLastError();
  })
}
#undef JFA_PICK_D

hipError_t launch_bwd_dkdv(const BwdArgs& a, int head_dim, int dtype, int act, int64_t grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (dtype == 0) return act == 0 ? dkdv_d<__bf16, 0>(a, head_dim, grid, stream) : dkdv_d<__bf16, 1>(a, head_dim, grid, stream);
  return act == 0 ? dkdv_d<float, 0>(a, head_dim, grid, stream) : dkdv_d<float, 1>(a, head_dim, grid, stream);
}

hipError_t launch_bwd_dq(const BwdArgs& a, int head_dim, int dtype, int act, int64_t grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (dtype == 0) return act == 0 ? dq_d<__bf16, 0>(a, head_dim, grid, stream) : dq_d<__bf16, 1>(a, head_dim, grid, stream);
  return act == 0 ? dq_d<float, 0>(a, head_dim, grid, stream) : dq_d<float, 1>(a, head_dim, grid, stream);
}

// The dQ pass when every sequence is short or has no keys: the dK/dV pass
// wrote the short sequences' dQ, and a sequence without keys gets zero rows.
// One workgroup per sequence.  Nothing is written when the list builder
// rejected the offsets (status word not 0), and offsets outside
// [0, total_q] write nothing either.
__global__ __launch_bounds__(256) void dq_keyless_kernel(BwdArgs a, const int* status, int row_bytes) {
  const int b = blockIdx.x;
  if (*status != 0 || a.ko[b + 1] != a.ko[b]) return;
  const int q0 = a.qo[b], q1 = a.qo[b + 1];
  if (q0 < 0 || q1 > a.total_q || q1 <= q0) return;
  u32x4* p = reinterpret_cast<u32x4*>(static_cast<char*>(a.dq) + (size_t)q0 * row_bytes);
  const int64_t n = (int64_t)(q1 - q0) * (row_bytes / 16);
  for (int64_t i = threadIdx.x; i < n; i += 256) p[i] = u32x4{0, 0, 0, 0};
}

hipError_t launch_bwd_dq_keyless(const BwdArgs& a, const int* status, int batch, int head_dim, int dtype,
                                 hipStream_t stream) {
  const int row_bytes = a.heads * head_dim * (dtype == 0 ? 2 : 4);
  if (batch <= 0 || row_bytes % 16 != 0 || !status) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dq_keyless_kernel, dim3(batch), dim3(256), 0, stream, a, status, row_bytes);
  return hipGetLastError();
}

hipError_t launch_bwd_stats(const StatsArgs& a, int head_dim, int dtype, hipStream_t stream) {
  return dtype == 0 ? stats_d<__bf16>(a, head_dim, stream) : stats_d<float>(a, head_dim, stream);
}

}  // namespace jfa

// MXFP8 jagged attention backward for gfx950: every product on the
// block-scaled matrix cores, with E4M3 operands in MX blocks of 32 along the
// product's own contraction axis (piletech.kr/articles/112134, section 핵심
// 포인트 / Key points, MXFP8 bullet, and section 상세 정리 / Detailed notes,
// MXFP8 item: training in MXFP8, the softmax side quantised online inside
// the kernel; number format: OCP Microscaling Formats (MX) v1.0).
//
// Per (query i, key j) pair, with t = scale q_i.k_j on the quantised rows:
//   P = exp(t - lse_i),  dP = dO_i . v_j,  dS = P (dP - delta_i)
//   dV_j += P dO_i,  dK_j += scale dS q_i,  dQ_i += scale dS k_j
// P and dS are formed in fp32 from exact P and quantised only as operands:
// along queries (blocks of 32 queries of a key, counted from the
// sequence's first query) for dV and dK, along keys (blocks of 32 keys of a
// query) for dQ.  Their block scale is the least power of two that keeps
// the block within E4M3's range, 2^k with max|x| <= 448 2^k: the vector
// conversion's 2^(floor(log2 max) - 8) saturates maxima in (1.75, 2) x 2^j,
// and its threshold lies exactly at P = 1, the weight of every query that
// sees a single key, where the last bit of P's evaluation would choose
// between 1 and 0.875.
//
// Two kernels, no atomics (each output row is owned by one workgroup):
//  * mx_dkdv_kernel, one workgroup per 64-key tile: two pairs of waves,
//    each pair owning 32 keys.  Wave A forms S = Q K^T and P, hands P to
//    wave B through LDS in fp32, quantises P and accumulates dV^T += dO^T P;
//    wave B forms dP = dO V^T and, one step later, dS from A's P, quantises
//    it and accumulates dK^T += Q^T dS.  A step is 64 queries: S and dP
//    come out one key per lane and 16 queries per lane half of each 32-query
//    block -- one MX block along queries is a lane-local max and one swap
//    between the wave's halves, and the packed codes are directly the B
//    operand of the dV / dK products, whose A operands (dO and Q along
//    queries) come from the column images.
//  * mx_dq_kernel, one workgroup per 128-query tile (4 waves x 32 queries),
//    the forward's layout: S^T = K Q^T and dP^T = V dO^T leave one query per
//    lane and 16 keys per lane half of each 32-key block, so dS quantised
//    along keys is again a lane-local max and one swap, and dQ^T += K^T dS^T
//    takes K's column image as its A operand.
#include <type_traits>

#include "jfa_common.hpp"
#include "jfa_internal.h"
#include "mx_common.hpp"

namespace jfa {

namespace {

__device__ __forceinline__ u32x4 gload16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }

typedef short s16x2 __attribute__((ext_vector_type(2)));

// Four elements of a block into one word (byte i = x_i), divided by the
// block's fitted scale in the conversion itself: v_cvt_scalef32_pk_fp8_f32
// divides by 2^(e - 127), e the exponent field of its scale operand (the
// significand is ignored), so the E8M0 code shifted into that field is the
// scale; measured on the hardware bit for bit equal to converting x 2^(127
// - code) for every code 0 .. 253, zero and subnormal inputs included.
// With the fitted scale no quotient exceeds 448, so the conversion needs no
// clamp.
__device__ __forceinline__ uint32_t codes4(const f32x16& x, int q, uint32_t code) {
  const float sc = __uint_as_float(code << 23);
  s16x2 w = {0, 0};
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, x[4 * q], x[4 * q + 1], sc, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, x[4 * q + 2], x[4 * q + 3], sc, true);
  return __builtin_bit_cast(uint32_t, w);
}

// E8M0 code of the fitted block scale of P and dS: the least 2^k with amax
// <= 448 2^k (biased by 127, at least 0), so that no element saturates.
// floor(log2 amax) - 8 is the exponent field minus 135; one more when the
// significand exceeds 1.75 (fraction field above 0x600000).
__device__ __forceinline__ uint32_t e8m0_code_fit(float amax) {
  const uint32_t u = __float_as_uint(amax);
  const int ef = (int)((u >> 23) & 0xff);
  return (uint32_t)max(ef - 8 + ((u & 0x7fffff) > 0x600000u ? 1 : 0), 0);
}

// Quantises two 32-element blocks held as accumulator columns (block c in
// x[c]: 16 values in this lane, the other 16 in lane l ^ 32) into the 32
// bytes of a block-scaled operand (block c in bytes 16c .. 16c+15), with the
// fitted scale, and returns the E8M0 code of block g (this lane half's
// scale byte).
template <bool POS>
__device__ __forceinline__ uint32_t quantise_pair(const f32x16* x, i32x8& out, int g) {
  uint32_t code[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    float amax = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) amax = fmaxf(amax, POS ? x[c][r] : fabsf(x[c][r]));
    code[c] = e8m0_code_fit(xor32_max(amax));
#pragma unroll
    for (int q = 0; q < 4; ++q) out[4 * c + q] = (int)codes4(x[c], q, code[c]);
  }
  return g ? code[1] : code[0];
}

// acc[dt] += A[dt] B for the 32-row blocks dt of a D-row product: A's
// scale word carries block dt's scale in byte dt.
template <int ND>
__device__ __forceinline__ void grad_products(f32x16* acc, const i32x8* a, const i32x8& b, uint32_t sa, uint32_t sb) {
  mma_mx<0, 0>(acc[0], a[0], b, sa, sb);
  mma_mx<1, 0>(acc[1], a[1], b, sa, sb);
  if constexpr (ND > 2) {
    mma_mx<2, 0>(acc[2], a[2], b, sa, sb);
    mma_mx<3, 0>(acc[3], a[3], b, sa, sb);
  }
}

// The A operands of one step's gradient product (ND fragments) and their
// scale word.
template <int ND>
struct ColFrags {
  i32x8 f[ND];
  uint32_t s;
};
template <int ND>
__device__ __forceinline__ void settle_frags(const ColFrags<ND>& c) {
#pragma unroll
  for (int i = 0; i < ND; ++i) settle(c.f[i]);
  settle(c.s);
}

}  // namespace

// ------------------------------------------------------------------ dK / dV

template <int D>
struct MxKvCfg {
  static constexpr int SQ = 64;                    // queries per step: two MX blocks
  static constexpr int CPR = D / 16;               // 16-byte chunks per image row
  static constexpr int TILE = SQ * D;              // one 64-row tile of a row image
  // a stage: [Q rows | dO rows | Q scales | dO scales | lse2 | delta]
  static constexpr int OFF_DO = TILE, OFF_QS = 2 * TILE, OFF_DOS = OFF_QS + 256, OFF_L = OFF_DOS + 256,
                       OFF_DL = OFF_L + 256, STAGE = OFF_DL + 256;
  static constexpr int XS = kWave * 32 * 4;        // one wave's P hand-over: 32 floats per lane
  static constexpr int PIPE = 2 * STAGE + 2 * 2 * XS;   // two stages; [slot][pair] hand-overs
  static constexpr int OUT = 4 * store_scratch_bytes<__bf16, D>();
  static constexpr int LDS = PIPE > OUT ? PIPE : OUT;
  static constexpr int NK = D / 64, ND = D / 32;
  static constexpr int RN = TILE / 16 / 128;       // chunks per thread of a role (128 threads) per tile
  static_assert(TILE / 16 % 128 == 0 && 64 * (D / 32) <= 256, "stage geometry");
};

template <int D>
__global__ __launch_bounds__(256, 2) void mx_dkdv_kernel(MxBwdArgs a) {
  using C = MxKvCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  const ItemMeta m = a.meta_kv[blockIdx.x];
  if (m.lq < 0) return;   // past the item count
  const int qs = m.qs, lq = m.lq, ks = m.ks, lk = m.lk, h = m.head, t = m.tile, b = m.seq;
  const int off = lk - lq;   // causal: query i sees keys j <= i + off
  // the wave index through readfirstlane: role-dependent values and
  // branches are then uniform to the compiler (scalar registers, no two
  // masked loads into one register)
  const int tid = threadIdx.x, l = lane_id(), w = __builtin_amdgcn_readfirstlane(tid >> 6), g = l >> 5, c32 = l & 31;
  const bool role_a = w < 2;   // A: S, P, dV;  B: dP, dS, dK
  const int pair = w & 1, tr = tid & 127;
  const int kw0 = t * 64 + 32 * pair;   // first key of this pair
  const int my_key = kw0 + c32;         // the key (column of S) this lane owns
  // 32-query blocks this tile's keys see, from the first one (32-aligned:
  // the MX blocks along queries are counted from the sequence's first query)
  const int q_first = kv_tile_first_q_block(lq, lk, t, 32, 64, a.causal) * 32;
  const int nst = (kv_tile_q_blocks(lq, lk, t, 32, 64, a.causal) + 1) / 2;
  const int qblocks = (lq + 31) / 32;

  // the sequence in the images
  const int64_t qb0 = qs / 32 + b, kb0 = ks / 32 + b;
  const int64_t nbq = a.rq / 32;
  const int64_t qrow = (int64_t)h * a.rq + 32 * qb0;   // image row of query 0
  const int64_t krow = (int64_t)h * a.rk + 32 * kb0;   // image row of key 0

  // this role's share of a stage (Q side for A, dO side for B), staged in
  // registers: the tile's chunks, and one row value per lane of the wave
  // (pair 0: the rows' scale words, pair 1: lse2 or delta)
  const MxImage rimg = role_a ? a.q : a.dout;
  const float* rstat = (role_a ? a.lse2 : a.delta) + (size_t)h * a.total_q + qs;
  u32x4 st_r[C::RN];
  uint32_t st_w = 0u;
  // Rows past the sequence repeat its last row (finite values, and every
  // weight of such a query is masked to 0): the loads are unconditional, so
  // that nothing has to wait for them before the stage is stored.
  auto stage_load = [&](int s) {
    const int q0 = q_first + 64 * s, last = lq - 1 - q0;
#pragma unroll
    for (int i = 0; i < C::RN; ++i) {
      const int p = i * 128 + tr, r = min(p / C::CPR, last), pc = p % C::CPR;
      st_r[i] = gload16(rimg.x + (qrow + q0 + r) * D + pc * 16);
    }
    const int r = min(l, last);
    if (pair == 0) st_w = scale_word<D>(rimg.s + (qrow + q0 + r) * (D / 32));
    else st_w = __float_as_uint(rstat[q0 + r]);
  };
  auto slot = [&](int s) { return smem + (s & 1) * C::STAGE; };
  auto stage_store = [&](int s) {
    char* st = slot(s);
    char* tile = st + (role_a ? 0 : C::OFF_DO);
#pragma unroll
    for (int i = 0; i < C::RN; ++i) {
      const int p = i * 128 + tr, r = p / C::CPR, pc = p % C::CPR;
      *reinterpret_cast<u32x4*>(tile + mx_k_off<D>(r, pc)) = st_r[i];
    }
    if (pair == 0) {
      char* sc = st + (role_a ? C::OFF_QS : C::OFF_DOS);
      if constexpr (D == 128) *reinterpret_cast<uint32_t*>(sc + 4 * l) = st_w;
      else *reinterpret_cast<uint16_t*>(sc + 2 * l) = (uint16_t)st_w;
    } else {
      *reinterpret_cast<uint32_t*>(st + (role_a ? C::OFF_L : C::OFF_DL) + 4 * l) = st_w;
    }
  };

  // A operand of this wave's gradient product for step s: the dO (A) or Q
  // (B) column image, blocks q_first/32 + 2s and + 1 (k blocks 0 and 1),
  // column 32 dt + c32, lane half g's 16 bytes; the scale word of block
  // q_first/32 + 2s + g, row c32 (byte dt: column 32 dt + c32).  A block
  // past the sequence is read as its last block instead: the B operand's
  // codes of those queries are 0 (their weights are masked), so the product
  // takes nothing from it, and the loads need no condition.
  const MxImage cimg = role_a ? a.doc : a.qc;
  const uint8_t* cx = cimg.x + ((int64_t)h * nbq + qb0) * (D * 32);
  const uint8_t* cs = cimg.s + ((int64_t)h * nbq + qb0) * D;
  auto col_load = [&](ColFrags<C::ND>& cf, int s) {
    const int blk = q_first / 32 + 2 * s, blk1 = min(blk + 1, qblocks - 1);
#pragma unroll
    for (int dt = 0; dt < C::ND; ++dt) {
      const int col = 32 * dt + c32;
      cf.f[dt] = cat8(gload16(cx + ((int64_t)blk * D + col) * 32 + 16 * g),
                      gload16(cx + ((int64_t)blk1 * D + col) * 32 + 16 * g));
    }
    cf.s = scale_word<D>(cs + ((int64_t)(g ? blk1 : blk) * 32 + c32) * (D / 32));
  };

  // B operand of S (A: the lane's key row) or dP (B: its value row): head
  // dims 64i + 16g .. +15 and 64i + 32 + 16g .. +15 for product i; the scale
  // word shifted so that byte 2i is the scale of block 2i + g
  i32x8 xf[C::NK];
  uint32_t xsc;
  {
    const int j = min(my_key, lk - 1);
    const MxImage x = role_a ? a.k : a.v;
    const uint8_t* p = x.x + (krow + j) * D + 16 * g;
#pragma unroll
    for (int i = 0; i < C::NK; ++i) xf[i] = cat8(gload16(p + 64 * i), gload16(p + 64 * i + 32));
    xsc = scale_word<D>(x.s + (krow + j) * (D / 32)) >> (8 * g);
  }
  if (nst > 0) stage_load(0);
#pragma unroll
  for (int i = 0; i < C::NK; ++i) settle(xf[i]);
  settle(xsc);
  if (nst > 0) stage_store(0);
  __syncthreads();

  f32x16 acc[C::ND];   // dV^T (A) or dK^T (B): lane = key, registers = head dims
#pragma unroll
  for (int i = 0; i < C::ND; ++i) acc[i] = f32x16{};

  auto visible = [&](int s) {
    const int q0 = q_first + 64 * s;
    return kw0 < lk && q0 < lq && !(a.causal && q0 + 63 + off < kw0);
  };
  auto needs_mask = [&](int s) {
    const int q0 = q_first + 64 * s;
    return q0 + 64 > lq || kw0 + 32 > lk || (a.causal && kw0 + 31 > q0 + off);
  };
  // the row statistic (lse2 or delta) of register r of block c, 4 at a time
  auto stat4 = [&](const char* st, int o, int c, int a4) {
    return *reinterpret_cast<const f32x4*>(st + o + 4 * (32 * c + 8 * a4 + 4 * g));
  };
  // x[c] = (Q or dO rows of step s) x (this lane's K or V row): block c's
  // query 32c + 8(r/4) + 4g + r%4 of the step in register r
  auto products = [&](f32x16* x, const char* tile, const char* sc) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = 32 * c + c32;
      const uint32_t sr = scale_word<D>(reinterpret_cast<const uint8_t*>(sc) + row * (D / 32)) >> (8 * g);
      x[c] = f32x16{};
      mma_mx<0, 0>(x[c], cat8(lds16(tile + mx_k_off<D>(row, g)), lds16(tile + mx_k_off<D>(row, 2 + g))), xf[0], sr,
                   xsc);
      if constexpr (C::NK > 1)
        mma_mx<2, 2>(x[c], cat8(lds16(tile + mx_k_off<D>(row, 4 + g)), lds16(tile + mx_k_off<D>(row, 6 + g))), xf[1],
                     sr, xsc);
    }
  };
  auto xslot = [&](int s) { return smem + 2 * C::STAGE + ((s & 1) * 2 + pair) * C::XS + l * 16; };

  // Wave A, step s: S, then P (handed to B) quantised into pc (returns the
  // scale byte of this lane half's block)
  auto a_p = [&](auto MASK, int s, i32x8& pc) {
    const char* st = slot(s);
    const int q0 = q_first + 64 * s;
    f32x16 x[2];
    products(x, st, st + C::OFF_QS);
    // visible iff lo <= query offset (32c + 8(r/4) + r%4) < lo + span
    const int lo = (a.causal ? my_key - off : 0) - q0 - 4 * g;
    const int span = my_key < lk ? max(lq - q0 - 4 * g - lo, 0) : 0;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 l4 = stat4(st, C::OFF_L, c, a4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * a4 + i;
          const float p = fast_exp2(fmaf(x[c][r], a.scale_log2, -l4[i]));
          bool masked = false;
          if constexpr (decltype(MASK)::value) masked = (unsigned)(32 * c + 8 * a4 + i - lo) >= (unsigned)span;
          x[c][r] = masked ? 0.f : p;
        }
      }
    }
    char* xo = xslot(s);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = k >> 2, q = k & 3;
      *reinterpret_cast<f32x4*>(xo + k * kWave * 16) = f32x4{x[c][4 * q], x[c][4 * q + 1], x[c][4 * q + 2], x[c][4 * q + 3]};
    }
    return quantise_pair<true>(x, pc, g);
  };

  // Wave B: dP - delta of step s (kept in registers until A's P arrives)
  f32x16 dd[2];
  auto b_dp = [&](int s) {
    const char* st = slot(s);
    products(dd, st + C::OFF_DO, st + C::OFF_DOS);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const f32x4 d4 = stat4(st, C::OFF_DL, c, a4);
#pragma unroll
        for (int i = 0; i < 4; ++i) dd[c][4 * a4 + i] -= d4[i];
      }
    }
  };
  // Wave B, one step behind: dS = P (dP - delta) of step s from A's P,
  // quantised into the B operand of dK^T += Q^T Q(dS) (its products run
  // after dP of the next step, giving the operand loads time to land)
  auto b_ds = [&](int s, i32x8& sc) {
    const char* xi = xslot(s);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = k >> 2, q = k & 3;
      const f32x4 p4 = *reinterpret_cast<const f32x4*>(xi + k * kWave * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i) dd[c][4 * q + i] *= p4[i];
    }
    return quantise_pair<false>(dd, sc, g);
  };

  // Step s: stage s+1 is read into registers first and written to LDS at
  // the end (its slot held stage s-1, which every wave finished before the
  // last barrier).  A works on step s; B finishes step s-1 (dS, then its dK
  // products after dP of step s) and forms dP(s).  Each wave loads the
  // gradient operands of the step it finishes next right after its
  // products have consumed the current ones.  Every load is issued without a branch (past the last step
  // they repeat it), which keeps the compiler's waits for them exact.  The
  // roles run loops of their own (each wave meets the same nst + 1
  // barriers), so that neither keeps the other's values live.  The
  // barriers order LDS only (lds_barrier), so that the operand loads stay in
  // flight across them.
  ColFrags<C::ND> cf;
  if (nst > 0 && role_a) {
    col_load(cf, 0);
    for (int s = 0; s < nst; ++s) {
      const int nx = min(s + 1, nst - 1);   // the last step reloads its own operands, unused
      stage_load(nx);
      if (visible(s)) {
        // one product site, so that the accumulators are updated in place
        i32x8 pc;
        uint32_t sp;
        if (needs_mask(s)) sp = a_p(std::true_type{}, s, pc);
        else sp = a_p(std::false_type{}, s, pc);
        grad_products<C::ND>(acc, cf.f, pc, cf.s, sp);
      }
      col_load(cf, nx);
      if (s + 1 < nst) stage_store(s + 1);
      lds_barrier();
    }
  } else if (nst > 0) {
    for (int s = 0; s <= nst; ++s) {
      stage_load(min(s + 1, nst - 1));
      const bool prev = s > 0 && visible(s - 1);
      const bool vis = s < nst && visible(s);
      i32x8 sc;
      uint32_t ss = 0u;
      if (prev) ss = b_ds(s - 1, sc);
      if (vis) b_dp(s);
      if (prev) grad_products<C::ND>(acc, cf.f, sc, cf.s, ss);
      col_load(cf, min(s, nst - 1));
      if (s + 1 < nst) stage_store(s + 1);
      if (s < nst) lds_barrier();
    }
  }

  // the ring is free once every wave is past the loop: stage the rows there
  __syncthreads();
  __bf16* op = static_cast<__bf16*>(role_a ? a.dv : a.dk) + (size_t)(ks + kw0) * (a.heads * D) + (size_t)h * D;
  store_rows_lds<__bf16, D>(op, a.heads * D, min(32, lk - kw0), acc, role_a ? 1.0f : a.scale,
                            smem + w * store_scratch_bytes<__bf16, D>());
}

// ------------------------------------------------------------------ dQ

template <int D>
struct MxDqCfg {
  static constexpr int BM = kFwdBM, BN = kFwdBN, NT = 256;
  static constexpr int KT = BN * D;          // a 64-row tile of a row image (K or V)
  static constexpr int CT = 2 * D * 32;      // two 32-key blocks of K's column image
  static constexpr int SC = 256;             // scale bytes per tile
  static constexpr int OFF_V = KT + SC, OFF_C = 2 * (KT + SC), STAGE = OFF_C + CT + SC;
  static constexpr int PIPE = 2 * STAGE;
  static constexpr int OUT = (NT / kWave) * store_scratch_bytes<__bf16, D>();
  static constexpr int LDS = PIPE > OUT ? PIPE : OUT;
  static constexpr int NK = D / 64, ND = D / 32;
  static constexpr int N = KT / 16 / NT;     // copies per thread per tile
  static_assert(KT / 16 % NT == 0 && CT == KT && BM == 128 && BN == 64, "tile geometry");
};

template <int D>
__global__ __launch_bounds__(256, 2) void mx_dq_kernel(MxBwdArgs a) {
  using C = MxDqCfg<D>;
  using F = MxCfg<D>;   // the forward's K-tile geometry (64 rows, same swizzle)
  static_assert(F::KT == C::KT, "K tiles shared with the forward's layout");
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];

  const ItemMeta m = a.meta_q[blockIdx.x];
  if (m.lq < 0) return;
  const int qs = m.qs, lq = m.lq, ks = m.ks, lk = m.lk, h = m.head, t = m.tile, b = m.seq;
  const int off = lk - lq;
  const int tid = threadIdx.x, l = lane_id(), w = tid >> 6, g = l >> 5, c32 = l & 31;
  const int wave0 = tid & ~(kWave - 1);
  const int row0 = t * C::BM + 32 * w;
  const int my_row = row0 + c32;
  const bool wave_live = row0 < lq;
  const int n_kv = q_tile_kv_blocks(lq, lk, t, C::BM, C::BN, a.causal);

  const int64_t qrow = (int64_t)h * a.rq + 32 * ((int64_t)(qs / 32) + b);
  const int64_t kb0 = ks / 32 + b;
  const int64_t krow = (int64_t)h * a.rk + 32 * kb0;
  const int64_t nbk = a.rk / 32;
  const uint8_t* kcx = a.kc.x + ((int64_t)h * nbk + kb0) * (D * 32);
  const uint8_t* kcs = a.kc.s + ((int64_t)h * nbk + kb0) * D;

  // this thread's chunks of a row tile and of a column tile (the forward's
  // swizzles: the LDS slot of copy i holds the global chunk mapped to it)
  int roff[C::N], coff[C::N];
#pragma unroll
  for (int i = 0; i < C::N; ++i) {
    const int p = i * C::NT + tid;
    const int r = p / F::CPR, pc = p % F::CPR;
    roff[i] = r * D + ((pc ^ ((r / F::RPL) % F::CPR)) * 16);
    const int c = p / (2 * D), d = (p >> 1) % D, ph = p & 1;
    coff[i] = c * D * 32 + d * 32 + ((ph ^ ((d >> 3) & 1)) * 16);
  }
  // Copies of key tile j into a stage: K rows, V rows, K columns; rows
  // past the sequence read as zeros.  Waves 0, 1, 2 also copy the K row,
  // V row and K column scales (whole dwords, as in the forward: the bytes
  // past an odd row count at D = 64 are a zero padding row).
  auto issue = [&](char* st, int j) {
    const int kv0 = j * C::BN, rows = min(C::BN, lk - kv0), nb = (rows + 31) / 32;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.k.x + (krow + kv0) * D), 0, rows * D, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a.v.x + (krow + kv0) * D), 0, rows * D, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(kcx + (int64_t)(2 * j) * (D * 32)), 0, nb * D * 32, kBufferWord3);
#pragma unroll
    for (int i = 0; i < C::N; ++i) {
      buffer_load_lds16(rk, roff[i], st + (i * C::NT + wave0) * 16);
      buffer_load_lds16(rv, roff[i], st + C::OFF_V + (i * C::NT + wave0) * 16);
      buffer_load_lds16(rc, coff[i], st + C::OFF_C + (i * C::NT + wave0) * 16);
    }
    const int sbytes = (rows * (D / 32) + 3) & ~3;
    if (w == 0) buffer_load_lds4(uniform_rsrc(a.k.s + (krow + kv0) * (D / 32), sbytes), l * 4, st + C::KT);
    if (w == 1) buffer_load_lds4(uniform_rsrc(a.v.s + (krow + kv0) * (D / 32), sbytes), l * 4, st + C::OFF_V + C::KT);
    if (w == 2) buffer_load_lds4(uniform_rsrc(kcs + (int64_t)(2 * j) * D, nb * D), l * 4, st + C::OFF_C + C::CT);
  };
  auto slot = [&](int j) { return smem + (j & 1) * C::STAGE; };
  if (n_kv > 0) issue(slot(0), 0);

  // B operands: the lane's Q row (for S^T) and dO row (for dP^T), product i
  // taking head dims 64i + 16g .. +15 and 64i + 32 + 16g .. +15, scale words
  // shifted so that byte 2i is block 2i + g; and the row's lse2 and delta
  i32x8 qf[C::NK], df[C::NK];
  uint32_t qsc, dsc;
  float lse2, delta;
  {
    const int r = min(my_row, lq - 1);
    const uint8_t* qp = a.q.x + (qrow + r) * D + 16 * g;
    const uint8_t* dp = a.dout.x + (qrow + r) * D + 16 * g;
#pragma unroll
    for (int i = 0; i < C::NK; ++i) {
      qf[i] = cat8(gload16(qp + 64 * i), gload16(qp + 64 * i + 32));
      df[i] = cat8(gload16(dp + 64 * i), gload16(dp + 64 * i + 32));
    }
    qsc = scale_word<D>(a.q.s + (qrow + r) * (D / 32)) >> (8 * g);
    dsc = scale_word<D>(a.dout.s + (qrow + r) * (D / 32)) >> (8 * g);
    lse2 = a.lse2[(size_t)h * a.total_q + qs + r];
    delta = a.delta[(size_t)h * a.total_q + qs + r];
#pragma unroll
    for (int i = 0; i < C::NK; ++i) {
      settle(qf[i]);
      settle(df[i]);
    }
    settle(qsc);
    settle(dsc);
    settle(lse2);
    settle(delta);
  }

  f32x16 acc[C::ND];   // dQ^T: lane = query, registers = head dims
#pragma unroll
  for (int i = 0; i < C::ND; ++i) acc[i] = f32x16{};

  auto wave_active = [&](int j) { return wave_live && (!a.causal || j * C::BN <= row0 + 31 + off); };
  const int row_limit = a.causal ? min(lk, my_row + off + 1) : lk;
  auto needs_mask = [&](int j) {
    const int kv0 = j * C::BN;
    return (kv0 + C::BN > lk) || (a.causal && kv0 + C::BN - 1 > row0 + off);
  };
  // x[c] = x0 + (K or V rows of the tile, block c) x (this lane's Q or dO
  // row): key 32c + 8(r/4) + 4g + r%4 of the tile in register r
  auto products = [&](f32x16* x, const char* tile, const i32x8* yf, uint32_t ysc, const f32x16& x0) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = 32 * c + c32;
      const uint32_t sr = scale_word<D>(reinterpret_cast<const uint8_t*>(tile + C::KT) + row * (D / 32)) >> (8 * g);
      x[c] = x0;
      mma_mx<0, 0>(x[c], cat8(lds16(tile + mx_k_off<D>(row, g)), lds16(tile + mx_k_off<D>(row, 2 + g))), yf[0], sr,
                   ysc);
      if constexpr (C::NK > 1)
        mma_mx<2, 2>(x[c], cat8(lds16(tile + mx_k_off<D>(row, 4 + g)), lds16(tile + mx_k_off<D>(row, 6 + g))), yf[1],
                     sr, ysc);
    }
  };
  // dP^T accumulates onto -delta (the lane's query), so that the products
  // leave dP - delta
  f32x16 ndelta;
#pragma unroll
  for (int r = 0; r < 16; ++r) ndelta[r] = -delta;
  // dS^T of key tile j quantised along keys into sc (returns the scale byte
  // of this lane half's block)
  auto ds_tile = [&](auto MASK, int j, i32x8& sc) {
    const char* st = slot(j);
    f32x16 s[2], ds[2];
    products(s, st, qf, qsc, f32x16{});
    products(ds, st + C::OFF_V, df, dsc, ndelta);
    const int lim = row_limit - j * C::BN - 4 * g;   // masked iff key offset >= lim
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[c][r], a.scale_log2, -lse2));
        bool masked = false;
        if constexpr (decltype(MASK)::value) masked = 32 * c + 8 * (r >> 2) + (r & 3) >= lim;
        ds[c][r] = masked ? 0.f : p * ds[c][r];
      }
    }
    return quantise_pair<false>(ds, sc, g);
  };
  // dQ^T += K^T Q(dS^T) over key tile j
  auto dq_products = [&](int j, const i32x8& sc, uint32_t ss) {
    const char* ct = slot(j) + C::OFF_C;
    const uint32_t skc = scale_word<D>(reinterpret_cast<const uint8_t*>(ct + C::CT) + g * D + c32 * (D / 32));
    auto dq = [&](auto DT) {
      constexpr int dt = decltype(DT)::value;
      const int d = 32 * dt + c32;
      mma_mx<dt, 0>(acc[dt], cat8(lds16(ct + mx_v_off<D>(0, d, g)), lds16(ct + mx_v_off<D>(1, d, g))), sc, skc, ss);
    };
    dq(std::integral_constant<int, 0>{});
    dq(std::integral_constant<int, 1>{});
    if constexpr (C::ND > 2) {
      dq(std::integral_constant<int, 2>{});
      dq(std::integral_constant<int, 3>{});
    }
  };

  dma_wait();
  __syncthreads();
  for (int j = 0; j < n_kv; ++j) {
    // stage j+1 goes into the slot of stage j-1, which every wave finished
    // before the last barrier
    if (j + 1 < n_kv) issue(slot(j + 1), j + 1);
    if (wave_active(j)) {
      // one product site, so that the accumulators are updated in place
      i32x8 sc;
      uint32_t ss;
      if (needs_mask(j)) ss = ds_tile(std::true_type{}, j, sc);
      else ss = ds_tile(std::false_type{}, j, sc);
      dq_products(j, sc, ss);
    }
    dma_wait();
    __syncthreads();
  }

  if (!wave_live) return;
  __bf16* op = static_cast<__bf16*>(a.dq) + (size_t)(qs + row0) * (a.heads * D) + (size_t)h * D;
  store_rows_lds<__bf16, D>(op, a.heads * D, min(32, lq - row0), acc, a.scale,
                            smem + w * store_scratch_bytes<__bf16, D>());
}

template __global__ void mx_dkdv_kernel<64>(MxBwdArgs);
template __global__ void mx_dkdv_kernel<128>(MxBwdArgs);
template __global__ void mx_dq_kernel<64>(MxBwdArgs);
template __global__ void mx_dq_kernel<128>(MxBwdArgs);

hipError_t launch_mx_bwd_dkdv(const MxBwdArgs& a, int head_dim, int64_t grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (head_dim == 64) hipLaunchKernelGGL(mx_dkdv_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  else if (head_dim == 128) hipLaunchKernelGGL(mx_dkdv_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_mx_bwd_dq(const MxBwdArgs& a, int head_dim, int64_t grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (head_dim == 64) hipLaunchKernelGGL(mx_dq_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  else if (head_dim == 128) hipLaunchKernelGGL(mx_dq_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace jfa

// MXFP8 jagged attention forward for gfx950: E4M3 operands with E8M0 block
// scales on the block-scaled matrix cores.
//
// Method: piletech.kr/articles/112134, section 핵심 포인트 (Key points), MXFP8
// bullet, and section 상세 정리 (Detailed notes), MXFP8 item: the model trains
// in a microscaled 8-bit format, the softmax output is quantised online from
// work the kernel does anyway, and the quantisation runs per wavefront on
// 32 x 32 blocks.  Number format: OCP Microscaling Formats (MX) v1.0 -- E4M3
// elements, one E8M0 scale per 32 elements, scale 2^(floor(log2 max) - 8),
// elements rounded to nearest even and clamped to 448.
//
// Two kernels:
//  * mx_quant_kernel turns bf16 Q, K and V into their MX images once per
//    call.  Q and K: "row images", blocks of 32 head-dim elements (the
//    contraction of Q K^T).  V: a "column image", blocks of 32 consecutive
//    keys of a sequence counted from its first key, per column (the
//    contraction of P V).  Both index a sequence's rows from a 32-row
//    boundary, row i of sequence b at image row 32 (off[b]/32 + b) + i, so
//    that the sequences' blocks never share a block row and no prefix sum
//    is needed.
//  * mx_fwd_kernel: one workgroup (4 waves x 32 queries) per 128-query
//    work item -- 2 waves when no sequence has more than 64 queries, so
//    that no wave of an item idles and twice the items fit a compute
//    unit --, K and V tiles of 64 keys copied into LDS by buffer loads
//    that write LDS.  S^T = K Q^T on the block-scaled matrix cores leaves
//    every lane one query and 16 keys of each 32-key block; those 32 keys
//    are exactly one MX block of P, so P's block max is a lane-local max and
//    one swap between the wave's halves -- the same reduction the row max
//    needs.  The row max is kept as an integer (log2 units): then the
//    block's elements are 2^(t - floor(block max) + 8), independent of the
//    row max, and the row max sets only the block's E8M0 scale.  The weights
//    go into the B operand of O^T += V^T P^T with no trip through LDS.
//
// Block-scaled product layout (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 on
// both sides, checked on the hardware): lane l holds row l%32 of A (column
// l%32 of B) in 32 bytes; bytes 0..15 of both lane halves form the first
// 32-element k block, bytes 16..31 the second, and byte p of lane half g
// meets byte p of the same half of the other operand.  The scale of row
// (column) r for k block kb is byte `opsel` of lane r + 32 kb's scale
// register.  The accumulator layout is that of the bf16 products
// (jfa_common.hpp).
#include <type_traits>

#include "jfa_common.hpp"
#include "jfa_internal.h"
#include "mx_common.hpp"

namespace jfa {

// ------------------------------------------------------------------ quantisation

// Row image block: rows row0 .. row0+31 (n of them real) of every head,
// blocks of 32 elements along a row.  The tile is read as it lies in memory
// (token-major, heads x D elements per token), 16 elements per thread and
// step: two neighbouring lanes hold a block.
template <int D>
__device__ __forceinline__ void mx_quant_rows(const __bf16* x, int heads, int64_t nrows, int row0, int n, int br,
                                              uint8_t* codes, uint8_t* scales, int tid) {
  constexpr int U = 4;               // chunks in flight per thread
  const int hd = heads * D;
  const int chunks = 32 * hd / 16;   // even: a block's two chunks are lanes t and t^1
  for (int base = 0; base < chunks; base += U * 256) {
    u32x4 raw[U][2];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int c = base + k * 256 + tid, e0 = c * 16, r = e0 / hd;
      if (c < chunks && r < n) {
        const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)(row0 + r) * hd + e0 % hd);
        raw[k][0] = src[0];
        raw[k][1] = src[1];
      } else {
        raw[k][0] = raw[k][1] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const int c = base + k * 256 + tid;
      if (c >= chunks) break;   // the pair t, t^1 leaves together (chunks is even)
      const int e0 = c * 16, r = e0 / hd, rem = e0 % hd, h = rem / D, d = rem % D;
      float v[16];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int e = 0; e < 4; ++e) bf16x2_to_float(raw[k][q][e], v[8 * q + 2 * e], v[8 * q + 2 * e + 1]);
      }
      float amax = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(v[e]));
      amax = fmaxf(amax, __shfl_xor(amax, 1));
      const uint32_t code = e8m0_code(amax);
      const float inv = e8m0_inverse(code);
      u32x4 w;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = fp8x4(v[4 * q] * inv, v[4 * q + 1] * inv, v[4 * q + 2] * inv, v[4 * q + 3] * inv);
      const int64_t row = (int64_t)h * nrows + 32 * (int64_t)br + r;
      *reinterpret_cast<u32x4*>(codes + row * D + d) = w;
      if ((c & 1) == 0) scales[row * (D / 32) + d / 32] = (uint8_t)code;
    }
  }
}

// Column image block: rows row0 .. row0+31 (n real) of every head, one block
// per column.  A thread takes two neighbouring columns (one 4-byte load per
// row: the wave reads whole token rows), keeps their 32 rows in registers
// and writes each column's 32 codes in the image's key order; the scales
// are staged in LDS and leave in 16-byte stores.
template <int D>
__device__ __forceinline__ void mx_quant_cols(const __bf16* x, int heads, int64_t nbr, int row0, int n, int br,
                                              uint8_t* codes, uint8_t* scales, int tid, uint8_t* lds) {
  const int hd = heads * D;
  for (int cp = tid; cp < hd / 2; cp += 256) {
    float a[32], b[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const uint32_t u = r < n ? *reinterpret_cast<const uint32_t*>(x + (size_t)(row0 + r) * hd + 2 * cp) : 0u;
      bf16x2_to_float(u, a[r], b[r]);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float* col = s ? b : a;
      float amax = 0.f;
#pragma unroll
      for (int r = 0; r < 32; ++r) amax = fmaxf(amax, fabsf(col[r]));
      const uint32_t code = e8m0_code(amax);
      const float inv = e8m0_inverse(code);
      const int cc = 2 * cp + s, h = cc / D, d = cc % D;
      // word w of the column holds keys 8 (w % 4) + 4 (w / 4) + 0..3
      u32x4 lo, hi;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int i = 8 * (w % 4) + 4 * (w / 4);
        const uint32_t x4 = fp8x4(col[i] * inv, col[i + 1] * inv, col[i + 2] * inv, col[i + 3] * inv);
        if (w < 4) lo[w] = x4;
        else hi[w - 4] = x4;
      }
      uint8_t* dst = codes + (((int64_t)h * nbr + br) * D + d) * 32;
      reinterpret_cast<u32x4*>(dst)[0] = lo;
      reinterpret_cast<u32x4*>(dst)[1] = hi;
      lds[h * D + (d % 32) * (D / 32) + d / 32] = (uint8_t)code;   // column 32 c + r at [r][c]
    }
  }
  __syncthreads();
  for (int c = tid; c < hd / 16; c += 256) {
    const int h = (16 * c) / D, o = (16 * c) % D;
    *reinterpret_cast<u32x4*>(scales + ((int64_t)h * nbr + br) * D + o) = reinterpret_cast<const u32x4*>(lds)[c];
  }
  __syncthreads();   // the staging is reused by the next block row
}

// One workgroup per kMxGroup consecutive block rows of a tensor, 32 rows of
// every head each: one search for the first block row's sequence, then a
// walk forward.  Dynamic LDS: heads * D bytes (a column block's scales).
constexpr int kMxGroup = 8;
template <int D>
__global__ __launch_bounds__(256) void mx_quant_kernel(MxQuantArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int z = blockIdx.y;
  const int nbr = a.nbr[z];
  const int br0 = blockIdx.x * kMxGroup;
  if (br0 >= nbr || a.batch <= 0) return;
  const int br1 = min(nbr, br0 + kMxGroup);
  const int32_t* off = a.off[z];
  // the last b with off[b]/32 + b <= br0 (b = 0 if none)
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] / 32 + mid <= br0) lo = mid;
    else hi = mid - 1;
  }
  const __bf16* x = static_cast<const __bf16*>(a.x[z]);
  int b = lo;
  for (int br = br0; br < br1; ++br) {   // every value here is uniform across the workgroup
    while (b + 1 < a.batch && off[b + 1] / 32 + b + 1 <= br) ++b;
    const int s = off[b], e = off[b + 1];
    const int i0 = 32 * (br - (s / 32 + b)), n = min(32, e - s - i0);
    if (i0 < 0 || n <= 0 || s < 0 || e > a.total[z]) continue;   // between sequences' blocks
    if (a.keys[z])
      mx_quant_cols<D>(x, a.heads, nbr, s + i0, n, br, a.codes[z], a.scales[z], threadIdx.x, lds);
    else
      mx_quant_rows<D>(x, a.heads, 32 * (int64_t)nbr, s + i0, n, br, a.codes[z], a.scales[z], threadIdx.x);
  }
}

hipError_t launch_mx_quant(const MxQuantArgs& a, int head_dim, int count, hipStream_t stream) {
  int nbr = 0;
  for (int z = 0; z < count; ++z) nbr = max(nbr, a.nbr[z]);
  if (count > kMxQuantMax) return hipErrorInvalidValue;
  if (nbr <= 0 || a.heads <= 0 || count <= 0) return hipSuccess;
  const dim3 grid((unsigned)((nbr + kMxGroup - 1) / kMxGroup), (unsigned)count);
  const size_t lds = (size_t)a.heads * head_dim;
  if (head_dim == 64) hipLaunchKernelGGL(mx_quant_kernel<64>, grid, dim3(256), lds, stream, a);
  else if (head_dim == 128) hipLaunchKernelGGL(mx_quant_kernel<128>, grid, dim3(256), lds, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// ------------------------------------------------------------------ attention

template <int D, int NW>
__global__ __launch_bounds__(64 * NW, 2) void mx_fwd_kernel(MxFwdArgs a) {
  using C = MxCfg<D, NW>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  char* const kslot0 = smem;                     // [K tile | K scales] x 2
  char* const vslot0 = smem + 2 * C::KSLOT;      // [V^T tile | V scales] x 2

  const ItemMeta m = a.meta[blockIdx.x];
  if (m.lq < 0) return;
  const int qs = m.qs, lq = m.lq, ks = m.ks, lk = m.lk, h = m.head, t = m.tile, b = m.seq;
  const int off = lk - lq;   // causal: query i sees keys j <= i + off
  const int tid = threadIdx.x, l = lane_id(), w = tid >> 6, g = l >> 5, c32 = l & 31;
  const int wave0 = tid & ~(kWave - 1);
  const int row0 = t * C::BM + 32 * w;
  const int my_row = row0 + c32;
  const bool wave_live = row0 < lq;
  const int n_kv = q_tile_kv_blocks(lq, lk, t, C::BM, C::BN, a.causal);

  // this sequence and head in the images
  const int64_t qrow0 = 32 * ((int64_t)(qs / 32) + b), krow0 = 32 * ((int64_t)(ks / 32) + b);
  const int64_t nbk = a.rk / 32;
  const uint8_t* kx = a.kx + ((int64_t)h * a.rk + krow0) * D;
  const uint8_t* ksc = a.ks + ((int64_t)h * a.rk + krow0) * (D / 32);
  const uint8_t* vx = a.vx + ((int64_t)h * nbk + krow0 / 32) * (D * 32);
  const uint8_t* vsc = a.vs + ((int64_t)h * nbk + krow0 / 32) * D;

  // global byte offsets of this thread's chunks within a K / V tile: the
  // chunk its LDS slot holds under the swizzles above
  int koff[C::N], voff[C::N];
#pragma unroll
  for (int i = 0; i < C::N; ++i) {
    const int p = i * C::NT + tid;
    const int r = p / C::CPR, pc = p % C::CPR;
    koff[i] = r * D + ((pc ^ ((r / C::RPL) % C::CPR)) * 16);
    const int c = p / (2 * D), d = (p >> 1) % D, ph = p & 1;
    voff[i] = c * D * 32 + d * 32 + ((ph ^ ((d >> 3) & 1)) * 16);
  }

  // Copies of key tile j: rows past the sequence read as zeros (each
  // buffer covers the sequence's rows only).  Wave 0 also copies the K
  // scales, wave 1 the V scales.
  auto issue_k = [&](char* slot, int j) {
    const int kv0 = j * C::BN, rows = min(C::BN, lk - kv0);
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kx + (int64_t)kv0 * D), 0, rows * D, kBufferWord3);
#pragma unroll
    for (int i = 0; i < C::N; ++i) buffer_load_lds16(r, koff[i], slot + (i * C::NT + wave0) * 16);
    // whole dwords: a copy that crosses the buffer's end reads as zero
    // entirely, so an odd row count at D = 64 would lose the last key's
    // scales; the extra bytes are the next image row, a zero padding row
    // of the sequence's last block
    if (w == 0)
      buffer_load_lds4(uniform_rsrc(ksc + (int64_t)kv0 * (D / 32), (rows * (D / 32) + 3) & ~3), l * 4, slot + C::KT);
  };
  auto issue_v = [&](char* slot, int j) {
    const int kv0 = j * C::BN, nb = (min(C::BN, lk - kv0) + 31) / 32;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(vx + (int64_t)(2 * j) * (D * 32)), 0, nb * D * 32, kBufferWord3);
#pragma unroll
    for (int i = 0; i < C::N; ++i) buffer_load_lds16(r, voff[i], slot + (i * C::NT + wave0) * 16);
    if (w == 1) buffer_load_lds4(uniform_rsrc(vsc + (int64_t)(2 * j) * D, nb * D), l * 4, slot + C::VT);
  };

  if (n_kv > 0) {
    issue_k(kslot0, 0);
    issue_v(vslot0, 0);
  }
  if (n_kv > 1) issue_k(kslot0 + C::KSLOT, 1);

  // Q fragments (B operand of S^T): product i takes head-dim elements
  // 64i + 16g .. +15 and 64i + 32 + 16g .. +15; the lane's scale word
  // shifted so that byte 2i is the scale of block 2i + g
  i32x8 qf[C::NK];
  uint32_t qsc;
  {
    const int r = min(my_row, lq - 1);
    const uint8_t* qp = a.qx + ((int64_t)h * a.rq + qrow0 + r) * D + 16 * g;
#pragma unroll
    for (int i = 0; i < C::NK; ++i)
      qf[i] = cat8(*reinterpret_cast<const u32x4*>(qp + 64 * i), *reinterpret_cast<const u32x4*>(qp + 64 * i + 32));
    qsc = scale_word<D>(a.qs + ((int64_t)h * a.rq + qrow0 + r) * (D / 32)) >> (8 * g);
#pragma unroll
    for (int i = 0; i < C::NK; ++i) settle(qf[i]);
    settle(qsc);
  }

  f32x16 o[C::ND];
#pragma unroll
  for (int i = 0; i < C::ND; ++i) o[i] = f32x16{};
  // running row max (an integer, log2 units) and sum of the exact weights
  float m_run = -INFINITY, l_run = 0.f;

  auto wave_active = [&](int j) { return wave_live && (!a.causal || j * C::BN <= row0 + 31 + off); };

  // S^T (64 keys x 32 queries) = K Q^T for the tile in K slot PAR, as two
  // 32-key blocks; a lane's K scale word is shifted like its Q word
  auto scores = [&](auto PAR, f32x16* s) {
    const char* kt = kslot0 + decltype(PAR)::value * C::KSLOT;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = 32 * c + c32;
      const uint32_t sk = scale_word<D>(reinterpret_cast<const uint8_t*>(kt + C::KT) + row * (D / 32)) >> (8 * g);
      s[c] = f32x16{};
      mma_mx<0, 0>(s[c], cat8(lds16(kt + mx_k_off<D>(row, g)), lds16(kt + mx_k_off<D>(row, 2 + g))), qf[0], sk, qsc);
      if constexpr (C::NK > 1)
        mma_mx<2, 2>(s[c], cat8(lds16(kt + mx_k_off<D>(row, 4 + g)), lds16(kt + mx_k_off<D>(row, 6 + g))), qf[1], sk,
                     qsc);
    }
  };

  // register r of score block c holds key 32c + 8(r/4) + 4g + r%4 of the tile
  const int row_limit = a.causal ? min(lk, my_row + off + 1) : lk;
  auto needs_mask = [&](int j) {
    const int kv0 = j * C::BN;
    return (kv0 + C::BN > lk) || (a.causal && kv0 + C::BN - 1 > row0 + off);
  };

  // Tile j in two halves, the scores of tile j+1 issued between them: the
  // masks, block maxima and lazy rescale (returns the two blocks' maxima in
  // log2 units); then the weights quantised into the P^T operand and
  // O^T += V^T P^T.  Each call site is single, so that the score and output
  // accumulators are written in place.
  struct BlockMax {
    float b0, b1;
  };
  auto tile_max = [&](auto MASK, f32x16* s, int j) {
    if constexpr (decltype(MASK)::value) {
      const int lim = row_limit - j * C::BN - 4 * g;   // masked iff key offset >= lim
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[c][r] -= (32 * c + 8 * (r >> 2) + (r & 3) >= lim) ? kMaskShift : 0.f;
      }
    }
    // the max of each 32-key block (one MX block of P): 16 keys here, 16 in
    // the other half of the wave
    float b0 = s[0][0], b1 = s[1][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      b0 = fmaxf(b0, s[0][r]);
      b1 = fmaxf(b1, s[1][r]);
    }
    return BlockMax{xor32_max(b0) * a.scale_log2, xor32_max(b1) * a.scale_log2};
  };
  auto rescale = [&](const BlockMax& bm) {
    const float mx = fmaxf(bm.b0, bm.b1);
    // lazy rescale, the max rounded up to an integer
    const bool grow = mx > m_run + kLazyRescale;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_use = grow ? ceilf(fmaxf(mx, kMaxFloor)) : m_run;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_use;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < C::ND; ++i) o[i] *= alpha;
    }
  };
  auto tile_pv = [&](auto PAR, const f32x16* s, const BlockMax& bm) {
    constexpr int kPar = decltype(PAR)::value;
    const float f0 = fmaxf(floorf(bm.b0), m_run - kMxFloorGap);
    const float f1 = fmaxf(floorf(bm.b1), m_run - kMxFloorGap);
    // elements 2^(t - floor + 8) of each block, their exact sums, the codes
    float sum0 = 0.f, sum1 = 0.f;
    i32x8 pc;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float nc = 8.f - (c == 0 ? f0 : f1);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = fast_exp2(fmaf(s[c][4 * q + i], a.scale_log2, nc));
        if (c == 0) sum0 += (e[0] + e[1]) + (e[2] + e[3]);
        else sum1 += (e[0] + e[1]) + (e[2] + e[3]);
        pc[4 * c + q] = (int)fp8x4_pos(e[0], e[1], e[2], e[3]);
      }
    }
    l_run += ldexpf(sum0, (int)(f0 - m_run) - 8) + ldexpf(sum1, (int)(f1 - m_run) - 8);
    // this half's block scale: 2^(floor - m - 8)
    const uint32_t sp = (uint32_t)((int)((g ? f1 : f0) - m_run) + 119);
    const char* vt = vslot0 + kPar * C::VSLOT;
    const uint32_t sv = scale_word<D>(reinterpret_cast<const uint8_t*>(vt + C::VT) + g * D + c32 * (D / 32));
    auto pv = [&](auto DT) {
      constexpr int dt = decltype(DT)::value;
      const int d = 32 * dt + c32;
      mma_mx<dt, 0>(o[dt], cat8(lds16(vt + mx_v_off<D>(0, d, g)), lds16(vt + mx_v_off<D>(1, d, g))), pc, sv, sp);
    };
    pv(std::integral_constant<int, 0>{});
    pv(std::integral_constant<int, 1>{});
    if constexpr (C::ND > 2) {
      pv(std::integral_constant<int, 2>{});
      pv(std::integral_constant<int, 3>{});
    }
  };

  // one pipelined step for key tile j (the bf16 forward's schedule): copy
  // K(j+2) over K(j) and V(j+1) over V(j-1), the maxima of j, the scores of
  // j+1, the weights and P V of j, then wait and barrier
  auto step = [&](auto PAR, int j, f32x16* s_cur, f32x16* s_nxt) {
    constexpr int kPar = decltype(PAR)::value;
    if (j + 2 < n_kv) issue_k(kslot0 + kPar * C::KSLOT, j + 2);
    if (j + 1 < n_kv) issue_v(vslot0 + (1 - kPar) * C::VSLOT, j + 1);
    const bool nxt = j + 1 < n_kv && wave_active(j + 1);
    const bool act = wave_active(j);
    BlockMax bm{0.f, 0.f};
    if (act) {
      bm = needs_mask(j) ? tile_max(std::true_type{}, s_cur, j) : tile_max(std::false_type{}, s_cur, j);
      rescale(bm);
    }
    if (nxt) scores(std::integral_constant<int, 1 - kPar>{}, s_nxt);
    if (act) tile_pv(PAR, s_cur, bm);
    dma_wait();
    __syncthreads();
  };

  dma_wait();
  __syncthreads();
  f32x16 sa[2], sb[2];
  if (n_kv > 0 && wave_active(0)) scores(std::integral_constant<int, 0>{}, sa);
  // the first step copies K(2) over K(0): every wave must be done reading it
  __syncthreads();
  for (int j = 0; j < n_kv; j += 2) {
    step(std::integral_constant<int, 0>{}, j, sa, sb);
    if (j + 1 < n_kv) step(std::integral_constant<int, 1>{}, j + 1, sb, sa);
  }

  if (!wave_live) return;
  const float l_tot = xor32_sum(l_run);
  const bool row_live = my_row < lq && lk > 0 && (!a.causal || my_row + off >= 0);
  const float f = row_live ? 1.0f / l_tot : 0.f;
  const int rs = a.heads * D;
  __bf16* op = static_cast<__bf16*>(a.out) + (size_t)(qs + row0) * rs + (size_t)h * D;
  store_rows_lds<__bf16, D>(op, rs, min(32, lq - row0), o, f, smem + w * store_scratch_bytes<__bf16, D>());
  if (g == 0 && my_row < lq)
    a.lse[(size_t)h * a.total_q + qs + my_row] = row_live ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template __global__ void mx_fwd_kernel<64, 4>(MxFwdArgs);
template __global__ void mx_fwd_kernel<128, 4>(MxFwdArgs);
template __global__ void mx_fwd_kernel<64, 2>(MxFwdArgs);
template __global__ void mx_fwd_kernel<128, 2>(MxFwdArgs);

// narrow: every sequence has at most 64 queries, so every item of the
// forward list is tile 0 and two waves cover its rows.
hipError_t launch_mx_fwd(const MxFwdArgs& a, int head_dim, bool narrow, int64_t grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  const dim3 g((unsigned)grid);
  if (head_dim == 64 && narrow) hipLaunchKernelGGL((mx_fwd_kernel<64, 2>), g, dim3(128), 0, stream, a);
  else if (head_dim == 128 && narrow) hipLaunchKernelGGL((mx_fwd_kernel<128, 2>), g, dim3(128), 0, stream, a);
  else if (head_dim == 64) hipLaunchKernelGGL((mx_fwd_kernel<64, 4>), g, dim3(256), 0, stream, a);
  else if (head_dim == 128) hipLaunchKernelGGL((mx_fwd_kernel<128, 4>), g, dim3(256), 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace jfa

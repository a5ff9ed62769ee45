// Shared device helpers of the MXFP8 kernels (mx.hip, mx_bwd.hip): the
// block-scaled product, E8M0 / E4M3 conversions, and the LDS tile layouts of
// row and column images.
//
// Block-scaled product layout (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 on
// both sides, checked on the hardware): lane l holds row l%32 of A (column
// l%32 of B) in 32 bytes; bytes 0..15 of both lane halves form the first
// 32-element k block, bytes 16..31 the second, and byte p of lane half g
// meets byte p of the same half of the other operand.  The scale of row
// (column) r for k block kb is byte `opsel` of lane r + 32 kb's scale
// register.  The accumulator layout is that of the bf16 products
// (jfa_common.hpp).
#pragma once

#include "jfa_common.hpp"
#include "jfa_internal.h"

namespace jfa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kE4M3Max = 448.f;
// A block's floor is kept at most this far below the row max (log2
// units): its E8M0 scale code floor - m - 8 + 127 then stays at 9 or more.
// Such a block weighs below 2^-100 of the row's largest weight.
constexpr float kMxFloorGap = 110.f;

template <int OA, int OB>
__device__ __forceinline__ void mma_mx(f32x16& acc, const i32x8& a, const i32x8& b, uint32_t sa, uint32_t sb) {
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, OA, (int)sa, OB, (int)sb);
}

// E8M0 code of a block whose largest magnitude is amax: floor(log2 amax) -
// 8, biased by 127, at least 0 (amax zero or below 2^-119).  For a normal
// amax floor(log2 amax) + 127 is its exponent field.
__device__ __forceinline__ uint32_t e8m0_code(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xff);
  return (uint32_t)max(ef - 8, 0);
}
// 2^(127 - code): takes a block's values to its elements (exact scaling).
__device__ __forceinline__ float e8m0_inverse(uint32_t code) { return __uint_as_float((254u - code) << 23); }

__device__ __forceinline__ float sat(float x) { return fminf(fmaxf(x, -kE4M3Max), kE4M3Max); }

// Four elements into one word (byte i = x_i): nearest even, clamped to 448
// (the conversion turns magnitudes beyond 464 into NaN).
__device__ __forceinline__ uint32_t fp8x4(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(x0), sat(x1), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(x2), sat(x3), w, true);
  return (uint32_t)w;
}
// The same for non-negative values (the weights).
__device__ __forceinline__ uint32_t fp8x4_pos(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(x0, kE4M3Max), fminf(x1, kE4M3Max), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(x2, kE4M3Max), fminf(x3, kE4M3Max), w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ void bf16x2_to_float(uint32_t u, float& lo, float& hi) {
  lo = __uint_as_float(u << 16);
  hi = __uint_as_float(u & 0xffff0000u);
}

// Byte position of key i (0..31) of a block within a column of the column
// image: lane half g of the P V product takes keys 8a + 4g + 0..3 (a =
// 0..3), the accumulator rows its scores arrive in, as 16 consecutive bytes.
__host__ __device__ constexpr int mx_key_pos(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

// NW waves of 32 queries per work item: 4 (the forward list's 128-row
// items), or 2 when no sequence has more than 64 queries (every item is then
// tile 0, rows 0 .. 63, and twice the items fit a compute unit).
template <int D, int NW = 4>
struct MxCfg {
  static constexpr int BM = 32 * NW, BN = kFwdBN, NT = 64 * NW;
  static_assert(NW == 2 || (NW == 4 && BM == kFwdBM), "two or four waves; four cover a forward tile");
  static constexpr int CPR = D / 16;          // 16-byte chunks per K row
  static constexpr int RPL = 256 / D;         // K rows per 256-byte LDS line
  static constexpr int KT = BN * D;           // K tile bytes
  static constexpr int VT = 2 * D * 32;       // V^T tile bytes: two 32-key blocks
  static constexpr int SC = 256;              // scale bytes per tile (one wave's dword copy)
  static constexpr int KSLOT = KT + SC, VSLOT = VT + SC;
  static constexpr int PIPE = 2 * KSLOT + 2 * VSLOT;
  static constexpr int OUT = (NT / kWave) * store_scratch_bytes<__bf16, D>();
  static constexpr int LDS = PIPE > OUT ? PIPE : OUT;
  static constexpr int NK = D / 64;           // block-scaled products per 32-key score block
  static constexpr int ND = D / 32;           // 32-row blocks of O^T
  static constexpr int CH = KT / 16;          // 16-byte chunks per K (and per V) tile
  static constexpr int N = CH / NT;           // copies per thread per tile
  static_assert(CH % NT == 0 && VT == KT, "tile chunks must split evenly over the threads");
};

// K tile in LDS: row r (key) of D bytes, 16-byte chunk c at chunk c ^ f(r),
// f(r) = (r / RPL) % CPR, so that 16 consecutive rows read at one chunk hit
// 16 distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ int mx_k_off(int r, int c) {
  using C = MxCfg<D>;
  return r * D + ((c ^ ((r / C::RPL) % C::CPR)) * 16);
}
// V^T tile in LDS: block c (keys 32c ..), column d, lane half g's 16 bytes
// at half g ^ bit 3 of d (16 consecutive columns at one half: distinct
// bank groups).
template <int D>
__device__ __forceinline__ int mx_v_off(int c, int d, int g) {
  return c * D * 32 + d * 32 + ((g ^ ((d >> 3) & 1)) * 16);
}

__device__ __forceinline__ i32x8 cat8(const u32x4& a, const u32x4& b) {
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ u32x4 lds16(const char* p) { return *reinterpret_cast<const u32x4*>(p); }

template <int D>
__device__ __forceinline__ uint32_t scale_word(const uint8_t* p) {
  if constexpr (D == 128) return *reinterpret_cast<const uint32_t*>(p);
  else return *reinterpret_cast<const uint16_t*>(p);
}

}  // namespace jfa

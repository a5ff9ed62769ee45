// Shared device helpers of the jagged attention kernels (gfx950 / CDNA4).
//
// Register layouts used throughout (v_mfma_f32_32x32x16_bf16, checked on the
// hardware; the fp32 path runs eight v_mfma_f32_32x32x2_f32 over the same
// fragment layout):
//   A operand (32 x 16):  lane l holds row l%32, k-slots 8*(l/32) + 0..7
//   B operand (16 x 32):  lane l holds column l%32, k-slots 8*(l/32) + 0..7
//   C/D (32 x 32, f32x16): lane l, register r holds
//                          row 8*(r/4) + 4*(l/32) + r%4, column l%32
// A "fragment" is the 8 k-slot values one lane contributes to an A or B
// operand.  Any permutation of k applied to both operands leaves a product
// unchanged; the kernels use that freedom so that an accumulator tile can be
// fed straight back as the B operand of the next product (see swap23 below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Masked scores are pushed down by this finite amount instead of being
// replaced by -inf: exp2 of (score - kMaskShift - rowmax) is exactly 0 in
// fp32 for any finite score, and no inf/NaN ever enters the running max.
constexpr float kMaskShift = 1.0e30f;
// The online softmax keeps a stale row max until the true max exceeds it by
// more than this (log2 units): weights then stay below 2^8, and O is rescaled
// only when a row's max really moves.
constexpr float kLazyRescale = 8.0f;
// Lower bound of the running max (log2 units): masked scores sit near
// -1.3e29 after scaling, so a fully masked row's weights exp2(x - max) stay 0.
constexpr float kMaxFloor = -1.0e20f;

constexpr int kWave = 64;

#define JFA_LDS __attribute__((address_space(3)))

template <typename T> struct Frag;
template <> struct Frag<__bf16> { using type = bf16x8; };
template <> struct Frag<float> { using type = f32x8; };
template <typename T> using frag_t = typename Frag<T>::type;

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Rows of a 32-row tile are stored (and produced) in an order whose bits 2
// and 3 are swapped.  With that order, accumulator register 8*s + e of lane
// group g = l/32 in a 32 x 32 C tile sits at logical row 16*s + 8*g + e, i.e.
// the 8 consecutive k-slots of a B-operand fragment.
__host__ __device__ constexpr int swap23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- MFMA

__device__ __forceinline__ void mma(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], acc, 0, 0, 0);
}

// ---------------------------------------------------------------- conversions

__device__ __forceinline__ bf16x8 to_frag_bf16(const float* x) {
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (__bf16)x[e];
  return f;
}

template <typename T>
__device__ __forceinline__ frag_t<T> pack_frag(const f32x16& acc, int s) {
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = acc[8 * s + e];
  if constexpr (sizeof(T) == 2) {
    return to_frag_bf16(x);
  } else {
    f32x8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = x[e];
    return f;
  }
}

// acc += sum of the 8 values of a fragment as it will enter the MFMA: one
// v_dot2c_f32_bf16 against (1.0, 1.0) per packed word, chained through the
// accumulator.  Issued as one inline-assembly block on plain 32-bit words
// (through the builtin's bf16-pair vector type this toolchain fed the first
// word to all four instructions).  The block ends with the 3 wait states a
// DOT result needs before another VALU instruction may read it; the
// compiler cannot insert them for inline assembly.
__device__ __forceinline__ void frag_sum_into(float& acc, const bf16x8& f) {
  const u32x4 w = __builtin_bit_cast(u32x4, f);
  const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
  asm("v_dot2c_f32_bf16 %0, %1, %2\n\t"
      "v_dot2c_f32_bf16 %0, %1, %3\n\t"
      "v_dot2c_f32_bf16 %0, %1, %4\n\t"
      "v_dot2c_f32_bf16 %0, %1, %5\n\t"
      "s_nop 2"
      : "+v"(acc)
      : "s"(0x3f803f80u), "v"(w0), "v"(w1), "v"(w2), "v"(w3));
}
__device__ __forceinline__ void frag_sum_into(float& acc, const f32x8& f) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc += f[i];
}

// ---------------------------------------------------------------- LDS access

// Dense LDS tiles of D-element rows, addressed in 16-byte chunks whose index
// is XOR-swizzled with a function of the row.  With 64 banks of 4 bytes a
// 256-byte line is served per cycle; the swizzle makes both read patterns
// of the kernels hit 16 distinct 16-byte bank groups:
//   - 16 consecutive rows, one chunk each (A/B operand rows, ds_read_b128);
//   - 4 consecutive aligned rows, 4 consecutive aligned chunks each
//     (transposed operand reads, ds_read_b64_tr_b16 over a half-wave).
template <typename T, int D>
struct Swz {
  static constexpr int CH = D * (int)sizeof(T) / 16;   // chunks per row
  static constexpr int ROW_BYTES = CH * 16;
  // byte offset of chunk c of row r
  __host__ __device__ static constexpr int off(int r, int c) {
    if constexpr (CH >= 16) {
      const int g = ((r & 3) << 2) ^ ((r >> 2) & 3);
      return r * ROW_BYTES + ((c & ~15) | ((c & 15) ^ g)) * 16;
    } else if constexpr (CH == 8) {            // two rows per 256-byte line
      const int line = r >> 1;
      const int g = ((line & 1) << 2) ^ ((line >> 1) & 3);
      return line * 256 + (((r & 1) << 3) | (c ^ g)) * 16;
    } else {                                   // CH == 4: four rows per line
      static_assert(CH == 4, "unsupported row size");
      const int line = r >> 2;
      return line * 256 + (((r & 3) << 2) | (c ^ (line & 3))) * 16;
    }
  }
  static constexpr int tile_bytes(int rows) { return rows * ROW_BYTES; }
  // inverse: physical 16-byte chunk index p -> (row r, chunk c)
  __device__ static __forceinline__ void inv(int p, int& r, int& c) {
    if constexpr (CH >= 16) {
      r = p / CH;
      const int g = ((r & 3) << 2) ^ ((r >> 2) & 3);
      const int q = p % CH;
      c = (q & ~15) | ((q & 15) ^ g);
    } else if constexpr (CH == 8) {
      const int line = p >> 4;
      r = 2 * line + ((p >> 3) & 1);
      c = (p & 7) ^ (((line & 1) << 2) ^ ((line >> 1) & 3));
    } else {
      const int line = p >> 4;
      r = 4 * line + ((p >> 2) & 3);
      c = (p & 3) ^ (line & 3);
    }
  }
};

// 8 consecutive elements (col .. col+7, col a multiple of 8) of row
// row0 + row, row0 a multiple of 16 (an immediate offset: the swizzle of a
// row depends on its low four bits only).
template <typename T, int D>
__device__ __forceinline__ frag_t<T> lds_row_frag(const char* tile, int row0, int row, int col) {
  using S = Swz<T, D>;
  tile += row0 * S::ROW_BYTES;
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tile + S::off(row, col >> 3)));
  } else {
    const u32x4 a = *reinterpret_cast<const u32x4*>(tile + S::off(row, col >> 2));
    const u32x4 b = *reinterpret_cast<const u32x4*>(tile + S::off(row, (col >> 2) + 1));
    f32x8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = __uint_as_float(a[e]);
      f[4 + e] = __uint_as_float(b[e]);
    }
    return f;
  }
}

// Transposed fragment: lane l gets the elements at logical rows
// row0 + 8*(l/32) + 0..7 of column col0 + l%32 (row0 a multiple of 16, col0
// a multiple of 32).  With SWAPPED, logical row r is stored at row swap23(r)
// (swap23 keeps aligned groups of four rows together).
// The swizzle of a row depends on its low four bits only and swap23 moves
// bits 2 and 3, so rows row0 + x sit at row0 * ROW_BYTES plus the offsets
// of rows x: the lane-dependent part is the same for every row0, and row0
// becomes an immediate offset of the read.
template <typename T, int D, bool SWAPPED>
__device__ __forceinline__ frag_t<T> lds_col_frag(const char* tile, int row0, int col0) {
  using S = Swz<T, D>;
  const int l = lane_id();
  tile += row0 * S::ROW_BYTES;
  row0 = 0;
  if constexpr (sizeof(T) == 2) {
    // ds_read_b64_tr_b16 (layout checked on the hardware): within each
    // 16-lane block, source lane s addresses the 4 elements at row r0 + s/4,
    // columns c0 + 4*(s%4) .. +3; output lane o receives column c0 + o at
    // rows r0 .. r0+3.  Two reads give the 8 rows of a fragment.
    const int blk = l >> 4, s = l & 15;
    const int g = blk >> 1, half = blk & 1;
    const int col = col0 + 16 * half + 4 * (s & 3);      // element column
    const int chunk = col >> 3, within = (col & 7) * 2;  // 16-byte chunk, byte in it
    u32x2 w[2];
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      int row = row0 + 8 * g + 4 * rd + (s >> 2);
      if (SWAPPED) row = swap23(row);
      const char* p = tile + S::off(row, chunk) + within;
      // whole 32-bit words only: per-element bf16 extraction of this
      // builtin's result is not compiled correctly by this toolchain
      w[rd] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((JFA_LDS i16x4*)(p)));
    }
    const u32x4 words = {w[0][0], w[0][1], w[1][0], w[1][1]};
    return __builtin_bit_cast(bf16x8, words);
  } else {
    const int g = l >> 5, c = col0 + (l & 31);
    f32x8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int row = row0 + 8 * g + e;
      if (SWAPPED) row = swap23(row);
      f[e] = *reinterpret_cast<const float*>(tile + S::off(row, c >> 2) + (c & 3) * 4);
    }
    return f;
  }
}

// One address register per operand.  In every swizzle above, moving a
// read by whole 16-column steps (row fragments), by whole 32-column blocks
// or to the second four rows (transposed fragments) flips address bits that
// the first read of each lane leaves fixed: every read is that first
// address XOR a compile-time constant.  valid() checks this for every lane.
// A kernel that refreshes the base inside its loop (see refresh) recomputes
// the reads' addresses with one XOR each instead of holding one register per
// read across the loop.
template <typename T, int D>
struct RowFragAddr {
  using S = Swz<T, D>;
  // lane l's read of columns 16*kk + 8*(l/32) .. +7 of row l%32
  __host__ __device__ static constexpr int lane_off(int l, int kk) {
    return S::off(l & 31, (16 * kk + 8 * (l >> 5)) * (int)sizeof(T) / 16);
  }
  __host__ __device__ static constexpr int xor_k(int kk) { return lane_off(0, kk) ^ lane_off(0, 0); }
  static constexpr bool valid() {
    for (int l = 0; l < kWave; ++l)
      for (int kk = 0; kk < D / 16; ++kk)
        if (lane_off(l, kk) != (lane_off(l, 0) ^ xor_k(kk))) return false;
    return true;
  }
  __device__ static __forceinline__ int base() { return lane_off(lane_id(), 0); }
};

template <typename T, int D, bool SWAPPED>
struct ColFragAddr {
  using S = Swz<T, D>;
  // lane l's rd-th ds_read_b64_tr_b16 of column block cb (layout as in
  // lds_col_frag), rows 0..15 of the tile
  __host__ __device__ static constexpr int lane_off(int l, int cb, int rd) {
    const int blk = l >> 4, s = l & 15, g = blk >> 1, half = blk & 1;
    const int col = 32 * cb + 16 * half + 4 * (s & 3);
    const int row = 8 * g + 4 * rd + (s >> 2);
    return S::off(SWAPPED ? swap23(row) : row, col >> 3) + (col & 7) * 2;
  }
  __host__ __device__ static constexpr int xor_k(int cb, int rd) { return lane_off(0, cb, rd) ^ lane_off(0, 0, 0); }
  static constexpr bool valid() {
    for (int l = 0; l < kWave; ++l)
      for (int cb = 0; cb < D / 32; ++cb)
        for (int rd = 0; rd < 2; ++rd)
          if (lane_off(l, cb, rd) != (lane_off(l, 0, 0) ^ xor_k(cb, rd))) return false;
    return true;
  }
  __device__ static __forceinline__ int base() { return lane_off(lane_id(), 0, 0); }
};

// An opaque copy of an address base: the compiler cannot hoist what is
// computed from it out of the loop it is refreshed in.
__device__ __forceinline__ int refresh(int base) {
  asm volatile("" : "+v"(base));
  return base;
}

// lds_row_frag of row row0 + l%32, columns 16*kk + 8*(l/32) .. +7, from a
// RowFragAddr base (bf16 only).
template <typename T, int D>
__device__ __forceinline__ frag_t<T> lds_row_frag_x(const char* tile, int row0, int kk, int base) {
  static_assert(sizeof(T) == 2 && RowFragAddr<T, D>::valid(), "XOR addressing needs bf16 rows");
  const char* p = tile + row0 * Swz<T, D>::ROW_BYTES + (base ^ RowFragAddr<T, D>::xor_k(kk));
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// lds_col_frag(tile, row0, 32 * cb) from a ColFragAddr base (bf16 only).
template <typename T, int D, bool SWAPPED>
__device__ __forceinline__ frag_t<T> lds_col_frag_x(const char* tile, int row0, int cb, int base) {
  using A = ColFragAddr<T, D, SWAPPED>;
  static_assert(sizeof(T) == 2 && A::valid(), "XOR addressing needs bf16 rows");
  tile += row0 * Swz<T, D>::ROW_BYTES;
  u32x2 w[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd)
    w[rd] = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((JFA_LDS i16x4*)(tile + (base ^ A::xor_k(cb, rd)))));
  const u32x4 words = {w[0][0], w[0][1], w[1][0], w[1][1]};
  return __builtin_bit_cast(bf16x8, words);
}

// ---------------------------------------------------------------- cross-lane

__device__ __forceinline__ float xor32_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xor32_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// ---------------------------------------------------------------- tile staging

// Buffer-resource word 3 for raw (untyped, unswizzled) dword buffer access.
constexpr int kBufferWord3 = 0x00020000;

// A ROWS x D tile of one head read from global memory into registers with
// raw buffer loads (16 bytes per access) and written to a swizzled LDS tile.
// The buffer of each load covers only the rows that belong to the sequence,
// so rows past its end read as zeros: nothing outside the sequence is read,
// and no per-row clamp or 64-bit address arithmetic is needed.  With SWAP,
// row r is stored at row swap23(r).
template <typename T, int D, int ROWS, bool SWAP, int NT = 256>
struct TileStage {
  using S = Swz<T, D>;
  static constexpr int CH = S::CH;
  static constexpr int N = ROWS * CH / NT;
  static_assert(ROWS * CH % NT == 0, "tile must split evenly over the threads");
  u32x4 r[N];

  // rows row0 .. row0+ROWS-1 of a sequence whose row j starts at
  // base + j*row_stride elements and which has nrows rows (row0 < nrows)
  __device__ __forceinline__ void load(const T* base, int row_stride, int row0, int nrows, int tid) {
    const int valid = min(ROWS, nrows - row0);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(base + (size_t)row0 * row_stride), 0, valid * row_stride * (int)sizeof(T), kBufferWord3);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + i * NT, row = c / CH, col = c % CH;
      r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rsrc, row * row_stride * (int)sizeof(T) + col * 16, 0, 0));
    }
  }
  __device__ __forceinline__ void store(char* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + i * NT, row = c / CH, col = c % CH;
      *reinterpret_cast<u32x4*>(tile + S::off(SWAP ? swap23(row) : row, col)) = r[i];
    }
  }
};

// One buffer load that writes LDS: every lane reads 16 bytes at byte offset
// `voff` of the buffer and the wave's 64 chunks land at lds .. lds + 1023
// (lane order).  Issued as inline assembly on purpose: for the builtin form
// the compiler cannot tell which LDS bytes the copy writes, and makes every
// later LDS read wait for all copies in flight, which would serialise the
// copies of stages that are meant to stay in flight behind the compute.
// Completion is the caller's business (vector-memory counter, then barrier).
// The assembly starts with 5 wait states: the buffer descriptor's scalar
// registers may have just been written by a vector instruction
// (readfirstlane), which a vector-memory read of them must not follow
// sooner, and M0 may have just been written by a scalar instruction, which
// an LDS copy must not follow in the next cycle.  The compiler inserts these
// waits for its own instructions but cannot see into inline assembly.
// NT: non-temporal (streaming) cache policy, for data read exactly once.
template <bool NT = false>
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, int voff, const char* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(JFA_LDS const char*)lds;   // the compiler moves it to M0
  if constexpr (NT)
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rsrc), "{m0}"(m0) : "memory");
  else
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(m0) : "memory");
}

// Raw buffer resource over `bytes` bytes at `base`, for values that are
// uniform across each wave but that the compiler cannot prove uniform (they
// depend on the wave index): passing them through readfirstlane lets it keep
// the descriptor in scalar registers, which the buffer instructions need.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int n = __builtin_amdgcn_readfirstlane(bytes);
  void* p = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, n, kBufferWord3);
}

// A ROWS x D tile of one head copied straight from global memory into a
// swizzled LDS tile with buffer loads that write LDS (no register staging).
// Each such load writes its 64 lanes' 16-byte chunks to 1 KB of consecutive
// LDS, so every lane loads the global chunk that the swizzle maps to its LDS
// slot.  Rows past the sequence's end read as zeros (the buffer covers only
// the sequence's rows).  With SWAP, LDS row r holds tile row swap23(r).
// When the tile has fewer chunks than N * NT, the surplus waves still issue
// their loads (so that every wave issues the same number), reading past the
// buffer (zeros) into `sink`, 1 KB of LDS per wave of the workgroup (each
// wave writes only its own KB).  Completion is tracked by the
// wave's vector-memory counter: wait for it and then barrier before any wave
// reads the tile.
template <typename T, int D, int ROWS, bool SWAP, int NT = 256>
struct TileDma {
  using S = Swz<T, D>;
  static constexpr int CH = S::CH;
  static constexpr int CHUNKS = ROWS * CH;
  static constexpr int N = (CHUNKS + NT - 1) / NT;   // loads per thread per tile
  static_assert(CHUNKS % kWave == 0, "a wave's loads must be all in the tile or all surplus");
  static constexpr int kPastEnd = 0x7ffffff0;        // offset beyond any buffer: reads zeros
  int voff[N];                                       // per-thread byte offsets into the tile's rows

  __device__ __forceinline__ void init(int row_stride, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int p = i * NT + tid;
      if (p < CHUNKS) {
        int r, c;
        S::inv(p, r, c);
        const int row = SWAP ? swap23(r) : r;
        voff[i] = row * row_stride * (int)sizeof(T) + c * 16;
      } else {
        voff[i] = kPastEnd;
      }
    }
  }
  // rows row0 .. row0+ROWS-1 of a sequence whose row j starts at
  // base + j*row_stride elements and which has nrows rows (row0 < nrows)
  __device__ __forceinline__ void issue(char* tile, const T* base, int row_stride, int row0, int nrows, int tid,
                                        char* sink = nullptr) const {
    const int valid = min(ROWS, nrows - row0);
    // base, row0 and nrows are uniform across the workgroup, so the
    // compiler keeps the descriptor in scalar registers
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T*>(base + (size_t)row0 * row_stride), 0, valid * row_stride * (int)sizeof(T), kBufferWord3);
    const int wave0 = tid & ~(kWave - 1);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const bool real = (N * NT == CHUNKS) || (i * NT + wave0 < CHUNKS);
      buffer_load_lds16(rsrc, voff[i], real ? tile + (i * NT + wave0) * 16 : sink + wave0 * 16);
    }
  }
};

// Workgroup barrier ordering LDS only: this wave's LDS reads and writes
// complete before it, and later LDS accesses stay after it.  Unlike
// __syncthreads it does not wait for the wave's global loads and stores
// (vector memory shares one counter with the LDS copies), so copies and
// loads issued for a later step, and stores to global memory, stay in
// flight across it.  For use where nothing in global memory passes between
// the workgroup's waves; copies into LDS are waited for explicitly
// (dma_wait*) before it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wait until this wave's outstanding global->LDS copies have landed.
__device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N of this wave's vector-memory operations are still in
// flight (they complete in issue order): the copies issued before the last N
// have landed.
template <int N>
__device__ __forceinline__ void dma_wait_all_but() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Makes the compiler wait here for the register load that produced x.  Its
// own wait bookkeeping cannot see the inline-assembly LDS copies; settling
// every register load before a loop keeps it from inserting waits inside
// the loop, where they would also drain the copies meant to stay in flight.
template <typename X>
__device__ __forceinline__ void settle(const X& x) {
  asm volatile("" ::"v"(x));
}

// One buffer load that writes LDS with 4 bytes per lane: lane l's dword
// lands at lds + 4*l (256 bytes per wave).  Same contract and the same
// leading wait states as buffer_load_lds16.
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t rsrc, int voff, const char* lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(JFA_LDS const char*)lds;   // the compiler moves it to M0
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(m0) : "memory");
}

// Per-row values base[row0 .. row0+63] of a sequence with nrows rows copied
// into this wave's own 256 bytes of LDS at `dst` (rows past the sequence
// read as zeros).  Each wave copies into a region no other wave writes.
__device__ __forceinline__ void rows_dma(char* dst, const float* base, int row0, int nrows) {
  buffer_load_lds4(uniform_rsrc(base + row0, min(64, nrows - row0) * (int)sizeof(float)), lane_id() * 4, dst);
}

template <typename T>
__device__ __forceinline__ frag_t<T> global_frag(const T* p) {
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
  } else {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p);
    const u32x4 b = *reinterpret_cast<const u32x4*>(p + 4);
    f32x8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = __uint_as_float(a[e]);
      f[4 + e] = __uint_as_float(b[e]);
    }
    return f;
  }
}

// Store 4 consecutive output elements (rounded to nearest even for bf16).
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ void store4(T* p, float x0, float x1, float x2, float x3) {
  if constexpr (sizeof(T) == 2) {
    bf16x4 f;
    f[0] = (__bf16)x0;
    f[1] = (__bf16)x1;
    f[2] = (__bf16)x2;
    f[3] = (__bf16)x3;
    *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, f);
  } else {
    f32x4 f = {x0, x1, x2, x3};
    *reinterpret_cast<f32x4*>(p) = f;
  }
}

// Write a D x 32 accumulator block set (ND blocks of 32 x 32, lane = column)
// as the lane's row of a [rows, heads, D] tensor, times f.
template <typename T, int ND>
__device__ __forceinline__ void store_row(T* row, const f32x16* acc, float f) {
  const int g = lane_id() >> 5;
  // register r of block dt holds element d = 32*dt + 8*(r/4) + 4*g + r%4
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      store4<T>(row + 32 * dt + 8 * q4 + 4 * g, acc[dt][4 * q4] * f, acc[dt][4 * q4 + 1] * f,
                acc[dt][4 * q4 + 2] * f, acc[dt][4 * q4 + 3] * f);
    }
  }
}

// Bytes of the per-wave LDS staging that store_rows_lds needs.
template <typename T, int D>
constexpr int store_scratch_bytes() {
  return 32 * (D * (int)sizeof(T) + 16);
}

// The same rows as store_row -- 32 rows starting at `base`, row i at
// base + i*row_stride elements, of which the first `nvalid` exist; lane
// l%32 owns row l%32 and register r of block dt holds element
// 32*dt + 8*(r/4) + 4*g + r%4, times the lane's `f` -- written with stores
// that cover whole rows: the wave assembles the rows in its own `scratch`
// (store_scratch_bytes of LDS, written by no other wave), then each 16-byte
// store lands next to its neighbours' in HBM.
template <typename T, int D>
__device__ __forceinline__ void store_rows_lds(T* base, int row_stride, int nvalid, const f32x16* acc, float f,
                                               char* scratch) {
  constexpr int ND = D / 32;
  constexpr int RB = D * (int)sizeof(T);   // bytes of one row
  constexpr int RS = RB + 16;              // padded LDS row stride
  const int l = lane_id(), g = l >> 5, c32 = l & 31;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      char* p = scratch + c32 * RS + (32 * dt + 8 * q4 + 4 * g) * (int)sizeof(T);
      const float x0 = acc[dt][4 * q4] * f, x1 = acc[dt][4 * q4 + 1] * f;
      const float x2 = acc[dt][4 * q4 + 2] * f, x3 = acc[dt][4 * q4 + 3] * f;
      if constexpr (sizeof(T) == 2) {
        bf16x4 v;
        v[0] = (__bf16)x0;
        v[1] = (__bf16)x1;
        v[2] = (__bf16)x2;
        v[3] = (__bf16)x3;
        *reinterpret_cast<u32x2*>(p) = __builtin_bit_cast(u32x2, v);
      } else {
        *reinterpret_cast<f32x4*>(p) = f32x4{x0, x1, x2, x3};
      }
    }
  }
  constexpr int CPR = RB / 16;             // 16-byte chunks per row
#pragma unroll
  for (int i = 0; i < 32 * CPR / kWave; ++i) {
    const int k = i * kWave + l, row = k / CPR, ch = k % CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(scratch + row * RS + ch * 16);
    if (row < nvalid) *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(base + (size_t)row * row_stride) + ch * 16) = v;
  }
}

// ---------------------------------------------------------------- rotary embedding

// BlockAttention's fused rotary embedding (rotate-half pairing): dimension
// i < d/2 of a Q or K row pairs with i + d/2, and the pair turns by angle
// p * theta_i at position p, theta_i = base^(-2i/d).  Angles are handled in
// revolutions, which is what the hardware sine and cosine take (their range,
// +-256 revolutions, covers positions within a block of 64 tokens with room
// to spare).  inverse turns the other way (the transpose of the rotation,
// for gradients).
__device__ __forceinline__ void rope_rotate(float& a, float& b, float rev, bool inverse) {
  const float c = __builtin_amdgcn_cosf(rev), s0 = __builtin_amdgcn_sinf(rev);
  const float s = inverse ? -s0 : s0;
  const float x = a * c - b * s, y = b * c + a * s;
  a = x;
  b = y;
}

// theta_i / (2 pi) for eight consecutive pairs i0 .. i0 + 7: one exp2, then
// the constant ratio base^(-2/d) between neighbours.  k2 = -2 log2(base) / d.
__device__ __forceinline__ void rope_revs8(int i0, float k2, float* rev) {
  constexpr float kInv2Pi = 0.15915494309189535f;
  const float step = __builtin_amdgcn_exp2f(k2);
  float th = __builtin_amdgcn_exp2f((float)i0 * k2) * kInv2Pi;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    rev[e] = th;
    th *= step;
  }
}

__device__ __forceinline__ void unpack_bf16x8(const u32x4& u, float* v) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(u[e] << 16);
    v[2 * e + 1] = __uint_as_float(u[e] & 0xffff0000u);
  }
}

// A row's fragments as the MFMA operands hold them (lane l: d-slots
// 16*kk + 8*(l/32) + e of fragment kk, e = 0..7), turned in place for
// position `pos`: pair (kk, e) with (kk + NK/2, e).  bf16 results are
// rounded to nearest even.
template <int NK>
__device__ __forceinline__ void rope_frags(bf16x8* f, int pos, float k2) {
  const int g = lane_id() >> 5;
#pragma unroll
  for (int kk = 0; kk < NK / 2; ++kk) {
    float a[8], b[8], rev[8];
    unpack_bf16x8(__builtin_bit_cast(u32x4, f[kk]), a);
    unpack_bf16x8(__builtin_bit_cast(u32x4, f[kk + NK / 2]), b);
    rope_revs8(16 * kk + 8 * g, k2, rev);
#pragma unroll
    for (int e = 0; e < 8; ++e) rope_rotate(a[e], b[e], (float)pos * rev[e], false);
    f[kk] = to_frag_bf16(a);
    f[kk + NK / 2] = to_frag_bf16(b);
  }
}

// Every row of a swizzled LDS tile of `rows` rows (bf16, D columns; with
// SWAPPED, LDS row r holds tile row swap23(r)) turned in place, tile row t
// at position pos0 + t; the nt threads of the workgroup share the work.
// The caller waits for the tile to land and barriers before and after.
template <int D, bool SWAPPED>
__device__ __forceinline__ void rope_lds_tile(char* tile, int rows, int pos0, float k2, int tid, int nt) {
  using S = Swz<__bf16, D>;
  constexpr int HC = S::CH / 2;   // 16-byte chunks in half a row
  for (int u = tid; u < rows * HC; u += nt) {
    const int r = u / HC, c = u % HC;
    const int pos = pos0 + (SWAPPED ? swap23(r) : r);
    u32x4* pa = reinterpret_cast<u32x4*>(tile + S::off(r, c));
    u32x4* pb = reinterpret_cast<u32x4*>(tile + S::off(r, c + HC));
    float a[8], b[8], rev[8];
    unpack_bf16x8(*pa, a);
    unpack_bf16x8(*pb, b);
    rope_revs8(8 * c, k2, rev);
#pragma unroll
    for (int e = 0; e < 8; ++e) rope_rotate(a[e], b[e], (float)pos * rev[e], false);
    *pa = __builtin_bit_cast(u32x4, to_frag_bf16(a));
    *pb = __builtin_bit_cast(u32x4, to_frag_bf16(b));
  }
}

// Accumulator blocks of one row per lane (lane l%32 = row, register r of
// block dt = element 32*dt + 8*(r/4) + 4*(l/32) + r%4) turned back in place
// (the transpose of the rotation) for the lane's position: pair (dt, r) with
// (dt + ND/2, r).
template <int ND>
__device__ __forceinline__ void rope_acc_inverse(f32x16* acc, int pos, float k2) {
  const int g = lane_id() >> 5;
#pragma unroll
  for (int dt = 0; dt < ND / 2; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float rev[8];
      rope_revs8(32 * dt + 8 * q4 + 4 * g, k2, rev);   // elements i0 .. i0 + 3 used
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * q4 + e;
        float lo = acc[dt][r], hi = acc[dt + ND / 2][r];
        rope_rotate(lo, hi, (float)pos * rev[e], true);
        acc[dt][r] = lo;
        acc[dt + ND / 2][r] = hi;
      }
    }
}

// ---------------------------------------------------------------- work items

// Number of `bn`-key blocks a `bm`-query tile visits (forward and dQ).
__device__ __forceinline__ int q_tile_kv_blocks(int lq, int lk, int t, int bm, int bn, int causal) {
  int last_row = min((t + 1) * bm, lq) - 1;
  int kv_end = lk;
  if (causal) kv_end = min(lk, max(0, last_row + lk - lq + 1));
  return ceil_div(kv_end, bn);
}

// Number of `bm`-query blocks a `bn`-key tile visits (dK/dV), and the first.
__device__ __forceinline__ int kv_tile_first_q_block(int lq, int lk, int t, int bm, int bn, int causal) {
  if (!causal) return 0;
  int first_row = max(0, t * bn - (lk - lq));
  return first_row / bm;
}
__device__ __forceinline__ int kv_tile_q_blocks(int lq, int lk, int t, int bm, int bn, int causal) {
  int nqb = ceil_div(lq, bm);
  if (!causal) return nqb;
  int first_row = max(0, t * bn - (lk - lq));
  return first_row < lq ? nqb - first_row / bm : 0;
}

}  // namespace jfa

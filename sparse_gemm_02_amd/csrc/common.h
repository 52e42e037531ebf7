// Shared device helpers of the SLoPe 2:4 library (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace slope {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ----------------------------------------------------------------- magnitudes
// Magnitude order key of a raw value: the absolute-value bits, with every NaN
// collapsed to one key just above +Inf (NaNs rank above numbers and tie).
__device__ __forceinline__ uint32_t mag_key(uint16_t b) {
  uint32_t m = b & 0x7FFFu;
  return m > 0x7F80u ? 0x7F81u : m;
}
// fp16 storage: NaN above the fp16 infinity 0x7C00
__device__ __forceinline__ uint32_t mag_key(_Float16 h) {
  uint32_t m = __builtin_bit_cast(uint16_t, h) & 0x7FFFu;
  return m > 0x7C00u ? 0x7C01u : m;
}
__device__ __forceinline__ uint32_t mag_key(uint32_t b) {
  uint32_t m = b & 0x7FFFFFFFu;
  return m > 0x7F800000u ? 0x7F800001u : m;
}

// 4-bit keep mask of the two largest of four keys; equal keys go to the lower
// position.  rank(j) counts the positions that outrank j: a lower position i
// outranks j when k_i >= k_j, a higher one when k_i > k_j.
__device__ __forceinline__ uint32_t top2_of_4(uint32_t k0, uint32_t k1, uint32_t k2, uint32_t k3) {
  uint32_t c01 = k0 >= k1, c02 = k0 >= k2, c03 = k0 >= k3;
  uint32_t c12 = k1 >= k2, c13 = k1 >= k3, c23 = k2 >= k3;
  uint32_t r0 = 3u - c01 - c02 - c03;
  uint32_t r1 = c01 + 2u - c12 - c13;
  uint32_t r2 = c02 + c12 + 1u - c23;
  uint32_t r3 = c03 + c13 + c23;
  return (uint32_t)(r0 < 2) | ((uint32_t)(r1 < 2) << 1) | ((uint32_t)(r2 < 2) << 2) | ((uint32_t)(r3 < 2) << 3);
}

// Nibble i0 | i1 << 2 of a 4-bit mask holding exactly two positions i0 < i1.
__device__ __forceinline__ uint32_t pair_nibble(uint32_t m) {
  uint32_t i0 = __builtin_ctz(m);
  uint32_t i1 = 31u - __builtin_clz(m);
  return i0 | (i1 << 2);
}

// ----------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float to_f32(uint16_t b) { return bf16_bits_to_f32(b); }
__device__ __forceinline__ float to_f32(uint32_t b) { return __uint_as_float(b); }

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// fp16 storage is the _Float16 type; conversions round to nearest even.
__device__ __forceinline__ float to_f32(_Float16 h) { return (float)h; }
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// Output element stores: uint16_t holds bf16 bits, _Float16 fp16, float fp32.
__device__ __forceinline__ void store_out(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
__device__ __forceinline__ void store_out(_Float16* p, float v) { *p = (_Float16)v; }
__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ float load_out(const uint16_t* p) { return bf16_bits_to_f32(*p); }
__device__ __forceinline__ float load_out(const _Float16* p) { return (float)*p; }
__device__ __forceinline__ float load_out(const float* p) { return *p; }

// 16-bit output patterns: bf16 for uint16_t outputs, fp16 for _Float16 ones.
template <typename O> __device__ __forceinline__ uint16_t out16_bits(float v);
template <> __device__ __forceinline__ uint16_t out16_bits<uint16_t>(float v) { return f32_to_bf16_bits(v); }
template <> __device__ __forceinline__ uint16_t out16_bits<_Float16>(float v) { return f32_to_f16_bits(v); }
// ... and 16-bit output patterns back to fp32.
template <typename O> __device__ __forceinline__ float out16_to_f32(uint32_t bits);
template <> __device__ __forceinline__ float out16_to_f32<uint16_t>(uint32_t b) { return bf16_bits_to_f32((uint16_t)b); }
template <> __device__ __forceinline__ float out16_to_f32<_Float16>(uint32_t b) { return f16_bits_to_f32((uint16_t)b); }

// The two 16-bit input formats of the matrix kernels, selected by H (fp16)
// or not (bf16): operand vectors, conversions of raw 16-bit patterns, and the
// MFMA / sparse MFMA instructions of that format.
template <bool H> struct Fmt16;
template <> struct Fmt16<false> {
  typedef bf16x8 v8;
  typedef bf16x16 v16;
  static __device__ __forceinline__ float to_f32(uint16_t b) { return bf16_bits_to_f32(b); }
  static __device__ __forceinline__ uint16_t from_f32(float f) { return f32_to_bf16_bits(f); }
  static __device__ __forceinline__ f32x16 mfma32x32x16(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16x16x32(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 smfmac32x32x32(v8 a, v16 b, f32x16 c, int idx) {
    return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(a, b, c, idx, 0, 0);
  }
};
template <> struct Fmt16<true> {
  typedef f16x8 v8;
  typedef f16x16 v16;
  static __device__ __forceinline__ float to_f32(uint16_t b) { return f16_bits_to_f32(b); }
  static __device__ __forceinline__ uint16_t from_f32(float f) { return f32_to_f16_bits(f); }
  static __device__ __forceinline__ f32x16 mfma32x32x16(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16x16x32(v8 a, v8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x16 smfmac32x32x32(v8 a, v16 b, f32x16 c, int idx) {
    return __builtin_amdgcn_smfmac_f32_32x32x32_f16(a, b, c, idx, 0, 0);
  }
};

__host__ __device__ constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tile-chunk form of a compressed 16-bit 2:4 matrix [rows, cols], the sparse
// products' operand format: chunk (t, s) holds rows 256t .. 256t+255 and dense
// columns 64s .. 64s+63 at byte offset (t * ceil(cols/64) + s) * kPackChunkBytes;
// first each row's 32 values (64 bytes at row*64, 16-byte granule c at
// c ^ ((row/4) % 4)), then each row's two metadata words (8 bytes at
// kPackValueBytes + row*8); rows past `rows` and columns past `cols` are 0.
constexpr int kPackRows = 256, kPackCols = 64;
constexpr int kPackValueBytes = kPackRows * 64, kPackChunkBytes = kPackValueBytes + kPackRows * 8;
__host__ __device__ constexpr int64_t pack_chunk_offset(int64_t row, int64_t col, int64_t cols) {
  return ((row / kPackRows) * cdiv(cols, kPackCols) + col / kPackCols) * kPackChunkBytes;
}

}  // namespace slope

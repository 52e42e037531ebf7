// Output-tile pieces shared by the sparse GEMM and the standalone adapter
// kernels: tile geometry, the fused low-rank adapter term and the tile store.
//
// A tile is the transposed output Out^T[m][t] (m = output feature, t = token)
// held by a grid of waves in 32 x 32 MFMA accumulators.  Element v of an
// accumulator is row 8*(v/4) + 4*(lane/32) + v%4, column lane%32 (measured
// layout of the gfx950 32x32 MFMA family).
#pragma once
#include "common.h"

namespace slope {

template <int BM_, int BT_, int NST_, int WGM_, int WGT_>
struct Geo {
  static constexpr int BM = BM_, BT = BT_;
  static constexpr int WGM = WGM_, WGT = WGT_, WAVES = WGM * WGT;  // wave grid over the tile
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int WM = BM / WGM, WT = BT / WGT;              // wave tile
  static constexpr int FM = WM / 32, FT = WT / 32;
  static constexpr int KS = 64;                   // dense k per LDS stage (two sparse-MFMA k steps)
  static constexpr int NST = NST_;                // operand stages in the LDS ring
  // stage layout (bytes): A [BM][64] (32 compressed values per row), B [BT][128] (64 values)
  static constexpr int A_BYTES = BM * 64, B_BYTES = BT * 128;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  // metadata: [BM][16] = four words (two stages) per row, in a ring of two slots,
  // plus a 256-byte landing area per wave for the placeholder loads that keep
  // every wave's per-stage load count equal
  static constexpr int META_SLOT = BM * 16, META_BYTES = 2 * META_SLOT, PAD_BYTES = 256 * WAVES;
  static constexpr int LDS_BYTES = NST * STAGE_BYTES + META_BYTES + PAD_BYTES;
  // buffer-to-LDS loads per wave and stage: A and B (1 KB each) and one metadata
  // load (a 1 KB slice every second stage for the first META_WAVES waves, else a
  // 256-byte placeholder that reads nothing)
  static constexpr int A_DMA = A_BYTES / 1024 / WAVES, B_DMA = B_BYTES / 1024 / WAVES;
  static constexpr int DMA_PER_STAGE = A_DMA + B_DMA + 1;
  static constexpr int META_WAVES = META_SLOT / 1024;  // waves that load one metadata KB each
  // packed operand (tile chunks): a chunk holds one stage of a 256-row tile,
  // the A slice (A_BYTES, already swizzled) then two metadata words per row;
  // the stage's metadata sits in LDS after its B slice (one 4-byte load per lane)
  static constexpr int META_STAGE = BM * 8, CHUNK_BYTES = A_BYTES + META_STAGE;
  static constexpr int PSTAGE_BYTES = STAGE_BYTES + META_STAGE, PLDS_BYTES = NST * PSTAGE_BYTES;
  static_assert(A_BYTES % (1024 * WAVES) == 0 && B_BYTES % (1024 * WAVES) == 0, "tile/wave split");
  static_assert(META_WAVES <= WAVES, "metadata split");
  static_assert(LDS_BYTES <= 160 * 1024 && PLDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(META_STAGE == 256 * WAVES, "one metadata load per wave and stage");
};

// acc[fm][ft] += R^T . (X L)^T over the adapter rank, from the prepared
// workspace: rt [Npad][rpad] (R transposed) and the hi / lo bf16 parts of
// X . L, xlh / xll [Tpad][rpad], in the input format (bf16, or fp16 with H);
// both padded with zeros so no bounds checks are needed.  Dense 32x32x16
// MFMA: A lane l = row l%32, k = 8*(l/32)+e; B lane l = column l%32, same k.
// hi and lo together keep about twice the format's mantissa of X . L.
template <class G, bool H = false>
__device__ __forceinline__ void adapter_mma(f32x16 (&acc)[G::FM][G::FT], const uint16_t* __restrict__ rt,
                                            const uint16_t* __restrict__ xlh, const uint16_t* __restrict__ xll,
                                            int rpad, int64_t m0, int64_t t0, int wm, int wt, int lane) {
  typedef Fmt16<H> F;
  typedef typename F::v8 v8;
  const int kofs = 8 * (lane >> 5);
  for (int jk = 0; jk < rpad; jk += 16) {
    v8 ra[G::FM];
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm) {
      const int64_t m = m0 + wm * G::WM + fm * 32 + (lane & 31);
      ra[fm] = *reinterpret_cast<const v8*>(rt + m * rpad + jk + kofs);
    }
#pragma unroll
    for (int ft = 0; ft < G::FT; ++ft) {
      const int64_t t = t0 + wt * G::WT + ft * 32 + (lane & 31);
      const v8 xh = *reinterpret_cast<const v8*>(xlh + t * rpad + jk + kofs);
      const v8 xo = *reinterpret_cast<const v8*>(xll + t * rpad + jk + kofs);
#pragma unroll
      for (int fm = 0; fm < G::FM; ++fm) {
        acc[fm][ft] = F::mfma32x32x16(ra[fm], xh, acc[fm][ft]);
        acc[fm][ft] = F::mfma32x32x16(ra[fm], xo, acc[fm][ft]);
      }
    }
  }
}

// Store the transposed tile to Out[t][m] (row-major [T, M]); four consecutive
// accumulator elements are four consecutive m: one 8-byte (16-bit output) or
// 16-byte (fp32) store.  Requires M % 4 == 0.
template <class G, typename O>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[G::FM][G::FT], O* __restrict__ Y, int64_t m0,
                                           int64_t t0, int M, int T, int wm, int wt, int lane) {
#pragma unroll
  for (int ft = 0; ft < G::FT; ++ft) {
    const int64_t t = t0 + wt * G::WT + ft * 32 + (lane & 31);
    if (t >= T) continue;
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t m = m0 + wm * G::WM + fm * 32 + 8 * q + 4 * (lane >> 5);
        if (m >= M) continue;
        O* p = Y + t * M + m;
        if constexpr (sizeof(O) == 2) {
          u32x2 w;
          w[0] = out16_bits<O>(acc[fm][ft][4 * q]) | ((uint32_t)out16_bits<O>(acc[fm][ft][4 * q + 1]) << 16);
          w[1] = out16_bits<O>(acc[fm][ft][4 * q + 2]) | ((uint32_t)out16_bits<O>(acc[fm][ft][4 * q + 3]) << 16);
          *reinterpret_cast<u32x2*>(p) = w;
        } else {
          f32x4 w = {acc[fm][ft][4 * q], acc[fm][ft][4 * q + 1], acc[fm][ft][4 * q + 2], acc[fm][ft][4 * q + 3]};
          *reinterpret_cast<f32x4*>(p) = w;
        }
      }
    }
  }
}

// Load the transposed tile from Out[t][m] (the inverse of store_tile; rows or
// columns outside [T, M] read as 0).  Four consecutive m per load (M % 4 ==
// 0: all in or all out), every load from a clamped valid address and then
// masked, so they are all in flight together.
template <class G, typename O>
__device__ __forceinline__ void load_tile(f32x16 (&acc)[G::FM][G::FT], const O* __restrict__ Y, int64_t m0,
                                          int64_t t0, int M, int T, int wm, int wt, int lane) {
#pragma unroll
  for (int ft = 0; ft < G::FT; ++ft) {
    const int64_t t = t0 + wt * G::WT + ft * 32 + (lane & 31);
    const int64_t tc = t < T ? t : T - 1;
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t m = m0 + wm * G::WM + fm * 32 + 8 * q + 4 * (lane >> 5);
        const bool ok = t < T && m < M;
        const O* p = Y + tc * M + (m < M ? m : M - 4);
        float x[4];
        if constexpr (sizeof(O) == 2) {
          const u32x2 w = *reinterpret_cast<const u32x2*>(p);
          x[0] = out16_to_f32<O>(w[0] & 0xFFFFu); x[1] = out16_to_f32<O>(w[0] >> 16);
          x[2] = out16_to_f32<O>(w[1] & 0xFFFFu); x[3] = out16_to_f32<O>(w[1] >> 16);
        } else {
          const f32x4 w = *reinterpret_cast<const f32x4*>(p);
          x[0] = w[0]; x[1] = w[1]; x[2] = w[2]; x[3] = w[3];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[fm][ft][4 * q + i] = ok ? x[i] : 0.f;
      }
    }
  }
}

}  // namespace slope

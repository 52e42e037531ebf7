// 8-bit (E4M3) variant of the sparse products: Y = (Xq . W_q^T) / (sx * sw)
// on gfx950's 8-bit sparse MFMA (v_smfmac_f32_32x32x64_fp8_fp8).
//
// The pages name N:M sparsity in general (explainer, Technical Summary 1) and
// count 16-bit values (discussion page, "Memory Footprint Reduction During
// Pretraining and Inference"); they give no 8-bit format or scaling rule.  The
// reading here: OCP FP8 E4M3 (bias 7, no infinities, 0x7F / 0xFF NaN, largest
// finite 448), one scale per tensor, scale = 448 / amax (one fp32 division;
// 1 when amax is 0 or not finite), codes = round_to_nearest_even(x * scale)
// with the product rounded to fp32 first and magnitudes beyond 448 saturated.
//
// Measured lane layout of v_smfmac_f32_32x32x64_fp8_fp8 on gfx950 (random
// exact-integer trials against a host model):
//   A (compressed, 16 bytes per lane): lane l holds row l%32 and the 16 kept
//     values of dense k 32*(l/32) .. 32*(l/32)+31 of the 64-wide k step (eight
//     groups of four, two values each, in group order); the index operand is
//     the eight groups' nibbles i0 | i1 << 2 at bits 4g, i.e. one stored
//     metadata word: lanes 0..31 take the k step's first word, 32..63 its second.
//   B (32 bytes per lane): lane l holds column l%32, k = 16*(l/32) + e for
//     e < 16 and 32 + 16*(l/32) + (e - 16) for e >= 16.
//   D: as every 32x32 MFMA (lane l column l%32, rows 8*(v/4) + 4*(l/32) + v%4).
// A stage of 128 dense k thus holds the same bytes per row as a 16-bit stage
// of 64 k (64 compressed bytes of A, 128 bytes of B), with twice the products.
#include "common.h"
#include "dma.h"
#include "gemm_tile.h"
#include "launch.h"
#include "tile_map.h"

namespace slope {

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kE4m3Max = 448.0f;

// Scale of a tensor from the bits of its largest magnitude (fp32 bits of |x|).
__device__ __forceinline__ float e4m3_scale_from_amax(uint32_t amax_bits) {
  if (amax_bits == 0u || amax_bits >= 0x7F800000u) return 1.0f;
  return kE4m3Max / __uint_as_float(amax_bits);
}

// fp32 -> E4M3 code, round to nearest even, magnitudes at or beyond 448 give
// +-448, NaN gives 0x7F, the sign of zero is kept.  Integer arithmetic on the
// fp32 bits (normal range) or one exact scaling by 2^9 and a nearest-even
// rounding (subnormal range, below 2^-6).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t mag = b & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return 0x7Fu;                       // NaN
  if (mag >= 0x43E00000u) return sign | 0x7Eu;               // >= 448 (and infinity): saturate
  if (mag < 0x3C800000u) {                                   // < 2^-6: subnormal codes 0 .. 8
    const float q = __builtin_rintf(__uint_as_float(mag) * 512.0f);
    return sign | (uint32_t)q;                               // 8 is the smallest normal, code 0x08
  }
  const uint32_t e = (mag >> 23) - 127u + 7u;                // biased E4M3 exponent, 1 .. 15
  uint32_t keep = (mag >> 20) & 7u;
  const uint32_t rest = mag & 0xFFFFFu;
  keep += (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
  uint32_t code = (e << 3) + keep;                           // a carry into the exponent is right
  return sign | (code > 0x7Eu ? 0x7Eu : code);
}

template <typename In>
__device__ __forceinline__ float in_to_f32(In v);
template <> __device__ __forceinline__ float in_to_f32<uint16_t>(uint16_t v) { return bf16_bits_to_f32(v); }
template <> __device__ __forceinline__ float in_to_f32<_Float16>(_Float16 v) { return (float)v; }

// amax word <- 0 (the next kernel takes the maximum into it)
__global__ void amax_clear_kernel(uint32_t* amax) { *amax = 0u; }

// amax <- max(amax, |x|) over n 16-bit values, as fp32 bits (an integer maximum
// of non-negative fp32 patterns: order independent, so deterministic).  Eight
// values per thread from each 16-byte load, four loads in flight, a block
// maximum by shuffles and LDS, one atomic per block (a few hundred blocks: the
// atomics on the one word are serialised at the cache).
template <typename In>
__global__ __launch_bounds__(256) void amax_kernel(const In* __restrict__ src, int64_t n, uint32_t* amax) {
  __shared__ uint32_t wmax[4];
  uint32_t m = 0u;
  const int64_t n8 = n / 8, stride = (int64_t)gridDim.x * 256;
  for (int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x; i0 < n8; i0 += 4 * stride) {
    u32x4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {                  // clamped addresses, masked below
      const int64_t i = i0 + u * stride;
      w[u] = *reinterpret_cast<const u32x4*>(src + 8 * (i < n8 ? i : i0));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const In lo = __builtin_bit_cast(In, (uint16_t)(w[u][e] & 0xFFFFu));
        const In hi = __builtin_bit_cast(In, (uint16_t)(w[u][e] >> 16));
        const uint32_t a = __float_as_uint(in_to_f32<In>(lo)) & 0x7FFFFFFFu;
        const uint32_t c = __float_as_uint(in_to_f32<In>(hi)) & 0x7FFFFFFFu;
        m = a > m ? a : m;                         // a clamped load repeats an element: harmless for a maximum
        m = c > m ? c : m;
      }
    }
  }
  for (int64_t i = n8 * 8 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const uint32_t a = __float_as_uint(in_to_f32<In>(src[i])) & 0x7FFFFFFFu;
    m = a > m ? a : m;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t x = (uint32_t)__shfl_xor((int)m, o);
    m = x > m ? x : m;
  }
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = wmax[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) b = wmax[w] > b ? wmax[w] : b;
    if (b != 0u) atomicMax(amax, b);
  }
}

// scale word: from the amax bits it holds to the scale (after every reader of amax)
__global__ void amax_to_scale_kernel(uint32_t* word) {
  *reinterpret_cast<float*>(word) = e4m3_scale_from_amax(*word);
}

// q[i] = E4M3 code of fp32(x[i] * scale), scale from the amax word; 16 values
// per thread (two 16-byte loads, one 16-byte store).
template <typename In>
__global__ __launch_bounds__(256) void quantize_kernel(const In* __restrict__ src, int64_t n,
                                                       const uint32_t* __restrict__ amax, uint8_t* __restrict__ dst) {
  const float s = e4m3_scale_from_amax(*amax);
  const int64_t n16 = n / 16;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (int64_t)gridDim.x * 256) {
    const u32x4 w0 = *reinterpret_cast<const u32x4*>(src + 16 * i);
    const u32x4 w1 = *reinterpret_cast<const u32x4*>(src + 16 * i + 8);
    u32x4 out;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 w = h ? w1 : w0;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        uint32_t word = 0u;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint32_t pair = w[2 * e + q];
          const float a = in_to_f32<In>(__builtin_bit_cast(In, (uint16_t)(pair & 0xFFFFu))) * s;
          const float c = in_to_f32<In>(__builtin_bit_cast(In, (uint16_t)(pair >> 16))) * s;
          word |= (f32_to_e4m3(a) | (f32_to_e4m3(c) << 8)) << (16 * q);
        }
        out[2 * h + e] = word;
      }
    }
    *reinterpret_cast<u32x4*>(dst + 16 * i) = out;
  }
  for (int64_t i = n16 * 16 + (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = (uint8_t)f32_to_e4m3(in_to_f32<In>(src[i]) * s);
}

// ---------------------------------------------------------------- tile chunks
// E4M3 tile chunk (t, s) of a compressed [rows, cols] matrix: rows 256t ..
// 256t+255, dense columns 128s .. 128s+127, at byte offset (t * ceil(cols/128)
// + s) * kChunk8Bytes: first each row's 64 codes (compressed values 64s ..
// 64s+63; 16-byte granule c at c ^ ((row/4) % 4)), then each row's four
// metadata words 4s .. 4s+3 (16 bytes at kChunk8ValueBytes + row*16).  Rows
// past `rows` and columns past `cols` are 0.
constexpr int kChunk8Rows = 256, kChunk8Cols = 128;
constexpr int kChunk8ValueBytes = kChunk8Rows * 64, kChunk8Bytes = kChunk8ValueBytes + kChunk8Rows * 16;

// Eight lanes per row: lane k of a row's group reads its 16-byte piece
// (compressed values 8k .. 8k+7 of the chunk's 64) and the group's first four
// lanes its metadata words, so each group reads one contiguous 128-byte line
// of values per row; 32 rows per pass, all eight passes' loads issued first.
// Lane k writes its eight codes (half of granule k / 2) and, k < 4, metadata
// word k.
template <typename In>
__global__ __launch_bounds__(256) void pack_e4m3_kernel(const In* __restrict__ vals, const uint32_t* __restrict__ meta,
                                                        int64_t M, int64_t Kred, int64_t stages, int64_t nchunks,
                                                        const uint32_t* __restrict__ amax, char* __restrict__ out) {
  const float sc = e4m3_scale_from_amax(*amax);
  const int k = threadIdx.x & 7, rsub = threadIdx.x >> 3;
  const int64_t wpr = (Kred / 4 + 7) / 8, half = Kred / 2;
  for (int64_t q = blockIdx.x; q < nchunks; q += gridDim.x) {
    const int64_t tm = q / stages, s = q % stages;
    char* chunk = out + q * kChunk8Bytes;
    const int64_t c0 = s * 64 + 8 * k;                // this lane's first compressed value of the row
    const int64_t word = 4 * s + (k & 3);             // this lane's metadata word (lanes 4..7 repeat 0..3)
    // every load from a clamped, valid address, masked afterwards (Kred % 16 == 0:
    // a piece of 8 values lies entirely inside or outside the row)
    u32x4 v[8];
    uint32_t mw[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int64_t row = tm * kChunk8Rows + 32 * p + rsub;
      const int64_t rc = row < M ? row : 0;
      v[p] = *reinterpret_cast<const u32x4*>(vals + rc * half + (c0 < half ? c0 : 0));
      mw[p] = meta[rc * wpr + (word < wpr ? word : 0)];
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r = 32 * p + rsub;
      const bool live = tm * kChunk8Rows + r < M;
      const bool ok = live && c0 < half;
      u32x2 o;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        uint32_t w = 0u;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t pair = v[p][2 * e + h];
          const float a = in_to_f32<In>(__builtin_bit_cast(In, (uint16_t)(pair & 0xFFFFu))) * sc;
          const float c = in_to_f32<In>(__builtin_bit_cast(In, (uint16_t)(pair >> 16))) * sc;
          w |= (f32_to_e4m3(a) | (f32_to_e4m3(c) << 8)) << (16 * h);
        }
        o[e] = ok ? w : 0u;
      }
      *reinterpret_cast<u32x2*>(chunk + r * 64 + (((k >> 1) ^ ((r >> 2) & 3)) << 4) + 8 * (k & 1)) = o;
      if (k < 4) *reinterpret_cast<uint32_t*>(chunk + kChunk8ValueBytes + r * 16 + 4 * k) = (live && word < wpr) ? mw[p] : 0u;
    }
  }
}

// ---------------------------------------------------------------- the GEMM
// 256 x 256 transposed output tile Out^T = W_q . Xq^T, eight waves of 128 x 64,
// stages of 128 dense k in a ring of three LDS slots filled by buffer-to-LDS
// loads: the weight's stage is one contiguous 20 KB chunk (values, then four
// metadata words per row), X's 256 token rows of 128 bytes each.  The schedule
// is the 16-bit kernel's: second k step's fragments read ahead of the first
// step's MFMAs, one barrier per stage, the slot refilled among the second
// step's MFMAs.  LDS granule swizzles as there (A row r: c ^ ((r>>2)&3); B row
// r: c ^ ((r^(r>>3))&7)), so fragment reads are conflict free.
struct Geo8 {
  static constexpr int BM = 256, BT = 256, WGM = 2, WGT = 4, WAVES = 8, THREADS = 512;
  static constexpr int WM = BM / WGM, WT = BT / WGT, FM = WM / 32, FT = WT / 32;
  static constexpr int KS = 128, NST = 3;
  static constexpr int A_BYTES = BM * 64, B_BYTES = BT * 128, META_STAGE = BM * 16;
  static constexpr int CHUNK_BYTES = A_BYTES + META_STAGE;
  static constexpr int SLOT = A_BYTES + B_BYTES + META_STAGE, LDS_BYTES = NST * SLOT;
  static constexpr int A_DMA = A_BYTES / 1024 / WAVES, B_DMA = B_BYTES / 1024 / WAVES, M_DMA = META_STAGE / 256 / WAVES;
  static constexpr int DMA_PER_STAGE = A_DMA + B_DMA + M_DMA;
  static_assert(CHUNK_BYTES == kChunk8Bytes && A_BYTES == kChunk8ValueBytes, "chunks are the stage slices");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <typename O>
__global__ __launch_bounds__(Geo8::THREADS, 1) void spmm_e4m3_kernel(const uint8_t* __restrict__ Xq,
                                                                   const char* __restrict__ packed, int M, int T,
                                                                   int Kred, const float* __restrict__ x_scale,
                                                                   const float* __restrict__ w_scale,
                                                                   O* __restrict__ Y) {
  typedef Geo8 G;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % G::WGM, wt = wave / G::WGM;
  const int tiles_m = (M + G::BM - 1) / G::BM, tiles_t = (T + G::BT - 1) / G::BT;
  int tm, tt;
  tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_t, 8, tm, tt);
  const int64_t m0 = (int64_t)tm * G::BM, t0 = (int64_t)tt * G::BT;
  const int stages = (Kred + G::KS - 1) / G::KS;
  const int rows_t = (int)((T - t0) < G::BT ? (T - t0) : G::BT);
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(packed + (int64_t)tm * stages * G::CHUNK_BYTES, (int64_t)stages * G::CHUNK_BYTES);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Xq + t0 * Kred, (int64_t)rows_t * Kred);

  uint32_t b_src[G::B_DMA];
  int b_k[G::B_DMA];
#pragma unroll
  for (int j = 0; j < G::B_DMA; ++j) {
    const int row = wave * (G::BT / G::WAVES) + j * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row ^ (row >> 3)) & 7);
    b_src[j] = (uint32_t)row * Kred + c * 16;
    b_k[j] = c * 16;                                 // first k of the granule within the stage
  }
  auto issue = [&](int s) {
    char* base = lds + (s % G::NST) * G::SLOT;
    const uint32_t chunk = (uint32_t)s * G::CHUNK_BYTES;
    const bool live = s < stages;
#pragma unroll
    for (int j = 0; j < G::A_DMA; ++j) {
      const uint32_t part = wave * (G::A_BYTES / G::WAVES) + j * 1024;
      dma16(ra, base + part, live ? chunk + part + lane * 16 : kOutOfRange);
    }
#pragma unroll
    for (int j = 0; j < G::B_DMA; ++j) {
      const bool ok = live && s * G::KS + b_k[j] < Kred;
      dma16(rb, base + G::A_BYTES + wave * (G::B_BYTES / G::WAVES) + j * 1024, ok ? b_src[j] + s * G::KS : kOutOfRange);
    }
#pragma unroll
    for (int j = 0; j < G::M_DMA; ++j) {
      const uint32_t part = wave * (G::META_STAGE / G::WAVES) + j * 256;
      dma4(ra, base + G::A_BYTES + G::B_BYTES + part, live ? chunk + G::A_BYTES + part + lane * 4 : kOutOfRange);
    }
  };

  int a_off[2][G::FM], m_off[2][G::FM], b_off[2][G::FT][2];
#pragma unroll
  for (int fm = 0; fm < G::FM; ++fm) {
    const int row = wm * G::WM + fm * 32 + (lane & 31);
    const int sw = (row >> 2) & 3;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      a_off[ks][fm] = row * 64 + (((2 * ks + (lane >> 5)) ^ sw) * 16);
      m_off[ks][fm] = G::A_BYTES + G::B_BYTES + row * 16 + (2 * ks + (lane >> 5)) * 4;
    }
  }
#pragma unroll
  for (int ft = 0; ft < G::FT; ++ft) {
    const int row = wt * G::WT + ft * 32 + (lane & 31);
    const int sw = (row ^ (row >> 3)) & 7;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      b_off[ks][ft][0] = G::A_BYTES + row * 128 + (((4 * ks + (lane >> 5)) ^ sw) * 16);
      b_off[ks][ft][1] = G::A_BYTES + row * 128 + (((4 * ks + 2 + (lane >> 5)) ^ sw) * 16);
    }
  }
  struct Frags {
    i32x4 a[G::FM];
    int ix[G::FM];
    i32x8 b[G::FT];
  };
  auto read_frags = [&](Frags& f, int s, int ks) {
    const char* base = lds + (s % G::NST) * G::SLOT;
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm) {
      f.a[fm] = *reinterpret_cast<const i32x4*>(base + a_off[ks][fm]);
      f.ix[fm] = *reinterpret_cast<const int*>(base + m_off[ks][fm]);
    }
#pragma unroll
    for (int ft = 0; ft < G::FT; ++ft) {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(base + b_off[ks][ft][0]);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(base + b_off[ks][ft][1]);
      f.b[ft] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };
  f32x16 acc[G::FM][G::FT];
#pragma unroll
  for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
    for (int ft = 0; ft < G::FT; ++ft) acc[fm][ft] = f32x16{};
  auto mma_col = [&](const Frags& f, int ft) {
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm)
      acc[fm][ft] = __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(f.a[fm], f.b[ft], acc[fm][ft], f.ix[fm], 0, 0);
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int ft = 0; ft < G::FT; ++ft) mma_col(f, ft);
  };

#pragma unroll
  for (int p = 0; p < G::NST; ++p) issue(p);
  wait_vmcnt<G::DMA_PER_STAGE * (G::NST - 1)>();
  barrier();
  compiler_fence();
  Frags f0, f1;
  read_frags(f0, 0, 0);
  for (int s = 0; s < stages; ++s) {
    read_frags(f1, s, 1);
    mma(f0);
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkmcnt0();
    wait_vmcnt<G::DMA_PER_STAGE * (G::NST - 2)>();
    barrier();
    if (s + 1 < stages) read_frags(f0, s + 1, 0);
    mma_col(f1, 0);
    __builtin_amdgcn_sched_barrier(0);
    issue(s + G::NST);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ft = 1; ft < G::FT; ++ft) mma_col(f1, ft);
  }
  wait_vmcnt<0>();
  // the two scales divided out once: one fp32 reciprocal of their product
  const float inv = 1.0f / (*x_scale * *w_scale);
#pragma unroll
  for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
    for (int ft = 0; ft < G::FT; ++ft) acc[fm][ft] *= inv;
  store_tile<G, O>(acc, Y, m0, t0, M, T, wm, wt, lane);
}

unsigned grid_for(int64_t work, int64_t per_block) {
  const int64_t b = cdiv(work, per_block);
  return (unsigned)(b < 1 ? 1 : (b > 16384 ? 16384 : b));
}

template <typename In>
hipError_t amax_into(const void* src, int64_t n, float* word, hipStream_t s) {
  uint32_t* w = reinterpret_cast<uint32_t*>(word);
  amax_clear_kernel<<<1, 1, 0, s>>>(w);
  if (n > 0) {
    const int64_t blocks = cdiv(n, 256 * 8 * 4);
    amax_kernel<In><<<(unsigned)(blocks < 512 ? blocks : 512), 256, 0, s>>>((const In*)src, n, w);
  }
  return hipGetLastError();
}

}  // namespace

int64_t packed_sparse_e4m3_bytes(int64_t rows, int64_t cols) {
  return cdiv(rows, kChunk8Rows) * cdiv(cols, kChunk8Cols) * kChunk8Bytes;
}

hipError_t launch_quantize_e4m3(Dt dt, const void* M, int64_t n, float* scale, uint8_t* q, hipStream_t s) {
  hipError_t e = dt == Dt::F16 ? amax_into<_Float16>(M, n, scale, s) : amax_into<uint16_t>(M, n, scale, s);
  if (e != hipSuccess) return e;
  uint32_t* w = reinterpret_cast<uint32_t*>(scale);
  if (n > 0) {
    if (dt == Dt::F16)
      quantize_kernel<_Float16><<<grid_for(n, 256 * 16 * 4), 256, 0, s>>>((const _Float16*)M, n, w, q);
    else
      quantize_kernel<uint16_t><<<grid_for(n, 256 * 16 * 4), 256, 0, s>>>((const uint16_t*)M, n, w, q);
  }
  amax_to_scale_kernel<<<1, 1, 0, s>>>(w);
  return hipGetLastError();
}

hipError_t launch_pack_sparse_e4m3(Dt dt, const void* values, const uint32_t* meta, int64_t M, int64_t Kred,
                                   float* scale, void* packed, hipStream_t s) {
  const int64_t n = M * (Kred / 2);
  hipError_t e =
      dt == Dt::F16 ? amax_into<_Float16>(values, n, scale, s) : amax_into<uint16_t>(values, n, scale, s);
  if (e != hipSuccess) return e;
  uint32_t* w = reinterpret_cast<uint32_t*>(scale);
  const int64_t stages = cdiv(Kred, kChunk8Cols), nchunks = cdiv(M, kChunk8Rows) * stages;
  if (nchunks > 0) {
    const unsigned grid = (unsigned)(nchunks < (1 << 20) ? nchunks : (1 << 20));
    if (dt == Dt::F16)
      pack_e4m3_kernel<_Float16><<<grid, 256, 0, s>>>((const _Float16*)values, meta, M, Kred, stages, nchunks, w,
                                                      (char*)packed);
    else
      pack_e4m3_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)values, meta, M, Kred, stages, nchunks, w,
                                                      (char*)packed);
  }
  amax_to_scale_kernel<<<1, 1, 0, s>>>(w);
  return hipGetLastError();
}

hipError_t launch_spmm_e4m3(Dt out, const uint8_t* Xq, const float* x_scale, int64_t T, int64_t Kred,
                            const void* packed, const float* w_scale, int64_t M, void* Y, hipStream_t s) {
  typedef Geo8 G;
  const int64_t nb = cdiv(M, G::BM) * cdiv(T, G::BT);
  if (nb == 0) return hipSuccess;
  if (out == Dt::BF16) {
    auto kern = spmm_e4m3_kernel<uint16_t>;
    static hipError_t attr = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS_BYTES);
    if (attr != hipSuccess) return attr;
    kern<<<(unsigned)nb, G::THREADS, G::LDS_BYTES, s>>>(Xq, (const char*)packed, (int)M, (int)T, (int)Kred, x_scale,
                                                        w_scale, (uint16_t*)Y);
  } else {
    auto kern = spmm_e4m3_kernel<float>;
    static hipError_t attr = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS_BYTES);
    if (attr != hipSuccess) return attr;
    kern<<<(unsigned)nb, G::THREADS, G::LDS_BYTES, s>>>(Xq, (const char*)packed, (int)M, (int)T, (int)Kred, x_scale,
                                                        w_scale, (float*)Y);
  }
  return hipGetLastError();
}

}  // namespace slope

// Sparse forward for a handful of tokens (T <= 64): the inference shapes of
// the discussion page's "SLoPe inference computation" (the unmerged adapter
// next to the 2:4 weight), where the layer streams its compressed weight once
// and the cost is HBM bandwidth, not matrix throughput.
//
// Y = X . W_s^T (+ (X . L) . R) with W_s in tile-chunk form (pack_sparse):
// the 256-row tiles are split along k so that enough waves stream the weight
// at once.  Each wave owns 64 rows of a tile and reads its operands straight
// from memory into registers (v_smfmac_f32_32x32x32_bf16, measured lane
// layouts as in spmm.hip); a block's four waves cover one tile over one
// k-range and write fp32 partial sums.  A second kernel adds the partial sums
// in split order (deterministic), adds the adapter term and rounds once.  The
// adapter's X . L is computed in fp32 by an extra row of blocks of the same
// launch, straight from L's own [K, r] layout, while the other blocks stream
// the weight; the up-projection reads R in its own layout (no transposed copy
// of R).
#include <atomic>
#include <mutex>

#include "common.h"
#include "dma.h"
#include "gemm_tile.h"
#include "launch.h"

namespace slope {

// Scratch of the allocation-free few-token forward: the split partial sums
// and X . L slices of one call, in a static device array (each GPU the library
// runs on holds its own copy until the process ends).  Every byte a call reads
// from it is written earlier by the same call, so nothing needs clearing; two
// calls that overlap on one GPU share it and race.  In host code the name is a
// host-side stand-in: only the address hipGetSymbolAddress returns for the
// current device may be handed to kernels.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];
std::mutex scratch_mu;
}  // namespace

hipError_t decode_scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {                                        // first call on this device: look the address up once
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

namespace {

typedef Geo<256, 256, 3, 2, 4> Chunk;            // the tile-chunk geometry written by pack_sparse
constexpr int kDecodeMaxT = 64;
constexpr int kUnroll = 4;                       // stages whose loads are issued together
constexpr int kXlTok = 4;                        // tokens per X . L block
constexpr int kXlRows = 2048;                    // rows of L per k-slice of X . L (up to four tokens), at most
static_assert(kXlRows / 256 <= 8, "up to four tokens a thread has at most 8 rows of a slice");
constexpr int kXlMaxSlices = 64;

// k-slices of the X . L blocks: up to four tokens the partial kernel is short,
// so K is cut into slices of at most kXlRows rows (the reduce adds them in
// order); with more tokens the weight streams long enough to hide one block
// walking all of K, and one slice keeps the reduce's staging cheap.
int xl_slices(int64_t T, int64_t K) {
  if (T > kXlTok) return 1;
  const int64_t n = cdiv(K, kXlRows);
  return (int)(n < 1 ? 1 : (n > kXlMaxSlices ? kXlMaxSlices : n));
}

// xl[t][8cg .. 8cg+7] = sum over k in [k0, k1) of X[t][k] L[k][8cg ..] for
// t < T <= 4 (columns past r are 0; X and xl start at the block's first
// token), fp32 with one fma per product.  Thread i
// takes rows k0 + i, k0 + i + 256, ...; the 256 per-thread sums are then added
// by a fixed butterfly within each wave and the four wave sums in wave order,
// so the result does not depend on timing.
template <bool H, int kXlBatch>
__device__ __forceinline__ void xl_columns(const uint16_t* __restrict__ X, const uint16_t* __restrict__ L, int T,
                                           int K, int r, int rpad, int cg, int k0, int k1, float* __restrict__ xl) {
  __shared__ float wsum[4][kXlTok * 8];
  typedef Fmt16<H> F;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c0 = 8 * cg;
  // with r % 8 == 0 a group starting below r lies inside the row: one 16-byte
  // load (L is 16-byte aligned); groups starting at or past r (the padding
  // up to rpad) read nothing and write zeros
  const bool vec = r % 8 == 0;
  float acc[kXlTok][8];
#pragma unroll
  for (int i = 0; i < kXlTok; ++i)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[i][c] = 0.f;
  // rows in batches of kXlBatch: every load of a batch (clamped to a valid
  // row, masked afterwards) is issued before the first product, since with
  // the weight streaming beside it each round trip to memory is long
  if (vec) {
    for (int kb = c0 < r ? k0 + (int)threadIdx.x : k1; kb < k1; kb += 256 * kXlBatch) {
      u32x4 lw[kXlBatch];
      uint16_t xr[kXlBatch][kXlTok];
#pragma unroll
      for (int j = 0; j < kXlBatch; ++j) {
        const int k = kb + 256 * j, kc = k < k1 ? k : k1 - 1;
        lw[j] = *reinterpret_cast<const u32x4*>(L + (int64_t)kc * r + c0);
#pragma unroll
        for (int i = 0; i < kXlTok; ++i) xr[j][i] = X[(int64_t)(i < T ? i : T - 1) * K + kc];
      }
#pragma unroll
      for (int j = 0; j < kXlBatch; ++j) {
        const bool live = kb + 256 * j < k1;
        float lv[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lv[2 * e] = F::to_f32((uint16_t)(lw[j][e] & 0xFFFFu));
          lv[2 * e + 1] = F::to_f32((uint16_t)(lw[j][e] >> 16));
        }
#pragma unroll
        for (int i = 0; i < kXlTok; ++i) {
          const float x = (live && i < T) ? F::to_f32(xr[j][i]) : 0.f;
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[i][c] = __builtin_fmaf(x, lv[c], acc[i][c]);
        }
      }
    }
  } else {
#pragma unroll 4
    for (int k = c0 < r ? k0 + (int)threadIdx.x : k1; k < k1; k += 256) {
      float lv[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {                // clamped columns, then masked (no branch per load)
        const float x = F::to_f32(L[(int64_t)k * r + (c0 + c < r ? c0 + c : r - 1)]);
        lv[c] = c0 + c < r ? x : 0.f;
      }
#pragma unroll
      for (int i = 0; i < kXlTok; ++i) {
        const float xv = F::to_f32(X[(int64_t)(i < T ? i : T - 1) * K + k]);
        const float x = i < T ? xv : 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[i][c] = __builtin_fmaf(x, lv[c], acc[i][c]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kXlTok; ++i)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v = acc[i][c];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
      acc[i][c] = v;
    }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < kXlTok; ++i)
#pragma unroll
      for (int c = 0; c < 8; ++c) wsum[wave][i * 8 + c] = acc[i][c];
  }
  __syncthreads();
  if (threadIdx.x < kXlTok * 8) {
    const int i = threadIdx.x / 8, c = threadIdx.x % 8;
    if (i < T && c0 + c < rpad)
      xl[i * rpad + c0 + c] = ((wsum[0][threadIdx.x] + wsum[1][threadIdx.x]) + wsum[2][threadIdx.x]) + wsum[3][threadIdx.x];
  }
}

// part[split][t][n] (n < Npad) = sum over this split's k of X[t][k] W_s[n][k].
// Block = 4 waves = one 256-row tile; wave w rows 64w .. 64w+63 (two 32-row
// A operands), FT = 1 or 2 token tiles of 32.  With XL (the adapter on) the
// grid has XR = ceil(XB / tiles) more rows of blocks, first, for the XB = G *
// TG * slices X . L blocks (G = rpad / 8 column groups, TG = ceil(T / 4) token
// groups): X . L block x (its index in those rows) writes the columns 8g ..
// 8g+7 (g = x % G) for tokens 4tg .. 4tg+3 (tg = (x / G) % TG) over k-slice
// s = x / (G * TG) of K to xl [s][T][rpad] (xl_columns, rows XB at a time)
// while the other rows stream the weight.  The grid keeps the tiles' width: rows padded with idle
// blocks to fit the X . L blocks measured up to twice as slow at T = 64.
//
// XS (more than four tokens): X's rows for each group of kUnrollXs stages go
// to LDS once per block, 128 bytes per token and stage (granule c at
// c ^ ((t ^ (t >> 3)) & 7), the sparse GEMM's B swizzle), in two buffers: the
// next group's rows are loaded into registers while the current group
// multiplies, and written behind one barrier per group.  The four waves then
// read their B fragments from LDS instead of each streaming all of X from the
// cache (at 64 tokens X's bytes per stage are 3.5x the weight's).  Groups of
// two stages (not four) halve the LDS a block holds, so more blocks share a
// compute unit (T = 64 layer 460 -> 441 us, the same at T = 16).  Each wave
// also loads the next group's weight into a second register set while the
// current group multiplies, so two groups of weight are in flight per wave.
constexpr int kXsRow = 128;                        // bytes of X per token and stage
constexpr int kUnrollXs = 2;                       // stages per X group
template <int FT>
constexpr int xs_lds_bytes() { return 2 * kUnrollXs * FT * 32 * kXsRow; }

template <int FT, bool H, int XB = 0, bool XS = false>
__global__ __launch_bounds__(256) void decode_partial_kernel(const uint16_t* __restrict__ X,
                                                             const char* __restrict__ packed, int T, int K,
                                                             int stages, int kc, int64_t Npad,
                                                             float* __restrict__ part,
                                                             const uint16_t* __restrict__ L, int r, int rpad,
                                                             int slices, float* __restrict__ xl) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = blockIdx.x;
  int xrows = 0;
  constexpr bool XL = XB > 0;
  if constexpr (XL) {
    const int groups = rpad / 8, tgroups = (T + kXlTok - 1) / kXlTok, xb = groups * tgroups * slices;
    xrows = (xb + (int)gridDim.x - 1) / (int)gridDim.x;
    if ((int)blockIdx.y < xrows) {
      const int x = blockIdx.y * gridDim.x + blockIdx.x;
      if (x < xb) {
        const int g = x % groups, tg = (x / groups) % tgroups, sl = x / (groups * tgroups);
        const int rows = (K + slices - 1) / slices, k0 = sl * rows, k1 = k0 + rows < K ? k0 + rows : K;
        const int t0 = tg * kXlTok, tn = T - t0 < kXlTok ? T - t0 : kXlTok;
        xl_columns<H, XB>(X + (int64_t)t0 * K, L, tn, K, r, rpad, g, k0, k1, xl + ((int64_t)sl * T + t0) * rpad);
      }
      return;
    }
  }
  const int split = blockIdx.y - xrows;
  const int s0 = split * kc, s1 = (s0 + kc < stages) ? s0 + kc : stages;
  const __amdgpu_buffer_rsrc_t ra =
      make_rsrc(packed + ((int64_t)tile * stages + s0) * Chunk::CHUNK_BYTES, (int64_t)(s1 - s0) * Chunk::CHUNK_BYTES);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (int64_t)T * K * 2);

  // per-lane offsets inside a chunk
  uint32_t a_off[2][2], m_off[2];
#pragma unroll
  for (int fm = 0; fm < 2; ++fm) {
    const int r = wave * 64 + fm * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) a_off[fm][ks] = r * 64 + (((2 * ks + (lane >> 5)) ^ ((r >> 2) & 3)) << 4);
    m_off[fm] = Chunk::A_BYTES + r * 8;
  }
  const int ix_shift = 16 * (lane >> 5);
  // X: token t = ft*32 + lane%32, k = 8*(lane/32) + e and 16 + 8*(lane/32) + e of each 32-wide step
  uint32_t x_off[FT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    const int t = ft * 32 + (lane & 31);
    x_off[ft] = t < T ? (uint32_t)(t * K + 8 * (lane >> 5)) * 2 : kOutOfRange;
  }

  f32x16 acc[2][FT];
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) acc[fm][ft] = f32x16{};

  if constexpr (XS) {
    extern __shared__ __attribute__((aligned(16))) char xs_lds[];
    typedef typename Fmt16<H>::v8 v8;
    constexpr int TOK = FT * 32, BUF = kUnrollXs * TOK * kXsRow;
    constexpr int GPT = TOK * kUnrollXs * 8 / 256;   // 16-byte granules of X per thread and group
    static_assert(GPT == 8 || GPT == 4 || GPT == 2, "fill mapping");
    // fill: granule q = threadIdx.x * GPT + j is row q / 8 = u * TOK + t, granule q % 8
    auto fill_load = [&](u32x4 (&xr)[GPT], int sb) {
#pragma unroll
      for (int j = 0; j < GPT; ++j) {
        const int q = (int)threadIdx.x * GPT + j, row = q >> 3, g = q & 7;
        const int u = row / TOK, t = row % TOK, st = sb + u;
        const bool ok = t < T && st < s1 && st * 64 + 8 * g < K;
        xr[j] = load16(rx, ok ? (uint32_t)(t * K + st * 64 + 8 * g) * 2 : kOutOfRange);
      }
    };
    auto fill_store = [&](const u32x4 (&xr)[GPT], char* buf) {
#pragma unroll
      for (int j = 0; j < GPT; ++j) {
        const int q = (int)threadIdx.x * GPT + j, row = q >> 3, g = q & 7;
        const int t = row % TOK;
        *reinterpret_cast<u32x4*>(buf + row * kXsRow + ((g ^ ((t ^ (t >> 3)) & 7)) << 4)) = xr[j];
      }
    };
    // per-lane B fragment offsets within a stage's rows: token ft*32 + lane%32,
    // granules 4ks + lane/32 and 4ks + 2 + lane/32
    int bo[FT][2][2];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      const int t = ft * 32 + (lane & 31), sw = (t ^ (t >> 3)) & 7;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bo[ft][ks][0] = t * kXsRow + (((4 * ks + (lane >> 5)) ^ sw) << 4);
        bo[ft][ks][1] = t * kXsRow + (((4 * ks + 2 + (lane >> 5)) ^ sw) << 4);
      }
    }
    // the weight of a group of stages, loaded one group ahead of its use into
    // the other of two register sets (the loop is unrolled by two, so no set
    // is copied while its loads are in flight).  Each lane loads its own 16-bit
    // half of a metadata word, so the index goes to the MFMA as loaded (a shift
    // after the load makes the wave wait for it there).
    uint32_t m16[2];
#pragma unroll
    for (int fm = 0; fm < 2; ++fm) m16[fm] = m_off[fm] + 2 * (lane >> 5);
    auto load_a = [&](v8 (&a)[kUnrollXs][2][2], int (&ix)[kUnrollXs][2][2], int sb) {
#pragma unroll
      for (int u = 0; u < kUnrollXs; ++u) {
        const int s = sb + u;
        const uint32_t dead = s < s1 ? 0u : kOutOfRange;
        const uint32_t c = (uint32_t)(s - s0) * Chunk::CHUNK_BYTES;
#pragma unroll
        for (int fm = 0; fm < 2; ++fm) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            a[u][fm][ks] = __builtin_bit_cast(v8, load16(ra, (c + a_off[fm][ks]) | dead));
            ix[u][fm][ks] = (int)__builtin_amdgcn_raw_buffer_load_b16(ra, (c + m16[fm] + ks * 4) | dead, 0, 0);
          }
        }
      }
    };
    int cur = 0, sb = s0;
    // one group: start the next group's X and weight loads (X first, so that
    // waiting for it before the barrier leaves the weight in flight), multiply
    // this group, then write the next group's X to the other buffer
    auto step = [&](v8 (&a)[kUnrollXs][2][2], int (&ix)[kUnrollXs][2][2], v8 (&an)[kUnrollXs][2][2],
                    int (&ixn)[kUnrollXs][2][2]) -> bool {
      const bool more = sb + kUnrollXs < s1;         // block-uniform
      u32x4 xr[GPT];
      if (more) {
        fill_load(xr, sb + kUnrollXs);
        load_a(an, ixn, sb + kUnrollXs);
      }
      const char* buf = xs_lds + cur * BUF;
#pragma unroll
      for (int u = 0; u < kUnrollXs; ++u)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int ft = 0; ft < FT; ++ft) {
            const char* rowp = buf + u * TOK * kXsRow;
            const v8 lo = *reinterpret_cast<const v8*>(rowp + bo[ft][ks][0]);
            const v8 hi = *reinterpret_cast<const v8*>(rowp + bo[ft][ks][1]);
            const typename Fmt16<H>::v16 b =
                __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
#pragma unroll
            for (int fm = 0; fm < 2; ++fm)
              acc[fm][ft] = Fmt16<H>::smfmac32x32x32(a[u][fm][ks], b, acc[fm][ft], ix[u][fm][ks]);
          }
      if (!more) return false;
      fill_store(xr, xs_lds + (cur ^ 1) * BUF);
      __syncthreads();                             // next buffer written; this one read by every wave
      cur ^= 1;
      sb += kUnrollXs;
      return true;
    };
    v8 a0[kUnrollXs][2][2], a1[kUnrollXs][2][2];
    int ix0[kUnrollXs][2][2], ix1[kUnrollXs][2][2];
    load_a(a0, ix0, s0);
    {
      u32x4 xr[GPT];
      fill_load(xr, s0);
      fill_store(xr, xs_lds);
    }
    __syncthreads();
    while (step(a0, ix0, a1, ix1) && step(a1, ix1, a0, ix0)) {
    }
  } else
  for (int sb = s0; sb < s1; sb += kUnroll) {
    typedef typename Fmt16<H>::v8 v8;
    v8 a[kUnroll][2][2];
    int ix[kUnroll][2][2];
    typename Fmt16<H>::v16 b[kUnroll][2][FT];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int s = sb + u;
      const bool live = s < s1;
      const uint32_t c = (uint32_t)(s - s0) * Chunk::CHUNK_BYTES;
#pragma unroll
      for (int fm = 0; fm < 2; ++fm) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          a[u][fm][ks] = __builtin_bit_cast(v8, load16(ra, live ? c + a_off[fm][ks] : kOutOfRange));
          const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(ra, live ? c + m_off[fm] + ks * 4 : kOutOfRange, 0, 0);
          ix[u][fm][ks] = (int)(w >> ix_shift);    // this lane's half of the word
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int k0 = s * 64 + ks * 32 + 8 * (lane >> 5);           // first k of this lane's low eight
        const uint32_t kb = (uint32_t)(s * 64 + ks * 32) * 2;       // byte offset of the k step in a row
        // K % 16 == 0: each group of eight k is entirely inside or outside the row
        const bool ok_lo = live && k0 < K, ok_hi = live && k0 + 16 < K;
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) {
          const bool valid = x_off[ft] != kOutOfRange;
          const u32x4 lo = load16(rx, valid && ok_lo ? x_off[ft] + kb : kOutOfRange);
          const u32x4 hi = load16(rx, valid && ok_hi ? x_off[ft] + kb + 32 : kOutOfRange);
          b[u][ks][ft] = __builtin_shufflevector(__builtin_bit_cast(v8, lo), __builtin_bit_cast(v8, hi), 0, 1, 2, 3, 4,
                                                 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int ft = 0; ft < FT; ++ft)
#pragma unroll
          for (int fm = 0; fm < 2; ++fm)
            acc[fm][ft] = Fmt16<H>::smfmac32x32x32(a[u][fm][ks], b[u][ks][ft], acc[fm][ft], ix[u][fm][ks]);
  }

  // lane holds token ft*32 + lane%32, rows 8*(v/4) + 4*(lane/32) + v%4 of each 32-row block
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    const int t = ft * 32 + (lane & 31);
    if (t >= T) continue;
    float* dst = part + ((int64_t)split * T + t) * Npad + (int64_t)tile * 256 + wave * 64;
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {acc[fm][ft][4 * q], acc[fm][ft][4 * q + 1], acc[fm][ft][4 * q + 2], acc[fm][ft][4 * q + 3]};
        *reinterpret_cast<f32x4*>(dst + fm * 32 + 8 * q + 4 * (lane >> 5)) = v;
      }
  }
}

// Y[t][n] = sum over the splits (in order) of part + sum_j xl[t][j] R[j][n],
// rounded once, with xl the sum in slice order of fp32 [xl_slices][T][rpad]
// (xlf, from the partial kernel).  Up to four tokens (more take the wide
// reduce below).  A block covers 64 consecutive n
// (one per lane) and TB tokens; its four waves split the work into quarters
// (wave w: the w-th quarter of the splits, in order, and the w-th quarter of
// the rank rows), each wave issuing its loads of partial sums (Q at a time)
// and of its R rows before using them, and the four partial sums are added in
// wave order through LDS (deterministic).  The block's xl rows are staged in
// LDS once and read as broadcasts; R is read in its own [r, N] layout.  R's
// rows and the staged X . L are read from clamped, valid addresses and then
// replaced by 0 where out of range: written as conditional loads they become
// branches with a wait after every load.
constexpr int kReduceMaxRank = 128;

template <typename O, int TB, int Q, bool H>
__global__ __launch_bounds__(256) void decode_reduce_kernel(const float* __restrict__ part, int splits, int T,
                                                            int64_t N, int64_t Npad, const uint16_t* __restrict__ R,
                                                            const float* __restrict__ xlf, int xl_slices, int r,
                                                            int rpad, O* __restrict__ Y) {
  constexpr int RQ = kReduceMaxRank / 4;           // rank rows per wave, at most
  __shared__ float xl[TB][kReduceMaxRank];
  __shared__ float sum[4][TB][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.x * 64 + lane;
  const bool col = n < N;
  const int tb = blockIdx.y * TB;
  // the wave's quarter of the (zero-padded) rank rows of R, loaded first
  const int rq = rpad / 4, j0 = wave * rq;
  const int64_t nc = col ? n : N - 1;             // a valid column for the clamped loads
  float rv[RQ];
  if (R) {
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const int j = j0 + q;
      const float x = Fmt16<H>::to_f32(R[(int64_t)(j < r ? j : r - 1) * N + nc]);
      rv[q] = (col && q < rq && j < r) ? x : 0.f;
    }
    // element e = threadIdx.x + 256 k of the TB x rpad values: every element's
    // loads of SB slices in flight together, the slices added in slice order
    constexpr int EPT = (TB * kReduceMaxRank + 255) / 256;
    constexpr int SB = EPT >= 8 ? 1 : 8 / EPT;
    float v[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) v[k] = 0.f;
    for (int sl0 = 0; sl0 < xl_slices; sl0 += SB) {
      float t8[SB][EPT];
#pragma unroll
      for (int q = 0; q < SB; ++q)
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
          const int e = threadIdx.x + 256 * k, ec = e < TB * rpad ? e : 0;
          const int i = ec / rpad, j = ec % rpad;
          const int t = tb + i < T ? tb + i : T - 1;
          const int sl = sl0 + q < xl_slices ? sl0 + q : xl_slices - 1;
          t8[q][k] = xlf[((int64_t)sl * T + t) * rpad + j];
        }
#pragma unroll
      for (int q = 0; q < SB; ++q)
#pragma unroll
        for (int k = 0; k < EPT; ++k)
          if (sl0 + q < xl_slices) v[k] += t8[q][k];
    }
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int e = threadIdx.x + 256 * k;
      if (e < TB * rpad) {
        const int i = e / rpad, j = e % rpad;
        xl[i][j] = tb + i < T ? v[k] : 0.f;
      }
    }
  }
  float y[TB];
#pragma unroll
  for (int i = 0; i < TB; ++i) y[i] = 0.f;
  // the wave's quarter of the splits, Q at a time
  const int sq = (splits + 3) / 4, sp0 = wave * sq, sp1 = sp0 + sq < splits ? sp0 + sq : splits;
  for (int c0 = sp0; c0 < sp1; c0 += Q) {
    float v[Q][TB];
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < TB; ++i)
        v[q][i] = (col && c0 + q < sp1 && tb + i < T) ? part[((int64_t)(c0 + q) * T + tb + i) * Npad + n] : 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < TB; ++i) y[i] += v[q][i];
  }
  __syncthreads();                                 // xl staged
  if (R) {
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      if (q >= rq) break;
#pragma unroll
      for (int i = 0; i < TB; ++i) y[i] += rv[q] * xl[i][j0 + q];
    }
  }
#pragma unroll
  for (int i = 0; i < TB; ++i) sum[wave][i][lane] = y[i];
  __syncthreads();
  if (wave == 0 && col) {
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      if (tb + i >= T) continue;
      const float out = ((sum[0][i][lane] + sum[1][i][lane]) + sum[2][i][lane]) + sum[3][i][lane];
      store_out(Y + (tb + i) * N + n, out);
    }
  }
}

// Above four tokens: Y for 64 consecutive n (one per lane) and a span of
// TBLK = 4 TW tokens per block, wave w taking tokens TW w .. TW w + TW - 1 of
// the span.  Each wave adds every split of its own tokens, in split order,
// so no sums cross waves; its partial sums are loaded Q splits at a time
// (Q TW = 32 values a lane) with the next batch in flight while one is added.
// With the adapter the block's xl rows (a single slice above four tokens)
// and R's rows for its 64 columns (as fp32, rows r .. rpad zero) are staged
// in LDS by 16- and 8-byte loads issued with the first partial sums, and the
// rank term is added after the splits, in rank order.  Every load is from a
// clamped, valid address (values past the ends are not used), so that none
// is a branch.  LDS: (TBLK + 64) rpad floats with the adapter, none without.
template <typename O, int TW, bool H>
__global__ __launch_bounds__(256) void decode_reduce_wide_kernel(const float* __restrict__ part, int splits, int T,
                                                                 int64_t N, int64_t Npad, const uint16_t* __restrict__ R,
                                                                 const float* __restrict__ xlf, int r, int rpad,
                                                                 O* __restrict__ Y) {
  constexpr int Q = 32 / TW, TBLK = 4 * TW;
  constexpr int XPT = TBLK * kReduceMaxRank / 4 / 256;   // 16-byte granules of xl per thread, at most
  constexpr int RPT = kReduceMaxRank * 16 / 256;          // 8-byte granules of R per thread, at most
  extern __shared__ __attribute__((aligned(16))) float wide_lds[];
  float* xs = wide_lds;                            // [TBLK][rpad]
  float* rs = wide_lds + TBLK * rpad;              // [rpad][64]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 64, n = n0 + lane;   // < Npad: N in 256s covers the grid's 64s
  const int tblk = blockIdx.y * TBLK, tw = tblk + wave * TW;
  auto load_parts = [&](int c0, float (&v)[Q][TW]) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        const int c = c0 + q < splits ? c0 + q : splits - 1;
        const int t = tw + i < T ? tw + i : T - 1;
        v[q][i] = part[((int64_t)c * T + t) * Npad + n];
      }
  };
  float va[Q][TW], vb[Q][TW];
  load_parts(0, va);
  if (Q < splits) load_parts(Q, vb);             // block-uniform
  if (R) {
    u32x4 xg[XPT];
    u32x2 rg[RPT];
    const int xn = TBLK * rpad / 4, rn = rpad * 16;
#pragma unroll
    for (int k = 0; k < XPT; ++k) {
      const int g = (int)threadIdx.x + 256 * k, e = (g < xn ? g : 0) * 4;
      const int i = e / rpad, j = e % rpad, t = tblk + i < T ? tblk + i : T - 1;
      xg[k] = *reinterpret_cast<const u32x4*>(xlf + (int64_t)t * rpad + j);
    }
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int g = (int)threadIdx.x + 256 * k, gc = g < rn ? g : 0;
      const int j = gc >> 4, c = (gc & 15) * 4;
      const int64_t col = n0 + c < N ? n0 + c : 0;   // N % 4 == 0: a granule is inside or past N
      rg[k] = *reinterpret_cast<const u32x2*>(R + (int64_t)(j < r ? j : 0) * N + col);
    }
#pragma unroll
    for (int k = 0; k < XPT; ++k) {
      const int g = (int)threadIdx.x + 256 * k, e = g * 4;
      if (g < xn) {
        const int i = e / rpad;
        *reinterpret_cast<u32x4*>(xs + e) = tblk + i < T ? xg[k] : u32x4{};
      }
    }
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
      const int g = (int)threadIdx.x + 256 * k;
      if (g < rn) {
        const int j = g >> 4, c = (g & 15) * 4;
        const bool ok = j < r && n0 + c < N;
        f32x4 f;
        f[0] = Fmt16<H>::to_f32((uint16_t)(rg[k][0] & 0xffffu));
        f[1] = Fmt16<H>::to_f32((uint16_t)(rg[k][0] >> 16));
        f[2] = Fmt16<H>::to_f32((uint16_t)(rg[k][1] & 0xffffu));
        f[3] = Fmt16<H>::to_f32((uint16_t)(rg[k][1] >> 16));
        *reinterpret_cast<f32x4*>(rs + j * 64 + c) = ok ? f : f32x4{};
      }
    }
  }
  float y[TW];
#pragma unroll
  for (int i = 0; i < TW; ++i) y[i] = 0.f;
  // the splits in order: add one batch while the next is in flight
  auto add = [&](int c0, float (&v)[Q][TW]) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if (c0 + q < splits)
#pragma unroll
        for (int i = 0; i < TW; ++i) y[i] += v[q][i];
  };
  for (int c0 = 0;;) {
    add(c0, va);
    if (c0 + 2 * Q < splits) load_parts(c0 + 2 * Q, va);
    c0 += Q;
    if (c0 >= splits) break;
    add(c0, vb);
    if (c0 + 2 * Q < splits) load_parts(c0 + 2 * Q, vb);
    c0 += Q;
    if (c0 >= splits) break;
  }
  if (R) {
    __syncthreads();                               // xl and R staged
    const float* xw = xs + wave * TW * rpad;
    for (int j = 0; j < rpad; j += 4) {
      const f32x4 rv = {rs[j * 64 + lane], rs[(j + 1) * 64 + lane], rs[(j + 2) * 64 + lane], rs[(j + 3) * 64 + lane]};
#pragma unroll
      for (int i = 0; i < TW; ++i) {
        const f32x4 xv = *reinterpret_cast<const f32x4*>(xw + i * rpad + j);
        y[i] += xv[0] * rv[0];
        y[i] += xv[1] * rv[1];
        y[i] += xv[2] * rv[2];
        y[i] += xv[3] * rv[3];
      }
    }
  }
  if (n < N) {
#pragma unroll
    for (int i = 0; i < TW; ++i)
      if (tw + i < T) store_out(Y + (int64_t)(tw + i) * N + n, y[i]);
  }
}

// dynamic LDS of the wide reduce: up to (4 TW + 64) x 128 floats
template <typename O, int TW, bool H>
void decode_wide_attr() {
  static const hipError_t e = hipFuncSetAttribute((const void*)decode_reduce_wide_kernel<O, TW, H>,
                                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                                  (4 * TW + 64) * kReduceMaxRank * (int)sizeof(float));
  (void)e;                                         // a failure shows as the launch's error
}

template <typename O, bool H>
void launch_decode_reduce(const float* part, int splits, int64_t T, int64_t N, int64_t Npad, const uint16_t* R,
                          const float* xf, int xs, int r, int rpad, O* Y, hipStream_t s) {
  if (T == 1) {
    dim3 g((unsigned)cdiv(N, 64), 1);
    decode_reduce_kernel<O, 1, 8, H><<<g, 256, 0, s>>>(part, splits, (int)T, N, Npad, R, xf, xs, r, rpad, Y);
  } else if (T <= 4) {
    dim3 g((unsigned)cdiv(N, 64), (unsigned)cdiv(T, 4));
    decode_reduce_kernel<O, 4, 8, H><<<g, 256, 0, s>>>(part, splits, (int)T, N, Npad, R, xf, xs, r, rpad, Y);
  } else {
    // token span per block: 16 up to 16 tokens, else 32, halved to 16 while
    // the grid has fewer than 512 blocks.  (A 64-token span needs 232 VGPRs,
    // two waves a SIMD: the OPT-66B layer at 64 tokens took 385 us with it
    // against 380 us with spans of 32 at most.)
    const int64_t nb = cdiv(N, 64);
    int span = T <= 16 ? 16 : 32;
    if (span > 16 && nb * cdiv(T, span) < 512) span = 16;
    const size_t lds = R ? (size_t)(span + 64) * rpad * sizeof(float) : 0;
    dim3 g((unsigned)nb, (unsigned)cdiv(T, span));
    // above four tokens X . L has one slice (xl_slices), read as [T][rpad]
    if (span == 32) decode_wide_attr<O, 8, H>();
    else decode_wide_attr<O, 4, H>();
    if (span == 32)
      decode_reduce_wide_kernel<O, 8, H><<<g, 256, lds, s>>>(part, splits, (int)T, N, Npad, R, xf, r, rpad, Y);
    else
      decode_reduce_wide_kernel<O, 4, H><<<g, 256, lds, s>>>(part, splits, (int)T, N, Npad, R, xf, r, rpad, Y);
  }
}

struct DecodePlan {
  int stages, splits, kc;
  int64_t tiles, Npad, part_bytes;
};

DecodePlan decode_plan(int64_t T, int64_t K, int64_t N) {
  DecodePlan p{};
  p.stages = (int)cdiv(K, 64);
  p.tiles = cdiv(N, 256);
  p.Npad = p.tiles * 256;
  // about 2048 blocks, with at most 0.02 K / T splits so that the partial sums
  // (splits x T x N x 8 bytes written and read) stay small next to the weight.
  // With many tokens a block spends long on each stage and the weight stream is
  // no longer the limit: then keep at least about 1024 blocks (latency hiding on
  // a few blocks per CU) as long as each still runs 16 stages or more.  Above
  // four tokens (X staged in LDS, two blocks per CU by registers, each with the
  // next group's weight in flight) fewer blocks pay, measured on the OPT-66B
  // linears: above 32 tokens about 512 (the floor, not 1024; 441 -> 406 us a
  // layer at 64 tokens), and up to 32 tokens with 48 tiles or more one round
  // of 512 blocks (QKV and FC1 at 16 tokens 10% faster, OPT-13B's 60-tile QKV
  // 3%; 36 tiles keep the cap).
  const int64_t tiles = p.tiles < 1 ? 1 : p.tiles;
  int64_t want = cdiv(2048, tiles);
  int64_t cap = (int64_t)(0.02 * (double)K / (double)(T < 1 ? 1 : T));
  const int64_t busy = std::min<int64_t>(cdiv(T > 32 ? 512 : 1024, tiles), p.stages / 16);
  if (cap < busy) cap = busy;
  if (want > cap) want = cap;
  if (T > kXlTok && T <= 32 && tiles >= 48) want = 512 / tiles;
  if (want > p.stages) want = p.stages;
  if (want < 1) want = 1;
  p.kc = (int)cdiv(p.stages, want);
  p.kc = (int)(cdiv(p.kc, kUnroll) * kUnroll);
  p.splits = p.stages == 0 ? 1 : (int)cdiv(p.stages, p.kc);
  p.part_bytes = cdiv((int64_t)p.splits * T * p.Npad * 4, 256) * 256;
  return p;
}

}  // namespace

// fp32 X . L slices [xl_slices][T][rpad] (rpad = r rounded up to 16)
int64_t xl_bytes(int64_t T, int64_t K, int64_t r) {
  return r > 0 ? cdiv((int64_t)xl_slices(T, K) * T * cdiv(r, 16) * 16 * 4, 256) * 256 : 0;
}

int64_t decode_workspace_bytes(int64_t T, int64_t K, int64_t r, int64_t N) {
  if (T == 0 || N == 0) return 0;
  return decode_plan(T, K, N).part_bytes + xl_bytes(T, K, r);
}

namespace {
// X staged through LDS above four tokens (XS); dynamic LDS of that variant
template <int FT, bool H, int XB>
hipError_t decode_xs_attr() {
  static hipError_t e = hipFuncSetAttribute((const void*)decode_partial_kernel<FT, H, XB, true>,
                                            hipFuncAttributeMaxDynamicSharedMemorySize, xs_lds_bytes<FT>());
  return e;
}

template <bool H>
hipError_t decode_partial_launch(int64_t T, dim3 grid, const void* X, const void* packed, int64_t K,
                                 const DecodePlan& p, float* part, const void* L, int64_t r, int64_t rpad, int xs,
                                 float* xl, hipStream_t s) {
  const uint16_t* Xb = (const uint16_t*)X;
  const char* pk = (const char*)packed;
  const uint16_t* Lb = (const uint16_t*)L;
  if (xl) {                                        // the adapter on: leading rows of blocks for X . L
    const int64_t xb = rpad / 8 * cdiv(T, kXlTok) * xs;
    dim3 g(grid.x, grid.y + (unsigned)cdiv(xb, grid.x));
    // up to four tokens a thread has at most eight rows of a slice: batches of 8
    if (T <= kXlTok) {
      decode_partial_kernel<1, H, 8><<<g, 256, 0, s>>>(Xb, pk, (int)T, (int)K, p.stages, p.kc, p.Npad, part, Lb,
                                                       (int)r, (int)rpad, xs, xl);
    } else if (T <= 32) {
      hipError_t e = decode_xs_attr<1, H, 16>();
      if (e != hipSuccess) return e;
      decode_partial_kernel<1, H, 16, true><<<g, 256, xs_lds_bytes<1>(), s>>>(
          Xb, pk, (int)T, (int)K, p.stages, p.kc, p.Npad, part, Lb, (int)r, (int)rpad, xs, xl);
    } else {
      hipError_t e = decode_xs_attr<2, H, 16>();
      if (e != hipSuccess) return e;
      decode_partial_kernel<2, H, 16, true><<<g, 256, xs_lds_bytes<2>(), s>>>(
          Xb, pk, (int)T, (int)K, p.stages, p.kc, p.Npad, part, Lb, (int)r, (int)rpad, xs, xl);
    }
  } else if (T <= kXlTok) {
    decode_partial_kernel<1, H><<<grid, 256, 0, s>>>(Xb, pk, (int)T, (int)K, p.stages, p.kc, p.Npad, part, nullptr,
                                                     0, 0, 0, nullptr);
  } else if (T <= 32) {
    hipError_t e = decode_xs_attr<1, H, 0>();
    if (e != hipSuccess) return e;
    decode_partial_kernel<1, H, 0, true><<<grid, 256, xs_lds_bytes<1>(), s>>>(
        Xb, pk, (int)T, (int)K, p.stages, p.kc, p.Npad, part, nullptr, 0, 0, 0, nullptr);
  } else {
    hipError_t e = decode_xs_attr<2, H, 0>();
    if (e != hipSuccess) return e;
    decode_partial_kernel<2, H, 0, true><<<grid, 256, xs_lds_bytes<2>(), s>>>(
        Xb, pk, (int)T, (int)K, p.stages, p.kc, p.Npad, part, nullptr, 0, 0, 0, nullptr);
  }
  return hipSuccess;
}
}  // namespace

hipError_t launch_spmm_decode(Dt in, Dt out, const void* X, int64_t T, int64_t K, const void* packed, int64_t N,
                              const void* L, const void* R, int64_t r, void* workspace, void* Y, hipStream_t s) {
  if (T == 0 || N == 0) return hipSuccess;
  const DecodePlan p = decode_plan(T, K, N);
  float* part = (float*)workspace;
  const bool ad = r > 0 && L != nullptr && R != nullptr;
  // the adapter's X . L: fp32 slices [xs][T][rpad] after the partial sums
  float* xl = ad ? (float*)((char*)workspace + p.part_bytes) : nullptr;
  const int64_t rpad = ad ? cdiv(r, 16) * 16 : 0;
  const int xs = ad ? xl_slices(T, K) : 0;
  dim3 grid((unsigned)p.tiles, (unsigned)p.splits);
  const hipError_t pe = in == Dt::F16 ? decode_partial_launch<true>(T, grid, X, packed, K, p, part, L, r, rpad, xs, xl, s)
                                       : decode_partial_launch<false>(T, grid, X, packed, K, p, part, L, r, rpad, xs, xl, s);
  if (pe != hipSuccess) return pe;
  const uint16_t* Ra = ad ? (const uint16_t*)R : nullptr;
  const int rp = (int)rpad;
  if (out == Dt::BF16)
    launch_decode_reduce<uint16_t, false>(part, p.splits, T, N, p.Npad, Ra, xl, xs, (int)r, rp, (uint16_t*)Y, s);
  else if (out == Dt::F16)
    launch_decode_reduce<_Float16, true>(part, p.splits, T, N, p.Npad, Ra, xl, xs, (int)r, rp, (_Float16*)Y, s);
  else if (in == Dt::F16)
    launch_decode_reduce<float, true>(part, p.splits, T, N, p.Npad, Ra, xl, xs, (int)r, rp, (float*)Y, s);
  else
    launch_decode_reduce<float, false>(part, p.splits, T, N, p.Npad, Ra, xl, xs, (int)r, rp, (float*)Y, s);
  return hipGetLastError();
}

static_assert(kDecodeMaxT == 64, "two 32-token tiles at most");
static_assert(kReduceMaxRank >= 128, "adapter ranks up to 128 (rank rows padded to 16)");

}  // namespace slope

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
// compute unit (T = 64 layer 460 -> 441 us, the same at T = 16).
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
    {
      u32x4 xr[GPT];
      fill_load(xr, s0);
      fill_store(xr, xs_lds);
    }
    __syncthreads();
    int cur = 0;
    for (int sb = s0; sb < s1; sb += kUnrollXs) {
      v8 a[kUnrollXs][2][2];
      int ix[kUnrollXs][2][2];
#pragma unroll
      for (int u = 0; u < kUnrollXs; ++u) {
        const int s = sb + u;
        const bool live = s < s1;
        const uint32_t c = (uint32_t)(s - s0) * Chunk::CHUNK_BYTES;
#pragma unroll
        for (int fm = 0; fm < 2; ++fm) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            a[u][fm][ks] = __builtin_bit_cast(v8, load16(ra, live ? c + a_off[fm][ks] : kOutOfRange));
            const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(ra, live ? c + m_off[fm] + ks * 4 : kOutOfRange, 0, 0);
            ix[u][fm][ks] = (int)(w >> ix_shift);
          }
        }
      }
      const bool more = sb + kUnrollXs < s1;         // block-uniform
      u32x4 xr[GPT];
      if (more) fill_load(xr, sb + kUnrollXs);
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
      if (more) fill_store(xr, xs_lds + (cur ^ 1) * BUF);
      __syncthreads();                             // next buffer written; this one read by every wave
      cur ^= 1;
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
// (xlf, from the partial kernel).  A block covers 64 consecutive n
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
    for (int e = threadIdx.x; e < TB * rpad; e += 256) {
      const int i = e / rpad, j = e % rpad;
      const int t = tb + i < T ? tb + i : T - 1;
      float v = 0.f;
      for (int sl0 = 0; sl0 < xl_slices; sl0 += 8) {   // eight slices' loads in flight, added in slice order
        float t8[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int sl = sl0 + q < xl_slices ? sl0 + q : xl_slices - 1;
          t8[q] = xlf[((int64_t)sl * T + t) * rpad + j];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (sl0 + q < xl_slices) v += t8[q];
      }
      xl[i][j] = tb + i < T ? v : 0.f;
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
    dim3 g((unsigned)cdiv(N, 64), (unsigned)cdiv(T, 16));
    decode_reduce_kernel<O, 16, 4, H><<<g, 256, 0, s>>>(part, splits, (int)T, N, Npad, R, xf, xs, r, rpad, Y);
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
  // a few blocks per CU) as long as each still runs 16 stages or more.
  int64_t want = cdiv(2048, p.tiles < 1 ? 1 : p.tiles);
  int64_t cap = (int64_t)(0.02 * (double)K / (double)(T < 1 ? 1 : T));
  const int64_t busy = std::min<int64_t>(cdiv(1024, p.tiles < 1 ? 1 : p.tiles), p.stages / 16);
  if (cap < busy) cap = busy;
  if (want > cap) want = cap;
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

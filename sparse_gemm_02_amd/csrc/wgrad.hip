// Masked weight gradient dW = (dY^T . X) kept at the static 2:4 mask.
//
// The discussion page ("Memory Footprint Reduction During Pretraining and
// Inference") stores the gradient as two 16-bit values per four weights, and
// ("SLoPe downstream finetuning") only the non-zero weights are updated.  The
// sparsity sits in the output, not in the reduction, so this is a dense MFMA
// contraction over tokens whose epilogue keeps two of every four results.
//
// The kernel computes the transposed tile dW^T[k][n] = sum_t X[t][k] dY[t][n]:
// in the 32x32 MFMA output layout lane l holds four consecutive rows
// 8*(v/4) + 4*(l/32) + v%4, i.e. one whole 2:4 group of k, so the epilogue picks
// its two kept values in registers and writes them in W_s's slot order.
//
// Both operands are stored with tokens (the reduction) as rows, so tiles go to
// LDS as they are in memory and the MFMA fragments are read with the gfx950
// transposing LDS load ds_read_b64_tr_b16.  Measured semantics: in each group of
// 16 lanes, lane j supplies the address of four consecutive 16-bit values; lane
// i receives value i%4 of the rows supplied by lanes i/4, i/4+4, i/4+8, i/4+12.
// With lane j pointing at row (t + j/4), columns (c + 4*(j%4)) .. +3, lane i
// receives column c + i of rows t .. t+3.
#include <algorithm>

#include "common.h"
#include "launch.h"
#include "tile_map.h"
#include "dma.h"

namespace slope {

hipError_t launch_wgrad_generic(Dt in, Dt out, const void* dY, const void* X, int64_t T, int64_t N, int64_t K,
                                const uint32_t* meta_s, void* dWv, void* dWd, int accumulate, hipStream_t s);

namespace {

constexpr int kThreads = 256;

// Rows of k tiles per group of the XCD-aware tile order (tile_map.h), as in
// the sparse products: eight with few k tiles; with many (FC2 of OPT-66B: 144
// k tiles, its X too large to stay in the infinity cache while dY does)
// narrower groups, six when each XCD's share of the order is a whole number of
// six-row groups, else four (FC2: 4.53 -> 4.40 ms; QKV and FC1, 36 k tiles,
// are 1-4% slower with four or six).  `nblocks` is the number of blocks the
// order covers, the same at every use for one launch.
__device__ __forceinline__ int wgrad_group(int nblocks, int tiles_k, int tiles_n) {
  if (tiles_k < 72) return 8;
  const int per_xcd = nblocks % 8 == 0 ? nblocks / 8 : 0;
  return per_xcd > 0 && per_xcd % (6 * tiles_n) == 0 ? 6 : 4;
}

template <int BK_, int BN_, int NST_, int WGK_, int WGN_>
struct WGeo {
  static constexpr int BK = BK_, BN = BN_;         // tile rows (k) x columns (n) of dW^T
  static constexpr int WGK = WGK_, WGN = WGN_, WAVES = WGK * WGN, THREADS = 64 * WAVES;
  static constexpr int WK = BK / WGK, WN = BN / WGN;  // wave tile
  static constexpr int FK = WK / 32, FN = WN / 32;
  static constexpr int TS = 32;                    // tokens per LDS stage (two 16-deep MFMA steps)
  static constexpr int NST = NST_;                 // stages in the LDS ring
  static constexpr int XROW = BK * 2, DROW = BN * 2;              // bytes per token row of each tile
  static constexpr int X_BYTES = TS * XROW, D_BYTES = TS * DROW;
  static constexpr int STAGE_BYTES = X_BYTES + D_BYTES;
  static constexpr int X_DMA = X_BYTES / 1024 / WAVES, D_DMA = D_BYTES / 1024 / WAVES;  // per wave per stage
  static constexpr int LDS_BYTES = NST * STAGE_BYTES;
  static_assert(XROW == 512 && DROW == 512, "DMA mapping assumes 512-byte token rows");
};

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Two adjacent outputs as one store (4-byte aligned for 16-bit outputs, 8-byte for fp32).
template <typename O>
__device__ __forceinline__ void store_pair(O* p, float a, float b) {
  if constexpr (sizeof(O) == 2) {
    *reinterpret_cast<uint32_t*>(p) = out16_bits<O>(a) | ((uint32_t)out16_bits<O>(b) << 16);
  } else {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
  }
}
// Four adjacent outputs (8-byte aligned for 16-bit outputs, 16-byte for fp32), optionally accumulated.
template <typename O>
__device__ __forceinline__ void store_quad(O* p, const float (&x)[4], int accumulate) {
  float y[4] = {x[0], x[1], x[2], x[3]};
  if (accumulate) {
    const u32x2 o = *reinterpret_cast<const u32x2*>(p);
    y[0] += out16_to_f32<O>(o[0] & 0xFFFF); y[1] += out16_to_f32<O>(o[0] >> 16);
    y[2] += out16_to_f32<O>(o[1] & 0xFFFF); y[3] += out16_to_f32<O>(o[1] >> 16);
  }
  u32x2 w;
  w[0] = out16_bits<O>(y[0]) | ((uint32_t)out16_bits<O>(y[1]) << 16);
  w[1] = out16_bits<O>(y[2]) | ((uint32_t)out16_bits<O>(y[3]) << 16);
  *reinterpret_cast<u32x2*>(p) = w;
}
__device__ __forceinline__ void store_quad(float* p, const float (&x)[4], int accumulate) {
  f32x4 y = {x[0], x[1], x[2], x[3]};
  if (accumulate) y += *reinterpret_cast<const f32x4*>(p);
  *reinterpret_cast<f32x4*>(p) = y;
}

// Operand fragment from a token-major LDS tile: eight consecutive tokens (rows
// tb .. tb+7) of column c0 + (lane % 32), with two transposing loads.  Tile rows
// are 512 bytes; row r keeps its 16-byte granule q at q ^ ((r & 3) << 2), which
// puts the four rows a 32-lane pass of the transposing load touches in four
// different 64-byte bank groups.
template <bool H>
__device__ __forceinline__ typename Fmt16<H>::v8 frag_tr(const char* tile, int tb, int c0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int col = c0 + 16 * (g & 1) + 4 * (j & 3);      // element column of this lane's 4 values
  const int t = tb + 8 * (g >> 1) + (j >> 2);
  const int q = col >> 3, within = (col & 7) * 2;
  const char* p0 = tile + t * 512 + ((q ^ ((t & 3) << 2)) << 4) + within;
  const char* p1 = tile + (t + 4) * 512 + ((q ^ (((t + 4) & 3) << 2)) << 4) + within;
  s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(typename Fmt16<H>::v8, v);
}

// Epilogue of both weight-gradient kernels: lane l of accumulator [a][b] holds
// column n = n0 + wn*WN + b*32 + l%32 and rows k = k0 + wk*WK + a*32 + 8q + 4(l/32)
// + i (i < 4) in elements 4q+i, i.e. one whole 2:4 group of k; keep the two
// positions meta_s names and write them in slot order (plus the masked dense copy).
//
// The metadata word of a lane's rows is the same for the four q of a 32-row
// block (k >> 5 does not depend on q or lane / 32), so the FN x FK words are
// loaded first, all in flight, from clamped addresses (a word past N or K is
// never used); with accumulate so are the previous values pairs.  Loads under
// the bounds branches would each be followed by a wait.
//
// dWv's rows are ldv elements apart (K/2 for the whole matrix; a tile's own
// compact buffer passes 128 and a base shifted by its first row and group).
template <class G, typename O>
__device__ __forceinline__ void wgrad_store(const f32x16 (&acc)[G::FK][G::FN], const uint32_t* __restrict__ meta,
                                            int K, int N, int64_t k0, int64_t n0, int wk, int wn, int lane,
                                            O* __restrict__ dWv, O* __restrict__ dWd, int accumulate,
                                            int64_t ldv) {
  const int64_t wpr = ((int64_t)K / 4 + 7) / 8;
  uint32_t words[G::FN][G::FK];
#pragma unroll
  for (int b = 0; b < G::FN; ++b) {
    const int64_t n = n0 + wn * G::WN + b * 32 + (lane & 31);
    const int64_t nc = n < N ? n : N - 1;
#pragma unroll
    for (int a = 0; a < G::FK; ++a) {
      const int64_t w = (k0 + wk * G::WK + a * 32) >> 5;
      words[b][a] = meta[nc * wpr + (w < wpr ? w : wpr - 1)];
    }
  }
  float prev[G::FN][G::FK][4][2];
  if (accumulate) {
#pragma unroll
    for (int b = 0; b < G::FN; ++b) {
      const int64_t n = n0 + wn * G::WN + b * 32 + (lane & 31);
#pragma unroll
      for (int a = 0; a < G::FK; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t k = k0 + wk * G::WK + a * 32 + 8 * q + 4 * (lane >> 5);
          const O* vp = (n < N && k < K) ? dWv + n * ldv + 2 * (k >> 2) : dWv + n0 * ldv + 2 * (k0 >> 2);
          prev[b][a][q][0] = load_out(vp);
          prev[b][a][q][1] = load_out(vp + 1);
        }
    }
  }
#pragma unroll
  for (int b = 0; b < G::FN; ++b) {
    const int64_t n = n0 + wn * G::WN + b * 32 + (lane & 31);
    if (n >= N) continue;
#pragma unroll
    for (int a = 0; a < G::FK; ++a) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t k = k0 + wk * G::WK + a * 32 + 8 * q + 4 * (lane >> 5);
        if (k >= K) continue;
        const int64_t g = k >> 2;
        const uint32_t nib = (words[b][a] >> (4 * (g & 7))) & 0xFu;
        const uint32_t i0 = nib & 3u, i1 = nib >> 2;
        const float r0 = acc[a][b][4 * q], r1 = acc[a][b][4 * q + 1];
        const float r2 = acc[a][b][4 * q + 2], r3 = acc[a][b][4 * q + 3];
        // i0 < i1: i0 in {0,1,2}, i1 in {1,2,3}; selects without indexing registers
        float v0 = i0 == 0 ? r0 : (i0 == 1 ? r1 : r2);
        float v1 = i1 == 3 ? r3 : (i1 == 2 ? r2 : r1);
        O* vp = dWv + n * ldv + 2 * g;
        if (accumulate) { v0 += prev[b][a][q][0]; v1 += prev[b][a][q][1]; }
        store_pair(vp, v0, v1);
        if (dWd) {
          O* dp = dWd + n * K + k;
          const float x[4] = {(i0 == 0) ? r0 : 0.f, (i0 == 1 || i1 == 1) ? r1 : 0.f,
                              (i0 == 2 || i1 == 2) ? r2 : 0.f, (i1 == 3) ? r3 : 0.f};
          store_quad(dp, x, accumulate);
        }
      }
    }
  }
}

// Requirements (host-checked): K % 8 == 0, N % 8 == 0, 16-byte aligned bases.
// Token rows of both operands stream through a ring of NST LDS stages filled
// by buffer loads that write LDS directly (one barrier per stage, fragments
// for the next 16 tokens read while the current ones multiply; a stage's slot
// is refilled as soon as every wave holds its fragments, so NST-1 stages stay
// in flight).  Columns past
// K or N and tokens past T read as 0.
template <class G, typename O, bool H>
__global__ __launch_bounds__(G::THREADS, 1) void wgrad_mfma_kernel(const uint16_t* __restrict__ dY,
                                                                 const uint16_t* __restrict__ X, int T, int N, int K,
                                                                 const uint32_t* __restrict__ meta,
                                                                 O* __restrict__ dWv, O* __restrict__ dWd,
                                                                 int accumulate) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wk = wave % G::WGK, wn = wave / G::WGK;
  const int tiles_k = (K + G::BK - 1) / G::BK, tiles_n = (N + G::BN - 1) / G::BN;
  int tk, tn;
  tile_of_block(blockIdx.x, gridDim.x, tiles_k, tiles_n, 8, tk, tn);
  const int64_t k0 = (int64_t)tk * G::BK, n0 = (int64_t)tn * G::BN;
  const int stages = (T + G::TS - 1) / G::TS;

  // DMA lanes: row (token within the stage) and logical granule of each load
  int x_row[G::X_DMA], x_q[G::X_DMA], d_row[G::D_DMA], d_q[G::D_DMA];
#pragma unroll
  for (int j = 0; j < G::X_DMA; ++j) {
    const int row = wave * (G::TS / G::WAVES) + 2 * j + (lane >> 5);
    x_row[j] = row;
    x_q[j] = (lane & 31) ^ ((row & 3) << 2);
  }
#pragma unroll
  for (int j = 0; j < G::D_DMA; ++j) {
    const int row = wave * (G::TS / G::WAVES) + 2 * j + (lane >> 5);
    d_row[j] = row;
    d_q[j] = (lane & 31) ^ ((row & 3) << 2);
  }
  auto issue = [&](int s) {
    char* base = lds + (s % G::NST) * G::STAGE_BYTES;
    const int64_t ts = (int64_t)s * G::TS;
    // resources from this stage's first token to the end of each matrix
    const int64_t xrem = (int64_t)T * K - (ts * K + k0), drem = (int64_t)T * N - (ts * N + n0);
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + ts * K + k0, xrem > 0 ? xrem * 2 : 0);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(dY + ts * N + n0, drem > 0 ? drem * 2 : 0);
#pragma unroll
    for (int j = 0; j < G::X_DMA; ++j) {
      const bool ok = k0 + 8 * x_q[j] + 8 <= K;
      dma16(rx, base + wave * (G::X_BYTES / G::WAVES) + j * 1024, ok ? (uint32_t)(x_row[j] * K * 2 + x_q[j] * 16) : kOutOfRange);
    }
#pragma unroll
    for (int j = 0; j < G::D_DMA; ++j) {
      const bool ok = n0 + 8 * d_q[j] + 8 <= N;
      dma16(rd, base + G::X_BYTES + wave * (G::D_BYTES / G::WAVES) + j * 1024,
            ok ? (uint32_t)(d_row[j] * N * 2 + d_q[j] * 16) : kOutOfRange);
    }
  };

  struct Frags {
    typename Fmt16<H>::v8 x[G::FK];
    typename Fmt16<H>::v8 d[G::FN];
  };
  auto read_frags = [&](Frags& f, int s, int sub) {
    const char* base = lds + (s % G::NST) * G::STAGE_BYTES;
#pragma unroll
    for (int a = 0; a < G::FK; ++a) f.x[a] = frag_tr<H>(base, 16 * sub, wk * G::WK + a * 32, lane);
#pragma unroll
    for (int b = 0; b < G::FN; ++b) f.d[b] = frag_tr<H>(base + G::X_BYTES, 16 * sub, wn * G::WN + b * 32, lane);
  };

  f32x16 acc[G::FK][G::FN];
#pragma unroll
  for (int a = 0; a < G::FK; ++a)
#pragma unroll
    for (int b = 0; b < G::FN; ++b) acc[a][b] = f32x16{};
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int b = 0; b < G::FN; ++b)
#pragma unroll
      for (int a = 0; a < G::FK; ++a)
        acc[a][b] = Fmt16<H>::mfma32x32x16(f.x[a], f.d[b], acc[a][b]);
  };

#pragma unroll
  for (int p = 0; p < G::NST; ++p) issue(p);
  wait_vmcnt<(G::X_DMA + G::D_DMA) * (G::NST - 1)>();
  barrier();
  compiler_fence();                                        // the first LDS reads stay after the barrier
  Frags f0, f1;
  read_frags(f0, 0, 0);
  for (int s = 0; s < stages; ++s) {
    read_frags(f1, s, 1);
    mma(f0);
    __builtin_amdgcn_sched_barrier(0);                     // MFMAs stay ahead of the waits
    wait_lgkmcnt0();                                       // this wave's reads of stage s are in registers
    wait_vmcnt<(G::X_DMA + G::D_DMA) * (G::NST - 2)>();   // stage s+1 landed (this wave's part)
    barrier();                                             // everyone's part; stage s fully read
    issue(s + G::NST);                                     // refill stage s's slot; past the end these read 0
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < stages) read_frags(f0, s + 1, 0);
    mma(f1);
  }
  wait_vmcnt<0>();

  wgrad_store<G, O>(acc, meta, K, N, k0, n0, wk, wn, lane, dWv, dWd, accumulate, K / 2);
}

// ---------------------------------------------------------------- packed path
// Both operands are first rewritten, transposed, into "token chunks": for a
// matrix M [T, C] (C = K for X, N for dY), chunk (c, s) holds columns
// 256c .. 256c+255 (rows of the chunk) x tokens 32s .. 32s+31, 16 KB, at element
// offset (c * Tch + s) * 8192 (Tch = ceil(T / 32)).  A chunk row is 64 bytes:
// four 16-byte granules of 8 tokens, granule g stored at g ^ ((row >> 2) & 3) so
// that MFMA fragment reads from LDS are free of bank conflicts.  Entries past T
// or C are 0.  Each stage of the GEMM then takes one contiguous chunk per
// operand, and every MFMA fragment is one 16-byte piece of a chunk row (a
// plain 128-bit LDS read for X, a 128-bit load from memory for dY).
constexpr int kChunkRows = 256, kChunkTokens = 32, kChunkElems = kChunkRows * kChunkTokens;

__global__ __launch_bounds__(256) void pack_tokens_kernel(const uint16_t* __restrict__ src, int T, int C,
                                                          int64_t chunks_c, int64_t Tch, uint16_t* __restrict__ dst) {
  constexpr int kPitch = 264;                       // LDS row pitch in elements (528 bytes)
  __shared__ __attribute__((aligned(16))) uint16_t tile[kChunkTokens * kPitch];
  const int tid = threadIdx.x;
  const int64_t nchunks = chunks_c * Tch;
  for (int64_t q = blockIdx.x; q < nchunks; q += gridDim.x) {
    const int64_t cb = q % chunks_c, ts = q / chunks_c;
    // 32 token rows x 512 bytes, 16 bytes per load; all four loads in flight
    // at once (clamped addresses, entries past T or C then zeroed: loads under
    // a bounds branch would each be waited for)
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int piece = tid + 256 * j, t = piece >> 5, g = piece & 31;
      const int64_t tg = ts * kChunkTokens + t, cg = cb * kChunkRows + 8 * g;
      const int64_t tc = tg < T ? tg : T - 1, cc = cg < C ? cg : C - 8;   // C % 8 == 0
      v[j] = *reinterpret_cast<const u32x4*>(src + tc * C + cc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int piece = tid + 256 * j, t = piece >> 5, g = piece & 31;
      const int64_t tg = ts * kChunkTokens + t, cg = cb * kChunkRows + 8 * g;
      *reinterpret_cast<u32x4*>(&tile[t * kPitch + 8 * g]) = (tg < T && cg < C) ? v[j] : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    // thread r writes chunk row r: 8 tokens per granule
    const int r = tid;
    uint16_t* out = dst + (cb * Tch + ts) * kChunkElems + r * kChunkTokens;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = (uint32_t)tile[(8 * g + 2 * e) * kPitch + r] | ((uint32_t)tile[(8 * g + 2 * e + 1) * kPitch + r] << 16);
      *reinterpret_cast<u32x4*>(out + 8 * (g ^ ((r >> 2) & 3))) = v;
    }
    __syncthreads();
  }
}


// dW^T tile [256 k][256 n] from packed X (xp) and dY (dp): a dense MFMA GEMM
// over tokens, 32 per stage.  X's chunk of each stage passes through a ring of
// NST LDS stages filled by buffer-to-LDS loads (one barrier per stage, the
// same schedule as the sparse GEMM); the dY operand goes straight from its
// token chunks into registers, PD stages ahead of use, through a ring of
// PD + 1 register sets (a wave's dY fragments are 16-byte pieces of its 64
// chunk rows; past the last token chunk the loads read 0).  Compared with
// staging both operands in LDS this halves the LDS fill traffic and cuts the
// LDS fragment reads by a third.  Operands meet the MFMAs in the same
// positions and order as in the token-major kernel, so results are identical.
//
// PP (ping-pong): the waves form two groups, 0-3 and 4-7, one wave of each on
// every SIMD, running half a stage apart with two barriers per stage.  While
// one group issues a stage's MFMAs, the other issues its loads, reads the next
// stage's X fragments from LDS and waits, so each SIMD's matrix pipe always has
// one wave with MFMAs ready instead of both waves draining it at the same
// barrier.  Every load is issued in the same per-wave order as without PP (one
// stage's X, then the dY set PD stages ahead), so one wait count serves both.
template <int NST_, int PD_, bool PP_ = false>
struct DGeo {
  static constexpr int BK = 256, BN = 256, WGK = 2, WGN = 4, WAVES = 8, THREADS = 512;
  static constexpr int WK = BK / WGK, WN = BN / WGN, FK = WK / 32, FN = WN / 32;
  static constexpr bool PP = PP_;
  static constexpr int NST = NST_, PD = PD_, RING = PD_ + 1;
  static constexpr int CHUNK_BYTES = kChunkElems * 2;
  static constexpr int LDS_BYTES = NST * CHUNK_BYTES;
  static constexpr int DMA = CHUNK_BYTES / 1024 / WAVES;           // X loads per wave and stage
  static constexpr int DLOADS = 2 * FN;                            // dY loads per wave and stage
  // outstanding vector-memory operations allowed when X's next stage must have landed:
  // the later of the prologue's and the steady state's counts (both exact at their first use)
  static constexpr int W1 = (DMA + DLOADS) * (NST - 2) + DLOADS;
  static constexpr int W0 = DMA * (NST - 2) + DLOADS * PD;
  static constexpr int XWAIT = W1 < W0 ? W1 : W0;
  // PP prologue: X's first stage landed while group 1 still holds back the
  // last prologue phase (it issues that in its first phase in the loop)
  static constexpr int PWAIT = DMA * (NST - 2) + DLOADS * (PD - 1);
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(NST >= 2 && PD >= 1, "pipeline depth");
  static_assert(!PP || (NST >= 3 && PD >= 2 && PD <= NST - 1 && XWAIT == W0), "ping-pong wait counts");
};

//
// Token split (MODE kSplit, part != NULL): the grid holds `splits` copies of
// the tile grid; copy j sums token chunks [j * kc, min((j + 1) * kc, Tch)) only
// and writes its kept values in fp32 to part + j * N * (K / 2) (W_s's slot
// order, no dense copy, no accumulation); wgrad_split_reduce_kernel then adds
// the copies in order.  Used when the tile grid alone would leave most compute
// units idle.
//
// Tail split (MODE kTail): the first nb_main blocks (whole rounds of the
// device) run logical tiles 0 .. nb_main-1 as the plain kernel does; the
// remaining ntail tiles, which would run alone in a last, partly filled
// round, are cut into token ranges of kc chunks: block nb_main + j sums range
// j / ntail of tail tile j % ntail and writes its kept values in fp32 to that
// tile's own 256 x 128 buffer in part (range-major); wgrad_tail_reduce_kernel
// adds the ranges in order.
constexpr int kPlain = 0, kSplit = 1, kTail = 2;
constexpr int kTileValues = 256 * 128;     // kept values of one 256 x 256 output tile

template <class G, typename O, bool H, int MODE = kPlain>
__global__ __launch_bounds__(G::THREADS, 1) void wgrad_direct_kernel(const uint16_t* __restrict__ dp,
                                                                   const uint16_t* __restrict__ xp, int T, int N,
                                                                   int K, const uint32_t* __restrict__ meta,
                                                                   O* __restrict__ dWv, O* __restrict__ dWd,
                                                                   int accumulate, float* __restrict__ part, int kc,
                                                                   int nb_main, int ntail) {
  static_assert(G::BK == 256 && G::BN == 256, "tail buffers hold 256 x 256 tiles");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  // the wave index in a scalar register: the LDS addresses of the
  // buffer-to-LDS loads are then computed without vector temporaries
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wk = wave % G::WGK, wn = wave / G::WGK;
  const int tiles_k = (K + G::BK - 1) / G::BK, tiles_n = (N + G::BN - 1) / G::BN;
  const int ntiles = tiles_k * tiles_n;
  const bool tail = MODE == kTail && (int)blockIdx.x >= nb_main;          // block-uniform
  const int tj = tail ? (int)blockIdx.x - nb_main : 0;
  const int split = MODE == kSplit ? (int)blockIdx.x / ntiles : (tail ? tj / ntail : 0);
  int tk, tn;
  const int order_blocks = MODE == kSplit ? ntiles : (MODE == kTail ? nb_main : (int)gridDim.x);
  const int group = wgrad_group(order_blocks, tiles_k, tiles_n);
  if (tail)
    logical_tile(nb_main + tj % ntail, tiles_k, tiles_n, group, tk, tn);
  else
    tile_of_block(MODE == kSplit ? (int)blockIdx.x % ntiles : (int)blockIdx.x, order_blocks, tiles_k, tiles_n, group,
                  tk, tn);
  const int64_t k0 = (int64_t)tk * G::BK, n0 = (int64_t)tn * G::BN;
  const int64_t Tch = (T + kChunkTokens - 1) / kChunkTokens;
  // this block's token chunks [s_first, stages)
  const bool ranged = MODE == kSplit || tail;
  const int s_first = ranged ? split * kc : 0;
  const int stages = ranged ? (s_first + kc < (int)Tch ? s_first + kc : (int)Tch) : (int)Tch;
  const uint16_t* const xs = xp + (int64_t)tk * Tch * kChunkElems;
  const uint16_t* const ds = dp + (int64_t)tn * Tch * kChunkElems;
  const uint32_t src0 = (uint32_t)(wave * G::DMA * 1024);
  const uint32_t lane_off = (uint32_t)(lane * 16);

  auto issue_x = [&](int s) {
    char* base = lds + (s % G::NST) * G::CHUNK_BYTES;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(xs + (int64_t)s * kChunkElems, s < stages ? G::CHUNK_BYTES : 0);
#pragma unroll
    for (int j = 0; j < G::DMA; ++j) dma16(rx, base + src0 + j * 1024, src0 + j * 1024 + lane_off);
  };

  int x_off[2][G::FK];
  uint32_t d_off[2][G::FN];
#pragma unroll
  for (int a = 0; a < G::FK; ++a) {
    const int row = wk * G::WK + a * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) x_off[ks][a] = row * 64 + (((2 * ks + (lane >> 5)) ^ ((row >> 2) & 3)) << 4);
  }
#pragma unroll
  for (int b = 0; b < G::FN; ++b) {
    const int row = wn * G::WN + b * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) d_off[ks][b] = (uint32_t)(row * 64 + (((2 * ks + (lane >> 5)) ^ ((row >> 2) & 3)) << 4));
  }

  struct DFrags {
    typename Fmt16<H>::v8 d[2][G::FN];
  };
  auto load_d = [&](DFrags& f, int s) {
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(ds + (int64_t)s * kChunkElems, s < stages ? G::CHUNK_BYTES : 0);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int b = 0; b < G::FN; ++b) f.d[ks][b] = __builtin_bit_cast(typename Fmt16<H>::v8, load16(rd, d_off[ks][b]));
  };
  struct XFrags {
    typename Fmt16<H>::v8 x[G::FK];
  };
  auto read_x = [&](XFrags& f, int s, int ks) {
    const char* base = lds + (s % G::NST) * G::CHUNK_BYTES;
#pragma unroll
    for (int a = 0; a < G::FK; ++a) f.x[a] = *reinterpret_cast<const typename Fmt16<H>::v8*>(base + x_off[ks][a]);
  };

  f32x16 acc[G::FK][G::FN];
#pragma unroll
  for (int a = 0; a < G::FK; ++a)
#pragma unroll
    for (int b = 0; b < G::FN; ++b) acc[a][b] = f32x16{};
  auto mma = [&](const XFrags& f, const DFrags& d, int ks) {
#pragma unroll
    for (int b = 0; b < G::FN; ++b)
#pragma unroll
      for (int a = 0; a < G::FK; ++a)
        acc[a][b] = Fmt16<H>::mfma32x32x16(f.x[a], d.d[ks][b], acc[a][b]);
  };

  DFrags ring[G::RING];
  // whole groups of RING stages, at least one (the ring index stays static, no
  // early exit leaves the compiler's wait counting pessimistic, and no branch
  // around the loop lets the prologue's loads sink past its wait); stages past
  // the last token chunk read zeros and add nothing
  const int span = stages - s_first;
  const int stages_pad = s_first + (span <= G::RING ? G::RING : (span + G::RING - 1) / G::RING * G::RING);
  if constexpr (G::PP) {
    // Ping-pong.  Phases between barriers: group 0 runs M(s) (the 16 MFMAs of
    // stage s) then L(s) (the loads of X stage s+NST and dY stage s+PD, X's
    // fragments of stage s+1 into registers); group 1 runs L(s-1) then M(s).
    // Before the barrier that ends M(s) of group 0 and L(s-1) of group 1,
    // every wave has waited for its part of X stage s+1, so that barrier makes
    // the stage visible to both groups' next reads; X stage s is read by group
    // 0 before the previous barrier and by group 1 before this one, so the
    // loads into its slot (stage s+NST) are issued after it.
    const bool g1 = wave >= 4;                                   // wave-uniform
    // a barrier that no instruction is scheduled across, MFMAs included
    auto phase_barrier = [] {
      __builtin_amdgcn_sched_barrier(0);
      barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    // The prologue issues as the phases L(s_first - NST) .. L(s_first - 1)
    // would (each stage's X, then the dY set of the stage PD later, where
    // that is one of this block's), so that every dY set has the same loads
    // after it on entry to the loop as in the loop, and the compiler's waits
    // for them are as loose in the first stages as in the rest; group 1
    // leaves the last of these phases to its first phase in the loop.  Each
    // group has a code path of its own from the prologue on, so that neither
    // inherits the other's pending loads at the loop head.
    XFrags x0, x1;
    auto prologue = [&](int phases) {
#pragma unroll
      for (int p = 0; p < G::NST; ++p) {
        if (p < phases) {
          issue_x(s_first + p);
          if (p >= G::NST - G::PD) load_d(ring[p - (G::NST - G::PD)], s_first + p - (G::NST - G::PD));
        }
      }
      compiler_fence();
      wait_vmcnt<G::PWAIT>();                                    // X's first stage landed (this wave's part)
      phase_barrier();
      compiler_fence();
    };
    int s0 = s_first;
    if (!g1) {
      prologue(G::NST);
      read_x(x0, s_first, 0);
      read_x(x1, s_first, 1);
      do {
#pragma unroll
        for (int u = 0; u < G::RING; ++u) {
          const int s = s0 + u;
          mma(x0, ring[u], 0);
          mma(x1, ring[u], 1);
          wait_vmcnt<G::XWAIT>();                                // X's stage s+1 landed (this wave's part)
          phase_barrier();
          compiler_fence();
          issue_x(s + G::NST);
          load_d(ring[(u + G::PD) % G::RING], s + G::PD);
          read_x(x0, s + 1, 0);
          read_x(x1, s + 1, 1);
          wait_lgkmcnt0();                                       // stage s+1's fragments in registers
          phase_barrier();
          compiler_fence();
        }
        s0 += G::RING;
      } while (s0 < stages_pad);
    } else {
      prologue(G::NST - 1);
      do {
#pragma unroll
        for (int u = 0; u < G::RING; ++u) {
          const int s = s0 + u;
          issue_x(s - 1 + G::NST);
          load_d(ring[(u + G::PD - 1) % G::RING], s - 1 + G::PD);
          read_x(x0, s, 0);
          read_x(x1, s, 1);
          wait_lgkmcnt0();                                       // stage s's fragments in registers
          wait_vmcnt<G::XWAIT>();                                // X's stage s+1 landed (this wave's part)
          phase_barrier();
          compiler_fence();
          mma(x0, ring[u], 0);
          mma(x1, ring[u], 1);
          phase_barrier();
          compiler_fence();
        }
        s0 += G::RING;
      } while (s0 < stages_pad);
    }
  } else {
#pragma unroll
  for (int p = 0; p < G::NST; ++p) issue_x(s_first + p);
#pragma unroll
  for (int p = 0; p < G::PD; ++p) load_d(ring[p], s_first + p);
  compiler_fence();                                              // the loads above are counted by the wait
  wait_vmcnt<G::DMA * (G::NST - 1) + G::DLOADS * G::PD>();     // X's first stage landed (this wave's part)
  barrier();
  compiler_fence();                                              // the first LDS reads stay after the barrier
  XFrags x0, x1;
  read_x(x0, s_first, 0);
  int s0 = s_first;
  do {
#pragma unroll
    for (int u = 0; u < G::RING; ++u) {
      const int s = s0 + u;
      read_x(x1, s, 1);                                  // issued ahead of the MFMAs they overlap
      __builtin_amdgcn_sched_barrier(0);
      mma(x0, ring[u], 0);
      __builtin_amdgcn_sched_barrier(0);
      wait_lgkmcnt0();                                   // this wave's reads of stage s are in registers
      wait_vmcnt<G::XWAIT>();                            // X's stage s+1 landed (this wave's part)
      barrier();                                         // everyone's part; stage s fully read
      issue_x(s + G::NST);
      load_d(ring[(u + G::PD) % G::RING], s + G::PD);    // the set consumed one stage ago
      read_x(x0, s + 1, 0);
      mma(x1, ring[u], 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    s0 += G::RING;
  } while (s0 < stages_pad);
  }
  wait_vmcnt<0>();
  if constexpr (MODE == kSplit) {
    wgrad_store<G, float>(acc, meta, K, N, k0, n0, wk, wn, lane, part + (int64_t)split * N * (K / 2), nullptr, 0,
                          K / 2);
  } else {
    if (tail) {
      // the tile's own buffer, rows 128 values apart, shifted by its first row and group
      float* tb = part + (int64_t)(split * ntail + tj % ntail) * kTileValues - n0 * 128 - 2 * (k0 >> 2);
      wgrad_store<G, float>(acc, meta, K, N, k0, n0, wk, wn, lane, tb, nullptr, 0, 128);
    } else {
      wgrad_store<G, O>(acc, meta, K, N, k0, n0, wk, wn, lane, dWv, dWd, accumulate, K / 2);
    }
  }
}

// dW from the token split's fp32 partials: one thread per 2:4 group (n, g)
// adds the splits' two kept values in split order (then the previous values
// with accumulate), rounds once and writes the pair in slot order, and the
// masked dense copy from the group's metadata nibble.
template <typename O>
__global__ __launch_bounds__(256) void wgrad_split_reduce_kernel(const float* __restrict__ part, int splits,
                                                                 int64_t N, int64_t K,
                                                                 const uint32_t* __restrict__ meta,
                                                                 O* __restrict__ dWv, O* __restrict__ dWd,
                                                                 int accumulate) {
  const int64_t groups = N * (K / 4), plane = N * (K / 2), wpr = (K / 4 + 7) / 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < groups; i += (int64_t)gridDim.x * 256) {
    const int64_t n = i / (K / 4), g = i % (K / 4);
    const float* p = part + 2 * i;
    float v0 = 0.f, v1 = 0.f;
    int sp = 0;
    for (; sp + 4 <= splits; sp += 4) {            // four splits' loads in flight, added in order
      float2 x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) x[q] = *reinterpret_cast<const float2*>(p + (int64_t)(sp + q) * plane);
#pragma unroll
      for (int q = 0; q < 4; ++q) { v0 += x[q].x; v1 += x[q].y; }
    }
    for (; sp < splits; ++sp) {
      const float2 x = *reinterpret_cast<const float2*>(p + (int64_t)sp * plane);
      v0 += x.x;
      v1 += x.y;
    }
    O* vp = dWv + 2 * i;
    // the dense copy from the new sums (store_quad adds its own previous values)
    if (dWd) {
      const uint32_t nib = (meta[n * wpr + (g >> 3)] >> (4 * (g & 7))) & 0xFu;
      const uint32_t i0 = nib & 3u, i1 = nib >> 2;
      const float x[4] = {i0 == 0 ? v0 : 0.f, i0 == 1 ? v0 : (i1 == 1 ? v1 : 0.f),
                          i0 == 2 ? v0 : (i1 == 2 ? v1 : 0.f), i1 == 3 ? v1 : 0.f};
      store_quad(dWd + n * K + 4 * g, x, accumulate);
    }
    if (accumulate) { v0 += load_out(vp); v1 += load_out(vp + 1); }
    store_pair(vp, v0, v1);
  }
}

// dW of the tail tiles from their token ranges' fp32 partials (part: range-major
// [ranges][ntail][256 n][128 values]): block (tile i, rows 4b .. 4b+3), thread
// (row, group) adds the ranges' two kept values in range order, then as
// wgrad_split_reduce_kernel (dense copy, accumulate, one rounding).
template <typename O>
__global__ __launch_bounds__(256) void wgrad_tail_reduce_kernel(const float* __restrict__ part, int ranges, int ntail,
                                                                int nb_main, int tiles_k, int tiles_n, int64_t N,
                                                                int64_t K, const uint32_t* __restrict__ meta,
                                                                O* __restrict__ dWv, O* __restrict__ dWd,
                                                                int accumulate) {
  const int i = (int)blockIdx.x / 64, rb = (int)blockIdx.x % 64;
  int tk, tn;
  logical_tile(nb_main + i, tiles_k, tiles_n, wgrad_group(nb_main, tiles_k, tiles_n), tk, tn);
  const int nl = rb * 4 + (int)(threadIdx.x >> 6), gl = (int)(threadIdx.x & 63);
  const int64_t n = (int64_t)tn * 256 + nl, g = (int64_t)tk * 64 + gl;
  if (n >= N || 4 * g >= K) return;
  const int64_t plane = (int64_t)ntail * kTileValues, wpr = (K / 4 + 7) / 8;
  const float* p = part + (int64_t)i * kTileValues + nl * 128 + 2 * gl;
  float v0 = 0.f, v1 = 0.f;
  int sp = 0;
  for (; sp + 4 <= ranges; sp += 4) {              // four ranges' loads in flight, added in order
    float2 x[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = *reinterpret_cast<const float2*>(p + (int64_t)(sp + q) * plane);
#pragma unroll
    for (int q = 0; q < 4; ++q) { v0 += x[q].x; v1 += x[q].y; }
  }
  for (; sp < ranges; ++sp) {
    const float2 x = *reinterpret_cast<const float2*>(p + (int64_t)sp * plane);
    v0 += x.x;
    v1 += x.y;
  }
  O* vp = dWv + n * (K / 2) + 2 * g;
  if (dWd) {
    const uint32_t nib = (meta[n * wpr + (g >> 3)] >> (4 * (g & 7))) & 0xFu;
    const uint32_t i0 = nib & 3u, i1 = nib >> 2;
    const float x[4] = {i0 == 0 ? v0 : 0.f, i0 == 1 ? v0 : (i1 == 1 ? v1 : 0.f),
                        i0 == 2 ? v0 : (i1 == 2 ? v1 : 0.f), i1 == 3 ? v1 : 0.f};
    store_quad(dWd + n * K + 4 * g, x, accumulate);
  }
  if (accumulate) { v0 += load_out(vp); v1 += load_out(vp + 1); }
  store_pair(vp, v0, v1);
}

typedef DGeo<8, 3, true> DGeoBig;

int64_t chunks_of(int64_t C) { return (C + kChunkRows - 1) / kChunkRows; }
int64_t token_chunks(int64_t T) { return (T + kChunkTokens - 1) / kChunkTokens; }

hipError_t launch_pack(const uint16_t* src, int64_t T, int64_t C, uint16_t* dst, hipStream_t s) {
  const int64_t n = chunks_of(C) * token_chunks(T);
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)(n < (1 << 20) ? n : (1 << 20));
  pack_tokens_kernel<<<grid, 256, 0, s>>>(src, (int)T, (int)C, chunks_of(C), token_chunks(T), dst);
  return hipGetLastError();
}

// Token split of the weight-gradient GEMM: when the tile grid fills fewer
// than half the compute units, run `splits` token ranges of kc chunks each
// (at least kMinSplitChunks chunks, 256 tokens, per range) so that about one
// round of blocks runs; 1 = no split.
constexpr int64_t kMinSplitChunks = 8;
struct WgradSplit {
  int64_t splits, kc;
};
WgradSplit wgrad_split_plan(int64_t T, int64_t N, int64_t K, int64_t cus) {
  const int64_t nb = chunks_of(K) * chunks_of(N), tch = token_chunks(T);
  WgradSplit p{1, tch};
  if (nb == 0 || tch < 2 * kMinSplitChunks || 2 * nb > cus) return p;
  int64_t want = cus / nb;
  const int64_t most = tch / kMinSplitChunks;
  if (want > most) want = most;
  if (want < 2) return p;
  p.kc = cdiv(tch, want);
  p.splits = cdiv(tch, p.kc);
  return p;
}

// Tail split of the weight-gradient GEMM: when the tiles fill more than one
// round of blocks and the last round is at most three quarters full, that
// round's tiles run in `ranges` token ranges of kc chunks (at least
// kMinSplitChunks each, about one round of blocks in all); ntail = 0: no tail split.
struct WgradTail {
  int64_t nb_main, ntail, ranges, kc;
};
WgradTail wgrad_tail_plan(int64_t T, int64_t N, int64_t K, int64_t cus) {
  const int64_t nb = chunks_of(K) * chunks_of(N), tch = token_chunks(T);
  WgradTail p{nb, 0, 1, tch};
  if (cus < 1 || nb <= cus) return p;
  const int64_t tail = nb % cus;
  if (tail == 0 || 4 * tail > 3 * cus) return p;
  int64_t want = cus / tail;
  const int64_t most = tch / kMinSplitChunks;
  if (want > most) want = most;
  if (want < 2) return p;
  p.kc = cdiv(tch, want);
  p.ranges = cdiv(tch, p.kc);
  if (p.ranges < 2) return p;
  p.nb_main = nb - tail;
  p.ntail = tail;
  return p;
}

template <typename O, bool H>
hipError_t launch_packed(const uint16_t* dp, const uint16_t* xp, int64_t T, int64_t N, int64_t K,
                         const uint32_t* meta, O* dWv, O* dWd, int accumulate, float* part, hipStream_t s) {
  typedef DGeoBig G;
  auto kern = wgrad_direct_kernel<G, O, H, kPlain>;
  auto kern_split = wgrad_direct_kernel<G, O, H, kSplit>;
  auto kern_tail = wgrad_direct_kernel<G, O, H, kTail>;
  static hipError_t attr = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  const int64_t nb = chunks_of(K) * chunks_of(N), cus = device_compute_units();
  const WgradSplit sp = part ? wgrad_split_plan(T, N, K, cus) : WgradSplit{1, token_chunks(T)};
  const WgradTail tp = part ? wgrad_tail_plan(T, N, K, cus) : WgradTail{nb, 0, 1, token_chunks(T)};
  if (tp.ntail > 0) {
    static hipError_t attr_tail =
        hipFuncSetAttribute((const void*)kern_tail, hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS_BYTES);
    if (attr_tail != hipSuccess) return attr_tail;
    kern_tail<<<(unsigned)(tp.nb_main + tp.ntail * tp.ranges), G::THREADS, G::LDS_BYTES, s>>>(
        dp, xp, (int)T, (int)N, (int)K, meta, dWv, dWd, accumulate, part, (int)tp.kc, (int)tp.nb_main,
        (int)tp.ntail);
    wgrad_tail_reduce_kernel<O><<<(unsigned)(tp.ntail * 64), 256, 0, s>>>(
        part, (int)tp.ranges, (int)tp.ntail, (int)tp.nb_main, (int)chunks_of(K), (int)chunks_of(N), N, K, meta, dWv,
        dWd, accumulate);
    return hipGetLastError();
  }
  if (sp.splits < 2) {
    kern<<<(unsigned)nb, G::THREADS, G::LDS_BYTES, s>>>(dp, xp, (int)T, (int)N, (int)K, meta, dWv, dWd, accumulate,
                                                        nullptr, 0, 0, 0);
    return hipGetLastError();
  }
  static hipError_t attr_split =
      hipFuncSetAttribute((const void*)kern_split, hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS_BYTES);
  if (attr_split != hipSuccess) return attr_split;
  kern_split<<<(unsigned)(nb * sp.splits), G::THREADS, G::LDS_BYTES, s>>>(dp, xp, (int)T, (int)N, (int)K, meta, dWv,
                                                                          dWd, accumulate, part, (int)sp.kc, 0, 0);
  const int64_t groups = N * (K / 4);
  const unsigned grid = (unsigned)std::min<int64_t>(cdiv(groups, 256), 4096);
  wgrad_split_reduce_kernel<O><<<grid, 256, 0, s>>>(part, (int)sp.splits, N, K, meta, dWv, dWd, accumulate);
  return hipGetLastError();
}

typedef WGeo<256, 256, 4, 2, 4> WGeoBig;

template <typename O, bool H>
hipError_t launch_token_major(const void* dY, const void* X, int64_t T, int64_t N, int64_t K, const uint32_t* meta,
                              O* dWv, O* dWd, int accumulate, hipStream_t s) {
  typedef WGeoBig G;
  const int64_t nb = cdiv(K, G::BK) * cdiv(N, G::BN);
  auto kern = wgrad_mfma_kernel<G, O, H>;
  static hipError_t attr = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  kern<<<(unsigned)nb, G::THREADS, G::LDS_BYTES, s>>>((const uint16_t*)dY, (const uint16_t*)X, (int)T, (int)N, (int)K,
                                                    meta, dWv, dWd, accumulate);
  return hipGetLastError();
}

}  // namespace

int64_t wgrad_workspace_bytes(int64_t T, int64_t N, int64_t K) {
  return (chunks_of(K) + chunks_of(N)) * token_chunks(T) * kChunkElems * 2;
}


int64_t packed_tokens_bytes(int64_t T, int64_t C) { return chunks_of(C) * token_chunks(T) * kChunkElems * 2; }

int64_t wgrad_split_bytes(int64_t T, int64_t N, int64_t K) {
  const int64_t cus = device_compute_units();
  const WgradSplit sp = wgrad_split_plan(T, N, K, cus);
  if (sp.splits >= 2) return cdiv(sp.splits * N * (K / 2) * 4, 256) * 256;
  const WgradTail tp = wgrad_tail_plan(T, N, K, cus);
  return tp.ntail > 0 ? cdiv(tp.ranges * tp.ntail * kTileValues * 4, 256) * 256 : 0;
}

hipError_t launch_pack_tokens(const void* M, int64_t T, int64_t C, void* packed, hipStream_t s) {
  return launch_pack((const uint16_t*)M, T, C, (uint16_t*)packed, s);
}

hipError_t launch_masked_wgrad_packed(Dt in, Dt out, const void* dY_packed, const void* X_packed, int64_t T,
                                      int64_t N, int64_t K, const uint32_t* meta_s, void* dW_values, void* dW_dense,
                                      int accumulate, void* split_part, hipStream_t s) {
  const uint16_t* dp = (const uint16_t*)dY_packed;
  const uint16_t* xp = (const uint16_t*)X_packed;
  float* part = (float*)split_part;
  if (out == Dt::BF16)
    return launch_packed<uint16_t, false>(dp, xp, T, N, K, meta_s, (uint16_t*)dW_values, (uint16_t*)dW_dense,
                                          accumulate, part, s);
  if (out == Dt::F16)
    return launch_packed<_Float16, true>(dp, xp, T, N, K, meta_s, (_Float16*)dW_values, (_Float16*)dW_dense,
                                         accumulate, part, s);
  if (in == Dt::F16)
    return launch_packed<float, true>(dp, xp, T, N, K, meta_s, (float*)dW_values, (float*)dW_dense, accumulate, part,
                                      s);
  return launch_packed<float, false>(dp, xp, T, N, K, meta_s, (float*)dW_values, (float*)dW_dense, accumulate, part,
                                     s);
}

hipError_t launch_masked_wgrad(Dt in, Dt out, const void* dY, const void* X, int64_t T, int64_t N, int64_t K,
                               const uint32_t* meta_s, void* dW_values, void* dW_dense, int accumulate,
                               void* workspace, hipStream_t s) {
  const bool fast = in != Dt::F32 && K % 8 == 0 && N % 8 == 0;
  if (!fast) return launch_wgrad_generic(in, out, dY, X, T, N, K, meta_s, dW_values, dW_dense, accumulate, s);
  if (workspace != nullptr) {
    // packed path: transpose both operands into token chunks, then one GEMM
    char* xp = (char*)workspace;
    char* dp = xp + packed_tokens_bytes(T, K);
    hipError_t e = launch_pack_tokens(X, T, K, xp, s);
    if (e != hipSuccess) return e;
    e = launch_pack_tokens(dY, T, N, dp, s);
    if (e != hipSuccess) return e;
    return launch_masked_wgrad_packed(in, out, dp, xp, T, N, K, meta_s, dW_values, dW_dense, accumulate, nullptr, s);
  }
  if (out == Dt::BF16)
    return launch_token_major<uint16_t, false>(dY, X, T, N, K, meta_s, (uint16_t*)dW_values, (uint16_t*)dW_dense,
                                               accumulate, s);
  if (out == Dt::F16)
    return launch_token_major<_Float16, true>(dY, X, T, N, K, meta_s, (_Float16*)dW_values, (_Float16*)dW_dense,
                                              accumulate, s);
  if (in == Dt::F16)
    return launch_token_major<float, true>(dY, X, T, N, K, meta_s, (float*)dW_values, (float*)dW_dense, accumulate,
                                           s);
  return launch_token_major<float, false>(dY, X, T, N, K, meta_s, (float*)dW_values, (float*)dW_dense, accumulate,
                                          s);
}

}  // namespace slope

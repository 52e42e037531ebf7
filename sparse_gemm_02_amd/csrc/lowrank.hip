// Low-rank adapter term Y += (X . L) . R (SLoPe explainer, Technical Summary
// 2.B: W_dense = W_sparse + L R; kept unmerged at inference per the discussion
// page's "SLoPe inference computation"; 2.C fuses it with the sparse product).
//
// The down-projection X . L is computed once per call into the caller's
// workspace (partial sums over k-splits, reduced in a fixed order, so results
// are deterministic); the up-projection is an MFMA epilogue over the rank,
// either fused into the sparse GEMM (spmm.hip) or run here on its own.
#include "common.h"
#include "dma.h"
#include "gemm_tile.h"
#include "launch.h"
#include "tile_map.h"

namespace slope {

hipError_t launch_lowrank_down_generic(Dt in, const void* X, const void* L, int64_t T, int64_t K, int64_t r,
                                       int splits, int64_t kc, float* xl, hipStream_t s);
hipError_t launch_lowrank_up_generic(Dt in, Dt out, const float* xl, int splits, const void* R, int64_t T,
                                     int64_t r, int64_t N, void* Y, hipStream_t s);

namespace {

constexpr int kDownWaveRows = 64;                  // tokens per down-projection wave
constexpr int kDownRows = 4 * kDownWaveRows;       // tokens per down-projection block
constexpr int kRankMax = 128;    // largest rank of the MFMA down-projection

int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// ------------------------------------------------------------------ layout helpers
struct Sizes {
  int splits;
  int64_t kc, rpad, Tpad, Kpad, Npad, part, xl, lt, rt;
};

// k splits of the down-projection: one block (256 tokens, one k range) per
// compute unit and round, so that whole rounds of blocks run (256 / token
// blocks splits), doubled as long as every block keeps 32 or more stages of
// 64 k; at most one split per 64 k.
int choose_splits(int64_t T, int64_t K) {
  const int64_t tblocks = cdiv(T, kDownRows) < 1 ? 1 : cdiv(T, kDownRows);
  int64_t want = 256 / tblocks < 1 ? 1 : 256 / tblocks;
  while (want * 2 * 64 * 32 <= K && want * 2 * tblocks <= 1024) want *= 2;
  const int64_t ksteps = cdiv(K, 64);
  if (want > ksteps) want = ksteps;
  if (want < 1) want = 1;
  return (int)want;
}

Sizes sizes(int64_t T, int64_t K, int64_t r, int64_t N) {
  Sizes z{};
  int splits = choose_splits(T, K);
  z.kc = round_up(cdiv(K, splits), 64);
  z.splits = z.kc > 0 ? (int)cdiv(K, z.kc) : 1;   // every split non-empty
  if (z.splits < 1) z.splits = 1;
  z.rpad = round_up(r, 16);
  z.Tpad = round_up(T, 256);
  z.Kpad = round_up(K, 8);
  z.Npad = round_up(N, 256);
  z.part = round_up((int64_t)z.splits * T * r * 4, 256);
  z.xl = round_up(z.Tpad * z.rpad * 2, 256);
  z.lt = round_up(z.rpad * z.Kpad * 2, 256);
  z.rt = round_up(z.Npad * z.rpad * 2, 256);
  return z;
}

// ------------------------------------------------------------------ prepare kernels
// lt[j][k] = L[k][j] for j < r, k < K; 0 in the padding.  Thread (k-group of
// eight, j) with j fastest: the reads of a wave cover consecutive j of eight
// rows of L, the write is one 16-byte piece of a row of lt (Kpad % 8 == 0).
__device__ __forceinline__ void transpose_l_body(int64_t bid, const uint16_t* __restrict__ L, int64_t K, int64_t r,
                                                 int64_t rpad, int64_t Kpad, uint16_t* __restrict__ lt) {
  const int64_t i = bid * 256 + threadIdx.x;
  if (i >= rpad * (Kpad / 8)) return;
  const int64_t j = i % rpad, k0 = (i / rpad) * 8;
  uint16_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (j < r && k0 + e < K) ? L[(k0 + e) * r + j] : (uint16_t)0;
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = v[2 * e] | ((uint32_t)v[2 * e + 1] << 16);
  *reinterpret_cast<u32x4*>(lt + j * Kpad + k0) = w;
}

// rt[n][j] = R[j][n] for j < r, n < N; 0 in the padding.  Thread (n, j-group
// of eight) with n fastest: reads cover consecutive n of eight rows of R, the
// write is one 16-byte piece of a row of rt (rpad % 8 == 0).
__device__ __forceinline__ void transpose_r_body(int64_t bid, const uint16_t* __restrict__ R, int64_t r, int64_t N,
                                                 int64_t rpad, int64_t Npad, uint16_t* __restrict__ rt) {
  const int64_t i = bid * 256 + threadIdx.x;
  if (i >= Npad * (rpad / 8)) return;
  const int64_t n = i % Npad, j0 = (i / Npad) * 8;
  uint16_t v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (j0 + e < r && n < N) ? R[(j0 + e) * N + n] : (uint16_t)0;
  u32x4 w;
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = v[2 * e] | ((uint32_t)v[2 * e + 1] << 16);
  *reinterpret_cast<u32x4*>(rt + n * rpad + j0) = w;
}

__global__ __launch_bounds__(256) void transpose_l_kernel(const uint16_t* __restrict__ L, int64_t K, int64_t r,
                                                          int64_t rpad, int64_t Kpad, uint16_t* __restrict__ lt) {
  transpose_l_body(blockIdx.x, L, K, r, rpad, Kpad, lt);
}

// Both transposes of the forward's adapter operands in one launch: blocks
// below nl transpose L, the others R.
__global__ __launch_bounds__(256) void transpose_lr_kernel(const uint16_t* __restrict__ L, int64_t K, int64_t r,
                                                           int64_t rpad, int64_t Kpad, uint16_t* __restrict__ lt,
                                                           unsigned nl, const uint16_t* __restrict__ R, int64_t N,
                                                           int64_t Npad, uint16_t* __restrict__ rt) {
  if (blockIdx.x < nl)
    transpose_l_body(blockIdx.x, L, K, r, rpad, Kpad, lt);
  else
    transpose_r_body(blockIdx.x - nl, R, r, N, rpad, Npad, rt);
}

// dst[i][j] = src[i][j] for i < rows, j < cols (src row-major, cols wide); 0 in
// the padding up to [rows_pad, cols_pad].  The adapter backward uses it for the
// operands that need no transposition there: R [r, N] as the down-projection's
// [rpad, Kpad] operand and L [K, r] as the epilogue's [Npad, rpad] operand.
__device__ __forceinline__ void pad_copy_body(int64_t bid, const uint16_t* __restrict__ src, int64_t rows,
                                              int64_t cols, int64_t rows_pad, int64_t cols_pad,
                                              uint16_t* __restrict__ dst) {
  const int64_t i = bid * 256 + threadIdx.x;
  if (i >= rows_pad * cols_pad) return;
  const int64_t a = i / cols_pad, b = i % cols_pad;
  dst[i] = (a < rows && b < cols) ? src[a * cols + b] : (uint16_t)0;
}

// Both padded copies of the dX product's adapter operands in one launch:
// blocks below n1 copy R as [rpad, Kpad], the others L as [Npad, rpad].
__global__ __launch_bounds__(256) void pad_copy2_kernel(const uint16_t* __restrict__ src1, int64_t rows1,
                                                        int64_t cols1, int64_t rows_pad1, int64_t cols_pad1,
                                                        uint16_t* __restrict__ dst1, unsigned n1,
                                                        const uint16_t* __restrict__ src2, int64_t rows2,
                                                        int64_t cols2, int64_t rows_pad2, int64_t cols_pad2,
                                                        uint16_t* __restrict__ dst2) {
  if (blockIdx.x < n1)
    pad_copy_body(blockIdx.x, src1, rows1, cols1, rows_pad1, cols_pad1, dst1);
  else
    pad_copy_body(blockIdx.x - n1, src2, rows2, cols2, rows_pad2, cols_pad2, dst2);
}

// xt[j][t] = x[t][j] for the hi and lo parts (x [Tpad][rpad] -> xt [rpad32][Tpad],
// rows j >= rpad zero).  Thread (j, t) with t fastest: coalesced writes.
// Two such transposes (X . L and dY . R^T for the adapter's gradients) in one
// launch: blocks below n1 take the first.
__global__ __launch_bounds__(256) void transpose_hilo2_kernel(const uint16_t* __restrict__ xh1,
                                                              const uint16_t* __restrict__ xl1, int64_t Tpad1,
                                                              int64_t rpad1, uint16_t* __restrict__ xht1,
                                                              uint16_t* __restrict__ xlt1, unsigned n1,
                                                              const uint16_t* __restrict__ xh2,
                                                              const uint16_t* __restrict__ xl2, int64_t Tpad2,
                                                              int64_t rpad2, uint16_t* __restrict__ xht2,
                                                              uint16_t* __restrict__ xlt2, int64_t rpad32) {
  const bool first = blockIdx.x < n1;
  const int64_t i = (int64_t)(first ? blockIdx.x : blockIdx.x - n1) * 256 + threadIdx.x;
  const int64_t Tpad = first ? Tpad1 : Tpad2, rpad = first ? rpad1 : rpad2;
  const uint16_t* xh = first ? xh1 : xh2;
  const uint16_t* xl = first ? xl1 : xl2;
  uint16_t* xht = first ? xht1 : xht2;
  uint16_t* xlt = first ? xlt1 : xlt2;
  if (i >= rpad32 * Tpad) return;
  const int64_t j = i / Tpad, t = i % Tpad;
  const bool in = j < rpad;
  xht[i] = in ? xh[t * rpad + j] : (uint16_t)0;
  xlt[i] = in ? xl[t * rpad + j] : (uint16_t)0;
}

// part[s][t][j] = sum over k in split s of X[t][k] lt[j][k], with both operands staged
// in LDS: each stage of 64 k brings the block's 256 token rows of X (128 bytes
// each, whole cache lines) and the same 64 k of the RP rows of L^T into a ring
// of three slots by buffer-to-LDS loads (rows and k past the block's range
// read 0), so X streams at line granularity and L^T is fetched once per block
// instead of once per wave.  16-byte granule c of a 128-byte LDS row r sits at
// c ^ ((r ^ (r >> 3)) & 7) (fragment reads of 16 rows hit distinct banks).  A
// wave owns 64 tokens (four 16-row MFMA A operands) and every rank column (NJ
// blocks of 16), 32 k per 16x16x32 MFMA step in order.  Dense 16x16x32 MFMA:
// A lane l = row l%16, k = 8*(l/16)+e; B lane l = column l%16, same k; D lane
// l = column l%16, rows 4*(l/16)+v.
template <int NJ>
struct DownLds {
  static constexpr int RP = NJ * 16;                          // rank rows of L^T per stage
  static constexpr int X_DMA = 256 * 128 / 1024 / 4;           // 1 KB loads per wave and stage: 8
  static constexpr int LT_DMA = (RP / 8 + 3) / 4;             // 8 rank rows per load, spread over 4 waves
  static constexpr int X_BYTES = 256 * 128, LT_BYTES = LT_DMA * 4 * 1024;
  static constexpr int SLOT = X_BYTES + LT_BYTES, NST = 3, LDS_BYTES = NST * SLOT;
  static constexpr int DMA_PER_STAGE = X_DMA + LT_DMA;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <int NJ, bool H>
__global__ __launch_bounds__(256, 1) void lowrank_down_lds_kernel(const uint16_t* __restrict__ X,
                                                                  const uint16_t* __restrict__ lt, int T, int K,
                                                                  int rpad, int Kpad, int kc, int r,
                                                                  float* __restrict__ part) {
  typedef DownLds<NJ> D;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int G = kDownWaveRows / 16;                         // 16-token operands per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int split = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kDownRows;
  const int kb = split * kc, ke = (kb + kc < K) ? kb + kc : K;
  const int stages = (ke - kb + 63) / 64;
  const int64_t rows_t = (T - t0) < kDownRows ? (T - t0) : kDownRows;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + t0 * K, rows_t * K * 2);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(lt, (int64_t)rpad * Kpad * 2);
  // DMA lanes: 8 rows x 8 granules per 1 KB load; lane i -> row i / 8, stored granule i % 8
  uint32_t x_src[D::X_DMA], l_src[D::LT_DMA];
  int x_k[D::X_DMA], l_k[D::LT_DMA];
  bool l_ok[D::LT_DMA];
#pragma unroll
  for (int j = 0; j < D::X_DMA; ++j) {
    const int row = (wave * D::X_DMA + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row ^ (row >> 3)) & 7);
    x_src[j] = (uint32_t)(row * K + kb + c * 8) * 2;
    x_k[j] = kb + c * 8;
  }
#pragma unroll
  for (int j = 0; j < D::LT_DMA; ++j) {
    const int row = (wave * D::LT_DMA + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row ^ (row >> 3)) & 7);
    l_src[j] = (uint32_t)(row * Kpad + kb + c * 8) * 2;
    l_k[j] = kb + c * 8;
    l_ok[j] = row < rpad;
  }
  auto issue = [&](int st) {
    char* base = lds + (st % D::NST) * D::SLOT;
#pragma unroll
    for (int j = 0; j < D::X_DMA; ++j) {
      const bool ok = st < stages && x_k[j] + st * 64 < ke;
      dma16(rx, base + (wave * D::X_DMA + j) * 1024, ok ? x_src[j] + st * 128 : kOutOfRange);
    }
#pragma unroll
    for (int j = 0; j < D::LT_DMA; ++j) {
      const bool ok = l_ok[j] && st < stages && l_k[j] + st * 64 < ke;
      dma16(rl, base + D::X_BYTES + (wave * D::LT_DMA + j) * 1024, ok ? l_src[j] + st * 128 : kOutOfRange);
    }
  };
  // fragment offsets: A row = token wave*64 + 16g + lane%16, B row = rank 16jb + lane%16;
  // k step ks takes logical granule 4ks + lane/16 of the stage's 128-byte row
  int a_off[2][G], b_off[2][NJ];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int row = wave * kDownWaveRows + g * 16 + (lane & 15);
      a_off[ks][g] = row * 128 + (((4 * ks + (lane >> 4)) ^ ((row ^ (row >> 3)) & 7)) << 4);
    }
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) {
      const int row = jb * 16 + (lane & 15);
      b_off[ks][jb] = D::X_BYTES + row * 128 + (((4 * ks + (lane >> 4)) ^ ((row ^ (row >> 3)) & 7)) << 4);
    }
  }
  f32x4 acc[G][NJ];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[g][j] = f32x4{};
  typedef typename Fmt16<H>::v8 v8;

#pragma unroll
  for (int p = 0; p < D::NST; ++p) issue(p);
  wait_vmcnt<D::DMA_PER_STAGE * (D::NST - 1)>();
  barrier();
  compiler_fence();
  for (int st = 0; st < stages; ++st) {
    const char* base = lds + (st % D::NST) * D::SLOT;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8 a[G], b[NJ];
#pragma unroll
      for (int g = 0; g < G; ++g) a[g] = *reinterpret_cast<const v8*>(base + a_off[ks][g]);
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb) b[jb] = *reinterpret_cast<const v8*>(base + b_off[ks][jb]);
#pragma unroll
      for (int jb = 0; jb < NJ; ++jb)
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g][jb] = Fmt16<H>::mfma16x16x32(a[g], b[jb], acc[g][jb]);
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkmcnt0();                                  // this wave's reads of stage st are in registers
    wait_vmcnt<D::DMA_PER_STAGE * (D::NST - 2)>();   // this wave's share of stage st+1 landed
    barrier();                                        // everyone's; stage st fully read
    compiler_fence();
    issue(st + D::NST);                               // refill st's slot (past the range: zeros)
  }
  wait_vmcnt<0>();
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb) {
    const int j = jb * 16 + (lane & 15);
    if (j >= r) continue;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t t = t0 + wave * kDownWaveRows + 16 * g + 4 * (lane >> 4) + v;
        if (t < T) part[((int64_t)split * T + t) * r + j] = acc[g][jb][v];
      }
  }
}

template <int NJ, bool H>
hipError_t down_nj_fmt(dim3 grid, const uint16_t* X, const uint16_t* lt, int64_t T, int64_t K, int64_t r,
                       const LowrankWs& w, hipStream_t s) {
  typedef DownLds<NJ> D;
  auto kern = lowrank_down_lds_kernel<NJ, H>;
  static hipError_t attr = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, D::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  kern<<<grid, 256, D::LDS_BYTES, s>>>(X, lt, (int)T, (int)K, (int)w.rpad, (int)w.Kpad, (int)w.kc, (int)r, w.part);
  return hipSuccess;
}

template <int NJ>
hipError_t down_nj(dim3 grid, const uint16_t* X, const uint16_t* lt, int64_t T, int64_t K, int64_t r,
                   const LowrankWs& w, hipStream_t s) {
  return w.h16 ? down_nj_fmt<NJ, true>(grid, X, lt, T, K, r, w, s) : down_nj_fmt<NJ, false>(grid, X, lt, T, K, r, w, s);
}

hipError_t launch_down(const uint16_t* X, const uint16_t* lt, int64_t T, int64_t K, int64_t r, const LowrankWs& w,
                       hipStream_t s) {
  const dim3 grid((unsigned)cdiv(T, kDownRows), (unsigned)w.splits);
  hipError_t e = hipSuccess;
  switch (w.rpad / 16) {
    case 1: e = down_nj<1>(grid, X, lt, T, K, r, w, s); break;
    case 2: e = down_nj<2>(grid, X, lt, T, K, r, w, s); break;
    case 3: e = down_nj<3>(grid, X, lt, T, K, r, w, s); break;
    case 4: e = down_nj<4>(grid, X, lt, T, K, r, w, s); break;
    case 5: e = down_nj<5>(grid, X, lt, T, K, r, w, s); break;
    case 6: e = down_nj<6>(grid, X, lt, T, K, r, w, s); break;
    case 7: e = down_nj<7>(grid, X, lt, T, K, r, w, s); break;
    case 8: e = down_nj<8>(grid, X, lt, T, K, r, w, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

// xl = sum over splits of part (in split order), split into a 16-bit hi + lo
// (bf16, or fp16 with H) with hi = rne(xl), lo = rne(xl - hi); zero in the
// padding.
template <bool H>
__global__ __launch_bounds__(256) void reduce_split_kernel(const float* __restrict__ part, int splits, int64_t T,
                                                           int64_t r, int64_t rpad, int64_t Tpad,
                                                           uint16_t* __restrict__ xlh, uint16_t* __restrict__ xll) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= Tpad * rpad) return;
  const int64_t t = i / rpad, j = i % rpad;
  float x = 0.f;
  if (t < T && j < r) {
#pragma unroll 8
    for (int s = 0; s < splits; ++s) x += part[((int64_t)s * T + t) * r + j];
  }
  const uint16_t hi = Fmt16<H>::from_f32(x);
  xlh[i] = hi;
  xll[i] = Fmt16<H>::from_f32(x - Fmt16<H>::to_f32(hi));
}

// ------------------------------------------------------------------ standalone up-projection
// Y[t][m] += (X . L)[t] . R[:, m] over one 256 x 256 output tile.
template <class G, typename O, bool H>
__global__ __launch_bounds__(G::THREADS, 1) void lowrank_up_add_kernel(const uint16_t* __restrict__ rt,
                                                                       const uint16_t* __restrict__ xlh,
                                                                       const uint16_t* __restrict__ xll, int rpad,
                                                                       int T, int M, O* __restrict__ Y) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % G::WGM, wt = wave / G::WGM;
  const int tiles_m = (M + G::BM - 1) / G::BM, tiles_t = (T + G::BT - 1) / G::BT;
  int tm, tt;
  tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_t, 8, tm, tt);
  const int64_t m0 = (int64_t)tm * G::BM, t0 = (int64_t)tt * G::BT;
  f32x16 acc[G::FM][G::FT];
  load_tile<G, O>(acc, Y, m0, t0, M, T, wm, wt, lane);
  adapter_mma<G, H>(acc, rt, xlh, xll, rpad, m0, t0, wm, wt, lane);
  store_tile<G, O>(acc, Y, m0, t0, M, T, wm, wt, lane);
}

typedef Geo<256, 256, 3, 2, 4> GeoUp;

unsigned blocks_for(int64_t n) { return (unsigned)cdiv(n, 256); }

void reduce_split(const LowrankWs& w, int64_t T, int64_t r, hipStream_t s) {
  if (w.h16)
    reduce_split_kernel<true><<<blocks_for(w.Tpad * w.rpad), 256, 0, s>>>(w.part, w.splits, T, r, w.rpad, w.Tpad,
                                                                        w.xlh, w.xll);
  else
    reduce_split_kernel<false><<<blocks_for(w.Tpad * w.rpad), 256, 0, s>>>(w.part, w.splits, T, r, w.rpad, w.Tpad,
                                                                         w.xlh, w.xll);
}

}  // namespace

int64_t lowrank_workspace_bytes(int64_t T, int64_t K, int64_t r, int64_t N) {
  if (T == 0 || r == 0) return 0;
  const Sizes z = sizes(T, K, r, N);
  return z.part + 2 * z.xl + z.lt + z.rt;
}

LowrankWs lowrank_layout(Dt in, void* ws, int64_t T, int64_t K, int64_t r, int64_t N) {
  const Sizes z = sizes(T, K, r, N);
  LowrankWs w;
  char* p = static_cast<char*>(ws);
  w.part = reinterpret_cast<float*>(p);
  w.xlh = reinterpret_cast<uint16_t*>(p + z.part);
  w.xll = reinterpret_cast<uint16_t*>(p + z.part + z.xl);
  w.lt = reinterpret_cast<uint16_t*>(p + z.part + 2 * z.xl);
  w.rt = reinterpret_cast<uint16_t*>(p + z.part + 2 * z.xl + z.lt);
  w.splits = z.splits;
  w.rpad = z.rpad;
  w.Tpad = z.Tpad;
  w.Kpad = z.Kpad;
  w.Npad = z.Npad;
  w.kc = z.kc;
  w.mfma = in != Dt::F32 && K % 8 == 0 && r <= kRankMax;
  w.h16 = in == Dt::F16;
  return w;
}

hipError_t launch_lowrank_prepare(Dt in, const void* X, const void* L, const void* R, int64_t T, int64_t K,
                                  int64_t r, int64_t N, const LowrankWs& w, hipStream_t s) {
  if (!w.mfma) return launch_lowrank_down_generic(in, X, L, T, K, r, w.splits, w.kc, w.part, s);
  // 16-bit inputs: transposed L and R, the split down-projection, the hi/lo reduction
  const unsigned nl = blocks_for(w.rpad * w.Kpad / 8), nr = blocks_for(w.Npad * w.rpad / 8);
  transpose_lr_kernel<<<nl + nr, 256, 0, s>>>((const uint16_t*)L, K, r, w.rpad, w.Kpad, w.lt, nl, (const uint16_t*)R, N,
                                             w.Npad, w.rt);
  const hipError_t ed = launch_down((const uint16_t*)X, w.lt, T, K, r, w, s);
  if (ed != hipSuccess) return ed;
  reduce_split(w, T, r, s);
  return hipGetLastError();
}

hipError_t launch_lowrank_down(Dt in, const void* X, const void* L, int64_t T, int64_t K, int64_t r,
                               const LowrankWs& w, hipStream_t s) {
  if (!w.mfma) return hipErrorInvalidValue;
  transpose_l_kernel<<<blocks_for(w.rpad * w.Kpad / 8), 256, 0, s>>>((const uint16_t*)L, K, r, w.rpad, w.Kpad, w.lt);
  const hipError_t ed = launch_down((const uint16_t*)X, w.lt, T, K, r, w, s);
  if (ed != hipSuccess) return ed;
  reduce_split(w, T, r, s);
  return hipGetLastError();
}

hipError_t launch_lowrank_prepare_bwd(const void* dY, const void* L, const void* R, int64_t T, int64_t N, int64_t r,
                                      int64_t K, const LowrankWs& w, hipStream_t s) {
  if (!w.mfma) return hipErrorInvalidValue;
  // down-projection operand: R as [rpad][Kpad] (its own layout, padded); epilogue operand: L as [Npad][rpad]
  const unsigned n1 = blocks_for(w.rpad * w.Kpad), n2 = blocks_for(w.Npad * w.rpad);
  pad_copy2_kernel<<<n1 + n2, 256, 0, s>>>((const uint16_t*)R, r, N, w.rpad, w.Kpad, w.lt, n1, (const uint16_t*)L, K, r,
                                          w.Npad, w.rpad, w.rt);
  const hipError_t ed = launch_down((const uint16_t*)dY, w.lt, T, N, r, w, s);
  if (ed != hipSuccess) return ed;
  reduce_split(w, T, r, s);
  return hipGetLastError();
}

hipError_t launch_transpose_hilo2(const LowrankWs& w1, const LowrankWs& w2, int64_t rpad32, uint16_t* xht1,
                                  uint16_t* xlt1, uint16_t* xht2, uint16_t* xlt2, hipStream_t s) {
  const unsigned n1 = blocks_for(rpad32 * w1.Tpad), n2 = blocks_for(rpad32 * w2.Tpad);
  transpose_hilo2_kernel<<<n1 + n2, 256, 0, s>>>(w1.xlh, w1.xll, w1.Tpad, w1.rpad, xht1, xlt1, n1, w2.xlh, w2.xll,
                                                w2.Tpad, w2.rpad, xht2, xlt2, rpad32);
  return hipGetLastError();
}

hipError_t launch_lowrank_up_add(Dt in, Dt out, const LowrankWs& w, const void* R, int64_t T, int64_t r,
                                 int64_t N, void* Y, hipStream_t s) {
  if (!w.mfma || N % 4 != 0) return launch_lowrank_up_generic(in, out, w.part, w.splits, R, T, r, N, Y, s);
  typedef GeoUp G;
  const int64_t nb = cdiv(N, G::BM) * cdiv(T, G::BT);
  if (out == Dt::BF16)
    lowrank_up_add_kernel<G, uint16_t, false><<<(unsigned)nb, G::THREADS, 0, s>>>(w.rt, w.xlh, w.xll, (int)w.rpad,
                                                                                 (int)T, (int)N, (uint16_t*)Y);
  else if (out == Dt::F16)
    lowrank_up_add_kernel<G, _Float16, true><<<(unsigned)nb, G::THREADS, 0, s>>>(w.rt, w.xlh, w.xll, (int)w.rpad,
                                                                                (int)T, (int)N, (_Float16*)Y);
  else if (w.h16)
    lowrank_up_add_kernel<G, float, true><<<(unsigned)nb, G::THREADS, 0, s>>>(w.rt, w.xlh, w.xll, (int)w.rpad,
                                                                             (int)T, (int)N, (float*)Y);
  else
    lowrank_up_add_kernel<G, float, false><<<(unsigned)nb, G::THREADS, 0, s>>>(w.rt, w.xlh, w.xll, (int)w.rpad,
                                                                              (int)T, (int)N, (float*)Y);
  return hipGetLastError();
}

}  // namespace slope

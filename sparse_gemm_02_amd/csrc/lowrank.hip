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
constexpr int kDownK = 32;       // k per MFMA step
constexpr int kRankMax = 128;    // largest rank of the MFMA down-projection

int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// ------------------------------------------------------------------ layout helpers
struct Sizes {
  int splits;
  int64_t kc, rpad, Tpad, Kpad, Npad, part, xl, lt, rt;
};

int choose_splits(int64_t T, int64_t K) {
  const int64_t tblocks = cdiv(T, kDownRows) < 1 ? 1 : cdiv(T, kDownRows);
  int64_t want = cdiv(1024, tblocks);            // enough blocks to fill 256 CUs
  if (want > (tblocks == 1 ? 64 : 16)) want = tblocks == 1 ? 64 : 16;   // one token block: split K further
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
__global__ __launch_bounds__(256) void transpose_l_kernel(const uint16_t* __restrict__ L, int64_t K, int64_t r,
                                                          int64_t rpad, int64_t Kpad, uint16_t* __restrict__ lt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
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
__global__ __launch_bounds__(256) void transpose_r_kernel(const uint16_t* __restrict__ R, int64_t r, int64_t N,
                                                          int64_t rpad, int64_t Npad, uint16_t* __restrict__ rt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
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

// dst[i][j] = src[i][j] for i < rows, j < cols (src row-major, cols wide); 0 in
// the padding up to [rows_pad, cols_pad].  The adapter backward uses it for the
// operands that need no transposition there: R [r, N] as the down-projection's
// [rpad, Kpad] operand and L [K, r] as the epilogue's [Npad, rpad] operand.
__global__ __launch_bounds__(256) void pad_copy_kernel(const uint16_t* __restrict__ src, int64_t rows, int64_t cols,
                                                       int64_t rows_pad, int64_t cols_pad,
                                                       uint16_t* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows_pad * cols_pad) return;
  const int64_t a = i / cols_pad, b = i % cols_pad;
  dst[i] = (a < rows && b < cols) ? src[a * cols + b] : (uint16_t)0;
}

// xt[j][t] = x[t][j] for the hi and lo parts (x [Tpad][rpad] -> xt [rpad32][Tpad],
// rows j >= rpad zero).  Thread (j, t) with t fastest: coalesced writes.
__global__ __launch_bounds__(256) void transpose_hilo_kernel(const uint16_t* __restrict__ xh,
                                                             const uint16_t* __restrict__ xl, int64_t Tpad,
                                                             int64_t rpad, int64_t rpad32, uint16_t* __restrict__ xht,
                                                             uint16_t* __restrict__ xlt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rpad32 * Tpad) return;
  const int64_t j = i / Tpad, t = i % Tpad;
  const bool in = j < rpad;
  xht[i] = in ? xh[t * rpad + j] : (uint16_t)0;
  xlt[i] = in ? xl[t * rpad + j] : (uint16_t)0;
}

// part[s][t][j] = sum over k in split s of X[t][k] lt[j][k].  A wave owns 64
// tokens (four 16-row MFMA A operands) and every rank column (NJ blocks of
// 16), so each 16-byte piece of lt it loads serves four operands; operands
// come straight from global memory and the next 32-wide k step's loads are
// issued before the current step's MFMAs.  Dense 16x16x32 MFMA: A lane l = row
// l%16, k = 8*(l/16)+e; B lane l = column l%16, same k; D lane l = column l%16,
// rows 4*(l/16)+v.
template <int NJ, bool H>
__global__ __launch_bounds__(256) void lowrank_down_kernel(const uint16_t* __restrict__ X,
                                                           const uint16_t* __restrict__ lt, int T, int K, int r,
                                                           int rpad, int Kpad, int kc, float* __restrict__ part) {
  constexpr int G = kDownWaveRows / 16;                         // 16-token operands per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s = blockIdx.y;
  const int64_t tw = (int64_t)blockIdx.x * kDownRows + wave * kDownWaveRows;   // first token of this wave
  const int kb = s * kc, ke = (kb + kc < K) ? kb + kc : K;
  // tokens past T read as 0 through the resource bound; k past the split is masked
  const int64_t rows_left = (int64_t)T - tw;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + (rows_left > 0 ? tw : 0) * K, rows_left > 0 ? rows_left * K * 2 : 0);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(lt, (int64_t)rpad * Kpad * 2);
  const int kl = 8 * (lane >> 4);
  uint32_t xa[G];
#pragma unroll
  for (int g = 0; g < G; ++g) xa[g] = (uint32_t)((g * 16 + (lane & 15)) * K) * 2;
  f32x4 acc[G][NJ];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[g][j] = f32x4{};
  struct Ops {
    u32x4 a[G], b[NJ];
  };
  auto load = [&](Ops& o, int k0) {
    const int k = k0 + kl;
    const bool ok = k0 < ke && k + 8 <= ke;
#pragma unroll
    for (int g = 0; g < G; ++g) o.a[g] = load16(rx, ok ? xa[g] + k * 2 : kOutOfRange);
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb)
      o.b[jb] = load16(rl, ok ? (uint32_t)((jb * 16 + (lane & 15)) * Kpad + k) * 2 : kOutOfRange);
  };
  auto mma = [&](const Ops& o) {
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) {
      typedef typename Fmt16<H>::v8 v8;
      const v8 bb = __builtin_bit_cast(v8, o.b[jb]);
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g][jb] = Fmt16<H>::mfma16x16x32(__builtin_bit_cast(v8, o.a[g]), bb, acc[g][jb]);
    }
  };
  Ops p0, p1;
  load(p0, kb);
  for (int k0 = kb; k0 < ke; k0 += 2 * kDownK) {
    load(p1, k0 + kDownK);
    mma(p0);
    load(p0, k0 + 2 * kDownK);
    mma(p1);
  }
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb) {
    const int j = jb * 16 + (lane & 15);
    if (j >= r) continue;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t t = tw + 16 * g + 4 * (lane >> 4) + v;
        if (t < T) part[((int64_t)s * T + t) * r + j] = acc[g][jb][v];
      }
  }
}

template <int NJ>
void down_nj(dim3 grid, const uint16_t* X, const uint16_t* lt, int64_t T, int64_t K, int64_t r, const LowrankWs& w,
             hipStream_t s) {
  if (w.h16)
    lowrank_down_kernel<NJ, true><<<grid, 256, 0, s>>>(X, lt, (int)T, (int)K, (int)r, (int)w.rpad, (int)w.Kpad,
                                                       (int)w.kc, w.part);
  else
    lowrank_down_kernel<NJ, false><<<grid, 256, 0, s>>>(X, lt, (int)T, (int)K, (int)r, (int)w.rpad, (int)w.Kpad,
                                                        (int)w.kc, w.part);
}

hipError_t launch_down(const uint16_t* X, const uint16_t* lt, int64_t T, int64_t K, int64_t r, const LowrankWs& w,
                       hipStream_t s) {
  const dim3 grid((unsigned)cdiv(T, kDownRows), (unsigned)w.splits);
  switch (w.rpad / 16) {
    case 1: down_nj<1>(grid, X, lt, T, K, r, w, s); break;
    case 2: down_nj<2>(grid, X, lt, T, K, r, w, s); break;
    case 3: down_nj<3>(grid, X, lt, T, K, r, w, s); break;
    case 4: down_nj<4>(grid, X, lt, T, K, r, w, s); break;
    case 5: down_nj<5>(grid, X, lt, T, K, r, w, s); break;
    case 6: down_nj<6>(grid, X, lt, T, K, r, w, s); break;
    case 7: down_nj<7>(grid, X, lt, T, K, r, w, s); break;
    case 8: down_nj<8>(grid, X, lt, T, K, r, w, s); break;
    default: return hipErrorInvalidValue;
  }
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
  transpose_l_kernel<<<blocks_for(w.rpad * w.Kpad / 8), 256, 0, s>>>((const uint16_t*)L, K, r, w.rpad, w.Kpad, w.lt);
  transpose_r_kernel<<<blocks_for(w.Npad * w.rpad / 8), 256, 0, s>>>((const uint16_t*)R, r, N, w.rpad, w.Npad, w.rt);
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
  pad_copy_kernel<<<blocks_for(w.rpad * w.Kpad), 256, 0, s>>>((const uint16_t*)R, r, N, w.rpad, w.Kpad, w.lt);
  pad_copy_kernel<<<blocks_for(w.Npad * w.rpad), 256, 0, s>>>((const uint16_t*)L, K, r, w.Npad, w.rpad, w.rt);
  const hipError_t ed = launch_down((const uint16_t*)dY, w.lt, T, N, r, w, s);
  if (ed != hipSuccess) return ed;
  reduce_split(w, T, r, s);
  return hipGetLastError();
}

hipError_t launch_transpose_hilo(const LowrankWs& w, int64_t rpad32, uint16_t* xht, uint16_t* xlt, hipStream_t s) {
  transpose_hilo_kernel<<<blocks_for(rpad32 * w.Tpad), 256, 0, s>>>(w.xlh, w.xll, w.Tpad, w.rpad, rpad32, xht, xlt);
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

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
// adapter's X . L comes from the down-projection of lowrank.hip; its
// up-projection reads R in its own layout (no transposed copy of R).
#include "common.h"
#include "dma.h"
#include "gemm_tile.h"
#include "launch.h"

namespace slope {

namespace {

typedef Geo<256, 256, 3, 2, 4> Chunk;            // the tile-chunk geometry written by pack_sparse
constexpr int kDecodeMaxT = 64;
constexpr int kUnroll = 4;                       // stages whose loads are issued together

// part[split][t][n] (n < Npad) = sum over this split's k of X[t][k] W_s[n][k].
// Block = 4 waves = one 256-row tile; wave w rows 64w .. 64w+63 (two 32-row
// A operands), FT = 1 or 2 token tiles of 32.
template <int FT, bool H>
__global__ __launch_bounds__(256) void decode_partial_kernel(const uint16_t* __restrict__ X,
                                                             const char* __restrict__ packed, int T, int K,
                                                             int stages, int kc, int64_t Npad,
                                                             float* __restrict__ part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = blockIdx.x, split = blockIdx.y;
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
// rounded once, with xl = xlh + xll (X . L as a bf16 hi/lo pair, prepared by
// the adapter's down-projection; their fp32 sum is exact).  A block covers 64
// consecutive n (one per lane) and TB tokens; its four waves split the work
// into quarters (wave w: the w-th quarter of the splits, in order, and the
// w-th quarter of the rank rows), each wave issuing a batch of Q loads before
// using them, and the four partial sums are added in wave order through LDS
// (deterministic).  The block's xl rows are staged in LDS once and read as
// broadcasts; R is read in its own [r, N] layout.
constexpr int kReduceMaxRank = 128;

template <typename O, int TB, int Q, bool H>
__global__ __launch_bounds__(256) void decode_reduce_kernel(const float* __restrict__ part, int splits, int T,
                                                            int64_t N, int64_t Npad, const uint16_t* __restrict__ R,
                                                            const uint16_t* __restrict__ xlh,
                                                            const uint16_t* __restrict__ xll, int r, int rpad,
                                                            O* __restrict__ Y) {
  __shared__ float xl[TB][kReduceMaxRank];
  __shared__ float sum[4][TB][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.x * 64 + lane;
  const bool col = n < N;
  const int tb = blockIdx.y * TB;
  if (R) {
    for (int e = threadIdx.x; e < TB * rpad; e += 256) {
      const int i = e / rpad, j = e % rpad;
      xl[i][j] = tb + i < T ? Fmt16<H>::to_f32(xlh[(tb + i) * rpad + j]) + Fmt16<H>::to_f32(xll[(tb + i) * rpad + j])
                           : 0.f;
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
    // the wave's quarter of the (zero-padded) rank rows
    const int rq = rpad / 4, j0 = wave * rq;
    for (int c0 = j0; c0 < j0 + rq; c0 += 4 * Q) {
      float rv[4 * Q];
#pragma unroll
      for (int q = 0; q < 4 * Q; ++q) {
        const int j = c0 + q;
        rv[q] = (col && j < j0 + rq && j < r) ? Fmt16<H>::to_f32(R[(int64_t)j * N + n]) : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 4 * Q; ++q) {
        if (c0 + q >= j0 + rq) break;
#pragma unroll
        for (int i = 0; i < TB; ++i) y[i] += rv[q] * xl[i][c0 + q];
      }
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
                          const uint16_t* xh, const uint16_t* xo, int r, int rpad, O* Y, hipStream_t s) {
  if (T <= 4) {
    dim3 g((unsigned)cdiv(N, 64), (unsigned)cdiv(T, 4));
    decode_reduce_kernel<O, 4, 16, H><<<g, 256, 0, s>>>(part, splits, (int)T, N, Npad, R, xh, xo, r, rpad, Y);
  } else {
    dim3 g((unsigned)cdiv(N, 64), (unsigned)cdiv(T, 16));
    decode_reduce_kernel<O, 16, 4, H><<<g, 256, 0, s>>>(part, splits, (int)T, N, Npad, R, xh, xo, r, rpad, Y);
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
  // (splits x T x N x 8 bytes written and read) stay small next to the weight
  int64_t want = cdiv(2048, p.tiles < 1 ? 1 : p.tiles);
  const int64_t cap = (int64_t)(0.02 * (double)K / (double)(T < 1 ? 1 : T));
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

int64_t decode_workspace_bytes(int64_t T, int64_t K, int64_t r, int64_t N) {
  if (T == 0 || N == 0) return 0;
  return decode_plan(T, K, N).part_bytes + (r > 0 ? lowrank_workspace_bytes(T, K, r, N) : 0);
}

namespace {
template <bool H>
void decode_partial_launch(int64_t T, dim3 grid, const void* X, const void* packed, int64_t K, const DecodePlan& p,
                           float* part, hipStream_t s) {
  if (T <= 32)
    decode_partial_kernel<1, H><<<grid, 256, 0, s>>>((const uint16_t*)X, (const char*)packed, (int)T, (int)K,
                                                     p.stages, p.kc, p.Npad, part);
  else
    decode_partial_kernel<2, H><<<grid, 256, 0, s>>>((const uint16_t*)X, (const char*)packed, (int)T, (int)K,
                                                     p.stages, p.kc, p.Npad, part);
}
}  // namespace

hipError_t launch_spmm_decode(Dt in, Dt out, const void* X, int64_t T, int64_t K, const void* packed, int64_t N,
                              const void* L, const void* R, int64_t r, void* workspace, void* Y, hipStream_t s) {
  if (T == 0 || N == 0) return hipSuccess;
  const DecodePlan p = decode_plan(T, K, N);
  float* part = (float*)workspace;
  const bool ad = r > 0 && L != nullptr && R != nullptr;
  LowrankWs w;
  if (ad) {
    w = lowrank_layout(in, (char*)workspace + p.part_bytes, T, K, r, N);
    const hipError_t e = launch_lowrank_down(in, X, L, T, K, r, w, s);
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)p.tiles, (unsigned)p.splits);
  if (in == Dt::F16)
    decode_partial_launch<true>(T, grid, X, packed, K, p, part, s);
  else
    decode_partial_launch<false>(T, grid, X, packed, K, p, part, s);
  const uint16_t* Ra = ad ? (const uint16_t*)R : nullptr;
  const uint16_t* xh = ad ? w.xlh : nullptr;
  const uint16_t* xo = ad ? w.xll : nullptr;
  const int rp = ad ? (int)w.rpad : 0;
  if (out == Dt::BF16)
    launch_decode_reduce<uint16_t, false>(part, p.splits, T, N, p.Npad, Ra, xh, xo, (int)r, rp, (uint16_t*)Y, s);
  else if (out == Dt::F16)
    launch_decode_reduce<_Float16, true>(part, p.splits, T, N, p.Npad, Ra, xh, xo, (int)r, rp, (_Float16*)Y, s);
  else if (in == Dt::F16)
    launch_decode_reduce<float, true>(part, p.splits, T, N, p.Npad, Ra, xh, xo, (int)r, rp, (float*)Y, s);
  else
    launch_decode_reduce<float, false>(part, p.splits, T, N, p.Npad, Ra, xh, xo, (int)r, rp, (float*)Y, s);
  return hipGetLastError();
}

static_assert(kDecodeMaxT == 64, "two 32-token tiles at most");
static_assert(kReduceMaxRank >= 128, "adapter ranks up to 128 (rank rows padded to 16)");

}  // namespace slope

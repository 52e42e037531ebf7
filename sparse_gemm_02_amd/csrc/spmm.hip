// Sparse 2:4 x dense GEMM on gfx950 sparse MFMA (v_smfmac_f32_32x32x32_bf16),
// with the low-rank adapter fused into the epilogue.
//
// Forward (SLoPe explainer, Technical Summary 2.A):   Y  = X . W_s^T
// Backward data (same section, double-pruned weight): dX = dY . W_dp
// Adapter (2.B, W_dense = W_sparse + L R; kept unmerged at inference per the
// discussion page's "SLoPe inference computation"):    Y += (X . L) . R
// Fusion of the sparse product with the low-rank term follows 2.C.
//
// Both products have the form Out[t][m] = sum_k B[t][k] * A[m][k] with A the
// 2:4 operand compressed along k and B row-major with k contiguous, so the
// kernel computes the transposed tile Out^T = A . B^T with A as the sparse
// MFMA operand (rows m = output features, reduction k).
//
// Lane layouts of v_smfmac_f32_32x32x32_bf16, measured on gfx950:
//   A (compressed): lane l holds row l%32, the 8 compressed values of groups
//     4*(l/32) .. 4*(l/32)+3 of the 32-wide k step (16 contiguous dense k), and
//     their four nibbles in bits 0..15 of the index operand (abid 0).
//   B: lane l holds column l%32, k = 8*(l/32) + e for e < 8 and
//     16 + 8*(l/32) + (e-8) for e >= 8.
//   D: lane l holds column l%32, rows 8*(v/4) + 4*(l/32) + v%4.
// The stored metadata word of a 32-wide k step therefore feeds lanes 0..31
// with its low half and lanes 32..63 with its high half.
#include "common.h"
#include "launch.h"
#include "tile_map.h"

namespace slope {

hipError_t launch_spmm_generic(Dt in, Dt out, const void* B, int64_t T, int64_t Kred, const void* values,
                               const uint32_t* meta, int64_t M, const float* xl, int splits, int64_t r,
                               const void* R, void* Y, hipStream_t s);
hipError_t launch_lowrank_down_generic(Dt in, const void* X, const void* L, int64_t T, int64_t K, int64_t r,
                                       int splits, int64_t kc, float* xl, hipStream_t s);
hipError_t launch_lowrank_up_generic(Dt in, Dt out, const float* xl, int splits, const void* R, int64_t T,
                                     int64_t r, int64_t N, void* Y, hipStream_t s);

namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------------ tile geometry
template <int BM_, int BT_>
struct Geo {
  static constexpr int BM = BM_, BT = BT_;
  static constexpr int WM = BM / 2, WT = BT / 2;  // 2 x 2 waves
  static constexpr int FM = WM / 32, FT = WT / 32;
  static constexpr int KS = 64;                   // dense k per LDS stage
  static constexpr int AP = 40;                   // A row pitch (bf16): 32 values + 8 pad
  static constexpr int BP = 72;                   // B row pitch (bf16): 64 values + 8 pad
  static constexpr int A_ELEMS = BM * AP, B_ELEMS = BT * BP, META_WORDS = 2 * BM;
  static constexpr int STAGE_BYTES = A_ELEMS * 2 + B_ELEMS * 2 + META_WORDS * 4;
  static constexpr int NA = BM * 4 / kThreads;    // 16-byte A chunks per thread per stage
  static constexpr int NB = BT * 8 / kThreads;    // 16-byte B chunks per thread per stage
  static constexpr int NMETA = 2 * BM / kThreads; // metadata words per thread per stage
  // adapter epilogue staging (reuses the operand buffers)
  static constexpr int RC = 32, RP = 40;
  static constexpr int ADAPTER_BYTES = (BM + 2 * BT) * RP * 2;
  static constexpr int LDS_BYTES = (2 * STAGE_BYTES > ADAPTER_BYTES) ? 2 * STAGE_BYTES : ADAPTER_BYTES;
};

// ------------------------------------------------------------------ adapter epilogue
// acc[fm][ft] (rows m, columns t of the transposed tile) += R^T . XL^T, with
// XL summed over its k-splits in fixed order and split into bf16 hi + lo
// parts so that the product keeps ~16 bits of XL.  Dense 32x32x16 MFMA:
// A lane l = row l%32, k = 8*(l/32)+e; B lane l = column l%32, same k.
template <class G>
__device__ __forceinline__ void adapter_accumulate(f32x16 (&acc)[G::FM][G::FT], char* lds, int64_t m0, int64_t t0,
                                                   int M, int T, const float* __restrict__ xl, int splits, int r,
                                                   const uint16_t* __restrict__ R, int wm, int wt, int lane) {
  uint16_t* Rt = reinterpret_cast<uint16_t*>(lds);        // [BM][RP]
  uint16_t* Xh = Rt + G::BM * G::RP;                       // [BT][RP]
  uint16_t* Xl = Xh + G::BT * G::RP;                       // [BT][RP]
  const int tid = threadIdx.x;
  for (int j0 = 0; j0 < r; j0 += G::RC) {
    __syncthreads();
    for (int i = tid; i < G::BM * G::RC; i += kThreads) {
      const int m = i % G::BM, jj = i / G::BM;
      const int64_t gm = m0 + m;
      uint16_t v = 0;
      if (j0 + jj < r && gm < M) v = R[(int64_t)(j0 + jj) * M + gm];
      Rt[m * G::RP + jj] = v;
    }
    for (int i = tid; i < G::BT * G::RC; i += kThreads) {
      const int jj = i % G::RC, t = i / G::RC;
      const int64_t gt = t0 + t;
      float x = 0.f;
      if (j0 + jj < r && gt < T)
        for (int s = 0; s < splits; ++s) x += xl[((int64_t)s * T + gt) * r + j0 + jj];
      const uint16_t hi = f32_to_bf16_bits(x);
      const uint16_t lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
      Xh[t * G::RP + jj] = hi;
      Xl[t * G::RP + jj] = lo;
    }
    __syncthreads();
#pragma unroll
    for (int jk = 0; jk < G::RC / 16; ++jk) {
      bf16x8 ra[G::FM];
#pragma unroll
      for (int fm = 0; fm < G::FM; ++fm)
        ra[fm] = *reinterpret_cast<const bf16x8*>(Rt + (wm * G::WM + fm * 32 + (lane & 31)) * G::RP + jk * 16 + 8 * (lane >> 5));
#pragma unroll
      for (int ft = 0; ft < G::FT; ++ft) {
        const int row = (wt * G::WT + ft * 32 + (lane & 31)) * G::RP + jk * 16 + 8 * (lane >> 5);
        const bf16x8 xh = *reinterpret_cast<const bf16x8*>(Xh + row);
        const bf16x8 xlo = *reinterpret_cast<const bf16x8*>(Xl + row);
#pragma unroll
        for (int fm = 0; fm < G::FM; ++fm) {
          acc[fm][ft] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[fm], xh, acc[fm][ft], 0, 0, 0);
          acc[fm][ft] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra[fm], xlo, acc[fm][ft], 0, 0, 0);
        }
      }
    }
  }
}

// Store the transposed tile: element v of acc[fm][ft] is Out[t][m] with
// m = m0 + wm*WM + fm*32 + 8*(v/4) + 4*(lane/32) + v%4, t = t0 + wt*WT + ft*32 + lane%32.
// Four consecutive v are four consecutive m: one 8-byte (bf16) or 16-byte store.
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
          w[0] = f32_to_bf16_bits(acc[fm][ft][4 * q]) | ((uint32_t)f32_to_bf16_bits(acc[fm][ft][4 * q + 1]) << 16);
          w[1] = f32_to_bf16_bits(acc[fm][ft][4 * q + 2]) | ((uint32_t)f32_to_bf16_bits(acc[fm][ft][4 * q + 3]) << 16);
          *reinterpret_cast<u32x2*>(p) = w;
        } else {
          f32x4 w = {acc[fm][ft][4 * q], acc[fm][ft][4 * q + 1], acc[fm][ft][4 * q + 2], acc[fm][ft][4 * q + 3]};
          *reinterpret_cast<f32x4*>(p) = w;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ main kernel
// Requirements (checked on the host): Kred % 16 == 0, M % 4 == 0, 16-byte
// aligned base pointers.  Ragged M, T and Kred % 64 are zero-filled.
template <class G, bool ADAPTER, typename O>
__global__ __launch_bounds__(kThreads, 1) void spmm_smfmac_kernel(
    const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ vals, const uint32_t* __restrict__ meta, int M,
    int T, int Kred, const float* __restrict__ xl, int splits, int r, const uint16_t* __restrict__ R,
    O* __restrict__ Y) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wt = wave >> 1;
  const int tiles_m = (M + G::BM - 1) / G::BM, tiles_t = (T + G::BT - 1) / G::BT;
  int tm, tt;
  tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_t, 8, tm, tt);
  const int64_t m0 = (int64_t)tm * G::BM, t0 = (int64_t)tt * G::BT;
  const int64_t vpitch = Kred / 2;                  // compressed values per row
  const int wpr = (Kred / 4 + 7) / 8;               // metadata words per row
  const int stages = (Kred + G::KS - 1) / G::KS;

  u32x4 pa[G::NA], pb[G::NB];
  uint32_t pm[G::NMETA];

  auto load = [&](int s) {
#pragma unroll
    for (int i = 0; i < G::NA; ++i) {
      const int c = tid + kThreads * i, row = c >> 2, p = c & 3;
      const int64_t gm = m0 + row;
      const int kd = s * G::KS + 16 * p;           // first dense k of this chunk
      pa[i] = (gm < M && kd + 16 <= Kred)
                  ? *reinterpret_cast<const u32x4*>(vals + gm * vpitch + (kd >> 1))
                  : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < G::NB; ++i) {
      const int c = tid + kThreads * i, row = c >> 3, p = c & 7;
      const int64_t gt = t0 + row;
      const int kd = s * G::KS + 8 * p;
      pb[i] = (gt < T && kd + 8 <= Kred) ? *reinterpret_cast<const u32x4*>(Bm + gt * Kred + kd)
                                         : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < G::NMETA; ++i) {
      const int c = tid + kThreads * i, row = c % G::BM, w = c / G::BM;
      const int64_t gm = m0 + row;
      const int wi = 2 * s + w;
      pm[i] = (gm < M && wi < wpr) ? meta[gm * wpr + wi] : 0u;
    }
  };
  auto store = [&](int buf) {
    uint16_t* A = reinterpret_cast<uint16_t*>(lds + buf * G::STAGE_BYTES);
    uint16_t* B = A + G::A_ELEMS;
    uint32_t* Mt = reinterpret_cast<uint32_t*>(B + G::B_ELEMS);
#pragma unroll
    for (int i = 0; i < G::NA; ++i) {
      const int c = tid + kThreads * i, row = c >> 2, p = c & 3;
      *reinterpret_cast<u32x4*>(A + row * G::AP + 8 * p) = pa[i];
    }
#pragma unroll
    for (int i = 0; i < G::NB; ++i) {
      const int c = tid + kThreads * i, row = c >> 3, p = c & 7;
      *reinterpret_cast<u32x4*>(B + row * G::BP + 8 * p) = pb[i];
    }
#pragma unroll
    for (int i = 0; i < G::NMETA; ++i) {
      const int c = tid + kThreads * i;
      Mt[c] = pm[i];  // [w][row]
    }
  };

  f32x16 acc[G::FM][G::FT];
#pragma unroll
  for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
    for (int ft = 0; ft < G::FT; ++ft) acc[fm][ft] = f32x16{};

  if (stages > 0) {
    load(0);
    store(0);
    __syncthreads();
  }
  for (int s = 0; s < stages; ++s) {
    const int buf = s & 1;
    if (s + 1 < stages) load(s + 1);
    const uint16_t* A = reinterpret_cast<const uint16_t*>(lds + buf * G::STAGE_BYTES);
    const uint16_t* B = A + G::A_ELEMS;
    const uint32_t* Mt = reinterpret_cast<const uint32_t*>(B + G::B_ELEMS);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 af[G::FM];
      int ix[G::FM];
#pragma unroll
      for (int fm = 0; fm < G::FM; ++fm) {
        const int row = wm * G::WM + fm * 32 + (lane & 31);
        af[fm] = *reinterpret_cast<const bf16x8*>(A + row * G::AP + ks * 16 + 8 * (lane >> 5));
        ix[fm] = (int)(Mt[ks * G::BM + row] >> (16 * (lane >> 5)));
      }
#pragma unroll
      for (int ft = 0; ft < G::FT; ++ft) {
        const int col = wt * G::WT + ft * 32 + (lane & 31);
        const uint16_t* bp = B + col * G::BP + ks * 32 + 8 * (lane >> 5);
        const bf16x8 lo = *reinterpret_cast<const bf16x8*>(bp);
        const bf16x8 hi = *reinterpret_cast<const bf16x8*>(bp + 16);
        const bf16x16 bfrag = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
#pragma unroll
        for (int fm = 0; fm < G::FM; ++fm)
          acc[fm][ft] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(af[fm], bfrag, acc[fm][ft], ix[fm], 0, 0);
      }
    }
    if (s + 1 < stages) store(buf ^ 1);
    __syncthreads();
  }
  if constexpr (ADAPTER) adapter_accumulate<G>(acc, lds, m0, t0, M, T, xl, splits, r, R, wm, wt, lane);
  store_tile<G, O>(acc, Y, m0, t0, M, T, wm, wt, lane);
}

// ------------------------------------------------------------------ standalone adapter
// Y[t][m] += XL[t] . R[:, m] over one output tile: the same epilogue with the
// accumulators loaded from Y.
template <class G, typename O>
__global__ __launch_bounds__(kThreads, 1) void lowrank_up_add_kernel(const float* __restrict__ xl, int splits,
                                                                     const uint16_t* __restrict__ R, int T, int r,
                                                                     int M, O* __restrict__ Y) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wt = wave >> 1;
  const int tiles_m = (M + G::BM - 1) / G::BM, tiles_t = (T + G::BT - 1) / G::BT;
  int tm, tt;
  tile_of_block(blockIdx.x, gridDim.x, tiles_m, tiles_t, 8, tm, tt);
  const int64_t m0 = (int64_t)tm * G::BM, t0 = (int64_t)tt * G::BT;
  f32x16 acc[G::FM][G::FT];
#pragma unroll
  for (int ft = 0; ft < G::FT; ++ft) {
    const int64_t t = t0 + wt * G::WT + ft * 32 + (lane & 31);
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm * G::WM + fm * 32 + 8 * (v / 4) + 4 * (lane >> 5) + v % 4;
        acc[fm][ft][v] = (t < T && m < M) ? load_out(Y + t * M + m) : 0.f;
      }
  }
  adapter_accumulate<G>(acc, lds, m0, t0, M, T, xl, splits, r, R, wm, wt, lane);
  store_tile<G, O>(acc, Y, m0, t0, M, T, wm, wt, lane);
}

// ------------------------------------------------------------------ down projection
// xl[s][t][j] = sum over split s of X[t][k] L[k][j].  Block: 64 tokens (16 per
// wave) x one k-split; L staged transposed in LDS per 64-wide k step; dense
// 16x16x32 MFMA (A lane l = row l%16, k = 8*(l/16)+e; B lane l = column l%16,
// same k; D lane l = column l%16, rows 4*(l/16)+v).
constexpr int LD_TT = 64, LD_KS = 64, LD_LP = 72, LD_RMAX = 128;

__global__ __launch_bounds__(kThreads) void lowrank_down_kernel(const uint16_t* __restrict__ X,
                                                                const uint16_t* __restrict__ L, int T, int K, int r,
                                                                int kc, float* __restrict__ xl) {
  __shared__ __attribute__((aligned(16))) uint16_t Lt[LD_RMAX * LD_LP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * LD_TT + wave * 16;
  const int kbeg = s * kc, kend = (kbeg + kc < K) ? kbeg + kc : K;
  const int rpad = (r + 15) & ~15;
  const int nj = rpad / 16;
  f32x4 acc[LD_RMAX / 16];
#pragma unroll
  for (int j = 0; j < LD_RMAX / 16; ++j) acc[j] = f32x4{};
  const int64_t trow = t0 + (lane & 15);
  for (int k0 = kbeg; k0 < kend; k0 += LD_KS) {
    __syncthreads();
    for (int i = tid; i < LD_KS * rpad; i += kThreads) {
      const int kk = i / rpad, j = i % rpad;
      const int k = k0 + kk;
      Lt[j * LD_LP + kk] = (j < r && k < kend) ? L[(int64_t)k * r + j] : (uint16_t)0;
    }
    __syncthreads();
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
      const int k = k0 + kk2 * 32 + 8 * (lane >> 4);
      const bf16x8 a = (trow < T && k + 8 <= kend) ? *reinterpret_cast<const bf16x8*>(X + trow * K + k) : bf16x8{};
#pragma unroll
      for (int jb = 0; jb < LD_RMAX / 16; ++jb) {
        if (jb < nj) {
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(Lt + (jb * 16 + (lane & 15)) * LD_LP + kk2 * 32 + 8 * (lane >> 4));
          acc[jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[jb], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int jb = 0; jb < LD_RMAX / 16; ++jb) {
    if (jb >= nj) break;
    const int j = jb * 16 + (lane & 15);
    if (j >= r) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t t = t0 + 4 * (lane >> 4) + v;
      if (t < T) xl[((int64_t)s * T + t) * r + j] = acc[jb][v];
    }
  }
}

typedef Geo<256, 256> GeoBig;

template <bool ADAPTER, typename O>
hipError_t launch_big(const uint16_t* B, int T, int Kred, const uint16_t* vals, const uint32_t* meta, int M,
                      const float* xl, int splits, int r, const uint16_t* R, O* Y, hipStream_t s) {
  typedef GeoBig G;
  auto kern = spmm_smfmac_kernel<G, ADAPTER, O>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t nb = cdiv(M, G::BM) * cdiv(T, G::BT);
  kern<<<(unsigned)nb, kThreads, G::LDS_BYTES, s>>>(B, vals, meta, M, T, Kred, xl, splits, r, R, Y);
  return hipGetLastError();
}

}  // namespace

int lowrank_splits(int64_t T, int64_t K) {
  const int64_t tblocks = cdiv(T, LD_TT);
  int64_t want = cdiv(1024, tblocks < 1 ? 1 : tblocks);
  if (want > 16) want = 16;
  const int64_t ksteps = cdiv(K, LD_KS);
  if (want > ksteps) want = ksteps;
  if (want < 1) want = 1;
  const int64_t kc = cdiv(cdiv(K, want), LD_KS) * LD_KS;
  return kc > 0 ? (int)cdiv(K, kc) : 1;
}

static int64_t split_width(int64_t K, int splits) { return cdiv(cdiv(K, splits), LD_KS) * LD_KS; }

hipError_t launch_lowrank_down(Dt in, const void* X, const void* L, int64_t T, int64_t K, int64_t r, int splits,
                               float* xl, hipStream_t s) {
  const int64_t kc = split_width(K, splits);
  if (in == Dt::BF16 && K % 8 == 0 && r <= LD_RMAX) {
    dim3 grid((unsigned)cdiv(T, LD_TT), (unsigned)splits);
    lowrank_down_kernel<<<grid, kThreads, 0, s>>>((const uint16_t*)X, (const uint16_t*)L, (int)T, (int)K, (int)r,
                                                  (int)kc, xl);
    return hipGetLastError();
  }
  return launch_lowrank_down_generic(in, X, L, T, K, r, splits, kc, xl, s);
}

hipError_t launch_spmm(Dt in, Dt out, const void* B, int64_t T, int64_t Kred, const void* values,
                       const uint32_t* meta, int64_t M, const float* xl, int splits, int64_t r, const void* R,
                       void* Y, hipStream_t s) {
  const bool fast = in == Dt::BF16 && Kred % 16 == 0 && M % 4 == 0;
  if (!fast) return launch_spmm_generic(in, out, B, T, Kred, values, meta, M, xl, splits, r, R, Y, s);
  const bool ad = xl != nullptr && r > 0;
  const uint16_t* Bb = (const uint16_t*)B;
  const uint16_t* vb = (const uint16_t*)values;
  const uint16_t* Rb = (const uint16_t*)R;
  if (out == Dt::BF16)
    return ad ? launch_big<true>(Bb, (int)T, (int)Kred, vb, meta, (int)M, xl, splits, (int)r, Rb, (uint16_t*)Y, s)
              : launch_big<false>(Bb, (int)T, (int)Kred, vb, meta, (int)M, xl, splits, (int)r, Rb, (uint16_t*)Y, s);
  return ad ? launch_big<true>(Bb, (int)T, (int)Kred, vb, meta, (int)M, xl, splits, (int)r, Rb, (float*)Y, s)
            : launch_big<false>(Bb, (int)T, (int)Kred, vb, meta, (int)M, xl, splits, (int)r, Rb, (float*)Y, s);
}

hipError_t launch_lowrank_up_add(Dt in, Dt out, const float* xl, int splits, const void* R, int64_t T, int64_t r,
                                 int64_t N, void* Y, hipStream_t s) {
  if (in != Dt::BF16 || N % 4 != 0) return launch_lowrank_up_generic(in, out, xl, splits, R, T, r, N, Y, s);
  typedef GeoBig G;
  const int64_t nb = cdiv(N, G::BM) * cdiv(T, G::BT);
  const int lds = G::ADAPTER_BYTES;
  if (out == Dt::BF16)
    lowrank_up_add_kernel<G, uint16_t><<<(unsigned)nb, kThreads, lds, s>>>(xl, splits, (const uint16_t*)R, (int)T, (int)r, (int)N, (uint16_t*)Y);
  else
    lowrank_up_add_kernel<G, float><<<(unsigned)nb, kThreads, lds, s>>>(xl, splits, (const uint16_t*)R, (int)T, (int)r, (int)N, (float*)Y);
  return hipGetLastError();
}

}  // namespace slope

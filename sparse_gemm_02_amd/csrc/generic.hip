// Generic LDS-tiled SIMT kernels: the fp32 path and the 16-bit paths (bf16,
// fp16) for shapes whose rows are not 16-byte aligned.  Accumulation in fp32.
//
// Operations (SLoPe explainer, Technical Summary 2.A and 2.B; discussion page,
// "Memory Footprint" and "SLoPe inference computation"):
//   forward        Y  = X . W_s^T (+ (X . L) . R)
//   backward data  dX = dY . W_dp   (same kernel on the compressed W_dp^T)
//   weight grad    dW = (dY^T . X) kept at the static mask
#include "common.h"
#include "launch.h"

namespace slope {

namespace {

constexpr int TILE = 64, KSTEP = 32, LPITCH = KSTEP + 1;

// Y[t][m] = sum_k B[t][k] * A[m][k], A given compressed (values, meta) along k.
template <typename E, typename O>
__global__ __launch_bounds__(256) void spmm_generic_kernel(const E* __restrict__ Bm, const E* __restrict__ vals,
                                                           const uint32_t* __restrict__ meta, int64_t M, int64_t T,
                                                           int64_t Kred, const float* __restrict__ xl, int splits,
                                                           int64_t r, const E* __restrict__ R, O* __restrict__ Y) {
  __shared__ float As[TILE * LPITCH];
  __shared__ float Bs[TILE * LPITCH];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t m0 = (int64_t)blockIdx.x * TILE, t0 = (int64_t)blockIdx.y * TILE;
  const int64_t gpr = Kred / 4, wpr = cdiv(gpr, 8);
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < Kred; k0 += KSTEP) {
    {  // decompress A: row = tid/4, groups 2*(tid%4), +1 of this 32-wide step
      const int row = threadIdx.x >> 2, gp = threadIdx.x & 3;
      float d[8] = {};
      const int64_t m = m0 + row;
      const int64_t g = k0 / 4 + 2 * gp;
      if (m < M) {
        for (int i = 0; i < 2; ++i) {
          if (g + i < gpr) {
            const uint32_t nib = (meta[m * wpr + (g + i) / 8] >> (4 * ((g + i) % 8))) & 0xFu;
            const E* v = vals + m * (Kred / 2) + 2 * (g + i);
            d[4 * i + (nib & 3u)] = to_f32(v[0]);
            d[4 * i + (nib >> 2)] = to_f32(v[1]);
          }
        }
      }
      for (int i = 0; i < 8; ++i) As[row * LPITCH + 8 * gp + i] = d[i];
    }
    for (int i = threadIdx.x; i < TILE * KSTEP; i += 256) {
      const int row = i / KSTEP, kk = i % KSTEP;
      const int64_t t = t0 + row, k = k0 + kk;
      Bs[row * LPITCH + kk] = (t < T && k < Kred) ? to_f32(Bm[t * Kred + k]) : 0.f;
    }
    __syncthreads();
    for (int kk = 0; kk < KSTEP; ++kk) {
      float a[4], b[4];
      for (int i = 0; i < 4; ++i) a[i] = As[(ty * 4 + i) * LPITCH + kk];
      for (int j = 0; j < 4; ++j) b[j] = Bs[(tx * 4 + j) * LPITCH + kk];
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= M) continue;
    for (int j = 0; j < 4; ++j) {
      const int64_t t = t0 + tx * 4 + j;
      if (t >= T) continue;
      float v = acc[i][j];
      if (xl) {
        float a = 0.f;
        for (int64_t q = 0; q < r; ++q) {
          float x = 0.f;
          for (int s = 0; s < splits; ++s) x += xl[((int64_t)s * T + t) * r + q];
          a = fmaf(x, to_f32(R[q * M + m]), a);
        }
        v += a;
      }
      store_out(Y + t * M + m, v);
    }
  }
}

// dW[n][k] = sum_t dY[t][n] * X[t][k], written at the static mask.
template <typename E, typename O>
__global__ __launch_bounds__(256) void wgrad_generic_kernel(const E* __restrict__ dY, const E* __restrict__ X,
                                                            int64_t T, int64_t N, int64_t K,
                                                            const uint32_t* __restrict__ meta, O* __restrict__ dWv,
                                                            O* __restrict__ dWd, int accumulate) {
  __shared__ float Ds[KSTEP * (TILE + 1)];
  __shared__ float Xs[KSTEP * (TILE + 1)];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t k0 = (int64_t)blockIdx.x * TILE, n0 = (int64_t)blockIdx.y * TILE;
  float acc[4][4] = {};  // [n][k]
  for (int64_t tb = 0; tb < T; tb += KSTEP) {
    for (int i = threadIdx.x; i < KSTEP * TILE; i += 256) {
      const int tt = i / TILE, c = i % TILE;
      const int64_t t = tb + tt;
      Ds[tt * (TILE + 1) + c] = (t < T && n0 + c < N) ? to_f32(dY[t * N + n0 + c]) : 0.f;
      Xs[tt * (TILE + 1) + c] = (t < T && k0 + c < K) ? to_f32(X[t * K + k0 + c]) : 0.f;
    }
    __syncthreads();
    for (int tt = 0; tt < KSTEP; ++tt) {
      float a[4], b[4];
      for (int i = 0; i < 4; ++i) a[i] = Ds[tt * (TILE + 1) + ty * 4 + i];
      for (int j = 0; j < 4; ++j) b[j] = Xs[tt * (TILE + 1) + tx * 4 + j];
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  const int64_t wpr = cdiv(K / 4, 8);
  const int64_t kg = k0 + tx * 4;  // this thread's four k form one 2:4 group
  if (kg >= K) return;
  const int64_t g = kg / 4;
  for (int i = 0; i < 4; ++i) {
    const int64_t n = n0 + ty * 4 + i;
    if (n >= N) continue;
    const uint32_t nib = (meta[n * wpr + g / 8] >> (4 * (g % 8))) & 0xFu;
    const uint32_t i0 = nib & 3u, i1 = nib >> 2;
    O* v = dWv + n * (K / 2) + 2 * g;
    float v0 = acc[i][i0], v1 = acc[i][i1];
    if (accumulate) { v0 += load_out(v); v1 += load_out(v + 1); }
    store_out(v, v0);
    store_out(v + 1, v1);
    if (dWd) {
      O* d = dWd + n * K + kg;
      for (int j = 0; j < 4; ++j) {
        float x = (j == (int)i0 || j == (int)i1) ? acc[i][j] : 0.f;
        if (accumulate) x += load_out(d + j);
        store_out(d + j, x);
      }
    }
  }
}

// xl[s][t][j] = sum over k in [s*kc, (s+1)*kc) of X[t][k] L[k][j].
template <typename E>
__global__ __launch_bounds__(256) void lowrank_down_generic_kernel(const E* __restrict__ X, const E* __restrict__ L,
                                                                   int64_t T, int64_t K, int64_t r, int64_t kc,
                                                                   float* __restrict__ xl) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * r) return;
  const int64_t s = blockIdx.y;
  const int64_t t = i / r, j = i % r;
  const int64_t kb = s * kc, ke = (kb + kc < K) ? kb + kc : K;
  float a = 0.f;
  for (int64_t k = kb; k < ke; ++k) a = fmaf(to_f32(X[t * K + k]), to_f32(L[k * r + j]), a);
  xl[s * T * r + i] = a;
}

// Y[t][m] += sum_s xl[s][t] . R[:, m]
template <typename E, typename O>
__global__ __launch_bounds__(256) void lowrank_up_generic_kernel(const float* __restrict__ xl, int splits,
                                                                 const E* __restrict__ R, int64_t T, int64_t r,
                                                                 int64_t N, O* __restrict__ Y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * N) return;
  const int64_t t = i / N, m = i % N;
  float a = 0.f;
  for (int64_t q = 0; q < r; ++q) {
    float x = 0.f;
    for (int s = 0; s < splits; ++s) x += xl[((int64_t)s * T + t) * r + q];
    a = fmaf(x, to_f32(R[q * N + m]), a);
  }
  store_out(Y + i, load_out(Y + i) + a);
}

template <typename O>
__global__ void fill_zero_kernel(O* __restrict__ Y, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) Y[i] = (O)0;
}

}  // namespace

namespace {

// storage type of each input format: bf16 bits, fp16, fp32 bits
template <typename E, typename O>
void spmm_generic(dim3 grid, const void* B, const void* values, const uint32_t* meta, int64_t M, int64_t T,
                  int64_t Kred, const float* xl, int splits, int64_t r, const void* R, void* Y, hipStream_t s) {
  spmm_generic_kernel<E, O><<<grid, 256, 0, s>>>((const E*)B, (const E*)values, meta, M, T, Kred, xl, splits, r,
                                                 (const E*)R, (O*)Y);
}
template <typename E, typename O>
void wgrad_generic(dim3 grid, const void* dY, const void* X, int64_t T, int64_t N, int64_t K, const uint32_t* meta,
                   void* dWv, void* dWd, int accumulate, hipStream_t s) {
  wgrad_generic_kernel<E, O><<<grid, 256, 0, s>>>((const E*)dY, (const E*)X, T, N, K, meta, (O*)dWv, (O*)dWd,
                                                  accumulate);
}
template <typename E, typename O>
void up_generic(unsigned grid, const float* xl, int splits, const void* R, int64_t T, int64_t r, int64_t N, void* Y,
                hipStream_t s) {
  lowrank_up_generic_kernel<E, O><<<grid, 256, 0, s>>>(xl, splits, (const E*)R, T, r, N, (O*)Y);
}

}  // namespace

// in: the input format; out: the input format or F32 (F32 inputs take F32 outputs)
hipError_t launch_spmm_generic(Dt in, Dt out, const void* B, int64_t T, int64_t Kred, const void* values,
                               const uint32_t* meta, int64_t M, const float* xl, int splits, int64_t r,
                               const void* R, void* Y, hipStream_t s) {
  dim3 grid((unsigned)cdiv(M, TILE), (unsigned)cdiv(T, TILE));
  if (in == Dt::BF16 && out == Dt::BF16)
    spmm_generic<uint16_t, uint16_t>(grid, B, values, meta, M, T, Kred, xl, splits, r, R, Y, s);
  else if (in == Dt::BF16)
    spmm_generic<uint16_t, float>(grid, B, values, meta, M, T, Kred, xl, splits, r, R, Y, s);
  else if (in == Dt::F16 && out == Dt::F16)
    spmm_generic<_Float16, _Float16>(grid, B, values, meta, M, T, Kred, xl, splits, r, R, Y, s);
  else if (in == Dt::F16)
    spmm_generic<_Float16, float>(grid, B, values, meta, M, T, Kred, xl, splits, r, R, Y, s);
  else
    spmm_generic<uint32_t, float>(grid, B, values, meta, M, T, Kred, xl, splits, r, R, Y, s);
  return hipGetLastError();
}

hipError_t launch_wgrad_generic(Dt in, Dt out, const void* dY, const void* X, int64_t T, int64_t N, int64_t K,
                                const uint32_t* meta_s, void* dWv, void* dWd, int accumulate, hipStream_t s) {
  dim3 grid((unsigned)cdiv(K, TILE), (unsigned)cdiv(N, TILE));
  if (in == Dt::BF16 && out == Dt::BF16)
    wgrad_generic<uint16_t, uint16_t>(grid, dY, X, T, N, K, meta_s, dWv, dWd, accumulate, s);
  else if (in == Dt::BF16)
    wgrad_generic<uint16_t, float>(grid, dY, X, T, N, K, meta_s, dWv, dWd, accumulate, s);
  else if (in == Dt::F16 && out == Dt::F16)
    wgrad_generic<_Float16, _Float16>(grid, dY, X, T, N, K, meta_s, dWv, dWd, accumulate, s);
  else if (in == Dt::F16)
    wgrad_generic<_Float16, float>(grid, dY, X, T, N, K, meta_s, dWv, dWd, accumulate, s);
  else
    wgrad_generic<uint32_t, float>(grid, dY, X, T, N, K, meta_s, dWv, dWd, accumulate, s);
  return hipGetLastError();
}

hipError_t launch_lowrank_down_generic(Dt in, const void* X, const void* L, int64_t T, int64_t K, int64_t r,
                                       int splits, int64_t kc, float* xl, hipStream_t s) {
  if (T * r == 0) return hipSuccess;
  dim3 grid((unsigned)cdiv(T * r, 256), (unsigned)splits);
  if (in == Dt::BF16)
    lowrank_down_generic_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)X, (const uint16_t*)L, T, K, r, kc, xl);
  else if (in == Dt::F16)
    lowrank_down_generic_kernel<_Float16><<<grid, 256, 0, s>>>((const _Float16*)X, (const _Float16*)L, T, K, r, kc, xl);
  else
    lowrank_down_generic_kernel<uint32_t><<<grid, 256, 0, s>>>((const uint32_t*)X, (const uint32_t*)L, T, K, r, kc, xl);
  return hipGetLastError();
}

hipError_t launch_lowrank_up_generic(Dt in, Dt out, const float* xl, int splits, const void* R, int64_t T,
                                     int64_t r, int64_t N, void* Y, hipStream_t s) {
  const unsigned grid = (unsigned)cdiv(T * N, 256);
  if (in == Dt::BF16 && out == Dt::BF16)
    up_generic<uint16_t, uint16_t>(grid, xl, splits, R, T, r, N, Y, s);
  else if (in == Dt::BF16)
    up_generic<uint16_t, float>(grid, xl, splits, R, T, r, N, Y, s);
  else if (in == Dt::F16 && out == Dt::F16)
    up_generic<_Float16, _Float16>(grid, xl, splits, R, T, r, N, Y, s);
  else if (in == Dt::F16)
    up_generic<_Float16, float>(grid, xl, splits, R, T, r, N, Y, s);
  else
    up_generic<uint32_t, float>(grid, xl, splits, R, T, r, N, Y, s);
  return hipGetLastError();
}

hipError_t launch_fill_zero(Dt out, void* Y, int64_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  const unsigned grid = (unsigned)(cdiv(count, 256) < 4096 ? cdiv(count, 256) : 4096);
  if (out == Dt::F32) fill_zero_kernel<float><<<grid, 256, 0, s>>>((float*)Y, count);
  else fill_zero_kernel<uint16_t><<<grid, 256, 0, s>>>((uint16_t*)Y, count);   // +0 in bf16 and fp16
  return hipGetLastError();
}

}  // namespace slope

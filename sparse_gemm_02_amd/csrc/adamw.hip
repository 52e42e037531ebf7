// AdamW on stored values: the compressed values of a 2:4 weight (moments only
// for the kept slots, the mask does not move) or a dense adapter factor.  An
// elementwise HBM-bound pass: 8 values per thread and iteration with 16-byte
// loads and stores, a scalar loop for the last n % 8.  The fused form that
// also double-prunes the updated weight lives with the double prune kernel.
#include <type_traits>

#include "adamw.h"

namespace slope {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float load1(const uint16_t* p) { return bf16_bits_to_f32(*p); }
__device__ __forceinline__ float load1(const _Float16* p) { return (float)*p; }
__device__ __forceinline__ float load1(const float* p) { return *p; }

template <typename PT, typename GT>
__global__ __launch_bounds__(kThreads) void adamw_kernel(PT* __restrict__ p, const GT* __restrict__ g,
                                                         float* __restrict__ m, float* __restrict__ v, int64_t n,
                                                         AdamWStep c) {
  const int64_t stride = (int64_t)gridDim.x * kThreads, t0 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t n8 = n / 8;
  for (int64_t i = t0; i < n8; i += stride) {
    const int64_t e = 8 * i;
    if constexpr (sizeof(PT) == 2) {
      constexpr bool H = std::is_same<PT, _Float16>::value;
      u32x4 w = *reinterpret_cast<const u32x4*>(p + e);
      *reinterpret_cast<u32x4*>(p + e) = adamw8_16<H>(w, g + e, m + e, v + e, c);
    } else {
      float pf[8], gf[8], mf[8], vf[8];
      load8_f32(p + e, pf);
      load8_f32(g + e, gf);
      load8_f32(m + e, mf);
      load8_f32(v + e, vf);
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[j] = adamw_apply(pf[j], gf[j], mf[j], vf[j], c);
      store8_f32(p + e, pf);
      store8_f32(m + e, mf);
      store8_f32(v + e, vf);
    }
  }
  for (int64_t e = 8 * n8 + t0; e < n; e += stride) {
    float mm = m[e], vv = v[e];
    const float np = adamw_apply(load1(p + e), load1(g + e), mm, vv, c);
    store_out(p + e, np);
    m[e] = mm;
    v[e] = vv;
  }
}

template <typename PT, typename GT>
hipError_t run(void* p, const void* g, float* m, float* v, int64_t n, const AdamWStep& c, hipStream_t s) {
  int64_t blocks = cdiv(cdiv(n, 8), kThreads);
  if (blocks > 256 * 16) blocks = 256 * 16;     // 16 blocks per CU, grid-stride beyond
  if (blocks < 1) blocks = 1;
  adamw_kernel<PT, GT><<<(unsigned)blocks, kThreads, 0, s>>>((PT*)p, (const GT*)g, m, v, n, c);
  return hipGetLastError();
}

}  // namespace

namespace {
template <typename PT>
hipError_t run_grad(Dt grad, void* params, const void* grads, float* m, float* v, int64_t n, const AdamWStep& c,
                    hipStream_t s) {
  if (grad == Dt::BF16) return run<PT, uint16_t>(params, grads, m, v, n, c, s);
  if (grad == Dt::F16) return run<PT, _Float16>(params, grads, m, v, n, c, s);
  return run<PT, float>(params, grads, m, v, n, c, s);
}
}  // namespace

hipError_t launch_adamw(Dt param, Dt grad, void* params, const void* grads, float* m, float* v, int64_t n,
                        const AdamWStep& c, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (param == Dt::BF16) return run_grad<uint16_t>(grad, params, grads, m, v, n, c, s);
  if (param == Dt::F16) return run_grad<_Float16>(grad, params, grads, m, v, n, c, s);
  return run_grad<float>(grad, params, grads, m, v, n, c, s);
}

}  // namespace slope

// Internal launchers of the SLoPe 2:4 library.  Arguments are validated by the
// C-ABI layer before any of these is called; each only enqueues kernels on the
// given stream and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace slope {

enum class Dt { F32 = 0, BF16 = 1 };

hipError_t launch_prune24(Dt dt, const void* W, int64_t rows, int64_t cols, uint8_t* mask, void* W_s,
                          hipStream_t s);
hipError_t launch_compress24(Dt dt, const void* W, const uint8_t* mask, int64_t rows, int64_t cols, void* values,
                             uint32_t* meta, int32_t* invalid, hipStream_t s);
hipError_t launch_double_prune(Dt dt, const void* values_s, const uint32_t* meta_s, int64_t N, int64_t K,
                               void* values_dpT, uint32_t* meta_dpT, uint8_t* mask_dpT, hipStream_t s);

// Number of K-splits of the adapter down-projection for T tokens and reduction K.
int lowrank_splits(int64_t T, int64_t K);

// xl[s][t][j] = partial sums of X[t, :] . L[:, j] over split s (fp32).
hipError_t launch_lowrank_down(Dt in, const void* X, const void* L, int64_t T, int64_t K, int64_t r, int splits,
                               float* xl, hipStream_t s);

// Y[t][m] = B[t, :] . Adense[m, :]  (+ sum_s xl[s][t, :] . R[:, m] when xl != nullptr)
// with Adense the decompressed 2:4 operand [M, Kred] and B row-major [T, Kred].
hipError_t launch_spmm(Dt in, Dt out, const void* B, int64_t T, int64_t Kred, const void* values,
                       const uint32_t* meta, int64_t M, const float* xl, int splits, int64_t r, const void* R,
                       void* Y, hipStream_t s);

// dW = (dY^T . X) kept at meta_s, written compressed (+ dense) with optional accumulation.
hipError_t launch_masked_wgrad(Dt in, Dt out, const void* dY, const void* X, int64_t T, int64_t N, int64_t K,
                               const uint32_t* meta_s, void* dW_values, void* dW_dense, int accumulate,
                               hipStream_t s);

// Y[t][m] += sum_s xl[s][t, :] . R[:, m]
hipError_t launch_lowrank_up_add(Dt in, Dt out, const float* xl, int splits, const void* R, int64_t T, int64_t r,
                                 int64_t N, void* Y, hipStream_t s);

// Y[t][m] = 0 (empty reductions).
hipError_t launch_fill_zero(Dt out, void* Y, int64_t count, hipStream_t s);

}  // namespace slope

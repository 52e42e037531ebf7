// Internal launchers of the SLoPe 2:4 library.  Arguments are validated by the
// C-ABI layer before any of these is called; each only enqueues kernels on the
// given stream and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace slope {

enum class Dt { F32 = 0, BF16 = 1, F16 = 2 };

// Compute units of the current device (256 on MI355X; that figure if the
// query fails, in which case the following launch reports the error).
inline int64_t device_compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return 256;
  return cus;
}

hipError_t launch_prune24(Dt dt, const void* W, int64_t rows, int64_t cols, uint8_t* mask, void* W_s,
                          hipStream_t s);
hipError_t launch_prune_nm(Dt dt, const void* W, int64_t rows, int64_t cols, int n, int m, uint8_t* mask, void* W_s,
                           hipStream_t s);
hipError_t launch_compress24(Dt dt, const void* W, const uint8_t* mask, int64_t rows, int64_t cols, void* values,
                             uint32_t* meta, int32_t* invalid, hipStream_t s);
hipError_t launch_double_prune(Dt dt, const void* values_s, const uint32_t* meta_s, int64_t N, int64_t K,
                               void* values_dpT, uint32_t* meta_dpT, uint8_t* mask_dpT, hipStream_t s);
// prune24 and compress24 in one pass (mask optional); with packed (16-bit,
// cols % 16 == 0) also W_s's tile chunks.
hipError_t launch_prune_compress24(Dt dt, const void* W, int64_t rows, int64_t cols, uint8_t* mask, void* values,
                                   uint32_t* meta, void* packed, hipStream_t s);

// Per-update constants of AdamW, derived on the host in double precision and
// rounded once to fp32:
//   p' = p * decay - step_size * m' / (sqrt(v') * inv_sqrt_bc2 + eps)
//   m' = beta1 m + omb1 g,  v' = beta2 v + omb2 g^2
struct AdamWStep {
  float decay, beta1, omb1, beta2, omb2, step_size, inv_sqrt_bc2, eps;
};
hipError_t launch_adamw(Dt param, Dt grad, void* params, const void* grads, float* m, float* v, int64_t n,
                        const AdamWStep& c, hipStream_t s);
// AdamW on the compressed values of W_s, then the double prune of the result.
hipError_t launch_adamw_double_prune(Dt dt, Dt grad, void* values_s, const uint32_t* meta_s, const void* grads,
                                     float* m, float* v, int64_t N, int64_t K, const AdamWStep& c,
                                     void* values_dpT, uint32_t* meta_dpT, uint8_t* mask_dpT, hipStream_t s);
// The same two steps with W_dp^T written as tile chunks, and the updated
// values also rewritten inside W_s's tile chunks (16-bit, K % 16 == 0,
// N % 16 == 0; checked by the caller).
hipError_t launch_double_prune_packed(Dt dt, const void* values_s, const uint32_t* meta_s, int64_t N, int64_t K,
                                      void* packed_dpT, hipStream_t s);
hipError_t launch_adamw_double_prune_packed(Dt dt, Dt grad, void* values_s, const uint32_t* meta_s,
                                            const void* grads, float* m, float* v, int64_t N, int64_t K,
                                            const AdamWStep& c, void* packed_s, void* packed_dpT, hipStream_t s);

// Adapter workspace (caller-owned device memory), carved into:
//   part [splits][T][r] fp32   partial sums of X . L over k-splits
//   xlh, xll [Tpad][rpad] bf16 X . L split into hi + lo bf16 parts (zero padded)
//   lt [rpad][Kpad] bf16       L transposed (zero padded)
//   rt [Npad][rpad] bf16       R transposed (zero padded)
// with rpad = r rounded up to 16, Tpad/Npad rounded up to 256, Kpad to 8.
struct LowrankWs {
  float* part = nullptr;
  uint16_t *xlh = nullptr, *xll = nullptr, *lt = nullptr, *rt = nullptr;
  int splits = 1;
  int64_t rpad = 0, Tpad = 0, Kpad = 0, Npad = 0, kc = 0;
  bool mfma = false;  // rt / xlh / xll are filled (16-bit inputs, K % 8 == 0, r <= 128)
  bool h16 = false;   // the 16-bit format is fp16 (else bf16): lt, rt, xlh, xll hold fp16
};
int64_t lowrank_workspace_bytes(int64_t T, int64_t K, int64_t r, int64_t N);
LowrankWs lowrank_layout(Dt in, void* ws, int64_t T, int64_t K, int64_t r, int64_t N);

// Fills the workspace for Y += (X . L) . R: the k-split partial sums and, on
// the bf16 path, the transposed L and R and the hi/lo split of X . L.
hipError_t launch_lowrank_prepare(Dt in, const void* X, const void* L, const void* R, int64_t T, int64_t K,
                                  int64_t r, int64_t N, const LowrankWs& w, hipStream_t s);

// Only the down-projection part (bf16, w.mfma): X . L as the hi/lo pair in w.
hipError_t launch_lowrank_down(Dt in, const void* X, const void* L, int64_t T, int64_t K, int64_t r,
                               const LowrankWs& w, hipStream_t s);

// Adapter backward, dX term: G = dY . R^T into w (hi/lo) with L as the
// epilogue operand, w laid out by lowrank_layout(BF16, ws, T, N, r, K): the
// forward's roles with (X, L, R, K, N) -> (dY, R^T, L^T, N, K).
hipError_t launch_lowrank_prepare_bwd(const void* dY, const void* L, const void* R, int64_t T, int64_t N, int64_t r,
                                      int64_t K, const LowrankWs& w, hipStream_t s);
// The hi/lo pairs of w1 and w2, each transposed to [rpad32][Tpad] (rows past
// rpad zero), in one launch.
hipError_t launch_transpose_hilo2(const LowrankWs& w1, const LowrankWs& w2, int64_t rpad32, uint16_t* xht1,
                                  uint16_t* xlt1, uint16_t* xht2, uint16_t* xlt2, hipStream_t s);

// Adapter weight gradients from token chunks: out = A^T . B over the tokens with
// A the chunks of a [T, C] matrix and B given as a transposed hi/lo pair
// [32*ceil(r/32)][Tpad]; written as out[j][c] (dR) or, trans, out[c][j] (dL).
// part: lr_wgrad_part_bytes(T, C, r) of fp32 scratch.
struct LrGrad {
  const void* chunks;
  int64_t C;
  const uint16_t* bh;
  const uint16_t* bl;
  int64_t Tpad;
  float* part;
  void* dst;
  bool trans;
};
int64_t lr_wgrad_part_bytes(int64_t T, int64_t C, int64_t r);
// Both gradients of one adapter (the same T and r) in one partial-sum launch
// and one reduce; T > 0, r in 1 .. 128, both C > 0.
hipError_t launch_lr_wgrad_pair(Dt in, Dt out, const LrGrad& g0, const LrGrad& g1, int64_t T, int64_t r,
                                int accumulate, hipStream_t s);

// Y[t][m] = B[t, :] . Adense[m, :]  (+ (X . L)[t, :] . R[:, m] when ws != nullptr)
// with Adense the decompressed 2:4 operand [M, Kred] and B row-major [T, Kred].
hipError_t launch_spmm(Dt in, Dt out, const void* B, int64_t T, int64_t Kred, const void* values,
                       const uint32_t* meta, int64_t M, const LowrankWs* ws, int64_t r, const void* R, void* Y,
                       hipStream_t s);

// Tile chunks of a compressed bf16 operand [M, Kred] (Kred % 16 == 0,
// Kred <= 2^21): size in bytes and the packing pass; launch_spmm_packed is
// launch_spmm on that form (bf16 B; ws with ws->mfma, or nullptr); with tok
// not null it also writes B's token chunks (pack_tokens' layout,
// packed_tokens_bytes(T, Kred) bytes) from the operand stages it loads.
int64_t packed_sparse_bytes(int64_t M, int64_t Kred);
hipError_t launch_pack_sparse(const void* values, const uint32_t* meta, int64_t M, int64_t Kred, void* packed,
                              hipStream_t s);
hipError_t launch_spmm_packed(Dt in, Dt out, const void* B, int64_t T, int64_t Kred, const void* packed, int64_t M,
                              const LowrankWs* ws, void* Y, void* tok, hipStream_t s);

// Forward for T <= 64 tokens on tile-chunk weights (bf16): split-k partial
// sums reduced in order, plus the adapter term when r > 0 (L [K, r],
// R [r, N]); workspace of decode_workspace_bytes(T, K, r, N) bytes.
int64_t decode_workspace_bytes(int64_t T, int64_t K, int64_t r, int64_t N);
// The few-token forward's own scratch (a static device array, one per GPU):
// its size, and its device address on the current device (looked up once per
// device, then cached).
constexpr int64_t kDecodeScratchBytes = int64_t(32) << 20;
hipError_t decode_scratch_address(void** ptr);
hipError_t launch_spmm_decode(Dt in, Dt out, const void* X, int64_t T, int64_t K, const void* packed, int64_t N,
                              const void* L, const void* R, int64_t r, void* workspace, void* Y, hipStream_t s);

// dW = (dY^T . X) kept at meta_s, written compressed (+ dense) with optional
// accumulation.  With a workspace of wgrad_workspace_bytes(T, N, K) bytes the
// bf16 path first packs X and dY into transposed token chunks there.
int64_t wgrad_workspace_bytes(int64_t T, int64_t N, int64_t K);
// Token chunks of a bf16 matrix [T, C] (C % 8 == 0): bytes, and the packing pass.
int64_t packed_tokens_bytes(int64_t T, int64_t C);
// fp32 partial sums of the weight gradient's token split on the current
// device (0 when the tile grid fills the device without it).
int64_t wgrad_split_bytes(int64_t T, int64_t N, int64_t K);
hipError_t launch_pack_tokens(const void* M, int64_t T, int64_t C, void* packed, hipStream_t s);
// The weight-gradient GEMM on packed bf16 operands (N % 8 == 0, K % 8 == 0).
hipError_t launch_masked_wgrad_packed(Dt in, Dt out, const void* dY_packed, const void* X_packed, int64_t T,
                                      int64_t N, int64_t K, const uint32_t* meta_s, void* dW_values, void* dW_dense,
                                      int accumulate, void* split_part, hipStream_t s);
hipError_t launch_masked_wgrad(Dt in, Dt out, const void* dY, const void* X, int64_t T, int64_t N, int64_t K,
                               const uint32_t* meta_s, void* dW_values, void* dW_dense, int accumulate,
                               void* workspace, hipStream_t s);

// Y[t][m] += (X . L)[t, :] . R[:, m] from a prepared workspace.
hipError_t launch_lowrank_up_add(Dt in, Dt out, const LowrankWs& w, const void* R, int64_t T, int64_t r,
                                 int64_t N, void* Y, hipStream_t s);

// Y[t][m] = 0 (empty reductions).
hipError_t launch_fill_zero(Dt out, void* Y, int64_t count, hipStream_t s);

// 8-bit (E4M3) variant: per-tensor scale 448 / amax and codes of a 16-bit
// tensor (scale: one device float, also used as the amax word while the
// kernels run); E4M3 tile chunks of a compressed 16-bit matrix with its scale;
// the 2:4 product on them, Y [T, M] = (Xq . W_q^T) / (x_scale * w_scale).
int64_t packed_sparse_e4m3_bytes(int64_t rows, int64_t cols);
hipError_t launch_quantize_e4m3(Dt dt, const void* M, int64_t n, float* scale, uint8_t* q, hipStream_t s);
hipError_t launch_pack_sparse_e4m3(Dt dt, const void* values, const uint32_t* meta, int64_t M, int64_t Kred,
                                   float* scale, void* packed, hipStream_t s);
hipError_t launch_spmm_e4m3(Dt out, const uint8_t* Xq, const float* x_scale, int64_t T, int64_t Kred,
                            const void* packed, const float* w_scale, int64_t M, void* Y, hipStream_t s);

}  // namespace slope

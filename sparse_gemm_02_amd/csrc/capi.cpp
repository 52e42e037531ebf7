// C ABI of the SLoPe 2:4 library: argument checks, then kernel launches.
// Every check happens before the first launch, so an error leaves all outputs
// untouched.  Declarations and the meaning of every argument: include/slope.h.
#include <hip/hip_runtime.h>

#include <cmath>

#include "../../include/slope.h"
#include "launch.h"

using slope::Dt;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dt_ok(int d) { return d == SLOPE_F32 || d == SLOPE_BF16 || d == SLOPE_F16; }

bool in_range(int64_t v) { return v >= 0 && v <= SLOPE_MAX_DIM; }

slope_status from_hip(hipError_t e) { return e == hipSuccess ? SLOPE_OK : SLOPE_ERR_HIP; }

slope_status check_io(slope_dtype in, slope_dtype out) {
  if (!dt_ok(in) || !dt_ok(out)) return SLOPE_ERR_INVALID_ARG;
  // outputs: the input's own format, or fp32
  if (out != SLOPE_F32 && out != in) return SLOPE_ERR_UNSUPPORTED;
  return SLOPE_OK;
}

// Pointer check: required pointers must be non-null; all non-null pointers aligned.
slope_status ptr(const void* p, bool required) {
  if (!p) return required ? SLOPE_ERR_INVALID_ARG : SLOPE_OK;
  return aligned16(p) ? SLOPE_OK : SLOPE_ERR_ALIGN;
}

#define SLOPE_TRY(x)                       \
  do {                                     \
    slope_status _st = (x);                \
    if (_st != SLOPE_OK) return _st;       \
  } while (0)

// Packed sparse operands: reduction width up to 2^21 (chunk resources stay
// below 2 GiB), adapter rank up to 128 (the MFMA epilogue).
constexpr int64_t kPackedMaxCols = 1 << 21, kPackedMaxRank = 128;
constexpr int64_t kDecodeMaxTokens = 64;   // the few-token forward

int64_t workspace_need(int64_t T, int64_t K, int64_t r, int64_t N) { return slope::lowrank_workspace_bytes(T, K, r, N); }

// Checks AdamW hyper-parameters and derives the per-update fp32 constants.
slope_status adamw_step(const slope_adamw_params* hp, slope::AdamWStep* c) {
  if (!hp) return SLOPE_ERR_INVALID_ARG;
  if (hp->step < 1 || !(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) ||
      !(hp->eps >= 0.0) || !std::isfinite(hp->eps) || !std::isfinite(hp->lr) || !std::isfinite(hp->weight_decay))
    return SLOPE_ERR_INVALID_ARG;
  const double t = (double)hp->step;
  const double bc1 = 1.0 - std::pow(hp->beta1, t), bc2 = 1.0 - std::pow(hp->beta2, t);
  c->decay = (float)(1.0 - hp->lr * hp->weight_decay);
  c->beta1 = (float)hp->beta1;
  c->omb1 = (float)(1.0 - hp->beta1);
  c->beta2 = (float)hp->beta2;
  c->omb2 = (float)(1.0 - hp->beta2);
  c->step_size = (float)(hp->lr / bc1);
  c->inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  c->eps = (float)hp->eps;
  return SLOPE_OK;
}

constexpr int64_t kAdamwMaxElems = int64_t(1) << 40;

// Adapter arguments: both factors with r > 0 (adapter on), or neither with any
// r >= 0 (adapter off).  One factor without the other, or factors with r == 0,
// is a caller error rather than a silent adapter-free product.
slope_status adapter_args(const void* L, const void* R, int64_t r, bool* on) {
  const bool have_l = L != nullptr, have_r = R != nullptr;
  if (have_l != have_r) return SLOPE_ERR_INVALID_ARG;
  if (have_l && r == 0) return SLOPE_ERR_INVALID_ARG;
  *on = have_l && r > 0;
  if (*on) {
    SLOPE_TRY(ptr(L, true));
    SLOPE_TRY(ptr(R, true));
  }
  return SLOPE_OK;
}

}  // namespace

extern "C" {

int slope_version(void) { return 200; }

const char* slope_status_string(int status) {
  switch (status) {
    case SLOPE_OK: return "ok";
    case SLOPE_ERR_INVALID_ARG: return "invalid argument (null pointer, unknown dtype or negative size)";
    case SLOPE_ERR_SHAPE: return "a 2:4 dimension is not a multiple of 4";
    case SLOPE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case SLOPE_ERR_WORKSPACE: return "workspace or operand buffer missing or too small";
    case SLOPE_ERR_HIP: return "HIP runtime error";
    case SLOPE_ERR_UNSUPPORTED: return "unsupported dtype combination or size";
    default: return "unknown status";
  }
}

slope_status slope_compressed_sizes(int64_t rows, int64_t cols, int64_t* n_values, int64_t* n_meta_words) {
  if (!n_values || !n_meta_words || rows < 0 || cols < 0) return SLOPE_ERR_INVALID_ARG;
  if (cols % 4) return SLOPE_ERR_SHAPE;
  *n_values = rows * (cols / 2);
  *n_meta_words = rows * ((cols / 4 + 7) / 8);
  return SLOPE_OK;
}

slope_status slope_lowrank_workspace_bytes(int64_t T, int64_t K, int64_t r, int64_t N, int64_t* bytes) {
  if (!bytes || T < 0 || K < 0 || r < 0 || N < 0) return SLOPE_ERR_INVALID_ARG;
  if (!in_range(T) || !in_range(K) || !in_range(r) || !in_range(N)) return SLOPE_ERR_UNSUPPORTED;
  *bytes = workspace_need(T, K, r, N);
  return SLOPE_OK;
}

slope_status slope_prune24(slope_dtype dt, const void* W, int64_t rows, int64_t cols, uint8_t* mask,
                           void* W_s_or_null, void* stream) {
  if (!dt_ok(dt) || rows < 0 || cols < 0) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(W, true));
  SLOPE_TRY(ptr(mask, true));
  SLOPE_TRY(ptr(W_s_or_null, false));
  if (cols % 4) return SLOPE_ERR_SHAPE;
  if (!in_range(rows) || !in_range(cols)) return SLOPE_ERR_UNSUPPORTED;
  return from_hip(slope::launch_prune24((Dt)dt, W, rows, cols, mask, W_s_or_null, (hipStream_t)stream));
}

slope_status slope_prune_nm(slope_dtype dt, const void* W, int64_t rows, int64_t cols, int n, int m, uint8_t* mask,
                           void* W_s_or_null, void* stream) {
  if (!dt_ok(dt) || rows < 0 || cols < 0) return SLOPE_ERR_INVALID_ARG;
  if (m != 4 && m != 8 && m != 16 && m != 32) return SLOPE_ERR_UNSUPPORTED;
  if (n < 1 || n > m) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(W, true));
  SLOPE_TRY(ptr(mask, true));
  SLOPE_TRY(ptr(W_s_or_null, false));
  if (cols % m) return SLOPE_ERR_SHAPE;
  if (!in_range(rows) || !in_range(cols)) return SLOPE_ERR_UNSUPPORTED;
  return from_hip(slope::launch_prune_nm((Dt)dt, W, rows, cols, n, m, mask, W_s_or_null, (hipStream_t)stream));
}

slope_status slope_prune_compress24(slope_dtype dt, const void* W, int64_t rows, int64_t cols, uint8_t* mask_or_null,
                                    void* values, uint32_t* meta, void* packed_or_null, int64_t packed_bytes,
                                    void* stream) {
  if (!dt_ok(dt) || rows < 0 || cols < 0 || packed_bytes < 0) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(W, true));
  SLOPE_TRY(ptr(mask_or_null, false));
  SLOPE_TRY(ptr(values, true));
  SLOPE_TRY(ptr(meta, true));
  SLOPE_TRY(ptr(packed_or_null, false));
  if (cols % 4) return SLOPE_ERR_SHAPE;
  if (!in_range(rows) || !in_range(cols)) return SLOPE_ERR_UNSUPPORTED;
  if (packed_or_null) {
    if (dt == SLOPE_F32) return SLOPE_ERR_UNSUPPORTED;   // tile chunks hold 16-bit values
    if (cols % 16) return SLOPE_ERR_SHAPE;
    if (cols > kPackedMaxCols) return SLOPE_ERR_UNSUPPORTED;
    if (packed_bytes < slope::packed_sparse_bytes(rows, cols)) return SLOPE_ERR_WORKSPACE;
  }
  return from_hip(slope::launch_prune_compress24((Dt)dt, W, rows, cols, mask_or_null, values, meta, packed_or_null,
                                                 (hipStream_t)stream));
}

slope_status slope_compress24(slope_dtype dt, const void* W, const uint8_t* mask, int64_t rows, int64_t cols,
                              void* values, uint32_t* meta, int32_t* invalid_groups_or_null, void* stream) {
  if (!dt_ok(dt) || rows < 0 || cols < 0) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(W, true));
  SLOPE_TRY(ptr(mask, true));
  SLOPE_TRY(ptr(values, true));
  SLOPE_TRY(ptr(meta, true));
  if (invalid_groups_or_null && (reinterpret_cast<uintptr_t>(invalid_groups_or_null) & 3u)) return SLOPE_ERR_ALIGN;
  if (cols % 4) return SLOPE_ERR_SHAPE;
  if (!in_range(rows) || !in_range(cols)) return SLOPE_ERR_UNSUPPORTED;
  return from_hip(slope::launch_compress24((Dt)dt, W, mask, rows, cols, values, meta, invalid_groups_or_null,
                                           (hipStream_t)stream));
}

slope_status slope_double_prune(slope_dtype dt, const void* values_s, const uint32_t* meta_s, int64_t N, int64_t K,
                                void* values_dpT, uint32_t* meta_dpT, uint8_t* mask_dpT_or_null, void* stream) {
  if (!dt_ok(dt) || N < 0 || K < 0) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(values_s, true));
  SLOPE_TRY(ptr(meta_s, true));
  SLOPE_TRY(ptr(values_dpT, true));
  SLOPE_TRY(ptr(meta_dpT, true));
  SLOPE_TRY(ptr(mask_dpT_or_null, false));
  if (N % 4 || K % 4) return SLOPE_ERR_SHAPE;
  if (!in_range(N) || !in_range(K)) return SLOPE_ERR_UNSUPPORTED;
  return from_hip(slope::launch_double_prune((Dt)dt, values_s, meta_s, N, K, values_dpT, meta_dpT,
                                             mask_dpT_or_null, (hipStream_t)stream));
}

slope_status slope_spmm_fwd(slope_dtype in_dt, slope_dtype out_dt, const void* X, int64_t T, int64_t K,
                            const void* values_s, const uint32_t* meta_s, int64_t N, const void* L_or_null,
                            const void* R_or_null, int64_t r, void* workspace_or_null, int64_t workspace_bytes,
                            void* Y, void* stream) {
  SLOPE_TRY(check_io(in_dt, out_dt));
  if (T < 0 || K < 0 || N < 0 || r < 0) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(X, true));
  SLOPE_TRY(ptr(values_s, true));
  SLOPE_TRY(ptr(meta_s, true));
  SLOPE_TRY(ptr(Y, true));
  bool adapter = false;
  SLOPE_TRY(adapter_args(L_or_null, R_or_null, r, &adapter));
  if (K % 4) return SLOPE_ERR_SHAPE;
  if (!in_range(T) || !in_range(K) || !in_range(N) || !in_range(r)) return SLOPE_ERR_UNSUPPORTED;
  if (adapter) {
    const int64_t need = workspace_need(T, K, r, N);
    if (need > 0 && (!workspace_or_null || workspace_bytes < need)) return SLOPE_ERR_WORKSPACE;
    if (workspace_or_null && !aligned16(workspace_or_null)) return SLOPE_ERR_ALIGN;
  }
  if (T == 0 || N == 0) return SLOPE_OK;
  hipStream_t s = (hipStream_t)stream;
  slope::LowrankWs w;
  if (adapter) {
    w = slope::lowrank_layout((Dt)in_dt, workspace_or_null, T, K, r, N);
    hipError_t e = slope::launch_lowrank_prepare((Dt)in_dt, X, L_or_null, R_or_null, T, K, r, N, w, s);
    if (e != hipSuccess) return SLOPE_ERR_HIP;
  }
  return from_hip(slope::launch_spmm((Dt)in_dt, (Dt)out_dt, X, T, K, values_s, meta_s, N, adapter ? &w : nullptr,
                                     adapter ? r : 0, R_or_null, Y, s));
}

slope_status slope_spmm_bwd_dx(slope_dtype in_dt, slope_dtype out_dt, const void* dY, int64_t T, int64_t N,
                               const void* values_dpT, const uint32_t* meta_dpT, int64_t K, void* dX,
                               void* stream) {
  SLOPE_TRY(check_io(in_dt, out_dt));
  if (T < 0 || K < 0 || N < 0) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(dY, true));
  SLOPE_TRY(ptr(values_dpT, true));
  SLOPE_TRY(ptr(meta_dpT, true));
  SLOPE_TRY(ptr(dX, true));
  if (N % 4) return SLOPE_ERR_SHAPE;
  if (!in_range(T) || !in_range(K) || !in_range(N)) return SLOPE_ERR_UNSUPPORTED;
  if (T == 0 || K == 0) return SLOPE_OK;
  // dX^T = W_dpT . dY^T: the forward kernel with reduction N and output rows K
  return from_hip(slope::launch_spmm((Dt)in_dt, (Dt)out_dt, dY, T, N, values_dpT, meta_dpT, K, nullptr, 0, nullptr,
                                     dX, (hipStream_t)stream));
}

slope_status slope_wgrad_workspace_bytes(int64_t T, int64_t N, int64_t K, int64_t* bytes) {
  if (!bytes || T < 0 || K < 0 || N < 0) return SLOPE_ERR_INVALID_ARG;
  if (!in_range(T) || !in_range(K) || !in_range(N)) return SLOPE_ERR_UNSUPPORTED;
  *bytes = slope::wgrad_workspace_bytes(T, N, K);
  return SLOPE_OK;
}

slope_status slope_masked_wgrad(slope_dtype in_dt, slope_dtype out_dt, const void* dY, const void* X, int64_t T,
                                int64_t N, int64_t K, const uint32_t* meta_s, void* dW_values,
                                void* dW_dense_or_null, int accumulate, void* workspace_or_null,
                                int64_t workspace_bytes, void* stream) {
  SLOPE_TRY(check_io(in_dt, out_dt));
  if (T < 0 || K < 0 || N < 0 || workspace_bytes < 0) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(dY, true));
  SLOPE_TRY(ptr(X, true));
  SLOPE_TRY(ptr(meta_s, true));
  SLOPE_TRY(ptr(dW_values, true));
  SLOPE_TRY(ptr(dW_dense_or_null, false));
  SLOPE_TRY(ptr(workspace_or_null, false));
  if (K % 4) return SLOPE_ERR_SHAPE;
  if (!in_range(T) || !in_range(K) || !in_range(N)) return SLOPE_ERR_UNSUPPORTED;
  if (workspace_or_null && workspace_bytes < slope::wgrad_workspace_bytes(T, N, K)) return SLOPE_ERR_WORKSPACE;
  if (N == 0 || K == 0) return SLOPE_OK;
  return from_hip(slope::launch_masked_wgrad((Dt)in_dt, (Dt)out_dt, dY, X, T, N, K, meta_s, dW_values,
                                             dW_dense_or_null, accumulate, workspace_or_null,
                                             (hipStream_t)stream));
}

slope_status slope_packed_sparse_bytes(int64_t rows, int64_t cols, int64_t* bytes) {
  if (!bytes || rows < 0 || cols < 0) return SLOPE_ERR_INVALID_ARG;
  if (cols % 16) return SLOPE_ERR_SHAPE;
  if (!in_range(rows) || cols > kPackedMaxCols) return SLOPE_ERR_UNSUPPORTED;
  *bytes = slope::packed_sparse_bytes(rows, cols);
  return SLOPE_OK;
}

slope_status slope_pack_sparse(slope_dtype dt, const void* values, const uint32_t* meta, int64_t rows, int64_t cols,
                               void* packed, int64_t packed_bytes, void* stream) {
  if (!dt_ok(dt) || rows < 0 || cols < 0 || packed_bytes < 0) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(values, true));
  SLOPE_TRY(ptr(meta, true));
  SLOPE_TRY(ptr(packed, true));
  if (dt == SLOPE_F32) return SLOPE_ERR_UNSUPPORTED;   // 16-bit values only
  if (cols % 16) return SLOPE_ERR_SHAPE;
  if (!in_range(rows) || cols > kPackedMaxCols) return SLOPE_ERR_UNSUPPORTED;
  if (packed_bytes < slope::packed_sparse_bytes(rows, cols)) return SLOPE_ERR_WORKSPACE;
  return from_hip(slope::launch_pack_sparse(values, meta, rows, cols, packed, (hipStream_t)stream));
}

namespace {
// The packed products, with an optional output of the dense operand's token
// chunks (tok == nullptr: none).
slope_status fwd_packed(slope_dtype in_dt, slope_dtype out_dt, const void* X, int64_t T, int64_t K,
                        const void* packed_s, int64_t packed_s_bytes, int64_t N, const void* L_or_null,
                        const void* R_or_null, int64_t r, void* workspace_or_null, int64_t workspace_bytes, void* Y,
                        void* tok, int64_t tok_bytes, void* stream) {
  SLOPE_TRY(check_io(in_dt, out_dt));
  if (T < 0 || K < 0 || N < 0 || r < 0 || packed_s_bytes < 0 || workspace_bytes < 0 || tok_bytes < 0)
    return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(X, true));
  SLOPE_TRY(ptr(packed_s, true));
  SLOPE_TRY(ptr(Y, true));
  SLOPE_TRY(ptr(tok, false));
  bool adapter = false;
  SLOPE_TRY(adapter_args(L_or_null, R_or_null, r, &adapter));
  if (in_dt == SLOPE_F32) return SLOPE_ERR_UNSUPPORTED;
  if (K % 16 || N % 4) return SLOPE_ERR_SHAPE;
  if (!in_range(T) || !in_range(N) || K > kPackedMaxCols || r > kPackedMaxRank) return SLOPE_ERR_UNSUPPORTED;
  if (packed_s_bytes < slope::packed_sparse_bytes(N, K)) return SLOPE_ERR_WORKSPACE;
  if (tok && tok_bytes < slope::packed_tokens_bytes(T, K)) return SLOPE_ERR_WORKSPACE;
  if (adapter) {
    const int64_t need = workspace_need(T, K, r, N);
    if (need > 0 && (!workspace_or_null || workspace_bytes < need)) return SLOPE_ERR_WORKSPACE;
    if (workspace_or_null && !aligned16(workspace_or_null)) return SLOPE_ERR_ALIGN;
  }
  hipStream_t s = (hipStream_t)stream;
  // no output rows: the token chunks (if asked for) come from the packing pass
  if (T == 0 || N == 0) return tok && T > 0 && K > 0 ? from_hip(slope::launch_pack_tokens(X, T, K, tok, s)) : SLOPE_OK;
  slope::LowrankWs w;
  if (adapter) {
    w = slope::lowrank_layout((Dt)in_dt, workspace_or_null, T, K, r, N);
    hipError_t e = slope::launch_lowrank_prepare((Dt)in_dt, X, L_or_null, R_or_null, T, K, r, N, w, s);
    if (e != hipSuccess) return SLOPE_ERR_HIP;
  }
  return from_hip(slope::launch_spmm_packed((Dt)in_dt, (Dt)out_dt, X, T, K, packed_s, N, adapter ? &w : nullptr, Y,
                                            tok, s));
}
}  // namespace

slope_status slope_decode_workspace_bytes(int64_t T, int64_t K, int64_t r, int64_t N, int64_t* bytes) {
  if (!bytes || T < 0 || K < 0 || r < 0 || N < 0) return SLOPE_ERR_INVALID_ARG;
  if (T > kDecodeMaxTokens || !in_range(K) || !in_range(N) || r > kPackedMaxRank) return SLOPE_ERR_UNSUPPORTED;
  *bytes = slope::decode_workspace_bytes(T, K, r, N);
  return SLOPE_OK;
}

slope_status slope_spmm_fwd_decode(slope_dtype in_dt, slope_dtype out_dt, const void* X, int64_t T, int64_t K,
                                   const void* packed_s, int64_t packed_s_bytes, int64_t N, const void* L_or_null,
                                   const void* R_or_null, int64_t r, void* workspace, int64_t workspace_bytes, void* Y,
                                   void* stream) {
  SLOPE_TRY(check_io(in_dt, out_dt));
  if (T < 0 || K < 0 || N < 0 || r < 0 || packed_s_bytes < 0 || workspace_bytes < 0) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(X, true));
  SLOPE_TRY(ptr(packed_s, true));
  SLOPE_TRY(ptr(Y, true));
  SLOPE_TRY(ptr(workspace, false));
  bool adapter = false;
  SLOPE_TRY(adapter_args(L_or_null, R_or_null, r, &adapter));
  if (in_dt == SLOPE_F32) return SLOPE_ERR_UNSUPPORTED;
  if (K % 16 || N % 4) return SLOPE_ERR_SHAPE;
  if (T > kDecodeMaxTokens || !in_range(N) || K > kPackedMaxCols || r > kPackedMaxRank) return SLOPE_ERR_UNSUPPORTED;
  if (packed_s_bytes < slope::packed_sparse_bytes(N, K)) return SLOPE_ERR_WORKSPACE;
  const int64_t need = slope::decode_workspace_bytes(T, K, adapter ? r : 0, N);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SLOPE_ERR_WORKSPACE;
  if (T == 0 || N == 0) return SLOPE_OK;
  return from_hip(slope::launch_spmm_decode((Dt)in_dt, (Dt)out_dt, X, T, K, packed_s, N, L_or_null, R_or_null, adapter ? r : 0,
                                            workspace, Y, (hipStream_t)stream));
}

slope_status slope_spmm_fwd_decode_noalloc(slope_dtype in_dt, slope_dtype out_dt, const void* X, int64_t T,
                                           int64_t K, const void* packed_s, int64_t packed_s_bytes, int64_t N,
                                           const void* L_or_null, const void* R_or_null, int64_t r, void* Y,
                                           void* stream) {
  SLOPE_TRY(check_io(in_dt, out_dt));
  if (T < 0 || K < 0 || N < 0 || r < 0 || packed_s_bytes < 0) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(X, true));
  SLOPE_TRY(ptr(packed_s, true));
  SLOPE_TRY(ptr(Y, true));
  bool adapter = false;
  SLOPE_TRY(adapter_args(L_or_null, R_or_null, r, &adapter));
  if (in_dt == SLOPE_F32) return SLOPE_ERR_UNSUPPORTED;
  if (K % 16 || N % 4) return SLOPE_ERR_SHAPE;
  if (T > kDecodeMaxTokens || !in_range(N) || K > kPackedMaxCols || r > kPackedMaxRank) return SLOPE_ERR_UNSUPPORTED;
  if (packed_s_bytes < slope::packed_sparse_bytes(N, K)) return SLOPE_ERR_WORKSPACE;
  // the call's scratch must fit the library's static array
  if (slope::decode_workspace_bytes(T, K, adapter ? r : 0, N) > slope::kDecodeScratchBytes)
    return SLOPE_ERR_UNSUPPORTED;
  if (T == 0 || N == 0) return SLOPE_OK;
  void* scratch = nullptr;
  hipError_t e = slope::decode_scratch_address(&scratch);
  if (e != hipSuccess) return SLOPE_ERR_HIP;
  return from_hip(slope::launch_spmm_decode((Dt)in_dt, (Dt)out_dt, X, T, K, packed_s, N, L_or_null, R_or_null,
                                            adapter ? r : 0, scratch, Y, (hipStream_t)stream));
}

namespace {
slope_status dx_packed(slope_dtype in_dt, slope_dtype out_dt, const void* dY, int64_t T, int64_t N,
                       const void* packed_dpT, int64_t packed_dpT_bytes, int64_t K, const void* L_or_null,
                       const void* R_or_null, int64_t r, void* workspace_or_null, int64_t workspace_bytes, void* dX,
                       void* tok, int64_t tok_bytes, void* stream) {
  SLOPE_TRY(check_io(in_dt, out_dt));
  if (T < 0 || K < 0 || N < 0 || r < 0 || packed_dpT_bytes < 0 || workspace_bytes < 0 || tok_bytes < 0)
    return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(dY, true));
  SLOPE_TRY(ptr(packed_dpT, true));
  SLOPE_TRY(ptr(dX, true));
  SLOPE_TRY(ptr(tok, false));
  bool adapter = false;
  SLOPE_TRY(adapter_args(L_or_null, R_or_null, r, &adapter));
  if (in_dt == SLOPE_F32) return SLOPE_ERR_UNSUPPORTED;
  if (N % 16 || K % 4) return SLOPE_ERR_SHAPE;
  if (!in_range(T) || !in_range(K) || N > kPackedMaxCols || r > kPackedMaxRank) return SLOPE_ERR_UNSUPPORTED;
  if (packed_dpT_bytes < slope::packed_sparse_bytes(K, N)) return SLOPE_ERR_WORKSPACE;
  if (tok && tok_bytes < slope::packed_tokens_bytes(T, N)) return SLOPE_ERR_WORKSPACE;
  if (adapter) {
    // the forward's adapter workspace with the roles of K and N exchanged
    const int64_t need = workspace_need(T, N, r, K);
    if (need > 0 && (!workspace_or_null || workspace_bytes < need)) return SLOPE_ERR_WORKSPACE;
    if (workspace_or_null && !aligned16(workspace_or_null)) return SLOPE_ERR_ALIGN;
  }
  hipStream_t s = (hipStream_t)stream;
  if (T == 0 || K == 0) return tok && T > 0 && N > 0 ? from_hip(slope::launch_pack_tokens(dY, T, N, tok, s)) : SLOPE_OK;
  slope::LowrankWs w;
  if (adapter) {
    w = slope::lowrank_layout((Dt)in_dt, workspace_or_null, T, N, r, K);
    hipError_t e = slope::launch_lowrank_prepare_bwd(dY, L_or_null, R_or_null, T, N, r, K, w, s);
    if (e != hipSuccess) return SLOPE_ERR_HIP;
  }
  return from_hip(slope::launch_spmm_packed((Dt)in_dt, (Dt)out_dt, dY, T, N, packed_dpT, K, adapter ? &w : nullptr,
                                            dX, tok, s));
}
}  // namespace

slope_status slope_spmm_fwd_packed(slope_dtype in_dt, slope_dtype out_dt, const void* X, int64_t T, int64_t K,
                                   const void* packed_s, int64_t packed_s_bytes, int64_t N, const void* L_or_null,
                                   const void* R_or_null, int64_t r, void* workspace_or_null, int64_t workspace_bytes,
                                   void* Y, void* stream) {
  return fwd_packed(in_dt, out_dt, X, T, K, packed_s, packed_s_bytes, N, L_or_null, R_or_null, r, workspace_or_null,
                    workspace_bytes, Y, nullptr, 0, stream);
}

slope_status slope_spmm_fwd_packed_tokens(slope_dtype in_dt, slope_dtype out_dt, const void* X, int64_t T, int64_t K,
                                          const void* packed_s, int64_t packed_s_bytes, int64_t N,
                                          const void* L_or_null, const void* R_or_null, int64_t r,
                                          void* workspace_or_null, int64_t workspace_bytes, void* Y, void* X_packed,
                                          int64_t X_packed_bytes, void* stream) {
  SLOPE_TRY(ptr(X_packed, true));
  return fwd_packed(in_dt, out_dt, X, T, K, packed_s, packed_s_bytes, N, L_or_null, R_or_null, r, workspace_or_null,
                    workspace_bytes, Y, X_packed, X_packed_bytes, stream);
}

slope_status slope_spmm_bwd_dx_packed(slope_dtype in_dt, slope_dtype out_dt, const void* dY, int64_t T, int64_t N,
                                      const void* packed_dpT, int64_t packed_dpT_bytes, int64_t K,
                                      const void* L_or_null, const void* R_or_null, int64_t r,
                                      void* workspace_or_null, int64_t workspace_bytes, void* dX, void* stream) {
  return dx_packed(in_dt, out_dt, dY, T, N, packed_dpT, packed_dpT_bytes, K, L_or_null, R_or_null, r,
                   workspace_or_null, workspace_bytes, dX, nullptr, 0, stream);
}

slope_status slope_spmm_bwd_dx_packed_tokens(slope_dtype in_dt, slope_dtype out_dt, const void* dY, int64_t T,
                                             int64_t N, const void* packed_dpT, int64_t packed_dpT_bytes, int64_t K,
                                             const void* L_or_null, const void* R_or_null, int64_t r,
                                             void* workspace_or_null, int64_t workspace_bytes, void* dX,
                                             void* dY_packed, int64_t dY_packed_bytes, void* stream) {
  SLOPE_TRY(ptr(dY_packed, true));
  return dx_packed(in_dt, out_dt, dY, T, N, packed_dpT, packed_dpT_bytes, K, L_or_null, R_or_null, r,
                   workspace_or_null, workspace_bytes, dX, dY_packed, dY_packed_bytes, stream);
}

namespace {
// Workspace of slope_lowrank_grads_packed: the forward adapter layout (X . L),
// the backward one (dY . R^T), both hi/lo pairs transposed, the two partial sums.
struct GradsWs {
  int64_t fwd, bwd, trans, part_r, part_l, total;
};
GradsWs grads_ws(int64_t T, int64_t K, int64_t r, int64_t N) {
  GradsWs g{};
  g.fwd = workspace_need(T, K, r, N);
  g.bwd = workspace_need(T, N, r, K);
  const int64_t Tpad = (T + 255) / 256 * 256, r32 = (r + 31) / 32 * 32;
  g.trans = (r32 * Tpad * 2 + 255) / 256 * 256;
  g.part_r = slope::lr_wgrad_part_bytes(T, N, r);
  g.part_l = slope::lr_wgrad_part_bytes(T, K, r);
  g.total = (T == 0 || r == 0) ? 0 : g.fwd + g.bwd + 4 * g.trans + g.part_r + g.part_l;
  return g;
}
}  // namespace

slope_status slope_lowrank_grads_workspace_bytes(int64_t T, int64_t K, int64_t r, int64_t N, int64_t* bytes) {
  if (!bytes || T < 0 || K < 0 || r < 0 || N < 0) return SLOPE_ERR_INVALID_ARG;
  if (!in_range(T) || !in_range(K) || !in_range(N) || r > kPackedMaxRank) return SLOPE_ERR_UNSUPPORTED;
  *bytes = grads_ws(T, K, r, N).total;
  return SLOPE_OK;
}

slope_status slope_lowrank_grads_packed(slope_dtype in_dt, slope_dtype out_dt, const void* X, const void* dY,
                                        const void* X_packed, int64_t X_packed_bytes, const void* dY_packed,
                                        int64_t dY_packed_bytes, int64_t T, int64_t K, int64_t r, int64_t N,
                                        const void* L, const void* R, const void* fwd_workspace_or_null,
                                        int64_t fwd_workspace_bytes, const void* bwd_workspace_or_null,
                                        int64_t bwd_workspace_bytes, void* workspace, int64_t workspace_bytes,
                                        void* dL, void* dR, int accumulate, void* stream) {
  SLOPE_TRY(check_io(in_dt, out_dt));
  if (T < 0 || K < 0 || N < 0 || r < 0 || workspace_bytes < 0 || X_packed_bytes < 0 || dY_packed_bytes < 0 ||
      fwd_workspace_bytes < 0 || bwd_workspace_bytes < 0)
    return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(X, true));
  SLOPE_TRY(ptr(dY, true));
  SLOPE_TRY(ptr(X_packed, true));
  SLOPE_TRY(ptr(dY_packed, true));
  SLOPE_TRY(ptr(L, true));
  SLOPE_TRY(ptr(R, true));
  SLOPE_TRY(ptr(dL, true));
  SLOPE_TRY(ptr(dR, true));
  SLOPE_TRY(ptr(workspace, false));
  SLOPE_TRY(ptr(fwd_workspace_or_null, false));
  SLOPE_TRY(ptr(bwd_workspace_or_null, false));
  if (in_dt == SLOPE_F32) return SLOPE_ERR_UNSUPPORTED;
  if (K % 8 || N % 8) return SLOPE_ERR_SHAPE;
  if (!in_range(T) || !in_range(K) || !in_range(N) || r > kPackedMaxRank) return SLOPE_ERR_UNSUPPORTED;
  const GradsWs g = grads_ws(T, K, r, N);
  if (g.total > 0 && (!workspace || workspace_bytes < g.total)) return SLOPE_ERR_WORKSPACE;
  // the token chunks and the handed-over adapter workspaces must be laid out
  // for these very sizes: each at least the size its own query reports
  if (r > 0 &&
      (X_packed_bytes < slope::packed_tokens_bytes(T, K) || dY_packed_bytes < slope::packed_tokens_bytes(T, N)))
    return SLOPE_ERR_WORKSPACE;
  if (fwd_workspace_or_null && fwd_workspace_bytes < g.fwd) return SLOPE_ERR_WORKSPACE;
  if (bwd_workspace_or_null && bwd_workspace_bytes < g.bwd) return SLOPE_ERR_WORKSPACE;
  if (r == 0 || K == 0 || N == 0) return SLOPE_OK;
  hipStream_t s = (hipStream_t)stream;
  if (T == 0) {   // empty sums: dL = dR = 0 (or unchanged when accumulating)
    if (accumulate) return SLOPE_OK;
    hipError_t e = slope::launch_fill_zero((Dt)out_dt, dL, K * r, s);
    if (e == hipSuccess) e = slope::launch_fill_zero((Dt)out_dt, dR, r * N, s);
    return from_hip(e);
  }
  char* p = static_cast<char*>(workspace);
  // X . L and dY . R^T: taken from the forward's / the dX product's adapter
  // workspace when the caller hands them over, else computed here
  const bool have_f = fwd_workspace_or_null != nullptr, have_b = bwd_workspace_or_null != nullptr;
  const slope::LowrankWs wf =
      slope::lowrank_layout((Dt)in_dt, have_f ? const_cast<void*>(fwd_workspace_or_null) : (void*)p, T, K, r, N);
  const slope::LowrankWs wb = slope::lowrank_layout(
      (Dt)in_dt, have_b ? const_cast<void*>(bwd_workspace_or_null) : (void*)(p + g.fwd), T, N, r, K);
  uint16_t* xh = reinterpret_cast<uint16_t*>(p + g.fwd + g.bwd);
  uint16_t* xl = reinterpret_cast<uint16_t*>(p + g.fwd + g.bwd + g.trans);
  uint16_t* gh = reinterpret_cast<uint16_t*>(p + g.fwd + g.bwd + 2 * g.trans);
  uint16_t* gl = reinterpret_cast<uint16_t*>(p + g.fwd + g.bwd + 3 * g.trans);
  float* pr = reinterpret_cast<float*>(p + g.fwd + g.bwd + 4 * g.trans);
  float* pl = reinterpret_cast<float*>(p + g.fwd + g.bwd + 4 * g.trans + g.part_r);
  const int64_t r32 = (r + 31) / 32 * 32;
  hipError_t e = hipSuccess;
  if (!have_f) e = slope::launch_lowrank_down((Dt)in_dt, X, L, T, K, r, wf, s);                      // X . L
  if (e == hipSuccess && !have_b) e = slope::launch_lowrank_prepare_bwd(dY, L, R, T, N, r, K, wb, s);  // dY . R^T
  if (e == hipSuccess) e = slope::launch_transpose_hilo2(wf, wb, r32, xh, xl, gh, gl, s);
  if (e == hipSuccess) {
    const slope::LrGrad grad_r{dY_packed, N, xh, xl, wf.Tpad, pr, dR, false};   // dR = (X . L)^T . dY
    const slope::LrGrad grad_l{X_packed, K, gh, gl, wb.Tpad, pl, dL, true};     // dL = X^T . (dY . R^T)
    e = slope::launch_lr_wgrad_pair((Dt)in_dt, (Dt)out_dt, grad_r, grad_l, T, r, accumulate, s);
  }
  return from_hip(e);
}

slope_status slope_packed_tokens_bytes(int64_t T, int64_t C, int64_t* bytes) {
  if (!bytes || T < 0 || C < 0) return SLOPE_ERR_INVALID_ARG;
  if (!in_range(T) || !in_range(C)) return SLOPE_ERR_UNSUPPORTED;
  *bytes = slope::packed_tokens_bytes(T, C);
  return SLOPE_OK;
}

slope_status slope_pack_tokens(slope_dtype dt, const void* M, int64_t T, int64_t C, void* packed,
                               int64_t packed_bytes, void* stream) {
  if (!dt_ok(dt)) return SLOPE_ERR_INVALID_ARG;
  if (T < 0 || C < 0 || packed_bytes < 0) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(M, true));
  SLOPE_TRY(ptr(packed, true));
  if (dt == SLOPE_F32) return SLOPE_ERR_UNSUPPORTED;   // 16-bit values only
  if (C % 8) return SLOPE_ERR_SHAPE;
  if (!in_range(T) || !in_range(C)) return SLOPE_ERR_UNSUPPORTED;
  if (packed_bytes < slope::packed_tokens_bytes(T, C)) return SLOPE_ERR_WORKSPACE;
  return from_hip(slope::launch_pack_tokens(M, T, C, packed, (hipStream_t)stream));
}

slope_status slope_wgrad_split_workspace_bytes(int64_t T, int64_t N, int64_t K, int64_t* bytes) {
  if (!bytes || T < 0 || K < 0 || N < 0) return SLOPE_ERR_INVALID_ARG;
  if (!in_range(T) || !in_range(K) || !in_range(N)) return SLOPE_ERR_UNSUPPORTED;
  *bytes = slope::wgrad_split_bytes(T, N, K);
  return SLOPE_OK;
}

slope_status slope_masked_wgrad_packed(slope_dtype in_dt, slope_dtype out_dt, const void* dY_packed,
                                       int64_t dY_packed_bytes, const void* X_packed, int64_t X_packed_bytes,
                                       int64_t T, int64_t N, int64_t K, const uint32_t* meta_s, void* dW_values,
                                       void* dW_dense_or_null, int accumulate, void* split_workspace_or_null,
                                       int64_t split_workspace_bytes, void* stream) {
  SLOPE_TRY(check_io(in_dt, out_dt));
  if (T < 0 || K < 0 || N < 0 || dY_packed_bytes < 0 || X_packed_bytes < 0 || split_workspace_bytes < 0)
    return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(split_workspace_or_null, false));
  SLOPE_TRY(ptr(dY_packed, true));
  SLOPE_TRY(ptr(X_packed, true));
  SLOPE_TRY(ptr(meta_s, true));
  SLOPE_TRY(ptr(dW_values, true));
  SLOPE_TRY(ptr(dW_dense_or_null, false));
  if (in_dt == SLOPE_F32) return SLOPE_ERR_UNSUPPORTED;
  if (K % 8 || N % 8) return SLOPE_ERR_SHAPE;
  if (!in_range(T) || !in_range(K) || !in_range(N)) return SLOPE_ERR_UNSUPPORTED;
  if (dY_packed_bytes < slope::packed_tokens_bytes(T, N) || X_packed_bytes < slope::packed_tokens_bytes(T, K))
    return SLOPE_ERR_WORKSPACE;
  // the token split runs only when a split workspace is given and the shape needs one
  const int64_t split_need = split_workspace_or_null ? slope::wgrad_split_bytes(T, N, K) : 0;
  if (split_need > 0 && split_workspace_bytes < split_need) return SLOPE_ERR_WORKSPACE;
  if (N == 0 || K == 0) return SLOPE_OK;
  return from_hip(slope::launch_masked_wgrad_packed((Dt)in_dt, (Dt)out_dt, dY_packed, X_packed, T, N, K, meta_s,
                                                    dW_values, dW_dense_or_null, accumulate,
                                                    split_need > 0 ? split_workspace_or_null : nullptr,
                                                    (hipStream_t)stream));
}

slope_status slope_lowrank_add(slope_dtype in_dt, slope_dtype out_dt, const void* X, const void* L, const void* R,
                               int64_t T, int64_t K, int64_t r, int64_t N, void* workspace,
                               int64_t workspace_bytes, void* Y, void* stream) {
  SLOPE_TRY(check_io(in_dt, out_dt));
  if (T < 0 || K < 0 || N < 0 || r < 0) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(X, true));
  SLOPE_TRY(ptr(L, true));
  SLOPE_TRY(ptr(R, true));
  SLOPE_TRY(ptr(Y, true));
  if (!in_range(T) || !in_range(K) || !in_range(N) || !in_range(r)) return SLOPE_ERR_UNSUPPORTED;
  const int64_t need = workspace_need(T, K, r, N);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SLOPE_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return SLOPE_ERR_ALIGN;
  if (T == 0 || N == 0 || r == 0) return SLOPE_OK;
  hipStream_t s = (hipStream_t)stream;
  const slope::LowrankWs w = slope::lowrank_layout((Dt)in_dt, workspace, T, K, r, N);
  hipError_t e = slope::launch_lowrank_prepare((Dt)in_dt, X, L, R, T, K, r, N, w, s);
  if (e != hipSuccess) return SLOPE_ERR_HIP;
  return from_hip(slope::launch_lowrank_up_add((Dt)in_dt, (Dt)out_dt, w, R, T, r, N, Y, s));
}

slope_status slope_adamw(slope_dtype param_dt, slope_dtype grad_dt, void* params, const void* grads, float* m,
                         float* v, int64_t n, const slope_adamw_params* hp, void* stream) {
  if (!dt_ok(param_dt) || !dt_ok(grad_dt) || n < 0) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(params, true));
  SLOPE_TRY(ptr(grads, true));
  SLOPE_TRY(ptr(m, true));
  SLOPE_TRY(ptr(v, true));
  slope::AdamWStep c;
  SLOPE_TRY(adamw_step(hp, &c));
  if (n > kAdamwMaxElems) return SLOPE_ERR_UNSUPPORTED;
  return from_hip(slope::launch_adamw((Dt)param_dt, (Dt)grad_dt, params, grads, m, v, n, c, (hipStream_t)stream));
}

slope_status slope_adamw_double_prune(slope_dtype dt, slope_dtype grad_dt, void* values_s, const uint32_t* meta_s,
                                      const void* dW_values, float* m, float* v, int64_t N, int64_t K,
                                      const slope_adamw_params* hp, void* values_dpT, uint32_t* meta_dpT,
                                      uint8_t* mask_dpT_or_null, void* stream) {
  if (!dt_ok(dt) || !dt_ok(grad_dt) || N < 0 || K < 0) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(values_s, true));
  SLOPE_TRY(ptr(meta_s, true));
  SLOPE_TRY(ptr(dW_values, true));
  SLOPE_TRY(ptr(m, true));
  SLOPE_TRY(ptr(v, true));
  SLOPE_TRY(ptr(values_dpT, true));
  SLOPE_TRY(ptr(meta_dpT, true));
  SLOPE_TRY(ptr(mask_dpT_or_null, false));
  slope::AdamWStep c;
  SLOPE_TRY(adamw_step(hp, &c));
  if (N % 4 || K % 4) return SLOPE_ERR_SHAPE;
  if (!in_range(N) || !in_range(K)) return SLOPE_ERR_UNSUPPORTED;
  return from_hip(slope::launch_adamw_double_prune((Dt)dt, (Dt)grad_dt, values_s, meta_s, dW_values, m, v, N, K, c,
                                                   values_dpT, meta_dpT, mask_dpT_or_null, (hipStream_t)stream));
}

slope_status slope_double_prune_packed(slope_dtype dt, const void* values_s, const uint32_t* meta_s, int64_t N,
                                       int64_t K, void* packed_dpT, int64_t packed_dpT_bytes, void* stream) {
  if (!dt_ok(dt) || N < 0 || K < 0 || packed_dpT_bytes < 0) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(values_s, true));
  SLOPE_TRY(ptr(meta_s, true));
  SLOPE_TRY(ptr(packed_dpT, true));
  if (dt == SLOPE_F32) return SLOPE_ERR_UNSUPPORTED;   // 16-bit values only
  if (N % 16 || K % 16) return SLOPE_ERR_SHAPE;
  if (!in_range(K) || N > kPackedMaxCols) return SLOPE_ERR_UNSUPPORTED;
  if (packed_dpT_bytes < slope::packed_sparse_bytes(K, N)) return SLOPE_ERR_WORKSPACE;
  return from_hip(slope::launch_double_prune_packed((Dt)dt, values_s, meta_s, N, K, packed_dpT, (hipStream_t)stream));
}

slope_status slope_adamw_double_prune_packed(slope_dtype dt, slope_dtype grad_dt, void* values_s,
                                             const uint32_t* meta_s, const void* dW_values, float* m, float* v,
                                             int64_t N, int64_t K, const slope_adamw_params* hp, void* packed_s,
                                             int64_t packed_s_bytes, void* packed_dpT, int64_t packed_dpT_bytes,
                                             void* stream) {
  if (!dt_ok(dt) || !dt_ok(grad_dt) || N < 0 || K < 0 || packed_s_bytes < 0 || packed_dpT_bytes < 0)
    return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(values_s, true));
  SLOPE_TRY(ptr(meta_s, true));
  SLOPE_TRY(ptr(dW_values, true));
  SLOPE_TRY(ptr(m, true));
  SLOPE_TRY(ptr(v, true));
  SLOPE_TRY(ptr(packed_s, true));
  SLOPE_TRY(ptr(packed_dpT, true));
  slope::AdamWStep c;
  SLOPE_TRY(adamw_step(hp, &c));
  if (dt == SLOPE_F32) return SLOPE_ERR_UNSUPPORTED;   // 16-bit values only
  if (N % 16 || K % 16) return SLOPE_ERR_SHAPE;
  if (K > kPackedMaxCols || N > kPackedMaxCols) return SLOPE_ERR_UNSUPPORTED;
  if (packed_s_bytes < slope::packed_sparse_bytes(N, K) || packed_dpT_bytes < slope::packed_sparse_bytes(K, N))
    return SLOPE_ERR_WORKSPACE;
  return from_hip(slope::launch_adamw_double_prune_packed((Dt)dt, (Dt)grad_dt, values_s, meta_s, dW_values, m, v, N,
                                                          K, c, packed_s, packed_dpT, (hipStream_t)stream));
}

// ---------------------------------------------------------------- 8-bit (E4M3) variant

slope_status slope_quantize_e4m3(slope_dtype dt, const void* M, int64_t n, float* scale, uint8_t* q, void* stream) {
  if ((dt != SLOPE_BF16 && dt != SLOPE_F16) || n < 0) return dt == SLOPE_F32 ? SLOPE_ERR_UNSUPPORTED : SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(M, true));
  SLOPE_TRY(ptr(q, true));
  if (!scale) return SLOPE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(scale) & 3u) return SLOPE_ERR_ALIGN;
  if (n > kAdamwMaxElems) return SLOPE_ERR_UNSUPPORTED;
  return from_hip(slope::launch_quantize_e4m3((Dt)dt, M, n, scale, q, (hipStream_t)stream));
}

slope_status slope_packed_sparse_e4m3_bytes(int64_t rows, int64_t cols, int64_t* bytes) {
  if (!bytes || rows < 0 || cols < 0) return SLOPE_ERR_INVALID_ARG;
  if (cols % 16) return SLOPE_ERR_SHAPE;
  if (!in_range(rows) || cols > kPackedMaxCols) return SLOPE_ERR_UNSUPPORTED;
  *bytes = slope::packed_sparse_e4m3_bytes(rows, cols);
  return SLOPE_OK;
}

slope_status slope_pack_sparse_e4m3(slope_dtype dt, const void* values, const uint32_t* meta, int64_t rows,
                                    int64_t cols, float* scale, void* packed, int64_t packed_bytes, void* stream) {
  if (!dt_ok(dt) || rows < 0 || cols < 0 || packed_bytes < 0) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(values, true));
  SLOPE_TRY(ptr(meta, true));
  SLOPE_TRY(ptr(packed, true));
  if (!scale) return SLOPE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(scale) & 3u) return SLOPE_ERR_ALIGN;
  if (dt == SLOPE_F32) return SLOPE_ERR_UNSUPPORTED;   // codes come from 16-bit values
  if (cols % 16) return SLOPE_ERR_SHAPE;
  if (!in_range(rows) || cols > kPackedMaxCols) return SLOPE_ERR_UNSUPPORTED;
  if (packed_bytes < slope::packed_sparse_e4m3_bytes(rows, cols)) return SLOPE_ERR_WORKSPACE;
  return from_hip(slope::launch_pack_sparse_e4m3((Dt)dt, values, meta, rows, cols, scale, packed, (hipStream_t)stream));
}

slope_status slope_spmm_e4m3_packed(slope_dtype out_dt, const uint8_t* Xq, const float* x_scale, int64_t T, int64_t K,
                                    const void* packed_w, int64_t packed_w_bytes, const float* w_scale, int64_t N,
                                    void* Y, void* stream) {
  if (!dt_ok(out_dt) || T < 0 || K < 0 || N < 0 || packed_w_bytes < 0) return SLOPE_ERR_INVALID_ARG;
  SLOPE_TRY(ptr(Xq, true));
  SLOPE_TRY(ptr(packed_w, true));
  SLOPE_TRY(ptr(Y, true));
  if (!x_scale || !w_scale) return SLOPE_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(x_scale) & 3u) || (reinterpret_cast<uintptr_t>(w_scale) & 3u)) return SLOPE_ERR_ALIGN;
  if (out_dt == SLOPE_F16) return SLOPE_ERR_UNSUPPORTED;   // bf16 or fp32 outputs
  if (K % 16 || N % 4) return SLOPE_ERR_SHAPE;
  if (!in_range(T) || !in_range(N) || K > kPackedMaxCols) return SLOPE_ERR_UNSUPPORTED;
  if (packed_w_bytes < slope::packed_sparse_e4m3_bytes(N, K)) return SLOPE_ERR_WORKSPACE;
  if (T == 0 || N == 0) return SLOPE_OK;
  return from_hip(slope::launch_spmm_e4m3((Dt)out_dt, Xq, x_scale, T, K, packed_w, w_scale, N, Y,
                                          (hipStream_t)stream));
}

}  // extern "C"

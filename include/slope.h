/*
 * slope.h - C ABI of the SLoPe 2:4 sparse linear layer for AMD MI355X (gfx950).
 *
 * The operations are those of "SLoPe: Double-Pruned Sparse Plus Lazy Low-Rank
 * Adapter Pretraining of LLMs" as described on its summary page (atlas.scime.ai,
 * sections Problem and Approach), its technical explainer (gist.science,
 * Technical Summary sections 2.A Double-Pruned Backward Pass, 2.B Lazy Low-Rank
 * Adapters, 2.C Optimized CUDA Kernels) and its OpenReview discussion
 * (paperhub.cn, sections "Memory Footprint Reduction During Pretraining and
 * Inference" and "Clarification on Inference Speedup and Sparse Pre-Training").
 *
 * Notation.  A linear layer has weight W [N, K] = [out, in] (row-major, as in
 * nn.Linear), input X [T, K], output Y [T, N] and output gradient dY [T, N].
 *   W_s   = W pruned 2:4 along K (two of every four consecutive inputs kept)
 *   W_dp  = the transpose of W_dpT = prune24(W_s^T): pruned 2:4 along N
 *   Y     = X . W_s^T (+ (X . L) . R),  L [K, r], R [r, N]
 *   dX    = dY . W_dp
 *   dW    = (dY^T . X) kept at W_s's mask
 *
 * Data types.  SLOPE_BF16 tensors hold raw bfloat16 values, SLOPE_F16 raw
 * IEEE binary16 values, SLOPE_F32 raw float32 values.  Products accumulate in
 * float32; 16-bit outputs are rounded to nearest even once, at the end.  A
 * call's outputs are in its input format or float32 (an F32-input call uses
 * F32 outputs).  The tile-chunk, token-chunk and few-token entry points take
 * the two 16-bit formats; the fp16 adapter keeps X . L as an fp16 hi/lo pair,
 * so |X . L| must stay below the fp16 range (65504).
 *
 * Selection rule (prune24, double_prune): within a group of four, the two
 * largest magnitudes are kept; equal magnitudes (including +0/-0 and x/-x) go
 * to the lower position; NaN ranks above every number and NaNs tie.  Pruned
 * entries become +0.  The pages fix 2:4 but not the score; magnitude and this
 * tie rule are the library's reading.
 *
 * Compressed 2:4 format of a [rows, cols] matrix (cols % 4 == 0):
 *   values [rows, cols/2]       the two kept values of every group, in
 *                               ascending position order, same dtype as input
 *   meta   [rows, ceil(cols/32)] uint32; group g of a row has nibble
 *                               i0 | i1 << 2 (its kept positions, i0 < i1) at
 *                               bits 4*(g%8) of word g/8; unused high nibbles
 *                               of a row's last word are 0
 * (two 16-bit values plus index bits per four weights: the discussion page's
 * memory accounting; the page counts 3 index bits, this format stores 4.)
 *
 * Memory and execution.  Every pointer argument is device memory owned by the
 * caller, contiguous row-major, 16-byte aligned; nothing is retained after a
 * call returns.  `stream` is a hipStream_t (NULL = the null stream).  Calls
 * only enqueue work and return without synchronising.  Arguments are checked
 * before anything is enqueued; on an error nothing is written and no kernel is
 * launched.  SLOPE_ERR_HIP reports a failed launch (hipGetLastError).  Calls
 * that overlap on one stream are ordered; the library keeps no state between
 * calls and is safe to call from several host threads.  Every buffer whose
 * layout depends on the sizes of a call (workspaces, tile and token chunks)
 * comes with its byte count, checked against the matching size query.
 *
 * Adapter arguments (L_or_null, R_or_null, r): both factors with r > 0 turn
 * the adapter on; both NULL (any r >= 0) turn it off.  Exactly one factor, or
 * factors with r == 0, is SLOPE_ERR_INVALID_ARG.
 *
 * Data checks.  Mask content is validated only where a mask comes from the
 * caller (slope_compress24): groups keeping more than two positions are
 * counted into a caller-owned device counter, read after the stream is
 * synchronised.  No device-side status is kept inside the library.
 */
#ifndef SLOPE_H_
#define SLOPE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SLOPE_F32 = 0, SLOPE_BF16 = 1, SLOPE_F16 = 2 } slope_dtype;

typedef enum {
  SLOPE_OK = 0,
  SLOPE_ERR_INVALID_ARG = -1, /* null pointer, unknown dtype, negative size */
  SLOPE_ERR_SHAPE = -2,       /* a 2:4 dimension not a multiple of 4 (8 where stated) */
  SLOPE_ERR_ALIGN = -3,       /* a pointer not 16-byte aligned */
  SLOPE_ERR_WORKSPACE = -4,   /* workspace or operand buffer missing, or fewer bytes than its size query */
  SLOPE_ERR_HIP = -5,         /* the HIP runtime reported an error */
  SLOPE_ERR_UNSUPPORTED = -6  /* dtype combination or size beyond the limits */
} slope_status;

/* Largest accepted size of any single dimension (rows, cols, T, N, K, r). */
#define SLOPE_MAX_DIM (1 << 22)

/* Library ABI version (major * 100 + minor). */
int slope_version(void);

/* Static text naming a status code (never NULL). */
const char* slope_status_string(int status);

/* Element counts of the compressed form of a [rows, cols] matrix: *n_values =
 * rows*cols/2 values, *n_meta_words = rows*ceil(cols/32) uint32 words.
 * Host-only; SLOPE_ERR_SHAPE if cols % 4 != 0. */
slope_status slope_compressed_sizes(int64_t rows, int64_t cols, int64_t* n_values, int64_t* n_meta_words);

/* Bytes of device workspace the low-rank adapter needs for T tokens, input
 * width K, rank r and output width N: the split partial sums of X . L
 * (float32), X . L as 16-bit hi + lo parts, and transposed copies of L and R.
 * Host-only; 0 when T == 0 or r == 0. */
slope_status slope_lowrank_workspace_bytes(int64_t T, int64_t K, int64_t r, int64_t N, int64_t* bytes);

/* Bytes of device workspace slope_masked_wgrad can use for T tokens, N
 * outputs and K inputs: X and dY rewritten, transposed, into 256-column x
 * 32-token chunks (16-bit, zero padded; see slope_pack_tokens), X's first.
 * Host-only. */
slope_status slope_wgrad_workspace_bytes(int64_t T, int64_t N, int64_t K, int64_t* bytes);

/* Magnitude 2:4 pruning of W [rows, cols] along its rows: the forward weight
 * W^R, pruned along rows (explainer 2.A; N:M = 2:4, summary page Approach).
 * The mask is chosen once, at initialisation, and then kept static (explainer
 * 2.A; summary page Approach).
 *   W         [rows, cols] dt, input
 *   mask      [rows, cols] uint8 output, 1 at kept positions, 0 elsewhere
 *             (one byte per weight, as in the discussion page's accounting)
 *   W_s       [rows, cols] dt output (kept values, +0 elsewhere) or NULL
 * Errors: SLOPE_ERR_SHAPE if cols % 4 != 0. */
slope_status slope_prune24(slope_dtype dt, const void* W, int64_t rows, int64_t cols, uint8_t* mask,
                           void* W_s_or_null, void* stream);

/* Magnitude N:M pruning of W [rows, cols] along its rows: in every group of m
 * consecutive columns the n highest-ranked elements are kept, ranked as in
 * slope_prune24 (n = 2, m = 4 gives slope_prune24's result).  The explainer's
 * Technical Summary 1 (Problem Statement) names N:M structured sparsity in
 * general; its "N zeros out of M" is read as n kept positions out of m.
 * With n <= 2 and m a multiple of four every aligned group of four keeps at
 * most two positions (1:4, 1:8, 2:8, 2:16, 2:32), so slope_compress24 of W_s
 * under this mask feeds the 2:4 products and the double prune unchanged.
 *   W         [rows, cols] dt, input
 *   n, m      m in {4, 8, 16, 32}, 1 <= n <= m
 *   mask      [rows, cols] uint8 output, 1 at kept positions, 0 elsewhere
 *   W_s       [rows, cols] dt output (kept values, +0 elsewhere) or NULL
 * Errors: SLOPE_ERR_UNSUPPORTED for another m; SLOPE_ERR_INVALID_ARG for n
 * outside [1, m]; SLOPE_ERR_SHAPE if cols % m != 0. */
slope_status slope_prune_nm(slope_dtype dt, const void* W, int64_t rows, int64_t cols, int n, int m, uint8_t* mask,
                           void* W_s_or_null, void* stream);

/* slope_prune24 followed by slope_compress24 of its mask, in one pass over W
 * (explainer 2.A: the forward weight pruned 2:4 along its rows, once, at
 * initialisation; discussion page, "Memory Footprint": two 16-bit non-zeros
 * plus their indices per four weights), optionally also writing W_s's
 * tile-chunk form for the *_packed products.
 *   W         [rows, cols] dt, input
 *   mask      [rows, cols] uint8 output as slope_prune24 writes it, or NULL
 *   values    [rows, cols/2] dt output, meta [rows, ceil(cols/32)] uint32 output
 *   packed    NULL, or caller-owned device memory of at least
 *             slope_packed_sparse_bytes(rows, cols) bytes (16-bit dt,
 *             cols % 16 == 0), overwritten with slope_pack_sparse's result
 * Results equal the separate calls, bit for bit.  Errors: SLOPE_ERR_SHAPE if
 * cols % 4 != 0 (cols % 16 != 0 with packed); SLOPE_ERR_UNSUPPORTED for a
 * packed float32 matrix or cols > 2^21 with packed; SLOPE_ERR_WORKSPACE if
 * packed_bytes is short. */
slope_status slope_prune_compress24(slope_dtype dt, const void* W, int64_t rows, int64_t cols, uint8_t* mask_or_null,
                                    void* values, uint32_t* meta, void* packed_or_null, int64_t packed_bytes,
                                    void* stream);

/* Compressed form of W under a mask (discussion page, "Memory Footprint":
 * two 16-bit non-zeros plus their indices per four weights).
 *   W, mask   [rows, cols] inputs (mask byte != 0 = kept)
 *   values    [rows, cols/2] dt output, meta [rows, ceil(cols/32)] uint32 output
 *   invalid   NULL, or a device int32 to which the number of groups whose mask
 *             keeps more than two positions is added (atomically).  Such a
 *             group keeps its two lowest kept positions; a group keeping fewer
 *             than two is filled with its lowest unkept positions and +0.
 * Errors: SLOPE_ERR_SHAPE if cols % 4 != 0. */
slope_status slope_compress24(slope_dtype dt, const void* W, const uint8_t* mask, int64_t rows, int64_t cols,
                              void* values, uint32_t* meta, int32_t* invalid_groups_or_null, void* stream);

/* Double pruning for the backward pass: W_dpT = prune24(W_s^T), the weight
 * W^{R,C} of explainer 2.A (the already 2:4-sparse weight is transposed and
 * pruned 2:4 once more), kept as the compressed transposed copy that the
 * discussion page counts next to the weight.
 * Deterministic; meant to run on every step so the column mask follows W_s.
 *   values_s, meta_s   compressed W_s of [N, K]
 *   values_dpT [K, N/2], meta_dpT [K, ceil(N/32)]  compressed W_dpT [K, N]
 *   mask_dpT   [K, N] uint8 output (1 = kept) or NULL
 * Errors: SLOPE_ERR_SHAPE unless N % 4 == 0 and K % 4 == 0. */
slope_status slope_double_prune(slope_dtype dt, const void* values_s, const uint32_t* meta_s, int64_t N, int64_t K,
                                void* values_dpT, uint32_t* meta_dpT, uint8_t* mask_dpT_or_null, void* stream);

/* Sparse forward with the fused unmerged adapter (explainer 2.A and 2.B; 2.C
 * fuses the sparse product with the low-rank term; discussion page: adapters
 * are not merged into the weights at inference):
 *   Y [T, N] = X [T, K] . W_s^T  (+ (X . L) . R  when L, R != NULL and r > 0)
 *   values_s [N, K/2], meta_s [N, ceil(K/32)]  compressed W_s
 *   L [K, r], R [r, N] in_dt; workspace: device memory of at least
 *   slope_lowrank_workspace_bytes(T, K, r, N) bytes (only used with an adapter;
 *   its contents are scratch, overwritten by every call)
 *   out_dt: dtype of Y (BF16 or F32 for BF16 inputs; F32 for F32 inputs)
 * Y is overwritten.  Errors: SLOPE_ERR_SHAPE if K % 4 != 0;
 * SLOPE_ERR_WORKSPACE if the adapter is on and the workspace is short. */
slope_status slope_spmm_fwd(slope_dtype in_dt, slope_dtype out_dt, const void* X, int64_t T, int64_t K,
                            const void* values_s, const uint32_t* meta_s, int64_t N, const void* L_or_null,
                            const void* R_or_null, int64_t r, void* workspace_or_null, int64_t workspace_bytes,
                            void* Y, void* stream);

/* Double-pruned backward data product (explainer 2.A: the backward pass runs
 * on the double-pruned weight):
 *   dX [T, K] = dY [T, N] . W_dp,  W_dp = transpose of W_dpT [K, N]
 *   values_dpT [K, N/2], meta_dpT [K, ceil(N/32)] from slope_double_prune
 * dX is overwritten.  Errors: SLOPE_ERR_SHAPE if N % 4 != 0. */
slope_status slope_spmm_bwd_dx(slope_dtype in_dt, slope_dtype out_dt, const void* dY, int64_t T, int64_t N,
                               const void* values_dpT, const uint32_t* meta_dpT, int64_t K, void* dX,
                               void* stream);

/* Weight gradient at the static mask (the discussion page counts two 16-bit
 * gradient values per four weights, and fine-tuning updates only the weights
 * that are not pruned):
 *   dW = (dY [T, N])^T . X [T, K], kept at the positions named by meta_s
 *   dW_values [N, K/2] out_dt: values in W_s's slot order (same layout as
 *             values_s)
 *   dW_dense  [N, K] out_dt masked dense copy, or NULL
 *   accumulate != 0: add to the existing contents instead of overwriting
 *   workspace: NULL, or device memory (16-byte aligned) of at least
 *             slope_wgrad_workspace_bytes(T, N, K) bytes, owned by the caller
 *             and overwritten; with it the 16-bit path packs both operands
 *             first and runs faster.  Results are identical either way.
 * Errors: SLOPE_ERR_SHAPE if K % 4 != 0; SLOPE_ERR_WORKSPACE if a workspace
 * is given and is short. */
slope_status slope_masked_wgrad(slope_dtype in_dt, slope_dtype out_dt, const void* dY, const void* X, int64_t T,
                                int64_t N, int64_t K, const uint32_t* meta_s, void* dW_values,
                                void* dW_dense_or_null, int accumulate, void* workspace_or_null,
                                int64_t workspace_bytes, void* stream);

/* Bytes of the tile-chunk form of a compressed 16-bit matrix [rows, cols] (see
 * slope_pack_sparse).  Host-only; SLOPE_ERR_SHAPE if cols % 16 != 0,
 * SLOPE_ERR_UNSUPPORTED if cols > 2^21. */
slope_status slope_packed_sparse_bytes(int64_t rows, int64_t cols, int64_t* bytes);

/* Tile-chunk copy of a compressed 16-bit matrix (values [rows, cols/2],
 * meta [rows, ceil(cols/32)] as written by slope_compress24 or
 * slope_double_prune), the operand format of the *_packed products.  Chunk
 * (t, s) holds rows 256t .. 256t+255 and dense columns 64s .. 64s+63, 18432
 * bytes at offset (t * ceil(cols/64) + s) * 18432: first the 32 values of
 * each row (64 bytes at row*64; the 16-byte granule c of a row sits at
 * c ^ ((row / 4) % 4)), then the row's two metadata words (8 bytes at
 * 16384 + row*8).  Rows past `rows` and columns past `cols` are 0.  packed:
 * caller-owned device memory of slope_packed_sparse_bytes(rows, cols) bytes,
 * overwritten.  Errors: SLOPE_ERR_UNSUPPORTED for float32 or cols > 2^21,
 * SLOPE_ERR_SHAPE if cols % 16 != 0, SLOPE_ERR_WORKSPACE if packed_bytes is
 * short. */
slope_status slope_pack_sparse(slope_dtype dt, const void* values, const uint32_t* meta, int64_t rows, int64_t cols,
                               void* packed, int64_t packed_bytes, void* stream);

/* slope_spmm_fwd with W_s given in tile-chunk form (slope_pack_sparse of
 * values_s, meta_s; rows N, cols K): same result, bitwise.  packed_s_bytes:
 * bytes of packed_s, at least slope_packed_sparse_bytes(N, K).  16-bit inputs
 * only; K % 16 == 0, K <= 2^21, N % 4 == 0, adapter rank r <= 128.  Errors as
 * slope_spmm_fwd, plus SLOPE_ERR_UNSUPPORTED / SLOPE_ERR_SHAPE for the limits
 * above and SLOPE_ERR_WORKSPACE for a short packed_s. */
slope_status slope_spmm_fwd_packed(slope_dtype in_dt, slope_dtype out_dt, const void* X, int64_t T, int64_t K,
                                   const void* packed_s, int64_t packed_s_bytes, int64_t N, const void* L_or_null,
                                   const void* R_or_null, int64_t r, void* workspace_or_null, int64_t workspace_bytes,
                                   void* Y, void* stream);

/* slope_spmm_bwd_dx with W_dpT given in tile-chunk form (slope_pack_sparse of
 * values_dpT, meta_dpT; rows K, cols N): same result, bitwise.  With L [K, r]
 * and R [r, N] (r > 0) it also adds the adapter's share of the input gradient
 * (the derivative of explainer 2.B's term):
 *   dX [T, K] = dY . W_dp (+ (dY . R^T) . L^T)
 * using workspace_or_null of slope_lowrank_workspace_bytes(T, N, r, K) bytes
 * (note the order: the reduction runs over N, the output over K).
 * packed_dpT_bytes: bytes of packed_dpT, at least slope_packed_sparse_bytes(K,
 * N).  16-bit inputs only; N % 16 == 0, N <= 2^21, K % 4 == 0, r <= 128.
 * Errors as slope_spmm_fwd_packed. */
slope_status slope_spmm_bwd_dx_packed(slope_dtype in_dt, slope_dtype out_dt, const void* dY, int64_t T, int64_t N,
                                      const void* packed_dpT, int64_t packed_dpT_bytes, int64_t K,
                                      const void* L_or_null, const void* R_or_null, int64_t r,
                                      void* workspace_or_null, int64_t workspace_bytes, void* dX, void* stream);

/* The two packed products that also write their dense operand as token
 * chunks (the layout of slope_pack_tokens, bitwise the same bytes), so that
 * the weight gradient's operands need no separate packing pass: the product
 * streams X (or dY) through its tiles anyway, and each stage of 64 columns of
 * each 256-token tile is written out once, by one of the blocks that read it.
 * The weight gradient dW = dY^T . X at the kept weights (explainer, Technical
 * Summary 2.A; discussion page, "Memory Footprint Reduction During
 * Pretraining and Inference") reads these chunks.  Arguments as
 * slope_spmm_fwd_packed / slope_spmm_bwd_dx_packed, plus X_packed (dY_packed):
 * caller-owned device memory of at least slope_packed_tokens_bytes(T, K)
 * (slope_packed_tokens_bytes(T, N)) bytes, 16-byte aligned, overwritten.
 * Results Y (dX) are bitwise those of the plain calls.  Errors: those of the
 * plain calls, SLOPE_ERR_INVALID_ARG for a NULL chunk buffer and
 * SLOPE_ERR_WORKSPACE for a short one. */
slope_status slope_spmm_fwd_packed_tokens(slope_dtype in_dt, slope_dtype out_dt, const void* X, int64_t T, int64_t K,
                                          const void* packed_s, int64_t packed_s_bytes, int64_t N,
                                          const void* L_or_null, const void* R_or_null, int64_t r,
                                          void* workspace_or_null, int64_t workspace_bytes, void* Y, void* X_packed,
                                          int64_t X_packed_bytes, void* stream);
slope_status slope_spmm_bwd_dx_packed_tokens(slope_dtype in_dt, slope_dtype out_dt, const void* dY, int64_t T,
                                             int64_t N, const void* packed_dpT, int64_t packed_dpT_bytes, int64_t K,
                                             const void* L_or_null, const void* R_or_null, int64_t r,
                                             void* workspace_or_null, int64_t workspace_bytes, void* dX,
                                             void* dY_packed, int64_t dY_packed_bytes, void* stream);

/* Bytes of device workspace slope_lowrank_grads_packed needs.  Host-only;
 * SLOPE_ERR_UNSUPPORTED if r > 128. */
slope_status slope_lowrank_grads_workspace_bytes(int64_t T, int64_t K, int64_t r, int64_t N, int64_t* bytes);

/* Weight gradients of the adapter term of explainer 2.B (Y += (X . L) . R):
 *   dL [K, r] = X^T . (dY . R^T),   dR [r, N] = (X . L)^T . dY
 * X [T, K], dY [T, N], L, R in_dt (BF16 or F16) row-major; X_packed, dY_packed: the same
 * matrices in token-chunk form (slope_pack_tokens), as the weight gradient
 * uses them, with their byte counts (at least slope_packed_tokens_bytes(T, K)
 * and (T, N)).  fwd_workspace_or_null / bwd_workspace_or_null: the adapter
 * workspaces that slope_spmm_fwd_packed (X, L, R) and slope_spmm_bwd_dx_packed
 * (dY, L, R) filled for these same operands, untouched since (they hold
 * X . L and dY . R^T, which are then not recomputed), with their byte counts
 * (at least slope_lowrank_workspace_bytes(T, K, r, N) and (T, N, r, K)); NULL
 * to compute them here.  A handed-over workspace must have been filled for the
 * same sizes and in_dt: only its size can be checked.  dL, dR in out_dt (in_dt
 * or F32), overwritten, or added to when accumulate != 0.  workspace:
 * slope_lowrank_grads_workspace_bytes(T, K, r, N) bytes, scratch.  Sums over
 * tokens run in a fixed order.  Errors: SLOPE_ERR_SHAPE unless K % 8 == 0 and
 * N % 8 == 0; SLOPE_ERR_UNSUPPORTED for r > 128; SLOPE_ERR_WORKSPACE for any
 * short buffer. */
slope_status slope_lowrank_grads_packed(slope_dtype in_dt, slope_dtype out_dt, const void* X, const void* dY,
                                        const void* X_packed, int64_t X_packed_bytes, const void* dY_packed,
                                        int64_t dY_packed_bytes, int64_t T, int64_t K, int64_t r, int64_t N,
                                        const void* L, const void* R, const void* fwd_workspace_or_null,
                                        int64_t fwd_workspace_bytes, const void* bwd_workspace_or_null,
                                        int64_t bwd_workspace_bytes, void* workspace, int64_t workspace_bytes,
                                        void* dL, void* dR, int accumulate, void* stream);

/* Bytes of device workspace slope_spmm_fwd_decode needs for T <= 64 tokens:
 * fp32 split partial sums, plus, when r > 0, X . L in fp32 as
 * [slices][T][rpad] (rpad = r rounded up to 16; one slice above four tokens,
 * ceil(K / 2048) up to 64 at or below).  Host-only; SLOPE_ERR_UNSUPPORTED if
 * T > 64 or r > 128. */
slope_status slope_decode_workspace_bytes(int64_t T, int64_t K, int64_t r, int64_t N, int64_t* bytes);

/* Few-token forward (T <= 64; the inference case of the discussion page's
 * "SLoPe inference computation": weight kept sparse, adapter unmerged):
 *   Y [T, N] = X [T, K] . W_s^T (+ (X . L) . R)
 * with W_s in tile-chunk form (slope_pack_sparse, rows N, cols K; packed_s_bytes
 * at least slope_packed_sparse_bytes(N, K)).  The compressed weight is
 * streamed once, split along K over enough waves to keep HBM busy; partial
 * sums are added in a fixed order (deterministic).  workspace: caller-owned
 * device memory of slope_decode_workspace_bytes(T, K, r, N) bytes (16-byte
 * aligned; scratch, overwritten).  16-bit inputs only; K % 16 == 0,
 * N % 4 == 0, r <= 128.  Errors: SLOPE_ERR_UNSUPPORTED for T > 64 or the
 * dtype/size limits, SLOPE_ERR_SHAPE, SLOPE_ERR_WORKSPACE. */
slope_status slope_spmm_fwd_decode(slope_dtype in_dt, slope_dtype out_dt, const void* X, int64_t T, int64_t K,
                                   const void* packed_s, int64_t packed_s_bytes, int64_t N, const void* L_or_null,
                                   const void* R_or_null, int64_t r, void* workspace, int64_t workspace_bytes, void* Y,
                                   void* stream);

/* Size of the static device scratch of slope_spmm_fwd_decode_noalloc: 32 MiB
 * on each GPU the library runs on, held until the process ends. */
#define SLOPE_DECODE_NOALLOC_SCRATCH_BYTES (32 << 20)

/* slope_spmm_fwd_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): same arguments except the workspace, same results bit for bit.
 * Its split partial sums and X . L go to a static device array of
 * SLOPE_DECODE_NOALLOC_SCRATCH_BYTES per GPU instead of a caller workspace;
 * the call allocates nothing (no hipMalloc or allocating library routine).
 * It accepts sizes whose slope_decode_workspace_bytes(T, K, r, N) fits that
 * array (at bf16 or fp16: every OPT-66B linear up to T = 16, every OPT-13B
 * linear up to T = 64) and returns SLOPE_ERR_UNSUPPORTED beyond it.  Every
 * call on one GPU uses that GPU's one array, which keeps the last call's
 * contents: calls that overlap on one GPU (several streams or host threads
 * at once) race and must be serialised by the caller; consecutive calls on one
 * stream are ordered and safe.  Errors: those of slope_spmm_fwd_decode, with
 * SLOPE_ERR_UNSUPPORTED for a scratch need above the array's size. */
slope_status slope_spmm_fwd_decode_noalloc(slope_dtype in_dt, slope_dtype out_dt, const void* X, int64_t T,
                                           int64_t K, const void* packed_s, int64_t packed_s_bytes, int64_t N,
                                           const void* L_or_null, const void* R_or_null, int64_t r, void* Y,
                                           void* stream);

/* Bytes of a 16-bit matrix M [T, C] rewritten as token chunks (see
 * slope_pack_tokens).  Host-only. */
slope_status slope_packed_tokens_bytes(int64_t T, int64_t C, int64_t* bytes);

/* Transposed token-chunk copy of a 16-bit (bf16 or fp16) matrix M [T, C]
 * (C % 8 == 0), the
 * operand format of slope_masked_wgrad_packed: chunk (c, s) holds columns
 * 256c .. 256c+255 (one 64-byte row each) x tokens 32s .. 32s+31, 16 KB, at
 * byte offset (c * ceil(T/32) + s) * 16384; in a row, the 16-byte granule of
 * tokens 8g .. 8g+7 sits at granule position g ^ ((row / 4) % 4); entries
 * past T or C are 0.  packed: caller-owned device memory of at least
 * slope_packed_tokens_bytes(T, C) bytes, overwritten.
 * Errors: SLOPE_ERR_UNSUPPORTED for float32, SLOPE_ERR_SHAPE if C % 8 != 0,
 * SLOPE_ERR_WORKSPACE if packed_bytes is short. */
slope_status slope_pack_tokens(slope_dtype dt, const void* M, int64_t T, int64_t C, void* packed,
                               int64_t packed_bytes, void* stream);

/* Bytes of the token-split workspace slope_masked_wgrad_packed can use for T
 * tokens, N outputs and K inputs on the current device: fp32 partial sums of
 * the kept gradient values, either one [N, K/2] plane per token range (when
 * the 256 x 256 output tiles fill at most half the compute units), or one
 * 256 x 128 buffer per token range and tile of a last, partly filled round
 * of tiles (when they fill more than one round and the last is at most three
 * quarters full).  0 when neither applies (no split is made).  Host-only. */
slope_status slope_wgrad_split_workspace_bytes(int64_t T, int64_t N, int64_t K, int64_t* bytes);

/* slope_masked_wgrad on operands already packed by slope_pack_tokens:
 * dY_packed from dY [T, N], X_packed from X [T, K], both in_dt (BF16 or
 * F16; the chunks do not record it), with their byte counts (at least
 * slope_packed_tokens_bytes(T, N) and (T, K)).  Same outputs, bitwise, as
 * slope_masked_wgrad when split_workspace_or_null is NULL.
 * split_workspace_or_null: NULL, or caller-owned device memory of at least
 * slope_wgrad_split_workspace_bytes(T, N, K) bytes (scratch, overwritten):
 * when the output tiles alone would leave more than half of the compute units
 * idle, or end in a partly filled last round, the token reduction of all
 * tiles, or of that round's tiles, is then split into ranges whose fp32
 * partial sums are added in a fixed order by a second kernel (deterministic;
 * the sums are grouped differently, so those outputs may differ from the
 * unsplit form in the last bits; the other tiles' are bitwise the same).  Errors: SLOPE_ERR_SHAPE if N % 8 != 0 or K % 8 != 0;
 * SLOPE_ERR_WORKSPACE if a packed operand or the given split workspace is
 * short. */
slope_status slope_masked_wgrad_packed(slope_dtype in_dt, slope_dtype out_dt, const void* dY_packed,
                                       int64_t dY_packed_bytes, const void* X_packed, int64_t X_packed_bytes,
                                       int64_t T, int64_t N, int64_t K, const uint32_t* meta_s, void* dW_values,
                                       void* dW_dense_or_null, int accumulate, void* split_workspace_or_null,
                                       int64_t split_workspace_bytes, void* stream);

/* Low-rank adapter term on its own (explainer 2.B: W_dense = W_sparse + L R):
 *   Y [T, N] += (X [T, K] . L [K, r]) . R [r, N]
 * X . L and transposed copies of L and R go to the workspace, which must hold
 * slope_lowrank_workspace_bytes(T, K, r, N) bytes.  Y (out_dt) is read and
 * written.  Errors: SLOPE_ERR_WORKSPACE if the workspace is short. */
slope_status slope_lowrank_add(slope_dtype in_dt, slope_dtype out_dt, const void* X, const void* L, const void* R,
                               int64_t T, int64_t K, int64_t r, int64_t N, void* workspace,
                               int64_t workspace_bytes, void* Y, void* stream);

/* Hyper-parameters of one AdamW update (the discussion page, "Choice of
 * Optimizer": SLoPe trains with AdamW).  Plain host struct, read during the
 * call only.  step numbers this update, counting from 1 (bias correction). */
typedef struct slope_adamw_params {
  double lr, beta1, beta2, eps, weight_decay;
  int64_t step;
} slope_adamw_params;

/* One AdamW step (decoupled weight decay, bias-corrected moments) on n stored
 * values, elementwise:
 *   m = beta1 m + (1 - beta1) g;   v = beta2 v + (1 - beta2) g^2
 *   p = p (1 - lr wd) - lr / (1 - beta1^step) * m / (sqrt(v) / sqrt(1 - beta2^step) + eps)
 * params [n] param_dt (updated in place): the compressed values of a 2:4
 * weight (the discussion page, "Memory Footprint", keeps optimizer state only
 * for the two non-zeros of every four) or a dense adapter factor L or R;
 * grads [n] grad_dt (BF16 or F32) in the same order; m, v [n] fp32 moments,
 * updated in place.  fp32 arithmetic (constants derived in double on the
 * host), one rounding of each new value to param_dt.  hp: host pointer.
 * Errors: SLOPE_ERR_INVALID_ARG for a null pointer, unknown dtype, n < 0,
 * step < 1, a beta outside [0, 1), eps < 0 or non-finite lr / weight_decay;
 * SLOPE_ERR_UNSUPPORTED for n > 2^40. */
slope_status slope_adamw(slope_dtype param_dt, slope_dtype grad_dt, void* params, const void* grads, float* m,
                         float* v, int64_t n, const slope_adamw_params* hp, void* stream);

/* The weight update of one SLoPe training step, fused: slope_adamw on the
 * compressed values of W_s (values_s [N, K/2] and m, v [N, K/2] updated in
 * place; meta_s unchanged, the mask is static), then slope_double_prune of the
 * updated W_s (explainer 2.A: the backward weight is pruned again from the
 * current weight) into values_dpT [K, N/2], meta_dpT [K, ceil(N/32)] and, if
 * given, mask_dpT [K, N].  dW_values [N, K/2] grad_dt, in W_s's slot order (as
 * slope_masked_wgrad writes it).  Results equal slope_adamw followed by
 * slope_double_prune.  Errors: those of both calls. */
slope_status slope_adamw_double_prune(slope_dtype dt, slope_dtype grad_dt, void* values_s, const uint32_t* meta_s,
                                      const void* dW_values, float* m, float* v, int64_t N, int64_t K,
                                      const slope_adamw_params* hp, void* values_dpT, uint32_t* meta_dpT,
                                      uint8_t* mask_dpT_or_null, void* stream);

/* slope_double_prune (explainer 2.A, the double-pruned backward weight) with
 * W_dpT written straight to its tile-chunk form: packed_dpT afterwards holds
 * exactly what slope_pack_sparse (rows K, cols N) makes of slope_double_prune's
 * values_dpT and meta_dpT, bitwise, without those canonical rows.  values_s
 * [N, K/2], meta_s [N, ceil(K/32)] dt (BF16 or F16); packed_dpT: caller-owned
 * device memory of at least slope_packed_sparse_bytes(K, N) bytes, overwritten
 * (padding included).  Errors: SLOPE_ERR_UNSUPPORTED for F32 or N > 2^21,
 * SLOPE_ERR_SHAPE unless N % 16 == 0 and K % 16 == 0, SLOPE_ERR_WORKSPACE if
 * packed_dpT_bytes is short. */
slope_status slope_double_prune_packed(slope_dtype dt, const void* values_s, const uint32_t* meta_s, int64_t N,
                                       int64_t K, void* packed_dpT, int64_t packed_dpT_bytes, void* stream);

/* The fused weight update of slope_adamw_double_prune for a layer whose GEMM
 * operands are kept in tile-chunk form (explainer 2.A: the backward weight is
 * pruned again from the updated weight; discussion page, "Memory Footprint":
 * optimizer state only for the kept values).  values_s, m, v are updated in
 * place as there; packed_s must hold slope_pack_sparse(values_s, meta_s, N, K)
 * of the values before the update, and afterwards holds that of the updated
 * values (only its value granules are rewritten: the mask is static);
 * packed_dpT receives slope_double_prune_packed of the updated W_s.  Results
 * equal slope_adamw_double_prune followed by slope_pack_sparse of both
 * operands, bitwise.  dt BF16 or F16; grad_dt BF16, F16 or F32.  Errors: those
 * of slope_adamw_double_prune and slope_double_prune_packed, SLOPE_ERR_UNSUPPORTED
 * for K > 2^21, SLOPE_ERR_WORKSPACE if either packed size is short. */
slope_status slope_adamw_double_prune_packed(slope_dtype dt, slope_dtype grad_dt, void* values_s,
                                             const uint32_t* meta_s, const void* dW_values, float* m, float* v,
                                             int64_t N, int64_t K, const slope_adamw_params* hp, void* packed_s,
                                             int64_t packed_s_bytes, void* packed_dpT, int64_t packed_dpT_bytes,
                                             void* stream);

/* ---------------------------------------------------------------- 8-bit variant
 * The explainer's Technical Summary 1 (Problem Statement) names N:M sparsity
 * in general and the discussion page ("Memory Footprint Reduction During
 * Pretraining and Inference") counts 16-bit values; the pages give no 8-bit
 * format or scaling rule.  This variant reads them as: OCP FP8 E4M3 codes
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities; 0x7F
 * and 0xFF are NaN; largest finite 448), one float32 scale per tensor,
 * scale = 448 / amax (amax = largest magnitude of the stored 16-bit values;
 * one fp32 division; 1 when amax is 0 or not finite), code = E4M3 value
 * nearest to fp32(x * scale), ties to the even code, magnitudes beyond 448
 * saturated to +-448.  Products accumulate in float32; the scales are
 * divided out at the end.  The 2:4 pattern and metadata are the 16-bit
 * weight's. */

/* Per-tensor scale and E4M3 codes of a 16-bit tensor M (n values, BF16 or
 * F16): *scale (device float, 4-byte aligned) <- 448 / amax, q [n] uint8 <- codes
 * (both overwritten; the scale word is scratch while the call runs).
 * Deterministic.  Errors: SLOPE_ERR_UNSUPPORTED for F32 or n > 2^40. */
slope_status slope_quantize_e4m3(slope_dtype dt, const void* M, int64_t n, float* scale, uint8_t* q, void* stream);

/* Bytes of the E4M3 tile-chunk form of a compressed [rows, cols] matrix (see
 * slope_pack_sparse_e4m3).  Host-only; SLOPE_ERR_SHAPE if cols % 16 != 0,
 * SLOPE_ERR_UNSUPPORTED if cols > 2^21. */
slope_status slope_packed_sparse_e4m3_bytes(int64_t rows, int64_t cols, int64_t* bytes);

/* E4M3 tile chunks of a compressed 16-bit 2:4 matrix (values [rows, cols/2],
 * meta [rows, ceil(cols/32)] as slope_compress24 / slope_double_prune write
 * them), quantized with the matrix's own scale: *scale (device float) <- 448 /
 * amax over the values; chunk (t, s) holds rows 256t .. 256t+255 and dense
 * columns 128s .. 128s+127, 20480 bytes at offset (t * ceil(cols/128) + s) *
 * 20480: first each row's 64 codes (64 bytes at row*64; 16-byte granule c at
 * c ^ ((row / 4) % 4)), then each row's four metadata words 4s .. 4s+3 (16
 * bytes at 16384 + row*16); rows past `rows` and columns past `cols` are 0.
 * packed: caller-owned, at least slope_packed_sparse_e4m3_bytes(rows, cols)
 * bytes, overwritten.  Errors: SLOPE_ERR_UNSUPPORTED for F32 or cols > 2^21,
 * SLOPE_ERR_SHAPE if cols % 16 != 0, SLOPE_ERR_WORKSPACE if packed is short. */
slope_status slope_pack_sparse_e4m3(slope_dtype dt, const void* values, const uint32_t* meta, int64_t rows,
                                    int64_t cols, float* scale, void* packed, int64_t packed_bytes, void* stream);

/* The 2:4 sparse product on E4M3 operands (explainer 2.A: the forward with
 * W_s, and dX with W_dp, in the 8-bit reading above):
 *   Y [T, N] = (Xq [T, K] . W_q^T) / (x_scale * w_scale)
 * Xq: E4M3 codes [T, K] (slope_quantize_e4m3 of X, or of dY for dX);
 * packed_w: slope_pack_sparse_e4m3 of W_s (rows N, cols K), or of W_dp^T
 * (rows K, cols N) for dX, with packed_w_bytes at least
 * slope_packed_sparse_e4m3_bytes(N, K); x_scale, w_scale: the device floats
 * those calls wrote.  out_dt BF16 or F32.  Y is overwritten.  No adapter
 * term (slope_lowrank_add adds it).  Errors: SLOPE_ERR_SHAPE unless
 * K % 16 == 0 and N % 4 == 0; SLOPE_ERR_UNSUPPORTED for F16 outputs or
 * K > 2^21; SLOPE_ERR_WORKSPACE if packed_w is short. */
slope_status slope_spmm_e4m3_packed(slope_dtype out_dt, const uint8_t* Xq, const float* x_scale, int64_t T, int64_t K,
                                    const void* packed_w, int64_t packed_w_bytes, const float* w_scale, int64_t N,
                                    void* Y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SLOPE_H_ */

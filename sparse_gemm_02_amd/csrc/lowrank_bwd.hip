// Weight gradients of the low-rank adapter (the adapter term Y += (X . L) . R
// of the SLoPe explainer, Technical Summary 2.B, differentiated):
//
//   dR = (X . L)^T . dY   [r, N]      dL = X^T . (dY . R^T)   [K, r]
//
// Both are reductions over the tokens with a small output (the rank is at
// most 128), so they share one kernel: out^T[c][j] = sum_t A[t][c] B[t][j]
// with A the large operand (dY or X) in token-chunk form (pack_tokens: one
// 64-byte row of 32 tokens per column c) and B the small one (X . L or
// dY . R^T) as a transposed 16-bit hi/lo pair [rpad32][Tpad] (the operands'
// format: bf16, or fp16 with H).  Each block takes
// one 256-column chunk column over a range of token chunks (B's slice staged
// in LDS once per chunk for the block's four waves); the fp32 partial
// sums are added in range order by a second kernel, which also writes the
// output in its own layout (dR row-major [r, N], dL row-major [K, r]).
#include "common.h"
#include "dma.h"
#include "launch.h"

namespace slope {

namespace {

constexpr int kChunkRows = 256, kChunkTokens = 32, kChunkBytes = kChunkRows * kChunkTokens * 2;

// part[split][j][c] (c < Cpad) = sum over the split's token chunks of A[t][c] B[t][j].
// Wave w: chunk rows 64w .. 64w+63 (two 32-row MFMA tiles) x FJ 32-wide rank
// tiles; 32x32x16 MFMA over 16 tokens, hi and lo parts of B.  A comes straight
// from memory; the block stages each chunk's slice of B (FJ*32 rows x 32
// tokens, hi and lo) in LDS once, in a double buffer, with 16-byte granule g
// of row j at g ^ ((j/4) % 4) so that fragment reads are free of conflicts.
template <int FJ, bool H>
__global__ __launch_bounds__(256) void lr_wgrad_partial_kernel(const char* __restrict__ chunks, int64_t Tch,
                                                               int per_split, const uint16_t* __restrict__ bh,
                                                               const uint16_t* __restrict__ bl, int64_t Tpad,
                                                               int64_t Cpad, float* __restrict__ part) {
  constexpr int BROWS = FJ * 32, SLICE = 2 * BROWS * 64;        // bytes of one chunk's B slice (hi and lo)
  __shared__ __attribute__((aligned(16))) char bs[2][SLICE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x, split = blockIdx.y;
  const int64_t s0 = (int64_t)split * per_split;
  const int64_t s1 = (s0 + per_split < Tch) ? s0 + per_split : Tch;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(chunks + ((int64_t)tile * Tch + s0) * kChunkBytes,
                                              s1 > s0 ? (s1 - s0) * kChunkBytes : 0);
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(bh, (int64_t)BROWS * Tpad * 2);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(bl, (int64_t)BROWS * Tpad * 2);
  uint32_t a_off[2][2];
#pragma unroll
  for (int fm = 0; fm < 2; ++fm) {
    const int r = wave * 64 + fm * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) a_off[fm][ks] = r * 64 + (((2 * ks + (lane >> 5)) ^ ((r >> 2) & 3)) << 4);
  }
  // staging: thread piece i < FJ: slice row q = piece / 4 (hi rows, then lo rows), granule g = piece % 4
  uint32_t st_src[FJ], st_dst[FJ];
  bool st_lo[FJ];
#pragma unroll
  for (int i = 0; i < FJ; ++i) {
    const int piece = tid + 256 * i, q = piece >> 2, g = piece & 3, j = q % BROWS;
    st_lo[i] = q >= BROWS;
    st_src[i] = (uint32_t)(j * Tpad + g * 8) * 2;
    st_dst[i] = q * 64 + ((g ^ ((j >> 2) & 3)) << 4);
  }
  // fragment reads: row j = 32 fj + lane%32 (hi at row j, lo at row BROWS + j), granule 2 ks + lane/32
  uint32_t b_off[2][FJ];
#pragma unroll
  for (int fj = 0; fj < FJ; ++fj) {
    const int j = fj * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) b_off[ks][fj] = j * 64 + (((2 * ks + (lane >> 5)) ^ ((j >> 2) & 3)) << 4);
  }

  f32x16 acc[2][FJ];
#pragma unroll
  for (int fm = 0; fm < 2; ++fm)
#pragma unroll
    for (int fj = 0; fj < FJ; ++fj) acc[fm][fj] = f32x16{};

  // chunk s's loads are issued while chunk s-1 is multiplied: the A
  // fragments and B's slice go to registers one chunk ahead (the buffer
  // resources return 0 past the split's chunks and past Tpad)
  typedef typename Fmt16<H>::v8 v8;
  v8 an[2][2];
  u32x4 bn[FJ];
  auto load_chunk = [&](int64_t s) {
    const uint32_t c = (uint32_t)(s - s0) * kChunkBytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int fm = 0; fm < 2; ++fm) an[ks][fm] = __builtin_bit_cast(v8, load16(ra, c + a_off[fm][ks]));
    const uint32_t tb = (uint32_t)(s * kChunkTokens) * 2;
#pragma unroll
    for (int i = 0; i < FJ; ++i) bn[i] = load16(st_lo[i] ? rl : rh, st_src[i] + tb);
  };
  if (s0 < s1) load_chunk(s0);
  for (int64_t s = s0; s < s1; ++s) {
    v8 a[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int fm = 0; fm < 2; ++fm) a[ks][fm] = an[ks][fm];
    char* buf = bs[s & 1];
#pragma unroll
    for (int i = 0; i < FJ; ++i) *reinterpret_cast<u32x4*>(buf + st_dst[i]) = bn[i];
    load_chunk(s + 1);                                 // past s1 these read 0 and are not used
    __syncthreads();                                   // slice s staged; slice s-2's buffer no longer read
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8 h[FJ], l[FJ];
#pragma unroll
      for (int fj = 0; fj < FJ; ++fj) {
        h[fj] = *reinterpret_cast<const v8*>(buf + b_off[ks][fj]);
        l[fj] = *reinterpret_cast<const v8*>(buf + BROWS * 64 + b_off[ks][fj]);
      }
#pragma unroll
      for (int fj = 0; fj < FJ; ++fj)
#pragma unroll
        for (int fm = 0; fm < 2; ++fm) {
          acc[fm][fj] = Fmt16<H>::mfma32x32x16(a[ks][fm], h[fj], acc[fm][fj]);
          acc[fm][fj] = Fmt16<H>::mfma32x32x16(a[ks][fm], l[fj], acc[fm][fj]);
        }
    }
  }
  // D: lane holds rank column fj*32 + lane%32, chunk rows 8*(v/4) + 4*(lane/32) + v%4
#pragma unroll
  for (int fj = 0; fj < FJ; ++fj) {
    const int j = fj * 32 + (lane & 31);
    float* dst = part + ((int64_t)split * FJ * 32 + j) * Cpad + (int64_t)tile * 256 + wave * 64;
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = {acc[fm][fj][4 * q], acc[fm][fj][4 * q + 1], acc[fm][fj][4 * q + 2], acc[fm][fj][4 * q + 3]};
        *reinterpret_cast<f32x4*>(dst + fm * 32 + 8 * q + 4 * (lane >> 5)) = v;
      }
  }
}

// out = sum over splits (in order) of part[s][j][c], for j < r, c < C, written
// as out[j][c] (TRANS false: dR [r, N]) or out[c][j] (TRANS true: dL [K, r]).
template <typename O, bool TRANS>
__global__ __launch_bounds__(256) void lr_wgrad_reduce_kernel(const float* __restrict__ part, int splits, int r,
                                                              int rows32, int64_t C, int64_t Cpad, int accumulate,
                                                              O* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)r * C) return;
  const int64_t j = i / C, c = i % C;
  float v = 0.f;
#pragma unroll 4
  for (int sp = 0; sp < splits; ++sp) v += part[((int64_t)sp * rows32 + j) * Cpad + c];
  O* p = TRANS ? out + c * r + j : out + j * C + c;
  if (accumulate) v += load_out(p);
  store_out(p, v);
}

// About 1024 blocks, but at most T / (16 * rows of B) token ranges: the fp32
// partial sums (splits x rows x C x 4 bytes, written and read) then stay
// within a quarter of the bytes of A itself.
int64_t split_count(int64_t tiles, int64_t Tch, int64_t brows) {
  int64_t want = cdiv(1024, tiles < 1 ? 1 : tiles);
  const int64_t cap = Tch * kChunkTokens / (16 * (brows < 1 ? 1 : brows));
  if (want > cap) want = cap;
  if (want > Tch) want = Tch;
  return want < 1 ? 1 : want;
}

template <int FJ>
void launch_partial(bool h16, const char* chunks, int64_t tiles, int64_t Tch, int per, int64_t splits,
                    const uint16_t* bh, const uint16_t* bl, int64_t Tpad, int64_t Cpad, float* part, hipStream_t s) {
  const dim3 grid((unsigned)tiles, (unsigned)splits);
  if (h16)
    lr_wgrad_partial_kernel<FJ, true><<<grid, 256, 0, s>>>(chunks, Tch, per, bh, bl, Tpad, Cpad, part);
  else
    lr_wgrad_partial_kernel<FJ, false><<<grid, 256, 0, s>>>(chunks, Tch, per, bh, bl, Tpad, Cpad, part);
}

template <typename O>
void launch_reduce(const float* part, int sp, int r, int rows, int64_t C, int64_t Cpad, int accumulate, bool trans,
                   void* dst, hipStream_t s) {
  const unsigned rb = (unsigned)cdiv((int64_t)r * C, 256);
  if (trans)
    lr_wgrad_reduce_kernel<O, true><<<rb, 256, 0, s>>>(part, sp, r, rows, C, Cpad, accumulate, (O*)dst);
  else
    lr_wgrad_reduce_kernel<O, false><<<rb, 256, 0, s>>>(part, sp, r, rows, C, Cpad, accumulate, (O*)dst);
}

}  // namespace

int64_t lr_wgrad_part_bytes(int64_t T, int64_t C, int64_t r) {
  const int64_t tiles = cdiv(C, kChunkRows), Tch = cdiv(T, kChunkTokens);
  const int64_t per = cdiv(Tch, split_count(tiles, Tch, cdiv(r, 32) * 32)), splits = Tch ? cdiv(Tch, per) : 1;
  return cdiv(splits * cdiv(r, 32) * 32 * tiles * kChunkRows * 4, 256) * 256;
}

hipError_t launch_lr_wgrad(Dt in, Dt out, const void* chunks, int64_t T, int64_t C, int64_t r, const uint16_t* bh,
                           const uint16_t* bl, int64_t Tpad, float* part, void* dst, bool trans, int accumulate,
                           hipStream_t s) {
  if (C == 0 || r == 0) return hipSuccess;
  const int64_t tiles = cdiv(C, kChunkRows), Tch = cdiv(T, kChunkTokens), Cpad = tiles * kChunkRows;
  const int64_t per = Tch ? cdiv(Tch, split_count(tiles, Tch, cdiv(r, 32) * 32)) : 1, splits = Tch ? cdiv(Tch, per) : 1;
  const int fj = (int)cdiv(r, 32);
  const char* ch = (const char*)chunks;
  const bool h16 = in == Dt::F16;
  if (Tch == 0) {
    // no tokens: the sums are empty (one split of zeros, cleared by a kernel)
    hipError_t e = launch_fill_zero(Dt::F32, part, (int64_t)fj * 32 * Cpad, s);
    if (e != hipSuccess) return e;
  } else if (fj == 1) {
    launch_partial<1>(h16, ch, tiles, Tch, (int)per, splits, bh, bl, Tpad, Cpad, part, s);
  } else if (fj == 2) {
    launch_partial<2>(h16, ch, tiles, Tch, (int)per, splits, bh, bl, Tpad, Cpad, part, s);
  } else if (fj == 3) {
    launch_partial<3>(h16, ch, tiles, Tch, (int)per, splits, bh, bl, Tpad, Cpad, part, s);
  } else {
    launch_partial<4>(h16, ch, tiles, Tch, (int)per, splits, bh, bl, Tpad, Cpad, part, s);
  }
  const int sp = Tch ? (int)splits : 1;
  if (out == Dt::BF16)
    launch_reduce<uint16_t>(part, sp, (int)r, fj * 32, C, Cpad, accumulate, trans, dst, s);
  else if (out == Dt::F16)
    launch_reduce<_Float16>(part, sp, (int)r, fj * 32, C, Cpad, accumulate, trans, dst, s);
  else
    launch_reduce<float>(part, sp, (int)r, fj * 32, C, Cpad, accumulate, trans, dst, s);
  return hipGetLastError();
}

}  // namespace slope

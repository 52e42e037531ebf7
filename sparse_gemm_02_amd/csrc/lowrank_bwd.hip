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
// format: bf16, or fp16 with H; rows from the rank up are zero, and the kernel
// reads the rank rounded up to 16 of them).  Each block takes
// one 256-column chunk column over a range of token chunks (B's slice staged
// in LDS once per chunk for the block's four waves); the fp32 partial
// sums are added in range order by a second kernel, which also writes the
// output in its own layout (dR row-major [r, N], dL row-major [K, r]).  One
// launch of each kernel computes both gradients of a layer.
#include "common.h"
#include "dma.h"
#include "launch.h"

namespace slope {

namespace {

constexpr int kChunkRows = 256, kChunkTokens = 32, kChunkBytes = kChunkRows * kChunkTokens * 2;

// part[split][j][c] (c < Cpad, j < 16 NJ) = sum over the split's token chunks of
// A[t][c] B[t][j].  Wave w: chunk rows 64w .. 64w+63 (four 16-row MFMA tiles) x
// NJ 16-wide rank tiles (a rank of 72 pads to 80, not 96); one 16x16x32 MFMA
// covers a whole 32-token chunk, for the hi and the lo part of B.  Dense
// 16x16x32 MFMA: A lane l = row l%16, k = 8*(l/16)+e; B lane l = column l%16,
// same k; D lane l = column l%16, rows 4*(l/16)+v.  A comes straight from
// memory; the block stages each chunk's slice of B (16 NJ rows x 32 tokens, hi
// and lo) in LDS once, in a double buffer, with 16-byte granule g of row j at
// g ^ ((j/4) % 4) so that fragment reads are free of bank conflicts.
// One product of the pair a launch computes: A's token chunks, B's hi/lo
// pair, the partial sums, and the grid of tiles x splits that covers it.
struct LrTask {
  const char* chunks;
  const uint16_t* bh;
  const uint16_t* bl;
  float* part;
  int64_t Tch, Tpad, Cpad;
  int per_split, tiles, splits;
};

// Blocks 0 .. t0.tiles * t0.splits - 1 compute t0 (tile fastest), the rest t1:
// both adapter products of a layer in one launch, so that the one with few
// column tiles (216 blocks for a 9216-wide operand) shares the device with the
// other instead of running alone.  Up to rank 80 the register budget of three
// blocks per compute unit holds the accumulators without spilling (four
// linears of OPT-66B at rank 72: 0.81 -> 0.79 ms with two blocks per unit).
template <int NJ, bool H>
__global__ __launch_bounds__(256, NJ <= 5 ? 3 : 2) void lr_wgrad_partial_kernel(const LrTask t0, const LrTask t1) {
  constexpr int BROWS = NJ * 16, SLICE = 2 * BROWS * 64;        // bytes of one chunk's B slice (hi and lo)
  constexpr int PIECES = SLICE / 16, PPT = (PIECES + 255) / 256;  // 16-byte staging pieces, per thread
  __shared__ __attribute__((aligned(16))) char bs[2][SLICE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = t0.tiles * t0.splits;
  const bool second = (int)blockIdx.x >= n0;                      // block-uniform
  const LrTask& t = second ? t1 : t0;
  const int b = second ? (int)blockIdx.x - n0 : (int)blockIdx.x;
  const int tile = b % t.tiles, split = b / t.tiles;
  const char* __restrict__ chunks = t.chunks;
  const uint16_t* __restrict__ bh = t.bh;
  const uint16_t* __restrict__ bl = t.bl;
  float* __restrict__ part = t.part;
  const int64_t Tch = t.Tch, Tpad = t.Tpad, Cpad = t.Cpad;
  const int per_split = t.per_split;
  const int64_t s0 = (int64_t)split * per_split;
  const int64_t s1 = (s0 + per_split < Tch) ? s0 + per_split : Tch;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(chunks + ((int64_t)tile * Tch + s0) * kChunkBytes,
                                              s1 > s0 ? (s1 - s0) * kChunkBytes : 0);
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(bh, (int64_t)BROWS * Tpad * 2);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(bl, (int64_t)BROWS * Tpad * 2);
  // A fragments: row tile rt, chunk row 64w + 16rt + l%16, granule l/16 (8 tokens)
  uint32_t a_off[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int r = wave * 64 + rt * 16 + (lane & 15);
    a_off[rt] = r * 64 + (((lane >> 4) ^ ((r >> 2) & 3)) << 4);
  }
  // staging: piece = slice row q (hi rows, then lo rows) x granule g; pieces past the slice load nothing
  uint32_t st_src[PPT], st_dst[PPT];
  bool st_lo[PPT], st_on[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int piece = tid + 256 * i, q = (piece >> 2) % (2 * BROWS), g = piece & 3, j = q % BROWS;
    st_on[i] = piece < PIECES;
    st_lo[i] = q >= BROWS;
    st_src[i] = (uint32_t)(j * Tpad + g * 8) * 2;
    st_dst[i] = q * 64 + ((g ^ ((j >> 2) & 3)) << 4);
  }
  // B fragments: rank tile jb, row j = 16jb + l%16, granule l/16
  uint32_t b_off[NJ];
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb) {
    const int j = jb * 16 + (lane & 15);
    b_off[jb] = j * 64 + (((lane >> 4) ^ ((j >> 2) & 3)) << 4);
  }

  f32x4 acc[4][NJ];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) acc[rt][jb] = f32x4{};

  // chunk s's loads are issued while chunk s-1 is multiplied: the A
  // fragments and B's slice go to registers one chunk ahead (the buffer
  // resources return 0 past the split's chunks and past Tpad)
  typedef typename Fmt16<H>::v8 v8;
  v8 an[4];
  u32x4 bn[PPT];
  auto load_chunk = [&](int64_t s) {
    const uint32_t c = (uint32_t)(s - s0) * kChunkBytes;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) an[rt] = __builtin_bit_cast(v8, load16(ra, c + a_off[rt]));
    const uint32_t tb = (uint32_t)(s * kChunkTokens) * 2;
#pragma unroll
    for (int i = 0; i < PPT; ++i) bn[i] = load16(st_lo[i] ? rl : rh, st_on[i] ? st_src[i] + tb : kOutOfRange);
  };
  if (s0 < s1) load_chunk(s0);
  for (int64_t s = s0; s < s1; ++s) {
    v8 a[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) a[rt] = an[rt];
    char* buf = bs[s & 1];
#pragma unroll
    for (int i = 0; i < PPT; ++i)
      if (st_on[i]) *reinterpret_cast<u32x4*>(buf + st_dst[i]) = bn[i];
    load_chunk(s + 1);                                 // past s1 these read 0 and are not used
    __syncthreads();                                   // slice s staged; slice s-2's buffer no longer read
#pragma unroll
    for (int jb = 0; jb < NJ; ++jb) {
      const v8 h = *reinterpret_cast<const v8*>(buf + b_off[jb]);
      const v8 l = *reinterpret_cast<const v8*>(buf + BROWS * 64 + b_off[jb]);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        acc[rt][jb] = Fmt16<H>::mfma16x16x32(a[rt], h, acc[rt][jb]);
        acc[rt][jb] = Fmt16<H>::mfma16x16x32(a[rt], l, acc[rt][jb]);
      }
    }
  }
  // D: lane holds rank column 16jb + lane%16, chunk rows 16rt + 4(lane/16) + v
#pragma unroll
  for (int jb = 0; jb < NJ; ++jb) {
    const int j = jb * 16 + (lane & 15);
    float* dst = part + ((int64_t)split * BROWS + j) * Cpad + (int64_t)tile * 256 + wave * 64 + 4 * (lane >> 4);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) *reinterpret_cast<f32x4*>(dst + rt * 16) = acc[rt][jb];
  }
}

// One output of the pair: its partial sums and where the sums go.
struct LrOut {
  const float* part;
  void* out;
  int64_t C, Cpad;
  int splits;
  bool trans;
};

// out = sum over splits (in order) of part[s][j][c], for j < r, c < C, written
// as out[j][c] (trans false: dR [r, N]) or out[c][j] (trans true: dL [K, r]);
// elements 0 .. r C0 - 1 are o0's, the rest o1's.
template <typename O>
__global__ __launch_bounds__(256) void lr_wgrad_reduce_kernel(const LrOut o0, const LrOut o1, int r, int rows,
                                                              int accumulate) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool second = i >= (int64_t)r * o0.C;
  if (second) i -= (int64_t)r * o0.C;
  const LrOut& o = second ? o1 : o0;
  if (i >= (int64_t)r * o.C) return;
  const int64_t j = i / o.C, c = i % o.C;
  float v = 0.f;
#pragma unroll 4
  for (int sp = 0; sp < o.splits; ++sp) v += o.part[((int64_t)sp * rows + j) * o.Cpad + c];
  O* p = o.trans ? (O*)o.out + c * r + j : (O*)o.out + j * o.C + c;
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

template <int NJ>
void launch_partial(bool h16, const LrTask& t0, const LrTask& t1, hipStream_t s) {
  const unsigned grid = (unsigned)(t0.tiles * t0.splits + t1.tiles * t1.splits);
  if (h16)
    lr_wgrad_partial_kernel<NJ, true><<<grid, 256, 0, s>>>(t0, t1);
  else
    lr_wgrad_partial_kernel<NJ, false><<<grid, 256, 0, s>>>(t0, t1);
}

template <typename O>
void launch_reduce(const LrOut& o0, const LrOut& o1, int r, int rows, int accumulate, hipStream_t s) {
  const unsigned rb = (unsigned)cdiv((int64_t)r * (o0.C + o1.C), 256);
  lr_wgrad_reduce_kernel<O><<<rb, 256, 0, s>>>(o0, o1, r, rows, accumulate);
}

}  // namespace

// rows of B and of the partial sums: the rank rounded up to 16
int64_t lr_rows(int64_t r) { return cdiv(r, 16) * 16; }

int64_t lr_wgrad_part_bytes(int64_t T, int64_t C, int64_t r) {
  const int64_t tiles = cdiv(C, kChunkRows), Tch = cdiv(T, kChunkTokens);
  const int64_t per = cdiv(Tch, split_count(tiles, Tch, lr_rows(r))), splits = Tch ? cdiv(Tch, per) : 1;
  return cdiv(splits * lr_rows(r) * tiles * kChunkRows * 4, 256) * 256;
}

hipError_t launch_lr_wgrad_pair(Dt in, Dt out, const LrGrad& g0, const LrGrad& g1, int64_t T, int64_t r,
                                int accumulate, hipStream_t s) {
  if (r == 0 || g0.C == 0 || g1.C == 0) return hipErrorInvalidValue;   // the caller returns before
  const int64_t Tch = cdiv(T, kChunkTokens), rows = lr_rows(r);
  if (Tch == 0) return hipErrorInvalidValue;                            // no tokens: the caller clears dL, dR
  auto task = [&](const LrGrad& g) {
    const int64_t tiles = cdiv(g.C, kChunkRows);
    const int64_t per = cdiv(Tch, split_count(tiles, Tch, rows)), splits = cdiv(Tch, per);
    return LrTask{(const char*)g.chunks, g.bh, g.bl, g.part, Tch, g.Tpad, tiles * kChunkRows, (int)per, (int)tiles,
                  (int)splits};
  };
  const LrTask t0 = task(g0), t1 = task(g1);
  const bool h16 = in == Dt::F16;
  switch (rows / 16) {
    case 1: launch_partial<1>(h16, t0, t1, s); break;
    case 2: launch_partial<2>(h16, t0, t1, s); break;
    case 3: launch_partial<3>(h16, t0, t1, s); break;
    case 4: launch_partial<4>(h16, t0, t1, s); break;
    case 5: launch_partial<5>(h16, t0, t1, s); break;
    case 6: launch_partial<6>(h16, t0, t1, s); break;
    case 7: launch_partial<7>(h16, t0, t1, s); break;
    case 8: launch_partial<8>(h16, t0, t1, s); break;
    default: return hipErrorInvalidValue;     // rank above 128: refused by the caller
  }
  const LrOut o0{g0.part, g0.dst, g0.C, t0.Cpad, t0.splits, g0.trans};
  const LrOut o1{g1.part, g1.dst, g1.C, t1.Cpad, t1.splits, g1.trans};
  if (out == Dt::BF16)
    launch_reduce<uint16_t>(o0, o1, (int)r, (int)rows, accumulate, s);
  else if (out == Dt::F16)
    launch_reduce<_Float16>(o0, o1, (int)r, (int)rows, accumulate, s);
  else
    launch_reduce<float>(o0, o1, (int)r, (int)rows, accumulate, s);
  return hipGetLastError();
}

}  // namespace slope

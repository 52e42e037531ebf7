// Magnitude 2:4 pruning, compression and double pruning (HBM-bound kernels).
//
// SLoPe explainer (gist.science), Technical Summary 2.A: the forward weight is
// pruned N:M (2:4) along its rows; the backward weight is the already sparse
// weight, transposed and pruned 2:4 again.  The discussion page's "Memory
// Footprint" section keeps each as two 16-bit values plus indices per group of
// four.  Selection rule: the two largest magnitudes, equal magnitudes to the
// lower position, NaN above every number.
#include "adamw.h"
#include "common.h"
#include "launch.h"

namespace slope {

namespace {

constexpr int kThreads = 256;

template <typename E> struct Vec4;                       // one group of four raw values
template <> struct Vec4<uint16_t> { typedef u32x2 T; };  // 8 bytes
template <> struct Vec4<_Float16> { typedef u32x2 T; };
template <> struct Vec4<uint32_t> { typedef u32x4 T; };  // 16 bytes

__device__ __forceinline__ void unpack(u32x2 v, uint16_t e[4]) {
  e[0] = (uint16_t)(v[0] & 0xFFFF); e[1] = (uint16_t)(v[0] >> 16);
  e[2] = (uint16_t)(v[1] & 0xFFFF); e[3] = (uint16_t)(v[1] >> 16);
}
__device__ __forceinline__ void unpack(u32x4 v, uint32_t e[4]) { e[0] = v[0]; e[1] = v[1]; e[2] = v[2]; e[3] = v[3]; }
__device__ __forceinline__ void unpack(u32x2 v, _Float16 e[4]) {
  uint16_t b[4];
  unpack(v, b);
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = __builtin_bit_cast(_Float16, b[i]);
}
__device__ __forceinline__ u32x2 pack(const uint16_t e[4]) {
  u32x2 v; v[0] = e[0] | ((uint32_t)e[1] << 16); v[1] = e[2] | ((uint32_t)e[3] << 16); return v;
}
__device__ __forceinline__ u32x4 pack(const uint32_t e[4]) { u32x4 v; v[0] = e[0]; v[1] = e[1]; v[2] = e[2]; v[3] = e[3]; return v; }
__device__ __forceinline__ u32x2 pack(const _Float16 e[4]) {
  uint16_t b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = __builtin_bit_cast(uint16_t, e[i]);
  return pack(b);
}

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef int16_t i16x2 __attribute__((ext_vector_type(2)));

// The rule of top2_of_4 for two groups at once: w[j] holds element j of one
// group of four in its low half and of another group in its high half.  Magnitude keys are at most 15 bits, so with packed 16-bit arithmetic
// the sign of k_j - k_i - 1 says whether i (< j) outranks j, ranks are sums of
// those signs and a position is kept when its rank is below two.  Per half:
// a / b = the values at the lower / higher kept position, nib = i0 | i1 << 2.
template <bool H>
__device__ __forceinline__ void top2_of_4_x2(const uint32_t w[4], uint32_t& a, uint32_t& b, uint32_t& nib,
                                             uint32_t keep[4]) {
  const uint16_t nan_key = H ? 0x7C01 : 0x7F81;     // every NaN ranks as this key (ties among NaNs)
  i16x2 k[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u16x2 m = __builtin_bit_cast(u16x2, w[j] & 0x7FFF7FFFu);
    k[j] = __builtin_bit_cast(i16x2, __builtin_elementwise_min(m, (u16x2){nan_key, nan_key}));
  }
  // o_ij = -1 where i outranks j (k_i >= k_j for i < j), else 0
  auto outranks = [&](int i, int j) { return (i16x2)((k[j] - k[i] - (i16x2){1, 1}) >> (i16x2){15, 15}); };
  const i16x2 o01 = outranks(0, 1), o02 = outranks(0, 2), o03 = outranks(0, 3);
  const i16x2 o12 = outranks(1, 2), o13 = outranks(1, 3), o23 = outranks(2, 3);
  // rank - 2 of each position
  const i16x2 r0 = (i16x2){1, 1} + o01 + o02 + o03;
  const i16x2 r1 = o12 + o13 - o01;
  const i16x2 r2 = o23 - o02 - o12 - (i16x2){1, 1};
  const i16x2 r3 = (i16x2){-2, -2} - o03 - o13 - o23;
  keep[0] = __builtin_bit_cast(uint32_t, (i16x2)(r0 >> (i16x2){15, 15}));
  keep[1] = __builtin_bit_cast(uint32_t, (i16x2)(r1 >> (i16x2){15, 15}));
  keep[2] = __builtin_bit_cast(uint32_t, (i16x2)(r2 >> (i16x2){15, 15}));
  keep[3] = __builtin_bit_cast(uint32_t, (i16x2)(r3 >> (i16x2){15, 15}));
  auto sel = [](uint32_t m, uint32_t x, uint32_t y) { return (x & m) | (y & ~m); };
  a = sel(keep[0], w[0], sel(keep[1], w[1], w[2]));
  b = sel(keep[3], w[3], sel(keep[2], w[2], w[1]));
  const uint32_t i0 = sel(keep[0], 0u, sel(keep[1], 0x00010001u, 0x00020002u));
  const uint32_t i1 = sel(keep[3], 0x00030003u, sel(keep[2], 0x00020002u, 0x00010001u));
  nib = i0 | (i1 << 2);
}

// ------------------------------------------------------------------ prune24
// One group of four per thread and iteration; groups never straddle rows
// because cols % 4 == 0, so the matrix is a flat array of groups.
template <typename E, int UNROLL>
__global__ __launch_bounds__(kThreads) void prune24_kernel(const E* __restrict__ W, int64_t groups,
                                                           uint32_t* __restrict__ mask4, E* __restrict__ W_s) {
  typedef typename Vec4<E>::T V;
  const V* in = reinterpret_cast<const V*>(W);
  V* out = reinterpret_cast<V*>(W_s);
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t g0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; g0 < groups; g0 += stride * UNROLL) {
    V v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      int64_t g = g0 + u * stride;
      if (g < groups) v[u] = __builtin_nontemporal_load(in + g);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      int64_t g = g0 + u * stride;
      if (g >= groups) break;
      E e[4];
      unpack(v[u], e);
      uint32_t keep = top2_of_4(mag_key(e[0]), mag_key(e[1]), mag_key(e[2]), mag_key(e[3]));
      // mask bytes 0/1 for the four positions, little-endian in one word
      uint32_t mb = (keep & 1u) | ((keep & 2u) << 7) | ((keep & 4u) << 14) | ((keep & 8u) << 21);
      mask4[g] = mb;
      if (W_s) {
        E o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (keep >> i) & 1u ? e[i] : (E)0;
        out[g] = pack(o);
      }
    }
  }
}

// ------------------------------------------------------------------ prune N:M
// General N:M (the explainer's Technical Summary 1 names N:M sparsity in
// general): per group of M consecutive elements the n highest-ranked are kept,
// ranked as in prune24 (magnitude key, equal keys to the lower position).  One
// group per thread: position j is kept when fewer than n positions outrank it.
// The group's M * sizeof(E) bytes move as 16-byte words (8 bytes for four
// 16-bit values); the mask bytes and W_s go out the same way.
template <typename E> __device__ __forceinline__ uint32_t elem_key(const uint32_t* w, int i) {
  if constexpr (sizeof(E) == 4) {
    return mag_key(w[i]);
  } else {
    const uint16_t b = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
    if constexpr (__is_same(E, _Float16)) return mag_key(__builtin_bit_cast(_Float16, b));
    else return mag_key(b);
  }
}

template <int WORDS> __device__ __forceinline__ void load_words(const uint32_t* p, uint32_t* w) {
  if constexpr (WORDS % 4 == 0) {
#pragma unroll
    for (int q = 0; q < WORDS / 4; ++q) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + q);
      w[4 * q] = v[0]; w[4 * q + 1] = v[1]; w[4 * q + 2] = v[2]; w[4 * q + 3] = v[3];
    }
  } else if constexpr (WORDS == 2) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    w[0] = v[0]; w[1] = v[1];
  } else {
    static_assert(WORDS == 1, "group sizes of 4, 8, 16 or 32 elements");
    w[0] = __builtin_nontemporal_load(p);
  }
}

template <int WORDS> __device__ __forceinline__ void store_words(uint32_t* p, const uint32_t* w) {
  if constexpr (WORDS % 4 == 0) {
#pragma unroll
    for (int q = 0; q < WORDS / 4; ++q) {
      u32x4 v; v[0] = w[4 * q]; v[1] = w[4 * q + 1]; v[2] = w[4 * q + 2]; v[3] = w[4 * q + 3];
      reinterpret_cast<u32x4*>(p)[q] = v;
    }
  } else if constexpr (WORDS == 2) {
    u32x2 v; v[0] = w[0]; v[1] = w[1];
    *reinterpret_cast<u32x2*>(p) = v;
  } else {
    p[0] = w[0];
  }
}

template <typename E, int M>
__global__ __launch_bounds__(kThreads) void prune_nm_kernel(const uint32_t* __restrict__ W, int64_t groups, int n,
                                                           uint32_t* __restrict__ mask, uint32_t* __restrict__ W_s) {
  constexpr int WORDS = M * (int)sizeof(E) / 4;   // 32-bit words of one group
  constexpr int PER = 4 / (int)sizeof(E);          // elements per word
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < groups; g += stride) {
    uint32_t w[WORDS];
    load_words<WORDS>(W + g * WORDS, w);
    uint32_t k[M];
#pragma unroll
    for (int i = 0; i < M; ++i) k[i] = elem_key<E>(w, i);
    uint32_t keep = 0;
#pragma unroll
    for (int j = 0; j < M; ++j) {
      int above = 0;
#pragma unroll
      for (int i = 0; i < M; ++i) {
        if (i < j) above += k[i] >= k[j];
        else if (i > j) above += k[i] > k[j];
      }
      keep |= (uint32_t)(above < n) << j;
    }
    uint32_t mb[M / 4];                             // mask bytes 0/1, four positions per word
#pragma unroll
    for (int q = 0; q < M / 4; ++q) {
      const uint32_t b = keep >> (4 * q);
      mb[q] = (b & 1u) | ((b & 2u) << 7) | ((b & 4u) << 14) | ((b & 8u) << 21);
    }
    store_words<M / 4>(mask + g * (M / 4), mb);
    if (W_s) {
#pragma unroll
      for (int q = 0; q < WORDS; ++q) {
        uint32_t clear = 0;
#pragma unroll
        for (int e = 0; e < PER; ++e)
          if (!((keep >> (q * PER + e)) & 1u)) clear |= (PER == 1 ? 0xFFFFFFFFu : 0xFFFFu << (16 * e));
        w[q] &= ~clear;
      }
      store_words<WORDS>(W_s + g * WORDS, w);
    }
  }
}

// ------------------------------------------------------------------ prune24 + compress24 in one pass
// Each lane takes one (row, pair p) of rows_pad x pairs_pad: groups 2p and
// 2p+1 of the row (columns 8p .. 8p+7), read as one 8- or 16-byte load, and
// writes its 4 kept values and 8 mask bytes (if asked for); the four lanes of
// a metadata word (groups 8w .. 8w+7) OR their nibbles together with shuffles
// and the first writes it.  Without PK the lanes of a wave take 64
// consecutive pairs of one row (one contiguous run in and out).  With PK
// (16-bit, cols % 16 == 0) the 8 bytes of values also go to W_s's tile chunk
// (lanes 2c, 2c+1 of a chunk row fill granule c) and the word to the chunk's
// metadata; rows_pad and pairs_pad cover whole chunks and lanes past the
// matrix write the chunks' zero padding.  There a block takes 16 rows x 16
// pairs (128 columns: two chunk columns), so that its chunk writes are whole
// 128-byte lines (16 rows x 64 bytes of values, 16 rows x 8 bytes of metadata
// per chunk) and so are its value rows (64 values of each row), instead of one
// 64-byte row piece of eight chunks per wave.  The selection is prune24's,
// and with a mask of exactly two per group compress24 keeps those two:
// results equal the two passes (and pack_sparse), bit for bit.
template <typename E, bool PK>
__global__ __launch_bounds__(kThreads) void prune_compress24_kernel(const E* __restrict__ W, int64_t rows,
                                                                   int64_t cols, int64_t rows_pad,
                                                                   int64_t pairs_pad, uint32_t* __restrict__ mask4,
                                                                   E* __restrict__ values, uint32_t* __restrict__ meta,
                                                                   char* __restrict__ packed) {
  typedef typename Vec4<E>::T V;
  const int64_t gpr = cols / 4, wpr = cdiv(gpr, 8);
  const int lane = threadIdx.x & 63;
  // PK: tasks of 16 rows x 16 pairs, one per block and iteration (pairs_pad is
  // a multiple of 8: a last task may reach a chunk column past the matrix,
  // whose lanes store nothing); else the lane's (row, pair) advances by a
  // fixed step each iteration (one division before the loop instead of a
  // 64-bit division per iteration); past the end the row is at least
  // rows_pad, so nothing is stored
  const int64_t total = PK ? (rows_pad / 16) * cdiv(pairs_pad, 16) : rows_pad * pairs_pad;
  const int64_t stride = PK ? (int64_t)gridDim.x : (int64_t)gridDim.x * kThreads;
  const int64_t base0 = PK ? (int64_t)blockIdx.x : (int64_t)blockIdx.x * kThreads + (threadIdx.x & ~63);
  const int cbs = (int)cdiv(pairs_pad, 16);
  const int drow = PK ? 0 : (int)(stride / pairs_pad), dpair = PK ? 0 : (int)(stride - (int64_t)drow * pairs_pad);
  const int npairs = (int)pairs_pad;
  int row = PK ? 0 : (int)((base0 + lane) / pairs_pad), p = PK ? 0 : (int)(base0 + lane - (int64_t)row * pairs_pad);
  // wave-uniform loop bound: every lane of a wave takes part in the shuffles
  for (int64_t base = base0; base < total; base += stride,
               row += drow + (p + dpair >= npairs ? 1 : 0), p += dpair - (p + dpair >= npairs ? npairs : 0)) {
    if constexpr (PK) {
      const int task = (int)base, rb = task / cbs, cb = task - rb * cbs;
      row = rb * 16 + (int)(threadIdx.x >> 4);
      p = cb * 16 + (int)(threadIdx.x & 15);
    }
    const bool slot = PK ? p < npairs : base + lane < total;   // inside rows_pad x pairs_pad
    const int64_t g0 = 2 * (int64_t)p;             // first group of the pair
    const bool in_row = row < rows;
    const int ng = in_row ? (g0 + 2 <= gpr ? 2 : (g0 < gpr ? 1 : 0)) : 0;   // groups of the pair in the matrix
    uint32_t nibs = 0, mb[2] = {0u, 0u};
    E kept[4] = {(E)0, (E)0, (E)0, (E)0};
    if (ng > 0) {
      V v[2];
      const V* src = reinterpret_cast<const V*>(W) + (int64_t)row * gpr + g0;
      v[0] = __builtin_nontemporal_load(src);
      v[1] = __builtin_nontemporal_load(src + (ng > 1 ? 1 : 0));
      if constexpr (sizeof(E) == 2) {
        // both groups ranked at once: element j of group 0 in the low half, of group 1 in the high
        uint32_t w[4], a, b, nib, keep[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          w[j] = __builtin_amdgcn_perm(v[1][j >> 1], v[0][j >> 1], (j & 1) ? 0x07060302u : 0x05040100u);
        top2_of_4_x2<__is_same(E, _Float16)>(w, a, b, nib, keep);
        nibs = (nib & 0xFu) | (ng > 1 ? ((nib >> 12) & 0xF0u) : 0u);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (j < ng)
            mb[j] = ((keep[0] >> (16 * j)) & 1u) | (((keep[1] >> (16 * j)) & 1u) << 8) |
                    (((keep[2] >> (16 * j)) & 1u) << 16) | (((keep[3] >> (16 * j)) & 1u) << 24);
        }
        kept[0] = __builtin_bit_cast(E, (uint16_t)(a & 0xFFFFu));
        kept[1] = __builtin_bit_cast(E, (uint16_t)(b & 0xFFFFu));
        if (ng > 1) {
          kept[2] = __builtin_bit_cast(E, (uint16_t)(a >> 16));
          kept[3] = __builtin_bit_cast(E, (uint16_t)(b >> 16));
        }
      } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        E e[4];
        unpack(v[j], e);
        const uint32_t keep = top2_of_4(mag_key(e[0]), mag_key(e[1]), mag_key(e[2]), mag_key(e[3]));
        const uint32_t nib = pair_nibble(keep);
        const uint32_t i0 = nib & 3u, i1 = nib >> 2;
        if (j < ng) {
          nibs |= nib << (4 * j);
          mb[j] = (keep & 1u) | ((keep & 2u) << 7) | ((keep & 4u) << 14) | ((keep & 8u) << 21);
          kept[2 * j] = i0 == 0 ? e[0] : (i0 == 1 ? e[1] : e[2]);
          kept[2 * j + 1] = i1 == 3 ? e[3] : (i1 == 2 ? e[2] : e[1]);
        }
      }
      }
      E* vp = values + (int64_t)row * (cols / 2) + 2 * g0;
      uint32_t* mp = mask4 ? mask4 + (int64_t)row * gpr + g0 : nullptr;
      constexpr uintptr_t kAlign = 4 * sizeof(E);             // the four kept values in one store
      if (ng == 2 && (reinterpret_cast<uintptr_t>(vp) & (kAlign - 1)) == 0) {
        if constexpr (sizeof(E) == 2)
          *reinterpret_cast<u32x2*>(vp) =
              u32x2{(uint32_t)__builtin_bit_cast(uint16_t, kept[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, kept[1]) << 16),
                    (uint32_t)__builtin_bit_cast(uint16_t, kept[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, kept[3]) << 16)};
        else
          *reinterpret_cast<u32x4*>(vp) = u32x4{(uint32_t)kept[0], (uint32_t)kept[1], (uint32_t)kept[2], (uint32_t)kept[3]};
      } else {
        for (int j = 0; j < 2 * ng; ++j) vp[j] = kept[j];
      }
      if (mp) {
        if (ng == 2 && (reinterpret_cast<uintptr_t>(mp) & 7) == 0)
          *reinterpret_cast<u32x2*>(mp) = u32x2{mb[0], mb[1]};
        else
          for (int j = 0; j < ng; ++j) mp[j] = mb[j];
      }
    }
    // the metadata word of groups 8w .. 8w+7 (w = p / 4) from its four lanes
    uint32_t word = nibs << (8 * (p & 3));
    word |= __shfl_xor(word, 1, 4);
    word |= __shfl_xor(word, 2, 4);
    if ((p & 3) == 0 && in_row && g0 < gpr) meta[row * wpr + (p >> 2)] = word;
    if constexpr (PK) {
      static_assert(sizeof(E) == 2, "tile chunks hold 16-bit values");
      if (slot && 8 * p < cdiv(cols, kPackCols) * kPackCols) {
        const int r = (int)(row % kPackRows), c = (int)((p >> 1) & 3), sw = (r >> 2) & 3;
        char* const chunk = packed + pack_chunk_offset(row, 8 * p, cols);
        const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, kept[0]) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, kept[1]) << 16);
        const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, kept[2]) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, kept[3]) << 16);
        *reinterpret_cast<u32x2*>(chunk + r * 64 + ((c ^ sw) << 4) + (p & 1) * 8) = u32x2{lo, hi};
        if ((p & 3) == 0) *reinterpret_cast<uint32_t*>(chunk + kPackValueBytes + r * 8 + ((p >> 2) & 1) * 4) = word;
      }
    }
  }
}

// ------------------------------------------------------------------ compress24
// Thread slot f -> (row, word, j): eight consecutive lanes build one metadata
// word (groups 8*word .. 8*word+7 of a row) and OR their nibbles together.
template <typename E>
__global__ __launch_bounds__(kThreads) void compress24_kernel(const E* __restrict__ W, const uint8_t* __restrict__ mask,
                                                              int64_t rows, int64_t cols, E* __restrict__ values,
                                                              uint32_t* __restrict__ meta, int32_t* invalid) {
  typedef typename Vec4<E>::T V;
  const int64_t gpr = cols / 4;             // groups per row
  const int64_t wpr = cdiv(gpr, 8);         // metadata words per row
  const int64_t slots = rows * wpr * 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  const int lane = threadIdx.x & 63;
  // wave-uniform loop bound so that every lane of a wave joins the shuffles
  const int64_t wave_base0 = (int64_t)blockIdx.x * kThreads + (threadIdx.x & ~63);
  for (int64_t base = wave_base0; base < slots; base += stride) {
    const int64_t f = base + lane;
    const bool in_range = f < slots;
    const int64_t w = f >> 3;
    const int j = (int)(f & 7);
    const int64_t row = in_range ? w / wpr : 0;
    const int64_t gw = in_range ? w - row * wpr : 0;
    const int64_t g = gw * 8 + j;
    const bool valid = in_range && g < gpr;
    uint32_t nib = 0;
    bool bad = false;
    if (valid) {
      const int64_t gidx = row * gpr + g;   // flat group index
      E e[4];
      unpack(reinterpret_cast<const V*>(W)[gidx], e);
      uint32_t mw = reinterpret_cast<const uint32_t*>(mask)[gidx];
      uint32_t kept = ((mw & 0xFFu) != 0) | (((mw >> 8) & 0xFFu) != 0) << 1 |
                      (((mw >> 16) & 0xFFu) != 0) << 2 | (((mw >> 24) & 0xFFu) != 0) << 3;
      uint32_t sel = kept;
      bad = __builtin_popcount(kept) > 2;
      if (bad) {  // keep the two lowest kept positions
        uint32_t lo = sel & (0u - sel);
        uint32_t rest = sel & ~lo;
        sel = lo | (rest & (0u - rest));
      }
      while (__builtin_popcount(sel) < 2) {  // fill with the lowest unkept positions
        uint32_t un = ~sel & 0xFu;
        sel |= un & (0u - un);
      }
      nib = pair_nibble(sel);
      const uint32_t i0 = nib & 3u, i1 = nib >> 2;
      E v0 = (kept >> i0) & 1u ? e[i0] : (E)0;
      E v1 = (kept >> i1) & 1u ? e[i1] : (E)0;
      values[2 * gidx] = v0;
      values[2 * gidx + 1] = v1;
    }
    uint32_t word = nib << (4 * j);
    word |= __shfl_xor(word, 1, 8);
    word |= __shfl_xor(word, 2, 8);
    word |= __shfl_xor(word, 4, 8);
    if (in_range && j == 0) meta[row * wpr + gw] = word;
    if (invalid) {
      uint64_t b = __ballot(bad);
      if (b && lane == 0) atomicAdd(invalid, (int32_t)__builtin_popcountll(b));
    }
  }
}

// ------------------------------------------------------------------ double prune
// Block tile: 64 rows n of W_s x 128 columns k.  Phase 1 decompresses the tile
// into LDS (one full metadata word, 32 columns, per thread).  Phase 2 gives each
// thread one row k of W_s^T and 32 consecutive n (one output metadata word),
// reads them down an LDS column, prunes 2:4 again and writes compressed rows.
constexpr int DP_TN = 64, DP_TK = 128;

template <typename E>
__global__ __launch_bounds__(kThreads) void double_prune_kernel(const E* __restrict__ vals, const uint32_t* __restrict__ meta,
                                                                int64_t N, int64_t K, E* __restrict__ out_vals,
                                                                uint32_t* __restrict__ out_meta, uint8_t* __restrict__ out_mask) {
  constexpr int PITCH = DP_TK + (sizeof(E) == 2 ? 2 : 1);  // odd word pitch: column reads spread over banks
  __shared__ E tile[DP_TN * PITCH];
  const int tid = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.y * DP_TN;
  const int64_t k0 = (int64_t)blockIdx.x * DP_TK;
  const int64_t in_wpr = cdiv(K / 4, 8), out_wpr = cdiv(N / 4, 8);
  const int64_t in_gpr = K / 4;

  {  // phase 1: decompress W_s[n0 + n][k0 + 32q .. +31]
    const int n = tid >> 2, q = tid & 3;
    const int64_t row = n0 + n;
    E dense[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) dense[i] = (E)0;
    const int64_t gbase = (k0 >> 2) + 8 * q;  // first group of this thread
    if (row < N && gbase < in_gpr) {
      const uint32_t word = meta[row * in_wpr + (gbase >> 3)];
      const E* v = vals + row * (K / 2) + 2 * gbase;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (gbase + i < in_gpr) {
          const uint32_t nib = (word >> (4 * i)) & 0xFu;
          dense[4 * i + (nib & 3u)] = v[2 * i];
          dense[4 * i + (nib >> 2)] = v[2 * i + 1];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) tile[n * PITCH + 32 * q + i] = dense[i];
  }
  __syncthreads();
  {  // phase 2: row k of W_s^T, columns n0 + 32h .. +31
    const int kk = tid & (DP_TK - 1), h = tid >> 7;
    const int64_t krow = k0 + kk;
    const int64_t g0 = (n0 >> 2) + 8 * h;  // first output group of this thread
    if (krow < K && g0 < N / 4) {
      uint32_t word = 0;
      E ov[16];
      uint32_t mbytes[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        E e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) e[j] = tile[(32 * h + 4 * i + j) * PITCH + kk];
        const uint32_t keep = top2_of_4(mag_key(e[0]), mag_key(e[1]), mag_key(e[2]), mag_key(e[3]));
        const uint32_t nib = pair_nibble(keep);
        word |= nib << (4 * i);
        ov[2 * i] = e[nib & 3u];
        ov[2 * i + 1] = e[nib >> 2];
        mbytes[i] = (keep & 1u) | ((keep & 2u) << 7) | ((keep & 4u) << 14) | ((keep & 8u) << 21);
      }
      const int64_t ngroups = N / 4 - g0 < 8 ? N / 4 - g0 : 8;
      if (ngroups < 8) word &= (1u << (4 * ngroups)) - 1u;
      out_meta[krow * out_wpr + (g0 >> 3)] = word;
      E* ovp = out_vals + krow * (N / 2) + 2 * g0;
      for (int i = 0; i < 2 * ngroups; ++i) ovp[i] = ov[i];
      if (out_mask) {
        uint32_t* mp = reinterpret_cast<uint32_t*>(out_mask + krow * N + 4 * g0);
        for (int i = 0; i < ngroups; ++i) mp[i] = mbytes[i];
      }
    }
  }
}

// Wide-access variant for 16-bit values (bf16; fp16 with H) with K % 16 == 0
// and N % 16 == 0.  Block tile: 128 rows n x 128 columns k.  Phase 1: eight lanes per row read one 128-byte
// line of compressed values and the matching metadata words, decompress four
// groups each with selects and write 32 bytes of the dense row to LDS.  Phase
// 2: thread (column pair cp, quarter q) reads rows 32q .. 32q+31 of columns
// 2cp and 2cp+1 as 32-bit words, prunes each column's eight groups of four and
// writes 32 bytes of values, one metadata word (and 32 mask bytes) per column;
// the four quarters of a column are adjacent lanes, so each output row is
// written as one 128-byte run.  LDS rows are 68 words (4 of padding) with word
// w of row n stored at w ^ (16 * ((n / 32) % 4)): both phases are free of bank
// conflicts.
constexpr int DW_T = 128, DW_PITCH = 68;  // tile edge; LDS row pitch in 32-bit words



//
// With UPD the kernel first applies one AdamW step to the compressed values it
// loads (gradient GT, fp32 moments m and v at the same element index), writes
// the new values and moments back in place and double-prunes the new values:
// the optimizer's pass over the weight and the double prune share one read.
//
// With PK the double-pruned W_dp^T goes straight to its tile-chunk form
// (pk_dpT) instead of values / metadata rows: each thread's 16 values of a row
// are two granules of one chunk row and its metadata word one of the row's
// two.  The grid then covers whole 256-row chunks, rows past K written as 0.
// UPD with PK also rewrites the updated values inside W_s's tile chunks
// (pk_s, which holds W_s packed: the mask is static, so only values change).
template <bool UPD, typename GT, bool H = false, bool PK = false>
__global__ __launch_bounds__(kThreads) void double_prune_wide_kernel(uint16_t* vals, const uint32_t* __restrict__ meta,
                                                                    int64_t N, int64_t K,
                                                                    uint16_t* __restrict__ out_vals,
                                                                    uint32_t* __restrict__ out_meta,
                                                                    uint8_t* __restrict__ out_mask,
                                                                    char* __restrict__ pk_dpT,
                                                                    char* __restrict__ pk_s,
                                                                    const GT* __restrict__ grads,
                                                                    float* __restrict__ m, float* __restrict__ v,
                                                                    AdamWStep hp) {
  __shared__ __attribute__((aligned(16))) uint32_t tile[DW_T * DW_PITCH];
  const int tid = threadIdx.x;
  // Workgroups are dealt to the eight XCDs in turn; give each XCD a contiguous
  // range of tiles, k fastest, so that the eight tiles sharing a 128-byte line
  // of metadata (1024 columns of a row) run on one XCD and read it once into
  // its L2 instead of once per XCD.
  const int64_t nb = (int64_t)gridDim.x * gridDim.y, bid = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
  const int64_t per = nb / 8, rem = nb % 8, xcd = bid % 8, slot = bid / 8;
  const int64_t lin = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  const int64_t n0 = (lin / gridDim.x) * DW_T, k0 = (lin % gridDim.x) * DW_T;
  const int64_t in_wpr = cdiv(K / 4, 8), out_wpr = cdiv(N / 4, 8);

  // phase 1: row r, dense columns 16c .. 16c+15 (compressed groups 4c .. 4c+3).
  // The loads of the thread's four rows (and with UPD their gradients and
  // moments) go out first, from clamped addresses: a row or column past the
  // matrix reads a valid element, is zeroed and never stored.  Loads under
  // bounds branches would each be waited for before the next was issued.
  const int c = tid & 7;
  const int64_t kc = k0 + 16 * c;
  const bool col_ok = kc < K;                         // K % 16 == 0: the 16 columns are all in or all out
  const int64_t kcc = col_ok ? kc : K - 16;
  u32x4 w4[4];
  uint32_t nibs[4];
  int64_t el[4];
  bool ok[4];
  float gf[UPD ? 4 : 1][8], mf[UPD ? 4 : 1][8], vf[UPD ? 4 : 1][8];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int64_t row = n0 + it * 32 + (tid >> 3);
    const int64_t rowc = row < N ? row : N - 1;
    ok[it] = row < N && col_ok;
    el[it] = rowc * (K / 2) + kcc / 2;                // the thread's eight compressed values
    w4[it] = *reinterpret_cast<const u32x4*>(vals + el[it]);
    nibs[it] = meta[rowc * in_wpr + (kcc >> 5)] >> (16 * (c & 1));
    if constexpr (UPD) {
      load8_f32(grads + el[it], gf[it]);
      load8_f32(m + el[it], mf[it]);
      load8_f32(v + el[it], vf[it]);
    }
  }
  // byte selectors (v_perm_b32 of a group's word with itself) giving the two
  // dense words of a group from its nibble: position p holds the high value
  // if p == i1, else the low value if p == i0, else 0 (the rule of the
  // selects this replaces, for every nibble)
  __shared__ uint32_t expand_sel[32];
  if (tid < 16) {
    const int i0 = tid & 3, i1 = tid >> 2;
    uint32_t h[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) h[p] = i1 == p ? 0x0302u : (i0 == p ? 0x0100u : 0x0C0Cu);
    expand_sel[2 * tid] = h[0] | (h[1] << 16);
    expand_sel[2 * tid + 1] = h[2] | (h[3] << 16);
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int r = it * 32 + (tid >> 3);
    if constexpr (UPD) {
      typedef Fmt16<H> F;
      u32x4 nw;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = adamw_apply(F::to_f32((uint16_t)(w4[it][i] & 0xFFFFu)), gf[it][2 * i], mf[it][2 * i],
                                     vf[it][2 * i], hp);
        const float hi = adamw_apply(F::to_f32((uint16_t)(w4[it][i] >> 16)), gf[it][2 * i + 1], mf[it][2 * i + 1],
                                     vf[it][2 * i + 1], hp);
        nw[i] = (uint32_t)F::from_f32(lo) | ((uint32_t)F::from_f32(hi) << 16);
      }
      w4[it] = nw;
      if (ok[it]) {
        const int64_t e = el[it];
        *reinterpret_cast<u32x4*>(vals + e) = nw;
        store8_f32(m + e, mf[it]);
        store8_f32(v + e, vf[it]);
        if constexpr (PK) {                           // the same granule of W_s's chunk row
          const int64_t row = n0 + r;
          const int rs = (int)(row % kPackRows), gs = (int)((kc % kPackCols) / 16);
          *reinterpret_cast<u32x4*>(pk_s + pack_chunk_offset(row, kc, K) + rs * 64 + ((gs ^ ((rs >> 2) & 3)) << 4)) = nw;
        }
      }
    }
    const u32x4 wv = ok[it] ? w4[it] : u32x4{0u, 0u, 0u, 0u};
    const uint32_t nb = ok[it] ? nibs[it] : 0u;
    uint32_t d[8];                                    // 16 dense 16-bit values, two per word
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t nib = (nb >> (4 * g)) & 0xFu;
      const u32x2 sel = *reinterpret_cast<const u32x2*>(&expand_sel[2 * nib]);
      d[2 * g] = __builtin_amdgcn_perm(wv[g], wv[g], sel[0]);
      d[2 * g + 1] = __builtin_amdgcn_perm(wv[g], wv[g], sel[1]);
    }
    const int swz = 16 * ((r >> 5) & 3);
    uint32_t* dst = tile + r * DW_PITCH;
    *reinterpret_cast<u32x4*>(dst + ((8 * c) ^ swz)) = u32x4{d[0], d[1], d[2], d[3]};
    *reinterpret_cast<u32x4*>(dst + ((8 * c + 4) ^ swz)) = u32x4{d[4], d[5], d[6], d[7]};
  }
  __syncthreads();

  // phase 2: columns 2cp, 2cp+1 of the tile, rows 32q .. 32q+31
  const int q = tid & 3, cp = tid >> 2;
  uint32_t col[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) col[i] = tile[(32 * q + i) * DW_PITCH + (cp ^ (16 * q))];
  const int64_t g0 = (n0 >> 2) + 8 * q;               // first output group (n / 4)
  const int64_t left = N / 4 - g0;
  const int ngroups = left <= 0 ? 0 : (left < 8 ? (int)left : 8);   // 0, 4 or 8 (N % 16 == 0)
  // both columns' groups at once (column 2cp in the low halves, 2cp+1 in the high)
  uint32_t words[2] = {0u, 0u}, ovs[2][8], mws[2][8];
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    uint32_t a, b, nib, keep[4];
    top2_of_4_x2<H>(&col[4 * g], a, b, nib, keep);
    words[0] |= (nib & 0xFu) << (4 * g);
    words[1] |= ((nib >> 16) & 0xFu) << (4 * g);
    ovs[0][g] = (a & 0xFFFFu) | (b << 16);
    ovs[1][g] = (a >> 16) | (b & 0xFFFF0000u);
    if constexpr (!PK) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        mws[h][g] = ((keep[0] >> (16 * h)) & 1u) | (((keep[1] >> (16 * h)) & 1u) << 8) |
                    (((keep[2] >> (16 * h)) & 1u) << 16) | (((keep[3] >> (16 * h)) & 1u) << 24);
    }
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t krow = k0 + 2 * cp + h;
    const bool live = krow < K && ngroups > 0;
    if (!PK && !live) continue;
    uint32_t word = words[h];
    const uint32_t* ov = ovs[h];
    const uint32_t* mw = mws[h];
    if (ngroups < 8) word &= 0xFFFFu;
    if constexpr (PK) {
      // chunk row krow % 256 of the chunk holding dense columns 4 g0 ..; groups
      // g0 .. g0+7 are its granules 2w, 2w+1 and metadata word w (w = (g0 / 8) % 2)
      if (g0 * 4 >= cdiv(N, kPackCols) * kPackCols) continue;        // past the last chunk column
      const bool hi = live && ngroups == 8;
      const int r = (int)(krow % kPackRows), w = (int)((g0 >> 3) & 1), sw = (r >> 2) & 3;
      char* const row_base = pk_dpT + pack_chunk_offset(krow, g0 * 4, N) + r * 64;
      *reinterpret_cast<u32x4*>(row_base + (((2 * w) ^ sw) << 4)) =
          live ? u32x4{ov[0], ov[1], ov[2], ov[3]} : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(row_base + (((2 * w + 1) ^ sw) << 4)) =
          hi ? u32x4{ov[4], ov[5], ov[6], ov[7]} : u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<uint32_t*>(pk_dpT + pack_chunk_offset(krow, g0 * 4, N) + kPackValueBytes + r * 8 + w * 4) =
          live ? word : 0u;
    } else {
      out_meta[krow * out_wpr + (g0 >> 3)] = word;
      uint32_t* ovp = reinterpret_cast<uint32_t*>(out_vals + krow * (N / 2) + 2 * g0);
      *reinterpret_cast<u32x4*>(ovp) = u32x4{ov[0], ov[1], ov[2], ov[3]};
      if (ngroups == 8) *reinterpret_cast<u32x4*>(ovp + 4) = u32x4{ov[4], ov[5], ov[6], ov[7]};
      if (out_mask) {
        uint32_t* mp = reinterpret_cast<uint32_t*>(out_mask + krow * N + 4 * g0);
        *reinterpret_cast<u32x4*>(mp) = u32x4{mw[0], mw[1], mw[2], mw[3]};
        if (ngroups == 8) *reinterpret_cast<u32x4*>(mp + 4) = u32x4{mw[4], mw[5], mw[6], mw[7]};
      }
    }
  }
}

int grid_for(int64_t work, int per_block) {
  int64_t b = cdiv(work, per_block);
  const int64_t cap = 256 * 32;  // enough waves in flight on 256 CUs
  return (int)(b < 1 ? 1 : (b > cap ? cap : b));
}

}  // namespace

hipError_t launch_prune24(Dt dt, const void* W, int64_t rows, int64_t cols, uint8_t* mask, void* W_s,
                          hipStream_t s) {
  const int64_t groups = rows * cols / 4;
  if (groups == 0) return hipSuccess;
  constexpr int U = 4;
  const int grid = grid_for(groups, kThreads * U);
  if (dt == Dt::BF16)
    prune24_kernel<uint16_t, U><<<grid, kThreads, 0, s>>>((const uint16_t*)W, groups, (uint32_t*)mask, (uint16_t*)W_s);
  else if (dt == Dt::F16)
    prune24_kernel<_Float16, U><<<grid, kThreads, 0, s>>>((const _Float16*)W, groups, (uint32_t*)mask, (_Float16*)W_s);
  else
    prune24_kernel<uint32_t, U><<<grid, kThreads, 0, s>>>((const uint32_t*)W, groups, (uint32_t*)mask, (uint32_t*)W_s);
  return hipGetLastError();
}

template <typename E>
hipError_t prune_nm_dispatch(const void* W, int64_t groups, int n, int m, uint8_t* mask, void* W_s, hipStream_t s) {
  const int grid = grid_for(groups, kThreads);
  const uint32_t* w = (const uint32_t*)W;
  uint32_t* mk = (uint32_t*)mask;
  uint32_t* ws = (uint32_t*)W_s;
  switch (m) {
    case 4: prune_nm_kernel<E, 4><<<grid, kThreads, 0, s>>>(w, groups, n, mk, ws); break;
    case 8: prune_nm_kernel<E, 8><<<grid, kThreads, 0, s>>>(w, groups, n, mk, ws); break;
    case 16: prune_nm_kernel<E, 16><<<grid, kThreads, 0, s>>>(w, groups, n, mk, ws); break;
    case 32: prune_nm_kernel<E, 32><<<grid, kThreads, 0, s>>>(w, groups, n, mk, ws); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prune_nm(Dt dt, const void* W, int64_t rows, int64_t cols, int n, int m, uint8_t* mask, void* W_s,
                           hipStream_t s) {
  const int64_t groups = rows * (cols / m);
  if (groups == 0) return hipSuccess;
  if (dt == Dt::BF16) return prune_nm_dispatch<uint16_t>(W, groups, n, m, mask, W_s, s);
  if (dt == Dt::F16) return prune_nm_dispatch<_Float16>(W, groups, n, m, mask, W_s, s);
  return prune_nm_dispatch<uint32_t>(W, groups, n, m, mask, W_s, s);
}

hipError_t launch_compress24(Dt dt, const void* W, const uint8_t* mask, int64_t rows, int64_t cols, void* values,
                             uint32_t* meta, int32_t* invalid, hipStream_t s) {
  const int64_t slots = rows * cdiv(cols / 4, 8) * 8;
  if (slots == 0) return hipSuccess;
  const int grid = grid_for(slots, kThreads);
  if (dt == Dt::BF16)
    compress24_kernel<uint16_t><<<grid, kThreads, 0, s>>>((const uint16_t*)W, mask, rows, cols, (uint16_t*)values, meta, invalid);
  else if (dt == Dt::F16)
    compress24_kernel<_Float16><<<grid, kThreads, 0, s>>>((const _Float16*)W, mask, rows, cols, (_Float16*)values, meta, invalid);
  else
    compress24_kernel<uint32_t><<<grid, kThreads, 0, s>>>((const uint32_t*)W, mask, rows, cols, (uint32_t*)values, meta, invalid);
  return hipGetLastError();
}

namespace {

// The wide double prune over a [N, K] W_s (16-bit, K % 16 == 0, N % 16 == 0):
// canonical W_dp^T rows, or (PK) W_dp^T tile chunks over whole 256-row chunks.
template <bool UPD, typename GT, bool H, bool PK>
hipError_t dp_wide(uint16_t* vals, const uint32_t* meta, int64_t N, int64_t K, uint16_t* out_vals,
                   uint32_t* out_meta, uint8_t* out_mask, char* pk_dpT, char* pk_s, const void* grads, float* m,
                   float* v, const AdamWStep& c, hipStream_t s) {
  const int64_t ktiles = PK ? cdiv(K, kPackRows) * (kPackRows / DW_T) : cdiv(K, DW_T);
  dim3 g((unsigned)ktiles, (unsigned)cdiv(N, DW_T));
  double_prune_wide_kernel<UPD, GT, H, PK><<<g, kThreads, 0, s>>>(vals, meta, N, K, out_vals, out_meta, out_mask,
                                                                 pk_dpT, pk_s, (const GT*)grads, m, v, c);
  return hipGetLastError();
}

template <bool UPD, bool H, bool PK>
hipError_t dp_wide_grad(Dt grad, uint16_t* vals, const uint32_t* meta, int64_t N, int64_t K, uint16_t* out_vals,
                        uint32_t* out_meta, uint8_t* out_mask, char* pk_dpT, char* pk_s, const void* grads,
                        float* m, float* v, const AdamWStep& c, hipStream_t s) {
  if (!UPD || grad == Dt::BF16)
    return dp_wide<UPD, uint16_t, H, PK>(vals, meta, N, K, out_vals, out_meta, out_mask, pk_dpT, pk_s, grads, m, v,
                                         c, s);
  if (grad == Dt::F16)
    return dp_wide<UPD, _Float16, H, PK>(vals, meta, N, K, out_vals, out_meta, out_mask, pk_dpT, pk_s, grads, m, v,
                                         c, s);
  return dp_wide<UPD, float, H, PK>(vals, meta, N, K, out_vals, out_meta, out_mask, pk_dpT, pk_s, grads, m, v, c,
                                    s);
}

template <bool UPD, bool PK>
hipError_t dp_wide_dt(Dt dt, Dt grad, void* vals, const uint32_t* meta, int64_t N, int64_t K, void* out_vals,
                      uint32_t* out_meta, uint8_t* out_mask, void* pk_dpT, void* pk_s, const void* grads, float* m,
                      float* v, const AdamWStep& c, hipStream_t s) {
  if (dt == Dt::F16)
    return dp_wide_grad<UPD, true, PK>(grad, (uint16_t*)vals, meta, N, K, (uint16_t*)out_vals, out_meta, out_mask,
                                       (char*)pk_dpT, (char*)pk_s, grads, m, v, c, s);
  return dp_wide_grad<UPD, false, PK>(grad, (uint16_t*)vals, meta, N, K, (uint16_t*)out_vals, out_meta, out_mask,
                                      (char*)pk_dpT, (char*)pk_s, grads, m, v, c, s);
}

bool wide_ok(Dt dt, int64_t N, int64_t K) { return dt != Dt::F32 && K % 16 == 0 && N % 16 == 0; }

}  // namespace

hipError_t launch_prune_compress24(Dt dt, const void* W, int64_t rows, int64_t cols, uint8_t* mask, void* values,
                                   uint32_t* meta, void* packed, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  // group pairs per row, four per metadata word; with packed output whole
  // 256-row chunks and eight pairs per chunk column
  const int64_t rows_pad = packed ? cdiv(rows, kPackRows) * kPackRows : rows;
  const int64_t words_pad = packed ? 4 * 2 * cdiv(cols, kPackCols) : 4 * cdiv(cols / 4, 8);
  // with chunks, one block per task of 16 rows x 16 pairs
  const int grid = packed ? grid_for((rows_pad / 16) * cdiv(words_pad, 16), 1) : grid_for(rows_pad * words_pad, kThreads);
  uint32_t* m4 = (uint32_t*)mask;
  char* pk = (char*)packed;
  if (dt == Dt::F32) {
    prune_compress24_kernel<uint32_t, false><<<grid, kThreads, 0, s>>>((const uint32_t*)W, rows, cols, rows_pad,
                                                                       words_pad, m4, (uint32_t*)values, meta, nullptr);
  } else if (dt == Dt::F16) {
    if (packed)
      prune_compress24_kernel<_Float16, true><<<grid, kThreads, 0, s>>>((const _Float16*)W, rows, cols, rows_pad,
                                                                        words_pad, m4, (_Float16*)values, meta, pk);
    else
      prune_compress24_kernel<_Float16, false><<<grid, kThreads, 0, s>>>((const _Float16*)W, rows, cols, rows_pad,
                                                                         words_pad, m4, (_Float16*)values, meta, nullptr);
  } else {
    if (packed)
      prune_compress24_kernel<uint16_t, true><<<grid, kThreads, 0, s>>>((const uint16_t*)W, rows, cols, rows_pad,
                                                                        words_pad, m4, (uint16_t*)values, meta, pk);
    else
      prune_compress24_kernel<uint16_t, false><<<grid, kThreads, 0, s>>>((const uint16_t*)W, rows, cols, rows_pad,
                                                                         words_pad, m4, (uint16_t*)values, meta, nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_double_prune(Dt dt, const void* values_s, const uint32_t* meta_s, int64_t N, int64_t K,
                               void* values_dpT, uint32_t* meta_dpT, uint8_t* mask_dpT, hipStream_t s) {
  if (N == 0 || K == 0) return hipSuccess;
  if (wide_ok(dt, N, K))
    return dp_wide_dt<false, false>(dt, dt, const_cast<void*>(values_s), meta_s, N, K, values_dpT, meta_dpT,
                                    mask_dpT, nullptr, nullptr, nullptr, nullptr, nullptr, AdamWStep{}, s);
  dim3 grid((unsigned)cdiv(K, DP_TK), (unsigned)cdiv(N, DP_TN));
  if (dt == Dt::BF16)
    double_prune_kernel<uint16_t><<<grid, kThreads, 0, s>>>((const uint16_t*)values_s, meta_s, N, K, (uint16_t*)values_dpT,
                                                            meta_dpT, mask_dpT);
  else if (dt == Dt::F16)
    double_prune_kernel<_Float16><<<grid, kThreads, 0, s>>>((const _Float16*)values_s, meta_s, N, K, (_Float16*)values_dpT,
                                                            meta_dpT, mask_dpT);
  else
    double_prune_kernel<uint32_t><<<grid, kThreads, 0, s>>>((const uint32_t*)values_s, meta_s, N, K, (uint32_t*)values_dpT,
                                                            meta_dpT, mask_dpT);
  return hipGetLastError();
}

hipError_t launch_double_prune_packed(Dt dt, const void* values_s, const uint32_t* meta_s, int64_t N, int64_t K,
                                      void* packed_dpT, hipStream_t s) {
  if (N == 0 || K == 0) return hipSuccess;
  return dp_wide_dt<false, true>(dt, dt, const_cast<void*>(values_s), meta_s, N, K, nullptr, nullptr, nullptr,
                                 packed_dpT, nullptr, nullptr, nullptr, nullptr, AdamWStep{}, s);
}

hipError_t launch_adamw_double_prune(Dt dt, Dt grad, void* values_s, const uint32_t* meta_s, const void* grads,
                                     float* m, float* v, int64_t N, int64_t K, const AdamWStep& c,
                                     void* values_dpT, uint32_t* meta_dpT, uint8_t* mask_dpT, hipStream_t s) {
  if (N == 0 || K == 0) return hipSuccess;
  if (wide_ok(dt, N, K))
    return dp_wide_dt<true, false>(dt, grad, values_s, meta_s, N, K, values_dpT, meta_dpT, mask_dpT, nullptr,
                                   nullptr, grads, m, v, c, s);
  // other shapes and fp32 weights: the elementwise update, then the double prune
  hipError_t e = launch_adamw(dt, grad, values_s, grads, m, v, N * (K / 2), c, s);
  if (e != hipSuccess) return e;
  return launch_double_prune(dt, values_s, meta_s, N, K, values_dpT, meta_dpT, mask_dpT, s);
}

hipError_t launch_adamw_double_prune_packed(Dt dt, Dt grad, void* values_s, const uint32_t* meta_s,
                                            const void* grads, float* m, float* v, int64_t N, int64_t K,
                                            const AdamWStep& c, void* packed_s, void* packed_dpT, hipStream_t s) {
  if (N == 0 || K == 0) return hipSuccess;
  return dp_wide_dt<true, true>(dt, grad, values_s, meta_s, N, K, nullptr, nullptr, nullptr, packed_dpT, packed_s,
                                grads, m, v, c, s);
}

}  // namespace slope

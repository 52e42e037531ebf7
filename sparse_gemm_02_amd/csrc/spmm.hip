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
#include "dma.h"
#include "gemm_tile.h"

namespace slope {

hipError_t launch_spmm_generic(Dt in, Dt out, const void* B, int64_t T, int64_t Kred, const void* values,
                               const uint32_t* meta, int64_t M, const float* xl, int splits, int64_t r,
                               const void* R, void* Y, hipStream_t s);

namespace {

// ------------------------------------------------------------------ main kernel
// Requirements (checked on the host): Kred % 16 == 0, M % 4 == 0, 16-byte
// aligned base pointers.  Operands stream through a ring of NST LDS stages
// filled by buffer loads that write LDS directly; rows past M or T and k past
// Kred read as 0 through the resources' bounds, so every load is unconditional.
//
// Each stage covers 64 dense k: a 64-byte segment of every compressed A row
// and a 128-byte segment of every B row, so each row of the tile costs one
// cache line per stage.  The metadata of a row (4 bytes per 32 k) comes four
// words at a time, every second stage.
//
// LDS granule swizzles keep fragment reads free of bank conflicts (measured on
// gfx950: 64 four-byte banks, a 128-bit read serves 16 lanes per pass, so the
// 16 rows of a pass must hit distinct 16-byte granules modulo 256 bytes):
// A row r keeps 16-byte granule c at c ^ ((r>>2)&3), B row r keeps granule c
// at c ^ ((r^(r>>3))&7).
//
// Schedule per stage s (one barrier): read the second k-step's fragments of s,
// issue the first k-step's MFMAs, wait for this wave's LDS reads and for stage
// s+1, barrier, read the first k-step's fragments of s+1, issue the second
// k-step's MFMAs with the loads of stage s+NST (into the slot stage s used,
// whose fragments are all in registers by then) placed among them.  NST-1
// stages stay in flight through most of the loop.  The metadata ring of two
// slots (four stages) holds stages s .. s+3, which needs NST == 3.  Each lane
// reads its own 16-bit half of a metadata word, so the index operand needs no
// shift.
//
// PK: the sparse operand comes as tile chunks (see pack_sparse_kernel): each
// stage loads one contiguous 18 KB chunk (values then metadata) instead of 256
// separate 64-byte row pieces and a strided metadata read.
//
// Block `bid` of `nblocks` computes one tile of the row tiles tm0 .. tm0 +
// tiles_m - 1 (BM rows each), any column tile.  A product whose full-width
// tiles would end in a partly filled round of blocks gives its last row tiles
// narrower tiles in the same launch (spmm_split_kernel).  Each output
// accumulates over k in the same order whatever the tile width, so the split
// does not change results.
// The adapter term of a tile, (X . L) . R added to its accumulators, with the
// operands staged through LDS: once the main loop is done the operand ring is
// idle, so the tile's rows of R^T and of X . L (hi and lo parts) come in by
// buffer-to-LDS loads, SL rank slices of 16 columns at a time: one round trip
// per chunk (one in all up to rank 96) instead of one per 16-deep rank step.
// A slice holds 32 bytes per row, the BM rows of R^T then the BT rows of the
// hi and the lo part; a lane reads its 16-byte half of a row, so eight
// consecutive lanes touch distinct banks.  The MFMAs are adapter_mma's, in the
// same order, so the results are identical.
template <class G, bool H, int LDS_AVAIL>
__device__ __forceinline__ void adapter_mma_lds(f32x16 (&acc)[G::FM][G::FT], char* lds,
                                                const uint16_t* __restrict__ rt, const uint16_t* __restrict__ xlh,
                                                const uint16_t* __restrict__ xll, int rpad, int64_t m0, int64_t t0,
                                                int wm, int wt, int wave, int lane) {
  typedef Fmt16<H> F;
  typedef typename F::v8 v8;
  constexpr int ROWS = G::BM + 2 * G::BT;
  constexpr int SLICE_BYTES = ROWS * 32, BLOCKS = ROWS / 32;   // 1 KB loads per slice
  constexpr int SL_FIT = LDS_AVAIL / SLICE_BYTES;
  constexpr int SL = SL_FIT < 8 ? SL_FIT : 8;
  static_assert(SL >= 1 && G::BM % 32 == 0 && G::BT % 32 == 0, "adapter slices fit the LDS ring");
  // the padded R^T [Mpad][rpad] and X . L [Tpad][rpad] hold every row of the tile
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(rt + m0 * rpad, (int64_t)G::BM * rpad * 2);
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(xlh + t0 * rpad, (int64_t)G::BT * rpad * 2);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(xll + t0 * rpad, (int64_t)G::BT * rpad * 2);
  const uint32_t pitch = (uint32_t)rpad * 2;
  const uint32_t lrow = (uint32_t)(lane >> 1), lhalf = (uint32_t)(lane & 1) * 16;
  const int slices = rpad / 16;
  for (int q0 = 0; q0 < slices; q0 += SL) {
    const int nq = slices - q0 < SL ? slices - q0 : SL;
    barrier();                                       // no wave reads the ring (or the last chunk) any more
    compiler_fence();
    for (int b = wave; b < nq * BLOCKS; b += G::WAVES) {
      const int q = b / BLOCKS, rb = b % BLOCKS;     // wave-uniform
      const uint32_t col = (uint32_t)(q0 + q) * 32 + lhalf;
      char* dst = lds + b * 1024;
      if (rb * 32 < G::BM)
        dma16(rr, dst, (rb * 32 + lrow) * pitch + col);
      else if (rb * 32 < G::BM + G::BT)
        dma16(rh, dst, (rb * 32 - G::BM + lrow) * pitch + col);
      else
        dma16(rl, dst, (rb * 32 - G::BM - G::BT + lrow) * pitch + col);
    }
    compiler_fence();
    wait_vmcnt<0>();                                 // this wave's slices landed
    barrier();                                       // everyone's
    compiler_fence();
    for (int q = 0; q < nq; ++q) {
      const char* base = lds + q * SLICE_BYTES + 16 * (lane >> 5);
      v8 ra[G::FM];
#pragma unroll
      for (int fm = 0; fm < G::FM; ++fm)
        ra[fm] = *reinterpret_cast<const v8*>(base + (wm * G::WM + fm * 32 + (lane & 31)) * 32);
#pragma unroll
      for (int ft = 0; ft < G::FT; ++ft) {
        const int tr = wt * G::WT + ft * 32 + (lane & 31);
        const v8 xh = *reinterpret_cast<const v8*>(base + (G::BM + tr) * 32);
        const v8 xo = *reinterpret_cast<const v8*>(base + (G::BM + G::BT + tr) * 32);
#pragma unroll
        for (int fm = 0; fm < G::FM; ++fm) {
          acc[fm][ft] = F::mfma32x32x16(ra[fm], xh, acc[fm][ft]);
          acc[fm][ft] = F::mfma32x32x16(ra[fm], xo, acc[fm][ft]);
        }
      }
    }
  }
}

// Token chunks of the dense operand (the layout pack_tokens_kernel writes:
// chunk (c, g) holds columns 256c .. 256c+255 as rows x tokens 32g .. 32g+31,
// 64-byte rows of four 16-byte granules of 8 tokens, granule j stored at
// j ^ ((row >> 2) & 3)), written from a stage's B slice in LDS: the stage's 64
// k are rows 64 (s % 4) .. of chunk column s / 4.  Wave w takes the tile's
// token group w, lane l the chunk row of k = l.  The gfx950 transposing LDS
// load does the transpose: in each group of 16 lanes, lane j names four
// consecutive k of token row t + j/4, and lane i receives k = c + i of tokens
// t .. t+3 (measured; see the weight-gradient kernels), so two loads give a
// lane the 8 tokens of one granule of its row.  The writer of the last stage
// also writes the rows of the last chunk column that no stage covers as zeros.
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <class G>
__device__ __forceinline__ void store_token_chunks(const char* __restrict__ bslot, uint16_t* __restrict__ chunks,
                                                   int s, int stages, int64_t t0, int64_t Tch, int lane_in,
                                                   int wave_in) {
  // Everything below is computed here, in the rare branch that calls this,
  // rather than hoisted into the main loop's registers: the lane index passes
  // through an empty asm statement the compiler cannot see through.
  int lane = lane_in;
  asm volatile("" : "+v"(lane));
  const int wave = __builtin_amdgcn_readfirstlane(wave_in);
  if (wave >= G::BT / 32) return;
  const int64_t gt = t0 / 32 + wave;
  if (gt >= Tch) return;
  const int r = 64 * (s & 3) + lane;
  uint16_t* row = chunks + ((int64_t)(s >> 2) * Tch + gt) * 8192 + r * 32;
  // the address this lane supplies: token 32w + 8j + 4h + rl, k 16 (l/16) + 4 (l%4);
  // B row t keeps granule c at c ^ ((t ^ (t >> 3)) & 7) = c ^ (4h + rl) ^ ((4w + j) & 7)
  const int rl = (lane & 15) >> 2;
  const int gsel = (2 * (lane >> 4) + ((lane >> 1) & 1)) ^ rl;
  const char* base = bslot + (32 * wave + rl) * 128 + 8 * (lane & 1);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = (4 * wave + j) & 7;
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 8 * j * 128 + ((gsel ^ q) << 4)));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(base + (8 * j + 4) * 128 + ((gsel ^ q ^ 4) << 4)));
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    *reinterpret_cast<u32x4*>(row + 8 * (j ^ ((r >> 2) & 3))) = u32x4{ua[0], ua[1], ub[0], ub[1]};
  }
  if (s == stages - 1) {
    for (int rz = 64 * ((s & 3) + 1) + lane; rz < 256; rz += 64) {
      uint16_t* zr = row + (rz - r) * 32;
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(zr + 8 * j) = u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// Row tiles per group of the XCD-aware tile order (tile_map.h).  With few row
// tiles every XCD's 32 blocks take 8 rows x 4 columns, the fewest operand
// bytes per stage.  With many row tiles the weight (several hundred MB) no
// longer stays in the infinity cache while the dense operand does, and
// narrower groups, each row tile's stages fetched in fewer rounds, measured
// faster on the OPT-66B shapes: 108 row tiles (QKV forward) 2.71 -> 2.61 ms
// with four rows, 144 (FC1 forward, FC2 dX) 3.57 -> 3.39 ms with six, where
// each XCD's share of the grid is a whole number of six-row groups (four
// rows: 3.48 ms).  36 row tiles lose 1-2% with four or six rows.
__device__ __forceinline__ int spmm_group(int nblocks, int tiles_m, int tiles_t) {
  if (tiles_m < 72) return 8;
  const int per_xcd = nblocks % 8 == 0 ? nblocks / 8 : 0;
  return per_xcd > 0 && per_xcd % (6 * tiles_t) == 0 ? 6 : 4;
}

template <class G, bool ADAPTER, typename O, bool PK, bool H, bool TOK>
__device__ __forceinline__ void spmm_tile(const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ vals,
                                          const uint32_t* __restrict__ meta, int M, int T, int Kred,
                                          const uint16_t* __restrict__ rt, const uint16_t* __restrict__ xlh,
                                          const uint16_t* __restrict__ xll, int rpad, O* __restrict__ Y, int bid,
                                          int nblocks, int tm0, int tiles_m, uint16_t* __restrict__ tok,
                                          int64_t Tch, int pack_rows) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % G::WGM, wt = wave / G::WGM;
  const int tiles_t = (T + G::BT - 1) / G::BT;
  int tm, tt;
  tile_of_block(bid, nblocks, tiles_m, tiles_t, spmm_group(nblocks, tiles_m, tiles_t), tm, tt);
  // token chunks: row tiles 0 .. pack_rows - 1 of this geometry share the
  // stages of each token tile, stage s going to row tile (s + tt) % pack_rows
  // (TOK: a separate instantiation, so that the plain product keeps its registers)
  int next_store = 0x7fffffff;
  if (TOK && tm < pack_rows) next_store = ((tm - tt) % pack_rows + pack_rows) % pack_rows;
  tm += tm0;
  static_assert(PK || G::NST == 3, "metadata ring holds four stages");
  constexpr int SLOT = PK ? G::PSTAGE_BYTES : G::STAGE_BYTES;
  const int64_t m0 = (int64_t)tm * G::BM, t0 = (int64_t)tt * G::BT;
  const int wpr = (Kred / 4 + 7) / 8;               // metadata words per row
  const int stages = (Kred + G::KS - 1) / G::KS;
  const int rows_m = (int)((M - m0) < G::BM ? (M - m0) : G::BM);
  const int rows_t = (int)((T - t0) < G::BT ? (T - t0) : G::BT);

  // resources cover exactly this block's valid rows
  const __amdgpu_buffer_rsrc_t ra =
      PK ? make_rsrc(vals + (int64_t)tm * stages * (G::CHUNK_BYTES / 2), (int64_t)stages * G::CHUNK_BYTES)
         : make_rsrc(vals + m0 * (Kred / 2), (int64_t)rows_m * Kred);
  const __amdgpu_buffer_rsrc_t rmeta = make_rsrc(meta + m0 * wpr, (int64_t)rows_m * wpr * 4);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(Bm + t0 * Kred, (int64_t)rows_t * Kred * 2);

  char* const meta_lds = lds + G::NST * G::STAGE_BYTES;
  // per-lane DMA sources (stage 0); stage s adds s*64 (A) / s*128 (B) bytes
  uint32_t a_src[G::A_DMA], b_src[G::B_DMA];
  int a_k[G::A_DMA], b_k[G::B_DMA];
#pragma unroll
  for (int j = 0; j < G::A_DMA; ++j) {
    const int row = wave * (G::BM / G::WAVES) + j * 16 + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    a_src[j] = (uint32_t)row * Kred + c * 16;
    a_k[j] = c * 16;                                // compressed bytes of the granule within the stage
  }
#pragma unroll
  for (int j = 0; j < G::B_DMA; ++j) {
    const int row = wave * (G::BT / G::WAVES) + j * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row ^ (row >> 3)) & 7);
    b_src[j] = (uint32_t)row * Kred * 2 + c * 16;
    b_k[j] = c * 8;                                 // first k of the granule within the stage
  }
  const uint32_t m_src = (uint32_t)(wave * 64 + lane) * wpr * 4;   // waves < META_WAVES

  auto issue = [&](int s) {
    char* base = lds + (s % G::NST) * SLOT;
    const uint32_t chunk = (uint32_t)s * G::CHUNK_BYTES;           // PK: this stage's chunk
#pragma unroll
    for (int j = 0; j < G::A_DMA; ++j) {
      const uint32_t part = wave * (G::A_BYTES / G::WAVES) + j * 1024;
      if (PK) {
        dma16(ra, base + part, s < stages ? chunk + part + lane * 16 : kOutOfRange);
      } else {
        const bool ok = s * 64 + a_k[j] < Kred;      // compressed bytes of a row = Kred
        dma16(ra, base + part, ok ? a_src[j] + s * 64 : kOutOfRange);
      }
    }
#pragma unroll
    for (int j = 0; j < G::B_DMA; ++j) {
      const bool ok = s * 64 + b_k[j] < Kred;
      dma16(rb, base + G::A_BYTES + wave * (G::B_BYTES / G::WAVES) + j * 1024, ok ? b_src[j] + s * 128 : kOutOfRange);
    }
    if (PK) {                                        // the stage's metadata words
      dma4(ra, base + G::A_BYTES + G::B_BYTES + wave * 256,
           s < stages ? chunk + G::A_BYTES + wave * 256 + lane * 4 : kOutOfRange);
    } else if ((s & 1) == 0 && wave < G::META_WAVES) {      // words 2s .. 2s+3 of every row
      const bool ok = 2 * s < wpr;
      dma16(rmeta, meta_lds + ((s >> 1) & 1) * G::META_SLOT + wave * 1024, ok ? m_src + s * 8 : kOutOfRange);
    } else {                                         // placeholder: same load count on every wave and stage
      dma4(rmeta, meta_lds + G::META_BYTES + wave * 256, kOutOfRange);
    }
  };

  // per-lane fragment offsets inside a stage (k-step ks adds nothing to the
  // row, only selects granules)
  int a_off[2][G::FM], m_off[G::FM], b_off[2][G::FT][2];
#pragma unroll
  for (int fm = 0; fm < G::FM; ++fm) {
    const int row = wm * G::WM + fm * 32 + (lane & 31);
    const int sw = (row >> 2) & 3;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) a_off[ks][fm] = row * 64 + (((2 * ks + (lane >> 5)) ^ sw) * 16);
    m_off[fm] = row * (PK ? 8 : 16) + 2 * (lane >> 5);   // this lane's 16-bit half of the word
  }
#pragma unroll
  for (int ft = 0; ft < G::FT; ++ft) {
    const int row = wt * G::WT + ft * 32 + (lane & 31);
    const int sw = (row ^ (row >> 3)) & 7;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      b_off[ks][ft][0] = G::A_BYTES + row * 128 + (((4 * ks + (lane >> 5)) ^ sw) * 16);
      b_off[ks][ft][1] = G::A_BYTES + row * 128 + (((4 * ks + 2 + (lane >> 5)) ^ sw) * 16);
    }
  }

  struct Frags {
    typename Fmt16<H>::v8 a[G::FM];
    int ix[G::FM];
    typename Fmt16<H>::v16 b[G::FT];
  };
  auto read_frags = [&](Frags& f, int s, int ks) {
    const char* base = lds + (s % G::NST) * SLOT;
    const char* mbase = PK ? base + G::A_BYTES + G::B_BYTES + ks * 4
                           : meta_lds + ((s >> 1) & 1) * G::META_SLOT + ((s & 1) * 2 + ks) * 4;
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm) {
      f.a[fm] = *reinterpret_cast<const typename Fmt16<H>::v8*>(base + a_off[ks][fm]);
      f.ix[fm] = (int)*reinterpret_cast<const uint16_t*>(mbase + m_off[fm]);
    }
#pragma unroll
    for (int ft = 0; ft < G::FT; ++ft) {
      const typename Fmt16<H>::v8 lo = *reinterpret_cast<const typename Fmt16<H>::v8*>(base + b_off[ks][ft][0]);
      const typename Fmt16<H>::v8 hi = *reinterpret_cast<const typename Fmt16<H>::v8*>(base + b_off[ks][ft][1]);
      f.b[ft] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
    }
  };

  f32x16 acc[G::FM][G::FT];
#pragma unroll
  for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
    for (int ft = 0; ft < G::FT; ++ft) acc[fm][ft] = f32x16{};
  auto mma_col = [&](const Frags& f, int ft) {
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm)
      acc[fm][ft] = Fmt16<H>::smfmac32x32x32(f.a[fm], f.b[ft], acc[fm][ft], f.ix[fm]);
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int ft = 0; ft < G::FT; ++ft) mma_col(f, ft);
  };

  // prologue: stages 0 .. NST-1 in flight; stage 0 landed and visible
#pragma unroll
  for (int p = 0; p < G::NST; ++p) issue(p);
  wait_vmcnt<G::DMA_PER_STAGE * (G::NST - 1)>();
  barrier();
  compiler_fence();                                   // the first LDS reads stay after the barrier
  Frags f0, f1;
  read_frags(f0, 0, 0);
  for (int s = 0; s < stages; ++s) {
    read_frags(f1, s, 1);
    mma(f0);
    // keep the first k-step's MFMAs ahead of the waits: they run meanwhile
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (TOK) {
      if (s == next_store) {                          // block-uniform; before the slot is refilled
        store_token_chunks<G>(lds + (s % G::NST) * SLOT + G::A_BYTES, tok, s, stages, t0, Tch, lane, wave);
        next_store += pack_rows;
      }
    }
    wait_lgkmcnt0();                                  // this wave's reads of stage s are in registers
    wait_vmcnt<G::DMA_PER_STAGE * (G::NST - 2)>();   // this wave's loads of stage s+1 landed
    barrier();                                        // everyone's have; stage s fully read
    if (s + 1 < stages) read_frags(f0, s + 1, 0);
    // the second k-step's MFMAs need nothing from the barrier: start them, and
    // refill stage s's slot while they run (past the end these loads read 0)
    mma_col(f1, 0);
    __builtin_amdgcn_sched_barrier(0);
    issue(s + G::NST);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ft = 1; ft < G::FT; ++ft) mma_col(f1, ft);
  }
  wait_vmcnt<0>();
  if constexpr (ADAPTER)
    adapter_mma_lds<G, H, PK ? G::PLDS_BYTES : G::LDS_BYTES>(acc, lds, rt, xlh, xll, rpad, m0, t0, wm, wt, wave, lane);
  store_tile<G, O>(acc, Y, m0, t0, M, T, wm, wt, lane);
}

// Every row tile in tiles of geometry G.
template <class G, bool ADAPTER, typename O, bool PK, bool H = false, bool TOK = false>
__global__ __launch_bounds__(G::THREADS, 1) void spmm_smfmac_kernel(
    const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ vals, const uint32_t* __restrict__ meta, int M,
    int T, int Kred, const uint16_t* __restrict__ rt, const uint16_t* __restrict__ xlh,
    const uint16_t* __restrict__ xll, int rpad, O* __restrict__ Y, uint16_t* __restrict__ tok, int64_t Tch) {
  const int tiles_m = (M + G::BM - 1) / G::BM;
  spmm_tile<G, ADAPTER, O, PK, H, TOK>(Bm, vals, meta, M, T, Kred, rt, xlh, xll, rpad, Y, blockIdx.x, gridDim.x, 0,
                                  tiles_m, tok, Tch, tiles_m);
}

// Row tiles 0 .. rows_full - 1 in tiles of geometry GF (the first blocks),
// the rest in the narrower tiles of GN (the last blocks, which the dispatcher
// hands to compute units as they come free).
template <class GF, class GN, bool ADAPTER, typename O, bool PK, bool H = false, bool TOK = false>
__global__ __launch_bounds__(GF::THREADS, 1) void spmm_split_kernel(
    const uint16_t* __restrict__ Bm, const uint16_t* __restrict__ vals, const uint32_t* __restrict__ meta, int M,
    int T, int Kred, const uint16_t* __restrict__ rt, const uint16_t* __restrict__ xlh,
    const uint16_t* __restrict__ xll, int rpad, O* __restrict__ Y, int rows_full, uint16_t* __restrict__ tok,
    int64_t Tch) {
  static_assert(GF::THREADS == GN::THREADS && GF::BM == GN::BM, "same block and row tiles");
  const int tiles_m = (M + GF::BM - 1) / GF::BM;
  const int nfull = rows_full * ((T + GF::BT - 1) / GF::BT);
  if ((int)blockIdx.x < nfull)
    spmm_tile<GF, ADAPTER, O, PK, H, TOK>(Bm, vals, meta, M, T, Kred, rt, xlh, xll, rpad, Y, blockIdx.x, nfull, 0,
                                     rows_full, tok, Tch, rows_full);
  else   // the narrow tiles store token chunks only when no row runs full width
    spmm_tile<GN, ADAPTER, O, PK, H, TOK>(Bm, vals, meta, M, T, Kred, rt, xlh, xll, rpad, Y, blockIdx.x - nfull,
                                     gridDim.x - nfull, rows_full, tiles_m - rows_full, tok, Tch,
                                     rows_full > 0 ? 0 : tiles_m);
}

typedef Geo<256, 256, 3, 2, 4> GeoBig;
static_assert(GeoBig::BM == kPackRows && GeoBig::KS == kPackCols && GeoBig::A_BYTES == kPackValueBytes &&
                  GeoBig::CHUNK_BYTES == kPackChunkBytes,
              "tile chunks are the stage slices of the wide tile");
// the narrower tile for the rows of a product's last, partly filled round
typedef Geo<256, 128, 3, 2, 4> GeoHalf;
static_assert(GeoHalf::BM == GeoBig::BM && GeoHalf::CHUNK_BYTES == GeoBig::CHUNK_BYTES, "same row tiles and chunks");

// Tile chunks of a compressed bf16 matrix [M, Kred] (values [M, Kred/2],
// metadata [M, ceil(Kred/32)]): chunk (tm, s) covers rows 256tm .. 256tm+255
// and dense columns 64s .. 64s+63, at byte offset (tm * S + s) * CHUNK_BYTES
// (S = ceil(Kred/64)): first the 32 values of each row (64 bytes at row*64,
// 16-byte granule c at c ^ ((row/4) % 4)), then the two metadata words of each
// row (8 bytes at A_BYTES + row*8).  Rows past M and columns past Kred are 0.
template <class G>
__global__ __launch_bounds__(256) void pack_sparse_kernel(const uint16_t* __restrict__ vals,
                                                          const uint32_t* __restrict__ meta, int64_t M, int64_t Kred,
                                                          int64_t stages, int64_t nchunks, char* __restrict__ out) {
  static_assert(G::BM == 256 && G::KS == 64, "chunk geometry");
  const int tid = threadIdx.x;
  const int64_t wpr = (Kred / 4 + 7) / 8;
  for (int64_t q = blockIdx.x; q < nchunks; q += gridDim.x) {
    const int64_t tm = q / stages, s = q % stages;
    char* chunk = out + q * G::CHUNK_BYTES;
#pragma unroll
    for (int it = 0; it < 4; ++it) {               // 256 rows x four 16-byte granules
      const int r = it * 64 + (tid >> 2), c = tid & 3;
      const int64_t row = tm * 256 + r, kb = s * 64 + c * 16;   // compressed byte offset within the row
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < M && kb < Kred) v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(vals) + row * Kred + kb);
      *reinterpret_cast<u32x4*>(chunk + r * 64 + ((c ^ ((r >> 2) & 3)) << 4)) = v;
    }
#pragma unroll
    for (int it = 0; it < 2; ++it) {               // 256 rows x two metadata words
      const int idx = it * 256 + tid, r = idx >> 1, w = idx & 1;
      const int64_t row = tm * 256 + r, word = 2 * s + w;
      const uint32_t m = (row < M && word < wpr) ? meta[row * wpr + word] : 0u;
      *reinterpret_cast<uint32_t*>(chunk + G::A_BYTES + r * 8 + w * 4) = m;
    }
  }
}

// Whole product: full-width tiles, or full-width rows plus half-width rows
// in one launch when the full-width grid would end in a partly filled round.
template <bool ADAPTER, typename O, bool PK, bool H, bool TOK>
hipError_t launch_big(const uint16_t* B, int T, int Kred, const uint16_t* vals, const uint32_t* meta, int M,
                      const LowrankWs* w, O* Y, uint16_t* tok, hipStream_t s) {
  const int64_t tiles_m = cdiv(M, GeoBig::BM), cols = cdiv(T, GeoBig::BT), cols_half = cdiv(T, GeoHalf::BT);
  const int64_t Tch = cdiv(T, 32);
  const int64_t rows = full_width_rows(tiles_m, cols, cols_half, device_compute_units());
  constexpr int lds_bytes = PK ? GeoBig::PLDS_BYTES : GeoBig::LDS_BYTES;
  static_assert((PK ? GeoHalf::PLDS_BYTES : GeoHalf::LDS_BYTES) <= lds_bytes, "the narrow tile fits the wide one's LDS");
  const uint16_t* rt = w ? w->rt : nullptr;
  const uint16_t* xlh = w ? w->xlh : nullptr;
  const uint16_t* xll = w ? w->xll : nullptr;
  const int rpad = w ? (int)w->rpad : 0;
  if (rows == tiles_m) {
    auto kern = spmm_smfmac_kernel<GeoBig, ADAPTER, O, PK, H, TOK>;
    // once per process (thread-safe static initialisation)
    static hipError_t attr = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (attr != hipSuccess) return attr;
    if (tiles_m * cols == 0) return hipSuccess;
    kern<<<(unsigned)(tiles_m * cols), GeoBig::THREADS, lds_bytes, s>>>(B, vals, meta, M, T, Kred, rt, xlh, xll,
                                                                        rpad, Y, tok, Tch);
  } else {
    auto kern = spmm_split_kernel<GeoBig, GeoHalf, ADAPTER, O, PK, H, TOK>;
    static hipError_t attr = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (attr != hipSuccess) return attr;
    const int64_t nb = rows * cols + (tiles_m - rows) * cols_half;
    kern<<<(unsigned)nb, GeoBig::THREADS, lds_bytes, s>>>(B, vals, meta, M, T, Kred, rt, xlh, xll, rpad, Y,
                                                          (int)rows, tok, Tch);
  }
  return hipGetLastError();
}

template <bool PK, bool H, typename O>
hipError_t dispatch_ad(const uint16_t* B, int64_t T, int64_t Kred, const uint16_t* vals, const uint32_t* meta,
                       int64_t M, const LowrankWs* ws, O* Y, uint16_t* tok, hipStream_t s) {
  if constexpr (PK) {   // token chunks: packed operands only
    if (tok)
      return ws ? launch_big<true, O, PK, H, true>(B, (int)T, (int)Kred, vals, meta, (int)M, ws, Y, tok, s)
                : launch_big<false, O, PK, H, true>(B, (int)T, (int)Kred, vals, meta, (int)M, nullptr, Y, tok, s);
  }
  return ws ? launch_big<true, O, PK, H, false>(B, (int)T, (int)Kred, vals, meta, (int)M, ws, Y, nullptr, s)
            : launch_big<false, O, PK, H, false>(B, (int)T, (int)Kred, vals, meta, (int)M, nullptr, Y, nullptr, s);
}

// in: BF16 or F16 (raw 16-bit operands); out: the input format or F32
template <bool PK>
hipError_t dispatch_big(Dt in, Dt out, const void* B, int64_t T, int64_t Kred, const void* values,
                        const uint32_t* meta, int64_t M, const LowrankWs* ws, void* Y, uint16_t* tok,
                        hipStream_t s) {
  const uint16_t* Bb = (const uint16_t*)B;
  const uint16_t* vb = (const uint16_t*)values;
  if (in == Dt::F16)
    return out == Dt::F16 ? dispatch_ad<PK, true>(Bb, T, Kred, vb, meta, M, ws, (_Float16*)Y, tok, s)
                          : dispatch_ad<PK, true>(Bb, T, Kred, vb, meta, M, ws, (float*)Y, tok, s);
  return out == Dt::BF16 ? dispatch_ad<PK, false>(Bb, T, Kred, vb, meta, M, ws, (uint16_t*)Y, tok, s)
                         : dispatch_ad<PK, false>(Bb, T, Kred, vb, meta, M, ws, (float*)Y, tok, s);
}

}  // namespace

hipError_t launch_spmm(Dt in, Dt out, const void* B, int64_t T, int64_t Kred, const void* values,
                       const uint32_t* meta, int64_t M, const LowrankWs* ws, int64_t r, const void* R, void* Y,
                       hipStream_t s) {
  // block resources stay below 2 GiB: 256 rows x Kred x 2 bytes
  const bool fast = in != Dt::F32 && Kred % 16 == 0 && M % 4 == 0 && Kred <= (1 << 21);
  const bool ad = ws != nullptr && r > 0;
  if (!fast || (ad && !ws->mfma))
    return launch_spmm_generic(in, out, B, T, Kred, values, meta, M, ad ? ws->part : nullptr, ad ? ws->splits : 1,
                               ad ? r : 0, R, Y, s);
  return dispatch_big<false>(in, out, B, T, Kred, values, meta, M, ad ? ws : nullptr, Y, nullptr, s);
}

int64_t packed_sparse_bytes(int64_t M, int64_t Kred) {
  return cdiv(M, GeoBig::BM) * cdiv(Kred, GeoBig::KS) * GeoBig::CHUNK_BYTES;
}

hipError_t launch_pack_sparse(const void* values, const uint32_t* meta, int64_t M, int64_t Kred, void* packed,
                              hipStream_t s) {
  const int64_t stages = cdiv(Kred, GeoBig::KS), n = cdiv(M, GeoBig::BM) * stages;
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)(n < (1 << 20) ? n : (1 << 20));
  pack_sparse_kernel<GeoBig><<<grid, 256, 0, s>>>((const uint16_t*)values, meta, M, Kred, stages, n, (char*)packed);
  return hipGetLastError();
}

hipError_t launch_spmm_packed(Dt in, Dt out, const void* B, int64_t T, int64_t Kred, const void* packed, int64_t M,
                              const LowrankWs* ws, void* Y, void* tok, hipStream_t s) {
  return dispatch_big<true>(in, out, B, T, Kred, packed, nullptr, M, ws, Y, (uint16_t*)tok, s);
}

}  // namespace slope

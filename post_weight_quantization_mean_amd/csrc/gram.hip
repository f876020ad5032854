// The Gram form of the search loss ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §1: the exact
// layer-output squared error carries the cross terms of X^T X).  For a candidate's error E,
//   sum_{m,n} (X E^T)[m,n]^2 = sum_n E[n,:] G E[n,:]^T,   G = X^T X  [K x K],
// so after G is formed once (2 M K^2 flop) every candidate costs 2 K^2 N flop instead of
// 2 M K N: less work whenever M > K (here 2 K, see below).
//
// gram_dma_kernel forms G on the bf16 matrix cores and stores it as two bf16 matrices,
// G_hi = bf16(G) and G_lo = bf16(G - G_hi), so G_hi + G_lo keeps 16 significand bits of G (a
// single bf16 G would lose the cancellation that the quadratic form depends on).  They are
// interleaved in one [K x 2K] matrix: row k' holds, for every 32-column chunk c, chunk c of row
// k' of G_hi and then of G_lo; Tp stores that matrix in matrix-core operand order (tp_at).
// gram_search_kernel multiplies both with E~^T (E rounded to bf16, the direct form's operand)
// into the same accumulators and dots each output (k', n) with E~[n, k'], read back from the E
// stages of the block's first 16 chunks, which hold exactly its rows k'.
//
// Triangular form (K > 512).  G is symmetric, so e G e^T = sum_k G[k,k] e_k^2 +
// 2 sum_{k < k'} G[k,k'] e_k e_k': the same quadratic form with T = diag(G) + 2 triu(G, 1) in
// place of G, which is zero below the diagonal.  Tp then holds T_hi and T_lo (T_hi = 2 G_hi and
// T_lo = 2 G_lo above the diagonal: doubling is exact), and a candidate block whose 512 rows
// start at row k0 of T needs only the columns k >= k0: the K loop of the block starts there,
// which cuts the candidate work to about (K + 512) / (2K) of the full form.  With K <= 512
// every block starts at column 0 and the symmetric G is kept.
//
// One workgroup = one 128 x 128 tile of G with k1b <= k2b (G is symmetric: the tile is also
// written transposed); four waves of 64 x 64, i.e. 2 x 2 tiles of v_mfma_f32_32x32x16_bf16.
// Accumulation: fp32 in the matrix cores over 1024 tokens, then added into a second fp32 sum,
// so the rounding of the long sum over M grows with M / 1024 + 1024, not with M.
#include <type_traits>
#include <utility>

#include "awq_internal.h"

namespace awq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int GT = 128;  // G tile

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  const bf16x2 h = __builtin_convertvector((f32x2){x, x}, bf16x2);  // round to nearest even
  return (uint16_t)(__builtin_bit_cast(uint32_t, h) & 0xffffu);
}

// The tiles are fed by LDS DMA.  X never passes through registers: each stage of TT tokens
// copies the tile's two 128-channel strips (TT rows x 256 bytes each) from global memory
// straight into LDS in X's own [token][channel] order (buffer loads with LDS destination, 1 KiB
// per instruction, TT / 8 per wave), NST stages deep.  The matrix cores need, per lane, eight
// consecutive tokens of one channel: ds_read_b64_tr_b16 delivers them from the [token][channel]
// layout.  In each group of 16 lanes, lane i receives element i % 4 of the 8-byte reads of lanes
// i / 4 + 4 r, r = 0..3 (measured on this part), so lanes j that read the 4 channels
// cb + 4 (j % 4) at token t0 + j / 4 give lane i tokens t0 .. t0 + 3 of channel cb + i; two such
// reads make one MFMA operand.  Each token row's 16-byte pieces are stored XOR 2 (row % 4), so
// the four rows of one transposed read fall on distinct banks.
typedef short v4i16 __attribute__((ext_vector_type(4)));
#define AWQ_LDS_AS __attribute__((address_space(3)))

__device__ __forceinline__ int gd_swz(int row) { return 2 * (row & 3); }

// Element (row, col) of part `part` (0: hi, 1: lo) in Tp.  The parts are interleaved by
// 32-column chunks into a [K x 2K] matrix (column pc = 64 (col / 32) + 32 part + col % 32), and
// that matrix is stored in matrix-core operand order: fragments of 32 rows x 16 columns, 1 KiB
// each, row block after row block (K / 8 fragments per block of 32 rows); lane l of a fragment
// holds row l % 32, columns 8 (l / 32) .. + 7 as 16 contiguous bytes, the 16 bytes that lane l
// of a v_mfma_f32_32x32x16_bf16 A operand takes.  The candidate kernel thus loads each of its A
// fragments with one coalesced 1 KiB load straight into registers.
__device__ __forceinline__ int64_t tp_at(int64_t K, int64_t row, int64_t col, int part) {
  const int64_t pc = 64 * (col >> 5) + 32 * part + (col & 31);
  const int64_t frag = (row >> 5) * (K >> 3) + (pc >> 4);
  const int64_t l = (row & 31) + 32 * ((pc >> 3) & 1);
  return (frag * 64 + l) * 8 + (pc & 7);
}
// Element (k1, k2) of G, g, from a tile with k1b <= k2b.  Off the tile diagonal (off_diag:
// k1b < k2b) the transposed element (k2, k1) is written too.  Triangular form: T[k1, k2] = 2 g
// above the diagonal, g on it, and 0 below it (so the transposed element of an off-diagonal
// tile is 0).
__device__ __forceinline__ void store_g(uint16_t* __restrict__ Tp, int64_t K, int64_t k1, int64_t k2, bool off_diag,
                                        bool tri, float g) {
  const float t = !tri || k1 == k2 ? g : (k1 < k2 ? 2.0f * g : 0.0f);
  const uint16_t hi = bf16_bits(t);
  const uint16_t lo = bf16_bits(t - __uint_as_float((uint32_t)hi << 16));
  Tp[tp_at(K, k1, k2, 0)] = hi;
  Tp[tp_at(K, k1, k2, 1)] = lo;
  if (off_diag) {
    Tp[tp_at(K, k2, k1, 0)] = tri ? (uint16_t)0 : hi;
    Tp[tp_at(K, k2, k1, 1)] = tri ? (uint16_t)0 : lo;
  }
}

// NST stages of TT tokens (LDS: NST x 2 x TT x 256 bytes).  Measured on the 16384 x 4096 X of
// the decoder block (528 tiles): 4 stages of 64 tokens (one block per CU) 382 us; 3, 4 or 5
// stages of 32 tokens (two blocks per CU) 426-439 us; 3 of 64, 474 us.  A kernel that transposed X
// in registers instead (each thread loaded an 8 x 8 block of X and stored channel rows into LDS)
// took 590 us.  What bounds this one is the LDS traffic: a 64 x 64 wave tile reads one 32 x 16
// operand per product, eight bytes per lane per transposed read.
template <int NST, int TT>
__global__ __launch_bounds__(256, (NST * TT * 512 <= 80 * 1024) ? 2 : 1) void gram_dma_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t K, int64_t ldx, uint16_t* __restrict__ Tp, int64_t full,
    int S, int64_t slice_tokens, float* __restrict__ partial, bool tri) {
  constexpr int STRIP = TT * GT * 2;  // one strip of a stage
  constexpr int STAGE = 2 * STRIP;
  constexpr int NDMA = TT / 8;        // 1 KiB copies per wave per stage
  constexpr int BLOCK_STAGES = 1024 / TT;
  static_assert(NST >= 3 && NST <= 6 && (TT == 32 || TT == 64), "stage shape");
  __shared__ __attribute__((aligned(1024))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[NST > 3 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t st4[NST > 4 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t st5[NST > 5 ? STAGE : 16];
  auto stg = [&](auto I) -> uint8_t* {
    constexpr int i = decltype(I)::value % NST;
    if constexpr (i == 0) return st0; else if constexpr (i == 1) return st1; else if constexpr (i == 2) return st2;
    else if constexpr (i == 3) return st3; else if constexpr (i == 4) return st4; else return st5;
  };
  const bool whole = blockIdx.x < full;
  const int64_t item = whole ? 0 : blockIdx.x - full;
  const int64_t tile = whole ? blockIdx.x : full + item / S;
  const int64_t mbeg = whole ? 0 : (item % S) * slice_tokens;
  const int64_t mend = whole ? M : (mbeg + slice_tokens < M ? mbeg + slice_tokens : M);
  const int64_t T = K / GT;
  int64_t i = 0, rem = tile;
  while (rem >= T - i) {
    rem -= T - i;
    ++i;
  }
  const int64_t k1b = i * GT, k2b = (i + rem) * GT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // copies: wave w fills strip w / 2 (0: channels k1b.., 1: k2b..), rows (TT / 2) (w % 2) + 4 c +
  // lane / 16 of the stage in instruction c; lane l's 16 bytes land in physical piece l % 16 of
  // its row, which holds logical piece (l % 16) ^ swz(row)
  const int dstrip = wave >> 1;
  const int64_t kb = dstrip ? k2b : k1b;
  uint32_t doff[NDMA];
#pragma unroll
  for (int c = 0; c < NDMA; ++c) {
    const int row = (TT / 2) * (wave & 1) + 4 * c + (lane >> 4);
    doff[c] = (uint32_t)((row * ldx + kb + 8 * ((lane & 15) ^ gd_swz(row))) * 2);
  }
  // stage s covers tokens mbeg + TT s ..; its rows past mend read as zero (the resource ends there)
  auto dma = [&](uint8_t* stage, int64_t s) {
    const int64_t m0 = mbeg + TT * s;
    const int64_t rows = mend - m0 < 0 ? 0 : (mend - m0 < TT ? mend - m0 : TT);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(X + (m0 < mend ? m0 : mend) * ldx), (short)0, (int)(rows * ldx * 2), 0x00020000);
#pragma unroll
    for (int c = 0; c < NDMA; ++c)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (AWQ_LDS_AS void*)(stage + dstrip * STRIP + ((TT / 2) * (wave & 1) + 4 * c) * 256), 16, (int)doff[c], 0,
          0, 0);
  };
  // fragment reads: lane block b = lane / 16 covers rows 16 (b % 2) .. of a 32-row operand and
  // tokens 8 (b / 2) .. of a 16-token slice; within it lane j reads token t0 + j / 4, channels
  // cb + 4 (j % 4)
  const int r1 = 64 * (wave >> 1), c2 = 64 * (wave & 1);  // this wave's rows (k1) and columns (k2)
  const int jb = lane >> 4, j = lane & 15;
  auto frag_off = [&](int t, int cb) {  // byte offset in a strip; t % 4 == j / 4
    const int ch = cb + 16 * (jb & 1) + 4 * (j & 3);
    return t * 256 + 16 * ((ch >> 3) ^ gd_swz(t)) + 2 * (ch & 7);
  };
  int aoff[2][2], boff[2][2];  // [operand][token half], for slice 0 (slice sl: + 16 sl rows)
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 8 * (jb >> 1) + 4 * h + (j >> 2);
      aoff[a][h] = frag_off(t, r1 + 32 * a);
      boff[a][h] = STRIP + frag_off(t, c2 + 32 * a);
    }
  f32x16 acc[2][2], tot[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][c][e] = tot[a][c][e] = 0.0f;
  auto rd = [](const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((AWQ_LDS_AS v4i16*)(AWQ_LDS_AS void*)p);
  };
  auto compute = [&](const uint8_t* stage) {
#pragma unroll
    for (int sl = 0; sl < TT / 16; ++sl) {  // 16-token slices: token rows 16 sl ..
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const v4i16 lo = rd(stage + aoff[a][0] + sl * 16 * 256), hi = rd(stage + aoff[a][1] + sl * 16 * 256);
        fa[a] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        const v4i16 blo = rd(stage + boff[a][0] + sl * 16 * 256), bhi = rd(stage + boff[a][1] + sl * 16 * 256);
        fb[a] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[c], acc[a][c], 0, 0, 0);
    }
  };
  // own copies of a stage done (the next NST - 2 stages' may still be in flight), then the barrier
  // after which every wave's copies of the stage are visible and every wave is done with the
  // stage that the next copies overwrite.  No workgroup fence: it would wait for the copies
  // still in flight too.
  auto sync_stage = [] {
    constexpr int vm = (NST - 2) * NDMA;  // vmcnt: bits 3:0 and 15:14; expcnt 7, lgkmcnt 15 (no wait)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt((vm & 15) | ((vm >> 4) << 14) | 0x0f70);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };
  const int64_t stages = (mend - mbeg + TT - 1) / TT;
  auto close_block = [&](int64_t s) {  // after stage s: close a 1024-token block of the sum
    if ((s + 1) % BLOCK_STAGES == 0) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          tot[a][c] += acc[a][c];
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[a][c][e] = 0.0f;
        }
    }
  };
  // step s (S = s mod NST known at compile time): wait for stage s, copy stage s + NST - 1 into
  // the buffer of stage s - 1, multiply stage s
  auto step = [&](int64_t s, auto Sc) {
    constexpr int Sv = decltype(Sc)::value;
    sync_stage();
    dma(stg(std::integral_constant<int, Sv + NST - 1>{}), s + NST - 1);
    compute(stg(std::integral_constant<int, Sv>{}));
    close_block(s);
  };
  dma(st0, 0);
  dma(st1, 1);
  if constexpr (NST > 3) dma(st2, 2);
  if constexpr (NST > 4) dma(st3, 3);
  if constexpr (NST > 5) dma(st4, 4);
  // stages past the last are copies of nothing (zero rows) and add zeros: the loop runs whole
  // rounds of NST so that every stage buffer has a fixed role
  for (int64_t s = 0; s < stages; s += NST) {
    step(s, std::integral_constant<int, 0>{});
    step(s + 1, std::integral_constant<int, 1>{});
    step(s + 2, std::integral_constant<int, 2>{});
    if constexpr (NST > 3) step(s + 3, std::integral_constant<int, 3>{});
    if constexpr (NST > 4) step(s + 4, std::integral_constant<int, 4>{});
    if constexpr (NST > 5) step(s + 5, std::integral_constant<int, 5>{});
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt 0: no copy outlives the block
  // 32x32 result layout: lane l holds column l % 32, rows 8 (e / 4) + 4 (l / 32) + e % 4.
  if (!whole) {
    float* P = partial + item * (GT * GT);
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int k1 = r1 + 32 * a + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
          const int k2 = c2 + 32 * c + (lane & 31);
          P[k1 * GT + k2] = tot[a][c][e] + acc[a][c][e];
        }
    return;
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t k1 = k1b + r1 + 32 * a + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
        const int64_t k2 = k2b + c2 + 32 * c + (lane & 31);
        store_g(Tp, K, k1, k2, k1b != k2b, tri, tot[a][c][e] + acc[a][c][e]);
      }
}

// The split tiles: element (k1, k2) of tile full + u is the sum of its S slices in slice order,
// starting from 0 -- the order in which a whole tile adds its 1024-token block sums, so with one
// block per slice the result is the same bits as the whole-tile kernel's.
__global__ __launch_bounds__(256) void gram_fixup_kernel(const float* __restrict__ partial, int64_t K,
                                                          int64_t full, int S, uint16_t* __restrict__ Tp, bool tri) {
  const int64_t u = blockIdx.y;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // k1 GT + k2, tile-local
  const int k1l = (int)(idx / GT), k2l = (int)(idx % GT);
  const int64_t T = K / GT;
  int64_t i = 0, rem = full + u;
  while (rem >= T - i) {
    rem -= T - i;
    ++i;
  }
  const int64_t k1b = i * GT, k2b = (i + rem) * GT;
  float g = 0.0f;
  for (int s = 0; s < S; ++s) g += partial[(u * S + s) * (GT * GT) + idx];
  store_g(Tp, K, k1b + k1l, k2b + k2l, k1b != k2b, tri, g);
}

// With tiles = q 512 + r (512: two rounds of one block on each of 256 CUs), the first q 512 tiles
// run whole; the r tiles of the last, partial round are cut into S token slices of whole
// 1024-token blocks, so that r S is about one round (K = 4096: 528 tiles, 16 of them in 16
// slices each).
constexpr int64_t kGramSlots = 512;
constexpr int64_t kGramBlockTokens = 1024;

struct GramPlan {
  int64_t tiles, full, r, slice_tokens;
  int S;
};

GramPlan gram_plan(int64_t M, int64_t K) {
  GramPlan p;
  const int64_t T = K / GT;
  p.tiles = T * (T + 1) / 2;
  p.r = p.tiles % kGramSlots;
  p.full = p.tiles - p.r;
  const int64_t nblk = (M + kGramBlockTokens - 1) / kGramBlockTokens;
  int64_t S = p.r > 0 ? kGramSlots / p.r : 1;
  if (S > nblk) S = nblk;
  if (S < 1) S = 1;
  const int64_t bps = (nblk + S - 1) / S;  // 1024-token blocks per slice
  p.slice_tokens = bps * kGramBlockTokens;
  p.S = (int)((nblk + bps - 1) / bps);
  if (p.S <= 1) {  // one slice: the leftover tiles run whole
    p.full = p.tiles;
    p.r = 0;
    p.S = 1;
  }
  return p;
}

// ---- the candidate kernel of the Gram form ------------------------------------------------
// The stack is stored as Tp (see tp_at): row k' of T_hi and row k' of T_lo interleaved by
// 32-column chunks, in matrix-core operand order.  Since (T_hi + T_lo) e^T = T_hi e^T + T_lo e^T, both parts accumulate into the same outputs:
// a block is a tile of 512 rows k' x 128 outputs n for one candidate, and its step c multiplies
// the hi and the lo part of chunk c with the same E chunk, 64 v_mfma_f32_32x32x16_bf16 per wave.
// Per matrix instruction that halves, against a [2K x K] stack of separate hi and lo rows, the
// quantization, the E stores and reads and the barriers, and the blocks' fixed prologue and
// epilogue; the bytes of T per instruction stay the same.
// The pipeline is the direct search kernel's (search.hip), with these differences:
//   * T never passes through LDS: the 64 matrix instructions of a step run K-half by K-half;
//     within one, row block r of the wave, hi then lo: group g = 32 h + 8 r + 4 part + cc, and
//     block blk = g / 4 of chunk c+1's A fragments (1 KiB of Tp each) is loaded straight into
//     registers right after the last product of chunk c that reads block blk, one step before
//     its use (the compiler's counters wait for it);
//   * the B fragments of the second K-half are read in groups 1-7 and the next chunk's first
//     K-half in groups 33-39, after the last use of the current ones;
//   * the quantization of chunk c+2 places element el in group 3 + 3 el, its two stores after
//     elements 7 and 15;
//   * the E stage of chunk c0 + j is slot j for j < 16 (kept to the end), later chunks rotate
//     through three more slots; the block's rows k' are its first 16 chunks, so the epilogue
//     reads the E~ it dots the outputs with from the kept slots (one 8-byte LDS read per four
//     outputs, against recomputing each e from W, s and the group's range).
// Triangular form: the block's K loop starts at its first row, chunk m0 / 32 (a multiple of 16).
constexpr int GS_BM = 512, GS_BN = 128, GS_KC = 32;
constexpr int GS_PROW = GS_KC * 2;            // bytes of an E row (one chunk)
constexpr int GS_ESTAGE = GS_BN * GS_PROW;    // 8 KiB
constexpr int GS_NES = 3;
constexpr int GS_KEEP = GS_BM / GS_KC;         // E stages kept for the epilogue: the block's first 16 chunks
constexpr int GS_SRG = kGroup * 8;            // one group's (s, 1/s) pairs: 1 KiB
#define AWQ_LDS_G __attribute__((address_space(3)))

__device__ __forceinline__ int gs_swz(int row) { return (row >> 2) & 3; }   // E rows
__device__ __forceinline__ float gs_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float gs_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ uint32_t gs_pack(float a, float b) {
  const bf16x2 h = __builtin_convertvector((f32x2){a, b}, bf16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}
struct GsWSet {
  uint4 w[2];  // this lane's 8 bf16 channels of its rows r0 and r1
};
// f(integral_constant<int, G>) for every G of the sequence, in order: the group index is a
// compile-time constant in every call, whatever the size of the step
template <typename F, int... G>
__device__ __forceinline__ void gs_each(F&& f, std::integer_sequence<int, G...>) {
  (f(std::integral_constant<int, G>{}), ...);
}
struct GsRowQ {
  float delta, inv, lo, hi;
};

__global__ __launch_bounds__(256, 1) void gram_search_kernel(
    const uint16_t* __restrict__ Tp, int64_t K, const WSegs segs, const float2* __restrict__ sr_tab,
    const float2* __restrict__ params, int n_grid, int64_t nt_count, int64_t tiles, bool tri,
    double* __restrict__ partial) {
  // E stages: slot j < 16 holds chunk c0 + j for good (the epilogue reads them back), later
  // chunks rotate through slots 16 .. 18; 152 KiB, with the scale tables the whole 160 KiB
  __shared__ __attribute__((aligned(1024))) uint8_t es[(GS_KEEP + GS_NES) * GS_ESTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t srs0[4 * GS_SRG];
  __shared__ __attribute__((aligned(1024))) uint8_t srs1[4 * GS_SRG];

  // XCD x (= b % 8) runs its blocks l = b / 8 in order: row tile mt = l / (spx n_grid), then
  // output tile ((x + mt) % 8) + 8 s, s < spx = ceil(nt_count / 8), candidate-fastest.  Blocks of
  // the triangular form differ in length with their row tile, so every XCD works on the same row
  // tile at a time; its resident blocks share that tile's rows and a few W tiles in its L2.
  const int64_t b = blockIdx.x;
  const int64_t spx = (nt_count + 7) >> 3, per_m = spx * n_grid, l = b >> 3;
  const int64_t mt = l / per_m, rr = l - mt * per_m, sj = rr / n_grid;
  const int64_t ntile = (((b & 7) + mt) & 7) + 8 * sj;
  if (mt * nt_count >= tiles || ntile >= nt_count) return;
  const int64_t tile = mt * nt_count + ntile;
  const int al = (int)(rr - sj * n_grid);
  const int64_t m0 = mt * GS_BM;      // first row of T
  const int64_t n0 = ntile * GS_BN;   // in the padded row space of all weights
  const WSel sel = select_wseg(segs, ntile);
  const uint16_t* __restrict__ W = static_cast<const uint16_t*>(sel.w);
  const int64_t N = sel.n, ldw = sel.ldw, n0w = sel.n0;
  const int G = (int)(K / kGroup);
  const int64_t NP = nt_count * GS_BN;
  const int nchunks = (int)(K / GS_KC);
  const int c0 = tri ? (int)(m0 / GS_KC) : 0;
  const int64_t ldx = 2 * K;
  // the E stage of chunk q (see es)
  auto eoff = [&](int q) {
    const int j = q - c0;
    return j < GS_KEEP ? j * GS_ESTAGE : (GS_KEEP + (j - GS_KEEP) % GS_NES) * GS_ESTAGE;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // rows of T past K (and rows of W past N) read as zero; offsets stay below 2^31 (host: 512
  // rows of Tp, 128 rows of W)
  auto rsrc = [](const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff), 0x00020000);
  };
  const __amdgpu_buffer_rsrc_t xrsrc = rsrc(Tp + m0 * ldx, (K - m0) * ldx * 2);
  const __amdgpu_buffer_rsrc_t wrsrc = rsrc(W + n0w * ldw, (N - n0w) * ldw * 2);
  const __amdgpu_buffer_rsrc_t srsrc = rsrc(sr_tab + (int64_t)al * K, K * 8);
  const __amdgpu_buffer_rsrc_t prsrc = rsrc(params + (int64_t)al * G * NP, (int64_t)G * NP * 8);
  // A fragment blk = 8 h + 2 r + part of chunk ch: row block 4 wave + r of the tile (K / 8
  // fragments of 1 KiB each), column block 4 ch + 2 part + h; this lane's 16 bytes at 16 lane
  const uint32_t avoff = (uint32_t)(lane * 16) + (uint32_t)(wave * 4) * (uint32_t)(K * 128);
  auto load_a = [&](int ch, int blk) {
    const int h = blk >> 3, r = (blk >> 1) & 3, part = blk & 1;
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                          xrsrc, (int)avoff, (int)(r * K * 128 + (4 * ch + 2 * part + h) * 1024), 0));
  };
  // quantization: rows r0, r1 of the E tile, channel piece q4 of each chunk
  const int q4 = lane & 3;
  const int r0 = wave * 32 + (lane >> 2), r1 = r0 + 16;
  const uint32_t woff0 = (uint32_t)(r0 * ldw * 2 + q4 * 16);
  const uint32_t woff1 = (uint32_t)(r1 * ldw * 2 + q4 * 16);
  const int eslot0 = r0 * GS_PROW + ((q4 ^ gs_swz(r0)) * 16);
  const int eslot1 = r1 * GS_PROW + ((q4 ^ gs_swz(r1)) * 16);
  const bool live0 = n0w + r0 < N, live1 = n0w + r1 < N;
  const int poff = (int)((n0 + 32 * wave + 2 * (lane >> 2)) * 8);
  // E fragment reads: lane reads row (32 t + fr), 16-byte piece 2 h + fh of K-half h
  const int fr = lane & 31, fh = lane >> 5;
  const int efoff0 = fr * GS_PROW + (((0 + fh) ^ gs_swz(fr)) * 16);
  const int efoff1 = fr * GS_PROW + (((2 + fh) ^ gs_swz(fr)) * 16);
  auto load_w = [&](GsWSet& S, int i, int cb, int j) {
    S.w[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           wrsrc, (int)(i == 0 ? woff0 : woff1) + j * (GS_KC * 2), cb, 0));
  };
  auto load_p = [&](int g) {
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(prsrc, poff, (int)(g * NP * 8), 0));
  };
  auto dma_sr = [&](uint8_t* table, int g) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(srsrc, (AWQ_LDS_G void*)(table + GS_SRG * wave), 16, 16 * lane,
                                             g * GS_SRG, 0, 0);
  };
  auto sr_addr = [&](const uint8_t* table, int c) {
    return table + GS_SRG * wave + (32 * (c & 3) + 8 * q4) * 8;
  };
  auto row_setup = [&](const float4& P, int i) {
    const bool live = i == 0 ? live0 : live1;
    GsRowQ q;
    q.delta = live ? (i == 0 ? P.x : P.z) : 1.0f;  // rows past N: Delta 1, z 0, w 0: e = 0
    const float z = live ? (i == 0 ? P.y : P.w) : 0.0f;
    q.inv = __builtin_amdgcn_rcpf(q.delta);  // search only; the pack divides exactly
    q.lo = -z;
    q.hi = 15.0f - z;
    return q;
  };
  auto elem = [&](const GsWSet& S, const float4* sv, const GsRowQ& q, int i, int j) {
    const uint4& w4 = S.w[i];
    const uint32_t u = j < 2 ? w4.x : j < 4 ? w4.y : j < 6 ? w4.z : w4.w;
    const float w = (j & 1) ? gs_hi(u) : gs_lo(u);
    const float s = (j & 1) ? sv[j >> 1].z : sv[j >> 1].x;
    const float rs = (j & 1) ? sv[j >> 1].w : sv[j >> 1].y;
    const float v = w * s;                                    // S W
    const float r = rintf(v * q.inv);                         // rne(v / Delta)
    const float qz = __builtin_amdgcn_fmed3f(r, q.lo, q.hi);  // clamp(r + z, 0, 15) - z
    return fmaf(-(qz * q.delta), rs, w);                      // w - Delta (q - z) / s
  };
  auto store_piece = [&](uint8_t* estage, int slot, const float* e8) {
    uint32_t pk[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) pk[h] = gs_pack(e8[2 * h], e8[2 * h + 1]);
    *reinterpret_cast<uint4*>(estage + slot) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  };
  auto quantize_all = [&](const GsWSet& S, const float4& P, int c, uint8_t* estage) {  // prologue only
    float4 sv[4];
    const uint8_t* sa = sr_addr(srs0, c);
#pragma unroll
    for (int t = 0; t < 4; ++t) sv[t] = *reinterpret_cast<const float4*>(sa + 16 * t);
    const GsRowQ q0 = row_setup(P, 0), q1 = row_setup(P, 1);
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = elem(S, sv, q0, 0, j);
    store_piece(estage, eslot0, e);
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = elem(S, sv, q1, 1, j);
    store_piece(estage, eslot1, e);
  };
  auto frag = [&](const uint8_t* base, int fo) { return *reinterpret_cast<const bf16x8*>(base + fo); };
  auto vm_wait = [](auto n) {  // s_waitcnt vmcnt(n), other counters untouched
    constexpr int v = decltype(n)::value;
    __builtin_amdgcn_s_waitcnt((v & 0xf) | (0x7 << 4) | (0xf << 8) | ((v >> 4) << 14));
  };
  constexpr int kWaitLgkm0 = 0xf | (0x7 << 4) | (0x0 << 8) | (0x3 << 14);

  f32x16 acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.0f;

  GsWSet S0, S1, S2, S3;  // W words of chunk c live in set c % 4
  float4 PC, PN;          // ranges of the group being quantized, of the next group
  GsRowQ q0, q1;
  // Prologue: group c0 / 4's scale table and ranges, W of chunks c0 .. c0 + 3, the A fragments
  // of chunk c0; chunks c0 and c0 + 1 are quantized.
  dma_sr(srs0, c0 >> 2);
  PC = load_p(c0 >> 2);
  load_w(S0, 0, c0 * (GS_KC * 2), 0);
  load_w(S1, 0, c0 * (GS_KC * 2), 1);
  load_w(S0, 1, c0 * (GS_KC * 2), 0);
  load_w(S1, 1, c0 * (GS_KC * 2), 1);
  __builtin_amdgcn_sched_barrier(0);
  bf16x8 a[16];  // A fragments of the step's chunk, block by block replaced by the next chunk's
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = load_a(c0, i);
  __builtin_amdgcn_sched_barrier(0);
  load_w(S2, 0, c0 * (GS_KC * 2), 2);
  load_w(S3, 0, c0 * (GS_KC * 2), 3);
  load_w(S2, 1, c0 * (GS_KC * 2), 2);
  load_w(S3, 1, c0 * (GS_KC * 2), 3);
  __builtin_amdgcn_sched_barrier(0);
  vm_wait(std::integral_constant<int, 0>{});
  __builtin_amdgcn_sched_barrier(0);
  quantize_all(S0, PC, 0, es + 0 * GS_ESTAGE);  // chunks c0, c0 + 1: positions 0, 1 of their group
  quantize_all(S1, PC, 1, es + 1 * GS_ESTAGE);
  q0 = row_setup(PC, 0);
  q1 = row_setup(PC, 1);
  bf16x8 b0[4];  // B fragments of K-half 0 of chunk c
  {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 4; ++t) b0[t] = frag(es + t * 32 * GS_PROW, efoff0);
    asm volatile("" ::"v"(S2.w[0].x), "v"(S2.w[0].y), "v"(S2.w[0].z), "v"(S2.w[0].w), "v"(S2.w[1].x),
                 "v"(S2.w[1].y), "v"(S2.w[1].z), "v"(S2.w[1].w));
    asm volatile("" ::"v"(S3.w[0].x), "v"(S3.w[0].y), "v"(S3.w[0].z), "v"(S3.w[0].w), "v"(S3.w[1].x),
                 "v"(S3.w[1].y), "v"(S3.w[1].z), "v"(S3.w[1].w));
  }

  // Step c (k = c % 4 known at compile time).  Loads: even steps 4 W in groups 0-3, when k = 0
  // the next group's ranges (group 4) and scale table DMA (group 5); every step 16 A fragments
  // in groups 4, 8, ..., 60 and 63.  The scale table DMA'd in a k = 0 step is read from the
  // k = 2 step on: 15 A loads of its own step and 16 of the next were issued after it.
  auto step = [&](int c8, auto jc, const GsWSet& Q, GsWSet& F4, GsWSet& F5, const uint8_t* srq, uint8_t* srn) {
    constexpr int j = decltype(jc)::value;
    constexpr int k = j & 3;
    constexpr bool even = (k & 1) == 0;
    const int c = c8 + j;
    const int cb = c8 * (GS_KC * 2);
    const int gn = (c8 >> 2) + (j >> 2) + 1;  // next group (k = 0 steps)
    const uint8_t* ec = es + eoff(c);
    const uint8_t* en = es + eoff(c + 1);
    uint8_t* eq = es + eoff(c + 2);
    const uint8_t* sa = sr_addr(srq, k + 2);
    if (k == 2) {  // chunks c+2 .. c+5 of this quad after the first two: next group
      PC = PN;
      q0 = row_setup(PC, 0);
      q1 = row_setup(PC, 1);
    }
    bf16x8 b1[4];
    float4 sv[4];
    float e[16];
    __builtin_amdgcn_sched_barrier(0);
    if (k == 2) vm_wait(std::integral_constant<int, 31>{});
    gs_each([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      constexpr int blk = g >> 2, h = blk >> 3, r = (blk >> 1) & 3, cc = g & 3;
      acc[r][cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[blk], h == 0 ? b0[cc] : b1[cc], acc[r][cc], 0, 0, 0);
      if (g == 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) sv[t] = *reinterpret_cast<const float4*>(sa + 16 * t);
      }
      if (g < 8 && (g & 1)) b1[g >> 1] = frag(ec + (g >> 1) * 32 * GS_PROW, efoff1);
      if (g >= 33 && g < 40 && (g & 1)) b0[(g - 33) >> 1] = frag(en + ((g - 33) >> 1) * 32 * GS_PROW, efoff0);
      // element el in group 3 + 3 el: row r0 in groups 3-24, row r1 in 27-48
      constexpr int el = g >= 3 && g <= 48 && g % 3 == 0 ? g / 3 - 1 : -1;
      if (el >= 0) {
        e[el] = el < 8 ? elem(Q, sv, q0, 0, el) : elem(Q, sv, q1, 1, el - 8);
        asm volatile("" : "+v"(e[el]));  // keep the element in this group
      }
      if (g == 25) store_piece(eq, eslot0, e);
      if (g == 49) store_piece(eq, eslot1, e + 8);
      if (even) {
        if (g == 0) load_w(F4, 0, cb, j + 4);
        if (g == 1) load_w(F5, 0, cb, j + 5);
        if (g == 2) load_w(F4, 1, cb, j + 4);
        if (g == 3) load_w(F5, 1, cb, j + 5);
        if (k == 0 && g == 4) PN = load_p(gn);
        if (k == 0 && g == 5) dma_sr(srn, gn);
      }
      // chunk c+1's A fragment of block blk - 1 (block 15: after the last product, group 63);
      // past the last chunk these read other rows of the tile or, past its end, zeros (unused)
      if (g >= 4 && (g & 3) == 0) a[(g >> 2) - 1] = load_a(c + 1, (g >> 2) - 1);
      if (g == 63) a[15] = load_a(c + 1, 15);
      __builtin_amdgcn_sched_barrier(0);
    }, std::make_integer_sequence<int, 64>{});
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // E stores of chunk c+2, fragment reads
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // The body covers two groups (8 steps) so that each scale table has a static role.  nchunks -
  // c0 is a multiple of 4 (c0 a multiple of 16).
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  using I6 = std::integral_constant<int, 6>;
  using I7 = std::integral_constant<int, 7>;
  int c = c0;
  for (; c + 8 <= nchunks; c += 8) {
    step(c, I0{}, S2, S0, S1, srs0, srs1);
    step(c, I1{}, S3, S0, S1, srs0, srs1);
    step(c, I2{}, S0, S2, S3, srs1, srs1);
    step(c, I3{}, S1, S2, S3, srs1, srs1);
    step(c, I4{}, S2, S0, S1, srs1, srs0);
    step(c, I5{}, S3, S0, S1, srs1, srs0);
    step(c, I6{}, S0, S2, S3, srs0, srs0);
    step(c, I7{}, S1, S2, S3, srs0, srs0);
  }
  if (c < nchunks) {  // K / 128 odd: one more group
    step(c, I0{}, S2, S0, S1, srs0, srs1);
    step(c, I1{}, S3, S0, S1, srs0, srs1);
    step(c, I2{}, S0, S2, S3, srs1, srs1);
    step(c, I3{}, S1, S2, S3, srs1, srs1);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt 0: no load (the last ones read past the end) outlives the block

  // This wave's 128 rows are rows kb .. kb + 127 of T: chunks c0 + 4 wave .. + 3 of K, whose E
  // stages are slots 4 wave .. + 3 (rows past K hold zeros and are skipped).  Lane l's outputs sit
  // at k' = kb + 32 r + 8 (i / 4) + 4 (l / 32) + i % 4 and n = n0 + 32 cc + l % 32; the lane reads
  // E~[n, k'] (E rounded to bf16, the operand the products used: rows past N hold zeros) four
  // channels at a time from slot 4 wave + r, and adds acc E~.
  double ss = 0.0;
  const int64_t kb = m0 + 128 * wave;
  if (kb < K) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint8_t* slot = es + (4 * wave + r) * GS_ESTAGE;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int nl = 32 * cc + (lane & 31);
        float t = 0.0f;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          // channels 8 i4 + 4 (l / 32) .. + 3 of row nl: piece i4, bytes 8 (l / 32) .. + 7
          const uint2 e4 = *reinterpret_cast<const uint2*>(slot + nl * GS_PROW + ((i4 ^ gs_swz(nl)) * 16) +
                                                           8 * (lane >> 5));
          t = fmaf(acc[r][cc][4 * i4 + 0], gs_lo(e4.x), t);
          t = fmaf(acc[r][cc][4 * i4 + 1], gs_hi(e4.x), t);
          t = fmaf(acc[r][cc][4 * i4 + 2], gs_lo(e4.y), t);
          t = fmaf(acc[r][cc][4 * i4 + 3], gs_hi(e4.y), t);
        }
        ss += (double)t;
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  // the rotating E stages are past their last access (the barrier ending the last step) and the
  // epilogue reads only the kept ones, so the first rotating stage can hold the four wave sums
  double* red = reinterpret_cast<double*>(es + GS_KEEP * GS_ESTAGE);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  if (tid == 0) partial[(int64_t)al * tiles + tile] = ((red[0] + red[1]) + red[2]) + red[3];
}

}  // namespace

size_t gram_partial_bytes(int64_t M, int64_t K) {
  const GramPlan p = gram_plan(M, K);
  return (size_t)(p.r * p.S) * GT * GT * sizeof(float);
}

hipError_t launch_gram(const uint16_t* X, int64_t M, int64_t K, int64_t ldx, uint16_t* Tp, float* partial,
                       hipStream_t st) {
  const GramPlan p = gram_plan(M, K);
  const bool tri = gram_triangular(K);
  gram_dma_kernel<4, 64><<<(unsigned)(p.full + p.r * p.S), 256, 0, st>>>(X, M, K, ldx, Tp, p.full, p.S,
                                                                        p.slice_tokens, partial, tri);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.r == 0) return e;
  gram_fixup_kernel<<<dim3((unsigned)(GT * GT / 256), (unsigned)p.r), 256, 0, st>>>(partial, K, p.full, p.S, Tp,
                                                                                     tri);
  return hipGetLastError();
}

hipError_t launch_search_gram(const uint16_t* Tp, int64_t K, const WSegs& W, const float2* sr_tab,
                              const float2* params, int n_grid, const SearchPlan& plan, double* partial,
                              hipStream_t st) {
  // eight XCD slots per row tile and output-tile group of eight (see the kernel)
  const dim3 grid((unsigned)(8 * plan.mt * ((plan.nt + 7) / 8) * n_grid));
  gram_search_kernel<<<grid, 256, 0, st>>>(Tp, K, W, sr_tab, params, n_grid, plan.nt, plan.tiles,
                                           gram_triangular(K), partial);
  return hipGetLastError();
}

}  // namespace awq

// The Gram form of the search loss ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §1: the exact
// layer-output squared error carries the cross terms of X^T X).  For a candidate's error E,
//   sum_{m,n} (X E^T)[m,n]^2 = sum_n E[n,:] G E[n,:]^T,   G = X^T X  [K x K],
// so after G is formed once (2 M K^2 flop) every candidate costs 2 K^2 N flop instead of
// 2 M K N: less work whenever M > K (here 2 K, see below).
//
// gram_dma_kernel forms G on the bf16 matrix cores and stores it as two bf16 matrices stacked
// along the rows, Gs = [G_hi; G_lo] [2K x K] with G_hi = bf16(G), G_lo = bf16(G - G_hi), so
// G_hi + G_lo keeps 16 significand bits of G (a single bf16 G would lose the cancellation
// that the quadratic form depends on).  The candidate kernel then multiplies Gs with E^T as
// it multiplies X with E^T, and dots each output row k' with E[:, k' mod K].
//
// Triangular form (K > 512).  G is symmetric, so e G e^T = sum_k G[k,k] e_k^2 +
// 2 sum_{k < k'} G[k,k'] e_k e_k': the same quadratic form with T = diag(G) + 2 triu(G, 1) in
// place of G, which is zero below the diagonal.  The stored stack is then [T_hi; T_lo]
// (T_hi = 2 G_hi and T_lo = 2 G_lo above the diagonal: doubling is exact), and a candidate
// block whose 512 rows start at row k0 of T needs only the columns k >= k0: the K loop of
// the block starts there, which cuts the candidate work to (K + 512) / (2K) of the full form.
// With K <= 512 every block starts at column 0 and the symmetric G is kept.
//
// One workgroup = one 128 x 128 tile of G with k1b <= k2b (G is symmetric: the tile is also
// written transposed); four waves of 64 x 64, i.e. 2 x 2 tiles of v_mfma_f32_32x32x16_bf16.
// Accumulation: fp32 in the matrix cores over 1024 tokens, then added into a second fp32 sum,
// so the rounding of the long sum over M grows with M / 1024 + 1024, not with M.
#include <type_traits>

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

// Element (k1, k2) of G, g, from a tile with k1b <= k2b: its hi and lo parts go to rows k1 and
// K + k1 of the stack.  Off the tile diagonal (off_diag: k1b < k2b) the transposed element
// (k2, k1) is written too.  Triangular form: T[k1, k2] = 2 g above the diagonal, g on it, and 0
// below it (so the transposed element of an off-diagonal tile is 0).
__device__ __forceinline__ void store_g(uint16_t* __restrict__ Gs, int64_t K, int64_t k1, int64_t k2, bool off_diag,
                                        bool tri, float g) {
  const float t = !tri || k1 == k2 ? g : (k1 < k2 ? 2.0f * g : 0.0f);
  const uint16_t hi = bf16_bits(t);
  const uint16_t lo = bf16_bits(t - __uint_as_float((uint32_t)hi << 16));
  Gs[k1 * K + k2] = hi;
  Gs[(K + k1) * K + k2] = lo;
  if (off_diag) {
    Gs[k2 * K + k1] = tri ? (uint16_t)0 : hi;
    Gs[(K + k2) * K + k1] = tri ? (uint16_t)0 : lo;
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
    const uint16_t* __restrict__ X, int64_t M, int64_t K, int64_t ldx, uint16_t* __restrict__ Gs, int64_t full,
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
        store_g(Gs, K, k1, k2, k1b != k2b, tri, tot[a][c][e] + acc[a][c][e]);
      }
}

// The split tiles: element (k1, k2) of tile full + u is the sum of its S slices in slice order,
// starting from 0 -- the order in which a whole tile adds its 1024-token block sums, so with one
// block per slice the result is the same bits as the whole-tile kernel's.
__global__ __launch_bounds__(256) void gram_fixup_kernel(const float* __restrict__ partial, int64_t K,
                                                          int64_t full, int S, uint16_t* __restrict__ Gs, bool tri) {
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
  store_g(Gs, K, k1b + k1l, k2b + k2l, k1b != k2b, tri, g);
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

}  // namespace

size_t gram_partial_bytes(int64_t M, int64_t K) {
  const GramPlan p = gram_plan(M, K);
  return (size_t)(p.r * p.S) * GT * GT * sizeof(float);
}

hipError_t launch_gram(const uint16_t* X, int64_t M, int64_t K, int64_t ldx, uint16_t* Gs, float* partial,
                       hipStream_t st) {
  const GramPlan p = gram_plan(M, K);
  const bool tri = gram_triangular(K);
  gram_dma_kernel<4, 64><<<(unsigned)(p.full + p.r * p.S), 256, 0, st>>>(X, M, K, ldx, Gs, p.full, p.S,
                                                                        p.slice_tokens, partial, tri);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.r == 0) return e;
  gram_fixup_kernel<<<dim3((unsigned)(GT * GT / 256), (unsigned)p.r), 256, 0, st>>>(partial, K, p.full, p.S, Gs,
                                                                                     tri);
  return hipGetLastError();
}

}  // namespace awq

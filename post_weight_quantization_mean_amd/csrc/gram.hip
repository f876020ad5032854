// The Gram form of the search loss ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §1: the exact
// layer-output squared error carries the cross terms of X^T X).  For a candidate's error E,
//   sum_{m,n} (X E^T)[m,n]^2 = sum_n E[n,:] G E[n,:]^T,   G = X^T X  [K x K],
// so after G is formed once (2 M K^2 flop) every candidate costs 2 K^2 N flop instead of
// 2 M K N: less work whenever M > K (here 2 K, see below).
//
// gram_kernel forms G on the bf16 matrix cores and stores it as two bf16 matrices stacked
// along the rows, Gs = [G_hi; G_lo] [2K x K] with G_hi = bf16(G), G_lo = bf16(G - G_hi), so
// G_hi + G_lo keeps 16 significand bits of G (a single bf16 G would lose the cancellation
// that the quadratic form depends on).  The candidate kernel then multiplies Gs with E^T as
// it multiplies X with E^T, and dots each output row k' with E[:, k' mod K].
//
// One workgroup = one 128 x 128 tile of G with k1b <= k2b (G is symmetric: the tile is also
// written transposed); four waves of 64 x 64, i.e. 2 x 2 tiles of v_mfma_f32_32x32x16_bf16.
// Per step 64 tokens: thread t holds an 8 x 8 block of X (tokens 8 (t % 8) .., channels
// 8 ((t / 8) % 16) .. of the k1 range for t < 128, of the k2 range otherwise), loaded as
// eight 16-byte rows, transposes it in registers (byte permutes pair the tokens of each
// channel) and stores eight 16-byte channel rows into LDS ([channel][token]); an MFMA
// fragment (one channel, eight tokens) is then one 16-byte read.  The next step's blocks are
// loaded while the current step multiplies.  Accumulation: fp32 in the matrix cores over
// 1024 tokens, then added into a second fp32 sum, so the rounding of the long sum over M
// grows with M / 1024 + 1024, not with M.
#include "awq_internal.h"

namespace awq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int GT = 128;              // G tile
constexpr int GS = 64;               // tokens per step
constexpr int GPITCH = GS + 8;       // LDS row pitch (bf16): 144 bytes
constexpr int kGramBlockSteps = 16;  // 1024 tokens per inner fp32 sum

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  const bf16x2 h = __builtin_convertvector((f32x2){x, x}, bf16x2);  // round to nearest even
  return (uint16_t)(__builtin_bit_cast(uint32_t, h) & 0xffffu);
}

// At most 256 registers a lane (two blocks per CU, 2 x 72 KiB of LDS): while one block waits for
// its next step's loads the other multiplies.  At one block per CU (264 registers) the one step
// of prefetch could not cover the load latency and G took 1.7x as long (measured; a second
// register set for two steps of prefetch instead gained half as much and does not fit with two
// blocks).
__global__ __launch_bounds__(256, 2) void gram_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                   int64_t ldx, uint16_t* __restrict__ Gs, int64_t full, int S,
                                                   int64_t slice_tokens, float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint16_t t1[2][GT][GPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t t2[2][GT][GPITCH];
  // Block b < full computes tile b over all M tokens and writes it to Gs.  Block full + u S + s
  // computes tile full + u over tokens [s slice_tokens, (s + 1) slice_tokens) (whole 1024-token
  // blocks) and writes the fp32 sum to partial[u S + s]; gram_fixup_kernel adds the slices.
  const bool whole = blockIdx.x < full;
  const int64_t item = whole ? 0 : blockIdx.x - full;
  const int64_t tile = whole ? blockIdx.x : full + item / S;
  const int64_t mbeg = whole ? 0 : (item % S) * slice_tokens;
  const int64_t mend = whole ? M : (mbeg + slice_tokens < M ? mbeg + slice_tokens : M);
  // upper-triangle tile (i, j), i <= j, of T x T tiles: tile = i T - i (i - 1) / 2 + (j - i)
  const int64_t T = K / GT;
  int64_t i = 0, rem = tile;
  while (rem >= T - i) {
    rem -= T - i;
    ++i;
  }
  const int64_t k1b = i * GT, k2b = (i + rem) * GT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // this thread's 8 x 8 block: tokens 8 tg .. + 7 of the step, channels 8 cg .. + 7 of its range
  const int tg = tid & 7, cg = (tid >> 3) & 15;
  const bool second = tid >= 128;
  const uint16_t* src = X + (second ? k2b : k1b) + 8 * cg;
  uint16_t (*dst)[GT][GPITCH] = second ? t2 : t1;
  u32x4 rows[8];
  int valid = 0;  // rows past mend: loaded from row mend - 1 (no branch, so no wait on the prefetch), zeroed at the store
  auto load = [&](int64_t m0) {
    valid = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t m = m0 + 8 * tg + r;
      rows[r] = *reinterpret_cast<const u32x4*>(src + (m < mend ? m : mend - 1) * ldx);
      valid |= (m < mend ? 1 : 0) << r;
    }
  };
  auto store = [&](int b) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (!((valid >> r) & 1)) rows[r] = (u32x4){0u, 0u, 0u, 0u};
    // pair the tokens of each channel: P[a][c] = (X[2a][c], X[2a+1][c]) as one 32-bit word
    uint32_t P[4][8];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = rows[2 * a][w], y = rows[2 * a + 1][w];
        P[a][2 * w] = __builtin_amdgcn_perm(y, x, 0x05040100u);      // (x.lo, y.lo)
        P[a][2 * w + 1] = __builtin_amdgcn_perm(y, x, 0x07060302u);  // (x.hi, y.hi)
      }
#pragma unroll
    for (int c = 0; c < 8; ++c)
      *reinterpret_cast<u32x4*>(&dst[b][8 * cg + c][8 * tg]) = (u32x4){P[0][c], P[1][c], P[2][c], P[3][c]};
  };
  f32x16 acc[2][2], tot[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][c][e] = tot[a][c][e] = 0.0f;
  const int r1 = 64 * (wave >> 1), c2 = 64 * (wave & 1);  // this wave's rows (k1) and columns (k2)
  const int fr = lane & 31, fk = 8 * (lane >> 5);
  // a slice starts on a 1024-token boundary, so the block sums below are the same blocks of
  // tokens as in a whole tile
  const int64_t steps = (mend - mbeg + GS - 1) / GS;
  load(mbeg);
  store(0);
  __syncthreads();
  for (int64_t st = 0; st < steps; ++st) {
    const int b = (int)(st & 1);
    if (st + 1 < steps) load(mbeg + (st + 1) * GS);
#pragma unroll
    for (int h = 0; h < GS / 16; ++h) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) fa[a] = *reinterpret_cast<const bf16x8*>(&t1[b][r1 + 32 * a + fr][16 * h + fk]);
#pragma unroll
      for (int c = 0; c < 2; ++c) fb[c] = *reinterpret_cast<const bf16x8*>(&t2[b][c2 + 32 * c + fr][16 * h + fk]);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[a], fb[c], acc[a][c], 0, 0, 0);
    }
    if ((st + 1) % kGramBlockSteps == 0) {  // close one 1024-token block of the sum
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          tot[a][c] += acc[a][c];
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[a][c][e] = 0.0f;
        }
    }
    if (st + 1 < steps) store(b ^ 1);  // the buffer read in step st - 1 (done before its barrier)
    __syncthreads();
  }
  // 32x32 result layout: lane l holds column l % 32, rows 8 (e / 4) + 4 (l / 32) + e % 4.
  if (!whole) {  // a slice: its fp32 sum, tile-local [k1][k2]
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
  // G[k1][k2] and, off the diagonal tiles, G[k2][k1]: rows of G_hi, then rows of G_lo.
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float g = tot[a][c][e] + acc[a][c][e];
        const int64_t k1 = k1b + r1 + 32 * a + 8 * (e / 4) + 4 * (lane >> 5) + (e % 4);
        const int64_t k2 = k2b + c2 + 32 * c + (lane & 31);
        const uint16_t hi = bf16_bits(g);
        const uint16_t lo = bf16_bits(g - __uint_as_float((uint32_t)hi << 16));  // g - hi: exact
        Gs[k1 * K + k2] = hi;
        Gs[(K + k1) * K + k2] = lo;
        if (k1b != k2b) {
          Gs[k2 * K + k1] = hi;
          Gs[(K + k2) * K + k1] = lo;
        }
      }
}

// The split tiles: element (k1, k2) of tile full + u is the sum of its S slices in slice order,
// starting from 0 -- the order in which a whole tile adds its 1024-token block sums, so with one
// block per slice the result is the same bits as the whole-tile kernel's.
__global__ __launch_bounds__(256) void gram_fixup_kernel(const float* __restrict__ partial, int64_t K,
                                                          int64_t full, int S, uint16_t* __restrict__ Gs) {
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
  const int64_t k1 = k1b + k1l, k2 = k2b + k2l;
  const uint16_t hi = bf16_bits(g);
  const uint16_t lo = bf16_bits(g - __uint_as_float((uint32_t)hi << 16));
  Gs[k1 * K + k2] = hi;
  Gs[(K + k1) * K + k2] = lo;
  if (k1b != k2b) {
    Gs[k2 * K + k1] = hi;
    Gs[(K + k2) * K + k1] = lo;
  }
}

// Two blocks per CU on 256 CUs.  With tiles = q 512 + r, the first q 512 tiles run whole; the r
// tiles of the last, partial round are cut into S token slices of whole 1024-token blocks, so
// that r S is about one round (K = 4096: 528 tiles, 16 of them in 16 slices each).
constexpr int64_t kGramSlots = 512;
constexpr int64_t kGramBlockTokens = GS * kGramBlockSteps;

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
  gram_kernel<<<(unsigned)(p.full + p.r * p.S), 256, 0, st>>>(X, M, K, ldx, Gs, p.full, p.S, p.slice_tokens,
                                                             partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.r == 0) return e;
  gram_fixup_kernel<<<dim3((unsigned)(GT * GT / 256), (unsigned)p.r), 256, 0, st>>>(partial, K, p.full, p.S, Gs);
  return hipGetLastError();
}

}  // namespace awq

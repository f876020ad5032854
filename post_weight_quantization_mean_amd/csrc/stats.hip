// Step 1 of the hot path: the per-input-channel activation statistic
//   a_j = (1/M) sum_m |X[m, j]|
// ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §1: the mean absolute activation per input
// channel; the dreamvfia.cn AWQ report, §二, writes it (1/B) sum_b |X_bk|).
//
// HBM-bound column reduction.  Each lane owns 16 bytes of a row (8 bf16 or 4 fp32 columns),
// so a wave reads 1 KiB contiguous per row.  The row splits are interleaved, not contiguous:
// in grid iteration t, split y, wave w reads rows ((t * splits + y) * 4 + w) * 4 + u,
// u = 0..3 (four independent loads in flight).  The whole grid therefore sweeps X as one
// moving window of a few hundred consecutive rows, which keeps the DRAM accesses local;
// with about two 4-wave blocks per CU a plain streaming read reaches ~7 TB/s on MI355X, where
// many more waves, or far-apart row ranges, stay near 5-6 TB/s (measured).  Every |x| is
// accumulated in fp64: for bf16/fp32 inputs of ordinary range the column sums are then exact
// and independent of summation order.  Partials per (split, column) go to the workspace and
// a second kernel sums them in a fixed order, divides by M and rounds once to fp32.  A NaN/Inf
// input makes its column sum non-finite, which the finalize kernel turns into
// AWQ_FLAG_NONFINITE_X.
#include "awq_internal.h"

namespace awq {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// X is streamed once: non-temporal loads keep it from displacing the caches' other contents

constexpr int kStatsWaves = 4;
constexpr int kStatsThreads = kStatsWaves * 64;
constexpr int kStatsRows = 4;  // consecutive rows per wave per iteration

template <bool F32>
__global__ __launch_bounds__(kStatsThreads) void stats_partial_kernel(
    const void* __restrict__ X, int64_t M, int64_t K, int64_t ldx, double* __restrict__ partial) {
  constexpr int VEC = F32 ? 4 : 8;   // columns per lane (16 bytes)
  constexpr int BCOLS = 64 * VEC;    // columns per block
  constexpr int U = kStatsRows;
  __shared__ double red[kStatsWaves][BCOLS];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t col = (int64_t)blockIdx.x * BCOLS + lane * VEC;
  const int64_t rstep = (int64_t)gridDim.y * kStatsWaves * U;  // rows per grid iteration
  int64_t r = ((int64_t)blockIdx.y * kStatsWaves + wave) * U;

  double acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.0;

  // |x| of one 16-byte piece into the lane's column sums
  auto add = [&](const u32x4& v) {
    if constexpr (F32) {
      const f32x4 f = __builtin_bit_cast(f32x4, v);
      acc[0] += fabs((double)f.x);
      acc[1] += fabs((double)f.y);
      acc[2] += fabs((double)f.z);
      acc[3] += fabs((double)f.w);
    } else {
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 word.
        // Clearing the sign bit gives |x| directly.
        acc[2 * i] += (double)__uint_as_float((u[i] << 16) & 0x7fffffffu);
        acc[2 * i + 1] += (double)__uint_as_float(u[i] & 0x7fff0000u);
      }
    }
  };
  if (col < K) {
    const uint8_t* base = static_cast<const uint8_t*>(X) + col * (F32 ? 4 : 2);
    const int64_t pitch = ldx * (F32 ? 4 : 2);
    auto row = [&](int64_t rr) { return reinterpret_cast<const u32x4*>(base + rr * pitch); };
#pragma unroll 2
    for (; r + U <= M; r += rstep) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(row(r + u));
#pragma unroll
      for (int u = 0; u < U; ++u) add(v[u]);
    }
    if (r < M) {  // the last, partial row quad (M % 4 rows)
      for (int u = 0; r + u < M; ++u) add(__builtin_nontemporal_load(row(r + u)));
    }
  }
#pragma unroll
  for (int i = 0; i < VEC; ++i) red[wave][lane * VEC + i] = acc[i];
  __syncthreads();
  // Fixed-order combine of the waves, then one store per column.
  for (int c = threadIdx.x; c < BCOLS; c += kStatsThreads) {
    const int64_t gc = (int64_t)blockIdx.x * BCOLS + c;
    if (gc < K) {
      double s = 0.0;
#pragma unroll
      for (int w = 0; w < kStatsWaves; ++w) s += red[w][c];
      partial[gc * gridDim.y + blockIdx.y] = s;  // [column][split]
    }
  }
}

// Eight lanes per column: lane t sums splits t, t + 8, t + 16, ... in order, then a fixed
// xor tree (1, 2, 4) combines the eight, so the result does not depend on scheduling.
constexpr int kFinThreads = 256;
constexpr int kFinCols = kFinThreads / 8;

__global__ __launch_bounds__(kFinThreads) void stats_finalize_kernel(const double* __restrict__ partial,
                                                                    int splits, int64_t M, int64_t K,
                                                                    float* __restrict__ a_out,
                                                                    uint32_t* __restrict__ flags) {
  const int64_t j = (int64_t)blockIdx.x * kFinCols + (threadIdx.x >> 3);
  const int t = threadIdx.x & 7;
  double s = 0.0;
  if (j < K) {
    const double* p = partial + j * splits;
    for (int i = t; i < splits; i += 8) s += p[i];
  }
  s += __shfl_xor(s, 1, 8);
  s += __shfl_xor(s, 2, 8);
  s += __shfl_xor(s, 4, 8);
  if (j < K && t == 0) {
    if (!isfinite(s)) atomicOr(flags, kFlagNonfiniteX);
    a_out[j] = (float)(s / (double)M);
  }
}

}  // namespace

StatsPlan stats_plan(int64_t M, int64_t K, bool f32) {
  const int vec = f32 ? 4 : 8;
  StatsPlan p;
  p.col_blocks = (int)((K + 64 * vec - 1) / (64 * vec));
  // At most two 4-wave blocks per CU (512 in all), but at least four iterations per wave so
  // that the fp64 partials stay a small fraction of the bytes read.  The bound is a hard one:
  // a grid a few blocks past 512 puts a third block on some CUs and ran 15% slower (measured:
  // 16384 x 14336 bf16 took 85 us with 532 blocks, 75 us with 504).
  int64_t want = 512 / p.col_blocks;
  if (want < 1) want = 1;
  int64_t max_splits = M / (4 * kStatsWaves * kStatsRows);
  if (max_splits < 1) max_splits = 1;
  p.splits = (int)(want < max_splits ? want : max_splits);
  return p;
}

hipError_t launch_stats(const void* X, bool f32, int64_t M, int64_t K, int64_t ldx, float* a_out,
                        double* partial, const StatsPlan& plan, uint32_t* flags, hipStream_t st) {
  dim3 grid(plan.col_blocks, plan.splits);
  if (f32)
    stats_partial_kernel<true><<<grid, kStatsThreads, 0, st>>>(X, M, K, ldx, partial);
  else
    stats_partial_kernel<false><<<grid, kStatsThreads, 0, st>>>(X, M, K, ldx, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  stats_finalize_kernel<<<(unsigned)((K + kFinCols - 1) / kFinCols), kFinThreads, 0, st>>>(
      partial, plan.splits, M, K, a_out, flags);
  return hipGetLastError();
}

}  // namespace awq

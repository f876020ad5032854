// Step 2 (the scale candidates), the per-group quantization ranges that step 3 needs, and the
// final reduction + argmin of steps 4-5.
//
// "AWQ：为什么 4-bit 权重量化要先观察 Activation", §3 and §4: twenty ratios alpha = i/20
// (0 .. 0.95), r_j = max(a_j^alpha, 1e-4) clamped BEFORE the normalisation by
// sqrt(max r * min r); alpha = 0 gives all ones; the first minimum of the loss wins.
// §7: groups of 128 consecutive input channels share a step Delta and a zero point z.
#include "awq_internal.h"

namespace awq {
namespace {

// ---- scale table ---------------------------------------------------------------------------
// fp64 power, clamp and normalisation, each s rounded once to fp32; rs = fp32(1 / s).
// x^alpha is non-decreasing in x for alpha >= 0, so max_j r_j = max((max_j a_j)^alpha, 1e-4)
// and likewise for the minimum: the normalisation needs only the extremes of a, and every
// (candidate, channel) is independent.  Each block reduces max / min of a itself (a is a few
// KiB and stays in L2) and writes 1024 channels of one candidate.
constexpr int kScaleThreads = 256;
constexpr int kScalePerThread = 4;
constexpr int kScaleCols = kScaleThreads * kScalePerThread;

// column block bx of candidate i
__device__ __forceinline__ void scale_table_block(const float* __restrict__ a, int64_t K, int n_grid,
                                                  float* __restrict__ s_tab, float* __restrict__ rs_tab,
                                                  float2* __restrict__ sr_tab, uint32_t* __restrict__ flags,
                                                  int bx, int i) {
  __shared__ double smax[kScaleThreads / 64];
  __shared__ double smin[kScaleThreads / 64];
  const double alpha = (double)i / (double)n_grid;
  double lmax = 0.0, lmin = INFINITY;
  bool bad = false;  // a_j negative, NaN or infinite
  for (int64_t j = threadIdx.x; j < K; j += kScaleThreads) {
    const double aj = (double)a[j];
    if (!(aj >= 0.0) || isinf(aj)) bad = true;
    lmax = fmax(lmax, aj);
    lmin = fmin(lmin, aj);
  }
  for (int off = 32; off > 0; off >>= 1) {
    lmax = fmax(lmax, __shfl_xor(lmax, off));
    lmin = fmin(lmin, __shfl_xor(lmin, off));
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) {
    smax[wave] = lmax;
    smin[wave] = lmin;
  }
  __syncthreads();
  double amax = smax[0], amin = smin[0];
  for (int w = 1; w < kScaleThreads / 64; ++w) {
    amax = fmax(amax, smax[w]);
    amin = fmin(amin, smin[w]);
  }
  const double norm = sqrt(fmax(pow(amax, alpha), 1e-4) * fmax(pow(amin, alpha), 1e-4));
  bool bad_s = false;
#pragma unroll
  for (int t = 0; t < kScalePerThread; ++t) {
    const int64_t j = (int64_t)bx * kScaleCols + t * kScaleThreads + threadIdx.x;
    if (j < K) {
      const double r = fmax(pow((double)a[j], alpha), 1e-4);
      const float sv = (float)(r / norm);
      const float rs = (float)(1.0 / (double)sv);
      if (!(sv > 0.0f) || isinf(sv) || isinf(rs)) bad_s = true;
      s_tab[(int64_t)i * K + j] = sv;
      rs_tab[(int64_t)i * K + j] = rs;
      sr_tab[(int64_t)i * K + j] = make_float2(sv, rs);
    }
  }
  // every block sees all of a; the ones of column block 0 report a bad statistic
  if (bad_s || (bad && bx == 0)) atomicOr(flags, kFlagScaleRange);
}

__global__ __launch_bounds__(kScaleThreads) void scale_table_kernel(const float* __restrict__ a, int64_t K,
                                                                   int n_grid, float* __restrict__ s_tab,
                                                                   float* __restrict__ rs_tab,
                                                                   float2* __restrict__ sr_tab,
                                                                   uint32_t* __restrict__ flags) {
  scale_table_block(a, K, n_grid, s_tab, rs_tab, sr_tab, flags, blockIdx.x, blockIdx.y);
}

// blocks 0 .. n_scale - 1: the scale table (column block b % cols of candidate b / cols); the
// rest: the copy of X in operand order (xfrag_block)
__global__ __launch_bounds__(kScaleThreads) void scale_table_xfrag_kernel(
    const float* __restrict__ a, int64_t K, int n_grid, float* __restrict__ s_tab, float* __restrict__ rs_tab,
    float2* __restrict__ sr_tab, uint32_t* __restrict__ flags, int cols, const uint16_t* __restrict__ X,
    int64_t M, int64_t ldx, uint16_t* __restrict__ Xf) {
  const int64_t n_scale = (int64_t)cols * n_grid;
  const int64_t b = blockIdx.x;
  if (b < n_scale)
    scale_table_block(a, K, n_grid, s_tab, rs_tab, sr_tab, flags, (int)(b % cols), (int)(b / cols));
  else
    xfrag_block(X, M, K, ldx, Xf, b - n_scale, threadIdx.x);
}

// ---- group ranges: Delta and z of every (candidate, output channel, group) ---------------
// Four lanes share one row's group of 128 (32 channels, 64 bytes each, so a load instruction
// covers 16 rows x 64 bytes); a block covers 64 consecutive rows of one group, whose range
// slots are contiguous for every candidate.  W is read once; every candidate's scales for the
// group come from LDS.  Per candidate a lane forms its 32 scaled values, their max and min
// (v_max3 / v_min3), and the four lanes of a row combine through lane swizzles.  The
// divisions Delta = max(max - min, 1e-5) / 15 and z = clamp(rne(-min / Delta), 0, 15) (both
// correctly rounded) are spread over the four lanes (candidates q, q + 4, ...), and the
// results are gathered in LDS and written as contiguous runs.
constexpr int kRangeThreads = 256;
constexpr int kRangeRows = kRangeThreads / 4;  // 64 rows per block

template <bool WF32>
__global__ __launch_bounds__(kRangeThreads) void group_range_kernel(const void* __restrict__ W, int64_t N,
                                                                   int64_t K, int64_t ldw,
                                                                   const float* __restrict__ s_tab,
                                                                   int n_grid, float2* __restrict__ params,
                                                                   int64_t row_base, int64_t NP,
                                                                   uint32_t* __restrict__ flags) {
  // dynamic LDS: this group's scales for every candidate (n_grid x 128 floats), then the
  // (Delta, z) of every candidate and row (n_grid x 64 float2)
  extern __shared__ float4 dyn[];
  float4* ss = dyn;
  float2* out = reinterpret_cast<float2*>(dyn + n_grid * (kGroup / 4));
  const int64_t G = K / kGroup;
  const int64_t NPw = padded_n(N);  // this weight's padded rows (of the NP in the table)
  const int64_t g = blockIdx.y;
  const int64_t nb = (int64_t)blockIdx.x * kRangeRows;   // first row of the block
  const int tid = threadIdx.x;
  const int row = tid >> 2, q = tid & 3;
  const int64_t n = nb + row;
  const bool live = n < N;

  for (int t = tid; t < n_grid * (kGroup / 4); t += kRangeThreads) {
    const int al = t / (kGroup / 4), c4 = t % (kGroup / 4);
    ss[t] = *reinterpret_cast<const float4*>(s_tab + (int64_t)al * K + g * kGroup + 4 * c4);
  }

  float w[32];
  if (live) {
    if constexpr (WF32) {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(W) + n * ldw + g * kGroup + 32 * q);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float4 u = p[t];
        w[4 * t] = u.x; w[4 * t + 1] = u.y; w[4 * t + 2] = u.z; w[4 * t + 3] = u.w;
      }
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + n * ldw + g * kGroup + 32 * q);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint4 u = p[t];
        const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          w[8 * t + 2 * h] = __uint_as_float(uu[h] << 16);
          w[8 * t + 2 * h + 1] = __uint_as_float(uu[h] & 0xffff0000u);
        }
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < 32; ++t) w[t] = 0.0f;
  }
  bool bad = false;
#pragma unroll
  for (int t = 0; t < 32; ++t) bad |= !isfinite(w[t]);
  __syncthreads();

  // candidates four at a time; afterwards lane q finishes candidate al4 + q of its row
#pragma unroll 1
  for (int al4 = 0; al4 < n_grid; al4 += 4) {
    float mxd[4], mnd[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int al = al4 + d < n_grid ? al4 + d : n_grid - 1;
      const float4* sp = ss + al * (kGroup / 4) + 8 * q;
      float mx = -INFINITY, mn = INFINITY;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float4 sv = sp[t];
        const float v0 = w[4 * t] * sv.x, v1 = w[4 * t + 1] * sv.y;
        const float v2 = w[4 * t + 2] * sv.z, v3 = w[4 * t + 3] * sv.w;
        mx = fmaxf(fmaxf(mx, v0), v1);
        mx = fmaxf(fmaxf(mx, v2), v3);
        mn = fminf(fminf(mn, v0), v1);
        mn = fminf(fminf(mn, v2), v3);
      }
      mxd[d] = max4(mx);
      mnd[d] = min4(mn);
    }
    const float mx = q == 0 ? mxd[0] : q == 1 ? mxd[1] : q == 2 ? mxd[2] : mxd[3];
    const float mn = q == 0 ? mnd[0] : q == 1 ? mnd[1] : q == 2 ? mnd[2] : mnd[3];
    const int al = al4 + q;
    if (al < n_grid) {
      const float range = mx - mn;
      if (live && !isfinite(range)) bad = true;
      const float delta = fmaxf(range, 1e-5f) / 15.0f;
      const float z = fminf(fmaxf(rintf(-mn / delta), 0.0f), 15.0f);
      out[al * kRangeRows + row] = make_float2(delta, z);
    }
  }
  __syncthreads();
  // rows nb .. nb + 63 occupy 64 consecutive slots starting at range_slot(nb), after the
  // row_base padded rows of the weights before this one
  const int64_t slot0 = row_base + range_slot(nb);
  for (int t = tid; t < n_grid * kRangeRows; t += kRangeThreads) {
    const int al = t / kRangeRows, j = t % kRangeRows;  // j: slot offset
    // slot offset j = 32 w' + 2 jj + i  <->  row offset 32 w' + 16 i + jj
    const int r = (j & ~31) + 16 * (j & 1) + ((j & 31) >> 1);
    if (nb + r < NPw) params[((int64_t)al * G + g) * NP + slot0 + j] = out[al * kRangeRows + r];
  }
  if (live && bad) atomicOr(flags, kFlagNonfiniteW);
}

// ---- fixed-order loss reduction, first argmin, copy of the winning scales ---------------
constexpr int kSelectThreads = 1024;

// per_tile: 1 (one sum per tile) or 4 (one per wave of the tile, added in wave order first: the
// same value the tile's block forms when it adds its four wave sums itself)
__global__ __launch_bounds__(kSelectThreads) void select_kernel(
    const double* __restrict__ partial, int64_t tiles, int n_grid, double count, int64_t K,
    const float* __restrict__ s_tab, double* __restrict__ losses, int32_t* __restrict__ best,
    float* __restrict__ s_best, uint32_t* __restrict__ flags, int per_tile) {
  __shared__ double sl[64];
  __shared__ int sbest;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int al = wave; al < n_grid; al += kSelectThreads / 64) {
    double s = 0.0;
    for (int64_t t = lane; t < tiles; t += 64) {
      const int64_t u = (int64_t)al * tiles + t;
      s += per_tile == 1 ? partial[u]
                         : ((partial[4 * u] + partial[4 * u + 1]) + partial[4 * u + 2]) + partial[4 * u + 3];
    }
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) sl[al] = s / count;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int b = 0;
    bool bad = false;
    for (int al = 0; al < n_grid; ++al) {
      losses[al] = sl[al];
      if (!isfinite(sl[al])) bad = true;
      if (sl[al] < sl[b]) b = al;
    }
    if (bad) atomicOr(flags, kFlagNonfiniteLoss);
    *best = b;
    sbest = b;
  }
  __syncthreads();
  const float* src = s_tab + (int64_t)sbest * K;
  for (int64_t j = threadIdx.x; j < K; j += kSelectThreads) s_best[j] = src[j];
}

}  // namespace

hipError_t launch_scale_table(const float* a, int64_t K, int n_grid, float* s_tab, float* rs_tab,
                              float2* sr_tab, uint32_t* flags, hipStream_t st) {
  const dim3 grid((unsigned)((K + kScaleCols - 1) / kScaleCols), (unsigned)n_grid);
  scale_table_kernel<<<grid, kScaleThreads, 0, st>>>(a, K, n_grid, s_tab, rs_tab, sr_tab, flags);
  return hipGetLastError();
}

hipError_t launch_scale_table_xfrag(const float* a, int64_t K, int n_grid, float* s_tab, float* rs_tab,
                                    float2* sr_tab, uint32_t* flags, const uint16_t* X, int64_t M,
                                    int64_t ldx, uint16_t* Xf, hipStream_t st) {
  if (K % 64 != 0) return hipErrorInvalidValue;
  const int64_t cols = (K + kScaleCols - 1) / kScaleCols;
  const int64_t blocks = cols * n_grid + (M + 31) / 32 * (K / 64);
  if (blocks <= 0 || blocks >= (int64_t)INT32_MAX) return hipErrorInvalidValue;
  scale_table_xfrag_kernel<<<(unsigned)blocks, kScaleThreads, 0, st>>>(a, K, n_grid, s_tab, rs_tab, sr_tab, flags,
                                                                      (int)cols, X, M, ldx, Xf);
  return hipGetLastError();
}

hipError_t launch_group_range(const void* W, bool wf32, int64_t N, int64_t K, int64_t ldw,
                              const float* s_tab, int n_grid, float2* params, int64_t row_base,
                              int64_t NP, uint32_t* flags, hipStream_t st) {
  const dim3 grid((unsigned)((N + kRangeRows - 1) / kRangeRows), (unsigned)(K / kGroup));
  const size_t lds = (size_t)n_grid * (kGroup * 4 + kRangeRows * 8);  // <= 64 KiB (n_grid <= 64)
  if (wf32)
    group_range_kernel<true><<<grid, kRangeThreads, lds, st>>>(W, N, K, ldw, s_tab, n_grid, params, row_base,
                                                               NP, flags);
  else
    group_range_kernel<false><<<grid, kRangeThreads, lds, st>>>(W, N, K, ldw, s_tab, n_grid, params, row_base,
                                                                NP, flags);
  return hipGetLastError();
}

hipError_t launch_select(const double* partial, int64_t tiles, int n_grid, int64_t M, int64_t N,
                         int64_t K, const float* s_tab, double* losses, int32_t* best,
                         float* s_best, uint32_t* flags, hipStream_t st, int per_tile) {
  const double count = (double)M * (double)N;
  select_kernel<<<1, kSelectThreads, 0, st>>>(partial, tiles, n_grid, count, K, s_tab, losses,
                                              best, s_best, flags, per_tile);
  return hipGetLastError();
}

}  // namespace awq

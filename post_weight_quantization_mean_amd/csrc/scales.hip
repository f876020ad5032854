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

// ---- scale table: one block per candidate -----------------------------------------------
// fp64 power, clamp and normalisation, each s rounded once to fp32; rs = fp32(1 / s).
constexpr int kScaleThreads = 1024;

__global__ __launch_bounds__(kScaleThreads) void scale_table_kernel(const float* __restrict__ a,
                                                                   int64_t K, int n_grid,
                                                                   float* __restrict__ s_tab,
                                                                   float* __restrict__ rs_tab,
                                                                   float2* __restrict__ sr_tab,
                                                                   uint32_t* __restrict__ flags) {
  __shared__ double smax[kScaleThreads / 64];
  __shared__ double smin[kScaleThreads / 64];
  const int i = blockIdx.x;
  const double alpha = (double)i / (double)n_grid;
  double lmax = 0.0, lmin = INFINITY;
  bool bad = false;
  for (int64_t j = threadIdx.x; j < K; j += kScaleThreads) {
    const double aj = (double)a[j];
    if (!(aj >= 0.0) || isinf(aj)) bad = true;
    const double r = fmax(pow(aj, alpha), 1e-4);
    lmax = fmax(lmax, r);
    lmin = fmin(lmin, r);
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
  double rmax = smax[0], rmin = smin[0];
  for (int w = 1; w < kScaleThreads / 64; ++w) {
    rmax = fmax(rmax, smax[w]);
    rmin = fmin(rmin, smin[w]);
  }
  const double norm = sqrt(rmax * rmin);
  for (int64_t j = threadIdx.x; j < K; j += kScaleThreads) {
    const double r = fmax(pow((double)a[j], alpha), 1e-4);
    const float s = (float)(r / norm);
    const float rs = (float)(1.0 / (double)s);
    if (!(s > 0.0f) || isinf(s) || isinf(rs)) bad = true;
    s_tab[(int64_t)i * K + j] = s;
    rs_tab[(int64_t)i * K + j] = rs;
    sr_tab[(int64_t)i * K + j] = make_float2(s, rs);
  }
  if (bad) atomicOr(flags, kFlagScaleRange);
}

// ---- group ranges: Delta and z of every (candidate, output channel, group) ---------------
// Sixteen lanes share one group of 128 (8 channels each); W is read once and every
// candidate's range is formed from it.  Delta = max(max - min, 1e-5) / 15 and
// z = clamp(rne(-min / Delta), 0, 15), both with correctly rounded fp32 division.
template <bool WF32>
__global__ __launch_bounds__(256) void group_range_kernel(const void* __restrict__ W, int64_t N,
                                                         int64_t K, int64_t ldw,
                                                         const float* __restrict__ s_tab,
                                                         int n_grid, float2* __restrict__ params,
                                                         uint32_t* __restrict__ flags) {
  const int64_t G = K / kGroup;
  const int64_t NP = padded_n(N);
  // 16 lanes per (group g, channel n); a block covers 16 consecutive channels of one group
  const int64_t grp = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const bool live = grp < N * G;
  const int64_t g = live ? grp / N : 0;
  const int64_t n = live ? grp % N : 0;
  const int64_t k0 = g * kGroup + sub * 8;

  float w[8];
  if (live) {
    if constexpr (WF32) {
      const float* p = static_cast<const float*>(W) + n * ldw + k0;
      const float4 u0 = *reinterpret_cast<const float4*>(p);
      const float4 u1 = *reinterpret_cast<const float4*>(p + 4);
      w[0] = u0.x; w[1] = u0.y; w[2] = u0.z; w[3] = u0.w;
      w[4] = u1.x; w[5] = u1.y; w[6] = u1.z; w[7] = u1.w;
    } else {
      const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + n * ldw + k0);
      const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[2 * i] = __uint_as_float(uu[i] << 16);
        w[2 * i + 1] = __uint_as_float(uu[i] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = 0.0f;
  }
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) bad |= !isfinite(w[i]);

  for (int al = 0; al < n_grid; ++al) {
    const float* sp = s_tab + (int64_t)al * K + k0;
    const float4 s0 = *reinterpret_cast<const float4*>(sp);
    const float4 s1 = *reinterpret_cast<const float4*>(sp + 4);
    const float s[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    float mx = -INFINITY, mn = INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = w[i] * s[i];
      mx = fmaxf(mx, v);
      mn = fminf(mn, v);
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      mx = fmaxf(mx, __shfl_xor(mx, off, 16));
      mn = fminf(mn, __shfl_xor(mn, off, 16));
    }
    if (live && sub == 0) {
      const float range = mx - mn;
      if (!isfinite(range)) bad = true;
      const float delta = fmaxf(range, 1e-5f) / 15.0f;
      const float z = fminf(fmaxf(rintf(-mn / delta), 0.0f), 15.0f);
      params[((int64_t)al * G + g) * NP + range_slot(n)] = make_float2(delta, z);
    }
  }
  if (live && bad) atomicOr(flags, kFlagNonfiniteW);
}

// ---- fixed-order loss reduction, first argmin, copy of the winning scales ---------------
constexpr int kSelectThreads = 1024;

__global__ __launch_bounds__(kSelectThreads) void select_kernel(
    const double* __restrict__ partial, int64_t tiles, int n_grid, double count, int64_t K,
    const float* __restrict__ s_tab, double* __restrict__ losses, int32_t* __restrict__ best,
    float* __restrict__ s_best, uint32_t* __restrict__ flags) {
  __shared__ double sl[64];
  __shared__ int sbest;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int al = wave; al < n_grid; al += kSelectThreads / 64) {
    double s = 0.0;
    for (int64_t t = lane; t < tiles; t += 64) s += partial[(int64_t)al * tiles + t];
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
  scale_table_kernel<<<n_grid, kScaleThreads, 0, st>>>(a, K, n_grid, s_tab, rs_tab, sr_tab, flags);
  return hipGetLastError();
}

hipError_t launch_group_range(const void* W, bool wf32, int64_t N, int64_t K, int64_t ldw,
                              const float* s_tab, int n_grid, float2* params, uint32_t* flags,
                              hipStream_t st) {
  const int64_t groups = N * (K / kGroup);
  const unsigned blocks = (unsigned)((groups + 15) / 16);
  if (wf32)
    group_range_kernel<true><<<blocks, 256, 0, st>>>(W, N, K, ldw, s_tab, n_grid, params, flags);
  else
    group_range_kernel<false><<<blocks, 256, 0, st>>>(W, N, K, ldw, s_tab, n_grid, params, flags);
  return hipGetLastError();
}

hipError_t launch_select(const double* partial, int64_t tiles, int n_grid, int64_t M, int64_t N,
                         int64_t K, const float* s_tab, double* losses, int32_t* best,
                         float* s_best, uint32_t* flags, hipStream_t st) {
  const double count = (double)M * (double)N;
  select_kernel<<<1, kSelectThreads, 0, st>>>(partial, tiles, n_grid, count, K, s_tab, losses,
                                              best, s_best, flags);
  return hipGetLastError();
}

}  // namespace awq

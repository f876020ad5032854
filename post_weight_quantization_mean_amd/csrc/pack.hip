// Step 5 of the hot path: real quantization of S W at the winning scales and packing of the
// codes ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §7: codes, group scales and zero
// points form the artefact; §8: g128 with fp16 scale and fp16 zero costs 4.25 bits/weight;
// "5. 核心模块", §5.3: INT4 codes are usually packed eight per int32).
//
// Exact fp32 contract, bit-identical to its definition: v = W*s (one rounding),
// Delta = max(max v - min v, 1e-5) / 15 and both quotients -min/Delta and v/Delta use
// correctly rounded division, rne() is round-half-to-even.  Each lane packs its codes eight per
// int32 (nibble i <- k = 8j+i).  Bandwidth-bound: 2 bytes of W read and 0.53 bytes written
// per weight.
#include "awq_internal.h"

namespace awq {
namespace {

// A block covers 64 rows of one group: four lanes share a row, lane q owning channels
// 32 q .. 32 q + 31 (64 bytes, so a load instruction covers 16 rows x 64 bytes); the group's
// scales come from LDS.  A row's Delta, reciprocal and zero point are formed by its four lanes
// alike and serve 32 values each.
constexpr int kPackThreads = 256;
constexpr int kPackRows = kPackThreads / 4;

template <bool WF32>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(const void* __restrict__ W, int64_t N, int64_t K,
                                                           int64_t ldw, const float* __restrict__ s,
                                                           int32_t* __restrict__ qweight,
                                                           uint16_t* __restrict__ scales,
                                                           uint16_t* __restrict__ zeros,
                                                           uint32_t* __restrict__ flags) {
  __shared__ float4 ss[kGroup / 4];
  const int64_t G = K / kGroup;
  const int64_t g = blockIdx.y;
  const int row = threadIdx.x >> 2, q = threadIdx.x & 3;
  const int64_t n = (int64_t)blockIdx.x * kPackRows + row;
  const int64_t nn = n < N ? n : N - 1;  // rows past N load row N-1 and store nothing
  const int64_t k0 = g * kGroup + 32 * q;

  uint32_t bad = 0;
  if (threadIdx.x < kGroup / 4) {
    const float4 sv = *reinterpret_cast<const float4*>(s + g * kGroup + 4 * threadIdx.x);
    if (!(sv.x > 0.0f) || !(sv.y > 0.0f) || !(sv.z > 0.0f) || !(sv.w > 0.0f) || isinf(sv.x) ||
        isinf(sv.y) || isinf(sv.z) || isinf(sv.w))
      bad |= kFlagScaleRange;
    ss[threadIdx.x] = sv;
  }
  float w[32];
  if constexpr (WF32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(W) + nn * ldw + k0);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float4 u = p[t];
      w[4 * t] = u.x; w[4 * t + 1] = u.y; w[4 * t + 2] = u.z; w[4 * t + 3] = u.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + nn * ldw + k0);
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
  __syncthreads();

  float v[32];
  float mx = -INFINITY, mn = INFINITY, sum = 0.0f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float4 sv = ss[8 * q + t];
    const float sc[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int i = 4 * t + h;
      v[i] = w[i] * sc[h];  // s is finite and positive: a non-finite w gives a non-finite v
      sum += v[i];          // NaN (and Inf - Inf) reach the sum, an Inf the range
      mx = fmaxf(mx, v[i]);
      mn = fminf(mn, v[i]);
    }
  }
  uint32_t rbad = 0;
  if (!isfinite(sum)) rbad |= kFlagNonfiniteW;
  mx = max4(mx);
  mn = min4(mn);
  const float range = mx - mn;
  if (!isfinite(range)) rbad |= kFlagNonfiniteW;
  // Correctly rounded quotients a / b from a reciprocal y = RN(1 / b) and FMA corrections:
  // q1 = RN(q0 + RN(a - b q0) y) with q0 = RN(a y) is within one ulp of a / b, so
  // r1 = a - b q1 is exact and RN(q1 + r1 y) = RN(a / b) (Markstein's theorem for a
  // reciprocal within half an ulp and a quotient within one ulp; b here is positive and
  // normal, and quotients below 2^-126 either round to code z or are the tiny Delta floor).
  auto quot = [](float a, float b, float y) {
    const float q0 = a * y;
    const float q1 = fmaf(fmaf(-q0, b, a), y, q0);
    return fmaf(fmaf(-q1, b, a), y, q1);
  };
  const float delta = quot(fmaxf(range, 1e-5f), 15.0f, 1.0f / 15.0f);  // RN(range' / 15)
  const float y = 1.0f / delta;
  const int z = (int)fminf(fmaxf(rintf(quot(-mn, delta, y)), 0.0f), 15.0f);
  const float zf = (float)z;
  uint32_t word[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t wd = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float c = __builtin_amdgcn_fmed3f(rintf(quot(v[8 * j + i], delta, y)) + zf, 0.0f, 15.0f);
      wd |= (uint32_t)(int)c << (4 * i);
    }
    word[j] = wd;
  }
  if (n < N) {
    *reinterpret_cast<uint4*>(qweight + n * (K / 8) + g * 16 + 4 * q) = make_uint4(word[0], word[1], word[2], word[3]);
    if (q == 0) {
      const _Float16 d16 = (_Float16)delta;  // round to nearest even
      if (isinf((float)d16)) rbad |= kFlagF16Range;
      scales[n * G + g] = __builtin_bit_cast(uint16_t, d16);
      zeros[n * G + g] = __builtin_bit_cast(uint16_t, (_Float16)z);
    }
    bad |= rbad;
  }
  if (bad) atomicOr(flags, bad);
}

}  // namespace

hipError_t launch_pack(const void* W, bool wf32, int64_t N, int64_t K, int64_t ldw, const float* s,
                       int32_t* qweight, uint16_t* scales, uint16_t* zeros, uint32_t* flags,
                       hipStream_t st) {
  const dim3 grid((unsigned)((N + kPackRows - 1) / kPackRows), (unsigned)(K / kGroup));
  if (wf32)
    pack_kernel<true><<<grid, kPackThreads, 0, st>>>(W, N, K, ldw, s, qweight, scales, zeros, flags);
  else
    pack_kernel<false><<<grid, kPackThreads, 0, st>>>(W, N, K, ldw, s, qweight, scales, zeros, flags);
  return hipGetLastError();
}

}  // namespace awq

// Step 5 of the hot path: real quantization of S W at the winning scales and packing of the
// codes ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §7: codes, group scales and zero
// points form the artefact; §8: g128 with fp16 scale and fp16 zero costs 4.25 bits/weight;
// "5. 核心模块", §5.3: INT4 codes are usually packed eight per int32).
//
// Exact fp32 contract, bit-identical to its definition: v = W*s (one rounding),
// Delta = max(max v - min v, 1e-5) / 15 and both quotients -min/Delta and v/Delta use
// correctly rounded division, rne() is round-half-to-even.  Sixteen lanes own one row's group of
// 128 (8 channels per lane); each lane packs its 8 codes into one int32 (nibble i <- k = 8j+i),
// so sixteen lanes store 64 contiguous bytes of qweight.  Bandwidth-bound: 2 bytes of W read
// and 0.53 bytes written per weight.
#include "awq_internal.h"

namespace awq {
namespace {

// A block covers 64 rows of one group: lane (slot, sub) handles the 8 channels sub * 8 .. +7 of
// rows slot, slot + 16, slot + 32, slot + 48, with all four W loads in flight at once and the
// group's scales loaded once.
constexpr int kPackThreads = 256;
constexpr int kPackRows = 64;
constexpr int kPackRowsPerLane = kPackRows / 16;

template <bool WF32>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(const void* __restrict__ W, int64_t N, int64_t K,
                                                           int64_t ldw, const float* __restrict__ s,
                                                           int32_t* __restrict__ qweight,
                                                           uint16_t* __restrict__ scales,
                                                           uint16_t* __restrict__ zeros,
                                                           uint32_t* __restrict__ flags) {
  const int64_t G = K / kGroup;
  const int64_t g = blockIdx.y;
  const int slot = threadIdx.x >> 4, sub = threadIdx.x & 15;
  const int64_t k0 = g * kGroup + sub * 8;

  const float4 s0 = *reinterpret_cast<const float4*>(s + k0);
  const float4 s1 = *reinterpret_cast<const float4*>(s + k0 + 4);
  const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  uint32_t bad = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (!(sc[i] > 0.0f) || isinf(sc[i])) bad |= kFlagScaleRange;

  float w[kPackRowsPerLane][8];
#pragma unroll
  for (int rr = 0; rr < kPackRowsPerLane; ++rr) {
    const int64_t n = (int64_t)blockIdx.x * kPackRows + rr * 16 + slot;
    const int64_t nn = n < N ? n : N - 1;  // rows past N load row N-1 and store nothing
    if constexpr (WF32) {
      const float* p = static_cast<const float*>(W) + nn * ldw + k0;
      const float4 u0 = *reinterpret_cast<const float4*>(p);
      const float4 u1 = *reinterpret_cast<const float4*>(p + 4);
      w[rr][0] = u0.x; w[rr][1] = u0.y; w[rr][2] = u0.z; w[rr][3] = u0.w;
      w[rr][4] = u1.x; w[rr][5] = u1.y; w[rr][6] = u1.z; w[rr][7] = u1.w;
    } else {
      const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + nn * ldw + k0);
      const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[rr][2 * i] = __uint_as_float(uu[i] << 16);
        w[rr][2 * i + 1] = __uint_as_float(uu[i] & 0xffff0000u);
      }
    }
  }

#pragma unroll
  for (int rr = 0; rr < kPackRowsPerLane; ++rr) {
    const int64_t n = (int64_t)blockIdx.x * kPackRows + rr * 16 + slot;
    float v[8];
    float mx = -INFINITY, mn = INFINITY, sum = 0.0f;
    uint32_t rbad = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = w[rr][i] * sc[i];  // s is finite and positive: a non-finite w gives a non-finite v
      sum += v[i];              // NaN (and Inf - Inf) reach the sum, an Inf the range
      mx = fmaxf(mx, v[i]);
      mn = fminf(mn, v[i]);
    }
    if (!isfinite(sum)) rbad |= kFlagNonfiniteW;
    mx = max16(mx);
    mn = min16(mn);
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
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float q = __builtin_amdgcn_fmed3f(rintf(quot(v[i], delta, y)) + zf, 0.0f, 15.0f);
      word |= (uint32_t)(int)q << (4 * i);
    }
    if (n < N) {
      qweight[n * (K / 8) + g * 16 + sub] = (int32_t)word;
      if (sub == 0) {
        const _Float16 d16 = (_Float16)delta;  // round to nearest even
        if (isinf((float)d16)) rbad |= kFlagF16Range;
        scales[n * G + g] = __builtin_bit_cast(uint16_t, d16);
        zeros[n * G + g] = __builtin_bit_cast(uint16_t, (_Float16)z);
      }
      bad |= rbad;
    }
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

// Step 5 of the hot path: real quantization of S W at the winning scales and packing of the
// codes ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §7: codes, group scales and zero
// points form the artefact; §8: g128 with fp16 scale and fp16 zero costs 4.25 bits/weight;
// "5. 核心模块", §5.3: INT4 codes are usually packed eight per int32).
//
// Exact fp32 contract, bit-identical to its definition: v = W*s (one rounding),
// Delta = max(max v - min v, 1e-5) / 15 and both quotients -min/Delta and v/Delta use
// correctly rounded division, rne() is round-half-to-even.  Sixteen lanes own one group of
// 128 (8 channels per lane); each lane packs its 8 codes into one int32 (nibble i <- k = 8j+i),
// so a wave stores 256 contiguous bytes of qweight.  Bandwidth-bound: 2 bytes of W read and
// 0.53 bytes written per weight.
#include "awq_internal.h"

namespace awq {
namespace {

template <bool WF32>
__global__ __launch_bounds__(256) void pack_kernel(const void* __restrict__ W, int64_t N, int64_t K,
                                                  int64_t ldw, const float* __restrict__ s,
                                                  int32_t* __restrict__ qweight,
                                                  uint16_t* __restrict__ scales,
                                                  uint16_t* __restrict__ zeros,
                                                  uint32_t* __restrict__ flags) {
  const int64_t G = K / kGroup;
  const int64_t grp = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  if (grp >= N * G) return;  // whole 16-lane rows exit together
  const int64_t n = grp / G;
  const int64_t g = grp % G;
  const int64_t k0 = g * kGroup + sub * 8;

  float w[8];
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
  const float4 s0 = *reinterpret_cast<const float4*>(s + k0);
  const float4 s1 = *reinterpret_cast<const float4*>(s + k0 + 4);
  const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};

  uint32_t bad = 0;
  float v[8];
  float mx = -INFINITY, mn = INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (!(sc[i] > 0.0f) || isinf(sc[i])) bad |= kFlagScaleRange;
    if (!isfinite(w[i])) bad |= kFlagNonfiniteW;
    v[i] = w[i] * sc[i];
    if (!isfinite(v[i])) bad |= kFlagNonfiniteW;
    mx = fmaxf(mx, v[i]);
    mn = fminf(mn, v[i]);
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, off, 16));
    mn = fminf(mn, __shfl_xor(mn, off, 16));
  }
  const float range = mx - mn;
  if (!isfinite(range)) bad |= kFlagNonfiniteW;
  const float delta = fmaxf(range, 1e-5f) / 15.0f;
  const int z = (int)fminf(fmaxf(rintf(-mn / delta), 0.0f), 15.0f);
  const float zf = (float)z;
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float q = fminf(fmaxf(rintf(v[i] / delta) + zf, 0.0f), 15.0f);
    word |= (uint32_t)(int)q << (4 * i);
  }
  qweight[n * (K / 8) + g * 16 + sub] = (int32_t)word;
  if (sub == 0) {
    const _Float16 d16 = (_Float16)delta;  // round to nearest even
    if (isinf((float)d16)) bad |= kFlagF16Range;
    scales[n * G + g] = __builtin_bit_cast(uint16_t, d16);
    zeros[n * G + g] = __builtin_bit_cast(uint16_t, (_Float16)z);
  }
  if (bad) atomicOr(flags, bad);
}

}  // namespace

hipError_t launch_pack(const void* W, bool wf32, int64_t N, int64_t K, int64_t ldw, const float* s,
                       int32_t* qweight, uint16_t* scales, uint16_t* zeros, uint32_t* flags,
                       hipStream_t st) {
  const int64_t groups = N * (K / kGroup);
  const unsigned blocks = (unsigned)((groups + 15) / 16);
  if (wf32)
    pack_kernel<true><<<blocks, 256, 0, st>>>(W, N, K, ldw, s, qweight, scales, zeros, flags);
  else
    pack_kernel<false><<<blocks, 256, 0, st>>>(W, N, K, ldw, s, qweight, scales, zeros, flags);
  return hipGetLastError();
}

}  // namespace awq

// Applying the chosen scales ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §6): the inverse
// scaling is absorbed by the producer of X -- a LayerNorm's gamma and beta, an RMSNorm's
// gamma, or a preceding Linear's output rows and bias (row k divided by s_k) -- while every
// projection that reads X multiplies its input column k by s_k.  Where no parameter can
// absorb it (after a non-linearity), the runtime form is act(x) / s: the division follows the
// activation, never precedes it.
//
// Each parameter is the exact quotient or product rounded once to its storage type.  fp32:
// correctly rounded division and multiplication.  bf16: the fp32 result p is rounded to nearest
// even, except where p falls exactly halfway between two bf16 values while the exact result
// does not -- possible because s carries 24 significand bits, e.g. -2.171875 * 1.7446043 rounds
// in fp32 to the bf16 midpoint -3.7890625 -- there the exact residual (one FMA) tells which
// side the exact result lies on.
// Elementwise and bandwidth-bound: 16-byte vectors where a row allows, single elements
// otherwise.
#include "awq_internal.h"

namespace awq {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float ld_el(const void* p, int64_t i, bool bf16) {
  return bf16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(p)[i] << 16)
              : static_cast<const float*>(p)[i];
}
__device__ __forceinline__ uint16_t to_bf16(float x) {
  const bf16x2 h = __builtin_convertvector((f32x2){x, x}, bf16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, h) & 0xffffu;
}
// RN_bf16(p + err) for p = RN32(x) and err = x - p exact: RNE of p unless p is a bf16
// midpoint and err != 0, when the magnitude goes up iff x lies beyond p
__device__ __forceinline__ uint16_t to_bf16_exact(float p, float err) {
  const uint32_t b = __float_as_uint(p);
  if ((b & 0xffffu) == 0x8000u && err != 0.0f) {
    const bool up = (err > 0.0f) == (p > 0.0f);
    return (uint16_t)((b >> 16) + (up ? 1u : 0u));
  }
  return to_bf16(p);
}
__device__ __forceinline__ void st_el(void* p, int64_t i, float v, float err, bool bf16) {
  if (bf16)
    static_cast<uint16_t*>(p)[i] = to_bf16_exact(v, err);
  else
    static_cast<float*>(p)[i] = v;
}

// exact GELU 0.5 x (1 + erf(x / sqrt 2)) written as 0.5 x erfc(-x / sqrt 2): no cancellation
// for large negative x; SiLU x / (1 + exp(-x))
__device__ __forceinline__ float act_f(float x, int act) {
  if (act == kActGelu) return 0.5f * x * erfcf(-x * 0.70710678118654752f);
  return x / (1.0f + expf(-x));
}

// op 0: A[r, c] /= s[r]; op 1: A[r, c] *= s[c]; op 2: Y[r, c] = act(X[r, c]) / s[c].
// Unit u covers V = 16 / element-size consecutive elements of one row (the row's last unit
// may be short).  vec: every row start is 16-byte aligned, so full units load as vectors.
template <int OP, bool BF16>
__global__ __launch_bounds__(256) void scale_kernel(const void* X, void* Y,  // Y may be X
                                                    int64_t rows, int64_t cols, int64_t ld,
                                                    const float* __restrict__ s, int act, bool vec,
                                                    uint32_t* __restrict__ flags) {
  constexpr int V = BF16 ? 8 : 4;
  const int64_t upr = (cols + V - 1) / V;
  const int64_t units = rows * upr;
  bool bad = false;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = u / upr, c0 = (u - r * upr) * V;
    const int64_t base = r * ld + c0;
    float v[V], f[V], er[V];  // result and its exact residual (x - f; 0 for the activation)
    const bool full = vec && c0 + V <= cols;
    if (full) {
      const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const char*>(X) + base * (BF16 ? 2 : 4));
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int t = 0; t < V; ++t)
        v[t] = BF16 ? __uint_as_float(t & 1 ? w[t / 2] & 0xffff0000u : w[t / 2] << 16) : __uint_as_float(w[t]);
    } else {
#pragma unroll
      for (int t = 0; t < V; ++t) v[t] = c0 + t < cols ? ld_el(X, base + t, BF16) : 0.0f;
    }
    if (OP == 0) {
      const float sr = s[r];
      bad |= !(sr > 0.0f) || isinf(sr);
#pragma unroll
      for (int t = 0; t < V; ++t) {
        f[t] = v[t] / sr;                  // correctly rounded
        er[t] = fmaf(-f[t], sr, v[t]);     // v - f s, exact; same sign as v / s - f
      }
    } else {
#pragma unroll
      for (int t = 0; t < V; ++t) {
        const float sc = c0 + t < cols ? s[c0 + t] : 1.0f;
        bad |= !(sc > 0.0f) || isinf(sc);
        if (OP == 1) {
          f[t] = v[t] * sc;
          er[t] = fmaf(v[t], sc, -f[t]);  // v s - f, exact
        } else {
          f[t] = act_f(v[t], act) / sc;
          er[t] = 0.0f;
        }
      }
    }
    if (full) {
      uint32_t w[4];
      if (BF16) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          w[t] = (uint32_t)to_bf16_exact(f[2 * t], er[2 * t]) | ((uint32_t)to_bf16_exact(f[2 * t + 1], er[2 * t + 1]) << 16);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) w[t] = __float_as_uint(f[t]);
      }
      *reinterpret_cast<uint4*>(static_cast<char*>(Y) + base * (BF16 ? 2 : 4)) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
#pragma unroll
      for (int t = 0; t < V; ++t)
        if (c0 + t < cols) st_el(Y, base + t, f[t], er[t], BF16);
    }
  }
  if (bad) atomicOr(flags, kFlagScaleRange);
}

}  // namespace

hipError_t launch_scale_op(int op, const void* X, void* Y, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                           const float* s, int act, bool vec, uint32_t* flags, hipStream_t st) {
  const int V = bf16 ? 8 : 4;
  const int64_t units = rows * ((cols + V - 1) / V);
  int64_t blocks = (units + 255) / 256;
  if (blocks > 2048) blocks = 2048;  // grid-stride beyond eight 256-thread blocks per CU
#define AWQ_SCALE_LAUNCH(OPV, B) \
  scale_kernel<OPV, B><<<(unsigned)blocks, 256, 0, st>>>(X, Y, rows, cols, ld, s, act, vec, flags)
  if (op == 0) { if (bf16) AWQ_SCALE_LAUNCH(0, true); else AWQ_SCALE_LAUNCH(0, false); }
  else if (op == 1) { if (bf16) AWQ_SCALE_LAUNCH(1, true); else AWQ_SCALE_LAUNCH(1, false); }
  else { if (bf16) AWQ_SCALE_LAUNCH(2, true); else AWQ_SCALE_LAUNCH(2, false); }
#undef AWQ_SCALE_LAUNCH
  return hipGetLastError();
}

}  // namespace awq

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
// side the exact result lies on.  The runtime form act(x) / s is the fp32 activation times the
// correctly rounded 1 / s, within a few fp32 ulps of the exact value.
// Elementwise: the scalings are bandwidth-bound, the activation (erfc / exp per element) is
// ALU-bound.  16-byte vectors where a row allows, single elements otherwise.
#include "awq_internal.h"

namespace awq {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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
// Unit = V = 16 / element-size consecutive elements of one row (the row's last unit may be
// short).  Thread (blockIdx.x, t) keeps column unit 256 blockIdx.x + t, so its s values are
// loaded once; the grid's rows are interleaved, so that in iteration i the blocks of column
// y handle rows (i gridDim.y + blockIdx.y) U .. + U - 1 and the whole grid sweeps the matrix
// as one window of consecutive rows, U 16-byte loads in flight per thread.
// vec: every row start is 16-byte aligned, so full units load and store as vectors.
// U = 8 rows for the bandwidth-bound scalings, 4 for the activation, whose erfc / exp make
// it ALU-bound: there more resident waves hide the latency better than more loads in flight.

template <int V, bool BF16>
__device__ __forceinline__ void unpack_unit(const u32x4 q, float* v) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int t = 0; t < V; ++t)
    v[t] = BF16 ? __uint_as_float(t & 1 ? w[t / 2] & 0xffff0000u : w[t / 2] << 16) : __uint_as_float(w[t]);
}

template <int OP, bool BF16, int kScaleU>
__global__ __launch_bounds__(256) void scale_kernel(const void* X, void* Y,  // Y may be X
                                                    int64_t rows, int64_t cols, int64_t ld,
                                                    const float* __restrict__ s, int act, bool vec,
                                                    uint32_t* __restrict__ flags) {
  constexpr int V = BF16 ? 8 : 4;
  constexpr int64_t ES = BF16 ? 2 : 4;
  const int64_t upr = (cols + V - 1) / V;
  const int64_t cu = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (cu >= upr) return;
  const int64_t c0 = cu * V;
  const bool full = vec && c0 + V <= cols;
  bool bad = false;
  float sc[V];  // s (op 1) or 1 / s correctly rounded (op 2)
  if (OP != 0) {
#pragma unroll
    for (int t = 0; t < V; ++t) {
      sc[t] = c0 + t < cols ? s[c0 + t] : 1.0f;
      bad |= !(sc[t] > 0.0f) || isinf(sc[t]);
      if (OP == 2) sc[t] = 1.0f / sc[t];
    }
  }
  const int64_t rstep = (int64_t)gridDim.y * kScaleU;
  for (int64_t rb = (int64_t)blockIdx.y * kScaleU; rb < rows; rb += rstep) {
    float v[kScaleU][V];
    if (full) {
      u32x4 q[kScaleU];
#pragma unroll
      for (int u = 0; u < kScaleU; ++u)
        if (rb + u < rows)
          q[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
              static_cast<const char*>(X) + ((rb + u) * ld + c0) * ES));
#pragma unroll
      for (int u = 0; u < kScaleU; ++u)
        if (rb + u < rows) unpack_unit<V, BF16>(q[u], v[u]);
    } else {
#pragma unroll
      for (int u = 0; u < kScaleU; ++u)
#pragma unroll
        for (int t = 0; t < V; ++t)
          v[u][t] = rb + u < rows && c0 + t < cols ? ld_el(X, (rb + u) * ld + c0 + t, BF16) : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kScaleU; ++u) {
      const int64_t r = rb + u;
      if (r >= rows) break;
      float f[V], er[V];  // result and its exact residual (x - f; 0 for the activation)
      if (OP == 0) {
        const float sr = s[r];
        bad |= !(sr > 0.0f) || isinf(sr);
#pragma unroll
        for (int t = 0; t < V; ++t) {
          f[t] = v[u][t] / sr;                // correctly rounded
          er[t] = fmaf(-f[t], sr, v[u][t]);   // v - f s, exact; same sign as v / s - f
        }
      } else {
#pragma unroll
        for (int t = 0; t < V; ++t) {
          if (OP == 1) {
            f[t] = v[u][t] * sc[t];
            er[t] = fmaf(v[u][t], sc[t], -f[t]);  // v s - f, exact
          } else {
            f[t] = act_f(v[u][t], act) * sc[t];  // within 1.5 ulp of act / s
            er[t] = 0.0f;
          }
        }
      }
      const int64_t base = r * ld + c0;
      if (full) {
        uint32_t w[4];
        if (BF16) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            w[t] = (uint32_t)to_bf16_exact(f[2 * t], er[2 * t]) |
                   ((uint32_t)to_bf16_exact(f[2 * t + 1], er[2 * t + 1]) << 16);
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) w[t] = __float_as_uint(f[t]);
        }
        __builtin_nontemporal_store((u32x4){w[0], w[1], w[2], w[3]},
                                    reinterpret_cast<u32x4*>(static_cast<char*>(Y) + base * ES));
      } else {
#pragma unroll
        for (int t = 0; t < V; ++t)
          if (c0 + t < cols) st_el(Y, base + t, f[t], er[t], BF16);
      }
    }
  }
  if (bad) atomicOr(flags, kFlagScaleRange);
}

}  // namespace

hipError_t launch_scale_op(int op, const void* X, void* Y, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                           const float* s, int act, bool vec, uint32_t* flags, hipStream_t st) {
  const int V = bf16 ? 8 : 4;
  const int U = op == 2 ? 4 : 8;
  const int64_t upr = (cols + V - 1) / V;
  const int64_t gx = (upr + 255) / 256;
  const int64_t row_blocks = (rows + U - 1) / U;
  // blocks in all: two 4-wave blocks per CU for the scalings keep the window of rows short
  // while U loads per thread keep enough bytes in flight; eight for the activation
  const int64_t nb = op == 2 ? 2048 : 512;
  int64_t gy = nb / gx;
  if (gy < 1) gy = 1;
  if (gy > row_blocks) gy = row_blocks;
  if (gy > 65535) gy = 65535;
  if (gx > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)gx, (unsigned)gy);
#define AWQ_SCALE_LAUNCH(OPV, B, UV) \
  scale_kernel<OPV, B, UV><<<grid, 256, 0, st>>>(X, Y, rows, cols, ld, s, act, vec, flags)
  if (op == 0) { if (bf16) AWQ_SCALE_LAUNCH(0, true, 8); else AWQ_SCALE_LAUNCH(0, false, 8); }
  else if (op == 1) { if (bf16) AWQ_SCALE_LAUNCH(1, true, 8); else AWQ_SCALE_LAUNCH(1, false, 8); }
  else { if (bf16) AWQ_SCALE_LAUNCH(2, true, 4); else AWQ_SCALE_LAUNCH(2, false, 4); }
#undef AWQ_SCALE_LAUNCH
  return hipGetLastError();
}

}  // namespace awq

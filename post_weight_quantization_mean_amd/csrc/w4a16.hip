// Using the artefact ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §7 and §8): the W4A16
// product Y = X' W_hat^T of 16-bit activations X' [M, K] (which already carry S^-1, folded
// into their producer) with the packed weight W_hat[n, k] = scales[n, g] (q[n, k] - zeros[n, g])
// (fp16 scale, integer zero point, nibble i of word j = code of k = 8 j + i).  The weight is
// decoded on the fly and never written back.
//
// Two kinds of kernel:
//   * decode, M <= 8 tokens (more with fp32 X, eight per launch): bandwidth-bound on the 4.25
//     bits per weight (bf16 activations use the two-products-per-instruction variant below the
//     fp32 one, or with three or more tokens the matrix-core variant after it).  A wave streams
//     four weight rows at a time with 1 KiB-contiguous loads; every lane keeps 32 channels
//     (one quarter of a group) and their activations.  A nibble becomes a float through a byte
//     mask and v_cvt_f32_ubyte (1.4 instructions per code), and the group's scale is applied
//     once per 32 channels: sum_k x_k Delta (q_k - z) = Delta (sum_k x_k q_k - z sum_k x_k).
//     Products x q are exact in fp32; only the fp32 sums round.
//   * prefill, M > 8: the bf16 matrix cores.  A 128-row tile of W_hat is decoded per 32-channel
//     chunk into LDS as bf16 (Delta (q - z) rounded once to bf16), X' is staged as bf16, and
//     each of four waves accumulates 128 tokens x 128 outputs in fp32.
#include <atomic>
#include <type_traits>

#include "awq_internal.h"

namespace awq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
// byte c of x as a float (one v_cvt_f32_ubyte<c>)
template <int C>
__device__ __forceinline__ float ubyte(uint32_t x) { return (float)((x >> (8 * C)) & 0xffu); }

// ---- decode ------------------------------------------------------------------------------
constexpr int kGvRows = 4;       // weight rows per wave step (fp32 activations)
constexpr int kGvWordOuter = 2;  // bf16 decode: up to this many tokens, word-outer order
constexpr int kGvThreads = 256;

// K is covered in passes of kc channels (4096 for up to two tokens, else 2048): X of the pass
// is staged in LDS as fp32 [M][kc] (at most 64 KiB), then every wave streams its rows over
// the pass.  Lane l owns, per 1 KiB segment t of a row's words, words 4 (64 t + l) .. + 3,
// i.e. 32 channels, a quarter of one group.  The wave that owns row n adds each pass's sum
// into Y itself, so the result does not depend on scheduling.
template <int M, bool XF32>
__global__ __launch_bounds__(kGvThreads) void w4a16_gemv_kernel(
    const void* __restrict__ X, int64_t ldx, int64_t K, const int32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int64_t N,
    float* __restrict__ Y, int64_t ldy, int64_t kc) {
  extern __shared__ float xs[];  // [M][kc]
  const int64_t G = K / kGroup;
  const int64_t words = K / 8;
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kGvThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kGvThreads) >> 6;
  for (int64_t c0 = 0; c0 < K; c0 += kc) {
    const int64_t kw = K - c0 < kc ? K - c0 : kc;  // channels in this pass (a multiple of 128)
    __syncthreads();  // the previous pass is done with xs
    {  // 16-byte pieces (8 bf16 or 4 fp32 values), four in flight per thread
      constexpr int PE = XF32 ? 4 : 8;
      const int64_t pieces = (int64_t)M * kw / PE;
      for (int64_t i0 = threadIdx.x; i0 < pieces; i0 += 4 * kGvThreads) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t i = i0 + u * kGvThreads;
          if (i < pieces) {
            const int64_t m = (i * PE) / kw, k = i * PE - m * kw;
            v[u] = *reinterpret_cast<const uint4*>(static_cast<const char*>(X) + (m * ldx + c0 + k) * (XF32 ? 4 : 2));
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t i = i0 + u * kGvThreads;
          if (i < pieces) {
            const int64_t m = (i * PE) / kw, k = i * PE - m * kw;
            float* dst = xs + m * kc + k;
            if constexpr (XF32) {
              *reinterpret_cast<uint4*>(dst) = v[u];
            } else {
              const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
              *reinterpret_cast<float4*>(dst) = make_float4(__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                                                            __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u));
              *reinterpret_cast<float4*>(dst + 4) = make_float4(__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xffff0000u),
                                                                __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xffff0000u));
            }
          }
        }
      }
    }
    __syncthreads();
    const int64_t pw = kw / 8;                 // words of a row in this pass
    const int64_t segs = (pw + 255) / 256;
    // the weight words, scales and zero points of one row group and segment, loaded one step
    // ahead of their use so that the next loads are in flight during the current math
    struct Slab {
      u32x4 q[kGvRows];
      uint16_t d[kGvRows], z[kGvRows];  // fp16 bits: converted where used, so that nothing
                                        // waits for the prefetch before the current math
    };
    auto fetch = [&](int64_t n0, int64_t t, Slab& S) {
      const int64_t lw = 4 * (64 * t + lane);
      const int64_t w0 = c0 / 8 + (lw < pw ? lw : 0);
      const int64_t g = (8 * w0) / kGroup;
#pragma unroll
      for (int r = 0; r < kGvRows; ++r) {
        const int64_t n = n0 + r < N ? n0 + r : N - 1;  // rows past N: load row N-1, store nothing
        S.q[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qweight + n * words + w0));
        S.d[r] = scales[n * G + g];
        S.z[r] = zeros[n * G + g];
      }
    };
    const int64_t step = nwaves * kGvRows;
    Slab cur, nxt;
    int64_t n0 = wave * kGvRows, t = 0;
    if (n0 < N) fetch(n0, 0, cur);
    while (n0 < N) {
      float acc[kGvRows][M];
#pragma unroll
      for (int r = 0; r < kGvRows; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
      for (t = 0; t < segs; ++t) {
        // next (row group, segment) in this wave's order
        const bool last_seg = t + 1 == segs;
        const int64_t nn = last_seg ? n0 + step : n0, tn = last_seg ? 0 : t + 1;
        fetch(nn < N ? nn : n0, tn, nxt);  // past the last row group: a harmless reload
        const int64_t lw = 4 * (64 * t + lane);  // first word of this lane within the pass
        if (lw < pw) {
          const int64_t k0 = 8 * lw;
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const float* xr = xs + (int64_t)m * kc + k0;
            float sx = 0.0f, sq[kGvRows];
#pragma unroll
            for (int r = 0; r < kGvRows; ++r) sq[r] = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {  // word j: codes 8 j .. 8 j + 7
              const float4 xa = *reinterpret_cast<const float4*>(xr + 8 * j);
              const float4 xb = *reinterpret_cast<const float4*>(xr + 8 * j + 4);
              const float x8[8] = {xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
#pragma unroll
              for (int c = 0; c < 8; ++c) sx += x8[c];
#pragma unroll
              for (int r = 0; r < kGvRows; ++r) {
                const uint32_t w = j == 0 ? cur.q[r].x : j == 1 ? cur.q[r].y : j == 2 ? cur.q[r].z : cur.q[r].w;
                const uint32_t ev = w & 0x0f0f0f0fu, od = (w >> 4) & 0x0f0f0f0fu;  // codes 0,2,4,6 / 1,3,5,7
                sq[r] = fmaf(x8[0], ubyte<0>(ev), sq[r]);
                sq[r] = fmaf(x8[1], ubyte<0>(od), sq[r]);
                sq[r] = fmaf(x8[2], ubyte<1>(ev), sq[r]);
                sq[r] = fmaf(x8[3], ubyte<1>(od), sq[r]);
                sq[r] = fmaf(x8[4], ubyte<2>(ev), sq[r]);
                sq[r] = fmaf(x8[5], ubyte<2>(od), sq[r]);
                sq[r] = fmaf(x8[6], ubyte<3>(ev), sq[r]);
                sq[r] = fmaf(x8[7], ubyte<3>(od), sq[r]);
              }
            }
            // Delta (sum x q - z sum x) for this quarter group
#pragma unroll
            for (int r = 0; r < kGvRows; ++r)
              acc[r][m] = fmaf(h2f(cur.d[r]), fmaf(-h2f(cur.z[r]), sx, sq[r]), acc[r][m]);
          }
        }
        cur = nxt;
      }
      // sum over the wave's lanes, one row and token at a time
#pragma unroll
      for (int r = 0; r < kGvRows; ++r)
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const float v = wave_sum(acc[r][m]);
          if (lane == 0 && n0 + r < N) {
            float* y = Y + (int64_t)m * ldy + n0 + r;
            *y = c0 == 0 ? v : *y + v;
          }
        }
      n0 += step;
    }
  }
}

// bf16 activations: the same layout with two products per instruction.  A word's eight codes
// become four bf16 pairs (q_i, q_{i+4}) biased to 128 + q (bf16 with exponent 2^7 holds the
// integers 128..255 exactly: bits 0x4300 | q), and v_dot2_f32_bf16 multiplies them with the
// activation pairs (x_i, x_{i+4}), staged in LDS in that order.  The bias comes off once per
// quarter group: sum x q - z sum x = sum x (128 + q) - (128 + z) sum x.  Products are exact;
// the sums carry the bias, so their rounding is relative to sum |x| (128 + q), about 2^7 times
// the unbiased sum's (still far below the bf16 precision of the activations).
// R weight rows per wave step: 2 for one or two tokens, 4 for more (see the launch).
template <int M, int R>
__global__ __launch_bounds__(kGvThreads) void w4a16_gemv_dot_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, int64_t K, const int32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int64_t N,
    float* __restrict__ Y, int64_t ldy, int64_t kc) {
  // LDS: [M][kc / 2] bf16 pairs, (x_i, x_{i+4}) per 8 channels, then [M][kc / 8] fp32 sums of
  // each 8 channels (the bias correction needs sum x per 32 channels, the same for every row)
  extern __shared__ __attribute__((aligned(16))) uint32_t xp[];
  float* xsum = reinterpret_cast<float*>(xp + (int64_t)M * (kc / 2));
  // 16-byte views for the reads (one ds_read_b128 each)
  const u32x4* xq = reinterpret_cast<const u32x4*>(xp);
  const f32x4* xs4 = reinterpret_cast<const f32x4*>(xsum);
  typedef __bf16 bfx2 __attribute__((ext_vector_type(2)));
  const int64_t G = K / kGroup;
  const int64_t words = K / 8;
  const int lane = threadIdx.x & 63;
  // wave-uniform row bookkeeping lives in scalar registers, so row addresses cost no VALU
  const int64_t wave = __builtin_amdgcn_readfirstlane((int)((blockIdx.x * kGvThreads + threadIdx.x) >> 6));
  const int64_t nwaves = ((int64_t)gridDim.x * kGvThreads) >> 6;
  const int64_t step = nwaves * R;
  auto dot = [](uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bfx2, a), __builtin_bit_cast(bfx2, b), c, false);
  };
  // the bias 0x43004300 as an opaque vector register: (x & mask) | bias is then one v_and_or_b32
  // (a VOP3 instruction takes no literal operand here, and at most one scalar one)
  uint32_t bias;
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(bias));
  // An item's rows use 16 groups of the pass (a segment of 256 words is 2048 channels), so its
  // scales and zeros are 32 R fp16 values: lane v of load h holds value 64 h + v, i.e. array
  // (scale, zero) (64 h + v) / (16 R), row ((64 h + v) / 16) % R, group 16 t + v % 16.  One
  // 2-byte load per lane per 64 values, against one per lane, row and array when every lane
  // loaded its own group's (the values each lane needs are taken from their holder with
  // ds_bpermute when the item is processed).
  constexpr int NDZ = (R + 1) / 2;
  struct Slab {
    u32x4 q[R];
    uint32_t dz[NDZ];  // fp16 bits, converted where used, so that nothing waits for the
                       // prefetch before the current math
  };
  // this wave's row groups n0 = R wave + i step (i < nrg), each in segs segments per pass: the
  // items (row group, segment) in that order, three slabs in a ring, two items in flight
  const int64_t first = wave * R;
  const int64_t nrg = first < N ? (N - 1 - first) / step + 1 : 0;
  for (int64_t c0 = 0; c0 < K; c0 += kc) {
    const int64_t kw = K - c0 < kc ? K - c0 : kc;  // a multiple of 128
    const int64_t pw = kw / 8;                      // words of a row in this pass
    const int64_t segs = (pw + 255) / 256;
    const int64_t T = nrg * segs;
    // cursor of the next item to fetch; rows past N load row N - 1 (in bounds, never stored)
    int64_t fn0 = first, ft = 0;
    auto fetch = [&](Slab& S) {
      const int lw = 4 * (64 * (int)ft + lane);
      const int w0 = lw < pw ? lw : 0;  // word within the pass
#pragma unroll
      for (int h = 0; h < NDZ; ++h) {
        const int v = 64 * h + lane;
        const int r = (v >> 4) % R;
        const int64_t n = fn0 + r < N ? fn0 + r : N - 1;
        const int gv = 16 * (int)ft + (v & 15);  // group within the pass; past its end: its last
        const int64_t gi = c0 / kGroup + (gv < pw / 16 ? gv : pw / 16 - 1);
        S.dz[h] = (v < 16 * R ? scales : zeros)[n * G + gi];
      }
      // the codes last: processing the item then waits for its newest loads, the codes, and
      // finds the scales and zeros landed (issued after the codes, they held up every item;
      // one token, back to back over eight 28672 x 4096 artefacts: 14.5 against 15.0 us)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t n = fn0 + r < N ? fn0 + r : N - 1;
        const int32_t* rowp = qweight + n * words + c0 / 8;
        S.q[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowp + w0));
      }
      if (++ft == segs) { ft = 0; fn0 += step; }
    };
    Slab sa, sb, sc;
    if (T > 0) {  // the first two items are in flight while X is staged
      fetch(sa);
      fetch(sb);
    }
    __syncthreads();  // the previous pass is done with xp
    {  // 8 channels (16 bytes) per piece, four pieces in flight per thread
      const int pieces = (int)(M * kw / 8);
      const int ppr = (int)(kw / 8);  // pieces per token row
      for (int i0 = threadIdx.x; i0 < pieces; i0 += 4 * kGvThreads) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * kGvThreads;
          if (i < pieces) {
            const int m = i / ppr, k = 8 * (i - m * ppr);
            v[u] = *reinterpret_cast<const uint4*>(X + m * ldx + c0 + k);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u * kGvThreads;
          if (i < pieces) {
            const int m = i / ppr, k = 8 * (i - m * ppr);
            // (x0,x1) (x2,x3) (x4,x5) (x6,x7) -> (x0,x4) (x1,x5) (x2,x6) (x3,x7)
            const uint32_t a = v[u].x, b = v[u].y, c = v[u].z, d = v[u].w;
            const uint4 pr = make_uint4((a & 0xffffu) | (c << 16), (a >> 16) | (c & 0xffff0000u),
                                        (b & 0xffffu) | (d << 16), (b >> 16) | (d & 0xffff0000u));
            *reinterpret_cast<uint4*>(xp + (int64_t)m * (kc / 2) + k / 2) = pr;
            float s8 = 0.0f;
            s8 = dot(pr.x, 0x3f803f80u, s8);  // (1, 1) in bf16: exact products
            s8 = dot(pr.y, 0x3f803f80u, s8);
            s8 = dot(pr.z, 0x3f803f80u, s8);
            s8 = dot(pr.w, 0x3f803f80u, s8);
            xsum[(int64_t)m * (kc / 8) + k / 8] = s8;
          }
        }
      }
    }
    __syncthreads();
    float acc[R][M];
    int64_t pn0 = first, pt = 0;  // cursor of the next item to process
    auto process = [&](const Slab& S) {
      if (pt == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int m = 0; m < M; ++m) acc[r][m] = 0.0f;
      }
      const int lw = 4 * (64 * (int)pt + lane);
      // this lane's group (16 pt + lane / 4) of each row: its scale and zero from their holders
      // (with every lane active: a holder may be past the end of a partial segment)
      float dv[R], zv[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int vd = 16 * r + (lane >> 2), vz = 16 * R + vd;
        dv[r] = h2f((uint16_t)__builtin_amdgcn_ds_bpermute(4 * (vd & 63), (int)S.dz[vd >> 6]));
        zv[r] = h2f((uint16_t)__builtin_amdgcn_ds_bpermute(4 * (vz & 63), (int)S.dz[vz >> 6]));
      }
      if (lw < pw) {
        // codes as biased bf16 pairs (q_i, q_{i+4}) + 128, i = 0..3, of word j of row r
        auto pairs = [&](int r, int j, uint32_t* qp) {
          const uint32_t w = j == 0 ? S.q[r].x : j == 1 ? S.q[r].y : j == 2 ? S.q[r].z : S.q[r].w;
          qp[0] = (w & 0x000f000fu) | bias;
          qp[1] = ((w >> 4) & 0x000f000fu) | bias;
          qp[2] = ((w >> 8) & 0x000f000fu) | bias;
          qp[3] = ((w >> 12) & 0x000f000fu) | bias;
        };
        auto finish = [&](int m, const float* sq) {
          const f32x4 s4 = xs4[(m * (kc / 8) + lw) / 4];
          const float sxm = (s4.x + s4.y) + (s4.z + s4.w);  // sum of the lane's 32 activations
#pragma unroll
          for (int r = 0; r < R; ++r) acc[r][m] = fmaf(dv[r], fmaf(-(128.0f + zv[r]), sxm, sq[r]), acc[r][m]);
        };
        if constexpr (M <= kGvWordOuter) {
          // few tokens: word by word, so that only one word's pairs are live
          float sq[M][R];
#pragma unroll
          for (int m = 0; m < M; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r) sq[m][r] = 0.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t qp[R][4];
#pragma unroll
            for (int r = 0; r < R; ++r) pairs(r, j, qp[r]);
#pragma unroll
            for (int m = 0; m < M; ++m) {
              const u32x4 x4 = xq[m * (kc / 8) + lw + j];
#pragma unroll
              for (int r = 0; r < R; ++r) {
                sq[m][r] = dot(x4.x, qp[r][0], sq[m][r]);
                sq[m][r] = dot(x4.y, qp[r][1], sq[m][r]);
                sq[m][r] = dot(x4.z, qp[r][2], sq[m][r]);
                sq[m][r] = dot(x4.w, qp[r][3], sq[m][r]);
              }
            }
          }
#pragma unroll
          for (int m = 0; m < M; ++m) finish(m, sq[m]);
        } else {
          // more tokens: all pairs once, then token by token
          uint32_t qp[R][4][4];
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) pairs(r, j, qp[r][j]);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            float sq[R];
#pragma unroll
            for (int r = 0; r < R; ++r) sq[r] = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const u32x4 x4 = xq[m * (kc / 8) + lw + j];
#pragma unroll
              for (int r = 0; r < R; ++r) {
                sq[r] = dot(x4.x, qp[r][j][0], sq[r]);
                sq[r] = dot(x4.y, qp[r][j][1], sq[r]);
                sq[r] = dot(x4.z, qp[r][j][2], sq[r]);
                sq[r] = dot(x4.w, qp[r][j][3], sq[r]);
              }
            }
            finish(m, sq);
          }
        }
      }
      if (pt + 1 == segs) {  // row group done: sum over the wave's lanes, one row and token at a time
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int m = 0; m < M; ++m) {
            const float v = wave_sum(acc[r][m]);
            if (lane == 0 && pn0 + r < N) {
              float* y = Y + (int64_t)m * ldy + pn0 + r;
              *y = c0 == 0 ? v : *y + v;
            }
          }
        pt = 0;
        pn0 += step;
      } else {
        ++pt;
      }
    };
    for (int64_t it = 0; it < T; it += 3) {  // static slab roles: item it in sa, it+1 in sb, it+2 in sc
      fetch(sc);
      process(sa);
      if (it + 1 < T) {
        fetch(sa);
        process(sb);
      }
      if (it + 2 < T) {
        fetch(sb);
        process(sc);
      }
    }
  }
}

// bf16 activations on the matrix cores: v_mfma_f32_16x16x32_bf16 with the tokens as its 16
// rows (M of them real; the rest repeat a staged token and are never stored) and 16 weight rows
// as its 16 columns.  Lane l supplies the A operand of token l % 16 and the B operand of weight
// row n0 + l % 16, both for its k-chunk c = l / 16: in MFMA j of a group, chunk c stands for
// word 4 c + j of the group (a fixed permutation of the sum over k, the same on both operands),
// so a lane's four words of a group are 16 contiguous bytes of the row.  Each word becomes four
// biased bf16 pairs (q_i, q_{i+4}) + 128, as in the dot kernel, against activation pairs
// (x_i, x_{i+4}) staged in LDS; the MFMA sums the group's 128 exact products in fp32, and the
// group's scale and zero come off once per group: Delta (sum x (128 + q) - (128 + z) sum x),
// with sum x per (token, group) staged beside the pairs.  The VALU work per code (the pair
// building, about 0.9 instructions, and the epilogue) no longer grows with the tokens, where the
// dot kernel spends one instruction per two products.  A wave owns 16 whole rows (all of K), so
// it writes its outputs itself; the codes of the next round of 8 groups are in flight while a
// round is multiplied.
constexpr int kMfDepth = 4;     // group pairs per round (8 groups)
constexpr int kMfPerCu = 4;     // blocks per CU of the matrix-core decode (2 measured the same)
constexpr int kMfMinTokens = 2;  // fewer tokens: the dot kernel (faster at one token)

__device__ __forceinline__ int mf_pitch(int64_t kc) { return (int)(kc / 2) + 4; }  // uint32 per token row (padded: no bank conflict across tokens)

__global__ __launch_bounds__(kGvThreads) void w4a16_gemv_mfma_kernel(
    const uint16_t* __restrict__ X, int64_t ldx, int M, int64_t K, const int32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int64_t N,
    float* __restrict__ Y, int64_t ldy, int64_t kc) {
  // LDS: [M][kc / 2 + 4] activation pairs, then [kc / 128][16] fp32 group sums (16 token slots),
  // then each wave's round of codes [16 rows][128 words]
  extern __shared__ __attribute__((aligned(16))) uint32_t xp[];
  const int pitch = mf_pitch(kc);
  float* gsum = reinterpret_cast<float*>(xp + (int64_t)M * pitch);
  uint32_t* wcodes = xp + (int64_t)M * pitch + (kc / kGroup) * 16 + (threadIdx.x >> 6) * (16 * 128);
  const int64_t G = K / kGroup, words = K / 8;
  const int lane = threadIdx.x & 63, tk = lane & 15, ch = lane >> 4;
  const int64_t wave = __builtin_amdgcn_readfirstlane((int)((blockIdx.x * kGvThreads + threadIdx.x) >> 6));
  const int64_t nwaves = ((int64_t)gridDim.x * kGvThreads) >> 6;
  const int64_t tiles = (N + 15) / 16;
  uint32_t bias;
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(bias));
  for (int64_t c0 = 0; c0 < K; c0 += kc) {
    const int64_t kw = K - c0 < kc ? K - c0 : kc;  // a multiple of 128
    const int gpp = (int)(kw / kGroup);             // groups in this pass
    __syncthreads();  // the previous pass is done with the LDS
    // activation pairs and group sums: one thread per (token, group), its 16 pieces of 8 channels
    // loaded at once; the sum over the group's 128 channels in a fixed order (fp32).  Group sums
    // of token slots M..15 stay unset: only product rows that are never stored read them.
    for (int i = threadIdx.x; i < M * gpp; i += kGvThreads) {
      const int m = i / gpp, gg = i - m * gpp;
      const uint16_t* src = X + m * ldx + c0 + gg * kGroup;
      uint4 v[16];
#pragma unroll
      for (int w = 0; w < 16; ++w) v[w] = *reinterpret_cast<const uint4*>(src + 8 * w);
      uint32_t* dst = xp + (int64_t)m * pitch + gg * 64;
      float sx = 0.0f;
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        const uint32_t a = v[w].x, b = v[w].y, c = v[w].z, d = v[w].w;
        *reinterpret_cast<uint4*>(dst + 4 * w) = make_uint4((a & 0xffffu) | (c << 16), (a >> 16) | (c & 0xffff0000u),
                                                            (b & 0xffffu) | (d << 16), (b >> 16) | (d & 0xffff0000u));
        float s8 = 0.0f;
        const uint32_t e[4] = {a, b, c, d};
#pragma unroll
        for (int q = 0; q < 4; ++q) s8 += __uint_as_float(e[q] << 16) + __uint_as_float(e[q] & 0xffff0000u);
        sx += s8;
      }
      gsum[gg * 16 + m] = sx;
    }
    __syncthreads();
    // this lane's A rows: token tk, or for tk >= M any staged token (rows M.. of the product are
    // never stored, and each row of the product depends only on its own row of A)
    const uint32_t* xa = xp + (int64_t)(tk < M ? tk : M - 1) * pitch + 16 * ch;
    for (int64_t tile = wave; tile < tiles; tile += nwaves) {
      const int64_t n = 16 * tile + tk;                 // this lane's weight row
      const int64_t nl = n < N ? n : N - 1;             // rows past N: load row N - 1, store nothing
      const uint16_t* drow = scales + nl * G + c0 / kGroup;
      const uint16_t* zrow = zeros + nl * G + c0 / kGroup;
      // Rounds of 8 groups: the tile's 16 rows x 512 bytes of codes.  The wave loads a round as
      // eight instructions of two rows each, whole 128-byte lines (lane l: row 2 i + l / 32,
      // 16-byte piece l % 32), and passes it through its own 8 KiB of LDS into the product's
      // layout (lane: row tk, piece 4 g + ch of the round's group g); the row's fp16 scales and
      // zeros of a round are one 16-byte load each.  Loading each lane's pieces directly touched
      // twice the lines per instruction and took the kernel from 14.6 to 18.8 us (one token).
      // Pieces are stored at piece ^ (row % 16), which keeps both the stores (8 lanes, one row)
      // and the reads (16 lanes, 16 rows) free of bank conflicts.  The codes of the next round
      // and its scales and zeros are in flight while a round is multiplied.  Tiles start at
      // different rounds (rot), so that waves do not all read the same bytes of rows 2 KiB apart
      // at once; the sum over groups is then taken in a rotated order, fixed per tile.
      const int rounds = gpp / (2 * kMfDepth);  // the pass width is a multiple of 1024 channels
      const int rot = (int)((tile * 5) % rounds);
      auto round_of = [&](int r) { return r + rot < rounds ? r + rot : r + rot - rounds; };
      u32x4 cq[2 * kMfDepth];
      u32x4 sdc, szc, sdn, szn;  // this and the next round's 8 scales and zeros (fp16 bits)
      const int lrow = lane >> 5, lpc = lane & 31;  // load layout: row 2 i + lrow, piece lpc
      // round r into cq (r clamped: a harmless reload); the scheduling barrier keeps rounds'
      // loads in issue order, so that the wait before a round's stores is for that round only
      auto fetch = [&](int r, u32x4* sd, u32x4* sz) {
        const int g0 = 2 * kMfDepth * round_of(r < rounds ? r : rounds - 1);
#pragma unroll
        for (int ii = 0; ii < 2 * kMfDepth; ++ii) {
          const int64_t rr = 16 * tile + 2 * ii + lrow;
          const int64_t rl = rr < N ? rr : N - 1;
          cq[ii] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(qweight + rl * words + c0 / 8 + 16 * g0 + 4 * lpc));
        }
        *sd = *reinterpret_cast<const u32x4*>(drow + g0);
        *sz = *reinterpret_cast<const u32x4*>(zrow + g0);
        __builtin_amdgcn_sched_barrier(0);
      };
      auto stash = [&] {  // cq -> this wave's LDS round, swizzled
#pragma unroll
        for (int ii = 0; ii < 2 * kMfDepth; ++ii) {
          const int row = 2 * ii + lrow;
          *reinterpret_cast<u32x4*>(wcodes + row * 128 + 4 * (lpc ^ (row & 15))) = cq[ii];
        }
      };
      float y[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      // groups gg and gg + 1 (codes w0, w1; fp16 scale and zero bits in the low / high halves of
      // dw, zw): two independent chains of four products, interleaved
      auto consume2 = [&](int gr, uint32_t dw, uint32_t zw, int gg) {  // round groups gr, gr + 1
        const u32x4 w0 = *reinterpret_cast<const u32x4*>(wcodes + tk * 128 + 4 * ((4 * gr + ch) ^ tk));
        const u32x4 w1 = *reinterpret_cast<const u32x4*>(wcodes + tk * 128 + 4 * ((4 * gr + 4 + ch) ^ tk));
        f32x4 acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
        const uint32_t wj[2][4] = {{w0.x, w0.y, w0.z, w0.w}, {w1.x, w1.y, w1.z, w1.w}};
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t w = wj[h][j];
            const u32x4 bq = {(w & 0x000f000fu) | bias, ((w >> 4) & 0x000f000fu) | bias,
                              ((w >> 8) & 0x000f000fu) | bias, ((w >> 12) & 0x000f000fu) | bias};
            const u32x4 aq = *reinterpret_cast<const u32x4*>(xa + (gg + h) * 64 + 4 * j);
            acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, aq),
                                                             __builtin_bit_cast(bf16x8, bq), acc[h], 0, 0, 0);
          }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float dv = h2f((uint16_t)(h ? dw >> 16 : dw & 0xffffu));
          const float zb = 128.0f + h2f((uint16_t)(h ? zw >> 16 : zw & 0xffffu));
          const f32x4 sg = *reinterpret_cast<const f32x4*>(gsum + (gg + h) * 16 + 4 * ch);  // tokens 4 ch ..
          y[0] = fmaf(dv, fmaf(-zb, sg.x, acc[h][0]), y[0]);
          y[1] = fmaf(dv, fmaf(-zb, sg.y, acc[h][1]), y[1]);
          y[2] = fmaf(dv, fmaf(-zb, sg.z, acc[h][2]), y[2]);
          y[3] = fmaf(dv, fmaf(-zb, sg.w, acc[h][3]), y[3]);
        }
      };
      fetch(0, &sdc, &szc);
      for (int r = 0; r < rounds; ++r) {
        const int g0 = 2 * kMfDepth * round_of(r);
        stash();  // round r's codes into LDS (this wave only; a wave's LDS accesses keep their order)
        const uint32_t dw[4] = {sdc.x, sdc.y, sdc.z, sdc.w}, zw[4] = {szc.x, szc.y, szc.z, szc.w};
        fetch(r + 1, &sdn, &szn);
#pragma unroll
        for (int sl = 0; sl < kMfDepth; ++sl) consume2(2 * sl, dw[sl], zw[sl], g0 + 2 * sl);  // groups g0 + 2 sl, + 1
        sdc = sdn;
        szc = szn;
      }
      // lane l holds row n (column l % 16 of the product), tokens 4 ch + i
      if (n < N) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 4 * ch + i;
          if (m < M) {
            float* yp = Y + (int64_t)m * ldy + n;
            *yp = c0 == 0 ? y[i] : *yp + y[i];
          }
        }
      }
    }
  }
}

// ---- prefill (bf16 X, more than 8 tokens) ----------------------------------------------------
#define AWQ_LDS __attribute__((address_space(3)))
constexpr int PBM = 512, PBN = 128, PKC = 32;

__device__ __forceinline__ uint32_t bf16x2_of(float a, float b) {
  const bf16x2 h = __builtin_convertvector((f32x2){a, b}, bf16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

// The tile (512 tokens x 128 outputs, four waves of 128 x 128 outputs, one per SIMD, 256 fp32
// accumulators a lane) and the pipeline of the candidate search's fused kernel, with the int4
// decode where the search quantizes.  Step c multiplies chunk c (32 channels: 32
// v_mfma_f32_32x32x16_bf16 per wave, back to back) and issues between them:
//   * the decode of chunk c+2 into W stage (c+2) % 3: wave w decodes W rows 32w .. 32w+31, lane l
//     rows 32w + l/4 and 32w + 16 + l/4, channels 8 (l%4) .. +7, i.e. one code word per row,
//     loaded four or five steps earlier; Delta (q - z) = fma(q, Delta, -z Delta) is exact in fp32
//     (q, z <= 15, Delta fp16) and is rounded once to bf16, the bf16 W~ of the other kernels;
//   * the fragment reads of chunk c's second K-half and of chunk c+1's B fragments and first two
//     A fragments;
//   * even steps: the code words of chunks c+4 and c+5 (one 4-byte load per row each) and, at a
//     group's first chunk, the next group's fp16 scales and zeros of the lane's two rows; every
//     step: half of the X pair that follows, copied from global memory straight into LDS.
// X lives in two pair stages (chunks 2p, 2p+1: a full 128-byte line of a row), each split into
// the first and the last 64 of every wave's rows (distinct LDS objects with a static role in
// each unrolled step, so the compiler's waits for the copies stay exact).  Each wave copies and
// reads only its own 128 X rows; the decoded W is shared, and one barrier per step, after every
// wave stored its part of chunk c+2, makes chunk c+1 readable.  Slots are permuted per row (X
// pair rows by (row >> 1) & 7, W rows by (row >> 2) & 3) so that the 32-row fragment reads are
// free of bank conflicts.  Rows past M or N read as zero through the buffer resources (a zero
// scale decodes to zero weights) and their outputs are not stored.
// XF: X is read instead from a copy in matrix-core operand order (xfrag_kernel of the search:
// the 16 bytes that lane l of an A operand takes for rows 32 rb.. and channels 16 kb.. are
// contiguous, 1 KiB per fragment), each A fragment with one load straight into registers, right
// after the last product of chunk c that reads its registers for chunk c+1; X then needs no LDS
// and no copies, as in the persistent search kernel.
constexpr int QXROW = 128;            // bytes of an X pair row (two chunks)
constexpr int QXPSTAGE = PBM * QXROW;  // 64 KiB
constexpr int QEROW = PKC * 2;        // bytes of a decoded W row of one chunk
constexpr int QESTAGE = PBN * QEROW;  // 8 KiB
constexpr int QNES = 3;               // W stages

__device__ __forceinline__ int qswz(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int qxswz(int row) { return (row >> 1) & 7; }

struct CodeSet {
  uint32_t w[2];  // this lane's code word of its rows r0 and r1 for one chunk
};
struct ScaleZero {
  uint32_t d0, d1, z0, z1;  // fp16 bits of the rows' scales and zeros for one group
};
struct RowDq {
  float d, nzd;  // Delta and -z Delta of one row's group
};

// X: row-major X [M, ldx] (XF false) or the operand-order copy (XF true, ldx ignored, rows
// padded to a multiple of 32 with zeros).
template <bool XF>
__global__ __launch_bounds__(256, 1) void w4a16_gemm_pipe_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t ldx, int64_t K, const int32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int64_t N,
    float* __restrict__ Y, int64_t ldy, int64_t ntiles, int64_t tiles, int64_t per_xcd) {
  constexpr int XST = XF ? 16 : QXPSTAGE / 2;  // the X stages are unused with the copy
  __shared__ __attribute__((aligned(1024))) uint8_t xp0lo[XST];
  __shared__ __attribute__((aligned(1024))) uint8_t xp0hi[XST];
  __shared__ __attribute__((aligned(1024))) uint8_t xp1lo[XST];
  __shared__ __attribute__((aligned(1024))) uint8_t xp1hi[XST];
  __shared__ __attribute__((aligned(1024))) uint8_t es[QNES * QESTAGE];
  // XCD x (= block % 8) takes the tiles x per_xcd .. (x + 1) per_xcd - 1 in order (token-tile
  // major), so its resident blocks share token tiles in its L2
  const int64_t L = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (L >= tiles) return;
  const int64_t m0 = (L / ntiles) * PBM, n0 = (L % ntiles) * PBN;
  const int64_t G = K / kGroup, words = K / 8;
  const int nchunks = (int)(K / PKC);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // buffer resources rebased at the tile: rows past M (or N) read as zero; offsets stay below
  // 2^31 (host: 512 rows of X; 128 rows of codes, scales or zeros are far smaller)
  auto rsrc = [](const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff), 0x00020000);
  };
  // the copy: rows m0.. are 64 K bytes per block of 32 rows; blocks past round_up(M, 32) read as
  // zero (512 rows of the copy span less than 2^31 bytes: host-checked for X)
  const int64_t Mp = (M + 31) / 32 * 32;
  const __amdgpu_buffer_rsrc_t xrsrc =
      XF ? rsrc(X + m0 * K, (Mp - m0) * K * 2) : rsrc(X + m0 * ldx, (M - m0) * ldx * 2);
  const __amdgpu_buffer_rsrc_t crsrc = rsrc(qweight + n0 * words, (N - n0) * words * 4);
  const __amdgpu_buffer_rsrc_t srsrc = rsrc(scales + n0 * G, (N - n0) * G * 2);
  const __amdgpu_buffer_rsrc_t zrsrc = rsrc(zeros + n0 * G, (N - n0) * G * 2);
  // X copy instruction i (0..15) of wave w fills pair rows 128 w + 8 i + lane / 8, slot lane % 8,
  // with the global 16-byte piece slot ^ qxswz(row); qxswz depends on i only through i % 2
  uint32_t xoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = wave * 128 + 8 * i + (lane >> 3);
    xoff[i] = (uint32_t)(row * ldx * 2 + (((lane & 7) ^ qxswz(row)) * 16));
  }
  const uint32_t xrow16 = (uint32_t)(16 * ldx * 2);
  const int xwave = wave * 64 * QXROW;  // this wave's 64 rows in a half stage
  auto dma_x_one = [&](uint8_t* xh, int i, int p) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xrsrc, (AWQ_LDS void*)(xh + xwave + (i & 7) * 1024), 16,
                                             (int)xoff[i & 1], (int)((uint32_t)(i >> 1) * xrow16 + (uint32_t)p * QXROW),
                                             0, 0);
  };
  // A fragment (row block r of this wave's 128 rows, chunk ch, K-half h) of the copy
  const uint32_t avoff = (uint32_t)(lane * 16) + (uint32_t)(wave * 4) * (uint32_t)(K * 64);
  auto load_a = [&](int ch, int h, int r) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                          xrsrc, (int)avoff, (int)(r * K * 64 + (2 * ch + h) * 1024), 0));
  };
  // decode: rows r0, r1 of the W tile, code word q4 of each chunk (channels 8 q4 .. 8 q4 + 7)
  const int q4 = lane & 3;
  const int r0 = wave * 32 + (lane >> 2), r1 = r0 + 16;
  const uint32_t coff0 = (uint32_t)(r0 * words * 4 + q4 * 4), coff1 = (uint32_t)(r1 * words * 4 + q4 * 4);
  const uint32_t soff0 = (uint32_t)(r0 * G * 2), soff1 = (uint32_t)(r1 * G * 2);
  const int eslot0 = r0 * QEROW + ((q4 ^ qswz(r0)) * 16);
  const int eslot1 = r1 * QEROW + ((q4 ^ qswz(r1)) * 16);
  // code word of row i for chunk (cb / 16 + j): the constant part goes in the immediate offset;
  // chunks past the end read other words of the row or zeros and are never used
  auto load_c = [&](CodeSet& S, int i, int cb, int j) {
    S.w[i] = __builtin_amdgcn_raw_buffer_load_b32(crsrc, (int)(i == 0 ? coff0 : coff1) + j * 16, cb, 0);
  };
  auto load_sz = [&](ScaleZero& P, int g) {
    P.d0 = __builtin_amdgcn_raw_buffer_load_b16(srsrc, (int)soff0, g * 2, 0);
    P.d1 = __builtin_amdgcn_raw_buffer_load_b16(srsrc, (int)soff1, g * 2, 0);
    P.z0 = __builtin_amdgcn_raw_buffer_load_b16(zrsrc, (int)soff0, g * 2, 0);
    P.z1 = __builtin_amdgcn_raw_buffer_load_b16(zrsrc, (int)soff1, g * 2, 0);
  };
  auto row_setup = [](uint32_t dh, uint32_t zh) {
    RowDq q;
    q.d = h2f((uint16_t)dh);
    q.nzd = -(h2f((uint16_t)zh) * q.d);  // exact: z <= 15 is an integer, Delta has 11 bits
    return q;
  };
  // weight j (0..7) of row i's word: Delta (q - z) with q = nibble j
  auto elem = [&](const CodeSet& S, const RowDq& q, int i, int j) {
    const uint32_t u = (j & 1) ? (S.w[i] >> 4) & 0x0f0f0f0fu : S.w[i] & 0x0f0f0f0fu;
    const int b = j >> 1;
    const float qf = b == 0 ? ubyte<0>(u) : b == 1 ? ubyte<1>(u) : b == 2 ? ubyte<2>(u) : ubyte<3>(u);
    return fmaf(qf, q.d, q.nzd);
  };
  auto store_piece = [&](uint8_t* estage, int slot, const float* e8) {
    uint32_t pk[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) pk[h] = bf16x2_of(e8[2 * h], e8[2 * h + 1]);
    *reinterpret_cast<uint4*>(estage + slot) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  };
  auto decode_all = [&](const CodeSet& S, const RowDq& q0, const RowDq& q1, uint8_t* estage) {  // prologue
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = elem(S, q0, 0, j);
    store_piece(estage, eslot0, e);
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = elem(S, q1, 1, j);
    store_piece(estage, eslot1, e);
  };
  // fragment reads: lane reads row (32 t + fr), 16-byte piece 2 h + fh of K-half h of its chunk
  const int fr = lane & 31, fh = lane >> 5;
  const int efoff0 = fr * QEROW + (((0 + fh) ^ qswz(fr)) * 16);
  const int efoff1 = fr * QEROW + (((2 + fh) ^ qswz(fr)) * 16);
  auto xfoff = [&](int half, int h) { return fr * QXROW + (((4 * half + 2 * h + fh) ^ qxswz(fr)) * 16); };
  auto frag = [&](const uint8_t* base, int fo) { return *reinterpret_cast<const bf16x8*>(base + fo); };
  auto vm_wait = [](auto n) {  // s_waitcnt vmcnt(n), other counters untouched
    constexpr int v = decltype(n)::value;
    __builtin_amdgcn_s_waitcnt((v & 0xf) | (0x7 << 4) | (0xf << 8) | ((v >> 4) << 14));
  };
  constexpr int kWaitLgkm0 = 0xf | (0x7 << 4) | (0x0 << 8) | (0x3 << 14);

  f32x16 acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.0f;

  CodeSet S0, S1, S2, S3;  // code words of chunk c live in set c % 4
  ScaleZero PC, PN;        // scales and zeros of the group being decoded, of the next group
  RowDq q0, q1;            // row_setup of PC (rows r0, r1)
  // Prologue: group 0's scales and zeros, codes of chunks 0-3, the X pair of chunks 0 and 1 (XF:
  // chunk 0's A fragments); then chunks 0 and 1 are decoded.
  bf16x8 a0[4], a1[4], b0[4];
  load_sz(PC, 0);
  load_c(S0, 0, 0, 0);
  load_c(S1, 0, 0, 1);
  load_c(S0, 1, 0, 0);
  load_c(S1, 1, 0, 1);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (XF) {
#pragma unroll
    for (int r = 0; r < 4; ++r) a0[r] = load_a(0, 0, r);
#pragma unroll
    for (int r = 0; r < 4; ++r) a1[r] = load_a(0, 1, r);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) dma_x_one(i < 8 ? xp0lo : xp0hi, i, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  load_c(S2, 0, 0, 2);
  load_c(S3, 0, 0, 3);
  load_c(S2, 1, 0, 2);
  load_c(S3, 1, 0, 3);
  __builtin_amdgcn_sched_barrier(0);
  vm_wait(std::integral_constant<int, 0>{});
  __builtin_amdgcn_sched_barrier(0);
  q0 = row_setup(PC.d0, PC.z0);
  q1 = row_setup(PC.d1, PC.z1);
  decode_all(S0, q0, q1, es + 0 * QESTAGE);
  decode_all(S1, q0, q1, es + 1 * QESTAGE);
  {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!XF) {
#pragma unroll
      for (int t = 0; t < 2; ++t) a0[t] = frag(xp0lo + xwave + t * 32 * QXROW, xfoff(0, 0));
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) b0[t] = frag(es + t * 32 * QEROW, efoff0);
    // use the code words of chunks 2 and 3 here, so that their loads are not sunk to the loop
    // head (where every iteration would wait for them)
    asm volatile("" ::"v"(S2.w[0]), "v"(S2.w[1]), "v"(S3.w[0]), "v"(S3.w[1]));
  }

  // One step, hand-scheduled in 32 groups, one per matrix instruction of chunk c (k = c % 4
  // known at compile time; xc is chunk c's pair stage, xn chunk c+1's):
  //   groups 0, 1: A fragments 2, 3 of chunk c (first used in groups 8 and 12);
  //   groups 0-7: second-half fragment reads of chunk c (A even, B odd groups);
  //   groups 3-25, two of every three: the sixteen weights of chunk c+2; W stores in groups 14
  //   and 26;
  //   groups 17-23 (odd): chunk c+1's B fragments of the first K-half; groups 24, 25: its A
  //   fragments 0, 1;
  //   vector memory: even steps the code words of chunks c+4 and c+5 (groups 0-3), when k = 0
  //   the next group's scales and zeros (groups 4, 5), and the copy of pair c/2 + 1, rows 0-63
  //   (groups 6, 9, ..., 27); odd steps the same pair's rows 64-127 (groups 0, 2, ..., 14).
  // vmcnt accounting (even steps: 4 code loads, 4 more when k = 0, 8 copies; odd steps: 8):
  //   * start of an even step: everything landed (the rows 64-127 of chunk c, copied by the
  //     previous step, are read now); start of an odd step: at most the previous step's last 12
  //     outstanding (chunk c's X comes from steps c-3 and c-2, the codes of chunk c+2 from step
  //     c-3 or c-2);
  //   * group 24 of an odd step: chunk c+1's rows 0-63 (copied by step c-1) landed, with this
  //     step's 8 copies after them; of an even step: nothing is awaited (those rows came from
  //     step c-2), the count is this step's loads before group 24.
  // XF: no copies and no explicit waits; the A fragments of chunk c+1 are loaded in groups 4, 8,
  // 12, 16 (K-half 0) and 20, 24, 28, 31 (K-half 1), and the compiler's counters wait for them
  // and for the code words, scales and zeros (all loaded into registers).
  auto step = [&](int c8, auto jc, const uint8_t* xclo, const uint8_t* xchi, const uint8_t* xnlo, uint8_t* xdlo,
                  uint8_t* xdhi, const CodeSet& Q, CodeSet& F4, CodeSet& F5, int& eo0, int& eo1, int& eo2) {
    constexpr int j = decltype(jc)::value;
    constexpr int k = j & 3;
    constexpr bool even = (k & 1) == 0;
    const int cb = c8 * 16;                    // chunk c8's byte offset in a row of code words
    const int pd = (c8 >> 1) + (j >> 1) + 1;   // pair being copied
    const int gn = (c8 >> 2) + (j >> 2) + 1;   // next group (k = 0 steps)
    const uint8_t* ec = es + eo0;
    const uint8_t* en = es + eo1;
    uint8_t* eq = es + eo2;
    const uint8_t* xwlo = xclo + xwave;
    const uint8_t* xwhi = xchi + xwave;
    const uint8_t* xnw = xnlo + xwave;
    auto xa = [&](int t) { return (t < 2 ? xwlo : xwhi) + (t & 1) * 32 * QXROW; };
    const int xo0 = xfoff(k & 1, 0), xo1 = xfoff(k & 1, 1), xn0 = xfoff((k + 1) & 1, 0);
    if (k == 2) {  // chunks c+2 .. c+5: the next group
      PC = PN;
      q0 = row_setup(PC.d0, PC.z0);
      q1 = row_setup(PC.d1, PC.z1);
    }
    bf16x8 b1[4];
    float e[16];
    const int ca = c8 + j + 1;  // XF: the chunk whose A fragments this step loads
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!XF) vm_wait(std::integral_constant<int, even ? 0 : 12>{});
#pragma unroll
    for (int g = 0; g < 32; ++g) {
      const int r = (g >> 2) & 3, cc = g & 3;
      if (g < 16)
        acc[r][cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[r], b0[cc], acc[r][cc], 0, 0, 0);
      else
        acc[r][cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[r], b1[cc], acc[r][cc], 0, 0, 0);
      if constexpr (XF) {
        // past the last chunk these read other rows of the tile or zeros (unused)
        if (g >= 4 && g <= 16 && (g & 3) == 0) a0[(g >> 2) - 1] = load_a(ca, 0, (g >> 2) - 1);
        if (g >= 20 && g <= 28 && (g & 3) == 0) a1[(g >> 2) - 5] = load_a(ca, 1, (g >> 2) - 5);
        if (g == 31) a1[3] = load_a(ca, 1, 3);
        if (g < 8 && (g & 1)) b1[g >> 1] = frag(ec + (g >> 1) * 32 * QEROW, efoff1);
      } else {
        if (g < 2) a0[2 + g] = frag(xa(2 + g), xo0);
        if (g < 8) {
          if (g & 1)
            b1[g >> 1] = frag(ec + (g >> 1) * 32 * QEROW, efoff1);
          else
            a1[g >> 1] = frag(xa(g >> 1), xo1);
        }
      }
      // weight el in group 3 + 3 (el / 2) + el % 2: groups 3-13 for row r0, 15-25 for r1
      const int el = g >= 3 && g <= 25 && (g - 3) % 3 != 2 ? 2 * ((g - 3) / 3) + (g - 3) % 3 : -1;
      if (el >= 0) {
        e[el] = el < 8 ? elem(Q, q0, 0, el) : elem(Q, q1, 1, el - 8);
        asm volatile("" : "+v"(e[el]));  // keep the weight in this group
      }
      if (g == 14) store_piece(eq, eslot0, e);
      if (g == 26) store_piece(eq, eslot1, e + 8);
      // every fragment read before group 8 has landed; only the W store of group 14 may be in
      // flight
      if (g == 15) __builtin_amdgcn_s_waitcnt(0xf | (0x7 << 4) | (0x1 << 8) | (0x3 << 14));
      if (g >= 16 && g < 24 && (g & 1)) b0[(g - 16) >> 1] = frag(en + ((g - 16) >> 1) * 32 * QEROW, efoff0);
      if constexpr (!XF) {
        if (g == 24) vm_wait(std::integral_constant<int, even ? (k == 0 ? 14 : 10) : 8>{});
        if (g == 24 || g == 25) a0[g - 24] = frag(xnw + (g - 24) * 32 * QXROW, xn0);
      }
      if (even) {
        if (g == 0) load_c(F4, 0, cb, j + 4);
        if (g == 1) load_c(F5, 0, cb, j + 5);
        if (g == 2) load_c(F4, 1, cb, j + 4);
        if (g == 3) load_c(F5, 1, cb, j + 5);
        if (k == 0 && g == 4) {
          PN.d0 = __builtin_amdgcn_raw_buffer_load_b16(srsrc, (int)soff0, gn * 2, 0);
          PN.d1 = __builtin_amdgcn_raw_buffer_load_b16(srsrc, (int)soff1, gn * 2, 0);
        }
        if (k == 0 && g == 5) {
          PN.z0 = __builtin_amdgcn_raw_buffer_load_b16(zrsrc, (int)soff0, gn * 2, 0);
          PN.z1 = __builtin_amdgcn_raw_buffer_load_b16(zrsrc, (int)soff1, gn * 2, 0);
        }
        if (!XF && g >= 6 && g <= 27 && (g - 6) % 3 == 0) dma_x_one(xdlo, (g - 6) / 3, pd);
      } else {
        if (!XF && g <= 14 && (g & 1) == 0) dma_x_one(xdhi, 8 + g / 2, pd);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // W stores of chunk c+2, fragment reads
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const int et = eo0;
    eo0 = eo1;
    eo1 = eo2;
    eo2 = et;
  };

  // nchunks = K / 32 is a multiple of 4.  Step c multiplies chunk c from pair stage (c / 2) % 2,
  // decodes set (c+2) % 4 into W stage (c+2) % 3, copies half of pair c/2 + 1 into stage
  // (c/2 + 1) % 2 and, when even, loads the codes of chunks c+4 and c+5 into sets c % 4 and
  // (c+1) % 4.  The unrolled body covers eight steps so that both pair stages keep static roles.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  using I6 = std::integral_constant<int, 6>;
  using I7 = std::integral_constant<int, 7>;
  int eo0 = 0, eo1 = QESTAGE, eo2 = 2 * QESTAGE;
  int c = 0;
  for (; c + 8 <= nchunks; c += 8) {
    step(c, I0{}, xp0lo, xp0hi, xp0lo, xp1lo, xp1hi, S2, S0, S1, eo0, eo1, eo2);
    step(c, I1{}, xp0lo, xp0hi, xp1lo, xp1lo, xp1hi, S3, S0, S1, eo0, eo1, eo2);
    step(c, I2{}, xp1lo, xp1hi, xp1lo, xp0lo, xp0hi, S0, S2, S3, eo0, eo1, eo2);
    step(c, I3{}, xp1lo, xp1hi, xp0lo, xp0lo, xp0hi, S1, S2, S3, eo0, eo1, eo2);
    step(c, I4{}, xp0lo, xp0hi, xp0lo, xp1lo, xp1hi, S2, S0, S1, eo0, eo1, eo2);
    step(c, I5{}, xp0lo, xp0hi, xp1lo, xp1lo, xp1hi, S3, S0, S1, eo0, eo1, eo2);
    step(c, I6{}, xp1lo, xp1hi, xp1lo, xp0lo, xp0hi, S0, S2, S3, eo0, eo1, eo2);
    step(c, I7{}, xp1lo, xp1hi, xp0lo, xp0lo, xp0hi, S1, S2, S3, eo0, eo1, eo2);
  }
  if (c < nchunks) {  // K / 128 odd: one more group
    step(c, I0{}, xp0lo, xp0hi, xp0lo, xp1lo, xp1hi, S2, S0, S1, eo0, eo1, eo2);
    step(c, I1{}, xp0lo, xp0hi, xp1lo, xp1lo, xp1hi, S3, S0, S1, eo0, eo1, eo2);
    step(c, I2{}, xp1lo, xp1hi, xp1lo, xp0lo, xp0hi, S0, S2, S3, eo0, eo1, eo2);
    step(c, I3{}, xp1lo, xp1hi, xp0lo, xp0lo, xp0hi, S1, S2, S3, eo0, eo1, eo2);
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt 0: no copy or load outlives the block
  // 32x32 result layout: lane l holds column l % 32, rows 8 (i / 4) + 4 (l / 32) + i % 4.
  if (m0 + PBM <= M) {
    // a whole token tile: stores through a buffer resource based at Y[m0, n0], with no branch
    // per store: the lane's offset is a VGPR, each store's row a scalar (512 rows of Y span
    // less than 2^31 bytes: host-checked), and columns past N are one lane mask per 32-column
    // block.  Every row addressed here is below M.
    const __amdgpu_buffer_rsrc_t yrsrc = rsrc(Y + m0 * ldy + n0, (PBM * ldy - n0) * 4);
    const uint32_t ldy4 = (uint32_t)ldy * 4u;
    const int yv = (int)((uint32_t)(wave * 128 + 4 * (lane / 32)) * ldy4 + (uint32_t)(lane % 32) * 4u);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      if (n0 + cc * 32 + (lane % 32) < N) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t so = (uint32_t)(r * 32 + 8 * (i / 4) + (i % 4)) * ldy4 + (uint32_t)(cc * 128);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[r][cc][i]), yrsrc, yv, (int)so, 0);
          }
      }
    }
  } else {
    // the last, partial token tile: each store checks its row and column
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t m = m0 + wave * 128 + r * 32 + 8 * (i / 4) + 4 * (lane / 32) + (i % 4);
          const int64_t n = n0 + cc * 32 + (lane % 32);
          if (m < M && n < N) Y[m * ldy + n] = acc[r][cc][i];
        }
  }
}

}  // namespace

// decode grid: one wave per row group, at most what is resident at once and at most
// max_per_cu blocks per CU (every wave then starts at the launch and loads its first rows while
// X is staged).  Fewer blocks sweeping the weight as a moving window stream it faster than a
// wave per row group: back to back over eight 28672 x 4096 artefacts, one token took 15.2 us
// per call at four blocks per CU and 16.4 us at all that is resident (eight); four tokens 26 us
// at two blocks per CU against 30 us.  The resident count is a property of the device and of
// the kernel instantiation (its LDS size is fixed by its token count), so it is queried once
// per device and kept: a decode launch costs ~15 us and the occupancy query is not free.  The
// cache packs (LDS bytes, resident blocks per CU, CUs) in one word; two threads that race on
// the first call store the same value.
template <typename Kern>
int64_t gemv_blocks(Kern kern, size_t lds, int64_t waves, int max_per_cu) {
  constexpr int kMaxDevices = 64;
  static std::atomic<uint64_t> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  std::atomic<uint64_t>* slot = dev < kMaxDevices ? &cache[dev] : nullptr;
  uint64_t packed = slot ? slot->load(std::memory_order_relaxed) : 0;
  if (packed == 0 || (packed >> 32) != (uint64_t)lds) {
    int cus = 256, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kGvThreads, lds) != hipSuccess || per_cu < 1)
      per_cu = 1;
    packed = ((uint64_t)lds << 32) | ((uint64_t)(per_cu < 255 ? per_cu : 255) << 24) | (uint64_t)(cus & 0xffffff);
    if (slot) slot->store(packed, std::memory_order_relaxed);
  }
  const int64_t per_cu = (int64_t)((packed >> 24) & 0xff), cus = (int64_t)(packed & 0xffffff);
  const int64_t resident = cus * (per_cu < max_per_cu ? per_cu : max_per_cu);
  const int64_t need = (waves + kGvThreads / 64 - 1) / (kGvThreads / 64);
  return need < resident ? need : resident;
}

// channels per decode pass: X of one pass takes at most 64 KiB of LDS (fp32)
int64_t w4a16_gemv_kc(int64_t M) { return M <= 2 ? 4096 : 2048; }

// channels per pass of the matrix-core decode and its LDS bytes: the widest multiple of 1024
// channels (whole rounds of kMfDepth groups) whose pairs and group sums fit, beside the four
// waves' 8 KiB code rounds, in 104 KiB, at most K.  (At 72 KiB, two blocks per CU, eight tokens
// took two K passes of 4096 channels and 22.9 us per call against 21.5 in one pass.)
size_t w4a16_mfma_lds(int64_t M, int64_t kc) {
  return (size_t)(M * (kc / 2 + 4) * 4 + (kc / kGroup) * 64 + (kGvThreads / 64) * 16 * 128 * 4);
}
int64_t w4a16_mfma_kc(int64_t M, int64_t K) {
  int64_t kc = K < 32768 ? K : 32768;
  if (kc > 1024) kc -= kc % 1024;
  while (kc > 1024 && w4a16_mfma_lds(M, kc) > 104 * 1024) kc -= 1024;
  return kc;
}

size_t w4a16_xcopy_bytes(bool xf32, int64_t M, int64_t K) {
  if (xf32 || M <= kW4a16GemvMax || K % 64 != 0) return 0;
  return (size_t)((M + 31) / 32 * 32) * (size_t)K * 2;
}

hipError_t launch_w4a16(const void* X, bool xf32, int64_t M, int64_t K, int64_t ldx, const int32_t* qweight,
                        const uint16_t* scales, const uint16_t* zeros, int64_t N, float* Y, int64_t ldy,
                        uint16_t* xcopy, hipStream_t st) {
  if (!xf32 && M > kW4a16GemvMax) {
    const int64_t mtiles = (M + PBM - 1) / PBM, ntiles = (N + PBN - 1) / PBN;
    const int64_t tiles = mtiles * ntiles, per_xcd = (tiles + 7) / 8;
    if (xcopy != nullptr) {
      hipError_t e = launch_xfrag(static_cast<const uint16_t*>(X), M, K, ldx, xcopy, st);
      if (e != hipSuccess) return e;
      w4a16_gemm_pipe_kernel<true><<<(unsigned)(8 * per_xcd), 256, 0, st>>>(
          xcopy, M, K, K, qweight, scales, zeros, N, Y, ldy, ntiles, tiles, per_xcd);
    } else {
      w4a16_gemm_pipe_kernel<false><<<(unsigned)(8 * per_xcd), 256, 0, st>>>(
          static_cast<const uint16_t*>(X), M, ldx, K, qweight, scales, zeros, N, Y, ldy, ntiles, tiles, per_xcd);
    }
    return hipGetLastError();
  }
  // decode path, up to 8 tokens per launch (fp32 X always takes it).  bf16 X with two or more
  // tokens goes to the matrix cores when its rounds of 8 groups line up: K a multiple of 1024 and
  // 16-byte aligned scales and zeros (their 16-byte loads); otherwise to the dot kernel.  Back to
  // back over eight 28672 x 4096 artefacts, per call: 2 tokens 16.9 us against 18.6 on the dot
  // kernel, 4 tokens 17.5 against 26.0, 8 tokens 21.5 against 40.4; one token 17.3 against 14.7.
  const bool mfma_ok = K % 1024 == 0 && (reinterpret_cast<uintptr_t>(scales) & 15u) == 0 &&
                       (reinterpret_cast<uintptr_t>(zeros) & 15u) == 0;
  for (int64_t m0 = 0; m0 < M; m0 += kW4a16GemvMax) {
    const int64_t mb = M - m0 < kW4a16GemvMax ? M - m0 : kW4a16GemvMax;
    const char* xp = static_cast<const char*>(X) + m0 * ldx * (xf32 ? 4 : 2);
    float* yp = Y + m0 * ldy;
    const int64_t kc = w4a16_gemv_kc(mb);
    const int64_t kcd = mb <= 2 ? 8192 : 4096;  // pairs + sums: at most 80 KiB, 4 segments
    const size_t lds = (size_t)mb * (size_t)kc * 4;
#define AWQ_GV(MV)                                                                                       \
  do {                                                                                                   \
    if (!xf32 && mfma_ok && mb >= kMfMinTokens) {                                                        \
      const int64_t kcm = w4a16_mfma_kc(mb, K);                                                          \
      const size_t ldsm = w4a16_mfma_lds(mb, kcm);                                                       \
      const int64_t blocks = gemv_blocks(w4a16_gemv_mfma_kernel, ldsm, (N + 15) / 16, kMfPerCu);         \
      w4a16_gemv_mfma_kernel<<<(unsigned)blocks, kGvThreads, ldsm, st>>>(                                \
          static_cast<const uint16_t*>(static_cast<const void*>(xp)), ldx, (int)mb, K, qweight, scales,  \
          zeros, N, yp, ldy, kcm);                                                                       \
    } else if (!xf32) {                                                                                  \
      constexpr int RV = MV <= 2 ? 2 : 4;                                                                \
      const size_t ldsd = (size_t)mb * kcd * 5 / 2;                                                      \
      const int64_t blocks = gemv_blocks(w4a16_gemv_dot_kernel<MV, RV>, ldsd, (N + RV - 1) / RV,         \
                                         MV <= 2 ? 4 : 2);                                               \
      w4a16_gemv_dot_kernel<MV, RV><<<(unsigned)blocks, kGvThreads, ldsd, st>>>(                         \
          static_cast<const uint16_t*>(static_cast<const void*>(xp)), ldx, K, qweight, scales, zeros, N, \
          yp, ldy, kcd);                                                                                 \
    } else {                                                                                             \
      const int64_t blocks = gemv_blocks(w4a16_gemv_kernel<MV, true>, lds, (N + kGvRows - 1) / kGvRows,  \
                                         64);                                                            \
      w4a16_gemv_kernel<MV, true><<<(unsigned)blocks, kGvThreads, lds, st>>>(xp, ldx, K, qweight, scales, \
                                                                            zeros, N, yp, ldy, kc);      \
    }                                                                                                    \
  } while (0)
    switch (mb) {
      case 1: AWQ_GV(1); break;
      case 2: AWQ_GV(2); break;
      case 3: AWQ_GV(3); break;
      case 4: AWQ_GV(4); break;
      case 5: AWQ_GV(5); break;
      case 6: AWQ_GV(6); break;
      case 7: AWQ_GV(7); break;
      default: AWQ_GV(8); break;
    }
#undef AWQ_GV
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace awq

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
  struct Slab {
    u32x4 q[R];
    uint16_t d[R], z[R];  // fp16 bits: converted where used, so that nothing
                                      // waits for the prefetch before the current math
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
      const int w0 = lw < pw ? lw : 0;                      // word within the pass
      const int g = (int)((c0 + 8 * (int64_t)w0) / kGroup);  // group of those words
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t n = fn0 + r < N ? fn0 + r : N - 1;
        const int32_t* rowp = qweight + n * words + c0 / 8;
        S.q[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowp + w0));
        S.d[r] = (scales + n * G)[g];
        S.z[r] = (zeros + n * G)[g];
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
          for (int r = 0; r < R; ++r)
            acc[r][m] = fmaf(h2f(S.d[r]), fmaf(-(128.0f + h2f(S.z[r])), sxm, sq[r]), acc[r][m]);
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

// ---- prefill -------------------------------------------------------------------------------
// A block of 8 waves (two per SIMD, at most 256 registers each) computes a 512-token x
// 128-output tile.  Each wave multiplies its own 64 tokens, so X never needs sharing: the wave
// copies its rows of every 32-channel chunk from global memory straight into LDS (buffer load
// with LDS destination, 1 KiB per instruction), three chunks deep, and nothing of X passes
// through registers or waits for a barrier.  The decoded weight tile is shared by all waves:
// its codes are loaded two chunks ahead, decoded after the chunk's matrix instructions and
// stored for the next chunk, which one barrier per chunk publishes.  The three X stages and
// the three W stages are distinct LDS objects with a fixed role in each step of the unrolled
// loop, so the compiler's wait counts for the copies stay exact.  LDS rows are 64 bytes,
// unpadded, their four 16-byte slots permuted per row (X by (row >> 2) & 3, W by wslot below)
// so that neither the fragment reads nor the stores meet a bank conflict.  (A 4-wave block,
// 128 tokens a wave at 512 registers, is the other instance of the template; it measured the
// same at 4096 tokens and slower at 512 and 16384.)
#define AWQ_LDS __attribute__((address_space(3)))
constexpr int PBM = 512, PBN = 128, PKC = 32;
constexpr int XSTAGE = PBM * PKC * 2;  // 32 KiB
constexpr int WSTAGE = PBN * PKC * 2;  // 8 KiB

__device__ __forceinline__ uint32_t bf16x2_of(float a, float b) {
  const bf16x2 h = __builtin_convertvector((f32x2){a, b}, bf16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ int pslot(int row, int s) { return (s ^ ((row >> 2) & 3)) * 16; }  // bytes
// W stage slots: f(row) = ((row >> 1) & 3) ^ 3 ((row >> 3) & 1).  LDS serves a 16-byte read for
// 16 lanes at a time over 64 four-byte banks and a 16-byte write for 8 lanes at a time over 32
// banks (measured with the bank-conflict counter); under this f both the 32-row fragment reads
// (16 consecutive rows, one slot) and the decode's stores (8 lanes: 4 rows x 2 slots) are
// conflict-free, where (row >> 2) & 3 doubled the stores' time.
__device__ __forceinline__ int wslot(int row, int s) {
  return (s ^ ((row >> 1) & 3) ^ (((row >> 3) & 1) * 3)) * 16;
}

// NW waves per block: wave w multiplies tokens RW w .. RW w + RW - 1 of the tile (RW = 512 / NW);
// a W row's four words of a chunk are decoded by TPR = NW / 2 threads, WPT = 4 / TPR words each.
template <int NW>
struct WRegs {
  uint32_t qv[8 / NW];  // this thread's words of its row: 8 codes each
};

template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void w4a16_gemm_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t ldx, int64_t K, const int32_t* __restrict__ qweight,
    const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros, int64_t N,
    float* __restrict__ Y, int64_t ldy, int64_t ntiles, int64_t tiles, int64_t per_xcd) {
  __shared__ __attribute__((aligned(1024))) uint8_t xs0[XSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs1[XSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs2[XSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ws0[WSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ws1[WSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t ws2[WSTAGE];
  const int64_t G = K / kGroup, words = K / 8;
  // Blocks go to the 8 XCDs round robin (block b to XCD b % 8); XCD x takes the tiles
  // x per_xcd .. (x + 1) per_xcd - 1 in order, so its blocks share token tiles and the tile's X
  // stays in that XCD's L2.  Blocks past the last tile (grid rounded up to 8) return at once.
  const int64_t L = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (L >= tiles) return;
  const int64_t mt = L / ntiles, nt = L % ntiles;
  const int64_t m0 = mt * PBM, n0 = nt * PBN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // X rows of this tile through a buffer resource: rows past M read as zero (host: 512 rows of
  // X span less than 2^31 bytes)
  const int64_t xbytes = (M - m0) * ldx * 2;
  const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(X + m0 * ldx), (short)0, (int)(xbytes < 0x7fffffff ? xbytes : 0x7fffffff), 0x00020000);
  constexpr int RW = PBM / NW, RT = RW / 32, NDMA = RW / 16, TPR = NW / 2, WPT = 4 / TPR;
  // copy instruction i (0 .. NDMA - 1) of this wave fills its rows 16 i + lane / 4 with 16 bytes
  // each: physical slot lane % 4 receives logical slot (lane % 4) ^ swizzle(row)
  uint32_t xoff[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int row = wave * RW + 16 * i + (lane >> 2);
    xoff[i] = (uint32_t)(row * ldx * 2 + (((lane & 3) ^ ((row >> 2) & 3)) * 16));
  }
  auto dma_x = [&](uint8_t* stage, int64_t c) {
#pragma unroll
    for (int i = 0; i < NDMA; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrsrc, (AWQ_LDS void*)(stage + (wave * RW + 16 * i) * 64), 16,
                                               (int)xoff[i], (int)(c * PKC * 2), 0, 0);
  };
  // W chunk: 128 rows x 4 words (32 channels); thread: row tid / TPR, words WPT (tid % TPR) ..
  const int wr = tid / TPR, wq = tid % TPR;
  const int64_t wn = n0 + wr;
  const bool wlive = wn < N;
  const int32_t* wrow = qweight + (wlive ? wn : 0) * words;
  const int64_t nch = K / PKC;  // a multiple of 4: a group is four chunks
  auto load_codes = [&](WRegs<NW>& R, int64_t c) {
    const int64_t cc = c < nch ? c : nch - 1;  // past the end: an in-bounds reload, never stored
    if constexpr (WPT == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(wrow + cc * (PKC / 8) + 2 * wq);
      R.qv[0] = v.x;
      R.qv[1] = v.y;
    } else {
      R.qv[0] = wrow[cc * (PKC / 8) + wq];
    }
  };
  // The row's fp16 scale and zero are loaded once per group, with the group's first chunk, into
  // register pair g mod 3; they stay fp16 bits until the decode, which comes two chunks later.
  uint32_t sd[3] = {0, 0, 0}, sz[3] = {0, 0, 0};
  auto load_group = [&](uint32_t& d, uint32_t& z, int64_t c) {
    const int64_t g = (c < nch ? c : nch - 1) / 4;
    d = scales[(wlive ? wn : 0) * G + g];
    z = zeros[(wlive ? wn : 0) * G + g];
  };
  auto store_w = [&](const WRegs<NW>& R, uint32_t dh, uint32_t zh, uint8_t* stage) {
    const float dv = wlive ? h2f((uint16_t)dh) : 0.0f, zv = h2f((uint16_t)zh);  // rows past N: weight 0
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      uint32_t pk[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float a = dv * ((float)((R.qv[j] >> (8 * c)) & 15u) - zv);  // exact in fp32
        const float bq = dv * ((float)((R.qv[j] >> (8 * c + 4)) & 15u) - zv);
        pk[c] = bf16x2_of(a, bq);
      }
      *reinterpret_cast<uint4*>(stage + wr * 64 + wslot(wr, WPT * wq + j)) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    }
  };
  f32x16 acc[RT][4];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.0f;
  const int frow = lane & 31, fs = lane >> 5;
  auto compute = [&](const uint8_t* xst, const uint8_t* wst) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 af[RT], bfr[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const int row = cc * 32 + frow;
        bfr[cc] = *reinterpret_cast<const bf16x8*>(wst + row * 64 + wslot(row, 2 * h + fs));
      }
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const int row = wave * RW + r * 32 + frow;
        af[r] = *reinterpret_cast<const bf16x8*>(xst + row * 64 + pslot(row, 2 * h + fs));
      }
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
          acc[r][cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[r], bfr[cc], acc[r][cc], 0, 0, 0);
    }
  };
  // stage i as the shared object itself (not through a pointer table), so that the compiler
  // knows which copy writes which stage and its wait counts stay exact
  auto xst = [&](auto I) -> uint8_t* {
    constexpr int i = decltype(I)::value % 3;
    if constexpr (i == 0) return xs0; else if constexpr (i == 1) return xs1; else return xs2;
  };
  auto wst = [&](auto I) -> uint8_t* {
    constexpr int i = decltype(I)::value % 3;
    if constexpr (i == 0) return ws0; else if constexpr (i == 1) return ws1; else return ws2;
  };
  // The barrier that publishes a W stage: this wave's LDS stores done (lgkmcnt 0), then
  // s_barrier.  No workgroup fence: a fence would also wait for every X copy still in flight
  // (they write LDS), though only the issuing wave reads those rows and its reads wait for
  // their own copies.  The signal fences keep the compiler from moving LDS accesses across.
  auto publish_w = [] {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // vmcnt 63, expcnt 7 (no wait), lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };
  WRegs<NW> rg[3];  // W codes of chunk c in set c % 3
  // Step c, with S = c mod 12 known at compile time (so that every stage, register set and
  // group pair is fixed and the step has no branch, which would cost the exact wait counts):
  // copy X chunk c + 2 into the X stage read two steps ago (past the end: a harmless re-copy
  // into a stage no later step reads), load W chunk c + 2's codes (and, at a group's first chunk,
  // its scale and zero), multiply chunk c, decode and store W chunk c + 1 into the W stage read
  // two steps ago, then the barrier that publishes it.
  auto step = [&](int64_t c, auto Sc) {
    constexpr int S = decltype(Sc)::value;
    dma_x(xst(std::integral_constant<int, S + 2>{}), c + 2 < nch ? c + 2 : nch - 1);
    load_codes(rg[(S + 2) % 3], c + 2);
    if constexpr ((S + 2) % 4 == 0) load_group(sd[((S + 2) / 4) % 3], sz[((S + 2) / 4) % 3], c + 2);
    __builtin_amdgcn_sched_barrier(0);  // the copies and loads ahead of the products they hide behind
    compute(xst(std::integral_constant<int, S>{}), wst(std::integral_constant<int, S>{}));
    store_w(rg[(S + 1) % 3], sd[((S + 1) / 4) % 3], sz[((S + 1) / 4) % 3], wst(std::integral_constant<int, S + 1>{}));
    publish_w();
  };
  dma_x(xs0, 0);
  dma_x(xs1, 1);
  load_codes(rg[0], 0);
  load_codes(rg[1], 1);
  load_group(sd[0], sz[0], 0);
  store_w(rg[0], sd[0], sz[0], ws0);
  __syncthreads();
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  using I6 = std::integral_constant<int, 6>;
  using I7 = std::integral_constant<int, 7>;
  using I8 = std::integral_constant<int, 8>;
  using I9 = std::integral_constant<int, 9>;
  using I10 = std::integral_constant<int, 10>;
  using I11 = std::integral_constant<int, 11>;
  int64_t c = 0;
  for (; c + 12 <= nch; c += 12) {
    step(c, I0{}); step(c + 1, I1{}); step(c + 2, I2{}); step(c + 3, I3{});
    step(c + 4, I4{}); step(c + 5, I5{}); step(c + 6, I6{}); step(c + 7, I7{});
    step(c + 8, I8{}); step(c + 9, I9{}); step(c + 10, I10{}); step(c + 11, I11{});
  }
  if (c < nch) {  // 4 or 8 chunks remain (nch is a multiple of 4)
    step(c, I0{}); step(c + 1, I1{}); step(c + 2, I2{}); step(c + 3, I3{});
    if (c + 4 < nch) {
      step(c + 4, I4{}); step(c + 5, I5{}); step(c + 6, I6{}); step(c + 7, I7{});
    }
  }
  // 32x32 result layout: lane l holds column l % 32, rows 8 (i / 4) + 4 (l / 32) + i % 4
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t m = m0 + wave * RW + r * 32 + 8 * (i / 4) + 4 * (lane / 32) + (i % 4);
        const int64_t n = n0 + cc * 32 + (lane % 32);
        if (m < M && n < N) Y[m * ldy + n] = acc[r][cc][i];
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

hipError_t launch_w4a16(const void* X, bool xf32, int64_t M, int64_t K, int64_t ldx, const int32_t* qweight,
                        const uint16_t* scales, const uint16_t* zeros, int64_t N, float* Y, int64_t ldy,
                        hipStream_t st) {
  if (!xf32 && M > kW4a16GemvMax) {
    const int64_t mtiles = (M + PBM - 1) / PBM, ntiles = (N + PBN - 1) / PBN;
    const int64_t tiles = mtiles * ntiles, per_xcd = (tiles + 7) / 8;
    constexpr int kGemmWaves = 8;
    w4a16_gemm_kernel<kGemmWaves><<<(unsigned)(8 * per_xcd), 64 * kGemmWaves, 0, st>>>(
        static_cast<const uint16_t*>(X), M, ldx, K, qweight, scales, zeros, N, Y, ldy, ntiles, tiles, per_xcd);
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

// After the scale search: the clipping search ("AWQ：为什么 4-bit 权重量化要先观察 Activation",
// §5).  With the chosen scales s, every output channel n and input group g of the scaled
// weight v = W s tries n_clip thresholds c_i = absmax_g |v| * (1 - i/20) (1, 0.95, ..., 0.55
// for the method's ten); the clipped group clamp(v, -c_i, c_i) goes through the same
// asymmetric quantizer as the scale search (§7), and the candidate's error is the mean over
// the given tokens of the squared error of the group's partial output,
//   err_i[n, g] = (1/M) sum_m ( sum_{k in g} X[m, k] E_i[n, k] )^2,
//   E_i = W - S^-1 Q(clamp(S W, -c_i, c_i)).
// Each (n, g) keeps the first candidate with the least error (§5: the thresholds are chosen
// per output channel and group independently).
//
// Three launches:
//   * clip_range_kernel: per (row, group) the absmax, the n_clip thresholds and the exact-
//     contract (Delta, z) of each clipped group; the first row block also writes 1/s;
//   * clip_err_kernel: per (candidate, 512-token tile, 128-row tile, block of groups) the
//     clipped qdq of W in registers (exact fp32 quotients), E in bf16 to LDS, Y = X E^T on the matrix cores group by
//     group, and after every group the column sums of Y^2 (fp32 over the tile's 512 tokens);
//   * clip_select_kernel: per (n, g) the fixed-order fp64 sum over token tiles, the mean and
//     the first minimum.
#include <type_traits>

#include "awq_internal.h"

namespace awq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int CBM = kClipBM;    // tokens per tile
constexpr int CBN = kClipBN;    // output channels per tile
constexpr int CTHREADS = 256;   // 4 waves, one per SIMD; wave w owns tokens 128 w .. 128 w + 127
constexpr int kClipRows = 64;   // rows per range block (four lanes per row)

__device__ __forceinline__ float lo16(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi16(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
// RN(a / b) from y = RN(1 / b) and two FMA residual corrections (Markstein): the codes of the
// product kernel are then exactly the contract's.  An error here is measured over one group
// of 128 weights, where a single code that differs would move it far more than the bf16
// rounding of E does.
__device__ __forceinline__ float exact_quot(float a, float b, float y) {
  const float q0 = a * y;
  const float q1 = fmaf(fmaf(-q0, b, a), y, q0);
  return fmaf(fmaf(-q1, b, a), y, q1);
}
__device__ __forceinline__ uint32_t to_bf16x2(float a, float b) {
  const bf16x2 h = __builtin_convertvector((f32x2){a, b}, bf16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

// ---- thresholds and clipped group ranges ---------------------------------------------------
// Block: 64 rows of one group, four lanes per row with 32 channels each.  params[i][g][n] =
// (Delta, z, c, 0) of candidate i; exact fp32 contract (correctly rounded division).
template <bool WF32>
__global__ __launch_bounds__(256) void clip_range_kernel(const void* __restrict__ W, int64_t N, int64_t K,
                                                         int64_t ldw, const float* __restrict__ s,
                                                         int n_clip, float4* __restrict__ params,
                                                         float* __restrict__ rs, uint32_t* __restrict__ flags) {
  const int64_t G = K / kGroup;
  const int64_t g = blockIdx.y;
  const int row = threadIdx.x >> 2, q = threadIdx.x & 3;
  const int64_t n = (int64_t)blockIdx.x * kClipRows + row;
  const int64_t nn = n < N ? n : N - 1;  // rows past N work on row N-1 and store nothing
  const int64_t k0 = g * kGroup + 32 * q;
  uint32_t bad = 0;
  float v[32];
  if constexpr (WF32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(W) + nn * ldw + k0);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float4 u = p[t];
      v[4 * t] = u.x; v[4 * t + 1] = u.y; v[4 * t + 2] = u.z; v[4 * t + 3] = u.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + nn * ldw + k0);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint4 u = p[t];
      const uint32_t uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        v[8 * t + 2 * h] = lo16(uu[h]);
        v[8 * t + 2 * h + 1] = hi16(uu[h]);
      }
    }
  }
  float peak = 0.0f, mx = -INFINITY, mn = INFINITY;
  bool nan = false;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float4 sv = *reinterpret_cast<const float4*>(s + k0 + 4 * t);
    const float sc[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      if (!(sc[h] > 0.0f) || isinf(sc[h])) bad |= kFlagScaleRange;
      const float x = v[4 * t + h] * sc[h];  // S W, one rounding
      nan |= x != x;
      peak = fmaxf(peak, fabsf(x));
      mx = fmaxf(mx, x);
      mn = fminf(mn, x);
    }
  }
  if (blockIdx.x == 0 && row == 0) {  // 1/s of this group's channels, for the product kernel
#pragma unroll
    for (int t = 0; t < 32; ++t) rs[k0 + t] = 1.0f / s[k0 + t];
  }
  peak = max4(peak);
  mx = max4(mx);
  mn = min4(mn);
  if (nan || isinf(peak)) bad |= kFlagNonfiniteW;
  if (n < N && q == 0) {
    for (int i = 0; i < n_clip; ++i) {
      const float f = (float)(1.0 - (double)i / 20.0);
      const float c = peak * f;  // threshold, one rounding
      const float hi = fminf(fmaxf(mx, -c), c), lo = fminf(fmaxf(mn, -c), c);  // of clamp(v)
      const float delta = fmaxf(hi - lo, 1e-5f) / 15.0f;
      const float z = fminf(fmaxf(rintf(-lo / delta), 0.0f), 15.0f);
      params[((int64_t)i * G + g) * N + n] = make_float4(delta, z, c, 0.0f);
    }
  }
  if (bad && n < N) atomicOr(flags, bad);
}

// ---- clipped qdq + error product, group by group ------------------------------------------
template <bool XF32>
struct ClipGeo {
  static constexpr int KC = XF32 ? 16 : 32;        // input channels per chunk
  static constexpr int PITCH = KC + 8;             // LDS row pitch in bf16 (16-byte pad)
  static constexpr int XPARTS = XF32 ? 2 : 1;      // bf16 terms of X
  static constexpr int XSZ = XF32 ? 4 : 2;
  static constexpr int XEL = XF32 ? 4 : 8;         // X elements per 16-byte piece
  static constexpr int XP = CBM * (KC / XEL) / CTHREADS;  // X pieces per thread (8)
  static constexpr int CPG = kGroup / KC;          // chunks per group
  static_assert(KC / XEL == 4, "X piece layout");
};

template <bool XF32, bool WF32>
__global__ __launch_bounds__(CTHREADS, 1) void clip_err_kernel(
    const void* __restrict__ X, int64_t M, int64_t ldx, const void* __restrict__ W, int64_t N,
    int64_t K, int64_t ldw, const float* __restrict__ s, const float* __restrict__ rs,
    const float4* __restrict__ params, int n_clip, int64_t mtiles, int64_t ntiles, int gpb,
    float* __restrict__ partial) {
  using Gm = ClipGeo<XF32>;
  constexpr int KC = Gm::KC;
  constexpr int PITCH = Gm::PITCH;
  constexpr int XPARTS = Gm::XPARTS;
  constexpr int XP = Gm::XP;
  constexpr int XSZ = Gm::XSZ;
  constexpr int WEL = WF32 ? 4 : 8;                 // W elements per 16-byte piece
  constexpr int WSZ = WF32 ? 4 : 2;
  constexpr int WPPR = KC / WEL;                    // W pieces per row per chunk
  constexpr int WP = CBN * WPPR / CTHREADS;         // W pieces per thread
  constexpr int WROW_STEP = CTHREADS / WPPR;

  __shared__ __attribute__((aligned(16))) uint16_t xs[2][XPARTS][CBM][PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t es[2][CBN][PITCH];
  __shared__ float red[4][CBN];

  const int64_t G = K / kGroup;
  const int64_t gblocks = (G + gpb - 1) / gpb;
  int64_t L = blockIdx.x;
  const int al = (int)(L % n_clip);
  L /= n_clip;
  const int64_t nt = L % ntiles;
  L /= ntiles;
  const int64_t mt = L % mtiles;
  const int64_t gb = L / mtiles;
  if (gb >= gblocks) return;
  const int64_t m0 = mt * CBM, n0 = nt * CBN;
  const int g0 = (int)(gb * gpb), g1 = (int)((g0 + gpb < G) ? g0 + gpb : G);
  const int c0 = g0 * Gm::CPG, c1 = g1 * Gm::CPG;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int xkp = tid & 3, xrow0 = tid >> 2;
  const int wkp = tid % WPPR, wrow0 = tid / WPPR;

  // buffer resources rebased at the tile: rows past M (or N) read as zero; offsets < 2^31
  // (host-checked: 512 rows of X, 128 rows of W)
  const int64_t xbytes = (M - m0) * ldx * XSZ, wbytes = (N - n0) * ldw * WSZ;
  const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const char*>(X) + m0 * ldx * XSZ), (short)0,
      (int)(xbytes < 0x7fffffff ? xbytes : 0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const char*>(W) + n0 * ldw * WSZ), (short)0,
      (int)(wbytes < 0x7fffffff ? wbytes : 0x7fffffff), 0x00020000);
  const uint32_t xoff0 = (uint32_t)(xrow0 * ldx * XSZ + xkp * 16);
  const uint32_t xstep = (uint32_t)(64 * ldx * XSZ);
  const uint32_t woff0 = (uint32_t)(wrow0 * ldw * WSZ + wkp * 16);
  const uint32_t wstep = (uint32_t)(WROW_STEP * ldw * WSZ);

  const float4* prow[WP];
  bool wlive[WP];
#pragma unroll
  for (int i = 0; i < WP; ++i) {
    const int64_t n = n0 + wrow0 + WROW_STEP * i;
    wlive[i] = n < N;
    prow[i] = params + (int64_t)al * G * N + (wlive[i] ? n : 0);
  }

  uint4 xr[XP], wr[WP];
  float4 sr[WEL / 4], rsr[WEL / 4], pr[WP];
  auto load_chunk = [&](int c) {
    const uint32_t kb = (uint32_t)(c * KC);
#pragma unroll
    for (int i = 0; i < XP; ++i)
      xr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            xrsrc, (int)(xoff0 + i * xstep + kb * XSZ), 0, 0));
#pragma unroll
    for (int i = 0; i < WP; ++i)
      wr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            wrsrc, (int)(woff0 + i * wstep + kb * WSZ), 0, 0));
#pragma unroll
    for (int t = 0; t < WEL / 4; ++t) {
      sr[t] = *reinterpret_cast<const float4*>(s + kb + wkp * WEL + 4 * t);
      rsr[t] = *reinterpret_cast<const float4*>(rs + kb + wkp * WEL + 4 * t);
    }
    const int g = (int)(kb / kGroup);
#pragma unroll
    for (int i = 0; i < WP; ++i) pr[i] = prow[i][(int64_t)g * N];
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int row = xrow0 + 64 * i;
      if constexpr (XF32) {
        const float f[4] = {__uint_as_float(xr[i].x), __uint_as_float(xr[i].y),
                            __uint_as_float(xr[i].z), __uint_as_float(xr[i].w)};
        uint32_t hi2[2], lo2[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x2 h = __builtin_convertvector((f32x2){f[2 * t], f[2 * t + 1]}, bf16x2);
          const f32x2 hf = __builtin_convertvector(h, f32x2);
          hi2[t] = __builtin_bit_cast(uint32_t, h);
          lo2[t] = to_bf16x2(f[2 * t] - hf.x, f[2 * t + 1] - hf.y);
        }
        *reinterpret_cast<uint2*>(&xs[buf][0][row][xkp * 4]) = make_uint2(hi2[0], hi2[1]);
        *reinterpret_cast<uint2*>(&xs[buf][1][row][xkp * 4]) = make_uint2(lo2[0], lo2[1]);
      } else {
        *reinterpret_cast<uint4*>(&xs[buf][0][row][xkp * 8]) = xr[i];
      }
    }
    float sv[WEL], rsv[WEL];
#pragma unroll
    for (int t = 0; t < WEL / 4; ++t) {
      sv[4 * t] = sr[t].x; sv[4 * t + 1] = sr[t].y; sv[4 * t + 2] = sr[t].z; sv[4 * t + 3] = sr[t].w;
      rsv[4 * t] = rsr[t].x; rsv[4 * t + 1] = rsr[t].y; rsv[4 * t + 2] = rsr[t].z; rsv[4 * t + 3] = rsr[t].w;
    }
#pragma unroll
    for (int i = 0; i < WP; ++i) {
      const int row = wrow0 + WROW_STEP * i;
      // rows past N: Delta 1, z 0, c 0 and w 0 give e = 0 exactly
      const float delta = wlive[i] ? pr[i].x : 1.0f;
      const float z = wlive[i] ? pr[i].y : 0.0f;
      const float c = wlive[i] ? pr[i].z : 0.0f;
      const float inv = 1.0f / delta;  // correctly rounded
      const float qlo = -z, qhi = 15.0f - z;
      float w[WEL];
      if constexpr (WF32) {
        w[0] = __uint_as_float(wr[i].x); w[1] = __uint_as_float(wr[i].y);
        w[2] = __uint_as_float(wr[i].z); w[3] = __uint_as_float(wr[i].w);
      } else {
        const uint32_t u[4] = {wr[i].x, wr[i].y, wr[i].z, wr[i].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          w[2 * t] = lo16(u[t]);
          w[2 * t + 1] = hi16(u[t]);
        }
      }
      float e[WEL];
#pragma unroll
      for (int j = 0; j < WEL; ++j) {
        const float v = __builtin_amdgcn_fmed3f(w[j] * sv[j], -c, c);  // clamp(S W, -c, c)
        const float r = rintf(exact_quot(v, delta, inv));              // rne(RN(v / Delta))
        const float qz = __builtin_amdgcn_fmed3f(r, qlo, qhi);         // clamp(r + z, 0, 15) - z
        e[j] = fmaf(-(qz * delta), rsv[j], w[j]);                      // w - Delta (q - z) / s
      }
      uint32_t pk[WEL / 2];
#pragma unroll
      for (int t = 0; t < WEL / 2; ++t) pk[t] = to_bf16x2(e[2 * t], e[2 * t + 1]);
      if constexpr (WEL == 8)
        *reinterpret_cast<uint4*>(&es[buf][row][wkp * 8]) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      else
        *reinterpret_cast<uint2*>(&es[buf][row][wkp * 4]) = make_uint2(pk[0], pk[1]);
    }
  };

  f32x16 acc[4][4];
  auto zero_acc = [&]() {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.0f;
  };
  zero_acc();
  const int frow = lane & 31, fk = (lane >> 5) * 8;
  auto mfma_chunk = [&](int buf) {
#pragma unroll
    for (int j = 0; j < KC / 16; ++j) {
      bf16x8 bfr[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) bfr[c] = *reinterpret_cast<const bf16x8*>(&es[buf][c * 32 + frow][j * 16 + fk]);
#pragma unroll
      for (int p = 0; p < XPARTS; ++p) {
        bf16x8 afr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          afr[r] = *reinterpret_cast<const bf16x8*>(&xs[buf][p][wave * 128 + r * 32 + frow][j * 16 + fk]);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[r], bfr[c], acc[r][c], 0, 0, 0);
      }
    }
  };
  // Column sums of Y^2 for group g: in the 32x32 result layout lane l holds column l % 32 of
  // its tile (16 rows, the other 16 in lane l ^ 32), so each lane squares and adds its 64
  // values per column tile, lanes l and l ^ 32 combine, and the four waves (token quarters)
  // are added in a fixed order through LDS.
  auto epilogue = [&](int g) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float t = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) t = fmaf(acc[r][c][i], acc[r][c][i], t);
      t += __shfl_xor(t, 32);
      if (lane < 32) red[wave][c * 32 + lane] = t;
    }
    __syncthreads();
    if (tid < CBN && n0 + tid < N) {
      const float tot = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
      partial[(((int64_t)al * G + g) * mtiles + mt) * N + n0 + tid] = tot;
    }
    zero_acc();
  };

  load_chunk(c0);
  store_chunk(0);
  __syncthreads();
  for (int c = c0; c < c1; ++c) {
    const int buf = (c - c0) & 1;
    load_chunk(c + 1 < c1 ? c + 1 : c);  // the last step reloads its own chunk (unused)
    mfma_chunk(buf);
    store_chunk(buf ^ 1);
    // after the group's last chunk (here the prefetched registers are already consumed); red
    // is written again only CPG barriers later
    if ((c + 1) % Gm::CPG == 0) epilogue(c / Gm::CPG);
    __syncthreads();
  }
}

// ---- bf16 X: one group's X resident in LDS for all candidates ----------------------------
// Block = (128-row tile, 512-token tile, block of groups); every candidate is handled inside
// the block.  Per group the block loads X[512 tokens x 128 channels] into LDS once (136 KiB,
// rows padded to 272 bytes: the 32-row fragment reads hit 16 distinct bank groups) and its W
// pieces into registers once; then for each candidate it quantizes the four 32-channel E
// chunks with that candidate's (Delta, z, c), multiplies, and writes the group's column sums
// of Y^2.  Each X and W byte serves n_clip candidates, so the product runs on data already in
// the CU instead of waiting for memory at every chunk.
constexpr int XGP = kGroup + 8;  // LDS pitch of a group row of X, in bf16

template <bool WF32>
__global__ __launch_bounds__(CTHREADS, 1) void clip_err_group_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t ldx, const void* __restrict__ W, int64_t N,
    int64_t K, int64_t ldw, const float* __restrict__ s, const float* __restrict__ rs,
    const float4* __restrict__ params, int n_clip, int64_t mtiles, int64_t ntiles, int gpb,
    float* __restrict__ partial) {
  constexpr int KC = 32;                      // channels per E chunk
  constexpr int EP = KC + 8;                  // LDS pitch of an E row
  constexpr int WEL = WF32 ? 4 : 8;           // W elements per 16-byte piece
  constexpr int WSZ = WF32 ? 4 : 2;
  constexpr int WPPR = KC / WEL;              // W pieces per row per chunk
  constexpr int WP = CBN * WPPR / CTHREADS;   // W pieces per thread per chunk
  constexpr int WROW_STEP = CTHREADS / WPPR;
  constexpr int CPG = kGroup / KC;            // 4 chunks per group
  constexpr int XPG = CBM * (kGroup / 8) / CTHREADS;  // 16-byte X pieces per thread per group (32)

  __shared__ __attribute__((aligned(16))) uint16_t xg[CBM][XGP];
  __shared__ __attribute__((aligned(16))) uint16_t es[2][CBN][EP];
  __shared__ __attribute__((aligned(16))) float2 srs[kGroup];  // (s, 1/s) of the group
  __shared__ float red[4][CBN];

  const int64_t G = K / kGroup;
  const int64_t gblocks = (G + gpb - 1) / gpb;
  int64_t L = blockIdx.x;
  const int64_t nt = L % ntiles;
  L /= ntiles;
  const int64_t mt = L % mtiles;
  const int64_t gb = L / mtiles;
  if (gb >= gblocks) return;
  const int64_t m0 = mt * CBM, n0 = nt * CBN;
  const int g0 = (int)(gb * gpb), g1 = (int)((g0 + gpb < G) ? g0 + gpb : G);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wkp = tid % WPPR, wrow0 = tid / WPPR;

  const int64_t xbytes = (M - m0) * ldx * 2, wbytes = (N - n0) * ldw * WSZ;
  const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(X + m0 * ldx), (short)0, (int)(xbytes < 0x7fffffff ? xbytes : 0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const char*>(W) + n0 * ldw * WSZ), (short)0,
      (int)(wbytes < 0x7fffffff ? wbytes : 0x7fffffff), 0x00020000);
  // X piece p (0..31) of this thread: row tid / 16 + 16 p, 16-byte piece tid % 16 of the group
  const int xpc = tid & 15, xr0 = tid >> 4;
  const uint32_t xoff0 = (uint32_t)(xr0 * ldx * 2 + xpc * 16);
  const uint32_t xstep = (uint32_t)(16 * ldx * 2);
  const uint32_t woff0 = (uint32_t)(wrow0 * ldw * WSZ + wkp * 16);
  const uint32_t wstep = (uint32_t)(WROW_STEP * ldw * WSZ);
  bool wlive[WP];
  int64_t prow[WP];
#pragma unroll
  for (int r = 0; r < WP; ++r) {
    const int64_t n = n0 + wrow0 + WROW_STEP * r;
    wlive[r] = n < N;
    prow[r] = wlive[r] ? n : 0;
  }

  f32x16 acc[4][4];
  auto zero_acc = [&]() {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.0f;
  };
  zero_acc();
  const int frow = lane & 31, fk = (lane >> 5) * 8;

  for (int g = g0; g < g1; ++g) {
    const uint32_t kb = (uint32_t)g * kGroup;
    // W of the group, all four chunks, in registers for every candidate
    uint4 wreg[CPG][WP];
#pragma unroll
    for (int j = 0; j < CPG; ++j)
#pragma unroll
      for (int r = 0; r < WP; ++r)
        wreg[j][r] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   wrsrc, (int)(woff0 + r * wstep + (kb + j * KC) * WSZ), 0, 0));
    __syncthreads();  // the previous group's X and scale reads are done
    if (tid < kGroup) srs[tid] = make_float2(s[kb + tid], rs[kb + tid]);
    // X of the group -> LDS, eight pieces in flight per step
#pragma unroll
    for (int h = 0; h < XPG / 8; ++h) {
      uint4 xv[8];
#pragma unroll
      for (int p = 0; p < 8; ++p)
        xv[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              xrsrc, (int)(xoff0 + (8 * h + p) * xstep + kb * 2), 0, 0));
#pragma unroll
      for (int p = 0; p < 8; ++p)
        *reinterpret_cast<uint4*>(&xg[xr0 + 16 * (8 * h + p)][xpc * 8]) = xv[p];
    }
    __syncthreads();

    // Steps t = 4 al + j (candidate al, chunk j): step t multiplies chunk t from E stage t % 2
    // with the matrix instructions issued one at a time, and between them quantizes chunk t+1
    // into the other stage (pinned by sched_barrier), so the vector ALU work runs under the
    // matrix work; one barrier per step.  A candidate's (Delta, z, c) are loaded one candidate
    // ahead.
    struct RowP { float delta, inv, lo, hi, c; };
    auto rowp = [&](const float4& P, int r) {
      RowP q;
      q.delta = wlive[r] ? P.x : 1.0f;  // rows past N: Delta 1, z 0, c 0 and w 0 give e = 0
      const float z = wlive[r] ? P.y : 0.0f;
      q.c = wlive[r] ? P.z : 0.0f;
      q.inv = 1.0f / q.delta;  // correctly rounded
      q.lo = -z;
      q.hi = 15.0f - z;
      return q;
    };
    auto load_params = [&](int al, float4* P) {
#pragma unroll
      for (int r = 0; r < WP; ++r) P[r] = params[((int64_t)al * G + g) * N + prow[r]];
    };
    // element t (0 .. WP*WEL-1) of chunk j: row t / WEL, channel t % WEL of this thread's piece
    auto elem = [&](int j, int t, const RowP* rp, const float* sv, const float* rsv) {
      const int r = t / WEL, k = t % WEL;
      const uint4 u4 = wreg[j][r];
      float w;
      if constexpr (WF32) {
        const uint32_t u = k == 0 ? u4.x : k == 1 ? u4.y : k == 2 ? u4.z : u4.w;
        w = __uint_as_float(u);
      } else {
        const uint32_t u = k < 2 ? u4.x : k < 4 ? u4.y : k < 6 ? u4.z : u4.w;
        w = (k & 1) ? hi16(u) : lo16(u);
      }
      const float v = __builtin_amdgcn_fmed3f(w * sv[k], -rp[r].c, rp[r].c);
      const float q = rintf(exact_quot(v, rp[r].delta, rp[r].inv));
      const float qz = __builtin_amdgcn_fmed3f(q, rp[r].lo, rp[r].hi);
      return fmaf(-(qz * rp[r].delta), rsv[k], w);
    };
    auto store_row = [&](uint16_t (*eb)[EP], int r, const float* e) {
      const int row = wrow0 + WROW_STEP * r;
      uint32_t pk[WEL / 2];
#pragma unroll
      for (int t = 0; t < WEL / 2; ++t) pk[t] = to_bf16x2(e[2 * t], e[2 * t + 1]);
      if constexpr (WEL == 8)
        *reinterpret_cast<uint4*>(&eb[row][wkp * 8]) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      else
        *reinterpret_cast<uint2*>(&eb[row][wkp * 4]) = make_uint2(pk[0], pk[1]);
    };
    auto load_sr = [&](int j, float* sv, float* rsv) {
#pragma unroll
      for (int t = 0; t < WEL; ++t) {
        const float2 p = srs[j * KC + wkp * WEL + t];
        sv[t] = p.x;
        rsv[t] = p.y;
      }
    };
    constexpr int NE = WP * WEL;  // elements per thread per chunk (16)
    float4 PC[WP], PN[WP];
    load_params(0, PC);
    RowP rq[WP];
#pragma unroll
    for (int r = 0; r < WP; ++r) rq[r] = rowp(PC[r], r);
    if (n_clip > 1) load_params(1, PN);
    {  // prologue: chunk 0 of candidate 0
      float sv[WEL], rsv[WEL], e[NE];
      load_sr(0, sv, rsv);
#pragma unroll
      for (int t = 0; t < NE; ++t) e[t] = elem(0, t, rq, sv, rsv);
#pragma unroll
      for (int r = 0; r < WP; ++r) store_row(es[0], r, e + r * WEL);
      __syncthreads();
    }
    // one step: chunk j of candidate al (j known at compile time)
    auto step = [&](int al, auto jc) {
      constexpr int j = decltype(jc)::value;
      constexpr int jn = (j + 1) % CPG;
      const bool more = j + 1 < CPG || al + 1 < n_clip;
      if (jn == 0 && more) {  // the next chunk belongs to the next candidate
#pragma unroll
        for (int r = 0; r < WP; ++r) rq[r] = rowp(PN[r], r);
        if (al + 2 < n_clip) load_params(al + 2, PN);
      }
      uint16_t (*ec)[EP] = es[j & 1];
      uint16_t (*en)[EP] = es[jn & 1];
      float sv[WEL], rsv[WEL], e[NE];
      if (more) load_sr(jn, sv, rsv);
      bf16x8 af[2][4], bfr[2][4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int c = 0; c < 4; ++c) bfr[h][c] = *reinterpret_cast<const bf16x8*>(&ec[c * 32 + frow][h * 16 + fk]);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          af[h][r] = *reinterpret_cast<const bf16x8*>(&xg[wave * 128 + r * 32 + frow][j * KC + h * 16 + fk]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int gi = 0; gi < 32; ++gi) {
        const int h = gi >> 4, r = (gi >> 2) & 3, c = gi & 3;
        acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[h][r], bfr[h][c], acc[r][c], 0, 0, 0);
        // the next chunk's elements, one per matrix instruction from the second on
        if (gi >= 1 && gi <= NE) {
          if (more) {
            e[gi - 1] = elem(jn, gi - 1, rq, sv, rsv);
            asm volatile("" : "+v"(e[gi - 1]));  // keep the element in this slot
            if (gi % WEL == 0) store_row(en, gi / WEL - 1, e + (gi / WEL - 1) * WEL);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (j == CPG - 1) {
        // column sums of Y^2 for (candidate al, group g), as in clip_err_kernel
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float tt = 0.0f;
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int i = 0; i < 16; ++i) tt = fmaf(acc[r][c][i], acc[r][c][i], tt);
          tt += __shfl_xor(tt, 32);
          if (lane < 32) red[wave][c * 32 + lane] = tt;
        }
        zero_acc();
        __syncthreads();
        if (tid < CBN && n0 + tid < N) {
          const float tot = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
          partial[(((int64_t)al * G + g) * mtiles + mt) * N + n0 + tid] = tot;
        }
      }
      // chunk t+1 is complete in its stage, chunk t's stage is free; red is written again
      // only after four more of these barriers
      __syncthreads();
    };
    for (int al = 0; al < n_clip; ++al) {
      step(al, std::integral_constant<int, 0>{});
      step(al, std::integral_constant<int, 1>{});
      step(al, std::integral_constant<int, 2>{});
      step(al, std::integral_constant<int, 3>{});
    }
  }
}

// ---- per (n, g): fixed-order sum over token tiles, mean, first minimum ---------------------
__global__ __launch_bounds__(256) void clip_select_kernel(const float* __restrict__ partial,
                                                          const float4* __restrict__ params, int n_clip,
                                                          int64_t M, int64_t N, int64_t G, int64_t mtiles,
                                                          float* __restrict__ max_val, int32_t* __restrict__ best_out,
                                                          double* __restrict__ err_out,
                                                          uint32_t* __restrict__ flags) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // n * G + g
  if (idx >= N * G) return;
  const int64_t n = idx / G, g = idx % G;
  int best = 0;
  double bl = 0.0;
  bool bad = false;
  for (int i = 0; i < n_clip; ++i) {
    double t = 0.0;
    for (int64_t m = 0; m < mtiles; ++m) t += (double)partial[(((int64_t)i * G + g) * mtiles + m) * N + n];
    const double e = t / (double)M;
    if (!isfinite(e)) bad = true;
    if (err_out) err_out[((int64_t)i * N + n) * G + g] = e;
    if (i == 0 || e < bl) {
      bl = e;
      best = i;
    }
  }
  max_val[idx] = params[((int64_t)best * G + g) * N + n].z;
  if (best_out) best_out[idx] = best;
  if (bad) atomicOr(flags, kFlagNonfiniteLoss);
}

#ifndef AWQ_CLIP_GPB
#define AWQ_CLIP_GPB 4
#endif
// groups per product block: four (16 chunks of work) unless K is smaller
int64_t clip_groups_per_block(int64_t G) { return G < AWQ_CLIP_GPB ? G : AWQ_CLIP_GPB; }

}  // namespace

hipError_t launch_clip(const void* X, bool xf32, int64_t M, int64_t K, int64_t ldx, const void* W,
                       bool wf32, int64_t N, int64_t ldw, const float* s, int n_clip, float* max_val,
                       int32_t* best, double* err, float4* params, float* rs, float* partial,
                       uint32_t* flags, hipStream_t st) {
  const int64_t G = K / kGroup;
  {
    const dim3 grid((unsigned)((N + kClipRows - 1) / kClipRows), (unsigned)G);
    if (wf32)
      clip_range_kernel<true><<<grid, 256, 0, st>>>(W, N, K, ldw, s, n_clip, params, rs, flags);
    else
      clip_range_kernel<false><<<grid, 256, 0, st>>>(W, N, K, ldw, s, n_clip, params, rs, flags);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t mtiles = (M + CBM - 1) / CBM, ntiles = (N + CBN - 1) / CBN;
  if (!xf32) {
    // enough blocks to fill the chip: split the groups so that the blocks number >= 2 per CU
    const int64_t tiles = mtiles * ntiles;
    int64_t gpb = (G * tiles + 511) / 512;
    if (gpb < 1) gpb = 1;
    const int64_t gblocks = (G + gpb - 1) / gpb;
    const unsigned blocks = (unsigned)(tiles * gblocks);
    if (wf32)
      clip_err_group_kernel<true><<<blocks, CTHREADS, 0, st>>>(static_cast<const uint16_t*>(X), M, ldx, W, N, K, ldw, s, rs,
                                                              params, n_clip, mtiles, ntiles, (int)gpb, partial);
    else
      clip_err_group_kernel<false><<<blocks, CTHREADS, 0, st>>>(static_cast<const uint16_t*>(X), M, ldx, W, N, K, ldw, s, rs,
                                                               params, n_clip, mtiles, ntiles, (int)gpb, partial);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    clip_select_kernel<<<(unsigned)((N * G + 255) / 256), 256, 0, st>>>(partial, params, n_clip, M, N, G,
                                                                       mtiles, max_val, best, err, flags);
    return hipGetLastError();
  }
  const int gpb = (int)clip_groups_per_block(G);
  const int64_t gblocks = (G + gpb - 1) / gpb;
  const unsigned blocks = (unsigned)(n_clip * ntiles * mtiles * gblocks);
#define AWQ_CLIP_LAUNCH(XF, WF)                                                                  \
  clip_err_kernel<XF, WF><<<blocks, CTHREADS, 0, st>>>(X, M, ldx, W, N, K, ldw, s, rs, params,   \
                                                       n_clip, mtiles, ntiles, gpb, partial)
  if (xf32 && wf32) AWQ_CLIP_LAUNCH(true, true);
  else if (xf32) AWQ_CLIP_LAUNCH(true, false);
  else if (wf32) AWQ_CLIP_LAUNCH(false, true);
  else AWQ_CLIP_LAUNCH(false, false);
#undef AWQ_CLIP_LAUNCH
  {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  clip_select_kernel<<<(unsigned)((N * G + 255) / 256), 256, 0, st>>>(partial, params, n_clip, M, N, G,
                                                                     mtiles, max_val, best, err, flags);
  return hipGetLastError();
}

}  // namespace awq

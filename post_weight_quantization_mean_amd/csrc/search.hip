// Steps 3 and 4 of the hot path, fused: for one scale candidate, group-wise asymmetric INT4
// quantize-dequantize of S W in registers, the error product Y = X E^T with
// E = W - S^-1 Q(S W) on the matrix cores, and the squared-error reduction of Y
// ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §1: the weight error is measured through
// the input, E_W = W - What; §3: equivalent scaling XW = (XS^-1)(SW); §4: every candidate
// scales the weight, pseudo-quantizes, divides the scale back and compares the module output;
// §7: round v/Delta, add z, clamp to [0, 15], reconstruct Delta (q - z)).
//
// One workgroup = one (512 tokens x 128 output channels) output tile for one candidate.
// The K loop walks chunks of 32 input channels (16 when X is fp32).  Per chunk:
//   * X[512 x 32] is copied to LDS as bf16 (fp32 X is split into bf16 hi + lo terms, so the
//     product keeps ~16 mantissa bits of X);
//   * W[128 x 32] is read once, quantized with that candidate's scales and its group ranges
//     (Delta, z precomputed per (candidate, channel, group) by the range pass), and the error
//     e = w - Delta (q - z) / s is rounded to bf16 and written to LDS.  The dequantized
//     weights never reach HBM;
//   * four waves each run a 128 x 128 slab of v_mfma_f32_32x32x16_bf16 from LDS.
// LDS is double buffered, so the next chunk's global loads are in flight during the current
// chunk's matrix work, and one barrier per chunk orders the two buffers.  At the end each
// lane squares its 256 accumulators (fp32 per 32x32 tile, fp64 across tiles) and the block
// writes one fp64 partial; a separate kernel sums partials in a fixed order.
//
// Block order is XCD-aware: the hardware places workgroup b on XCD b % 8, so logical index
// L = (b % 8) * ceil(G/8) + b / 8 gives every XCD a contiguous run of L.  L runs candidate-
// fastest, so the ~32 blocks resident on one XCD share the same X rows and W rows in its L2.
#include "awq_internal.h"

namespace awq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = kSearchBM;      // 512 tokens
constexpr int BN = kSearchBN;      // 128 output channels
constexpr int THREADS = 256;       // 4 waves, one per SIMD
constexpr int WAVE_ROWS = BM / 4;  // 128 tokens per wave

template <bool XF32, bool WF32>
struct Geo {
  static constexpr int KC = XF32 ? 16 : 32;     // input channels per chunk
  static constexpr int PITCH = KC + 8;          // LDS row pitch in bf16 (16-byte pad)
  static constexpr int XPARTS = XF32 ? 2 : 1;   // bf16 terms of X
  static constexpr int XEL = XF32 ? 4 : 8;      // X elements per 16-byte piece
  static constexpr int XPPR = KC / XEL;         // X pieces per row per chunk (4)
  static constexpr int XP = BM * XPPR / THREADS;  // X pieces per thread (8)
  static constexpr int WEL = WF32 ? 4 : 8;      // W elements per 16-byte piece
  static constexpr int WPPR = KC / WEL;         // W pieces per row per chunk
  static constexpr int WP = BN * WPPR / THREADS;  // W pieces per thread
  static constexpr int WROW_STEP = THREADS / WPPR;  // row distance between a thread's pieces
  static_assert(XPPR == 4, "X piece layout");
  static_assert(WP >= 1, "W piece layout");
};

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 h = __builtin_convertvector((f32x2){a, b}, bf16x2);  // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

template <bool XF32, bool WF32>
__global__ __launch_bounds__(THREADS, 1) void search_fused_kernel(
    const void* __restrict__ X, int64_t M, int64_t ldx, const void* __restrict__ W, int64_t N,
    int64_t K, int64_t ldw, const float* __restrict__ s_tab, const float* __restrict__ rs_tab,
    const float2* __restrict__ params, int n_grid, int64_t nt_count, int64_t tiles,
    int64_t per_xcd, double* __restrict__ partial) {
  using Gm = Geo<XF32, WF32>;
  constexpr int KC = Gm::KC;
  constexpr int PITCH = Gm::PITCH;
  constexpr int XPARTS = Gm::XPARTS;
  constexpr int XP = Gm::XP;
  constexpr int WP = Gm::WP;
  constexpr int WEL = Gm::WEL;

  __shared__ __attribute__((aligned(16))) uint16_t xs[2][XPARTS][BM][PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t es[2][BN][PITCH];
  __shared__ double red[4];

  const int64_t b = blockIdx.x;
  const int64_t L = (b & 7) * per_xcd + (b >> 3);
  if (L >= tiles * n_grid) return;
  const int64_t tile = L / n_grid;
  const int al = (int)(L - tile * n_grid);
  const int64_t m0 = (tile / nt_count) * BM;
  const int64_t n0 = (tile % nt_count) * BN;
  const int64_t G = K / kGroup;
  const int64_t nchunks = K / KC;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ---- this thread's pieces -------------------------------------------------------------
  const int xkp = tid & 3;     // X: piece column within the chunk row
  const int xrow0 = tid >> 2;  // X rows xrow0 + 64 i
  const int wkp = tid % Gm::WPPR;
  const int wrow0 = tid / Gm::WPPR;  // W rows wrow0 + WROW_STEP i
  constexpr int XSZ = XF32 ? 4 : 2;
  constexpr int WSZ = WF32 ? 4 : 2;

  // Buffer resources rebased at this tile: rows past M (or N) fall outside num_records and
  // read as zero, so tail tiles need no branches.  Offsets stay below 2^31 (host-checked).
  const int64_t xrows = M - m0, wrows = N - n0;
  const int64_t xbytes = xrows * ldx * XSZ, wbytes = wrows * ldw * WSZ;
  const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const char*>(X) + m0 * ldx * XSZ), (short)0,
      (int)(xbytes < 0x7fffffff ? xbytes : 0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const char*>(W) + n0 * ldw * WSZ), (short)0,
      (int)(wbytes < 0x7fffffff ? wbytes : 0x7fffffff), 0x00020000);
  const uint32_t xoff0 = (uint32_t)(xrow0 * ldx * XSZ + xkp * 16);
  const uint32_t xstep = (uint32_t)(64 * ldx * XSZ);
  const uint32_t woff0 = (uint32_t)(wrow0 * ldw * WSZ + wkp * 16);
  const uint32_t wstep = (uint32_t)(Gm::WROW_STEP * ldw * WSZ);

  const float* srow = s_tab + (int64_t)al * K + wkp * WEL;
  const float* rsrow = rs_tab + (int64_t)al * K + wkp * WEL;
  // group ranges of this thread's W rows (rows past N read row N-1 and are masked)
  const float2* prow[WP];
  bool wlive[WP];
#pragma unroll
  for (int i = 0; i < WP; ++i) {
    const int64_t n = n0 + wrow0 + Gm::WROW_STEP * i;
    wlive[i] = n < N;
    prow[i] = params + ((int64_t)al * N + (wlive[i] ? n : N - 1)) * G;
  }

  uint4 xr[XP];
  uint4 wr[WP];
  float4 sr[WEL / 4], rsr[WEL / 4];
  float2 pr[WP];

  // Global -> registers only; nothing loaded here is used until store_chunk, so the loads of
  // chunk c+1 stay in flight while chunk c runs on the matrix cores.
  auto load_chunk = [&](int64_t c) {
    const uint32_t k0b = (uint32_t)(c * KC);
#pragma unroll
    for (int i = 0; i < XP; ++i)
      xr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            xrsrc, (int)(xoff0 + i * xstep + k0b * XSZ), 0, 0));
#pragma unroll
    for (int i = 0; i < WP; ++i)
      wr[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                            wrsrc, (int)(woff0 + i * wstep + k0b * WSZ), 0, 0));
#pragma unroll
    for (int q = 0; q < WEL / 4; ++q) {
      sr[q] = *reinterpret_cast<const float4*>(srow + k0b + 4 * q);
      rsr[q] = *reinterpret_cast<const float4*>(rsrow + k0b + 4 * q);
    }
    const uint32_t g = k0b / kGroup;
#pragma unroll
    for (int i = 0; i < WP; ++i) pr[i] = prow[i][g];
  };

  auto store_chunk = [&](int buf) {
    // X -> LDS (bf16, or bf16 hi + lo for fp32 X)
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int row = xrow0 + 64 * i;
      if constexpr (XF32) {
        const float f[4] = {__uint_as_float(xr[i].x), __uint_as_float(xr[i].y),
                            __uint_as_float(xr[i].z), __uint_as_float(xr[i].w)};
        uint32_t hi2[2], lo2[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const bf16x2 h = __builtin_convertvector((f32x2){f[2 * q], f[2 * q + 1]}, bf16x2);
          const f32x2 hf = __builtin_convertvector(h, f32x2);
          hi2[q] = __builtin_bit_cast(uint32_t, h);
          lo2[q] = pack_bf16x2(f[2 * q] - hf.x, f[2 * q + 1] - hf.y);
        }
        *reinterpret_cast<uint2*>(&xs[buf][0][row][xkp * 4]) = make_uint2(hi2[0], hi2[1]);
        *reinterpret_cast<uint2*>(&xs[buf][1][row][xkp * 4]) = make_uint2(lo2[0], lo2[1]);
      } else {
        *reinterpret_cast<uint4*>(&xs[buf][0][row][xkp * 8]) = xr[i];
      }
    }
    float sv[WEL], rsv[WEL];
#pragma unroll
    for (int q = 0; q < WEL / 4; ++q) {
      sv[4 * q + 0] = sr[q].x; sv[4 * q + 1] = sr[q].y; sv[4 * q + 2] = sr[q].z; sv[4 * q + 3] = sr[q].w;
      rsv[4 * q + 0] = rsr[q].x; rsv[4 * q + 1] = rsr[q].y; rsv[4 * q + 2] = rsr[q].z; rsv[4 * q + 3] = rsr[q].w;
    }
    // W -> qdq -> E (bf16) -> LDS
#pragma unroll
    for (int i = 0; i < WP; ++i) {
      const int row = wrow0 + Gm::WROW_STEP * i;
      // rows past N: Delta = 1, z = 0 and w = 0 give e = 0 exactly
      const float delta = wlive[i] ? pr[i].x : 1.0f;
      const float z = wlive[i] ? pr[i].y : 0.0f;
      const float inv = __builtin_amdgcn_rcpf(delta);  // search only; pack divides exactly
      const float lo = -z, hi = 15.0f - z;
      float w[WEL];
      if constexpr (WF32) {
        w[0] = __uint_as_float(wr[i].x); w[1] = __uint_as_float(wr[i].y);
        w[2] = __uint_as_float(wr[i].z); w[3] = __uint_as_float(wr[i].w);
      } else {
        const uint32_t u[4] = {wr[i].x, wr[i].y, wr[i].z, wr[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          w[2 * q] = bf16_lo(u[q]);
          w[2 * q + 1] = bf16_hi(u[q]);
        }
      }
      float e[WEL];
#pragma unroll
      for (int j = 0; j < WEL; ++j) {
        const float v = w[j] * sv[j];                            // S W
        const float r = rintf(v * inv);                          // rne(v / Delta)
        const float qz = __builtin_amdgcn_fmed3f(r, lo, hi);     // clamp(r + z, 0, 15) - z
        const float d = qz * delta;                              // Delta (q - z)
        e[j] = fmaf(-d, rsv[j], w[j]);                           // w - Delta (q - z) / s
      }
      uint32_t pk[WEL / 2];
#pragma unroll
      for (int q = 0; q < WEL / 2; ++q) pk[q] = pack_bf16x2(e[2 * q], e[2 * q + 1]);
      if constexpr (WEL == 8)
        *reinterpret_cast<uint4*>(&es[buf][row][wkp * 8]) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      else
        *reinterpret_cast<uint2*>(&es[buf][row][wkp * 4]) = make_uint2(pk[0], pk[1]);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.0f;

  const int frow = lane & 31;
  const int fk = (lane >> 5) * 8;

  auto mfma_chunk = [&](int buf) {
#pragma unroll
    for (int j = 0; j < KC / 16; ++j) {
      bf16x8 bfr[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        bfr[c] = *reinterpret_cast<const bf16x8*>(&es[buf][c * 32 + frow][j * 16 + fk]);
#pragma unroll
      for (int p = 0; p < XPARTS; ++p) {
        bf16x8 afr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          afr[r] = *reinterpret_cast<const bf16x8*>(
              &xs[buf][p][wave * WAVE_ROWS + r * 32 + frow][j * 16 + fk]);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[r], bfr[c], acc[r][c], 0, 0, 0);
      }
    }
  };

  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int64_t c = 0; c < nchunks; ++c) {
    const int buf = (int)(c & 1);
    // The last iteration reloads and restages its own chunk into the idle buffer; keeping
    // the body free of branches lets the scheduler interleave the quantization VALU work
    // with the matrix instructions.
    load_chunk(c + 1 < nchunks ? c + 1 : c);
    mfma_chunk(buf);
    store_chunk(buf ^ 1);
    __syncthreads();
  }

  // ---- squared error of this tile ----------------------------------------------------------
  double ss = 0.0;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float t = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) t = fmaf(acc[r][c][i], acc[r][c][i], t);
      ss += (double)t;
    }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  if (tid == 0) partial[(int64_t)al * tiles + tile] = ((red[0] + red[1]) + red[2]) + red[3];
}


// ---- pipelined kernel for bf16 X and bf16 W (the production path) ----------------------
// Same tile and arithmetic as above; the K loop is software-pipelined:
//   * X chunks go global -> LDS directly (buffer_load ... lds), two chunks ahead, into four
//     LDS stages; no VGPRs or ds_write instructions are spent on X;
//   * W chunks (and their scales, reciprocals and group ranges) are loaded into registers
//     two chunks ahead, alternating between two register sets;
//   * iteration c runs the matrix instructions of chunk c while the VALU quantizes chunk
//     c+1 into the other E stage, so the two overlap on each SIMD.
// LDS tiles are unpadded [rows][32 bf16] with the four 16-byte slots of a row permuted by
// swz(row) = ((row >> 1) ^ (row >> 3)) & 3, which spreads the 32 rows of an MFMA fragment
// read over all banks.  The loop is unrolled by 4 (4 X stages, 2 E stages, 2 register sets)
// so every stage is a distinct LDS object and the compiler's wait counters stay exact.
// Each wave waits for its own chunk-(c+1) DMA before the barrier that ends iteration c, so
// after the barrier every wave may read rows that other waves fetched.
#define AWQ_LDS __attribute__((address_space(3)))

constexpr int PKC = 32;           // input channels per chunk
constexpr int PROW = PKC * 2;     // bytes per LDS row
constexpr int XSTAGE = BM * PROW; // 32 KiB
constexpr int ESTAGE = BN * PROW; // 8 KiB

__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

struct WSet {
  uint4 w[2];
  float4 s[2], rs[2];
  float2 p[2];
};

__global__ __launch_bounds__(THREADS, 1) void search_pipelined_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t ldx, const uint16_t* __restrict__ W,
    int64_t N, int64_t K, int64_t ldw, const float* __restrict__ s_tab,
    const float* __restrict__ rs_tab, const float2* __restrict__ params, int n_grid,
    int64_t nt_count, int64_t tiles, int64_t per_xcd, double* __restrict__ partial) {
  __shared__ __attribute__((aligned(1024))) uint8_t xs0[XSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs1[XSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs2[XSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs3[XSTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t es0[ESTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t es1[ESTAGE];
  __shared__ double red[4];

  const int64_t b = blockIdx.x;
  const int64_t L = (b & 7) * per_xcd + (b >> 3);
  if (L >= tiles * n_grid) return;
  const int64_t tile = L / n_grid;
  const int al = (int)(L - tile * n_grid);
  const int64_t m0 = (tile / nt_count) * BM;
  const int64_t n0 = (tile % nt_count) * BN;
  const int64_t G = K / kGroup;
  const int nchunks = (int)(K / PKC);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // X: DMA instruction i of this wave fills LDS rows (4 i + wave) * 16 + lane / 4, slot
  // lane % 4, with global piece kp = slot ^ swz(row).
  const int64_t xrows = M - m0, wrows = N - n0;
  const int64_t xbytes = xrows * ldx * 2, wbytes = wrows * ldw * 2;
  const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(X + m0 * ldx), (short)0, (int)(xbytes < 0x7fffffff ? xbytes : 0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + n0 * ldw), (short)0, (int)(wbytes < 0x7fffffff ? wbytes : 0x7fffffff), 0x00020000);
  uint32_t xoff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = (4 * i + wave) * 16 + (lane >> 2);
    const int kp = (lane & 3) ^ swz(row);
    xoff[i] = (uint32_t)(row * ldx * 2 + kp * 16);
  }
  // W: thread owns rows wrow0 and wrow0 + 64, piece wkp (8 channels)
  const int wkp = tid & 3;
  const int wrow0 = tid >> 2;
  const uint32_t woff0 = (uint32_t)(wrow0 * ldw * 2 + wkp * 16);
  const uint32_t woff1 = (uint32_t)((wrow0 + 64) * ldw * 2 + wkp * 16);
  const int eslot0 = (wrow0 * PROW) + ((wkp ^ swz(wrow0)) * 16);
  const int eslot1 = ((wrow0 + 64) * PROW) + ((wkp ^ swz(wrow0 + 64)) * 16);
  const float* srow = s_tab + (int64_t)al * K + wkp * 8;
  const float* rsrow = rs_tab + (int64_t)al * K + wkp * 8;
  const bool live0 = n0 + wrow0 < N, live1 = n0 + wrow0 + 64 < N;
  const float2* prow0 = params + ((int64_t)al * N + (live0 ? n0 + wrow0 : N - 1)) * G;
  const float2* prow1 = params + ((int64_t)al * N + (live1 ? n0 + wrow0 + 64 : N - 1)) * G;

  // fragment reads: lane reads row (.. + fr), slot (2 j + fh) ^ swz(fr)
  const int fr = lane & 31, fh = lane >> 5;
  const int fsw = swz(fr);
  const int foff0 = fr * PROW + (((0 + fh) ^ fsw) * 16);
  const int foff1 = fr * PROW + (((2 + fh) ^ fsw) * 16);
  const int xwave = wave * WAVE_ROWS * PROW;

  auto dma_x = [&](uint8_t* stage, int c) {
    const uint32_t kb = (uint32_t)c * (PKC * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xrsrc, (AWQ_LDS void*)(stage + (4 * i + wave) * 1024), 16, (int)(xoff[i] + kb), 0, 0, 0);
  };
  auto load_w = [&](WSet& S, int c) {
    const uint32_t kb = (uint32_t)c * (PKC * 2);
    S.w[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, (int)(woff0 + kb), 0, 0));
    S.w[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, (int)(woff1 + kb), 0, 0));
    const int k0 = c * PKC;
    S.s[0] = *reinterpret_cast<const float4*>(srow + k0);
    S.s[1] = *reinterpret_cast<const float4*>(srow + k0 + 4);
    S.rs[0] = *reinterpret_cast<const float4*>(rsrow + k0);
    S.rs[1] = *reinterpret_cast<const float4*>(rsrow + k0 + 4);
    const int g = k0 / kGroup;
    S.p[0] = prow0[g];
    S.p[1] = prow1[g];
  };
  auto qdq_store = [&](const WSet& S, uint8_t* estage) {
    const float sv[8] = {S.s[0].x, S.s[0].y, S.s[0].z, S.s[0].w, S.s[1].x, S.s[1].y, S.s[1].z, S.s[1].w};
    const float rv[8] = {S.rs[0].x, S.rs[0].y, S.rs[0].z, S.rs[0].w,
                         S.rs[1].x, S.rs[1].y, S.rs[1].z, S.rs[1].w};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const bool live = i == 0 ? live0 : live1;
      const float delta = live ? S.p[i].x : 1.0f;  // rows past N: e = 0 exactly
      const float z = live ? S.p[i].y : 0.0f;
      const float inv = __builtin_amdgcn_rcpf(delta);
      const float lo = -z, hi = 15.0f - z;
      const uint32_t u[4] = {S.w[i].x, S.w[i].y, S.w[i].z, S.w[i].w};
      uint32_t pk[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float e2[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = 2 * q + h;
          const float w = h == 0 ? bf16_lo(u[q]) : bf16_hi(u[q]);
          const float v = w * sv[j];                                // S W
          const float r = rintf(v * inv);                           // rne(v / Delta)
          const float qz = __builtin_amdgcn_fmed3f(r, lo, hi);      // clamp(r + z, 0, 15) - z
          e2[h] = fmaf(-(qz * delta), rv[j], w);                    // w - Delta (q - z) / s
        }
        pk[q] = pack_bf16x2(e2[0], e2[1]);
      }
      *reinterpret_cast<uint4*>(estage + (i == 0 ? eslot0 : eslot1)) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.0f;

  auto mfma_chunk = [&](const uint8_t* xst, const uint8_t* est) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int fo = j == 0 ? foff0 : foff1;
      bf16x8 bfr[4], afr[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) bfr[c] = *reinterpret_cast<const bf16x8*>(est + c * 32 * PROW + fo);
#pragma unroll
      for (int r = 0; r < 4; ++r) afr[r] = *reinterpret_cast<const bf16x8*>(xst + xwave + r * 32 * PROW + fo);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[r][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[r], bfr[c], acc[r][c], 0, 0, 0);
    }
  };

  // vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
  // lgkmcnt[11:8] | vmcnt[5:4] at [15:14]); n = 16 = loads issued per iteration.
  constexpr int kLoadsPerIter = 8 + 2 + 4 + 2;
  constexpr int kWaitVm = (kLoadsPerIter & 0xf) | (0x7 << 4) | (0xf << 8) | ((kLoadsPerIter >> 4) << 14);
  constexpr int kWaitLgkm0 = 0xf | (0x7 << 4) | (0x0 << 8) | (0x3 << 14);

  WSet A, B;
  // Prologue: W(0), X(0), W(1), X(1) in flight; chunk 0 quantized into E stage 0.  Every
  // step then issues W(c+2) before X(c+2), so at the end of step c exactly the 16 loads of
  // that step were issued after X(c+1): vmcnt(16) means this wave's X(c+1) has landed.
  load_w(A, 0);
  dma_x(xs0, 0);
  load_w(B, 1);
  dma_x(xs1, 1);
  qdq_store(A, es0);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kWaitVm);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // One pipeline step: matrix work of chunk c from (xc, ec); quantize chunk c+1 from `next`
  // into en; prefetch chunk c+2 into `fill` and xn.  Past the end the prefetch repeats the
  // last chunk into stages nobody reads again.
  auto step = [&](int c, const uint8_t* xc, uint8_t* xn, const uint8_t* ec, uint8_t* en,
                  const WSet& next, WSet& fill) {
    const int cp = c + 2 < nchunks ? c + 2 : nchunks - 1;
    load_w(fill, cp);
    dma_x(xn, cp);
    mfma_chunk(xc, ec);
    qdq_store(next, en);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVm);  // this wave's chunk c+1 DMA has landed
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // nchunks = K / 32 is a multiple of 4 (K is a multiple of 128)
  for (int c = 0; c < nchunks; c += 4) {
    step(c + 0, xs0, xs2, es0, es1, B, A);
    step(c + 1, xs1, xs3, es1, es0, A, B);
    step(c + 2, xs2, xs0, es0, es1, B, A);
    step(c + 3, xs3, xs1, es1, es0, A, B);
  }

  double ss = 0.0;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float t = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) t = fmaf(acc[r][c][i], acc[r][c][i], t);
      ss += (double)t;
    }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  if (tid == 0) partial[(int64_t)al * tiles + tile] = ((red[0] + red[1]) + red[2]) + red[3];
}

}  // namespace

SearchPlan search_plan(int64_t M, int64_t K, int64_t N, int n_grid) {
  SearchPlan p;
  p.mt = (M + BM - 1) / BM;
  p.nt = (N + BN - 1) / BN;
  p.tiles = p.mt * p.nt;
  const int64_t total = p.tiles * n_grid;
  p.blocks = ((total + 7) / 8) * 8;
  p.groups = K / kGroup;
  return p;
}

hipError_t launch_search_fused(const void* X, bool xf32, int64_t M, int64_t ldx, const void* W,
                               bool wf32, int64_t N, int64_t K, int64_t ldw, const float* s_tab,
                               const float* rs_tab, const float2* params, int n_grid,
                               const SearchPlan& plan, double* partial, hipStream_t st) {
  const int64_t per_xcd = plan.blocks / 8;
  const dim3 grid((unsigned)plan.blocks);
#define AWQ_LAUNCH(XF, WF)                                                                      \
  search_fused_kernel<XF, WF><<<grid, THREADS, 0, st>>>(X, M, ldx, W, N, K, ldw, s_tab, rs_tab, \
                                                        params, n_grid, plan.nt, plan.tiles,    \
                                                        per_xcd, partial)
  if (!xf32 && !wf32) {
    search_pipelined_kernel<<<grid, THREADS, 0, st>>>(
        static_cast<const uint16_t*>(X), M, ldx, static_cast<const uint16_t*>(W), N, K, ldw, s_tab,
        rs_tab, params, n_grid, plan.nt, plan.tiles, per_xcd, partial);
    return hipGetLastError();
  }
  if (xf32 && wf32)
    AWQ_LAUNCH(true, true);
  else if (xf32)
    AWQ_LAUNCH(true, false);
  else if (wf32)
    AWQ_LAUNCH(false, true);
  else
    AWQ_LAUNCH(false, false);
#undef AWQ_LAUNCH
  return hipGetLastError();
}

}  // namespace awq

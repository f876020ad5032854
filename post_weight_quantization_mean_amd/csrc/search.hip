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
  const int64_t NP = padded_n(N);
  const float2* prow[WP];  // this thread's rows in the range table of candidate al
  bool wlive[WP];
#pragma unroll
  for (int i = 0; i < WP; ++i) {
    const int64_t n = n0 + wrow0 + Gm::WROW_STEP * i;  // < NP (tiles never pass NP)
    wlive[i] = n < N;
    prow[i] = params + (int64_t)al * G * NP + range_slot(n);
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
    for (int i = 0; i < WP; ++i) pr[i] = prow[i][g * NP];
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
// Same tile and arithmetic as above; the K loop is software-pipelined three chunks deep:
//   * X chunks go global -> LDS directly (buffer_load ... lds) into four LDS stages; no
//     VGPRs or ds_write instructions are spent on X;
//   * wave w quantizes the 8-channel piece w of every chunk, for rows `lane` and `lane + 64`:
//     its W words and group ranges come in through two and one 16-byte vector loads; the
//     chunk's 32 (s, 1/s) pairs come in through one 4-byte-per-lane load of an interleaved
//     table and reach SGPRs with v_readlane (scalar loads would share lgkmcnt with LDS and
//     turn every fragment wait into a full drain);
//   * step c issues the 32 matrix instructions of chunk c one by one, and behind each the
//     VALU work of quantizing chunk c+1 (one element every other MFMA), the prefetch loads
//     of chunk c+3 and the second-half fragment reads; sched_barrier pins that order so the
//     matrix core, the VALU and the memory pipes run concurrently on each SIMD.
// Measured on the 4096^3 layer, the vector-memory address path is the scarce resource, so
// every wave issues 12 vector loads per chunk (8 X DMA, 2 W, 1 group range, 1 scale pair),
// spread one per two matrix instructions.
// LDS tiles are unpadded [rows][32 bf16] with the four 16-byte slots of a row permuted by
// swz(row) = (row >> 2) & 3; with it the 32-row MFMA fragment reads (ds_read_b128) measure
// zero bank-conflict cycles on gfx950, where unswizzled 64-byte rows cost 12 per read.
// The loop is unrolled by 4 (4 X stages, 2 E stages, 4 register sets) so every stage is a
// distinct LDS object and the compiler's wait counters stay exact.  Each wave waits for its
// own chunk-(c+1) DMA before the barrier that ends step c, so after the barrier every wave
// may read rows that other waves fetched.
#define AWQ_LDS __attribute__((address_space(3)))

constexpr int PKC = 32;            // input channels per chunk
constexpr int PROW = PKC * 2;      // bytes per LDS row
constexpr int XSTAGE = BM * PROW;  // 32 KiB
constexpr int ESTAGE = BN * PROW;  // 8 KiB

__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

struct WSet {
  uint4 w[2];   // 8 bf16 channels of rows lane and lane + 64
  float4 p;     // (Delta, z) of row lane, then of row lane + 64, for this chunk's group
  float sr;     // lane l holds s (l even) or 1/s (l odd) of channel l / 2 of the chunk
};
struct SVal {
  float s[8];   // wave-uniform (SGPRs, via v_readlane): s of this wave's 8 channels
  float rs[8];  // 1 / s
};

struct RowQ {
  float delta, inv, lo, hi;
};

__global__ __launch_bounds__(THREADS, 1) void search_pipelined_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t ldx, const uint16_t* __restrict__ W,
    int64_t N, int64_t K, int64_t ldw, const float* __restrict__ s_tab,
    const float* __restrict__ rs_tab, const float2* __restrict__ sr_tab,
    const float2* __restrict__ params, int n_grid, int64_t nt_count, int64_t tiles,
    int64_t per_xcd, double* __restrict__ partial) {
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
  const int64_t NP = padded_n(N);
  const int nchunks = (int)(K / PKC);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // X: DMA instruction i of this wave fills LDS rows (4 i + wave) * 16 + lane / 4, slot
  // lane % 4, with the global piece kp = slot ^ swz(row).  Buffer resources are rebased at
  // this tile so rows past M (or N) read as zero; offsets stay below 2^31 (host-checked).
  const int64_t xbytes = (M - m0) * ldx * 2, wbytes = (N - n0) * ldw * 2;
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
  // W side: this wave's piece is channels 8 wave .. 8 wave + 7 of each chunk
  const uint32_t woff0 = (uint32_t)(lane * ldw * 2 + wave * 16);
  const uint32_t woff1 = (uint32_t)((lane + 64) * ldw * 2 + wave * 16);
  const int eslot0 = lane * PROW + ((wave ^ swz(lane)) * 16);
  const int eslot1 = (lane + 64) * PROW + ((wave ^ swz(lane + 64)) * 16);
  const bool live0 = n0 + lane < N, live1 = n0 + lane + 64 < N;
  const float* srbase = reinterpret_cast<const float*>(sr_tab) + (int64_t)al * K * 2 + lane;
  // ranges of rows lane and lane + 64 are adjacent (range_slot); rows past N are masked
  const float4* pbase = reinterpret_cast<const float4*>(params + (int64_t)al * G * NP + n0 + 2 * lane);

  // fragment reads: lane reads row (... + fr), slot (2 j + fh) ^ swz(fr)
  const int fr = lane & 31, fh = lane >> 5;
  const int fsw = swz(fr);
  const int foff0 = fr * PROW + (((0 + fh) ^ fsw) * 16);
  const int foff1 = fr * PROW + (((2 + fh) ^ fsw) * 16);
  const int xwave = wave * WAVE_ROWS * PROW;

  auto dma_x_one = [&](uint8_t* stage, int i, uint32_t kb) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xrsrc, (AWQ_LDS void*)(stage + (4 * i + wave) * 1024), 16,
                                             (int)(xoff[i] + kb), 0, 0, 0);
  };
  auto load_w0 = [&](WSet& S, uint32_t kb) {
    S.w[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, (int)(woff0 + kb), 0, 0));
  };
  auto load_w1 = [&](WSet& S, uint32_t kb) {
    S.w[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, (int)(woff1 + kb), 0, 0));
  };
  auto load_p = [&](WSet& S, int k0) { S.p = pbase[(int64_t)(k0 / kGroup) * (NP / 2)]; };
  auto load_sr = [&](WSet& S, int k0) { S.sr = srbase[2 * k0]; };
  auto get_s = [&](const WSet& S) {
    SVal v;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v.s[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(S.sr), 16 * wave + 2 * j));
      v.rs[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(S.sr), 16 * wave + 2 * j + 1));
    }
    return v;
  };
  auto load_all = [&](WSet& S, uint8_t* stage, int c) {
    const uint32_t kb = (uint32_t)c * (PKC * 2);
    load_sr(S, c * PKC);
    load_w0(S, kb);
    load_w1(S, kb);
    load_p(S, c * PKC);
#pragma unroll
    for (int i = 0; i < 8; ++i) dma_x_one(stage, i, kb);
  };
  auto row_setup = [&](const WSet& S, int i) {
    const bool live = i == 0 ? live0 : live1;
    RowQ q;
    q.delta = live ? (i == 0 ? S.p.x : S.p.z) : 1.0f;  // rows past N: Delta 1, z 0, w 0: e = 0
    const float z = live ? (i == 0 ? S.p.y : S.p.w) : 0.0f;
    q.inv = __builtin_amdgcn_rcpf(q.delta);  // search only; the pack divides exactly
    q.lo = -z;
    q.hi = 15.0f - z;
    return q;
  };
  // e = w - Delta (q - z) / s for channel j (0..7) of row i (0/1)
  auto elem = [&](const WSet& S, const SVal& T, const RowQ& q, int i, int j) {
    const uint4& w4 = S.w[i];
    const uint32_t u = j < 2 ? w4.x : j < 4 ? w4.y : j < 6 ? w4.z : w4.w;
    const float w = (j & 1) ? bf16_hi(u) : bf16_lo(u);
    const float v = w * T.s[j];                               // S W
    const float r = rintf(v * q.inv);                         // rne(v / Delta)
    const float qz = __builtin_amdgcn_fmed3f(r, q.lo, q.hi);  // clamp(r + z, 0, 15) - z
    return fmaf(-(qz * q.delta), T.rs[j], w);                 // w - Delta (q - z) / s
  };
  auto store_piece = [&](uint8_t* estage, int slot, const float* e8) {
    uint32_t pk[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) pk[h] = pack_bf16x2(e8[2 * h], e8[2 * h + 1]);
    *reinterpret_cast<uint4*>(estage + slot) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  };
  auto frag = [&](const uint8_t* base, int fo) { return *reinterpret_cast<const bf16x8*>(base + fo); };

  f32x16 acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[r][c][i] = 0.0f;

  // vmcnt(n) with the other counters left alone (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
  // lgkmcnt[11:8] | vmcnt[5:4] at [15:14]); n = 24 = vector loads issued by two steps.
  constexpr int kLoadsPerStep = 1 + 2 + 1 + 8;
  constexpr int kPending = 2 * kLoadsPerStep;
  constexpr int kWaitVm = (kPending & 0xf) | (0x7 << 4) | (0xf << 8) | ((kPending >> 4) << 14);
  constexpr int kWaitLgkm0 = 0xf | (0x7 << 4) | (0x0 << 8) | (0x3 << 14);

  WSet S0, S1, S2, S3;  // three chunks ahead
  // Prologue: chunks 0, 1 and 2 in flight (the X DMA last in each), chunk 0 quantized into
  // E stage 0.  Every step c then issues the 12 vector loads of chunk c+3, X DMA last, so at
  // the end of step c vmcnt(24) means this wave's X DMA of chunk c+1 has landed.
  load_all(S0, xs0, 0);
  load_all(S1, xs1, 1);
  load_all(S2, xs2, 2);
  {
    float e[8];
    const SVal T0 = get_s(S0);
    const RowQ q0 = row_setup(S0, 0), q1 = row_setup(S0, 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = elem(S0, T0, q0, 0, j);
    store_piece(es0, eslot0, e);
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = elem(S0, T0, q1, 1, j);
    store_piece(es0, eslot1, e);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(kWaitVm);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // One pipeline step, hand-scheduled in 32 groups, one per matrix instruction of chunk c.
  // Group g: MFMA g; in odd groups one element of the quantization of chunk c+1; in groups
  // 0-7 one second-half fragment read; in even groups 0-22 one prefetch load of chunk c+3
  // (scales, W words, group ranges, then the 8 X DMA), so no group carries more than one
  // vector-memory instruction behind its 32-cycle MFMA.
  auto step = [&](int c, const uint8_t* xc, uint8_t* xn, const uint8_t* ec, uint8_t* en,
                  const WSet& next, WSet& fill) {
    const int cp = c + 3 < nchunks ? c + 3 : nchunks - 1;  // past the end: harmless reload
    const uint32_t kb = (uint32_t)cp * (PKC * 2);
    const int k0 = cp * PKC;
    const uint8_t* xw = xc + xwave;
    bf16x8 a0[4], b0[4], a1[4], b1[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      a0[t] = frag(xw + t * 32 * PROW, foff0);
      b0[t] = frag(ec + t * 32 * PROW, foff0);
    }
    const SVal tv = get_s(next);
    const RowQ q0 = row_setup(next, 0);
    const RowQ q1 = row_setup(next, 1);
    __builtin_amdgcn_sched_barrier(0);
    float e[16];
#pragma unroll
    for (int g = 0; g < 32; ++g) {
      const int r = (g >> 2) & 3, cc = g & 3;
      if (g < 16)
        acc[r][cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[r], b0[cc], acc[r][cc], 0, 0, 0);
      else
        acc[r][cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[r], b1[cc], acc[r][cc], 0, 0, 0);
      if (g & 1) {
        const int el = g >> 1;
        e[el] = el < 8 ? elem(next, tv, q0, 0, el) : elem(next, tv, q1, 1, el - 8);
        asm volatile("" : "+v"(e[el]));  // keep the element in this group (no IR sinking)
      }
      if (g < 8) {
        if (g & 1)
          b1[g >> 1] = frag(ec + (g >> 1) * 32 * PROW, foff1);
        else
          a1[g >> 1] = frag(xw + (g >> 1) * 32 * PROW, foff1);
      }
      if (g == 0) {
        load_sr(fill, k0);
      } else if (g == 2) {
        load_w0(fill, kb);
      } else if (g == 4) {
        load_w1(fill, kb);
      } else if (g == 6) {
        load_p(fill, k0);
      } else if (g >= 8 && g <= 22 && (g & 1) == 0) {
        dma_x_one(xn, (g - 8) >> 1, kb);
      } else if (g == 17) {
        store_piece(en, eslot0, e);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    store_piece(en, eslot1, e + 8);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitVm);  // this wave's chunk c+1 loads (X DMA too) landed
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // nchunks = K / 32 is a multiple of 4 (K is a multiple of 128).  Step c reads X stage
  // c % 4 and E stage c % 2, quantizes register set (c+1) % 4 into E stage (c+1) % 2 and
  // fills register set (c+3) % 4 and X stage (c+3) % 4 (last read in step c-1).
  for (int c = 0; c < nchunks; c += 4) {
    step(c + 0, xs0, xs3, es0, es1, S1, S3);
    step(c + 1, xs1, xs0, es1, es0, S2, S0);
    step(c + 2, xs2, xs1, es0, es1, S3, S1);
    step(c + 3, xs3, xs2, es1, es0, S0, S2);
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
                               const float* rs_tab, const float2* sr_tab, const float2* params,
                               int n_grid, const SearchPlan& plan, double* partial, hipStream_t st) {
  const int64_t per_xcd = plan.blocks / 8;
  const dim3 grid((unsigned)plan.blocks);
#define AWQ_LAUNCH(XF, WF)                                                                      \
  search_fused_kernel<XF, WF><<<grid, THREADS, 0, st>>>(X, M, ldx, W, N, K, ldw, s_tab, rs_tab, \
                                                        params, n_grid, plan.nt, plan.tiles,    \
                                                        per_xcd, partial)
  if (!xf32 && !wf32) {
    search_pipelined_kernel<<<grid, THREADS, 0, st>>>(
        static_cast<const uint16_t*>(X), M, ldx, static_cast<const uint16_t*>(W), N, K, ldw, s_tab,
        rs_tab, sr_tab, params, n_grid, plan.nt, plan.tiles, per_xcd, partial);
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

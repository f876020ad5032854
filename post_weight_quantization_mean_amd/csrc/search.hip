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
//
// Three kernels share this tile and arithmetic: search_fused_kernel (above description; any
// dtype), search_pipelined_kernel (bf16: a software pipeline with X staged through LDS by the
// buffer-to-LDS DMA) and search_persistent_kernel (bf16, the production path: one block per CU
// carrying that pipeline across tiles, with X read straight into registers from a copy of X in
// matrix-core operand order that xfrag_kernel writes first).
#include <atomic>
#include <type_traits>

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
    const void* __restrict__ X, int64_t M, int64_t ldx, const WSegs segs, int64_t K,
    const float* __restrict__ s_tab, const float* __restrict__ rs_tab,
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
  const int64_t n0 = (tile % nt_count) * BN;  // in the padded row space of all weights
  // the weight this tile belongs to; n0w: the tile's first row within it
  const WSel sel = select_wseg(segs, tile % nt_count);
  const void* __restrict__ W = sel.w;
  const int64_t N = sel.n, ldw = sel.ldw, n0w = sel.n0;
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
  const int64_t xrows = M - m0, wrows = N - n0w;
  const int64_t xbytes = xrows * ldx * XSZ, wbytes = wrows * ldw * WSZ;
  const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const char*>(X) + m0 * ldx * XSZ), (short)0,
      (int)(xbytes < 0x7fffffff ? xbytes : 0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(static_cast<const char*>(W) + n0w * ldw * WSZ), (short)0,
      (int)(wbytes < 0x7fffffff ? wbytes : 0x7fffffff), 0x00020000);
  const uint32_t xoff0 = (uint32_t)(xrow0 * ldx * XSZ + xkp * 16);
  const uint32_t xstep = (uint32_t)(64 * ldx * XSZ);
  const uint32_t woff0 = (uint32_t)(wrow0 * ldw * WSZ + wkp * 16);
  const uint32_t wstep = (uint32_t)(Gm::WROW_STEP * ldw * WSZ);

  const float* srow = s_tab + (int64_t)al * K + wkp * WEL;
  const float* rsrow = rs_tab + (int64_t)al * K + wkp * WEL;
  // group ranges of this thread's W rows (rows past the weight's N are masked)
  const int64_t NP = nt_count * BN;
  const float2* prow[WP];  // this thread's rows in the range table of candidate al
  bool wlive[WP];
#pragma unroll
  for (int i = 0; i < WP; ++i) {
    const int64_t r = wrow0 + Gm::WROW_STEP * i;
    wlive[i] = n0w + r < N;
    prow[i] = params + (int64_t)al * G * NP + range_slot(n0 + r);  // n0 + r < NP
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
// Same tile and arithmetic as above, software-pipelined so that every step is a run of 32
// back-to-back matrix instructions with the other work of the step issued between them.
// Step c (one chunk of 32 input channels) issues the MFMAs of chunk c and, between them:
//   * the quantization of chunk c+2 into E stage (c+2) % 3: wave w quantizes E rows
//     32w .. 32w+31, lane l rows 32w + l/4 and 32w + 16 + l/4, channels 8 (l%4) .. +7, from
//     W words loaded two steps earlier, the group ranges of its two rows and the chunk's
//     (s, 1/s) pairs, read from a per-group table in LDS;
//   * the fragment reads of chunk c's second K-half, chunk c+1's B fragments of the first
//     K-half, and the first two (of four) A fragments of chunk c+1; the other two are read as
//     step c+1 starts and first used eight matrix instructions later;
//   * the vector-memory traffic for later steps (below).
// X lives in LDS as pair stages: 2 chunks (64 channels, a full 128-byte line of a row) per
// stage, two stages.  The global -> LDS DMA (buffer_load ... lds) of a pair moves 8 rows x
// 128 bytes per instruction: an instruction that fills whole lines costs the vector-memory
// address path about 1.5x fewer cycles per byte than one that fills 64-byte halves (measured),
// and every line crosses from L2 once.  Pair p+1 (chunks 2p+2, 2p+3) is DMA'd during steps
// 2p (this wave's rows 0-63) and 2p+1 (rows 64-127), into the stage pair p-1 used.  Even steps
// also load the W words of chunks c+4 and c+5 (the two 64-byte halves of the same lines, back
// to back, so the second is an L1 hit); when c % 4 = 0, the next group's ranges and its
// (s, 1/s) table.
// Each wave DMAs only the 128 X rows it multiplies, so X needs no barrier: a wave reads its
// rows once its own vmcnt says they landed.  E is shared by the four waves; the one barrier
// per step, after every wave stored its part of E for chunk c+2, makes E of chunk c+1 (stored
// a step earlier) readable during step c.  X stages are distinct LDS objects with a static role
// per unrolled step (the compiler's wait counters for the DMA stay exact); the three E stages
// are addressed at run time.
// LDS rows are unpadded with their 16-byte slots permuted: X pair rows (128 bytes, 8 slots)
// by (row >> 1) & 7, E rows (64 bytes, 4 slots) by (row >> 2) & 3.  With them the 32-row MFMA
// fragment reads (ds_read_b128) are free of bank conflicts on gfx950.
#define AWQ_LDS __attribute__((address_space(3)))

constexpr int PKC = 32;                // input channels per chunk
constexpr int PROW = PKC * 2;          // bytes per E row
constexpr int XROW = 2 * PROW;         // bytes per X pair row (two chunks)
constexpr int XPSTAGE = BM * XROW;     // 64 KiB
constexpr int ESTAGE = BN * PROW;      // 8 KiB
constexpr int NES = 3;                 // E stages
constexpr int SRG = kGroup * 8;        // one group's (s, 1/s) pairs: 1 KiB

__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int xswz(int row) { return (row >> 1) & 7; }

struct WSet {
  uint4 w[2];  // this lane's 8 bf16 channels of its rows r0 and r1
};

struct RowQ {
  float delta, inv, lo, hi;
};

__global__ __launch_bounds__(THREADS, 1) void search_pipelined_kernel(
    const uint16_t* __restrict__ X, int64_t M, int64_t ldx, const WSegs segs, int64_t K,
    const float2* __restrict__ sr_tab, const float2* __restrict__ params, int n_grid,
    int64_t nt_count, int64_t tiles, int64_t per_xcd, double* __restrict__ partial) {
  // X pair stages (pairs 0, 2, 4, ... in xp0; 1, 3, 5, ... in xp1), each split into the first
  // and the last 64 of every wave's 128 rows: distinct LDS objects, so reads of one half never
  // wait for the DMA into the other
  __shared__ __attribute__((aligned(1024))) uint8_t xp0lo[XPSTAGE / 2];
  __shared__ __attribute__((aligned(1024))) uint8_t xp0hi[XPSTAGE / 2];
  __shared__ __attribute__((aligned(1024))) uint8_t xp1lo[XPSTAGE / 2];
  __shared__ __attribute__((aligned(1024))) uint8_t xp1hi[XPSTAGE / 2];
  __shared__ __attribute__((aligned(1024))) uint8_t es[NES * ESTAGE];
  // per-wave copies of one group's scale pairs: even groups in srs0, odd groups in srs1
  __shared__ __attribute__((aligned(1024))) uint8_t srs0[4 * SRG];
  __shared__ __attribute__((aligned(1024))) uint8_t srs1[4 * SRG];

  const int64_t b = blockIdx.x;
  const int64_t L = (b & 7) * per_xcd + (b >> 3);
  if (L >= tiles * n_grid) return;
  const int64_t tile = L / n_grid;
  const int al = (int)(L - tile * n_grid);
  const int64_t m0 = (tile / nt_count) * BM;
  const int64_t n0 = (tile % nt_count) * BN;  // in the padded row space of all weights
  // the weight this tile belongs to; n0w: the tile's first row within it
  const WSel sel = select_wseg(segs, tile % nt_count);
  const uint16_t* __restrict__ W = static_cast<const uint16_t*>(sel.w);
  const int64_t N = sel.n, ldw = sel.ldw, n0w = sel.n0;
  const int G = (int)(K / kGroup);
  const int64_t NP = nt_count * BN;
  const int nchunks = (int)(K / PKC);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // Buffer resources are rebased at this tile so rows past M (or N) read as zero; offsets
  // stay below 2^31 (host-checked: 512 rows of X, 128 rows of W).
  const int64_t xbytes = (M - m0) * ldx * 2, wbytes = (N - n0w) * ldw * 2;
  const __amdgpu_buffer_rsrc_t xrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(X + m0 * ldx), (short)0, (int)(xbytes < 0x7fffffff ? xbytes : 0x7fffffff), 0x00020000);
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(W + n0w * ldw), (short)0, (int)(wbytes < 0x7fffffff ? wbytes : 0x7fffffff), 0x00020000);
  // this candidate's (s, 1/s) pairs: K float2 = 8 K bytes (< 2^24: K <= ldx < 2^21 follows
  // from the host check on 512 rows of X)
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(sr_tab + (int64_t)al * K), (short)0, (int)(K * 8), 0x00020000);
  // X DMA instruction i (0..15) of wave w fills pair rows 128 w + 8 i + lane / 8, slot lane % 8,
  // with the global 16-byte piece slot ^ xswz(row).  xswz depends on i only through i % 2, so
  // two lane offsets serve all sixteen; the rest of the row offset goes in soffset.
  uint32_t xoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = wave * WAVE_ROWS + 8 * i + (lane >> 3);
    xoff[i] = (uint32_t)(row * ldx * 2 + (((lane & 7) ^ xswz(row)) * 16));
  }
  const uint32_t xrow16 = (uint32_t)(16 * ldx * 2);  // 16 rows of X, bytes
  // quantization: rows r0, r1 of the E tile, channel piece q4 of each chunk
  const int q4 = lane & 3;
  const int r0 = wave * 32 + (lane >> 2), r1 = r0 + 16;
  const uint32_t woff0 = (uint32_t)(r0 * ldw * 2 + q4 * 16);
  const uint32_t woff1 = (uint32_t)(r1 * ldw * 2 + q4 * 16);
  const int eslot0 = r0 * PROW + ((q4 ^ swz(r0)) * 16);
  const int eslot1 = r1 * PROW + ((q4 ^ swz(r1)) * 16);
  const bool live0 = n0w + r0 < N, live1 = n0w + r1 < N;
  // ranges of rows r0 and r1 are adjacent (range_slot); rows past N are masked.  A buffer
  // resource over this candidate's ranges (G Npad float2 < 2^31 bytes: host-checked) reads
  // groups past the end as zero.
  const __amdgpu_buffer_rsrc_t prsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(params + (int64_t)al * G * NP), (short)0, (int)((int64_t)G * NP * 8), 0x00020000);
  const int poff = (int)((n0 + 32 * wave + 2 * (lane >> 2)) * 8);

  // fragment reads: lane reads row (32 t + fr), 16-byte piece 2 h + fh of K-half h of its chunk
  const int fr = lane & 31, fh = lane >> 5;
  const int efoff0 = fr * PROW + (((0 + fh) ^ swz(fr)) * 16);
  const int efoff1 = fr * PROW + (((2 + fh) ^ swz(fr)) * 16);
  // in an X pair row the chunk's pieces are 4 (c % 2) + 2 h + fh
  auto xfoff = [&](int half, int h) { return fr * XROW + (((4 * half + 2 * h + fh) ^ xswz(fr)) * 16); };
  const int xwave = wave * (WAVE_ROWS / 2) * XROW;  // this wave's 64 rows in a half stage

  // DMA instruction i of pair p into half stage xh (i < 8: the wave's rows 0-63, else 64-127)
  auto dma_x_one = [&](uint8_t* xh, int i, int p) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(xrsrc, (AWQ_LDS void*)(xh + xwave + (i & 7) * 1024), 16,
                                             (int)xoff[i & 1], (int)((uint32_t)(i >> 1) * xrow16 + (uint32_t)p * XROW),
                                             0, 0);
  };
  // W words of row i of chunk (cb / 64 + j): the constant part of the offset goes in the
  // instruction's immediate field; chunks past the end read other bytes of the tile (unused)
  auto load_w = [&](WSet& S, int i, int cb, int j) {
    S.w[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           wrsrc, (int)(i == 0 ? woff0 : woff1) + j * (PKC * 2), cb, 0));
  };
  auto load_p = [&](int g) {
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(prsrc, poff, (int)(g * NP * 8), 0));
  };
  // each wave copies group g's 1 KiB of pairs into its own slot of table (g even: srs0), one
  // 16-byte-per-lane DMA (a 4-byte DMA costs several times more per instruction)
  auto dma_sr = [&](uint8_t* table, int g) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(srsrc, (AWQ_LDS void*)(table + SRG * wave), 16, 16 * lane,
                                             g * SRG, 0, 0);
  };
  // (s, 1/s) of channels 8 q4 .. 8 q4 + 7 of chunk c: four float4 (s_2t, rs_2t, s_2t+1, rs_2t+1)
  auto sr_addr = [&](const uint8_t* table, int c) {
    return table + SRG * wave + (32 * (c & 3) + 8 * q4) * 8;
  };
  auto row_setup = [&](const float4& P, int i) {
    const bool live = i == 0 ? live0 : live1;
    RowQ q;
    q.delta = live ? (i == 0 ? P.x : P.z) : 1.0f;  // rows past N: Delta 1, z 0, w 0: e = 0
    const float z = live ? (i == 0 ? P.y : P.w) : 0.0f;
    q.inv = __builtin_amdgcn_rcpf(q.delta);  // search only; the pack divides exactly
    q.lo = -z;
    q.hi = 15.0f - z;
    return q;
  };
  // e = w - Delta (q - z) / s for channel j (0..7) of row i (0/1)
  auto elem = [&](const WSet& S, const float4* sv, const RowQ& q, int i, int j) {
    const uint4& w4 = S.w[i];
    const uint32_t u = j < 2 ? w4.x : j < 4 ? w4.y : j < 6 ? w4.z : w4.w;
    const float w = (j & 1) ? bf16_hi(u) : bf16_lo(u);
    const float s = (j & 1) ? sv[j >> 1].z : sv[j >> 1].x;
    const float rs = (j & 1) ? sv[j >> 1].w : sv[j >> 1].y;
    const float v = w * s;                                    // S W
    const float r = rintf(v * q.inv);                         // rne(v / Delta)
    const float qz = __builtin_amdgcn_fmed3f(r, q.lo, q.hi);  // clamp(r + z, 0, 15) - z
    return fmaf(-(qz * q.delta), rs, w);                      // w - Delta (q - z) / s
  };
  auto store_piece = [&](uint8_t* estage, int slot, const float* e8) {
    uint32_t pk[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) pk[h] = pack_bf16x2(e8[2 * h], e8[2 * h + 1]);
    *reinterpret_cast<uint4*>(estage + slot) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  };
  auto quantize_all = [&](const WSet& S, const float4& P, int c, uint8_t* estage) {  // prologue only
    float4 sv[4];
    const uint8_t* sa = sr_addr(srs0, c);
#pragma unroll
    for (int t = 0; t < 4; ++t) sv[t] = *reinterpret_cast<const float4*>(sa + 16 * t);
    const RowQ q0 = row_setup(P, 0), q1 = row_setup(P, 1);
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = elem(S, sv, q0, 0, j);
    store_piece(estage, eslot0, e);
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = elem(S, sv, q1, 1, j);
    store_piece(estage, eslot1, e);
  };
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

  WSet S0, S1, S2, S3;  // W words of chunk c live in set c % 4
  float4 PC, PN;        // ranges of the group being quantized, of the next group
  RowQ q0, q1;          // row_setup of PC (rows r0, r1), renewed when PC changes
  // Prologue (once per block): group 0's scale table and ranges, W of chunks 0-3 and the X
  // pair of chunks 0 and 1, then chunks 0 and 1 are quantized.
  dma_sr(srs0, 0);
  PC = load_p(0);
  load_w(S0, 0, 0, 0);
  load_w(S1, 0, 0, 1);
  load_w(S0, 1, 0, 0);
  load_w(S1, 1, 0, 1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < 16; ++i) dma_x_one(i < 8 ? xp0lo : xp0hi, i, 0);
  __builtin_amdgcn_sched_barrier(0);
  load_w(S2, 0, 0, 2);
  load_w(S3, 0, 0, 3);
  load_w(S2, 1, 0, 2);
  load_w(S3, 1, 0, 3);
  __builtin_amdgcn_sched_barrier(0);
  vm_wait(std::integral_constant<int, 0>{});
  __builtin_amdgcn_sched_barrier(0);
  quantize_all(S0, PC, 0, es + 0 * ESTAGE);
  quantize_all(S1, PC, 1, es + 1 * ESTAGE);
  q0 = row_setup(PC, 0);
  q1 = row_setup(PC, 1);
  bf16x8 a0[4], b0[4];
  {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 2; ++t) a0[t] = frag(xp0lo + xwave + t * 32 * XROW, xfoff(0, 0));
#pragma unroll
    for (int t = 0; t < 4; ++t) b0[t] = frag(es + t * 32 * PROW, efoff0);
    // Consume the W words of chunks 2 and 3 here: left unused before the loop, their loads
    // would be sunk to the loop entry, and the loop head would then wait for them on every
    // iteration.
    auto consume = [](const WSet& S) {
      asm volatile("" ::"v"(S.w[0].x), "v"(S.w[0].y), "v"(S.w[0].z), "v"(S.w[0].w), "v"(S.w[1].x),
                   "v"(S.w[1].y), "v"(S.w[1].z), "v"(S.w[1].w));
    };
    consume(S2);
    consume(S3);
  }

  // One pipeline step, hand-scheduled in 32 groups, one per matrix instruction of chunk c
  // (k = c % 4, known at compile time; xc is chunk c's pair stage, xn chunk c+1's):
  //   groups 0, 1: A fragments 2, 3 of chunk c (first used in groups 8 and 12);
  //   groups 0-7:  second-half fragment reads of chunk c (A even, B odd groups);
  //   group 0:     the (s, 1/s) pairs for the quantization of chunk c+2 (row ranges are set up
  //                when the group changes);
  //   groups 3-25, two of every three: its sixteen elements; E stores in groups 14 and 26;
  //   groups 17-23 (odd): chunk c+1's B fragments of the first K-half; groups 24, 25: its A
  //   fragments 0, 1;
  //   vector memory (below): even steps W words of chunks c+4 and c+5 (groups 0-3), when k = 0
  //   the next group's ranges and scale table (4, 5), and X DMA of pair c/2 + 1, rows 0-63
  //   (groups 6, 9, ..., 27); odd steps the same pair's rows 64-127 (groups 0, 2, ..., 14).
  // vmcnt accounting (even steps: 4 W + 8 X loads, plus 2 when k = 0; odd steps 8 X):
  //   * start of an even step: all loads landed (the X rows 64-127 of chunk c, DMA'd by the
  //     previous step, are read now); start of an odd step: at most the previous step's 12
  //     outstanding (W of chunk c+2 is from step c-3, chunk c's X from steps c-3, c-2);
  //   * group 24: chunk c+1's rows 0-63 (from step c-1 at the latest) landed;
  //   * end of a k = 1 step: this wave's scale table DMA of step k = 0 (followed by 16 X) landed.
  // c8: first chunk of the 8-step body, j: step within it (c = c8 + j); eo0, eo1, eo2: byte
  // offsets of the E stages of chunks c, c+1, c+2, rotated after every step (in the unrolled
  // body the rotation is register renaming).  Loads past the last chunk, pair or group read
  // other bytes of their tiles or zeros (buffer bounds) and are never used.
  auto step = [&](int c8, auto jc, const uint8_t* xclo, const uint8_t* xchi, const uint8_t* xnlo,
                  uint8_t* xdlo, uint8_t* xdhi, const WSet& Q, WSet& F4, WSet& F5, const uint8_t* srq,
                  uint8_t* srn, int& eo0, int& eo1, int& eo2) {
    constexpr int j = decltype(jc)::value;
    constexpr int k = j & 3;
    constexpr bool even = (k & 1) == 0;
    const int c = c8 + j;
    const int cb = c8 * (PKC * 2);                 // chunk c8's byte offset in a row
    const int pd = (c8 >> 1) + (j >> 1) + 1;       // pair being DMA'd
    const int gn = (c8 >> 2) + (j >> 2) + 1;       // next group (k = 0 steps)
    const uint8_t* ec = es + eo0;
    const uint8_t* en = es + eo1;
    uint8_t* eq = es + eo2;
    const uint8_t* sa = sr_addr(srq, k + 2);
    const uint8_t* xwlo = xclo + xwave;
    const uint8_t* xwhi = xchi + xwave;
    const uint8_t* xnw = xnlo + xwave;
    // A fragment t of chunk c: rows 32 t .. 32 t + 31 of the wave, in the lo (t < 2) or hi half
    auto xa = [&](int t) { return (t < 2 ? xwlo : xwhi) + (t & 1) * 32 * XROW; };
    const int xo0 = xfoff(k & 1, 0), xo1 = xfoff(k & 1, 1), xn0 = xfoff((k + 1) & 1, 0);
    if (k == 2) {  // chunks c+2 .. c+5 of this quad after the first two: next group
      PC = PN;
      q0 = row_setup(PC, 0);
      q1 = row_setup(PC, 1);
    }
    bf16x8 a1[4], b1[4];
    float4 sv[4];
    float e[16];
    __builtin_amdgcn_sched_barrier(0);
    vm_wait(std::integral_constant<int, even ? 0 : 12>{});
#pragma unroll
    for (int g = 0; g < 32; ++g) {
      const int r = (g >> 2) & 3, cc = g & 3;
      if (g < 16)
        acc[r][cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[r], b0[cc], acc[r][cc], 0, 0, 0);
      else
        acc[r][cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[r], b1[cc], acc[r][cc], 0, 0, 0);
      if (g < 2) a0[2 + g] = frag(xa(2 + g), xo0);
      if (g == 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) sv[t] = *reinterpret_cast<const float4*>(sa + 16 * t);
      }
      if (g < 8) {
        if (g & 1)
          b1[g >> 1] = frag(ec + (g >> 1) * 32 * PROW, efoff1);
        else
          a1[g >> 1] = frag(xa(g >> 1), xo1);
      }
      // element el in group 3 + 3 (el / 2) + el % 2: groups 3-13 for row r0, 15-25 for r1
      const int el = g >= 3 && g <= 25 && (g - 3) % 3 != 2 ? 2 * ((g - 3) / 3) + (g - 3) % 3 : -1;
      if (el >= 0) {
        e[el] = el < 8 ? elem(Q, sv, q0, 0, el) : elem(Q, sv, q1, 1, el - 8);
        asm volatile("" : "+v"(e[el]));  // keep the element in this group (no IR sinking)
      }
      if (g == 14) store_piece(eq, eslot0, e);
      if (g == 26) store_piece(eq, eslot1, e + 8);
      // every fragment read before group 8 (a1, b1) has landed; only the E store of group 14
      // may be in flight.  One wait here spares the compiler's per-use waits in groups 16-31.
      if (g == 15) __builtin_amdgcn_s_waitcnt(0xf | (0x7 << 4) | (0x1 << 8) | (0x3 << 14));
      if (g >= 16 && g < 24 && (g & 1)) b0[(g - 16) >> 1] = frag(en + ((g - 16) >> 1) * 32 * PROW, efoff0);
      // chunk c+1's rows 0-63 landed: they come from step c-1 at the latest, followed by this
      // step's loads before group 24 (even: 4 W, 2 when k = 0, 6 X; odd: 8 X)
      if (g == 24) vm_wait(std::integral_constant<int, even ? 10 : 8>{});
      if (g == 24 || g == 25) a0[g - 24] = frag(xnw + (g - 24) * 32 * XROW, xn0);
      if (even) {
        if (g == 0) load_w(F4, 0, cb, j + 4);
        if (g == 1) load_w(F5, 0, cb, j + 5);
        if (g == 2) load_w(F4, 1, cb, j + 4);
        if (g == 3) load_w(F5, 1, cb, j + 5);
        if (k == 0 && g == 4) PN = load_p(gn);
        if (k == 0 && g == 5) dma_sr(srn, gn);
        if (g >= 6 && g <= 27 && (g - 6) % 3 == 0) dma_x_one(xdlo, (g - 6) / 3, pd);
      } else {
        if (g <= 14 && (g & 1) == 0) dma_x_one(xdhi, 8 + g / 2, pd);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (k == 1) vm_wait(std::integral_constant<int, 16>{});  // this wave's scale table landed
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // E stores of chunk c+2, fragment reads
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const int et = eo0;
    eo0 = eo1;
    eo1 = eo2;
    eo2 = et;
  };

  // nchunks = K / 32 is a multiple of 4 (K is a multiple of 128).  Step c multiplies chunk c
  // from pair stage (c / 2) % 2, quantizes W set (c+2) % 4 into E stage (c+2) % 3, DMAs half
  // of pair c/2 + 1 into stage (c/2 + 1) % 2 (last read by chunk c-1, in step c-1) and, when
  // even, loads the W words of chunks c+4 and c+5 into sets c % 4 and (c+1) % 4 (quantized in
  // steps c-2 and c-1).  The body covers two groups (8 steps) so that each scale table and
  // each X pair stage has a static role: reads of one never wait for the DMA into the other.
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  using I6 = std::integral_constant<int, 6>;
  using I7 = std::integral_constant<int, 7>;
  int eo0 = 0, eo1 = ESTAGE, eo2 = 2 * ESTAGE;
  int c = 0;
  for (; c + 8 <= nchunks; c += 8) {
    step(c, I0{}, xp0lo, xp0hi, xp0lo, xp1lo, xp1hi, S2, S0, S1, srs0, srs1, eo0, eo1, eo2);
    step(c, I1{}, xp0lo, xp0hi, xp1lo, xp1lo, xp1hi, S3, S0, S1, srs0, srs1, eo0, eo1, eo2);
    step(c, I2{}, xp1lo, xp1hi, xp1lo, xp0lo, xp0hi, S0, S2, S3, srs1, srs1, eo0, eo1, eo2);
    step(c, I3{}, xp1lo, xp1hi, xp0lo, xp0lo, xp0hi, S1, S2, S3, srs1, srs1, eo0, eo1, eo2);
    step(c, I4{}, xp0lo, xp0hi, xp0lo, xp1lo, xp1hi, S2, S0, S1, srs1, srs0, eo0, eo1, eo2);
    step(c, I5{}, xp0lo, xp0hi, xp1lo, xp1lo, xp1hi, S3, S0, S1, srs1, srs0, eo0, eo1, eo2);
    step(c, I6{}, xp1lo, xp1hi, xp1lo, xp0lo, xp0hi, S0, S2, S3, srs0, srs0, eo0, eo1, eo2);
    step(c, I7{}, xp1lo, xp1hi, xp0lo, xp0lo, xp0hi, S1, S2, S3, srs0, srs0, eo0, eo1, eo2);
  }
  if (c < nchunks) {  // K / 128 odd: one more group
    step(c, I0{}, xp0lo, xp0hi, xp0lo, xp1lo, xp1hi, S2, S0, S1, srs0, srs1, eo0, eo1, eo2);
    step(c, I1{}, xp0lo, xp0hi, xp1lo, xp1lo, xp1hi, S3, S0, S1, srs0, srs1, eo0, eo1, eo2);
    step(c, I2{}, xp1lo, xp1hi, xp1lo, xp0lo, xp0hi, S0, S2, S3, srs1, srs1, eo0, eo1, eo2);
    step(c, I3{}, xp1lo, xp1hi, xp0lo, xp0lo, xp0hi, S1, S2, S3, srs1, srs1, eo0, eo1, eo2);
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
  // every wave is past its last LDS access (the barrier ending the last step), so the first
  // E stage can hold the four wave sums
  double* red = reinterpret_cast<double*>(es);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  if (tid == 0) partial[(int64_t)al * tiles + tile] = ((red[0] + red[1]) + red[2]) + red[3];
}

// ---- persistent variant of the pipelined kernel -------------------------------------------
// One block per CU walks its tiles (those of its XCD's run of logical indices, every PX-th, PX
// = blocks per XCD) and carries the pipeline across tiles.
// X never passes through LDS here.  The kernel reads it from a copy in fragment order
// (xfrag_kernel), where the 16 bytes that lane l holds of the MFMA A operand for rows
// 32 rb .. 32 rb + 31 and channels 16 kb .. 16 kb + 15 sit together, so each A fragment is one
// coalesced 1 KiB load straight into registers.  Per step and CU, LDS then carries the 8 KiB of
// E written and 32 KiB of B fragments read, against 104 KiB when X is staged there (the X
// copies into LDS were the largest cost of a step).
// Step c loads the A fragments of chunk c+1, each right after the last product of chunk c that
// reads the same registers, about one step before its first use; the compiler's counters wait
// for them.  The rest of the look-ahead is the pipelined kernel's: W of chunks c+4, c+5 on even
// steps, the next group's ranges and (s, 1/s) table when c % 4 = 0.  In the last steps of a
// tile these read the next tile's data, so the next tile starts with its first A fragments,
// W sets and two E chunks in place and no prologue.
// At a tile boundary each wave squares its accumulators and reduces them across its lanes; the
// first step of the next tile starts the products from zero and stores that wave's sum (one per
// wave: partial[4 (al tiles + tile) + wave]), so nothing waits for the store.
// Needs K / 32 to be a multiple of 8 (K / 128 even) and at least 16 (the first and the last
// eight steps of a tile are distinct).
struct TileRes {
  __amdgpu_buffer_rsrc_t x, w, sr, p;  // Xf from row m0, W rows n0w.., the candidate's (s, 1/s), ranges
  uint32_t woff0, woff1;               // this lane's W rows r0, r1
  int poff;                            // this lane's range slots
  bool live0, live1;                   // rows r0, r1 inside the weight
  int64_t slot;                        // al * tiles + tile
};

// MULTI: the tiles come from several weights (the segment table is scanned per tile); otherwise
// every tile is one of segs' first weight, whose fields alone are read.
template <bool MULTI>
__global__ __launch_bounds__(THREADS, 1) void search_persistent_kernel(
    const uint16_t* __restrict__ Xf, int64_t Mp, const WSegs segs, int64_t K,
    const float2* __restrict__ sr_tab, const float2* __restrict__ params, int n_grid,
    int64_t nt_count, int64_t tiles, int64_t per_xcd, double* __restrict__ partial) {
  __shared__ __attribute__((aligned(1024))) uint8_t es[NES * ESTAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t srs0[4 * SRG];
  __shared__ __attribute__((aligned(1024))) uint8_t srs1[4 * SRG];

  // this block's tiles: logical indices L0, L0 + PX, ... below its XCD's end
  const int64_t PX = gridDim.x >> 3;
  const int64_t xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
  const int64_t total = tiles * n_grid;
  const int64_t lend0 = (xcd + 1) * per_xcd, lend = lend0 < total ? lend0 : total;
  const int64_t L0 = xcd * per_xcd + jx;
  if (L0 >= lend) return;
  const int G = (int)(K / kGroup);
  const int64_t NP = nt_count * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane & 3;
  const int r0 = wave * 32 + (lane >> 2), r1 = r0 + 16;
  auto rsrc = [](const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff), 0x00020000);
  };
  // (logical indices fit in 31 bits: host-checked)
  const uint32_t ng = (uint32_t)n_grid, ntc = (uint32_t)nt_count;
  auto make_res = [&](int64_t L, TileRes& T) {
    const uint32_t tile = (uint32_t)L / ng;
    const int al = (int)((uint32_t)L - tile * ng);
    const uint32_t mt = tile / ntc, nt = tile - mt * ntc;
    const int64_t m0 = (int64_t)mt * BM, n0 = (int64_t)nt * BN;
    const WSel sel = MULTI ? select_wseg(segs, nt) : WSel{segs.w[0], segs.ldw[0], segs.n[0], (int64_t)nt * BN};
    const uint16_t* W = static_cast<const uint16_t*>(sel.w);
    const int64_t N = sel.n, ldw = sel.ldw, n0w = sel.n0;
    // row blocks past Mp (a tile's rows past M) read as zero; 512 rows of Xf span less than
    // 2^31 bytes (host-checked)
    T.x = rsrc(Xf + m0 * K, (Mp - m0) * K * 2);
    T.w = rsrc(W + n0w * ldw, (N - n0w) * ldw * 2);
    T.sr = rsrc(sr_tab + (int64_t)al * K, K * 8);
    T.p = rsrc(params + (int64_t)al * G * NP, (int64_t)G * NP * 8);
    T.woff0 = (uint32_t)(r0 * ldw * 2 + q4 * 16);
    T.woff1 = (uint32_t)(r1 * ldw * 2 + q4 * 16);
    T.poff = (int)((n0 + 32 * wave + 2 * (lane >> 2)) * 8);
    T.live0 = n0w + r0 < N;
    T.live1 = n0w + r1 < N;
    T.slot = (int64_t)al * tiles + tile;
  };

  const int eslot0 = r0 * PROW + ((q4 ^ swz(r0)) * 16);
  const int eslot1 = r1 * PROW + ((q4 ^ swz(r1)) * 16);
  const int fr = lane & 31, fh = lane >> 5;
  const int efoff0 = fr * PROW + (((0 + fh) ^ swz(fr)) * 16);
  const int efoff1 = fr * PROW + (((2 + fh) ^ swz(fr)) * 16);

  // A fragment (row block r of this wave's 128 rows, chunk ch, K-half h): 1 KiB of Xf, this
  // lane's 16 bytes at 16 lane; a row block is 64 K bytes
  const uint32_t avoff = (uint32_t)(lane * 16) + (uint32_t)(wave * 4) * (uint32_t)(K * 64);
  auto load_a = [&](const TileRes& T, int ch, int h, int r) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                          T.x, (int)avoff, (int)(r * K * 64 + (2 * ch + h) * 1024), 0));
  };
  auto load_w = [&](const TileRes& T, WSet& S, int i, int cb, int j) {
    S.w[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           T.w, (int)(i == 0 ? T.woff0 : T.woff1) + j * (PKC * 2), cb, 0));
  };
  auto load_p = [&](const TileRes& T, int g) {
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(T.p, T.poff, (int)(g * NP * 8), 0));
  };
  auto dma_sr = [&](const TileRes& T, uint8_t* table, int g) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(T.sr, (AWQ_LDS void*)(table + SRG * wave), 16, 16 * lane, g * SRG, 0, 0);
  };
  auto sr_addr = [&](const uint8_t* table, int c) {
    return table + SRG * wave + (32 * (c & 3) + 8 * q4) * 8;
  };
  auto row_setup = [&](const TileRes& T, const float4& P, int i) {
    const bool live = i == 0 ? T.live0 : T.live1;
    RowQ q;
    q.delta = live ? (i == 0 ? P.x : P.z) : 1.0f;  // rows past N: Delta 1, z 0, w 0: e = 0
    const float z = live ? (i == 0 ? P.y : P.w) : 0.0f;
    q.inv = __builtin_amdgcn_rcpf(q.delta);  // search only; the pack divides exactly
    q.lo = -z;
    q.hi = 15.0f - z;
    return q;
  };
  auto elem = [&](const WSet& S, const float4* sv, const RowQ& q, int i, int j) {
    const uint4& w4 = S.w[i];
    const uint32_t u = j < 2 ? w4.x : j < 4 ? w4.y : j < 6 ? w4.z : w4.w;
    const float w = (j & 1) ? bf16_hi(u) : bf16_lo(u);
    const float s = (j & 1) ? sv[j >> 1].z : sv[j >> 1].x;
    const float rs = (j & 1) ? sv[j >> 1].w : sv[j >> 1].y;
    const float v = w * s;                                    // S W
    const float r = rintf(v * q.inv);                         // rne(v / Delta)
    const float qz = __builtin_amdgcn_fmed3f(r, q.lo, q.hi);  // clamp(r + z, 0, 15) - z
    return fmaf(-(qz * q.delta), rs, w);                      // w - Delta (q - z) / s
  };
  auto store_piece = [&](uint8_t* estage, int slot, const float* e8) {
    uint32_t pk[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) pk[h] = pack_bf16x2(e8[2 * h], e8[2 * h + 1]);
    *reinterpret_cast<uint4*>(estage + slot) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  };
  auto quantize_all = [&](const TileRes& T, const WSet& S, const float4& P, int c, uint8_t* estage) {  // prologue
    float4 sv[4];
    const uint8_t* sa = sr_addr(srs0, c);
#pragma unroll
    for (int t = 0; t < 4; ++t) sv[t] = *reinterpret_cast<const float4*>(sa + 16 * t);
    const RowQ q0 = row_setup(T, P, 0), q1 = row_setup(T, P, 1);
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = elem(S, sv, q0, 0, j);
    store_piece(estage, eslot0, e);
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = elem(S, sv, q1, 1, j);
    store_piece(estage, eslot1, e);
  };
  auto frag = [&](const uint8_t* base, int fo) { return *reinterpret_cast<const bf16x8*>(base + fo); };
  auto vm_wait = [](auto n) {
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
  const f32x16 zero16 = acc[0][0];

  TileRes cur, nxt;
  make_res(L0, cur);
  WSet S0, S1, S2, S3;
  float4 PC, PN;
  RowQ q0, q1;
  bf16x8 a0[4], a1[4], b0[4];
  // prologue of the first tile: its table, ranges, W of chunks 0-3 and A fragments of chunk 0
  dma_sr(cur, srs0, 0);
  PC = load_p(cur, 0);
  load_w(cur, S0, 0, 0, 0);
  load_w(cur, S1, 0, 0, 1);
  load_w(cur, S0, 1, 0, 0);
  load_w(cur, S1, 1, 0, 1);
  load_w(cur, S2, 0, 0, 2);
  load_w(cur, S3, 0, 0, 3);
  load_w(cur, S2, 1, 0, 2);
  load_w(cur, S3, 1, 0, 3);
#pragma unroll
  for (int r = 0; r < 4; ++r) a0[r] = load_a(cur, 0, 0, r);
#pragma unroll
  for (int r = 0; r < 4; ++r) a1[r] = load_a(cur, 0, 1, r);
  __builtin_amdgcn_sched_barrier(0);
  vm_wait(std::integral_constant<int, 0>{});
  __builtin_amdgcn_sched_barrier(0);
  quantize_all(cur, S0, PC, 0, es + 0 * ESTAGE);
  quantize_all(cur, S1, PC, 1, es + 1 * ESTAGE);
  q0 = row_setup(cur, PC, 0);
  q1 = row_setup(cur, PC, 1);
  {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < 4; ++t) b0[t] = frag(es + t * 32 * PROW, efoff0);
  }
  double pend = 0.0;             // the sum of the wave's squares of the previous tile
  int64_t pend_slot = cur.slot;  // its slot (the first tile's own slot, overwritten by its sum)

  // Step c.  FIRST: the tile's first step (products start from zero; the previous tile's wave
  // sum is stored in group 1).  LAST: the tile's last eight steps, whose look-ahead past the
  // tile's end uses the next tile (nxt: its resources; chunk and group indices relative to its
  // start).
  auto step = [&](int c8, auto jc, auto firstc, auto lastc, const WSet& Q, WSet& F4, WSet& F5,
                  const uint8_t* srq, uint8_t* srn, int& eo0, int& eo1, int& eo2) {
    constexpr int j = decltype(jc)::value;
    constexpr bool FIRST = decltype(firstc)::value, LAST = decltype(lastc)::value;
    constexpr int k = j & 3;
    constexpr bool even = (k & 1) == 0;
    // which look-ahead of this step falls past the tile's end (last eight steps only)
    constexpr bool nw = LAST && j >= 4;  // W of chunks c+4, c+5 and the next group's ranges / table
    constexpr bool na = LAST && j == 7;  // the A fragments of chunk c+1
    constexpr bool nq = LAST && j == 6;  // the row setup of chunk c+2's group
    const TileRes& TW = nw ? nxt : cur;
    const TileRes& TA = na ? nxt : cur;
    // the next tile's chunks j + 4 - 8, j + 5 - 8 (offsets stay non-negative) and 0, group 0
    constexpr int jw = nw ? j - 8 : j;
    const int cb = nw ? 0 : c8 * (PKC * 2);
    const int ca = na ? 0 : c8 + j + 1;
    const int gn = nw ? 0 : (c8 >> 2) + (j >> 2) + 1;
    const uint8_t* ec = es + eo0;
    const uint8_t* en = es + eo1;
    uint8_t* eq = es + eo2;
    const uint8_t* sa = sr_addr(srq, k + 2);
    if (k == 2) {
      PC = PN;
      q0 = row_setup(nq ? nxt : cur, PC, 0);
      q1 = row_setup(nq ? nxt : cur, PC, 1);
    }
    bf16x8 b1[4];
    float4 sv[4];
    float e[16];
    __builtin_amdgcn_sched_barrier(0);
    // k == 2 reads the (s, 1/s) table copied into LDS two steps earlier (group 5 of step k = 0):
    // 7 A loads of that step and 8 of the next were issued after it
    if (k == 2) vm_wait(std::integral_constant<int, 15>{});
#pragma unroll
    for (int g = 0; g < 32; ++g) {
      const int r = (g >> 2) & 3, cc = g & 3;
      if (g < 16)
        acc[r][cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[r], b0[cc], FIRST ? zero16 : acc[r][cc], 0, 0, 0);
      else
        acc[r][cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[r], b1[cc], acc[r][cc], 0, 0, 0);
      if (FIRST && g == 1) {
        // the previous tile's wave sum, the same value from every lane
        double* dst = partial + 4 * pend_slot + wave;
        *dst = pend;
      }
      // chunk c+1's A fragments, each after the last product that reads chunk c's in its place
      if (g >= 4 && g <= 16 && (g & 3) == 0) a0[(g >> 2) - 1] = load_a(TA, ca, 0, (g >> 2) - 1);
      if (g >= 20 && g <= 28 && (g & 3) == 0) a1[(g >> 2) - 5] = load_a(TA, ca, 1, (g >> 2) - 5);
      if (g == 31) a1[3] = load_a(TA, ca, 1, 3);
      if (g == 0) {
#pragma unroll
        for (int t = 0; t < 4; ++t) sv[t] = *reinterpret_cast<const float4*>(sa + 16 * t);
      }
      if (g < 8 && (g & 1)) b1[g >> 1] = frag(ec + (g >> 1) * 32 * PROW, efoff1);
      const int el = g >= 3 && g <= 25 && (g - 3) % 3 != 2 ? 2 * ((g - 3) / 3) + (g - 3) % 3 : -1;
      if (el >= 0) {
        e[el] = el < 8 ? elem(Q, sv, q0, 0, el) : elem(Q, sv, q1, 1, el - 8);
        asm volatile("" : "+v"(e[el]));
      }
      if (g == 14) store_piece(eq, eslot0, e);
      if (g == 26) store_piece(eq, eslot1, e + 8);
      if (g == 15) __builtin_amdgcn_s_waitcnt(0xf | (0x7 << 4) | (0x1 << 8) | (0x3 << 14));
      if (g >= 16 && g < 24 && (g & 1)) b0[(g - 16) >> 1] = frag(en + ((g - 16) >> 1) * 32 * PROW, efoff0);
      if (even) {
        if (g == 0) load_w(TW, F4, 0, cb, jw + 4);
        if (g == 1) load_w(TW, F5, 0, cb, jw + 5);
        if (g == 2) load_w(TW, F4, 1, cb, jw + 4);
        if (g == 3) load_w(TW, F5, 1, cb, jw + 5);
        if (k == 0 && g == 4) PN = load_p(TW, gn);
        if (k == 0 && g == 5) dma_sr(TW, srn, gn);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const int et = eo0;
    eo0 = eo1;
    eo1 = eo2;
    eo2 = et;
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  using I6 = std::integral_constant<int, 6>;
  using I7 = std::integral_constant<int, 7>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  // eight steps: step j quantizes chunk c+j+2 from the W set loaded four steps before (Q) and,
  // when even, loads chunks c+j+4, c+j+5 into F4, F5; the (s, 1/s) tables alternate by group
  auto body = [&](int c, auto firstc, auto lastc, int& eo0, int& eo1, int& eo2) {
    step(c, I0{}, firstc, lastc, S2, S0, S1, srs0, srs1, eo0, eo1, eo2);
    step(c, I1{}, F_{}, lastc, S3, S0, S1, srs0, srs1, eo0, eo1, eo2);
    step(c, I2{}, F_{}, lastc, S0, S2, S3, srs1, srs1, eo0, eo1, eo2);
    step(c, I3{}, F_{}, lastc, S1, S2, S3, srs1, srs1, eo0, eo1, eo2);
    step(c, I4{}, F_{}, lastc, S2, S0, S1, srs1, srs0, eo0, eo1, eo2);
    step(c, I5{}, F_{}, lastc, S3, S0, S1, srs1, srs0, eo0, eo1, eo2);
    step(c, I6{}, F_{}, lastc, S0, S2, S3, srs0, srs0, eo0, eo1, eo2);
    step(c, I7{}, F_{}, lastc, S1, S2, S3, srs0, srs0, eo0, eo1, eo2);
  };
  const int nchunks = (int)(K / PKC);
  int eo0 = 0, eo1 = ESTAGE, eo2 = 2 * ESTAGE;
  for (int64_t L = L0;; L += PX) {
    const bool more = L + PX < lend;
    if (more)
      make_res(L + PX, nxt);
    else
      nxt = cur;  // nothing follows: the look-ahead re-reads this tile's first chunks, unused
    body(0, T_{}, F_{}, eo0, eo1, eo2);
    for (int c = 8; c + 8 < nchunks; c += 8) body(c, F_{}, F_{}, eo0, eo1, eo2);
    body(nchunks - 8, F_{}, T_{}, eo0, eo1, eo2);
    // this tile's squares: fp32 per 32x32 tile, fp64 across tiles and lanes
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
    pend = ss;
    pend_slot = cur.slot;
    if (!more) break;
    cur = nxt;
  }
  partial[4 * pend_slot + wave] = pend;
  __builtin_amdgcn_s_waitcnt(0);  // every load (the last ones read ahead past the end) has landed
}

// X bf16 [M, K] (row stride ldx) into the fragment order of the persistent kernel, one
// xfrag_block per block.
__global__ __launch_bounds__(256) void xfrag_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                   int64_t ldx, uint16_t* __restrict__ Xf) {
  xfrag_block(X, M, K, ldx, Xf, blockIdx.x, threadIdx.x);
}

}  // namespace

namespace {
// compute units of the current device, queried once per device (the persistent grid's size)
int64_t device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  int v = dev < kMaxDevices ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (v <= 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) cus = 256;
    v = cus;
    if (dev < kMaxDevices) cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}
// blocks of the persistent kernel (one per CU, a multiple of 8), or 0 when the pipelined kernel
// runs instead: bf16 operands, K / 32 a multiple of 8 and at least 16, and at least two tiles
// per block
int64_t persistent_blocks(bool xf32, bool wf32, int64_t K, const SearchPlan& plan, int n_grid) {
  const int64_t total = plan.tiles * n_grid;
  static_assert(PKC * 8 == 256, "persistent_k: K / 32 a multiple of 8 and at least 16");
  if (xf32 || wf32 || !persistent_k(K) || total >= (int64_t)INT32_MAX) return 0;
  const int64_t P = device_cus() / 8 * 8;
  return P >= 8 && total >= 2 * P ? P : 0;
}
}  // namespace

bool search_persistent(bool xf32, bool wf32, int64_t K, const SearchPlan& plan, int n_grid) {
  return persistent_blocks(xf32, wf32, K, plan, n_grid) > 0;
}

hipError_t launch_xfrag(const uint16_t* X, int64_t M, int64_t K, int64_t ldx, uint16_t* Xf, hipStream_t st) {
  if (K % 64 != 0) return hipErrorInvalidValue;
  const int64_t blocks = (M + 31) / 32 * (K / 64);
  if (blocks <= 0 || blocks >= (int64_t)INT32_MAX) return hipErrorInvalidValue;
  xfrag_kernel<<<(unsigned)blocks, 256, 0, st>>>(X, M, K, ldx, Xf);
  return hipGetLastError();
}

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

hipError_t launch_search_fused(const void* X, const uint16_t* Xf, bool xf32, int64_t M, int64_t ldx,
                               const WSegs& W, bool wf32, int64_t K, const float* s_tab,
                               const float* rs_tab, const float2* sr_tab, const float2* params,
                               int n_grid, const SearchPlan& plan, double* partial, hipStream_t st) {
  const int64_t per_xcd = plan.blocks / 8;
  const dim3 grid((unsigned)plan.blocks);
#define AWQ_LAUNCH(XF, WF)                                                                  \
  search_fused_kernel<XF, WF><<<grid, THREADS, 0, st>>>(X, M, ldx, W, K, s_tab, rs_tab, params, \
                                                        n_grid, plan.nt, plan.tiles, per_xcd,   \
                                                        partial)
  if (Xf != nullptr) {
    const int64_t pb = persistent_blocks(xf32, wf32, K, plan, n_grid);
    if (pb <= 0) return hipErrorInvalidValue;  // the caller checks search_persistent first
    if (W.count == 1)
      search_persistent_kernel<false><<<(unsigned)pb, THREADS, 0, st>>>(
          Xf, (M + 31) / 32 * 32, W, K, sr_tab, params, n_grid, plan.nt, plan.tiles, per_xcd, partial);
    else
      search_persistent_kernel<true><<<(unsigned)pb, THREADS, 0, st>>>(
          Xf, (M + 31) / 32 * 32, W, K, sr_tab, params, n_grid, plan.nt, plan.tiles, per_xcd, partial);
    return hipGetLastError();
  }
  if (!xf32 && !wf32) {
    search_pipelined_kernel<<<grid, THREADS, 0, st>>>(static_cast<const uint16_t*>(X), M, ldx, W, K, sr_tab,
                                                      params, n_grid, plan.nt, plan.tiles, per_xcd, partial);
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

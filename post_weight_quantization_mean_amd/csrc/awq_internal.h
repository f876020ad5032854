// Internal declarations shared by the HIP translation units of libawq (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

constexpr int kGroup = 128;  // quantization group along K
constexpr int kQMax = 15;    // unsigned 4-bit codes 0..15

// Flag bits, identical to the AWQ_FLAG_* values of the public header.
constexpr uint32_t kFlagNonfiniteX = 0x1u;
constexpr uint32_t kFlagNonfiniteW = 0x2u;
constexpr uint32_t kFlagScaleRange = 0x4u;
constexpr uint32_t kFlagF16Range = 0x8u;
constexpr uint32_t kFlagNonfiniteLoss = 0x10u;

// ---- statistic -------------------------------------------------------------------------
struct StatsPlan {
  int col_blocks;  // blocks across K
  int splits;      // interleaved row splits (partials per column)
};
StatsPlan stats_plan(int64_t M, int64_t K, bool f32);
hipError_t launch_stats(const void* X, bool f32, int64_t M, int64_t K, int64_t ldx, float* a_out,
                        double* partial, const StatsPlan& plan, uint32_t* flags, hipStream_t st);

// ---- lane permutations (DPP: plain VALU operands, no LDS traffic) -------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]: lane i reads lane i ^ 1
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]: lane i reads lane i ^ 2
constexpr int kDppHalfMirror = 0x141;  // within 8 lanes, lane i reads lane 7 - i
constexpr int kDppMirror = 0x140;      // within 16 lanes, lane i reads lane 15 - i
// max / min over each group of four, or of sixteen, consecutive lanes (every lane gets it)
__device__ __forceinline__ float max4(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  return fmaxf(x, dpp<kDppXor2>(x));
}
__device__ __forceinline__ float min4(float x) {
  x = fminf(x, dpp<kDppXor1>(x));
  return fminf(x, dpp<kDppXor2>(x));
}
__device__ __forceinline__ float max16(float x) {
  x = max4(x);
  x = fmaxf(x, dpp<kDppHalfMirror>(x));
  return fmaxf(x, dpp<kDppMirror>(x));
}
__device__ __forceinline__ float min16(float x) {
  x = min4(x);
  x = fminf(x, dpp<kDppHalfMirror>(x));
  return fminf(x, dpp<kDppMirror>(x));
}

// sum over the 64 lanes of a wave, the same value in every lane: DPP butterflies within each
// 16-lane row, then the four row sums read from lanes 0, 16, 32, 48 (no LDS round trip)
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  x += dpp<kDppMirror>(x);
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
  const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
  const float d = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
  return (a + b) + (c + d);
}

// ---- search ----------------------------------------------------------------------------
constexpr int kSearchBM = 512;  // tokens per block tile
constexpr int kSearchBN = 128;  // output channels per block tile

// Group ranges (Delta, z) of every (candidate, group, output channel) live in the workspace
// as float2 [n_grid][K/128][Npad] with Npad = N rounded up to 128.  Within each 128-channel
// tile, channel r = 32 w + 16 i + j (w < 4, i < 2, j < 16) sits at slot 32 w + 2 j + i, so
// rows r and r + 16 are side by side and one 16-byte load gives a thread the ranges of both
// rows it quantizes.
__host__ __device__ inline int64_t padded_n(int64_t N) { return (N + 127) / 128 * 128; }
__host__ __device__ inline int64_t range_slot(int64_t n) {
  const int64_t r = n % 128;
  return (n / 128) * 128 + (r / 32) * 32 + 2 * (r % 16) + (r % 32) / 16;
}

// Projections that read the same X and share one scale vector (query/key/value, gate/up) are
// searched as one layer: their weights are segments of one row space, each padded to a whole
// number of 128-row tiles so that a tile never mixes two weights.  Passed to kernels by value
// and read with constant indices only (a run-time index into kernel arguments would copy them
// to scratch memory).
constexpr int kMaxWSegs = 8;
struct WSegs {
  const void* w[kMaxWSegs];
  int64_t ldw[kMaxWSegs];
  int64_t n[kMaxWSegs];              // rows of each weight
  int64_t tile0[kMaxWSegs + 1];      // first 128-row tile of each weight; tile0[count] = all tiles
  int count;
};
struct WSel {
  const void* w;
  int64_t ldw, n;  // the tile's weight, its row stride and rows
  int64_t n0;      // first row of the tile within that weight
};
__host__ __device__ inline WSel select_wseg(const WSegs& S, int64_t tile_n) {
  WSel r{S.w[0], S.ldw[0], S.n[0], tile_n * 128};
#pragma unroll
  for (int i = 1; i < kMaxWSegs; ++i)
    if (i < S.count && tile_n >= S.tile0[i]) r = WSel{S.w[i], S.ldw[i], S.n[i], (tile_n - S.tile0[i]) * 128};
  return r;
}

struct SearchPlan {
  int64_t mt, nt;    // tiles along M and N
  int64_t tiles;     // mt * nt
  int64_t blocks;    // launched blocks (multiple of 8)
  int64_t groups;    // K / 128
};
// N: rows of the padded row space (the sum of the weights' rows, each rounded up to 128)
SearchPlan search_plan(int64_t M, int64_t K, int64_t N, int n_grid);

// s_tab, rs_tab: fp32 [n_grid, K]; sr_tab: the same pairs interleaved, float2 [n_grid, K]
hipError_t launch_scale_table(const float* a, int64_t K, int n_grid, float* s_tab, float* rs_tab,
                              float2* sr_tab, uint32_t* flags, hipStream_t st);
// params: float2 [n_grid, K/128, NP] over the padded row space of NP rows; one launch per
// weight, whose rows start at padded row row_base (a multiple of 128)
hipError_t launch_group_range(const void* W, bool wf32, int64_t N, int64_t K, int64_t ldw,
                              const float* s_tab, int n_grid, float2* params, int64_t row_base,
                              int64_t NP, uint32_t* flags, hipStream_t st);
// The persistent search kernel (one block per CU carrying its pipeline across tiles) takes bf16
// X and W, K a multiple of 256 and at least 512 (persistent_k), and at least two tiles per CU.
// It reads X from a copy in fragment order (launch_xfrag): bf16 [round_up(M, 32), K], the
// 16 bytes of lane l of the MFMA operand for rows 32 rb.. and channels 16 kb.. at
// ((rb K/16 + kb) 64 + l) 16 bytes, rows past M zero.  It writes 4 fp64 sums per (candidate,
// tile), one per wave; the other kernels write 1 (the workspace holds 4 for every tile).
inline bool persistent_k(int64_t K) { return K % 256 == 0 && K >= 512; }
bool search_persistent(bool xf32, bool wf32, int64_t K, const SearchPlan& plan, int n_grid);
hipError_t launch_xfrag(const uint16_t* X, int64_t M, int64_t K, int64_t ldx, uint16_t* Xf, hipStream_t st);
// One block (256 threads) of that copy: rows 32 rb .. + 31 and channels 64 cb .. + 63 of X (four
// fragments, 4 KiB), with rb, cb from block index b; thread t reads 16 bytes (t % 8) of row
// 32 rb + t / 8, so eight lanes read one 128-byte run of a row.  The 16-byte piece of row
// 32 rb + l % 32, channels 16 kb + 8 (l / 32) .. + 7 goes to byte ((rb K/16 + kb) 64 + l) 16 of
// Xf; rows M .. Mp - 1 are zero.
__device__ __forceinline__ void xfrag_block(const uint16_t* __restrict__ X, int64_t M, int64_t K, int64_t ldx,
                                            uint16_t* __restrict__ Xf, int64_t b, int t) {
  const int64_t kc = K / 64;
  const int64_t rb = b / kc, cb = b - rb * kc;
  const int rl = t >> 3, piece = t & 7;
  const int64_t row = rb * 32 + rl;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (row < M) v = *reinterpret_cast<const uint4*>(X + row * ldx + cb * 64 + piece * 8);
  const int64_t frag_index = rb * (K / 16) + cb * 4 + (piece >> 1);
  const int l = rl + 32 * (piece & 1);
  *reinterpret_cast<uint4*>(Xf + (frag_index * 64 + l) * 8) = v;
}
// The scale table and that copy in one launch (they are independent): the scale table's few,
// latency-bound blocks first, then the copy's blocks, which run beside them.
hipError_t launch_scale_table_xfrag(const float* a, int64_t K, int n_grid, float* s_tab, float* rs_tab,
                                    float2* sr_tab, uint32_t* flags, const uint16_t* X, int64_t M,
                                    int64_t ldx, uint16_t* Xf, hipStream_t st);
// Xf: the fragment-ordered copy of X when search_persistent(...) holds (the persistent kernel
// runs), else null (the pipelined kernel for bf16 operands, the plain fused kernel otherwise)
hipError_t launch_search_fused(const void* X, const uint16_t* Xf, bool xf32, int64_t M, int64_t ldx,
                               const WSegs& W, bool wf32, int64_t K, const float* s_tab,
                               const float* rs_tab, const float2* sr_tab, const float2* params,
                               int n_grid, const SearchPlan& plan, double* partial, hipStream_t st);
// Gram form: Tp bf16 [K, 2K], row k' = chunks of 32 columns of G_hi and G_lo interleaved
// (bf16(G) and bf16(G - bf16(G)), G = X^T X for bf16 X [M, K]); when gram_triangular(K), G there
// stands for T = diag(X^T X) + 2 triu(X^T X, 1) (zero below the diagonal), and each candidate
// block's K loop starts at its first row of T
inline bool gram_triangular(int64_t K) { return K > kSearchBM; }
// bytes of fp32 slice sums that launch_gram needs beside Tp (0 when no tile is split)
size_t gram_partial_bytes(int64_t M, int64_t K);
hipError_t launch_gram(const uint16_t* X, int64_t M, int64_t K, int64_t ldx, uint16_t* Tp, float* partial,
                       hipStream_t st);
// the candidate losses' partial sums in the Gram form (plan: search_plan with K rows)
hipError_t launch_search_gram(const uint16_t* Tp, int64_t K, const WSegs& W, const float2* sr_tab,
                              const float2* params, int n_grid, const SearchPlan& plan, double* partial,
                              hipStream_t st);
// partial: per_tile fp64 sums per (candidate, tile): 4 after the persistent kernel, else 1
hipError_t launch_select(const double* partial, int64_t tiles, int n_grid, int64_t M, int64_t N,
                         int64_t K, const float* s_tab, double* losses, int32_t* best,
                         float* s_best, uint32_t* flags, hipStream_t st, int per_tile = 1);

// ---- pack ------------------------------------------------------------------------------
// clip: fp32 [N, K/128] thresholds of the clipped pack, or null
hipError_t launch_pack(const void* W, bool wf32, int64_t N, int64_t K, int64_t ldw, const float* s,
                       const float* clip, int32_t* qweight, uint16_t* scales, uint16_t* zeros,
                       uint32_t* flags, hipStream_t st);

// ---- applying the scales ----------------------------------------------------------------
constexpr int kActGelu = 0;  // the values of the ABI's activation codes
constexpr int kActSilu = 1;
// op 0: A[r, c] /= s[r] (fold into a producer); 1: A[r, c] *= s[c] (scale a consumer);
// 2: Y[r, c] = act(X[r, c]) / s[c].  vec: X (and Y) rows start 16-byte aligned.
hipError_t launch_scale_op(int op, const void* X, void* Y, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                           const float* s, int act, bool vec, uint32_t* flags, hipStream_t st);

// ---- W4A16 products over the artefact -----------------------------------------------------
constexpr int64_t kW4a16GemvMax = 8;  // tokens per decode launch; bf16 X above this runs on MFMA
constexpr int kW4a16BM = 512;         // tokens per prefill tile
// bytes of the operand-order copy of X that the prefill reads X from (bf16 X, more than
// kW4a16GemvMax tokens; the xfrag layout of the search), else 0
size_t w4a16_xcopy_bytes(bool xf32, int64_t M, int64_t K);
// xcopy: w4a16_xcopy_bytes of device memory for that copy, or null (the prefill stages X itself)
hipError_t launch_w4a16(const void* X, bool xf32, int64_t M, int64_t K, int64_t ldx, const int32_t* qweight,
                        const uint16_t* scales, const uint16_t* zeros, int64_t N, float* Y, int64_t ldy,
                        uint16_t* xcopy, hipStream_t st);

// ---- clipping search --------------------------------------------------------------------
constexpr int kClipBM = 512;  // tokens per product tile
constexpr int kClipBN = 128;  // output channels per product tile
// params: float4 [n_clip][K/128][N] (Delta, z, c, 0); rs: fp32 [K]; partial: fp32
// [n_clip][K/128][ceil(M/512)][N]
hipError_t launch_clip(const void* X, bool xf32, int64_t M, int64_t K, int64_t ldx, const void* W,
                       bool wf32, int64_t N, int64_t ldw, const float* s, int n_clip, float* max_val,
                       int32_t* best, double* err, float4* params, float* rs, float* partial,
                       uint32_t* flags, hipStream_t st);

}  // namespace awq

// Step 5 of the hot path: real quantization of S W at the winning scales and packing of the
// codes ("AWQ：为什么 4-bit 权重量化要先观察 Activation", §7: codes, group scales and zero
// points form the artefact; §8: g128 with fp16 scale and fp16 zero costs 4.25 bits/weight;
// "5. 核心模块", §5.3: INT4 codes are usually packed eight per int32).
//
// Exact fp32 contract, bit-identical to its definition: v = W*s (one rounding),
// Delta = max(max v - min v, 1e-5) / 15 and both quotients -min/Delta and v/Delta use
// correctly rounded division, rne() is round-half-to-even.  Each lane packs its codes eight per
// int32 (nibble i <- k = 8j+i).  Bandwidth-bound: 2 bytes of W read and 0.53 bytes written
// per weight.
#include "awq_internal.h"

namespace awq {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Work unit: one (row n, group g), i.e. 128 weights.  Four lanes share a unit, lane q owning
// channels 32 q .. 32 q + 31; a unit's Delta, reciprocal and zero point are formed by its four
// lanes alike and serve 32 values each.  Units are numbered u = n G + g, the order of W, of
// qweight and of scales / zeros in memory.  The grid is persistent: with U units per grid
// iteration (a whole number R of rows, U = R G), iteration t covers units t U .. t U + U - 1,
// so the grid sweeps W as one moving window of R consecutive rows (about 8 MiB), and the
// code, scale and zero stores of neighbouring lanes and waves fill whole cache lines.  As U is
// a multiple of G, a lane keeps one group for the whole kernel and holds that group's 32
// scales in registers.
constexpr int kPackThreads = 256;
constexpr int kPackUnits = kPackThreads / 4;  // units per block per iteration
constexpr int kWaveUnits = 16;                // units per wave per iteration
constexpr int64_t kPackWindow = 32768;  // target units per grid iteration

// Correctly rounded quotients a / b from a reciprocal y = RN(1 / b) and FMA corrections:
// q1 = RN(q0 + RN(a - b q0) y) with q0 = RN(a y) is within one ulp of a / b, so
// r1 = a - b q1 is exact and RN(q1 + r1 y) = RN(a / b) (Markstein's theorem for a
// reciprocal within half an ulp and a quotient within one ulp; b here is positive and
// normal, and quotients below 2^-126 either round to code z or are the tiny Delta floor).
__device__ __forceinline__ float quot(float a, float b, float y) {
  const float q0 = a * y;
  const float q1 = fmaf(fmaf(-q0, b, a), y, q0);
  return fmaf(fmaf(-q1, b, a), y, q1);
}

// The lane's 32 scales (channels k0 .. k0 + 31); a scale that is not finite and positive
// sets the range flag.
__device__ __forceinline__ void load_scales(const float* __restrict__ s, int64_t k0, float (&sc)[32],
                                            uint32_t& bad) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float4 sv = *reinterpret_cast<const float4*>(s + k0 + 4 * t);
    sc[4 * t] = sv.x; sc[4 * t + 1] = sv.y; sc[4 * t + 2] = sv.z; sc[4 * t + 3] = sv.w;
  }
#pragma unroll
  for (int i = 0; i < 32; ++i)
    if (!(sc[i] > 0.0f) || isinf(sc[i])) bad |= kFlagScaleRange;
}

// Quantize the lane's 32 weights w of unit (n, g) and store its four code words (and, lane
// q = 0, the unit's scale and zero point).  All four lanes of the unit's quad must be active.
// CLIP: the scaled weights are first clamped to [-clip[n G + g], clip[n G + g]] (the
// threshold chosen by the clipping search); a negative or non-finite threshold sets the range
// flag.
template <bool CLIP>
__device__ __forceinline__ void encode_unit(const float (&w)[32], const float (&sc)[32], int64_t n,
                                            int64_t g, int q, int64_t K, const float* __restrict__ clip,
                                            int32_t* __restrict__ qweight, uint16_t* __restrict__ scales,
                                            uint16_t* __restrict__ zeros, uint32_t& bad) {
  const int64_t G = K / kGroup;
  float c = 0.0f;
  if constexpr (CLIP) {
    c = clip[n * G + g];
    if (!(c >= 0.0f) || isinf(c)) bad |= kFlagScaleRange;
  }
  float v[32];
  float mx = -INFINITY, mn = INFINITY;
  bool nan = false;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    v[i] = w[i] * sc[i];  // s is finite and positive: a non-finite w gives a non-finite v
  }
#pragma unroll
  for (int i = 0; i < 32; i += 2) nan |= __builtin_isunordered(v[i], v[i + 1]);
  if (nan) bad |= kFlagNonfiniteW;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if constexpr (CLIP) v[i] = fminf(fmaxf(v[i], -c), c);  // exact
    mx = fmaxf(mx, v[i]);  // an Inf reaches the range
    mn = fminf(mn, v[i]);
  }
  mx = max4(mx);
  mn = min4(mn);
  const float range = mx - mn;
  if (!isfinite(range)) bad |= kFlagNonfiniteW;
  const float delta = quot(fmaxf(range, 1e-5f), 15.0f, 1.0f / 15.0f);  // RN(range' / 15)
  const float y = 1.0f / delta;
  const int z = (int)fminf(fmaxf(rintf(quot(-mn, delta, y)), 0.0f), 15.0f);
  const float zf = (float)z;
  // rne(RN(v / Delta)) + z from u = RN(v y + z) (one FMA).  With A = |v / Delta|,
  // y = (1 + e1) / Delta and u = (v y + z)(1 + e2), |e1|, |e2| <= 2^-24, so
  // |u - (v / Delta + z)| <= 2^-24 (2A + z) (1 + 2^-23), and |RN(v / Delta) - v / Delta| <=
  // 2^-24 A: u is within 2^-24 (3A + 16) of RN(v / Delta) + z.  When every u lies farther than
  // m = (|v|max y + 16) 2^-21 (> 2.6x that bound) from a half-integer, i.e.
  // |u - rint u| <= 0.5 - m, RN(v / Delta) + z lies strictly on the same side, is no tie, and
  // rint(u) = rne(RN(v / Delta)) + z.  Otherwise the lane forms its 32 quotients exactly: on
  // bf16 weights with smoothly varying scales about one lane in 10^3, with s = 1 (where exact
  // ties RN(v / Delta) = k + 1/2 occur in about 0.2% of the values) one lane in 16.
  float r[32];
  float far = 0.0f;  // max |u - rint(u)|; u - rint(u) is exact in fp32
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float u = fmaf(v[i], y, zf);
    r[i] = rintf(u);
    far = fmaxf(far, fabsf(u - r[i]));
  }
  if (far > 0.5f - (fmaxf(fabsf(mx), fabsf(mn)) * y + 16.0f) * 0x1p-21f) {
#pragma unroll
    for (int i = 0; i < 32; ++i) r[i] = rintf(quot(v[i], delta, y)) + zf;
  }
  // code = clamp(r, 0, 15); bytes of lo / hi hold the even / odd codes of a word, and
  // lo | hi << 4 puts code i at nibble i
  uint32_t word[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_fmed3f(r[8 * j + 2 * i], 0.0f, 15.0f), i, lo);
      hi = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_amdgcn_fmed3f(r[8 * j + 2 * i + 1], 0.0f, 15.0f), i, hi);
    }
    word[j] = lo | (hi << 4);
  }
  *reinterpret_cast<uint4*>(qweight + n * (K / 8) + g * 16 + 4 * q) = make_uint4(word[0], word[1], word[2], word[3]);
  if (q == 0) {
    const _Float16 d16 = (_Float16)delta;  // round to nearest even
    if (isinf((float)d16)) bad |= kFlagF16Range;
    scales[n * G + g] = __builtin_bit_cast(uint16_t, d16);
    zeros[n * G + g] = __builtin_bit_cast(uint16_t, (_Float16)z);
  }
}

// bf16 W.  A wave's 16 units of one iteration are 16 x 256 bytes, contiguous in memory when
// they lie in one row (or rows are dense).  The wave reads them with four load instructions
// of 1 KiB each (lane l, instruction t: 16-byte slot 64 t + l, i.e. piece l % 16 of the
// wave's unit 4 t + l / 16), so every instruction fills eight whole cache lines; loading each
// lane's own 64 bytes instead made every instruction touch 32 lines, a quarter of each, and
// ran the kernel 1.3x slower (measured).  The slots then pass through a wave-private 4 KiB of
// LDS into the four-lanes-per-unit layout.  LDS slot s is stored at s ^ ((s >> 4) & 15):
// both the slot-order writes and the unit-order reads hit 16 distinct 16-byte bank groups per
// 16 lanes.  Two iterations of loads are in flight per wave.
template <bool CLIP>
__global__ __launch_bounds__(kPackThreads) void pack_bf16_kernel(
    const uint16_t* __restrict__ W, int64_t N, int64_t K, int64_t ldw, const float* __restrict__ s,
    const float* __restrict__ clip, int64_t R, int32_t* __restrict__ qweight,
    uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros, uint32_t* __restrict__ flags) {
  __shared__ __attribute__((aligned(16))) u32x4 lds[kPackThreads / 64][kWaveUnits * 16];
  const int64_t G = K / kGroup;
  const int64_t U = R * G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t uw = (int64_t)blockIdx.x * kPackUnits + wave * kWaveUnits;  // wave's first unit
  if (uw >= U) return;  // a spare wave of the last block (no barrier in this kernel)
  const int q = lane & 3;
  const int64_t ui = uw + (lane >> 2);
  const bool mine = ui < U;  // this quad's unit exists
  const int64_t g = ui % G;
  const int64_t n0 = ui / G;

  uint32_t bad = 0;
  float sc[32];
  load_scales(s, g * kGroup + 32 * q, sc, bad);

  // the four slots this lane loads: unit j = 4 t + lane / 16 of the wave, piece lane % 16
  // W through a buffer resource of N ldw 2 bytes (< 2^31, host-checked): 32-bit byte offsets
  // that advance by a scalar row step, and slots past the last row read zero in hardware, so
  // the loads need neither a per-slot row test nor a branch (a guarded load compiles to a
  // branch, after which the wait counts could no longer keep both iterations in flight).
  // Slots of units that do not exist start at the end of W and stay past it.
  const uint32_t wbytes = (uint32_t)(N * ldw * 2);
  const __amdgpu_buffer_rsrc_t wrsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)W, (short)0, (int)wbytes, 0x00020000);
  uint32_t boff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t uj = uw + 4 * t + (lane >> 4);
    boff[t] = uj < U ? (uint32_t)(((uj / G) * ldw + (uj % G) * kGroup + 8 * (lane & 15)) * 2) : wbytes;
  }
  const uint32_t rowb = (uint32_t)(ldw * 2);
  auto phys = [](int slot) { return slot ^ ((slot >> 4) & 15); };
  auto issue = [&](u32x4* raw, int64_t kk) {  // loads of iteration kk (rows + kk), non-temporal
#pragma unroll
    for (int t = 0; t < 4; ++t)
      raw[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             wrsrc, (int)(boff[t] + (uint32_t)kk * rowb), 0, 2));
  };
  auto process = [&](u32x4* raw, int64_t kk) {
    // slot order -> unit order through LDS (a wave's LDS operations complete in issue order)
#pragma unroll
    for (int t = 0; t < 4; ++t) lds[wave][phys(64 * t + lane)] = raw[t];
    __builtin_amdgcn_wave_barrier();
    u32x4 mw[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) mw[t] = lds[wave][phys((lane >> 2) * 16 + 4 * q + t)];
    __builtin_amdgcn_wave_barrier();
    issue(raw, kk + 2 * R);  // two iterations ahead, in flight during this one's math
    const int64_t n = n0 + kk;
    if (mine && n < N) {
      float w[32];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t uu[4] = {mw[t].x, mw[t].y, mw[t].z, mw[t].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          w[8 * t + 2 * h] = __uint_as_float(uu[h] << 16);
          w[8 * t + 2 * h + 1] = __uint_as_float(uu[h] & 0xffff0000u);
        }
      }
      encode_unit<CLIP>(w, sc, n, g, q, K, clip, qweight, scales, zeros, bad);
    }
  };
  // the wave's first row is uw / G: the loop runs while any of its units has a row left
  const int64_t wrow = uw / G;
  u32x4 ra[4], rb[4];
  issue(ra, 0);
  __builtin_amdgcn_sched_barrier(0);  // ra's loads strictly before rb's, as in the loop
  issue(rb, R);
  for (int64_t kk = 0; wrow + kk < N; kk += 2 * R) {
    process(ra, kk);
    process(rb, kk + R);  // unconditional (its units past N encode nothing): a branch here would
                          // leave the wait counts at the loop head unable to keep rb in flight
  }
  if (bad) atomicOr(flags, bad);
}

// fp32 W (small layers and mixed inputs): each lane loads its own 128 bytes per row, one row
// ahead.
template <bool CLIP>
__global__ __launch_bounds__(kPackThreads) void pack_f32_kernel(
    const float* __restrict__ W, int64_t N, int64_t K, int64_t ldw, const float* __restrict__ s,
    const float* __restrict__ clip, int64_t R, int32_t* __restrict__ qweight,
    uint16_t* __restrict__ scales, uint16_t* __restrict__ zeros, uint32_t* __restrict__ flags) {
  const int64_t G = K / kGroup;
  const int64_t ui = (int64_t)blockIdx.x * kPackUnits + (threadIdx.x >> 2);
  if (ui >= R * G) return;  // the last block's spare units (whole quads; no barrier here)
  const int q = threadIdx.x & 3;
  const int64_t g = ui % G;
  const int64_t k0 = g * kGroup + 32 * q;
  uint32_t bad = 0;
  float sc[32];
  load_scales(s, k0, sc, bad);
  float4 raw[8];
  auto load = [&](int64_t row) {
    const float4* p = reinterpret_cast<const float4*>(W + row * ldw + k0);
#pragma unroll
    for (int t = 0; t < 8; ++t) raw[t] = p[t];
  };
  int64_t n = ui / G;
  if (n < N) load(n);
  for (; n < N; n += R) {
    float w[32];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      w[4 * t] = raw[t].x; w[4 * t + 1] = raw[t].y; w[4 * t + 2] = raw[t].z; w[4 * t + 3] = raw[t].w;
    }
    if (n + R < N) load(n + R);
    encode_unit<CLIP>(w, sc, n, g, q, K, clip, qweight, scales, zeros, bad);
  }
  if (bad) atomicOr(flags, bad);
}

}  // namespace

hipError_t launch_pack(const void* W, bool wf32, int64_t N, int64_t K, int64_t ldw, const float* s,
                       const float* clip, int32_t* qweight, uint16_t* scales, uint16_t* zeros,
                       uint32_t* flags, hipStream_t st) {
  const int64_t G = K / kGroup;
  int64_t R = (kPackWindow + G / 2) / G;  // rows per grid iteration
  if (R < 1) R = 1;
  if (R > N) R = N;
  const unsigned blocks = (unsigned)((R * G + kPackUnits - 1) / kPackUnits);
  const float* Wf = static_cast<const float*>(W);
  const uint16_t* Wh = static_cast<const uint16_t*>(W);
  if (wf32 && clip)
    pack_f32_kernel<true><<<blocks, kPackThreads, 0, st>>>(Wf, N, K, ldw, s, clip, R, qweight, scales, zeros, flags);
  else if (wf32)
    pack_f32_kernel<false><<<blocks, kPackThreads, 0, st>>>(Wf, N, K, ldw, s, clip, R, qweight, scales, zeros, flags);
  else {
    // the bf16 kernel addresses W with 32-bit offsets: row slabs of at most 2^30 bytes, so that
    // offsets two iterations past a slab's end stay below 2^31
    int64_t slab = ((int64_t)1 << 30) / (ldw * 2);
    if (slab < 1) slab = 1;
    for (int64_t r0 = 0; r0 < N; r0 += slab) {
      const int64_t n = N - r0 < slab ? N - r0 : slab;
      const int64_t Rs = R < n ? R : n;
      const unsigned bs = (unsigned)((Rs * G + kPackUnits - 1) / kPackUnits);
      const float* cs = clip ? clip + r0 * G : nullptr;
      if (clip)
        pack_bf16_kernel<true><<<bs, kPackThreads, 0, st>>>(Wh + r0 * ldw, n, K, ldw, s, cs, Rs, qweight + r0 * (K / 8),
                                                            scales + r0 * G, zeros + r0 * G, flags);
      else
        pack_bf16_kernel<false><<<bs, kPackThreads, 0, st>>>(Wh + r0 * ldw, n, K, ldw, s, cs, Rs, qweight + r0 * (K / 8),
                                                             scales + r0 * G, zeros + r0 * G, flags);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipGetLastError();
}

}  // namespace awq

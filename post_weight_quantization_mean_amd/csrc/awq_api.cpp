// Host side of libawq: argument validation, workspace carving and kernel launches behind the
// C ABI declared in include/awq.h.  Validation is plain host code that runs before any HIP
// call, so every argument error is reported without touching the device.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <mutex>

#include "awq.h"
#include "awq_internal.h"

namespace {

using awq::kGroup;

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool valid_dtype(int t) { return t == AWQ_DTYPE_F32 || t == AWQ_DTYPE_BF16; }
int64_t dsize(int t) { return t == AWQ_DTYPE_F32 ? 4 : 2; }

// a * b without overflow (both non-negative), else -1
int64_t mul_ok(int64_t a, int64_t b) {
  if (a < 0 || b < 0) return -1;
  if (a != 0 && b > INT64_MAX / a) return -1;
  return a * b;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Common checks of one [rows, K] operand with row stride ld.
int check_matrix(const void* p, int dtype, int64_t rows, int64_t K, int64_t ld) {
  if (p == nullptr) return AWQ_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return AWQ_ERR_UNSUPPORTED;
  if (rows <= 0 || K <= 0 || ld < K) return AWQ_ERR_INVALID_ARG;
  if (K % kGroup != 0) return AWQ_ERR_SHAPE;
  const int64_t bytes = mul_ok(mul_ok(rows, ld), dsize(dtype));
  if (bytes < 0) return AWQ_ERR_SHAPE;
  // 16-byte vector loads: the base and every row start must be 16-byte aligned
  if (!aligned16(p) || (ld * dsize(dtype)) % 16 != 0) return AWQ_ERR_INVALID_ARG;
  return AWQ_OK;
}

int map_hip(hipError_t e) { return e == hipSuccess ? AWQ_OK : AWQ_ERR_HIP; }

struct SearchLayout {
  size_t s_tab, rs_tab, sr_tab, params, partial, total;
};

bool search_layout(int64_t M, int64_t K, int64_t N, int n_grid, SearchLayout* out) {
  const awq::SearchPlan plan = awq::search_plan(M, K, N, n_grid);
  const int64_t tab = mul_ok(mul_ok(n_grid, K), 4);
  const int64_t par = mul_ok(mul_ok(mul_ok(n_grid, awq::padded_n(N)), K / kGroup), 8);
  const int64_t part = mul_ok(mul_ok(n_grid, plan.tiles), 8 * 4);  // up to four sums per tile
  if (tab < 0 || par < 0 || part < 0) return false;
  SearchLayout L;
  L.s_tab = 0;
  L.rs_tab = L.s_tab + align_up((size_t)tab);
  L.sr_tab = L.rs_tab + align_up((size_t)tab);
  L.params = L.sr_tab + align_up((size_t)tab * 2);
  L.partial = L.params + align_up((size_t)par);
  L.total = L.partial + align_up((size_t)part);
  *out = L;
  return true;
}

// Bytes of the fragment-ordered copy of X that the persistent search kernel reads (bf16
// [round_up(M, 32), K]), or 0 when K does not take that kernel, -1 on overflow.
int64_t xfrag_bytes(int64_t M, int64_t K) {
  if (!awq::persistent_k(K)) return 0;
  if (M > INT64_MAX - 31) return -1;
  return mul_ok(mul_ok((M + 31) / 32 * 32, K), 2);
}

// A search workspace of `total` bytes plus room for the copy of X where K takes it (0 on
// overflow).
size_t with_xfrag(size_t total, int64_t M, int64_t K) {
  const int64_t xb = xfrag_bytes(M, K);
  if (xb < 0) return 0;
  return total + align_up((size_t)xb);
}

// Checks of an elementwise operand [rows, cols] with row stride ld (no group constraint).
int check_elems(const void* p, int dtype, int64_t rows, int64_t cols, int64_t ld) {
  if (p == nullptr) return AWQ_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return AWQ_ERR_UNSUPPORTED;
  if (rows <= 0 || cols <= 0 || ld < cols) return AWQ_ERR_INVALID_ARG;
  if (mul_ok(mul_ok(rows, ld), dsize(dtype)) < 0) return AWQ_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(p) % (uintptr_t)dsize(dtype)) != 0) return AWQ_ERR_INVALID_ARG;
  return AWQ_OK;
}

int scale_op(int op, const void* X, void* Y, int dtype, int64_t rows, int64_t cols, int64_t ld, const float* s,
             int act, uint32_t* flags, awq_stream_t stream) {
  int st = check_elems(X, dtype, rows, cols, ld);
  if (st != AWQ_OK) return st;
  if (Y == nullptr || s == nullptr || flags == nullptr) return AWQ_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(Y) % (uintptr_t)dsize(dtype)) != 0 || (reinterpret_cast<uintptr_t>(s) & 3u) != 0)
    return AWQ_ERR_INVALID_ARG;
  if (op == 2 && act != awq::kActGelu && act != awq::kActSilu) return AWQ_ERR_UNSUPPORTED;
  const bool vec = aligned16(X) && aligned16(Y) && (ld * dsize(dtype)) % 16 == 0;
  return map_hip(awq::launch_scale_op(op, X, Y, dtype == AWQ_DTYPE_BF16, rows, cols, ld, s, act, vec, flags,
                                      reinterpret_cast<hipStream_t>(stream)));
}

struct ClipLayout {
  size_t rs, params, partial, total;
};

bool clip_layout(int64_t M, int64_t K, int64_t N, int n_clip, ClipLayout* out) {
  const int64_t G = K / kGroup;
  const int64_t mtiles = (M + awq::kClipBM - 1) / awq::kClipBM;
  const int64_t rs = mul_ok(K, 4);
  const int64_t par = mul_ok(mul_ok(mul_ok(n_clip, G), N), 16);
  const int64_t part = mul_ok(mul_ok(mul_ok(mul_ok(n_clip, G), mtiles), N), 4);
  if (rs < 0 || par < 0 || part < 0) return false;
  ClipLayout L;
  L.rs = 0;
  L.params = L.rs + align_up((size_t)rs);
  L.partial = L.params + align_up((size_t)par);
  L.total = L.partial + align_up((size_t)part);
  *out = L;
  return true;
}

// ---- the allocation-free search: its workspace in a static device array -------------------
// awq_search_static is for callers that cannot allocate device memory.  Its workspace is this
// array: AWQ_STATIC_SCRATCH_BYTES on every GPU the library is used on, held from its module
// load on that GPU until the process ends.  Every call on one GPU shares that GPU's copy.
__device__ __align__(256) unsigned char scratch[AWQ_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // the device address of `scratch` on each device, once known

// The device address of `scratch` on the current device.  In host code the array's name is a
// host-side stand-in, not a device address, so it is looked up once per device, with that
// device current, and only this pointer is ever handed to kernels.
hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

AWQ_API int awq_abi_version(void) { return AWQ_ABI_VERSION; }

AWQ_API const char* awq_status_string(int status) {
  switch (status) {
    case AWQ_OK: return "ok";
    case AWQ_ERR_INVALID_ARG: return "invalid argument (null pointer, size, stride or alignment)";
    case AWQ_ERR_SHAPE: return "shape error (K not a multiple of the group size, or size overflow)";
    case AWQ_ERR_UNSUPPORTED: return "unsupported dtype or group size";
    case AWQ_ERR_WORKSPACE: return "workspace missing or too small";
    case AWQ_ERR_HIP: return "HIP runtime or launch error";
    case AWQ_ERR_SCRATCH:
      return "the call needs more workspace than the static scratch of awq_search_static holds "
             "(AWQ_STATIC_SCRATCH_BYTES); use awq_search with a workspace";
    default: return "unknown status";
  }
}

AWQ_API size_t awq_stats_workspace_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0) return 0;
  const awq::StatsPlan p = awq::stats_plan(M, K, false);
  const awq::StatsPlan q = awq::stats_plan(M, K, true);
  const int64_t splits = p.splits > q.splits ? p.splits : q.splits;
  const int64_t bytes = mul_ok(mul_ok(splits, K), 8);
  return bytes < 0 ? 0 : align_up((size_t)bytes);
}

AWQ_API int awq_stats(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx, float* a_out,
                      void* ws, size_t ws_bytes, uint32_t* flags, awq_stream_t stream) {
  int st = check_matrix(X, x_dtype, M, K, ldx);
  if (st != AWQ_OK) return st;
  if (a_out == nullptr || flags == nullptr) return AWQ_ERR_INVALID_ARG;
  const size_t need = awq_stats_workspace_bytes(M, K);
  if (need == 0) return AWQ_ERR_SHAPE;
  if (ws == nullptr || ws_bytes < need) return AWQ_ERR_WORKSPACE;
  const bool f32 = x_dtype == AWQ_DTYPE_F32;
  const awq::StatsPlan plan = awq::stats_plan(M, K, f32);
  return map_hip(awq::launch_stats(X, f32, M, K, ldx, a_out, static_cast<double*>(ws), plan, flags,
                                   reinterpret_cast<hipStream_t>(stream)));
}

AWQ_API size_t awq_search_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t group,
                                          int32_t n_grid) {
  if (M <= 0 || K <= 0 || N <= 0 || group != kGroup || K % kGroup != 0 || n_grid < 1 || n_grid > 64)
    return 0;
  SearchLayout L;
  if (!search_layout(M, K, N, n_grid, &L)) return 0;
  return with_xfrag(L.total, M, K);
}

}  // extern "C"

namespace {

// The search over one layer whose weight is given as n_weights row blocks that share X
// (a single weight is the case n_weights = 1).  Ws, Ns, ldws: host arrays.
int search_impl(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx, const void* const* Ws,
                int w_dtype, const int64_t* Ns, const int64_t* ldws, int32_t n_weights, const float* a,
                int32_t group, int32_t n_grid, double* losses_out, int32_t* best_out, float* s_best_out,
                float* s_table_out, void* ws, size_t ws_bytes, uint32_t* flags, awq_stream_t stream,
                awq_event_t fused_begin, awq_event_t fused_end, bool gram = false,
                bool static_ws = false) {
  int st = check_matrix(X, x_dtype, M, K, ldx);
  if (st != AWQ_OK) return st;
  if (Ws == nullptr || Ns == nullptr || ldws == nullptr || n_weights < 1 || n_weights > awq::kMaxWSegs)
    return AWQ_ERR_INVALID_ARG;
  awq::WSegs segs{};
  segs.count = n_weights;
  int64_t n_total = 0, tiles = 0;
  for (int i = 0; i < n_weights; ++i) {
    st = check_matrix(Ws[i], w_dtype, Ns[i], K, ldws[i]);
    if (st != AWQ_OK) return st;
    // block-relative buffer offsets are 32-bit: 128 rows of each weight span less than 2^31 bytes
    if (mul_ok(mul_ok(awq::kSearchBN, ldws[i]), dsize(w_dtype)) >= (int64_t)INT32_MAX) return AWQ_ERR_SHAPE;
    segs.w[i] = Ws[i];
    segs.ldw[i] = ldws[i];
    segs.n[i] = Ns[i];
    segs.tile0[i] = tiles;
    tiles += awq::padded_n(Ns[i]) / 128;
    n_total += Ns[i];
  }
  segs.tile0[n_weights] = tiles;
  const int64_t NP = tiles * 128;  // the padded row space
  if (group != kGroup) return AWQ_ERR_UNSUPPORTED;
  if (n_grid < 1 || n_grid > 64) return AWQ_ERR_INVALID_ARG;
  if (a == nullptr || losses_out == nullptr || best_out == nullptr || s_best_out == nullptr ||
      flags == nullptr)
    return AWQ_ERR_INVALID_ARG;
  // 512 rows of X in 32-bit block-relative offsets
  if (mul_ok(mul_ok(awq::kSearchBM, ldx), dsize(x_dtype)) >= (int64_t)INT32_MAX) return AWQ_ERR_SHAPE;
  // one candidate's group ranges (float2 [K/128][NP]) are addressed with 32-bit offsets
  if (mul_ok(mul_ok(K / kGroup, NP), 8) >= (int64_t)INT32_MAX) return AWQ_ERR_SHAPE;
  // Gram form: the product's left operand is Tp [K, 2K] bf16 (G_hi and G_lo interleaved by
  // 32-column chunks); 512 of its rows are addressed with 32-bit offsets
  if (gram && (x_dtype != AWQ_DTYPE_BF16 || w_dtype != AWQ_DTYPE_BF16)) return AWQ_ERR_UNSUPPORTED;
  if (gram && mul_ok(mul_ok(awq::kSearchBM, 2 * K), 2) >= (int64_t)INT32_MAX) return AWQ_ERR_SHAPE;
  const int64_t rows = gram ? K : M;  // rows of the product's left operand
  SearchLayout L;
  if (!search_layout(rows, K, NP, n_grid, &L)) return AWQ_ERR_SHAPE;
  size_t total = L.total, gs_off = 0, gp_off = 0;
  if (gram) {
    const int64_t gsb = mul_ok(mul_ok(2 * K, K), 2);
    if (gsb < 0) return AWQ_ERR_SHAPE;
    gs_off = total;
    total += align_up((size_t)gsb);
    gp_off = total;  // fp32 sums of the G tiles split along the tokens
    total += align_up(awq::gram_partial_bytes(M, K));
  }
  if (static_ws) {
    // every argument is checked above; the first HIP call of this path comes after them
    if (total > (size_t)AWQ_STATIC_SCRATCH_BYTES) return AWQ_ERR_SCRATCH;
    if (!aligned16(a) || (s_table_out != nullptr && !aligned16(s_table_out))) return AWQ_ERR_INVALID_ARG;
    const hipError_t se = static_scratch(&ws);
    if (se != hipSuccess) return AWQ_ERR_HIP;
    ws_bytes = (size_t)AWQ_STATIC_SCRATCH_BYTES;
  }
  if (ws == nullptr || ws_bytes < total) return AWQ_ERR_WORKSPACE;
  if (!aligned16(ws) || !aligned16(a)) return AWQ_ERR_INVALID_ARG;
  if (s_table_out != nullptr && !aligned16(s_table_out)) return AWQ_ERR_INVALID_ARG;
  const bool xf32 = x_dtype == AWQ_DTYPE_F32, wf32 = w_dtype == AWQ_DTYPE_F32;
  const awq::SearchPlan plan = awq::search_plan(rows, K, NP, n_grid);
  // The persistent kernel reads X from a fragment-ordered copy placed after the rest of the
  // workspace; without room for it the pipelined kernel runs (the same losses bit for bit).
  const int64_t xfb = gram ? 0 : xfrag_bytes(M, K);
  const bool persistent = xfb > 0 && ws_bytes >= total + (size_t)xfb &&
                          awq::search_persistent(xf32, wf32, K, plan, n_grid);

  char* base = static_cast<char*>(ws);
  float* s_tab = s_table_out != nullptr ? s_table_out : reinterpret_cast<float*>(base + L.s_tab);
  float* rs_tab = reinterpret_cast<float*>(base + L.rs_tab);
  float2* sr_tab = reinterpret_cast<float2*>(base + L.sr_tab);
  float2* params = reinterpret_cast<float2*>(base + L.params);
  double* partial = reinterpret_cast<double*>(base + L.partial);
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint16_t* Xf = persistent ? reinterpret_cast<uint16_t*>(base + total) : nullptr;  // total: 256-aligned
  uint16_t* Tp = gram ? reinterpret_cast<uint16_t*>(base + gs_off) : nullptr;  // [K, 2K] bf16
  float* gpart = gram ? reinterpret_cast<float*>(base + gp_off) : nullptr;

  // the copy of X shares the scale table's launch (both only read X and a)
  hipError_t e = persistent ? awq::launch_scale_table_xfrag(a, K, n_grid, s_tab, rs_tab, sr_tab, flags,
                                                             static_cast<const uint16_t*>(X), M, ldx, Xf, s)
                            : awq::launch_scale_table(a, K, n_grid, s_tab, rs_tab, sr_tab, flags, s);
  if (e == hipSuccess && gram) e = awq::launch_gram(static_cast<const uint16_t*>(X), M, K, ldx, Tp, gpart, s);
  for (int i = 0; i < n_weights && e == hipSuccess; ++i)
    e = awq::launch_group_range(Ws[i], wf32, Ns[i], K, ldws[i], s_tab, n_grid, params, segs.tile0[i] * 128,
                                NP, flags, s);
  if (e == hipSuccess && fused_begin != nullptr)
    e = hipEventRecord(reinterpret_cast<hipEvent_t>(fused_begin), s);
  if (e == hipSuccess && gram)
    e = awq::launch_search_gram(Tp, K, segs, sr_tab, params, n_grid, plan, partial, s);
  else if (e == hipSuccess)
    e = awq::launch_search_fused(X, Xf, xf32, M, ldx, segs, wf32, K, s_tab, rs_tab, sr_tab, params, n_grid,
                                 plan, partial, s);
  if (e == hipSuccess && fused_end != nullptr)
    e = hipEventRecord(reinterpret_cast<hipEvent_t>(fused_end), s);
  if (e == hipSuccess)
    e = awq::launch_select(partial, plan.tiles, n_grid, M, n_total, K, s_tab, losses_out, best_out,
                           s_best_out, flags, s,
                           persistent ? 4 : 1);
  return map_hip(e);
}

}  // namespace

extern "C" {

AWQ_API int awq_search_timed(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                             const void* W, int w_dtype, int64_t N, int64_t ldw, const float* a,
                             int32_t group, int32_t n_grid, double* losses_out,
                             int32_t* best_out, float* s_best_out, float* s_table_out, void* ws,
                             size_t ws_bytes, uint32_t* flags, awq_stream_t stream,
                             awq_event_t fused_begin, awq_event_t fused_end) {
  const void* Ws[1] = {W};
  return search_impl(X, x_dtype, M, K, ldx, Ws, w_dtype, &N, &ldw, 1, a, group, n_grid, losses_out, best_out,
                     s_best_out, s_table_out, ws, ws_bytes, flags, stream, fused_begin, fused_end);
}

AWQ_API int awq_search(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                       const void* W, int w_dtype, int64_t N, int64_t ldw, const float* a,
                       int32_t group, int32_t n_grid, double* losses_out, int32_t* best_out,
                       float* s_best_out, float* s_table_out, void* ws, size_t ws_bytes,
                       uint32_t* flags, awq_stream_t stream) {
  return awq_search_timed(X, x_dtype, M, K, ldx, W, w_dtype, N, ldw, a, group, n_grid,
                          losses_out, best_out, s_best_out, s_table_out, ws, ws_bytes, flags,
                          stream, nullptr, nullptr);
}

AWQ_API int awq_search_static(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                              const void* W, int w_dtype, int64_t N, int64_t ldw, const float* a,
                              int32_t group, int32_t n_grid, double* losses_out, int32_t* best_out,
                              float* s_best_out, float* s_table_out, uint32_t* flags, awq_stream_t stream) {
  const void* Ws[1] = {W};
  return search_impl(X, x_dtype, M, K, ldx, Ws, w_dtype, &N, &ldw, 1, a, group, n_grid, losses_out, best_out,
                     s_best_out, s_table_out, nullptr, 0, flags, stream, nullptr, nullptr, false, true);
}

AWQ_API size_t awq_search_gram_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t group, int32_t n_grid) {
  if (M <= 0 || K <= 0 || N <= 0 || group != kGroup || K % kGroup != 0 || n_grid < 1 || n_grid > 64 ||
      K > INT64_MAX / 8)
    return 0;
  SearchLayout L;
  if (!search_layout(K, K, N, n_grid, &L)) return 0;
  const int64_t gsb = mul_ok(mul_ok(2 * K, K), 2);
  if (gsb < 0) return 0;
  return L.total + align_up((size_t)gsb) + align_up(awq::gram_partial_bytes(M, K));
}

AWQ_API int awq_search_gram(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx, const void* W,
                            int w_dtype, int64_t N, int64_t ldw, const float* a, int32_t group, int32_t n_grid,
                            double* losses_out, int32_t* best_out, float* s_best_out, float* s_table_out,
                            void* ws, size_t ws_bytes, uint32_t* flags, awq_stream_t stream) {
  const void* Ws[1] = {W};
  return search_impl(X, x_dtype, M, K, ldx, Ws, w_dtype, &N, &ldw, 1, a, group, n_grid, losses_out, best_out,
                     s_best_out, s_table_out, ws, ws_bytes, flags, stream, nullptr, nullptr, true);
}

AWQ_API size_t awq_search_multi_workspace_bytes(int64_t M, int64_t K, const int64_t* Ns, int32_t n_weights,
                                                int32_t group, int32_t n_grid) {
  if (M <= 0 || K <= 0 || Ns == nullptr || n_weights < 1 || n_weights > awq::kMaxWSegs || group != kGroup ||
      K % kGroup != 0 || n_grid < 1 || n_grid > 64)
    return 0;
  int64_t NP = 0;
  for (int i = 0; i < n_weights; ++i) {
    if (Ns[i] <= 0 || Ns[i] > INT64_MAX / 4) return 0;
    NP += awq::padded_n(Ns[i]);
    if (NP < 0 || NP > INT64_MAX / 4) return 0;
  }
  SearchLayout L;
  if (!search_layout(M, K, NP, n_grid, &L)) return 0;
  return with_xfrag(L.total, M, K);
}

AWQ_API int awq_search_multi(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                             const void* const* Ws, int w_dtype, const int64_t* Ns, const int64_t* ldws,
                             int32_t n_weights, const float* a, int32_t group, int32_t n_grid,
                             double* losses_out, int32_t* best_out, float* s_best_out, float* s_table_out,
                             void* ws, size_t ws_bytes, uint32_t* flags, awq_stream_t stream) {
  return search_impl(X, x_dtype, M, K, ldx, Ws, w_dtype, Ns, ldws, n_weights, a, group, n_grid, losses_out,
                     best_out, s_best_out, s_table_out, ws, ws_bytes, flags, stream, nullptr, nullptr);
}

AWQ_API int awq_pack_clipped(const void* W, int w_dtype, int64_t N, int64_t K, int64_t ldw,
                             const float* s, const float* max_val, int32_t group,
                             int32_t* qweight, uint16_t* scales, uint16_t* zeros,
                             uint32_t* flags, awq_stream_t stream) {
  int st = check_matrix(W, w_dtype, N, K, ldw);
  if (st != AWQ_OK) return st;
  if (group != kGroup) return AWQ_ERR_UNSUPPORTED;
  if (s == nullptr || qweight == nullptr || scales == nullptr || zeros == nullptr ||
      flags == nullptr)
    return AWQ_ERR_INVALID_ARG;
  if (!aligned16(s)) return AWQ_ERR_INVALID_ARG;
  if (mul_ok(N, K) < 0) return AWQ_ERR_SHAPE;
  return map_hip(awq::launch_pack(W, w_dtype == AWQ_DTYPE_F32, N, K, ldw, s, max_val, qweight,
                                  scales, zeros, flags, reinterpret_cast<hipStream_t>(stream)));
}

AWQ_API int awq_pack(const void* W, int w_dtype, int64_t N, int64_t K, int64_t ldw,
                     const float* s, int32_t group, int32_t* qweight, uint16_t* scales,
                     uint16_t* zeros, uint32_t* flags, awq_stream_t stream) {
  return awq_pack_clipped(W, w_dtype, N, K, ldw, s, nullptr, group, qweight, scales, zeros, flags,
                          stream);
}

AWQ_API size_t awq_clip_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t group,
                                        int32_t n_clip) {
  if (M <= 0 || K <= 0 || N <= 0 || group != kGroup || K % kGroup != 0 || n_clip < 1 || n_clip > 20)
    return 0;
  ClipLayout L;
  if (!clip_layout(M, K, N, n_clip, &L)) return 0;
  return L.total;
}

AWQ_API int awq_clip(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                     const void* W, int w_dtype, int64_t N, int64_t ldw, const float* s,
                     int32_t group, int32_t n_clip, float* max_val_out, int32_t* best_out,
                     double* err_out, void* ws, size_t ws_bytes, uint32_t* flags,
                     awq_stream_t stream) {
  int st = check_matrix(X, x_dtype, M, K, ldx);
  if (st != AWQ_OK) return st;
  st = check_matrix(W, w_dtype, N, K, ldw);
  if (st != AWQ_OK) return st;
  if (group != kGroup) return AWQ_ERR_UNSUPPORTED;
  if (n_clip < 1 || n_clip > 20) return AWQ_ERR_INVALID_ARG;
  if (s == nullptr || max_val_out == nullptr || flags == nullptr) return AWQ_ERR_INVALID_ARG;
  if (!aligned16(s)) return AWQ_ERR_INVALID_ARG;
  // block-relative 32-bit buffer offsets: 512 rows of X and 128 rows of W
  if (mul_ok(mul_ok(awq::kClipBM, ldx), dsize(x_dtype)) >= (int64_t)INT32_MAX ||
      mul_ok(mul_ok(awq::kClipBN, ldw), dsize(w_dtype)) >= (int64_t)INT32_MAX)
    return AWQ_ERR_SHAPE;
  ClipLayout L;
  if (!clip_layout(M, K, N, n_clip, &L)) return AWQ_ERR_SHAPE;
  if (ws == nullptr || ws_bytes < L.total) return AWQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return AWQ_ERR_INVALID_ARG;
  char* base = static_cast<char*>(ws);
  return map_hip(awq::launch_clip(X, x_dtype == AWQ_DTYPE_F32, M, K, ldx, W, w_dtype == AWQ_DTYPE_F32,
                                  N, ldw, s, n_clip, max_val_out, best_out, err_out,
                                  reinterpret_cast<float4*>(base + L.params),
                                  reinterpret_cast<float*>(base + L.rs),
                                  reinterpret_cast<float*>(base + L.partial), flags,
                                  reinterpret_cast<hipStream_t>(stream)));
}

AWQ_API int awq_fold_rows(void* A, int dtype, int64_t rows, int64_t cols, int64_t lda, const float* s,
                          uint32_t* flags, awq_stream_t stream) {
  return scale_op(0, A, A, dtype, rows, cols, lda, s, 0, flags, stream);
}

AWQ_API int awq_scale_cols(void* W, int dtype, int64_t N, int64_t K, int64_t ldw, const float* s,
                           uint32_t* flags, awq_stream_t stream) {
  return scale_op(1, W, W, dtype, N, K, ldw, s, 0, flags, stream);
}

AWQ_API int awq_scaled_act(const void* X, void* Y, int dtype, int64_t M, int64_t K, int64_t ld, int act,
                           const float* s, uint32_t* flags, awq_stream_t stream) {
  return scale_op(2, X, Y, dtype, M, K, ld, s, act, flags, stream);
}

AWQ_API size_t awq_w4a16_workspace_bytes(int64_t M, int64_t K, int x_dtype) {
  if (M <= 0 || K <= 0 || K % kGroup != 0 || !valid_dtype(x_dtype) || M > INT64_MAX / 2 / K) return 0;
  return awq::w4a16_xcopy_bytes(x_dtype == AWQ_DTYPE_F32, M, K);
}

AWQ_API int awq_w4a16_ws(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx, const int32_t* qweight,
                         const uint16_t* scales, const uint16_t* zeros, int64_t N, int32_t group, float* Y,
                         int64_t ldy, void* ws, size_t ws_bytes, awq_stream_t stream) {
  int st = check_matrix(X, x_dtype, M, K, ldx);
  if (st != AWQ_OK) return st;
  if (group != kGroup) return AWQ_ERR_UNSUPPORTED;
  if (qweight == nullptr || scales == nullptr || zeros == nullptr || Y == nullptr || N <= 0 || ldy < N)
    return AWQ_ERR_INVALID_ARG;
  if (!aligned16(qweight) || (reinterpret_cast<uintptr_t>(scales) & 1u) != 0 ||
      (reinterpret_cast<uintptr_t>(zeros) & 1u) != 0 || (reinterpret_cast<uintptr_t>(Y) & 3u) != 0)
    return AWQ_ERR_INVALID_ARG;
  if (mul_ok(mul_ok(M, ldy), 4) < 0 || mul_ok(N, K) < 0) return AWQ_ERR_SHAPE;
  // prefill tiles use 32-bit offsets within 512 rows of X (and of its copy, K <= ldx) and of Y
  if (mul_ok(mul_ok(awq::kW4a16BM, ldx), dsize(x_dtype)) >= (int64_t)INT32_MAX) return AWQ_ERR_SHAPE;
  if (mul_ok(mul_ok(awq::kW4a16BM, ldy), 4) >= (int64_t)INT32_MAX) return AWQ_ERR_SHAPE;
  if (ws != nullptr && !aligned16(ws)) return AWQ_ERR_INVALID_ARG;
  // the copy of X when the workspace holds it; otherwise the prefill stages X itself
  const size_t xb = awq::w4a16_xcopy_bytes(x_dtype == AWQ_DTYPE_F32, M, K);
  uint16_t* xcopy = xb > 0 && ws != nullptr && ws_bytes >= xb ? static_cast<uint16_t*>(ws) : nullptr;
  return map_hip(awq::launch_w4a16(X, x_dtype == AWQ_DTYPE_F32, M, K, ldx, qweight, scales, zeros, N, Y, ldy,
                                   xcopy, reinterpret_cast<hipStream_t>(stream)));
}

AWQ_API int awq_w4a16(const void* X, int x_dtype, int64_t M, int64_t K, int64_t ldx, const int32_t* qweight,
                      const uint16_t* scales, const uint16_t* zeros, int64_t N, int32_t group, float* Y,
                      int64_t ldy, awq_stream_t stream) {
  return awq_w4a16_ws(X, x_dtype, M, K, ldx, qweight, scales, zeros, N, group, Y, ldy, nullptr, 0, stream);
}

}  // extern "C"

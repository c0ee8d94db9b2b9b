// C ABI of the column-sparse delta library: argument validation (before any
// HIP call), kernel launches, status codes, thread-local error text, and the
// optional per-kernel event timer.  Declarations and contracts: chipmunk.h.
#include "chipmunk.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

static_assert(CHIPMUNK_NOALLOC_SCRATCH_BYTES == chipmunk::kNoAllocScratchBytes, "scratch array size");

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return CHIPMUNK_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int64_t kMaxGridY = 65535;
// Workgroups of 256 threads in one launch (the grid's work-item count is 32-bit).
constexpr int64_t kMaxGroups = (int64_t)UINT32_MAX / 256;

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CHIPMUNK_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Common MLP layer checks.  need_score: the dense step writes the scores.
int check_mlp(const chipmunk_mlp* L, bool need_score) {
  if (!L) return fail(CHIPMUNK_E_NULLPTR, "layer is NULL");
  if (L->n < 1) return fail(CHIPMUNK_E_SHAPE, "n must be >= 1 (got %lld)", (long long)L->n);
  if (L->d < 128 || L->d % 128 != 0) return fail(CHIPMUNK_E_SHAPE, "d must be a positive multiple of 128 (got %d)", L->d);
  if (L->h < 64 || L->h % 64 != 0) return fail(CHIPMUNK_E_SHAPE, "h must be a positive multiple of 64 (got %d)", L->h);
  if (chipmunk::row_blocks(L->n) > kMaxGridY)
    return fail(CHIPMUNK_E_SHAPE, "n too large: %lld row blocks exceed %lld", (long long)chipmunk::row_blocks(L->n),
                (long long)kMaxGridY);
  if (L->flags & ~(CHIPMUNK_MLP_RESCORE | CHIPMUNK_MLP_FP8 | CHIPMUNK_MLP_FP8_W2))
    return fail(CHIPMUNK_E_SHAPE, "unknown layer flags 0x%x", L->flags);
  const bool fp8w = (L->flags & CHIPMUNK_MLP_FP8_W2) != 0;
  if (fp8w && (!L->w2_f8 || !L->w2_scale))
    return fail(CHIPMUNK_E_NULLPTR, "layer w2_f8 and w2_scale are required by CHIPMUNK_MLP_FP8_W2");
  if (fp8w && !aligned(L->w2_f8, 16)) return fail(CHIPMUNK_E_ALIGN, "w2_f8 must be 16-byte aligned");
  const bool fp8 = (L->flags & CHIPMUNK_MLP_FP8) != 0;
  if ((!fp8 && !L->w1t) || !L->w2 || !L->a_cache)
    return fail(CHIPMUNK_E_NULLPTR, "layer w1t (unless FP8), w2 and a_cache are required");
  if (fp8 && (!L->w1t_f8 || !L->w1t_scale))
    return fail(CHIPMUNK_E_NULLPTR, "layer w1t_f8 and w1t_scale are required by CHIPMUNK_MLP_FP8");
  if (need_score && !L->score) return fail(CHIPMUNK_E_NULLPTR, "layer score is required by the dense step");
  if ((L->flags & CHIPMUNK_MLP_RESCORE) && !L->score)
    return fail(CHIPMUNK_E_NULLPTR, "layer score is required by CHIPMUNK_MLP_RESCORE");
  if ((L->w1t && !aligned(L->w1t, 16)) || !aligned(L->w2, 16) || !aligned(L->a_cache, 16) ||
      (fp8 && !aligned(L->w1t_f8, 16)))
    return fail(CHIPMUNK_E_ALIGN, "w1t, w1t_f8, w2 and a_cache must be 16-byte aligned");
  if ((L->b1 && !aligned(L->b1, 4)) || (L->b2 && !aligned(L->b2, 4)) || (L->score && !aligned(L->score, 4)))
    return fail(CHIPMUNK_E_ALIGN, "b1, b2 and score must be 4-byte aligned");
  return CHIPMUNK_OK;
}

int check_attn(const chipmunk_attn* L) {
  if (!L) return fail(CHIPMUNK_E_NULLPTR, "layer is NULL");
  if (L->n < 1) return fail(CHIPMUNK_E_SHAPE, "n must be >= 1 (got %lld)", (long long)L->n);
  if (L->heads < 1) return fail(CHIPMUNK_E_SHAPE, "heads must be >= 1 (got %d)", L->heads);
  if (L->head_dim != CHIPMUNK_HEAD_DIM)
    return fail(CHIPMUNK_E_UNSUPPORTED, "head_dim must be %d (got %d)", CHIPMUNK_HEAD_DIM, L->head_dim);
  if (!std::isfinite(L->scale)) return fail(CHIPMUNK_E_SHAPE, "scale must be finite");
  if (L->n >= (int64_t)1 << 24)
    return fail(CHIPMUNK_E_SHAPE, "n must be below 2^24 (32-bit byte offsets of gathered K/V rows)");
  if (chipmunk::row_blocks(L->n) * (int64_t)L->heads > kMaxGroups)
    return fail(CHIPMUNK_E_SHAPE, "heads * row blocks exceeds the grid limit (%lld workgroups)", (long long)kMaxGroups);
  if (!L->m || !L->num || !L->den) return fail(CHIPMUNK_E_NULLPTR, "layer m, num and den are required");
  if (!aligned(L->m, 4) || !aligned(L->den, 4) || !aligned(L->num, 16) || (L->score && !aligned(L->score, 4)))
    return fail(CHIPMUNK_E_ALIGN, "num must be 16-byte aligned; m, den, score 4-byte aligned");
  return CHIPMUNK_OK;
}

int check_bf16_in(const void* p, const char* name) {
  if (!p) return fail(CHIPMUNK_E_NULLPTR, "%s is NULL", name);
  if (!aligned(p, 16)) return fail(CHIPMUNK_E_ALIGN, "%s must be 16-byte aligned", name);
  return CHIPMUNK_OK;
}

// D tiles [nb][kp/32][128][32] bf16 (kp = k rounded up to 64).
size_t sparse_mlp_ws(int64_t n, int32_t k) {
  return (size_t)chipmunk::row_blocks(n) * (size_t)chipmunk::padded_k(k) * chipmunk::kRowBlock * sizeof(uint16_t);
}
// fp8 copy of x: [n][d] e4m3 codes, then n scale bytes, rounded up to 16.
size_t fp8_x_ws(int64_t n, int32_t d) { return ((size_t)n * (size_t)d + (size_t)n + 15) / 16 * 16; }
bool is_fp8(const chipmunk_mlp* L) { return (L->flags & CHIPMUNK_MLP_FP8) != 0; }
// Operands of the fp8 second product, or nullptr.
const chipmunk::Fp8Cols* fp8_second(const chipmunk_mlp* L, chipmunk::Fp8Cols* buf) {
  if (!(L->flags & CHIPMUNK_MLP_FP8_W2)) return nullptr;
  *buf = {L->w2_f8, L->w2_scale};
  return buf;
}
// Workspace of the sparse MLP delta of layer L at keep count k.
size_t layer_sparse_ws(const chipmunk_mlp* L, int32_t k) {
  return sparse_mlp_ws(L->n, k) + (is_fp8(L) ? fp8_x_ws(L->n, L->d) : 0);
}
// Quantizes x into ws + off (fp8 layers) and returns the operands of the first
// product; nullptr for bf16 layers.
hipError_t prepare_fp8(const chipmunk_mlp* L, const uint16_t* x, void* ws, size_t off, chipmunk::Fp8Rows* f8,
                       const chipmunk::Fp8Rows** out, hipStream_t s) {
  *out = nullptr;
  if (!is_fp8(L)) return hipSuccess;
  uint8_t* xq = static_cast<uint8_t*>(ws) + off;
  uint8_t* xsc = xq + (size_t)L->n * (size_t)L->d;
  *f8 = {xq, xsc, L->w1t_f8, L->w1t_scale};
  *out = f8;
  return chipmunk::launch_quantize_fp8(x, L->n, L->d, xq, xsc, s);
}

// Scores the sparse delta rewrites (NULL: S stays fixed until the next dense step).
float* rescore_target(const chipmunk_mlp* L) { return (L->flags & CHIPMUNK_MLP_RESCORE) ? L->score : nullptr; }

// Arguments of the sparse MLP delta.
int check_sparse_mlp(const chipmunk_mlp* L, const uint16_t* x, const int32_t* idx, int32_t k, const float* y,
                     const uint16_t* a_new_packed, const void* ws, size_t ws_bytes) {
  int rc = check_mlp(L, false);
  if (rc) return rc;
  if (k < 0 || k > L->h) return fail(CHIPMUNK_E_SHAPE, "k must be in [0, h] (k=%d, h=%d)", k, L->h);
  if ((rc = check_bf16_in(x, "x"))) return rc;
  if (!y) return fail(CHIPMUNK_E_NULLPTR, "y is NULL");
  if (!aligned(y, 16)) return fail(CHIPMUNK_E_ALIGN, "y must be 16-byte aligned");
  if (k > 0 && !idx) return fail(CHIPMUNK_E_NULLPTR, "idx is NULL");
  if (idx && !aligned(idx, 4)) return fail(CHIPMUNK_E_ALIGN, "idx must be 4-byte aligned");
  if (a_new_packed && !aligned(a_new_packed, 16)) return fail(CHIPMUNK_E_ALIGN, "a_new_packed must be 16-byte aligned");
  const size_t need = layer_sparse_ws(L, k);
  if (k > 0 && (!ws || ws_bytes < need))
    return fail(CHIPMUNK_E_WORKSPACE, "workspace of %zu bytes required (got %zu)", need, ws ? ws_bytes : (size_t)0);
  if (ws && !aligned(ws, 16)) return fail(CHIPMUNK_E_ALIGN, "ws must be 16-byte aligned");
  return CHIPMUNK_OK;
}

// Arguments of the sparse attention delta.
int check_sparse_attn(const chipmunk_attn* L, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int32_t* idx, int32_t kk, int mode, const float* o) {
  int rc = check_attn(L);
  if (rc) return rc;
  if (mode != CHIPMUNK_ATTN_SPARSE && mode != CHIPMUNK_ATTN_REFRESH)
    return fail(CHIPMUNK_E_SHAPE, "mode must be CHIPMUNK_ATTN_SPARSE or CHIPMUNK_ATTN_REFRESH (got %d)", mode);
  if (kk < 0 || (int64_t)kk > L->n) return fail(CHIPMUNK_E_SHAPE, "kk must be in [0, n] (kk=%d)", kk);
  if ((rc = check_bf16_in(q, "q")) || (rc = check_bf16_in(k, "k")) || (rc = check_bf16_in(v, "v"))) return rc;
  if (kk > 0 && !idx) return fail(CHIPMUNK_E_NULLPTR, "idx is NULL");
  if (idx && !aligned(idx, 4)) return fail(CHIPMUNK_E_ALIGN, "idx must be 4-byte aligned");
  if (mode == CHIPMUNK_ATTN_SPARSE) {
    if (!o) return fail(CHIPMUNK_E_NULLPTR, "o is NULL");
    if (!aligned(o, 16)) return fail(CHIPMUNK_E_ALIGN, "o must be 16-byte aligned");
  }
  return CHIPMUNK_OK;
}

// A byte range [p, p + bytes) of one buffer named in an error message.
struct Span {
  const void* p;
  size_t bytes;
  const char* name;
};

bool overlap(const Span& a, const Span& b) {
  if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Arguments of the re-identifying attention step, including that no buffer it
// writes (o, num, den, score: updated in place while the inputs are read)
// shares memory with another buffer of the call.
int check_reident(const chipmunk_attn* L, const uint16_t* q_prev, const uint16_t* k_prev, const uint16_t* v_prev,
                  const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* idx, int32_t kk,
                  const float* o) {
  int rc = check_sparse_attn(L, q, k, v, idx, kk, CHIPMUNK_ATTN_SPARSE, o);
  if (rc) return rc;
  if ((rc = check_bf16_in(q_prev, "q_prev")) || (rc = check_bf16_in(k_prev, "k_prev")) ||
      (rc = check_bf16_in(v_prev, "v_prev")))
    return rc;
  if (!L->score) return fail(CHIPMUNK_E_NULLPTR, "layer score is required (the step rescores its keys)");
  const size_t toks = (size_t)L->heads * (size_t)L->n, hd = CHIPMUNK_HEAD_DIM;
  const size_t nba = (size_t)chipmunk::row_blocks(L->n), ak = kk > 0 ? (size_t)kk : 0;
  const Span wr[] = {{o, toks * hd * 4, "o"},
                     {L->num, toks * hd * 4, "num"},
                     {L->den, toks * 4, "den"},
                     {L->score, (size_t)L->heads * nba * (size_t)L->n * 4, "score"}};
  const Span rd[] = {{q_prev, toks * hd * 2, "q_prev"}, {k_prev, toks * hd * 2, "k_prev"},
                     {v_prev, toks * hd * 2, "v_prev"}, {q, toks * hd * 2, "q"},
                     {k, toks * hd * 2, "k"},           {v, toks * hd * 2, "v"},
                     {idx, (size_t)L->heads * nba * ak * 4, "idx"}, {L->m, toks * 4, "m"}};
  for (size_t i = 0; i < sizeof wr / sizeof wr[0]; ++i) {
    for (size_t j = i + 1; j < sizeof wr / sizeof wr[0]; ++j)
      if (overlap(wr[i], wr[j])) return fail(CHIPMUNK_E_SHAPE, "%s overlaps %s", wr[i].name, wr[j].name);
    for (const Span& r : rd)
      if (overlap(wr[i], r)) return fail(CHIPMUNK_E_SHAPE, "%s overlaps %s", wr[i].name, r.name);
  }
  return CHIPMUNK_OK;
}


}  // namespace

// ------------------------------------------------------------------ timer ---
namespace chipmunk {
namespace {
struct Rec {
  int kid;
  hipEvent_t a, b;
};
std::mutex g_tmu;
bool g_ton = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;
thread_local hipEvent_t g_open = nullptr;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

const char* kernel_name(int kid) {
  static const char* names[K_COUNT] = {"mlp_gemm1_sparse", "mlp_gemm1_dense", "mlp_gemm2_sparse", "mlp_gemm2_dense",
                                       "topk_rows",        "cache_writeback", "attn_stats",       "attn_dense",
                                       "attn_sparse",      "attn_refresh",     "sparse_step_fused",
                                       "attn_reident",     "quantize_fp8",     "sparse_step_reident_fused"};
  return (kid >= 0 && kid < K_COUNT) ? names[kid] : "";
}

void timing_before(int kid, hipStream_t s) {
  (void)kid;
  std::lock_guard<std::mutex> g(g_tmu);
  if (!g_ton) return;
  g_open = take_event();
  // A start event that could not be recorded is dropped (back to the pool):
  // that launch is then simply not timed.
  if (g_open && hipEventRecord(g_open, s) != hipSuccess) {
    g_pool.push_back(g_open);
    g_open = nullptr;
  }
}

void timing_after(int kid, hipStream_t s) {
  std::lock_guard<std::mutex> g(g_tmu);
  if (!g_ton || !g_open) return;
  hipEvent_t e = take_event();
  if (e && hipEventRecord(e, s) == hipSuccess) {
    g_recs.push_back({kid, g_open, e});
  } else {
    if (e) g_pool.push_back(e);
    g_pool.push_back(g_open);
  }
  g_open = nullptr;
}
}  // namespace chipmunk

extern "C" int chipmunk_timing_enable(int on) {
  using namespace chipmunk;
  std::lock_guard<std::mutex> g(g_tmu);
  if (on) {
    // Records of the previous window are discarded; their events return to the
    // pool once complete.  A failed wait leaves the events out of the pool
    // (they may still be pending) and is reported.
    hipError_t first = hipSuccess;
    for (auto& r : g_recs) {
      const hipError_t e = hipEventSynchronize(r.b);
      if (e == hipSuccess) {
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
      } else if (first == hipSuccess) {
        first = e;
      }
    }
    g_recs.clear();
    if (first != hipSuccess) {
      g_ton = false;
      return hip_status(first, "hipEventSynchronize");
    }
  }
  g_ton = on != 0;
  return ok();
}

extern "C" int chipmunk_timing_read(int kid, double* total_ms, int64_t* launches) {
  using namespace chipmunk;
  if (kid < 0 || kid >= K_COUNT) return fail(CHIPMUNK_E_SHAPE, "kernel id %d out of range", kid);
  if (!total_ms || !launches) return fail(CHIPMUNK_E_NULLPTR, "total_ms and launches are required");
  std::lock_guard<std::mutex> g(g_tmu);
  double sum = 0.0;
  int64_t cnt = 0;
  for (auto& r : g_recs) {
    if (r.kid != kid) continue;
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_status(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return hip_status(e, "hipEventElapsedTime");
    sum += ms;
    ++cnt;
  }
  *total_ms = sum;
  *launches = cnt;
  return ok();
}

extern "C" int chipmunk_kernel_count(void) { return chipmunk::K_COUNT; }
extern "C" const char* chipmunk_kernel_name(int kid) { return chipmunk::kernel_name(kid); }

// ------------------------------------------------------------ entry points ---
extern "C" const char* chipmunk_last_error(void) { return g_err.c_str(); }
extern "C" int chipmunk_abi_version(void) { return CHIPMUNK_ABI_VERSION; }

// Set by the build from the digest of the sources it compiled.
#ifndef CHIPMUNK_SOURCE_DIGEST
#define CHIPMUNK_SOURCE_DIGEST "unknown"
#endif
extern "C" const char* chipmunk_source_digest(void) { return CHIPMUNK_SOURCE_DIGEST; }

extern "C" size_t chipmunk_workspace_bytes(int op, int64_t n, int32_t d, int32_t h, int32_t k) {
  (void)d;
  (void)h;
  if (n < 1 || k < 0) return 0;
  switch (op) {
    case CHIPMUNK_OP_SPARSE_MLP:
      return sparse_mlp_ws(n, k);
    case CHIPMUNK_OP_SPARSE_MLP_FP8:
      return d > 0 ? sparse_mlp_ws(n, k) + fp8_x_ws(n, d) : 0;
    case CHIPMUNK_OP_DENSE_MLP_FP8:
      return d > 0 ? fp8_x_ws(n, d) : 0;
    default:
      return 0;
  }
}

extern "C" int chipmunk_dense_step(int kind, const void* layer, const uint16_t* x_or_q, const uint16_t* k,
                                   const uint16_t* v, float* out, void* ws, size_t ws_bytes, void* stream) {
  try {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!layer) return fail(CHIPMUNK_E_NULLPTR, "layer is NULL");
    if (kind == CHIPMUNK_MLP) {
      const chipmunk_mlp* L = static_cast<const chipmunk_mlp*>(layer);
      int rc = check_mlp(L, true);
      if (rc) return rc;
      if ((rc = check_bf16_in(x_or_q, "x"))) return rc;
      if (k || v) return fail(CHIPMUNK_E_SHAPE, "k and v must be NULL for an MLP layer");
      if (!out) return fail(CHIPMUNK_E_NULLPTR, "out (y) is NULL");
      if (!aligned(out, 16)) return fail(CHIPMUNK_E_ALIGN, "out (y) must be 16-byte aligned");
      if (is_fp8(L)) {
        const size_t need = fp8_x_ws(L->n, L->d);
        if (!ws || ws_bytes < need)
          return fail(CHIPMUNK_E_WORKSPACE, "workspace of %zu bytes required (got %zu)", need, ws ? ws_bytes : (size_t)0);
        if (!aligned(ws, 16)) return fail(CHIPMUNK_E_ALIGN, "ws must be 16-byte aligned");
      }
      chipmunk::Fp8Rows f8buf;
      const chipmunk::Fp8Rows* f8 = nullptr;
      hipError_t e = prepare_fp8(L, x_or_q, ws, 0, &f8buf, &f8, s);
      if (e != hipSuccess) return hip_status(e, "quantize_fp8 launch");
      // The second product reads the freshly written activation cache directly
      // ([nb][h][128] is the [unit][row] layout it streams).
      e = chipmunk::launch_mlp_gemm1(true, x_or_q, L->w1t, L->b1, nullptr, L->a_cache, nullptr, nullptr, L->score,
                                     L->n, L->d, L->h, L->h, s, f8);
      if (e != hipSuccess) return hip_status(e, "mlp_gemm1 (dense) launch");
      e = chipmunk::launch_mlp_gemm2(true, L->a_cache, L->w2, nullptr, L->b2, out, L->n, L->d, L->h, L->h, L->h, s);
      return hip_status(e, "mlp_gemm2 (dense) launch");
    }
    if (kind == CHIPMUNK_ATTN) {
      const chipmunk_attn* L = static_cast<const chipmunk_attn*>(layer);
      int rc = check_attn(L);
      if (rc) return rc;
      if ((rc = check_bf16_in(x_or_q, "q")) || (rc = check_bf16_in(k, "k")) || (rc = check_bf16_in(v, "v"))) return rc;
      if (!out || !L->score) return fail(CHIPMUNK_E_NULLPTR, "out (o) and layer score are required");
      if (!aligned(out, 16)) return fail(CHIPMUNK_E_ALIGN, "out (o) must be 16-byte aligned");
      hipError_t e = chipmunk::launch_attn_dense(x_or_q, k, v, L->m, L->num, L->den, out, L->score, L->n, L->heads,
                                                 L->scale, s);
      return hip_status(e, "attention refresh launch");
    }
    return fail(CHIPMUNK_E_SHAPE, "unknown kind %d", kind);
  } catch (...) {
    return fail(CHIPMUNK_E_INTERNAL, "internal error in chipmunk_dense_step");
  }
}

extern "C" int chipmunk_identify_topk(const float* score, int64_t rows, int64_t cols, int32_t k, int32_t* idx,
                                      void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  try {
    if (rows < 0) return fail(CHIPMUNK_E_SHAPE, "rows must be >= 0");
    if (cols < 1) return fail(CHIPMUNK_E_SHAPE, "cols must be >= 1");
    if (k < 0 || k > cols) return fail(CHIPMUNK_E_SHAPE, "k must be in [0, cols] (k=%d, cols=%lld)", k, (long long)cols);
    if (rows > INT32_MAX) return fail(CHIPMUNK_E_SHAPE, "rows exceeds the grid limit");
    if (!score || !idx) return fail(CHIPMUNK_E_NULLPTR, "score and idx are required");
    if (!aligned(score, 4) || !aligned(idx, 4)) return fail(CHIPMUNK_E_ALIGN, "score and idx must be 4-byte aligned");
    if (rows == 0 || k == 0) return ok();
    return hip_status(chipmunk::launch_topk(score, rows, cols, k, idx, static_cast<hipStream_t>(stream)),
                      "topk launch");
  } catch (...) {
    return fail(CHIPMUNK_E_INTERNAL, "internal error in chipmunk_identify_topk");
  }
}

extern "C" int chipmunk_check_index_sets(const int32_t* idx, int64_t rows, int32_t k, int64_t cols, int64_t* result,
                                         void* stream) {
  try {
    if (rows < 0) return fail(CHIPMUNK_E_SHAPE, "rows must be >= 0");
    if (cols < 1) return fail(CHIPMUNK_E_SHAPE, "cols must be >= 1");
    if (k < 0 || k > cols) return fail(CHIPMUNK_E_SHAPE, "k must be in [0, cols] (k=%d, cols=%lld)", k, (long long)cols);
    // four rows per workgroup of the check kernel
    if ((rows + 3) / 4 > INT32_MAX) return fail(CHIPMUNK_E_SHAPE, "rows exceeds the grid limit");
    if (!result) return fail(CHIPMUNK_E_NULLPTR, "result is required");
    if (rows > 0 && k > 0 && !idx) return fail(CHIPMUNK_E_NULLPTR, "idx is required");
    if (!aligned(result, 8)) return fail(CHIPMUNK_E_ALIGN, "result must be 8-byte aligned");
    if (idx && !aligned(idx, 4)) return fail(CHIPMUNK_E_ALIGN, "idx must be 4-byte aligned");
    return hip_status(chipmunk::launch_check_index_sets(idx, rows, k, cols, result, static_cast<hipStream_t>(stream)),
                      "index-set check launch");
  } catch (...) {
    return fail(CHIPMUNK_E_INTERNAL, "internal error in chipmunk_check_index_sets");
  }
}

extern "C" int chipmunk_sparse_mlp_delta(const chipmunk_mlp* L, const uint16_t* x, const int32_t* idx, int32_t k,
                                         float* y, uint16_t* a_new_packed, void* ws, size_t ws_bytes, void* stream) {
  try {
    int rc = check_sparse_mlp(L, x, idx, k, y, a_new_packed, ws, ws_bytes);
    if (rc) return rc;
    if (k == 0) return ok();
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint16_t* dbuf = static_cast<uint16_t*>(ws);
    chipmunk::Fp8Rows f8buf;
    const chipmunk::Fp8Rows* f8 = nullptr;
    hipError_t e = prepare_fp8(L, x, ws, sparse_mlp_ws(L->n, k), &f8buf, &f8, s);
    if (e != hipSuccess) return hip_status(e, "quantize_fp8 launch");
    chipmunk::Fp8Cols f8wbuf;
    const chipmunk::Fp8Cols* f8w = fp8_second(L, &f8wbuf);
    e = chipmunk::launch_mlp_gemm1(false, x, L->w1t, L->b1, idx, L->a_cache, dbuf, a_new_packed, rescore_target(L),
                                   L->n, L->d, L->h, k, s, f8, f8w != nullptr);
    if (e != hipSuccess) return hip_status(e, "mlp_gemm1 (sparse) launch");
    e = chipmunk::launch_mlp_gemm2(false, dbuf, L->w2, idx, nullptr, y, L->n, L->d, L->h, k, chipmunk::padded_k(k), s,
                                   f8w);
    return hip_status(e, "mlp_gemm2 (sparse) launch");
  } catch (...) {
    return fail(CHIPMUNK_E_INTERNAL, "internal error in chipmunk_sparse_mlp_delta");
  }
}

extern "C" int chipmunk_sparse_mlp_delta_noalloc(const chipmunk_mlp* L, const uint16_t* x, const int32_t* idx,
                                                 int32_t k, float* y, uint16_t* a_new_packed, void* stream) {
  try {
    // Every argument is checked before any HIP call, the scratch size against
    // the library's array; only then is the array's device address taken.
    int rc = check_mlp(L, false);
    if (rc) return rc;
    if (k < 0 || k > L->h) return fail(CHIPMUNK_E_SHAPE, "k must be in [0, h] (k=%d, h=%d)", k, L->h);
    const size_t need = layer_sparse_ws(L, k);
    if (need > chipmunk::kNoAllocScratchBytes)
      return fail(CHIPMUNK_E_WORKSPACE,
                  "this call needs %zu bytes of scratch, above the %zu-byte array of the allocation-free entry "
                  "point; call chipmunk_sparse_mlp_delta with a workspace instead",
                  need, chipmunk::kNoAllocScratchBytes);
    // A stand-in workspace (aligned, never dereferenced) for the shared checks.
    void* const stand_in = reinterpret_cast<void*>(static_cast<uintptr_t>(256));
    if ((rc = check_sparse_mlp(L, x, idx, k, y, a_new_packed, stand_in, chipmunk::kNoAllocScratchBytes))) return rc;
    if (k == 0) return ok();
    void* ws = nullptr;
    hipError_t e = chipmunk::noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_status(e, "scratch array address");
    return chipmunk_sparse_mlp_delta(L, x, idx, k, y, a_new_packed, ws, chipmunk::kNoAllocScratchBytes, stream);
  } catch (...) {
    return fail(CHIPMUNK_E_INTERNAL, "internal error in chipmunk_sparse_mlp_delta_noalloc");
  }
}

extern "C" int chipmunk_sparse_attn_delta(const chipmunk_attn* L, const uint16_t* q, const uint16_t* k,
                                          const uint16_t* v, const int32_t* idx, int32_t kk, int mode, float* o,
                                          void* stream) {
  try {
    int rc = check_sparse_attn(L, q, k, v, idx, kk, mode, o);
    if (rc) return rc;
    if (mode == CHIPMUNK_ATTN_REFRESH && kk == 0) return ok();
    hipError_t e = chipmunk::launch_attn_sparse(mode == CHIPMUNK_ATTN_REFRESH, q, k, v, idx, L->m, L->num, L->den, o,
                                                L->n, L->heads, kk, L->scale, static_cast<hipStream_t>(stream));
    return hip_status(e, "attention delta launch");
  } catch (...) {
    return fail(CHIPMUNK_E_INTERNAL, "internal error in chipmunk_sparse_attn_delta");
  }
}

extern "C" int chipmunk_sparse_attn_reident(const chipmunk_attn* L, const uint16_t* q_prev, const uint16_t* k_prev,
                                            const uint16_t* v_prev, const uint16_t* q, const uint16_t* k,
                                            const uint16_t* v, const int32_t* idx, int32_t kk, float* o,
                                            void* stream) {
  try {
    int rc = check_reident(L, q_prev, k_prev, v_prev, q, k, v, idx, kk, o);
    if (rc) return rc;
    hipError_t e = chipmunk::launch_attn_reident(q_prev, k_prev, v_prev, q, k, v, idx, L->m, L->num, L->den, L->score,
                                                 o, L->n, L->heads, kk, L->scale, static_cast<hipStream_t>(stream));
    return hip_status(e, "re-identifying attention delta launch");
  } catch (...) {
    return fail(CHIPMUNK_E_INTERNAL, "internal error in chipmunk_sparse_attn_reident");
  }
}

namespace {
// Both deltas in one grid: nothing one of them writes may share memory with
// anything the other reads or writes.  att_w / att_r: the attention side's
// written and read buffers.
template <size_t NW, size_t NR>
int check_step_overlap(const chipmunk_mlp* M, const uint16_t* x, const int32_t* mlp_idx, int32_t k, const float* y,
                       const uint16_t* a_new_packed, const void* ws, const Span (&att_w)[NW], const Span (&att_r)[NR],
                       int64_t attn_groups) {
  const size_t nb = (size_t)chipmunk::row_blocks(M->n);
  const size_t mk = k > 0 ? (size_t)k : 0;
  const Span mlp_w[] = {{y, (size_t)M->n * M->d * 4, "y"},
                        {M->a_cache, nb * M->h * 128 * 2, "mlp a_cache"},
                        {a_new_packed, nb * mk * 128 * 2, "a_new_packed"},
                        {ws, k > 0 ? layer_sparse_ws(M, k) : 0, "ws"},
                        {rescore_target(M), rescore_target(M) ? nb * M->h * 4 : 0, "mlp score"}};
  const Span mlp_r[] = {{x, (size_t)M->n * M->d * 2, "x"},
                        {M->w1t, (size_t)M->h * M->d * 2, "w1t"},
                        {is_fp8(M) ? M->w1t_f8 : nullptr, (size_t)M->h * M->d, "w1t_f8"},
                        {is_fp8(M) ? M->w1t_scale : nullptr, (size_t)M->h, "w1t_scale"},
                        {(M->flags & CHIPMUNK_MLP_FP8_W2) ? M->w2_f8 : nullptr, (size_t)M->h * M->d, "w2_f8"},
                        {(M->flags & CHIPMUNK_MLP_FP8_W2) ? M->w2_scale : nullptr, (size_t)M->d, "w2_scale"},
                        {M->w2, (size_t)M->h * M->d * 2, "w2"},
                        {M->b1, M->b1 ? (size_t)M->h * 4 : 0, "b1"},
                        {mlp_idx, nb * mk * 4, "mlp idx"}};
  // Each part of the grid is at most 7 workgroups of padding above its units.
  const int64_t groups = (k > 0 ? (int64_t)(M->d / 128) * (int64_t)nb + 8 : 0) + attn_groups + 8;
  if (groups > kMaxGroups) return fail(CHIPMUNK_E_SHAPE, "the fused grid exceeds %lld workgroups", (long long)kMaxGroups);
  for (const Span& w : mlp_w) {
    for (const Span& r : att_w)
      if (overlap(w, r)) return fail(CHIPMUNK_E_SHAPE, "%s overlaps %s", w.name, r.name);
    for (const Span& r : att_r)
      if (overlap(w, r)) return fail(CHIPMUNK_E_SHAPE, "%s overlaps %s", w.name, r.name);
  }
  for (const Span& w : att_w)
    for (const Span& r : mlp_r)
      if (overlap(w, r)) return fail(CHIPMUNK_E_SHAPE, "%s overlaps %s", w.name, r.name);
  return CHIPMUNK_OK;
}
}  // namespace

extern "C" int chipmunk_sparse_step(const chipmunk_mlp* M, const uint16_t* x, const int32_t* mlp_idx, int32_t k,
                                    float* y, uint16_t* a_new_packed, void* ws, size_t ws_bytes,
                                    const chipmunk_attn* A, const uint16_t* q, const uint16_t* kx, const uint16_t* v,
                                    const int32_t* attn_idx, int32_t kk, float* o, void* stream) {
  try {
    int rc = check_sparse_mlp(M, x, mlp_idx, k, y, a_new_packed, ws, ws_bytes);
    if (rc) return rc;
    if ((rc = check_sparse_attn(A, q, kx, v, attn_idx, kk, CHIPMUNK_ATTN_SPARSE, o))) return rc;
    const size_t nba = (size_t)chipmunk::row_blocks(A->n);
    const size_t toks = (size_t)A->heads * (size_t)A->n, hd = CHIPMUNK_HEAD_DIM;
    const size_t ak = kk > 0 ? (size_t)kk : 0;
    const Span att_w[] = {{o, toks * hd * 4, "o"}};
    const Span att_r[] = {{q, toks * hd * 2, "q"},          {kx, toks * hd * 2, "k"},
                          {v, toks * hd * 2, "v"},          {attn_idx, (size_t)A->heads * nba * ak * 4, "attn idx"},
                          {A->m, toks * 4, "m"},            {A->num, toks * hd * 4, "num"},
                          {A->den, toks * 4, "den"}};
    if ((rc = check_step_overlap(M, x, mlp_idx, k, y, a_new_packed, ws, att_w, att_r,
                                 (int64_t)A->heads * (int64_t)nba)))
      return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    chipmunk::Fp8Rows f8buf;
    const chipmunk::Fp8Rows* f8 = nullptr;
    if (k > 0) {
      hipError_t e = prepare_fp8(M, x, ws, sparse_mlp_ws(M->n, k), &f8buf, &f8, s);
      if (e != hipSuccess) return hip_status(e, "quantize_fp8 launch");
    }
    chipmunk::Fp8Cols f8wbuf;
    const chipmunk::Fp8Cols* f8w = fp8_second(M, &f8wbuf);
    hipError_t e = chipmunk::launch_sparse_step(x, M->w1t, M->b1, mlp_idx, M->a_cache, static_cast<uint16_t*>(ws),
                                                a_new_packed, rescore_target(M), M->w2, y, M->n, M->d, M->h, k, q,
                                                kx, v, attn_idx, A->m, A->num, A->den, o, A->n, A->heads, kk,
                                                A->scale, s, f8, f8w);
    return hip_status(e, "sparse step launch");
  } catch (...) {
    return fail(CHIPMUNK_E_INTERNAL, "internal error in chipmunk_sparse_step");
  }
}

extern "C" int chipmunk_sparse_step_reident(const chipmunk_mlp* M, const uint16_t* x, const int32_t* mlp_idx,
                                            int32_t k, float* y, uint16_t* a_new_packed, void* ws, size_t ws_bytes,
                                            const chipmunk_attn* A, const uint16_t* q_prev, const uint16_t* k_prev,
                                            const uint16_t* v_prev, const uint16_t* q, const uint16_t* kx,
                                            const uint16_t* v, const int32_t* attn_idx, int32_t kk, float* o,
                                            void* stream) {
  try {
    int rc = check_sparse_mlp(M, x, mlp_idx, k, y, a_new_packed, ws, ws_bytes);
    if (rc) return rc;
    if ((rc = check_reident(A, q_prev, k_prev, v_prev, q, kx, v, attn_idx, kk, o))) return rc;
    const size_t nba = (size_t)chipmunk::row_blocks(A->n);
    const size_t toks = (size_t)A->heads * (size_t)A->n, hd = CHIPMUNK_HEAD_DIM;
    const size_t ak = kk > 0 ? (size_t)kk : 0;
    const Span att_w[] = {{o, toks * hd * 4, "o"},
                          {A->num, toks * hd * 4, "num"},
                          {A->den, toks * 4, "den"},
                          {A->score, (size_t)A->heads * nba * (size_t)A->n * 4, "attn score"}};
    const Span att_r[] = {{q_prev, toks * hd * 2, "q_prev"}, {k_prev, toks * hd * 2, "k_prev"},
                          {v_prev, toks * hd * 2, "v_prev"}, {q, toks * hd * 2, "q"},
                          {kx, toks * hd * 2, "k"},          {v, toks * hd * 2, "v"},
                          {attn_idx, (size_t)A->heads * nba * ak * 4, "attn idx"}, {A->m, toks * 4, "m"}};
    if ((rc = check_step_overlap(M, x, mlp_idx, k, y, a_new_packed, ws, att_w, att_r,
                                 (int64_t)A->heads * (int64_t)nba)))
      return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    chipmunk::Fp8Rows f8buf;
    const chipmunk::Fp8Rows* f8 = nullptr;
    if (k > 0) {
      hipError_t e = prepare_fp8(M, x, ws, sparse_mlp_ws(M->n, k), &f8buf, &f8, s);
      if (e != hipSuccess) return hip_status(e, "quantize_fp8 launch");
    }
    chipmunk::Fp8Cols f8wbuf;
    const chipmunk::Fp8Cols* f8w = fp8_second(M, &f8wbuf);
    hipError_t e = chipmunk::launch_sparse_step_reident(
        x, M->w1t, M->b1, mlp_idx, M->a_cache, static_cast<uint16_t*>(ws), a_new_packed, rescore_target(M), M->w2, y,
        M->n, M->d, M->h, k, q_prev, k_prev, v_prev, q, kx, v, attn_idx, A->m, A->num, A->den, A->score, o, A->n,
        A->heads, kk, A->scale, s, f8, f8w);
    return hip_status(e, "re-identifying sparse step launch");
  } catch (...) {
    return fail(CHIPMUNK_E_INTERNAL, "internal error in chipmunk_sparse_step_reident");
  }
}

extern "C" int chipmunk_quantize_fp8(const uint16_t* src, int64_t rows, int32_t cols, uint8_t* dst, uint8_t* scale,
                                     void* stream) {
  try {
    if (rows < 0) return fail(CHIPMUNK_E_SHAPE, "rows must be >= 0");
    if (cols < 8 || cols % 8 != 0) return fail(CHIPMUNK_E_SHAPE, "cols must be a positive multiple of 8 (got %d)", cols);
    if ((rows + 3) / 4 > (int64_t)UINT32_MAX) return fail(CHIPMUNK_E_SHAPE, "rows exceeds the grid limit");
    if (!src || !dst || !scale) return fail(CHIPMUNK_E_NULLPTR, "src, dst and scale are required");
    if (!aligned(src, 16) || !aligned(dst, 16)) return fail(CHIPMUNK_E_ALIGN, "src and dst must be 16-byte aligned");
    const Span in{src, (size_t)rows * (size_t)cols * 2, "src"};
    const Span o1{dst, (size_t)rows * (size_t)cols, "dst"}, o2{scale, (size_t)rows, "scale"};
    if (overlap(in, o1) || overlap(in, o2) || overlap(o1, o2))
      return fail(CHIPMUNK_E_SHAPE, "src, dst and scale must not overlap");
    if (rows == 0) return ok();
    return hip_status(chipmunk::launch_quantize_fp8(src, rows, cols, dst, scale, static_cast<hipStream_t>(stream)),
                      "quantize_fp8 launch");
  } catch (...) {
    return fail(CHIPMUNK_E_INTERNAL, "internal error in chipmunk_quantize_fp8");
  }
}

extern "C" int chipmunk_quantize_fp8_cols(const uint16_t* src, int64_t rows, int32_t cols, uint8_t* dst,
                                          uint8_t* scale, void* stream) {
  try {
    if (rows < 0) return fail(CHIPMUNK_E_SHAPE, "rows must be >= 0");
    if (cols < 8 || cols % 8 != 0) return fail(CHIPMUNK_E_SHAPE, "cols must be a positive multiple of 8 (got %d)", cols);
    if (!src || !dst || !scale) return fail(CHIPMUNK_E_NULLPTR, "src, dst and scale are required");
    if (!aligned(src, 16) || !aligned(dst, 16)) return fail(CHIPMUNK_E_ALIGN, "src and dst must be 16-byte aligned");
    const Span in{src, (size_t)rows * (size_t)cols * 2, "src"};
    const Span o1{dst, (size_t)rows * (size_t)cols, "dst"}, o2{scale, (size_t)cols, "scale"};
    if (overlap(in, o1) || overlap(in, o2) || overlap(o1, o2))
      return fail(CHIPMUNK_E_SHAPE, "src, dst and scale must not overlap");
    if (rows == 0) return ok();
    return hip_status(
        chipmunk::launch_quantize_fp8_cols(src, rows, cols, dst, scale, static_cast<hipStream_t>(stream)),
        "quantize_fp8_cols launch");
  } catch (...) {
    return fail(CHIPMUNK_E_INTERNAL, "internal error in chipmunk_quantize_fp8_cols");
  }
}

extern "C" int chipmunk_cache_writeback(const chipmunk_mlp* L, const uint16_t* a_new_packed, const int32_t* idx,
                                        int32_t k, void* stream) {
  try {
    int rc = check_mlp(L, false);
    if (rc) return rc;
    if (k < 0 || k > L->h) return fail(CHIPMUNK_E_SHAPE, "k must be in [0, h] (k=%d, h=%d)", k, L->h);
    if (k == 0) return ok();
    if ((rc = check_bf16_in(a_new_packed, "a_new_packed"))) return rc;
    if (!idx) return fail(CHIPMUNK_E_NULLPTR, "idx is NULL");
    if (!aligned(idx, 4)) return fail(CHIPMUNK_E_ALIGN, "idx must be 4-byte aligned");
    return hip_status(chipmunk::launch_writeback(a_new_packed, idx, L->a_cache, L->n, L->h, k,
                                                 static_cast<hipStream_t>(stream)),
                      "writeback launch");
  } catch (...) {
    return fail(CHIPMUNK_E_INTERNAL, "internal error in chipmunk_cache_writeback");
  }
}

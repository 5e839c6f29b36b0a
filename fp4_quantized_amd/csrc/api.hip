// C ABI of libaveris (declared in include/averis.h): argument validation, workspace sizing,
// and dispatch to the split/quant and GEMM launchers.  Nothing is enqueued unless every
// argument check passes.
#include <cstring>
#include <mutex>

#include "launch.h"

using namespace av;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool fmt_ok(int32_t f) { return f == AVERIS_NVFP4 || f == AVERIS_MXFP4; }
bool dtype_ok(int32_t d) { return d == AVERIS_F32 || d == AVERIS_BF16; }
int64_t elem_size(int32_t d) { return d == AVERIS_BF16 ? 2 : 4; }
int64_t block_of(int32_t f) { return f == AVERIS_MXFP4 ? 32 : 16; }

// A qtensor the call writes or reads must have exactly the expected shape and format.
int32_t check_qp(const averis_qtensor* q, int64_t outer, int64_t k, int64_t k_pad, int32_t fmt, uint32_t rot) {
  const bool empty = outer == 0 || k == 0;
  if (!empty && (!q->codes || !q->scales)) return AVERIS_E_NULL;
  if (fmt == AVERIS_NVFP4 && !q->tensor_scale) return AVERIS_E_NULL;
  if (q->fmt != fmt) return AVERIS_E_FORMAT;
  if (q->outer != outer || q->k != k || q->k_pad != k_pad) return AVERIS_E_SHAPE;
  if ((q->flags & ~AVERIS_HADAMARD16) != 0) return AVERIS_E_FLAGS;
  if ((q->flags & AVERIS_HADAMARD16) != rot) return AVERIS_E_FLAGS;
  if (!aligned16(q->codes) || !aligned16(q->scales)) return AVERIS_E_ALIGN;
  return AVERIS_OK;
}
int32_t check_q(const averis_qtensor* q, int64_t outer, int64_t k, int32_t fmt, uint32_t rot) {
  return check_qp(q, outer, k, round_up(k, kKPad), fmt, rot);
}

// Group offsets: E >= 1, both copies given, host copy starts at 0 and never decreases.
// Returns the total row count, or -1.
int64_t check_offsets(const int64_t* d_offsets, const int64_t* h_offsets, int32_t E) {
  if (E < 1 || E > (1 << 20) || !d_offsets || !h_offsets) return -1;
  if (h_offsets[0] != 0) return -1;
  for (int32_t e = 0; e < E; ++e)
    if (h_offsets[e + 1] < h_offsets[e]) return -1;
  return h_offsets[E];
}
int64_t sum_round(const int64_t* h, int32_t E, int64_t m) {
  int64_t s = 0;
  for (int32_t e = 0; e < E; ++e) s += round_up(h[e + 1] - h[e], m);
  return s;
}

// Operand consumed by a GEMM: shape taken from the struct, only consistency checked.
int32_t check_in(const averis_qtensor* q) {
  if (!q) return AVERIS_E_NULL;
  if (!fmt_ok(q->fmt)) return AVERIS_E_FORMAT;
  if (q->outer < 0 || q->k < 0 || q->k_pad != round_up(q->k, kKPad)) return AVERIS_E_SHAPE;
  return check_q(q, q->outer, q->k, q->fmt, q->flags & AVERIS_HADAMARD16);
}

}  // namespace

extern "C" {

int32_t averis_abi_version(void) { return AVERIS_ABI_VERSION; }

#ifndef AVERIS_SOURCE_DIGEST
#define AVERIS_SOURCE_DIGEST "unknown"
#endif
const char* averis_source_digest(void) { return AVERIS_SOURCE_DIGEST; }

const char* averis_status_string(int32_t s) {
  switch (s) {
    case AVERIS_OK: return "ok";
    case AVERIS_E_NULL: return "required pointer is NULL";
    case AVERIS_E_SHAPE: return "inconsistent or unsupported sizes";
    case AVERIS_E_ALIGN: return "pointer or leading dimension not 16-byte aligned";
    case AVERIS_E_DTYPE: return "unknown element type";
    case AVERIS_E_FORMAT: return "unknown FP4 format or mixed formats";
    case AVERIS_E_FLAGS: return "unknown or contradictory flags";
    case AVERIS_E_WORKSPACE: return "workspace missing or too small";
    case AVERIS_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t averis_split_quant_workspace_size(int64_t rows, int64_t cols, int32_t fmt, uint32_t flags) {
  (void)fmt; (void)flags;
  if (rows < 0 || cols <= 0) return 0;
  return split_quant_ws_bytes(rows, cols);
}

// Validates one split + quantization request and fills its plan (nothing is launched).
static int32_t split_quant_plan(const void* x, int32_t xdt, int64_t rows, int64_t cols, int64_t ldx, int32_t fmt,
                                uint32_t flags, float* mean, const averis_qtensor* q_row,
                                const averis_qtensor* q_col, const averis_qtensor* q_mean, void* ws,
                                size_t ws_bytes, void* stream, bool sr, uint64_t seed,
                                const averis_colstats* stats, SplitQuantPlan& p) {
  if (!dtype_ok(xdt)) return AVERIS_E_DTYPE;
  if (!fmt_ok(fmt)) return AVERIS_E_FORMAT;
  if (flags & ~(AVERIS_SPLIT | AVERIS_HADAMARD16 | AVERIS_MEAN_GIVEN | AVERIS_CHECK_FINITE)) return AVERIS_E_FLAGS;
  const bool split = flags & AVERIS_SPLIT, h16 = flags & AVERIS_HADAMARD16, given = flags & AVERIS_MEAN_GIVEN;
  if (given && !split) return AVERIS_E_FLAGS;
  if (rows < 0 || cols <= 0 || cols % kColMult != 0 || ldx < cols) return AVERIS_E_SHAPE;
  if (rows > ((int64_t)1 << 31) || cols > ((int64_t)1 << 24)) return AVERIS_E_SHAPE;
  if (!q_row && !q_col) return AVERIS_E_NULL;
  if (rows > 0 && !x) return AVERIS_E_NULL;
  if (x && (!aligned16(x) || (ldx * elem_size(xdt)) % 16 != 0)) return AVERIS_E_ALIGN;
  const uint32_t rot = h16 ? AVERIS_HADAMARD16 : 0u;
  int32_t st;
  if (q_row && (st = check_q(q_row, rows, cols, fmt, rot)) != AVERIS_OK) return st;
  if (q_col && (st = check_q(q_col, cols, rows, fmt, rot)) != AVERIS_OK) return st;
  if (split) {
    if (!mean || !q_mean) return AVERIS_E_NULL;
    if (!aligned16(mean)) return AVERIS_E_ALIGN;
    if ((st = check_q(q_mean, 1, cols, fmt, rot)) != AVERIS_OK) return st;
  } else if (q_mean) {
    return AVERIS_E_FLAGS;
  }
  if (stats) {
    if (!split || given) return AVERIS_E_FLAGS;
    if (!stats->sum || (stats->min == nullptr) != (stats->max == nullptr)) return AVERIS_E_NULL;
    if (fmt == AVERIS_NVFP4 && !h16 && !stats->min) return AVERIS_E_NULL;
    if (stats->rows != rows || stats->cols != cols || stats->part_rows <= 0 ||
        stats->parts != ceil_div(rows, stats->part_rows) || stats->parts * cols > stats->capacity)
      return AVERIS_E_SHAPE;
  }
  if (!ws || ws_bytes < split_quant_ws_bytes(rows, cols)) return AVERIS_E_WORKSPACE;
  if (!aligned16(ws)) return AVERIS_E_ALIGN;

  p = SplitQuantPlan{x, xdt, rows, cols, ldx, fmt, split, h16, given, mean, q_row, q_col, q_mean, ws,
                     reinterpret_cast<hipStream_t>(stream)};
  p.sr = sr;
  p.seed = seed;
  p.check = (flags & AVERIS_CHECK_FINITE) != 0;
  if (stats) {
    p.st_sum = stats->sum; p.st_parts = stats->parts;
    if (fmt == AVERIS_NVFP4 && !h16) { p.st_min = stats->min; p.st_max = stats->max; }
  }
  return AVERIS_OK;
}

static int32_t split_quant_common(const void* x, int32_t xdt, int64_t rows, int64_t cols, int64_t ldx, int32_t fmt,
                                  uint32_t flags, float* mean, const averis_qtensor* q_row,
                                  const averis_qtensor* q_col, const averis_qtensor* q_mean, void* ws,
                                  size_t ws_bytes, void* stream, bool sr, uint64_t seed,
                                  const averis_colstats* stats = nullptr) {
  SplitQuantPlan p{};
  const int32_t st = split_quant_plan(x, xdt, rows, cols, ldx, fmt, flags, mean, q_row, q_col, q_mean, ws, ws_bytes,
                                      stream, sr, seed, stats, p);
  if (st != AVERIS_OK) return st;
  return split_quant_launch(p) == hipSuccess ? AVERIS_OK : AVERIS_E_HIP;
}

int32_t averis_split_quant_batch(int32_t n, const averis_split_quant_item* items, int32_t xdt, int32_t fmt,
                                 uint32_t flags, void* stream) {
  if (n < 1 || n > AVERIS_BATCH_MAX || n > batch_max()) return AVERIS_E_SHAPE;
  if (!items) return AVERIS_E_NULL;
  if (flags & AVERIS_CHECK_FINITE) return AVERIS_E_FLAGS;
  SplitQuantPlan ps[AVERIS_BATCH_MAX];
  for (int i = 0; i < n; ++i) {
    const averis_split_quant_item& it = items[i];
    const int32_t st = split_quant_plan(it.x, xdt, it.rows, it.cols, it.ldx, fmt, flags, it.mean, it.q_row, it.q_col,
                                        it.q_mean, it.ws, it.ws_bytes, stream, false, 0, nullptr, ps[i]);
    if (st != AVERIS_OK) return st;
    // each tensor needs a workspace of its own (counters, partials and amax slots)
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(it.ws), e0 = b0 + split_quant_ws_bytes(it.rows, it.cols);
    for (int j = 0; j < i; ++j) {
      const uintptr_t b1 = reinterpret_cast<uintptr_t>(items[j].ws);
      const uintptr_t e1 = b1 + split_quant_ws_bytes(items[j].rows, items[j].cols);
      if (b0 < e1 && b1 < e0) return AVERIS_E_WORKSPACE;
    }
  }
  return split_quant_batch_launch(ps, n) == hipSuccess ? AVERIS_OK : AVERIS_E_HIP;
}

int32_t averis_split_quant(const void* x, int32_t xdt, int64_t rows, int64_t cols, int64_t ldx, int32_t fmt,
                           uint32_t flags, float* mean, const averis_qtensor* q_row, const averis_qtensor* q_col,
                           const averis_qtensor* q_mean, void* ws, size_t ws_bytes, void* stream) {
  return split_quant_common(x, xdt, rows, cols, ldx, fmt, flags, mean, q_row, q_col, q_mean, ws, ws_bytes, stream,
                            false, 0);
}

int32_t averis_split_quant_stats(const void* x, int32_t xdt, int64_t rows, int64_t cols, int64_t ldx, int32_t fmt,
                                 uint32_t flags, const averis_colstats* stats, float* mean, const averis_qtensor* q_row,
                                 const averis_qtensor* q_col, const averis_qtensor* q_mean, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (!stats) return AVERIS_E_NULL;
  return split_quant_common(x, xdt, rows, cols, ldx, fmt, flags, mean, q_row, q_col, q_mean, ws, ws_bytes, stream,
                            false, 0, stats);
}

int32_t averis_split_quant_sr(const void* x, int32_t xdt, int64_t rows, int64_t cols, int64_t ldx, int32_t fmt,
                              uint32_t flags, uint64_t seed, float* mean, const averis_qtensor* q_row,
                              const averis_qtensor* q_col, const averis_qtensor* q_mean, void* ws, size_t ws_bytes,
                              void* stream) {
  return split_quant_common(x, xdt, rows, cols, ldx, fmt, flags, mean, q_row, q_col, q_mean, ws, ws_bytes, stream,
                            true, seed);
}

// ------------------------------------------------------------------------------------------
// The allocation-free split + quantization: its workspace is this file's device array, one copy
// per GPU, resolved to a device address once per device (the array's name in host code is only
// a stand-in for the symbol).  The first call on a device also clears the array with a fill
// kernel on the caller's stream; every later call finds the strip counters at zero again, as
// every split+quant leaves them.
// ------------------------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ void k_zero_words(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this GPU's scratch array, cleared on first use; nullptr on a HIP error.
void* scratch_for_current_device(hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    hipLaunchKernelGGL(k_zero_words, dim3(256), dim3(256), 0, stream, reinterpret_cast<uint32_t*>(ptr),
                       kScratchBytes / 4);
    if (hipGetLastError() != hipSuccess) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}
}  // namespace

size_t averis_split_quant_noalloc_max_bytes(void) { return kScratchBytes; }

int32_t averis_split_quant_noalloc(const void* x, int32_t xdt, int64_t rows, int64_t cols, int64_t ldx, int32_t fmt,
                                   uint32_t flags, float* mean, const averis_qtensor* q_row,
                                   const averis_qtensor* q_col, const averis_qtensor* q_mean, void* stream) {
  if (rows < 0 || cols <= 0) return AVERIS_E_SHAPE;
  if (flags & AVERIS_CHECK_FINITE) return AVERIS_E_FLAGS;  // its status word would sit in the hidden array
  if (split_quant_ws_bytes(rows, cols) > kScratchBytes) return AVERIS_E_WORKSPACE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = scratch_for_current_device(s);
  if (!ws) return AVERIS_E_HIP;
  return split_quant_common(x, xdt, rows, cols, ldx, fmt, flags, mean, q_row, q_col, q_mean, ws, kScratchBytes,
                            stream, false, 0);
}

size_t averis_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t fmt) {
  if (M < 0 || N < 0 || K < 0) return 0;
  const int64_t kp = round_up(K, kKPad);
  return gemm_ws_bytes(M, N, kp, choose_splits(fmt, M, N, kp));
}

size_t averis_linear_bwd_dw_workspace_size(int64_t m, int64_t n, int64_t l, int32_t fmt) {
  if (m < 0 || n < 0 || l < 0) return 0;
  const int64_t K = round_up(l, kKPad);
  return gemm_ws_bytes(m, n, K, choose_splits(fmt, m, n, K));
}

// Leading dimensions of GEMM outputs are below 2^23 elements: a wave's 64 output rows then span
// under 2^31 bytes, the reach of a buffer store's 32-bit offset.
constexpr int64_t kMaxLd = int64_t(1) << 23;

// Column-statistics partials are at least 64 rows each (the smallest epilogue row block).
constexpr int64_t kStatsMinPartRows = 64;

static int32_t linear_common(const averis_qtensor* a, const averis_qtensor* mu, const averis_qtensor* w, void* out,
                             int32_t odt, int64_t ldo, void* ws, size_t ws_bytes, void* stream,
                             averis_colstats* stats = nullptr, bool want_stats = false) {
  int32_t st;
  if ((st = check_in(a)) != AVERIS_OK) return st;
  if ((st = check_in(w)) != AVERIS_OK) return st;
  if (!dtype_ok(odt)) return AVERIS_E_DTYPE;
  if (a->fmt != w->fmt) return AVERIS_E_FORMAT;
  if (a->k != w->k) return AVERIS_E_SHAPE;
  if ((a->flags ^ w->flags) & AVERIS_HADAMARD16) return AVERIS_E_FLAGS;
  if (mu) {
    if ((st = check_in(mu)) != AVERIS_OK) return st;
    if (mu->fmt != a->fmt) return AVERIS_E_FORMAT;
    if (mu->outer != 1 || mu->k != a->k) return AVERIS_E_SHAPE;
    if ((mu->flags ^ a->flags) & AVERIS_HADAMARD16) return AVERIS_E_FLAGS;
  }
  if (ldo < w->outer || ldo >= kMaxLd || w->outer % 8 != 0) return AVERIS_E_SHAPE;
  if (a->outer > 0 && w->outer > 0) {
    if (!out) return AVERIS_E_NULL;
    if (!aligned16(out) || (ldo * elem_size(odt)) % 16 != 0) return AVERIS_E_ALIGN;
  }
  const int splits = choose_splits(a->fmt, a->outer, w->outer, a->k_pad);
  if (!ws || ws_bytes < gemm_ws_bytes(a->outer, w->outer, a->k_pad, splits)) return AVERIS_E_WORKSPACE;
  if (!aligned16(ws)) return AVERIS_E_ALIGN;
  GemmPlan p{};
  p.a = a; p.b = w; p.c = out; p.ldc = ldo; p.c_bf16 = odt == AVERIS_BF16;
  p.mu = mu; p.splits = splits; p.ws = ws; p.stream = reinterpret_cast<hipStream_t>(stream);
  GemmPlan::Stats cs{};
  if (want_stats) {
    if (!stats || !stats->sum || (stats->min == nullptr) != (stats->max == nullptr)) return AVERIS_E_NULL;
    if (stats->capacity < averis_colstats_capacity(a->outer, w->outer)) return AVERIS_E_SHAPE;
    cs = GemmPlan::Stats{stats->sum, stats->min, stats->max, 0};
    p.stats = &cs;
  }
  if (gemm_launch(p) != hipSuccess) return AVERIS_E_HIP;
  if (want_stats) {
    stats->rows = a->outer; stats->cols = w->outer; stats->part_rows = cs.part_rows;
    stats->parts = ceil_div(a->outer, cs.part_rows);
  }
  return AVERIS_OK;
}

int64_t averis_colstats_capacity(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return 0;
  return ceil_div(rows, kStatsMinPartRows) * cols;
}

static int32_t producer_common(int op, const void* x, const void* u, int32_t dt, int64_t rows, int64_t cols,
                               int64_t ldx, const float* w, float eps, void* y, int64_t ldy, averis_colstats* stats,
                               void* stream) {
  if (!dtype_ok(dt)) return AVERIS_E_DTYPE;
  if (rows < 0 || cols <= 0 || cols % kColMult != 0 || ldx < cols || ldy < cols) return AVERIS_E_SHAPE;
  if (rows > ((int64_t)1 << 31) || cols > ((int64_t)1 << 24)) return AVERIS_E_SHAPE;
  if (op == 0 && !(eps >= 0.0f)) return AVERIS_E_SHAPE;
  if (rows > 0 && (!x || !y || (op == 0 && !w) || (op == 1 && !u))) return AVERIS_E_NULL;
  const int64_t es = elem_size(dt);
  if ((x && !aligned16(x)) || (u && !aligned16(u)) || (y && !aligned16(y)) || (ldx * es) % 16 != 0 ||
      (ldy * es) % 16 != 0)
    return AVERIS_E_ALIGN;
  if (stats) {
    if (!stats->sum || (stats->min == nullptr) != (stats->max == nullptr)) return AVERIS_E_NULL;
    if (stats->capacity < averis_colstats_capacity(rows, cols)) return AVERIS_E_SHAPE;
  }
  if (producer_launch(op, dt, x, u, rows, cols, ldx, w, eps, y, ldy, stats ? stats->sum : nullptr,
                      stats ? stats->min : nullptr, stats ? stats->max : nullptr,
                      reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return AVERIS_E_HIP;
  if (stats) {
    stats->rows = rows; stats->cols = cols; stats->part_rows = producer_part_rows();
    stats->parts = ceil_div(rows, producer_part_rows());
  }
  return AVERIS_OK;
}

int32_t averis_rmsnorm_stats(const void* x, int32_t dt, int64_t rows, int64_t cols, int64_t ldx, const float* weight,
                             float eps, void* y, int64_t ldy, averis_colstats* stats, void* stream) {
  return producer_common(0, x, nullptr, dt, rows, cols, ldx, weight, eps, y, ldy, stats, stream);
}

int32_t averis_swiglu_stats(const void* gate, const void* up, int32_t dt, int64_t rows, int64_t cols, int64_t ld,
                            void* y, int64_t ldy, averis_colstats* stats, void* stream) {
  return producer_common(1, gate, up, dt, rows, cols, ld, nullptr, 0.0f, y, ldy, stats, stream);
}

int32_t averis_linear_fwd_stats(const averis_qtensor* xr, const averis_qtensor* mu_x, const averis_qtensor* w, void* y,
                                int32_t ydt, int64_t ldy, averis_colstats* stats, void* ws, size_t ws_bytes,
                                void* stream) {
  return linear_common(xr, mu_x, w, y, ydt, ldy, ws, ws_bytes, stream, stats, true);
}

int32_t averis_linear_bwd_dx_stats(const averis_qtensor* dr, const averis_qtensor* mu_d, const averis_qtensor* w,
                                   void* dx, int32_t dxdt, int64_t lddx, averis_colstats* stats, void* ws,
                                   size_t ws_bytes, void* stream) {
  return linear_common(dr, mu_d, w, dx, dxdt, lddx, ws, ws_bytes, stream, stats, true);
}

int32_t averis_linear_fwd(const averis_qtensor* xr, const averis_qtensor* mu_x, const averis_qtensor* w, void* y,
                          int32_t ydt, int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  return linear_common(xr, mu_x, w, y, ydt, ldy, ws, ws_bytes, stream);
}

int32_t averis_linear_bwd_dx(const averis_qtensor* dr, const averis_qtensor* mu_d, const averis_qtensor* w, void* dx,
                             int32_t dxdt, int64_t lddx, void* ws, size_t ws_bytes, void* stream) {
  return linear_common(dr, mu_d, w, dx, dxdt, lddx, ws, ws_bytes, stream);
}

int32_t averis_linear_bwd_dw(const averis_qtensor* xr_t, const averis_qtensor* dr_t, const averis_qtensor* mu_x,
                             const averis_qtensor* mu_d, int64_t l, float* dw, int64_t lddw, uint32_t flags, void* ws,
                             size_t ws_bytes, void* stream) {
  int32_t st;
  if (flags & ~AVERIS_ACCUMULATE) return AVERIS_E_FLAGS;
  if ((st = check_in(xr_t)) != AVERIS_OK) return st;
  if ((st = check_in(dr_t)) != AVERIS_OK) return st;
  if (xr_t->fmt != dr_t->fmt) return AVERIS_E_FORMAT;
  if (xr_t->k != l || dr_t->k != l) return AVERIS_E_SHAPE;
  if ((xr_t->flags ^ dr_t->flags) & AVERIS_HADAMARD16) return AVERIS_E_FLAGS;
  if ((mu_x == nullptr) != (mu_d == nullptr)) return AVERIS_E_NULL;
  if (mu_x) {
    if ((st = check_in(mu_x)) != AVERIS_OK) return st;
    if ((st = check_in(mu_d)) != AVERIS_OK) return st;
    if (mu_x->fmt != xr_t->fmt || mu_d->fmt != xr_t->fmt) return AVERIS_E_FORMAT;
    if (mu_x->outer != 1 || mu_d->outer != 1 || mu_x->k != xr_t->outer || mu_d->k != dr_t->outer) return AVERIS_E_SHAPE;
    if ((mu_x->flags ^ mu_d->flags) & AVERIS_HADAMARD16) return AVERIS_E_FLAGS;
  }
  const int64_t m = xr_t->outer, n = dr_t->outer;
  if (lddw < n || lddw >= kMaxLd || n % 8 != 0) return AVERIS_E_SHAPE;
  if (m > 0 && n > 0) {
    if (!dw) return AVERIS_E_NULL;
    if (!aligned16(dw) || (lddw * 4) % 16 != 0) return AVERIS_E_ALIGN;
  }
  const int splits = choose_splits(xr_t->fmt, m, n, xr_t->k_pad);
  if (!ws || ws_bytes < gemm_ws_bytes(m, n, xr_t->k_pad, splits)) return AVERIS_E_WORKSPACE;
  if (!aligned16(ws)) return AVERIS_E_ALIGN;
  GemmPlan p{};
  p.a = xr_t; p.b = dr_t; p.c = dw; p.ldc = lddw; p.c_bf16 = 0;
  p.mu_u = mu_x; p.mu_v = mu_d; p.r1 = (float)l;
  p.accumulate = (flags & AVERIS_ACCUMULATE) ? 1 : 0;
  p.splits = splits; p.ws = ws; p.stream = reinterpret_cast<hipStream_t>(stream);
  return gemm_launch(p) == hipSuccess ? AVERIS_OK : AVERIS_E_HIP;
}

// ------------------------------------------------------------------------------------------
// Grouped (MoE) variants
// ------------------------------------------------------------------------------------------
size_t averis_split_quant_grouped_workspace_size(int64_t rows, int64_t cols, int32_t E, int32_t fmt, uint32_t flags) {
  (void)fmt; (void)flags;
  if (rows < 0 || cols <= 0 || E < 1) return 0;
  return split_quant_grouped_ws_bytes(rows, cols, E);
}

int32_t averis_split_quant_grouped(const void* x, int32_t xdt, int64_t cols, int64_t ldx, const int64_t* d_offsets,
                                   const int64_t* h_offsets, int32_t E, int32_t fmt, uint32_t flags, float* means,
                                   const averis_qtensor* q_row, const averis_qtensor* q_col,
                                   const averis_qtensor* q_mean, void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_ok(xdt)) return AVERIS_E_DTYPE;
  if (!fmt_ok(fmt)) return AVERIS_E_FORMAT;
  if (flags & ~(AVERIS_SPLIT | AVERIS_HADAMARD16 | AVERIS_MEAN_GIVEN | AVERIS_CHECK_FINITE)) return AVERIS_E_FLAGS;
  const bool split = flags & AVERIS_SPLIT, h16 = flags & AVERIS_HADAMARD16, given = flags & AVERIS_MEAN_GIVEN;
  if (given && !split) return AVERIS_E_FLAGS;
  const int64_t rows = check_offsets(d_offsets, h_offsets, E);
  if (rows < 0) return E < 1 || !d_offsets || !h_offsets ? (E < 1 ? AVERIS_E_SHAPE : AVERIS_E_NULL) : AVERIS_E_SHAPE;
  if (cols <= 0 || cols % kColMult != 0 || ldx < cols) return AVERIS_E_SHAPE;
  if (rows > ((int64_t)1 << 31) || cols > ((int64_t)1 << 24)) return AVERIS_E_SHAPE;
  if (!q_row && !q_col) return AVERIS_E_NULL;
  if (rows > 0 && !x) return AVERIS_E_NULL;
  if (x && (!aligned16(x) || (ldx * elem_size(xdt)) % 16 != 0)) return AVERIS_E_ALIGN;
  if (!aligned16(d_offsets)) return AVERIS_E_ALIGN;
  const uint32_t rot = h16 ? AVERIS_HADAMARD16 : 0u;
  int32_t st;
  if (q_row && (st = check_q(q_row, sum_round(h_offsets, E, 32), cols, fmt, rot)) != AVERIS_OK) return st;
  if (q_col && (st = check_qp(q_col, cols, rows, sum_round(h_offsets, E, kKPad), fmt, rot)) != AVERIS_OK) return st;
  if (split) {
    if (!means || !q_mean) return AVERIS_E_NULL;
    if (!aligned16(means)) return AVERIS_E_ALIGN;
    if ((st = check_q(q_mean, E, cols, fmt, rot)) != AVERIS_OK) return st;
  } else if (q_mean) {
    return AVERIS_E_FLAGS;
  }
  if (!ws || ws_bytes < split_quant_grouped_ws_bytes(rows, cols, E)) return AVERIS_E_WORKSPACE;
  if (!aligned16(ws)) return AVERIS_E_ALIGN;

  SplitQuantPlan p{x, xdt, rows, cols, ldx, fmt, split, h16, given, means, q_row, q_col, q_mean, ws,
                   reinterpret_cast<hipStream_t>(stream), d_offsets, h_offsets, E};
  p.check = (flags & AVERIS_CHECK_FINITE) != 0;
  return split_quant_launch(p) == hipSuccess ? AVERIS_OK : AVERIS_E_HIP;
}

size_t averis_linear_grouped_workspace_size(int64_t N, int32_t E, int32_t fmt) {
  (void)fmt;
  if (N < 0 || E < 1) return 0;
  return gemm_grouped_ws_bytes(0, N, E);
}

static int32_t linear_grouped_common(const averis_qtensor* a, const averis_qtensor* mu, const averis_qtensor* w,
                                     const int64_t* d_offsets, const int64_t* h_offsets, int32_t E, void* out,
                                     int32_t odt, int64_t ldo, void* ws, size_t ws_bytes, void* stream) {
  int32_t st;
  const int64_t rows = check_offsets(d_offsets, h_offsets, E);
  if (rows < 0) return (!d_offsets || !h_offsets) && E >= 1 ? AVERIS_E_NULL : AVERIS_E_SHAPE;
  if (!aligned16(d_offsets)) return AVERIS_E_ALIGN;
  if ((st = check_in(a)) != AVERIS_OK) return st;
  if ((st = check_in(w)) != AVERIS_OK) return st;
  if (!dtype_ok(odt)) return AVERIS_E_DTYPE;
  if (a->fmt != w->fmt) return AVERIS_E_FORMAT;
  if (a->k != w->k) return AVERIS_E_SHAPE;
  if ((a->flags ^ w->flags) & AVERIS_HADAMARD16) return AVERIS_E_FLAGS;
  if (a->outer != sum_round(h_offsets, E, 32)) return AVERIS_E_SHAPE;
  if (w->outer % E != 0) return AVERIS_E_SHAPE;
  const int64_t N = w->outer / E;
  if (N % 32 != 0) return AVERIS_E_SHAPE;  // per-group weight blocks align with the 32-row scale groups
  if (mu) {
    if ((st = check_in(mu)) != AVERIS_OK) return st;
    if (mu->fmt != a->fmt) return AVERIS_E_FORMAT;
    if (mu->outer != E || mu->k != a->k) return AVERIS_E_SHAPE;
    if ((mu->flags ^ a->flags) & AVERIS_HADAMARD16) return AVERIS_E_FLAGS;
  }
  if (ldo < N || ldo >= kMaxLd) return AVERIS_E_SHAPE;
  if (rows > 0 && N > 0) {
    if (!out) return AVERIS_E_NULL;
    if (!aligned16(out) || (ldo * elem_size(odt)) % 16 != 0) return AVERIS_E_ALIGN;
  }
  if (!ws || ws_bytes < gemm_grouped_ws_bytes(0, N, E)) return AVERIS_E_WORKSPACE;
  if (!aligned16(ws)) return AVERIS_E_ALIGN;
  GemmPlan p{};
  p.a = a; p.b = w; p.c = out; p.ldc = ldo; p.c_bf16 = odt == AVERIS_BF16;
  p.mu = mu; p.splits = 1; p.ws = ws; p.stream = reinterpret_cast<hipStream_t>(stream);
  p.grouped = 1; p.d_offsets = d_offsets; p.h_offsets = h_offsets; p.E = E;
  return gemm_launch(p) == hipSuccess ? AVERIS_OK : AVERIS_E_HIP;
}

int32_t averis_linear_fwd_grouped(const averis_qtensor* xr, const averis_qtensor* mu_x, const averis_qtensor* w,
                                  const int64_t* d_offsets, const int64_t* h_offsets, int32_t E, void* y, int32_t ydt,
                                  int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  return linear_grouped_common(xr, mu_x, w, d_offsets, h_offsets, E, y, ydt, ldy, ws, ws_bytes, stream);
}

int32_t averis_linear_bwd_dx_grouped(const averis_qtensor* dr, const averis_qtensor* mu_d, const averis_qtensor* w,
                                     const int64_t* d_offsets, const int64_t* h_offsets, int32_t E, void* dx,
                                     int32_t dxdt, int64_t lddx, void* ws, size_t ws_bytes, void* stream) {
  return linear_grouped_common(dr, mu_d, w, d_offsets, h_offsets, E, dx, dxdt, lddx, ws, ws_bytes, stream);
}

size_t averis_linear_bwd_dw_grouped_workspace_size(int64_t m, int64_t n, int32_t E, int32_t fmt) {
  (void)fmt;
  if (m < 0 || n < 0 || E < 1) return 0;
  return gemm_grouped_dw_ws_bytes(m, n, E);
}

int32_t averis_linear_bwd_dw_grouped(const averis_qtensor* xr_t, const averis_qtensor* dr_t,
                                     const averis_qtensor* mu_x, const averis_qtensor* mu_d, const int64_t* d_offsets,
                                     const int64_t* h_offsets, int32_t E, float* dw, int64_t lddw, uint32_t flags,
                                     void* ws, size_t ws_bytes, void* stream) {
  int32_t st;
  if (flags & ~AVERIS_ACCUMULATE) return AVERIS_E_FLAGS;
  const int64_t rows = check_offsets(d_offsets, h_offsets, E);
  if (rows < 0) return (!d_offsets || !h_offsets) && E >= 1 ? AVERIS_E_NULL : AVERIS_E_SHAPE;
  if (!aligned16(d_offsets)) return AVERIS_E_ALIGN;
  if (!xr_t || !dr_t) return AVERIS_E_NULL;
  if (!fmt_ok(xr_t->fmt)) return AVERIS_E_FORMAT;
  const uint32_t rot = xr_t->flags & AVERIS_HADAMARD16;
  const int64_t tpad = sum_round(h_offsets, E, kKPad);
  if ((st = check_qp(xr_t, xr_t->outer, rows, tpad, xr_t->fmt, rot)) != AVERIS_OK) return st;
  if ((st = check_qp(dr_t, dr_t->outer, rows, tpad, xr_t->fmt, rot)) != AVERIS_OK) return st;
  if ((mu_x == nullptr) != (mu_d == nullptr)) return AVERIS_E_NULL;
  const int64_t m = xr_t->outer, n = dr_t->outer;
  if (mu_x) {
    if ((st = check_q(mu_x, E, m, xr_t->fmt, rot)) != AVERIS_OK) return st;
    if ((st = check_q(mu_d, E, n, xr_t->fmt, rot)) != AVERIS_OK) return st;
  }
  if (lddw < n || lddw >= kMaxLd || n % 8 != 0) return AVERIS_E_SHAPE;
  if (m > 0 && n > 0) {
    if (!dw) return AVERIS_E_NULL;
    if (!aligned16(dw) || (lddw * 4) % 16 != 0) return AVERIS_E_ALIGN;
  }
  if (!ws || ws_bytes < gemm_grouped_dw_ws_bytes(m, n, E)) return AVERIS_E_WORKSPACE;
  if (!aligned16(ws)) return AVERIS_E_ALIGN;
  GemmPlan p{};
  p.a = xr_t; p.b = dr_t; p.c = dw; p.ldc = lddw; p.c_bf16 = 0;
  p.mu_u = mu_x; p.mu_v = mu_d; p.r1 = 0.0f;  // the factor is each group's own token count
  p.accumulate = (flags & AVERIS_ACCUMULATE) ? 1 : 0;
  p.splits = 1; p.ws = ws; p.stream = reinterpret_cast<hipStream_t>(stream);
  p.grouped = 2; p.d_offsets = d_offsets; p.h_offsets = h_offsets; p.E = E;
  return gemm_launch(p) == hipSuccess ? AVERIS_OK : AVERIS_E_HIP;
}

}  // extern "C"

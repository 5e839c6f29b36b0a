// Split + FP4 quantization kernels for gfx950.
//
// Method: "The Curse and Blessing of Mean Bias in FP4-Quantized LLM Training", explainer page
// "均值偏置的诅咒与祝福：FP4量化大语言模型训练" (paper.rainbus.top), section 方法步骤详情: column mean
// mu = (1/l) 1^T X over the tokens, residual X_R = X - 1 mu, and Q_b applied independently to
// mu and X_R; section 块量化: one scale per block set by the block's largest magnitude;
// section Hadamard变换: optional 16x16 Hadamard on [.., 16] tiles.  The paperlayer.ai summary
// (§3 Method) adds that the mean matrix is broadcast, never materialized: here X_R exists only
// in registers between the load of X and the store of its FP4 codes.
//
// Pass structure (X is read twice; the second read usually hits the 256 MB Infinity Cache):
//   k_colstats  per (512-row slab, 64-column strip) column sums: fp32 over 8 rows, fp64 beyond;
//               NVFP4 also column min and max.  The last workgroup of each strip reduces the
//               strip's slabs in fixed order -> mu (fp32), and the strip's maxima of the
//               residual (exact from min / max: fl(x - mu) is monotone in x) and of the mean
//   k_quant     re-read a 32-row tile into LDS, subtract, rotate, block amax, scale, E2M1,
//               and emit both layouts: K = features (row layout) one 64-byte unit per thread,
//               K = tokens (column layout) one column per thread; row tile 0 also quantizes
//               the mean, and each tile zeroes the padding it owns.  With NVFP4 + Hadamard
//               the rotated amax is not available from min / max, so k_quant first runs once
//               in amax-only mode.
// A vanilla MXFP4 operand (no split) needs k_quant only.
#include <algorithm>

#include "launch.h"

namespace av {

constexpr int kThreads = 256;

// ------------------------------------------------------------------------------------------
// 16-point Hadamard butterflies (Sylvester order, stages h = 1, 2, 4, 8), then x 0.25.
// In-register on 16 consecutive values.
// ------------------------------------------------------------------------------------------
__device__ inline void h16_inreg(float* v) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if ((j & h) == 0) {
        const float a = v[j], b = v[j + h];
        v[j] = __fadd_rn(a, b);
        v[j + h] = __fsub_rn(a, b);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = __fmul_rn(v[j], 0.25f);
}

// Butterflies on 16-element blocks spread over 16/VEC lanes, VEC consecutive per lane.
template <int VEC>
__device__ inline void h16_lanes(float* v, int lane) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
    if (h < VEC) {
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        if ((j & h) == 0) {
          const float a = v[j], b = v[j + h];
          v[j] = __fadd_rn(a, b);
          v[j + h] = __fsub_rn(a, b);
        }
      }
    } else {
      const int lm = h / VEC;
      const bool upper = (lane & lm) != 0;
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const float p = __shfl_xor(v[j], lm, 64);
        v[j] = upper ? __fsub_rn(p, v[j]) : __fadd_rn(v[j], p);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < VEC; ++j) v[j] = __fmul_rn(v[j], 0.25f);
}

// ------------------------------------------------------------------------------------------
// k_colstats: column statistics and, in the last workgroup of each column strip, the mean.
// Grid (n_strips, nslab): workgroup (s, b) covers columns [64 s, 64 s + 64) of the rows of
// slab b (kCsRows rows; grouped launches number the slabs group after group, at least one per
// group so empty groups still get their mean of 0).  Thread t holds VEC columns (t % LPR) * VEC
// of rows t / LPR + RPB k, loaded in batches of 16 before use.  Column sums: fp32 over each
// group of 8 rows, fp64 across groups and threads (fixed order); MINMAX (NVFP4): column min
// and max too.  The partials go to the workspace; the workgroup then counts its arrival on its
// strip's counter (agent-scope atomics; see the arrival below).  The last one to arrive
// finalizes the strip:
// fixed-order fp64 reduction of the strip's slabs -> mu (fp32; SPLIT without MEAN_GIVEN), the
// strip's max |residual| (MINMAX: exact from the column min / max, since fl(x - mu) is
// monotone in x) and max |(rotated) mean| as per-strip partials, and resets the counter to 0.
// The counters must be zero before the first call on a workspace and are zero after every call.
// mode bit 0 = SPLIT, bit 1 = MEAN_GIVEN.
// ------------------------------------------------------------------------------------------
// 64-column strips with 512-row slabs measured fastest on the sweep shapes (256-column strips
// read longer row segments but leave the finalizing workgroup 4x the slabs to reduce).
constexpr int kCsRows = 512;            // rows per column-statistics workgroup
constexpr int kCsCols = 64;             // columns per column-statistics workgroup (one strip)
constexpr int kCsWaves = kCsCols / 64;  // finalize: one wave per 64 columns of the strip
// Each strip's arrival counter has a 128-byte line of its own: the 32 slabs of a strip arrive
// within a microsecond, and counters sharing a line would serialize every strip's atomics.
constexpr int kCounterStride = 32;  // uint32 per counter line

struct ColArgs {
  const void* x; int64_t rows, cols, ldx;
  double* psum; float* pmin; float* pmax;  // [nslab][cols]
  uint32_t* slots; int n_slots;            // amax slots, zeroed here for later kernels
  uint32_t* counters;                      // [groups][n_strips], kCounterStride apart
  float* mean;                             // [groups][cols]
  float* ramax_part; float* mamax_part;    // [groups][n_strips]
  int n_strips, mode, h16;
  const int64_t* offsets; int E;
  // PARTS launches: fp32 partials [slab][cols] of each slab's column sum (min, max), no finalize
  float* o_sum; float* o_min; float* o_max;
  // k_colstats_given: fp32 partials [g_parts][cols] of the column sums (min, max) of the rows
  const float* g_sum; const float* g_min; const float* g_max; int64_t g_parts;
  int64_t g_per;  // k_colstats_given: parts per workgroup
};

__device__ __host__ inline int64_t cs_slabs(int64_t len) {
  const int64_t n = ceil_div(len, kCsRows);
  return n > 0 ? n : 1;
}

// Finalization of one 64-column group of a strip, shared by both statistics kernels: the mean of
// column c from its sum S over glen rows (SPLIT without MEAN_GIVEN; MEAN_GIVEN reads it), and
// the wave's maxima of |residual| (MINMAX: exact from the column min / max, since fl(x - mu) is
// monotone in x) and of |(rotated) mean|, one partial each.  Called by all 64 lanes of a wave.
template <bool MINMAX>
__device__ __forceinline__ void strip_finalize(const ColArgs& a, int e, int strip, int cw, int lane, int64_t c,
                                               bool cin, int64_t glen, double S, float lo, float hi) {
  float* mean = a.mean ? a.mean + (int64_t)e * a.cols : nullptr;
  float mu = 0.0f;
  if (cin && (a.mode & 1)) {
    if (a.mode & 2) mu = mean[c];
    else { mu = glen > 0 ? (float)(S / (double)glen) : 0.0f; mean[c] = mu; }
  }
  float ra = 0.0f;
  if (MINMAX && cin && glen > 0) ra = fmaxf(__fsub_rn(hi, mu), __fsub_rn(mu, lo));
  // |mu| per column, rotated within 16-column blocks when the mean is quantized rotated
  float mv[1] = {cin ? mu : 0.0f};
  if (a.h16) h16_lanes<1>(mv, lane);
  float ma = fabsf(mv[0]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) { ra = wave_xor_max(ra, m); ma = wave_xor_max(ma, m); }
  if (lane == 0) {
    const int64_t o = ((int64_t)e * a.n_strips + strip) * kCsWaves + cw;  // per 64 columns
    a.ramax_part[o] = ra; a.mamax_part[o] = ma;
  }
}

// PARTS: write the slab's column partials (fp32) to o_sum / o_min / o_max and stop (no
// counters, no slots, no finalize): the column statistics of an output whose producer could not
// take them in its epilogue.
// The workgroup (bx, by) = (column strip, slab) of launch a.
template <typename T, bool MINMAX, bool PARTS = false>
__device__ __forceinline__ void colstats_body(const ColArgs& a, int bx, int by) {
  constexpr int VEC = Elem<T>::VEC;
  constexpr int LPR = kCsCols / VEC;   // lanes per row
  constexpr int RPB = kThreads / LPR;  // rows per pass of the workgroup
  constexpr int PER = kCsRows / RPB;   // rows per thread (16 bf16, 32 fp32)
  constexpr int BATCH = 16;            // loads in flight per thread
  static_assert(PER % BATCH == 0 && BATCH % 8 == 0, "row batches");
  __shared__ double s_sum[RPB][kCsCols];
  __shared__ float s_min[MINMAX ? RPB : 1][kCsCols];
  __shared__ float s_max[MINMAX ? RPB : 1][kCsCols];
  __shared__ double f_sum[4][kCsCols];
  __shared__ float f_min[4][kCsCols], f_max[4][kCsCols];
  __shared__ int s_last;

  const int t = threadIdx.x;
  if (!PARTS && bx == 0 && by == 0)
    for (int i = t; i < a.n_slots; i += kThreads) a.slots[i] = 0u;  // maxed by later kernels

  // this workgroup's rows [rb, re) and its group's slabs [s0, s0 + nsl)
  int64_t rb = (int64_t)by * kCsRows, re = a.rows, s0 = 0, glen = a.rows;
  int e = 0, nsl = (int)cs_slabs(a.rows);
  if (a.offsets) {
    const GroupPos gp = group_scan(a.offsets, a.E, by, true, [](int64_t len) { return cs_slabs(len); });
    if (gp.e < 0) return;
    e = gp.e;
    rb = gp.off + gp.local * kCsRows;
    re = gp.off + gp.len;
    s0 = gp.base;
    nsl = (int)cs_slabs(gp.len);
    glen = gp.len;
  }
  if (re > rb + kCsRows) re = rb + kCsRows;
  const int strip = bx;
  const int64_t c0 = (int64_t)strip * kCsCols;
  const int lc = t % LPR, rr = t / LPR;
  const int64_t col = c0 + lc * VEC;
  const bool col_ok = col < a.cols;
  const T* x = reinterpret_cast<const T*>(a.x);

  double sum[VEC];
  float mn[VEC], mx[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) { sum[j] = 0.0; mn[j] = __builtin_huge_valf(); mx[j] = -__builtin_huge_valf(); }
#pragma unroll
  for (int b0 = 0; b0 < PER; b0 += BATCH) {
    uint4 w[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
      const int64_t r = rb + rr + (int64_t)RPB * (b0 + i);
      w[i] = (col_ok && r < re) ? *reinterpret_cast<const uint4*>(x + r * a.ldx + col) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int g8 = 0; g8 < BATCH; g8 += 8) {
      float part[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) part[j] = 0.0f;
#pragma unroll
      for (int i = g8; i < g8 + 8; ++i) {
        float v[VEC];
        Elem<T>::unpack(w[i], v);  // rows past the end are zeros: harmless in the sum
#pragma unroll
        for (int j = 0; j < VEC; ++j) part[j] = __fadd_rn(part[j], v[j]);
        if (MINMAX && rb + rr + (int64_t)RPB * (b0 + i) < re) {
#pragma unroll
          for (int j = 0; j < VEC; ++j) { mn[j] = fminf(mn[j], v[j]); mx[j] = fmaxf(mx[j], v[j]); }
        }
      }
#pragma unroll
      for (int j = 0; j < VEC; ++j) sum[j] += (double)part[j];
    }
  }
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    s_sum[rr][lc * VEC + j] = sum[j];
    if (MINMAX) { s_min[rr][lc * VEC + j] = mn[j]; s_max[rr][lc * VEC + j] = mx[j]; }
  }
  __syncthreads();
  if (t < kCsCols && c0 + t < a.cols) {
    double sacc = 0.0;
    float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
    for (int q = 0; q < RPB; ++q) {
      sacc += s_sum[q][t];
      if (MINMAX) { lo = fminf(lo, s_min[q][t]); hi = fmaxf(hi, s_max[q][t]); }
    }
    if constexpr (PARTS) {
      const int64_t o = (int64_t)by * a.cols + c0 + t;
      a.o_sum[o] = (float)sacc;
      if (MINMAX) { a.o_min[o] = lo; a.o_max[o] = hi; }
      return;
    }
    // agent-scope atomic stores: complete only at the coherence point all XCDs read from
    const int64_t o = (int64_t)by * a.cols + c0 + t;
    __hip_atomic_store(a.psum + o, sacc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (MINMAX) {
      __hip_atomic_store(a.pmin + o, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.pmax + o, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ---- arrival on the strip's counter; the last workgroup finalizes the strip ----
  // Every value exchanged between workgroups is an agent-scope atomic access: on gfx950 the
  // partial stores are written through to the agent's coherence point (sc1), the counter
  // update is performed there, and the finalizer's partial loads are served from there (sc1).
  // Each thread waits until its partial stores have completed (vmcnt 0; a workgroup barrier
  // alone does not wait for global stores, and a store and a later atomic to another address
  // may complete in either order), then the barrier lets thread 0 count the arrival; the
  // finalizer issues its loads only after its own update returned, so it reads every other
  // workgroup's completed partials.  The language-level form (release on the update, acquire in
  // the finalizer) compiles to a full L2 write-back and invalidate per workgroup and measured
  // 2.1x slower for this pass on the layer shapes; every exchanged value is written through, so
  // the completion wait is the part of the release these accesses need.
  if constexpr (PARTS) return;
  wait_vm<0>();
  __syncthreads();
  uint32_t* counter = a.counters + ((int64_t)e * a.n_strips + strip) * kCounterStride;
  if (t == 0)
    s_last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(nsl - 1);
  __syncthreads();
  if (!s_last) return;

  // kCsWaves == 1: the four waves split the slabs; otherwise wave q takes columns 64 q ..
  constexpr int SPLITS = kCsWaves == 1 ? 4 : 1;
  const int q = t >> 6, lane = t & 63;
  const int cw = kCsWaves == 1 ? 0 : q;  // this wave's 64-column group of the strip
  const int64_t c = c0 + 64 * cw + lane;
  const bool cin = c < a.cols;
  double* psum = a.psum + s0 * a.cols;
  float* pmin = a.pmin + s0 * a.cols;
  float* pmax = a.pmax + s0 * a.cols;
  const int per = (nsl + SPLITS - 1) / SPLITS;
  const int pb = SPLITS == 1 ? 0 : q * per, pe = SPLITS == 1 ? nsl : (pb + per < nsl ? pb + per : nsl);
  double sacc = 0.0;
  float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
  // agent-scope loads of the other workgroups' partials, whatever XCD wrote them
  // (eight slabs per batch of loads, summed in slab order)
  if (cin && (a.mode & 1) && !(a.mode & 2))
    for (int p0 = pb; p0 < pe; p0 += 8) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = p0 + u < pe ? __hip_atomic_load(psum + (int64_t)(p0 + u) * a.cols + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                           : 0.0;
#pragma unroll
      for (int u = 0; u < 8; ++u) sacc += v[u];
    }
  if (cin && MINMAX)
    for (int p0 = pb; p0 < pe; p0 += 8) {
      float l8[8], h8[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool ok = p0 + u < pe;
        const int64_t o = (int64_t)(p0 + u) * a.cols + c;
        l8[u] = ok ? __hip_atomic_load(pmin + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : __builtin_huge_valf();
        h8[u] = ok ? __hip_atomic_load(pmax + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : -__builtin_huge_valf();
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) { lo = fminf(lo, l8[u]); hi = fmaxf(hi, h8[u]); }
    }
  if (SPLITS == 4) {
    f_sum[q][lane] = sacc; f_min[q][lane] = lo; f_max[q][lane] = hi;
  }
  __syncthreads();
  if (SPLITS == 1 || q == 0) {
    const double S = SPLITS == 1 ? sacc : ((f_sum[0][lane] + f_sum[1][lane]) + f_sum[2][lane]) + f_sum[3][lane];
    if (SPLITS == 4) {
      lo = fminf(fminf(f_min[0][lane], f_min[1][lane]), fminf(f_min[2][lane], f_min[3][lane]));
      hi = fmaxf(fmaxf(f_max[0][lane], f_max[1][lane]), fmaxf(f_max[2][lane], f_max[3][lane]));
    }
    strip_finalize<MINMAX>(a, e, strip, cw, lane, c, cin, glen, S, lo, hi);
    if (lane == 0 && cw == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // for the next call
  }
}


template <typename T, bool MINMAX, bool PARTS = false>
__global__ __launch_bounds__(kThreads) void k_colstats(ColArgs a) {
  colstats_body<T, MINMAX, PARTS>(a, (int)blockIdx.x, (int)blockIdx.y);
}

// Batched launches: several independent tensors' statistics passes in one grid.  Workgroup b
// belongs to the tensor i with start[i] <= b < start[i + 1] and is workgroup b - start[i] of that
// tensor's own (strip, slab) grid, strips first.
constexpr int kBatchMax = 8;
struct ColBatch { ColArgs a[kBatchMax]; int start[kBatchMax + 1]; int n; };

template <typename T, bool MINMAX>
__global__ __launch_bounds__(kThreads) void k_colstats_batch(ColBatch b) {
  const int blk = (int)blockIdx.x;
  int i = 0;
  while (i + 1 < b.n && blk >= b.start[i + 1]) ++i;
  const int local = blk - b.start[i], ns = b.a[i].n_strips;
  colstats_body<T, MINMAX>(b.a[i], local % ns, local / ns);
}

// ------------------------------------------------------------------------------------------
// k_colstats_given: the mean and the strip maxima from column partials that the producer of X
// computed (a GEMM epilogue, RMSNorm, SwiGLU, or k_colstats in PARTS mode): g_parts rows of
// fp32 sums (and, for MINMAX, minima and maxima) per column.  Grid (n_strips, groups of g_per
// parts): workgroup (s, k) sums parts [k g_per, (k + 1) g_per) of strip s's 64 columns
// in fp64 (wave q takes every fourth batch of eight parts, in part order; the four waves are
// added in wave order) and stores the sums as slab k of the workspace's partials.  The slabs
// meet as k_colstats' do: agent-scope stores, an arrival on the strip's counter, and the last
// workgroup to arrive reduces the slabs in slab order and finalizes the strip (the same
// coherence argument).  Block (0, 0) also zeroes the amax slots.  Dense SPLIT only.
// ------------------------------------------------------------------------------------------
constexpr int kGivenParts = 32;  // producer parts per workgroup (at most the workspace's slabs)

template <bool MINMAX>
__global__ __launch_bounds__(kThreads) void k_colstats_given(ColArgs a) {
  static_assert(kCsWaves == 1, "one wave per strip");
  __shared__ double f_sum[4][kCsCols];
  __shared__ float f_min[4][kCsCols], f_max[4][kCsCols];
  __shared__ int s_last;
  const int t = threadIdx.x, q = t >> 6, lane = t & 63;
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = t; i < a.n_slots; i += kThreads) a.slots[i] = 0u;
  const int strip = blockIdx.x, slab = blockIdx.y, nsl = (int)gridDim.y;
  const int64_t c = (int64_t)strip * kCsCols + lane;
  const bool cin = c < a.cols;
  const int64_t pb = (int64_t)slab * a.g_per, pe = pb + a.g_per < a.g_parts ? pb + a.g_per : a.g_parts;
  double sacc = 0.0;
  float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
  if (cin)
    for (int64_t p0 = pb + 8 * q; p0 < pe; p0 += 32) {
      float v[8], l8[MINMAX ? 8 : 1], h8[MINMAX ? 8 : 1];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool ok = p0 + u < pe;
        const int64_t o = (p0 + u) * a.cols + c;
        v[u] = ok ? a.g_sum[o] : 0.0f;
        if constexpr (MINMAX) {
          l8[u] = ok ? a.g_min[o] : __builtin_huge_valf();
          h8[u] = ok ? a.g_max[o] : -__builtin_huge_valf();
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        sacc += (double)v[u];
        if constexpr (MINMAX) { lo = fminf(lo, l8[u]); hi = fmaxf(hi, h8[u]); }
      }
    }
  f_sum[q][lane] = sacc; f_min[q][lane] = lo; f_max[q][lane] = hi;
  __syncthreads();
  uint32_t* counter = a.counters + (int64_t)strip * kCounterStride;
  if (q == 0 && cin) {
    const double S = ((f_sum[0][lane] + f_sum[1][lane]) + f_sum[2][lane]) + f_sum[3][lane];
    const int64_t o = (int64_t)slab * a.cols + c;
    __hip_atomic_store(a.psum + o, S, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (MINMAX) {
      __hip_atomic_store(a.pmin + o, fminf(fminf(f_min[0][lane], f_min[1][lane]), fminf(f_min[2][lane], f_min[3][lane])),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.pmax + o, fmaxf(fmaxf(f_max[0][lane], f_max[1][lane]), fmaxf(f_max[2][lane], f_max[3][lane])),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  wait_vm<0>();      // this thread's partial stores have completed (the barrier alone does not wait)
  __syncthreads();  // ... and every thread's
  if (t == 0)
    s_last = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(nsl - 1);
  __syncthreads();
  if (!s_last || q != 0) return;
  double S = 0.0;
  lo = __builtin_huge_valf(); hi = -__builtin_huge_valf();
  if (cin)
    for (int k = 0; k < nsl; ++k) {
      const int64_t o = (int64_t)k * a.cols + c;
      S += __hip_atomic_load(a.psum + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (MINMAX) {
        lo = fminf(lo, __hip_atomic_load(a.pmin + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        hi = fmaxf(hi, __hip_atomic_load(a.pmax + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      }
    }
  strip_finalize<MINMAX>(a, 0, strip, 0, lane, c, cin, a.rows, S, lo, hi);
  if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // for the next call
}

// ------------------------------------------------------------------------------------------
// k_quant: one workgroup per 32-row x TC-column tile (TC = 32 * VEC: 256 bf16 or 128 fp32
// columns), row tile fastest in the tile numbering.  The tile is loaded with coalesced 16-byte
// loads and staged in LDS in the plane layout below, the column means in a swizzled order; both
// layouts then read from LDS:
//   row layout     thread t quantizes one 64-byte unit of row t / 8 (two units for fp32 MXFP4,
//                  whose 32-element block spans two): whole blocks, no lane exchange;
//   column layout  thread t quantizes column t over the tile's 32 rows.
// MXFP4 divides by the power-of-two block scale inside the E2M1 conversion (exact); tiles whose
// rows all hold data skip the per-element row masks.
//
// The tiles of row tile 0 also quantize the mean's blocks in their columns, and every tile
// zeroes the padding it owns (row-layout K tail, scale rows up to the 32-row group, the
// quantized mean's tail and rows 1..31), so one launch writes every output byte.  Grouped
// launches number the tiles group after group; a tile belongs to one group.
//
// AMAX_ONLY: compute max |rotated residual| of each layout and atomically max it into
// amax_slots[1] (row) and amax_slots[2] (column); nothing is stored.
// ------------------------------------------------------------------------------------------
constexpr int kQRows = 32;                  // rows per tile
// LDS layout of a tile: a tile row (512 bytes) is 8 units of 64 bytes, a unit 4 chunks of 16
// bytes.  Chunk j of unit u of row r sits in plane j at slot r * 8 + u; planes are kQPlane
// slots apart.  A thread reading its whole unit (row layout) and 64 lanes reading one element
// each of 64 consecutive columns (column layout) then hit distinct LDS banks.
constexpr int kQPlane = kQRows * 8 + 2;     // slots per plane (2 slots of padding)
constexpr int kQBufBytes = 4 * kQPlane * 16;
// Column means of a tile: unit u's float chunk i (4 floats) at 16-byte slot i * 8 + u, so that
// the 8 units' chunks read together are contiguous.
template <int EPU>
__device__ __forceinline__ int mean_slot(int c) { return ((c % EPU) >> 2) * 8 + c / EPU; }

struct QuantArgs {
  const void* x;
  int64_t rows, cols, ldx;
  const float* mean;           // nullptr: no subtraction
  const uint32_t* amax_slots;  // NVFP4 with rotation: [1] rotated row amax, [2] rotated col amax
  uint32_t* amax_out;          // AMAX_ONLY target (same buffer as amax_slots)
  int want_row_amax, want_col_amax;  // AMAX_ONLY: the layouts the quantizing pass will write
  const float* ramax_part;     // NVFP4: per-strip max |residual| from k_colstats
  const float* mamax_part;     // NVFP4: per-workgroup max |(rotated) mean|
  int n_part;
  uint8_t* mean_codes;         // quantized mean (nullptr: none)
  uint8_t* mean_scales;
  float* mean_ts;
  int64_t mean_kpad;
  uint8_t* row_codes;          // nullptr: row layout not written
  uint8_t* row_scales;
  float* row_ts;
  uint8_t* col_codes;          // nullptr: column layout not written
  uint8_t* col_scales;
  float* col_ts;
  int64_t col_kpad;            // padded token count of the column layout
  int64_t row_kpad;            // padded column count of the row layout (its row stride in elements)
  int tiles_r, tiles_c;
  int64_t rows_out;            // rows of the row layout written (rows past `rows` are zero residuals)
  int mean_row, mean_rows;     // row of the quantized mean written here; its rows in total
  int cover_kpad;              // row tiles cover the column layout's padded token count
  uint32_t sr_k0, sr_k1;        // stochastic rounding: the Philox key (the caller's seed)
  uint32_t* status;             // CHECK_FINITE: status bits ORed here (workspace word 0), or null
  // grouped launches: group e = input rows [offsets[e], offsets[e+1]), quantized on its own
  // (own mean row, tensor scales and amax partials); row layout rows start at the group's
  // 32-aligned offset, column layout tokens at its 256-aligned offset
  const int64_t* offsets; int E;
};

// ------------------------------------------------------------------------------------------
// Stochastic rounding (averis_split_quant_sr).  Random bits: Philox4x32-10 (Salmon, Moraes,
// Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011) under the caller's 64-bit
// seed; element k of outer index i of a layout (0 row, 1 column, 2 mean) takes the 16-bit half
// k % 2 (low first) of word (k % 8) / 2 at counter (k / 8, i, layout, 0).  The magnitude of the
// scaled value lies between grid neighbours lo <= a < hi and rounds to hi when u16 / 2^16 is
// below (a - lo) / (hi - lo), which is exact in fp32 (Sterbenz, and a power-of-two step).
// ------------------------------------------------------------------------------------------
__device__ inline uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c.x), lo0 = 0xD2511F53u * c.x;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c.z), lo1 = 0xCD9E8D57u * c.z;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// The 16-bit draws of n (multiple of 8) consecutive elements from k0 on (k0 % 8 == 0).
__device__ __forceinline__ void sr_draws(const QuantArgs& a, int64_t outer, int64_t k0, int layout, int n,
                                         uint32_t* u) {
  for (int q = 0; q < n / 8; ++q) {
    const uint4 w = philox4x32_10(make_uint4((uint32_t)((k0 >> 3) + q), (uint32_t)outer, (uint32_t)layout, 0u),
                                  a.sr_k0, a.sr_k1);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) u[8 * q + j] = (ws[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
  }
}

__device__ __forceinline__ uint32_t e2m1_sr(float v, uint32_t u16) {
  const float a = fabsf(v);
  uint32_t c = 7u;
  if (a < 6.0f) {
    float lo, inv_step;
    if (a < 2.0f) { c = (uint32_t)(a * 2.0f); lo = (float)c * 0.5f; inv_step = 2.0f; }
    else if (a < 3.0f) { c = 4u; lo = 2.0f; inv_step = 1.0f; }
    else if (a < 4.0f) { c = 5u; lo = 3.0f; inv_step = 1.0f; }
    else { c = 6u; lo = 4.0f; inv_step = 0.5f; }
    const float p = __fmul_rn(__fsub_rn(a, lo), inv_step);
    if ((float)u16 * (1.0f / 65536.0f) < p) ++c;
  }
  return c | ((__float_as_uint(v) >> 31) << 3);
}

// E2M1 codes of n values of one block with stochastic rounding, after its scale decision.
template <int FMT>
__device__ __forceinline__ void block_codes_sr(float* v, int n, const BlockQ& q, const uint32_t* u, uint32_t* dst) {
  for (int k = 0; k < n / 8; ++k) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) w |= e2m1_sr(__fmul_rn(v[8 * k + j], q.mul), u[8 * k + j]) << (4 * j);
    dst[k] = q.dead ? 0u : w;
  }
}

// CHECK_FINITE: OR `bits` of any lane of the wave into the status word (one atomic per wave
// that found something).  Status bits: 1 = non-finite input, 2 = a nonzero block zeroed or
// clamped because its scale underflowed.
__device__ __forceinline__ void status_or(const QuantArgs& a, uint32_t bits) {
  const uint64_t any1 = __ballot((bits & 1u) != 0), any2 = __ballot((bits & 2u) != 0);
  if ((any1 | any2) && (threadIdx.x & 63) == __builtin_ctzll(any1 | any2))
    atomicOr(a.status, (any1 ? 1u : 0u) | (any2 ? 2u : 0u));
}

// A block's scale lost its range: NVFP4 zeroes a nonzero block (E4M3 underflow or a decode
// scale below 2^-126); MXFP4 clamps the exponent of a block whose amax is below 2^-125.
template <int FMT>
__device__ __forceinline__ bool scale_underflow(float amax, const BlockQ& q) {
  if (!(amax > 0.0f)) return false;
  return FMT == AVERIS_MXFP4 ? amax < 2.35098870e-38f : q.dead;
}

// Mean quantization (row tile 0) and padding zeroes for tile (tr, tc) of ROWS rows.
template <int FMT, bool H16, int TC, int ROWS, bool SR = false>
__device__ __forceinline__ void quant_extras(const QuantArgs& a, int tr, int tc, int64_t r0, int64_t c0) {
  constexpr int G = FMT == AVERIS_MXFP4 ? 32 : 16;
  const int t = threadIdx.x;
  const bool last_tc = tc == a.tiles_c - 1;
  const int64_t cend = c0 + TC < a.cols ? c0 + TC : a.cols;
  // ---- row layout: K tail of codes and scales, and scale rows up to the 32-row group ----
  if (a.row_codes) {
    const int64_t kp = a.row_kpad, rp = round_up(a.rows_out, 32);
    const int64_t rend_d = r0 + ROWS < a.rows_out ? r0 + ROWS : a.rows_out;
    const int64_t rend_p = r0 + ROWS < rp ? r0 + ROWS : rp;
    if (last_tc && kp > a.cols) {
      const int nq = (int)((kp - a.cols) / 32);  // 16-byte chunks of code tail per row
      for (int64_t i = t; i < (rend_d - r0) * nq; i += kThreads) {
        const int64_t r = r0 + i / nq;
        *reinterpret_cast<uint4*>(a.row_codes + r * (kp / 2) + a.cols / 2 + (i % nq) * 16) = make_uint4(0, 0, 0, 0);
      }
      const int nt = (int)((kp - a.cols) / G);
      for (int64_t i = t; i < (rend_p - r0) * nt; i += kThreads)
        a.row_scales[scale_offset(r0 + i / nt, a.cols / G + i % nt, kp, G)] = 0;
    }
    const int64_t pr0 = r0 > a.rows_out ? r0 : a.rows_out;
    const int nb = (int)((cend - c0) / G);
    for (int64_t i = t; i < (rend_p - pr0) * nb; i += kThreads)
      a.row_scales[scale_offset(pr0 + i / nb, c0 / G + i % nb, kp, G)] = 0;
  }
  if (!a.mean_codes || tr != 0) return;
  // ---- quantized mean: this tile's blocks of its row, the row's K tail, and (first group)
  // the zero rows up to the 32-row group ----
  const int64_t kp = a.mean_kpad, mr = a.mean_row;
  float s_dec = 0.0f;
  if (FMT == AVERIS_NVFP4) {
    float m = 0.0f;
    for (int i = t & 63; i < a.n_part; i += 64) m = fmaxf(m, a.mamax_part[i]);
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) m = wave_xor_max(m, s);
    s_dec = nvfp4_tensor_scale(m);
    if (tc == 0 && t == 0) a.mean_ts[mr] = s_dec;
  }
  for (int64_t c = c0 + (int64_t)t * G; c < cend; c += (int64_t)kThreads * G) {
    float v[32];
#pragma unroll
    for (int j = 0; j < G; ++j) v[j] = a.mean[c + j];
    if (H16) {
      h16_inreg(v);
      if (G == 32) h16_inreg(v + 16);
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < G; ++j) amax = fmaxf(amax, fabsf(v[j]));
    const BlockQ q = block_params<FMT>(amax, s_dec);
    if (a.status && scale_underflow<FMT>(amax, q)) atomicOr(a.status, 2u);
    if constexpr (SR) {
      uint32_t u[G], w[G / 8];
      sr_draws(a, 0, c, 2, G, u);
      block_codes_sr<FMT>(v, G, q, u, w);
#pragma unroll
      for (int j = 0; j < G / 8; ++j) *reinterpret_cast<uint32_t*>(a.mean_codes + mr * (kp / 2) + c / 2 + 4 * j) = w[j];
    } else {
#pragma unroll
      for (int j = 0; j < G; ++j) v[j] = __fmul_rn(v[j], q.mul);
#pragma unroll
      for (int j = 0; j < G / 8; ++j)
        *reinterpret_cast<uint32_t*>(a.mean_codes + mr * (kp / 2) + c / 2 + 4 * j) = q.dead ? 0u : pack8_fp4(v + 8 * j);
    }
    a.mean_scales[scale_offset(mr, c / G, kp, G)] = (uint8_t)q.sbyte;
  }
  const int nt = (int)((kp - a.cols) / G);  // K-tail blocks per row
  if (last_tc && kp > a.cols) {
    const int nq = (int)((kp - a.cols) / 32);
    if (t < nq) *reinterpret_cast<uint4*>(a.mean_codes + mr * (kp / 2) + a.cols / 2 + t * 16) = make_uint4(0, 0, 0, 0);
    for (int i = t; i < nt; i += kThreads) a.mean_scales[scale_offset(mr, a.cols / G + i, kp, G)] = 0;
  }
  if (mr == 0) {
    const int64_t z0 = a.mean_rows, zn = round_up(a.mean_rows, 32) - a.mean_rows;
    const int nb = (int)((cend - c0) / G) + (last_tc ? nt : 0);
    for (int64_t i = t; i < zn * nb; i += kThreads) {
      const int64_t r = z0 + i / nb, bi = i % nb;
      const int64_t blk = bi < (cend - c0) / G ? c0 / G + bi : a.cols / G + (bi - (cend - c0) / G);
      a.mean_scales[scale_offset(r, blk, kp, G)] = 0;
    }
  }
}

// Row tiles of a group of `len` rows.
template <int ROWS>
__device__ __host__ inline int64_t quant_row_tiles(int64_t len, int cover_kpad) {
  const int64_t t = ceil_div(cover_kpad ? round_up(len, kKPad) : round_up(len, 32), ROWS);
  return t > 0 ? t : 1;
}

// NVFP4 tensor decode scales of one launch (or group): from the rotated amax slots (H16), else
// from k_colstats' per-strip maxima of |residual|.  Every lane of the wave gets them.
template <bool H16>
__device__ __forceinline__ void nvfp4_scales(const QuantArgs& a, float& sd_row, float& sd_col) {
  float ar, ac;
  if (H16) {
    ar = __uint_as_float(a.amax_slots[1]);
    ac = __uint_as_float(a.amax_slots[2]);
  } else {
    float m = 0.0f;
    for (int i = threadIdx.x & 63; i < a.n_part; i += 64) m = fmaxf(m, a.ramax_part[i]);
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) m = wave_xor_max(m, s);
    ar = ac = m;
  }
  sd_row = nvfp4_tensor_scale(ar);
  sd_col = nvfp4_tensor_scale(ac);
}

// Per-wave maxima of the AMAX_ONLY pass -> at most one atomic max per slot and workgroup.  Every
// wave of the workgroup calls it (it holds a barrier); waves >= `nw` contribute nothing.  The
// atomic is skipped when the slot already holds at least this workgroup's maximum (the slot only
// grows, and non-negative floats order like their bits): tens of thousands of workgroups
// otherwise serialize on the two addresses (measured: a 6.6x slower pass at 65536 x 4096).
__device__ __forceinline__ void amax_commit(const QuantArgs& a, float ra, float ca, float (*s_red)[8], int nw) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    ra = wave_xor_max(ra, m);
    ca = wave_xor_max(ca, m);
  }
  if (lane == 0 && wave < nw) { s_red[0][wave] = ra; s_red[1][wave] = ca; }
  lds_barrier();
  if (threadIdx.x == 0) {
    float u = s_red[0][0], v = s_red[1][0];
    for (int i = 1; i < nw; ++i) { u = fmaxf(u, s_red[0][i]); v = fmaxf(v, s_red[1][i]); }
    if (__float_as_uint(u) > __hip_atomic_load(a.amax_out + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      atomicMax(a.amax_out + 1, __float_as_uint(u));
    if (__float_as_uint(v) > __hip_atomic_load(a.amax_out + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      atomicMax(a.amax_out + 2, __float_as_uint(v));
  }
}

// E2M1 codes of n (8 or 16) values of one block into dst words, after its scale decision.
template <int FMT>
__device__ __forceinline__ void block_codes(float* v, int n, const BlockQ& q, uint32_t* dst) {
  if (FMT == AVERIS_MXFP4) {
    const float sc = mx_scale_value(q.sbyte);
    for (int k = 0; k < n / 8; ++k) dst[k] = q.dead ? 0u : pack8_fp4_div(v + 8 * k, sc);
  } else {
    for (int j = 0; j < n; ++j) v[j] = __fmul_rn(v[j], q.mul);
    for (int k = 0; k < n / 8; ++k) dst[k] = q.dead ? 0u : pack8_fp4(v + 8 * k);
  }
}

// Row layout of a tile: thread t quantizes one 64-byte unit (two for fp32 MXFP4, whose
// 32-element block spans two units) of row t * UPT / 8: whole blocks, so no lane exchange.
// FULL: every row of the tile holds data.
template <typename T, int FMT, bool H16, bool AMAX_ONLY, bool FULL, bool SR = false>
__device__ __forceinline__ void tile_rows(const QuantArgs& a, int64_t r0, int64_t c0, const uint8_t* tile,
                                            const float* means, float sd_row, float& amax_acc) {
  constexpr int SZ = (int)sizeof(T);
  constexpr int G = FMT == AVERIS_MXFP4 ? 32 : 16;
  constexpr int UPT = G * SZ > 64 ? G * SZ / 64 : 1;  // units per thread
  constexpr int EPU = 64 / SZ;                         // elements per unit
  constexpr int EPT = UPT * EPU;                       // elements per thread
  constexpr int NT = kQRows * 8 / UPT;                 // threads with work
  const int t = threadIdx.x;
  if (t >= NT) return;
  const int r = (t * UPT) >> 3, u0 = (t * UPT) & 7;
  const int64_t row = r0 + r, cbase = c0 + u0 * EPU;
  uint32_t d[EPT * SZ / 4];
#pragma unroll
  for (int q = 0; q < UPT; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 c = *reinterpret_cast<const uint4*>(tile + (j * kQPlane + r * 8 + u0 + q) * 16);
      d[q * 16 + j * 4] = c.x; d[q * 16 + j * 4 + 1] = c.y; d[q * 16 + j * 4 + 2] = c.z; d[q * 16 + j * 4 + 3] = c.w;
    }
  float v[EPT];
#pragma unroll
  for (int i = 0; i < EPT * SZ / 16; ++i) {
    const int e0 = i * (16 / SZ);  // first element of chunk i of the thread
    const float4 m4 = *reinterpret_cast<const float4*>(means + 4 * mean_slot<EPU>(u0 * EPU + e0));
    float x[4 * (SZ == 2 ? 2 : 1)];
    Elem<T>::unpack(make_uint4(d[4 * i], d[4 * i + 1], d[4 * i + 2], d[4 * i + 3]), x);
    if (SZ == 2) {
      const float4 m5 = *reinterpret_cast<const float4*>(means + 4 * mean_slot<EPU>(u0 * EPU + e0 + 4));
      const float mm[8] = {m4.x, m4.y, m4.z, m4.w, m5.x, m5.y, m5.z, m5.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[8 * i + e] = __fsub_rn(x[e], mm[e]);
    } else {
      const float mm[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * i + e] = __fsub_rn(x[e], mm[e]);
    }
  }
  if (!FULL && row >= a.rows) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) v[e] = 0.0f;  // rows past the data are zero residuals
  }
  if (H16) {
#pragma unroll
    for (int h = 0; h < EPT / 16; ++h) h16_inreg(v + 16 * h);
  }
  const bool col_ok = cbase < a.cols;
  uint32_t codes[EPT / 8];
  uint32_t sb = 0, flags = 0;
  uint32_t u[SR ? EPT : 1];
  if constexpr (SR) sr_draws(a, row, cbase, 0, EPT, u);
#pragma unroll
  for (int b = 0; b < EPT / G; ++b) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < G; ++j) m = fmaxf(m, fabsf(v[b * G + j]));
    if (AMAX_ONLY) {
      if ((FULL || row < a.rows) && col_ok) amax_acc = fmaxf(amax_acc, m);
      continue;
    }
    const BlockQ q = block_params<FMT>(m, sd_row);
    if (a.status && (FULL || row < a.rows) && col_ok && scale_underflow<FMT>(m, q)) flags |= 2u;
    if constexpr (SR) block_codes_sr<FMT>(v + b * G, G, q, u + b * G, codes + b * (G / 8));
    else block_codes<FMT>(v + b * G, G, q, codes + b * (G / 8));
    sb |= q.sbyte << (8 * b);
  }
  if (AMAX_ONLY) return;
  if (a.status) status_or(a, flags);
  if (row < a.rows_out && col_ok) {
    uint8_t* dst = a.row_codes + row * (a.row_kpad / 2) + cbase / 2;
    if constexpr (EPT == 32) *reinterpret_cast<uint4*>(dst) = make_uint4(codes[0], codes[1], codes[2], codes[3]);
    else *reinterpret_cast<uint2*>(dst) = make_uint2(codes[0], codes[1]);
    uint8_t* sd = a.row_scales + scale_offset(row, cbase / G, a.row_kpad, G);
    if (EPT / G == 2) *reinterpret_cast<uint16_t*>(sd) = (uint16_t)sb;
    else *sd = (uint8_t)sb;
  }
}

// Column layout of a tile: thread t quantizes column t over the tile's 32 rows.
template <typename T, int FMT, bool H16, bool AMAX_ONLY, bool FULL, bool SR = false>
__device__ __forceinline__ void tile_cols(const QuantArgs& a, int64_t r0, int64_t c0, const uint8_t* tile,
                                            const float* means, float sd_col, float& amax_acc) {
  constexpr int SZ = (int)sizeof(T);
  constexpr int TC = 32 * Elem<T>::VEC;
  constexpr int G = FMT == AVERIS_MXFP4 ? 32 : 16;
  constexpr int EPU = 64 / SZ, EPC = 16 / SZ;  // elements per unit, per chunk
  const int c = threadIdx.x;
  if (c >= TC) return;
  const int64_t col = c0 + c;
  const uint8_t* p = tile + ((c % EPU) / EPC * kQPlane + c / EPU) * 16 + (c % EPC) * SZ;  // + 128 bytes a row
  const float m_c = means[4 * mean_slot<EPU>(c) + (c & 3)];
  float v[32];
#pragma unroll
  for (int rr = 0; rr < 32; ++rr) {
    const float xv = Elem<T>::load1(reinterpret_cast<const T*>(p + rr * 128));
    v[rr] = (FULL || r0 + rr < a.rows) ? __fsub_rn(xv, m_c) : 0.0f;
  }
  if (H16) { h16_inreg(v); h16_inreg(v + 16); }
  uint32_t codes[4];
  uint32_t sb = 0, flags = 0;
  uint32_t u[SR ? 32 : 1];
  if constexpr (SR) sr_draws(a, col, r0, 1, 32, u);
#pragma unroll
  for (int b = 0; b < 32 / G; ++b) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < G; ++j) m = fmaxf(m, fabsf(v[b * G + j]));
    if (AMAX_ONLY) {
      if (col < a.cols) amax_acc = fmaxf(amax_acc, m);
      continue;
    }
    const BlockQ q = block_params<FMT>(m, sd_col);
    if (a.status && col < a.cols && scale_underflow<FMT>(m, q)) flags |= 2u;
    if constexpr (SR) block_codes_sr<FMT>(v + b * G, G, q, u + b * G, codes + b * (G / 8));
    else block_codes<FMT>(v + b * G, G, q, codes + b * (G / 8));
    sb |= q.sbyte << (8 * b);
  }
  if (AMAX_ONLY) return;
  if (a.status) status_or(a, flags);
  if (col < a.cols && r0 < a.col_kpad) {
    *reinterpret_cast<uint4*>(a.col_codes + col * (a.col_kpad / 2) + r0 / 2) = make_uint4(codes[0], codes[1], codes[2], codes[3]);
    uint8_t* sd = a.col_scales + scale_offset(col, r0 / G, a.col_kpad, G);
    if (G == 16) *reinterpret_cast<uint16_t*>(sd) = (uint16_t)sb;
    else *sd = (uint8_t)sb;
  }
}

// Tile `tile` (row tiles first) of launch ain.
template <typename T, int FMT, bool H16, bool AMAX_ONLY, bool SR = false>
__device__ __forceinline__ void quant_body(const QuantArgs& ain, const int tile) {
  constexpr int SZ = (int)sizeof(T);
  constexpr int TC = 32 * Elem<T>::VEC;
  constexpr int EPU = 64 / SZ, EPC = 16 / SZ;  // elements per unit, per chunk
  constexpr int G = FMT == AVERIS_MXFP4 ? 32 : 16;
  static_assert(TC * SZ == 512, "tile rows are 512 bytes");
  __shared__ __align__(16) uint8_t s_tile[kQBufBytes];
  __shared__ __align__(16) float s_mean[256];
  __shared__ float s_red[2][8];

  QuantArgs a = ain;  // this workgroup's view (grouped launches retarget it to one group)
  int tr, tc;
  if (ain.offsets) {
    const int tcs = ain.tiles_c, cov = ain.cover_kpad;
    const GroupPos gp = group_scan(ain.offsets, ain.E, tile, true,
                                   [tcs, cov](int64_t len) { return quant_row_tiles<kQRows>(len, cov) * tcs; });
    if (gp.e < 0) return;
    const int64_t trs = quant_row_tiles<kQRows>(gp.len, cov);
    tr = (int)(gp.local % trs); tc = (int)(gp.local / trs);
    const int e = gp.e;
    a.x = reinterpret_cast<const T*>(ain.x) + gp.off * ain.ldx;
    a.rows = gp.len;
    a.rows_out = round_up(gp.len, 32);
    if (a.mean) a.mean += (int64_t)e * ain.cols;
    a.ramax_part += (int64_t)e * ain.n_part;
    a.mamax_part += (int64_t)e * ain.n_part;
    a.amax_slots += 2 * e;
    a.amax_out += 2 * e;
    a.mean_row = e;
    if (a.row_codes) {
      a.row_codes += gp.p32 * (ain.row_kpad / 2);
      a.row_scales += scale_offset(gp.p32, 0, ain.row_kpad, G);
    }
    if (a.row_ts) a.row_ts += e;
    if (a.col_codes) {
      a.col_codes += ain.cols * gp.p256 / 2;
      a.col_scales += ain.cols * gp.p256 / G;
    }
    if (a.col_ts) a.col_ts += e;
    a.col_kpad = round_up(gp.len, kKPad);
  } else {
    tr = tile % ain.tiles_r; tc = tile / ain.tiles_r;
  }
  const int64_t r0 = (int64_t)tr * kQRows, c0 = (int64_t)tc * TC;
  const int t = threadIdx.x;
  const T* x = reinterpret_cast<const T*>(a.x);

  // ---- loads first (rows >= a.rows and columns >= a.cols read as 0), staged in LDS before any
  // store is issued, so no later step waits for this workgroup's stores.  Load k of thread t
  // is 16-byte chunk q = 256 k + t of the tile (row q / 32, chunk q % 32 of the row).  The
  // quantizing pass's loads are non-temporal (the rotated-amax pass before it keeps the default
  // policy): the input is not read again, and the L2 then keeps the column
  // layout's partial output lines, which neighbouring row tiles complete (measured on the
  // layer's split + quantization: 12-15 % faster with vanilla MXFP4 and NVFP4, 3.5 % with the
  // MXFP4 split, whose statistics pass has just read the same input). ----
  uint4 w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int q = k * kThreads + t;
    const int64_t row = r0 + (q >> 5), col = c0 + (int64_t)(q & 31) * EPC;
    const T* src = x + row * a.ldx + col;
    w[k] = (row < a.rows && col < a.cols) ? (AMAX_ONLY ? *reinterpret_cast<const uint4*>(src) : load_nt16(src))
                                          : make_uint4(0, 0, 0, 0);
  }
  if (!AMAX_ONLY && a.status) {  // CHECK_FINITE: an all-ones exponent field is a NaN or an infinity
    uint32_t bad = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t ws[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (SZ == 2) bad |= ((ws[i] & 0x7F80u) == 0x7F80u) | ((ws[i] & 0x7F800000u) == 0x7F800000u);
        else bad |= (ws[i] & 0x7F800000u) == 0x7F800000u;
      }
    }
    status_or(a, bad ? 1u : 0u);
  }
  float4 m4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (t < TC / 4 && a.mean && c0 + 4 * t < a.cols) m4 = *reinterpret_cast<const float4*>(a.mean + c0 + 4 * t);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int q = k * kThreads + t, ch = q & 31;
    *reinterpret_cast<uint4*>(s_tile + ((ch & 3) * kQPlane + (q >> 5) * 8 + (ch >> 2)) * 16) = w[k];
  }
  if (t < TC / 4) *reinterpret_cast<float4*>(s_mean + 4 * mean_slot<EPU>(4 * t)) = m4;

  float sd_row = 0.0f, sd_col = 0.0f;
  if (FMT == AVERIS_NVFP4 && !AMAX_ONLY) {
    nvfp4_scales<H16>(a, sd_row, sd_col);
    if (tr == 0 && tc == 0 && t == 0) {
      if (a.row_ts) a.row_ts[0] = sd_row;
      if (a.col_ts) a.col_ts[0] = sd_col;
    }
  }
  if (!AMAX_ONLY) quant_extras<FMT, H16, TC, kQRows, SR>(a, tr, tc, r0, c0);
  lds_barrier();

  float amax_row = 0.0f, amax_col = 0.0f;
  if (r0 + kQRows <= a.rows) {
    if (AMAX_ONLY ? a.want_row_amax : a.row_codes != nullptr)
      tile_rows<T, FMT, H16, AMAX_ONLY, true, SR>(a, r0, c0, s_tile, s_mean, sd_row, amax_row);
    if (AMAX_ONLY ? a.want_col_amax : a.col_codes != nullptr)
      tile_cols<T, FMT, H16, AMAX_ONLY, true, SR>(a, r0, c0, s_tile, s_mean, sd_col, amax_col);
  } else {
    if (AMAX_ONLY ? a.want_row_amax : a.row_codes != nullptr)
      tile_rows<T, FMT, H16, AMAX_ONLY, false, SR>(a, r0, c0, s_tile, s_mean, sd_row, amax_row);
    if (AMAX_ONLY ? a.want_col_amax : a.col_codes != nullptr)
      tile_cols<T, FMT, H16, AMAX_ONLY, false, SR>(a, r0, c0, s_tile, s_mean, sd_col, amax_col);
  }
  if (AMAX_ONLY) amax_commit(a, amax_row, amax_col, s_red, kThreads / 64);
}

template <typename T, int FMT, bool H16, bool AMAX_ONLY, bool SR = false>
__global__ __launch_bounds__(kThreads, 4) void k_quant(QuantArgs ain) {
  quant_body<T, FMT, H16, AMAX_ONLY, SR>(ain, xcd_remap(blockIdx.x, (int)gridDim.x));
}

// Batched quantization: tile b (after the XCD remap) belongs to the tensor i with start[i] <= b <
// start[i + 1] and is tile b - start[i] of it.
struct QuantBatch { QuantArgs a[kBatchMax]; int start[kBatchMax + 1]; int n; };
static_assert(sizeof(QuantBatch) <= 4096 && sizeof(ColBatch) <= 4096, "kernel argument size");

template <typename T, int FMT, bool H16, bool AMAX_ONLY>
__global__ __launch_bounds__(kThreads, 4) void k_quant_batch(QuantBatch b) {
  const int blk = xcd_remap(blockIdx.x, (int)gridDim.x);
  int i = 0;
  while (i + 1 < b.n && blk >= b.start[i + 1]) ++i;
  quant_body<T, FMT, H16, AMAX_ONLY>(b.a[i], blk - b.start[i]);
}

__global__ void k_fill_f32(float* p, int n, float v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ------------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------------
// workspace: [0, hdr) amax slots (3 + 2 E uint32, 256-byte aligned end), then strip counters
// (E x n_strips, one 128-byte line each, zero between calls) | per-strip partial maxima
// (2 x E x n_part fp32) | column statistics: psum [nslab][cols] fp64, pmin and pmax [nslab][cols]
// fp32
struct SqLayout {
  uint32_t* slots; int n_slots; uint32_t* counters; float* ramax; float* mamax; double* psum; float* pmin;
  float* pmax; int n_part; int64_t nslab;
};
static int64_t n_strips(int64_t cols) { return ceil_div(cols, kCsCols); }
static int64_t n_parts(int64_t cols) { return n_strips(cols) * kCsWaves; }  // per-64-column partial maxima
static size_t sq_slots_bytes(int64_t E) { return (size_t)round_up((3 + 2 * E) * 4, 256); }
static size_t sq_header(int64_t cols, int64_t E) {
  return sq_slots_bytes(E) + (size_t)round_up(E * n_strips(cols) * kCounterStride * 4, 256);
}
static SqLayout sq_layout(void* ws, int64_t nslab, int64_t cols, int64_t E) {
  SqLayout L;
  uint8_t* b = reinterpret_cast<uint8_t*>(ws);
  L.n_part = (int)n_parts(cols);
  L.nslab = nslab;
  const size_t h = sq_header(cols, E), pb = (size_t)round_up(E * L.n_part * 4, 256);
  L.slots = reinterpret_cast<uint32_t*>(b);
  L.n_slots = (int)(3 + 2 * E);
  L.counters = reinterpret_cast<uint32_t*>(b + sq_slots_bytes(E));
  L.ramax = reinterpret_cast<float*>(b + h);
  L.mamax = reinterpret_cast<float*>(b + h + pb);
  L.psum = reinterpret_cast<double*>(b + h + 2 * pb);
  L.pmin = reinterpret_cast<float*>(b + h + 2 * pb + (size_t)L.nslab * cols * 8);
  L.pmax = L.pmin + (size_t)L.nslab * cols;
  return L;
}
static size_t sq_bytes(int64_t nslab, int64_t cols, int64_t E) {
  return sq_header(cols, E) + 2 * (size_t)round_up(E * n_parts(cols) * 4, 256) + (size_t)nslab * cols * (8 + 4 + 4) +
         256;
}

size_t split_quant_ws_bytes(int64_t rows, int64_t cols) { return sq_bytes(cs_slabs(rows), cols, 1); }
// grouped: at most ceil(rows / kCsRows) + E slabs
size_t split_quant_grouped_ws_bytes(int64_t rows, int64_t cols, int64_t E) {
  return sq_bytes(ceil_div(rows, kCsRows) + E + 1, cols, E);
}

// Arguments of the quantizing pass for plan p (before the output pointers: the rotated-amax pass
// takes the same ones); ntiles = its workgroups.
template <typename T>
static QuantArgs quant_args(const SplitQuantPlan& p, const SqLayout& L, int64_t& ntiles) {
  constexpr int TC = 32 * Elem<T>::VEC;
  const bool grouped = p.E > 0;
  QuantArgs a{};
  a.x = p.x; a.rows = p.rows; a.cols = p.cols; a.ldx = p.ldx;
  a.mean = p.split ? p.mean : nullptr;
  a.amax_slots = L.slots; a.amax_out = L.slots;
  a.status = p.check ? L.slots : nullptr;  // word 0 (the amax slots start at word 1)
  a.ramax_part = L.ramax; a.mamax_part = L.mamax; a.n_part = L.n_part;
  const int64_t col_kpad = round_up(p.rows, kKPad);
  a.col_kpad = col_kpad;
  a.row_kpad = round_up(p.cols, kKPad);
  a.tiles_c = (int)ceil_div(p.cols, TC);
  a.rows_out = p.rows;
  a.mean_row = 0; a.mean_rows = grouped ? (int)p.E : 1;
  a.cover_kpad = p.q_col ? 1 : 0;
  if (grouped) {
    a.offsets = p.d_offsets; a.E = (int)p.E;
    int64_t tr = 0;
    for (int64_t e = 0; e < p.E; ++e) tr += quant_row_tiles<kQRows>(p.h_offsets[e + 1] - p.h_offsets[e], a.cover_kpad);
    a.tiles_r = (int)tr;
    ntiles = tr * a.tiles_c;
  } else {
    // column layout covers the padding rows too (they are zero residuals); at least one row tile
    // so that the tensor scales, the quantized mean and the padding are written for rows == 0
    a.tiles_r = (int)quant_row_tiles<kQRows>(p.rows, a.cover_kpad);
    ntiles = (int64_t)a.tiles_r * a.tiles_c;
  }
  return a;
}

// The rotated-amax pass's view of a (NVFP4 with H16), and the quantizing pass's outputs.
static QuantArgs amax_view(const QuantArgs& a, const SplitQuantPlan& p) {
  QuantArgs m = a;
  m.want_row_amax = p.q_row != nullptr;
  m.want_col_amax = p.q_col != nullptr;
  return m;
}
static void set_outputs(QuantArgs& a, const SplitQuantPlan& p) {
  if (p.q_row) { a.row_codes = p.q_row->codes; a.row_scales = p.q_row->scales; a.row_ts = p.q_row->tensor_scale; }
  if (p.q_col) { a.col_codes = p.q_col->codes; a.col_scales = p.q_col->scales; a.col_ts = p.q_col->tensor_scale; }
  if (p.split && p.q_mean) {
    a.mean_codes = p.q_mean->codes; a.mean_scales = p.q_mean->scales; a.mean_ts = p.q_mean->tensor_scale;
    a.mean_kpad = p.q_mean->k_pad;
  }
  if (p.sr) {
    a.sr_k0 = (uint32_t)p.seed;
    a.sr_k1 = (uint32_t)(p.seed >> 32);
  }
}

template <typename T, int FMT, bool H16>
static hipError_t launch_quant_t(const SplitQuantPlan& p, const SqLayout& L) {
  const bool grouped = p.E > 0;
  int64_t ntiles = 0;
  QuantArgs a = quant_args<T>(p, L, ntiles);
  if (ntiles == 0) {  // no columns or no groups: still define the tensor scales (0)
    if (FMT == AVERIS_NVFP4 && !grouped) {
      float* ts[3] = {p.q_row ? p.q_row->tensor_scale : nullptr, p.q_col ? p.q_col->tensor_scale : nullptr,
                      p.q_mean ? p.q_mean->tensor_scale : nullptr};
      for (float* t : ts)
        if (t) hipLaunchKernelGGL(k_fill_f32, dim3(1), dim3(64), 0, p.stream, t, 1, 0.0f);
    }
    return hipGetLastError();
  }
  if (FMT == AVERIS_NVFP4 && H16)
    hipLaunchKernelGGL((k_quant<T, FMT, H16, true>), dim3((unsigned)ntiles), dim3(kThreads), 0, p.stream, amax_view(a, p));
  set_outputs(a, p);
  if (p.sr) hipLaunchKernelGGL((k_quant<T, FMT, H16, false, true>), dim3((unsigned)ntiles), dim3(kThreads), 0, p.stream, a);
  else hipLaunchKernelGGL((k_quant<T, FMT, H16, false>), dim3((unsigned)ntiles), dim3(kThreads), 0, p.stream, a);
  return hipGetLastError();
}

template <int FMT, bool H16>
static hipError_t launch_quant_f(const SplitQuantPlan& p, const SqLayout& L) {
  return p.xdt == AVERIS_BF16 ? launch_quant_t<uint16_t, FMT, H16>(p, L) : launch_quant_t<float, FMT, H16>(p, L);
}

static ColArgs col_args(const SplitQuantPlan& p, const SqLayout& L) {
  const bool grouped = p.E > 0;
  ColArgs a{};
  a.x = p.x; a.rows = p.rows; a.cols = p.cols; a.ldx = p.ldx;
  a.psum = L.psum; a.pmin = L.pmin; a.pmax = L.pmax;
  a.slots = L.slots; a.n_slots = L.n_slots; a.counters = L.counters;
  a.mean = p.mean; a.ramax_part = L.ramax; a.mamax_part = L.mamax;
  a.n_strips = (int)n_strips(p.cols);
  a.mode = (p.split ? 1 : 0) | (p.mean_given ? 2 : 0);
  a.h16 = (p.split && p.h16) ? 1 : 0;
  a.offsets = grouped ? p.d_offsets : nullptr;
  a.E = grouped ? (int)p.E : 1;
  return a;
}

template <typename T, bool MINMAX>
static void launch_stats_t(const SplitQuantPlan& p, const SqLayout& L) {
  const dim3 grid((unsigned)n_strips(p.cols), (unsigned)L.nslab);
  hipLaunchKernelGGL((k_colstats<T, MINMAX>), grid, dim3(kThreads), 0, p.stream, col_args(p, L));
}

template <bool MINMAX>
static void launch_stats_given(const SplitQuantPlan& p, const SqLayout& L) {
  ColArgs a{};
  a.rows = p.rows; a.cols = p.cols;
  a.slots = L.slots; a.n_slots = L.n_slots; a.counters = L.counters;
  a.psum = L.psum; a.pmin = L.pmin; a.pmax = L.pmax;
  a.mean = p.mean; a.ramax_part = L.ramax; a.mamax_part = L.mamax;
  a.n_strips = (int)n_strips(p.cols);
  a.mode = 1;
  a.h16 = p.h16 ? 1 : 0;
  a.E = 1;
  a.g_sum = p.st_sum; a.g_min = p.st_min; a.g_max = p.st_max; a.g_parts = p.st_parts;
  // groups of about kGivenParts parts, at most the workspace's slabs
  const int64_t groups = std::max<int64_t>(1, std::min<int64_t>(ceil_div(p.st_parts, kGivenParts), L.nslab));
  a.g_per = std::max<int64_t>(1, ceil_div(p.st_parts, groups));
  hipLaunchKernelGGL((k_colstats_given<MINMAX>), dim3((unsigned)n_strips(p.cols), (unsigned)groups), dim3(kThreads), 0,
                     p.stream, a);
}

template <typename T, bool MINMAX>
static void launch_colparts_t(const void* c, int64_t M, int64_t N, int64_t ldc, float* sum, float* mn, float* mx,
                              hipStream_t s) {
  ColArgs a{};
  a.x = c; a.rows = M; a.cols = N; a.ldx = ldc;
  a.n_strips = (int)n_strips(N);
  a.E = 1;
  a.o_sum = sum; a.o_min = mn; a.o_max = mx;
  hipLaunchKernelGGL((k_colstats<T, MINMAX, true>), dim3((unsigned)n_strips(N), (unsigned)ceil_div(M, kCsRows)),
                     dim3(kThreads), 0, s, a);
}

int64_t colparts_rows() { return kCsRows; }

void colparts_launch(const void* c, int cdt, int64_t M, int64_t N, int64_t ldc, float* sum, float* mn, float* mx,
                     hipStream_t s) {
  if (M <= 0 || N <= 0) return;
  if (cdt == AVERIS_BF16) {
    if (mn) launch_colparts_t<uint16_t, true>(c, M, N, ldc, sum, mn, mx, s);
    else launch_colparts_t<uint16_t, false>(c, M, N, ldc, sum, mn, mx, s);
  } else {
    if (mn) launch_colparts_t<float, true>(c, M, N, ldc, sum, mn, mx, s);
    else launch_colparts_t<float, false>(c, M, N, ldc, sum, mn, mx, s);
  }
}

hipError_t split_quant_launch(const SplitQuantPlan& p) {
  const bool grouped = p.E > 0;
  int64_t nslab = cs_slabs(p.rows);
  if (grouped) {
    nslab = 0;
    for (int64_t e = 0; e < p.E; ++e) nslab += cs_slabs(p.h_offsets[e + 1] - p.h_offsets[e]);
  }
  const SqLayout L = sq_layout(p.ws, nslab, p.cols, grouped ? p.E : 1);
  const bool nv = p.fmt == AVERIS_NVFP4;
  // column statistics: the mean (SPLIT without MEAN_GIVEN) and, for NVFP4, the residual amax;
  // from the producer's column partials when it computed them
  if (p.st_sum) {
    if (p.st_min) launch_stats_given<true>(p, L); else launch_stats_given<false>(p, L);
  } else if (p.cols > 0 && (nv || (p.split && !p.mean_given))) {
    if (p.xdt == AVERIS_BF16) {
      if (nv) launch_stats_t<uint16_t, true>(p, L); else launch_stats_t<uint16_t, false>(p, L);
    } else {
      if (nv) launch_stats_t<float, true>(p, L); else launch_stats_t<float, false>(p, L);
    }
  }
  else if (p.check) {
    // the status word is cleared by k_colstats (with the amax slots); without it, here
    hipLaunchKernelGGL(k_fill_f32, dim3(1), dim3(64), 0, p.stream, reinterpret_cast<float*>(L.slots), 1, 0.0f);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nv) return p.h16 ? launch_quant_f<AVERIS_NVFP4, true>(p, L) : launch_quant_f<AVERIS_NVFP4, false>(p, L);
  return p.h16 ? launch_quant_f<AVERIS_MXFP4, true>(p, L) : launch_quant_f<AVERIS_MXFP4, false>(p, L);
}

// ------------------------------------------------------------------------------------------
// Batched split + quantization of independent dense tensors that share the input type, format
// and flags: one statistics launch over every tensor's (strip, slab) workgroups, then one
// quantizing launch over every tensor's tiles (NVFP4 with H16: one rotated-amax launch before
// it).  Each tensor keeps its own workspace (counters, partials, amax slots), so the kernels do
// per tensor exactly what the single launches do.
// ------------------------------------------------------------------------------------------
int batch_max() { return kBatchMax; }

template <typename T, int FMT, bool H16>
static void launch_batch_t(const SplitQuantPlan* ps, const SqLayout* L, int n) {
  const SplitQuantPlan& p0 = ps[0];
  const bool nv = FMT == AVERIS_NVFP4;
  if (nv || (p0.split && !p0.mean_given)) {
    ColBatch b{};
    int total = 0;
    for (int i = 0; i < n; ++i) {
      b.a[i] = col_args(ps[i], L[i]);
      b.start[i] = total;
      total += (int)(n_strips(ps[i].cols) * L[i].nslab);
    }
    b.start[n] = total;
    b.n = n;
    hipLaunchKernelGGL((k_colstats_batch<T, nv>), dim3((unsigned)total), dim3(kThreads), 0, p0.stream, b);
  }
  QuantBatch q{};
  int total = 0;
  for (int i = 0; i < n; ++i) {
    int64_t nt = 0;
    q.a[i] = quant_args<T>(ps[i], L[i], nt);
    q.start[i] = total;
    total += (int)nt;
  }
  q.start[n] = total;
  q.n = n;
  if (FMT == AVERIS_NVFP4 && H16) {
    QuantBatch m = q;
    for (int i = 0; i < n; ++i) m.a[i] = amax_view(q.a[i], ps[i]);
    hipLaunchKernelGGL((k_quant_batch<T, FMT, H16, true>), dim3((unsigned)total), dim3(kThreads), 0, p0.stream, m);
  }
  for (int i = 0; i < n; ++i) set_outputs(q.a[i], ps[i]);
  hipLaunchKernelGGL((k_quant_batch<T, FMT, H16, false>), dim3((unsigned)total), dim3(kThreads), 0, p0.stream, q);
}

template <int FMT, bool H16>
static void launch_batch_f(const SplitQuantPlan* ps, const SqLayout* L, int n) {
  if (ps[0].xdt == AVERIS_BF16) launch_batch_t<uint16_t, FMT, H16>(ps, L, n);
  else launch_batch_t<float, FMT, H16>(ps, L, n);
}

hipError_t split_quant_batch_launch(const SplitQuantPlan* ps, int n) {
  if (n <= 0) return hipSuccess;
  SqLayout L[kBatchMax];
  for (int i = 0; i < n; ++i) L[i] = sq_layout(ps[i].ws, cs_slabs(ps[i].rows), ps[i].cols, 1);
  const bool nv = ps[0].fmt == AVERIS_NVFP4, h16 = ps[0].h16;
  if (nv) {
    if (h16) launch_batch_f<AVERIS_NVFP4, true>(ps, L, n); else launch_batch_f<AVERIS_NVFP4, false>(ps, L, n);
  } else {
    if (h16) launch_batch_f<AVERIS_MXFP4, true>(ps, L, n); else launch_batch_f<AVERIS_MXFP4, false>(ps, L, n);
  }
  return hipGetLastError();
}

}  // namespace av

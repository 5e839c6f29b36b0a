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
//   k_stats     per-slab column sum (fp64 over fp32 groups of 8 rows), min and max
//   k_finalize  fixed-order reduction of the slabs -> mu (fp32), residual amax from min/max
//               (exact: fl(x - mu) is monotone in x), integer atomic max into one slot
//   k_quant_mean  Q_b of the mean vector (own tensor scale), optional rotation
//   k_quant     re-read a 64-row tile, subtract, rotate, block amax, scale, E2M1, and emit
//               both layouts: K = features (row layout) from registers, K = tokens (column
//               layout) through an LDS transpose.  With NVFP4 + Hadamard the rotated amax is
//               not available from min/max, so k_quant first runs once in amax-only mode.
#include "launch.h"

namespace av {

constexpr int kThreads = 256;
constexpr int kSlab = 256;     // rows per k_stats workgroup
constexpr int kTileRows = 64;  // rows per k_quant tile

// ------------------------------------------------------------------------------------------
// k_stats: grid (ceil(cols / TC), nslab); TC = 32 lanes * VEC columns.  Thread t covers VEC
// columns at (t % 32) * VEC and rows slab0 + t / 32 + 8 i.
// ------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void k_stats(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                    int64_t ldx, double* __restrict__ psum,
                                                    float* __restrict__ pmin, float* __restrict__ pmax,
                                                    uint32_t* __restrict__ amax_slots) {
  constexpr int VEC = Elem<T>::VEC;
  constexpr int TC = 32 * VEC;
  __shared__ double s_sum[8][TC];
  __shared__ float s_min[8][TC];
  __shared__ float s_max[8][TC];

  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 4) amax_slots[threadIdx.x] = 0u;

  const int lane_c = threadIdx.x & 31, phase = threadIdx.x >> 5;
  const int64_t c0 = (int64_t)blockIdx.x * TC + lane_c * VEC;
  const int64_t r_begin = (int64_t)blockIdx.y * kSlab;
  const int64_t r_end = r_begin + kSlab < rows ? r_begin + kSlab : rows;
  const bool col_ok = c0 < cols;

  double sum[VEC];
  float mn[VEC], mx[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) { sum[j] = 0.0; mn[j] = __builtin_huge_valf(); mx[j] = -__builtin_huge_valf(); }

  if (col_ok) {
    // groups of 8 rows per thread: fp32 partial over the group, then one fp64 add
    for (int64_t g = r_begin + phase; g < r_end; g += 8 * 8) {
      uint4 w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t r = g + 8 * i;
        w[i] = r < r_end ? *reinterpret_cast<const uint4*>(x + r * ldx + c0) : make_uint4(0, 0, 0, 0);
      }
      float part[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) part[j] = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (g + 8 * i < r_end) {
          float v[VEC];
          Elem<T>::unpack(w[i], v);
#pragma unroll
          for (int j = 0; j < VEC; ++j) {
            part[j] += v[j];
            mn[j] = fminf(mn[j], v[j]);
            mx[j] = fmaxf(mx[j], v[j]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < VEC; ++j) sum[j] += (double)part[j];
    }
  }
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    s_sum[phase][lane_c * VEC + j] = sum[j];
    s_min[phase][lane_c * VEC + j] = mn[j];
    s_max[phase][lane_c * VEC + j] = mx[j];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < TC; c += kThreads) {
    const int64_t col = (int64_t)blockIdx.x * TC + c;
    if (col >= cols) continue;
    double s = 0.0;
    float a = __builtin_huge_valf(), b = -__builtin_huge_valf();
#pragma unroll
    for (int p = 0; p < 8; ++p) { s += s_sum[p][c]; a = fminf(a, s_min[p][c]); b = fmaxf(b, s_max[p][c]); }
    const int64_t o = (int64_t)blockIdx.y * cols + col;
    psum[o] = s; pmin[o] = a; pmax[o] = b;
  }
}

// ------------------------------------------------------------------------------------------
// k_finalize: one thread per column.  mode bit 0 = SPLIT, bit 1 = MEAN_GIVEN.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_finalize(const double* __restrict__ psum, const float* __restrict__ pmin,
                                                       const float* __restrict__ pmax, int nslab, int64_t rows,
                                                       int64_t cols, int mode, float* __restrict__ mean,
                                                       uint32_t* __restrict__ amax_slot) {
  __shared__ float s_red[kThreads / 64];
  const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  float amax = 0.0f;
  if (c < cols && rows > 0) {
    double s = 0.0;
    float a = __builtin_huge_valf(), b = -__builtin_huge_valf();
    for (int p = 0; p < nslab; ++p) {
      const int64_t o = (int64_t)p * cols + c;
      s += psum[o]; a = fminf(a, pmin[o]); b = fmaxf(b, pmax[o]);
    }
    float mu = 0.0f;
    if (mode & 1) {
      if (mode & 2) mu = mean[c];
      else { mu = (float)(s / (double)rows); mean[c] = mu; }
    }
    amax = fmaxf(__fsub_rn(b, mu), __fsub_rn(mu, a));
  } else if (c < cols && (mode & 1) && !(mode & 2)) {
    mean[c] = 0.0f;
  }
  // workgroup max, then one integer atomic max (amax >= 0, so its bits order like uints)
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) amax = wave_xor_max(amax, m);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = amax;
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = s_red[0];
    for (int i = 1; i < kThreads / 64; ++i) v = fmaxf(v, s_red[i]);
    atomicMax(amax_slot, __float_as_uint(v));
  }
}

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
// k_quant_mean: one workgroup quantizes mu [cols] along its length.
// ------------------------------------------------------------------------------------------
template <int FMT, bool H16>
__global__ __launch_bounds__(kThreads) void k_quant_mean(const float* __restrict__ mean, int64_t cols, int64_t k_pad,
                                                         uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                         float* __restrict__ tscale) {
  constexpr int G = FMT == AVERIS_MXFP4 ? 32 : 16;
  __shared__ float s_red[kThreads / 64];
  const int64_t nblk = cols / G;
  float s_dec = 0.0f;
  if (FMT == AVERIS_NVFP4) {
    float amax = 0.0f;
    for (int64_t b = threadIdx.x; b < nblk; b += kThreads) {
      float v[32];
#pragma unroll
      for (int j = 0; j < G; ++j) v[j] = mean[b * G + j];
      if (H16) h16_inreg(v);
#pragma unroll
      for (int j = 0; j < G; ++j) amax = fmaxf(amax, fabsf(v[j]));
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = wave_xor_max(amax, m);
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = s_red[0];
    for (int i = 1; i < kThreads / 64; ++i) amax = fmaxf(amax, s_red[i]);
    s_dec = nvfp4_tensor_scale(amax);
    if (threadIdx.x == 0) tscale[0] = s_dec;
  }
  for (int64_t b = threadIdx.x; b < nblk; b += kThreads) {
    float v[32];
#pragma unroll
    for (int j = 0; j < G; ++j) v[j] = mean[b * G + j];
    if (H16) {
      h16_inreg(v);
      if (G == 32) h16_inreg(v + 16);
    }
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < G; ++j) amax = fmaxf(amax, fabsf(v[j]));
    const BlockQ q = block_params<FMT>(amax, s_dec);
#pragma unroll
    for (int j = 0; j < G; ++j) v[j] = __fmul_rn(v[j], q.mul);
#pragma unroll
    for (int j = 0; j < G / 8; ++j) {
      const uint32_t w = q.dead ? 0u : pack8_fp4(v + 8 * j);
      *reinterpret_cast<uint32_t*>(codes + b * (G / 2) + 4 * j) = w;
    }
    scales[scale_offset(0, b, k_pad, G)] = (uint8_t)q.sbyte;
  }
}

// ------------------------------------------------------------------------------------------
// k_quant: one workgroup per 64-row x TC-column tile (TC = 32 * VEC: 256 bf16 or 128 fp32
// columns).  Grid is 1-D over tiles_r x tiles_c, XCD-remapped with the row tile fastest.
//
// Row layout: thread t holds VEC consecutive columns (t % 32) * VEC of rows t / 32 + 8 i; a
// block of G columns spans G / VEC lanes and its amax is a lane-shuffle max.
// Column layout: the raw tile goes to LDS; thread t then takes column t % TC and the 32-row
// half (t / TC + j * (256 / TC)) and quantizes down the column in registers.
//
// AMAX_ONLY: compute max |rotated residual| of each layout and atomically max it into
// amax_slots[1] (row) and amax_slots[2] (column); nothing is stored.
// ------------------------------------------------------------------------------------------
struct QuantArgs {
  const void* x;
  int64_t rows, cols, ldx;
  const float* mean;           // nullptr: no subtraction
  const uint32_t* amax_slots;  // NVFP4: [0] residual amax, [1] rotated row amax, [2] rotated col amax
  uint32_t* amax_out;          // AMAX_ONLY target (same buffer as amax_slots)
  uint8_t* row_codes;          // nullptr: row layout not written
  uint8_t* row_scales;
  float* row_ts;
  uint8_t* col_codes;          // nullptr: column layout not written
  uint8_t* col_scales;
  float* col_ts;
  int64_t col_kpad;            // padded token count of the column layout
  int64_t row_kpad;            // padded column count of the row layout (its row stride in elements)
  int tiles_r, tiles_c;
};

template <typename T, int FMT, bool H16, bool AMAX_ONLY>
__global__ __launch_bounds__(kThreads) void k_quant(QuantArgs a) {
  constexpr int VEC = Elem<T>::VEC;
  constexpr int TC = 32 * VEC;
  constexpr int G = FMT == AVERIS_MXFP4 ? 32 : 16;
  constexpr int LPB = G / VEC;  // lanes per row-layout block
  __shared__ T s_tile[kTileRows][TC];
  __shared__ float s_red[2][kThreads / 64];

  const int tile = xcd_remap(blockIdx.x, a.tiles_r * a.tiles_c);
  const int tr = tile % a.tiles_r, tc = tile / a.tiles_r;
  const int64_t r0 = (int64_t)tr * kTileRows, c0 = (int64_t)tc * TC;
  const int lane_c = threadIdx.x & 31, phase = threadIdx.x >> 5;
  const int lane = threadIdx.x & 63;
  const T* x = reinterpret_cast<const T*>(a.x);

  // tensor decode scales (NVFP4): residual amax, or the rotated amax per layout
  float sd_row = 0.0f, sd_col = 0.0f;
  if (FMT == AVERIS_NVFP4 && !AMAX_ONLY) {
    const float ar = __uint_as_float(a.amax_slots[H16 ? 1 : 0]);
    const float ac = __uint_as_float(a.amax_slots[H16 ? 2 : 0]);
    sd_row = nvfp4_tensor_scale(ar);
    sd_col = nvfp4_tensor_scale(ac);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      if (a.row_ts) a.row_ts[0] = sd_row;
      if (a.col_ts) a.col_ts[0] = sd_col;
    }
  }

  // ---- load the tile (rows >= a.rows read as 0) ----
  const int64_t cc = c0 + lane_c * VEC;
  const bool col_ok = cc < a.cols;
  uint4 w[kTileRows / 8];
#pragma unroll
  for (int i = 0; i < kTileRows / 8; ++i) {
    const int64_t r = r0 + phase + 8 * i;
    w[i] = (col_ok && r < a.rows) ? *reinterpret_cast<const uint4*>(x + r * a.ldx + cc) : make_uint4(0, 0, 0, 0);
  }
  float mu[VEC];
#pragma unroll
  for (int j = 0; j < VEC; ++j) mu[j] = (a.mean && col_ok) ? a.mean[cc + j] : 0.0f;

  float amax_row_acc = 0.0f, amax_col_acc = 0.0f;

  // ---- row layout (K = cols) ----
  if (a.row_codes || AMAX_ONLY) {
#pragma unroll
    for (int i = 0; i < kTileRows / 8; ++i) {
      const int64_t r = r0 + phase + 8 * i;
      float v[VEC];
      Elem<T>::unpack(w[i], v);
#pragma unroll
      for (int j = 0; j < VEC; ++j) v[j] = __fsub_rn(v[j], mu[j]);
      if (H16) h16_lanes<VEC>(v, lane);
      float m = 0.0f;
#pragma unroll
      for (int j = 0; j < VEC; ++j) m = fmaxf(m, fabsf(v[j]));
#pragma unroll
      for (int s = 1; s < LPB; s <<= 1) m = wave_xor_max(m, s);
      if (AMAX_ONLY) {
        if (r < a.rows && col_ok) amax_row_acc = fmaxf(amax_row_acc, m);
        continue;
      }
      const BlockQ q = block_params<FMT>(m, sd_row);
#pragma unroll
      for (int j = 0; j < VEC; ++j) v[j] = __fmul_rn(v[j], q.mul);
      if (r < a.rows && col_ok) {
        uint8_t* dst = a.row_codes + r * (a.row_kpad / 2) + cc / 2;
        if (VEC == 8) *reinterpret_cast<uint32_t*>(dst) = q.dead ? 0u : pack8_fp4(v);
        else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(q.dead ? 0u : pack4_fp4(v));
        if ((lane_c % LPB) == 0) a.row_scales[scale_offset(r, cc / G, a.row_kpad, G)] = (uint8_t)q.sbyte;
      }
    }
  }

  // ---- column layout (K = rows) through LDS ----
  if (a.col_codes || AMAX_ONLY) {
#pragma unroll
    for (int i = 0; i < kTileRows / 8; ++i)
      *reinterpret_cast<uint4*>(&s_tile[phase + 8 * i][lane_c * VEC]) = w[i];
    __syncthreads();
    constexpr int HALVES = kTileRows / 32;       // 32-row groups per tile
    constexpr int ITEMS = TC * HALVES / kThreads; // items per thread
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int item = threadIdx.x + it * kThreads;
      const int c = item % TC, half = item / TC;
      const int64_t col = c0 + c;
      const float m_c = (a.mean && col < a.cols) ? a.mean[col] : 0.0f;
      float v[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const int rr = half * 32 + j;
        const float xv = Elem<T>::load1(&s_tile[rr][c]);
        v[j] = (r0 + rr < a.rows) ? __fsub_rn(xv, m_c) : 0.0f;
      }
      if (H16) { h16_inreg(v); h16_inreg(v + 16); }
#pragma unroll
      for (int b = 0; b < 32 / G; ++b) {
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < G; ++j) m = fmaxf(m, fabsf(v[b * G + j]));
        if (AMAX_ONLY) {
          if (col < a.cols) amax_col_acc = fmaxf(amax_col_acc, m);
          continue;
        }
        const BlockQ q = block_params<FMT>(m, sd_col);
#pragma unroll
        for (int j = 0; j < G; ++j) v[b * G + j] = __fmul_rn(v[b * G + j], q.mul);
        if (col < a.cols) {
          const int64_t k0 = r0 + half * 32 + b * G;  // first token of this block
          uint8_t* dst = a.col_codes + col * (a.col_kpad / 2) + k0 / 2;
          if (G == 32) {
            uint4 o;
            o.x = q.dead ? 0u : pack8_fp4(v + b * G);
            o.y = q.dead ? 0u : pack8_fp4(v + b * G + 8);
            o.z = q.dead ? 0u : pack8_fp4(v + b * G + 16);
            o.w = q.dead ? 0u : pack8_fp4(v + b * G + 24);
            *reinterpret_cast<uint4*>(dst) = o;
          } else {
            uint2 o;
            o.x = q.dead ? 0u : pack8_fp4(v + b * G);
            o.y = q.dead ? 0u : pack8_fp4(v + b * G + 8);
            *reinterpret_cast<uint2*>(dst) = o;
          }
          a.col_scales[scale_offset(col, k0 / G, a.col_kpad, G)] = (uint8_t)q.sbyte;
        }
      }
    }
  }

  if (AMAX_ONLY) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      amax_row_acc = wave_xor_max(amax_row_acc, m);
      amax_col_acc = wave_xor_max(amax_col_acc, m);
    }
    if (lane == 0) { s_red[0][threadIdx.x >> 6] = amax_row_acc; s_red[1][threadIdx.x >> 6] = amax_col_acc; }
    __syncthreads();
    if (threadIdx.x == 0) {
      float u = s_red[0][0], v = s_red[1][0];
      for (int i = 1; i < kThreads / 64; ++i) { u = fmaxf(u, s_red[0][i]); v = fmaxf(v, s_red[1][i]); }
      atomicMax(a.amax_out + 1, __float_as_uint(u));
      atomicMax(a.amax_out + 2, __float_as_uint(v));
    }
  }
}

// Zero bytes [start, start + len) of each of `rows` rows of stride ld (K padding of a layout).
__global__ void k_zero_tail(uint8_t* __restrict__ base, int64_t rows, int64_t ld, int64_t start, int64_t len) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = i / len, b = i % len;
  if (r < rows) base[r * ld + start + b] = 0;
}

// Zero the tiled scale bytes outside the data: blocks [k/g, k_pad/g) of rows [0, outer) and
// every block of the group-padding rows [outer, round_up(outer, 32)).
__global__ void k_zero_scale_pad(uint8_t* __restrict__ scales, int64_t outer, int64_t k, int64_t k_pad, int g) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nb = k_pad / g, kb = k / g, tail = nb - kb;
  const int64_t n1 = outer * tail, n2 = (round_up(outer, 32) - outer) * nb;
  int64_t r, b;
  if (i < n1) { r = i / tail; b = kb + i % tail; }
  else if (i < n1 + n2) { r = outer + (i - n1) / nb; b = (i - n1) % nb; }
  else return;
  scales[scale_offset(r, b, k_pad, g)] = 0;
}

__global__ void k_fill_f32(float* p, int n, float v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ------------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------------
static int64_t slab_count(int64_t rows) {
  const int64_t n = ceil_div(rows, kSlab);
  return n > 0 ? n : 1;  // one (empty) slab when rows == 0
}

size_t split_quant_ws_bytes(int64_t rows, int64_t cols) {
  const int64_t nslab = slab_count(rows);
  return 256 + (size_t)nslab * cols * (8 + 4 + 4) + 256;
}



template <typename T, int FMT, bool H16>
static hipError_t launch_quant_t(const SplitQuantPlan& p, uint32_t* slots) {
  constexpr int TC = 32 * Elem<T>::VEC;
  QuantArgs a{};
  a.x = p.x; a.rows = p.rows; a.cols = p.cols; a.ldx = p.ldx;
  a.mean = p.split ? p.mean : nullptr;
  a.amax_slots = slots; a.amax_out = slots;
  const int64_t col_kpad = round_up(p.rows, kKPad);
  a.col_kpad = col_kpad;
  a.row_kpad = round_up(p.cols, kKPad);
  a.tiles_c = (int)ceil_div(p.cols, TC);
  // column layout covers the padding rows too (they are zero residuals)
  a.tiles_r = (int)ceil_div(p.q_col ? col_kpad : p.rows, kTileRows);
  const int ntiles = a.tiles_r * a.tiles_c;
  if (ntiles == 0) {  // empty operands: still define their tensor scales (0)
    if (FMT == AVERIS_NVFP4) {
      float* ts[2] = {p.q_row ? p.q_row->tensor_scale : nullptr, p.q_col ? p.q_col->tensor_scale : nullptr};
      for (float* t : ts)
        if (t) hipLaunchKernelGGL(k_fill_f32, dim3(1), dim3(64), 0, p.stream, t, 1, 0.0f);
    }
    return hipGetLastError();
  }
  if (FMT == AVERIS_NVFP4 && H16) {
    QuantArgs m = a;
    hipLaunchKernelGGL((k_quant<T, FMT, H16, true>), dim3(ntiles), dim3(kThreads), 0, p.stream, m);
  }
  if (p.q_row) { a.row_codes = p.q_row->codes; a.row_scales = p.q_row->scales; a.row_ts = p.q_row->tensor_scale; }
  if (p.q_col) { a.col_codes = p.q_col->codes; a.col_scales = p.q_col->scales; a.col_ts = p.q_col->tensor_scale; }
  hipLaunchKernelGGL((k_quant<T, FMT, H16, false>), dim3(ntiles), dim3(kThreads), 0, p.stream, a);
  return hipGetLastError();
}

template <int FMT, bool H16>
static hipError_t launch_quant_f(const SplitQuantPlan& p, uint32_t* slots) {
  return p.xdt == AVERIS_BF16 ? launch_quant_t<uint16_t, FMT, H16>(p, slots) : launch_quant_t<float, FMT, H16>(p, slots);
}

// Zero the padding of an operand the quantizer writes: codes [k, k_pad) of every row, and the
// scale bytes outside the data (K tail and the rows that pad the last 32-row group).
static void zero_padding(const averis_qtensor* q, int fmt, hipStream_t s) {
  const int G = fmt == AVERIS_MXFP4 ? 32 : 16;
  if (!q || q->outer == 0 || q->k_pad == 0) return;
  if (q->k_pad > q->k) {
    const int64_t cl = (q->k_pad - q->k) / 2;
    hipLaunchKernelGGL(k_zero_tail, dim3((unsigned)ceil_div(q->outer * cl, 256)), dim3(256), 0, s, q->codes, q->outer,
                       q->k_pad / 2, q->k / 2, cl);
  }
  const int64_t n = q->outer * (q->k_pad / G - q->k / G) + (round_up(q->outer, 32) - q->outer) * (q->k_pad / G);
  if (n > 0)
    hipLaunchKernelGGL(k_zero_scale_pad, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, q->scales, q->outer, q->k,
                       q->k_pad, G);
}

hipError_t split_quant_launch(const SplitQuantPlan& p) {
  uint8_t* ws = reinterpret_cast<uint8_t*>(p.ws);
  uint32_t* slots = reinterpret_cast<uint32_t*>(ws);
  const int64_t nslab = slab_count(p.rows);
  double* psum = reinterpret_cast<double*>(ws + 256);
  float* pmin = reinterpret_cast<float*>(ws + 256 + (size_t)nslab * p.cols * 8);
  float* pmax = pmin + (size_t)nslab * p.cols;

  const bool need_stats = p.fmt == AVERIS_NVFP4 || (p.split && !p.mean_given);
  if (need_stats) {
    const int tc = p.xdt == AVERIS_BF16 ? 256 : 128;
    const dim3 grid((unsigned)ceil_div(p.cols, tc), (unsigned)nslab);
    if (p.xdt == AVERIS_BF16)
      hipLaunchKernelGGL(k_stats<uint16_t>, grid, dim3(kThreads), 0, p.stream, (const uint16_t*)p.x, p.rows, p.cols,
                         p.ldx, psum, pmin, pmax, slots);
    else
      hipLaunchKernelGGL(k_stats<float>, grid, dim3(kThreads), 0, p.stream, (const float*)p.x, p.rows, p.cols, p.ldx,
                         psum, pmin, pmax, slots);
    const int mode = (p.split ? 1 : 0) | (p.mean_given ? 2 : 0);
    hipLaunchKernelGGL(k_finalize, dim3((unsigned)ceil_div(p.cols, kThreads)), dim3(kThreads), 0, p.stream, psum, pmin,
                       pmax, (int)ceil_div(p.rows, kSlab), p.rows, p.cols, mode, p.mean, slots);
  }
  if (p.split) {
    if (p.fmt == AVERIS_NVFP4) {
      if (p.h16) hipLaunchKernelGGL((k_quant_mean<AVERIS_NVFP4, true>), dim3(1), dim3(kThreads), 0, p.stream, p.mean, p.cols, p.q_mean->k_pad, p.q_mean->codes, p.q_mean->scales, p.q_mean->tensor_scale);
      else hipLaunchKernelGGL((k_quant_mean<AVERIS_NVFP4, false>), dim3(1), dim3(kThreads), 0, p.stream, p.mean, p.cols, p.q_mean->k_pad, p.q_mean->codes, p.q_mean->scales, p.q_mean->tensor_scale);
    } else {
      if (p.h16) hipLaunchKernelGGL((k_quant_mean<AVERIS_MXFP4, true>), dim3(1), dim3(kThreads), 0, p.stream, p.mean, p.cols, p.q_mean->k_pad, p.q_mean->codes, p.q_mean->scales, (float*)nullptr);
      else hipLaunchKernelGGL((k_quant_mean<AVERIS_MXFP4, false>), dim3(1), dim3(kThreads), 0, p.stream, p.mean, p.cols, p.q_mean->k_pad, p.q_mean->codes, p.q_mean->scales, (float*)nullptr);
    }
  }
  zero_padding(p.q_row, p.fmt, p.stream);  // the column layout's padding rows are written by k_quant
  zero_padding(p.q_mean, p.fmt, p.stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.fmt == AVERIS_NVFP4) return p.h16 ? launch_quant_f<AVERIS_NVFP4, true>(p, slots) : launch_quant_f<AVERIS_NVFP4, false>(p, slots);
  return p.h16 ? launch_quant_f<AVERIS_MXFP4, true>(p, slots) : launch_quant_f<AVERIS_MXFP4, false>(p, slots);
}

}  // namespace av

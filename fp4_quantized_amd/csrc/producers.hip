// Producers of a linear layer's input that also write its column statistics (gfx950).
//
// The Averis split ("均值偏置的诅咒与祝福" explainer, paper.rainbus.top, section 方法步骤详情)
// needs the column mean of X over all token rows before any element can be quantized; computed
// by the split itself that is a second pass over X.  The kernel that writes X can sum its
// columns as it stores them.  In a transformer block the linears' inputs are written by the
// normalization (q/k/v and gate/up read RMSNorm's output) and by the activation (down reads
// SwiGLU's output), so these two producers write the same column partials as the GEMM epilogue
// (fp32 sums, optionally minima and maxima, of the values as stored, per 64-row part), and
// averis_split_quant_stats starts the split from them.
//
//   RMSNorm: y = x * (1 / sqrt(mean_c(x^2) + eps)) * w      (Zhang and Sennrich, 2019)
//   SwiGLU:  y = silu(g) * u,  silu(g) = g / (1 + exp(-g))  (Shazeer, 2020)
//
// One workgroup of eight waves per 64-row part and 512-column block; wave w takes rows
// [8 w, 8 w + 8) of the part.  Lane l owns the eight columns 8 l + 512 b of each
// 512-column block b.  Per block the wave loads its eight rows at once, computes and stores
// them, and sums its columns over them in row order; the eight waves' sums meet in LDS and are
// added in wave order.  RMSNorm first reads its rows in full for their sums of squares (every
// column block's workgroup does; the repeats come from the caches).
#include "launch.h"

namespace av {

constexpr int kProdRows = 64;   // rows per workgroup = rows per statistics part
constexpr int kProdWaves = 8;
constexpr int kProdWaveRows = kProdRows / kProdWaves;
constexpr int kProdBlock = 512;  // columns per block (64 lanes x 8)

struct ProdArgs {
  const void* x; const void* u;  // RMSNorm: x; SwiGLU: gate x, up u
  int64_t rows, cols, ldx;
  const float* w; float eps;     // RMSNorm weight [cols] and epsilon
  void* y; int64_t ldy;
  float* st_sum; float* st_min; float* st_max;  // [part][cols], or st_sum null: no statistics
};

// Raw 16-byte loads of 8 elements (two for fp32), unpacked when used.
template <typename T>
struct Raw8 {
  uint4 w[sizeof(T) / 2];
  __device__ __forceinline__ void load(const T* p) {
#pragma unroll
    for (int k = 0; k < (int)(sizeof(T) / 2); ++k) w[k] = *reinterpret_cast<const uint4*>(p + 4 * k);
  }
  __device__ __forceinline__ void unpack(float* v) const {
    if constexpr (sizeof(T) == 2) Elem<T>::unpack(w[0], v);
    else { Elem<T>::unpack(w[0], v); Elem<T>::unpack(w[1], v + 4); }
  }
};

// Store 8 values as T; v becomes the values as stored.
template <typename T>
__device__ __forceinline__ void store8(T* p, float* v) {
  if constexpr (sizeof(T) == 2) {
    const uint4 o = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                               pack_bf16x2(v[6], v[7]));
    *reinterpret_cast<uint4*>(p) = o;
    Elem<T>::unpack(o, v);
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = __fadd_rn(v, __shfl_xor(v, m, 64));
  return v;
}

// OP 0: RMSNorm, OP 1: SwiGLU.  MINMAX: column minima and maxima too.
template <typename T, int OP, bool MINMAX>
__global__ __launch_bounds__(64 * kProdWaves) void k_producer(ProdArgs a) {
  constexpr int W = kProdWaves, kProdBatch = kProdWaveRows;
  __shared__ float s_sum[W][kProdBlock];
  __shared__ float s_min[MINMAX ? W : 1][MINMAX ? kProdBlock : 1], s_max[MINMAX ? W : 1][MINMAX ? kProdBlock : 1];
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
  const int64_t part = blockIdx.x, r0 = part * kProdRows + (int64_t)wave * kProdWaveRows;
  const int nr = (int)(a.rows - r0 < kProdWaveRows ? (a.rows - r0 > 0 ? a.rows - r0 : 0) : kProdWaveRows);
  const T* x = reinterpret_cast<const T*>(a.x);
  const T* up = reinterpret_cast<const T*>(a.u);
  T* y = reinterpret_cast<T*>(a.y);
  const int nblk = (int)ceil_div(a.cols, kProdBlock);
  // one column block per workgroup (grid y); RMSNorm reads its rows in full for their sums of
  // squares first
  const int b_first = (int)blockIdx.y, b_end = b_first + 1;
  const bool stats = a.st_sum != nullptr;

  // RMSNorm: 1 / sqrt(mean of squares + eps) of each of the wave's rows (fp32 sum of squares:
  // each lane's columns in order, then a butterfly over the lanes)
  float rs[kProdWaveRows];
  if constexpr (OP == 0) {
    float ss[kProdWaveRows];
#pragma unroll
    for (int i = 0; i < kProdWaveRows; ++i) ss[i] = 0.0f;
    for (int b = 0; b < nblk; ++b) {
      const int64_t c = (int64_t)b * kProdBlock + lane * 8;
      if (c >= a.cols) continue;
#pragma unroll
      for (int i0 = 0; i0 < kProdWaveRows; i0 += kProdBatch) {
        Raw8<T> rx[kProdBatch];
#pragma unroll
        for (int i = 0; i < kProdBatch; ++i)
          if (i0 + i < nr) rx[i].load(x + (r0 + i0 + i) * a.ldx + c);
#pragma unroll
        for (int i = 0; i < kProdBatch; ++i) {
          if (i0 + i < nr) {
            float v[8];
            rx[i].unpack(v);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss[i0 + i] = __fadd_rn(ss[i0 + i], __fmul_rn(v[e], v[e]));
          }
        }
      }
    }
    const float inv_cols = __fdiv_rn(1.0f, (float)a.cols);
#pragma unroll
    for (int i = 0; i < kProdWaveRows; ++i) {
      const float ms = __fmul_rn(wave_sum(ss[i]), inv_cols);
      rs[i] = __fdiv_rn(1.0f, __fsqrt_rn(__fadd_rn(ms, a.eps)));
    }
  }

  for (int b = b_first; b < b_end; ++b) {
    const int64_t c = (int64_t)b * kProdBlock + lane * 8;
    const bool cin = c < a.cols;
    float wv[8];
    if constexpr (OP == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) wv[e] = cin ? a.w[c + e] : 0.0f;
    }
    float cs[8], cmn[8], cmx[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) { cs[e] = 0.0f; cmn[e] = __builtin_huge_valf(); cmx[e] = -__builtin_huge_valf(); }
#pragma unroll
    for (int i0 = 0; i0 < kProdWaveRows; i0 += kProdBatch) {
      Raw8<T> rx[kProdBatch], ru[OP == 1 ? kProdBatch : 1];
#pragma unroll
      for (int i = 0; i < kProdBatch; ++i) {
        if (cin && i0 + i < nr) {
          rx[i].load(x + (r0 + i0 + i) * a.ldx + c);
          if constexpr (OP == 1) ru[i].load(up + (r0 + i0 + i) * a.ldx + c);
        }
      }
#pragma unroll
      for (int i = 0; i < kProdBatch; ++i) {
        if (cin && i0 + i < nr) {
          float v[8], o[8];
          rx[i].unpack(v);
          if constexpr (OP == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = __fmul_rn(__fmul_rn(v[e], rs[i0 + i]), wv[e]);
          } else {
            float uu[8];
            ru[i].unpack(uu);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = __fmul_rn(__fdiv_rn(v[e], __fadd_rn(1.0f, expf(-v[e]))), uu[e]);
          }
          store8(y + (r0 + i0 + i) * a.ldy + c, o);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            cs[e] = __fadd_rn(cs[e], o[e]);
            if constexpr (MINMAX) { cmn[e] = fminf(cmn[e], o[e]); cmx[e] = fmaxf(cmx[e], o[e]); }
          }
        }
      }
    }
    if (!stats) continue;
    // the waves' column sums, added in wave order
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s_sum[wave][lane * 8 + e] = cs[e];
      if constexpr (MINMAX) { s_min[wave][lane * 8 + e] = cmn[e]; s_max[wave][lane * 8 + e] = cmx[e]; }
    }
    __syncthreads();
    for (int k = threadIdx.x; k < kProdBlock; k += 64 * W) {
      const int64_t col = (int64_t)b * kProdBlock + k;
      if (col < a.cols) {
        float t = s_sum[0][k], lo = MINMAX ? s_min[0][k] : 0.0f, hi = MINMAX ? s_max[0][k] : 0.0f;
#pragma unroll
        for (int q = 1; q < W; ++q) {
          t = __fadd_rn(t, s_sum[q][k]);
          if constexpr (MINMAX) { lo = fminf(lo, s_min[q][k]); hi = fmaxf(hi, s_max[q][k]); }
        }
        a.st_sum[part * a.cols + col] = t;
        if constexpr (MINMAX) { a.st_min[part * a.cols + col] = lo; a.st_max[part * a.cols + col] = hi; }
      }
    }
    __syncthreads();
  }
}

int64_t producer_part_rows() { return kProdRows; }

template <typename T, int OP>
static void launch_prod_t(const ProdArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(a.rows, kProdRows), (unsigned)ceil_div(a.cols, kProdBlock));
  if (a.st_min) hipLaunchKernelGGL((k_producer<T, OP, true>), grid, dim3(64 * kProdWaves), 0, s, a);
  else hipLaunchKernelGGL((k_producer<T, OP, false>), grid, dim3(64 * kProdWaves), 0, s, a);
}

hipError_t producer_launch(int op, int dt, const void* x, const void* u, int64_t rows, int64_t cols, int64_t ldx,
                           const float* w, float eps, void* y, int64_t ldy, float* st_sum, float* st_min,
                           float* st_max, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  ProdArgs a{x, u, rows, cols, ldx, w, eps, y, ldy, st_sum, st_min, st_max};
  if (dt == AVERIS_BF16) {
    if (op == 0) launch_prod_t<uint16_t, 0>(a, s); else launch_prod_t<uint16_t, 1>(a, s);
  } else {
    if (op == 0) launch_prod_t<float, 0>(a, s); else launch_prod_t<float, 1>(a, s);
  }
  return hipGetLastError();
}

}  // namespace av

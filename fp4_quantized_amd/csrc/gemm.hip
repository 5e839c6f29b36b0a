// Quantized GEMMs of the Averis linear layer for gfx950.
//
// "均值偏置的诅咒与祝福：FP4量化大语言模型训练" explainer (paper.rainbus.top), section 方法步骤详情:
//   Y = 1 (mu_X W) + X_R W,  dL/dX = 1 (mu_D W^T) + D_R W^T,  dL/dW = X_R^T D_R + l mu_X^T mu_D
// with every operand FP4-quantized; the mean term of Y and dX is a broadcast row, and in dW it
// is a rank-one outer product (the cross terms vanish for zero-mean residuals).
//
// One tile loop C[M, N] = A[M, K] B[N, K]^T over K-inner packed E2M1 operands:
//   MXFP4: v_mfma_scale_f32_32x32x64_f8f6f4 consumes the codes and the E8M0 block scales
//          directly (lane l holds row l % 32, K elements 32 (l / 32) .. + 31 = one MX block).
//   NVFP4: E4M3 scales are not powers of two, which the scaled MFMA cannot apply, so each
//          lane dequantizes its 32 codes exactly to bf16 (code x E4M3 value has <= 6
//          significant bits) and issues four v_mfma_f32_32x32x16_bf16; the fp32 tensor scales
//          multiply the accumulator in the epilogue.
// Epilogue: out = alpha * acc + bias[col] + r1 * u[row] * v[col] (+ C when accumulating),
// alpha = product of the operands' tensor decode scales (NVFP4) or 1.
#include "launch.h"

namespace av {

constexpr int kGemmThreads = 256;
constexpr int BM = 128, BN = 128;
constexpr int BKB = 128;           // bytes of codes per row per K-step (256 elements)
constexpr int BKE = 2 * BKB;       // elements per K-step
constexpr int LDS_ROW = BKB + 16;  // padded LDS row stride (bytes)

struct GemmArgs {
  const uint8_t* a_codes; const uint8_t* a_scales; int64_t lda_b; int64_t lds_a;  // row strides: bytes of codes, bytes of scales
  const uint8_t* b_codes; const uint8_t* b_scales; int64_t ldb_b; int64_t lds_b;
  const float* a_ts; const float* b_ts;  // tensor decode scales (NVFP4) or nullptr
  int64_t M, N, K;                      // K = padded length (multiple of 128)
  void* c; int64_t ldc; int c_bf16;     // output (or split-K partials base when splits > 1)
  const float* bias;                    // [N] or nullptr
  const float* r1u; const float* r1v; float r1;  // rank-one term r1 * u[row] * v[col], or nullptr
  int accumulate;
  int splits; int64_t k_chunk;          // K range per split (multiple of BKE), partials at c + s * M * N
  int tiles_m, tiles_n;
};

__device__ inline uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// 32 E2M1 codes (16 bytes) times two block scales (elements 0-15: s0, 16-31: s1) -> 4 x 8 bf16.
__device__ inline void dequant32_bf16(const uint4& c, float s0, float s1, v8bf* out) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float s = q < 2 ? s0 : s1;
    uint32_t h[4];
#pragma unroll
    for (int bsel = 0; bsel < 4; ++bsel) {
      float2 f;
      switch (bsel) {
        case 0: { auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 0); f = make_float2(r[0], r[1]); break; }
        case 1: { auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 1); f = make_float2(r[0], r[1]); break; }
        case 2: { auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 2); f = make_float2(r[0], r[1]); break; }
        default: { auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 3); f = make_float2(r[0], r[1]); break; }
      }
      // exact products, so dropping the low 16 bits is an exact bf16 conversion
      const uint32_t lo = __float_as_uint(f.x * s) >> 16, hi = __float_as_uint(f.y * s) & 0xFFFF0000u;
      h[bsel] = lo | hi;
    }
    out[q] = __builtin_bit_cast(v8bf, make_uint4(h[0], h[1], h[2], h[3]));
  }
}

template <int FMT>
__global__ __launch_bounds__(kGemmThreads) void k_gemm(GemmArgs g) {
  constexpr int G = FMT == AVERIS_MXFP4 ? 32 : 16;
  constexpr int SB = BKE / G;  // scale bytes per row per K-step (8 or 16)
  __shared__ __attribute__((aligned(16))) uint8_t sA[BM * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint8_t sB[BN * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint8_t sSA[BM * SB];
  __shared__ __attribute__((aligned(16))) uint8_t sSB[BN * SB];

  const int ntiles = g.tiles_m * g.tiles_n;
  const int lin = xcd_remap(blockIdx.x, ntiles * g.splits);
  const int split = lin / ntiles;
  const int tile = lin % ntiles;
  const int tm = tile / g.tiles_n, tn = tile % g.tiles_n;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t kb = (int64_t)split * g.k_chunk;
  const int64_t ke = kb + g.k_chunk < g.K ? kb + g.k_chunk : g.K;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;  // 2 x 2 waves, 64 x 64 each

  // global -> register staging: 16 KB of codes per operand = 4 x 16 B per thread
  const int ld_chunk = tid & 7, ld_row = tid >> 3;  // 8 threads per 128-byte row, 32 rows per pass
  uint4 ra[4], rb[4];
  uint32_t rsa[SB / 8], rsb[SB / 8];  // scales: BM * SB bytes = 1 or 2 KB -> 4 or 8 bytes/thread

  auto gload = [&](int64_t k0) {
    const int64_t kbyte = k0 / 2;
    const bool kin = k0 + (int64_t)(ld_chunk + 1) * 32 <= ke;  // this 16-byte chunk (32 elems) in range
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t ra_row = m0 + ld_row + 32 * i, rb_row = n0 + ld_row + 32 * i;
      ra[i] = (kin && ra_row < g.M) ? *reinterpret_cast<const uint4*>(g.a_codes + ra_row * g.lda_b + kbyte + ld_chunk * 16) : make_uint4(0, 0, 0, 0);
      rb[i] = (kin && rb_row < g.N) ? *reinterpret_cast<const uint4*>(g.b_codes + rb_row * g.ldb_b + kbyte + ld_chunk * 16) : make_uint4(0, 0, 0, 0);
    }
    // scales: thread t covers row t / (256 / BM) ... one dword (4 scale bytes) per load
#pragma unroll
    for (int i = 0; i < SB / 8; ++i) {
      const int idx = tid + i * kGemmThreads;     // dword index within the BM x SB tile
      const int row = idx / (SB / 4), dw = idx % (SB / 4);
      const int64_t kblk = k0 / G + dw * 4;        // first block of this dword
      const bool sin = kblk * G + 4 * G <= ke;      // all 4 blocks inside the K range
      const int64_t ar = m0 + row, br = n0 + row;
      rsa[i] = (sin && ar < g.M) ? *reinterpret_cast<const uint32_t*>(g.a_scales + ar * g.lds_a + kblk) : 0u;
      rsb[i] = (sin && br < g.N) ? *reinterpret_cast<const uint32_t*>(g.b_scales + br * g.lds_b + kblk) : 0u;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4*>(sA + (ld_row + 32 * i) * LDS_ROW + ld_chunk * 16) = ra[i];
      *reinterpret_cast<uint4*>(sB + (ld_row + 32 * i) * LDS_ROW + ld_chunk * 16) = rb[i];
    }
#pragma unroll
    for (int i = 0; i < SB / 8; ++i) {
      const int idx = tid + i * kGemmThreads;
      reinterpret_cast<uint32_t*>(sSA)[idx] = rsa[i];
      reinterpret_cast<uint32_t*>(sSB)[idx] = rsb[i];
    }
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

  const int fr = lane & 31, fk = lane >> 5;  // fragment row, K half
  for (int64_t k0 = kb; k0 < ke; k0 += BKE) {
    gload(k0);
    __syncthreads();  // previous compute done with LDS
    lstore();
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKE / 64; ++kk) {
      uint4 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fa[i] = *reinterpret_cast<const uint4*>(sA + (wm * 64 + i * 32 + fr) * LDS_ROW + kk * 32 + fk * 16);
        fb[i] = *reinterpret_cast<const uint4*>(sB + (wn * 64 + i * 32 + fr) * LDS_ROW + kk * 32 + fk * 16);
      }
      if (FMT == AVERIS_MXFP4) {
        int sa[2], sb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          sa[i] = sSA[(wm * 64 + i * 32 + fr) * SB + kk * 2 + fk];
          sb[i] = sSB[(wn * 64 + i * 32 + fr) * SB + kk * 2 + fk];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const v8i av = {(int)fa[i].x, (int)fa[i].y, (int)fa[i].z, (int)fa[i].w, 0, 0, 0, 0};
            const v8i bv = {(int)fb[j].x, (int)fb[j].y, (int)fb[j].z, (int)fb[j].w, 0, 0, 0, 0};
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[i][j], 4, 4, 0, sa[i], 0, sb[j]);
          }
      } else {
        v8bf da[2][4], db[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const uint8_t* pa = sSA + (wm * 64 + i * 32 + fr) * SB + kk * 4 + fk * 2;
          const uint8_t* pb = sSB + (wn * 64 + i * 32 + fr) * SB + kk * 4 + fk * 2;
          dequant32_bf16(fa[i], e4m3_value(pa[0]), e4m3_value(pa[1]), da[i]);
          dequant32_bf16(fb[i], e4m3_value(pb[0]), e4m3_value(pb[1]), db[i]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[i][q], db[j][q], acc[i][j], 0, 0, 0);
      }
    }
  }

  // ---- epilogue ----
  float alpha = 1.0f;
  if (FMT == AVERIS_NVFP4) alpha = __fmul_rn(g.a_ts[0], g.b_ts[0]);
  const bool partial = g.splits > 1;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + fr;
      if (col >= g.N) continue;
      const float bcol = (!partial && g.bias) ? g.bias[col] : 0.0f;
      const float vcol = (!partial && g.r1u) ? g.r1v[col] : 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * 64 + i * 32 + (e >> 2) * 8 + fk * 4 + (e & 3);
        if (row >= g.M) continue;
        float out = __fmul_rn(acc[i][j][e], alpha);
        if (partial) {
          reinterpret_cast<float*>(g.c)[(int64_t)split * g.M * g.N + row * g.N + col] = out;
          continue;
        }
        if (g.bias) out = __fadd_rn(out, bcol);
        if (g.r1u) out = __fadd_rn(out, __fmul_rn(__fmul_rn(g.r1, g.r1u[row]), vcol));
        if (g.c_bf16) {
          reinterpret_cast<uint16_t*>(g.c)[row * g.ldc + col] = (uint16_t)f32_to_bf16_rne(out);
        } else {
          float* p = reinterpret_cast<float*>(g.c) + row * g.ldc + col;
          *p = g.accumulate ? __fadd_rn(*p, out) : out;
        }
      }
    }
}

// Split-K reduce: C = (accumulate ? C : 0) + sum_s P[s] (fixed order) + r1 * u[row] * v[col].
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part, int splits, int64_t M, int64_t N,
                                                       float* __restrict__ c, int64_t ldc, const float* __restrict__ u,
                                                       const float* __restrict__ v, float r1, int accumulate) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * N) return;
  const int64_t row = idx / N, col = idx % N;
  float s = part[idx];
  for (int p = 1; p < splits; ++p) s = __fadd_rn(s, part[(int64_t)p * M * N + idx]);
  if (u) s = __fadd_rn(s, __fmul_rn(__fmul_rn(r1, u[row]), v[col]));
  float* dst = c + row * ldc + col;
  *dst = accumulate ? __fadd_rn(*dst, s) : s;
}

// Dequantized value of element k of a packed row (fp64, exact).
template <int FMT>
__device__ inline double dq_elem(const uint8_t* codes, const uint8_t* scales, int64_t k) {
  const uint32_t byte = codes[k >> 1];
  const uint32_t c = (k & 1) ? (byte >> 4) : (byte & 15u);
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  double v = e == 0 ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  if (c & 8u) v = -v;
  if (FMT == AVERIS_MXFP4) return v * ldexp(1.0, (int)scales[k >> 5] - 127);
  return v * (double)e4m3_value(scales[k >> 4]);
}

// Mean-term GEMV: out[j] = alpha * sum_k DQ(mu)[k] DQ(B)[j][k], one wave per output, fp64
// accumulation with a fixed-order lane reduction.  alpha = s_mu * s_B (NVFP4) or 1.
template <int FMT>
__global__ __launch_bounds__(256) void k_gemv_mean(const uint8_t* __restrict__ mu_codes, const uint8_t* __restrict__ mu_scales,
                                                   const float* __restrict__ mu_ts, const uint8_t* __restrict__ b_codes,
                                                   const uint8_t* __restrict__ b_scales, int64_t ldb_b, int64_t lds_b,
                                                   const float* __restrict__ b_ts, int64_t N, int64_t K, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= N) return;
  const uint8_t* bc = b_codes + j * ldb_b;
  const uint8_t* bs = b_scales + j * lds_b;
  double s = 0.0;
  for (int64_t k = lane; k < K; k += 64) s += dq_elem<FMT>(mu_codes, mu_scales, k) * dq_elem<FMT>(bc, bs, k);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  if (lane == 0) {
    double alpha = 1.0;
    if (FMT == AVERIS_NVFP4) alpha = (double)mu_ts[0] * (double)b_ts[0];
    out[j] = (float)(s * alpha);
  }
}

// Dequantized mean vector for the rank-one dW term, rotation undone in fp64 if `rotated`.
template <int FMT>
__global__ __launch_bounds__(256) void k_mean_vec(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                  const float* __restrict__ ts, int64_t K, int rotated, float* __restrict__ out) {
  const int64_t blk = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 16-element chunk
  if (blk * 16 >= K) return;
  const double sd = FMT == AVERIS_NVFP4 ? (double)ts[0] : 1.0;
  double v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = dq_elem<FMT>(codes, scales, blk * 16 + j) * sd;
  if (rotated) {
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if ((j & h) == 0) { const double a = v[j], b = v[j + h]; v[j] = a + b; v[j + h] = a - b; }
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] *= 0.25;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (blk * 16 + j < K) out[blk * 16 + j] = (float)v[j];
}

// ------------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------------


static int g_count(int fmt) { return fmt == AVERIS_MXFP4 ? 32 : 16; }

int choose_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ceil_div(M, BM) * ceil_div(N, BN);
  int64_t s = 512 / (tiles > 0 ? tiles : 1);
  const int64_t ksteps = ceil_div(K, BKE);
  if (s > ksteps) s = ksteps;
  if (s > 8) s = 8;
  return s < 1 ? 1 : (int)s;
}

// workspace: [256 B][bias N][u M][v N] fp32, then split-K partials [splits][M][N] fp32
static size_t partials_offset(int64_t M, int64_t N) { return 256 + (size_t)round_up((N + M + N) * 4, 1024); }

size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, int splits) {
  size_t b = partials_offset(M, N);
  if (splits > 1) b += (size_t)splits * M * N * 4;
  return b;
}

hipError_t gemm_launch(const GemmPlan& p) {
  const averis_qtensor& A = *p.a;
  const averis_qtensor& B = *p.b;
  const int fmt = A.fmt;
  const int G = g_count(fmt);
  uint8_t* ws = reinterpret_cast<uint8_t*>(p.ws);
  float* bias = reinterpret_cast<float*>(ws + 256);
  float* u = bias + B.outer;
  float* v = u + A.outer;
  float* partials = reinterpret_cast<float*>(ws + partials_offset(A.outer, B.outer));

  GemmArgs g{};
  g.a_codes = A.codes; g.a_scales = A.scales; g.lda_b = A.k_pad / 2; g.lds_a = A.k_pad / G;
  g.b_codes = B.codes; g.b_scales = B.scales; g.ldb_b = B.k_pad / 2; g.lds_b = B.k_pad / G;
  g.a_ts = A.tensor_scale; g.b_ts = B.tensor_scale;
  g.M = A.outer; g.N = B.outer; g.K = A.k_pad;
  g.tiles_m = (int)ceil_div(g.M, BM); g.tiles_n = (int)ceil_div(g.N, BN);
  g.accumulate = p.accumulate;
  if (g.M == 0 || g.N == 0) return hipSuccess;

  if (p.mu) {
    const averis_qtensor& U = *p.mu;
    const unsigned blocks = (unsigned)ceil_div(g.N, 4);
    if (fmt == AVERIS_MXFP4)
      hipLaunchKernelGGL(k_gemv_mean<AVERIS_MXFP4>, dim3(blocks), dim3(256), 0, p.stream, U.codes, U.scales, U.tensor_scale,
                         B.codes, B.scales, g.ldb_b, g.lds_b, B.tensor_scale, g.N, B.k_pad, bias);
    else
      hipLaunchKernelGGL(k_gemv_mean<AVERIS_NVFP4>, dim3(blocks), dim3(256), 0, p.stream, U.codes, U.scales, U.tensor_scale,
                         B.codes, B.scales, g.ldb_b, g.lds_b, B.tensor_scale, g.N, B.k_pad, bias);
    g.bias = bias;
  }
  if (p.mu_u) {
    const averis_qtensor* vs[2] = {p.mu_u, p.mu_v};
    float* outs[2] = {u, v};
    for (int t = 0; t < 2; ++t) {
      const averis_qtensor& Q = *vs[t];
      const unsigned blocks = (unsigned)ceil_div(ceil_div(Q.k, 16), 256);
      const int rot = (Q.flags & AVERIS_HADAMARD16) ? 1 : 0;
      if (fmt == AVERIS_MXFP4)
        hipLaunchKernelGGL(k_mean_vec<AVERIS_MXFP4>, dim3(blocks), dim3(256), 0, p.stream, Q.codes, Q.scales, Q.tensor_scale, Q.k, rot, outs[t]);
      else
        hipLaunchKernelGGL(k_mean_vec<AVERIS_NVFP4>, dim3(blocks), dim3(256), 0, p.stream, Q.codes, Q.scales, Q.tensor_scale, Q.k, rot, outs[t]);
    }
    g.r1u = u; g.r1v = v; g.r1 = p.r1;
  }
  g.splits = p.splits;
  const int64_t ksteps = ceil_div(g.K, BKE);
  g.k_chunk = ceil_div(ksteps, p.splits) * BKE;
  if (p.splits > 1) {
    g.c = partials; g.ldc = g.N; g.c_bf16 = 0;
  } else {
    g.c = p.c; g.ldc = p.ldc; g.c_bf16 = p.c_bf16;
  }
  const unsigned grid = (unsigned)(g.tiles_m * g.tiles_n * p.splits);
  if (fmt == AVERIS_MXFP4) hipLaunchKernelGGL(k_gemm<AVERIS_MXFP4>, dim3(grid), dim3(kGemmThreads), 0, p.stream, g);
  else hipLaunchKernelGGL(k_gemm<AVERIS_NVFP4>, dim3(grid), dim3(kGemmThreads), 0, p.stream, g);
  if (p.splits > 1) {
    const int64_t n = g.M * g.N;
    hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, p.stream, partials, p.splits, g.M,
                       g.N, reinterpret_cast<float*>(p.c), p.ldc, g.r1u, g.r1v, g.r1, p.accumulate);
  }
  return hipGetLastError();
}

}  // namespace av

// Quantized GEMMs of the Averis linear layer for gfx950.
//
// "均值偏置的诅咒与祝福：FP4量化大语言模型训练" explainer (paper.rainbus.top), section 方法步骤详情:
//   Y = 1 (mu_X W) + X_R W,  dL/dX = 1 (mu_D W^T) + D_R W^T,  dL/dW = X_R^T D_R + l mu_X^T mu_D
// with every operand FP4-quantized; the mean term of Y and dX is a broadcast row, and in dW it
// is a rank-one outer product (the cross terms vanish for zero-mean residuals).
//
// One tile loop C[M, N] = A[M, K] B[N, K]^T over K-inner packed E2M1 operands:
//   MXFP4: v_mfma_scale_f32_32x32x64_f8f6f4 consumes the codes and the E8M0 block scales
//          directly; a lane holds one row and 32 K elements (= one MX block) per instruction.
//   NVFP4: E4M3 scales are not powers of two, which the scaled MFMA cannot apply (it uses only
//          a scale's exponent), so each lane dequantizes its 32 codes exactly to f16 (code x
//          E4M3 value has <= 6 significant bits; one conversion and one packed multiply per two
//          codes) and issues four v_mfma_f32_32x32x16_f16; the fp32 tensor scales multiply the
//          accumulator in the epilogue.
// K order inside a K-step is permuted (the same way for A and B, so products pair up): lane
// half h takes the step's 32-element chunks h*S .. h*S+S-1 for its S MFMAs, which makes its
// block scales for the whole step one contiguous LDS load.
// Pipeline: operands go straight from global memory to LDS (gfx950 global_load_lds) into a
// ring of stages; while K-step i is multiplied, steps i+1 .. i+STAGES-1 are in flight.  One
// barrier per K-step, no fence: each wave waits on its own vmcnt, then all meet at s_barrier.
// MXFP4 dense launches use a warp-specialized form (k_gemm_ws): loader waves keep a 4-stage ring
// filled across tile boundaries while the multiplying waves only multiply and store.
// Epilogue: out = alpha * acc + bias[col] + r1 * u[row] * v[col] (+ C when accumulating),
// alpha = product of the operands' tensor decode scales (NVFP4) or 1.
#include <algorithm>
#include <cmath>
#include <utility>
#include <vector>

#include "launch.h"

namespace av {

// A quantized mean read in place: element k of row `row` of a [rows, k_pad] FP4 operand (codes,
// tiled scales, NVFP4 per-row tensor scales), quantized after the 16x16 rotation when rot != 0.
struct MeanVec { const uint8_t* codes; const uint8_t* scales; const float* ts; int64_t k_pad; int rot; };

struct GemmArgs {
  const uint8_t* a_codes; const uint8_t* a_scales; int64_t lda_b;  // codes row stride (bytes); scales tiled
  const uint8_t* b_codes; const uint8_t* b_scales; int64_t ldb_b;
  const float* a_ts; const float* b_ts;  // tensor decode scales (NVFP4) or nullptr
  int64_t M, N, K;                      // K = padded length (multiple of 128)
  void* c; int64_t ldc; int c_bf16;     // output (or split-K partials base when splits > 1)
  const float* bias;                    // [N] or nullptr
  // broadcast mean term computed inside the tile loop (kernels with MU): row mu_row of the
  // quantized mean [rows, K] (codes, tiled scales, NVFP4 tensor scales) times B
  const uint8_t* mu_codes; const uint8_t* mu_scales; const float* mu_ts; int64_t mu_row;
  // rank-one term r1 * u[row] * v[col] (has_r1): u, v = dequantized means ru, rv (row r1_row)
  MeanVec ru, rv; int has_r1; float r1; int64_t r1_row;
  int accumulate;
  int splits; int64_t k_chunk;          // K range per split (multiple of the K-step), partials at c + s * M * N
  int tiles_m, tiles_n;
  int group_m;                          // tile rows per group in the tile order (L2 locality)
  // Grouped (MoE) launches: group e covers rows [offsets[e], offsets[e+1]) of the token axis.
  //   grouped == 1 (forward / input gradient): A = grouped row layout (group e starts at row
  //     p32[e]), B = E stacked [N, K] operands, C rows offsets[e] + r, bias [E][N], M = l_e.
  //   grouped == 2 (weight gradient): A, B = per-group column layouts ([M, K_e] and [N, K_e],
  //     K_e = round_up(l_e, 256), at token offset p256[e]), C = [E][M][ldc], rank-one factor
  //     l_e with u [E][M] and v [E][N].  Every group has tiles_m x tiles_n tiles.
  const int64_t* offsets; int E; int grouped;
  int n_work;                           // logical tiles of the launch (a workgroup may take several)
  // STATS kernels: per-column sums of the stored output over each wave's rows, [part][N] with
  // part = row / (32 TM)
  float* st_sum;
};

__device__ inline uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ inline float2 fp4x2_to_f32(uint32_t w, int sel) {
  // exact decode of the two codes in byte `sel` (low nibble first), unit scale
  switch (sel) {
    case 0: { auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); return make_float2(r[0], r[1]); }
    case 1: { auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); return make_float2(r[0], r[1]); }
    case 2: { auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); return make_float2(r[0], r[1]); }
    default: { auto r = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); return make_float2(r[0], r[1]); }
  }
}

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// The gfx950 conversions below apply only the power-of-two part of their scale operand, so they
// run with scale 1.0 and stay exact: E2M1 codes and E4M3 scales are all f16 values.
__device__ inline v2h fp4x2_to_f16(uint32_t w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  }
}
// The two E4M3 scale bytes in the low (hi = 0) or high 16 bits of w, as f16.
__device__ inline v2h e4m3x2_to_f16(uint32_t w, int hi) {
  return hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
            : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}

// 32 E2M1 codes (16 bytes) times two block scales (elements 0-15: sc.x, 16-31: sc.y) -> 4 x 8
// f16.  A code has at most 2 significant bits and an E4M3 value at most 4, so each product (one
// packed f16 multiply per two codes) is exact: magnitudes lie in [2^-10, 2688], all normal f16.
__device__ inline void dequant32_f16(const uint4& c, v2h sc, v8h* out) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const v2h s = q < 2 ? v2h{sc.x, sc.x} : v2h{sc.y, sc.y};
    v2h h[4];
#pragma unroll
    for (int bsel = 0; bsel < 4; ++bsel) h[bsel] = fp4x2_to_f16(w[q], bsel) * s;
    out[q] = v8h{h[0].x, h[0].y, h[1].x, h[1].y, h[2].x, h[2].y, h[3].x, h[3].y};
  }
}

// Dequantized element k of row `row` of a quantized mean operand with padded length k_pad
// (fp32; exact for codes times an E8M0 scale, one rounding for NVFP4's decode scale).
template <int FMT>
__device__ inline float dq_one(const uint8_t* codes, const uint8_t* scales, const float* ts, int64_t row, int64_t k,
                               int64_t k_pad) {
  constexpr int G = FMT == AVERIS_MXFP4 ? 32 : 16;
  const uint32_t byte = codes[row * (k_pad / 2) + (k >> 1)];
  const uint32_t c = (k & 1) ? (byte >> 4) : (byte & 15u);
  const float v = fp4x2_to_f32(c, 0).x;
  const uint32_t s = scales[scale_offset(row, k / G, k_pad, G)];
  if (FMT == AVERIS_MXFP4) return ldexpf(v, (int)s - 127);
  return __fmul_rn(__fmul_rn(v, e4m3_value(s)), ts[row]);
}

// Element k of a dequantized mean vector, the rotation undone when the mean was quantized
// rotated: 0.25 * sum_j H16[p][j] DQ(q[16 b + j]), k = 16 b + p, H16[p][j] = (-1)^popcount(p & j)
// (Sylvester order).  The 16 terms are fp32 values within a factor 12 of each other, so their
// fp64 sum is exact in any order and the result is one rounding of the exact value.
template <int FMT>
__device__ inline float mean_value(const MeanVec& mv, int64_t row, int64_t k) {
  if (!mv.rot) return dq_one<FMT>(mv.codes, mv.scales, mv.ts, row, k, mv.k_pad);
  constexpr int G = FMT == AVERIS_MXFP4 ? 32 : 16;
  const int64_t b = k >> 4;
  const int p = (int)(k & 15);
  // the block's 16 codes (8 bytes) and the one scale they share, each one load
  const uint2 cw = *reinterpret_cast<const uint2*>(mv.codes + row * (mv.k_pad / 2) + b * 8);
  const uint32_t sc = mv.scales[scale_offset(row, b * 16 / G, mv.k_pad, G)];
  const float ts = FMT == AVERIS_NVFP4 ? mv.ts[row] : 1.0f;
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t c = ((j < 8 ? cw.x : cw.y) >> (4 * (j & 7))) & 15u;
    const float e = fp4x2_to_f32(c, 0).x;  // the same per-element decode as dq_one
    const float v = FMT == AVERIS_MXFP4 ? ldexpf(e, (int)sc - 127) : __fmul_rn(__fmul_rn(e, e4m3_value(sc)), ts);
    s += (__popc(p & j) & 1) ? -(double)v : (double)v;
  }
  return (float)(s * 0.25);
}

// Tile order: consecutive logical tiles walk down a group of `gm` tile rows, then move one
// tile column right.  With the XCD remap each XCD owns a contiguous run of logical tiles, so
// it works on a compact (group rows x run / group columns) block and re-reads little of A or B
// from beyond its L2.
__device__ __forceinline__ void tile_coords(int t, int tiles_m, int tiles_n, int gm, int& tm, int& tn) {
  const int per_group = gm * tiles_n;
  const int group = t / per_group, first_m = group * gm;
  const int rows = tiles_m - first_m < gm ? tiles_m - first_m : gm;
  const int r = t % per_group;
  tm = first_m + r % rows;
  tn = r / rows;
}

// LDS row swizzle (16-byte slot index within a 128-byte row): conflict-free fragment reads of
// 32 consecutive rows for 32- and 64-bank LDS.  Depends only on the row's low 4 bits.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

template <int FMT, int WM, int WN, int TM, int TN, int STAGES, int AUX = 0>
struct GemmCfg {
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int BM = WM * TM * 32, BN = WN * TN * 32;
  static constexpr int BKB = 128, BKE = 256;     // bytes / elements per row per K-step
  static constexpr int G = FMT == AVERIS_MXFP4 ? 32 : 16;
  static constexpr int SB = BKE / G;             // scale bytes per row per K-step (8 or 16)
  static constexpr int PIECE = 32 * SB;          // tiled scale bytes of one 32-row group per K-step
  static constexpr int NKK = BKE / 64;           // MFMA K-substeps per K-step
  static constexpr int A_OFF = 0, B_OFF = BM * BKB, SA_OFF = (BM + BN) * BKB, SB_OFF = SA_OFF + BM * SB;
  static constexpr int DUMMY_OFF = SB_OFF + BN * SB;            // sink for padding scale loads
  static constexpr int STAGE = DUMMY_OFF + 256;
  static constexpr int IA = BM / 8, IB = BN / 8;                // 1 KB code loads per step
  static constexpr int ISA = BM * SB / 256, ISB = BN * SB / 256;  // 256-byte scale loads per step
  // scale loads are padded to a multiple of the wave count (extra ones load zeros into the
  // sink) so that every wave issues the same number of loads per step
  static constexpr int ISA_P = (ISA + NW - 1) / NW * NW, ISB_P = (ISB + NW - 1) / NW * NW;
  static_assert(IA % NW == 0 && IB % NW == 0, "code loads must split evenly over waves");
  static constexpr int NLA = IA / NW, NLB = IB / NW, NLSA = ISA_P / NW, NLSB = ISB_P / NW;
  static constexpr int LPS = NLA + NLB + NLSA + NLSB;          // load instructions per wave per step
  static_assert(LPS * (STAGES - 2) < 64, "vmcnt range");
};

// The mean term (MU): longest K whose quantized mean row fits the tile's LDS copy.
constexpr int kMuMaxK = 8192;
constexpr int kMuCodes = kMuMaxK / 2, kMuBytes = kMuCodes + 1024;  // codes, then 4 x 256 scale bytes

template <int FMT, int WM, int WN, int TM, int TN, int STAGES, int AUX = 0, bool MU = false>
struct GemmTile {
  using C = GemmCfg<FMT, WM, WN, TM, TN, STAGES, AUX>;
  static_assert(!MU || TN == WM, "the mean term splits a wave's column blocks over the wave rows");
  __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
  int va[C::NLA], vb[C::NLB], vsa[C::NLSA], vsb[C::NLSB];  // per-lane byte offsets (loop invariant)
  int ldsa[C::NLSA], ldsb[C::NLSB];                          // LDS destinations of the scale loads
  int frag_off[C::NKK];   // lane's LDS byte offset of its fragment chunk for each substep
  int scale_off;          // lane's LDS byte offset of its scale bytes within a fragment row block
  int wave, wm, wn;
  int mu_off, mu_soff;    // lane half's byte offsets within a K-step of the mean's codes / scales
  v16f acc[TM][TN];
  v16f acc_mu;            // MU: 32 x 32 block (every row the mean) x this wave's column block wm

  // Operand views of tile (m0, n0); the accumulators are left alone (clear() resets them).
  // as_wave >= 0: the views of wave as_wave's share of the loads (a loader wave issuing them).
  __device__ __forceinline__ void bind(const GemmArgs& g, int64_t m0, int64_t n0, int as_wave = -1) {
    const int lane = threadIdx.x & 63;
    // wave-uniform, and known to be: the epilogue's buffer resources then stay scalar
    wave = as_wave >= 0 ? as_wave : __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    wm = wave / WN; wn = wave % WN;
    const int fr = lane & 31, fk = lane >> 5;
    // operands restricted to this tile's rows: offsets past the last row read as zero
    const int64_t rows_a = g.M - m0 < C::BM ? g.M - m0 : C::BM, rows_b = g.N - n0 < C::BN ? g.N - n0 : C::BN;
    ra = make_rsrc(g.a_codes + m0 * g.lda_b, rows_a * g.lda_b);
    rb = make_rsrc(g.b_codes + n0 * g.ldb_b, rows_b * g.ldb_b);
    // tiled scales: this tile's 32-row groups start at group m0 / 32; a group spans K / 256 pieces
    const int64_t gstride = (g.K / C::BKE) * C::PIECE;
    rsa = make_rsrc(g.a_scales + (m0 / 32) * gstride, ceil_div(rows_a, 32) * gstride);
    rsb = make_rsrc(g.b_scales + (n0 / 32) * gstride, ceil_div(rows_b, 32) * gstride);
    const int lr = lane >> 3, sl = lane & 7;
#pragma unroll
    for (int i = 0; i < C::NLA; ++i) {
      const int t = i * C::NW + wave, r = t * 8 + lr;
      va[i] = (int)(r * g.lda_b) + ((sl ^ swz(r)) << 4);
    }
#pragma unroll
    for (int i = 0; i < C::NLB; ++i) {
      const int t = i * C::NW + wave, r = t * 8 + lr;
      vb[i] = (int)(r * g.ldb_b) + ((sl ^ swz(r)) << 4);
    }
    // scale load t (256 bytes) covers piece t * 256 / PIECE of the step, part t % (PIECE / 256)
    constexpr int PP = C::PIECE / 256;
#pragma unroll
    for (int i = 0; i < C::NLSA; ++i) {
      const int t = i * C::NW + wave;
      vsa[i] = t < C::ISA ? (int)((t / PP) * gstride) + (t % PP) * 256 + lane * 4 : 0x7FFFFFF0;
      ldsa[i] = t < C::ISA ? C::SA_OFF + t * 256 : C::DUMMY_OFF;
    }
#pragma unroll
    for (int i = 0; i < C::NLSB; ++i) {
      const int t = i * C::NW + wave;
      vsb[i] = t < C::ISB ? (int)((t / PP) * gstride) + (t % PP) * 256 + lane * 4 : 0x7FFFFFF0;
      ldsb[i] = t < C::ISB ? C::SB_OFF + t * 256 : C::DUMMY_OFF;
    }
    const int sw = swz(fr);
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) frag_off[kk] = fr * C::BKB + (((fk * C::NKK + kk) ^ sw) << 4);
    scale_off = fr * C::SB + fk * (C::SB / 2);
    mu_off = fk * C::NKK * 16;
    mu_soff = fk * (C::SB / 2);
  }
  __device__ __forceinline__ void clear() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = v16f{};
    acc_mu = v16f{};
  }

  // MU: DMA of the mean row (codes, then per K-step scale bytes) into smu.  Issued before the
  // prologue, so the first pipeline wait covers it (vector memory ops complete in order).
  __device__ __forceinline__ void issue_mean(const GemmArgs& g, uint8_t* smu) const {
    const int lane = threadIdx.x & 63, i = wave * 64 + lane;
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(g.mu_codes + g.mu_row * (g.K / 2), g.K / 2);
    dma16<AUX>(rc, smu + wave * 1024, i * 16, 0);
    const int64_t pieces = g.K / C::BKE;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(g.mu_scales + (g.mu_row >> 5) * pieces * C::PIECE, pieces * C::PIECE);
    constexpr int LPP = C::SB / 4;  // lanes per K-step piece (4 bytes each)
    const int voff = (i / LPP) * C::PIECE + (int)(g.mu_row & 31) * C::SB + (i % LPP) * 4;
    dma4<AUX>(rs, smu + kMuCodes + wave * 256, voff, 0);
  }

  // This wave's share of the loads of the K-step starting at byte `kbyte` into stage s.
  __device__ __forceinline__ void issue(int kbyte, int sbyte, uint8_t* s) const {
#pragma unroll
    for (int i = 0; i < C::NLA; ++i) dma16<AUX>(ra, s + C::A_OFF + (i * C::NW + wave) * 1024, va[i], kbyte);
#pragma unroll
    for (int i = 0; i < C::NLB; ++i) dma16<AUX>(rb, s + C::B_OFF + (i * C::NW + wave) * 1024, vb[i], kbyte);
#pragma unroll
    for (int i = 0; i < C::NLSA; ++i) dma4<AUX>(rsa, s + ldsa[i], vsa[i], sbyte);
#pragma unroll
    for (int i = 0; i < C::NLSB; ++i) dma4<AUX>(rsb, s + ldsb[i], vsb[i], sbyte);
  }

  // One K-step from stage s; with MU also the mean's K-step `kstep` from smu.
  // MSO: byte offset of the mean's scale bytes from its codes in smu
  template <int MSO = kMuCodes>
  __device__ __forceinline__ void compute(const uint8_t* s, const uint8_t* smu, int kstep) {
    constexpr int LSB = C::SB / 2;  // scale bytes per lane half per K-step (4 or 8)
    uint32_t msc[LSB / 4];          // MU: the mean's scale bytes of this lane half's chunks
    if constexpr (MU) {
#pragma unroll
      for (int w = 0; w < LSB / 4; ++w)
        msc[w] = *reinterpret_cast<const uint32_t*>(smu + MSO + kstep * C::SB + mu_soff + 4 * w);
    }
    uint32_t sa[TM][LSB / 4], sb[TN][LSB / 4];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int w = 0; w < LSB / 4; ++w)
        sa[i][w] = *reinterpret_cast<const uint32_t*>(s + C::SA_OFF + (wm * TM * 32 + i * 32) * C::SB + scale_off + 4 * w);
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int w = 0; w < LSB / 4; ++w)
        sb[j][w] = *reinterpret_cast<const uint32_t*>(s + C::SB_OFF + (wn * TN * 32 + j * 32) * C::SB + scale_off + 4 * w);
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
      uint4 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = *reinterpret_cast<const uint4*>(s + C::A_OFF + (wm * TM * 32 + i * 32) * C::BKB + frag_off[kk]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[j] = *reinterpret_cast<const uint4*>(s + C::B_OFF + (wn * TN * 32 + j * 32) * C::BKB + frag_off[kk]);
      if (FMT == AVERIS_MXFP4) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const v8i av = {(int)fa[i].x, (int)fa[i].y, (int)fa[i].z, (int)fa[i].w, 0, 0, 0, 0};
            const v8i bv = {(int)fb[j].x, (int)fb[j].y, (int)fb[j].z, (int)fb[j].w, 0, 0, 0, 0};
            // B rows feed the MFMA's first operand, so a lane ends up holding four consecutive
            // output columns of one output row
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bv, av, acc[i][j], 4, 4, 0, (int)__builtin_amdgcn_ubfe(sb[j][0], 8 * kk, 8), 0,
                (int)__builtin_amdgcn_ubfe(sa[i][0], 8 * kk, 8));
          }
        if constexpr (MU) {
          // every row of the A block is the mean (one broadcast LDS read per lane half);
          // column block wm of this wave's columns
          const uint4 fm = *reinterpret_cast<const uint4*>(smu + kstep * C::BKB + mu_off + kk * 16);
          const uint4 fbm = wm ? fb[TN - 1] : fb[0];
          const uint32_t sbm = wm ? sb[TN - 1][0] : sb[0][0];
          const v8i mv = {(int)fm.x, (int)fm.y, (int)fm.z, (int)fm.w, 0, 0, 0, 0};
          const v8i bv = {(int)fbm.x, (int)fbm.y, (int)fbm.z, (int)fbm.w, 0, 0, 0, 0};
          acc_mu = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              bv, mv, acc_mu, 4, 4, 0, (int)__builtin_amdgcn_ubfe(sbm, 8 * kk, 8), 0,
              (int)__builtin_amdgcn_ubfe(msc[0], 8 * kk, 8));
        }
      } else {
        v8h da[TM][4], db[TN][4];
        const int wsel = kk / 2, hi = kk % 2;  // two scale bytes per chunk
#pragma unroll
        for (int i = 0; i < TM; ++i) dequant32_f16(fa[i], e4m3x2_to_f16(sa[i][wsel], hi), da[i]);
#pragma unroll
        for (int j = 0; j < TN; ++j) dequant32_f16(fb[j], e4m3x2_to_f16(sb[j][wsel], hi), db[j]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(db[j][q], da[i][q], acc[i][j], 0, 0, 0);
        if constexpr (MU) {
          const uint4 fm = *reinterpret_cast<const uint4*>(smu + kstep * C::BKB + mu_off + kk * 16);
          v8h dm[4];
          dequant32_f16(fm, e4m3x2_to_f16(msc[wsel], hi), dm);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            acc_mu = __builtin_amdgcn_mfma_f32_32x32x16_f16(wm ? db[TN - 1][q] : db[0][q], dm[q], acc_mu, 0, 0, 0);
        }
      }
    }
  }
  // MXFP4 K-step with every fragment of the step read from LDS before the first MFMA: a wave that
  // is alone on its SIMD (the warp-specialized kernel) then waits for LDS once per step instead of
  // once per 64-element substep.
  // MSO: byte offset of the mean's scale bytes from its codes in smu
  template <int MSO = kMuCodes>
  __device__ __forceinline__ void compute_mx_preload(const uint8_t* s, const uint8_t* smu, int kstep) {
    static_assert(FMT == AVERIS_MXFP4, "MXFP4 only");
    uint32_t msc = 0;
    if constexpr (MU) msc = *reinterpret_cast<const uint32_t*>(smu + MSO + kstep * C::SB + mu_soff);
    uint32_t sa[TM], sb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      sa[i] = *reinterpret_cast<const uint32_t*>(s + C::SA_OFF + (wm * TM * 32 + i * 32) * C::SB + scale_off);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      sb[j] = *reinterpret_cast<const uint32_t*>(s + C::SB_OFF + (wn * TN * 32 + j * 32) * C::SB + scale_off);
    uint4 fa[C::NKK][TM], fb[C::NKK][TN], fm[C::NKK];
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[kk][i] = *reinterpret_cast<const uint4*>(s + C::A_OFF + (wm * TM * 32 + i * 32) * C::BKB + frag_off[kk]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[kk][j] = *reinterpret_cast<const uint4*>(s + C::B_OFF + (wn * TN * 32 + j * 32) * C::BKB + frag_off[kk]);
      if constexpr (MU) fm[kk] = *reinterpret_cast<const uint4*>(smu + kstep * C::BKB + mu_off + kk * 16);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep every read ahead of the MFMAs (the scheduler would sink them)
#pragma unroll
    for (int kk = 0; kk < C::NKK; ++kk) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const v8i av = {(int)fa[kk][i].x, (int)fa[kk][i].y, (int)fa[kk][i].z, (int)fa[kk][i].w, 0, 0, 0, 0};
          const v8i bv = {(int)fb[kk][j].x, (int)fb[kk][j].y, (int)fb[kk][j].z, (int)fb[kk][j].w, 0, 0, 0, 0};
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              bv, av, acc[i][j], 4, 4, 0, (int)__builtin_amdgcn_ubfe(sb[j], 8 * kk, 8), 0,
              (int)__builtin_amdgcn_ubfe(sa[i], 8 * kk, 8));
        }
      if constexpr (MU) {
        const uint4 fbm = wm ? fb[kk][TN - 1] : fb[kk][0];
        const uint32_t sbm = wm ? sb[TN - 1] : sb[0];
        const v8i mv = {(int)fm[kk].x, (int)fm[kk].y, (int)fm[kk].z, (int)fm[kk].w, 0, 0, 0, 0};
        const v8i bv = {(int)fbm.x, (int)fbm.y, (int)fbm.z, (int)fbm.w, 0, 0, 0, 0};
        acc_mu = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            bv, mv, acc_mu, 4, 4, 0, (int)__builtin_amdgcn_ubfe(sbm, 8 * kk, 8), 0,
            (int)__builtin_amdgcn_ubfe(msc, 8 * kk, 8));
      }
    }
  }
};

// One pipeline step: wait until K-step `step` has landed (STAGES - 2 younger steps may stay in
// flight), meet at the barrier (all waves are then done with the stage refilled next), refill
// that stage with K-step step + STAGES - 1, multiply.  Every step issues the same loads (steps
// past the end re-load step 0's bytes into a stage nobody reads) so the vmcnt arithmetic is exact.
template <class T, int STAGES>
__device__ __forceinline__ void pipe_step(T& t, int step, int nsteps, int kb_byte, int kb_sbyte, uint8_t* cur,
                                          uint8_t* nxt, const uint8_t* smu, int k0) {
  using C = typename T::C;
  wait_vm<C::LPS * (STAGES - 2)>();
  __builtin_amdgcn_s_barrier();
  const int ns = step + STAGES - 1;
  const bool live = ns < nsteps;
  t.issue(live ? kb_byte + ns * C::BKB : 0, live ? kb_sbyte + ns * C::PIECE : 0, nxt);
  if (step < nsteps) t.compute(cur, smu, k0 + step);
}

__device__ __forceinline__ void lgkm_wait0() { __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14)); }

// Epilogue of one wave, straight from the accumulators: acc[i][j][4q + r] holds
// C[row i*32 + lane%32][col j*32 + 8q + 4h + r], h = lane / 32.
//   fp32 output (and split-K partials): a lane's 4 consecutive columns are 16 bytes; a transpose
//   within lane quads makes each store whole 128-byte row segments, written non-temporally.
//   bf16 output: v_permlane32_swap exchanges quad q+1 of the low half with quad q of the high
//   half, after which lane (fr, h) holds the 8 consecutive columns j*32 + 16p + 8h of its row
//   (p = q / 2), 16 bytes of bf16; with two column blocks (TN = 2) a transpose within lane quads
//   makes each store whole 128-byte row segments, written non-temporally.
// Per-column terms (bias, v) and per-row terms (u) are loaded once per tile, in one batch,
// before the first store; u (times r1) and v come from the tile's LDS copy (su: this wave's rows,
// sv: its columns).
//   out = alpha * acc (+ bias[col]) (+ r1 * u[row] * v[col]) (+ C when accumulating), each step
//   rounded once in fp32; split-K partials get alpha * acc only.
// ALL = false: the launch has no bias vector, rank-one term or accumulation (the epilogue then
// issues no global loads).
// Value of lane t ^ M within each 16-lane row (DPP moves: quad permutations for M = 1, 2; row
// half-mirror then quad reversal for 4; row rotation by 8 for 8).
template <int M>
__device__ __forceinline__ float row_xor(float v) {
  const int x = __float_as_int(v);
  if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
  else if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
  else if constexpr (M == 4)
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false), 0x1B, 0xF, 0xF, false));
  else return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false));
}

template <int W, class OP>
__device__ __forceinline__ void rs_step(float (&v)[16], bool upper, OP op) {
#pragma unroll
  for (int k = 0; k < W; ++k) {
    float a = v[k], b = v[k + W];
    asm("" : "+v"(a), "+v"(b));  // keep the lane choice a register select, not an indexed load
    const float keep = upper ? b : a, send = upper ? a : b;
    v[k] = op(keep, row_xor<W>(send));
  }
}

// Reduce-scatter of 16 per-lane values over the 32 lanes of each lane half, in a fixed order:
// afterwards lane t of the half holds OP over the half's 32 lanes of value t % 16 (15 DPP
// exchanges within 16-lane rows and one row swap, instead of the 80 exchanges of a butterfly
// on every value).  Both lanes of a pair combine in the same order.
template <class OP>
__device__ __forceinline__ float half_reduce_scatter16(float (&v)[16], int lane, OP op) {
  rs_step<8>(v, (lane & 8) != 0, op);
  rs_step<4>(v, (lane & 4) != 0, op);
  rs_step<2>(v, (lane & 2) != 0, op);
  rs_step<1>(v, (lane & 1) != 0, op);
  // rows 2r and 2r + 1 (lanes t and t ^ 16): both get op(row 2r, row 2r + 1)
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[0]), __float_as_uint(v[0]), false, false);
  return op(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// 4 x 4 transpose of 16-byte chunks within each quad of lanes: chunk s of lane 4 q + k moves to
// chunk k of lane 4 q + s.  Two exchange rounds (lane bit 0 with chunk bit 0, then bit 1 with
// bit 1); in each a lane keeps two chunks and swaps the other two with its partner through DPP
// quad permutations.
__device__ __forceinline__ void quad_transpose(v4u (&c)[4], int lane) {
  const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
#pragma unroll
  for (int m = 0; m < 4; m += 2)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t a = c[m][d], b = c[m + 1][d];
      asm("" : "+v"(a), "+v"(b));  // keep the lane choice a register select
      const uint32_t send = b0 ? a : b;
      const uint32_t recv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, 0xB1, 0xF, 0xF, false);  // lane ^ 1
      c[m][d] = b0 ? recv : a;
      c[m + 1][d] = b0 ? b : recv;
    }
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t a = c[m][d], b = c[m + 2][d];
      asm("" : "+v"(a), "+v"(b));
      const uint32_t send = b1 ? a : b;
      const uint32_t recv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, 0x4E, 0xF, 0xF, false);  // lane ^ 2
      c[m][d] = b1 ? recv : a;
      c[m + 2][d] = b1 ? b : recv;
    }
}

// STATS: column sums of the stored output over each wave's rows (fp32 partials [part][N],
// part = row / (32 TM)).
// 16-byte buffer store, non-temporal or with the default policy.
__device__ __forceinline__ void store16(v4u v, __amdgpu_buffer_rsrc_t r, int off, bool nt) {
  if (nt) __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kNonTemporal);
  else __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

// ST: 2 = whole-line stores, non-temporal for outputs (split-K partials, re-read at once by the
// reduction, with the default policy); 1 = whole-line stores, default policy; 0 = each lane's
// 16-byte pieces as they come.
// BIAS = false: the launch never has a bias vector (its registers are not kept).
template <int FMT, int TM, int TN, bool MU, bool ALL = true, bool STATS = false, int ST = 2, bool BIAS = true>
__device__ __forceinline__ void epilogue_regs(const GemmArgs& g, const v16f (&acc)[TM][TN], int64_t rbase,
                                              int64_t cbase, int split, int lane, const float* su, const float* sv,
                                              const float* sbias) {
  const int fr = lane & 31, h = lane >> 5;
  const bool bf = g.c_bf16 && g.splits == 1;
  const bool terms = g.splits == 1;
  // mean term: from the tile's MFMAs (MU; split-K partials carry their share) or a precomputed
  // bias vector (dense launches without MU)
  const bool hb = MU || (BIAS && ALL && terms && g.bias), hr = ALL && terms && g.has_r1;
  float alpha_mu = 1.0f;
  if (FMT == AVERIS_NVFP4 && MU) alpha_mu = __fmul_rn(g.mu_ts[g.mu_row], g.b_ts[0]);
  // this lane's columns: bf16 -> j*32 + 16p + 8h + (0..7); fp32 -> j*32 + 8q + 4h + (0..3)
  // VLAZY (256-row tiles): v is read from LDS where it is used instead of held in registers
  constexpr bool VLAZY = TM >= 4;
  float bias[TN][16], vv[TN][16], uu[TM];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const int off = bf ? j * 32 + 16 * (c4 >> 1) + 8 * h + 4 * (c4 & 1) : j * 32 + 8 * c4 + 4 * h;
      const int64_t col = cbase + off;
      const bool ok = col < g.N;
      float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
      if (MU) {
        b = *reinterpret_cast<const float4*>(sbias + off);
        if (FMT == AVERIS_NVFP4) {
          b.x = __fmul_rn(alpha_mu, b.x); b.y = __fmul_rn(alpha_mu, b.y);
          b.z = __fmul_rn(alpha_mu, b.z); b.w = __fmul_rn(alpha_mu, b.w);
        }
      } else if (hb && ok) {
        b = *reinterpret_cast<const float4*>(g.bias + col);
      }
      const float4 r = (hr && !VLAZY) ? *reinterpret_cast<const float4*>(sv + off) : make_float4(0.f, 0.f, 0.f, 0.f);
      bias[j][4 * c4] = b.x; bias[j][4 * c4 + 1] = b.y; bias[j][4 * c4 + 2] = b.z; bias[j][4 * c4 + 3] = b.w;
      vv[j][4 * c4] = r.x; vv[j][4 * c4 + 1] = r.y; vv[j][4 * c4 + 2] = r.z; vv[j][4 * c4 + 3] = r.w;
    }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t row = rbase + i * 32 + fr;
    uu[i] = (hr && row < g.M) ? su[i * 32 + fr] : 0.0f;
  }
  float alpha = 1.0f;
  if (FMT == AVERIS_NVFP4) alpha = __fmul_rn(g.a_ts[0], g.b_ts[0]);
  // Output stores (accumulation aside) go through a buffer over this wave's rows: rows past M
  // lie beyond its range and columns past N get an out-of-range offset, which the hardware
  // drops (no branches around the stores).
  const bool acc_in = ALL && g.splits == 1 && g.accumulate;
  const int esz = bf ? 2 : 4;
  const int64_t ldo = g.splits > 1 ? g.N : g.ldc;
  uint8_t* obase = g.splits > 1 ? reinterpret_cast<uint8_t*>(g.c) + (((int64_t)split * g.M + rbase) * g.N) * 4
                                : reinterpret_cast<uint8_t*>(g.c) + rbase * g.ldc * esz;
  const int64_t nrows = g.M - rbase < TM * 32 ? g.M - rbase : TM * 32;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(obase, nrows > 0 ? (nrows - 1) * ldo * esz + g.N * esz : 0);
  // STATS: column sums of the stored values over this wave's rows in fp32: each lane's TM rows
  // in order, then across the lanes of each half in the fixed reduce-scatter order, after which
  // lane t of a half holds value t % 16 of each column block.
  float csum[STATS ? TN : 1][16];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t row = rbase + i * 32 + fr;
    const bool row_ok = row < g.M;
    const int roff = (i * 32 + fr) * (int)(ldo * esz);
    v4u ob[4];  // bf16, TN == 2: this row's four 16-byte chunks (j, p) at 2 j + p
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      float x[16];
      if (bf) {
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i][j][8 * p + r]),
                                                             __float_as_uint(acc[i][j][8 * p + 4 + r]), false, false);
            x[8 * p + r] = __uint_as_float(sw[0]);
            x[8 * p + 4 + r] = __uint_as_float(sw[1]);
          }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = acc[i][j][e];
      }
      if (FMT == AVERIS_NVFP4) {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = __fmul_rn(x[e], alpha);
      }
      if (hb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[e] = __fadd_rn(x[e], bias[j][e]);
      }
      if (hr) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float ve = vv[j][e];
          if constexpr (VLAZY) {
            const int c4 = e >> 2;
            const int off = bf ? j * 32 + 16 * (c4 >> 1) + 8 * h + 4 * (c4 & 1) : j * 32 + 8 * c4 + 4 * h;
            ve = sv[off + (e & 3)];
          }
          x[e] = __fadd_rn(x[e], __fmul_rn(uu[i], ve));
        }
      }
      if (bf) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int64_t col = cbase + j * 32 + 16 * p + 8 * h;
          const v4u o = {pack_bf16x2(x[8 * p], x[8 * p + 1]), pack_bf16x2(x[8 * p + 2], x[8 * p + 3]),
                         pack_bf16x2(x[8 * p + 4], x[8 * p + 5]), pack_bf16x2(x[8 * p + 6], x[8 * p + 7])};
          if constexpr (TN == 2 && ST > 0) ob[2 * j + p] = o;  // stored below, after the quad transpose
          else __builtin_amdgcn_raw_buffer_store_b128(o, ro, col < g.N ? roff + (int)col * 2 : 0x7FFFFFF0, 0, 0);
          if constexpr (STATS) {  // the values as stored
#pragma unroll
            for (int r = 0; r < 8; ++r)
              x[8 * p + r] = __uint_as_float(r & 1 ? (o[r >> 1] & 0xFFFF0000u) : (o[r >> 1] << 16));
          }
        }
      } else if (!acc_in) {
        // fp32 (outputs and split-K partials): lane (fr, h) holds 4 chunks of 4 columns
        // j*32 + 8q + 4h of row fr; after the quad transpose store s writes row 4 (fr / 4) + s and
        // the eight lanes of a quad pair cover the block's 32 columns, one whole 128-byte line
        // (non-temporal, as for bf16)
        v4u of[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          of[q] = v4u{__float_as_uint(x[4 * q]), __float_as_uint(x[4 * q + 1]), __float_as_uint(x[4 * q + 2]),
                      __float_as_uint(x[4 * q + 3])};
        if constexpr (ST > 0) {
          quad_transpose(of, lane);
          const int64_t col = cbase + j * 32 + 8 * (fr & 3) + 4 * h;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int rs = (i * 32 + (fr & ~3) + s) * (int)(ldo * esz);
            store16(of[s], ro, col < g.N ? rs + (int)col * 4 : 0x7FFFFFF0, ST == 2 && g.splits == 1);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t col = cbase + j * 32 + 8 * q + 4 * h;
            store16(of[q], ro, col < g.N ? roff + (int)col * 4 : 0x7FFFFFF0, false);
          }
        }
      } else {  // accumulate into fp32 C (no STATS)
        if (!row_ok) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t col = cbase + j * 32 + 8 * q + 4 * h;
          if (col >= g.N) continue;
          float* dst = reinterpret_cast<float*>(g.c) + row * g.ldc + col;
          const float4 c = *reinterpret_cast<const float4*>(dst);
          *reinterpret_cast<float4*>(dst) = make_float4(__fadd_rn(c.x, x[4 * q]), __fadd_rn(c.y, x[4 * q + 1]),
                                                        __fadd_rn(c.z, x[4 * q + 2]), __fadd_rn(c.w, x[4 * q + 3]));
        }
      }
      if constexpr (STATS) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float v = row_ok ? x[e] : 0.0f;
          csum[j][e] = i == 0 ? v : __fadd_rn(csum[j][e], v);
        }
      }
    }
    if constexpr (TN == 2 && ST > 0) {
      // bf16 with two column blocks: lane (fr, h) holds 64 bytes of row fr in four chunks; after
      // the transpose within its lane quad, store s writes row 4 (fr / 4) + s and the eight lanes
      // of a quad pair (both halves) cover that row's 64 columns, one whole 128-byte line.  The
      // stores are non-temporal: the output is not re-read here, and whole lines streamed past
      // the L2 leave the operands that the next tiles re-read resident (partial-line
      // non-temporal stores are much slower).
      if (bf) {
        quad_transpose(ob, lane);
        const int k = fr & 3;
        const int64_t col = cbase + 32 * (k >> 1) + 16 * (k & 1) + 8 * h;
        const int coff = col < g.N ? (int)col * 2 : -1;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int rs = (i * 32 + (fr & ~3) + s) * (int)(ldo * esz);
          store16(ob[s], ro, coff >= 0 ? rs + coff : 0x7FFFFFF0, ST == 2);
        }
      }
    }
  }
  if constexpr (STATS) {
    // lane t < 16 of each half writes the totals of value t of each column block: column
    // j*32 + 16p + 8h + r (bf16, t = 8p + r) or j*32 + 8q + 4h + r (fp32, t = 4q + r)
    if (rbase < g.M) {
      const int t = lane & 15;
      const int64_t part = rbase / (TM * 32);
      const int64_t coff = bf ? 16 * (t >> 3) + 8 * h + (t & 7) : 8 * (t >> 2) + 4 * h + (t & 3);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t col = cbase + j * 32 + coff;
        const float sj = half_reduce_scatter16(csum[j], lane, [](float a, float b) { return __fadd_rn(a, b); });
        if ((lane & 31) < 16 && col < g.N) g.st_sum[part * g.N + col] = sj;
      }
    }
  }
}

// Two-stage 2 x 2 wave tiles run two workgroups per CU (two waves per SIMD): the register budget
// is held to that occupancy.
// MU: the launch carries a broadcast mean term, computed by one extra MFMA per wave and substep
// on the tile's B fragments (every row of that A block is the quantized mean).
//
// A workgroup takes a strided run of logical tiles within its XCD's contiguous share of the
// launch (one tile when the grid covers every tile).  Each tile runs prologue, K loop and
// epilogue in turn: the epilogue reads no stage memory and every wave has finished with the
// stages before it starts, so the next tile's prologue may refill them at once.  (The next
// tile's first loads cannot be issued ahead of the epilogue's stores: loads and stores share
// one vector-memory counter and may complete out of order, so no wait could single out the
// loads.)
template <int FMT, int WM, int WN, int TM, int TN, int STAGES, int AUX = 0, bool MU = false, bool STATS = false>
__global__ __launch_bounds__(64 * WM * WN, (STAGES == 2 && TM * TN <= 4) ? 2 : 1) void k_gemm(GemmArgs gin) {
  using T = GemmTile<FMT, WM, WN, TM, TN, STAGES, AUX, MU>;
  using C = typename T::C;
  static_assert(STAGES == 2 || STAGES == 3 || STAGES == 4, "stages");
  __shared__ __attribute__((aligned(1024))) uint8_t st0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[STAGES >= 3 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[STAGES >= 4 ? C::STAGE : 16];
  __shared__ float s_uv[C::BM + C::BN];  // rank-one term: r1 * u over the tile's rows, then v over its columns
  __shared__ __attribute__((aligned(16))) uint8_t s_mu[MU ? kMuBytes : 16];  // the mean row (MU)
  __shared__ float s_bias[MU ? WN * TN * 32 : 1];  // the tile's mean term, per column
  static_assert(C::BM + C::BN <= C::NT, "one rank-one element per thread");

  int first, stride, end;
  xcd_tiles((int)blockIdx.x, (int)gridDim.x, gin.n_work, first, stride, end);
  T t;
  t.clear();
  bool mu_loaded = false;
  for (int lin = first; lin < end; lin += stride) {
    GemmArgs g = gin;  // this tile's view (grouped launches retarget it to one group)
    int ntiles = g.tiles_m * g.tiles_n;
    int split = 0, tm, tn;
    if (gin.grouped == 1) {
      const int tn_all = gin.tiles_n;
      const GroupPos gp = group_scan(gin.offsets, gin.E, lin, true,
                                     [tn_all](int64_t len) { return ceil_div(len, (int64_t)C::BM) * tn_all; });
      if (gp.e < 0) continue;
      const int tms = (int)ceil_div(gp.len, (int64_t)C::BM);
      tile_coords((int)gp.local, tms, tn_all, gin.group_m < tms ? gin.group_m : tms, tm, tn);
      const int64_t gsa = (gin.K / C::BKE) * C::PIECE;  // tiled scale bytes per 32-row group
      g.M = gp.len;
      g.a_codes += gp.p32 * gin.lda_b;
      g.a_scales += (gp.p32 / 32) * gsa;
      g.b_codes += (int64_t)gp.e * gin.N * gin.ldb_b;
      g.b_scales += ((int64_t)gp.e * gin.N / 32) * gsa;
      if (FMT == AVERIS_NVFP4) { g.a_ts += gp.e; g.b_ts += gp.e; }
      if (gin.bias) g.bias += (int64_t)gp.e * gin.N;
      g.mu_row = gp.e;
      g.c = reinterpret_cast<uint8_t*>(gin.c) + gp.off * gin.ldc * (gin.c_bf16 ? 2 : 4);
    } else if (gin.grouped == 2) {
      const int e = lin / ntiles;
      tile_coords(lin % ntiles, g.tiles_m, g.tiles_n, g.group_m, tm, tn);
      const GroupPos gp = group_scan(gin.offsets, gin.E, e, false, [](int64_t) { return (int64_t)1; });
      const int64_t ke_pad = round_up(gp.len, (int64_t)C::BKE);
      g.K = ke_pad; g.k_chunk = ke_pad;
      g.lda_b = ke_pad / 2; g.ldb_b = ke_pad / 2;
      g.a_codes += gin.M * gp.p256 / 2;
      g.a_scales += gin.M * gp.p256 / C::G;
      g.b_codes += gin.N * gp.p256 / 2;
      g.b_scales += gin.N * gp.p256 / C::G;
      if (FMT == AVERIS_NVFP4) { g.a_ts += e; g.b_ts += e; }
      g.r1 = (float)gp.len;
      g.r1_row = e;
      g.c = reinterpret_cast<float*>(gin.c) + (int64_t)e * gin.M * gin.ldc;
    } else {
      split = lin / ntiles;
      tile_coords(lin % ntiles, g.tiles_m, g.tiles_n, g.group_m, tm, tn);
    }
    const int64_t m0 = (int64_t)tm * C::BM, n0 = (int64_t)tn * C::BN;
    const int64_t kb = (int64_t)split * g.k_chunk;
    const int64_t ke = kb + g.k_chunk < g.K ? kb + g.k_chunk : g.K;
    const int nsteps = (int)((ke - kb) / C::BKE);  // K and k_chunk are multiples of the K-step
    const int kb_byte = (int)(kb / 2), kb_sbyte = (int)(kb / C::BKE) * C::PIECE;
    const int k0 = (int)(kb / C::BKE);  // absolute index of the first K-step

    t.bind(g, m0, n0);
    // the mean row: once for a dense launch, per tile for a grouped one (its group's row)
    if constexpr (MU) {
      if (!mu_loaded || gin.grouped) t.issue_mean(g, s_mu);
      mu_loaded = true;
    }
    // prologue: K-steps 0 .. STAGES-2
    t.issue(kb_byte, kb_sbyte, st0);
    if (STAGES >= 3) t.issue(1 < nsteps ? kb_byte + C::BKB : 0, 1 < nsteps ? kb_sbyte + C::PIECE : 0, st1);
    if (STAGES >= 4) t.issue(2 < nsteps ? kb_byte + 2 * C::BKB : 0, 2 < nsteps ? kb_sbyte + 2 * C::PIECE : 0, st2);
    // this thread's rank-one element (loads overlap the prologue; used in the epilogue)
    const bool hr = g.splits == 1 && g.has_r1;
    float uv = 0.0f;
    if (hr && (int)threadIdx.x < C::BM + C::BN) {
      const int i = threadIdx.x;
      if (i < C::BM) {
        const int64_t row = m0 + i;
        if (row < g.M) uv = __fmul_rn(g.r1, mean_value<FMT>(g.ru, g.r1_row, row));
      } else {
        const int64_t col = n0 + (i - C::BM);
        if (col < g.N) uv = mean_value<FMT>(g.rv, g.r1_row, col);
      }
    }
    for (int it = 0; it < nsteps; it += STAGES) {
      if (STAGES == 2) {
        pipe_step<T, STAGES>(t, it, nsteps, kb_byte, kb_sbyte, st0, st1, s_mu, k0);
        pipe_step<T, STAGES>(t, it + 1, nsteps, kb_byte, kb_sbyte, st1, st0, s_mu, k0);
      } else if (STAGES == 3) {
        pipe_step<T, STAGES>(t, it, nsteps, kb_byte, kb_sbyte, st0, st2, s_mu, k0);
        pipe_step<T, STAGES>(t, it + 1, nsteps, kb_byte, kb_sbyte, st1, st0, s_mu, k0);
        pipe_step<T, STAGES>(t, it + 2, nsteps, kb_byte, kb_sbyte, st2, st1, s_mu, k0);
      } else {
        pipe_step<T, STAGES>(t, it, nsteps, kb_byte, kb_sbyte, st0, st3, s_mu, k0);
        pipe_step<T, STAGES>(t, it + 1, nsteps, kb_byte, kb_sbyte, st1, st0, s_mu, k0);
        pipe_step<T, STAGES>(t, it + 2, nsteps, kb_byte, kb_sbyte, st2, st1, s_mu, k0);
        pipe_step<T, STAGES>(t, it + 3, nsteps, kb_byte, kb_sbyte, st3, st2, s_mu, k0);
      }
    }
    wait_vm<0>();                 // no load may still be writing LDS
    __builtin_amdgcn_s_barrier();  // every wave is done reading the stages

    // ---- epilogue ----
    // no wave still reads the previous tile's s_uv / s_bias.  MU: row 0 of a wave's mean block
    // (lanes 0 and 32) holds the mean term of its column block wm; waves (0, wn) and (1, wn)
    // cover the two blocks of columns wn.
    if constexpr (MU) {
      if ((threadIdx.x & 31) == 0) {
        float* sb = s_bias + (t.wn * TN + t.wm) * 32 + 4 * ((threadIdx.x >> 5) & 1);
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int r = 0; r < 4; ++r) sb[8 * q + r] = t.acc_mu[4 * q + r];
      }
    }
    if (hr && (int)threadIdx.x < C::BM + C::BN) s_uv[threadIdx.x] = uv;
    if (MU || hr) lds_barrier();
    // (plain per-lane stores: in these kernels, whose multiplying waves also issue the operand
    // loads, whole-line non-temporal stores measured 1-2 % slower)
    epilogue_regs<FMT, TM, TN, MU, true, STATS, 0>(g, t.acc, m0 + t.wm * TM * 32, n0 + t.wn * TN * 32, split, threadIdx.x & 63,
                                   s_uv + t.wm * TM * 32, s_uv + C::BM + t.wn * TN * 32, s_bias + t.wn * TN * 32);
    t.clear();
  }
}

// Warp-specialized form of the 128 x 128 tile for MXFP4 dense launches without a bias vector or
// accumulation whose K-steps split evenly: waves 0-3 multiply and store, waves 4 .. 4+L-1 issue
// every operand load (loader l takes the shares of waves l, l+L, ..).  A workgroup's K-steps form
// one stream across its (tile, split) units, each of nsteps = k_chunk / 256 steps; global step q
// lives in ring stage q % S.  The loaders keep S - 1 steps in flight, crossing unit boundaries,
// and since their waits count only their own loads (no stores, no other waves' operations) a
// counted vmcnt singles out the oldest step: loads complete in order.
// Barrier sequence, the same for every wave: one barrier per K-step (a loader first waits until
// its loads of that step have landed; after the barrier stage (q - 1) % S is free, its last reader
// being step q - 1, and it refills it with step q + S - 1), plus one epilogue barrier per unit
// with the mean or the rank-one term.  Steps past the stream's end re-load the last unit's first
// step into the stage just freed, which nobody reads again, so every wait covers the same number
// of loads.
// MU: the mean term of the forward and input-gradient GEMMs (one more MFMA per four).  R1 (one
// split only): the weight gradient's rank-one term; the multiplying waves dequantize u and v for
// each tile before its K-steps (their only global loads) and add r1 u v^T in the epilogue.
// TMW: MFMA tiles per wave along M (2: 128 x 128 workgroup tiles; 4: 256 x 128, each wave 128 x
// 64, which reads 6 fragments from LDS per 8 MFMAs instead of 4 per 4).
template <int FMT, bool MU, bool R1, int S, int L, int TMW = 2, bool STATS = false>
__global__ __launch_bounds__(64 * (4 + L), 2) void k_gemm_ws(GemmArgs g) {
  constexpr int WM = 2, WN = 2, TM = TMW, TN = 2;
  using T = GemmTile<FMT, WM, WN, TM, TN, 2, 0, MU>;
  using C = typename T::C;
  constexpr int SSZ = TM == 2 ? (C::STAGE + 1023) / 1024 * 1024 : (C::STAGE + 255) / 256 * 256;  // 3 x 51 KB fit
  constexpr int SH = C::NW / L;                  // shares per loader wave
  constexpr int LPW = C::LPS * SH;               // loads per loader wave per K-step
  static_assert(C::NW % L == 0 && LPW * (S - 2) < 64, "vmcnt range");
  static_assert(!R1 || C::BM + C::BN == 256, "one rank-one factor per multiplying thread");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[S * SSZ];
  __shared__ __attribute__((aligned(16))) uint8_t s_mu[MU ? kMuBytes : 16];
  __shared__ float s_bias[MU ? WN * TN * 32 : 1];
  __shared__ float s_uv[R1 ? C::BM + C::BN : 1];  // r1 * u over the tile's rows, then v over its columns
  constexpr bool ebar = MU || R1;                 // the epilogue barrier

  int first, stride, end;
  xcd_tiles((int)blockIdx.x, (int)gridDim.x, g.n_work, first, stride, end);
  if (first >= end) return;
  const int nsteps = (int)(g.k_chunk / C::BKE);  // >= 1, the same for every (tile, split)
  const int ntw = (end - first + stride - 1) / stride;  // this workgroup's (tile, split) units
  const int total = ntw * nsteps;               // its K-steps
  const int ntiles = g.tiles_m * g.tiles_n;
  auto origin = [&](int ti, int64_t& m0, int64_t& n0, int& split) {
    const int lin = first + ti * stride;
    int tm, tn;
    split = lin / ntiles;
    tile_coords(lin % ntiles, g.tiles_m, g.tiles_n, g.group_m, tm, tn);
    m0 = (int64_t)tm * C::BM;
    n0 = (int64_t)tn * C::BN;
  };
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));

  if (wave >= C::NW) {
    // ---- loader wave l ----
    const int l = wave - C::NW;
    T lt[SH];
    int bound = 0;  // unit whose views lt holds
    int64_t m0, n0;
    int split;
    origin(0, m0, n0, split);
#pragma unroll
    for (int i = 0; i < SH; ++i) lt[i].bind(g, m0, n0, l + i * L);
    if constexpr (MU) {
#pragma unroll
      for (int i = 0; i < SH; ++i) lt[i].issue_mean(g, s_mu);
    }
    auto issue = [&](int q) {  // global step q into stage q % S
      int st = 0;
      if (q < total) {
        const int ti = q / nsteps;
        st = q - ti * nsteps;
        if (ti != bound) {
          bound = ti;
          origin(ti, m0, n0, split);
#pragma unroll
          for (int i = 0; i < SH; ++i) lt[i].bind(g, m0, n0, l + i * L);
        }
      }
      uint8_t* stg = ring + (q % S) * SSZ;
      const int kstep = (int)((int64_t)split * g.k_chunk / C::BKE) + st;  // absolute K-step
#pragma unroll
      for (int i = 0; i < SH; ++i) lt[i].issue(kstep * C::BKB, kstep * C::PIECE, stg);
    };
    for (int q = 0; q < S - 1; ++q) issue(q);
    for (int q = 0; q < total; ++q) {
      wait_vm<LPW * (S - 2)>();
      __builtin_amdgcn_s_barrier();
      issue(q + S - 1);
      if (ebar && q % nsteps == nsteps - 1) __builtin_amdgcn_s_barrier();  // the epilogue barrier
    }
    wait_vm<0>();  // the trailing re-loads land before the workgroup ends
    return;
  }

  // ---- multiplying waves ----
  T t;
  t.bind(g, 0, 0);  // lane constants (this wave loads nothing)
  int q = 0;
  for (int ti = 0; ti < ntw; ++ti) {
    int64_t m0, n0;
    int split;
    origin(ti, m0, n0, split);
    const int k0 = (int)((int64_t)split * g.k_chunk / C::BKE);
    t.clear();
    float uv = 0.0f;
    if constexpr (R1) {
      const int i = threadIdx.x;  // 256 multiplying threads = BM + BN
      if (i < C::BM) {
        if (m0 + i < g.M) uv = __fmul_rn(g.r1, mean_value<FMT>(g.ru, g.r1_row, m0 + i));
      } else if (n0 + (i - C::BM) < g.N) {
        uv = mean_value<FMT>(g.rv, g.r1_row, n0 + (i - C::BM));
      }
    }
    for (int st = 0; st < nsteps; ++st, ++q) {
      __builtin_amdgcn_s_barrier();
      if constexpr (TM == 2) t.compute_mx_preload(ring + (q % S) * SSZ, s_mu, k0 + st);
      else t.compute(ring + (q % S) * SSZ, s_mu, k0 + st);
    }
    if constexpr (MU) {
      if ((threadIdx.x & 31) == 0) {
        float* sb = s_bias + (t.wn * TN + t.wm) * 32 + 4 * ((threadIdx.x >> 5) & 1);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
          for (int r = 0; r < 4; ++r) sb[8 * qq + r] = t.acc_mu[4 * qq + r];
      }
    }
    if constexpr (R1) s_uv[threadIdx.x] = uv;
    if constexpr (ebar) lds_barrier();
    epilogue_regs<FMT, TM, TN, MU, R1, STATS, (STATS && TM == 4) ? 0 : 2>(g, t.acc, m0 + t.wm * TM * 32, n0 + t.wn * TN * 32, split, threadIdx.x & 63,
                                       s_uv + t.wm * TM * 32, s_uv + C::BM + t.wn * TN * 32,
                                       s_bias + t.wn * TN * 32);
  }
}

// Warp-specialized form of the grouped weight gradient (both formats, 128 x 128 tiles; NVFP4 takes
// the group's two tensor scales in the epilogue): unit lin is
// tile lin % (tiles_m tiles_n) of group e = lin / (tiles_m tiles_n), whose K is the group's token
// count padded to 256, so units differ in their number of K-steps (none for an empty group).
// Waves as in k_gemm_ws; the loaders walk a cursor over the flattened (unit, K-step) sequence and
// keep S - 1 steps in flight across units.  One barrier per K-step, the same for every wave, and
// no other: a unit's epilogue overlaps the loaders' next K-steps, and its stores drain while the
// multiplying waves go on to the next unit (they issue no global loads that would wait for them).
//   * Each group's token count and first 256-token block sit in an LDS table built once per
//     workgroup, so a unit switch reads no global memory (a loader's vector load there would have
//     to wait for every operand load in flight).
//   * R1: the rank-one factors l_e u and v come from fp32 tables written by k_rank_one_vectors;
//     with every K-step the loaders also copy the unit's 128 + 128 factors into the stage, and the
//     multiplying waves read them from the stage of the unit's last K-step during its epilogue
//     (the loaders refill that stage only after the next K-step's barrier).  Empty units store
//     zeros (their rank-one factor l_e is 0).
//   * Schedule: groups differ widely in K (a skewed routing gives one expert 30 K-steps per
//     tile and another 1), so units are dealt by work, not by count.  The host ranks the groups
//     by K-steps, longest first (kernel argument `order`); unit rank k is tile k % T of group
//     order[k / T] (T tiles per group).  Round r hands ranks r G .. r G + G - 1 to the G
//     workgroups, in reverse order on odd rounds (a snake deal), so every workgroup gets a
//     near-equal sum of K-steps.  Workgroups are numbered XCD by XCD (dispatch puts workgroup b
//     on XCD b % 8), so one XCD takes consecutive ranks: neighbouring tiles of one group, whose
//     operands then meet in that XCD's L2.
// Steps past the stream's end re-load the last step issued into the stage just freed, which
// nobody reads.
constexpr int kDwMaxGroups = 1024;  // groups of the LDS table (more: the three-stage kernel)

struct DwOrder { uint16_t e[kDwMaxGroups]; };  // groups, most K-steps first

struct DwUnit { int e, ns; int64_t m0, n0; };

// Logical index of workgroup b when the G workgroups are numbered XCD by XCD.
__device__ __forceinline__ int xcd_local(int b, int G) {
  const int x = b & 7, k = b >> 3, q = G >> 3, r = G & 7;
  return x * q + (x < r ? x : r) + k;
}

// Rank of the u-th unit of logical workgroup lw in the snake deal over G workgroups.
__device__ __forceinline__ int dw_rank(int u, int lw, int G) { return u * G + ((u & 1) ? G - 1 - lw : lw); }

template <class C>
__device__ __forceinline__ DwUnit dw_unit(const GemmArgs& gin, int rank, const DwOrder& ord, const int* s_len,
                                          const int* s_t256, GemmArgs& g) {
  g = gin;
  const int ntiles = gin.tiles_m * gin.tiles_n;
  DwUnit u;
  u.e = ord.e[uniform32(rank / ntiles)];
  int tm, tn;
  tile_coords(rank % ntiles, gin.tiles_m, gin.tiles_n, gin.group_m, tm, tn);
  const int64_t len = uniform32(s_len[u.e]), t0 = (int64_t)uniform32(s_t256[u.e]) * C::BKE;
  const int64_t ke_pad = round_up(len, (int64_t)C::BKE);
  g.K = ke_pad; g.k_chunk = ke_pad;
  g.lda_b = ke_pad / 2; g.ldb_b = ke_pad / 2;
  g.a_codes += gin.M * t0 / 2;
  g.a_scales += gin.M * t0 / C::G;
  g.b_codes += gin.N * t0 / 2;
  g.b_scales += gin.N * t0 / C::G;
  g.c = reinterpret_cast<float*>(gin.c) + (int64_t)u.e * gin.M * gin.ldc;
  if (C::G == 16) { g.a_ts = gin.a_ts + u.e; g.b_ts = gin.b_ts + u.e; }  // NVFP4: per-group tensor scales
  g.has_r1 = gin.has_r1 && len > 0;
  u.m0 = (int64_t)tm * C::BM;
  u.n0 = (int64_t)tn * C::BN;
  u.ns = (int)(ke_pad / C::BKE);
  return u;
}

// Rank-one factors of the grouped weight gradient, one fp32 table row per group: u_tab[e][i] =
// l_e * u_e[i] (i < M) and v_tab[e][j] = v_e[j] (j < N), the dequantized means (rotation undone).
template <int FMT>
__global__ __launch_bounds__(256) void k_rank_one_vectors(GemmArgs g, float* __restrict__ u_tab,
                                                          float* __restrict__ v_tab, int64_t mpad, int64_t npad) {
  const int e = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const float len = (float)(g.offsets[e + 1] - g.offsets[e]);
  if (i < g.M) u_tab[e * mpad + i] = __fmul_rn(len, mean_value<FMT>(g.ru, e, i));
  else if (i < g.M + g.N) v_tab[e * npad + (i - g.M)] = mean_value<FMT>(g.rv, e, i - g.M);
}

// TMW = 4: 256 x 128 tiles (a 3-stage ring; the group tables hold kDwMaxGroupsWide groups so that
// the ring and the tables fit the LDS).
constexpr int kDwMaxGroupsWide = 128;
template <int FMT, bool R1, int S, int L, int TMW = 2>
__global__ __launch_bounds__(64 * (4 + L), 1) void k_gemm_ws_dw(GemmArgs g, const float* __restrict__ u_tab,
                                                                const float* __restrict__ v_tab, int64_t mpad,
                                                                int64_t npad, DwOrder ord) {
  constexpr int WM = 2, WN = 2, TM = TMW, TN = 2;
  using T = GemmTile<FMT, WM, WN, TM, TN, 2, 0, false>;
  using C = typename T::C;
  constexpr int UV_OFF = (C::STAGE + 255) / 256 * 256;
  constexpr int MAXG = TMW == 2 ? kDwMaxGroups : kDwMaxGroupsWide;
  constexpr int UV_BYTES = (C::BM + C::BN) * 4;  // R1: u over the tile's rows, then v over its columns
  constexpr int ALIGN = TM == 2 ? 1024 : 256;     // (256 x 128: three stages and the tables fit)
  constexpr int SSZ = (UV_OFF + (R1 ? UV_BYTES : 0) + ALIGN - 1) / ALIGN * ALIGN;
  constexpr int SH = C::NW / L;                     // shares per loader wave
  constexpr int LPW = C::LPS * SH + (R1 ? 1 : 0);  // loads per loader wave per K-step
  static_assert(C::NW % L == 0 && LPW * (S - 2) < 64, "vmcnt range");
  static_assert(!R1 || (L == 2 && C::BM <= 256 && C::BN == 128), "one rank-one slice per loader");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[S * SSZ];
  __shared__ int s_len[MAXG], s_t256[MAXG];

  const int G = (int)gridDim.x, lw = xcd_local((int)blockIdx.x, G);
  int ntw = 0;  // this workgroup's units
  while (dw_rank(ntw, lw, G) < g.n_work) ++ntw;
  if (ntw == 0) return;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;

  // group table: length and first 256-token block of every group (wave 0, one pass of
  // 64-group prefix scans), before any operand load is in flight
  if (wave == 0) {
    int64_t base = 0;
    for (int e0 = 0; e0 < g.E; e0 += 64) {
      const int e = e0 + lane;
      const int64_t len = e < g.E ? g.offsets[e + 1] - g.offsets[e] : 0;
      const int64_t c = ceil_div(len, (int64_t)C::BKE);
      int64_t sc = c;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int64_t x = __shfl_up(sc, d, 64);
        if (lane >= d) sc += x;
      }
      if (e < g.E) { s_len[e] = (int)len; s_t256[e] = (int)(base + sc - c); }
      base += __shfl(sc, 63, 64);
    }
  }
  __syncthreads();

  if (wave >= C::NW) {
    // ---- loader wave l: the cursor is unit cu, its K-step cs of cns; lt holds the views of the
    // last unit with K-steps (the lambdas are forced inline: a call would keep what they capture
    // in scratch memory) ----
    const int l = wave - C::NW;
    T lt[SH];
    __amdgpu_buffer_rsrc_t ruv = make_rsrc(u_tab, 0);  // R1: this loader's rank-one slice
    int cu = 0, cs = 0, cns = 0, last = 0;
    bool have = false;  // some unit of this workgroup has K-steps
    auto open_unit = [&](int u) __attribute__((always_inline)) {
      GemmArgs v;
      const DwUnit du = dw_unit<C>(g, dw_rank(u, lw, G), ord, s_len, s_t256, v);
      cns = du.ns;
      if (cns > 0) {
#pragma unroll
        for (int i = 0; i < SH; ++i) lt[i].bind(v, du.m0, du.n0, l + i * L);
        if constexpr (R1) {
          const int64_t o0 = l == 0 ? du.m0 : du.n0, lim = l == 0 ? g.M : g.N;
          const float* base = (l == 0 ? u_tab + du.e * mpad : v_tab + du.e * npad) + o0;
          ruv = make_rsrc(base, (lim - o0) * 4);
        }
        have = true;
      }
    };
    auto skip_empty = [&]() __attribute__((always_inline)) {
      while (cu < ntw && cs >= cns) {
        ++cu;
        cs = 0;
        if (cu < ntw) open_unit(cu);
      }
    };
    auto issue_next = [&](int q) __attribute__((always_inline)) {  // into stage q % S
      if (!have) return;  // nothing to load, and no K-step barriers either
      int kstep = last;
      if (cu < ntw) {
        kstep = cs++;
        last = kstep;
      }
      uint8_t* stg = ring + (q % S) * SSZ;
#pragma unroll
      for (int i = 0; i < SH; ++i) lt[i].issue(kstep * C::BKB, kstep * C::PIECE, stg);
      // BM / 4 (u) or BN / 4 (v) lanes x 16 bytes = the factors, packed u then v.  Only those
      // lanes issue the copy: a direct-to-LDS load writes every active lane's bytes (zeros past
      // the range), and the packed slots have no room for the rest.
      if constexpr (R1) {
        if (lane < (l == 0 ? C::BM : C::BN) / 4) dma16<0>(ruv, stg + UV_OFF + (l == 0 ? 0 : C::BM * 4), lane * 16, 0);
      }
      skip_empty();
    };
    open_unit(0);
    skip_empty();
    for (int q = 0; q < S - 1; ++q) issue_next(q);
    int q = 0;
    for (int u = 0; u < ntw; ++u) {
      GemmArgs gu;
      const int ns = dw_unit<C>(g, dw_rank(u, lw, G), ord, s_len, s_t256, gu).ns;
      for (int st = 0; st < ns; ++st, ++q) {
        wait_vm<LPW * (S - 2)>();
        __builtin_amdgcn_s_barrier();
        issue_next(q + S - 1);
      }
    }
    wait_vm<0>();  // the trailing re-loads land before the workgroup ends
    return;
  }

  // ---- multiplying waves ----
  T t;
  t.bind(g, 0, 0);  // lane constants (this wave loads nothing)
  int q = 0;
  for (int u = 0; u < ntw; ++u) {
    GemmArgs gu;
    const DwUnit du = dw_unit<C>(g, dw_rank(u, lw, G), ord, s_len, s_t256, gu);
    t.clear();
    for (int st = 0; st < du.ns; ++st, ++q) {
      __builtin_amdgcn_s_barrier();
      if constexpr (TM == 2 && FMT == AVERIS_MXFP4) t.compute_mx_preload(ring + (q % S) * SSZ, ring, st);
      else t.compute(ring + (q % S) * SSZ, ring, st);
    }
    // R1 with K-steps: the factors sit in the stage of the unit's last K-step
    const float* uv = reinterpret_cast<const float*>(ring + ((q + S - 1) % S) * SSZ + UV_OFF);
    epilogue_regs<FMT, TM, TN, false, R1, false, 2, false>(gu, t.acc, du.m0 + t.wm * TM * 32, du.n0 + t.wn * TN * 32, 0, lane,
                                          uv + t.wm * TM * 32, uv + C::BM + t.wn * TN * 32, uv);
  }
}

// Warp-specialized grouped forward / input gradient (MXFP4, 128 x 128 tiles, or 256 x 128 with
// TMW = 4): logical tile lin
// enumerates, group after group, the ceil(l_e / 128) x tiles_n tiles of every group (expert);
// every tile has the same K, so a workgroup's K-steps form one stream as in k_gemm_ws.  Each
// group's first row, first 32-row-padded row and first logical tile sit in an LDS table built
// once per workgroup, so a tile switch reads no global memory.  MU: the mean row differs per
// group, so with every K-step the loaders also copy that step's 128 mean code bytes and 8 scale
// bytes of the tile's group into the stage (both loaders copy the same bytes), and the
// multiplying waves read them from there.
constexpr int kWsgMaxGroups = 256;

struct GTile { int e; int64_t m0, n0; };

template <class C>
__device__ __forceinline__ GTile wsg_tile(const GemmArgs& gin, int lin, const int* s_off, const int* s_p32,
                                          const int* s_t0, GemmArgs& g) {
  int lo = 0, hi = gin.E;  // the last group whose first tile is <= lin (it is not empty)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_t0[mid] <= lin) lo = mid; else hi = mid;
  }
  GTile t;
  t.e = uniform32(lo);
  const int64_t off = uniform32(s_off[t.e]), len = uniform32(s_off[t.e + 1]) - off, p32 = uniform32(s_p32[t.e]);
  const int tms = (int)ceil_div(len, (int64_t)C::BM);
  int tm, tn;
  tile_coords(lin - uniform32(s_t0[t.e]), tms, gin.tiles_n, gin.group_m < tms ? gin.group_m : tms, tm, tn);
  const int64_t gsa = (gin.K / C::BKE) * C::PIECE;  // tiled scale bytes per 32-row group
  g = gin;
  g.M = len;
  g.a_codes += p32 * gin.lda_b;
  g.a_scales += (p32 / 32) * gsa;
  g.b_codes += (int64_t)t.e * gin.N * gin.ldb_b;
  g.b_scales += ((int64_t)t.e * gin.N / 32) * gsa;
  g.c = reinterpret_cast<uint8_t*>(gin.c) + off * gin.ldc * (gin.c_bf16 ? 2 : 4);
  t.m0 = (int64_t)tm * C::BM;
  t.n0 = (int64_t)tn * C::BN;
  return t;
}

template <int FMT, bool MU, int S, int L, int TMW = 2>
__global__ __launch_bounds__(64 * (4 + L), 1) void k_gemm_ws_g(GemmArgs g) {
  constexpr int WM = 2, WN = 2, TM = TMW, TN = 2;
  using T = GemmTile<FMT, WM, WN, TM, TN, 2, 0, MU>;
  using C = typename T::C;
  constexpr int MU_OFF = (C::STAGE + 255) / 256 * 256;  // the K-step's mean codes, then at +256 its scales
  constexpr int SSZ = (MU_OFF + (MU ? 512 : 0) + 1023) / 1024 * 1024;
  constexpr int SH = C::NW / L;
  constexpr int LPW = C::LPS * SH + (MU ? 2 : 0);  // loads per loader wave per K-step
  static_assert(C::NW % L == 0 && LPW * (S - 2) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t ring[S * SSZ];
  __shared__ float s_bias[MU ? WN * TN * 32 : 1];
  __shared__ int s_off[kWsgMaxGroups + 1], s_p32[kWsgMaxGroups], s_t0[kWsgMaxGroups + 1];

  int first, stride, end;
  xcd_tiles((int)blockIdx.x, (int)gridDim.x, g.n_work, first, stride, end);
  if (first >= end) return;
  const int nsteps = (int)(g.K / C::BKE);
  const int ntw = (end - first + stride - 1) / stride;
  const int total = ntw * nsteps;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;

  // group table (wave 0, 64-group prefix scans), before any operand load is in flight
  if (wave == 0) {
    int bp = 0, bt = 0;
    for (int e0 = 0; e0 < g.E; e0 += 64) {
      const int e = e0 + lane;
      const int64_t o = e < g.E ? g.offsets[e] : 0;
      const int len = e < g.E ? (int)(g.offsets[e + 1] - o) : 0;
      const int p = (int)round_up(len, 32), tl = (int)ceil_div(len, (int64_t)C::BM) * g.tiles_n;
      int sp = p, st = tl;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int xp = __shfl_up(sp, d, 64), xt = __shfl_up(st, d, 64);
        if (lane >= d) { sp += xp; st += xt; }
      }
      if (e < g.E) { s_off[e] = (int)o; s_p32[e] = bp + sp - p; s_t0[e] = bt + st - tl; }
      bp += __shfl(sp, 63, 64);
      bt += __shfl(st, 63, 64);
    }
    if (lane == 0) { s_off[g.E] = (int)g.offsets[g.E]; s_t0[g.E] = bt; }
  }
  __syncthreads();

  if (wave >= C::NW) {
    // ---- loader wave l ----
    const int l = wave - C::NW;
    T lt[SH];
    int bound = -1;
    __amdgpu_buffer_rsrc_t rmc = make_rsrc(g.mu_codes, 0), rms = make_rsrc(g.mu_scales, 0);
    int ms_off = 0x7FFFFFF0;
    auto issue = [&](int q) __attribute__((always_inline)) {  // global step q into stage q % S
      const int qq = q < total ? q : total - 1;  // past the end: re-load the last step (unread)
      const int ti = qq / nsteps, st = qq - ti * nsteps;
      if (ti != bound) {
        bound = ti;
        GemmArgs v;
        const GTile gt = wsg_tile<C>(g, first + ti * stride, s_off, s_p32, s_t0, v);
#pragma unroll
        for (int i = 0; i < SH; ++i) lt[i].bind(v, gt.m0, gt.n0, l + i * L);
        if constexpr (MU) {
          rmc = make_rsrc(g.mu_codes + (int64_t)gt.e * (g.K / 2), g.K / 2);
          rms = make_rsrc(g.mu_scales, (int64_t)round_up(g.E, 32) * (g.K / C::G));
          ms_off = lane < 2 ? (int)(((int64_t)(gt.e >> 5) * (g.K / C::BKE)) * C::PIECE + (gt.e & 31) * C::SB) + lane * 4
                            : 0x7FFFFFF0;
        }
      }
      uint8_t* stg = ring + (q % S) * SSZ;
#pragma unroll
      for (int i = 0; i < SH; ++i) lt[i].issue(st * C::BKB, st * C::PIECE, stg);
      if constexpr (MU) {
        dma4<0>(rmc, stg + MU_OFF, lane < 32 ? lane * 4 : 0x7FFFFFF0, st * C::BKB);
        dma4<0>(rms, stg + MU_OFF + 256, ms_off, st * C::PIECE);
      }
    };
    for (int q = 0; q < S - 1; ++q) issue(q);
    for (int q = 0; q < total; ++q) {
      wait_vm<LPW * (S - 2)>();
      __builtin_amdgcn_s_barrier();
      issue(q + S - 1);
      if (MU && q % nsteps == nsteps - 1) __builtin_amdgcn_s_barrier();  // the epilogue barrier
    }
    wait_vm<0>();  // the trailing re-loads land before the workgroup ends
    return;
  }

  // ---- multiplying waves ----
  T t;
  t.bind(g, 0, 0);  // lane constants (this wave loads nothing)
  int q = 0;
  for (int ti = 0; ti < ntw; ++ti) {
    GemmArgs gu;
    const GTile gt = wsg_tile<C>(g, first + ti * stride, s_off, s_p32, s_t0, gu);
    t.clear();
    for (int st = 0; st < nsteps; ++st, ++q) {
      __builtin_amdgcn_s_barrier();
      const uint8_t* stg = ring + (q % S) * SSZ;
      if constexpr (TM == 2) t.template compute_mx_preload<256>(stg, stg + MU_OFF, 0);
      else t.template compute<256>(stg, stg + MU_OFF, 0);
    }
    if constexpr (MU) {
      if ((threadIdx.x & 31) == 0) {
        float* sb = s_bias + (t.wn * TN + t.wm) * 32 + 4 * ((threadIdx.x >> 5) & 1);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
#pragma unroll
          for (int r = 0; r < 4; ++r) sb[8 * qq + r] = t.acc_mu[4 * qq + r];
      }
      lds_barrier();
    }
    epilogue_regs<FMT, TM, TN, MU, false>(gu, t.acc, gt.m0 + t.wm * TM * 32, gt.n0 + t.wn * TN * 32, 0, lane,
                                          s_bias, s_bias, s_bias + t.wn * TN * 32);
  }
}

// Split-K reduce: C = (accumulate ? C : 0) + (sum_s P[s] in split order + bias[col]
// + r1 * u[row] * v[col]), four columns per thread (N % 8 == 0); fp32 or bf16 output; u and v
// dequantized from the quantized means in place.
template <int FMT>
__global__ __launch_bounds__(256) void k_splitk_reduce(const float* __restrict__ part, int splits, GemmArgs g,
                                                       void* __restrict__ c, int64_t ldc, int c_bf16) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nq = g.N / 4;
  if (q >= g.M * nq) return;
  const int64_t row = q / nq, col = (q % nq) * 4;
  const int64_t idx = row * g.N + col;
  float4 s = *reinterpret_cast<const float4*>(part + idx);
  for (int p = 1; p < splits; ++p) {
    const float4 t = *reinterpret_cast<const float4*>(part + (int64_t)p * g.M * g.N + idx);
    s.x = __fadd_rn(s.x, t.x); s.y = __fadd_rn(s.y, t.y); s.z = __fadd_rn(s.z, t.z); s.w = __fadd_rn(s.w, t.w);
  }
  float v[4] = {s.x, s.y, s.z, s.w};
  const float ru = g.has_r1 ? __fmul_rn(g.r1, mean_value<FMT>(g.ru, g.r1_row, row)) : 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (g.bias) v[e] = __fadd_rn(v[e], g.bias[col + e]);
    if (g.has_r1) v[e] = __fadd_rn(v[e], __fmul_rn(ru, mean_value<FMT>(g.rv, g.r1_row, col + e)));
  }
  if (c_bf16) {
    uint2 o;
    o.x = pack_bf16x2(v[0], v[1]); o.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(c) + row * ldc + col) = o;
  } else {
    float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(c) + row * ldc + col);
    if (g.accumulate) {
      const float4 o = *dst;
      v[0] = __fadd_rn(o.x, v[0]); v[1] = __fadd_rn(o.y, v[1]); v[2] = __fadd_rn(o.z, v[2]); v[3] = __fadd_rn(o.w, v[3]);
    }
    *dst = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Mean-term GEMV: out[j] = alpha * sum_k DQ(mu)[k] DQ(B)[j][k], one wave per output row.
// Grouped launches (gridDim.y = E): group e uses row e of mu, rows e N .. of B, out + e N.
// Each lane takes 32-element chunks; code products summed exactly in fp32 within a chunk, the
// chunk sums scaled and accumulated in fp64; fixed-order lane reduction.
template <int FMT>
__global__ __launch_bounds__(256) void k_gemv_mean(const uint8_t* __restrict__ mu_codes, const uint8_t* __restrict__ mu_scales,
                                                   const float* __restrict__ mu_ts, const uint8_t* __restrict__ b_codes,
                                                   const uint8_t* __restrict__ b_scales, int64_t ldb_b,
                                                   const float* __restrict__ b_ts, int64_t N, int64_t K, float* __restrict__ out) {
  constexpr int G = FMT == AVERIS_MXFP4 ? 32 : 16;
  const int lane = threadIdx.x & 63;
  const int64_t e = blockIdx.y;
  const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= N) return;
  const int64_t jb = e * N + j;  // row of B
  mu_codes += e * (K / 2);
  const uint8_t* bc = b_codes + jb * ldb_b;
  double s = 0.0;
  for (int64_t ch = lane; ch * 32 < K; ch += 64) {
    const uint4 ca = *reinterpret_cast<const uint4*>(mu_codes + ch * 16);
    const uint4 cb = *reinterpret_cast<const uint4*>(bc + ch * 16);
    const uint32_t wa[4] = {ca.x, ca.y, ca.z, ca.w}, wb[4] = {cb.x, cb.y, cb.z, cb.w};
    float part[2] = {0.0f, 0.0f};  // exact: sums of products of E2M1 values
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int bsel = 0; bsel < 4; ++bsel) {
        const float2 a = fp4x2_to_f32(wa[q], bsel), b = fp4x2_to_f32(wb[q], bsel);
        part[q >> 1] = __fadd_rn(part[q >> 1], __fadd_rn(__fmul_rn(a.x, b.x), __fmul_rn(a.y, b.y)));
      }
    if (FMT == AVERIS_MXFP4) {
      const int ex = (int)mu_scales[scale_offset(e, ch, K, G)] + (int)b_scales[scale_offset(jb, ch, K, G)] - 254;
      s += ldexp((double)part[0] + (double)part[1], ex);
    } else {
      const int64_t b0 = 2 * ch, b1 = 2 * ch + 1;
      s += (double)part[0] * ((double)e4m3_value(mu_scales[scale_offset(e, b0, K, G)]) *
                              (double)e4m3_value(b_scales[scale_offset(jb, b0, K, G)])) +
           (double)part[1] * ((double)e4m3_value(mu_scales[scale_offset(e, b1, K, G)]) *
                              (double)e4m3_value(b_scales[scale_offset(jb, b1, K, G)]));
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  if (lane == 0) {
    double alpha = 1.0;
    if (FMT == AVERIS_NVFP4) alpha = (double)mu_ts[e] * (double)b_ts[e];
    out[e * N + j] = (float)(s * alpha);
  }
}

// ------------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------------
static int g_count(int fmt) { return fmt == AVERIS_MXFP4 ? 32 : 16; }

// Configurations: 128 x 128 tiles of 2 x 2 multiplying waves with 2 x 2 MFMA tiles each, except
// KCFG_LONG96 (measured on MI355X against 256 x 128 (4 and 8 waves), 128 x 256, 256 x 192 and
// 256 x 256 tiles, and against 128-element K-steps with 3 and 4 stages, at the Qwen3-0.6B-shaped
// linears):
//   KCFG_WS     warp-specialized (k_gemm_ws): two loader waves keep three K-steps of a 4-stage
//               ring in flight across tiles, one workgroup per CU; every MXFP4 dense launch
//               without accumulation whose K-steps split evenly (forward and input-gradient
//               GEMMs: 8-16 % faster than KCFG_SHORT; weight gradients: 23-27 % faster than
//               KCFG_LONG);
//   KCFG_WSW    the warp-specialized kernel on 256 x 128 tiles (waves of 128 x 64: 0.75x the LDS
//               bytes per flop, the bound of the 128 x 128 form), a 3-stage ring; short-K launches
//               without the rank-one term that still give every CU a tile: 7-14 % faster;
//   KCFG_SHORT  two LDS stages, two workgroups per CU (70 KB LDS, <= 256 VGPRs each): the other
//               short-K launches (NVFP4, grouped, accumulate, GEMV mean term);
//   KCFG_LONG   three stages, one workgroup per CU, deeper prefetch, for the other long-K
//               launches (NVFP4, and grouped weight gradients past the warp-specialized
//               kernel's group table);
//   KCFG_LONG96 the long-K kernel on 128 x 96 tiles (4 x 1 waves of 32 x 96), for dense
//               single-split long-K launches whose 128 x 128 tiles would leave CUs idle in
//               their last round (the NVFP4 1024 x 3072 weight gradient: 192 tiles -> 256).
constexpr int KCFG_LONG = 0, KCFG_SHORT = 1, KCFG_WS = 2, KCFG_LONG96 = 3, KCFG_WSW = 4, KCFG_WSDW = 5, KCFG_WSG = 6,
              KCFG_WSGW = 7, KCFG_WSDWW = 8;
constexpr int kWsStages = 4, kWsLoaders = 2;  // warp-specialized kernel: ring depth, loader waves
constexpr bool kWsLongK = true;               // warp-specialized kernel for long K too
constexpr bool kWsWide = true;                // 256 x 128 warp-specialized tiles for short K
constexpr bool kWsgWide = true;               // 256 x 128 tiles for the grouped forward / input gradient
constexpr bool kDwWide = true;                // 256 x 128 tiles for the grouped weight gradient
struct TileCfg { int bm, bn; };
static TileCfg tile_of(int cfg) {
  return cfg == KCFG_LONG96                                            ? TileCfg{128, 96}
         : (cfg == KCFG_WSW || cfg == KCFG_WSGW || cfg == KCFG_WSDWW) ? TileCfg{256, 128}
                                                                      : TileCfg{128, 128};
}
constexpr int kBKE = 256;
// Short K: the warp-specialized kernel (MXFP4 dense launches; the rest fall back to the two-stage
// kernel).  Long K: three stages, one workgroup per CU (MXFP4 dense launches: warp-specialized).
static int pick_cfg(int64_t K) { return K >= 4096 ? KCFG_LONG : KCFG_WS; }

static int splits_for(int cfg, int64_t M, int64_t N, int64_t K) {
  const TileCfg tc = tile_of(cfg);
  const int64_t tiles = ceil_div(M, tc.bm) * ceil_div(N, tc.bn);
  if (tiles >= 192) return 1;
  int64_t s = ceil_div(256, tiles > 0 ? tiles : 1);
  const int64_t ksteps = ceil_div(K, kBKE);
  if (s > ksteps) s = ksteps;
  if (s > 8) s = 8;
  return s < 1 ? 1 : (int)s;
}
int choose_splits(int fmt, int64_t M, int64_t N, int64_t K) {
  (void)fmt;
  return splits_for(pick_cfg(K), M, N, K);
}

// workspace: [256 B][mean-term bias E x N fp32], then split-K partials [splits][M][N] fp32
// (dense launches only)
static size_t partials_offset(int64_t N, int64_t E) { return 256 + (size_t)round_up(E * N * 4, 1024); }

size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, int splits) {
  (void)K;
  size_t b = partials_offset(N, 1);
  if (splits > 1) b += (size_t)splits * M * N * 4;
  return b;
}
size_t gemm_grouped_ws_bytes(int64_t M, int64_t N, int64_t E) {
  (void)M;
  return partials_offset(N, E);
}
// grouped weight gradient: [256 B][u_tab E x round_up(M, 128) fp32][v_tab E x round_up(N, 128) fp32]
size_t gemm_grouped_dw_ws_bytes(int64_t M, int64_t N, int64_t E) {
  return 256 + (size_t)E * (round_up(M, 128) + round_up(N, 128)) * 4;
}

// stats: the STATS form of the kernels that take the output's column sums in the epilogue
// (MXFP4 warp-specialized, NVFP4 two-stage)
template <int F>
static void launch_cfg(int cfg, bool mu, const GemmArgs& g, unsigned grid, hipStream_t s, void* ws,
                       const int64_t* h_offsets, bool stats = false) {
  if (cfg == KCFG_WSDW || cfg == KCFG_WSDWW) {  // grouped weight gradient
    constexpr int S = kWsStages, L = kWsLoaders;
    const bool wide = cfg == KCFG_WSDWW;
    const int64_t mpad = round_up(g.M, 128), npad = round_up(g.N, 128);
    float* u_tab = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + 256);
    float* v_tab = u_tab + g.E * mpad;
    // groups ranked by K-steps, most first (stable: ties keep group order)
    DwOrder ord;
    std::vector<std::pair<int64_t, int>> ks((size_t)g.E);
    for (int e = 0; e < g.E; ++e) ks[e] = {-ceil_div(h_offsets[e + 1] - h_offsets[e], (int64_t)kBKE), e};
    std::stable_sort(ks.begin(), ks.end());
    for (int e = 0; e < g.E; ++e) ord.e[e] = (uint16_t)ks[e].second;
    if (g.has_r1)
      hipLaunchKernelGGL(k_rank_one_vectors<F>, dim3((unsigned)ceil_div(g.M + g.N, 256), (unsigned)g.E), dim3(256), 0,
                         s, g, u_tab, v_tab, mpad, npad);
    // 256 x 128 tiles (MXFP4 only: three NVFP4 stages of that size exceed the LDS)
    if constexpr (F == AVERIS_MXFP4) {
      if (wide) {
        if (g.has_r1)
          hipLaunchKernelGGL((k_gemm_ws_dw<F, true, 3, L, 4>), dim3(grid), dim3(64 * (4 + L)), 0, s, g, u_tab, v_tab,
                             mpad, npad, ord);
        else
          hipLaunchKernelGGL((k_gemm_ws_dw<F, false, 3, L, 4>), dim3(grid), dim3(64 * (4 + L)), 0, s, g, u_tab, v_tab,
                             mpad, npad, ord);
        return;
      }
    }
    if (g.has_r1)
      hipLaunchKernelGGL((k_gemm_ws_dw<F, true, S, L>), dim3(grid), dim3(64 * (4 + L)), 0, s, g, u_tab, v_tab, mpad,
                         npad, ord);
    else
      hipLaunchKernelGGL((k_gemm_ws_dw<F, false, S, L>), dim3(grid), dim3(64 * (4 + L)), 0, s, g, u_tab, v_tab, mpad,
                         npad, ord);
    return;
  }
  if constexpr (F == AVERIS_MXFP4) {
    if (cfg == KCFG_WSG) {  // grouped forward / input gradient
      constexpr int S = kWsStages, L = kWsLoaders;
      if (g.mu_codes) hipLaunchKernelGGL((k_gemm_ws_g<F, true, S, L>), dim3(grid), dim3(64 * (4 + L)), 0, s, g);
      else hipLaunchKernelGGL((k_gemm_ws_g<F, false, S, L>), dim3(grid), dim3(64 * (4 + L)), 0, s, g);
      return;
    }
    if (cfg == KCFG_WSGW) {  // the same on 256 x 128 tiles: a 3-stage ring
      constexpr int L = kWsLoaders;
      if (g.mu_codes) hipLaunchKernelGGL((k_gemm_ws_g<F, true, 3, L, 4>), dim3(grid), dim3(64 * (4 + L)), 0, s, g);
      else hipLaunchKernelGGL((k_gemm_ws_g<F, false, 3, L, 4>), dim3(grid), dim3(64 * (4 + L)), 0, s, g);
      return;
    }
    if (cfg == KCFG_WSW) {  // 256 x 128 tiles: a 3-stage ring of 51 KB stages
      constexpr int L = kWsLoaders;
      if (stats) {
        if (mu) hipLaunchKernelGGL((k_gemm_ws<F, true, false, 3, L, 4, true>), dim3(grid), dim3(64 * (4 + L)), 0, s, g);
        else hipLaunchKernelGGL((k_gemm_ws<F, false, false, 3, L, 4, true>), dim3(grid), dim3(64 * (4 + L)), 0, s, g);
        return;
      }
      if (mu) hipLaunchKernelGGL((k_gemm_ws<F, true, false, 3, L, 4>), dim3(grid), dim3(64 * (4 + L)), 0, s, g);
      else hipLaunchKernelGGL((k_gemm_ws<F, false, false, 3, L, 4>), dim3(grid), dim3(64 * (4 + L)), 0, s, g);
      return;
    }
    if (cfg == KCFG_WS) {
      constexpr int S = kWsStages, L = kWsLoaders;
      if (stats) {
        if (mu) hipLaunchKernelGGL((k_gemm_ws<F, true, false, S, L, 2, true>), dim3(grid), dim3(64 * (4 + L)), 0, s, g);
        else hipLaunchKernelGGL((k_gemm_ws<F, false, false, S, L, 2, true>), dim3(grid), dim3(64 * (4 + L)), 0, s, g);
        return;
      }
      if (mu) hipLaunchKernelGGL((k_gemm_ws<F, true, false, S, L>), dim3(grid), dim3(64 * (4 + L)), 0, s, g);
      else if (g.has_r1 && g.splits == 1)
        hipLaunchKernelGGL((k_gemm_ws<F, false, true, S, L>), dim3(grid), dim3(64 * (4 + L)), 0, s, g);
      else hipLaunchKernelGGL((k_gemm_ws<F, false, false, S, L>), dim3(grid), dim3(64 * (4 + L)), 0, s, g);
      return;
    }
  }
  if constexpr (F == AVERIS_MXFP4) {
    if (mu) {
      if (cfg == KCFG_LONG) hipLaunchKernelGGL((k_gemm<F, 2, 2, 2, 2, 3, 0, true>), dim3(grid), dim3(256), 0, s, g);
      else hipLaunchKernelGGL((k_gemm<F, 2, 2, 2, 2, 2, 0, true>), dim3(grid), dim3(256), 0, s, g);
      return;
    }
  }
  if constexpr (F == AVERIS_NVFP4) {
    if (stats && cfg == KCFG_SHORT) {
      hipLaunchKernelGGL((k_gemm<F, 2, 2, 2, 2, 2, 0, false, true>), dim3(grid), dim3(256), 0, s, g);
      return;
    }
  }
  if (cfg == KCFG_SHORT) hipLaunchKernelGGL((k_gemm<F, 2, 2, 2, 2, 2>), dim3(grid), dim3(256), 0, s, g);
  else if (cfg == KCFG_LONG96) hipLaunchKernelGGL((k_gemm<F, 4, 1, 1, 3, 3>), dim3(grid), dim3(256), 0, s, g);
  else hipLaunchKernelGGL((k_gemm<F, 2, 2, 2, 2, 3>), dim3(grid), dim3(256), 0, s, g);
}
// Workgroups resident per CU: two for the two-stage configuration, one for the three-stage one
// (105 KB of LDS) and for the warp-specialized one (a 4 x 35 KB ring).
static int resident_per_cu(int cfg) { return cfg == KCFG_SHORT ? 2 : 1; }
static int cu_count() {
  static int cached[64] = {};  // per device id
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cached[dev] = n;
  return n;
}

hipError_t gemm_launch(const GemmPlan& p) {
  const averis_qtensor& A = *p.a;
  const averis_qtensor& B = *p.b;
  const int fmt = A.fmt;
  const int64_t E = p.grouped ? p.E : 1;
  // per-group GEMM sizes: rows of A (grouped forward: the largest group), rows of B, padded K
  int64_t M = A.outer, N = B.outer, K = A.k_pad;
  int64_t total_tiles_m = 0;
  if (p.grouped == 1) {
    N = B.outer / E;
    M = 0;
    for (int64_t e = 0; e < E; ++e) M = std::max<int64_t>(M, p.h_offsets[e + 1] - p.h_offsets[e]);
  } else if (p.grouped == 2) {
    K = 0;
    for (int64_t e = 0; e < E; ++e) K = std::max<int64_t>(K, round_up(p.h_offsets[e + 1] - p.h_offsets[e], kBKE));
  }
  uint8_t* ws = reinterpret_cast<uint8_t*>(p.ws);
  float* bias = reinterpret_cast<float*>(ws + 256);
  float* partials = reinterpret_cast<float*>(ws + partials_offset(N, E));

  GemmArgs g{};
  g.a_codes = A.codes; g.a_scales = A.scales; g.lda_b = A.k_pad / 2;
  g.b_codes = B.codes; g.b_scales = B.scales; g.ldb_b = B.k_pad / 2;
  g.a_ts = A.tensor_scale; g.b_ts = B.tensor_scale;
  g.M = M; g.N = N; g.K = K;
  g.offsets = p.d_offsets; g.E = (int)E; g.grouped = p.grouped;
  // mean term inside the GEMM: MXFP4 while the mean row fits the tile's LDS copy (see below)
  const bool mu_row_fits = p.mu && fmt == AVERIS_MXFP4 && K <= kMuMaxK;
  int cfg = p.grouped == 2 ? KCFG_LONG : pick_cfg(K);  // grouped dW: long, varying K
  // the warp-specialized kernel: MXFP4 dense launches with K > 0 split into equal K chunks (every
  // (tile, split) unit then has the same nonzero number of K-steps), no accumulation and no bias
  // vector
  const bool ws_ok = fmt == AVERIS_MXFP4 && !p.grouped && !p.accumulate && (!p.mu || mu_row_fits) && K > 0 &&
                     ceil_div(K, (int64_t)kBKE) % p.splits == 0;
  if (cfg == KCFG_WS && !ws_ok) cfg = KCFG_SHORT;
  // grouped weight gradient: the warp-specialized form with per-group K (NVFP4 too: measured 1.5x
  // faster over the MoE step than the three-stage kernel's per-tile K loop)
  if (p.grouped == 2 && !p.accumulate && !p.mu && K > 0 && K < (int64_t(1) << 30) &&
      E <= kDwMaxGroups)
    cfg = kDwWide && fmt == AVERIS_MXFP4 && E <= kDwMaxGroupsWide ? KCFG_WSDWW : KCFG_WSDW;  // (group lengths in the LDS table are int)
  // grouped forward / input gradient, MXFP4: the warp-specialized form with the group's mean
  // K-step in every stage (group offsets in the LDS table are int)
  if (p.grouped == 1 && fmt == AVERIS_MXFP4 && !p.accumulate && K > 0 && E <= kWsgMaxGroups &&
      p.h_offsets[E] < (int64_t(1) << 31))
    cfg = KCFG_WSG;
  if (kWsLongK && cfg == KCFG_LONG && ws_ok) cfg = KCFG_WS;
  if (kWsWide && cfg == KCFG_WS && K < 4096 && !p.mu_u &&
      ceil_div(M, (int64_t)256) * ceil_div(N, (int64_t)128) * p.splits >= cu_count())
    cfg = KCFG_WSW;
  if (cfg == KCFG_LONG && !p.grouped && !p.mu && p.splits == 1 && N % 96 == 0) {
    // fuller last round of the one-per-CU grid with 128 x 96 tiles?
    const int64_t cus = cu_count();
    auto fill = [cus](int64_t t) { return (double)t / (double)(cus * ceil_div(t, cus)); };
    const int64_t t128 = ceil_div(M, (int64_t)128) * ceil_div(N, (int64_t)128), t96 = ceil_div(M, (int64_t)128) * (N / 96);
    if (fill(t96) > fill(t128) + 0.05) cfg = KCFG_LONG96;
  }
  // (the grouped warp-specialized kernel carries each K-step of the mean in its stages: any K)
  if (cfg == KCFG_WSG && kWsgWide) cfg = KCFG_WSGW;
  const bool mu_in = mu_row_fits || (p.mu && (cfg == KCFG_WSG || cfg == KCFG_WSGW));
  const TileCfg tc = tile_of(cfg);
  g.tiles_m = (int)ceil_div(M, tc.bm); g.tiles_n = (int)ceil_div(N, tc.bn);
  if (p.grouped == 1)
    for (int64_t e = 0; e < E; ++e) total_tiles_m += ceil_div(p.h_offsets[e + 1] - p.h_offsets[e], tc.bm);
  {
    // Group height: the tiles an XCD runs at once (one workgroup per CU) form a gm x (R / gm)
    // block; its A and B rows, re-read by the XCD's next round, should stay in that XCD's L2
    // while the outputs stream through it.  The block's operand bytes, gm BM + (R / gm) BN per
    // K-step, are least at gm ~ sqrt(R BN / BM); rounded down to a power of two.  (Measured on
    // the layer's GEMMs against the square-block choice: 2x less fetched beyond L2 for the
    // forward GEMMs, 4 % less GEMM time over the layer.)
    const int64_t tiles = p.grouped == 1 ? total_tiles_m * g.tiles_n : (int64_t)g.tiles_m * g.tiles_n * p.splits * E;
    const int64_t per_round = std::min<int64_t>(ceil_div(tiles, 8), (int64_t)resident_per_cu(cfg) * cu_count() / 8);
    const double best = std::sqrt((double)per_round * tc.bn / tc.bm);
    int gm = 1;
    while (gm * 2 <= best && gm * 2 <= g.tiles_m) gm *= 2;
    g.group_m = gm;
  }
  g.accumulate = p.accumulate;
  g.splits = p.grouped ? 1 : p.splits;
  // column statistics of the output: sums in the epilogue of the warp-specialized MXFP4 kernels
  // and of the two-stage NVFP4 kernel on single-split dense launches; otherwise (and whenever
  // minima and maxima are wanted: three reductions in the epilogue spill the two-stage kernel)
  // a pass over the stored output after the GEMM
  const bool st_fused = p.stats && !p.stats->min && !p.grouped && g.splits == 1 && !p.accumulate &&
                        ((fmt == AVERIS_MXFP4 && (cfg == KCFG_WS || cfg == KCFG_WSW)) ||
                         (fmt == AVERIS_NVFP4 && cfg == KCFG_SHORT));
  if (p.stats) {
    p.stats->part_rows = st_fused ? (cfg == KCFG_WSW ? 128 : 64) : colparts_rows();
    if (st_fused) g.st_sum = p.stats->sum;
  }
  if (M == 0 || N == 0 || E == 0) return hipSuccess;

  // mean term: MXFP4 computes it inside the GEMM (one scaled MFMA more per four) while the mean
  // row fits the tile's LDS copy.  Otherwise, and for NVFP4 (whose f16 MFMAs on dequantized
  // fragments would need four more per sixteen, measured 12 % slower), a GEMV writes the
  // workspace's bias vector, added in the epilogue.
  if (mu_in) {
    g.mu_codes = p.mu->codes; g.mu_scales = p.mu->scales; g.mu_ts = p.mu->tensor_scale; g.mu_row = 0;
  } else if (p.mu) {
    const averis_qtensor& U = *p.mu;
    const dim3 blocks((unsigned)ceil_div(N, 4), (unsigned)E);
    if (fmt == AVERIS_MXFP4)
      hipLaunchKernelGGL(k_gemv_mean<AVERIS_MXFP4>, blocks, dim3(256), 0, p.stream, U.codes, U.scales, U.tensor_scale,
                         B.codes, B.scales, g.ldb_b, B.tensor_scale, N, B.k_pad, bias);
    else
      hipLaunchKernelGGL(k_gemv_mean<AVERIS_NVFP4>, blocks, dim3(256), 0, p.stream, U.codes, U.scales, U.tensor_scale,
                         B.codes, B.scales, g.ldb_b, B.tensor_scale, N, B.k_pad, bias);
    g.bias = bias;
  }
  if (p.mu_u) {
    // rank-one term: the kernels dequantize the means in place (undoing the rotation if any)
    const averis_qtensor& Qu = *p.mu_u;
    const averis_qtensor& Qv = *p.mu_v;
    g.has_r1 = 1;
    g.r1 = p.r1;
    g.r1_row = 0;
    g.ru = MeanVec{Qu.codes, Qu.scales, Qu.tensor_scale, Qu.k_pad, (Qu.flags & AVERIS_HADAMARD16) ? 1 : 0};
    g.rv = MeanVec{Qv.codes, Qv.scales, Qv.tensor_scale, Qv.k_pad, (Qv.flags & AVERIS_HADAMARD16) ? 1 : 0};
  }
  const int64_t ksteps = ceil_div(K, kBKE);
  g.k_chunk = ceil_div(ksteps, g.splits) * kBKE;
  if (g.splits > 1) {
    g.c = partials; g.ldc = N; g.c_bf16 = 0;
  } else {
    g.c = p.c; g.ldc = p.ldc; g.c_bf16 = p.c_bf16;
  }
  const int64_t work = p.grouped == 1 ? total_tiles_m * g.tiles_n : (int64_t)g.tiles_m * g.tiles_n * g.splits * E;
  if (work == 0) return hipGetLastError();
  // one resident round of workgroups, each looping over its tiles
  g.n_work = (int)work;
  const int64_t grid = std::min<int64_t>(work, (int64_t)resident_per_cu(cfg) * cu_count());
  if (fmt == AVERIS_MXFP4) launch_cfg<AVERIS_MXFP4>(cfg, mu_in, g, (unsigned)grid, p.stream, p.ws, p.h_offsets, st_fused);
  else launch_cfg<AVERIS_NVFP4>(cfg, mu_in, g, (unsigned)grid, p.stream, p.ws, p.h_offsets, st_fused);
  if (g.splits > 1) {
    const unsigned blocks = (unsigned)ceil_div(M * (N / 4), 256);
    if (fmt == AVERIS_MXFP4)
      hipLaunchKernelGGL(k_splitk_reduce<AVERIS_MXFP4>, dim3(blocks), dim3(256), 0, p.stream, partials, g.splits, g, p.c,
                         p.ldc, p.c_bf16);
    else
      hipLaunchKernelGGL(k_splitk_reduce<AVERIS_NVFP4>, dim3(blocks), dim3(256), 0, p.stream, partials, g.splits, g, p.c,
                         p.ldc, p.c_bf16);
  }
  if (p.stats && !st_fused)
    colparts_launch(p.c, p.c_bf16 ? AVERIS_BF16 : AVERIS_F32, M, N, p.ldc, p.stats->sum, p.stats->min, p.stats->max,
                    p.stream);
  return hipGetLastError();
}

}  // namespace av

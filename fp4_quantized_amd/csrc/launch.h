// Internal launch plans shared by the C ABI layer and the kernel files.
#pragma once

#include "common.h"

namespace av {

struct SplitQuantPlan {
  const void* x; int xdt; int64_t rows, cols, ldx;
  int fmt; bool split, h16, mean_given;
  float* mean;
  const averis_qtensor *q_row, *q_col, *q_mean;
  void* ws;
  hipStream_t stream;
  // grouped (MoE) operands: E > 0 groups of input rows [offsets[e], offsets[e+1]); device
  // offsets for the kernels, a host copy for grid sizing
  const int64_t* d_offsets; const int64_t* h_offsets; int64_t E;
  // stochastic rounding of the E2M1 codes with this Philox key (dense launches only)
  bool sr; uint64_t seed;
  bool check;  // CHECK_FINITE: status bits into workspace word 0
  // column partials from X's producer (dense SPLIT): st_parts rows of [cols] fp32 sums, and
  // minima / maxima or null; replace the statistics pass over X
  const float* st_sum = nullptr; const float* st_min = nullptr; const float* st_max = nullptr;
  int64_t st_parts = 0;
};
// Column partials of an output that its GEMM could not take in the epilogue: rows of
// colparts_rows() rows each, fp32 sums (and minima / maxima when mn is set), [part][N].
int64_t colparts_rows();
void colparts_launch(const void* c, int cdt, int64_t M, int64_t N, int64_t ldc, float* sum, float* mn, float* mx,
                     hipStream_t s);
size_t split_quant_ws_bytes(int64_t rows, int64_t cols);
size_t split_quant_grouped_ws_bytes(int64_t rows, int64_t cols, int64_t E);
hipError_t split_quant_launch(const SplitQuantPlan& p);
// Batched form: n <= batch_max() dense plans with one input type, format and flags (no
// stochastic rounding, producer statistics or CHECK_FINITE), each with its own workspace.
int batch_max();
hipError_t split_quant_batch_launch(const SplitQuantPlan* ps, int n);

struct GemmPlan {
  const averis_qtensor* a; const averis_qtensor* b;   // C = A B^T, both K-inner
  void* c; int64_t ldc; int c_bf16;
  const averis_qtensor* mu;                            // broadcast-row mean term (fwd / dX), or null
  const averis_qtensor* mu_u; const averis_qtensor* mu_v; float r1;  // rank-one term (dW), or null
  int accumulate;
  int splits;
  // grouped (MoE) launches: 1 = token rows grouped (forward / input gradient), 2 = token axis
  // grouped (weight gradient); offsets [E + 1] on the device and a host copy for sizing
  int grouped;
  const int64_t* d_offsets; const int64_t* h_offsets; int64_t E;
  void* ws;
  hipStream_t stream;
  // column statistics of the stored output (dense launches): fp32 partials [part][N] of rows
  // [part * part_rows, ...), sums, and minima / maxima when min is set; part_rows is written
  struct Stats { float* sum; float* min; float* max; int64_t part_rows; }* stats = nullptr;
};
// Producers with column statistics (producers.hip): op 0 RMSNorm of x with weight w, op 1
// SwiGLU of gate x and up u; y written as dt; statistics per producer_part_rows() rows when
// st_sum is set.
int64_t producer_part_rows();
hipError_t producer_launch(int op, int dt, const void* x, const void* u, int64_t rows, int64_t cols, int64_t ldx,
                           const float* w, float eps, void* y, int64_t ldy, float* st_sum, float* st_min,
                           float* st_max, hipStream_t s);

int choose_splits(int fmt, int64_t M, int64_t N, int64_t K);
size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, int splits);
size_t gemm_grouped_ws_bytes(int64_t M, int64_t N, int64_t E);
size_t gemm_grouped_dw_ws_bytes(int64_t M, int64_t N, int64_t E);
hipError_t gemm_launch(const GemmPlan& p);

}  // namespace av

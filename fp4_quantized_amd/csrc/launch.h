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
};
size_t split_quant_ws_bytes(int64_t rows, int64_t cols);
size_t split_quant_grouped_ws_bytes(int64_t rows, int64_t cols, int64_t E);
hipError_t split_quant_launch(const SplitQuantPlan& p);

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
};
int choose_splits(int fmt, int64_t M, int64_t N, int64_t K);
size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, int splits);
size_t gemm_grouped_ws_bytes(int64_t M, int64_t N, int64_t E);
hipError_t gemm_launch(const GemmPlan& p);

}  // namespace av

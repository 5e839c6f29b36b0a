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
};
size_t split_quant_ws_bytes(int64_t rows, int64_t cols);
hipError_t split_quant_launch(const SplitQuantPlan& p);

struct GemmPlan {
  const averis_qtensor* a; const averis_qtensor* b;   // C = A B^T, both K-inner
  void* c; int64_t ldc; int c_bf16;
  const averis_qtensor* mu;                            // broadcast-row mean term (fwd / dX), or null
  const averis_qtensor* mu_u; const averis_qtensor* mu_v; float r1;  // rank-one term (dW), or null
  int accumulate;
  int splits;
  void* ws;
  hipStream_t stream;
};
int choose_splits(int fmt, int64_t M, int64_t N, int64_t K);
size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, int splits);
hipError_t gemm_launch(const GemmPlan& p);

}  // namespace av

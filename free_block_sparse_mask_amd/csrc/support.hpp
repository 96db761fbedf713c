// Internal declarations of the support code outside the attention path:
// token orders and the L1 sums of the hyper-parameter search.
#pragma once

#include "common.hpp"

namespace sparge {

// host-side raster / time-fastest orders (the Hilbert order is in common.hpp)
void simple_order(int T, int H, int W, int order, int32_t* perm, int32_t* inv);

// relative L1 sums: deterministic two-kernel float64 reduction
constexpr int kL1Blocks = 1024;
struct L1Args {
  const void* o;
  const void* r;
  int64_t o_sb, o_sh, o_sn;   // element strides
  int64_t r_sb, r_sh, r_sn;
  int64_t B, H, N, d;
  int dtype_o, dtype_r;
  double* partial;            // [kL1Blocks][2]
  double* out;                // [2]
};
hipError_t launch_l1(const L1Args& a, hipStream_t st);

}  // namespace sparge

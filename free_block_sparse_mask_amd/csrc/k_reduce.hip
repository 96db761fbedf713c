// Relative L1 sums for the hyper-parameter search.
//
// Pages: [Review] "SpargeAttn: Accurate and Training-free Sparse Attention
// Accelerating Any Model Inference" (xllm-io paper-review blog), the
// hyper-parameter determination paragraph: L1 = sum|O - O'| / sum|O|.
//
// Two kernels make the float64 sums independent of timing: l1_partial gives
// every workgroup a fixed set of rows (grid stride over rows, one wavefront
// per row, lanes over d) and reduces its lanes through LDS in a fixed tree;
// l1_final sums the kL1Blocks partials in a fixed order.  The inputs are
// read once (HBM-bound; the search calls it a few dozen times on
// calibration-sized tensors).
#include "support.hpp"

namespace sparge {

namespace {

__device__ __forceinline__ double load_elem(const void* base, int64_t off, int dtype) {
  if (dtype == SPARGE_F32) return (double)static_cast<const float*>(base)[off];
  const unsigned short bits = static_cast<const unsigned short*>(base)[off];
  if (dtype == SPARGE_BF16) return (double)__uint_as_float((unsigned int)bits << 16);
  return (double)__builtin_bit_cast(_Float16, bits);
}

// sum of v over the 256 threads of the workgroup, in a fixed order
__device__ __forceinline__ void block_sum2(double (&red)[2][256], double a, double b, int tid) {
  red[0][tid] = a;
  red[1][tid] = b;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) {
      red[0][tid] += red[0][tid + s];
      red[1][tid] += red[1][tid + s];
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void l1_partial(L1Args a) {
  __shared__ double red[2][256];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t rows = a.B * a.H * a.N;
  double sd = 0.0, sr = 0.0;
  for (int64_t row = (int64_t)blockIdx.x * 4 + wave; row < rows; row += (int64_t)kL1Blocks * 4) {
    const int64_t n = row % a.N, bh = row / a.N;
    const int64_t h = bh % a.H, b = bh / a.H;
    const int64_t oo = b * a.o_sb + h * a.o_sh + n * a.o_sn;
    const int64_t ro = b * a.r_sb + h * a.r_sh + n * a.r_sn;
    for (int64_t c = lane; c < a.d; c += 64) {
      const double x = load_elem(a.o, oo + c, a.dtype_o);
      const double r = load_elem(a.r, ro + c, a.dtype_r);
      sd += fabs(x - r);
      sr += fabs(r);
    }
  }
  block_sum2(red, sd, sr, tid);
  if (tid == 0) {
    a.partial[2 * blockIdx.x] = red[0][0];
    a.partial[2 * blockIdx.x + 1] = red[1][0];
  }
}

__global__ __launch_bounds__(256) void l1_final(L1Args a) {
  __shared__ double red[2][256];
  const int tid = threadIdx.x;
  double sd = 0.0, sr = 0.0;
  for (int p = tid; p < kL1Blocks; p += 256) {
    sd += a.partial[2 * p];
    sr += a.partial[2 * p + 1];
  }
  block_sum2(red, sd, sr, tid);
  if (tid == 0) {
    a.out[0] = red[0][0];
    a.out[1] = red[1][0];
  }
}

}  // namespace

hipError_t launch_l1(const L1Args& a, hipStream_t st) {
  hipLaunchKernelGGL(l1_partial, dim3(kL1Blocks), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(l1_final, dim3(1), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace sparge

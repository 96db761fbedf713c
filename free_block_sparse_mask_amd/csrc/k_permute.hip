// Token gather / scatter along N for the 3D Hilbert-curve order of visual
// tokens on gfx950.
//
// Pages: [Review] "SpargeAttn: Accurate and Training-free Sparse Attention
// Accelerating Any Model Inference" (xllm-io paper-review blog), "HilbertCurve
// Permutation": Q, K, V in T x H x W x d are reordered into L x d along a
// Hilbert curve so that neighbouring tokens share a block; [Rebuttal] reply
// "Weaknesses3.2": attention itself is permutation invariant, so the output
// is mapped back with the inverse order.
//
// A pure HBM copy: each lane moves 16 bytes; the lanes of one token row are
// consecutive, so every row read and write is one contiguous segment.  The
// permutation index is read once per row; an index outside [0, N) (a stale
// or malformed order) moves nothing, so it cannot reach outside x or y.
#include "common.hpp"

namespace sparge {

namespace {

__global__ __launch_bounds__(kThreads) void permute_rows(PermuteArgs a, int lanes_per_row,
                                                         long long total_rows) {
  const long long g = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long row = g / lanes_per_row;
  const int part = (int)(g % lanes_per_row);
  if (row >= total_rows) return;
  const int p = (int)(row % a.N);
  const long long bh = row / a.N;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int q = a.perm[p];
  if ((unsigned)q >= (unsigned)a.N) return;
  const int src = a.inverse ? p : q;
  const int dst = a.inverse ? q : p;
  const unsigned char* xs = static_cast<const unsigned char*>(a.x) + b * a.x_sb + h * a.x_sh + src * a.x_sn;
  unsigned char* yd = static_cast<unsigned char*>(a.y) + b * a.y_sb + h * a.y_sh + dst * a.y_sn;
  *reinterpret_cast<u32x4*>(yd + 16 * part) = *reinterpret_cast<const u32x4*>(xs + 16 * part);
}

}  // namespace

hipError_t launch_permute(const PermuteArgs& a, hipStream_t st) {
  const int lanes = a.row_bytes / 16;
  const long long rows = (long long)a.B * a.H * a.N;
  const long long threads = rows * lanes;
  hipLaunchKernelGGL(permute_rows, dim3((unsigned)ceil_div(threads, kThreads)), dim3(kThreads), 0, st, a,
                     lanes, rows);
  return hipGetLastError();
}

}  // namespace sparge

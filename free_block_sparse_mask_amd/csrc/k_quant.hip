// int8 per-block quantisation of Q and K on gfx950 (SageAttention-style, as
// integrated by SpargeAttn).
//
// Pages: [Review] "SpargeAttn: Accurate and Training-free Sparse Attention
// Accelerating Any Model Inference" (xllm-io paper-review blog), "Algorithm 1"
// step 2 (Q^_i, K^_j, delta_Q, delta_K = Quant(Q_i, K_j)) and the components
// table (per-block quantisation, FP16 -> INT8).
//
// All arithmetic that decides a code is float64: the K mean, K - mean, the
// block maximum, x / delta and the rounding (ties to even), so every code is
// decided exactly as the float64 definition decides it (a product with
// 1 / delta stands in for the division wherever it provably rounds alike).
// HBM-bound kernels:
//   kmean_partial  column sums of K over chunks of 1024 tokens
//   kmean_final    mean over the chunks, in chunk order (deterministic)
//   quant_blocks   one workgroup per Q or K block: max |x|, then the codes
#include "common.hpp"

namespace sparge {

namespace {

__device__ __forceinline__ double widen16(unsigned short u, bool bf16) {
  if (bf16) return (double)__uint_as_float((unsigned int)u << 16);
  return (double)(float)__builtin_bit_cast(_Float16, u);
}

template <int D>
__global__ __launch_bounds__(kThreads) void kmean_partial(QuantArgs a, int nchunks) {
  constexpr int DCH = D / 8;
  constexpr int SLOTS = kThreads / DCH;
  __shared__ double red[SLOTS][D + 1];
  const int chunk = blockIdx.x % nchunks;
  const int bh = blockIdx.x / nchunks;
  const int b = bh / a.Hkv, h = bh % a.Hkv;
  const int tid = threadIdx.x, c = tid % DCH, slot = tid / DCH;
  const unsigned short* base = static_cast<const unsigned short*>(a.k) + b * a.k_sb + h * a.k_sh;
  const int r0 = chunk * kQuantChunkRows, r1 = min(a.N, r0 + kQuantChunkRows);
  const bool bf = a.bf16 != 0;
  double s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.0;
  // four rows requested before their sums (the same order of additions)
  constexpr int U = 4;
  for (int rb = r0 + slot; rb < r1; rb += U * SLOTS) {
    u32x4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = rb + u * SLOTS;
      w[u] = r < r1 ? *reinterpret_cast<const u32x4*>(base + (long long)r * a.k_sn + 8 * c) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (rb + u * SLOTS >= r1) break;
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += widen16((unsigned short)(w[u][e >> 1] >> ((e & 1) * 16)), bf);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[slot][8 * c + e] = s[e];
  __syncthreads();
  if (tid < D) {
    double t = 0.0;
    for (int sl = 0; sl < SLOTS; ++sl) t += red[sl][tid];
    a.ws.ksum_part[((long long)bh * nchunks + chunk) * D + tid] = t;
  }
}

__global__ void kmean_final(QuantArgs a, int nchunks) {
  const int bh = blockIdx.x;
  const int c = threadIdx.x;
  if (c >= a.d) return;
  double t = 0.0;
  // the partial sums are added in chunk order; unrolling only lets their
  // loads be in flight together
#pragma unroll 16
  for (int k = 0; k < nchunks; ++k) t += a.ws.ksum_part[((long long)bh * nchunks + k) * a.d + c];
  a.ws.kmean[(long long)bh * a.d + c] = t / (double)a.N;
}

template <int D>
__global__ __launch_bounds__(kThreads) void quant_blocks(QuantArgs a) {
  constexpr int DCH = D / 8;
  constexpr int SLOTS = kThreads / DCH;
  __shared__ double red[kThreads / 64];
  __shared__ double mu[D];
  const long long nq = (long long)a.B * a.H * a.Tm;
  long long blk = blockIdx.x;
  const bool is_q = blk < nq;
  int b, h, t, brows;
  const unsigned short* base;
  long long sn;
  int8_t* out;
  if (is_q) {
    t = (int)(blk % a.Tm);
    const long long bh = blk / a.Tm;
    b = (int)(bh / a.H);
    h = (int)(bh % a.H);
    brows = kBq;
    base = static_cast<const unsigned short*>(a.q) + b * a.q_sb + h * a.q_sh;
    sn = a.q_sn;
    out = a.q8 + bh * (long long)a.N * D;
  } else {
    blk -= nq;
    t = (int)(blk % a.Tn);
    const long long bh = blk / a.Tn;
    b = (int)(bh / a.Hkv);
    h = (int)(bh % a.Hkv);
    brows = kBk;
    base = static_cast<const unsigned short*>(a.k) + b * a.k_sb + h * a.k_sh;
    sn = a.k_sn;
    out = a.k8 + bh * (long long)a.N * D;
  }
  const int tid = threadIdx.x, c = tid % DCH, slot = tid / DCH;
  if (tid < D) mu[tid] = is_q ? 0.0 : a.ws.kmean[((long long)b * a.Hkv + h) * D + tid];
  __syncthreads();
  const int r0 = t * brows;
  const int nrows = min(a.N, r0 + brows) - r0;
  const bool bf = a.bf16 != 0;

  // the thread's rows, all requested at once and read from HBM once for
  // both the maximum and the codes
  constexpr int RPT = kBq / SLOTS;           // rows per thread (Q blocks; K blocks use half)
  u32x4 wr[RPT];
#pragma unroll
  for (int it = 0; it < RPT; ++it) {
    const int r = slot + it * SLOTS;
    wr[it] = r < nrows ? *reinterpret_cast<const u32x4*>(base + (long long)(r0 + r) * sn + 8 * c)
                       : u32x4{0, 0, 0, 0};
  }
  double amax = 0.0;
#pragma unroll
  for (int it = 0; it < RPT; ++it) {
    if (slot + it * SLOTS >= nrows) break;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double x = widen16((unsigned short)(wr[it][e >> 1] >> ((e & 1) * 16)), bf) - mu[8 * c + e];
      amax = fmax(amax, fabs(x));
    }
  }
  // the maximum is the same in any order: within each wavefront, then over
  // the four
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmax(amax, __shfl_xor(amax, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  double m = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) m = fmax(m, red[w]);
  const double delta = m > 0.0 ? m / 127.0 : 1.0;
  // The code is rint of the rounded quotient x / delta, and |x / delta| <= 127.
  // y = x * (1 / delta) lies within 2^-44 of that quotient (two roundings of
  // relative size 2^-53 on a value below 2^7, plus the quotient's own), so
  // both round to the same integer unless y is within that distance of a
  // half-integer; inside a guard band of 2^-40 the division itself decides.
  const double rdelta = 1.0 / delta;
#pragma unroll
  for (int it = 0; it < RPT; ++it) {
    const int r = slot + it * SLOTS;
    if (r >= nrows) break;
    unsigned int packed[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double x = widen16((unsigned short)(wr[it][e >> 1] >> ((e & 1) * 16)), bf) - mu[8 * c + e];
      const double y = x * rdelta;
      double qv = rint(y);
      if (fabs(fabs(y - trunc(y)) - 0.5) < 0x1p-40) qv = rint(x / delta);
      qv = fmin(127.0, fmax(-127.0, qv));
      const unsigned int byte = (unsigned int)(unsigned char)(signed char)(int)qv;
      packed[e >> 2] |= byte << ((e & 3) * 8);
    }
    *reinterpret_cast<u32x2*>(out + (long long)(r0 + r) * D + 8 * c) = u32x2{packed[0], packed[1]};
  }
  if (tid == 0) {
    if (is_q)
      a.q_scale[((long long)b * a.H + h) * a.Tm + t] = (float)delta;
    else
      a.k_scale[((long long)b * a.Hkv + h) * a.Tn + t] = (float)delta;
  }
}

}  // namespace

hipError_t launch_quant(const QuantArgs& a, hipStream_t st) {
  const int nchunks = (int)ceil_div(a.N, kQuantChunkRows);
  const unsigned pblocks = (unsigned)((long long)a.B * a.Hkv * nchunks);
  if (a.d == 64)
    hipLaunchKernelGGL(kmean_partial<64>, dim3(pblocks), dim3(kThreads), 0, st, a, nchunks);
  else
    hipLaunchKernelGGL(kmean_partial<128>, dim3(pblocks), dim3(kThreads), 0, st, a, nchunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kmean_final, dim3((unsigned)(a.B * a.Hkv)), dim3(128), 0, st, a, nchunks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long qb = (long long)a.B * a.H * a.Tm + (long long)a.B * a.Hkv * a.Tn;
  if (a.d == 64)
    hipLaunchKernelGGL(quant_blocks<64>, dim3((unsigned)qb), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(quant_blocks<128>, dim3((unsigned)qb), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace sparge

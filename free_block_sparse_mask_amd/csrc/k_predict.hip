// Stage 1 of SpargeAttn on gfx950: predict the block mask M_g.
//
// Pages: [Review] "SpargeAttn: Accurate and Training-free Sparse Attention
// Accelerating Any Model Inference" (xllm-io paper-review blog), "Core
// formulas" eqs. (4)-(9) and "Algorithm 1" steps 3-5; [Rebuttal] OpenReview
// author rebuttal, reply "Weaknesses3.1" (CosSim is one mean cosine
// similarity per block) and "Weaknesses1" (only self-similar blocks are
// compressed; the others are always computed).
//
// Every quantity that decides a mask bit (block means, self-similarity, the
// compressed map, its softmax and the TopCdf prefix sums) is computed in
// float64.  Three kernels:
//   pool_cossim   one workgroup per Q or K block: coalesced 16-byte loads,
//                 per-token norms summed over their 16 lanes with DPP moves,
//                 column sums of x and x/|x| combined across lanes and then
//                 the four wavefronts through LDS; s = |mean x/|x||^2.
//   shat_gemm     Shat = qbar kbar^T / sqrt(d) per (batch, head) on 64 x 64
//                 tiles staged through LDS and multiplied on the float64
//                 matrix cores (tiles wholly in the causal future are
//                 skipped).
//   mask_rows     one workgroup per query block row: softmax over the live
//                 selective columns, the TopCdf cut by a radix select over
//                 the probabilities with fixed-point sums (no sort), eq. 9
//                 forcing, then the M_g row and its compacted ascending list
//                 (a fix row skips straight to its list of live tiles).
#include "common.hpp"

namespace sparge {

namespace {

constexpr double kNegInfD = -__builtin_huge_val();

// 1/sqrt(x) for x > 0 in float64: the hardware estimate refined by two
// Newton steps y <- y (3 - x y^2) / 2, each of which squares the relative
// error, so the result is within a few ulp of the rounded reciprocal root.
__device__ __forceinline__ double rsqrt_f64(double x) {
  double y = __builtin_amdgcn_rsq(x);
  y = y * fma(-0.5 * x, y * y, 1.5);
  y = y * fma(-0.5 * x, y * y, 1.5);
  return y;
}

__device__ __forceinline__ double bits_to_double(unsigned short u, bool bf16) {
  if (bf16) return (double)__uint_as_float((unsigned int)u << 16);
  return (double)(float)__builtin_bit_cast(_Float16, u);
}

// Lane exchanges of a double as two 32-bit halves.  dpp_f64<CTRL> reads the
// lane that the DPP control names (0xB1: quad lanes 1,0,3,2; 0x4E: quad lanes
// 2,3,0,1; 0x141: the mirror within each 8 lanes; 0x140: the mirror within
// each 16 lanes).  These run on the vector ALU instead of the LDS crossbar.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(unsigned)u, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(unsigned)(u >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}

// Sum over aligned groups of W lanes (W = 2, 4, 8 or 16), every lane of a
// group left with the same total.  Each step adds the value of a lane in the
// other half of the current group; after the first two steps all lanes of a
// quad agree, so a mirror pairs the same halves as an xor would and the sums
// equal those of an xor butterfly (x ^ 1, x ^ 2, x ^ 4, x ^ 8) bit for bit.
template <int W>
__device__ __forceinline__ double group_sum(double v) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16, "group of 2 to 16 lanes");
  v += dpp_f64<0xB1>(v);
  if constexpr (W >= 4) v += dpp_f64<0x4E>(v);
  if constexpr (W >= 8) v += dpp_f64<0x141>(v);
  if constexpr (W >= 16) v += dpp_f64<0x140>(v);
  return v;
}

// x[l] + x[l ^ 32] in every lane (v_permlane32_swap of both halves)
__device__ __forceinline__ double sum_halves_f64(double x) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const auto lo = __builtin_amdgcn_permlane32_swap((unsigned)u, (unsigned)u, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap((unsigned)(u >> 32), (unsigned)(u >> 32), false, false);
  const double a = __longlong_as_double((long long)(((unsigned long long)hi[0] << 32) | lo[0]));
  const double b = __longlong_as_double((long long)(((unsigned long long)hi[1] << 32) | lo[1]));
  return a + b;
}

constexpr int kWaves = kThreads / 64;

// Workgroup-wide exclusive scan of one int per thread (256 threads): a scan
// within each wavefront, then the wavefront totals through LDS (lds holds at
// least kWaves ints).
__device__ int block_excl_scan_int(int v, int* lds, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(incl, off, 64);
    if (lane >= off) incl += t;
  }
  if (lane == 63) lds[w] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int x = 0; x < kWaves; ++x) {
    const int t = lds[x];
    before += x < w ? t : 0;
    total += t;
  }
  __syncthreads();
  return before + incl - v;
}

// Workgroup reductions of one value per thread (256 threads), all taken as
// the tree x[t] op x[t + off] for off = 128, 64, ..., 1: the two steps across
// wavefronts through LDS, the six within wavefront 0 as an xor butterfly
// (lane t < off meets lane t + off, the same operands in the same order), so
// a floating-point sum is the same number whichever way the tree is walked.
template <typename T, typename Op>
__device__ __forceinline__ T block_reduce(T v, T* lds, Op op) {
  static_assert(kThreads == 256, "the two cross-wavefront steps assume four wavefronts");
  const int tid = threadIdx.x;
  lds[tid] = v;
  __syncthreads();
  if (tid < 64) {
    T x = op(op(lds[tid], lds[tid + 128]), op(lds[tid + 64], lds[tid + 192]));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = op(x, __shfl_xor(x, off, 64));
    if (tid == 0) lds[0] = x;
  }
  __syncthreads();
  const T r = lds[0];
  __syncthreads();
  return r;
}

__device__ double block_reduce_max(double v, double* lds) {
  return block_reduce(v, lds, [](double x, double y) { return fmax(x, y); });
}

__device__ double block_reduce_sum(double v, double* lds) {
  return block_reduce(v, lds, [](double x, double y) { return x + y; });
}

__device__ uint64_t block_reduce_u64(uint64_t v, unsigned long long* lds) {
  return block_reduce((unsigned long long)v, lds,
                      [](unsigned long long x, unsigned long long y) { return x + y; });
}

// ceil(tau * F) exactly, for 0 < tau <= 1 and a 64-bit integer F: tau is
// m * 2^-s with an integer mantissa m < 2^53 (s >= 52 since tau <= 1), so
// the 117-bit product m * F shifted right by s, rounded up, is the value.
// An integer prefix c satisfies c < tau * F exactly when c < ceil(tau * F).
__device__ __forceinline__ uint64_t ceil_tau_times(double tau, uint64_t F) {
  const uint64_t bits = (uint64_t)__double_as_longlong(tau);
  const int ex = (int)((bits >> 52) & 0x7ff);
  uint64_t m = bits & ((1ull << 52) - 1);
  int s = 1074;                                   // subnormal tau: m * 2^-1074
  if (ex != 0) {
    m |= 1ull << 52;
    s = 1075 - ex;
  }
  if (m == 0 || F == 0) return 0;
  if (s >= 117) return 1;                         // 0 < tau * F < 1
  const unsigned __int128 prod = (unsigned __int128)m * F;
  return (uint64_t)((prod + (((unsigned __int128)1 << s) - 1)) >> s);
}

// Writes the M_g row (Tn bytes) and the ascending list of its ones.
// keep(j) must be readable by every thread.
template <typename Keep>
__device__ void write_row(int Tn, Keep keep, uint8_t* mg_row, int32_t* cnt_out, uint16_t* idx_row,
                          int* scan_lds) {
  const int tid = threadIdx.x;
  const int per = (Tn + kThreads - 1) / kThreads;
  const int lo = min(Tn, tid * per), hi = min(Tn, lo + per);
  int mine = 0;
  for (int j = lo; j < hi; ++j) mine += keep(j) ? 1 : 0;
  int total;
  int pos = block_excl_scan_int(mine, scan_lds, total);
  for (int j = lo; j < hi; ++j)
    if (keep(j)) idx_row[pos++] = (uint16_t)j;
  if (mg_row != nullptr)
    for (int j = tid; j < Tn; j += kThreads) mg_row[j] = keep(j) ? 1 : 0;
  if (tid == 0) *cnt_out = total;
}

// ---------------------------------------------------------------------------
// pool_cossim: eqs. (4)-(6)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void pool_cossim(PredictArgs a) {
  constexpr int DCH = D / 8;                 // lanes per token row
  constexpr int SLOTS = kThreads / DCH;      // token rows in flight
  constexpr int NWV = kThreads / 64;         // wavefronts
  __shared__ double red_x[NWV][D];
  __shared__ double red_h[NWV][D];
  __shared__ double red_s[NWV];

  const long long nq = (long long)a.B * a.H * a.Tm;
  long long blk = blockIdx.x;
  const bool is_q = blk < nq;
  int b, h, t, brows;
  const unsigned short* base;
  long long sn;
  if (is_q) {
    t = (int)(blk % a.Tm);
    const long long bh = blk / a.Tm;
    b = (int)(bh / a.H);
    h = (int)(bh % a.H);
    brows = kBq;
    base = static_cast<const unsigned short*>(a.q) + b * a.q_sb + h * a.q_sh;
    sn = a.q_sn;
  } else {
    blk -= nq;
    t = (int)(blk % a.Tn);
    const long long bh = blk / a.Tn;
    b = (int)(bh / a.Hkv);
    h = (int)(bh % a.Hkv);
    brows = kBk;
    base = static_cast<const unsigned short*>(a.k) + b * a.k_sb + h * a.k_sh;
    sn = a.k_sn;
  }
  const int r0 = t * brows;
  const int nrows = min(a.N, r0 + brows) - r0;
  const int tid = threadIdx.x;
  const int c = tid % DCH, slot = tid / DCH;
  const bool bf = a.bf16 != 0;

  // every row this thread reads is requested before any arithmetic, so the
  // block's 16-32 KB are in flight at once (one load per row at a time left
  // the kernel at a third of the HBM bandwidth)
  constexpr int RPT = kBq / SLOTS;           // rows per thread (Q blocks; K blocks use half)
  u32x4 wr[RPT];
#pragma unroll
  for (int it = 0; it < RPT; ++it) {
    const int r = slot + it * SLOTS;
    wr[it] = r < nrows ? *reinterpret_cast<const u32x4*>(base + (long long)(r0 + r) * sn + 8 * c)
                       : u32x4{0, 0, 0, 0};
  }
  double sx[8], sh[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) sx[e] = sh[e] = 0.0;
#pragma unroll
  for (int it = 0; it < RPT; ++it) {
    if (slot + it * SLOTS >= nrows) break;
    const u32x4 w = wr[it];
    double x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = bits_to_double((unsigned short)(w[e >> 1] >> ((e & 1) * 16)), bf);
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
    ss = group_sum<DCH>(ss);
    const double inv = ss > 0.0 ? rsqrt_f64(ss) : 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sx[e] += x[e];
      sh[e] += x[e] * inv;
    }
  }
  // column sums: first over the row slots of a wavefront (lanes that differ
  // in the bits above the DCH lanes of a row), then over the wavefronts
#pragma unroll
  for (int off = DCH; off < 32; off <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sx[e] += __shfl_xor(sx[e], off, 64);
      sh[e] += __shfl_xor(sh[e], off, 64);
    }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    sx[e] = sum_halves_f64(sx[e]);
    sh[e] = sum_halves_f64(sh[e]);
  }
  const int wv = tid >> 6, lane = tid & 63;
  if (lane < DCH) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      red_x[wv][8 * lane + e] = sx[e];
      red_h[wv][8 * lane + e] = sh[e];
    }
  }
  __syncthreads();
  double contrib = 0.0;
  if (tid < D) {
    double tx = 0.0, th = 0.0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      tx += red_x[w][tid];
      th += red_h[w][tid];
    }
    const double mean = tx / nrows;
    const double mh = th / nrows;
    contrib = mh * mh;
    if (is_q)
      a.ws.qbar[(((long long)b * a.H + h) * a.Tm + t) * D + tid] = mean;
    else
      a.ws.kbar[(((long long)b * a.Hkv + h) * a.Tn + t) * D + tid] = mean;
  }
  // s = the sum of the D values of contrib (threads >= D hold 0)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) contrib += __shfl_xor(contrib, off, 64);
  if (lane == 0) red_s[wv] = contrib;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) s += red_s[w];
  if (tid == 0) {
    if (is_q) {
      const long long o = ((long long)b * a.H + h) * a.Tm + t;
      a.ws.sq[o] = s;
      if (a.s_q_out) a.s_q_out[o] = s;
    } else {
      const long long o = ((long long)b * a.Hkv + h) * a.Tn + t;
      a.ws.sk[o] = s;
      if (a.s_k_out) a.s_k_out[o] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// shat_gemm: Shat = qbar kbar^T / sqrt(d) (eq. 7 before the -inf columns)
// ---------------------------------------------------------------------------
constexpr int kGT = 64;     // tile rows (query blocks)
constexpr int kGTJ = 128;   // tile columns (key blocks)
constexpr int kGK = 16;     // d chunk
typedef double f64x4 __attribute__((ext_vector_type(4)));
// Each wavefront owns 32 rows x kGTJ/2 columns of the tile as 2 x NJ blocks of
// the float64 matrix core's 16 x 16 x 4 product.  Operand lane l holds row
// (or column) l % 16 at k = l / 16; accumulator element r of lane l is row
// l / 16 + 4 r, column l % 16.  Two 8-byte LDS reads per lane feed 1024 FMAs
// per wavefront, where a 4 x 4 per-thread FMA tile needed 64 bytes of LDS
// reads per 16 FMAs and waited on LDS bandwidth; the wide tile gives each
// chunk's loads and barriers twice the MFMA work to hide behind.
// three wavefronts per SIMD (144 VGPRs, no spills) against two by default
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3)))
void shat_gemm(PredictArgs a, double inv_sqrt_d) {
  constexpr int NJ = kGTJ / 32;                // 16-column blocks per wavefront
  // k-major tiles: rows padded by 2 doubles so that the transposing stores of
  // 16 consecutive k land in distinct banks
  __shared__ double qt[kGK][kGT + 2];
  __shared__ double kt[kGK][kGTJ + 2];
  const int it = blockIdx.x, jt = blockIdx.y;
  const int bh = blockIdx.z;
  const int b = bh / a.H, h = bh % a.H;
  const int hk = h / (a.H / a.Hkv);
  const int i0 = it * kGT, j0 = jt * kGTJ;
  if (a.causal) {
    const int i_last = min(a.Tm - 1, i0 + kGT - 1);
    const int last_q = min(a.N, (i_last + 1) * kBq) - 1;
    if (j0 * kBk > last_q) return;
  }
  const double* qb = a.ws.qbar + ((long long)b * a.H + h) * a.Tm * a.d;
  const double* kb = a.ws.kbar + ((long long)b * a.Hkv + hk) * a.Tn * a.d;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  const int wr = 32 * (wv >> 1), wc = (kGTJ / 2) * (wv & 1);    // the wavefront's quarter
  const int l16 = lane & 15, l4 = lane >> 4;
  f64x4 acc[2][NJ];
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < NJ; ++y) acc[x][y] = f64x4{0.0, 0.0, 0.0, 0.0};
  // the next d chunk is loaded into registers while this one is used
  constexpr int PQ = kGT * kGK / kThreads, PK = kGTJ * kGK / kThreads;
  double pq[PQ], pk[PK];
  auto load_chunk = [&](int k0) {
#pragma unroll
    for (int u = 0; u < PQ; ++u) {
      const int e = tid + u * kThreads;
      const int gi = i0 + e / kGK;
      pq[u] = gi < a.Tm ? qb[(long long)gi * a.d + k0 + e % kGK] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < PK; ++u) {
      const int e = tid + u * kThreads;
      const int gj = j0 + e / kGK;
      pk[u] = gj < a.Tn ? kb[(long long)gj * a.d + k0 + e % kGK] : 0.0;
    }
  };
  load_chunk(0);
  for (int k0 = 0; k0 < a.d; k0 += kGK) {
#pragma unroll
    for (int u = 0; u < PQ; ++u) {
      const int e = tid + u * kThreads;
      qt[e % kGK][e / kGK] = pq[u];
    }
#pragma unroll
    for (int u = 0; u < PK; ++u) {
      const int e = tid + u * kThreads;
      kt[e % kGK][e / kGK] = pk[u];
    }
    __syncthreads();
    if (k0 + kGK < a.d) load_chunk(k0 + kGK);
#pragma unroll
    for (int ks = 0; ks < kGK; ks += 4) {
      const double qa0 = qt[ks + l4][wr + l16], qa1 = qt[ks + l4][wr + 16 + l16];
#pragma unroll
      for (int y = 0; y < NJ; ++y) {
        const double kby = kt[ks + l4][wc + 16 * y + l16];
        acc[0][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(qa0, kby, acc[0][y], 0, 0, 0);
        acc[1][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(qa1, kby, acc[1][y], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  double* out = a.ws.shat + ((long long)b * a.H + h) * a.Tm * a.Tn;
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int gi = i0 + wr + 16 * x + l4 + 4 * r;
      if (gi >= a.Tm) continue;
#pragma unroll
      for (int y = 0; y < NJ; ++y) {
        const int gj = j0 + wc + 16 * y + l16;
        if (gj < a.Tn) out[(long long)gi * a.Tn + gj] = acc[x][y][r] * inv_sqrt_d;
      }
    }
}

// ---------------------------------------------------------------------------
// mask_rows: eqs. (7)-(9) for one query block row, then its compacted list
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void mask_rows(PredictArgs a, int cap) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  double* pv = reinterpret_cast<double*>(dyn);                        // [cap >= Tn]
  int* pj = reinterpret_cast<int*>(dyn + 8 * (size_t)cap);              // [cap]
  uint8_t* flag = dyn + 12 * (size_t)cap;                             // [Tn]: bit0 fix_k, bit1 kept
  __shared__ double dred[kThreads];
  __shared__ int ired[kThreads];
  __shared__ unsigned long long ured[kThreads];
  __shared__ unsigned int hcnt[256];
  __shared__ unsigned long long hsum[256];
  __shared__ int s_digit;
  __shared__ uint64_t s_above;
  __shared__ uint64_t s_key;
  static_assert(kThreads == 256, "one histogram bin per thread");

  const long long row = blockIdx.x;               // (b*H + h)*Tm + i
  const int i = (int)(row % a.Tm);
  const int bh = (int)(row / a.Tm);
  const int b = bh / a.H, h = bh % a.H;
  const int hk = h / (a.H / a.Hkv);
  const int tid = threadIdx.x;
  const int last_q = min(a.N, (i + 1) * kBq) - 1;
  const int n_live = a.causal ? min(a.Tn, last_q / kBk + 1) : a.Tn;
  const bool fix_q = a.ws.sq[row] < a.theta;
  // a fix row keeps every live tile (eq. 9) and needs no column flags
  if (!fix_q) {
    const double* skr = a.ws.sk + ((long long)b * a.Hkv + hk) * a.Tn;
#pragma unroll 8
    for (int j = tid; j < a.Tn; j += kThreads) flag[j] = (skr[j] < a.theta) ? 1 : 0;
    __syncthreads();
    // gather the live selective columns in ascending j
    const int per = (n_live + kThreads - 1) / kThreads;
    const int lo = min(n_live, tid * per), hi = min(n_live, lo + per);
    int mine = 0;
    for (int j = lo; j < hi; ++j) mine += (flag[j] & 1) ? 0 : 1;
    int m;
    int pos = block_excl_scan_int(mine, ired, m);
    const double* srow = a.ws.shat + row * a.Tn;
    // every j < hi is a column of the row, so its value is loaded before the
    // test and the unrolled loads overlap
#pragma unroll 8
    for (int j = lo; j < hi; ++j) {
      const double sv = srow[j];
      if (!(flag[j] & 1)) {
        pv[pos] = sv;
        pj[pos] = j;
        ++pos;
      }
    }
    __syncthreads();
    if (m > 0) {
      // softmax over the m finite entries (eq. 8's P^[i])
      double mx = kNegInfD;
      for (int r = tid; r < m; r += kThreads) mx = fmax(mx, pv[r]);
      mx = block_reduce_max(mx, dred);
      double se = 0.0;
      for (int r = tid; r < m; r += kThreads) {
        const double e = exp(pv[r] - mx);
        pv[r] = e;
        se += e;
      }
      se = block_reduce_sum(se, dred);
      // ---- TopCdf (eq. 8) without a sort.  In the order (P desc, j asc) the
      // kept entries are the prefix up to and including the first entry whose
      // inclusive cumulative sum reaches tau * sum.  A radix select over the
      // probabilities' bit patterns (positive doubles order like their bits)
      // finds that entry's value 8 bits per pass; entries of equal value are
      // then kept in ascending j.  Sums are taken in 2^-62 fixed point, so they
      // are exact integers, independent of the order of the atomic adds.
      constexpr int MAXE = SPARGE_MAX_TN / kThreads;
      const int per2 = (m + kThreads - 1) / kThreads;
      const int lo2 = min(m, tid * per2);
      const int n2 = min(m, lo2 + per2) - lo2;
      uint64_t key[MAXE], fx[MAXE];
      uint64_t fsum = 0;
#pragma unroll
      for (int x = 0; x < MAXE; ++x) {
        const double pr = x < n2 ? pv[lo2 + x] / se : 0.0;
        key[x] = (uint64_t)__double_as_longlong(pr);
        fx[x] = (uint64_t)(pr * 0x1p62);
        fsum += fx[x];
      }
      const uint64_t F = block_reduce_u64(fsum, ured);
      // kept iff exclusive prefix < tau * F, i.e. < TF = ceil(tau * F), taken
      // exactly: 1 <= TF <= F, so the running sums always cross TF inside
      // some bin, the first entry is always kept, and tau = 1 keeps every
      // entry whose fixed-point value is non-zero.  (A float64 product
      // tau * (double)F would not do: (double)F is F rounded to a multiple of
      // 2^9 near 2^62, on either side of F.)
      const uint64_t TF = ceil_tau_times(a.tau, F);
      if (tid == 0) {
        s_digit = 0;
        s_above = 0;
      }
      uint64_t prefix = 0, above = 0;
      for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        hcnt[tid] = 0u;
        hsum[tid] = 0ull;
        __syncthreads();
#pragma unroll
        for (int x = 0; x < MAXE; ++x)
          if (x < n2 && ((key[x] >> shift) >> 8) == prefix) {     // in the selected range
            const int d = (int)((key[x] >> shift) & 255u);
            atomicAdd(&hcnt[d], 1u);
            atomicAdd(&hsum[d], (unsigned long long)fx[x]);
          }
        __syncthreads();
        if (tid < 64) {
          // lane l scans bins 255-4l .. 252-4l: the crossing bin is the first,
          // in descending digit order, where above + (sum before it) < TF <=
          // above + (sum through it)
          uint64_t sb[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) sb[q] = hsum[255 - 4 * tid - q];
          const uint64_t mine = sb[0] + sb[1] + sb[2] + sb[3];
          uint64_t incl = mine;
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const uint64_t t = __shfl_up(incl, off, 64);
            if (tid >= off) incl += t;
          }
          uint64_t cum = above + (incl - mine);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (cum < TF && TF <= cum + sb[q]) {
              s_digit = 255 - 4 * tid - q;
              s_above = cum;
            }
            cum += sb[q];
          }
        }
        __syncthreads();
        prefix = (prefix << 8) | (uint64_t)s_digit;
        above = s_above;
        // a crossing bin with one entry: that entry is the boundary value
        // (the entries above it are exactly those summed in `above`), so the
        // remaining passes would only spell out its key
        if (pass < 7 && hcnt[s_digit] == 1u) {
#pragma unroll
          for (int x = 0; x < MAXE; ++x)
            if (x < n2 && (key[x] >> shift) == prefix) s_key = key[x];
          __syncthreads();
          prefix = s_key;
          break;
        }
      }
      // prefix is now the value v of the boundary entry and above the sum of
      // the entries greater than v; among the entries equal to v, the one of
      // rank t (ascending j) is kept iff above + t * f(v) < TF
      int my_ties = 0;
#pragma unroll
      for (int x = 0; x < MAXE; ++x) my_ties += (x < n2 && key[x] == prefix) ? 1 : 0;
      int n_ties;
      int rank = block_excl_scan_int(my_ties, ired, n_ties);
      const uint64_t fv = (uint64_t)(__longlong_as_double((long long)prefix) * 0x1p62);
      const uint64_t room = TF - above;             // >= 1
      const long long tie_keep = fv == 0 ? n_ties : (long long)min((uint64_t)n_ties, (room + fv - 1) / fv);
#pragma unroll
      for (int x = 0; x < MAXE; ++x) {
        if (x >= n2) continue;
        bool keep = key[x] > prefix;
        if (key[x] == prefix) keep = rank++ < tie_keep;
        if (keep) flag[pj[lo2 + x]] |= 2;
      }
      __syncthreads();
    }
  }

  uint8_t* mg_row = a.mg + row * a.Tn;
  const int Tn = a.Tn;
  write_row(
      Tn, [&](int j) { return j < n_live && (fix_q || (flag[j] & 3) != 0); }, mg_row,
      a.row_cnt + row, a.row_idx + row * Tn, ired);
}

// compaction of a caller's mask (live tiles only)
__global__ __launch_bounds__(kThreads) void compact_rows(const uint8_t* mg, int Tm, int Tn, int N,
                                                         int causal, int32_t* cnt, uint16_t* idx) {
  __shared__ int ired[kThreads];
  const long long row = blockIdx.x;
  const int i = (int)(row % Tm);
  const int last_q = min(N, (i + 1) * kBq) - 1;
  const int n_live = causal ? min(Tn, last_q / kBk + 1) : Tn;
  const uint8_t* m = mg + row * Tn;
  write_row(
      Tn, [&](int j) { return j < n_live && m[j] != 0; }, nullptr, cnt + row, idx + row * Tn, ired);
}

}  // namespace

hipError_t launch_compact(const uint8_t* mg, int64_t rows, int Tm, int Tn, int N, int causal,
                          int32_t* cnt, uint16_t* idx, hipStream_t st) {
  hipLaunchKernelGGL(compact_rows, dim3((unsigned)rows), dim3(kThreads), 0, st, mg, Tm, Tn, N,
                     causal, cnt, idx);
  return hipGetLastError();
}

hipError_t launch_predict(const PredictArgs& a, hipStream_t st) {
  const long long pool_blocks = (long long)a.B * a.H * a.Tm + (long long)a.B * a.Hkv * a.Tn;
  if (a.d == 64)
    hipLaunchKernelGGL(pool_cossim<64>, dim3((unsigned)pool_blocks), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(pool_cossim<128>, dim3((unsigned)pool_blocks), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 g((unsigned)ceil_div(a.Tm, kGT), (unsigned)ceil_div(a.Tn, kGTJ), (unsigned)(a.B * a.H));
  hipLaunchKernelGGL(shat_gemm, g, dim3(kThreads), 0, st, a, 1.0 / sqrt((double)a.d));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = 13 * (size_t)a.Tn;
  hipLaunchKernelGGL(mask_rows, dim3((unsigned)((long long)a.B * a.H * a.Tm)), dim3(kThreads), lds, st,
                     a, a.Tn);
  return hipGetLastError();
}

}  // namespace sparge

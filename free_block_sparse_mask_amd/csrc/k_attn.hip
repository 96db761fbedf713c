// Stage 2 of SpargeAttn on gfx950: block-sparse FlashAttention forward with
// the lambda (sparse warp online softmax) rule.
//
// Pages: [Review] "SpargeAttn: Accurate and Training-free Sparse Attention
// Accelerating Any Model Inference" (xllm-io paper-review blog), "Core
// formulas" eqs. (1)-(3), the sparse warp online softmax paragraph and
// "Algorithm 1" (steps 6-17).
//
// Design (CDNA4 first, not the pages' CUDA warp layout):
// * One workgroup of 4 wavefronts per query block i of 128 rows; wavefront w
//   owns rows [32w, 32w + 32) of the block, so the lambda vote is one ballot
//   over a 64-lane wavefront (both lane halves hold the same 32 rows).
// * S^T = K_j Q_i^T on v_mfma_f32_32x32x16 (bf16/f16) or v_mfma_i32_32x32x32_i8:
//   the accumulator layout of S^T puts one query row per lane (lane % 32) and
//   16 of its 32 keys per 32x32 tile in registers, so the row max is an
//   in-lane reduction plus one exchange with lane ^ 32, and P~ can feed the
//   P~V MFMA as its B operand straight from registers.
// * O^T = V_j^T P~^T: V is transposed into LDS as it is staged, so the A
//   operand (8 keys of one d_v column) is two 8-byte LDS reads.
// * K_j and V_j for the next listed block are fetched into registers while
//   the current block is computed (one LDS buffer, two barriers per block).
// * The key blocks come from the compacted ascending list of M_g's ones.
// * Grid order: heaviest query blocks (largest i) first; when the number of
//   (batch, kv head) pairs is a multiple of 8, all query heads of one kv head
//   land on one XCD (workgroup id % 8), so their K/V tiles share that XCD's L2.
#include "common.hpp"

namespace sparge {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

template <bool BF16>
__device__ __forceinline__ unsigned int pack2(float a, float b) {
  if constexpr (BF16) {
    __bf16 x = (__bf16)a, y = (__bf16)b;
    return (unsigned int)__builtin_bit_cast(unsigned short, x) |
           ((unsigned int)__builtin_bit_cast(unsigned short, y) << 16);
  } else {
    _Float16 x = (_Float16)a, y = (_Float16)b;
    return (unsigned int)__builtin_bit_cast(unsigned short, x) |
           ((unsigned int)__builtin_bit_cast(unsigned short, y) << 16);
  }
}

template <bool BF16>
__device__ __forceinline__ f32x16 mfma16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Workgroup id -> (b, h, i); returns false for padding workgroups.
__device__ __forceinline__ bool map_block(const AttnArgs& p, int& b, int& h, int& i) {
  const int group = p.H / p.Hkv;
  const int pairs = p.B * p.Hkv;
  const long long id = blockIdx.x;
  if ((pairs & 7) == 0) {
    const int per_xcd = pairs >> 3;
    const int xcd = (int)(id & 7);
    const long long k = id >> 3;
    const long long per_i = (long long)per_xcd * group;
    const int irank = (int)(k / per_i);
    const int rem = (int)(k % per_i);
    const int pp = rem / group, g = rem % group;
    const int pair = xcd + 8 * pp;
    b = pair / p.Hkv;
    h = (pair % p.Hkv) * group + g;
    i = p.Tm - 1 - irank;
  } else {
    const long long bh = (long long)p.B * p.H;
    const int irank = (int)(id / bh);
    const int rem = (int)(id % bh);
    b = rem / p.H;
    h = rem % p.H;
    i = p.Tm - 1 - irank;
  }
  return i >= 0 && b < p.B;
}

// KIND: 0 f16, 1 bf16, 2 int8 QK + f16 PV, 3 int8 QK + bf16 PV
template <int D, int KIND, bool CAUSAL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd(AttnArgs p) {
  constexpr bool I8 = KIND >= 2;
  constexpr bool PVBF = (KIND == 1 || KIND == 3);
  constexpr int KSB = I8 ? (D + 16) : (D + 8) * 2;   // K row stride in bytes (16-byte aligned)
  constexpr int VSE = kBk + 4;                       // V^T row stride in 16-bit elements
  constexpr int K_BYTES = kBk * KSB;
  constexpr int V_BYTES = D * VSE * 2;
  constexpr int DCH = D / 8;                         // 16-byte chunks per 16-bit row
  constexpr int KCH = I8 ? D / 16 : DCH;             // 16-byte chunks per K row
  constexpr int K_LOADS = kBk * KCH / kThreads;      // per thread
  constexpr int V_UNITS = 16 * DCH;                  // (4 keys x 8 columns) units
  constexpr int QS = I8 ? D / 32 : D / 16;           // k-steps of the QK^T MFMA
  constexpr int OT = D / 32;                         // 32-column tiles of O^T

  __shared__ __attribute__((aligned(16))) unsigned char smem[K_BYTES + V_BYTES];
  __shared__ unsigned long long red[kWavesPerBlock][4];
  unsigned char* klds = smem;
  unsigned short* vlds = reinterpret_cast<unsigned short*>(smem + K_BYTES);

  int b, h, i;
  if (!map_block(p, b, h, i)) return;
  const int group = p.H / p.Hkv;
  const int hk = h / group;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int q0 = i * kBq + wave * kRowsPerWave;
  const int qrow = q0 + l32;
  const bool qvalid = qrow < p.N;
  const int last_q = min(p.N, (i + 1) * kBq) - 1;
  const int n_live = CAUSAL ? min(p.Tn, last_q / kBk + 1) : p.Tn;

  // ---- Q fragment (B operand of S^T = K Q^T), kept in registers ----
  u32x4 qf[QS];
  if constexpr (I8) {
    const int8_t* qb = static_cast<const int8_t*>(p.q) + ((long long)(b * p.H + h) * p.N) * D;
#pragma unroll
    for (int s = 0; s < QS; ++s)
      qf[s] = qvalid ? *reinterpret_cast<const u32x4*>(qb + (long long)qrow * D + 32 * s + 16 * hl)
                     : u32x4{0, 0, 0, 0};
  } else {
    const unsigned short* qb = static_cast<const unsigned short*>(p.q) + b * p.q_sb + h * p.q_sh;
#pragma unroll
    for (int s = 0; s < QS; ++s)
      qf[s] = qvalid ? *reinterpret_cast<const u32x4*>(qb + (long long)qrow * p.q_sn + 16 * s + 8 * hl)
                     : u32x4{0, 0, 0, 0};
  }
  float qscale = 1.0f;
  if constexpr (I8) qscale = p.q_scale[(long long)(b * p.H + h) * p.Tm + i];

  const unsigned char* kbase;
  long long k_sn_bytes;
  if constexpr (I8) {
    kbase = static_cast<const unsigned char*>(p.k) + ((long long)(b * p.Hkv + hk) * p.N) * D;
    k_sn_bytes = D;
  } else {
    kbase = static_cast<const unsigned char*>(p.k) + (b * p.k_sb + hk * p.k_sh) * 2;
    k_sn_bytes = p.k_sn * 2;
  }
  const unsigned short* vbase = static_cast<const unsigned short*>(p.v) + b * p.v_sb + hk * p.v_sh;
  const float* kscale_row = I8 ? p.k_scale + (long long)(b * p.Hkv + hk) * p.Tn : nullptr;

  const long long row_id = (long long)(b * p.H + h) * p.Tm + i;
  const int cnt = p.row_cnt[row_id];
  const uint16_t* list = p.row_idx + row_id * p.Tn;

  // ---- staging registers for the next K/V tile ----
  u32x4 kreg[K_LOADS > 0 ? K_LOADS : 1];
  u32x4 vreg[4];
  const int vu_c = tid % DCH, vu_g = tid / DCH;      // V unit: column chunk, key group

  auto fetch = [&](int j) {
#pragma unroll
    for (int r = 0; r < K_LOADS; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / KCH, ch = c % KCH;
      const int key = j * kBk + row;
      kreg[r] = key < p.N ? *reinterpret_cast<const u32x4*>(kbase + key * k_sn_bytes + ch * 16)
                          : u32x4{0, 0, 0, 0};
    }
    if (tid < V_UNITS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = j * kBk + 4 * vu_g + r;
        vreg[r] = key < p.N ? *reinterpret_cast<const u32x4*>(vbase + (long long)key * p.v_sn + 8 * vu_c)
                            : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int r = 0; r < K_LOADS; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / KCH, ch = c % KCH;
      *reinterpret_cast<u32x4*>(klds + row * KSB + ch * 16) = kreg[r];
    }
    if (tid < V_UNITS) {
      // transpose 4 keys x 8 columns: column e gets keys 4g..4g+3 as one 8-byte word
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        const int sh = (e & 1) * 16;
        const unsigned int k0 = (vreg[0][w] >> sh) & 0xffffu, k1 = (vreg[1][w] >> sh) & 0xffffu;
        const unsigned int k2 = (vreg[2][w] >> sh) & 0xffffu, k3 = (vreg[3][w] >> sh) & 0xffffu;
        u32x2 word = {k0 | (k1 << 16), k2 | (k3 << 16)};
        *reinterpret_cast<u32x2*>(vlds + (8 * vu_c + e) * VSE + 4 * vu_g) = word;
      }
    }
  };

  f32x16 oacc[OT];
#pragma unroll
  for (int t = 0; t < OT; ++t) oacc[t] = f32x16{};
  float m_run = kNegInf;      // running max, log2 units
  float l_half = 0.0f;        // this lane half's share of the row sum
  unsigned long long n_exec = 0, n_skip = 0, n_void = 0, n_qk = 0;

  if (cnt > 0) fetch(list[0]);
  for (int n = 0; n < cnt; ++n) {
    const int j = list[n];
    __syncthreads();                      // previous tile fully consumed
    stage();
    __syncthreads();
    if (n + 1 < cnt) fetch(list[n + 1]);  // overlaps with the math below
    if (j >= n_live) continue;            // not a live tile (never in lists from M_g of live tiles)
    ++n_qk;

    // ---- S^T = K_j Q_i^T : two 32-key x 32-row tiles ----
    float sv[2][16];
    if constexpr (I8) {
      const float sc = qscale * kscale_row[j] * p.scale_log2;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        i32x16 acc = {};
#pragma unroll
        for (int s = 0; s < QS; ++s) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(klds + (32 * t + l32) * KSB + 32 * s + 16 * hl);
          acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                     __builtin_bit_cast(i32x4, qf[s]), acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[t][r] = (float)acc[r] * sc;
      }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < QS; ++s) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(klds + (32 * t + l32) * KSB + 32 * s + 16 * hl);
          acc = mfma16<KIND == 1>(a, qf[s], acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[t][r] = acc[r] * p.scale_log2;
      }
    }

    // ---- masking: keys beyond N, causal future, rows beyond N ----
    const bool need_mask = (j * kBk + kBk > p.N) || (q0 + kRowsPerWave > p.N) ||
                           (CAUSAL && j * kBk + kBk - 1 > q0);
    if (need_mask) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * kBk + 32 * t + 8 * (r >> 2) + 4 * hl + (r & 3);
          const bool dead = !qvalid || key >= p.N || (CAUSAL && key > qrow);
          sv[t][r] = dead ? kNegInf : sv[t][r];
        }
    }

    // ---- online softmax (eq. 1), log2 units ----
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[t][r]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const bool finite_row = mx > kNegInf;
    // lambda vote over the wavefront's 32 rows
    const bool wants_pv = finite_row && !(mx - m_new < p.lam_log2);
    const bool any_finite = __any(finite_row);
    const bool exec = __any(wants_pv);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = (m_new == kNegInf) ? 1.0f : exp2f(m_run - m_new);
    float psum = 0.0f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sv[t][r] = exp2f(sv[t][r] - m_use);
        psum += sv[t][r];
      }
    l_half = alpha * l_half + psum;
    m_run = m_new;

    unsigned char code;
    if (!any_finite) {
      code = 3;
      ++n_void;
    } else if (!exec) {
      code = 2;
      ++n_skip;
    } else {
      code = 1;
      ++n_exec;
      if (__any(alpha != 1.0f)) {
#pragma unroll
        for (int t = 0; t < OT; ++t) oacc[t] *= alpha;
      }
      // ---- O^T += V_j^T P~^T ----
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int tt = s >> 1, r0 = 8 * (s & 1);
        u32x4 pb;
        pb[0] = pack2<PVBF>(sv[tt][r0 + 0], sv[tt][r0 + 1]);
        pb[1] = pack2<PVBF>(sv[tt][r0 + 2], sv[tt][r0 + 3]);
        pb[2] = pack2<PVBF>(sv[tt][r0 + 4], sv[tt][r0 + 5]);
        pb[3] = pack2<PVBF>(sv[tt][r0 + 6], sv[tt][r0 + 7]);
#pragma unroll
        for (int t = 0; t < OT; ++t) {
          const unsigned short* vrow = vlds + (32 * t + l32) * VSE + 16 * s + 4 * hl;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
          const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
          oacc[t] = mfma16<PVBF>(a, pb, oacc[t]);
        }
      }
    }
    if (p.dbg != nullptr && lane == 0 && q0 < p.N)
      p.dbg[(row_id * p.Tn + j) * kWavesPerBlock + wave] = code;
  }

  // ---- epilogue: O / l ----
  const float l_tot = l_half + xor32(l_half);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qvalid && p.out_f32) {
    float* ob = static_cast<float*>(p.o) + b * p.o_sb + h * p.o_sh + (long long)qrow * p.o_sn;
#pragma unroll
    for (int t = 0; t < OT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x4 w = {__float_as_uint(oacc[t][4 * g + 0] * inv), __float_as_uint(oacc[t][4 * g + 1] * inv),
                   __float_as_uint(oacc[t][4 * g + 2] * inv), __float_as_uint(oacc[t][4 * g + 3] * inv)};
        *reinterpret_cast<u32x4*>(ob + 32 * t + 8 * g + 4 * hl) = w;
      }
  } else if (qvalid) {
    // each float32 quotient is materialised (the empty asm keeps the compiler
    // from fusing multiply and narrowing into one differently rounded op), so
    // this output is exactly the float32 output rounded to the 16-bit type
    unsigned short* ob = static_cast<unsigned short*>(p.o) + b * p.o_sb + h * p.o_sh + (long long)qrow * p.o_sn;
#pragma unroll
    for (int t = 0; t < OT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y[e] = oacc[t][4 * g + e] * inv;
          asm volatile("" : "+v"(y[e]));
        }
        u32x2 w = {pack2<PVBF>(y[0], y[1]), pack2<PVBF>(y[2], y[3])};
        *reinterpret_cast<u32x2*>(ob + 32 * t + 8 * g + 4 * hl) = w;
      }
  }

  // ---- counters ----
  const bool empty = qvalid && hl == 0 && !(l_tot > 0.0f);
  const unsigned long long n_empty = __popcll(__ballot(empty));
  if (lane == 0) {
    red[wave][0] = n_exec;
    red[wave][1] = n_skip;
    red[wave][2] = n_void;
    red[wave][3] = n_empty;
  }
  __syncthreads();
  if (tid == 0 && p.counts != nullptr) {
    unsigned long long e = 0, s = 0, v = 0, em = 0;
    for (int w = 0; w < kWavesPerBlock; ++w) {
      // waves whose 32 rows all lie beyond N hold no group
      if (i * kBq + w * kRowsPerWave >= p.N) continue;
      e += red[w][0];
      s += red[w][1];
      v += red[w][2];
      em += red[w][3];
    }
    atomicAdd(p.counts + SPARGE_CNT_LIVE, (unsigned long long)n_live);
    atomicAdd(p.counts + SPARGE_CNT_QK_EXEC, n_qk);
    atomicAdd(p.counts + SPARGE_CNT_QK_SKIP, (unsigned long long)(n_live - n_qk));
    atomicAdd(p.counts + SPARGE_CNT_PV_EXEC, e);
    atomicAdd(p.counts + SPARGE_CNT_PV_SKIP, s);
    atomicAdd(p.counts + SPARGE_CNT_PV_VOID, v);
    atomicAdd(p.counts + SPARGE_CNT_EMPTY_ROWS, em);
    atomicAdd(p.counts + SPARGE_CNT_ROWS, (unsigned long long)(last_q - i * kBq + 1));
  }
}

__global__ void zero_u64(unsigned long long* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0ull;
}

template <int D, int KIND>
hipError_t launch_d_kind(const AttnArgs& a, hipStream_t st) {
  const long long blocks = (long long)a.B * a.H * a.Tm;
  if (a.causal)
    hipLaunchKernelGGL((attn_fwd<D, KIND, true>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_fwd<D, KIND, false>), dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t st) {
  switch (a.kind) {
    case 0: return launch_d_kind<D, 0>(a, st);
    case 1: return launch_d_kind<D, 1>(a, st);
    case 2: return launch_d_kind<D, 2>(a, st);
    default: return launch_d_kind<D, 3>(a, st);
  }
}

}  // namespace

hipError_t launch_zero_counts(unsigned long long* counts, int n, hipStream_t st) {
  hipLaunchKernelGGL(zero_u64, dim3(1), dim3(64), 0, st, counts, n);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
  return a.d == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace sparge

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
//   in-lane reduction plus one exchange with lane ^ 32, and P~ feeds the P~V
//   MFMA as its B operand straight from registers.
// * O^T = V_j^T P~^T with V^T from a once-per-call transposed copy of V whose
//   keys are ordered so that the A operand (the 8 keys one lane half feeds
//   one MFMA) is a single 16-byte LDS read.
// * K_j and V_j^T tiles go from global memory straight into LDS
//   (global_load_lds_dwordx4, no staging registers) into two alternating
//   buffers: the next listed tile streams in while the current one is used,
//   with one barrier per tile.  The 16-byte granules of each LDS row are
//   XOR-swizzled by row so the MFMA operand reads hit distinct banks.
// * The key blocks come from the compacted ascending list of M_g's ones.
// * Grid order: heaviest query blocks (largest i) first, in phases of a few
//   kv heads with one kv head per XCD (see map_block).
#include <type_traits>

#include "common.hpp"

namespace sparge {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// v_permlane32_swap(x, x) leaves x[l % 32] in one result and x[32 + l % 32]
// in the other, so combining the two gives every lane the pair (l, l ^ 32).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// two floats -> two 16-bit values (round to nearest even) in one 32-bit word;
// the vector form maps to one v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32
template <bool BF16>
__device__ __forceinline__ unsigned int pack2(float a, float b) {
  const f32x2 v = {a, b};
  if constexpr (BF16)
    return __builtin_bit_cast(unsigned int, __builtin_convertvector(v, bf16x2));
  else
    return __builtin_bit_cast(unsigned int, __builtin_convertvector(v, f16x2));
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

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 16 bytes per lane from global memory straight into LDS: lane L's bytes land
// at lds_dst + 16 L (lds_dst must be the same for the whole wavefront).
__device__ __forceinline__ void dma16(const unsigned char* src, unsigned char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_dst, 16, 0, 0);
}

// Workgroup id -> (b, h, i).  Workgroups are dispatched to the 8 XCDs round
// robin (id % 8).  When the query heads of 8 / G kv heads fill one row of 8
// slots (G = H / H_kv), the grid runs in phases of 8 / G kv heads: slot s of
// every row is XCD s, which always serves query head s % G of kv head
// s / G of the phase, heaviest block rows first.  Each XCD's L2 then sees one
// kv head, and only 8 / G kv heads (a few tens of MB to a few hundred MB of
// K and V) are live in the Infinity Cache at a time.  Other shapes fall back
// to block rows outermost, heaviest first.
__device__ __forceinline__ bool map_block(const AttnArgs& p, int& b, int& h, int& i) {
  const int group = p.H / p.Hkv;
  const int pairs = p.B * p.Hkv;
  const long long id = blockIdx.x;
  if ((8 % group) == 0 && (pairs % (8 / group)) == 0) {
    const int per_phase = 8 / group;
    const int slot = (int)(id & 7);
    const long long k = id >> 3;
    const int phase = (int)(k / p.Tm);
    const int irank = (int)(k % p.Tm);
    const int pair = phase * per_phase + slot / group;
    b = pair / p.Hkv;
    h = (pair % p.Hkv) * group + slot % group;
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
  constexpr int KROW = I8 ? D : 2 * D;          // bytes per K row
  constexpr int KG = KROW / 16;                 // 16-byte granules per K row
  constexpr int KSW = 16 / KG;                  // rows sharing one swizzle step
  constexpr int K_BYTES = kBk * KROW;
  constexpr int VROW = kBk * 2;                 // bytes per V^T row (64 keys)
  constexpr int V_BYTES = D * VROW;
  constexpr int KCW = K_BYTES / 1024 / kWavesPerBlock;   // 1 KB chunks per wave
  constexpr int VCW = V_BYTES / 1024 / kWavesPerBlock;
  constexpr int QS = I8 ? D / 32 : D / 16;      // k-steps of the QK^T MFMA
  constexpr int OT = D / 32;                    // 32-column tiles of O^T
  static_assert(KCW >= 1 && VCW >= 1, "tile must span every wave");

  __shared__ __attribute__((aligned(1024))) unsigned char kbuf[2][K_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char vbuf[2][V_BYTES];
  __shared__ unsigned long long red[kWavesPerBlock][4];

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
  const unsigned char* vtbase =
      reinterpret_cast<const unsigned char*>(p.vt) + ((long long)(b * p.Hkv + hk) * D) * p.Np * 2;
  const float* kscale_row = I8 ? p.k_scale + (long long)(b * p.Hkv + hk) * p.Tn : nullptr;

  const long long row_id = (long long)(b * p.H + h) * p.Tm + i;
  const int cnt = p.row_cnt[row_id];
  const uint16_t* list = p.row_idx + row_id * p.Tn;

  // ---- global -> LDS tile loads (one 1 KB chunk per wave instruction) ----
  // A chunk holds R = 1024 / row_bytes consecutive rows.  The swizzle repeats
  // every 16 rows, so chunk c of wavefront w is placed at rows
  // 16 (c (4/G) + w / G) + R (w % G) + lane / granules_per_row, G = 16 / R:
  // every chunk of a wavefront then has the same lane offset (one register),
  // and the chunk only moves the uniform base.
  constexpr int KR = 1024 / KROW, KGRP = 16 / KR;
  constexpr int VR = 1024 / VROW, VGRP = 16 / VR;
  const int k_row0 = 16 * (wave / KGRP) + KR * (wave % KGRP) + lane / KG;
  const uint32_t k_off = (uint32_t)(k_row0 * k_sn_bytes) + (uint32_t)(((lane % KG) ^ ((k_row0 / KSW) % KG)) * 16);
  const int v_row0 = 16 * (wave / VGRP) + VR * (wave % VGRP) + lane / 8;
  const uint32_t v_off = (uint32_t)(v_row0 * p.Np * 2) + (uint32_t)(((lane % 8) ^ ((v_row0 / 2) % 8)) * 16);
  auto issue_k = [&](int j, int st) {
    const bool ragged = j * kBk + kBk > p.N;
#pragma unroll
    for (int c = 0; c < KCW; ++c) {
      const int row_c = 16 * c * (4 / KGRP);                  // rows added by chunk c
      const unsigned char* src = kbase + ((long long)j * kBk + row_c) * k_sn_bytes + k_off;
      if (ragged) {
        // rows past N re-read row N-1 (their scores are masked); the address is
        // formed from the clamped key in signed 64-bit arithmetic
        const long long key = (long long)j * kBk + row_c + min(k_row0, p.N - 1 - j * kBk - row_c);
        src = kbase + key * k_sn_bytes + (k_off - (uint32_t)(k_row0 * k_sn_bytes));
      }
      dma16(src, &kbuf[st][(row_c + 16 * (wave / KGRP) + KR * (wave % KGRP)) * KROW]);
    }
  };
  auto issue_v = [&](int j, int st) {
#pragma unroll
    for (int c = 0; c < VCW; ++c) {
      const int row_c = 16 * c * (4 / VGRP);
      const unsigned char* base = vtbase + ((long long)row_c * p.Np + (long long)j * kBk) * 2;
      dma16(base + v_off, &vbuf[st][(row_c + 16 * (wave / VGRP) + VR * (wave % VGRP)) * VROW]);
    }
  };

  // LDS read bases: the swizzled offset of k-step s is base ^ (32 s), and the
  // second 32-row tile sits a fixed distance further (see the layout above).
  const int ksw = (l32 / KSW) % KG;
  uint32_t k_rd = (uint32_t)(l32 * KROW) + (uint32_t)((ksw & ~1) * 16) + (uint32_t)((hl ^ (ksw & 1)) * 16);
  const int vsw = (l32 / 2) % 8;
  uint32_t v_rd = (uint32_t)(l32 * VROW) + (uint32_t)((vsw & ~1) * 16) + (uint32_t)((hl ^ (vsw & 1)) * 16);

  // S^T of one tile: two 32-key x 32-row MFMA accumulators (raw dot products)
  using Acc = typename std::conditional<I8, i32x16, f32x16>::type;
  auto qk = [&](const unsigned char* kt, Acc (&acc)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      acc[t] = Acc{};
#pragma unroll
      for (int s = 0; s < QS; ++s) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(kt + t * 32 * KROW + (k_rd ^ (32u * s)));
        if constexpr (I8)
          acc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                        __builtin_bit_cast(i32x4, qf[s]), acc[t], 0, 0, 0);
        else
          acc[t] = mfma16<KIND == 1>(a, qf[s], acc[t]);
      }
    }
  };

  f32x16 oacc[OT];
#pragma unroll
  for (int t = 0; t < OT; ++t) oacc[t] = f32x16{};
  float m_run = kNegInf;      // running max, log2 units
  float l_half = 0.0f;        // this lane half's share of the row sum
  // per-wavefront tallies (wave-uniform; one workgroup visits at most Tn tiles)
  int n_exec = 0, n_skip = 0, n_void = 0;
  uint8_t* dbg_row = p.dbg != nullptr ? p.dbg + row_id * p.Tn * kWavesPerBlock + wave : nullptr;
  const bool write_dbg = dbg_row != nullptr && q0 < p.N;

  // Software pipeline: while the softmax of listed tile n runs on the VALU,
  // the QK^T MFMAs of tile n+1 are already in flight.  K_{n+2} and V_{n+1}
  // stream into the buffers that tiles n and n-1 have released.  The MFMAs of
  // the next tile and the whole softmax of this one form one branch-free
  // block, so the scheduler can interleave them; only P~V sits behind the
  // wavefront's vote.  After the last tile the next-tile MFMAs recompute a
  // stale buffer and are discarded.
  auto step = [&](int n, Acc (&cur)[2], Acc (&nxt)[2]) {
    const int j = list[n];
    wait_vmem();                          // K_{n+1} and V_n have landed (this wave's part)
    __syncthreads();                      // everyone's have; everyone is done with tile n-1
    asm volatile("" : "+v"(k_rd), "+v"(v_rd));
    if (n + 2 < cnt) issue_k(list[n + 2], n & 1);
    if (n + 1 < cnt) issue_v(list[n + 1], (n + 1) & 1);
    const unsigned char* vt = vbuf[n & 1];
    const unsigned char* kn = kbuf[(n + 1) & 1];

    float c_scale = p.scale_log2;
    if constexpr (I8) c_scale = qscale * kscale_row[j] * p.scale_log2;
    float sv[2][16];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[t][r] = (float)cur[t][r];
    // masking: keys beyond N, causal future, rows beyond N (diagonal and ragged tiles only)
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

    // ---- next tile's S^T on the matrix cores ----
    qk(kn, nxt);

    // ---- online softmax (eq. 1) in log2 units; the scale is folded into an FMA ----
    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sv[t][r]);
    mx = max_halves(mx);
    const float mloc = mx * c_scale;                 // c_scale > 0: max commutes with the scale
    const float m_new = fmaxf(m_run, mloc);
    const bool finite_row = mloc > kNegInf;
    // lambda vote over the wavefront's 32 rows
    const bool wants_pv = finite_row && !(mloc - m_new < p.lam_log2);
    const bool any_finite = __any(finite_row);
    const bool exec = __any(wants_pv);
    const float neg_m = (m_new == kNegInf) ? 0.0f : -m_new;
    const float alpha = (m_new == kNegInf) ? 1.0f : fast_exp2(m_run - m_new);
    // P~ (eq. 1); it always feeds l (Algorithm 1 computes it before the M_pv
    // test) and is packed in the P~V input type as the B operand of 4 k-steps
    float psum = 0.0f;
    u32x4 pb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int tt = s >> 1, r0 = 8 * (s & 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = fast_exp2(fmaf(sv[tt][r0 + 2 * e], c_scale, neg_m));
        const float x1 = fast_exp2(fmaf(sv[tt][r0 + 2 * e + 1], c_scale, neg_m));
        psum += x0 + x1;
        pb[s][e] = pack2<PVBF>(x0, x1);
      }
    }
    l_half = alpha * l_half + psum;
    m_run = m_new;
    const unsigned char code = exec ? 1 : (any_finite ? 2 : 3);
    n_exec += exec ? 1 : 0;
    n_skip += (!exec && any_finite) ? 1 : 0;
    n_void += any_finite ? 0 : 1;
    if (exec) {
#pragma unroll
      for (int t = 0; t < OT; ++t) oacc[t] *= alpha;
      // ---- O^T += V_j^T P~^T ----
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t off = v_rd ^ (32u * s);
#pragma unroll
        for (int t = 0; t < OT; ++t) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(vt + t * 32 * VROW + off);
          oacc[t] = mfma16<PVBF>(a, pb[s], oacc[t]);
        }
      }
    }
    if (write_dbg && lane == 0) dbg_row[j * kWavesPerBlock] = code;
  };

  Acc s_a[2], s_b[2];
  if (cnt > 0) {
    issue_k(list[0], 0);
    issue_v(list[0], 0);
    if (cnt > 1) issue_k(list[1], 1);
    wait_vmem();
    __syncthreads();
    qk(kbuf[0], s_a);
  }
  int n = 0;
  for (; n + 1 < cnt; n += 2) {           // unrolled by two so the score buffers swap roles
    step(n, s_a, s_b);
    step(n + 1, s_b, s_a);
  }
  if (n < cnt) step(n, s_a, s_b);
  const int n_qk = cnt;

  // ---- epilogue: O / l ----
  const float l_tot = sum_halves(l_half);
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
    red[wave][0] = (unsigned long long)n_exec;
    red[wave][1] = (unsigned long long)n_skip;
    red[wave][2] = (unsigned long long)n_void;
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
    atomicAdd(p.counts + SPARGE_CNT_QK_EXEC, (unsigned long long)n_qk);
    atomicAdd(p.counts + SPARGE_CNT_QK_SKIP, (unsigned long long)(n_live - n_qk));
    atomicAdd(p.counts + SPARGE_CNT_PV_EXEC, e);
    atomicAdd(p.counts + SPARGE_CNT_PV_SKIP, s);
    atomicAdd(p.counts + SPARGE_CNT_PV_VOID, v);
    atomicAdd(p.counts + SPARGE_CNT_EMPTY_ROWS, em);
    atomicAdd(p.counts + SPARGE_CNT_ROWS, (unsigned long long)(last_q - i * kBq + 1));
  }
}

// V [B,Hkv,N,D] (strided, 16-bit) -> V^T [B,Hkv,D,Np], zero past N; 64 x 64 tiles.
__global__ __launch_bounds__(kThreads) void transpose_v(AttnArgs p) {
  __shared__ __attribute__((aligned(16))) unsigned short tile[64][72];
  const int kt = blockIdx.x, dt = blockIdx.y, bh = blockIdx.z;
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const int tid = threadIdx.x;
  const unsigned short* vb = static_cast<const unsigned short*>(p.v) + b * p.v_sb + hk * p.v_sh;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int key = tid / 8 + 32 * r, ch = tid % 8;
    const int gk = kt * 64 + key;
    u32x4 val = {0, 0, 0, 0};
    if (gk < p.N) val = *reinterpret_cast<const u32x4*>(vb + (long long)gk * p.v_sn + dt * 64 + 8 * ch);
    *reinterpret_cast<u32x4*>(&tile[key][8 * ch]) = val;
  }
  __syncthreads();
  unsigned short* out = p.vt + ((long long)bh * p.d) * p.Np;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int dv = tid / 8 + 32 * r, kc = tid % 8;
    // positions 8kc..8kc+7 of the row; inside each group of 16 keys the
    // middle quarters are swapped, so the 16 bytes at positions 8h..8h+7 hold
    // keys {4h..4h+3, 8+4h..8+4h+3}: the 8 keys one lane half feeds one MFMA
    const int base = 16 * (kc / 2) + 4 * (kc % 2);
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = base + (e < 2 ? 2 * e : 8 + 2 * (e - 2));
      w[e] = (unsigned int)tile[key][dv] | ((unsigned int)tile[key + 1][dv] << 16);
    }
    *reinterpret_cast<u32x4*>(out + (long long)(dt * 64 + dv) * p.Np + kt * 64 + 8 * kc) = w;
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
  dim3 g((unsigned)(a.Np / 64), (unsigned)(a.d / 64), (unsigned)(a.B * a.Hkv));
  hipLaunchKernelGGL(transpose_v, g, dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return a.d == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace sparge

// Stage 2 of SpargeAttn on gfx950: block-sparse FlashAttention forward with
// the lambda (sparse warp online softmax) rule.
//
// Pages: [Review] "SpargeAttn: Accurate and Training-free Sparse Attention
// Accelerating Any Model Inference" (xllm-io paper-review blog), "Core
// formulas" eqs. (1)-(3), the sparse warp online softmax paragraph and
// "Algorithm 1" (steps 6-17).
//
// Two passes over the listed tiles:
//
// attn_stats (pass 1) runs the online softmax of eq. (1) over the listed key
//   blocks of one query block in ascending order: S = Q K^T, the running max
//   m, the row sum l, and the lambda vote of every wavefront on every tile.
//   The vote only needs the running max, so pass 1 decides exactly which
//   (tile, wavefront) pairs run P~V without touching V.  It writes m and l of
//   every row and, per query block, the ascending list of tiles on which at
//   least one wavefront voted to run P~V, with the wavefront mask.
// attn_pv (pass 2) visits only those tiles.  A wavefront that voted on a
//   tile recomputes its S (the same MFMA sequence, so the same values) and
//   adds exp(S - m_final) V to O; O / l is stored at the end.  Unrolling the
//   rescaling of eq. (1) gives the same sum: a tile's P~ = exp(S - m_t) is
//   multiplied by exp(m_t - m_final) through the later rescales, and a
//   skipped group leaves m unchanged.
//
// At the workloads this path is built for, about one listed tile in eight
// has a voting wavefront, so V (half of the bytes of a K/V pass) is read for
// a small fraction of the tiles, and pass 1 holds only K in LDS: a two-slot
// ring for a single block, small enough that four workgroups share a CU, and
// a four-slot (int8: six-slot) ring for a pair of blocks, two workgroups per
// CU.
//
// attn_fused is the one-pass form (Algorithm 1's shape) for calls in which
//   nearly every wavefront votes or rows are short: K and V^T tiles share
//   its ring (for a single block two slots, or four where they fit in 64 KB;
//   for a pair of dense blocks four, one barrier per two tiles), and the P~V
//   of a voted tile follows its vote, for every Q/K and P~V type the passes
//   take.  attn_pilot samples the call's
//   blocks on the device and pilot_decide writes which path the call takes;
//   the kernels of the other path read that flag and return at once.
//
// Most of pass 1's tiles belong to query blocks whose row of M_g is all
// ones on the live tiles (the fix blocks of eq. (9) force it), so their
// lists are 0, 1, ..., live - 1 and prefixes of one another.  build_packs
// pairs such blocks of one kv head, heaviest first, and one workgroup of 8
// wavefronts runs a pair on one K stream (half the tile loads); the other
// blocks keep a workgroup of their own in a second launch, and sum_counts
// adds up the partial counters of both.
//
// Layout (CDNA4 first, not the pages' CUDA warp layout):
// * 4 wavefronts per query block i of 128 rows; wavefront w owns rows
//   [32w, 32w + 32) of the block, so the lambda vote is one ballot over a
//   64-lane wavefront (both lane halves hold the same 32 rows).
// * S^T = K_j Q_i^T on v_mfma_f32_32x32x16 (bf16/f16) or v_mfma_i32_32x32x32_i8:
//   the accumulator layout of S^T puts one query row per lane (lane % 32) and
//   16 of its 32 keys per 32x32 tile in registers, so the row max is an
//   in-lane reduction plus one exchange with lane ^ 32, and P~ feeds the P~V
//   MFMA as its B operand straight from registers.
// * O^T = V_j^T P~^T with V^T from a once-per-call transposed copy of V whose
//   keys are ordered so that the A operand (the 8 keys one lane half feeds
//   one MFMA) is a single 16-byte LDS read.
// * Tiles go from global memory straight into LDS (global_load_lds_dwordx4)
//   into a ring of slots.  These loads are issued as inline assembly: the
//   compiler neither tracks them nor adds waits for them, and every wait on
//   them is explicit (a vmcnt that leaves the younger tiles in flight,
//   followed by a barrier).  The 16-byte granules of each LDS row are
//   XOR-swizzled by row so the MFMA operand reads hit distinct banks.
// * Grid order: heaviest query blocks (largest i) first, in phases of a few
//   kv heads with one kv head per XCD (see map_block); the pairs of pass 1
//   come from per-kv-head queues, each XCD starting on its own kv heads.
#include <type_traits>

#include "common.hpp"

namespace sparge {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
// log2-units distance below the running max past which a whole tile's
// exponentials are skipped: each of its P~ is below 2^-32, so it adds less
// than 64 * 2^-32 = 2^-26 to a row sum l >= 1 (a quarter of float32's half
// ulp at 1), and the 4096 tiles of the longest row less than 2^-14 of l
// (see attn_stats)
constexpr float kFarLog2 = 32.0f;
// attention pass 1: K ring slots and tiles loaded ahead, for one query block
// per workgroup and for packs of dense blocks
constexpr int kStatsSlots = 2;
constexpr int kStatsAhead = 1;
// pair kernel: K slots, tiles loaded ahead, entries per workgroup barrier.
// int8 K tiles are half the size, so their ring is deeper and its barriers
// fewer (six slots, three per barrier: 20.4 against 20.9 ms at 128K GQA).
template <bool I8>
struct PackRing {
  static constexpr int slots = I8 ? 6 : 4;
  static constexpr int ahead = I8 ? 3 : 2;
  static constexpr int per = I8 ? 3 : 2;
};

// The larger of two floats that are not NaN (scores, their maxima, -inf) in
// one v_max_f32: fmaxf first quiets each operand the compiler cannot prove
// canonical (a lane exchange's result, a loop-carried max), one more
// instruction apiece.
__device__ __forceinline__ float max_nn(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// v_permlane32_swap(x, x) leaves x[l % 32] in one result and x[32 + l % 32]
// in the other, so combining the two gives every lane the pair (l, l ^ 32).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ int max_halves_i(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
  return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Whether x holds on any active lane: the lane mask of the compare itself
// (an SGPR pair), so a vote and everything built from it stay scalar; HIP's
// __any() takes the predicate through a VGPR and back.
__device__ __forceinline__ bool wave_any(bool x) { return __builtin_amdgcn_ballot_w64(x) != 0; }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
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

// LDS byte address of a pointer into shared memory
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ const unsigned char* uniform_ptr(const unsigned char* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return reinterpret_cast<const unsigned char*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

// 16 bytes per lane from sbase + voff (sbase wavefront-uniform) into LDS at
// lds + 16 * lane (lds wavefront-uniform).  M0 carries the LDS address; no
// other code in these kernels uses M0 (no LDS-DMA builtins, no indirect
// register indexing, no messages).  The instruction writes no register, so
// nothing the compiler allocates is pending when the statement ends.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const unsigned char* sbase, uint32_t voff, uint32_t lds) {
  // lds is uniform by contract; the read makes it an SGPR wherever the
  // compiler kept it in a vector register
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Waits until at most N vector-memory operations of this wavefront are in
// flight and its LDS operations are done, then joins the workgroup barrier.
// LGKM = false leaves the LDS and scalar-load counter alone: for a loop
// whose LDS reads have all been consumed before it gets here, so scalar
// loads may stay in flight across the barrier.
template <int N, bool LGKM = true>
__device__ __forceinline__ void wait_barrier() {
  if constexpr (LGKM)
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
// the same with N = pending * PER, pending (wavefront-uniform) clamped to [0, P]
template <int PER, int P, bool LGKM = true>
__device__ __forceinline__ void wait_pending(int pending) {
  if constexpr (P <= 0) {
    wait_barrier<0, LGKM>();
  } else {
    if (pending >= P)
      wait_barrier<P * PER, LGKM>();
    else
      wait_pending<PER, P - 1, LGKM>(pending);
  }
}

// Workgroup id -> (b, h, r) for T row groups per head (r = T - 1 for the
// heaviest).  Workgroups are dispatched to the 8 XCDs round robin (id % 8).
// When the query heads of 8 / G kv heads fill one row of 8 slots
// (G = H / H_kv), the grid runs in phases of 8 / G kv heads: slot s of every
// row is XCD s, which always serves query head s % G of kv head s / G of the
// phase, heaviest rows first.  Each XCD's L2 then sees one kv head, and only
// 8 / G kv heads (a few tens of MB to a few hundred MB of K and V) are live
// in the Infinity Cache at a time.  Other shapes fall back to rows
// outermost, heaviest first.
__device__ __forceinline__ bool map_block(const AttnArgs& p, int T, int& b, int& h, int& r) {
  const int group = p.H / p.Hkv;
  const int pairs = p.B * p.Hkv;
  const long long id = blockIdx.x;
  if ((8 % group) == 0 && (pairs % (8 / group)) == 0) {
    const int per_phase = 8 / group;
    const int slot = (int)(id & 7);
    const long long k = id >> 3;
    const int phase = (int)(k / T);
    const int rank = (int)(k % T);
    const int pair = phase * per_phase + slot / group;
    b = pair / p.Hkv;
    h = (pair % p.Hkv) * group + slot % group;
    r = T - 1 - rank;
  } else {
    const long long bh = (long long)p.B * p.H;
    const int rank = (int)(id / bh);
    const int rem = (int)(id % bh);
    b = rem / p.H;
    h = rem % p.H;
    r = T - 1 - rank;
  }
  return r >= 0 && b < p.B;
}

// Whether the call's path flag (written on the device by pilot_decide) names
// `path`; a call without a flag always takes two passes.
__device__ __forceinline__ bool path_is(const AttnArgs& p, int path) {
  return p.path_flag != nullptr && __builtin_amdgcn_readfirstlane(*p.path_flag) == path;
}

// ---------------------------------------------------------------------------
// Geometry shared by both passes
// ---------------------------------------------------------------------------
template <int D, int KIND>
struct Geo {
  static constexpr bool I8 = KIND >= 2;
  static constexpr bool PVBF = (KIND == 1 || KIND == 3);
  static constexpr int KROW = I8 ? D : 2 * D;          // bytes per K row
  static constexpr int KG = KROW / 16;                 // 16-byte granules per K row
  static constexpr int KSW = 16 / KG;                  // rows sharing one swizzle step
  static constexpr int K_BYTES = kBk * KROW;
  static constexpr int KCH = K_BYTES / 1024;           // 1 KB chunks per K tile
  static constexpr int KR = 1024 / KROW;               // K rows per 1 KB chunk
  static constexpr int VROW = kBk * 2;                 // bytes per V^T row (64 keys)
  static constexpr int V_BYTES = D * VROW;
  static constexpr int VCW = V_BYTES / 1024 / kWavesPerBlock;
  static constexpr int VR = 1024 / VROW;
  static constexpr int VGRP = 16 / VR;
  static constexpr int QS = I8 ? D / 32 : D / 16;      // k-steps of the QK^T MFMA
  static constexpr int OT = D / 32;                    // 32-column tiles of O^T
  static constexpr int EPM = 32 / (2 * QS);            // scores per lane per QK^T MFMA
  // pass 2: (K, V^T) slots
  static constexpr int E_BYTES = K_BYTES + V_BYTES;
  static constexpr int NS2 = (65536 / E_BYTES) >= 4 ? 4 : 2;
  // pass 2 with fp8 P~V: V^T tiles of one byte per value (64 keys per row)
  static constexpr int V8_BYTES = D * kBk;
  static constexpr int V8CW = V8_BYTES / 1024 / kWavesPerBlock;
  static constexpr int E8_BYTES = K_BYTES + V8_BYTES;
  // as many slots (up to 4) as keep the ring at 72 KB, so two workgroups
  // still share a CU
  static constexpr int NS8 = 4 * E8_BYTES <= 65536 ? 4 : (3 * E8_BYTES <= 73728 ? 3 : 2);
  static_assert(VCW >= 1, "tile must span every wave");
  static_assert(EPM * 2 * QS == 32, "scores must split evenly over the MFMAs");
};

template <int D, int KIND, int NP>
size_t stats_lds_bytes(int Tn) {
  using G = Geo<D, KIND>;
  return (size_t)(NP == 1 ? kStatsSlots : PackRing<G::I8>::slots) * G::K_BYTES + (NP == 1 ? (size_t)2 * ((Tn + 1) & ~1) : 0) +
         (size_t)4 * NP * kWavesPerBlock * ((Tn + 15) / 16) + (G::I8 ? (size_t)4 * Tn : 0);
}
// Pass 2 at d = 128 with (K, V^T) entries of at most 24 KB (int8 K with
// 16-bit V^T, 16-bit K with fp8 V^T, int8 K with fp8 V^T) runs a two-slot
// ring and reads its entry list (and the int8 K block scales) with scalar
// loads, one step ahead, instead of staging them in LDS: the ring alone
// (48 or 32 KB) is then the workgroup's LDS, and three workgroups share a
// CU instead of two.
template <int D, int KIND, bool PV8>
constexpr bool pv_scalar_list() {
  using G = Geo<D, KIND>;
  return D == 128 && (PV8 ? G::E8_BYTES : G::E_BYTES) <= 24576;
}
template <int D, int KIND, bool PV8>
constexpr int pv_slots() {
  using G = Geo<D, KIND>;
  return pv_scalar_list<D, KIND, PV8>() ? 2 : (PV8 ? G::NS8 : G::NS2);
}
template <int D, int KIND, bool PV8>
constexpr int pv_waves_per_eu() {
  return pv_scalar_list<D, KIND, PV8>() ? 3 : 2;
}
template <int D, int KIND, bool PV8>
size_t pv_lds_bytes(int Tn) {
  using G = Geo<D, KIND>;
  const size_t ring = (size_t)pv_slots<D, KIND, PV8>() * (PV8 ? G::E8_BYTES : G::E_BYTES);
  if (pv_scalar_list<D, KIND, PV8>()) return ring;
  return ring + (size_t)4 * Tn + (G::I8 ? (size_t)4 * Tn : 0);
}

// A 32-bit load that the compiler issues as a scalar (SMEM) load: the
// address must be wavefront-uniform, and the memory is not written while
// the kernel runs (the constant address space promises that).
typedef const __attribute__((address_space(4))) uint32_t const_u32;
__device__ __forceinline__ uint32_t load_scalar(const void* base, long long idx) {
  return ((const_u32*)base)[idx];
}

// Per-lane pieces common to both passes: Q fragment, K DMA offsets, read bases.
// NW wavefronts share the loads of a K tile: its 1 KB chunk q (rows
// KR q .. KR q + KR - 1) is loaded by wavefront q % NW, so chunk c of
// wavefront w holds rows KR (c NW + w) + lane / KG.  The XOR swizzle of a row
// repeats every 16 rows and KR NW is a multiple of 16, so all chunks of a
// wavefront share one lane offset.
template <int D, int KIND, int NW>
struct Lane {
  using G = Geo<D, KIND>;
  static constexpr int KCW = G::KCH >= NW ? G::KCH / NW : 1;   // chunks per loading wavefront
  static_assert((G::KR * NW) % 16 == 0, "chunk rows must keep the swizzle phase");
  int b, h, i, hk, tid, wave, lane, l32, hl, q0, qrow;
  bool qvalid, loads_k;
  long long row_id;
  u32x4 qf[G::QS];
  float qscale;
  const unsigned char* kbase;
  long long k_sn_bytes;
  int k_row0;
  uint32_t k_gran;
  uint32_t k_voff[KCW];      // lane offset of chunk c inside a full tile
  uint32_t k_wl;             // this wavefront's LDS offset inside a tile (uniform)
  uint32_t k_rd;

  // wq: wavefront index inside its query block (0..3)
  __device__ __forceinline__ void init(const AttnArgs& p, int b_, int h_, int i_, int wq) {
    b = b_;
    h = h_;
    i = i_;
    hk = h / (p.H / p.Hkv);
    tid = threadIdx.x;
    wave = tid >> 6;
    lane = tid & 63;
    l32 = lane & 31;
    hl = lane >> 5;
    q0 = i * kBq + wq * kRowsPerWave;
    qrow = q0 + l32;
    qvalid = qrow < p.N;
    row_id = (long long)(b * p.H + h) * p.Tm + i;
    if constexpr (G::I8) {
      const int8_t* qb = static_cast<const int8_t*>(p.q) + ((long long)(b * p.H + h) * p.N) * D;
#pragma unroll
      for (int s = 0; s < G::QS; ++s)
        qf[s] = qvalid ? *reinterpret_cast<const u32x4*>(qb + (long long)qrow * D + 32 * s + 16 * hl)
                       : u32x4{0, 0, 0, 0};
      qscale = p.q_scale[row_id];
      kbase = static_cast<const unsigned char*>(p.k) + ((long long)(b * p.Hkv + hk) * p.N) * D;
      k_sn_bytes = D;
    } else {
      const unsigned short* qb = static_cast<const unsigned short*>(p.q) + b * p.q_sb + h * p.q_sh;
#pragma unroll
      for (int s = 0; s < G::QS; ++s)
        qf[s] = qvalid ? *reinterpret_cast<const u32x4*>(qb + (long long)qrow * p.q_sn + 16 * s + 8 * hl)
                       : u32x4{0, 0, 0, 0};
      qscale = 1.0f;
      kbase = static_cast<const unsigned char*>(p.k) + (b * p.k_sb + hk * p.k_sh) * 2;
      k_sn_bytes = p.k_sn * 2;
    }
    // The Q loads complete here.  The compiler counts only the loads it
    // emitted, so a wait it placed at their first use inside a tile loop
    // would run every iteration, and vmcnt also counts the K tiles in flight
    // through LDS-DMA: each tile would wait for the next one to land.
#pragma unroll
    for (int s = 0; s < G::QS; ++s) asm volatile("" : "+v"(qf[s]));
    asm volatile("" : "+v"(qscale));   // the int8 row-block scale, likewise
    loads_k = wave < G::KCH;
    k_row0 = G::KR * wave + lane / G::KG;
    k_gran = (uint32_t)(((lane % G::KG) ^ ((k_row0 / G::KSW) % G::KG)) * 16);
#pragma unroll
    for (int c = 0; c < KCW; ++c)
      k_voff[c] = (uint32_t)((k_row0 + c * G::KR * NW) * k_sn_bytes) + k_gran;
    k_wl = (uint32_t)__builtin_amdgcn_readfirstlane((int)(G::KR * wave * G::KROW));
    // LDS read base: the swizzled offset of k-step s is k_rd ^ (32 s), and the
    // second 32-row tile sits 32 rows further
    const int ksw = (l32 / G::KSW) % G::KG;
    k_rd = (uint32_t)(l32 * G::KROW) + (uint32_t)((ksw & ~1) * 16) + (uint32_t)((hl ^ (ksw & 1)) * 16);
  }

  // this wavefront's chunks of K tile j into the LDS tile at `slot_lds`
  // (j and slot_lds wavefront-uniform); KCW loads, or none
  __device__ __forceinline__ void issue_k(const AttnArgs& p, int j, uint32_t slot_lds) const {
    if (!loads_k) return;
    const unsigned char* tb = uniform_ptr(kbase + (long long)j * kBk * k_sn_bytes);
    if (j * kBk + kBk <= p.N) {
#pragma unroll
      for (int c = 0; c < KCW; ++c)
        dma16(tb, k_voff[c], slot_lds + (uint32_t)(c * NW * 1024) + k_wl);
    } else {
      // ragged last tile: rows past N re-read row N-1 (their scores are masked)
      const int lim = p.N - 1 - j * kBk;   // >= 0: tile j is live
#pragma unroll
      for (int c = 0; c < KCW; ++c)
        dma16(tb, (uint32_t)(min(k_row0 + c * G::KR * NW, lim) * k_sn_bytes) + k_gran,
              slot_lds + (uint32_t)(c * NW * 1024) + k_wl);
    }
  }

  // the A operands of S^T = K Q^T for one tile: 2 x QS 16-byte LDS reads
  __device__ __forceinline__ void read_k(const unsigned char* kt, u32x4 (&kf)[2][G::QS]) const {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < G::QS; ++s)
        kf[t][s] = *reinterpret_cast<const u32x4*>(kt + t * 32 * G::KROW + (k_rd ^ (32u * s)));
  }
};

template <int KIND>
__device__ __forceinline__ auto mfma_qk(u32x4 a, u32x4 b,
                                        typename std::conditional<(KIND >= 2), i32x16, f32x16>::type c) {
  if constexpr (KIND >= 2)
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c,
                                                 0, 0, 0);
  else
    return mfma16<KIND == 1>(a, b, c);
}

// Tile j has dead scores for the wavefront whose rows start at q0 (keys
// beyond N, rows beyond N, or, causal, keys after some row) exactly when
// j >= first_masked_tile(q0): with rows past N every tile has them; else
// j*64 + 64 > N holds from j = floor(N / 64) on, and j*64 + 63 > q0 from
// j = floor((q0 + 1) / 64) on.
template <bool CAUSAL>
__device__ __forceinline__ int first_masked_tile(const AttnArgs& p, int q0) {
  if (q0 + kRowsPerWave > p.N) return 0;
  const int jn = p.N / kBk;
  return CAUSAL ? min(jn, (q0 + 1) / kBk) : jn;
}

// Dead scores of one tile set to -inf in place: keys beyond N, causal future,
// rows beyond N (only diagonal and ragged tiles, j >= jm, need it).
template <bool CAUSAL>
__device__ __forceinline__ void mask_scores(const AttnArgs& p, f32x16 (&sv)[2], int j, int jm, int qrow, bool qvalid,
                                            int hl) {
  if (j >= jm) {
    // key = j*64 + 4*hl + off(t, r) is dead iff key > last, the last visible
    // key of this row (-1 for a row beyond N): off > last - j*64 - 4*hl
    const int last = !qvalid ? -1 : (CAUSAL ? min(qrow, p.N - 1) : p.N - 1);
    const int thr = last - j * kBk - 4 * hl;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 32 * t + 8 * (r >> 2) + (r & 3);
        sv[t][r] = off > thr ? kNegInf : sv[t][r];
      }
  }
}

// ---------------------------------------------------------------------------
// Pass 1: running max, row sums, lambda votes; K only
// ---------------------------------------------------------------------------
// Live K tiles of query block i (the causal ones end at the diagonal)
template <bool CAUSAL>
__device__ __forceinline__ int live_tiles(const AttnArgs& p, int i) {
  const int last_q = min(p.N, (i + 1) * kBq) - 1;
  return CAUSAL ? min(p.Tn, last_q / kBk + 1) : p.Tn;
}

// Dense query blocks (those whose list holds every live tile, so the list
// is 0, 1, ..., live - 1) of one (b, kv head), heaviest first (block index
// descending, then query head), in packs of kPackBlocks; the last pack is
// padded with -1.  One workgroup of 1024 threads per (b, kv head).  It also
// resets the kv head's pack queue, and workgroup 0 the partial counters.
template <bool CAUSAL>
__global__ __launch_bounds__(1024) void build_packs(AttnArgs p) {
  __shared__ int wsum[16];
  const int g = blockIdx.x, b = g / p.Hkv, hk = g % p.Hkv;
  const int G = p.H / p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (g == 0)
    for (int x = tid; x < kCountSlots * SPARGE_NUM_COUNTERS; x += 1024) p.cnt_part[x] = 0ull;
  const int n_cand = G * p.Tm;
  int32_t* out = p.packs + (long long)g * pack_slots(p.H, p.Hkv, p.Tm);
  int base = 0;
  for (int c0 = 0; c0 < n_cand; c0 += 1024) {
    const int c = c0 + tid;
    bool dense = false;
    int row = 0;
    if (c < n_cand) {
      const int i = p.Tm - 1 - c / G;
      row = (b * p.H + hk * G + c % G) * p.Tm + i;
      dense = p.row_cnt[row] == live_tiles<CAUSAL>(p, i);
    }
    const unsigned long long bal = __ballot(dense);
    if (lane == 0) wsum[wave] = (int)__popcll(bal);
    __syncthreads();
    int off = 0, tot = 0;
    for (int w = 0; w < 16; ++w) {
      const int x = wsum[w];
      off += w < wave ? x : 0;
      tot += x;
    }
    if (dense) out[base + off + (int)__popcll(bal & ((1ull << lane) - 1ull))] = row;
    base += tot;
    __syncthreads();
  }
  const int np = (base + kPackBlocks - 1) / kPackBlocks;
  for (int x = base + tid; x < np * kPackBlocks; x += 1024) out[x] = -1;
  if (tid == 0) {
    p.npack[g] = np;
    p.pack_next[g] = 0;
  }
}

// counters = the sums of the partial counters
__global__ void sum_counts(AttnArgs p) {
  const int c = threadIdx.x;
  if (c >= SPARGE_NUM_COUNTERS) return;
  unsigned long long t = 0;
  for (int s = 0; s < kCountSlots; ++s) t += p.cnt_part[s * SPARGE_NUM_COUNTERS + c];
  p.counts[c] = t;
}

// NP = 1: one workgroup of 4 wavefronts per query block that lists some but
// not all of its live tiles (all blocks when p.packs is null).  The block's
// listed K tiles stream through a two-slot LDS ring, one barrier per tile.
// A wavefront keeps only the scores of the current tile, and the LDS of a
// workgroup (two 16 KB slots, the list, the votes) stays under a quarter of
// the CU's 160 KB, so four workgroups share a CU: four wavefronts per SIMD
// hide each other's MFMA, exponential and LDS latencies.
// NP = kPackBlocks: one workgroup of 4 NP wavefronts per pack of dense query
// blocks of one kv head (build_packs).  Their lists are prefixes of one
// another, so one K stream serves all of them: the workgroup walks the
// longest list, and a block whose list has ended only takes its share of the
// tile loads and the barriers.  With pairs (NP = 2), two workgroups share a
// CU, four wavefronts per SIMD, and drift against each other as the single
// workgroups do; one workgroup of four blocks per CU measured slower.
// The next pack of dense blocks for this workgroup (pick: 2 ints of shared
// memory).  Each (b, kv head) hands out its packs in order, heaviest first,
// from a counter.  Workgroups go to the 8 XCDs round robin (id % 8), and the
// workgroups of XCD x start at kv head x ng / 8 of the ng, moving on to the
// next kv heads once those are handed out.  So the workgroups resident on
// one XCD hold neighbouring packs (one kv head, close block indices) that
// start together and walk the same K tiles through its L2, different XCDs
// read different K, and an XCD whose kv heads run out takes over the rest of
// the others'.  r0 is the pack's first (heaviest) row id, r the one of slot
// `member` (-1 for a padding slot); false when every queue is empty.
template <int NP>
__device__ __forceinline__ bool take_pack(const AttnArgs& p, int* pick, int member, int& r0, int& r) {
  const int per = pack_slots(p.H, p.Hkv, p.Tm);
  const int ng = p.B * p.Hkv;
  if (threadIdx.x == 0) {
    const int g0 = (int)((long long)(blockIdx.x % 8u) * ng / 8);
    int pg = -1, pk = 0;
    for (int s = 0; s < ng && pg < 0; ++s) {
      const int gg = (g0 + s) % ng;
      // the queue head only grows, so an old value never hides packs left
      if (__hip_atomic_load(p.pack_next + gg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= p.npack[gg])
        continue;
      const int kk = atomicAdd(p.pack_next + gg, 1);
      if (kk < p.npack[gg]) {
        pg = gg;
        pk = kk;
      }
    }
    pick[0] = pg;
    pick[1] = pk;
  }
  __syncthreads();
  const int g = pick[0], k = pick[1];
  if (g < 0) return false;
  const int32_t* pr = p.packs + (long long)g * per + (long long)k * NP;
  // the slots are wavefront-uniform
  r0 = __builtin_amdgcn_readfirstlane(pr[0]);
  r = __builtin_amdgcn_readfirstlane(pr[__builtin_amdgcn_readfirstlane(member)]);
  return true;
}

template <int D, int KIND, bool CAUSAL, int NP>
__global__ __launch_bounds__(NP * kThreads) __attribute__((amdgpu_waves_per_eu(4)))
void attn_stats(AttnArgs p) {
  using G = Geo<D, KIND>;
  using Acc = typename std::conditional<G::I8, i32x16, f32x16>::type;
  constexpr bool PACK = NP > 1;
  constexpr int NW = NP * kWavesPerBlock;
  constexpr int NT = NP * kThreads;
  using LN = Lane<D, KIND, NW>;
  constexpr int NSLOT = PACK ? PackRing<G::I8>::slots : kStatsSlots;
  constexpr int PD = PACK ? PackRing<G::I8>::ahead : kStatsAhead;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __shared__ unsigned long long red[NW][4];
  __shared__ int pick[2];

  if (path_is(p, kPathFused)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int member = wave / kWavesPerBlock, wq = wave % kWavesPerBlock;
  int b, h, i;
  int UC;                     // this block's list length
  int UCU;                    // entries the workgroup walks (the longest list)
  bool active = true;         // the wavefront's pack slot holds a block
  if constexpr (!PACK) {
    if (!map_block(p, p.Tm, b, h, i)) return;
    UC = p.row_cnt[(long long)(b * p.H + h) * p.Tm + i];
    if (p.packs != nullptr && UC == live_tiles<CAUSAL>(p, i)) return;   // a packed dense block
    UCU = UC;
  } else {
    // the next pack from the per-kv-head queues (take_pack); the grid has a
    // workgroup for every pack slot, and those that find every queue empty
    // return
    int r0, r;
    if (!take_pack<NP>(p, pick, member, r0, r)) return;
    active = r >= 0;
    r = active ? r : r0;
    i = r % p.Tm;
    h = (r / p.Tm) % p.H;
    b = r / p.Tm / p.H;
    UC = active ? live_tiles<CAUSAL>(p, i) : 0;
    UCU = live_tiles<CAUSAL>(p, r0 % p.Tm);
  }
  LN L;
  L.init(p, b, h, i, wq);
  const int jm = __builtin_amdgcn_readfirstlane(first_masked_tile<CAUSAL>(p, L.q0));   // q0 is wavefront-uniform
  const long long row_id = L.row_id;
  const int last_q = min(p.N, (i + 1) * kBq) - 1;
  const int n_live = live_tiles<CAUSAL>(p, i);

  // LDS: K ring | the block's list (NP = 1) | votes (2 bits per wavefront and
  // entry) | int8 K scales of the walked entries
  const int nwords = (p.Tn + 15) / 16;
  unsigned char* ring = smem;
  uint16_t* lst = reinterpret_cast<uint16_t*>(smem + NSLOT * G::K_BYTES);
  uint32_t* votes = reinterpret_cast<uint32_t*>(smem + NSLOT * G::K_BYTES + (PACK ? 0 : 2 * ((p.Tn + 1) & ~1)));
  float* ksc = reinterpret_cast<float*>(votes + NW * nwords);
  {
    const float* kscale_row = G::I8 ? p.k_scale + (long long)(b * p.Hkv + L.hk) * p.Tn : nullptr;
    if constexpr (PACK) {
      if constexpr (G::I8)
        for (int e = tid; e < UCU; e += NT) ksc[e] = kscale_row[e];
    } else {
      const uint16_t* gl = p.row_idx + row_id * p.Tn;
      for (int e = tid; e < UC; e += NT) {
        const int j = gl[e];
        lst[e] = (uint16_t)j;
        if constexpr (G::I8) ksc[e] = kscale_row[j];
      }
    }
  }
  __syncthreads();
  const uint32_t ring_lds = lds_addr(ring);
  // tile of entry e (a packed list is 0, 1, 2, ...)
  auto entry_tile = [&](int e) -> int { return PACK ? e : (int)lst[e]; };

  float m_run = kNegInf;      // running max, log2 units
  float l_half = 0.0f;        // this lane half's share of the row sum
  uint32_t vw = 0;            // votes of the current 16 entries

  // tile(e): entry e's scores and softmax for this wavefront (the tile has
  // landed in slot SL and the workgroup has passed the barrier that covers it)
  // The refill of the other slot is issued after this tile's first operand
  // reads, so its address arithmetic runs in the shadow of the MFMAs instead
  // of delaying them.
  constexpr int KLA = 2;      // k-steps the operand reads run ahead of the MFMAs
  auto tile = [&](int e, auto slot_c, auto&& refill) {
    constexpr int SL = decltype(slot_c)::value;
    const int j = __builtin_amdgcn_readfirstlane(entry_tile(e));
    float c_scale = p.scale_log2;
    if constexpr (G::I8) c_scale = L.qscale * ksc[e] * p.scale_log2;
    // K operands in k-step order, both 32-key halves per step, so the two
    // accumulator chains alternate and each operand is read a few steps
    // before its MFMA
    const unsigned char* kt = ring + SL * G::K_BYTES;
    u32x4 kf[G::QS][2];
#pragma unroll
    for (int s = 0; s < G::QS; ++s) {
      if (s == 1) refill();
#pragma unroll
      for (int t = 0; t < 2; ++t)
        kf[s][t] = *reinterpret_cast<const u32x4*>(kt + t * 32 * G::KROW + (L.k_rd ^ (32u * s)));
    }
    Acc acc[2] = {Acc{}, Acc{}};
#pragma unroll
    for (int s = 0; s < G::QS; ++s)
#pragma unroll
      for (int t = 0; t < 2; ++t) acc[t] = mfma_qk<KIND>(kf[s][t], L.qf[s], acc[t]);
    // issue order: the reads run KLA k-steps ahead of the MFMAs that use them
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * KLA, 0);
#pragma unroll
    for (int s = 0; s < G::QS - KLA; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * KLA, 0);
    // ---- online softmax (eq. 1) in log2 units; the scale is folded into an FMA ----
    // The scores as floats, masked in place, and the row max: 4 independent
    // chains of 8 values, then 4 -> 1.  An int8 tile without dead scores
    // takes the max on the int32 sums instead (exact in float: at most
    // 127 * 127 * 128 < 2^24 in magnitude) and converts the scores only when
    // its exponentials run.
    f32x16 sv[2];
    float mx;
    bool have_sv = true;
    if constexpr (G::I8) {
      if (j < jm) {
        int mi[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int o = 8 * (q & 1);
          int m = max(acc[q >> 1][o], acc[q >> 1][o + 1]);
#pragma unroll
          for (int x = 2; x < 8; x += 2) m = max(max(m, acc[q >> 1][o + x]), acc[q >> 1][o + x + 1]);
          mi[q] = m;
        }
        mx = (float)max_halves_i(max(max(mi[0], mi[1]), max(mi[2], mi[3])));
        have_sv = false;
      }
    }
    auto to_float = [&]() {
      if constexpr (G::I8) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[t][r] = (float)acc[t][r];
      } else {
        sv[0] = acc[0];
        sv[1] = acc[1];
      }
    };
    if (have_sv) {
      to_float();
      mask_scores<CAUSAL>(p, sv, j, jm, L.qrow, L.qvalid, L.hl);
      float mq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int o = 8 * (q & 1);
        float m = kNegInf;
#pragma unroll
        for (int x = 0; x < 8; x += 2) m = fmaxf(fmaxf(m, sv[q >> 1][o + x]), sv[q >> 1][o + x + 1]);
        mq[q] = m;
      }
      mx = max_halves(fmaxf(fmaxf(fmaxf(mq[0], mq[1]), mq[2]), mq[3]));
    }
    const float mloc = mx * c_scale;               // c_scale > 0: max commutes with the scale
    const float m_new = max_nn(m_run, mloc);
    const bool finite_row = mloc > kNegInf;
    // lambda vote over the wavefront's 32 rows
    // (ballots of single compares, so each is the compare's lane mask)
    const unsigned long long fin_mask = __builtin_amdgcn_ballot_w64(finite_row);
    const bool any_finite = fin_mask != 0;
    const bool exec = (fin_mask & __builtin_amdgcn_ballot_w64(!(mloc - m_new < p.lam_log2))) != 0;
    // P~ always feeds l (Algorithm 1 computes it before the M_pv test).  When
    // every row's tile maximum lies more than kFarLog2 below its running max,
    // m does not move and each P~ is below 2^-kFarLog2: the tile adds less
    // than 64 * 2^-32 to l >= 1, under half an ulp of l, so its exponentials
    // are not evaluated.
    const bool far = (fin_mask & __builtin_amdgcn_ballot_w64(!(mloc - m_new < -kFarLog2))) == 0;
    if (!far) {
      if (!have_sv) to_float();
      const float neg_m = (m_new == kNegInf) ? 0.0f : -m_new;
      const float alpha = (m_new == kNegInf) ? 1.0f : fast_exp2(m_run - m_new);
      float ps[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const f32x16& vv = sv[q >> 2];
        const int o = 4 * (q & 3);
        ps[q] = (fast_exp2(fmaf(vv[o], c_scale, neg_m)) + fast_exp2(fmaf(vv[o + 1], c_scale, neg_m))) +
                (fast_exp2(fmaf(vv[o + 2], c_scale, neg_m)) + fast_exp2(fmaf(vv[o + 3], c_scale, neg_m)));
      }
      const float psum = ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));
      l_half = alpha * l_half + psum;
    }
    m_run = m_new;
    // 1: P~V runs, 2: skipped, 3: no finite score (a vote implies a finite one)
    const uint32_t code = 3u - (any_finite ? 1u : 0u) - (exec ? 1u : 0u);
    vw |= code << (2 * (e & 15));
    if ((e & 15) == 15 || e == UC - 1) {
      votes[wave * nwords + (e >> 4)] = vw;
      vw = 0;
    }
  };

  // A ring of NSLOT K slots, PD tiles loaded ahead, one barrier per TPB
  // entries.  Single blocks (TPB = 1): at entry e's barrier its tile has
  // landed (the younger loads may still be in flight) and every wavefront is
  // done with entry e-1, whose slot then takes entry e+PD.  Pairs (TPB = PD,
  // 2 PD slots): the barrier before entries e .. e+PD-1 follows the landing
  // of all of them, and every wavefront is done with e-PD .. e-1, whose slots
  // then take e+PD .. e+2PD-1; between barriers the wavefronts drift by up
  // to PD - 1 tiles.
  static_assert(PD >= 1 && PD < NSLOT, "the refilled slot must be free");
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  int jd_v = 0;               // tile of the next refill (read one entry early)
  for (int t = 0; t < min(PD, UCU); ++t)
    L.issue_k(p, __builtin_amdgcn_readfirstlane(entry_tile(t)), ring_lds + (uint32_t)((t % NSLOT) * G::K_BYTES));
  if (UCU > 0) jd_v = entry_tile(min(PD, UCU - 1));
  // step(e): the barrier, then tile e, which refills entry e-1's slot with
  // e+PD; a packed block whose list has ended only refills
  constexpr int TPB = PACK ? PackRing<G::I8>::per : 1;
  static_assert(TPB + PD <= NSLOT && NSLOT % TPB == 0 && PD >= TPB, "a period's slots must be free");
  auto step = [&](int e, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    if constexpr (SL % TPB == 0)
      wait_pending<LN::KCW, PD - TPB>(min(UCU - 1, e + PD - 1) - min(UCU - 1, e + TPB - 1));
    auto refill = [&]() {
      const int jn = __builtin_amdgcn_readfirstlane(jd_v);
      if (e + PD < UCU) L.issue_k(p, jn, ring_lds + (uint32_t)(((SL + PD) % NSLOT) * G::K_BYTES));
      jd_v = entry_tile(min(e + PD + 1, UCU - 1));
    };
    if (!PACK || e < UC)
      tile(e, slot_c, refill);
    else
      refill();
  };
  int e = 0;
  if constexpr (NSLOT == 2) {
    for (; e + 2 <= UCU; e += 2) {
      step(e, I0{});
      step(e + 1, I1{});
    }
    if (e < UCU) step(e, I0{});
  } else if constexpr (NSLOT == 3) {
    for (; e + 3 <= UCU; e += 3) {
      step(e, I0{});
      step(e + 1, I1{});
      step(e + 2, I2{});
    }
    if (e < UCU) step(e, I0{});
    if (e + 1 < UCU) step(e + 1, I1{});
  } else if constexpr (NSLOT == 4) {
    for (; e + 4 <= UCU; e += 4) {
      step(e, I0{});
      step(e + 1, I1{});
      step(e + 2, I2{});
      step(e + 3, I3{});
    }
    if (e < UCU) step(e, I0{});
    if (e + 1 < UCU) step(e + 1, I1{});
    if (e + 2 < UCU) step(e + 2, I2{});
  } else {
    static_assert(NSLOT == 6, "two, three, four or six slots");
    using I4 = std::integral_constant<int, 4>;
    using I5 = std::integral_constant<int, 5>;
    for (; e + 6 <= UCU; e += 6) {
      step(e, I0{});
      step(e + 1, I1{});
      step(e + 2, I2{});
      step(e + 3, I3{});
      step(e + 4, I4{});
      step(e + 5, I5{});
    }
    if (e < UCU) step(e, I0{});
    if (e + 1 < UCU) step(e + 1, I1{});
    if (e + 2 < UCU) step(e + 2, I2{});
    if (e + 3 < UCU) step(e + 3, I3{});
    if (e + 4 < UCU) step(e + 4, I4{});
  }
  wait_barrier<0>();                       // every vote word is written

  // ---- the block's executed-tile list (listed tiles with a voting wavefront) ----
  const int wv0 = member * kWavesPerBlock;   // the block's first wavefront
  if (active && wq == 0) {
    uint32_t* ul = p.ulist + row_id * p.Tn;
    int n = 0;
    for (int base = 0; base < UC; base += 64) {
      const int x = base + lane;
      uint32_t m = 0, j = 0;
      if (x < UC) {
        j = (uint32_t)entry_tile(x);
#pragma unroll
        for (int w = 0; w < kWavesPerBlock; ++w) {
          const uint32_t c = (votes[(wv0 + w) * nwords + (x >> 4)] >> (2 * (x & 15))) & 3u;
          m |= (c == 1u ? 1u : 0u) << w;
        }
      }
      const unsigned long long bal = __ballot(m != 0);
      const int pos = n + (int)__popcll(bal & ((1ull << lane) - 1ull));
      if (m != 0) ul[pos] = j | (m << 16);
      n += (int)__popcll(bal);
    }
    if (lane == 0) p.ucnt[row_id] = n;
  }
  const float l_tot = sum_halves(l_half);
  if (active && L.qvalid && L.hl == 0) {
    const long long r = (long long)(b * p.H + h) * p.N + L.qrow;
    p.row_m[r] = m_run;
    p.row_l[r] = l_tot;
  }
  const int btid = tid % kThreads;          // thread index inside the block's wavefronts
  if (active && p.dbg != nullptr) {
    uint8_t* drow = p.dbg + row_id * p.Tn * kWavesPerBlock;
    for (int x = btid; x < UC * kWavesPerBlock; x += kThreads) {
      const int e2 = x / kWavesPerBlock, w = x % kWavesPerBlock;
      if (i * kBq + w * kRowsPerWave < p.N)
        drow[entry_tile(e2) * kWavesPerBlock + w] =
            (uint8_t)((votes[(wv0 + w) * nwords + (e2 >> 4)] >> (2 * (e2 & 15))) & 3u);
    }
  }

  // ---- counters: the wavefront's vote codes, counted from its vote words ----
  int n_exec = 0, n_skip = 0, n_void = 0;
  for (int x = lane; x < (UC + 15) / 16; x += 64) {
    const uint32_t w = votes[wave * nwords + x];
    const uint32_t lo = w & 0x55555555u, hi = (w >> 1) & 0x55555555u;
    n_exec += __popc(lo & ~hi);
    n_skip += __popc(hi & ~lo);
    n_void += __popc(lo & hi);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    n_exec += __shfl_xor(n_exec, o);
    n_skip += __shfl_xor(n_skip, o);
    n_void += __shfl_xor(n_void, o);
  }
  const bool empty = L.qvalid && L.hl == 0 && !(l_tot > 0.0f);
  const unsigned long long n_empty = __popcll(__ballot(empty));
  if (lane == 0) {
    red[wave][0] = (unsigned long long)n_exec;
    red[wave][1] = (unsigned long long)n_skip;
    red[wave][2] = (unsigned long long)n_void;
    red[wave][3] = n_empty;
  }
  __syncthreads();
  if (active && btid == 0) {
    unsigned long long ex = 0, sk = 0, vo = 0, em = 0;
    unsigned long long* cp = p.cnt_part + (blockIdx.x % kCountSlots) * SPARGE_NUM_COUNTERS;
    for (int w = 0; w < kWavesPerBlock; ++w) {
      // waves whose 32 rows all lie beyond N hold no group
      if (i * kBq + w * kRowsPerWave >= p.N) continue;
      ex += red[wv0 + w][0];
      sk += red[wv0 + w][1];
      vo += red[wv0 + w][2];
      em += red[wv0 + w][3];
    }
    atomicAdd(cp + SPARGE_CNT_LIVE, (unsigned long long)n_live);
    atomicAdd(cp + SPARGE_CNT_QK_EXEC, (unsigned long long)UC);
    atomicAdd(cp + SPARGE_CNT_QK_SKIP, (unsigned long long)(n_live - UC));
    atomicAdd(cp + SPARGE_CNT_PV_EXEC, ex);
    atomicAdd(cp + SPARGE_CNT_PV_SKIP, sk);
    atomicAdd(cp + SPARGE_CNT_PV_VOID, vo);
    atomicAdd(cp + SPARGE_CNT_EMPTY_ROWS, em);
    atomicAdd(cp + SPARGE_CNT_ROWS, (unsigned long long)(last_q - i * kBq + 1));
  }
}

// ---------------------------------------------------------------------------
// Pass 2: P~V on the executed tiles, then O / l
// ---------------------------------------------------------------------------
// PV8: P~V on fp8 E4M3 ([Review] Fig. 9, "SpargeAttn + Sage2"): P~ is scaled
// by 2^8 and rounded to E4M3, V^T holds E4M3 codes of V / delta_c (delta_c a
// per-channel power of two), and one v_mfma_scale_f32_32x32x64_f8f6f4 takes a
// whole 64-key tile per 32 output rows; O = delta_c * O^T / 2^8 / l.
template <int D, int KIND, bool CAUSAL, bool PV8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(pv_waves_per_eu<D, KIND, PV8>())))
void attn_pv(AttnArgs p) {
  using G = Geo<D, KIND>;
  using Acc = typename std::conditional<G::I8, i32x16, f32x16>::type;
  constexpr int NS = pv_slots<D, KIND, PV8>();
  constexpr int EB = PV8 ? G::E8_BYTES : G::E_BYTES;
  constexpr int VCWX = PV8 ? G::V8CW : G::VCW;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

  if (path_is(p, kPathFused)) return;
  int b, h, i;
  if (!map_block(p, p.Tm, b, h, i)) return;
  Lane<D, KIND, kWavesPerBlock> L;
  L.init(p, b, h, i, (int)(threadIdx.x >> 6));
  const int jm = __builtin_amdgcn_readfirstlane(first_masked_tile<CAUSAL>(p, L.q0));   // q0 is wavefront-uniform
  const int tid = L.tid, wave = L.wave, lane = L.lane, l32 = L.l32, hl = L.hl;
  const long long row_id = L.row_id;
  constexpr bool SLIST = pv_scalar_list<D, KIND, PV8>();
  const int U = __builtin_amdgcn_readfirstlane(p.ucnt[row_id]);
  const uint32_t* gul = p.ulist + row_id * p.Tn;
  const float* kscale_row = G::I8 ? p.k_scale + (long long)(b * p.Hkv + L.hk) * p.Tn : nullptr;
  uint32_t* ent = reinterpret_cast<uint32_t*>(smem + NS * EB);
  float* ksc = reinterpret_cast<float*>(ent + p.Tn);
  if constexpr (!SLIST) {
    for (int e = tid; e < U; e += kThreads) {
      const uint32_t en = gul[e];
      ent[e] = en;
      if constexpr (G::I8) ksc[e] = kscale_row[en & 0xffffu];
    }
  }
  // SLIST: entry e and its K scale (en_c, ks_c), entry e + 1 (en_n)
  uint32_t en_c = 0, en_n = 0;
  float ks_c = 0.0f;
  if constexpr (SLIST) {
    if (U > 0) {
      en_c = load_scalar(gul, 0);
      if constexpr (G::I8) ks_c = __uint_as_float(load_scalar(kscale_row, en_c & 0xffffu));
    }
    if (U > 1) en_n = load_scalar(gul, 1);
  }
  const long long srow = (long long)(b * p.H + h) * p.N + L.qrow;
  float m_row = L.qvalid ? p.row_m[srow] : kNegInf;
  float l_row = L.qvalid ? p.row_l[srow] : 0.0f;
  // both loads complete before the first tile is issued (a wait the compiler
  // placed at their first use would also wait for that tile)
  asm volatile("" : "+v"(m_row), "+v"(l_row));
  __syncthreads();

  const unsigned char* vtbase =
      reinterpret_cast<const unsigned char*>(p.vt) + ((long long)(b * p.Hkv + L.hk) * D) * p.Np * (PV8 ? 1 : 2);
  // 16-bit V^T: rows of 128 bytes, granules XOR-swizzled by row / 2
  const int v_row0 = 16 * (wave / G::VGRP) + G::VR * (wave % G::VGRP) + lane / 8;
  const uint32_t v_off = (uint32_t)(v_row0 * p.Np * 2) + (uint32_t)(((lane % 8) ^ ((v_row0 / 2) % 8)) * 16);
  const uint32_t v_wl = (uint32_t)((16 * (wave / G::VGRP) + G::VR * (wave % G::VGRP)) * G::VROW);
  const int vsw = (l32 / 2) % 8;
  const uint32_t v_rd = (uint32_t)(l32 * G::VROW) + (uint32_t)((vsw & ~1) * 16) + (uint32_t)((hl ^ (vsw & 1)) * 16);
  // fp8 V^T: rows of 64 bytes (4 granules), granule g of row m stored at
  // position g ^ ((m >> 2) & 3); a 1 KB chunk holds 16 rows, lane -> (row
  // lane / 4, position lane % 4)
  const uint32_t v8_off = (uint32_t)((lane / 4) * p.Np) + (uint32_t)(((lane % 4) ^ ((lane / 16) & 3)) * 16);
  const int f8 = (l32 >> 2) & 3;
  const uint32_t v8_rd0 = (uint32_t)(l32 * 64 + (((2 * hl) ^ f8) * 16));
  const uint32_t v8_rd1 = (uint32_t)(l32 * 64 + (((2 * hl + 1) ^ f8) * 16));
  const uint32_t ring_lds = lds_addr(smem);

  // entry e -> slot: its K tile, then its V^T tile (KCW + VCWX loads per wavefront)
  auto issue = [&](int e, int slot) {
    const int j = __builtin_amdgcn_readfirstlane(SLIST ? (int)((e == 0 ? en_c : en_n) & 0xffffu)
                                                       : (int)(ent[e] & 0xffffu));
    const uint32_t sl = ring_lds + (uint32_t)(slot * EB);
    L.issue_k(p, j, sl);
    if constexpr (PV8) {
#pragma unroll
      for (int c = 0; c < VCWX; ++c) {
        const int q = c * kWavesPerBlock + wave;            // rows 16q .. 16q + 15
        const unsigned char* base = uniform_ptr(vtbase + (long long)(16 * q) * p.Np + (long long)j * kBk);
        dma16(base, v8_off, (uint32_t)__builtin_amdgcn_readfirstlane((int)(sl + G::K_BYTES + q * 1024)));
      }
    } else {
#pragma unroll
      for (int c = 0; c < VCWX; ++c) {
        const int row_c = 16 * c * (4 / G::VGRP);
        const unsigned char* base = uniform_ptr(vtbase + ((long long)row_c * p.Np + (long long)j * kBk) * 2);
        dma16(base, v_off,
              (uint32_t)__builtin_amdgcn_readfirstlane((int)(sl + G::K_BYTES + row_c * G::VROW + v_wl)));
      }
    }
  };

  f32x16 oacc[G::OT];
#pragma unroll
  for (int t = 0; t < G::OT; ++t) oacc[t] = f32x16{};
  const float neg_m = (m_row == kNegInf) ? 0.0f : -m_row;

  // Entry e is used in step e; entries e+1 .. e+NS-2 are in flight when step
  // e starts, and step e refills the slot entry e-1 used with entry e+NS-1.
  const int pre = min(U, NS - 1);
  for (int t = 0; t < pre; ++t) issue(t, t);
  for (int e = 0; e < U; ++e) {
    const int pend = min(U - 1, e + NS - 2) - e;    // entries issued after entry e
    // (SLIST: every LDS read of the previous step fed its MFMAs, and the
    // loop writes no LDS but through the tile loads)
    wait_pending<Lane<D, KIND, kWavesPerBlock>::KCW + VCWX, NS - 2, !SLIST>(pend);
    if (e + NS - 1 < U) issue(e + NS - 1, (e + NS - 1) % NS);
    const uint32_t en = SLIST ? en_c : (uint32_t)__builtin_amdgcn_readfirstlane((int)ent[e]);
    const int j = (int)(en & 0xffffu);
    // SLIST: the next step's entries, loaded while this step runs
    float ks_n = 0.0f;
    uint32_t en_nn = 0;
    if constexpr (SLIST) {
      if constexpr (G::I8)
        if (e + 1 < U) ks_n = __uint_as_float(load_scalar(kscale_row, en_n & 0xffffu));
      if (e + 2 < U) en_nn = load_scalar(gul, e + 2);
    }
    if ((en >> (16 + wave)) & 1u) {       // this wavefront's group ran P~V on tile j
      const unsigned char* kt = smem + (e % NS) * EB;
      const unsigned char* vt = kt + G::K_BYTES;
      u32x4 kf[2][G::QS];
      L.read_k(kt, kf);
      Acc acc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        acc[t] = Acc{};
#pragma unroll
        for (int s = 0; s < G::QS; ++s) acc[t] = mfma_qk<KIND>(kf[t][s], L.qf[s], acc[t]);
      }
      float c_scale = p.scale_log2;
      if constexpr (G::I8) c_scale = L.qscale * (SLIST ? ks_c : ksc[e]) * p.scale_log2;
      f32x16 sv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[t][r] = (float)acc[t][r];
      mask_scores<CAUSAL>(p, sv, j, jm, L.qrow, L.qvalid, hl);
      if constexpr (PV8) {
        // P = exp(S - m_final) * 2^8 as E4M3: byte 16t + r of the lane's 32
        // holds sv[t][r], the key order the fp8 V^T rows use
        i32x8 pb;
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const int t = v >> 2, r0 = 4 * (v & 3);
          float y[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) y[q] = fminf(fast_exp2(fmaf(sv[t][r0 + q], c_scale, neg_m)) * 256.0f, 448.0f);
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
          pb[v] = w;
        }
        // ---- O^T += V_j^T P^T, one 64-key MFMA per 32 output rows ----
#pragma unroll
        for (int t = 0; t < G::OT; ++t) {
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(vt + t * 32 * 64 + v8_rd0);
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(vt + t * 32 * 64 + v8_rd1);
          const i32x8 av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                            (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
          oacc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pb, oacc[t], 0, 0, 0, 127, 0, 127);
        }
      } else {
        // P = exp(S - m_final), packed in the P~V input type as the B operand of 4 k-steps
        u32x4 pb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int tt = s >> 1, r0 = 8 * (s & 1);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float x0 = fast_exp2(fmaf(sv[tt][r0 + 2 * q], c_scale, neg_m));
            const float x1 = fast_exp2(fmaf(sv[tt][r0 + 2 * q + 1], c_scale, neg_m));
            pb[s][q] = pack2<G::PVBF>(x0, x1);
          }
        }
        // ---- O^T += V_j^T P^T ----
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t off = v_rd ^ (32u * s);
#pragma unroll
          for (int t = 0; t < G::OT; ++t) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(vt + t * 32 * G::VROW + off);
            oacc[t] = mfma16<G::PVBF>(a, pb[s], oacc[t]);
          }
        }
      }
    }
    if constexpr (SLIST) {
      en_c = en_n;
      ks_c = ks_n;
      en_n = en_nn;
    }
  }

  // ---- epilogue: O / l (fp8: times delta_c / 2^8) ----
  const float inv = l_row > 0.0f ? 1.0f / l_row : 0.0f;
  if constexpr (PV8) {
    const float* vs = p.vscale + (long long)(b * p.Hkv + L.hk) * D;
#pragma unroll
    for (int t = 0; t < G::OT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) oacc[t][4 * g + q] *= vs[32 * t + 8 * g + 4 * hl + q] * (1.0f / 256.0f);
  }
  if (L.qvalid && p.out_f32) {
    float* ob = static_cast<float*>(p.o) + b * p.o_sb + h * p.o_sh + (long long)L.qrow * p.o_sn;
#pragma unroll
    for (int t = 0; t < G::OT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x4 w = {__float_as_uint(oacc[t][4 * g + 0] * inv), __float_as_uint(oacc[t][4 * g + 1] * inv),
                   __float_as_uint(oacc[t][4 * g + 2] * inv), __float_as_uint(oacc[t][4 * g + 3] * inv)};
        *reinterpret_cast<u32x4*>(ob + 32 * t + 8 * g + 4 * hl) = w;
      }
  } else if (L.qvalid) {
    // each float32 quotient is materialised (the empty asm keeps the compiler
    // from fusing multiply and narrowing into one differently rounded op), so
    // this output is exactly the float32 output rounded to the 16-bit type
    unsigned short* ob =
        static_cast<unsigned short*>(p.o) + b * p.o_sb + h * p.o_sh + (long long)L.qrow * p.o_sn;
#pragma unroll
    for (int t = 0; t < G::OT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float y[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          y[q] = oacc[t][4 * g + q] * inv;
          asm volatile("" : "+v"(y[q]));
        }
        u32x2 w = {pack2<G::PVBF>(y[0], y[1]), pack2<G::PVBF>(y[2], y[3])};
        *reinterpret_cast<u32x2*>(ob + 32 * t + 8 * g + 4 * hl) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// One fused pass in Algorithm 1's order, and the pilot that chooses it
// ---------------------------------------------------------------------------
// The two passes above pay for their split with a second QK^T on every tile
// some wavefront votes for.  When most (tile, wavefront) pairs vote that is
// most of the tiles, and one pass that streams V beside K is cheaper.  The
// pilot estimates the vote rate of the call from a sample; pilot_decide
// writes the path every later kernel of the call reads.

// The factor that takes tile j's raw scores to log2 units: 1/sqrt(d) log2(e),
// times the two block scales on the int8 path (the same product, in the same
// order, as pass 1 forms).  `ks_row`: the kv head's int8 K block scales.
template <int D, int KIND, int NW>
__device__ __forceinline__ float tile_scale(const AttnArgs& p, const Lane<D, KIND, NW>& L, const float* ks_row,
                                            int j) {
  float c = p.scale_log2;
  if constexpr (Geo<D, KIND>::I8) c = L.qscale * ks_row[j] * p.scale_log2;
  return c;
}

// Row maxima of one tile of S^T for this wavefront (log2 units: the raw
// maxima times c_scale > 0): the QK^T MFMAs on the K tile at `kt`, the dead
// scores masked.  The raw scores stay in `sv` (as floats: int8 sums are
// exact in float32, below 2^24 in magnitude).
template <int D, int KIND, bool CAUSAL, int NW = kWavesPerBlock>
__device__ __forceinline__ float tile_scores(const AttnArgs& p, const Lane<D, KIND, NW>& L,
                                             const unsigned char* kt, int j, int jm, float c_scale,
                                             f32x16 (&sv)[2]) {
  using G = Geo<D, KIND>;
  using Acc = typename std::conditional<G::I8, i32x16, f32x16>::type;
  constexpr int KLA = 2;      // k-steps the operand reads run ahead of the MFMAs
  u32x4 kf[G::QS][2];
#pragma unroll
  for (int s = 0; s < G::QS; ++s)
#pragma unroll
    for (int t = 0; t < 2; ++t)
      kf[s][t] = *reinterpret_cast<const u32x4*>(kt + t * 32 * G::KROW + (L.k_rd ^ (32u * s)));
  Acc acc[2] = {Acc{}, Acc{}};
#pragma unroll
  for (int s = 0; s < G::QS; ++s)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[t] = mfma_qk<KIND>(kf[s][t], L.qf[s], acc[t]);
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * KLA, 0);
#pragma unroll
  for (int s = 0; s < G::QS - KLA; ++s) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 2 * KLA, 0);
  if constexpr (G::I8) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[t][r] = (float)acc[t][r];
  } else {
    sv[0] = acc[0];
    sv[1] = acc[1];
  }
  mask_scores<CAUSAL>(p, sv, j, jm, L.qrow, L.qvalid, L.hl);
  float mq[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int o = 8 * (q & 1);
    float m = kNegInf;
#pragma unroll
    for (int x = 0; x < 8; x += 2) m = fmaxf(fmaxf(m, sv[q >> 1][o + x]), sv[q >> 1][o + x + 1]);
    mq[q] = m;
  }
  return max_halves(fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]))) * c_scale;
}

// Pilot: sampled query block g * stride + stride / 2 of the B H Tm (in
// (b, h, i) order).  Its first listed tile seeds the running max; up to
// kPilotTiles - 1 further listed tiles, one from each equal stratum of the
// rest of the list, are visited in list order, each voting per wavefront
// against the running max of the sample so far, as the lambda rule votes
// against the running max.  Every sampled tile stands for the listed tiles
// of its stratum (the first for itself), so the counts weigh long rows by
// their work.  The workgroup's weighted votes and (tile, wavefront) pairs
// with a visible key go to its own pair of pilot_cnt slots (no atomics: one
// address shared by every workgroup serialised them); pilot_decide adds the
// slots up.  The sampled K tiles go through kPilotSlots LDS slots, that many
// loads in flight at a time.
constexpr int kPilotSlots = 4;
template <int D, int KIND>
size_t pilot_lds_bytes() {
  return (size_t)kPilotSlots * Geo<D, KIND>::K_BYTES;
}
template <int D, int KIND, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void attn_pilot(AttnArgs p, int stride) {
  static_assert(kPilotTiles % kPilotSlots == 0, "whole rounds of slots");
  static_assert(kPilotTiles - 1 <= 7 && 840 % 7 == 0, "840 = lcm(1..8) divides by every stratum count");
  using G = Geo<D, KIND>;
  using LN = Lane<D, KIND, kWavesPerBlock>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __shared__ unsigned long long part[kWavesPerBlock][2];
  const long long total = (long long)p.B * p.H * p.Tm;
  long long g = (long long)blockIdx.x * stride + stride / 2;
  if (g >= total) g = (long long)blockIdx.x * stride;
  if (g >= total) {           // (not reached: the grid is ceil(total / stride))
    if (threadIdx.x == 0)
      for (int c = 0; c < kPilotCounts; ++c) p.pilot_cnt[kPilotCounts * blockIdx.x + c] = 0;
    return;
  }
  const int i = (int)(g % p.Tm);
  const int bh = (int)(g / p.Tm);
  const int b = bh / p.H, h = bh % p.H;
  const int wave = (int)(threadIdx.x >> 6), lane = (int)(threadIdx.x & 63);
  LN L;
  L.init(p, b, h, i, wave);
  const int jm = __builtin_amdgcn_readfirstlane(first_masked_tile<CAUSAL>(p, L.q0));   // q0 is wavefront-uniform
  const int n_live = live_tiles<CAUSAL>(p, i);
  const int UC = p.row_cnt[L.row_id];
  const bool dense = UC == n_live;
  const uint16_t* gl = p.row_idx + L.row_id * p.Tn;
  const float* ks_row = G::I8 ? p.k_scale + (long long)(b * p.Hkv + L.hk) * p.Tn : nullptr;
  // the same in every wavefront of the block: strata after the first tile,
  // and tiles loaded
  const int S = UC > 1 ? min(kPilotTiles - 1, UC - 1) : 0;
  const int NL = UC > 0 ? 1 + S : 0;
  const uint32_t slots = lds_addr(smem);
  // sample k: the first listed entry (k = 0), or the middle of stratum k - 1
  // of entries 1 .. UC - 1
  auto tile_of = [&](int k) -> int {
    const int e = k == 0 ? 0 : 1 + (int)((long long)(2 * k - 1) * (UC - 1) / (2 * S));
    return __builtin_amdgcn_readfirstlane(dense ? e : (int)gl[e]);
  };
  float mk[kPilotTiles];
#pragma unroll
  for (int r0 = 0; r0 < kPilotTiles; r0 += kPilotSlots) {
    if (r0 < NL) {
#pragma unroll
      for (int u = 0; u < kPilotSlots; ++u)
        if (r0 + u < NL) L.issue_k(p, tile_of(r0 + u), slots + (uint32_t)(u * G::K_BYTES));
      wait_barrier<0>();      // the round's tiles have landed for every wavefront
#pragma unroll
      for (int u = 0; u < kPilotSlots; ++u) {
        mk[r0 + u] = kNegInf;
        if (r0 + u < NL) {
          f32x16 sv[2];
          const int j = tile_of(r0 + u);
          mk[r0 + u] = tile_scores<D, KIND, CAUSAL>(p, L, smem + u * G::K_BYTES, j, jm,
                                                    tile_scale(p, L, ks_row, j), sv);
        }
      }
      __syncthreads();        // every wavefront is done with the slots
    } else {
#pragma unroll
      for (int u = 0; u < kPilotSlots; ++u) mk[r0 + u] = kNegInf;
    }
  }
  // the first tile votes wherever a row sees a key (m_new = its own max)
  unsigned long long v_first = wave_any(mk[0] > kNegInf) ? 1 : 0;
  unsigned long long votes = 0, pairs = 0;
  float m_run = mk[0];
#pragma unroll
  for (int k = 1; k < kPilotTiles; ++k) {
    if (k < NL) {
      const float m_new = fmaxf(m_run, mk[k]);
      const bool fin = mk[k] > kNegInf;
      const bool v = fin && !(mk[k] - m_new < p.lam_log2);
      if (wave_any(fin)) {
        pairs += 1;
        votes += wave_any(v) ? 1 : 0;
      }
      m_run = m_new;
    }
  }
  const unsigned long long w_first = 840, w_stratum = S > 0 ? (unsigned long long)(UC - 1) * (840 / S) : 0;
  if (lane == 0) {
    part[wave][0] = votes * w_stratum + v_first * w_first;
    part[wave][1] = pairs * w_stratum + v_first * w_first;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long v = 0, n = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
      v += part[w][0];
      n += part[w][1];
    }
    unsigned long long* pc = p.pilot_cnt + kPilotCounts * blockIdx.x;
    pc[0] = v;
    pc[1] = n;
    pc[2] = (unsigned long long)UC;       // the sampled block's listed tiles
    pc[3] = 1;
  }
}

// The call's path: the requested one, or for kPathAuto the fused pass when
// at least nine tenths of the pilot's weighted (tile, wavefront) pairs voted,
// or when the sampled blocks list at most `mean_tiles` tiles on average.
// A short sample sets new maxima more often than the whole row does, so the
// pilot overstates lower rates and hardly separates them: it reads 0.64 to
// 0.72 on the llm recipe from N 4096 (36% of the pairs vote) to 131072 (5%),
// and 1.0 where all vote (image, video).  The fused pass wins near full
// rates (about 30% faster on image and video) and on short rows: bf16 9 to
// 21% faster at N 8192 to 32768 (some 150 listed tiles per block or fewer),
// fp8 P~V (half the V bytes) 4 to 23% faster up to 65536 (some 300), int8
// Q/K, whose first pass costs less, 6 to 20% at N 8192 and 16384 (some 80
// or fewer) but 15% slower at 32768, and int8 Q/K with fp8 P~V 14% faster
// at 8192 (some 40) but 4% slower at 16384.  It loses on long rows of low
// rates (bf16 15% slower at 131072, fp8 8%; int8 17% at 65536).
// `groups`: the pilot's workgroups (0 when the path is forced).
__global__ void pilot_decide(AttnArgs p, int groups, int mean_tiles) {
  unsigned long long v = 0, n = 0, uc = 0, nb = 0;
  for (int x = (int)threadIdx.x; x < groups; x += 64) {
    const unsigned long long* pc = p.pilot_cnt + kPilotCounts * x;
    v += pc[0];
    n += pc[1];
    uc += pc[2];
    nb += pc[3];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    v += __shfl_xor(v, o);
    n += __shfl_xor(n, o);
    uc += __shfl_xor(uc, o);
    nb += __shfl_xor(nb, o);
  }
  if (threadIdx.x != 0) return;
  int path = p.path;
  if (path != kPathTwoPass && path != kPathFused)
    path = (n > 0 && (10 * v >= 9 * n || uc <= (unsigned long long)mean_tiles * nb)) ? kPathFused
                                                                                      : kPathTwoPass;
  *p.path_flag = path;
}

// The fused pass runs dense blocks in packs only when rows are long: a mean
// of at least 192 live tiles per query block (Tn, or Tn / 2 causal).  Packs
// halve the K and V^T streams but couple two blocks' wavefronts at every
// barrier; on short rows that costs more than it saves (llm recipe: 0.43
// against 0.38 ms at N 8192, 3.56 against 3.97 ms at 32768; video 24.96
// against 25.45 ms).
template <bool CAUSAL>
__device__ __forceinline__ bool fused_packs(const AttnArgs& p) {
  return (CAUSAL ? p.Tn / 2 : p.Tn) >= 192;
}

// the fused pass's ring: bytes of a (K, V^T) slot (fp8 V^T with PV8), and
// slots: four for a pack; for a single block as many as keep the ring at
// 64 KB (two or four)
template <int D, int KIND, bool PV8>
constexpr int fused_slot_bytes() {
  return PV8 ? Geo<D, KIND>::E8_BYTES : Geo<D, KIND>::E_BYTES;
}
template <int D, int KIND, int NP, bool PV8>
constexpr int fused_slots() {
  return NP > 1 ? 4 : ((65536 / fused_slot_bytes<D, KIND, PV8>()) >= 4 ? 4 : 2);
}
template <int D, int KIND, int NP, bool PV8>
size_t fused_lds_bytes(int Tn) {
  return (size_t)fused_slots<D, KIND, NP, PV8>() * fused_slot_bytes<D, KIND, PV8>() +
         (NP == 1 ? (size_t)2 * ((Tn + 1) & ~1) : 0) + (size_t)4 * NP * kWavesPerBlock * ((Tn + 15) / 16);
}

// The fused pass: the query blocks of a call in the grid order of attn_pv
// (NP = 1, one workgroup of 4 wavefronts each), except the dense ones, which
// run in the packs of attn_stats (NP = 2, one workgroup of 8 wavefronts per
// pack of two blocks of one kv head, handed out from the same per-kv-head
// queues): the pack's blocks list the same tiles (prefixes, causal), so one
// stream of K and V^T tiles through a ring of LDS slots (the slots and loads
// of attn_pv) serves both.  Per tile, as Algorithm 1 orders it: S = Q K^T,
// the running max m and row sum l (eq. 1), the wavefront's lambda vote, and,
// when the vote runs P~V, O = exp(m_old - m_new) O + P~ V with P~ = exp(S -
// m_new) rounded to V's type (PV8: 2^8 P~ rounded to E4M3 at the running
// max, as Algorithm 1 orders the steps, against attn_pv's fp8 V^T, and the
// sum scaled by delta_c / 2^8 at the end).  A tile whose rows all lie more
// than kFarLog2 below their running max leaves m, l and O as they are (their
// P~ are below 2^-32; see attn_stats); its vote is still counted.  The votes,
// the decision map and the counters are those of attn_stats.
template <int D, int KIND, bool CAUSAL, int NP, bool PV8>
__global__ __launch_bounds__(NP * kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fused(AttnArgs p) {
  using G = Geo<D, KIND>;
  constexpr bool PACK = NP > 1;
  constexpr int NW = NP * kWavesPerBlock;
  constexpr int NT = NP * kThreads;
  using LN = Lane<D, KIND, NW>;
  // ring slots, tiles loaded ahead, tiles per barrier: a pack's workgroup
  // (alone on its CU) passes one barrier per two tiles, as pass 1's pairs do
  constexpr int NS = fused_slots<D, KIND, NP, PV8>();
  constexpr int PD = PACK ? 2 : NS - 1;
  constexpr int TPB = PACK ? 2 : 1;
  constexpr int EB = fused_slot_bytes<D, KIND, PV8>();
  // 1 KB chunks of a V^T tile, and per loading wavefront.  Where a tile has
  // fewer chunks (of K or V^T) than the workgroup has wavefronts, some load
  // fewer than others, and each barrier must then wait for every load.
  constexpr int VCH = (PV8 ? G::V8_BYTES : G::V_BYTES) / 1024;
  constexpr int VCWN = VCH >= NW ? VCH / NW : 1;
  static_assert(VCH % NW == 0 || (VCH < NW && PD == TPB), "V^T tiles must split over the wavefronts");
  static_assert(G::KCH % NW == 0 || (G::KCH < NW && PD == TPB), "K tiles must split over the wavefronts");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __shared__ unsigned long long red[NW][4];
  __shared__ int pick[2];

  if (!path_is(p, kPathFused)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int member = wave / kWavesPerBlock, wq = wave % kWavesPerBlock;
  int b, h, i;
  int UC;                     // this block's list length
  int UCU;                    // entries the workgroup walks (the longest list)
  bool active = true;         // the wavefront's pack slot holds a block
  if constexpr (!PACK) {
    if (!map_block(p, p.Tm, b, h, i)) return;
    UC = p.row_cnt[(long long)(b * p.H + h) * p.Tm + i];
    // a dense block taken by the pack kernel
    if (p.packs != nullptr && fused_packs<CAUSAL>(p) && UC == live_tiles<CAUSAL>(p, i)) return;
    UCU = UC;
  } else {
    if (!fused_packs<CAUSAL>(p)) return;
    int r0, r;
    if (!take_pack<NP>(p, pick, member, r0, r)) return;
    active = r >= 0;
    r = active ? r : r0;
    i = r % p.Tm;
    h = (r / p.Tm) % p.H;
    b = r / p.Tm / p.H;
    UC = active ? live_tiles<CAUSAL>(p, i) : 0;
    UCU = live_tiles<CAUSAL>(p, r0 % p.Tm);
  }
  LN L;
  L.init(p, b, h, i, wq);
  const int jm = __builtin_amdgcn_readfirstlane(first_masked_tile<CAUSAL>(p, L.q0));   // q0 is wavefront-uniform
  const int l32 = L.l32, hl = L.hl;
  const long long row_id = L.row_id;
  const int last_q = min(p.N, (i + 1) * kBq) - 1;
  const int n_live = live_tiles<CAUSAL>(p, i);
  const bool dense = PACK || UC == n_live;     // the list is 0, 1, ..., live - 1
  const float* ks_row = G::I8 ? p.k_scale + (long long)(b * p.Hkv + L.hk) * p.Tn : nullptr;
  const int nwords = (p.Tn + 15) / 16;
  uint16_t* lst = reinterpret_cast<uint16_t*>(smem + NS * EB);
  uint32_t* votes = reinterpret_cast<uint32_t*>(smem + NS * EB + (PACK ? 0 : 2 * ((p.Tn + 1) & ~1)));
  if (!dense) {
    const uint16_t* gl = p.row_idx + row_id * p.Tn;
    for (int e = tid; e < UC; e += NT) lst[e] = gl[e];
  }
  __syncthreads();
  auto entry_tile = [&](int e) -> int { return dense ? e : (int)lst[e]; };

  // 16-bit V^T tiles: rows of 128 bytes, granules XOR-swizzled by row / 2
  // (attn_pv); wavefront w loads rows 8w .. 8w + 7 of every 8 NW rows.  fp8
  // V^T (PV8): attn_pv's layout, 1 KB chunk q (rows 16q .. 16q + 15) loaded
  // by wavefront q % NW.
  const unsigned char* vtbase =
      reinterpret_cast<const unsigned char*>(p.vt) + ((long long)(b * p.Hkv + L.hk) * D) * p.Np * (PV8 ? 1 : 2);
  const uint32_t v8_off = (uint32_t)((lane / 4) * p.Np) + (uint32_t)(((lane % 4) ^ ((lane / 16) & 3)) * 16);
  const int f8 = (l32 >> 2) & 3;
  const uint32_t v8_rd0 = (uint32_t)(l32 * 64 + (((2 * hl) ^ f8) * 16));
  const uint32_t v8_rd1 = (uint32_t)(l32 * 64 + (((2 * hl + 1) ^ f8) * 16));
  const int v_row0 = 16 * (wave / G::VGRP) + G::VR * (wave % G::VGRP) + lane / 8;
  const uint32_t v_off = (uint32_t)(v_row0 * p.Np * 2) + (uint32_t)(((lane % 8) ^ ((v_row0 / 2) % 8)) * 16);
  const uint32_t v_wl = (uint32_t)((16 * (wave / G::VGRP) + G::VR * (wave % G::VGRP)) * G::VROW);
  const int vsw = (l32 / 2) % 8;
  const uint32_t v_rd = (uint32_t)(l32 * G::VROW) + (uint32_t)((vsw & ~1) * 16) + (uint32_t)((hl ^ (vsw & 1)) * 16);
  const uint32_t ring_lds = lds_addr(smem);
  auto issue = [&](int e, int slot) {
    const int j = __builtin_amdgcn_readfirstlane(entry_tile(e));
    const uint32_t sl = ring_lds + (uint32_t)(slot * EB);
    L.issue_k(p, j, sl);
    if constexpr (PV8) {
#pragma unroll
      for (int c = 0; c < VCWN; ++c) {
        const int q = c * NW + wave;
        if (q < VCH) {
          const unsigned char* base = uniform_ptr(vtbase + (long long)(16 * q) * p.Np + (long long)j * kBk);
          dma16(base, v8_off, (uint32_t)__builtin_amdgcn_readfirstlane((int)(sl + G::K_BYTES + q * 1024)));
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < VCWN; ++c) {
        const int row_c = 16 * c * (NW / G::VGRP);
        const unsigned char* base = uniform_ptr(vtbase + ((long long)row_c * p.Np + (long long)j * kBk) * 2);
        dma16(base, v_off,
              (uint32_t)__builtin_amdgcn_readfirstlane((int)(sl + G::K_BYTES + row_c * G::VROW + v_wl)));
      }
    }
  };

  f32x16 oacc[G::OT];
#pragma unroll
  for (int t = 0; t < G::OT; ++t) oacc[t] = f32x16{};
  float m_run = kNegInf;      // running max, log2 units
  float l_half = 0.0f;        // this lane half's share of the row sum
  int n_exec = 0, n_skip = 0, n_void = 0;
  uint32_t vw = 0;

  // Entry e is used in step e, and step e loads entry e+PD into the slot of
  // entry e+PD-NS.  Single blocks (TPB = 1, PD = NS-1): at step e's barrier
  // entry e has landed (e+1 .. e+NS-2 may still be in flight) and every
  // wavefront is done with e-1.  Packs (TPB = PD = 2, four slots): the
  // barrier before entries e and e+1 follows the landing of both, and every
  // wavefront is done with e-2 and e-1, whose slots then take e+2 and e+3;
  // between barriers the wavefronts drift by up to a tile.  The steps run NS
  // at a time with the slot a constant, so its LDS offsets fold into the
  // reads.  A packed block whose list has ended only loads.
  const int pre = min(UCU, PD);
  for (int t = 0; t < pre; ++t) issue(t, t);
  static_assert(TPB + PD <= NS && NS % TPB == 0 && PD >= TPB, "a period's slots must be free");
  auto step = [&](int e, auto slot_c) {
    constexpr int SL = decltype(slot_c)::value;
    if constexpr (SL % TPB == 0)
      wait_pending<LN::KCW + VCWN, PD - TPB>(min(UCU - 1, e + PD - 1) - min(UCU - 1, e + TPB - 1));
    if (e + PD < UCU) issue(e + PD, (SL + PD) % NS);
    if (PACK && e >= UC) return;
    const int j = __builtin_amdgcn_readfirstlane(entry_tile(e));
    const unsigned char* kt = smem + SL * EB;
    const unsigned char* vt = kt + G::K_BYTES;
    f32x16 sv[2];
    const float c_scale = tile_scale(p, L, ks_row, j);
    const float mloc = tile_scores<D, KIND, CAUSAL, NW>(p, L, kt, j, jm, c_scale, sv);
    const float m_new = max_nn(m_run, mloc);
    const bool finite_row = mloc > kNegInf;
    // (ballots of single compares, so each is the compare's lane mask)
    const unsigned long long fin_mask = __builtin_amdgcn_ballot_w64(finite_row);
    const bool any_finite = fin_mask != 0;
    const bool exec = (fin_mask & __builtin_amdgcn_ballot_w64(!(mloc - m_new < p.lam_log2))) != 0;
    const bool far = (fin_mask & __builtin_amdgcn_ballot_w64(!(mloc - m_new < -kFarLog2))) == 0;
    if (!far) {
      // P~ against the running max itself, so a row's largest score gives
      // exactly 1 (a trailing reference saved O rescales but rounded that
      // dominant term to 16 bits too: 2^-9 of its V value, over 1e-2 where
      // |V| > 5)
      const float neg_m = (m_new == kNegInf) ? 0.0f : -m_new;
      const float alpha = (m_new == kNegInf) ? 1.0f : fast_exp2(m_run - m_new);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) sv[t][r] = fast_exp2(fmaf(sv[t][r], c_scale, neg_m));
      float ps[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const f32x16& vv = sv[q >> 2];
        const int o = 4 * (q & 3);
        ps[q] = (vv[o] + vv[o + 1]) + (vv[o + 2] + vv[o + 3]);
      }
      l_half = alpha * l_half + (((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7])));
      if (wave_any(alpha != 1.0f)) {
#pragma unroll
        for (int t = 0; t < G::OT; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[t][r] *= alpha;
      }
      if (exec && PV8) {
        // 2^8 P~ as E4M3 (P~ <= 1 at the running max, so 2^8 P~ <= 256 is in
        // range): byte 16t + r of the lane's 32 holds sv[t][r], the key order
        // of the fp8 V^T rows; then one 64-key MFMA per 32 rows of O^T
        i32x8 pb8;
#pragma unroll
        for (int x = 0; x < 8; ++x) {
          const int t = x >> 2, r0 = 4 * (x & 3);
          float y[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) y[q] = fminf(sv[t][r0 + q] * 256.0f, 448.0f);
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
          pb8[x] = w;
        }
#pragma unroll
        for (int t = 0; t < G::OT; ++t) {
          const u32x4 a0 = *reinterpret_cast<const u32x4*>(vt + t * 32 * 64 + v8_rd0);
          const u32x4 a1 = *reinterpret_cast<const u32x4*>(vt + t * 32 * 64 + v8_rd1);
          const i32x8 av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                            (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
          oacc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pb8, oacc[t], 0, 0, 0, 127, 0, 127);
        }
      } else if (exec) {
        // P~ in V's type as the B operand of 4 k-steps, then O^T += V_j^T P~^T
        u32x4 pb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int tt = s >> 1, r0 = 8 * (s & 1);
#pragma unroll
          for (int q = 0; q < 4; ++q) pb[s][q] = pack2<G::PVBF>(sv[tt][r0 + 2 * q], sv[tt][r0 + 2 * q + 1]);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t off = v_rd ^ (32u * s);
#pragma unroll
          for (int t = 0; t < G::OT; ++t) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(vt + t * 32 * G::VROW + off);
            oacc[t] = mfma16<G::PVBF>(a, pb[s], oacc[t]);
          }
        }
      }
    }
    m_run = m_new;
    const uint32_t code = exec ? 1u : (any_finite ? 2u : 3u);
    n_exec += exec ? 1 : 0;
    n_skip += (!exec && any_finite) ? 1 : 0;
    n_void += any_finite ? 0 : 1;
    vw |= code << (2 * (e & 15));
    if ((e & 15) == 15 || e == UC - 1) {
      votes[wave * nwords + (e >> 4)] = vw;
      vw = 0;
    }
  };
  static_assert(NS == 2 || NS == 4, "the fused ring has two or four slots");
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  int e = 0;
  if constexpr (NS == 2) {
    for (; e + 2 <= UCU; e += 2) {
      step(e, I0{});
      step(e + 1, I1{});
    }
    if (e < UCU) step(e, I0{});
  } else {
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    for (; e + 4 <= UCU; e += 4) {
      step(e, I0{});
      step(e + 1, I1{});
      step(e + 2, I2{});
      step(e + 3, I3{});
    }
    if (e < UCU) step(e, I0{});
    if (e + 1 < UCU) step(e + 1, I1{});
    if (e + 2 < UCU) step(e + 2, I2{});
  }
  wait_barrier<0>();                       // every vote word is written

  // ---- epilogue: O / l, as attn_pv stores it (fp8: times delta_c / 2^8) ----
  const float l_tot = sum_halves(l_half);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if constexpr (PV8) {
    const float* vs = p.vscale + (long long)(b * p.Hkv + L.hk) * D;
#pragma unroll
    for (int t = 0; t < G::OT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) oacc[t][4 * g + q] *= vs[32 * t + 8 * g + 4 * hl + q] * (1.0f / 256.0f);
  }
  if (active && L.qvalid && p.out_f32) {
    float* ob = static_cast<float*>(p.o) + b * p.o_sb + h * p.o_sh + (long long)L.qrow * p.o_sn;
#pragma unroll
    for (int t = 0; t < G::OT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x4 w = {__float_as_uint(oacc[t][4 * g + 0] * inv), __float_as_uint(oacc[t][4 * g + 1] * inv),
                   __float_as_uint(oacc[t][4 * g + 2] * inv), __float_as_uint(oacc[t][4 * g + 3] * inv)};
        *reinterpret_cast<u32x4*>(ob + 32 * t + 8 * g + 4 * hl) = w;
      }
  } else if (active && L.qvalid) {
    unsigned short* ob =
        static_cast<unsigned short*>(p.o) + b * p.o_sb + h * p.o_sh + (long long)L.qrow * p.o_sn;
#pragma unroll
    for (int t = 0; t < G::OT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float y[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          y[q] = oacc[t][4 * g + q] * inv;
          asm volatile("" : "+v"(y[q]));
        }
        u32x2 w = {pack2<G::PVBF>(y[0], y[1]), pack2<G::PVBF>(y[2], y[3])};
        *reinterpret_cast<u32x2*>(ob + 32 * t + 8 * g + 4 * hl) = w;
      }
  }

  // ---- decision map and counters, as attn_stats writes them ----
  const int wv0 = member * kWavesPerBlock;   // the block's first wavefront
  const int btid = tid % kThreads;           // thread index inside the block's wavefronts
  if (active && p.dbg != nullptr) {
    uint8_t* drow = p.dbg + row_id * p.Tn * kWavesPerBlock;
    for (int x = btid; x < UC * kWavesPerBlock; x += kThreads) {
      const int e2 = x / kWavesPerBlock, w = x % kWavesPerBlock;
      if (i * kBq + w * kRowsPerWave < p.N)
        drow[entry_tile(e2) * kWavesPerBlock + w] =
            (uint8_t)((votes[(wv0 + w) * nwords + (e2 >> 4)] >> (2 * (e2 & 15))) & 3u);
    }
  }
  const bool empty = L.qvalid && hl == 0 && !(l_tot > 0.0f);
  const unsigned long long n_empty = __popcll(__ballot(empty));
  if (lane == 0) {
    red[wave][0] = (unsigned long long)n_exec;
    red[wave][1] = (unsigned long long)n_skip;
    red[wave][2] = (unsigned long long)n_void;
    red[wave][3] = n_empty;
  }
  __syncthreads();
  if (active && btid == 0) {
    unsigned long long ex = 0, sk = 0, vo = 0, em = 0;
    unsigned long long* cp = p.cnt_part + (blockIdx.x % kCountSlots) * SPARGE_NUM_COUNTERS;
    for (int w = 0; w < kWavesPerBlock; ++w) {
      if (i * kBq + w * kRowsPerWave >= p.N) continue;   // no rows: no group
      ex += red[wv0 + w][0];
      sk += red[wv0 + w][1];
      vo += red[wv0 + w][2];
      em += red[wv0 + w][3];
    }
    atomicAdd(cp + SPARGE_CNT_LIVE, (unsigned long long)n_live);
    atomicAdd(cp + SPARGE_CNT_QK_EXEC, (unsigned long long)UC);
    atomicAdd(cp + SPARGE_CNT_QK_SKIP, (unsigned long long)(n_live - UC));
    atomicAdd(cp + SPARGE_CNT_PV_EXEC, ex);
    atomicAdd(cp + SPARGE_CNT_PV_SKIP, sk);
    atomicAdd(cp + SPARGE_CNT_PV_VOID, vo);
    atomicAdd(cp + SPARGE_CNT_EMPTY_ROWS, em);
    atomicAdd(cp + SPARGE_CNT_ROWS, (unsigned long long)(last_q - i * kBq + 1));
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

// fp8 P~V, step 1: per chunk of kQuantChunkRows tokens, the channel maxima of
// |V| (grid: chunks x B*Hkv; 8 channels per lane, rows strided over the
// workgroup, then a reduction over the row slots in LDS).
template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void v_absmax_partial(AttnArgs p) {
  constexpr int CG = D / 8;                 // lanes per row
  constexpr int SLOTS = kThreads / CG;
  __shared__ float red[SLOTS][D + 1];
  const int chunk = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const int tid = threadIdx.x, c = tid % CG, slot = tid / CG;
  const unsigned short* vb = static_cast<const unsigned short*>(p.v) + b * p.v_sb + hk * p.v_sh;
  const int r0 = chunk * kQuantChunkRows, r1 = min(p.N, r0 + kQuantChunkRows);
  float mx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = r0 + slot; r < r1; r += SLOTS) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(vb + (long long)r * p.v_sn + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const unsigned short u = (unsigned short)(w[e >> 1] >> (16 * (e & 1)));
      const float x = BF16 ? __uint_as_float((unsigned int)u << 16) : (float)__builtin_bit_cast(_Float16, u);
      mx[e] = fmaxf(mx[e], fabsf(x));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[slot][8 * c + e] = mx[e];
  __syncthreads();
  if (tid < D) {
    float m = 0.0f;
    for (int s = 0; s < SLOTS; ++s) m = fmaxf(m, red[s][tid]);
    p.vpart[((long long)bh * gridDim.x + chunk) * D + tid] = m;
  }
}

// fp8 P~V, step 2: delta_c = 2^e, e the least integer with max|V_c| <= 448 2^e
// (clamped to 2^-100 for a channel that is all but zero; 1 for a zero one).
__global__ void v_scale_final(AttnArgs p, int chunks) {
  const int bh = blockIdx.x, c = threadIdx.x;
  if (c >= p.d) return;
  float m = 0.0f;
  for (int k = 0; k < chunks; ++k) m = fmaxf(m, p.vpart[((long long)bh * chunks + k) * p.d + c]);
  float delta = 1.0f;
  if (m > 0.0f) {
    int e = (int)ceilf(log2f(m / 448.0f));
    e = max(-100, min(e, 127));
    while (e < 127 && m > ldexpf(448.0f, e)) ++e;
    while (e > -100 && m <= ldexpf(448.0f, e - 1)) --e;
    delta = ldexpf(1.0f, e);
  }
  p.vscale[(long long)bh * p.d + c] = delta;
}

// fp8 P~V, step 3: V [B,Hkv,N,D] -> E4M3 codes of V / delta_c in V^T order
// [B,Hkv,D,Np] (zero past N).  Inside each 64-key row, byte 32h + b holds key
// 32 (b / 16) + 8 ((b % 16) / 4) + 4h + b % 4: the keys lane half h of the
// P~V MFMA holds, in the order of its score registers.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void transpose_v8(AttnArgs p) {
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
  const int dv = tid / 4, g = tid % 4;             // channel dt*64 + dv, bytes 16g .. 16g + 15
  const float inv = 1.0f / p.vscale[(long long)bh * p.d + dt * 64 + dv];   // a power of two: exact
  u32x4 w;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float y[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pos = 16 * g + 4 * v + q, hh = pos / 32, bb = pos % 32;
      const int key = 32 * (bb / 16) + 8 * ((bb % 16) / 4) + 4 * hh + (bb % 4);
      const unsigned short u = tile[key][dv];
      const float x = BF16 ? __uint_as_float((unsigned int)u << 16) : (float)__builtin_bit_cast(_Float16, u);
      y[q] = fminf(fmaxf(x * inv, -448.0f), 448.0f);
    }
    int c = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    w[v] = (unsigned int)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], c, true);
  }
  unsigned char* out = reinterpret_cast<unsigned char*>(p.vt) + ((long long)bh * p.d) * p.Np;
  *reinterpret_cast<u32x4*>(out + (long long)(dt * 64 + dv) * p.Np + kt * 64 + 16 * g) = w;
}

__global__ void zero_u64(unsigned long long* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0ull;
}

template <int D, int KIND, bool CAUSAL, bool PV8>
hipError_t launch_passes(const AttnArgs& a0, hipStream_t st) {
  AttnArgs a = a0;
  const long long blocks = (long long)a.B * a.H * a.Tm;
  const long long packs = (long long)a.B * a.Hkv * (pack_slots(a.H, a.Hkv, a.Tm) / kPackBlocks);
  const size_t lds1 = stats_lds_bytes<D, KIND, 1>(a.Tn);
  const size_t lds1p = stats_lds_bytes<D, KIND, kPackBlocks>(a.Tn);
  const size_t lds2 = pv_lds_bytes<D, KIND, PV8>(a.Tn);
  hipError_t e = hipSuccess;
  {
    // the path of this call, on the device: the pilot's estimate or the
    // request (every call may take the fused pass: 16-bit or int8 Q/K,
    // 16-bit or fp8 P~V)
    int groups = 0;
    if (a.path != kPathTwoPass && a.path != kPathFused) {
      const long long stride = (blocks + kPilotBlocks - 1) / kPilotBlocks;
      const long long n = (blocks + stride - 1) / stride;   // <= kPilotBlocks
      groups = (int)n;
      const size_t ldsp = pilot_lds_bytes<D, KIND>();
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_pilot<D, KIND, CAUSAL>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)ldsp);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((attn_pilot<D, KIND, CAUSAL>), dim3((unsigned)n), dim3(kThreads), ldsp, st, a,
                         (int)stride);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(pilot_decide, dim3(1), dim3(64), 0, st, a, groups,
                       Geo<D, KIND>::I8 ? (PV8 ? kFusedMeanTilesI8F8 : kFusedMeanTilesI8)
                                        : (PV8 ? kFusedMeanTilesF8 : kFusedMeanTiles));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fused<D, KIND, CAUSAL, 1, PV8>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)fused_lds_bytes<D, KIND, 1, PV8>(a.Tn));
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fused<D, KIND, CAUSAL, kPackBlocks, PV8>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)fused_lds_bytes<D, KIND, kPackBlocks, PV8>(a.Tn));
    if (e != hipSuccess) return e;
  }
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_stats<D, KIND, CAUSAL, 1>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_stats<D, KIND, CAUSAL, kPackBlocks>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1p);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_pv<D, KIND, CAUSAL, PV8>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds2);
  if (e != hipSuccess) return e;
  // pass 1: the dense query blocks in packs, then the others
  hipLaunchKernelGGL(build_packs<CAUSAL>, dim3((unsigned)(a.B * a.Hkv)), dim3(1024), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_stats<D, KIND, CAUSAL, kPackBlocks>), dim3((unsigned)packs),
                     dim3(kPackBlocks * kThreads), lds1p, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_stats<D, KIND, CAUSAL, 1>), dim3((unsigned)blocks), dim3(kThreads), lds1, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    // the fused pass: dense blocks in packs, then the others
    const size_t ldsfp = fused_lds_bytes<D, KIND, kPackBlocks, PV8>(a.Tn);
    hipLaunchKernelGGL((attn_fused<D, KIND, CAUSAL, kPackBlocks, PV8>), dim3((unsigned)packs),
                       dim3(kPackBlocks * kThreads), ldsfp, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t ldsf = fused_lds_bytes<D, KIND, 1, PV8>(a.Tn);
    hipLaunchKernelGGL((attn_fused<D, KIND, CAUSAL, 1, PV8>), dim3((unsigned)blocks), dim3(kThreads), ldsf, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(sum_counts, dim3(1), dim3(64), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_pv<D, KIND, CAUSAL, PV8>), dim3((unsigned)blocks), dim3(kThreads), lds2, st, a);
  return hipGetLastError();
}

template <int D, int KIND>
hipError_t launch_d_kind(const AttnArgs& a, hipStream_t st) {
  if (a.pv8) return a.causal ? launch_passes<D, KIND, true, true>(a, st) : launch_passes<D, KIND, false, true>(a, st);
  return a.causal ? launch_passes<D, KIND, true, false>(a, st) : launch_passes<D, KIND, false, false>(a, st);
}

// the fp8 V^T: channel maxima, power-of-two scales, E4M3 codes
template <int D>
hipError_t launch_v8(const AttnArgs& a, hipStream_t st) {
  const bool bf = (a.kind == 1 || a.kind == 3);
  const int chunks = (int)ceil_div(a.N, kQuantChunkRows);
  const dim3 g1((unsigned)chunks, (unsigned)(a.B * a.Hkv));
  if (bf)
    hipLaunchKernelGGL((v_absmax_partial<D, true>), g1, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((v_absmax_partial<D, false>), g1, dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(v_scale_final, dim3((unsigned)(a.B * a.Hkv)), dim3(128), 0, st, a, chunks);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g3((unsigned)(a.Np / 64), (unsigned)(a.d / 64), (unsigned)(a.B * a.Hkv));
  if (bf)
    hipLaunchKernelGGL(transpose_v8<true>, g3, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(transpose_v8<false>, g3, dim3(kThreads), 0, st, a);
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
  hipError_t e;
  if (a.pv8) {
    e = a.d == 64 ? launch_v8<64>(a, st) : launch_v8<128>(a, st);
  } else {
    dim3 g((unsigned)(a.Np / 64), (unsigned)(a.d / 64), (unsigned)(a.B * a.Hkv));
    hipLaunchKernelGGL(transpose_v, g, dim3(kThreads), 0, st, a);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  return a.d == 64 ? launch_d<64>(a, st) : launch_d<128>(a, st);
}

}  // namespace sparge

// Internal declarations shared by the HIP kernels and the C ABI of libsparge.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/sparge.h"

namespace sparge {

constexpr int kBq = SPARGE_BQ;              // query block rows
constexpr int kBk = SPARGE_BK;              // key/value block rows
constexpr int kRowsPerWave = 32;            // rows voting together (one wavefront)
constexpr int kWavesPerBlock = kBq / kRowsPerWave;
constexpr int kThreads = 256;
// attention pass 1: query blocks that list every live tile share one
// workgroup (and one K stream) in packs of this many blocks of one kv head
constexpr int kPackBlocks = 2;

// attention pass 1: slots of partial counters (workgroup id % kCountSlots),
// so that short workgroups do not all add to the same eight addresses
constexpr int kCountSlots = 64;

// slots per (b, kv head) of the dense-block packs: G * Tm rounded up to a
// whole number of packs
inline __host__ __device__ int pack_slots(int H, int Hkv, int Tm) {
  const int n = (H / Hkv) * Tm;
  return (n + kPackBlocks - 1) / kPackBlocks * kPackBlocks;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// Workspace layout (all regions 256-byte aligned, carved in this order)
// ---------------------------------------------------------------------------
struct Workspace {
  // stage 1
  double* qbar;        // [B,H,Tm,d]
  double* kbar;        // [B,Hkv,Tn,d]
  double* sq;          // [B,H,Tm]
  double* sk;          // [B,Hkv,Tn]
  double* shat;        // [B,H,Tm,Tn]
  // int8 quantisation: per-chunk column sums of K, then the mean
  double* ksum_part;   // [B,Hkv,kQuantChunks,d]
  double* kmean;       // [B,Hkv,d]
  // attention: row lists built from a caller's mask, and V transposed
  int32_t* list_cnt;   // [B,H,Tm]
  uint16_t* list_idx;  // [B,H,Tm,Tn]
  unsigned short* vt;  // [B,Hkv,d,Tn*64] 16-bit V^T, zero past N
  // attention pass 1 -> pass 2: per-row softmax statistics and, per query
  // block, the listed tiles on which at least one wavefront ran P~V
  float* row_m;        // [B,H,N] final running max (log2 units)
  float* row_l;        // [B,H,N] final row sum l
  uint32_t* ulist;     // [B,H,Tm,Tn] j | (wavefront mask << 16), ascending j
  int32_t* ucnt;       // [B,H,Tm]
  // fp8 P~V: per-channel power-of-two V scales (the fp8 V^T shares vt)
  float* vscale;       // [B,Hkv,d]
  // attention pass 1: dense query blocks in packs, and packs per kv head
  int32_t* packs;      // [B,Hkv,pack_slots] row ids (b H + h) Tm + i, -1 pads
  int32_t* npack;      // [B,Hkv]
  int32_t* pack_next;  // [B,Hkv] next unclaimed pack of each kv head
  unsigned long long* cnt_part;   // [kCountSlots][SPARGE_NUM_COUNTERS]
  // attention path of the call (two passes or one fused pass) and the
  // pilot's vote counts that choose it
  int32_t* path_flag;             // [1]
  unsigned long long* pilot_cnt;  // [kPilotBlocks][kPilotCounts]: per pilot workgroup, weighted votes and
                                  // pairs, the sampled block's listed tiles, 1
  size_t total;
};

// attention paths (the values of SPARGE_PATH_* in include/sparge.h)
constexpr int kPathAuto = 0;
constexpr int kPathTwoPass = 1;
constexpr int kPathFused = 2;
// pilot: at most this many sampled query blocks, this many listed tiles each
constexpr int kPilotBlocks = 256;
constexpr int kPilotCounts = 4;
// the automatic path takes the fused pass when the sampled blocks list at
// most this many tiles on average: 16-bit Q/K and P~V; fp8 P~V, whose V
// stream is half as large, twice as many; int8 Q/K, whose first pass is
// cheaper, half as many; int8 Q/K with fp8 P~V, whose first pass is cheap
// and whose second reads the fewest bytes, a quarter
constexpr int kFusedMeanTiles = 224;
constexpr int kFusedMeanTilesF8 = 448;
constexpr int kFusedMeanTilesI8 = 112;
constexpr int kFusedMeanTilesI8F8 = 64;
constexpr int kPilotTiles = 4;

constexpr int kQuantChunkRows = 1024;       // tokens per partial K column sum

Workspace carve_workspace(void* base, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d);

// ---------------------------------------------------------------------------
// Kernel launchers (return hipError_t of the launch)
// ---------------------------------------------------------------------------
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  unsigned short* vt;  // workspace V^T [B,Hkv,d,Np]
  int64_t Np;          // padded token count of V^T rows (Tn * 64)
  float* row_m;        // workspace: pass 1 final max per row (log2 units)
  float* row_l;        // workspace: pass 1 row sum per row
  uint32_t* ulist;     // workspace: executed-tile lists (j | mask << 16)
  int32_t* ucnt;       // workspace: their lengths
  int32_t* packs;      // workspace: dense query blocks in packs (see Workspace)
  int32_t* npack;      // workspace: packs per (b, kv head)
  int32_t* pack_next;  // workspace: next unclaimed pack per (b, kv head)
  unsigned long long* cnt_part;   // workspace: partial counters
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t o_sb, o_sh, o_sn;
  int B, H, Hkv, N, Tm, Tn, d;
  int kind;           // 0 f16, 1 bf16, 2 i8 QK + f16 PV, 3 i8 QK + bf16 PV
  int pv8;            // P~V on fp8 E4M3 (V stored in the kind's P~V type)
  float* vscale;      // workspace: per-channel V scales of the fp8 P~V
  float* vpart;       // workspace: per-chunk channel maxima of |V|
  int out_f32;        // store float32 O instead of the P~V type
  int causal;
  const int32_t* row_cnt;
  const uint16_t* row_idx;
  const float* q_scale;
  const float* k_scale;
  float scale_log2;   // log2(e) / sqrt(d)
  float lam_log2;     // lambda * log2(e)
  unsigned long long* counts;
  uint8_t* dbg;
  int path;           // kPathAuto, kPathTwoPass or kPathFused (requested)
  int32_t* path_flag;             // workspace: the path the call takes; null: two passes, no flag
  unsigned long long* pilot_cnt;  // workspace: the pilot's counts per workgroup
};
hipError_t launch_attn(const AttnArgs& a, hipStream_t st);

hipError_t launch_zero_counts(unsigned long long* counts, int n, hipStream_t st);

// M_g rows -> ascending lists of live j with M_g = 1
hipError_t launch_compact(const uint8_t* mg, int64_t rows, int Tm, int Tn, int N, int causal,
                          int32_t* cnt, uint16_t* idx, hipStream_t st);

struct PredictArgs {
  const void* q;
  const void* k;
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int B, H, Hkv, N, Tm, Tn, d;
  int bf16;
  int causal;
  double tau, theta;
  uint8_t* mg;
  int32_t* row_cnt;
  uint16_t* row_idx;
  double* s_q_out;    // may be null
  double* s_k_out;    // may be null
  Workspace ws;
};
hipError_t launch_predict(const PredictArgs& a, hipStream_t st);

struct QuantArgs {
  const void* q;
  const void* k;
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int B, H, Hkv, N, Tm, Tn, d;
  int bf16;
  int8_t* q8;
  int8_t* k8;
  float* q_scale;
  float* k_scale;
  Workspace ws;
};
hipError_t launch_quant(const QuantArgs& a, hipStream_t st);

struct PermuteArgs {
  const void* x;
  void* y;
  int64_t x_sb, x_sh, x_sn;   // in bytes
  int64_t y_sb, y_sh, y_sn;   // in bytes
  int B, H, N;
  int row_bytes;
  const int32_t* perm;
  int inverse;
};
hipError_t launch_permute(const PermuteArgs& a, hipStream_t st);

// host-side 3D Hilbert order
int hilbert_order(int T, int H, int W, int32_t* perm, int32_t* inv);

}  // namespace sparge

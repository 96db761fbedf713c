// C ABI of libsparge: argument checks, workspace carving and kernel launches.
// Every check runs on the host before anything is enqueued.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "support.hpp"

namespace sparge {

namespace {

thread_local std::string g_last_error;
std::atomic<int> g_attn_path{kPathAuto};   // sparge_attn_path()

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return SPARGE_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SPARGE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_size(int dtype) {
  switch (dtype) {
    case SPARGE_F16:
    case SPARGE_BF16: return 2;
    case SPARGE_I8: return 1;
    case SPARGE_F32: return 4;
    default: return 0;
  }
}

// Checks one tensor descriptor: sizes, d contiguous rows, 16-byte aligned strides.
int check_tensor(const char* name, const sparge_tensor* t, int esize) {
  if (t == nullptr) return fail(SPARGE_EINVAL, "%s: null descriptor", name);
  if (t->B < 0 || t->H < 0 || t->N < 0 || t->d <= 0)
    return fail(SPARGE_EINVAL, "%s: negative size or d <= 0 (B=%lld H=%lld N=%lld d=%lld)", name,
                (long long)t->B, (long long)t->H, (long long)t->N, (long long)t->d);
  if (t->sn < t->d) return fail(SPARGE_EINVAL, "%s: token stride %lld < d", name, (long long)t->sn);
  if (t->sb < 0 || t->sh < 0) return fail(SPARGE_EINVAL, "%s: negative stride", name);
  if ((t->sb * esize) % 16 || (t->sh * esize) % 16 || (t->sn * esize) % 16)
    return fail(SPARGE_EINVAL, "%s: byte strides must be multiples of 16", name);
  return SPARGE_OK;
}

int check_qk_shapes(const sparge_tensor* q, const sparge_tensor* k) {
  if (q->B != k->B || q->N != k->N || q->d != k->d)
    return fail(SPARGE_EINVAL, "q and k differ in B, N or d");
  if (q->H > 0 && (k->H <= 0 || q->H % k->H != 0))
    return fail(SPARGE_EINVAL, "H (%lld) must be a positive multiple of H_kv (%lld)", (long long)q->H,
                (long long)k->H);
  if (q->d != 64 && q->d != 128) return fail(SPARGE_EUNSUPPORTED, "head dim %lld: only 64 and 128", (long long)q->d);
  if (ceil_div(q->N, kBk) > SPARGE_MAX_TN)
    return fail(SPARGE_EUNSUPPORTED, "N = %lld exceeds %d key blocks", (long long)q->N, SPARGE_MAX_TN);
  if (q->B * q->H * ceil_div(q->N, kBq) > 0x7fffffffLL || q->B * q->H * q->N > (1LL << 40))
    return fail(SPARGE_EUNSUPPORTED, "too many blocks for one launch");
  return SPARGE_OK;
}

bool empty_problem(const sparge_tensor* q) { return q->B == 0 || q->H == 0 || q->N == 0; }

// Byte range [lo, hi) a non-empty tensor's elements span (strides are >= 0).
void byte_span(const void* base, const sparge_tensor* t, int esize, uintptr_t& lo, uintptr_t& hi) {
  lo = (uintptr_t)base;
  hi = lo + (uintptr_t)(((t->B - 1) * t->sb + (t->H - 1) * t->sh + (t->N - 1) * t->sn + t->d) * esize);
}

bool spans_overlap(const void* x, const sparge_tensor* xs, const void* y, const sparge_tensor* ys, int esize) {
  uintptr_t xl, xh, yl, yh;
  byte_span(x, xs, esize, xl, xh);
  byte_span(y, ys, esize, yl, yh);
  return xl < yh && yl < xh;
}

}  // namespace

Workspace carve_workspace(void* base, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d) {
  Workspace w{};
  const int64_t Tm = ceil_div(N, kBq), Tn = ceil_div(N, kBk);
  const int64_t chunks = ceil_div(N, kQuantChunkRows);
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* r = p ? p + off : nullptr;
    off = align256(off + bytes);
    return r;
  };
  w.qbar = reinterpret_cast<double*>(take(8 * (size_t)(B * H * Tm * d)));
  w.kbar = reinterpret_cast<double*>(take(8 * (size_t)(B * Hkv * Tn * d)));
  w.sq = reinterpret_cast<double*>(take(8 * (size_t)(B * H * Tm)));
  w.sk = reinterpret_cast<double*>(take(8 * (size_t)(B * Hkv * Tn)));
  w.shat = reinterpret_cast<double*>(take(8 * (size_t)(B * H * Tm * Tn)));
  w.ksum_part = reinterpret_cast<double*>(take(8 * (size_t)(B * Hkv * chunks * d)));
  w.kmean = reinterpret_cast<double*>(take(8 * (size_t)(B * Hkv * d)));
  w.list_cnt = reinterpret_cast<int32_t*>(take(4 * (size_t)(B * H * Tm)));
  w.list_idx = reinterpret_cast<uint16_t*>(take(2 * (size_t)(B * H * Tm * Tn)));
  w.vt = reinterpret_cast<unsigned short*>(take(2 * (size_t)(B * Hkv * d * Tn * kBk)));
  w.row_m = reinterpret_cast<float*>(take(4 * (size_t)(B * H * N)));
  w.row_l = reinterpret_cast<float*>(take(4 * (size_t)(B * H * N)));
  w.ulist = reinterpret_cast<uint32_t*>(take(4 * (size_t)(B * H * Tm * Tn)));
  w.ucnt = reinterpret_cast<int32_t*>(take(4 * (size_t)(B * H * Tm)));
  w.vscale = reinterpret_cast<float*>(take(4 * (size_t)(B * Hkv * d)));
  w.packs = reinterpret_cast<int32_t*>(take(4 * (size_t)(B * Hkv) * (size_t)pack_slots((int)H, (int)Hkv, (int)Tm)));
  w.npack = reinterpret_cast<int32_t*>(take(4 * (size_t)(B * Hkv)));
  w.pack_next = reinterpret_cast<int32_t*>(take(4 * (size_t)(B * Hkv)));
  w.cnt_part = reinterpret_cast<unsigned long long*>(take(8 * (size_t)kCountSlots * SPARGE_NUM_COUNTERS));
  w.path_flag = reinterpret_cast<int32_t*>(take(4));
  w.pilot_cnt = reinterpret_cast<unsigned long long*>(take(8 * (size_t)kPilotCounts * kPilotBlocks));
  w.total = off;
  return w;
}

}  // namespace sparge

using namespace sparge;

extern "C" {

int sparge_version(void) { return 10000; }

const char* sparge_last_error(void) { return g_last_error.c_str(); }

int sparge_rows_per_wave(void) { return kRowsPerWave; }

int sparge_attn_path(int path) {
  if (path != -1 && path != SPARGE_PATH_AUTO && path != SPARGE_PATH_TWO_PASS && path != SPARGE_PATH_FUSED)
    return fail(SPARGE_EINVAL, "unknown attention path %d", path);
  if (path == -1) return g_attn_path.load();
  return g_attn_path.exchange(path);
}

size_t sparge_workspace_size(const sparge_tensor* q, const sparge_tensor* k) {
  if (q == nullptr || k == nullptr || q->B < 0 || q->H < 0 || q->N < 0 || q->d <= 0 || k->H <= 0)
    return 0;
  if (k->B != q->B || k->N != q->N || k->d != q->d || q->H % k->H != 0) return 0;
  return carve_workspace(nullptr, q->B, q->H, k->H, q->N, q->d).total + 256;
}

int sparge_hilbert_index(int T, int H, int W, int32_t* perm, int32_t* inv) {
  if (T <= 0 || H <= 0 || W <= 0) return fail(SPARGE_EINVAL, "grid sizes must be positive");
  if (perm == nullptr || inv == nullptr) return fail(SPARGE_EINVAL, "null output");
  if ((int64_t)T * H * W >= (1LL << 31)) return fail(SPARGE_EUNSUPPORTED, "grid too large");
  if (std::max(T, std::max(H, W)) > (1 << 20)) return fail(SPARGE_EUNSUPPORTED, "grid side too large");
  hilbert_order(T, H, W, perm, inv);
  return ok();
}

int sparge_grid_order(int T, int H, int W, int order, int32_t* perm, int32_t* inv) {
  if (T <= 0 || H <= 0 || W <= 0) return fail(SPARGE_EINVAL, "grid sizes must be positive");
  if (perm == nullptr || inv == nullptr) return fail(SPARGE_EINVAL, "null output");
  if (order != SPARGE_ORDER_HILBERT && order != SPARGE_ORDER_ROWMAJOR && order != SPARGE_ORDER_TIMEMAJOR)
    return fail(SPARGE_EINVAL, "unknown order %d", order);
  if ((int64_t)T * H * W >= (1LL << 31)) return fail(SPARGE_EUNSUPPORTED, "grid too large");
  if (order == SPARGE_ORDER_HILBERT) return sparge_hilbert_index(T, H, W, perm, inv);
  simple_order(T, H, W, order, perm, inv);
  return ok();
}

size_t sparge_l1_workspace_size(void) { return (size_t)16 * kL1Blocks + 256; }

int sparge_l1_sums(const void* o, const sparge_tensor* os, int dtype_o, const void* ref,
                   const sparge_tensor* rs, int dtype_ref, double* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  const int eo = dtype_o == SPARGE_I8 ? 0 : elem_size(dtype_o);
  const int er = dtype_ref == SPARGE_I8 ? 0 : elem_size(dtype_ref);
  if (eo == 0 || er == 0) return fail(SPARGE_EINVAL, "dtypes must be F16, BF16 or F32");
  int r = check_tensor("o", os, eo);
  if (r) return r;
  r = check_tensor("ref", rs, er);
  if (r) return r;
  if (os->B != rs->B || os->H != rs->H || os->N != rs->N || os->d != rs->d)
    return fail(SPARGE_EINVAL, "o and ref differ in shape");
  if (out == nullptr) return fail(SPARGE_EINVAL, "null output");
  if (workspace == nullptr || workspace_bytes < sparge_l1_workspace_size())
    return fail(SPARGE_EWORKSPACE, "workspace needs %zu bytes", sparge_l1_workspace_size());
  const bool empty = empty_problem(os);
  if (!empty && (o == nullptr || ref == nullptr)) return fail(SPARGE_EINVAL, "null pointer");
  if (!empty && (!aligned16(o) || !aligned16(ref))) return fail(SPARGE_EINVAL, "o and ref must be 16-byte aligned");
  L1Args a{};
  a.o = o;
  a.r = ref;
  a.o_sb = os->sb;
  a.o_sh = os->sh;
  a.o_sn = os->sn;
  a.r_sb = rs->sb;
  a.r_sh = rs->sh;
  a.r_sn = rs->sn;
  a.B = empty ? 0 : os->B;   // an empty tensor still writes (0, 0)
  a.H = os->H;
  a.N = os->N;
  a.d = os->d;
  a.dtype_o = dtype_o;
  a.dtype_r = dtype_ref;
  a.partial = reinterpret_cast<double*>(align256((size_t)workspace));
  a.out = out;
  const hipError_t e = launch_l1(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "l1 launch");
  return ok();
}

int sparge_hilbert_permute(const void* x, const sparge_tensor* xs, void* y, const sparge_tensor* ys,
                           int dtype, const int32_t* perm, int inverse, void* stream) {
  const int es = elem_size(dtype);
  if (es == 0) return fail(SPARGE_EINVAL, "unknown dtype %d", dtype);
  int r = check_tensor("x", xs, es);
  if (r) return r;
  r = check_tensor("y", ys, es);
  if (r) return r;
  if (xs->B != ys->B || xs->H != ys->H || xs->N != ys->N || xs->d != ys->d)
    return fail(SPARGE_EINVAL, "x and y differ in shape");
  if ((xs->d * es) % 16) return fail(SPARGE_EUNSUPPORTED, "row bytes must be a multiple of 16");
  if (xs->N >= (1LL << 31)) return fail(SPARGE_EUNSUPPORTED, "N too large");
  if (inverse != 0 && inverse != 1) return fail(SPARGE_EINVAL, "inverse must be 0 or 1");
  if (empty_problem(xs)) return ok();
  if (x == nullptr || y == nullptr) return fail(SPARGE_EINVAL, "null pointer");
  if (!aligned16(x) || !aligned16(y)) return fail(SPARGE_EINVAL, "x and y must be 16-byte aligned");
  if (spans_overlap(x, xs, y, ys, es)) return fail(SPARGE_EINVAL, "x and y must not overlap");
  if (perm == nullptr) return fail(SPARGE_EINVAL, "null perm");
  PermuteArgs a{};
  a.x = x;
  a.y = y;
  a.x_sb = xs->sb * es;
  a.x_sh = xs->sh * es;
  a.x_sn = xs->sn * es;
  a.y_sb = ys->sb * es;
  a.y_sh = ys->sh * es;
  a.y_sn = ys->sn * es;
  a.B = (int)xs->B;
  a.H = (int)xs->H;
  a.N = (int)xs->N;
  a.row_bytes = (int)(xs->d * es);
  a.perm = perm;
  a.inverse = inverse;
  const hipError_t e = launch_permute(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hilbert_permute launch");
  return ok();
}

int sparge_quant_qk_int8(const void* q, const sparge_tensor* qs, const void* k,
                         const sparge_tensor* ks, int dtype, int8_t* q8, int8_t* k8,
                         float* q_scale, float* k_scale, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (dtype != SPARGE_F16 && dtype != SPARGE_BF16)
    return fail(SPARGE_EINVAL, "q/k dtype must be F16 or BF16");
  int r = check_tensor("q", qs, 2);
  if (r) return r;
  r = check_tensor("k", ks, 2);
  if (r) return r;
  r = check_qk_shapes(qs, ks);
  if (r) return r;
  if (empty_problem(qs)) return ok();
  if (!q || !k || !q8 || !k8 || !q_scale || !k_scale) return fail(SPARGE_EINVAL, "null pointer");
  if (!aligned16(q) || !aligned16(k) || !aligned16(q8) || !aligned16(k8))
    return fail(SPARGE_EINVAL, "q, k, q8, k8 must be 16-byte aligned");
  if (workspace == nullptr || workspace_bytes < sparge_workspace_size(qs, ks))
    return fail(SPARGE_EWORKSPACE, "workspace needs %zu bytes", sparge_workspace_size(qs, ks));
  QuantArgs a{};
  a.q = q;
  a.k = k;
  a.q_sb = qs->sb;
  a.q_sh = qs->sh;
  a.q_sn = qs->sn;
  a.k_sb = ks->sb;
  a.k_sh = ks->sh;
  a.k_sn = ks->sn;
  a.B = (int)qs->B;
  a.H = (int)qs->H;
  a.Hkv = (int)ks->H;
  a.N = (int)qs->N;
  a.Tm = (int)ceil_div(qs->N, kBq);
  a.Tn = (int)ceil_div(qs->N, kBk);
  a.d = (int)qs->d;
  a.bf16 = dtype == SPARGE_BF16;
  a.q8 = q8;
  a.k8 = k8;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  void* base = reinterpret_cast<void*>(align256((size_t)workspace));
  a.ws = carve_workspace(base, a.B, a.H, a.Hkv, a.N, a.d);
  const hipError_t e = launch_quant(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "quant launch");
  return ok();
}

int sparge_predict_mask(const void* q, const sparge_tensor* qs, const void* k,
                        const sparge_tensor* ks, int dtype, double tau, double theta, int causal,
                        uint8_t* mg, int32_t* row_cnt, uint16_t* row_idx, double* s_q,
                        double* s_k, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != SPARGE_F16 && dtype != SPARGE_BF16)
    return fail(SPARGE_EINVAL, "q/k dtype must be F16 or BF16");
  int r = check_tensor("q", qs, 2);
  if (r) return r;
  r = check_tensor("k", ks, 2);
  if (r) return r;
  r = check_qk_shapes(qs, ks);
  if (r) return r;
  if (!(tau > 0.0 && tau <= 1.0)) return fail(SPARGE_EINVAL, "tau must lie in (0, 1]");
  if (!std::isfinite(theta)) return fail(SPARGE_EINVAL, "theta must be finite");
  if (causal != 0 && causal != 1) return fail(SPARGE_EINVAL, "causal must be 0 or 1");
  if (empty_problem(qs)) return ok();
  if (!q || !k || !mg || !row_cnt || !row_idx) return fail(SPARGE_EINVAL, "null pointer");
  if (!aligned16(q) || !aligned16(k)) return fail(SPARGE_EINVAL, "q and k must be 16-byte aligned");
  if (workspace == nullptr || workspace_bytes < sparge_workspace_size(qs, ks))
    return fail(SPARGE_EWORKSPACE, "workspace needs %zu bytes", sparge_workspace_size(qs, ks));
  PredictArgs a{};
  a.q = q;
  a.k = k;
  a.q_sb = qs->sb;
  a.q_sh = qs->sh;
  a.q_sn = qs->sn;
  a.k_sb = ks->sb;
  a.k_sh = ks->sh;
  a.k_sn = ks->sn;
  a.B = (int)qs->B;
  a.H = (int)qs->H;
  a.Hkv = (int)ks->H;
  a.N = (int)qs->N;
  a.Tm = (int)ceil_div(qs->N, kBq);
  a.Tn = (int)ceil_div(qs->N, kBk);
  a.d = (int)qs->d;
  a.bf16 = dtype == SPARGE_BF16;
  a.causal = causal;
  a.tau = tau;
  a.theta = theta;
  a.mg = mg;
  a.row_cnt = row_cnt;
  a.row_idx = row_idx;
  a.s_q_out = s_q;
  a.s_k_out = s_k;
  void* base = reinterpret_cast<void*>(align256((size_t)workspace));
  a.ws = carve_workspace(base, a.B, a.H, a.Hkv, a.N, a.d);
  const hipError_t e = launch_predict(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "predict launch");
  return ok();
}

}  // extern "C"

namespace {

// One attention call after its arguments have been checked: the launch
// arguments (workspace pointers still unset), the caller's mask and lists,
// and whether the lists must be built from the mask.
struct AttnCall {
  AttnArgs a{};
  const uint8_t* mg = nullptr;
  bool need_lists = false;
  bool done = false;        // an empty problem: nothing (more) to launch
  hipStream_t st = nullptr;
};

// Every host-side check of sparge_attn except the workspace's; on success
// fills `c`.  An empty problem zeroes the counters and sets c.done.
int attn_prepare(const void* q, const sparge_tensor* qs, const void* k, const sparge_tensor* ks,
                 const void* v, const sparge_tensor* vs, void* o, const sparge_tensor* os,
                 int qk_dtype, int pv_dtype, int o_dtype, const float* q_scale, const float* k_scale,
                 const uint8_t* mg, const int32_t* row_cnt, const uint16_t* row_idx,
                 double lambda, int causal, int64_t* counts, uint8_t* pv_dbg, void* stream, bool pv8,
                 AttnCall& c) {
  int kind;
  if (qk_dtype == SPARGE_F16 && pv_dtype == SPARGE_F16) kind = 0;
  else if (qk_dtype == SPARGE_BF16 && pv_dtype == SPARGE_BF16) kind = 1;
  else if (qk_dtype == SPARGE_I8 && pv_dtype == SPARGE_F16) kind = 2;
  else if (qk_dtype == SPARGE_I8 && pv_dtype == SPARGE_BF16) kind = 3;
  else return fail(SPARGE_EINVAL, "unsupported dtype pair (qk %d, pv %d)", qk_dtype, pv_dtype);
  const int qk_es = elem_size(qk_dtype);
  int r = check_tensor("q", qs, qk_es);
  if (r) return r;
  r = check_tensor("k", ks, qk_es);
  if (r) return r;
  r = check_tensor("v", vs, 2);
  if (r) return r;
  if (o_dtype != pv_dtype && o_dtype != SPARGE_F32)
    return fail(SPARGE_EINVAL, "o dtype must be the P~V dtype or F32");
  r = check_tensor("o", os, o_dtype == SPARGE_F32 ? 4 : 2);
  if (r) return r;
  r = check_qk_shapes(qs, ks);
  if (r) return r;
  if (vs->B != ks->B || vs->H != ks->H || vs->N != ks->N || vs->d != ks->d)
    return fail(SPARGE_EINVAL, "v must have the shape of k");
  if (os->B != qs->B || os->H != qs->H || os->N != qs->N || os->d != qs->d)
    return fail(SPARGE_EINVAL, "o must have the shape of q");
  // the attention kernel forms per-lane offsets of 64 K rows in 32 bits
  if (ks->sn * qk_es * (int64_t)kBk >= (1LL << 31) || qs->sn * qk_es * (int64_t)kBk >= (1LL << 31))
    return fail(SPARGE_EUNSUPPORTED, "token stride too large (64 rows must span < 2 GiB)");
  if (kind >= 2) {
    // int8 codes are the contiguous output of sparge_quant_qk_int8
    const int64_t d = qs->d;
    if (qs->sn != d || qs->sh != qs->N * d || qs->sb != qs->H * qs->N * d || ks->sn != d ||
        ks->sh != ks->N * d || ks->sb != ks->H * ks->N * d)
      return fail(SPARGE_EINVAL, "int8 q/k must be contiguous [B,H,N,d]");
  }
  if (std::isnan(lambda) || !(lambda < 0.0)) return fail(SPARGE_EINVAL, "lambda must be < 0");
  if (causal != 0 && causal != 1) return fail(SPARGE_EINVAL, "causal must be 0 or 1");
  if ((row_cnt == nullptr) != (row_idx == nullptr))
    return fail(SPARGE_EINVAL, "row_cnt and row_idx are given together or not at all");
  c.st = static_cast<hipStream_t>(stream);
  if (empty_problem(qs)) {
    if (counts != nullptr) {
      const hipError_t e =
          launch_zero_counts(reinterpret_cast<unsigned long long*>(counts), SPARGE_NUM_COUNTERS, c.st);
      if (e != hipSuccess) return hip_fail(e, "counter reset");
    }
    c.done = true;
    return SPARGE_OK;
  }
  if (!q || !k || !v || !o || !mg || !counts) return fail(SPARGE_EINVAL, "null pointer");
  if (kind >= 2 && (!q_scale || !k_scale)) return fail(SPARGE_EINVAL, "int8 needs q_scale and k_scale");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(SPARGE_EINVAL, "q, k, v, o must be 16-byte aligned");
  AttnArgs& a = c.a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.q_sb = qs->sb;
  a.q_sh = qs->sh;
  a.q_sn = qs->sn;
  a.k_sb = ks->sb;
  a.k_sh = ks->sh;
  a.k_sn = ks->sn;
  a.v_sb = vs->sb;
  a.v_sh = vs->sh;
  a.v_sn = vs->sn;
  a.o_sb = os->sb;
  a.o_sh = os->sh;
  a.o_sn = os->sn;
  a.B = (int)qs->B;
  a.H = (int)qs->H;
  a.Hkv = (int)ks->H;
  a.N = (int)qs->N;
  a.Tm = (int)ceil_div(qs->N, kBq);
  a.Tn = (int)ceil_div(qs->N, kBk);
  a.d = (int)qs->d;
  a.kind = kind;
  a.pv8 = pv8 ? 1 : 0;
  a.out_f32 = o_dtype == SPARGE_F32;
  a.causal = causal;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)qs->d));
  a.lam_log2 = (float)(lambda * 1.4426950408889634);
  a.counts = reinterpret_cast<unsigned long long*>(counts);
  a.dbg = pv_dbg;
  a.row_cnt = row_cnt;
  a.row_idx = row_idx;
  c.mg = mg;
  c.need_lists = row_cnt == nullptr;
  return SPARGE_OK;
}

// Points the call at its scratch regions in `w` and launches it.
int attn_launch(AttnCall& c, const Workspace& w) {
  AttnArgs& a = c.a;
  a.vt = w.vt;
  a.Np = (int64_t)a.Tn * kBk;
  a.row_m = w.row_m;
  a.row_l = w.row_l;
  a.ulist = w.ulist;
  a.ucnt = w.ucnt;
  a.vscale = w.vscale;
  a.packs = w.packs;
  a.npack = w.npack;
  a.pack_next = w.pack_next;
  a.cnt_part = w.cnt_part;
  a.vpart = reinterpret_cast<float*>(w.ksum_part);   // free during an attention call
  a.path_flag = w.path_flag;
  a.pilot_cnt = w.pilot_cnt;
  a.path = g_attn_path.load(std::memory_order_relaxed);
  hipError_t e = hipSuccess;   // the attention kernels overwrite every counter
  if (c.need_lists) {
    e = launch_compact(c.mg, (int64_t)a.B * a.H * a.Tm, a.Tm, a.Tn, a.N, a.causal, w.list_cnt, w.list_idx, c.st);
    if (e != hipSuccess) return hip_fail(e, "mask compaction launch");
    a.row_cnt = w.list_cnt;
    a.row_idx = w.list_idx;
  }
  e = launch_attn(a, c.st);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return ok();
}

int attn_impl(const void* q, const sparge_tensor* qs, const void* k, const sparge_tensor* ks,
              const void* v, const sparge_tensor* vs, void* o, const sparge_tensor* os,
              int qk_dtype, int pv_dtype, int o_dtype, const float* q_scale, const float* k_scale,
              const uint8_t* mg, const int32_t* row_cnt, const uint16_t* row_idx,
              double lambda, int causal, int64_t* counts, uint8_t* pv_dbg, void* workspace,
              size_t workspace_bytes, void* stream, bool pv8) {
  AttnCall c;
  int r = attn_prepare(q, qs, k, ks, v, vs, o, os, qk_dtype, pv_dtype, o_dtype, q_scale, k_scale, mg, row_cnt,
                       row_idx, lambda, causal, counts, pv_dbg, stream, pv8, c);
  if (r != SPARGE_OK || c.done) return r == SPARGE_OK ? ok() : r;
  if (workspace == nullptr || workspace_bytes < sparge_workspace_size(qs, ks))
    return fail(SPARGE_EWORKSPACE, "workspace needs %zu bytes", sparge_workspace_size(qs, ks));
  void* base = reinterpret_cast<void*>(align256((size_t)workspace));
  return attn_launch(c, carve_workspace(base, c.a.B, c.a.H, c.a.Hkv, c.a.N, c.a.d));
}

// ---------------------------------------------------------------------------
// sparge_attn_noalloc: the scratch of one attention call in a static array
// ---------------------------------------------------------------------------
// Each GPU the library runs on holds its own copy of `scratch` for the life of
// the process.  In host code the array's name is only a host-side stand-in:
// its device address comes from hipGetSymbolAddress, once per device, and only
// that address is ever handed to kernels.
constexpr size_t kScratchBytes = SPARGE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device that work on `st` runs on.
int stream_device(hipStream_t st, int& dev) {
  hipError_t e = st == nullptr ? hipGetDevice(&dev) : hipStreamGetDevice(st, &dev);
  if (e != hipSuccess) return hip_fail(e, "finding the stream's device");
  if (dev < 0 || dev >= kMaxDevices) return fail(SPARGE_EUNSUPPORTED, "device %d out of range", dev);
  return SPARGE_OK;
}

// Device address of `scratch` on `dev`, looked up on the first call there
// (with that device current) and kept.
int scratch_on(int dev, void*& ptr) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess && e2 != hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(SPARGE_EHIP, "hipGetSymbolAddress(scratch) returned null");
    g_scratch_ptr[dev] = p;
  }
  ptr = g_scratch_ptr[dev];
  return SPARGE_OK;
}

// The attention share of the workspace layout: only the regions the attention
// kernels touch (the same regions, in a tighter layout, as in the full one).
Workspace carve_attn_workspace(void* base, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d) {
  Workspace w{};
  const int64_t Tm = ceil_div(N, kBq), Tn = ceil_div(N, kBk);
  const int64_t chunks = ceil_div(N, kQuantChunkRows);
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* r = p ? p + off : nullptr;
    off = align256(off + bytes);
    return r;
  };
  w.ksum_part = reinterpret_cast<double*>(take(8 * (size_t)(B * Hkv * chunks * d)));
  w.list_cnt = reinterpret_cast<int32_t*>(take(4 * (size_t)(B * H * Tm)));
  w.list_idx = reinterpret_cast<uint16_t*>(take(2 * (size_t)(B * H * Tm * Tn)));
  w.vt = reinterpret_cast<unsigned short*>(take(2 * (size_t)(B * Hkv * d * Tn * kBk)));
  w.row_m = reinterpret_cast<float*>(take(4 * (size_t)(B * H * N)));
  w.row_l = reinterpret_cast<float*>(take(4 * (size_t)(B * H * N)));
  w.ulist = reinterpret_cast<uint32_t*>(take(4 * (size_t)(B * H * Tm * Tn)));
  w.ucnt = reinterpret_cast<int32_t*>(take(4 * (size_t)(B * H * Tm)));
  w.vscale = reinterpret_cast<float*>(take(4 * (size_t)(B * Hkv * d)));
  w.packs = reinterpret_cast<int32_t*>(take(4 * (size_t)(B * Hkv) * (size_t)pack_slots((int)H, (int)Hkv, (int)Tm)));
  w.npack = reinterpret_cast<int32_t*>(take(4 * (size_t)(B * Hkv)));
  w.pack_next = reinterpret_cast<int32_t*>(take(4 * (size_t)(B * Hkv)));
  w.cnt_part = reinterpret_cast<unsigned long long*>(take(8 * (size_t)kCountSlots * SPARGE_NUM_COUNTERS));
  w.path_flag = reinterpret_cast<int32_t*>(take(4));
  w.pilot_cnt = reinterpret_cast<unsigned long long*>(take(8 * (size_t)kPilotCounts * kPilotBlocks));
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

int sparge_attn_noalloc(const void* q, const sparge_tensor* qs, const void* k, const sparge_tensor* ks,
                        const void* v, const sparge_tensor* vs, void* o, const sparge_tensor* os,
                        int qk_dtype, int pv_dtype, int o_dtype, const float* q_scale, const float* k_scale,
                        const uint8_t* mg, const int32_t* row_cnt, const uint16_t* row_idx,
                        double lambda, int causal, int64_t* counts, uint8_t* pv_dbg, void* stream) {
  AttnCall c;
  int r = attn_prepare(q, qs, k, ks, v, vs, o, os, qk_dtype, pv_dtype, o_dtype, q_scale, k_scale, mg, row_cnt,
                       row_idx, lambda, causal, counts, pv_dbg, stream, false, c);
  if (r != SPARGE_OK || c.done) return r == SPARGE_OK ? ok() : r;
  const size_t need = carve_attn_workspace(nullptr, qs->B, qs->H, ks->H, qs->N, qs->d).total;
  if (need > kScratchBytes)
    return fail(SPARGE_EWORKSPACE, "the problem needs %zu bytes of scratch; the static scratch holds %zu", need,
                kScratchBytes);
  int dev = 0;
  if ((r = stream_device(c.st, dev)) != SPARGE_OK) return r;
  void* base = nullptr;
  if ((r = scratch_on(dev, base)) != SPARGE_OK) return r;
  return attn_launch(c, carve_attn_workspace(base, c.a.B, c.a.H, c.a.Hkv, c.a.N, c.a.d));
}

int sparge_attn(const void* q, const sparge_tensor* qs, const void* k, const sparge_tensor* ks,
                const void* v, const sparge_tensor* vs, void* o, const sparge_tensor* os,
                int qk_dtype, int pv_dtype, int o_dtype, const float* q_scale, const float* k_scale,
                const uint8_t* mg, const int32_t* row_cnt, const uint16_t* row_idx,
                double lambda, int causal, int64_t* counts, uint8_t* pv_dbg, void* workspace,
                size_t workspace_bytes, void* stream) {
  return attn_impl(q, qs, k, ks, v, vs, o, os, qk_dtype, pv_dtype, o_dtype, q_scale, k_scale, mg, row_cnt,
                   row_idx, lambda, causal, counts, pv_dbg, workspace, workspace_bytes, stream, false);
}

int sparge_attn_fp8pv(const void* q, const sparge_tensor* qs, const void* k, const sparge_tensor* ks,
                      const void* v, const sparge_tensor* vs, void* o, const sparge_tensor* os,
                      int qk_dtype, int v_dtype, int o_dtype, const float* q_scale, const float* k_scale,
                      const uint8_t* mg, const int32_t* row_cnt, const uint16_t* row_idx,
                      double lambda, int causal, int64_t* counts, uint8_t* pv_dbg, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return attn_impl(q, qs, k, ks, v, vs, o, os, qk_dtype, v_dtype, o_dtype, q_scale, k_scale, mg, row_cnt,
                   row_idx, lambda, causal, counts, pv_dbg, workspace, workspace_bytes, stream, true);
}

}  // extern "C"

/*
 * sparge.h -- C ABI of the MI355X (gfx950) SpargeAttn hot path.
 *
 * The method is SpargeAttn's two-stage online filter on a FlashAttention
 * tiling.  Pages cited by title and section:
 *   [Review]   "SpargeAttn: Accurate and Training-free Sparse Attention
 *              Accelerating Any Model Inference" (xllm-io paper-review blog):
 *              "Core formulas" eqs. (1)-(9), the sparse warp online softmax,
 *              "Algorithm 1", the components table, "HilbertCurve Permutation".
 *   [Rebuttal] "SpargeAttention: ..." OpenReview author rebuttal, replies
 *              "Weaknesses1", "Weaknesses3", "Weaknesses3.1", "Weaknesses3.2".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are 4-D [B, heads, N, d] with the d axis contiguous.  A
 *   sparge_tensor gives the sizes and the strides (in elements) of the other
 *   three axes.  Base pointers and the byte strides must be 16-byte aligned.
 * - Query blocks hold SPARGE_BQ rows, key/value blocks SPARGE_BK rows:
 *   Tm = ceil(N / SPARGE_BQ), Tn = ceil(N / SPARGE_BK).  A ragged last block
 *   holds the remaining rows.
 * - GQA: query head h reads key/value head h / (H / H_kv); H % H_kv == 0.
 * - Every device pointer is owned by the caller.  The library never
 *   allocates device memory: scratch lives in the caller's `workspace`,
 *   sized by sparge_workspace_size().
 * - Every device call is asynchronous on `stream` (a hipStream_t; NULL is
 *   the default stream).  Arguments are checked on the host before anything
 *   is enqueued; on a negative return nothing was launched (SPARGE_EHIP: a
 *   launch failed).  sparge_last_error() gives the calling thread's message.
 * - A device call enqueues kernel launches only (no allocation, copy, memset
 *   or synchronisation), and every launch rewrites whatever scratch a later
 *   one reads, so a sequence of calls may be captured into a HIP graph and
 *   replayed; calls that share a workspace must not overlap.
 * - N == 0, B == 0 or H == 0 is valid and launches nothing.
 */
#ifndef SPARGE_H
#define SPARGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPARGE_OK 0
#define SPARGE_EINVAL (-1)        /* bad argument (null pointer, shape, range)  */
#define SPARGE_EUNSUPPORTED (-2)  /* valid but not supported (d, N, dtype)  */
#define SPARGE_EWORKSPACE (-3)    /* workspace smaller than sparge_workspace_size */
#define SPARGE_EHIP (-4)          /* a HIP call or kernel launch failed           */

#define SPARGE_BQ 128             /* query block rows b_q                        */
#define SPARGE_BK 64              /* key/value block rows b_k                    */
#define SPARGE_MAX_TN 4096        /* largest Tn (so N <= 262144)                 */

/* element types */
#define SPARGE_F16 0
#define SPARGE_BF16 1
#define SPARGE_I8 2
#define SPARGE_F32 3              /* output only                                 */

/* counters written by sparge_attn, int64 each, in this order */
#define SPARGE_CNT_LIVE 0         /* live tiles (causal: tiles with a visible pair)   */
#define SPARGE_CNT_QK_EXEC 1      /* live tiles with M_g = 1: QK^T computed          */
#define SPARGE_CNT_QK_SKIP 2      /* live tiles with M_g = 0 (= LIVE - QK_EXEC)       */
#define SPARGE_CNT_PV_EXEC 3      /* (tile, row group) pairs whose P~V ran            */
#define SPARGE_CNT_PV_SKIP 4      /* pairs skipped by the lambda vote                 */
#define SPARGE_CNT_PV_VOID 5      /* pairs with no visible key in the tile (causal)   */
#define SPARGE_CNT_EMPTY_ROWS 6   /* query rows whose executed tiles held no key: O=0 */
#define SPARGE_CNT_ROWS 7         /* query rows                                       */
#define SPARGE_NUM_COUNTERS 8

typedef struct {
  int64_t B, H, N, d;   /* batch, heads, tokens, head dim                        */
  int64_t sb, sh, sn;   /* element strides of the batch, head and token axes     */
} sparge_tensor;

/* Library version (major * 10000 + minor * 100 + patch). */
int sparge_version(void);

/* Message of the calling thread's last failed call ("" if none). */
const char* sparge_last_error(void);

/* Query rows that take the lambda decision together: b_q / c_w, one 64-lane
 * wavefront of the attention kernel ([Review] sparse warp online softmax: the
 * rows I_w of warp i_w). */
int sparge_rows_per_wave(void);

/*
 * How sparge_attn, sparge_attn_fp8pv and sparge_attn_noalloc run stage 2,
 * for every Q/K and P~V type they take.  Both paths compute the same method ([Review] eq. 1, the sparse warp online
 * softmax rule, Algorithm 1) with the same lambda decisions and counters;
 * they round P~ at different points:
 *   SPARGE_PATH_TWO_PASS: a statistics pass (running max, row sums, votes;
 *     K only) and a P~V pass over the tiles some wavefront voted for, which
 *     recomputes S there and uses P~ = exp(S - final row max).  Cheap when few
 *     (tile, wavefront) pairs vote.
 *   SPARGE_PATH_FUSED: one pass streaming K and V together, Algorithm 1's own
 *     order (P~ = exp(S - running max), O rescaled as the max grows), P~V
 *     skipped for the wavefronts whose vote says so.  Cheap when most vote,
 *     or when rows are short.
 *   SPARGE_PATH_AUTO (the default): per call, a pilot on the device takes
 *     up to 256 sampled query blocks, seeds a running max with each block's
 *     first listed tile, and votes 3 more listed tiles (one per stratum of
 *     the list) against it; the call takes the fused path when at least nine
 *     tenths of the sampled (tile, wavefront) pairs vote, each sample
 *     weighted by the listed tiles it stands for, or when the sampled blocks
 *     list at most 224 tiles on average (448 with fp8 P~V, whose V stream is
 *     half as large; 112 with int8 Q/K, whose first pass is cheaper; 64 with
 *     both).  Nothing is read back to the host.
 * sparge_attn_path(p) sets the path of later calls process-wide and returns
 * the previous setting; sparge_attn_path(-1) only returns it.  An unknown p
 * returns SPARGE_EINVAL.
 */
#define SPARGE_PATH_AUTO 0
#define SPARGE_PATH_TWO_PASS 1
#define SPARGE_PATH_FUSED 2
int sparge_attn_path(int path);

/* Bytes of device workspace any entry point below needs for Q of `q` and K/V
 * of `k` (same B, N, d; k->H = H_kv).  0 for invalid shapes. */
size_t sparge_workspace_size(const sparge_tensor* q, const sparge_tensor* k);

/*
 * Host only.  3D Hilbert order of a T x H x W token grid stored in raster
 * order (token id (t*H + h)*W + w) ([Review] "HilbertCurve Permutation";
 * [Rebuttal] Weaknesses3): every point gets its index on the Hilbert curve of
 * the enclosing 2^b cube (Skilling's transpose algorithm, axes t, h, w, axis t
 * most significant), and tokens are sorted by index.  perm[p] = token of rank
 * p, inv[perm[p]] = p; both hold T*H*W int32 and are written by the library.
 * Returns SPARGE_EINVAL for non-positive sizes or null pointers,
 * SPARGE_EUNSUPPORTED if T*H*W >= 2^31.
 */
int sparge_hilbert_index(int T, int H, int W, int32_t* perm, int32_t* inv);

/*
 * Token gather or scatter along N of one tensor x -> y (same sizes; dtype
 * SPARGE_F16, SPARGE_BF16, SPARGE_I8 or SPARGE_F32 only sets the element
 * size; a row of d elements must be a multiple of 16 bytes).
 * inverse = 0: y[b,h,p,:] = x[b,h,perm[p],:] (Q, K, V into curve order).
 * inverse = 1: y[b,h,perm[p],:] = x[b,h,p,:] (the output back to raster order).
 * perm is a device int32 array of N entries forming a permutation of 0..N-1.
 * It is not validated: an entry outside [0, N) moves nothing (that row of y
 * is left as it was), so a malformed order cannot read or write outside x
 * and y.  The byte ranges x and y span must not overlap (SPARGE_EINVAL).
 */
int sparge_hilbert_permute(const void* x, const sparge_tensor* xs, void* y, const sparge_tensor* ys,
                           int dtype, const int32_t* perm, int inverse, void* stream);

/*
 * Per-block symmetric int8 quantisation of Q and K ([Review] Algorithm 1
 * step 2, components table: per-block quantisation, FP16 -> INT8).
 * K first has its mean over all N tokens of each (b, kv head) subtracted.
 * Per block X (SPARGE_BQ rows of Q, SPARGE_BK rows of K - mean):
 *   delta = max|X| / 127 (1 if X is all zero), code = clamp(rint(X/delta), +-127)
 * with ties to even, all in float64.  Outputs are contiguous:
 *   q8 [B,H,N,d] int8, k8 [B,H_kv,N,d] int8, q_scale [B,H,Tm] float,
 *   k_scale [B,H_kv,Tn] float (delta rounded to float).
 * dtype is the element type of q and k (SPARGE_F16 or SPARGE_BF16).
 */
int sparge_quant_qk_int8(const void* q, const sparge_tensor* qs, const void* k,
                         const sparge_tensor* ks, int dtype, int8_t* q8, int8_t* k8,
                         float* q_scale, float* k_scale, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Stage 1: predict the block mask M_g ([Review] eqs. (4)-(9), Algorithm 1
 * steps 3-5), in float64:
 *   qbar_i, kbar_j = block means (eqs. 4-5);
 *   s = mean pairwise cosine similarity of the block's tokens, computed as
 *       || mean_a x_a / ||x_a|| ||^2 (eq. 6 as corrected in [Rebuttal]
 *       Weaknesses3.1; a zero token counts as a zero unit vector);
 *   Shat[i,j] = qbar_i . kbar_j / sqrt(d), -inf where s_k[j] < theta or the
 *       key block is wholly in the future (causal) (eq. 7);
 *   P^[i] = softmax of the finite entries; TopCdf keeps, in order of
 *       descending P^ (ties: lower j), every entry whose exclusive prefix sum
 *       is below tau * sum(P^[i]) (eq. 8);
 *   M_g[i,:] = 1 on live tiles if s_q[i] < theta, M_g[:,j] = 1 on live tiles
 *       if s_k[j] < theta (eq. 9); tiles wholly in the future are 0.
 * Outputs (device, caller-allocated):
 *   mg      [B,H,Tm,Tn] uint8 (0/1)
 *   row_cnt [B,H,Tm] int32: number of ones in the row
 *   row_idx [B,H,Tm,Tn] uint16: the row's j with M_g = 1, ascending, in the
 *           first row_cnt entries (the rest is unspecified)
 *   s_q [B,H,Tm], s_k [B,H_kv,Tn] float64 self-similarities (may be NULL).
 * tau in (0, 1]; theta finite (theta > 1 makes every block fix: M_g = live).
 * dtype: SPARGE_F16 or SPARGE_BF16.
 */
int sparge_predict_mask(const void* q, const sparge_tensor* qs, const void* k,
                        const sparge_tensor* ks, int dtype, double tau, double theta, int causal,
                        uint8_t* mg, int32_t* row_cnt, uint16_t* row_idx, double* s_q,
                        double* s_k, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Stage 2: block-sparse FlashAttention with the lambda rule ([Review] eqs.
 * (1)-(3), sparse warp online softmax, Algorithm 1 steps 6-17).  For every
 * query block i, key blocks j with M_g[i,j] = 1 on live tiles are visited in
 * ascending j:  S = Q_i K_j^T / sqrt(d) (causal: -inf above the diagonal),
 * m_new = max(m, rowmax S), P~ = exp(S - m_new),
 * l = exp(m - m_new) l + rowsum P~, and, for each group of
 * sparge_rows_per_wave() rows, unless every row with a finite rowmax has
 * rowmax S - m_new < lambda (natural-log units), O = exp(m - m_new) O + P~ V.
 * Finally O = O / l (0 where l = 0), stored in the element type of v.
 *
 * qk_dtype / pv_dtype: (F16, F16), (BF16, BF16), or (I8, F16) / (I8, BF16).
 *   I8: q and k are the contiguous codes of sparge_quant_qk_int8 and
 *   S = (q8 . k8) * q_scale[i] * k_scale[j] / sqrt(d); otherwise the scales
 *   are ignored (may be NULL).  P~ is rounded to pv_dtype before P~V.
 * o_dtype: pv_dtype, or SPARGE_F32 to store the float32 result before its
 *   final rounding (the 16-bit output is exactly that value rounded to
 *   nearest even).
 * mg [B,H,Tm,Tn] uint8 is required.  row_cnt/row_idx (as written by
 *   sparge_predict_mask) are optional: if both are NULL the row lists are
 *   built from mg in the workspace.  Only live tiles are visited.  A given
 *   list must be ascending and hold live tiles only; a row whose count
 *   equals its number of live tiles is run as the list 0, 1, ..., live - 1.
 * workspace (sparge_workspace_size bytes) is required: it holds a
 *   transposed copy of V, the per-row softmax statistics and executed-tile
 *   lists passed from the first to the second attention kernel, the row
 *   lists built from mg, the grouping of the query blocks that list every
 *   live tile, and partial counters.  Everything in it is rewritten by each
 *   call: calls on one stream may share a workspace, calls that can overlap
 *   may not.
 * lambda < 0 (-inf disables the rule).
 * counts: int64[SPARGE_NUM_COUNTERS], overwritten (see SPARGE_CNT_*).
 * pv_dbg: optional uint8 [B,H,Tm,Tn,SPARGE_BQ/sparge_rows_per_wave()] with
 *   1 = group's P~V ran, 2 = skipped by the vote, 3 = no visible key,
 *   0 = tile not visited; the caller clears it beforehand.
 * o: [B,H,N,d] in o_dtype.
 */
int sparge_attn(const void* q, const sparge_tensor* qs, const void* k, const sparge_tensor* ks,
                const void* v, const sparge_tensor* vs, void* o, const sparge_tensor* os,
                int qk_dtype, int pv_dtype, int o_dtype, const float* q_scale, const float* k_scale,
                const uint8_t* mg, const int32_t* row_cnt, const uint16_t* row_idx,
                double lambda, int causal, int64_t* counts, uint8_t* pv_dbg, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * sparge_attn for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * arguments, results and errors are those of sparge_attn (SPARGE_F16 /
 * SPARGE_BF16 / int8 QK with 16-bit P~V), without `workspace` and
 * `workspace_bytes`: the call's scratch (the transposed V, the per-row
 * softmax statistics and executed-tile lists passed between the two
 * attention kernels, the row lists built from mg when row_cnt/row_idx are
 * NULL, the pairing of dense query blocks, the partial counters and the
 * pilot's counts and path flag) lives
 * in a static device array of SPARGE_NOALLOC_SCRATCH_BYTES that each GPU the
 * library runs on holds until the process ends.  The call allocates nothing
 * and frees nothing; its first use on a device looks up that device's copy
 * of the array.
 * A problem whose scratch exceeds the array returns SPARGE_EWORKSPACE before
 * anything is launched; the scratch grows as
 *   2 B H_kv d 64 Tn + 8 B H N + 6 B H Tm Tn + 8 B H_kv d ceil(N / 1024)
 *   + small terms (bytes), which allows, e.g., B = 1, H = 8, H_kv = 2,
 *   d = 128 up to N = 65536.
 * Every call on one GPU shares that GPU's array and leaves its last contents
 * there; each call rewrites every region it reads before reading it.  Calls
 * that can overlap on one GPU (different streams, or host threads) race on
 * the array and must not be issued.
 */
#define SPARGE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int sparge_attn_noalloc(const void* q, const sparge_tensor* qs, const void* k, const sparge_tensor* ks,
                        const void* v, const sparge_tensor* vs, void* o, const sparge_tensor* os,
                        int qk_dtype, int pv_dtype, int o_dtype, const float* q_scale, const float* k_scale,
                        const uint8_t* mg, const int32_t* row_cnt, const uint16_t* row_idx,
                        double lambda, int causal, int64_t* counts, uint8_t* pv_dbg, void* stream);

/*
 * The "SpargeAttn + Sage2" variant of stage 2 ([Review] Fig. 9): the same
 * block-sparse attention and lambda rule as sparge_attn, with P~V on 8-bit
 * floats (OCP E4M3: 4 exponent bits, bias 7, 3 mantissa bits, largest 448,
 * round to nearest even).  The pages only name the variant; the formats
 * taken here are:
 *   V is scaled per channel by delta_c = 2^e, e the least integer with
 *     max_n |V[n, c]| <= 448 * 2^e (clamped at 2^-100; 1 for a zero
 *     channel), so V / delta_c is exact before its one rounding to E4M3;
 *   P~ = exp(S - m) is scaled by 2^8 and rounded to E4M3, m the running max
 *     at that tile on the fused path (Algorithm 1's order), the row's final
 *     running max on the two-pass path;
 *   O = delta_c * sum(P8 V8) / 2^8 / l, with l the float32 row sum of the
 *     unrounded P~ and the products summed in float32 on the matrix cores.
 * Arguments as sparge_attn, except v_dtype (SPARGE_F16 or SPARGE_BF16): the
 * element type v is stored in (qk_dtype equal to it, or SPARGE_I8); o_dtype
 * is v_dtype or SPARGE_F32.  The workspace also holds the fp8 copy of V^T
 * and the scales.  Same error behaviour as sparge_attn.
 */
int sparge_attn_fp8pv(const void* q, const sparge_tensor* qs, const void* k, const sparge_tensor* ks,
                      const void* v, const sparge_tensor* vs, void* o, const sparge_tensor* os,
                      int qk_dtype, int v_dtype, int o_dtype, const float* q_scale, const float* k_scale,
                      const uint8_t* mg, const int32_t* row_cnt, const uint16_t* row_idx,
                      double lambda, int causal, int64_t* counts, uint8_t* pv_dbg, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Token orders of a T x H x W grid of visual tokens (host), the alternatives
 * the permutation comparison of [Review] (Table 4: random, row-major,
 * time-major, HilbertCurve) sets against each other.  Grid token (t, h, w)
 * has raster index (t H + h) W + w.  perm[p] is the raster index of the
 * token at position p; inv is its inverse.  Both are host int32[T H W]
 * owned by the caller.
 *   SPARGE_ORDER_HILBERT:   as sparge_hilbert_index.
 *   SPARGE_ORDER_ROWMAJOR:  raster order, w fastest, then h, then t (the
 *                           identity).
 *   SPARGE_ORDER_TIMEMAJOR: t fastest, then w, then h: the frames of one
 *                           pixel are adjacent.
 * A random order is the caller's (any permutation works with
 * sparge_hilbert_permute).  Errors: SPARGE_EINVAL for non-positive sizes, an
 * unknown order or null outputs; SPARGE_EUNSUPPORTED past 2^31 tokens.
 */
#define SPARGE_ORDER_HILBERT 0
#define SPARGE_ORDER_ROWMAJOR 1
#define SPARGE_ORDER_TIMEMAJOR 2
int sparge_grid_order(int T, int H, int W, int order, int32_t* perm, int32_t* inv);

/*
 * The two sums of the relative L1 error that bounds the hyper-parameter
 * search of [Review] ("hyper-parameter determination": L1 = sum|O - O'| /
 * sum|O|, O the full-attention output, O' the sparse one):
 * out[0] = sum |o - ref|, out[1] = sum |ref|, over every element.
 * o, ref: [B,H,N,d] of the same sizes, element types dtype_o / dtype_ref
 *   (SPARGE_F16, SPARGE_BF16 or SPARGE_F32), d contiguous.
 * out: device double[2], overwritten.  The sums are taken in float64 in a
 *   fixed order: the same inputs give the same bits on every call.
 * workspace: device scratch of at least sparge_l1_workspace_size() bytes.
 * An empty tensor gives (0, 0).
 */
size_t sparge_l1_workspace_size(void);
int sparge_l1_sums(const void* o, const sparge_tensor* os, int dtype_o, const void* ref,
                   const sparge_tensor* rs, int dtype_ref, double* out, void* workspace,
                   size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARGE_H */

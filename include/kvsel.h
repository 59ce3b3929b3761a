/*
 * kvsel.h -- C ABI of the query-guided KV selection library (libkvsel.so),
 * built for AMD Instinct MI355X (gfx950).
 *
 * The library runs the selection path shared by three methods:
 *   [ACRE]       "Boosting Long-Context Management via Query-Guided Activation
 *                 Refilling" (arXiv 2412.12486)
 *   [CacheFocus] "CacheFocus: Dynamic Cache Re-Positioning for Efficient
 *                 Retrieval-Augmented Generation" (arXiv 2502.11101)
 *   [InfoFlow]   "InfoFlow KV: Information-Flow-Aware KV Recomputation for Long
 *                 Context" (arXiv 2603.05353)
 * in six calls: re-position -> score -> aggregate -> top-k -> gather/refill ->
 * decode attention, plus two calls that fuse neighbouring steps with results
 * defined as those of the pair they replace (kvsel_score_reposition,
 * kvsel_gather_decode).  Three more serve CacheFocus's layer-wise pruning
 * (§2.4-2.5): kvsel_score_units scores a list of units of a cache, re-positioned
 * to their slots, without copying them; kvsel_take composes index lists;
 * kvsel_order lists a kept set by score.  Two serve InfoFlow's chunk reordering
 * (§4.3): kvsel_unit_fractions and kvsel_slot_starts.  kvsel_index_attn
 * attends selected tokens causally to the context (InfoFlow's recomputation).
 *
 * Conventions for every call
 * --------------------------
 * - Tensor pointers are DEVICE pointers, owned by the caller.  The library
 *   allocates nothing and keeps no state between calls; scratch memory is
 *   passed in as (ws, ws_bytes) and sized by the *_workspace() queries.  The
 *   one exception is kvsel_gather_decode_noalloc, whose scratch is a fixed
 *   array of the library's own device memory (see there).
 * - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *   default stream).  It returns KVSEL_OK once its kernels are enqueued.
 * - Arguments are validated before anything is enqueued.  On a negative status
 *   nothing was launched and no output was written; kvsel_last_error() gives a
 *   message.  A fault during execution surfaces at the caller's next
 *   synchronisation, as with any HIP kernel.
 * - Caches are [B][N][H][D]: instance, cached row, kv head, head dim.  Within a
 *   row the H*D elements are contiguous; rows and instances may be strided
 *   (kvsel_cache.stride_n / stride_b, in elements, multiples of 8; stride_n
 *   below 2^24, else KVSEL_ERR_UNSUPPORTED).  Pointers
 *   must be 16-byte aligned.  Query blocks are contiguous [B][T][Hq][D] in the
 *   cache dtype.  Per-row statistics are [B][Hq][T] (a "row" is one query head
 *   and query token).  Hq must be a multiple of H; query head h reads kv head
 *   h / (Hq / H).
 * - Supported: head dim D in {64, 128}; dtype bf16 or fp32 (the query, the
 *   cache and any second cache of one call share the dtype).  Dot products of
 *   the cache dtype's operands accumulate in fp32 (packed bf16 dots or the
 *   matrix cores for bf16); softmax arithmetic is fp32; re-rotation is fp64
 *   with one rounding to the cache dtype.
 * - A "unit" is unit_len consecutive cached rows: a chunk, a document, an L1
 *   entry's L2 block, or a single token (unit_len = 1).  N must be a multiple
 *   of unit_len; M = N / unit_len.
 * - `scale` (the logit scale, usually 1/sqrt(D)) must be finite and > 0 in
 *   every call that takes it, else KVSEL_ERR_SHAPE: the kernels take the
 *   maximum of the unscaled dot products, which is the maximum logit only for
 *   a positive scale.
 */
#ifndef KVSEL_H
#define KVSEL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define KVSEL_OK               0
#define KVSEL_ERR_NULL        -1  /* a required pointer is NULL                  */
#define KVSEL_ERR_SHAPE       -2  /* sizes are inconsistent or out of range      */
#define KVSEL_ERR_DTYPE       -3  /* dtype is not bf16 / fp32                    */
#define KVSEL_ERR_UNSUPPORTED -4  /* head dim, alignment or stride not supported */
#define KVSEL_ERR_WORKSPACE   -5  /* workspace smaller than the query returned   */
#define KVSEL_ERR_HIP         -6  /* the HIP runtime rejected a launch           */

/* Element types of caches and query blocks. */
#define KVSEL_BF16 0
#define KVSEL_FP32 1

/* Which dimensions form RoPE's 2-D slices: (i, i + D/2) or (2i, 2i + 1). */
#define KVSEL_ROPE_HALF        0
#define KVSEL_ROPE_INTERLEAVED 1

/* Aggregation signal. */
#define KVSEL_SIG_MASS  0  /* softmax attention weight                      */
#define KVSEL_SIG_VNORM 1  /* attention weight x L2 norm of the value row    */

/* A cache tensor [B][N][H][D]. */
typedef struct kvsel_cache {
  int64_t B;         /* instances (requests x layers, layers, ...)        */
  int64_t N;         /* cached rows per instance                          */
  int64_t H;         /* kv heads                                          */
  int64_t D;         /* head dim: 64 or 128                               */
  int64_t stride_b;  /* elements between instances, >= N * stride_n       */
  int64_t stride_n;  /* elements between rows, >= H * D and < 2^24       */
  int32_t dtype;     /* KVSEL_BF16 or KVSEL_FP32                          */
} kvsel_cache;

/* One key/value segment of the cache read by the final attention pass. */
typedef struct kvsel_segment {
  const void* k;     /* device pointer, cache layout of `kc`              */
  const void* v;     /* device pointer, same layout                       */
  kvsel_cache kc;
} kvsel_segment;

/*
 * kvsel_reposition -- cache re-positioning ([CacheFocus §2.3]: a rotation's
 * inverse is its transpose, so a cached key is un-rotated and rotated again at
 * its new position; [InfoFlow §4.2]: global position reconstruction
 * g(t) = Delta_i + p_i(t); the rotation matrix is [InfoFlow §3.2]).
 *
 * Every row of unit u is rotated by delta[u] positions:
 *   k_out = R(p_old + delta) R(p_old)^T k_in = R(delta) k_in,
 * pair i turning by delta * theta_i with theta_i = rope_base^(-2i/D).  The
 * angle and the 2x2 rotation are computed in fp64 and the result is rounded
 * once to the cache dtype (nearest even).  Values are not touched (only keys
 * carry RoPE).
 *
 *   k_in, k_out  cache `kc`; k_out may equal k_in (in place), else it must not
 *                overlap k_in and uses the same strides.
 *   unit_len     rows per unit (N % unit_len == 0).
 *   delta        device int64: [M] shared by all instances, or [B][M] when
 *                delta_per_instance != 0.  |delta| < 2^31.
 *   rope_style   KVSEL_ROPE_HALF or KVSEL_ROPE_INTERLEAVED.
 */
int kvsel_reposition(const void* k_in, void* k_out, kvsel_cache kc,
                     int64_t unit_len, const int64_t* delta,
                     int32_t delta_per_instance, double rope_base,
                     int32_t rope_style, hipStream_t stream);

/*
 * kvsel_score -- the query block attends the cached keys ([ACRE §2.4]:
 * A = softmax(Q_q K^T / sqrt(d)); [ACRE §2.1 Eq. 4]).
 *
 * With l[b,h,j,t] = scale * q[b,j,h,:] . k[b,t,kv(h),:] and the softmax over
 * all N cached rows of the instance (no mask), computes
 *   row_max[b,h,j] = max_t l,   row_sum[b,h,j] = sum_t exp(l - row_max)
 * and, per unit u, the partials
 *   part[b,h,j,u] = (m_u, S_u),  m_u = max_{t in u} l,  S_u = sum_{t in u} exp(l - m_u).
 *
 *   q            [B][T][Hq][D], cache dtype.
 *   k            keys in the scoring frame (after kvsel_reposition if any).
 *   scale        usually 1/sqrt(D).
 *   row_max, row_sum  fp32 [B][Hq][T]; both NULL or both set.
 *   part         fp32 [B][Hq][T][M][2], or NULL.  Requires unit_len > 1.
 *   At least one of (row_max, part) must be set.  When only `part` is set a
 *   single kernel runs and needs no workspace.
 *   ws           kvsel_score_workspace(...) bytes (may be 0 -> ws NULL).
 */
int kvsel_score(const void* q, int64_t T, int64_t Hq, const void* k,
                kvsel_cache kc, float scale, int64_t unit_len, float* row_max,
                float* row_sum, float* part, void* ws, size_t ws_bytes,
                hipStream_t stream);
size_t kvsel_score_workspace(int64_t B, int64_t N, int64_t Hq, int64_t T,
                             int64_t unit_len, int32_t want_row_stats,
                             int32_t want_part);

/*
 * kvsel_score_reposition -- kvsel_reposition followed by kvsel_score on the
 * re-positioned keys, in one pass where the shape allows it ([CacheFocus §2.3]
 * re-positions the cached keys before the query-document attention;
 * [InfoFlow §4.2] scores after global position reconstruction).
 *
 * Same results as kvsel_reposition(k -> k_out, rot_unit_len, delta, ...) and
 * then kvsel_score(q, ..., k_out, ...): the keys are rotated with the same
 * fp64 arithmetic and single rounding, so the scores are those of the
 * rounded re-positioned keys.  Where bf16 query blocks have >= 16 rows per kv
 * head, the scoring segment (unit_len with `part`, else 256) and rot_unit_len
 * are multiples of 64, the rotation happens while the keys are staged for
 * scoring: the keys are read once, and k_out (when not NULL) receives the
 * re-positioned keys.  Otherwise the two passes run, through k_out or, when
 * it is NULL, through the tail of the workspace.
 *   k_out        NULL or a cache with the layout of `kc`; must not overlap k.
 *   rot_unit_len, delta, delta_per_instance, rope_base, rope_style
 *                as unit_len, delta, ... of kvsel_reposition.
 *   ws           kvsel_score_reposition_workspace(..., have_k_out) bytes.
 *   other arguments as for kvsel_score.
 */
int kvsel_score_reposition(const void* q, int64_t T, int64_t Hq, const void* k,
                           void* k_out, kvsel_cache kc, float scale,
                           int64_t unit_len, int64_t rot_unit_len,
                           const int64_t* delta, int32_t delta_per_instance,
                           double rope_base, int32_t rope_style,
                           float* row_max, float* row_sum, float* part,
                           void* ws, size_t ws_bytes, hipStream_t stream);
size_t kvsel_score_reposition_workspace(int64_t T, int64_t Hq, kvsel_cache kc,
                                        int64_t unit_len, int64_t rot_unit_len,
                                        int32_t want_row_stats, int32_t want_part,
                                        int32_t have_k_out);

/*
 * kvsel_score_units -- kvsel_score_reposition over a list of units of the
 * cache: instance b scores the cache formed by concatenating, in list order,
 * the n_units units units[b][0..n_units) of its own cache (unit_len rows each),
 * with virtual unit j re-positioned by delta[j] (delta_per_instance: by
 * delta[b][j]) positions, or not re-positioned when delta is NULL.  This is
 * one layer of [CacheFocus §2.4]: the caches of the current cache IDs are
 * concatenated, re-positioned (§2.3 / §2.3.1: each cache to its slot's
 * start) and attended by the query.
 *
 * Results are those of copying the listed units into a compact cache of
 * n_units * unit_len rows, kvsel_reposition on it with unit_len and delta,
 * then kvsel_score: row_max/row_sum [B][Hq][T] over the n_units * unit_len
 * scored rows, part [B][Hq][T][n_units][2] (segment j = virtual unit j).
 * Where bf16 query blocks have >= 16 rows per kv head and unit_len (and the
 * scoring segment, unit_len with part, else 256) is a multiple of 64, the
 * listed units are read in place, rotated while staged and scored in one
 * kernel (no copy); otherwise the copy goes through the workspace.
 *   kc           the source caches (B instances of kc.N rows, any strides).
 *   units        int32 [B][n_units]; each entry in [0, kc.N / unit_len)
 *                (repeats allowed).  An entry outside that range reads no
 *                memory; its rows' contribution is unspecified.
 *   delta        int64 [n_units] or [B][n_units], or NULL; rope_base > 1 and
 *                rope_style as kvsel_reposition when set.
 *   ws           kvsel_score_units_workspace(...) bytes (may be 0 -> ws NULL).
 *   other arguments as for kvsel_score.
 */
int kvsel_score_units(const void* q, int64_t T, int64_t Hq, const void* k,
                      kvsel_cache kc, float scale, int64_t unit_len,
                      const int32_t* units, int64_t n_units,
                      const int64_t* delta, int32_t delta_per_instance,
                      double rope_base, int32_t rope_style, float* row_max,
                      float* row_sum, float* part, void* ws, size_t ws_bytes,
                      hipStream_t stream);
size_t kvsel_score_units_workspace(int64_t T, int64_t Hq, kvsel_cache kc,
                                   int64_t unit_len, int64_t n_units,
                                   int32_t want_row_stats, int32_t want_part);

/*
 * kvsel_aggregate -- per-unit relevance from the softmax-normalised
 * attention, with alpha = exp(l - row_max) / row_sum:
 *   KVSEL_SIG_MASS:  S[g,u] = sum_{b in g} sum_h sum_j sum_{t in u} alpha
 *                    ([ACRE §2.4 Eq. 15] pooling over heads and query tokens,
 *                    as a sum: the mean times Hq*T, same ranking;
 *                    [CacheFocus §2.4 footnote 3] document-wise accumulation)
 *   KVSEL_SIG_VNORM: S[g,u] = sum_{b in g} sum_h sum_j sum_{t in u}
 *                    alpha * ||v[b,t,kv(h),:]||_2
 *                    ([InfoFlow §4.2] attention-norm token score s_j = sum_i A_ij)
 * where group g is `group` consecutive instances (e.g. the layers whose scores
 * are summed).  Output unit_score fp32 [B/group][M].  With accumulate != 0
 * the result is added to what unit_score holds (a running total over calls,
 * [CacheFocus §2.4 footnote 3]: document-wise attention accumulated layer by
 * layer); the call's own sum is formed first, in a fixed order, then added.
 *
 * Two paths:
 *  - chunk path (signal MASS and part != NULL): combines the partials of
 *    kvsel_score; q, k, v are not read and may be NULL; row_max/row_sum may be
 *    NULL (then derived from part).
 *  - token path (otherwise): re-reads q and k (and v for VNORM) and needs
 *    row_max/row_sum from kvsel_score; works for any unit_len >= 1.  Its
 *    workspace holds per-token sums: B*N floats, or 16*B*N when B*N < 2^19
 *    (small caches split the kv heads over groups of workgroups, each with
 *    its own partial sums, added in a fixed order).
 *   ws           kvsel_aggregate_workspace(...) bytes (both paths need one).
 */
int kvsel_aggregate(const void* q, int64_t T, int64_t Hq, const void* k,
                    const void* v, kvsel_cache kc, float scale,
                    const float* row_max, const float* row_sum,
                    const float* part, int32_t signal, int64_t unit_len,
                    int64_t group, float* unit_score, int32_t accumulate,
                    void* ws, size_t ws_bytes, hipStream_t stream);
size_t kvsel_aggregate_workspace(int64_t B, int64_t N, int64_t Hq, int64_t T,
                                 int64_t unit_len, int32_t chunk_path,
                                 int32_t have_row_stats);

/*
 * kvsel_topk -- arg-top-k per row of scores ([ACRE §2.4 Eq. 16]
 * I = argtop_k(S); [InfoFlow §4.2] global budget k).
 *
 * Order: score descending, ties by smaller index (-0.0 equals +0.0); NaN
 * scores are not allowed.  The k kept indices are written in ASCENDING index
 * order (the order-preserving refill of [ACRE Eq. 18-19]).
 *   score  fp32 [G][M];  idx int32 [G][k];  val fp32 [G][k] (score of each
 *   kept index, same order) or NULL.  0 <= k <= M, M < 2^31, G < 2^21.
 *   k == 0 is a no-op.
 */
int kvsel_topk(const float* score, int64_t G, int64_t M, int64_t k,
               int32_t* idx, float* val, hipStream_t stream);

/*
 * kvsel_take -- out[g][j] = src[g][idx[g][j]] for j < k: composes two index
 * lists, e.g. the positions kvsel_topk kept in the current list of cache IDs
 * with that list, giving the cache IDs left after a pruning layer
 * ([CacheFocus §2.4]).
 *   src   int32 [G][m];  idx int32 [G][k];  out int32 [G][k], not overlapping
 *   src or idx.  An idx entry outside [0, m) gives -1.  G * k < 2^31.
 *   k == 0 is a no-op.
 */
int kvsel_take(const int32_t* src, int64_t G, int64_t m, const int32_t* idx,
               int64_t k, int32_t* out, hipStream_t stream);

/*
 * kvsel_order -- list k given indices of each row by their scores
 * ([CacheFocus §2.5] attention-guided "sort" allocation: the remaining caches
 * are placed in order of their aggregated attention).
 *
 * Rank of an entry = number of entries before it in the order (score
 * descending, index ascending, list position ascending): the same order as
 * kvsel_topk, made total.  descending != 0: idx_out[g][r] is the entry of
 * rank r (most relevant first); descending == 0: the exact reverse (most
 * relevant last, i.e. nearest a query that follows the caches).
 *   score    fp32 [G][M];  idx int32 [G][k] (entries in [0, M); an entry
 *            outside ranks as the lowest score and gets value 0).
 *   idx_out  int32 [G][k], not overlapping idx;  val_out fp32 [G][k] (the
 *            score of each listed index) or NULL.  k == 0 is a no-op.
 *   G * ceil(k / 256) < 2^23.  Cost: k^2 comparisons per row (meant for
 *   kept sets, not whole caches).
 */
int kvsel_order(const float* score, int64_t G, int64_t M, const int32_t* idx,
                int64_t k, int32_t descending, int32_t* idx_out,
                float* val_out, hipStream_t stream);

/*
 * kvsel_index_attn -- attention of selected tokens to the context under a
 * causal constraint: the recomputation of selected tokens at their global
 * positions ([InfoFlow §4.2] KV recomputation; [InfoFlow §8] the index-based
 * causal pattern, neither dense nor strictly causal).
 *
 * Selected token j of instance b sits at context position pos[b][j]; its query
 * row for head h attends to keys 0 .. min(pos[b][j], N - 1), its own row
 * included:
 *   out[b,j,h,:] = sum_{t <= pos} softmax_t(scale * q[b,j,h,:] . k[b,t,kv(h),:]) v[b,t,kv(h),:]
 *   lse[b,h,j]   = natural log of sum_{t <= pos} exp(scale * q . k_t)
 * A negative position attends to nothing: a zero row and lse = -inf.
 *
 *   q      [B][S][Hq][D] bf16, the selected tokens' queries.
 *   pos    int32 [B][S], device; any order (ascending keeps a workgroup's
 *          rows close together and is fastest).
 *   k, v   the context, cache `kc` (bf16 only: the matrix-core kernel).
 *   out    fp32 [B][S][Hq][D];  lse fp32 [B][Hq][S] or NULL.
 *   S * Hq < 2^31.  No workspace: every row's output is written once.
 * As in kvsel_decode_attn's matrix-core pass, the weights exp(l - ref) are
 * rounded to bf16 before they multiply V, and the sum that normalises them
 * adds the same rounded weights, in fp32.
 */
int kvsel_index_attn(const void* q, int64_t S, int64_t Hq, float scale,
                     const void* k, const void* v, kvsel_cache kc,
                     const int32_t* pos, float* out, float* lse,
                     hipStream_t stream);

/*
 * kvsel_unit_fractions -- r[g][u] = |sel_g ∩ unit u| / unit_len: the share of
 * unit u's rows (unit u = rows [u*unit_len, (u+1)*unit_len)) in the index set
 * sel_g ([InfoFlow §4.3], r_i = |S^(1) ∩ C_i| / |C_i| for equal chunks).
 *   sel   int32 [G][k], ascending within each row (kvsel_topk's order);
 *         another order gives unspecified fractions (no fault).
 *   r     fp32 [G][M]; count / unit_len with one rounding, so equal counts
 *         give equal values and larger counts larger ones.
 *   G * M < 2^31, unit_len * M < 2^31.  k may be 0 (all fractions 0).
 */
int kvsel_unit_fractions(const int32_t* sel, int64_t G, int64_t k,
                         int64_t unit_len, int64_t M, float* r,
                         hipStream_t stream);

/*
 * kvsel_slot_starts -- the start position of every unit once the units are
 * concatenated in a new order ([InfoFlow §4.3]: GLOBAL positions
 * reconstructed for the reordered chunks, g(t) = Delta_i + p_i(t)):
 *   delta[g*rep + i][order[g][p]] = base + p * unit_len,   i < rep.
 * With units stored at unit-local positions, delta is the rotation each unit
 * needs (kvsel_reposition / kvsel_score_reposition with
 * delta_per_instance = 1; rep = the instances that share a selection row,
 * e.g. layers).
 *   order  int32 [G][M], a permutation of 0..M-1 per row (kvsel_order's
 *          output); entries outside [0, M) are skipped, and units they leave
 *          out keep what delta held.
 *   delta  int64 [G*rep][M], not overlapping order.
 *   G * M < 2^31, 1 <= rep <= 65536, 0 <= base, base + unit_len * M < 2^31.
 */
int kvsel_slot_starts(const int32_t* order, int64_t G, int64_t M,
                      int64_t unit_len, int64_t base, int64_t rep,
                      int64_t* delta, hipStream_t stream);

/*
 * kvsel_gather -- copy the kept units into a compact cache ("refill",
 * [ACRE §2.4 Eq. 18-19]; final cache of [CacheFocus §2.4]).
 *
 * Instance b uses index row b / idx_group of idx (int32 [B/idx_group][k],
 * ascending, each in [0, M); a slot whose index is outside that range is
 * skipped and its output rows are left as they were).  Unit u of the source is rows
 * [u*unit_len, (u+1)*unit_len) -- with unit_len = l this is the L1-entry ->
 * L2-block proxy map of [ACRE Eq. 11-12].
 *
 * Output layout:
 *  - compact (proxy == NULL): dst [B][k*unit_len][H][D] contiguous, the kept
 *    units in ascending order;
 *  - nested (proxy != NULL, [ACRE Eq. 18-19]): dst [B][m + k*unit_len][H][D]
 *    where m = proxy->N; walking the proxy (L1) entries j in order, a selected
 *    entry is preceded by its unit of source rows, an unselected one stands
 *    alone.  k_proxy / v_proxy use cache `*proxy` (same B, H, D, dtype).
 *
 * Re-positioning on the fly ([CacheFocus §2.5] "align"): when align_base >= 0
 * the kept keys are rotated so that the r-th kept unit occupies positions
 * align_base + r*unit_len + (0..unit_len-1); src_start (device int64 [M], or
 * NULL = all 0) gives the position of each source unit's first row.  Values
 * are copied unchanged.  Not available in nested mode.
 *
 *   v_src / v_dst (and v_proxy) may be NULL to gather keys only.
 *
 * Host-resident source ([ACRE §2.2, §2.4]: the L2 cache offloaded to CPU
 * memory, the L1 cache kept on the GPU): k_src / v_src may be pinned host
 * memory (hipHostMalloc).  The same kernel then reads only the kept rows,
 * over the host link, through the device address the runtime maps them to.
 * Pageable host memory is refused with KVSEL_ERR_UNSUPPORTED before anything
 * is enqueued.  Every other pointer is device memory.
 */
int kvsel_gather(const void* k_src, const void* v_src, kvsel_cache kc,
                 int64_t unit_len, const int32_t* idx, int64_t k,
                 int64_t idx_group, const int64_t* src_start,
                 int64_t align_base, double rope_base, int32_t rope_style,
                 const void* k_proxy, const void* v_proxy,
                 const kvsel_cache* proxy, void* k_dst, void* v_dst,
                 hipStream_t stream);

/*
 * kvsel_decode_attn -- one attention pass of the query rows over the compact
 * cache ([ACRE §2.1 Eq. 4]; decoding on the refilled cache, [ACRE §2.4]).
 *
 *   o[b,j,h,:] = sum_t softmax_t(scale * q[b,j,h,:] . k_t) v_t
 * over the concatenation of the n_seg segments (a HOST array; all share B, H,
 * D and dtype with the query), no mask.  Output fp32 [B][T][Hq][D]; lse (fp32
 * [B][Hq][T], natural log of sum_t exp(l)) or NULL.  1 <= n_seg <= 4; every
 * segment has N >= 1.  For bf16 query blocks with >= 5 rows per kv head the
 * pass runs on the matrix cores (5 to 15 rows padded to one 16-row block) and
 * the attention weights exp(l - ref) are rounded to bf16 before they multiply
 * V; the sum that normalises them adds the same rounded weights, in fp32.
 *   ws  kvsel_decode_workspace(...) bytes (returns 0 for invalid arguments).
 */
int kvsel_decode_attn(const void* q, int64_t T, int64_t Hq, float scale,
                      const kvsel_segment* segs, int32_t n_seg, float* out,
                      float* lse, void* ws, size_t ws_bytes,
                      hipStream_t stream);
size_t kvsel_decode_workspace(int64_t T, int64_t Hq, const kvsel_segment* segs,
                              int32_t n_seg);

/*
 * kvsel_gather_decode -- refill and the final attention pass in one call
 * ([ACRE §2.4 Eq. 18-19] refill of the kept entries, then decoding over the
 * refilled cache, [ACRE §2.4] and [ACRE §2.1 Eq. 4]).
 *
 * Same result as kvsel_gather in the compact layout (no re-positioning, no
 * proxy cache) into (k_dst, v_dst), followed by kvsel_decode_attn over the
 * segments extra[0 .. n_extra) plus that compact cache.  Where the shape
 * allows it (bf16, head dim 128, H in {1,2,4,8} and 1 <= (Hq / H) * T <= 8)
 * one kernel reads every kept row once, writes it to the compact cache and
 * attends to it from registers; otherwise the kernels of the two separate
 * calls run back to back.
 *
 *   q, T, Hq, scale   as in kvsel_decode_attn.
 *   k_src, v_src, kc, unit_len, idx, k, idx_group   as in kvsel_gather
 *                     (pinned host memory allowed for k_src / v_src).  Every
 *                     index must lie in [0, M); a slot outside that range is
 *                     never read from or written to, and the output is then
 *                     unspecified.
 *   k_dst, v_dst      compact cache [B][k * unit_len][H][D], contiguous (may
 *                     be NULL when k == 0).
 *   extra, n_extra    HOST array of 0 .. 3 further segments attended as they
 *                     are (e.g. the L1 cache of [ACRE]); same B, H, D, dtype.
 *                     k == 0 needs at least one extra segment.
 *   out, lse          as in kvsel_decode_attn.
 *   ws                kvsel_gather_decode_workspace(...) bytes.
 */
int kvsel_gather_decode(const void* q, int64_t T, int64_t Hq, float scale,
                        const void* k_src, const void* v_src, kvsel_cache kc,
                        int64_t unit_len, const int32_t* idx, int64_t k,
                        int64_t idx_group, void* k_dst, void* v_dst,
                        const kvsel_segment* extra, int32_t n_extra,
                        float* out, float* lse, void* ws, size_t ws_bytes,
                        hipStream_t stream);
size_t kvsel_gather_decode_workspace(int64_t T, int64_t Hq, kvsel_cache kc,
                                     int64_t unit_len, int64_t k,
                                     const kvsel_segment* extra,
                                     int32_t n_extra);

/*
 * kvsel_gather_decode_noalloc -- for callers that cannot allocate: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments and results as kvsel_gather_decode without (ws, ws_bytes):
 * the split partials live in a fixed array of the library's own device memory,
 * kvsel_noalloc_scratch_bytes() = 128 MiB per GPU, held from the first use on
 * that GPU until the process ends.  The call allocates nothing.
 *   - A shape whose kvsel_gather_decode_workspace() exceeds that size gets
 *     KVSEL_ERR_WORKSPACE before anything is enqueued (16 requests x 8 layers
 *     of one-token queries over 64 chunks of 256 tokens needs 65 MiB).
 *   - The array belongs to the CURRENT device; a stream of another device gets
 *     KVSEL_ERR_UNSUPPORTED.
 *   - Every call on one GPU shares its array, which keeps the last call's
 *     contents: calls that overlap on one GPU (other streams, other host
 *     threads) race.  Run one at a time per GPU.
 */
int kvsel_gather_decode_noalloc(const void* q, int64_t T, int64_t Hq, float scale,
                                const void* k_src, const void* v_src,
                                kvsel_cache kc, int64_t unit_len,
                                const int32_t* idx, int64_t k, int64_t idx_group,
                                void* k_dst, void* v_dst,
                                const kvsel_segment* extra, int32_t n_extra,
                                float* out, float* lse, hipStream_t stream);
size_t kvsel_noalloc_scratch_bytes(void);

/* Text of a status code; message of the last failed call on this thread. */
const char* kvsel_status_str(int status);
const char* kvsel_last_error(void);
/* Library version, major*10000 + minor*100 + patch. */
int kvsel_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVSEL_H */

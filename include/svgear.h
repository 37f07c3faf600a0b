/*
 * svgear.h — C ABI of the MI355X (gfx950) routed sparse-attention library.
 *
 * The library computes the hot path of SVG-EAR ("SVG-EAR: Parameter-Free
 * Linear Compensation for Sparse Video Generation via Error-aware Routing",
 * arXiv 2603.08982) for one attention layer:
 *
 *   svgear_cluster   k-means of each head's Q rows or K rows      (paper §4.1)
 *   svgear_permute   stable cluster-contiguous permutation + means (§3.1, §4.1, §4.3)
 *   svgear_cluster_permute  both in one call, the last Lloyd pass doing the permutation
 *   svgear_probe     query-centroid error probe -> block ratios    (§4.2, Eq. 5)
 *   svgear_probe_values  the same probe with the value-aware error   (§4.2, §4.3)
 *   svgear_route     greedy error-to-cost selection per query cluster (§4.2, §5)
 *   svgear_route_global  the same greedy selection under one budget per head (§4.1, §4.2)
 *
 * and, for the error analysis of block selections (§5.3, Fig. 6a):
 *
 *   svgear_block_scores  centroid-estimated attention mass of every block (top-p ranking)
 *   svgear_map_error     squared distance of a block-sparse attention map from the full one
 *   svgear_row_spread    squared distance of every permuted row from its cluster mean
 *   svgear_attend    exact selected blocks + centroid compensation (§4.1, §4.3)
 *   svgear_unpermute inverse permutation of the output rows        (§3.1)
 *   svgear_attend_unpermute  svgear_attend writing each output row at its
 *                    query's original position (§3.1, §4.1, §4.3)
 *
 * and two measurement helpers outside the method: svgear_clock_probe and
 * svgear_realtime_khz (the shader clock under matrix-core load).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensors are DEVICE pointers, row-major, head-major: X[h][n][j] at
 *    X + (h*N + n)*d + j. Index arrays are int32 device pointers.
 *  - svgear_dtype names the element type of Q/K/V-like tensors: SVGEAR_F32
 *    (float) or SVGEAR_BF16 (bfloat16 stored as uint16). Centroid tables,
 *    ratios and normalisers are always float32.
 *  - Supported head dimension d: 64 or 128. Cluster counts: 1 <= C <= min(N, 1024).
 *    One head holds fewer than 2^31 elements (N*d < 2^31) and all heads
 *    together at most 2^40.
 *  - Ownership: the caller allocates and frees every buffer, including the
 *    workspace; the library never allocates, frees or synchronises. Work is
 *    enqueued on the caller's stream `s` (0 = the legacy default stream) and
 *    every buffer must stay valid until that work has completed.
 *  - Errors: argument problems are reported synchronously, before anything
 *    is enqueued (SVGEAR_ERR_INVALID_ARG, SVGEAR_ERR_UNSUPPORTED,
 *    SVGEAR_ERR_WORKSPACE). Once the arguments pass, every call that launches
 *    work checks that the calling thread's current HIP device is a gfx950
 *    (looked up once per device, then cached) and returns
 *    SVGEAR_ERR_UNSUPPORTED otherwise, also when no device is present. A
 *    failed kernel launch returns SVGEAR_ERR_HIP.
 *    Faults inside kernels surface at the caller's next synchronisation, as
 *    for any asynchronous HIP work.
 *  - Calls hold no state between invocations and may be made from several
 *    host threads on different streams; two calls that share an output or a
 *    workspace buffer must be ordered by the caller.
 *  - Results are deterministic: the same inputs give bitwise identical
 *    outputs (no floating-point atomics).
 */
#ifndef SVGEAR_H
#define SVGEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* svgear_stream_t; /* same object as hipStream_t */

typedef enum {
  SVGEAR_OK = 0,
  SVGEAR_ERR_INVALID_ARG = 1, /* null pointer, size out of range, inconsistent sizes */
  SVGEAR_ERR_UNSUPPORTED = 2, /* dtype or head dimension not built, or the current
                                 device is not a gfx950 (MI355X) GPU */
  SVGEAR_ERR_WORKSPACE = 3,   /* workspace smaller than the matching *_workspace() */
  SVGEAR_ERR_HIP = 4          /* the HIP runtime refused a launch */
} svgear_status;

typedef enum { SVGEAR_F32 = 0, SVGEAR_BF16 = 1 } svgear_dtype;

/* Human-readable name of a status code (static storage, never NULL). */
const char* svgear_status_string(svgear_status st);

/* Bytes of workspace svgear_cluster needs for H heads of N rows, dimension d,
 * C clusters, element type dt. Returns 0 for arguments svgear_cluster would reject. */
size_t svgear_cluster_workspace(svgear_dtype dt, int H, int N, int d, int C);

/*
 * k-means clustering of every head's rows (paper §4.1: Q and K are clustered
 * into C_q and C_k clusters).
 *
 * Runs `iters` (>= 1) Lloyd iterations from the caller's initial centroids:
 * each row goes to the centroid with the smallest squared Euclidean distance
 * (ties to the lowest index), then every centroid with members becomes their
 * mean; a centroid without members keeps its value. The distance is formed
 * from the centroid rounded to the input element type (bf16 or f32),
 * accumulated in f32; means are accumulated in f32 in a fixed order.
 *
 *   X         [H][N][d] dt, input rows.
 *   centroids [H][C][d] f32, in: initial centroids; out: means of the final labels
 *             (empty clusters keep their last value).
 *   labels    [H][N] int32 out: cluster of every row from the last assignment.
 *   counts    [H][C] int32 out: members per cluster under those labels.
 *   ws        device workspace of at least svgear_cluster_workspace(...) bytes.
 */
svgear_status svgear_cluster(svgear_dtype dt, int H, int N, int d, int C, int iters,
                             const void* X, float* centroids, int32_t* labels, int32_t* counts,
                             void* ws, size_t ws_bytes, svgear_stream_t s);

/* Bytes of workspace svgear_permute needs. */
size_t svgear_permute_workspace(svgear_dtype dt, int H, int N, int d, int C);

/*
 * Stable permutation that lays every cluster out contiguously (paper §3.1),
 * applied to one or two tensors that share the labels, with the mean row of
 * every cluster (the centroids q-bar, k-bar and mean values v-bar of §4.1/§4.3;
 * V takes K's labels).
 *
 *   labels    [H][N] int32 in, each in [0, C) (values outside are clamped into
 *             that range, so no access leaves its buffer).
 *   perm      [H][N] int32 out: perm[p] = source row placed in slot p; rows of
 *             one cluster keep their original order.
 *   offsets   [H][C+1] int32 out: cluster c occupies slots offsets[c]..offsets[c+1]-1.
 *   ntensors  1 or 2.
 *   src       host array of ntensors device pointers, [H][N][d] dt each.
 *   dst       host array of ntensors device pointers, [H][N][d] dt each (permuted
 *             rows: dst[p] = src[perm[p]]); must not alias src.
 *   means     host array of ntensors device pointers, [H][C][d] f32 each, or NULL
 *             entries to skip; empty clusters get a zero row. `means` itself may be NULL.
 */
svgear_status svgear_permute(svgear_dtype dt, int H, int N, int d, int C, const int32_t* labels,
                             int32_t* perm, int32_t* offsets, int ntensors,
                             const void* const* src, void* const* dst, float* const* means,
                             void* ws, size_t ws_bytes, svgear_stream_t s);

/* Bytes of workspace svgear_probe needs. */
size_t svgear_probe_workspace(int H, int Nk, int Cq, int Ck);

/*
 * svgear_cluster followed by svgear_permute on its labels, in one call
 * (paper §4.1: Q and K are clustered, then each cluster is made contiguous).
 * The last Lloyd iteration's counting sort is the final permutation, so its
 * segment-sum pass also writes the permuted copies and the means, and the
 * separate permutation's extra read of the inputs and its sort are saved.
 * Every output is bitwise what the two calls produce.
 *
 *   src[0] is the clustered tensor X [H][N][d] dt; src[1] (ntensors = 2) follows
 *   X's labels (V with K). dst[k] [H][N][d] dt receives src[k] in permuted
 *   order; means[k] [H][C][d] f32 (entries may be NULL) its segment means (0
 *   for an empty cluster).
 *   centroids [H][C][d] f32 in: initial table; out: the k-means centroids (an
 *   empty cluster keeps its centroid, otherwise the mean of X over the final
 *   labels). labels [H][N], counts [H][C], perm [H][N], offsets [H][C+1] int32
 *   out, as in svgear_cluster and svgear_permute.
 *   ws: svgear_cluster_permute_workspace(dt, H, N, d, C) bytes.
 * Errors as svgear_cluster and svgear_permute.
 */
size_t svgear_cluster_permute_workspace(svgear_dtype dt, int H, int N, int d, int C);
svgear_status svgear_cluster_permute(svgear_dtype dt, int H, int N, int d, int C, int iters,
                                     int ntensors, const void* const* src, void* const* dst,
                                     float* const* means, float* centroids, int32_t* labels,
                                     int32_t* counts, int32_t* perm, int32_t* offsets, void* ws,
                                     size_t ws_bytes, svgear_stream_t s);

/*
 * Query-centroid error probe (paper §4.2, Eq. 5) and block error-to-size ratio.
 *
 * For query centroid c and permuted key j of key cluster k(j), with
 * s = scale*qbar_c.k_j, s~ = scale*qbar_c.kbar_k(j), m_c = max_j s and
 * Z_c = sum_j exp(s - m_c):
 *     eps_cj = (exp(s - m_c) - exp(s~ - m_c)) / Z_c
 *     ratio[c][c'] = (1/|k_c'|) * sum_{j in c'} eps_cj^2      (-1 if |k_c'| = 0)
 *     log_norm[c]  = m_c + ln Z_c
 * The logits are formed from q-bar split into a bf16 high part and a bf16
 * remainder (about 16 significant bits) against the bf16 or f32 keys, f32 accumulation.
 *
 *   q_centroids [H][Cq][d] f32;  Kp [H][Nk][d] dt (permuted keys);
 *   k_centroids [H][Ck][d] f32;  k_offsets [H][Ck+1] int32 (offsets[Ck] = Nk);
 *   ratio       [H][Cq][Ck] f32 out;  log_norm [H][Cq] f32 out, may be NULL.
 */
svgear_status svgear_probe(svgear_dtype dt, int H, int Nk, int d, int Cq, int Ck, float scale,
                           const float* q_centroids, const void* Kp, const float* k_centroids,
                           const int32_t* k_offsets, float* ratio, float* log_norm, void* ws,
                           size_t ws_bytes, svgear_stream_t s);

/*
 * Value-aware query-centroid error probe (paper §4.2's value-aware estimate,
 * which brings the values of the linear-compensation output of §4.3 into the
 * error). Its display was lost; the reading implemented: with the two weights
 * of svgear_probe, p = exp(s - m)/Z (raw key) and p~ = exp(s~ - m)/Z (key
 * centroid), key j of key cluster c' contributes
 *     eps_cj = || p_cj v_j - p~_cj vbar_c' ||^2
 * and ratio[c][c'] = (1/|k_c'|) sum_{j in c'} eps_cj.
 *
 * Arguments as svgear_probe, plus
 *   Vp          [H][Nk][d] dt (permuted values, the keys' order);
 *   v_centroids [H][Ck][d] f32 (mean value of every key cluster).
 * The split p^2 ||v_j - vbar||^2 + 2 p (p - p~) (v_j - vbar).vbar + (p - p~)^2 ||vbar||^2
 * is summed with f32 accumulation from per-key terms computed once per call.
 * ws: svgear_probe_values_workspace(H, Nk, Cq, Ck) bytes. Errors as svgear_probe.
 */
size_t svgear_probe_values_workspace(int H, int Nk, int Cq, int Ck);
svgear_status svgear_probe_values(svgear_dtype dt, int H, int Nk, int d, int Cq, int Ck,
                                  float scale, const float* q_centroids, const void* Kp,
                                  const float* k_centroids, const void* Vp,
                                  const float* v_centroids, const int32_t* k_offsets,
                                  float* ratio, float* log_norm, void* ws, size_t ws_bytes,
                                  svgear_stream_t s);

/*
 * Greedy error-to-cost routing per query cluster (paper §4.2 "Error
 * estimation", §5 "Implementation": routing at query-cluster granularity).
 *
 * For every (head, non-empty query cluster): non-empty key clusters are
 * ordered by ratio, highest first, equal ratios by lower index; walking that
 * order once, a key cluster is selected when its keys still fit in
 * `budget_keys` (clusters that do not fit are passed over; later, smaller ones
 * may still fit). A query cluster without queries selects nothing.
 * budget_keys = floor(rho * Nk) is computed by the caller.
 *
 *   ratio     [H][Cq][Ck] f32 in (>= 0 for non-empty clusters; NaN and negative
 *             values count as 0; the value of empty clusters is ignored).
 *   q_offsets [H][Cq+1] int32 in, or NULL (then every query cluster is routed).
 *   k_offsets [H][Ck+1] int32 in.
 *   sel_mask  [H][Cq][Ck] uint8 out (1 = exact).
 *   sel_list  [H][Cq][Ck] int32 out: selected key clusters ascending, -1 padded. May be NULL.
 *   sel_count [H][Cq] int32 out: number selected. May be NULL.
 *   sel_keys  [H][Cq] int32 out: exact keys used (<= budget_keys). May be NULL.
 *   ws        svgear_route_workspace(H, Cq, Ck) bytes; that size is 0 (the sort
 *             runs in on-chip memory), so ws may be NULL and ws_bytes 0.
 * Returns SVGEAR_ERR_INVALID_ARG for sizes outside 1..1024, a negative budget or
 * a NULL required pointer; nothing is launched then.
 */
size_t svgear_route_workspace(int H, int Cq, int Ck);
svgear_status svgear_route(int H, int Cq, int Ck, const float* ratio, const int32_t* q_offsets,
                           const int32_t* k_offsets, int32_t budget_keys, uint8_t* sel_mask,
                           int32_t* sel_list, int32_t* sel_count, int32_t* sel_keys, void* ws,
                           size_t ws_bytes, svgear_stream_t s);

/*
 * Greedy error-to-cost routing under one budget for the whole attention map of
 * a head (paper §4.1: at most rho * Nq * Nk exact entries in the block mask;
 * §4.2: blocks taken in decreasing order of estimated error per entry while
 * the budget lasts). Unlike svgear_route, the budget is not split per query
 * cluster.
 *
 * Every block (c, c') whose query cluster and key cluster are both non-empty
 * competes for `budget_entries` exact (query, key) entries and costs
 * |q_c| * |k_c'| of them. Blocks are ordered by ratio, highest first; equal
 * ratios by lower c, then lower c'. Walking that order once, a block is
 * selected when its cost still fits (blocks that do not fit are passed over;
 * later, cheaper ones may still fit). budget_entries = floor(rho * Nq * Nk) is
 * computed by the caller.
 *
 *   ratio        [H][Cq][Ck] f32 in (>= 0 for non-empty clusters; NaN and
 *                negative values count as 0; values of empty clusters are ignored).
 *   q_offsets    [H][Cq+1] int32 in;  k_offsets [H][Ck+1] int32 in.
 *   sel_mask     [H][Cq][Ck] uint8 out (1 = exact).
 *   sel_list     [H][Cq][Ck] int32 out: selected key clusters ascending, -1 padded. May be NULL.
 *   sel_count    [H][Cq] int32 out. May be NULL.
 *   sel_keys     [H][Cq] int32 out: exact keys of each query cluster. May be NULL.
 *   used_entries [H] int64 out: exact entries used (<= budget_entries). May be NULL.
 *   ws           svgear_route_global_workspace(H, Cq, Ck) bytes (sort buffers).
 *
 * Returns SVGEAR_ERR_INVALID_ARG for sizes outside 1..1024, a negative budget
 * or a NULL required pointer, SVGEAR_ERR_WORKSPACE for a missing or short
 * workspace; nothing is launched then.
 */
size_t svgear_route_global_workspace(int H, int Cq, int Ck);
svgear_status svgear_route_global(int H, int Cq, int Ck, const float* ratio,
                                  const int32_t* q_offsets, const int32_t* k_offsets,
                                  int64_t budget_entries, uint8_t* sel_mask, int32_t* sel_list,
                                  int32_t* sel_count, int32_t* sel_keys, int64_t* used_entries,
                                  void* ws, size_t ws_bytes, svgear_stream_t s);

/*
 * Compensated block-sparse attention on permuted Q, K, V (paper §4.1 block
 * mask, §4.3 linear compensation).
 *
 * Query i of query cluster c gets one softmax over (a) scale*q_i.k_j for every
 * key j of every key cluster c' with sel_mask[c][c'] = 1, value v_j, and (b) for
 * every other non-empty key cluster c', scale*q_i.kbar_c' + ln|k_c'| with value
 * vbar_c'. QK^T and PV run on bf16 (or f32) matrix cores with f32 accumulation;
 * the softmax is f32; for bf16 the probabilities and the centroid rows are
 * rounded to bf16 as matrix operands.
 *
 *   Qp [H][Nq][d], Kp/Vp [H][Nk][d] dt;  q_offsets [H][Cq+1], k_offsets [H][Ck+1];
 *   k_centroids, v_centroids [H][Ck][d] f32;  sel_mask [H][Cq][Ck] uint8;
 *   Op [H][Nq][d] dt out (rows in the permuted query order);
 *   ws  workspace of svgear_attend_workspace(...) bytes (it holds the centroid
 *       rows rounded to dt); may be NULL when that size is 0.
 * One head's K (and V) must span fewer than 2^32 bytes (Nk * d * element
 * bytes); larger heads return SVGEAR_ERR_INVALID_ARG.
 * The selection enters as the mask alone: every block derives both its
 * ascending list of selected key clusters and the list of skipped ones (which
 * the compensation needs) from its mask row in one pass, so svgear_route's
 * sel_list / sel_count are not taken here (a second description of the same
 * selection could only disagree with the first).
 * Inputs must be finite: the kernel is compiled on the assumption that no
 * logit is NaN (running maxima skip NaN quieting); NaN inputs give undefined
 * output values (never an out-of-bounds access).
 */
size_t svgear_attend_workspace(svgear_dtype dt, int H, int Ck, int d);

svgear_status svgear_attend(svgear_dtype dt, int H, int Nq, int Nk, int d, int Cq, int Ck,
                            float scale, const void* Qp, const void* Kp, const void* Vp,
                            const int32_t* q_offsets, const int32_t* k_offsets,
                            const float* k_centroids, const float* v_centroids,
                            const uint8_t* sel_mask, void* Op, void* ws, size_t ws_bytes,
                            svgear_stream_t s);

/*
 * svgear_attend followed by svgear_unpermute in one pass (paper §3.1: the
 * output of the permuted layout is mapped back to the original token order;
 * §4.1, §4.3: the attention itself). Arguments as svgear_attend, except
 *   q_perm [H][Nq] int32: the query permutation (q_perm[h][p] is the original
 *          row of permuted row p; a permutation of 0..Nq-1 per head);
 *   O      [H][Nq][d] dt out, in the original query order: O[h][q_perm[h][p]]
 *          is the result for permuted query p, bitwise what svgear_attend then
 *          svgear_unpermute write. Rows whose q_perm value lies outside
 *          [0, Nq) are not written. O must not alias Qp.
 * Errors as svgear_attend; a NULL q_perm is SVGEAR_ERR_INVALID_ARG.
 */
svgear_status svgear_attend_unpermute(svgear_dtype dt, int H, int Nq, int Nk, int d, int Cq,
                                      int Ck, float scale, const void* Qp, const void* Kp,
                                      const void* Vp, const int32_t* q_offsets,
                                      const int32_t* k_offsets, const float* k_centroids,
                                      const float* v_centroids, const uint8_t* sel_mask,
                                      const int32_t* q_perm, void* O, void* ws, size_t ws_bytes,
                                      svgear_stream_t s);

/*
 * svgear_attend_unpermute without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * with a fixed memory plan, harnesses that forbid hipMalloc). Arguments,
 * results and errors as svgear_attend_unpermute, bitwise the same output.
 *
 * Its scratch (the centroid rows rounded to dt, 2 * H * Ck * d elements of dt
 * for bf16, none for f32) lives in a 32 MiB array of device memory that the
 * library reserves on every GPU it runs on until the process ends; sizes that
 * need more (bf16 with H * Ck * d above about 8.3 million) return
 * SVGEAR_ERR_WORKSPACE before anything is enqueued. The call allocates and
 * frees nothing. All calls on one GPU share that GPU's array: two calls that
 * may overlap on one GPU (different streams, or host threads without
 * ordering) race on it and must be ordered by the caller.
 */
svgear_status svgear_attend_unpermute_noalloc(svgear_dtype dt, int H, int Nq, int Nk, int d,
                                              int Cq, int Ck, float scale, const void* Qp,
                                              const void* Kp, const void* Vp,
                                              const int32_t* q_offsets, const int32_t* k_offsets,
                                              const float* k_centroids, const float* v_centroids,
                                              const uint8_t* sel_mask, const int32_t* q_perm,
                                              void* O, svgear_stream_t s);

/*
 * Inverse permutation of output rows: X[h][perm[h][p]] = Xp[h][p] (paper §3.1).
 *   perm [H][N] int32 (a permutation of 0..N-1 per head); Xp, X [H][N][d] dt, not aliased.
 */
svgear_status svgear_unpermute(svgear_dtype dt, int H, int N, int d, const int32_t* perm,
                               const void* Xp, void* X, svgear_stream_t s);

/*
 * Score-based block ranking of the top-p baseline compared in §5.3 (blocks
 * selected by approximated attention scores, §1 and §4.2): for every query
 * centroid c and key cluster c',
 *     scores[c][c'] = |k_c'| exp(scale qbar_c.kbar_c') / sum over non-empty c''
 * (the block's share of the centroid query's attention mass estimated from the
 * centroids), -1 for empty key clusters. Passed to svgear_route as `ratio` it
 * fills the same budget in decreasing score. f32 throughout.
 *
 *   q_centroids [H][Cq][d] f32;  k_centroids [H][Ck][d] f32;  k_offsets [H][Ck+1];
 *   scores      [H][Cq][Ck] f32 out.
 * Returns SVGEAR_ERR_INVALID_ARG for sizes outside 1..1024, d not 64 or 128, a
 * non-positive scale or a NULL pointer.
 */
svgear_status svgear_block_scores(int H, int d, int Cq, int Ck, float scale,
                                  const float* q_centroids, const float* k_centroids,
                                  const int32_t* k_offsets, float* scores, svgear_stream_t s);

/*
 * Distance of a block-sparse attention map from the full map (§5.3, "Strategy
 * of block selection": (1/(Nq Nk)) ||A_sparse - A_full||_F^2, Fig. 6a).
 *
 * On permuted queries and keys, A_full is softmax(scale q_i.k_j) over all keys.
 * A_sparse keeps the exact weight of every key in a block (query cluster of i,
 * key cluster c') with sel_mask = 1; each key of a skipped non-empty key cluster
 * gets the centroid weight exp(scale q_i.kbar_c') when `compensate` is non-zero
 * (§4.3) and 0 otherwise (top-p without compensation); every sparse row is
 * normalised by its own sum (a row that keeps nothing stays 0).
 *
 *   Qp [H][Nq][d], Kp [H][Nk][d] dt;  q_offsets [H][Cq+1], k_offsets [H][Ck+1];
 *   k_centroids [H][Ck][d] f32;  sel_mask [H][Cq][Ck] uint8;
 *   err      [H][Nq] f32 out: sum_j (A_sparse - A_full)_ij^2 for each query;
 *   z_full   [H][Nq] f32 out: sum_j exp(s_ij - max_j s_ij);
 *   z_sparse [H][Nq] f32 out: the sparse row's normaliser on the same scale.
 * The caller forms the mean squared error as sum(err) / (Nq Nk) and the
 * normaliser change as |z_sparse / z_full - 1|. Logits from bf16 (or f32)
 * matrix cores with f32 accumulation, centroid logits and sums in f32.
 * ws: svgear_map_error_workspace(H, Nq, Ck) bytes (the centroid logits).
 * Errors as svgear_attend; SVGEAR_ERR_WORKSPACE for a missing or short workspace.
 */
size_t svgear_map_error_workspace(int H, int Nq, int Ck);
svgear_status svgear_map_error(svgear_dtype dt, int H, int Nq, int Nk, int d, int Cq, int Ck,
                               float scale, const void* Qp, const void* Kp,
                               const int32_t* q_offsets, const int32_t* k_offsets,
                               const float* k_centroids, const uint8_t* sel_mask, int compensate,
                               float* err, float* z_full, float* z_sparse, void* ws,
                               size_t ws_bytes, svgear_stream_t s);

/*
 * Clustering spread of permuted rows (§4's bound on the map error carries a
 * residual proportional to the queries' clustering error delta_q^2, plotted
 * against C_q in §5.3 Fig. 6b; its formula was lost). For every permuted row p
 * of cluster c:
 *     spread[h][p] = || Xp[h][p] - means[h][c] ||^2   (f32)
 * The mean over rows is the k-means objective per row (delta_q^2 for Q).
 *
 *   Xp [H][N][d] dt (cluster-contiguous rows);  means [H][C][d] f32;
 *   offsets [H][C+1] int32;  spread [H][N] f32 out.
 * Errors as svgear_permute's shape checks; NULL pointers are SVGEAR_ERR_INVALID_ARG.
 */
svgear_status svgear_row_spread(svgear_dtype dt, int H, int N, int d, int C, const void* Xp,
                                const float* means, const int32_t* offsets, float* spread,
                                svgear_stream_t s);

/*
 * Measurement helpers (not part of the method): the shader clock the chip
 * holds while its matrix cores are busy, so that a kernel's fraction of the
 * bf16 matrix peak can also be taken at the clock it actually ran at (the
 * nominal 2.4 GHz drops under matrix load).
 *
 * svgear_clock_probe enqueues `blocks` blocks of four wavefronts, each
 * running `iters` rounds of eight independent bf16 16x16x32 MFMA chains on
 * register operands (no memory traffic). The first wavefront of block 0
 * reads the shader clock counter and the constant-rate real-time counter
 * before and after its chains. Enough blocks to fill the GPU (8 per compute
 * unit) keep every matrix core busy meanwhile.
 *   out  device buffer of at least 4 + blocks uint64 words:
 *        out[0], out[1]  shader clock counter at start and end (cycles),
 *        out[2], out[3]  real-time counter at start and end (ticks),
 *        out[4 + b]      a checksum of block b's products (bits of a float).
 *   blocks, iters in [1, 2^20], out not NULL: else SVGEAR_ERR_INVALID_ARG.
 * svgear_realtime_khz writes the real-time counter's rate for the current
 * device (kHz). The clock in MHz is
 *   (out[1] - out[0]) / (out[3] - out[2]) * khz / 1000.
 */
svgear_status svgear_clock_probe(int blocks, int iters, uint64_t* out, svgear_stream_t s);
svgear_status svgear_realtime_khz(int* khz);

#ifdef __cplusplus
}
#endif

#endif /* SVGEAR_H */

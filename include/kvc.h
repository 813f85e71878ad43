/*
 * kvc.h -- centroid-indexed KV-cache retrieval on MI355X (gfx950).
 *
 * The method is LouisKV's ("LouisKV: Efficient KV Cache Retrieval for Long
 * Input-Output Sequences", papernotes.org note; edgentiq blog of the same
 * method). At prefill each KV head's keys are clustered with K-means and
 * every cluster is indexed by the mean of its keys; at decode, generated KV
 * is cut into temporal segments at semantic boundaries, each indexed by its
 * key mean; a retrieval happens only when the adjacent-query cosine r_t
 * falls below tau, and then selects whole units under a token budget, one
 * set per GQA group; attention runs over the selected rows.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers are DEVICE pointers unless marked [host]. Every call validates
 *   its arguments on the host, enqueues kernels on `stream` and returns; it
 *   never synchronises, never allocates device memory and keeps no global
 *   state. The caller owns every buffer, including workspaces.
 * - Return value: KV_OK (0) or a negative kv_status. Argument errors are
 *   reported before anything is enqueued. Conditions that depend on device
 *   data (running out of pool rows or units while appending) are written to
 *   the pool's device status word; the caller reads it after its own sync.
 * - Element types: KV_BF16 (stored as raw bfloat16 bits) or KV_F32. Head
 *   dimension 64 or 128. Index arithmetic is int32.
 * - Layouts are dense, row-major, innermost dimension last, as written in
 *   brackets. "BH" means batch * n_kv_heads (sequence-major).
 * - GQA: query head h belongs to KV head h / (n_q_heads / n_kv_heads).
 * - Workspaces must be 256-byte aligned. Workspaces of kv_select and
 *   kv_gather_attend hold completion counters: zero-fill them once before
 *   first use; every completed call leaves them zero again. Calls that share
 *   a workspace must not run concurrently.
 * - Determinism: every output is bitwise reproducible for identical inputs
 *   (no floating-point atomics anywhere).
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KV_OK = 0,
  KV_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, inconsistent shapes */
  KV_ERR_UNSUPPORTED = -2, /* head_dim or dtype not supported */
  KV_ERR_WORKSPACE = -3,   /* workspace too small or misaligned */
  KV_ERR_CAPACITY = -4,    /* pool rows/units or selection capacity exceeded */
  KV_ERR_HIP = -5          /* a HIP launch failed */
} kv_status;

typedef enum { KV_F32 = 0, KV_BF16 = 1 } kv_dtype;

/*
 * The unified KV pool of one layer ("Key designs" item 2 of the LouisKV note:
 * prefill clusters and decode segments share one pool and one scoring
 * mechanism). The pool's tables live in HBM; its K and V rows live in HBM
 * or, as in the note's deployment (the full KV cache kept in CPU memory,
 * "Background"), in pinned host memory mapped into the device's address
 * space (see kv_host_device_pointer). Rows of each (sequence, KV head)
 * are stored cluster by cluster (CSR) after kv_cluster_build, then decode
 * rows are appended in time order. Units are contiguous row ranges:
 * clusters have ids 0..C-1, segments C, C+1, ... in closing order.
 * Bookkeeping counters are per sequence (all KV heads of a sequence share
 * cluster count and segment boundaries).
 *
 * The struct itself is [host] memory; every pointer in it is device memory
 * owned by the caller (k and v: device memory, or the device address of
 * mapped host memory). Every kernel reads and writes k and v in place
 * wherever they live; with host memory each access crosses the host link.
 */
typedef struct kv_pool {
  int32_t batch;      /* sequences */
  int32_t n_kv_heads; /* KV heads per sequence */
  int32_t head_dim;   /* 64 or 128 */
  int32_t dtype;      /* kv_dtype of k, v and unit_index */
  int32_t row_cap;    /* rows per (sequence, KV head) */
  int32_t unit_cap;   /* units per (sequence, KV head) */
  void *k;            /* [batch][n_kv_heads][row_cap][head_dim] */
  void *v;            /* same */
  int32_t *unit_start; /* [batch][n_kv_heads][unit_cap] first row of each unit */
  int32_t *unit_size;  /* [batch][n_kv_heads][unit_cap] rows of each unit (0 = empty) */
  float *unit_mean;    /* [batch][n_kv_heads][unit_cap][head_dim] fp32 key mean */
  void *unit_index;    /* same shape, dtype: the scoring copy, RNE of unit_mean */
  int32_t *n_rows;     /* [batch] rows in use */
  int32_t *n_units;    /* [batch] units written (clusters + closed segments) */
  int32_t *n_cand;     /* [batch] selectable units: clusters + evicted segments */
  int32_t buf_cap;     /* local-buffer rows; 0 = no decode segments */
  int32_t *buf_begin;  /* [batch] first row of the local buffer */
  int32_t *seg_begin;  /* [batch] first row of the open segment */
  float *seg_sum;      /* [batch][n_kv_heads][head_dim] fp32 key sum of the open
                          segment; may be NULL when buf_cap == 0 */
  int32_t *status;     /* [1] device status word (kv_status of async errors) */
  /* Optional HBM copy of the local buffer, for a pool whose k and v live in
   * host memory (the note's "Key designs" item 2 keeps only a fixed-size local
   * buffer on the GPU): pool row r of the buffer is also stored at slot
   * r % buf_ring. Both NULL: the buffer rows are read from k and v. */
  void *buf_k;        /* [batch][n_kv_heads][buf_ring][head_dim] or NULL */
  void *buf_v;        /* same */
  int32_t buf_ring;   /* slots per (sequence, KV head); >= buf_cap when set */
} kv_pool;

/* Human-readable name of a status code (static string). */
const char *kv_status_string(kv_status s);

/* ------------------------------------------------------------------------
 * Prefill: K-means over each (sequence, KV head)'s keys, then the CSR pack.
 * LouisKV note, "Key designs" item 2: similar keys are grouped with K-means
 * and each cluster's centroid, the mean of its keys, is its retrieval index.
 *
 * Lloyd's algorithm, exactly `iters` rounds of
 *   assign: a(x) = argmin_k ||x - c_k||^2, with c_k rounded to the storage
 *           dtype (bf16 RNE of the fp32 master copy) and fp32 accumulation.
 *           For KV_BF16 the minimum is taken over the upper 28 bits of each
 *           fp32 score, so centroids whose scores agree in those bits (exact
 *           ties, and near-ties within about 2^-19 relative) go to the lowest
 *           k; for KV_F32 exact ties go to the lowest k;
 *   update: c_k = mean of its members in fp32; members are read in key order
 *           and dealt round-robin to a fixed number of partial sums, which are
 *           then combined in a fixed order, so the sum is the same bit for bit
 *           on every run (not the left-to-right sum in key order);
 *           an empty cluster keeps its previous centroid.
 * n_clusters <= 8192 (KV_ERR_UNSUPPORTED above).
 * Init: c_k = keys[init_idx[k]]. Then rows are packed cluster by cluster
 * (stable in key order) into pool->k / pool->v and the unit tables, and the
 * per-sequence counters are set (n_rows = n_keys, n_units = n_cand =
 * n_clusters, buf_begin = seg_begin = n_keys, seg_sum = 0).
 *
 * keys, values: [batch][n_kv_heads][n_keys][head_dim] in pool->dtype.
 * init_idx:     [batch][n_kv_heads][n_clusters] distinct indices in
 *               [0, n_keys) (distinctness is a precondition, not checked; an
 *               index outside [0, n_keys) is clamped into it and
 *               *pool->status is set to KV_ERR_INVALID_ARG).
 * assign_in:    NULL, or [BH][n_keys] labels in [0, n_clusters): skip Lloyd
 *               and pack this clustering (centroids = its member means;
 *               empty clusters take keys[init_idx[k]]). A key whose label is
 *               outside [0, n_clusters) is left out of every unit (its row is
 *               not packed) and *pool->status is set to KV_ERR_INVALID_ARG.
 * assign_out:   NULL, or [BH][n_keys]: the final labels.
 * rounds_out:   NULL, or [BH] int32: the rounds whose assignment ran for
 *               each head. A head whose assignment changes no label has
 *               reached a fixed point of the iteration (the update then
 *               reproduces its centroids bit for bit, and so on), so for
 *               KV_BF16 keys its later rounds are skipped: the labels,
 *               centroids and pool are those of exactly `iters` rounds. It
 *               is iters where no such round came before the last (always
 *               for KV_F32), 0 with assign_in.
 * sweeps_out:   NULL, or [BH] float: the assignment work each head took, in
 *               whole sweeps of n_keys x n_clusters distance evaluations. For
 *               KV_BF16 keys a round after the second scores only the
 *               centroids that moved in the last update (every one of them
 *               for the keys whose own centroid moved), which gives the
 *               labels of a whole sweep bit for bit at a fraction of its
 *               work; otherwise it equals rounds_out.
 * iters >= 1 unless assign_in is given. n_clusters <= n_keys,
 * n_keys <= pool->row_cap, n_clusters <= pool->unit_cap.
 */
size_t kv_cluster_build_workspace(int32_t batch, int32_t n_kv_heads, int32_t n_keys,
                                  int32_t head_dim, int32_t n_clusters, kv_dtype dtype);
kv_status kv_cluster_build(const kv_pool *pool, const void *keys, const void *values,
                           int32_t n_keys, int32_t n_clusters, int32_t iters,
                           const int32_t *init_idx, const int32_t *assign_in,
                           int32_t *assign_out, int32_t *rounds_out, float *sweeps_out,
                           void *ws, size_t ws_bytes, hipStream_t stream);

/* One Lloyd assignment step (the same kernel kv_cluster_build runs).
 * keys [n_heads][n_keys][head_dim] (dtype); centroids [n_heads][n_clusters]
 * [head_dim] fp32 master copies; labels out [n_heads][n_keys] int32.
 * For KV_BF16 the distance uses bf16(centroid) on the matrix cores. */
size_t kv_kmeans_assign_workspace(int32_t n_heads, int32_t n_clusters, int32_t head_dim,
                                  kv_dtype dtype);
kv_status kv_kmeans_assign(const void *keys, const float *centroids, int32_t n_heads,
                           int32_t n_keys, int32_t head_dim, int32_t n_clusters,
                           kv_dtype dtype, int32_t *labels, void *ws, size_t ws_bytes,
                           hipStream_t stream);

/* The assignment step split in two, for callers that assign several key
 * sets against one set of centroids (the centroids are converted once).
 * kv_kmeans_prepare writes the centroids' assignment form into ws (same size
 * as kv_kmeans_assign_workspace: for KV_BF16 the bf16 MFMA fragments and fp32
 * half norms, for KV_F32 the half norms). kv_kmeans_assign_prepared then
 * labels keys exactly as kv_kmeans_assign would with those centroids; it
 * reads ws without modifying it, so ws stays valid until the caller
 * overwrites it. centroids must be the array given to kv_kmeans_prepare (the
 * fp32 path reads it; the bf16 path reads only ws). Both calls validate like
 * kv_kmeans_assign. kv_kmeans_assign = kv_kmeans_prepare followed by
 * kv_kmeans_assign_prepared on the same stream. */
kv_status kv_kmeans_prepare(const float *centroids, int32_t n_heads, int32_t head_dim,
                            int32_t n_clusters, kv_dtype dtype, void *ws, size_t ws_bytes,
                            hipStream_t stream);
kv_status kv_kmeans_assign_prepared(const void *keys, const float *centroids, int32_t n_heads,
                                    int32_t n_keys, int32_t head_dim, int32_t n_clusters,
                                    kv_dtype dtype, int32_t *labels, const void *ws,
                                    size_t ws_bytes, hipStream_t stream);

/* One Lloyd update step: centroids_out[k] = mean of keys labelled k, or
 * centroids_in[k] when the cluster is empty (summation order as in
 * kv_cluster_build). counts (nullable) receives the member counts
 * [n_heads][n_clusters]. centroids_out may alias centroids_in. A key whose
 * label is outside [0, n_clusters) takes part in no cluster. */
size_t kv_kmeans_update_workspace(int32_t n_heads, int32_t n_keys, int32_t n_clusters);
kv_status kv_kmeans_update(const void *keys, const int32_t *labels, const float *centroids_in,
                           float *centroids_out, int32_t *counts, int32_t n_heads,
                           int32_t n_keys, int32_t head_dim, int32_t n_clusters,
                           kv_dtype dtype, void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Decode step 1: the semantic-boundary test. LouisKV note, "Key designs"
 * item 1 and the flowchart of "Overall framework":
 *   r = (1/H) * sum_h cos(q_prev^h, q_cur^h) over all n_q_heads heads,
 *   flag = (r < tau), strict. cos is 0 when either norm is 0.
 * q_prev NULL means the first decode step: flag = 1 and r = NaN.
 * q_prev, q_cur: [batch][n_q_heads][head_dim] (dtype). flag: [batch] uint8.
 * r: NULL or [batch] fp32.
 */
kv_status kv_boundary(const void *q_prev, const void *q_cur, int32_t batch, int32_t n_q_heads,
                      int32_t head_dim, kv_dtype dtype, float tau, uint8_t *flag, float *r,
                      hipStream_t stream);

/* ------------------------------------------------------------------------
 * Decode step 2 (long-output workloads, pool->buf_cap > 0): temporal
 * segments and the fixed-size local buffer. LouisKV note, "Key designs"
 * item 2 (decode half): generated KV is cut at the semantic boundaries into
 * segments indexed by their key mean; the most recent segments stay in a
 * fixed-size local buffer and the oldest moves to the pool when it is full.
 * Per sequence b, in this order:
 *   1. close the open segment when flag[b] and it is non-empty, or when it
 *      already holds buf_cap rows: it becomes unit n_units[b] with
 *      unit_mean = seg_sum / size and unit_index = dtype(unit_mean);
 *   2. append k_t, v_t as row n_rows[b] and add k_t to seg_sum (and, when
 *      the pool keeps an HBM copy of its buffer, also to slot
 *      n_rows[b] % buf_ring of buf_k / buf_v);
 *   3. while the buffer [buf_begin, n_rows) holds more than buf_cap rows,
 *      evict the oldest closed segment: n_cand[b]++ and buf_begin moves past
 *      it (no data moves; the pool and the buffer share the row store).
 * The buffer therefore never holds more than buf_cap rows after a step, so
 * buf_ring = buf_cap slots keep every buffered row.
 * k_t, v_t: [batch][n_kv_heads][head_dim] (dtype). flag: [batch] uint8 from
 * kv_boundary of the same step. Out of rows or units: *pool->status =
 * KV_ERR_CAPACITY and that sequence's step is skipped.
 */
kv_status kv_segment_append(const kv_pool *pool, const void *k_t, const void *v_t,
                            const uint8_t *flag, hipStream_t stream);

/* Decode steps 1 and 2 in one launch: exactly kv_boundary(q_prev, q_cur,
 * pool->batch, n_q_heads, pool->head_dim, pool->dtype, tau, flag, r)
 * followed by kv_segment_append(pool, k_t, v_t, flag), with the same results
 * bit for bit. The append workgroup of each sequence evaluates that
 * sequence's boundary test itself. flag: [batch] uint8 out (the selection of
 * the same step reads it); r: NULL or [batch] fp32 out. Validation as the
 * two calls (pool->buf_cap > 0 required). */
kv_status kv_boundary_segment_append(const kv_pool *pool, const void *q_prev, const void *q_cur,
                                     int32_t n_q_heads, float tau, const void *k_t,
                                     const void *v_t, uint8_t *flag, float *r,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * Decode step 3: group-consistent scoring and budgeted selection. LouisKV
 * note, flowchart (on a boundary, q_t is compared with every unit's centroid
 * and the Top-B units are fetched) and "Key designs" item 3 (one unit set per
 * GQA group; batched selection under a token budget over units of variable
 * size). For every (b, g) with flag[b] != 0 (or flag == NULL):
 *   s_u = sum over the group's query heads h of q[b][h] . unit_index[b][g][u]
 *         (fp32) for u < n_cand[b];
 *   rank non-empty units by (s_u descending, u ascending) and keep the
 *   longest prefix whose total unit_size is <= budget.
 * The selected ids are written ascending to sel_units[b][g][0..sel_n), with
 * sel_n[b][g] and sel_rows[b][g] (total rows). sel_spans (nullable):
 * [BH][sel_cap][2] int32 receives (unit_start[u], unit_size[u]) of each
 * selected unit at the same positions, the row ranges kv_gather_attend
 * needs. When flag[b] == 0 nothing of sequence b is touched, so the
 * previous selection is reused.
 * q: [batch][n_q_heads][head_dim] (dtype). sel_units: [BH][sel_cap] with
 * sel_cap >= min(budget, unit_cap). scores_out: NULL or [BH][unit_cap] fp32
 * (entries u >= n_cand[b] untouched). pool->unit_cap <= 8192
 * (KV_ERR_UNSUPPORTED above: each of the 512 threads of a (b, g)'s last
 * workgroup holds at most 16 candidates' sort keys in registers).
 */
size_t kv_select_workspace(const kv_pool *pool, int32_t n_q_heads);
kv_status kv_select(const kv_pool *pool, const void *q, int32_t n_q_heads, int32_t budget,
                    const uint8_t *flag, int32_t *sel_units, int32_t sel_cap, int32_t *sel_n,
                    int32_t *sel_rows, int32_t *sel_spans, float *scores_out, void *ws,
                    size_t ws_bytes, hipStream_t stream);

/* Decode steps 1 and 3 in one launch: exactly kv_boundary(q_prev, q_cur,
 * pool->batch, n_q_heads, pool->head_dim, pool->dtype, tau, flag, r)
 * followed by kv_select(pool, q_cur, n_q_heads, budget, flag, ...), with the
 * same results bit for bit (flag, r, selection, scores_out). Each select
 * workgroup evaluates the boundary test of its own sequence, so a step
 * without a boundary costs one memory round trip and no second launch.
 * Pools with a local buffer (buf_cap > 0) get KV_ERR_UNSUPPORTED: there
 * kv_segment_append of the step runs between the boundary test and the
 * selection, so the three calls stay separate. Workspace:
 * kv_select_workspace. flag: [batch] uint8 out; r: NULL or [batch] fp32 out. */
kv_status kv_boundary_select(const kv_pool *pool, const void *q_prev, const void *q_cur,
                             int32_t n_q_heads, float tau, int32_t budget, uint8_t *flag,
                             float *r, int32_t *sel_units, int32_t sel_cap, int32_t *sel_n,
                             int32_t *sel_rows, int32_t *sel_spans, float *scores_out, void *ws,
                             size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Decode step 4: gather the selected rows and attend. LouisKV note,
 * flowchart: the retrieved (or reused) critical KV feeds attention. For each
 * query head h of KV head g:
 *   out[b][h] = softmax(scale * K_S q[b][h]) V_S   (fp32; 0 if S is empty)
 * where S = rows of the units sel_units[b][g][0..sel_n[b][g]) followed, when
 * pool->buf_cap > 0, by the local-buffer rows [buf_begin[b], n_rows[b])
 * (read from the pool's HBM copy of the buffer when buf_k is set).
 * When sel_spans ([BH][sel_cap][2] int32, as written by kv_select) is given,
 * the units' row ranges are read from it instead of looking the ids up in
 * the unit table (one dependent memory round trip less; sel_units may then
 * be NULL). Row indices are clamped into [0, row_cap).
 * q: [batch][n_q_heads][head_dim] (dtype). out: [batch][n_q_heads][head_dim]
 * fp32. max_rows: expected upper bound on selected pool rows per (b, g) (the
 * budget); it sizes the launch and the workspace and, through the split of
 * the rows over workgroups, the order of the fp32 sums (for equal max_rows,
 * equal rows in equal order give bitwise equal outputs). sel_cap <= 4096.
 */
size_t kv_gather_attend_workspace(const kv_pool *pool, int32_t n_q_heads, int32_t max_rows);
kv_status kv_gather_attend(const kv_pool *pool, const void *q, int32_t n_q_heads, float scale,
                           const int32_t *sel_units, const int32_t *sel_spans, int32_t sel_cap,
                           const int32_t *sel_n, int32_t max_rows, float *out, void *ws,
                           size_t ws_bytes, hipStream_t stream);

/* kv_gather_attend for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same kernels and results, bit for bit, as
 * kv_gather_attend with the same arguments, but the completion counters and
 * split partials live in a static device array of the library (4 MiB, one
 * per device, held until the process ends) instead of a caller workspace.
 * It calls no allocating routine. The first call on a device looks the array up and
 * clears it with a kernel on `stream`; every completed call leaves its
 * counters zero again. All calls on one device share the array, so calls
 * that overlap in time on one device (different streams, or concurrent
 * graph replays) race and must not be issued. Arguments and validation as
 * kv_gather_attend; a call whose kv_gather_attend_workspace(pool, n_q_heads,
 * max_rows) exceeds 4 MiB (4194304 bytes) returns KV_ERR_WORKSPACE. */
kv_status kv_gather_attend_noalloc(const kv_pool *pool, const void *q, int32_t n_q_heads,
                                   float scale, const int32_t *sel_units,
                                   const int32_t *sel_spans, int32_t sel_cap,
                                   const int32_t *sel_n, int32_t max_rows, float *out,
                                   hipStream_t stream);

/* ------------------------------------------------------------------------
 * The GPU-side working set of a pool kept in host memory. LouisKV note,
 * flowchart: on a boundary the top units are fetched from the CPU pool to
 * the GPU, and the steps inside the segment reuse them; "Key designs" item 3:
 * the chosen rows of the CPU tensor are copied straight to the GPU, without
 * first gathering them on the CPU. Here the copy is a gather kernel that
 * reads the selected rows where the pool keeps them (mapped host memory, or
 * HBM) and writes them into `dst`, a second pool in HBM that holds one span
 * per (b, g).
 *
 * For every sequence b with flag[b] != 0 and every KV head g: the rows of
 * the selection (sel_units / sel_spans / sel_n exactly as kv_gather_attend
 * reads them) are written in selection order to dst->k / dst->v rows
 * [0, R) of (b, g), R = min(selected rows, dst->row_cap), and
 * dst_spans[b][g] = {0, R}, dst_n[b][g] = (R > 0). Sequences with flag 0 are
 * left untouched, so their previous working set is reused.
 * kv_gather_attend(dst, q, ..., sel_spans = dst_spans, sel_cap = 1,
 * sel_n = dst_n, max_rows) then attends over the same rows in the same order
 * as kv_gather_attend(pool, q, ..., the selection, max_rows), with bitwise
 * equal output. More selected rows than dst->row_cap sets *pool->status to
 * KV_ERR_CAPACITY and keeps the first dst->row_cap rows.
 * dst: same batch, n_kv_heads, head_dim and dtype as pool, buf_cap 0, its
 * own k and v (only k, v and row_cap are used). dst_spans: [BH][2] int32;
 * dst_n: [BH] int32. The local buffer of a pool with decode segments is not
 * part of a selection and is not copied (kv_fetch_attend reads it from the
 * pool's HBM copy of it). sel_cap <= 4096. No workspace. */
kv_status kv_fetch_selected(const kv_pool *pool, const uint8_t *flag, const int32_t *sel_units,
                            const int32_t *sel_spans, int32_t sel_cap, const int32_t *sel_n,
                            const kv_pool *dst, int32_t *dst_spans, int32_t *dst_n,
                            hipStream_t stream);

/* kv_fetch_selected followed by kv_gather_attend over the working set, in
 * one launch for bf16 pools: exactly
 *   kv_fetch_selected(pool, flag, sel_units, sel_spans, sel_cap, sel_n,
 *                     dst, dst_spans, dst_n);
 *   kv_gather_attend(dst, q, n_q_heads, scale, NULL, dst_spans, 1, dst_n,
 *                    max_rows, out, ws, ws_bytes);
 * with the same working set, spans, status and output bit for bit. On a
 * retrieval step (flag[b] != 0) each attention workgroup stores the rows it
 * attends, as it loads them from the pool, into the working set (from the
 * same registers, so each row is read once, also over the host link); with
 * a local buffer it copies them in a pass of its own first. On other steps
 * it reads the working set only, requesting its first rows together with
 * the flag and the span, so a step without retrieval costs one launch and
 * one memory round trip before the rows arrive. fp32 pools run the two
 * launches.
 * A pool with decode segments (buf_cap > 0; bf16, with buf_k / buf_v set)
 * is supported too: the attended rows are then the working set followed by
 * the local buffer, read from the pool's HBM copy, i.e. exactly the rows
 * and order of kv_gather_attend(pool, q, ..., the selection, max_rows),
 * with bitwise equal output; other pools with buf_cap > 0 get
 * KV_ERR_UNSUPPORTED. Arguments as for those two calls; workspace:
 * kv_gather_attend_workspace(pool, n_q_heads, max_rows). */
kv_status kv_fetch_attend(const kv_pool *pool, const void *q, int32_t n_q_heads, float scale,
                          const uint8_t *flag, const int32_t *sel_units, const int32_t *sel_spans,
                          int32_t sel_cap, const int32_t *sel_n, int32_t max_rows,
                          const kv_pool *dst, int32_t *dst_spans, int32_t *dst_n, float *out,
                          void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * A whole decode step of one layer in one launch. LouisKV note, flowchart
 * of "Overall framework": at every step the semantic-boundary test decides,
 * and only on a boundary are the units scored and the Top-B fetched; between
 * boundaries the KV fetched last time is reused for attention. Exactly
 *   kv_boundary_select(pool, q_prev, q_cur, n_q_heads, tau, budget, flag, r,
 *                      sel_units, sel_cap, sel_n, sel_rows, sel_spans, NULL);
 *   kv_fetch_attend(pool, q_cur, n_q_heads, scale, flag, NULL, sel_spans,
 *                   sel_cap, sel_n, max_rows = budget, dst, dst_spans, dst_n,
 *                   out);
 * with the same flag, r, selection, working set, status and output bit for
 * bit, but one launch: every attention workgroup evaluates the boundary test
 * of its sequence itself; on a step without retrieval it goes straight to
 * the working set; on a retrieval step the workgroups of (b, g) first score
 * the units (each its share), the last to finish selects and publishes the
 * selection (device-coherent stores, acknowledged before a generation
 * counter moves), the others wait for the counter (the selecting workgroup
 * is already running and waits for nothing, so the wait ends) and read it
 * with device-coherent loads, and all of them then fetch and attend as
 * kv_fetch_attend does. A wait that does not end after about 2^22 sleeps
 * would set *pool->status to KV_ERR_HIP. bf16 pools without a local buffer (buf_cap 0), in device or
 * host memory; unit_cap <= 8192; sel_cap >= min(budget, unit_cap), <= 4096.
 * sel_units and sel_spans are outputs ([BH][sel_cap] and [BH][sel_cap][2]
 * int32), written on retrieval steps only, like sel_n and sel_rows ([BH]).
 * flag: [batch] uint8 out; r: NULL or [batch] fp32 out. dst, dst_spans,
 * dst_n: the working set, as for kv_fetch_attend. ws:
 * kv_decode_step_workspace(pool, n_q_heads, budget) bytes, zero-filled once
 * before first use (its counters return to zero after every call); calls
 * sharing a workspace must not overlap. */
size_t kv_decode_step_workspace(const kv_pool *pool, int32_t n_q_heads, int32_t budget);
kv_status kv_decode_step(const kv_pool *pool, const void *q_prev, const void *q_cur,
                         int32_t n_q_heads, float tau, float scale, int32_t budget, uint8_t *flag,
                         float *r, int32_t *sel_units, int32_t *sel_spans, int32_t sel_cap,
                         int32_t *sel_n, int32_t *sel_rows, const kv_pool *dst,
                         int32_t *dst_spans, int32_t *dst_n, float *out, void *ws,
                         size_t ws_bytes, hipStream_t stream);

/* Device address of pinned host memory (hipHostMalloc, mapped), to place a
 * pool's k and v in host memory. *dev receives the address the kernels use.
 * KV_ERR_INVALID_ARG if `host` is not such memory. host, dev: [host]. */
kv_status kv_host_device_pointer(void *host, void **dev);

#ifdef __cplusplus
}
#endif
#endif /* KVC_H */

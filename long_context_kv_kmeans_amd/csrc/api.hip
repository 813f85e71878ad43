// C ABI of libkvc: argument validation on the host, workspace carving and
// kernel composition. Every entry point validates before touching HIP, so
// argument errors are reported without a device.
#include <mutex>

#include "kvc_internal.hpp"

using namespace kvc;

namespace {

bool dims_ok(int d) { return d == 64 || d == 128; }
bool dtype_ok(int dt) { return dt == KV_F32 || dt == KV_BF16; }
bool aligned256(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

kv_status check_pool(const kv_pool *p) {
  if (!p) return KV_ERR_INVALID_ARG;
  if (p->batch <= 0 || p->n_kv_heads <= 0 || p->row_cap <= 0 || p->unit_cap <= 0)
    return KV_ERR_INVALID_ARG;
  if (!dtype_ok(p->dtype) || !dims_ok(p->head_dim)) return KV_ERR_UNSUPPORTED;
  if (!p->k || !p->v || !p->unit_start || !p->unit_size || !p->unit_mean || !p->unit_index ||
      !p->n_rows || !p->n_units || !p->n_cand || !p->buf_begin || !p->seg_begin || !p->status)
    return KV_ERR_INVALID_ARG;
  if (p->buf_cap < 0) return KV_ERR_INVALID_ARG;
  if (p->buf_cap > 0 && !p->seg_sum) return KV_ERR_INVALID_ARG;
  if ((p->buf_k == nullptr) != (p->buf_v == nullptr)) return KV_ERR_INVALID_ARG;
  if (p->buf_k && (p->buf_cap <= 0 || p->buf_ring < p->buf_cap)) return KV_ERR_INVALID_ARG;
  return KV_OK;
}

size_t cluster_ws_layout(int bh, int n, int d, int c, kv_dtype dt, size_t *off_cent,
                         size_t *off_labels, size_t *off_assign, size_t *off_update,
                         size_t *off_skip = nullptr, size_t *off_inc = nullptr) {
  size_t o = 0;
  *off_cent = o;
  o += align_up((size_t)bh * c * d * sizeof(float), 256);
  *off_labels = o;
  o += align_up((size_t)bh * n * sizeof(int32_t), 256);
  *off_assign = o;
  o += assign_ws_bytes(bh, c, d, dt);
  *off_update = o;
  o += update_ws_bytes(bh, n, c);
  if (off_skip) *off_skip = o;  // fixed-point flags conv[bh], chg[bh]; work counters [bh] (u64)
  o += align_up((size_t)4 * bh * sizeof(int32_t), 256);
  if (off_inc) *off_inc = o;  // incremental assignment (bf16)
  if (dt == KV_BF16) o += assign_inc_ws_bytes(bh, n, c, d);
  return o;
}


}  // namespace

// ---------------------------------------------------------------- static scratch
// Device memory of kv_gather_attend_noalloc: the attention's completion
// counters and split partials live in this file-scope array instead of a
// caller workspace. Each device the library runs on holds its own copy until
// the process ends. Host code never passes the array's name to a kernel (on
// the host it is only a stand-in for the device symbol): the device address
// comes from hipGetSymbolAddress, once per device, and is kept in
// g_scratch_dev.
constexpr size_t kScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

__global__ void k_zero_words(uint32_t *p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// The current device's scratch address; on the first call on a device, looks
// it up and clears the whole array on `stream` (with a kernel, so that the
// clear can also be recorded into a graph).
kv_status scratch_for_current_device(void **out, hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return KV_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return KV_ERR_HIP;
    }
    k_zero_words<<<256, 256, 0, stream>>>(static_cast<uint32_t *>(ptr), kScratchBytes / 4);
    if (hipGetLastError() != hipSuccess) return KV_ERR_HIP;
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return KV_OK;
}
}  // namespace

extern "C" {

const char *kv_status_string(kv_status s) {
  switch (s) {
    case KV_OK: return "KV_OK";
    case KV_ERR_INVALID_ARG: return "KV_ERR_INVALID_ARG";
    case KV_ERR_UNSUPPORTED: return "KV_ERR_UNSUPPORTED";
    case KV_ERR_WORKSPACE: return "KV_ERR_WORKSPACE";
    case KV_ERR_CAPACITY: return "KV_ERR_CAPACITY";
    case KV_ERR_HIP: return "KV_ERR_HIP";
  }
  return "KV_ERR_UNKNOWN";
}

// ---------------------------------------------------------------- K-means steps
size_t kv_kmeans_assign_workspace(int32_t n_heads, int32_t n_clusters, int32_t head_dim,
                                  kv_dtype dtype) {
  if (n_heads <= 0 || n_clusters <= 0 || !dims_ok(head_dim) || !dtype_ok(dtype)) return 0;
  return assign_ws_bytes(n_heads, n_clusters, head_dim, dtype);
}

kv_status kv_kmeans_assign(const void *keys, const float *centroids, int32_t n_heads,
                           int32_t n_keys, int32_t head_dim, int32_t n_clusters, kv_dtype dtype,
                           int32_t *labels, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (!keys || !centroids || !labels) return KV_ERR_INVALID_ARG;
  if (n_heads <= 0 || n_keys <= 0 || n_clusters <= 0) return KV_ERR_INVALID_ARG;
  if (!dims_ok(head_dim) || !dtype_ok(dtype)) return KV_ERR_UNSUPPORTED;
  if (n_clusters > kMaxClusters) return KV_ERR_UNSUPPORTED;
  if (!ws || !aligned256(ws) || ws_bytes < assign_ws_bytes(n_heads, n_clusters, head_dim, dtype))
    return KV_ERR_WORKSPACE;
  return launch_assign(keys, centroids, n_heads, n_keys, head_dim, n_clusters, dtype, labels, ws,
                       stream);
}

kv_status kv_kmeans_prepare(const float *centroids, int32_t n_heads, int32_t head_dim,
                            int32_t n_clusters, kv_dtype dtype, void *ws, size_t ws_bytes,
                            hipStream_t stream) {
  if (!centroids) return KV_ERR_INVALID_ARG;
  if (n_heads <= 0 || n_clusters <= 0) return KV_ERR_INVALID_ARG;
  if (!dims_ok(head_dim) || !dtype_ok(dtype)) return KV_ERR_UNSUPPORTED;
  if (n_clusters > kMaxClusters) return KV_ERR_UNSUPPORTED;
  if (!ws || !aligned256(ws) || ws_bytes < assign_ws_bytes(n_heads, n_clusters, head_dim, dtype))
    return KV_ERR_WORKSPACE;
  return launch_assign_prepare(centroids, n_heads, head_dim, n_clusters, dtype, ws, stream);
}

kv_status kv_kmeans_assign_prepared(const void *keys, const float *centroids, int32_t n_heads,
                                    int32_t n_keys, int32_t head_dim, int32_t n_clusters,
                                    kv_dtype dtype, int32_t *labels, const void *ws,
                                    size_t ws_bytes, hipStream_t stream) {
  if (!keys || !centroids || !labels) return KV_ERR_INVALID_ARG;
  if (n_heads <= 0 || n_keys <= 0 || n_clusters <= 0) return KV_ERR_INVALID_ARG;
  if (!dims_ok(head_dim) || !dtype_ok(dtype)) return KV_ERR_UNSUPPORTED;
  if (n_clusters > kMaxClusters) return KV_ERR_UNSUPPORTED;
  if (!ws || !aligned256(ws) || ws_bytes < assign_ws_bytes(n_heads, n_clusters, head_dim, dtype))
    return KV_ERR_WORKSPACE;
  return launch_assign_prepared(keys, centroids, n_heads, n_keys, head_dim, n_clusters, dtype,
                                labels, ws, stream);
}

size_t kv_kmeans_update_workspace(int32_t n_heads, int32_t n_keys, int32_t n_clusters) {
  if (n_heads <= 0 || n_keys <= 0 || n_clusters <= 0) return 0;
  return update_ws_bytes(n_heads, n_keys, n_clusters);
}

kv_status kv_kmeans_update(const void *keys, const int32_t *labels, const float *centroids_in,
                           float *centroids_out, int32_t *counts, int32_t n_heads, int32_t n_keys,
                           int32_t head_dim, int32_t n_clusters, kv_dtype dtype, void *ws,
                           size_t ws_bytes, hipStream_t stream) {
  if (!keys || !labels || !centroids_in || !centroids_out) return KV_ERR_INVALID_ARG;
  if (n_heads <= 0 || n_keys <= 0 || n_clusters <= 0) return KV_ERR_INVALID_ARG;
  if (!dims_ok(head_dim) || !dtype_ok(dtype)) return KV_ERR_UNSUPPORTED;
  if (n_clusters > kMaxClusters) return KV_ERR_UNSUPPORTED;
  if (!ws || !aligned256(ws) || ws_bytes < update_ws_bytes(n_heads, n_keys, n_clusters))
    return KV_ERR_WORKSPACE;
  return launch_update(keys, labels, centroids_in, centroids_out, counts, n_heads, n_keys,
                       head_dim, n_clusters, dtype, ws, stream, nullptr, nullptr, nullptr);
}

// ---------------------------------------------------------------- cluster build
size_t kv_cluster_build_workspace(int32_t batch, int32_t n_kv_heads, int32_t n_keys,
                                  int32_t head_dim, int32_t n_clusters, kv_dtype dtype) {
  if (batch <= 0 || n_kv_heads <= 0 || n_keys <= 0 || n_clusters <= 0 || !dims_ok(head_dim) ||
      !dtype_ok(dtype))
    return 0;
  size_t a, b, c, d;
  return cluster_ws_layout(batch * n_kv_heads, n_keys, head_dim, n_clusters, dtype, &a, &b, &c,
                           &d);
}

kv_status kv_cluster_build(const kv_pool *pool, const void *keys, const void *values,
                           int32_t n_keys, int32_t n_clusters, int32_t iters,
                           const int32_t *init_idx, const int32_t *assign_in, int32_t *assign_out,
                           int32_t *rounds_out, float *sweeps_out, void *ws, size_t ws_bytes,
                           hipStream_t stream) {
  kv_status st = check_pool(pool);
  if (st != KV_OK) return st;
  if (!keys || !values || !init_idx) return KV_ERR_INVALID_ARG;
  if (n_keys <= 0 || n_clusters <= 0 || n_clusters > n_keys) return KV_ERR_INVALID_ARG;
  if (!assign_in && iters < 1) return KV_ERR_INVALID_ARG;
  if (n_clusters > kMaxClusters) return KV_ERR_UNSUPPORTED;
  if (n_keys > pool->row_cap || n_clusters > pool->unit_cap) return KV_ERR_CAPACITY;
  const int bh = pool->batch * pool->n_kv_heads, d = pool->head_dim;
  const kv_dtype dt = (kv_dtype)pool->dtype;
  size_t o_cent, o_lab, o_asg, o_upd, o_skip, o_inc;
  const size_t need = cluster_ws_layout(bh, n_keys, d, n_clusters, dt, &o_cent, &o_lab, &o_asg,
                                        &o_upd, &o_skip, &o_inc);
  if (!ws || !aligned256(ws) || ws_bytes < need) return KV_ERR_WORKSPACE;
  char *w = static_cast<char *>(ws);
  float *cent = reinterpret_cast<float *>(w + o_cent);
  int32_t *labels = assign_out ? assign_out : reinterpret_cast<int32_t *>(w + o_lab);
  void *asg_ws = w + o_asg;
  void *upd_ws = w + o_upd;
  // Heads that reach a fixed point of Lloyd's iteration (an assignment that
  // changes no label) skip the rest of their rounds: the later rounds would
  // give the same labels and centroids bit for bit (bf16 keys; the flags are
  // zeroed with the initial centroids).
  LloydSkip skip;
  AssignIncWs inc{};
  if (dt == KV_BF16 && !assign_in) {
    skip.conv = reinterpret_cast<int32_t *>(w + o_skip);
    skip.chg = skip.conv + bh;
    // Centroids that did not move score every key exactly as before, so
    // later rounds sweep only the moved ones (and every centroid for the keys
    // whose own centroid moved): the labels of a whole sweep, bit for bit.
    assign_inc_ws_carve(w + o_inc, bh, n_keys, n_clusters, d, &inc);
    inc.work = reinterpret_cast<unsigned long long *>(skip.conv + 2 * bh);
  }

  st = launch_init_centroids(keys, init_idx, cent, bh, n_keys, n_clusters, d, dt, pool->status,
                             stream, skip.conv, skip.conv ? 4 * bh : 0);
  if (st != KV_OK) return st;
  const int32_t *perm = nullptr, *start = nullptr, *tot = nullptr;
  if (assign_in) {
    st = launch_update(keys, assign_in, cent, cent, nullptr, bh, n_keys, d, n_clusters, dt, upd_ws,
                       stream, &perm, &start, &tot, nullptr, pool->status);
    if (st != KV_OK) return st;
    if (assign_out && assign_out != assign_in)
      if (hipMemcpyAsync(assign_out, assign_in, (size_t)bh * n_keys * 4, hipMemcpyDeviceToDevice,
                         stream) != hipSuccess)
        return KV_ERR_HIP;
  } else {
    // bf16: the first round's fragments come from the init centroids; later
    // rounds get theirs from the update kernel that produced the centroids.
    const bool fused = dt == KV_BF16;
    if (fused) {
      st = launch_prep_frags(cent, bh, d, n_clusters, asg_ws, stream);
      if (st != KV_OK) return st;
    }
    for (int it = 0; it < iters; ++it) {
      // from the second round on, compare with the previous round's labels
      LloydSkip round_skip = it > 0 ? skip : LloydSkip{};
      round_skip.round = it + 1;
      // from the second round on the assignment marks the clusters its label
      // changes touch; the member sums of the others stand (not in the last
      // round, whose update also lays out the pack)
      if (it > 0 && it + 1 < iters && skip.conv != nullptr) round_skip.touched = inc.flags[(it + 1) & 1];
      if (skip.conv != nullptr)
        st = launch_assign_round(keys, bh, n_keys, d, n_clusters, labels, asg_ws, inc, it + 1,
                                 round_skip, stream);
      else
        st = launch_assign(keys, cent, bh, n_keys, d, n_clusters, dt, labels, asg_ws, stream,
                           fused, round_skip);
      if (st != KV_OK) return st;
      void *next_frags = (fused && it + 1 < iters) ? asg_ws : nullptr;
      if (it + 1 < iters && update_local_ok(bh, n_keys, n_clusters))  // the pack reads the last only
        st = launch_update_local(keys, labels, cent, cent, bh, n_keys, d, n_clusters, dt, upd_ws,
                                 stream, next_frags, round_skip);
      else if (it + 1 < iters)
        st = launch_update(keys, labels, cent, cent, nullptr, bh, n_keys, d, n_clusters, dt,
                           upd_ws, stream, &perm, &start, &tot, next_frags, nullptr, round_skip);
      else  // the last round runs whole: the pack reads its order, starts and counts
        st = launch_update(keys, labels, cent, cent, nullptr, bh, n_keys, d, n_clusters, dt,
                           upd_ws, stream, &perm, &start, &tot, next_frags);
      if (st != KV_OK) return st;
    }
  }
  if (rounds_out || sweeps_out) {
    st = launch_rounds_out(skip.conv, skip.conv ? inc.work : nullptr, rounds_out, sweeps_out, bh,
                           assign_in ? 0 : iters, n_keys, n_clusters, stream);
    if (st != KV_OK) return st;
  }
  return launch_pack(pool, keys, values, cent, perm, start, tot, n_keys, n_clusters, stream);
}

// ---------------------------------------------------------------- decode
kv_status kv_boundary(const void *q_prev, const void *q_cur, int32_t batch, int32_t n_q_heads,
                      int32_t head_dim, kv_dtype dtype, float tau, uint8_t *flag, float *r,
                      hipStream_t stream) {
  if (!q_cur || !flag) return KV_ERR_INVALID_ARG;
  if (batch <= 0 || n_q_heads <= 0) return KV_ERR_INVALID_ARG;
  if (!dims_ok(head_dim) || !dtype_ok(dtype)) return KV_ERR_UNSUPPORTED;
  if (tau != tau) return KV_ERR_INVALID_ARG;
  return launch_boundary(q_prev, q_cur, batch, n_q_heads, head_dim, dtype, tau, flag, r, stream);
}

kv_status kv_segment_append(const kv_pool *pool, const void *k_t, const void *v_t,
                            const uint8_t *flag, hipStream_t stream) {
  kv_status st = check_pool(pool);
  if (st != KV_OK) return st;
  if (!k_t || !v_t || !flag) return KV_ERR_INVALID_ARG;
  if (pool->buf_cap <= 0) return KV_ERR_INVALID_ARG;
  return launch_segment_append(pool, k_t, v_t, flag, false, nullptr, nullptr, 0, 0.f, nullptr,
                               nullptr, stream);
}

kv_status kv_boundary_segment_append(const kv_pool *pool, const void *q_prev, const void *q_cur,
                                     int32_t n_q_heads, float tau, const void *k_t,
                                     const void *v_t, uint8_t *flag, float *r,
                                     hipStream_t stream) {
  kv_status st = check_pool(pool);
  if (st != KV_OK) return st;
  if (!q_cur || !k_t || !v_t || !flag) return KV_ERR_INVALID_ARG;
  if (n_q_heads <= 0 || tau != tau) return KV_ERR_INVALID_ARG;
  if (pool->buf_cap <= 0) return KV_ERR_INVALID_ARG;
  return launch_segment_append(pool, k_t, v_t, nullptr, true, q_prev, q_cur, n_q_heads, tau,
                               flag, r, stream);
}

size_t kv_select_workspace(const kv_pool *pool, int32_t n_q_heads) {
  if (check_pool(pool) != KV_OK || n_q_heads <= 0) return 0;
  const size_t bh = (size_t)pool->batch * pool->n_kv_heads;
  return align_up(bh * sizeof(int32_t), 256) + align_up(bh * pool->unit_cap * sizeof(float), 256);
}

namespace {
kv_status select_common(const kv_pool *pool, const void *q, int32_t n_q_heads, int32_t budget,
                        const uint8_t *flag, int32_t *sel_units, int32_t sel_cap, int32_t *sel_n,
                        int32_t *sel_rows, int32_t *sel_spans, float *scores_out, void *ws,
                        size_t ws_bytes, bool fused, const void *q_prev, float tau, uint8_t *flag_out,
                        float *r_out, hipStream_t stream) {
  kv_status st = check_pool(pool);
  if (st != KV_OK) return st;
  if (!q || !sel_units || !sel_n || !sel_rows) return KV_ERR_INVALID_ARG;
  if (n_q_heads <= 0 || n_q_heads % pool->n_kv_heads != 0 || budget < 0 || sel_cap <= 0)
    return KV_ERR_INVALID_ARG;
  if (fused && (!flag_out || tau != tau)) return KV_ERR_INVALID_ARG;
  const int G = n_q_heads / pool->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KV_ERR_UNSUPPORTED;
  if (sel_cap < (budget < pool->unit_cap ? budget : pool->unit_cap)) return KV_ERR_CAPACITY;
  if (pool->unit_cap > kSelectBlockThreads * kSelectMaxKeysPerThread) return KV_ERR_UNSUPPORTED;
  const size_t need = kv_select_workspace(pool, n_q_heads);
  if (!ws || !aligned256(ws) || ws_bytes < need) return KV_ERR_WORKSPACE;
  const size_t bh = (size_t)pool->batch * pool->n_kv_heads;
  int32_t *counters = static_cast<int32_t *>(ws);
  float *scores = scores_out ? scores_out
                             : reinterpret_cast<float *>(static_cast<char *>(ws) +
                                                         align_up(bh * sizeof(int32_t), 256));
  return launch_select(pool, q, n_q_heads, budget, flag, sel_units, sel_cap, sel_n, sel_rows,
                       sel_spans, scores, counters, fused, q_prev, tau, flag_out, r_out, stream);
}
}  // namespace

kv_status kv_select(const kv_pool *pool, const void *q, int32_t n_q_heads, int32_t budget,
                    const uint8_t *flag, int32_t *sel_units, int32_t sel_cap, int32_t *sel_n,
                    int32_t *sel_rows, int32_t *sel_spans, float *scores_out, void *ws,
                    size_t ws_bytes, hipStream_t stream) {
  return select_common(pool, q, n_q_heads, budget, flag, sel_units, sel_cap, sel_n, sel_rows,
                       sel_spans, scores_out, ws, ws_bytes, false, nullptr, 0.f, nullptr, nullptr,
                       stream);
}

kv_status kv_boundary_select(const kv_pool *pool, const void *q_prev, const void *q_cur,
                             int32_t n_q_heads, float tau, int32_t budget, uint8_t *flag,
                             float *r, int32_t *sel_units, int32_t sel_cap, int32_t *sel_n,
                             int32_t *sel_rows, int32_t *sel_spans, float *scores_out, void *ws,
                             size_t ws_bytes, hipStream_t stream) {
  if (pool && pool->buf_cap > 0) return KV_ERR_UNSUPPORTED;  // the segment append goes between
  return select_common(pool, q_cur, n_q_heads, budget, nullptr, sel_units, sel_cap, sel_n,
                       sel_rows, sel_spans, scores_out, ws, ws_bytes, true, q_prev, tau, flag, r,
                       stream);
}

size_t kv_gather_attend_workspace(const kv_pool *pool, int32_t n_q_heads, int32_t max_rows) {
  if (check_pool(pool) != KV_OK || n_q_heads <= 0 || n_q_heads % pool->n_kv_heads != 0 ||
      max_rows < 0)
    return 0;
  const size_t bh = (size_t)pool->batch * pool->n_kv_heads;
  const size_t G = (size_t)(n_q_heads / pool->n_kv_heads);
  const size_t ns = (size_t)attend_num_splits(pool, max_rows);
  return align_up(bh * sizeof(int32_t), 256) +
         align_up(bh * ns * G * (pool->head_dim + 2) * sizeof(float), 256);
}

kv_status kv_gather_attend(const kv_pool *pool, const void *q, int32_t n_q_heads, float scale,
                           const int32_t *sel_units, const int32_t *sel_spans, int32_t sel_cap,
                           const int32_t *sel_n, int32_t max_rows, float *out, void *ws,
                           size_t ws_bytes, hipStream_t stream) {
  kv_status st = check_pool(pool);
  if (st != KV_OK) return st;
  if (!q || (!sel_units && !sel_spans) || !sel_n || !out) return KV_ERR_INVALID_ARG;
  if (n_q_heads <= 0 || n_q_heads % pool->n_kv_heads != 0 || sel_cap <= 0 || max_rows < 0)
    return KV_ERR_INVALID_ARG;
  if (!(scale == scale)) return KV_ERR_INVALID_ARG;
  const int G = n_q_heads / pool->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KV_ERR_UNSUPPORTED;
  if (sel_cap > kMaxSel) return KV_ERR_UNSUPPORTED;
  const size_t need = kv_gather_attend_workspace(pool, n_q_heads, max_rows);
  if (!ws || !aligned256(ws) || ws_bytes < need) return KV_ERR_WORKSPACE;
  const size_t bh = (size_t)pool->batch * pool->n_kv_heads;
  int32_t *counters = static_cast<int32_t *>(ws);
  float *partials = reinterpret_cast<float *>(static_cast<char *>(ws) +
                                              align_up(bh * sizeof(int32_t), 256));
  return launch_gather_attend(pool, q, n_q_heads, scale, sel_units, sel_spans, sel_cap, sel_n,
                              attend_num_splits(pool, max_rows), attend_row_bound(pool, max_rows),
                              out, partials, counters, stream);
}

kv_status kv_gather_attend_noalloc(const kv_pool *pool, const void *q, int32_t n_q_heads,
                                   float scale, const int32_t *sel_units,
                                   const int32_t *sel_spans, int32_t sel_cap,
                                   const int32_t *sel_n, int32_t max_rows, float *out,
                                   hipStream_t stream) {
  kv_status st = check_pool(pool);
  if (st != KV_OK) return st;
  if (!q || (!sel_units && !sel_spans) || !sel_n || !out) return KV_ERR_INVALID_ARG;
  if (n_q_heads <= 0 || n_q_heads % pool->n_kv_heads != 0 || sel_cap <= 0 || max_rows < 0)
    return KV_ERR_INVALID_ARG;
  if (!(scale == scale)) return KV_ERR_INVALID_ARG;
  const int G = n_q_heads / pool->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KV_ERR_UNSUPPORTED;
  if (sel_cap > kMaxSel) return KV_ERR_UNSUPPORTED;
  const size_t need = kv_gather_attend_workspace(pool, n_q_heads, max_rows);
  if (need == 0 || need > kScratchBytes) return KV_ERR_WORKSPACE;
  void *ws = nullptr;
  st = scratch_for_current_device(&ws, stream);
  if (st != KV_OK) return st;
  const size_t bh = (size_t)pool->batch * pool->n_kv_heads;
  int32_t *counters = static_cast<int32_t *>(ws);
  float *partials = reinterpret_cast<float *>(static_cast<char *>(ws) +
                                              align_up(bh * sizeof(int32_t), 256));
  return launch_gather_attend(pool, q, n_q_heads, scale, sel_units, sel_spans, sel_cap, sel_n,
                              attend_num_splits(pool, max_rows), attend_row_bound(pool, max_rows),
                              out, partials, counters, stream);
}

// ---------------------------------------------------------------- working set
kv_status kv_fetch_selected(const kv_pool *pool, const uint8_t *flag, const int32_t *sel_units,
                            const int32_t *sel_spans, int32_t sel_cap, const int32_t *sel_n,
                            const kv_pool *dst, int32_t *dst_spans, int32_t *dst_n,
                            hipStream_t stream) {
  kv_status st = check_pool(pool);
  if (st != KV_OK) return st;
  st = check_pool(dst);
  if (st != KV_OK) return st;
  if (!flag || (!sel_units && !sel_spans) || !sel_n || !dst_spans || !dst_n)
    return KV_ERR_INVALID_ARG;
  if (sel_cap <= 0) return KV_ERR_INVALID_ARG;
  if (sel_cap > kMaxSel) return KV_ERR_UNSUPPORTED;
  if (dst->batch != pool->batch || dst->n_kv_heads != pool->n_kv_heads ||
      dst->head_dim != pool->head_dim || dst->dtype != pool->dtype)
    return KV_ERR_INVALID_ARG;
  if (dst->k == pool->k || dst->v == pool->v) return KV_ERR_INVALID_ARG;
  if (dst->buf_cap > 0) return KV_ERR_UNSUPPORTED;  // a working set has no local buffer
  return launch_fetch_rows(pool, flag, sel_units, sel_spans, sel_cap, sel_n, dst, dst_spans,
                           dst_n, stream);
}

kv_status kv_fetch_attend(const kv_pool *pool, const void *q, int32_t n_q_heads, float scale,
                          const uint8_t *flag, const int32_t *sel_units, const int32_t *sel_spans,
                          int32_t sel_cap, const int32_t *sel_n, int32_t max_rows,
                          const kv_pool *dst, int32_t *dst_spans, int32_t *dst_n, float *out,
                          void *ws, size_t ws_bytes, hipStream_t stream) {
  kv_status st = check_pool(pool);
  if (st != KV_OK) return st;
  st = check_pool(dst);
  if (st != KV_OK) return st;
  if (!q || !flag || (!sel_units && !sel_spans) || !sel_n || !dst_spans || !dst_n || !out)
    return KV_ERR_INVALID_ARG;
  if (n_q_heads <= 0 || n_q_heads % pool->n_kv_heads != 0 || sel_cap <= 0 || max_rows < 0)
    return KV_ERR_INVALID_ARG;
  if (!(scale == scale)) return KV_ERR_INVALID_ARG;
  if (dst->batch != pool->batch || dst->n_kv_heads != pool->n_kv_heads ||
      dst->head_dim != pool->head_dim || dst->dtype != pool->dtype)
    return KV_ERR_INVALID_ARG;
  if (dst->k == pool->k || dst->v == pool->v) return KV_ERR_INVALID_ARG;
  if (dst->buf_cap > 0) return KV_ERR_UNSUPPORTED;  // a working set has no local buffer
  // a local buffer is attended from the pool's HBM copy of it (bf16 kernel only)
  if (pool->buf_cap > 0 && (!pool->buf_k || pool->dtype != KV_BF16)) return KV_ERR_UNSUPPORTED;
  const int G = n_q_heads / pool->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KV_ERR_UNSUPPORTED;
  if (sel_cap > kMaxSel) return KV_ERR_UNSUPPORTED;
  const size_t need = kv_gather_attend_workspace(pool, n_q_heads, max_rows);
  if (!ws || !aligned256(ws) || ws_bytes < need) return KV_ERR_WORKSPACE;
  const size_t bh = (size_t)pool->batch * pool->n_kv_heads;
  int32_t *counters = static_cast<int32_t *>(ws);
  float *partials = reinterpret_cast<float *>(static_cast<char *>(ws) +
                                              align_up(bh * sizeof(int32_t), 256));
  return launch_fetch_attend(pool, q, n_q_heads, scale, flag, sel_units, sel_spans, sel_cap,
                             sel_n, attend_num_splits(pool, max_rows),
                             attend_row_bound(pool, max_rows), dst, dst_spans, dst_n, out,
                             partials, counters, stream);
}

// ---------------------------------------------------------------- one launch per step
namespace {
struct StepWs {
  size_t counters, partials, sel_counters, gen, scores, total;
};
StepWs step_ws_layout(const kv_pool *pool, int32_t n_q_heads, int32_t budget) {
  const size_t bh = (size_t)pool->batch * pool->n_kv_heads;
  const size_t G = (size_t)(n_q_heads / pool->n_kv_heads);
  const size_t ns = (size_t)attend_num_splits(pool, budget);
  StepWs w;
  size_t o = 0;
  w.counters = o;
  o += align_up(bh * sizeof(int32_t), 256);
  w.partials = o;
  o += align_up(bh * ns * G * (pool->head_dim + 2) * sizeof(float), 256);
  w.sel_counters = o;
  o += align_up(bh * sizeof(int32_t), 256);
  w.gen = o;
  o += align_up(bh * sizeof(int32_t), 256);
  w.scores = o;
  o += align_up(bh * pool->unit_cap * sizeof(float), 256);
  w.total = o;
  return w;
}
}  // namespace

size_t kv_decode_step_workspace(const kv_pool *pool, int32_t n_q_heads, int32_t budget) {
  if (check_pool(pool) != KV_OK || n_q_heads <= 0 || n_q_heads % pool->n_kv_heads != 0 ||
      budget < 0)
    return 0;
  return step_ws_layout(pool, n_q_heads, budget).total;
}

kv_status kv_decode_step(const kv_pool *pool, const void *q_prev, const void *q_cur,
                         int32_t n_q_heads, float tau, float scale, int32_t budget, uint8_t *flag,
                         float *r, int32_t *sel_units, int32_t *sel_spans, int32_t sel_cap,
                         int32_t *sel_n, int32_t *sel_rows, const kv_pool *dst,
                         int32_t *dst_spans, int32_t *dst_n, float *out, void *ws,
                         size_t ws_bytes, hipStream_t stream) {
  kv_status st = check_pool(pool);
  if (st != KV_OK) return st;
  st = check_pool(dst);
  if (st != KV_OK) return st;
  if (!q_cur || !flag || !sel_units || !sel_spans || !sel_n || !sel_rows || !dst_spans ||
      !dst_n || !out)
    return KV_ERR_INVALID_ARG;
  if (n_q_heads <= 0 || n_q_heads % pool->n_kv_heads != 0 || budget < 0 || sel_cap <= 0)
    return KV_ERR_INVALID_ARG;
  if (tau != tau || !(scale == scale)) return KV_ERR_INVALID_ARG;
  if (pool->dtype != KV_BF16 || pool->buf_cap > 0) return KV_ERR_UNSUPPORTED;
  const int G = n_q_heads / pool->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return KV_ERR_UNSUPPORTED;
  if (pool->unit_cap > kSelectBlockThreads * kSelectMaxKeysPerThread) return KV_ERR_UNSUPPORTED;
  if (sel_cap > kMaxSel) return KV_ERR_UNSUPPORTED;
  if (sel_cap < (budget < pool->unit_cap ? budget : pool->unit_cap)) return KV_ERR_CAPACITY;
  if (dst->batch != pool->batch || dst->n_kv_heads != pool->n_kv_heads ||
      dst->head_dim != pool->head_dim || dst->dtype != pool->dtype)
    return KV_ERR_INVALID_ARG;
  if (dst->k == pool->k || dst->v == pool->v) return KV_ERR_INVALID_ARG;
  if (dst->buf_cap > 0) return KV_ERR_UNSUPPORTED;  // a working set has no local buffer
  const StepWs w = step_ws_layout(pool, n_q_heads, budget);
  if (!ws || !aligned256(ws) || ws_bytes < w.total) return KV_ERR_WORKSPACE;
  char *c = static_cast<char *>(ws);
  return launch_decode_step(
      pool, q_prev, q_cur, n_q_heads, tau, scale, budget, flag, r, sel_units, sel_spans, sel_cap,
      sel_n, sel_rows, attend_num_splits(pool, budget), attend_row_bound(pool, budget), dst,
      dst_spans, dst_n, out, reinterpret_cast<float *>(c + w.partials),
      reinterpret_cast<int32_t *>(c + w.counters), reinterpret_cast<float *>(c + w.scores),
      reinterpret_cast<int32_t *>(c + w.sel_counters), reinterpret_cast<int32_t *>(c + w.gen),
      stream);
}

kv_status kv_host_device_pointer(void *host, void **dev) {
  if (!host || !dev) return KV_ERR_INVALID_ARG;
  void *d = nullptr;
  if (hipHostGetDevicePointer(&d, host, 0) != hipSuccess || !d) {
    (void)hipGetLastError();
    return KV_ERR_INVALID_ARG;
  }
  *dev = d;
  return KV_OK;
}

}  // extern "C"

// Decode-step kernels for centroid-indexed KV retrieval, gfx950.
//
//  k_boundary        -- r = mean over query heads of cos(q_prev, q_cur); flag = r < tau
//                       (LouisKV note, "Key designs" item 1).
//  k_segment_append  -- temporal segments + fixed-size local buffer
//                       (LouisKV note, "Key designs" item 2, decode half).
//  k_select          -- group-summed q . index for every pool unit, then the
//                       longest (score desc, id asc) prefix within the token
//                       budget (flowchart Top-B; "Key designs" item 3).
//  k_gather_attend   -- softmax attention of the group's query heads over the
//                       selected rows (+ local buffer), split over workgroups
//                       with an online softmax and a deterministic merge.
//
// Multi-block kernels finish with a "last block" step: each block publishes
// its results, fences at agent scope and bumps a per-(sequence, head)
// counter; the block that brings the counter to the grid size does the final
// reduction in a fixed order and resets the counter to zero.
#include "kvc_internal.hpp"

namespace kvc {

// Completion protocol for the last-block steps. After the block barrier all
// of the block's stores sit in this XCD's L2; one release fence by thread 0
// makes them visible device-wide before the counter moves, and only the
// block that completes the count pays for an acquire (L2/L1 invalidate)
// before reading the other blocks' results. Returns true in that block.
__device__ __forceinline__ bool last_block_arrives(int32_t *counter, int nblocks, int *s_last) {
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_last = (old == nblocks - 1);
    if (*s_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  return *s_last != 0;
}

// ---------------------------------------------------------------- boundary
// One workgroup per sequence; each wave owns up to 8 query heads and issues
// all of their loads before reducing, so the step costs one memory round trip.
// Summation order is fixed (heads in order within a wave, then waves in
// order), so r is reproducible bit for bit.
constexpr int kBoundaryHeadsPerWave = 8;

template <typename T, int D>
__global__ void __launch_bounds__(256) k_boundary(const T *__restrict__ q_prev,
                                                  const T *__restrict__ q_cur, int hq, float tau,
                                                  uint8_t *__restrict__ flag, float *__restrict__ r) {
  constexpr int EPL = D / 64;
  constexpr int HPW = kBoundaryHeadsPerWave;
  __shared__ float part[4];
  const int b = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (q_prev == nullptr) {
    if (threadIdx.x == 0) {
      flag[b] = 1;
      if (r) r[b] = __builtin_nanf("");
    }
    return;
  }
  float csum = 0.f;
  for (int h0 = wave * HPW; h0 < hq; h0 += 4 * HPW) {
    T a[HPW][EPL], c[HPW][EPL];
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
      const int h = h0 + i;
      const size_t o = ((size_t)b * hq + (h < hq ? h : 0)) * D + lane * EPL;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        a[i][e] = q_prev[o + e];
        c[i][e] = q_cur[o + e];
      }
    }
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
      float dot = 0.f, n1 = 0.f, n2 = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float x = Elem<T>::to_f32(a[i][e]), y = Elem<T>::to_f32(c[i][e]);
        dot = fmaf(x, y, dot);
        n1 = fmaf(x, x, n1);
        n2 = fmaf(y, y, n2);
      }
      dot = wave_sum(dot);
      n1 = wave_sum(n1);
      n2 = wave_sum(n2);
      const float cosv = (n1 > 0.f && n2 > 0.f) ? dot / (sqrtf(n1) * sqrtf(n2)) : 0.f;
      if (h0 + i < hq) csum += cosv;
    }
  }
  if (lane == 0) part[wave] = csum;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float rv = (((part[0] + part[1]) + part[2]) + part[3]) / (float)hq;
    flag[b] = rv < tau ? 1 : 0;
    if (r) r[b] = rv;
  }
}

kv_status launch_boundary(const void *q_prev, const void *q_cur, int batch, int hq, int d,
                          kv_dtype dt, float tau, uint8_t *flag, float *r, hipStream_t s) {
  if (dt == KV_BF16) {
    if (d == 128)
      k_boundary<uint16_t, 128><<<batch, 256, 0, s>>>((const uint16_t *)q_prev,
                                                      (const uint16_t *)q_cur, hq, tau, flag, r);
    else
      k_boundary<uint16_t, 64><<<batch, 256, 0, s>>>((const uint16_t *)q_prev,
                                                     (const uint16_t *)q_cur, hq, tau, flag, r);
  } else {
    if (d == 128)
      k_boundary<float, 128><<<batch, 256, 0, s>>>((const float *)q_prev, (const float *)q_cur,
                                                   hq, tau, flag, r);
    else
      k_boundary<float, 64><<<batch, 256, 0, s>>>((const float *)q_prev, (const float *)q_cur, hq,
                                                  tau, flag, r);
  }
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

// ---------------------------------------------------------------- segments
// One workgroup per sequence. Thread 0 does the scalar bookkeeping; all
// threads move the (head, element) data. Segment boundaries are shared by
// the sequence's KV heads, so head 0's unit table is read for evictions.
template <typename T>
__global__ void __launch_bounds__(256) k_segment_append(kv_pool pool, const T *__restrict__ k_t,
                                                        const T *__restrict__ v_t,
                                                        const uint8_t *__restrict__ flag) {
  __shared__ int s_close, s_ok, s_open_len, s_seg_begin, s_n_rows, s_n_units;
  const int b = blockIdx.x;
  const int H = pool.n_kv_heads, D = pool.head_dim;
  if (threadIdx.x == 0) {
    const int n_rows = pool.n_rows[b], seg_begin = pool.seg_begin[b], n_units = pool.n_units[b];
    const int open_len = n_rows - seg_begin;
    const int close = ((flag[b] != 0) && open_len > 0) || open_len >= pool.buf_cap;
    int ok = n_rows < pool.row_cap && (!close || n_units < pool.unit_cap);
    if (!ok) __hip_atomic_store(pool.status, (int)KV_ERR_CAPACITY, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
    s_close = close;
    s_ok = ok;
    s_open_len = open_len;
    s_seg_begin = seg_begin;
    s_n_rows = n_rows;
    s_n_units = n_units;
  }
  __syncthreads();
  if (!s_ok) return;
  const int close = s_close, open_len = s_open_len, n_rows = s_n_rows, n_units = s_n_units;
  const size_t HD = (size_t)H * D;
  for (int i = threadIdx.x; i < H * D; i += blockDim.x) {
    const int g = i / D, e = i % D;
    const size_t bg = (size_t)b * H + g;
    float sum = pool.seg_sum[b * HD + i];
    if (close) {
      const float mean = sum / (float)open_len;
      const size_t uo = (bg * pool.unit_cap + n_units) * D + e;
      pool.unit_mean[uo] = mean;
      static_cast<T *>(pool.unit_index)[uo] = Elem<T>::from_f32(mean);
      if (e == 0) {
        pool.unit_start[bg * pool.unit_cap + n_units] = s_seg_begin;
        pool.unit_size[bg * pool.unit_cap + n_units] = open_len;
      }
      sum = 0.f;
    }
    const T kv = k_t[b * HD + i];
    const size_t ro = (bg * pool.row_cap + n_rows) * D + e;
    static_cast<T *>(pool.k)[ro] = kv;
    static_cast<T *>(pool.v)[ro] = v_t[b * HD + i];
    pool.seg_sum[b * HD + i] = sum + Elem<T>::to_f32(kv);
  }
  if (threadIdx.x == 0) {
    const int new_rows = n_rows + 1;
    const int new_units = n_units + close;
    int seg_begin = close ? n_rows : s_seg_begin;
    int buf_begin = pool.buf_begin[b];
    int n_cand = pool.n_cand[b];
    const int32_t *us = pool.unit_start + (size_t)b * H * pool.unit_cap;
    const int32_t *uz = pool.unit_size + (size_t)b * H * pool.unit_cap;
    while (new_rows - buf_begin > pool.buf_cap && n_cand < new_units) {
      // the segment closed in this step is still in registers
      const int st = (n_cand == n_units) ? s_seg_begin : us[n_cand];
      const int sz = (n_cand == n_units) ? open_len : uz[n_cand];
      buf_begin = st + sz;
      ++n_cand;
    }
    pool.n_rows[b] = new_rows;
    pool.n_units[b] = new_units;
    pool.n_cand[b] = n_cand;
    pool.buf_begin[b] = buf_begin;
    pool.seg_begin[b] = seg_begin;
  }
}

kv_status launch_segment_append(const kv_pool *pool, const void *k_t, const void *v_t,
                                const uint8_t *flag, hipStream_t s) {
  if (pool->dtype == KV_BF16)
    k_segment_append<uint16_t><<<pool->batch, 256, 0, s>>>(*pool, (const uint16_t *)k_t,
                                                           (const uint16_t *)v_t, flag);
  else
    k_segment_append<float><<<pool->batch, 256, 0, s>>>(*pool, (const float *)k_t,
                                                        (const float *)v_t, flag);
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

// ---------------------------------------------------------------- select
// Scoring: 1024-thread workgroups each score up to 1024 units; a unit's index
// vector is read as 16-byte pieces, so one wave instruction covers 64 / LPU
// units. Selection: the last workgroup of (b, g) holds every candidate as a
// 64-bit key (orderable score << 32 | ~id) in registers, KPT consecutive
// units per thread, and finds the first unit that no longer fits the budget
// with an MSB-first weighted radix select (per-wave LDS histograms, one
// digit of 8 bits per pass, early exit once the crossing bucket holds a
// single unit). Every unit ranked before it is selected.
constexpr int kSelectThreads = 1024;
constexpr int kSelectWaves = kSelectThreads / 64;
constexpr int kScoreUnitsPerBlock = kSelectThreads;

// Wave 0 helper: given per-digit weights w[0..255] (LDS), the weight already
// above the range and the budget, find the highest digit whose inclusion
// makes the running total (taken from the top digit down) exceed the budget.
// Returns -1 if even all digits fit. *above_out = weight of digits above it.
__device__ int find_crossing_digit(const int *w, long above, long budget, long *above_out) {
  const int lane = threadIdx.x & 63;
  // lane l owns digits 255 - 4l .. 252 - 4l (descending)
  long local = 0;
  int dg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dg[i] = w[255 - 4 * lane - i];
    local += dg[i];
  }
  long incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  const long excl = incl - local;
  int found = -1;
  long found_above = 0;
  long run = above + excl;
  if (run <= budget && above + incl > budget) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (found < 0 && run + dg[i] > budget) {
        found = 255 - 4 * lane - i;
        found_above = run;
      }
      run += dg[i];
    }
  }
  const uint64_t who = __ballot(found >= 0);
  if (who == 0) return -1;
  const int src = __ffsll((unsigned long long)who) - 1;
  *above_out = __shfl(found_above, src);
  return __shfl(found, src);
}

__device__ __forceinline__ unsigned long long unit_key(float score, int u) {
  return ((unsigned long long)float_order_key(score) << 32) | (uint32_t)(0xffffffffu - (uint32_t)u);
}

template <typename T, int D, int KPT>
__global__ void __launch_bounds__(kSelectThreads)
    k_select(kv_pool pool, const T *__restrict__ q, int hq, int group, int budget,
             const uint8_t *__restrict__ flag, int32_t *__restrict__ sel_units, int sel_cap,
             int32_t *__restrict__ sel_n, int32_t *__restrict__ sel_rows, float *__restrict__ scores,
             int32_t *counters) {
  constexpr int EPL = 16 / Elem<T>::kBytes;  // elements per 16-byte lane load
  constexpr int LPU = D / EPL;               // lanes per index vector
  constexpr int UPW = 64 / LPU;              // units per wave instruction
  constexpr int UNR = 4;
  const int H = pool.n_kv_heads;
  const int bg = blockIdx.y, b = bg / H, g = bg % H;
  if (flag != nullptr && flag[b] == 0) return;
  const int U = min(max(pool.n_cand[b], 0), pool.unit_cap);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int part = lane % LPU, slot = lane / LPU;

  // ---- scoring: s_u = (sum_h q_h) . idx_u, fp32
  float qs[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qs[e] = 0.f;
  for (int h = 0; h < group; ++h) {
    const uint4 v =
        *reinterpret_cast<const uint4 *>(q + ((size_t)b * hq + g * group + h) * D + part * EPL);
    float f[EPL];
    unpack16<T>(v, f);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qs[e] += f[e];
  }
  const T *idx = static_cast<const T *>(pool.unit_index) + (size_t)bg * pool.unit_cap * D;
  float *sc = scores + (size_t)bg * pool.unit_cap;
  const int wbase = blockIdx.x * kScoreUnitsPerBlock + wave * 64;
#pragma unroll
  for (int j0 = 0; j0 < 64; j0 += UPW * UNR) {
    uint4 v[UNR];
#pragma unroll
    for (int i = 0; i < UNR; ++i) {
      const int u = wbase + j0 + i * UPW + slot;
      v[i] = u < U ? *reinterpret_cast<const uint4 *>(idx + (size_t)u * D + part * EPL)
                   : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < UNR; ++i) {
      float f[EPL];
      unpack16<T>(v[i], f);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dot = fmaf(qs[e], f[e], dot);
#pragma unroll
      for (int o = LPU / 2; o >= 1; o >>= 1) dot += __shfl_xor(dot, o);
      const int u = wbase + j0 + i * UPW + slot;
      if (part == 0 && u < U) sc[u] = dot;
    }
  }

  // ---- completion: the last block of (b, g) selects
  __shared__ int s_last;
  if (!last_block_arrives(&counters[bg], (int)gridDim.x, &s_last)) return;

  const int32_t *usz = pool.unit_size + (size_t)bg * pool.unit_cap;
  unsigned long long key[KPT];
  int sz[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int u = tid * KPT + j;
    const int s = u < U ? usz[u] : 0;
    sz[j] = s > 0 ? s : 0;
    key[j] = (u < U && s > 0) ? unit_key(sc[u], u) : 0ull;
  }

  __shared__ int hw[kSelectWaves][256];
  __shared__ int hc[kSelectWaves][256];
  __shared__ int tw[256];
  __shared__ int tc[256];
  __shared__ int hu[256];
  __shared__ long s_above;
  __shared__ int s_done, s_none;
  __shared__ unsigned long long s_prefix, s_kstar;
  if (tid == 0) {
    s_above = 0;
    s_prefix = 0ull;
    s_done = 0;
    s_none = 0;
  }
  for (int sh = 56; sh >= 0; sh -= 8) {
    for (int i = tid; i < kSelectWaves * 256; i += kSelectThreads) {
      (&hw[0][0])[i] = 0;
      (&hc[0][0])[i] = 0;
    }
    __syncthreads();
    const unsigned long long prefix = s_prefix;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (sz[j] == 0) continue;
      if (sh < 56 && (key[j] >> (sh + 8)) != (prefix >> (sh + 8))) continue;
      const int dgt = (int)((key[j] >> sh) & 255ull);
      atomicAdd(&hw[wave][dgt], sz[j]);
      atomicAdd(&hc[wave][dgt], 1);
      hu[dgt] = tid * KPT + j;  // any member; read only when the bucket holds one unit
    }
    __syncthreads();
    if (tid < 256) {
      int w = 0, c = 0;
#pragma unroll
      for (int v = 0; v < kSelectWaves; ++v) {
        w += hw[v][tid];
        c += hc[v][tid];
      }
      tw[tid] = w;
      tc[tid] = c;
    }
    __syncthreads();
    if (wave == 0) {
      long above_out = 0;
      const int dgt = find_crossing_digit(tw, s_above, budget, &above_out);
      if (lane == 0) {
        if (dgt < 0) {
          s_none = 1;  // everything in range fits (only possible at the top level)
          s_done = 1;
        } else {
          s_above = above_out;
          s_prefix = prefix | ((unsigned long long)dgt << sh);
          if (tc[dgt] == 1) {
            const int u = hu[dgt];
            s_kstar = unit_key(sc[u], u);
            s_done = 1;
          } else if (sh == 0) {
            s_kstar = s_prefix;
            s_done = 1;
          }
        }
      }
    }
    __syncthreads();
    if (s_done) break;
  }
  const bool take_all = s_none != 0;
  const unsigned long long kstar = s_kstar;

  // ---- compaction in ascending unit id (thread t owns units t*KPT .. t*KPT+KPT-1)
  int cnt = 0, rows = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (sz[j] > 0 && (take_all || key[j] > kstar)) {
      ++cnt;
      rows += sz[j];
    }
  __shared__ int wsum[kSelectWaves], wrows[kSelectWaves];
  int incl = cnt, rincl = rows;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o), z = __shfl_up(rincl, o);
    if (lane >= o) {
      incl += y;
      rincl += z;
    }
  }
  if (lane == 63) {
    wsum[wave] = incl;
    wrows[wave] = rincl;
  }
  __syncthreads();
  int off = 0, total = 0, total_rows = 0;
  for (int w = 0; w < kSelectWaves; ++w) {
    if (w < wave) off += wsum[w];
    total += wsum[w];
    total_rows += wrows[w];
  }
  int pos = off + incl - cnt;
  int32_t *out = sel_units + (size_t)bg * sel_cap;
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if (sz[j] > 0 && (take_all || key[j] > kstar)) {
      if (pos < sel_cap) out[pos] = tid * KPT + j;
      ++pos;
    }
  if (tid == 0) {
    if (total > sel_cap) {
      __hip_atomic_store(pool.status, (int)KV_ERR_CAPACITY, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      total = sel_cap;
    }
    sel_n[bg] = total;
    sel_rows[bg] = total_rows;
    __hip_atomic_store(&counters[bg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

int select_num_blocks(const kv_pool *pool) {
  const int nb = (pool->unit_cap + kScoreUnitsPerBlock - 1) / kScoreUnitsPerBlock;
  return nb < 1 ? 1 : nb;
}

template <typename T, int D>
static kv_status select_dispatch(const kv_pool *pool, const void *q, int hq, int budget,
                                 const uint8_t *flag, int32_t *sel_units, int sel_cap,
                                 int32_t *sel_n, int32_t *sel_rows, float *scores,
                                 int32_t *counters, hipStream_t s) {
  const int G = hq / pool->n_kv_heads;
  const dim3 grid(select_num_blocks(pool), pool->batch * pool->n_kv_heads);
  const int per = (pool->unit_cap + kSelectThreads - 1) / kSelectThreads;
#define KVC_SEL(K)                                                                            \
  k_select<T, D, K><<<grid, kSelectThreads, 0, s>>>(*pool, (const T *)q, hq, G, budget, flag,  \
                                                     sel_units, sel_cap, sel_n, sel_rows,      \
                                                     scores, counters)
  if (per <= 2) KVC_SEL(2);
  else if (per <= 8) KVC_SEL(8);
  else if (per <= kSelectMaxKeysPerThread) KVC_SEL(kSelectMaxKeysPerThread);
  else return KV_ERR_UNSUPPORTED;
#undef KVC_SEL
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

kv_status launch_select(const kv_pool *pool, const void *q, int hq, int budget,
                        const uint8_t *flag, int32_t *sel_units, int sel_cap, int32_t *sel_n,
                        int32_t *sel_rows, float *scores, int32_t *counters, hipStream_t s) {
  if (pool->dtype == KV_BF16)
    return pool->head_dim == 128
               ? select_dispatch<uint16_t, 128>(pool, q, hq, budget, flag, sel_units, sel_cap,
                                                sel_n, sel_rows, scores, counters, s)
               : select_dispatch<uint16_t, 64>(pool, q, hq, budget, flag, sel_units, sel_cap,
                                               sel_n, sel_rows, scores, counters, s);
  return pool->head_dim == 128
             ? select_dispatch<float, 128>(pool, q, hq, budget, flag, sel_units, sel_cap, sel_n,
                                           sel_rows, scores, counters, s)
             : select_dispatch<float, 64>(pool, q, hq, budget, flag, sel_units, sel_cap, sel_n,
                                          sel_rows, scores, counters, s);
}

// ---------------------------------------------------------------- gather + attend
// Rows of (b, g): the selected units' row ranges (CSR order of the selection
// list) followed by the local-buffer rows. A workgroup of 8 waves takes one
// contiguous share of those rows; each wave keeps 32 rows of K and V in
// flight (16 bytes per lane per row piece) and folds them into a per-lane
// online softmax for the group's G query heads; waves merge through LDS.
// With one share per (b, g) the workgroup writes the output directly;
// otherwise it publishes (m, l, acc) and the last workgroup merges the
// shares in order.
constexpr int kAttendThreads = 512;
constexpr int kAttendWaves = kAttendThreads / 64;
constexpr int kAttendRowsPerWave = 32;    // rows in flight per wave
constexpr int kAttendMinRowsPerSplit = 128;
constexpr int kAttendTargetBlocks = 256;  // one wave of workgroups across the CUs

__device__ __forceinline__ float safe_scale(float m_old, float m_new) {
  return m_old == -INFINITY ? 0.f : exp2f(m_old - m_new);
}

template <typename T, int D, int G>
__global__ void __launch_bounds__(kAttendThreads)
    k_gather_attend(kv_pool pool, const T *__restrict__ q, int hq, float scale_log2,
                    const int32_t *__restrict__ sel_units, int sel_cap,
                    const int32_t *__restrict__ sel_n, float *__restrict__ out,
                    float *__restrict__ partials, int32_t *counters) {
  constexpr int EPL = 16 / Elem<T>::kBytes;  // elements per lane (one 16-byte load)
  constexpr int LPR = D / EPL;               // lanes per row
  constexpr int RPI = 64 / LPR;              // rows per wave instruction
  constexpr int UNR = kAttendRowsPerWave / RPI;
  constexpr int NW = kAttendWaves;
  __shared__ int s_psum[kMaxSel];
  __shared__ int s_start[kMaxSel];
  __shared__ int s_rowtab[kAttendThreads];
  __shared__ int s_wsum[NW];
  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ float s_acc[NW][G][D];
  __shared__ int s_last;

  const int H = pool.n_kv_heads;
  const int bg = blockIdx.y, b = bg / H, g = bg % H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int part = lane % LPR, slot = lane / LPR;
  const int nsplit = gridDim.x, split = blockIdx.x;

  // ---- queries of the group, pre-scaled so that exp2 gives the softmax
  float qf[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 v =
        *reinterpret_cast<const uint4 *>(q + ((size_t)b * hq + g * G + h) * D + part * EPL);
    unpack16<T>(v, qf[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[h][e] *= scale_log2;
  }

  // ---- selected units -> LDS prefix table (block-wide scan of sizes)
  const int n = min(min(sel_n[bg], sel_cap), kMaxSel);
  const int32_t *su = sel_units + (size_t)bg * sel_cap;
  const int32_t *ust = pool.unit_start + (size_t)bg * pool.unit_cap;
  const int32_t *usz = pool.unit_size + (size_t)bg * pool.unit_cap;
  int carry = 0;
  for (int base = 0; base < n; base += kAttendThreads) {
    const int i = base + tid;
    int sz = 0;
    if (i < n) {
      const int u = su[i];
      const bool valid = u >= 0 && u < pool.unit_cap;  // foreign ids count as empty units
      sz = valid ? max(usz[u], 0) : 0;
      s_start[i] = valid ? ust[u] : 0;
    }
    int incl = sz;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int off = carry, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wave) off += s_wsum[w];
      tot += s_wsum[w];
    }
    if (i < n) s_psum[i] = off + incl - sz;
    carry += tot;
    __syncthreads();
  }
  const int r_sel = carry;
  int r_buf = 0, buf_begin = 0;
  if (pool.buf_cap > 0) {
    buf_begin = pool.buf_begin[b];
    r_buf = max(pool.n_rows[b] - buf_begin, 0);
  }
  const int R = r_sel + r_buf;
  const int chunk = (R + nsplit - 1) / nsplit;
  const int r_lo = min(R, split * chunk), r_hi = min(R, r_lo + chunk);

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  const T *kbase = static_cast<const T *>(pool.k) + (size_t)bg * pool.row_cap * D + part * EPL;
  const T *vbase = static_cast<const T *>(pool.v) + (size_t)bg * pool.row_cap * D + part * EPL;

  for (int p0 = r_lo; p0 < r_hi; p0 += kAttendThreads) {
    const int plen = min(kAttendThreads, r_hi - p0);
    if (tid < plen) {
      const int j = p0 + tid;
      int row;
      if (j < r_sel) {
        int lo = 0, hi = n - 1;  // last i with s_psum[i] <= j
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_psum[mid] <= j) lo = mid; else hi = mid - 1;
        }
        row = s_start[lo] + (j - s_psum[lo]);
      } else {
        row = buf_begin + (j - r_sel);
      }
      s_rowtab[tid] = min(max(row, 0), pool.row_cap - 1);
    }
    __syncthreads();
    for (int it = wave * kAttendRowsPerWave; it < plen; it += NW * kAttendRowsPerWave) {
      uint4 kv[UNR], vv[UNR];
      bool ok[UNR];
#pragma unroll
      for (int uu = 0; uu < UNR; ++uu) {
        const int li = it + uu * RPI + slot;
        ok[uu] = li < plen;
        const size_t row = ok[uu] ? (size_t)s_rowtab[li] : 0;
        kv[uu] = *reinterpret_cast<const uint4 *>(kbase + row * D);
        vv[uu] = *reinterpret_cast<const uint4 *>(vbase + row * D);
      }
      float s[UNR][G];
#pragma unroll
      for (int uu = 0; uu < UNR; ++uu) {
        float kf[EPL];
        unpack16<T>(kv[uu], kf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float d0 = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) d0 = fmaf(qf[h][e], kf[e], d0);
#pragma unroll
          for (int o = LPR / 2; o >= 1; o >>= 1) d0 += __shfl_xor(d0, o);
          s[uu][h] = ok[uu] ? d0 : -INFINITY;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mx = m[h];
#pragma unroll
        for (int uu = 0; uu < UNR; ++uu) mx = fmaxf(mx, s[uu][h]);
        const float alpha = safe_scale(m[h], mx);
        float p[UNR];
        float psum = 0.f;
#pragma unroll
        for (int uu = 0; uu < UNR; ++uu) {
          p[uu] = ok[uu] ? exp2f(s[uu][h] - mx) : 0.f;
          psum += p[uu];
        }
        l[h] = l[h] * alpha + psum;
        m[h] = mx;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
#pragma unroll
        for (int uu = 0; uu < UNR; ++uu) {
          float vf[EPL];
          unpack16<T>(vv[uu], vf);
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p[uu], vf[e], acc[h][e]);
        }
      }
    }
    __syncthreads();
  }

  // ---- merge the row groups of the wave (lanes with equal `part`)
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float om = __shfl_xor(m[h], o);
      const float ol = __shfl_xor(l[h], o);
      const float mx = fmaxf(m[h], om);
      const float a1 = safe_scale(m[h], mx), a2 = safe_scale(om, mx);
      l[h] = l[h] * a1 + ol * a2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float oa = __shfl_xor(acc[h][e], o);
        acc[h][e] = acc[h][e] * a1 + oa * a2;
      }
      m[h] = mx;
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (part == 0) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][h][part * EPL + e] = acc[h][e];
    }
  }
  __syncthreads();
  // ---- merge the waves (in order); one share: write the output directly
  const size_t pstride = (size_t)G * (D + 2);
  float *mine = partials + ((size_t)bg * nsplit + split) * pstride;
  for (int i = tid; i < G * D; i += kAttendThreads) {
    const int h = i / D, e = i % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, s_m[w][h]);
    float a = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sc = safe_scale(s_m[w][h], mx);
      a += s_acc[w][h][e] * sc;
      lsum += s_l[w][h] * sc;
    }
    if (nsplit == 1) {
      out[((size_t)b * hq + g * G + h) * D + e] = lsum > 0.f ? a / lsum : 0.f;
    } else {
      mine[h * (D + 2) + e] = a;
      if (e == 0) {
        mine[h * (D + 2) + D] = mx;
        mine[h * (D + 2) + D + 1] = lsum;
      }
    }
  }
  if (nsplit == 1) return;
  if (!last_block_arrives(&counters[bg], nsplit, &s_last)) return;
  // ---- final merge over shares, in share order
  const float *allp = partials + (size_t)bg * nsplit * pstride;
  for (int i = tid; i < G * D; i += kAttendThreads) {
    const int h = i / D, e = i % D;
    float mx = -INFINITY;
    for (int sp = 0; sp < nsplit; ++sp) mx = fmaxf(mx, allp[sp * pstride + h * (D + 2) + D]);
    float a = 0.f, lsum = 0.f;
    for (int sp = 0; sp < nsplit; ++sp) {
      const float *pp = allp + sp * pstride + h * (D + 2);
      const float sc = safe_scale(pp[D], mx);
      a += pp[e] * sc;
      lsum += pp[D + 1] * sc;
    }
    out[((size_t)b * hq + g * G + h) * D + e] = lsum > 0.f ? a / lsum : 0.f;
  }
  if (tid == 0) __hip_atomic_store(&counters[bg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int attend_num_splits(const kv_pool *pool, int max_rows) {
  const long rows = (long)(max_rows > 0 ? max_rows : 0) + (pool->buf_cap > 0 ? pool->buf_cap : 0);
  const long bh = (long)pool->batch * pool->n_kv_heads;
  long by_rows = (rows + kAttendMinRowsPerSplit - 1) / kAttendMinRowsPerSplit;
  long by_grid = (kAttendTargetBlocks + bh - 1) / bh;
  long ns = by_rows < by_grid ? by_rows : by_grid;
  if (ns < 1) ns = 1;
  if (ns > 64) ns = 64;
  return (int)ns;
}

template <typename T, int D>
static kv_status attend_dispatch(const kv_pool *pool, const void *q, int hq, float scale_log2,
                                 const int32_t *sel_units, int sel_cap, const int32_t *sel_n,
                                 int nsplit, float *out, float *partials, int32_t *counters,
                                 hipStream_t s) {
  const int G = hq / pool->n_kv_heads;
  const dim3 grid(nsplit, pool->batch * pool->n_kv_heads);
#define KVC_ATT(GG)                                                                            \
  k_gather_attend<T, D, GG><<<grid, kAttendThreads, 0, s>>>(*pool, (const T *)q, hq,           \
                                                            scale_log2, sel_units, sel_cap,    \
                                                            sel_n, out, partials, counters)
  switch (G) {
    case 1: KVC_ATT(1); break;
    case 2: KVC_ATT(2); break;
    case 4: KVC_ATT(4); break;
    case 8: KVC_ATT(8); break;
    default: return KV_ERR_UNSUPPORTED;
  }
#undef KVC_ATT
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

kv_status launch_gather_attend(const kv_pool *pool, const void *q, int hq, float scale,
                               const int32_t *sel_units, int sel_cap, const int32_t *sel_n,
                               int nsplit, float *out, float *partials, int32_t *counters,
                               hipStream_t s) {
  const float sl2 = scale * 1.4426950408889634f;  // log2(e): exp(x) = exp2(x log2 e)
  if (pool->dtype == KV_BF16)
    return pool->head_dim == 128
               ? attend_dispatch<uint16_t, 128>(pool, q, hq, sl2, sel_units, sel_cap, sel_n,
                                                nsplit, out, partials, counters, s)
               : attend_dispatch<uint16_t, 64>(pool, q, hq, sl2, sel_units, sel_cap, sel_n,
                                               nsplit, out, partials, counters, s);
  return pool->head_dim == 128
             ? attend_dispatch<float, 128>(pool, q, hq, sl2, sel_units, sel_cap, sel_n, nsplit,
                                           out, partials, counters, s)
             : attend_dispatch<float, 64>(pool, q, hq, sl2, sel_units, sel_cap, sel_n, nsplit,
                                          out, partials, counters, s);
}

}  // namespace kvc

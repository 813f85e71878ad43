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
// its results with device-coherent stores and bumps a per-(sequence, head)
// counter; the block that brings the counter to the grid size does the final
// reduction in a fixed order and resets the counter to zero.
#include <algorithm>
#include <utility>

#include "kvc_internal.hpp"

namespace kvc {

// Zero in a register the compiler cannot prove uniform across the wave: a load
// indexed by it stays a vector memory load. Scalar loads of the same data
// would return out of order with the kernel-argument loads, so a later wait
// for any argument would also wait for them.
__device__ __forceinline__ int opaque_zero() {
  int z = 0;
  asm volatile("" : "+v"(z));
  return z;
}

// Completion protocol for the last-block steps. Results that another
// workgroup will read are written with device-coherent stores (relaxed
// agent-scope atomic stores: `sc1` on gfx950, so they do not sit in this
// XCD's non-coherent L2). Every wave waits for its stores to be acknowledged
// (vmcnt(0)) before the workgroup barrier; only then does thread 0 bump the
// counter, so a workgroup that sees the final count also sees every
// published result when it reads them with device-coherent loads. This
// avoids the L2-wide writeback / invalidate that agent-scope fences cost.
// Returns true in the workgroup that completes the count.
__device__ __forceinline__ void coherent_store(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store_i(int32_t *p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t coherent_load_i(const int32_t *p) {
  return __hip_atomic_load(const_cast<int32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store_i2(int32_t *p, int2 v) {
  const unsigned long long u = (unsigned long long)(uint32_t)v.x | ((unsigned long long)(uint32_t)v.y << 32);
  __hip_atomic_store(reinterpret_cast<unsigned long long *>(p), u, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int2 coherent_load_i2(const int32_t *p) {
  const unsigned long long u = __hip_atomic_load(
      reinterpret_cast<unsigned long long *>(const_cast<int32_t *>(p)), __ATOMIC_RELAXED,
      __HIP_MEMORY_SCOPE_AGENT);
  return int2{(int)(uint32_t)u, (int)(uint32_t)(u >> 32)};
}
__device__ __forceinline__ bool last_block_arrives(int32_t *counter, int nblocks, int *s_last) {
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's coherent stores are acknowledged
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_last = (old == nblocks - 1);
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

// r of sequence b, computed by waves 0..3 of the calling workgroup (all of
// its threads must call: the partial sums meet in LDS `part`[4]). Every
// thread receives r. Callers of any workgroup size get the same bits.
// A head is read by LPH lanes with one 16-byte load each, so one wave
// instruction covers HPI heads and the per-head sums reduce over LPH lanes
// for all HPI heads at once; the HPI cosines then sum across lane groups.
// The loads of each wave's first HPW heads can be requested ahead
// (boundary_prefetch), so that a caller with other loads in flight does not
// wait for them before the test; boundary_r_pre then finishes the test with
// the same arithmetic as boundary_r.
template <typename T, int D> struct BoundaryFirst {
  static constexpr int EPL = 16 / (int)sizeof(T);  // elements per 16-byte load
  static constexpr int LPH = D / EPL;              // lanes per head
  static constexpr int HPI = 64 / LPH;             // heads per wave instruction
  static constexpr int HPW = kBoundaryHeadsPerWave;
  static constexpr int NI = HPW / HPI;             // load instructions per tensor and wave step
  static_assert(HPW % HPI == 0 && (LPH == 8 || LPH == 16 || LPH == 32), "head layout");
  uint4 a[NI], c[NI];
};

template <typename T, int D>
__device__ __forceinline__ void boundary_load_step(const T *__restrict__ q_prev,
                                                   const T *__restrict__ q_cur, int hq, int b,
                                                   int h0, BoundaryFirst<T, D> &f) {
  using F = BoundaryFirst<T, D>;
  const int lane = threadIdx.x & 63;
  const int sub = lane / F::LPH, piece = lane % F::LPH;
#pragma unroll
  for (int i = 0; i < F::NI; ++i) {
    const int h = h0 + i * F::HPI + sub;
    const size_t o = ((size_t)b * hq + (h < hq ? h : 0)) * D + piece * F::EPL;
    f.a[i] = *reinterpret_cast<const uint4 *>(q_prev + o);
    f.c[i] = *reinterpret_cast<const uint4 *>(q_cur + o);
  }
}

// W0: the first of the four waves that run the test (its role 0); the roles,
// not the wave numbers, decide the arithmetic.
template <typename T, int D, int W0 = 0>
__device__ __forceinline__ void boundary_prefetch(const T *__restrict__ q_prev,
                                                  const T *__restrict__ q_cur, int hq, int b,
                                                  BoundaryFirst<T, D> &f) {
  const int wave = (int)(threadIdx.x >> 6) - W0;
  if (wave >= 0 && wave < 4 && wave * kBoundaryHeadsPerWave < hq)
    boundary_load_step<T, D>(q_prev, q_cur, hq, b, wave * kBoundaryHeadsPerWave, f);
}

// The four test waves' share: each writes its cosine sum to part[role].
template <typename T, int D, int W0 = 0>
__device__ __forceinline__ void boundary_partial(const T *__restrict__ q_prev,
                                                 const T *__restrict__ q_cur, int hq, int b,
                                                 float *part, const BoundaryFirst<T, D> &first) {
  using F = BoundaryFirst<T, D>;
  constexpr int EPL = F::EPL, LPH = F::LPH, HPI = F::HPI, HPW = F::HPW, NI = F::NI;
  const int wave = (int)(threadIdx.x >> 6) - W0, lane = threadIdx.x & 63;
  const int sub = lane / LPH;
  if (wave >= 0 && wave < 4) {
    float csum = 0.f;
    for (int h0 = wave * HPW; h0 < hq; h0 += 4 * HPW) {
      F f;
      if (h0 == wave * HPW)
        f = first;
      else
        boundary_load_step<T, D>(q_prev, q_cur, hq, b, h0, f);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float x[EPL], y[EPL];
        unpack16<T>(f.a[i], x);
        unpack16<T>(f.c[i], y);
        float dot = 0.f, n1 = 0.f, n2 = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          dot = fmaf(x[e], y[e], dot);
          n1 = fmaf(x[e], x[e], n1);
          n2 = fmaf(y[e], y[e], n2);
        }
        dot = group_sum<LPH>(dot);
        n1 = group_sum<LPH>(n1);
        n2 = group_sum<LPH>(n2);
        const float cosv = (n1 > 0.f && n2 > 0.f) ? dot / (sqrtf(n1) * sqrtf(n2)) : 0.f;
        csum += sum_stride<LPH>(h0 + i * HPI + sub < hq ? cosv : 0.f);
      }
    }
    if (lane == 0) part[wave] = csum;
  }
}

// r from the four shares (every thread of the workgroup must call).
__device__ __forceinline__ float boundary_combine(const float *part, int hq) {
  __syncthreads();
  return (((part[0] + part[1]) + part[2]) + part[3]) / (float)hq;
}

template <typename T, int D, int W0 = 0>
__device__ float boundary_r_pre(const T *__restrict__ q_prev, const T *__restrict__ q_cur, int hq,
                                int b, float *part, const BoundaryFirst<T, D> &first) {
  boundary_partial<T, D, W0>(q_prev, q_cur, hq, b, part, first);
  return boundary_combine(part, hq);
}

template <typename T, int D>
__device__ __forceinline__ float boundary_r(const T *__restrict__ q_prev, const T *__restrict__ q_cur, int hq,
                            int b, float *part) {
  BoundaryFirst<T, D> f;
  boundary_prefetch<T, D>(q_prev, q_cur, hq, b, f);
  return boundary_r_pre<T, D>(q_prev, q_cur, hq, b, part, f);
}

template <typename T, int D>
__global__ void __launch_bounds__(256) k_boundary(const T *__restrict__ q_prev,
                                                  const T *__restrict__ q_cur, int hq, float tau,
                                                  uint8_t *__restrict__ flag, float *__restrict__ r) {
  __shared__ float part[4];
  const int b = blockIdx.x;
  if (q_prev == nullptr) {
    if (threadIdx.x == 0) {
      flag[b] = 1;
      if (r) r[b] = __builtin_nanf("");
    }
    return;
  }
  const float rv = boundary_r<T, D>(q_prev, q_cur, hq, b, part);
  if (threadIdx.x == 0) {
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
// BD > 0: the workgroup first runs the boundary test of its sequence
// (head_dim BD) on (q_prev, q_cur) itself and writes flag / r, instead of
// reading flag.
constexpr int kAppendPrefetch = 8;  // (head, element) pairs per thread loaded up front

template <typename T, int BD>
__global__ void __launch_bounds__(256) k_segment_append(kv_pool pool, const T *__restrict__ k_t,
                                                        const T *__restrict__ v_t,
                                                        const uint8_t *__restrict__ flag,
                                                        const T *__restrict__ q_prev,
                                                        const T *__restrict__ q_cur, int hq,
                                                        float tau, uint8_t *__restrict__ flag_out,
                                                        float *__restrict__ r_out) {
  constexpr int PER = kAppendPrefetch;
  __shared__ int s_close, s_ok, s_open_len, s_seg_begin, s_n_rows, s_n_units;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int H = pool.n_kv_heads, D = pool.head_dim;
  const int HD = H * D;
  // Everything that does not depend on the boundary decision is requested
  // first, so it shares one memory round trip with the boundary test's loads.
  int c_rows = 0, c_seg = 0, c_units = 0, c_buf = 0, c_cand = 0;
  if (tid == 0) {
    c_rows = pool.n_rows[b];
    c_seg = pool.seg_begin[b];
    c_units = pool.n_units[b];
    c_buf = pool.buf_begin[b];
    c_cand = pool.n_cand[b];
  }
  float sums[PER];
  T kvs[PER], vvs[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid + j * 256;
    if (i < HD) {
      sums[j] = pool.seg_sum[(size_t)b * HD + i];
      kvs[j] = k_t[(size_t)b * HD + i];
      vvs[j] = v_t[(size_t)b * HD + i];
    }
  }
  int f;
  if constexpr (BD > 0) {
    __shared__ float s_part[4];
    float rv = __builtin_nanf("");
    f = 1;
    if (q_prev != nullptr) {
      rv = boundary_r<T, BD>(q_prev, q_cur, hq, b, s_part);
      f = rv < tau ? 1 : 0;
    }
    if (tid == 0) {
      flag_out[b] = (uint8_t)f;
      if (r_out) r_out[b] = rv;
    }
  } else {
    f = tid == 0 ? flag[b] != 0 : 0;
  }
  if (tid == 0) {
    const int open_len = c_rows - c_seg;
    const int close = (f && open_len > 0) || open_len >= pool.buf_cap;
    int ok = c_rows < pool.row_cap && (!close || c_units < pool.unit_cap);
    if (!ok) __hip_atomic_store(pool.status, (int)KV_ERR_CAPACITY, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
    s_close = close;
    s_ok = ok;
    s_open_len = open_len;
    s_seg_begin = c_seg;
    s_n_rows = c_rows;
    s_n_units = c_units;
  }
  __syncthreads();
  if (!s_ok) return;
  const int close = s_close, open_len = s_open_len, n_rows = s_n_rows, n_units = s_n_units;
  auto move = [&](int i, float sum, T kv, T vv) {
    const int g = i / D, e = i % D;
    const size_t bg = (size_t)b * H + g;
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
    const size_t ro = (bg * pool.row_cap + n_rows) * D + e;
    static_cast<T *>(pool.k)[ro] = kv;
    static_cast<T *>(pool.v)[ro] = vv;
    if (pool.buf_k != nullptr) {  // the local buffer's HBM copy: slot n_rows % buf_ring
      const size_t bo = (bg * pool.buf_ring + n_rows % pool.buf_ring) * D + e;
      static_cast<T *>(pool.buf_k)[bo] = kv;
      static_cast<T *>(pool.buf_v)[bo] = vv;
    }
    pool.seg_sum[(size_t)b * HD + i] = sum + Elem<T>::to_f32(kv);
  };
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = tid + j * 256;
    if (i < HD) move(i, sums[j], kvs[j], vvs[j]);
  }
  for (int i = tid + PER * 256; i < HD; i += 256)  // more than PER elements per thread
    move(i, pool.seg_sum[(size_t)b * HD + i], k_t[(size_t)b * HD + i], v_t[(size_t)b * HD + i]);
  if (tid == 0) {
    const int new_rows = n_rows + 1;
    const int new_units = n_units + close;
    int seg_begin = close ? n_rows : s_seg_begin;
    int buf_begin = c_buf;
    int n_cand = c_cand;
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
                                const uint8_t *flag, bool fused, const void *q_prev,
                                const void *q_cur, int hq, float tau, uint8_t *flag_out,
                                float *r_out, hipStream_t s) {
#define KVC_SA(T, BD)                                                                         \
  k_segment_append<T, BD><<<pool->batch, 256, 0, s>>>(                                        \
      *pool, (const T *)k_t, (const T *)v_t, flag, (const T *)q_prev, (const T *)q_cur, hq, \
      tau, flag_out, r_out)
  const bool d128 = pool->head_dim == 128;
  if (pool->dtype == KV_BF16) {
    if (!fused) KVC_SA(uint16_t, 0);
    else if (d128) KVC_SA(uint16_t, 128);
    else KVC_SA(uint16_t, 64);
  } else {
    if (!fused) KVC_SA(float, 0);
    else if (d128) KVC_SA(float, 128);
    else KVC_SA(float, 64);
  }
#undef KVC_SA
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

// ---------------------------------------------------------------- select
// Scoring: 512-thread workgroups each score up to 512 units; a unit's index
// vector is read as 16-byte pieces, so one wave instruction covers 64 / LPU
// units, and a wave's 64 scores leave in one store. Selection: the last
// workgroup of (b, g) holds every candidate as a 64-bit key (orderable score
// << 32 | ~id) in registers, KPT units per thread, and finds the first unit
// that no longer fits the budget (select_prefix_block: a pass over score
// buckets, then a direct ranking or radix passes within the crossing bucket).
// Every unit ranked before it is selected.
constexpr int kSelectThreads = kSelectBlockThreads;
constexpr int kSelectWaves = kSelectThreads / 64;
constexpr int kScoreUnitsPerBlock = kSelectThreads;

// Wave 0 helper: lane l holds the weights wd[i] of digits 255 - 4 l - i
// (i = 0..3, descending). Given the weight already above the range and the
// budget, finds the highest digit whose inclusion makes the running total
// (taken from the top digit down) exceed the budget: returns it, or -1 if
// every digit fits, with *above_out = the weight of the digits above it and
// *lane_out = the lane that owns it.
__device__ int find_crossing_digit(const long (&wd)[4], long above, long budget, long *above_out,
                                   int *lane_out) {
  const int lane = threadIdx.x & 63;
  long local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) local += wd[i];
  const long incl = wave_incl_scan_i64(local);
  const long excl = incl - local;
  int found = -1;
  long found_above = 0;
  long run = above + excl;
  if (run <= budget && above + incl > budget) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (found < 0 && run + wd[i] > budget) {
        found = 255 - 4 * lane - i;
        found_above = run;
      }
      run += wd[i];
    }
  }
  const uint64_t who = __ballot(found >= 0);
  if (who == 0) return -1;
  const int src = __ffsll((unsigned long long)who) - 1;
  *above_out = lane_value_i64(found_above, src);
  *lane_out = src;
  return lane_value(found, src);
}

__device__ __forceinline__ unsigned long long unit_key(float score, int u) {
  return ((unsigned long long)float_order_key(score) << 32) | (uint32_t)(0xffffffffu - (uint32_t)u);
}

// ---- pieces of the selection shared by k_select and k_decode_step

// The group's query pieces for scoring: lane part p of head h holds elements
// EPL p .. EPL p + EPL - 1 (requested early, summed later).
template <typename T, int D>
__device__ __forceinline__ void score_query_load(const T *__restrict__ q, int hq, int b, int g,
                                                 int group, int lane, uint4 (&qv)[8]) {
  constexpr int EPL = 16 / Elem<T>::kBytes;
  constexpr int LPU = D / EPL;
  const int part = lane % LPU;
#pragma unroll
  for (int h = 0; h < 8; ++h)
    if (h < group)
      qv[h] = *reinterpret_cast<const uint4 *>(q + ((size_t)b * hq + g * group + h) * D + part * EPL);
}

// Summed group query (heads in order), this lane's EPL elements.
template <typename T, int D>
__device__ __forceinline__ void score_query_sum(const uint4 (&qv)[8], int group,
                                                float (&qs)[16 / Elem<T>::kBytes]) {
  constexpr int EPL = 16 / Elem<T>::kBytes;
#pragma unroll
  for (int e = 0; e < EPL; ++e) qs[e] = 0.f;
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    if (h < group) {
      float f[EPL];
      unpack16<T>(qv[h], f);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qs[e] += f[e];
    }
  }
}

// One wave scores units [u0, u0 + 64) (those below U): s_u = qs . idx_u in
// fp32, a fixed summation order per unit whichever wave computes it; scores
// go out with device-coherent stores.
template <typename T, int D>
__device__ __forceinline__ void score_units64(const T *__restrict__ idx, float *sc,
                                              const float (&qs)[16 / Elem<T>::kBytes], int u0,
                                              int U, int lane) {
  constexpr int EPL = 16 / Elem<T>::kBytes;  // elements per 16-byte lane load
  constexpr int LPU = D / EPL;               // lanes per index vector
  constexpr int UPW = 64 / LPU;              // units per wave instruction
  // every load of the wave's 64 units in flight at once (one round trip)
  constexpr int UNR = 64 / UPW < 16 ? 64 / UPW : 16;
  const int part = lane % LPU, slot = lane / LPU;
  const int ulast = max(U - 1, 0);  // loads at clamped units (in the pool), masked at the store
#pragma unroll
  for (int j0 = 0; j0 < 64; j0 += UPW * UNR) {
    uint4 v[UNR];
#pragma unroll
    for (int i = 0; i < UNR; ++i) {
      const int u = min(u0 + j0 + i * UPW + slot, ulast);
      v[i] = *reinterpret_cast<const uint4 *>(idx + (size_t)u * D + part * EPL);
    }
    float dots[UNR];
#pragma unroll
    for (int i = 0; i < UNR; ++i) {
      float f[EPL];
      unpack16<T>(v[i], f);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dot = fmaf(qs[e], f[e], dot);
      dots[i] = group_sum<LPU>(dot);
    }
    if constexpr (UNR * UPW == 64) {
      // one store instruction for the 64 units: lane s offers the dot of its
      // group's unit i = s % LPU, and lane l takes unit l's from lane
      // (l % UPW) LPU + l / UPW
      float w = dots[0];
#pragma unroll
      for (int i = 1; i < UNR; ++i) w = (part == i) ? dots[i] : w;
      const int src = (lane % UPW) * LPU + lane / UPW;
      const float mine = __int_as_float(__builtin_amdgcn_ds_bpermute(src * 4, __float_as_int(w)));
      if (u0 + lane < U) coherent_store(&sc[u0 + lane], mine);
    } else {
#pragma unroll
      for (int i = 0; i < UNR; ++i) {
        const int u = u0 + j0 + i * UPW + slot;
        if (part == 0 && u < U) coherent_store(&sc[u], dots[i]);
      }
    }
  }
}

// The selection's units: slot j (< KPT) of wave w, lane l holds unit
// (w KPT + j) 64 + l, so that each wave instruction that reads or writes a
// per-unit value touches 64 consecutive units (the scores, written by other
// workgroups, are read past the L2s: 256 contiguous bytes per instruction
// rather than one dword from each of 64 lines).
template <int KPT> __device__ __forceinline__ int select_unit(int j) {
  return (((int)threadIdx.x >> 6) * KPT + j) * 64 + ((int)threadIdx.x & 63);
}

// Unit sizes (0 past U) and first rows of this thread's KPT units.
template <int KPT>
__device__ __forceinline__ void select_sizes(const kv_pool &pool, int bg, int U, int (&sz)[KPT],
                                             int (&ust)[KPT]) {
  const int32_t *usz = pool.unit_size + (size_t)bg * pool.unit_cap;
  const int32_t *ustp = pool.unit_start + (size_t)bg * pool.unit_cap;
  // Every load is issued, at a clamped index, and masked afterwards: a load
  // under a per-lane condition whose result is reshaped inside the branch
  // makes the compiler wait for it there, one round trip per load.
  int raw[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    raw[j] = usz[min(select_unit<KPT>(j), pool.unit_cap - 1)];
    ust[j] = ustp[min(select_unit<KPT>(j), pool.unit_cap - 1)];
  }
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int u = select_unit<KPT>(j);
    sz[j] = (u < U && raw[j] > 0) ? raw[j] : 0;
  }
}

// The selection proper, run by the one workgroup of NT threads that holds all
// of (b, g)'s scores: every candidate becomes a 64-bit key (orderable score
// << 32 | ~id), KPT units per thread (select_unit). The first unit that no
// longer fits the budget (the crossing unit) is found by counting passes into
// per-wave LDS histograms hw / hc [NT / 64][256] (weight, count; a thread's
// run of equal digits counted once, a wave whose keys share one digit counted
// with one update): first over 256 equal-width buckets of the score between
// the lowest and highest score (when all scores are finite and differ); a
// crossing bucket of <= 64 units is then ranked directly by wave 0; otherwise
// MSB-first 8-bit digits of the keys in that bucket, from the highest bit in
// which the keys differ, until the crossing digit holds a single unit. Every
// unit ranked before the crossing unit is written, in ascending id, to
// sel_units (and its row span to sel_spans), with sel_n and sel_rows. Ends
// with a barrier.
template <int NT, int KPT, bool COH = false>
__device__ void select_prefix_block(const kv_pool &pool, int bg, int budget, const float *sc,
                                    const int (&sz)[KPT], const int (&ustv)[KPT],
                                    int32_t *__restrict__ sel_units,
                                    int sel_cap, int32_t *__restrict__ sel_n,
                                    int32_t *__restrict__ sel_rows,
                                    int32_t *__restrict__ sel_spans, int (*hw)[256],
                                    int (*hc)[256]) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  unsigned long long key[KPT];
  unsigned long long kor = 0ull, kand = ~0ull;
  uint32_t vmax = 0u, vmin = 0xffffffffu;  // score parts of the keys
  float scv[KPT];  // all requested at once (clamped index), masked below
#pragma unroll
  for (int j = 0; j < KPT; ++j) scv[j] = coherent_load(&sc[min(select_unit<KPT>(j), pool.unit_cap - 1)]);
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int u = select_unit<KPT>(j);
    key[j] = sz[j] > 0 ? unit_key(scv[j], u) : 0ull;
    if (sz[j] > 0) {
      kor |= key[j];
      kand &= key[j];
      vmax = max(vmax, (uint32_t)(key[j] >> 32));
      vmin = min(vmin, (uint32_t)(key[j] >> 32));
    }
  }

  __shared__ unsigned long long hk[256];
  __shared__ unsigned long long s_or[NW], s_and[NW];
  __shared__ uint32_t s_vmax[NW], s_vmin[NW];
  __shared__ long s_above;
  __shared__ int s_done, s_none, s_cnt, s_cn;
  __shared__ unsigned long long s_prefix, s_kstar;
  __shared__ unsigned long long s_ck[64];
  __shared__ int s_cs[64];
  // The bits in which the candidates' keys differ (the bit passes start at the
  // highest of them: the bits above are common to every key) and the range of
  // their scores.
  kor = wave_bits64<true>(kor);
  kand = wave_bits64<false>(kand);
  vmax = wave_max_u32(vmax);
  vmin = wave_min_u32(vmin);
  if (lane == 0) {
    s_or[wave] = kor;
    s_and[wave] = kand;
    s_vmax[wave] = vmax;
    s_vmin[wave] = vmin;
  }
  if (tid == 0) {
    s_above = 0;
    s_done = 0;
    s_none = 0;
    s_cn = 0;
  }
  __syncthreads();
  kor = 0ull;
  kand = ~0ull;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    kor |= s_or[v];
    kand &= s_and[v];
    vmax = max(vmax, s_vmax[v]);
    vmin = min(vmin, s_vmin[v]);
  }

  // One counting pass: every candidate with in(j) adds its weight and count to
  // the bucket dig(j) (0..255) of its wave's histogram row; wave 0 then finds
  // the crossing bucket over the rows (digits from 255 down, after the weight
  // s_above already above them). Sets s_prefix's digit field through `mark`,
  // s_above, s_cnt (the crossing bucket's units), or s_none / s_done.
  auto count_pass = [&](auto in, auto dig, auto mark) {
    // each wave counts into its own histogram row: cleared and filled in
    // program order, so no barrier between
    for (int i = lane; i < 256; i += 64) {
      hw[wave][i] = 0;
      hc[wave][i] = 0;
    }
    // runs of equal digits among this thread's units count once
    int rd = -1, rw = 0, rc = 0;
    unsigned long long rk = 0ull;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (!in(j)) continue;
      const int dgt = dig(j);
      if (dgt != rd) {
        if (rc > 0) {
          atomicAdd(&hw[wave][rd], rw);
          atomicAdd(&hc[wave][rd], rc);
          hk[rd] = rk;  // any member; read only when the bucket holds one unit
        }
        rd = dgt;
        rw = 0;
        rc = 0;
      }
      rw += sz[j];
      rc += 1;
      rk = key[j];
    }
    const uint64_t act = __ballot(rc > 0);
    if (act != 0) {
      const int src = __ffsll((unsigned long long)act) - 1;
      const int d0 = lane_value(rd, src);
      if (__ballot(rc > 0 && rd != d0) == 0) {
        // one digit for the whole wave (keys concentrated in a bucket): one
        // update instead of 64 conflicting ones
        const int w = wave_sum_i32(rc > 0 ? rw : 0), c = wave_sum_i32(rc);
        if (lane == src) {
          hw[wave][d0] += w;
          hc[wave][d0] += c;
          hk[d0] = rk;
        }
      } else if (rc > 0) {
        atomicAdd(&hw[wave][rd], rw);
        atomicAdd(&hc[wave][rd], rc);
        hk[rd] = rk;
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane l: digits 255 - 4 l .. 252 - 4 l, summed over the waves' rows
      long wd[4];
      int cd[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 255 - 4 * lane - i;
        int w = 0, c = 0;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
          w += hw[v][d];
          c += hc[v][d];
        }
        wd[i] = w;
        cd[i] = c;
      }
      long above_out = 0;
      int owner = 0;
      const int dgt = find_crossing_digit(wd, s_above, budget, &above_out, &owner);
      const int i_own = dgt >= 0 ? (255 - dgt) & 3 : 0;
      const int cnt =
          lane_value(i_own == 0 ? cd[0] : i_own == 1 ? cd[1] : i_own == 2 ? cd[2] : cd[3], owner);
      if (lane == 0) {
        if (dgt < 0) {
          s_none = 1;  // everything in range fits (only possible in the first pass)
          s_done = 1;
        } else {
          s_above = above_out;
          s_cnt = cnt;
          mark(dgt);
          if (cnt == 1) {
            s_kstar = hk[dgt];
            s_done = 1;
          }
        }
      }
    }
    __syncthreads();
  };

  // First pass over score values: 256 equal-width buckets between the lowest
  // and the highest score (monotone in the score, so in key order), which
  // spread the candidates where the top bits of their keys do not. Skipped
  // when a score is not finite or all are equal.
  const float smax = order_key_float(vmax), smin = order_key_float(vmin);
  const float vrange = smax - smin, vscale = 256.0f / vrange;
  const bool vpass = vmax > vmin && isfinite(smax) && isfinite(smin) && vrange > 0.f &&
                     isfinite(vscale);
  auto vdigit = [&](int j) {
    const float sj = order_key_float((uint32_t)(key[j] >> 32));
    return min(255, (int)((sj - smin) * vscale));
  };
  int vstar = -1;  // the crossing value bucket
  if (vpass) {
    count_pass([&](int j) { return sz[j] > 0; }, vdigit, [&](int d) { s_prefix = (unsigned long long)d; });
    vstar = (int)s_prefix;
    if (!s_done && s_cnt <= 64) {
      // few units in the crossing bucket: wave 0 ranks them directly (the
      // weight of the bucket's units above each, added to the weight above
      // the bucket) and the unit whose own weight crosses the budget ends it
      for (int j = 0; j < KPT; ++j)
        if (sz[j] > 0 && vdigit(j) == vstar) {
          const int p = atomicAdd(&s_cn, 1);
          s_ck[p] = key[j];
          s_cs[p] = sz[j];
        }
      __syncthreads();
      if (wave == 0) {
        const int n = s_cn;
        const unsigned long long mine = lane < n ? s_ck[lane] : 0ull;
        const long base = s_above;
        long ab = base;
        for (int k = 0; k < n; ++k)
          if (s_ck[k] > mine) ab += s_cs[k];
        const bool cross = lane < n && ab <= budget && ab + (lane < n ? s_cs[lane] : 0) > budget;
        const uint64_t who = __ballot(cross);
        if (lane == 0) {
          s_kstar = who ? s_ck[__ffsll((unsigned long long)who) - 1] : s_ck[0];
          s_done = 1;
        }
      }
      __syncthreads();
    }
  }
  if (!s_done) {
    // MSB-first bit passes: bits [sh, sh + width) of the keys that agree with
    // the prefix above them (and lie in the crossing value bucket)
    const unsigned long long diff = kor ^ kand;
    const int hibit = diff ? 63 - __clzll((long long)diff) : 0;
    int sh = max(hibit - 7, 0), width = 8;
    unsigned long long prefix = (sh + width >= 64) ? 0ull : (kand >> (sh + width)) << (sh + width);
    for (;;) {
      const int top = sh + width;
      const unsigned long long dmask = (1ull << width) - 1ull;
      count_pass(
          [&](int j) {
            return sz[j] > 0 && (top >= 64 || (key[j] >> top) == (prefix >> top)) &&
                   (vstar < 0 || vdigit(j) == vstar);
          },
          [&](int j) { return (int)((key[j] >> sh) & dmask); },
          [&](int d) {
            s_prefix = prefix | ((unsigned long long)d << sh);
            if (sh == 0) {
              s_kstar = s_prefix;
              s_done = 1;
            }
          });
      if (s_done) break;
      prefix = s_prefix;
      if (sh >= 8) {
        sh -= 8;
      } else {
        width = sh;
        sh = 0;
      }
    }
  }
  const bool take_all = s_none != 0;
  const unsigned long long kstar = s_kstar;

  // ---- compaction in ascending unit id: units go in (wave, slot, lane)
  // order, so a unit's position is the selected count of the earlier waves,
  // of this wave's earlier slots and of the slot's lower lanes (ballots)
  int32_t *out = sel_units + (size_t)bg * sel_cap;
  int32_t *spans = sel_spans ? sel_spans + (size_t)bg * sel_cap * 2 : nullptr;
  uint64_t bsel[KPT];
  int cnt = 0, rows = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool sj = sz[j] > 0 && (take_all || key[j] > kstar);
    bsel[j] = __ballot(sj);
    cnt += __popcll(bsel[j]);
    rows += sj ? sz[j] : 0;
  }
  rows = wave_sum_i32(rows);
  __shared__ int wsum[NW], wrows[NW];
  if (lane == 0) {
    wsum[wave] = cnt;
    wrows[wave] = rows;
  }
  __syncthreads();
  int pos = 0, total = 0, total_rows = 0;
  for (int w = 0; w < NW; ++w) {
    if (w < wave) pos += wsum[w];
    total += wsum[w];
    total_rows += wrows[w];
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int p = pos + __popcll(bsel[j] & below);
    if (((bsel[j] >> lane) & 1ull) && p < sel_cap) {
      out[p] = select_unit<KPT>(j);
      if (spans) {
        if constexpr (COH)
          coherent_store_i2(spans + 2 * p, int2{ustv[j], sz[j]});
        else
          *reinterpret_cast<int2 *>(spans + 2 * p) = int2{ustv[j], sz[j]};
      }
    }
    pos += __popcll(bsel[j]);
  }
  if (tid == 0) {
    if (total > sel_cap) {
      __hip_atomic_store(pool.status, (int)KV_ERR_CAPACITY, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      total = sel_cap;
    }
    if constexpr (COH)
      coherent_store_i(&sel_n[bg], total);
    else
      sel_n[bg] = total;
    sel_rows[bg] = total_rows;
  }
  __syncthreads();
}

// FUSED: the workgroup first runs the boundary test of its sequence on
// (q_prev, q) itself (flag_out / r_out written once per sequence) instead of
// reading flag. The unit count and the group's queries are requested in the
// same memory round trip as the decision's inputs.
template <typename T, int D, int KPT, bool FUSED>
__global__ void __launch_bounds__(kSelectThreads)
    k_select(kv_pool pool, const T *__restrict__ q, int hq, int group, int budget,
             const uint8_t *__restrict__ flag, int32_t *__restrict__ sel_units, int sel_cap,
             int32_t *__restrict__ sel_n, int32_t *__restrict__ sel_rows,
             int32_t *__restrict__ sel_spans, float *__restrict__ scores,
             int32_t *counters, const T *__restrict__ q_prev, float tau,
             uint8_t *__restrict__ flag_out, float *__restrict__ r_out) {
  constexpr int EPL = 16 / Elem<T>::kBytes;
  const int H = pool.n_kv_heads;
  const int bg = blockIdx.y, b = bg / H, g = bg % H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n_cand = pool.n_cand[b];
  uint4 qv[8];
  score_query_load<T, D>(q, hq, b, g, group, lane, qv);
  if constexpr (FUSED) {
    __shared__ float s_part[4];
    int f = 1;
    float rv = __builtin_nanf("");
    if (q_prev != nullptr) {
      rv = boundary_r<T, D>(q_prev, q, hq, b, s_part);
      f = rv < tau ? 1 : 0;
    }
    if (blockIdx.x == 0 && g == 0 && tid == 0) {
      flag_out[b] = (uint8_t)f;
      if (r_out) r_out[b] = rv;
    }
    if (!f) return;
  } else {
    if (flag != nullptr && flag[b] == 0) return;
  }
  const int U = min(max(n_cand, 0), pool.unit_cap);

  // ---- scoring: s_u = (sum_h q_h) . idx_u, fp32
  float qs[EPL];
  score_query_sum<T, D>(qv, group, qs);
  const T *idx = static_cast<const T *>(pool.unit_index) + (size_t)bg * pool.unit_cap * D;
  float *sc = scores + (size_t)bg * pool.unit_cap;
  score_units64<T, D>(idx, sc, qs, blockIdx.x * kScoreUnitsPerBlock + wave * 64, U, lane);

  // ---- completion: the last block of (b, g) selects. Unit sizes are
  // requested before the arrival so that they land with the store acks.
  int sz[KPT], ust[KPT];
  select_sizes<KPT>(pool, bg, U, sz, ust);
  __shared__ int s_last;
  if (!last_block_arrives(&counters[bg], (int)gridDim.x, &s_last)) return;
  __shared__ int hw[kSelectWaves][256];
  __shared__ int hc[kSelectWaves][256];
  select_prefix_block<kSelectThreads, KPT>(pool, bg, budget, sc, sz, ust, sel_units, sel_cap, sel_n,
                                           sel_rows, sel_spans, hw, hc);
  if (tid == 0) __hip_atomic_store(&counters[bg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int select_num_blocks(const kv_pool *pool) {
  const int nb = (pool->unit_cap + kScoreUnitsPerBlock - 1) / kScoreUnitsPerBlock;
  return nb < 1 ? 1 : nb;
}

template <typename T, int D>
static kv_status select_dispatch(const kv_pool *pool, const void *q, int hq, int budget,
                                 const uint8_t *flag, int32_t *sel_units, int sel_cap,
                                 int32_t *sel_n, int32_t *sel_rows, int32_t *sel_spans,
                                 float *scores, int32_t *counters, bool fused, const void *q_prev,
                                 float tau, uint8_t *flag_out, float *r_out, hipStream_t s) {
  const int G = hq / pool->n_kv_heads;
  const dim3 grid(select_num_blocks(pool), pool->batch * pool->n_kv_heads);
  const int per = (pool->unit_cap + kSelectThreads - 1) / kSelectThreads;
#define KVC_SEL(K, F)                                                                          \
  k_select<T, D, K, F><<<grid, kSelectThreads, 0, s>>>(                                        \
      *pool, (const T *)q, hq, G, budget, flag, sel_units, sel_cap, sel_n, sel_rows,           \
      sel_spans, scores, counters, (const T *)q_prev, tau, flag_out, r_out)
#define KVC_SEL2(K)         \
  do {                      \
    if (fused)              \
      KVC_SEL(K, true);     \
    else                    \
      KVC_SEL(K, false);    \
  } while (0)
  static_assert(kSelectMaxKeysPerThread == 16, "one instantiation per key count");
  if (per <= 4) KVC_SEL2(4);
  else if (per <= 16) KVC_SEL2(16);
  else return KV_ERR_UNSUPPORTED;
#undef KVC_SEL2
#undef KVC_SEL
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

kv_status launch_select(const kv_pool *pool, const void *q, int hq, int budget,
                        const uint8_t *flag, int32_t *sel_units, int sel_cap, int32_t *sel_n,
                        int32_t *sel_rows, int32_t *sel_spans, float *scores, int32_t *counters,
                        bool fused,
                        const void *q_prev, float tau, uint8_t *flag_out, float *r_out,
                        hipStream_t s) {
#define KVC_SD(T, D)                                                                          \
  select_dispatch<T, D>(pool, q, hq, budget, flag, sel_units, sel_cap, sel_n, sel_rows,         \
                        sel_spans, scores, counters, fused, q_prev, tau, flag_out, r_out, s)
  kv_status st;
  if (pool->dtype == KV_BF16)
    st = pool->head_dim == 128 ? KVC_SD(uint16_t, 128) : KVC_SD(uint16_t, 64);
  else
    st = pool->head_dim == 128 ? KVC_SD(float, 128) : KVC_SD(float, 64);
#undef KVC_SD
  return st;
}

// ---------------------------------------------------------------- gather + attend
// Rows of (b, g): the selected units' row ranges (CSR order of the selection
// list) followed by the local-buffer rows, or the working set's contiguous
// rows. A workgroup takes one contiguous share of those rows (shares of
// ceil(max(R, bound) / splits) rows, bound = max_rows + the buffer's
// capacity) and folds them into an online softmax for the group's G query
// heads; waves merge through LDS. With one share per (b, g) the workgroup
// writes the output directly; otherwise it publishes (m, l, acc) and the
// last workgroup merges the shares in order.
//
// bf16 keys: q.k for 16 rows x 16 query columns (G used) is one
// v_mfma_f32_16x16x32_bf16 chain over the head dimension; p.v runs on the
// same tiles for head dimension 128 (the V rows transposed in registers,
// see AttendAcc) and on the VALU for 64, where the probabilities reach the
// lanes holding the V rows by row broadcasts. fp32 keys take an all-VALU
// variant.
constexpr int kAttendMinRowsPerSplit = 64;
constexpr int kAttendTargetBlocks = 256;  // one 8-wave workgroup per CU

__device__ __forceinline__ float safe_scale(float m_old, float m_new) {
  return m_old == -INFINITY ? 0.f : exp2f(m_old - m_new);
}

// Selected units of (b, g) -> LDS: s_start[i] first row, s_psum[i] rows before
// unit i in the concatenated selection. Thread t owns the contiguous run of
// list positions [t per, (t + 1) per), per = ceil(sel_cap / NT), and loads its
// ids before the list length is known (positions past the length are simply
// not used), so the ids, the length and the unit table cost two dependent
// memory round trips whatever the length. Sets *n_out to the list length
// (clamped to [0, sel_cap]) and returns the selection's row count.
template <int NT, bool COH = false>
__device__ int attend_load_selection(const kv_pool &pool, int bg, const int32_t *su,
                                     const int32_t *spans, const int32_t *sel_n, int sel_cap,
                                     int *n_out, int *s_psum, int *s_start, int *s_wsum) {
  constexpr int NW = NT / 64;
  constexpr int PER_MAX = kMaxSel / NT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int per = (sel_cap + NT - 1) / NT;  // sel_cap <= kMaxSel
  const int i0 = tid * per;
  int sz[PER_MAX], st[PER_MAX];
  int n;
  // Loads are issued for every slot at a clamped index (sel_cap >= 1) and
  // masked afterwards, so that all of them are in flight together: a load
  // under a per-lane condition makes the compiler wait for it in its branch.
  if (spans != nullptr) {
    // row spans given: ids are not needed, one round trip
#pragma unroll
    for (int j = 0; j < PER_MAX; ++j) {
      const int i = min(i0 + j, sel_cap - 1);
      const int2 v = COH ? coherent_load_i2(spans + 2 * i)
                         : *reinterpret_cast<const int2 *>(spans + 2 * i);
      st[j] = v.x;
      sz[j] = v.y;
    }
    n = min(max(COH ? coherent_load_i(&sel_n[bg]) : sel_n[bg], 0), sel_cap);
#pragma unroll
    for (int j = 0; j < PER_MAX; ++j) {
      const bool valid = j < per && i0 + j < n;
      sz[j] = valid ? max(sz[j], 0) : 0;
      st[j] = valid ? st[j] : 0;
    }
  } else {
    int uid[PER_MAX];
#pragma unroll
    for (int j = 0; j < PER_MAX; ++j) uid[j] = su[min(i0 + j, sel_cap - 1)];
    n = min(max(sel_n[bg], 0), sel_cap);
    const int32_t *ust = pool.unit_start + (size_t)bg * pool.unit_cap;
    const int32_t *usz = pool.unit_size + (size_t)bg * pool.unit_cap;
    int rs[PER_MAX], rz[PER_MAX];
#pragma unroll
    for (int j = 0; j < PER_MAX; ++j) {
      // foreign ids count as empty units (their loads read unit 0)
      const int u = (uid[j] >= 0 && uid[j] < pool.unit_cap) ? uid[j] : 0;
      rz[j] = usz[u];
      rs[j] = ust[u];
    }
#pragma unroll
    for (int j = 0; j < PER_MAX; ++j) {
      const int u = uid[j];
      const bool valid = j < per && i0 + j < n && u >= 0 && u < pool.unit_cap;
      sz[j] = valid ? max(rz[j], 0) : 0;
      st[j] = valid ? rs[j] : 0;
    }
  }
  int run = 0;
#pragma unroll
  for (int j = 0; j < PER_MAX; ++j) run += sz[j];
  const int incl = wave_incl_scan_i32(run);
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int off = incl - run, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) off += s_wsum[w];
    tot += s_wsum[w];
  }
#pragma unroll
  for (int j = 0; j < PER_MAX; ++j) {
    if (j < per && i0 + j < n) {
      s_psum[i0 + j] = off;
      s_start[i0 + j] = st[j];
    }
    off += sz[j];
  }
  __syncthreads();
  *n_out = n;
  return tot;
}

// Pool row of position j (< r_sel: inside the selection, else the buffer).
// ring > 0 (the pool keeps an HBM copy of its local buffer): a buffer row r
// is returned as ~(r % ring), its slot in the copy, so that negative entries
// of a row table name buffer slots.
__device__ __forceinline__ int attend_row_of(int j, int n, int r_sel, int buf_begin,
                                             const int *s_psum, const int *s_start, int row_cap,
                                             int ring = 0) {
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
    if (ring > 0) return ~(max(row, 0) % ring);
  }
  return min(max(row, 0), row_cap - 1);
}

// Merge NW wave states (m, l, acc over D) per head, then either write the
// output (one share) or publish the share and let the last workgroup merge.
// The last workgroup reads every share with all loads in flight at once: one
// wave per head reduces (m, l) across the shares (lane = share), then each
// thread folds its output elements over the shares in batches of kMergeBatch.
constexpr int kMaxSplits = 64;
constexpr int kMergeBatch = 16;

// Share values (output element tid + k NT, shares sp0 .. sp0 + kMergeBatch - 1).
template <int NT, int G, int D, int EPT>
__device__ __forceinline__ void merge_load_batch(float (&v)[EPT][kMergeBatch], const float *allp,
                                                 size_t pstride, int sp0, int nsplit) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int i = tid + k * NT, h = i / D, e = i % D;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j)
      v[k][j] = (i < G * D && sp0 + j < nsplit)
                    ? coherent_load(&allp[(sp0 + j) * pstride + h * (D + 2) + e])
                    : 0.f;
  }
}

template <int NT, int G, int D>
__device__ __forceinline__ void attend_finish(int bg, int b, int g, int hq, int nsplit, int split,
                              const float (*s_m)[G], const float (*s_l)[G],
                              const float (*s_acc)[G][D], float *out, float *partials,
                              int32_t *counters, int *s_last) {
  constexpr int NW = NT / 64;
  constexpr int EPT = (G * D + NT - 1) / NT;  // output elements per thread
  __shared__ float s_scale[kMaxSplits][G];
  __shared__ float s_lsum[G];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const size_t pstride = (size_t)G * (D + 2);
  float *mine = partials + ((size_t)bg * nsplit + split) * pstride;
  for (int i = tid; i < G * D; i += NT) {
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
      coherent_store(&mine[h * (D + 2) + e], a);
      if (e == 0) {
        coherent_store(&mine[h * (D + 2) + D], mx);
        coherent_store(&mine[h * (D + 2) + D + 1], lsum);
      }
    }
  }
  if (nsplit == 1) return;
  if (!last_block_arrives(&counters[bg], nsplit, s_last)) return;
  const float *allp = partials + (size_t)bg * nsplit * pstride;
  // The first batch of share values is requested before (m, l) so that both
  // arrive in one memory round trip.
  float v[EPT][kMergeBatch];
  merge_load_batch<NT, G, D, EPT>(v, allp, pstride, 0, nsplit);
  for (int h = wave; h < G; h += NW) {
    const bool on = lane < nsplit;
    const float m = on ? coherent_load(&allp[lane * pstride + h * (D + 2) + D]) : -INFINITY;
    const float l = on ? coherent_load(&allp[lane * pstride + h * (D + 2) + D + 1]) : 0.f;
    const float mx = wave_max(m);
    const float sc = safe_scale(m, mx);
    const float lsum = wave_sum(l * sc);
    if (on) s_scale[lane][h] = sc;
    if (lane == 0) s_lsum[h] = lsum;
  }
  __syncthreads();
  float a[EPT];
#pragma unroll
  for (int k = 0; k < EPT; ++k) a[k] = 0.f;
  for (int sp0 = 0;;) {
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int h = ((tid + k * NT) / D) % G;
#pragma unroll
      for (int j = 0; j < kMergeBatch; ++j)
        if (sp0 + j < nsplit) a[k] += v[k][j] * s_scale[sp0 + j][h];
    }
    sp0 += kMergeBatch;
    if (sp0 >= nsplit) break;
    merge_load_batch<NT, G, D, EPT>(v, allp, pstride, sp0, nsplit);
  }
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int i = tid + k * NT;
    if (i < G * D) {
      const int h = i / D, e = i % D;
      const float lsum = s_lsum[h];
      out[((size_t)b * hq + g * G + h) * D + e] = lsum > 0.f ? a[k] / lsum : 0.f;
    }
  }
  if (tid == 0) __hip_atomic_store(&counters[bg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- bf16: MFMA q.k, VALU p.v -------------------------------------------------
constexpr int kAttendThreads = 512;
constexpr int kAttendWaves = kAttendThreads / 64;
constexpr int kAttendChunk = 32;  // rows per wave step: two 16-row MFMA tiles
constexpr int kAttendMfmaPiece = 1024;  // rows resolved per row-table pass

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8a_t __attribute__((ext_vector_type(8)));

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F> __device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Lane H of each 16-lane row, broadcast to the row.
template <int H> __device__ __forceinline__ float row_bcast(float v) {
  static_assert(H >= 0 && H < 16, "lane");
  return dpp_mov<kDppRowBcast0 + H>(v);
}

// One wave step's operands for 32 rows (two 16-row MFMA tiles). K fragments
// (A operand): lane holds row l%16 of a tile and head-dimension entries
// 32 s + 8 (l/16) .. +7 of k-step s. The score of row 16 t + 4 q + r (tile t)
// for query head c then sits in lane 16 q + c; V rows are dealt so that the
// 16-lane row q holds exactly rows {16 t + 4 q + r}: lane l loads, for
// i < VU, row 16 t + 4 q + r with k = 4 t + r = i RPL + sub (q = l/16,
// sub = (l%16) / LPR), elements 8 (l % LPR) .. +7. A probability then
// reaches its V lanes by a broadcast within the 16-lane row.
template <int D> struct AttendChunk {
  static constexpr int KS = D / 32;
  static constexpr int LPR = D / 8;     // lanes per V row
  static constexpr int RPL = 16 / LPR;  // V rows per 16-lane row and instruction
  static constexpr int VU = 8 / RPL;    // V loads per lane
  bf16x8a_t kf[2][KS];
  uint4 vv[VU];
};

// A wave's p.v sums, relative to m_run.
// D = 128 (kMfma): the products run on MFMA. For D = 128 a lane's V loads are
// eight rows (the k-slots of its 16-lane row q = l/16, in load order) times
// elements 8 (l%16) .. +7, which is the A operand of 16x16x32 tile j (M = the
// elements 8 m + j, K = the 32 rows) once transposed in registers; the
// probabilities of the same rows for head l%16 are already the B operand.
// t[j] then holds, in lane l, element 8 (4 q + r) + j (entry r) for head l%16.
// Other D: VALU sums a[h][e] of this lane's eight V elements per head h.
template <int D, int G> struct AttendAcc {
  static constexpr bool kMfma = D == 128;
  f32x4_t t[kMfma ? 8 : 1];
  float a[kMfma ? 1 : G][8];
};

// A row-table entry r >= 0 is row r of kbase / vbase; with BUF (the pool keeps
// an HBM copy of its local buffer) r < 0 is slot ~r of that copy (kbuf / vbuf).
template <int D, bool BUF>
__device__ __forceinline__ const uint16_t *attend_row_ptr(const uint16_t *base,
                                                          const uint16_t *buf, int r) {
  if constexpr (BUF) return r >= 0 ? base + (size_t)r * D : buf + (size_t)(~r) * D;
  return base + (size_t)r * D;
}

template <int D, bool BUF>
__device__ __forceinline__ void attend_chunk_load(AttendChunk<D> &c, const int *s_rowtab, int it,
                                                  int plen, const uint16_t *kbase,
                                                  const uint16_t *vbase, const uint16_t *kbuf,
                                                  const uint16_t *vbuf, int lane) {
  using C = AttendChunk<D>;
  const int col = lane & 15, quad = lane >> 4;
  const int vpart = lane % C::LPR, sub = (lane & 15) / C::LPR;
#pragma unroll
  for (int tk = 0; tk < 2; ++tk) {
    const int li = it + tk * 16 + col;
    const uint16_t *kr = attend_row_ptr<D, BUF>(kbase, kbuf, li < plen ? s_rowtab[li] : 0);
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      c.kf[tk][s] = __builtin_bit_cast(
          bf16x8a_t, *reinterpret_cast<const uint4 *>(kr + 32 * s + 8 * quad));
  }
#pragma unroll
  for (int i = 0; i < C::VU; ++i) {
    const int k = i * C::RPL + sub;
    const int li = it + 16 * (k >> 2) + 4 * quad + (k & 3);
    const uint16_t *vr = attend_row_ptr<D, BUF>(vbase, vbuf, li < plen ? s_rowtab[li] : 0);
    c.vv[i] = *reinterpret_cast<const uint4 *>(vr + 8 * vpart);
  }
}

// Rows rbase + position of a contiguous row range (clamped to rmax), in the
// lane layout of attend_chunk_load: needs no row table, so it can be issued
// before the range's length is known.
template <int D>
__device__ __forceinline__ void attend_chunk_load_direct(AttendChunk<D> &c, int rbase, int rmax,
                                                         const uint16_t *kbase,
                                                         const uint16_t *vbase, int lane) {
  using C = AttendChunk<D>;
  const int col = lane & 15, quad = lane >> 4;
  const int vpart = lane % C::LPR, sub = (lane & 15) / C::LPR;
#pragma unroll
  for (int tk = 0; tk < 2; ++tk) {
    const uint16_t *kr = kbase + (size_t)min(rbase + tk * 16 + col, rmax) * D;
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      c.kf[tk][s] = __builtin_bit_cast(
          bf16x8a_t, *reinterpret_cast<const uint4 *>(kr + 32 * s + 8 * quad));
  }
#pragma unroll
  for (int i = 0; i < C::VU; ++i) {
    const int k = i * C::RPL + sub;
    const uint16_t *vr = vbase + (size_t)min(rbase + 16 * (k >> 2) + 4 * quad + (k & 3), rmax) * D;
    c.vv[i] = *reinterpret_cast<const uint4 *>(vr + 8 * vpart);
  }
}

// A chunk's valid rows (positions it .. it + 31 below plen of the piece that
// starts at position p0) stored from the registers they were loaded into to
// rows p0 + position of a working set (wk, wv: its K and V of (b, g)): the
// inverse of attend_chunk_load's lane layout, so each row is written whole,
// once.
template <int D>
__device__ __forceinline__ void attend_chunk_store(const AttendChunk<D> &c, int it, int plen,
                                                   int p0, uint16_t *wk, uint16_t *wv, int lane) {
  using C = AttendChunk<D>;
  const int col = lane & 15, quad = lane >> 4;
  const int vpart = lane % C::LPR, sub = (lane & 15) / C::LPR;
#pragma unroll
  for (int tk = 0; tk < 2; ++tk) {
    const int li = it + tk * 16 + col;
    if (li < plen) {
      uint16_t *kr = wk + (size_t)(p0 + li) * D;
#pragma unroll
      for (int s = 0; s < C::KS; ++s)
        *reinterpret_cast<uint4 *>(kr + 32 * s + 8 * quad) = __builtin_bit_cast(uint4, c.kf[tk][s]);
    }
  }
#pragma unroll
  for (int i = 0; i < C::VU; ++i) {
    const int k = i * C::RPL + sub;
    const int li = it + 16 * (k >> 2) + 4 * quad + (k & 3);
    if (li < plen) *reinterpret_cast<uint4 *>(wv + (size_t)(p0 + li) * D + 8 * vpart) = c.vv[i];
  }
}

// Working-set mode of the attention (fetch fused in): flag null = off.
struct AttendFetch {
  const uint8_t *flag;  // [batch]: 1 = retrieval step (fetch), 0 = read the working set
  void *k, *v;          // working set [BH][cap][D]
  int cap;
  int32_t *spans;       // [BH][2]
  int32_t *count;       // [BH]
  int reread;           // retrieval step: 1 = attend the working set once the copy has
                        // landed (pool rows behind the host link), 0 = attend the pool
                        // rows the copy has just read (pool in device memory)
};

// One whole decode step in the attention launch (kv_decode_step): the
// boundary test and, on a retrieval step, the scoring and the selection run
// inside it; otherwise as working-set mode. Null q_prev: first step.
struct DecodeStep {
  const uint16_t *q_prev;
  float tau;
  int budget;
  int group;
  uint8_t *flag;           // [batch] out
  float *r;                // [batch] out, or null
  int32_t *sel_units;      // [BH][sel_cap] out on retrieval steps
  int32_t *sel_n;          // [BH]
  int32_t *sel_rows;       // [BH]
  int32_t *sel_spans;      // [BH][sel_cap][2]
  int sel_cap;
  float *scores;           // [BH][unit_cap] scratch
  int32_t *sel_counters;   // [BH] scoring arrivals; zero between calls
  int32_t *gen;            // [BH] selection generation; any start value
  int32_t *status;         // pool status word
};

// Bounded wait of a workgroup for the selection of its (b, g) (a spin that
// has not seen it after this many sleeps reports KV_ERR_HIP and goes on).
constexpr int kStepSpinLimit = 1 << 22;

// Retrieval step of kv_decode_step, run by all nsplit workgroups of (b, g):
// each scores its share of the units, the last one to finish selects (the
// same functions and arithmetic as k_select, so the same scores and the same
// set bit for bit), publishes the spans and the count with device-coherent
// stores, waits for their acknowledgements and bumps gen[bg] (the completion
// protocol of last_block_arrives); the others wait for gen[bg] to move past
// the value they read at launch (gen0, thread 0 only) and then read the
// selection with device-coherent loads. The selecting workgroup is already
// running when the others wait, and it waits for nobody, so the wait always
// ends. hw / hc: LDS for the radix histograms.
template <int NT, int D, int KPT>
__device__ void step_select(const kv_pool &pool, const DecodeStep &st,
                            const uint16_t *__restrict__ q, int hq, int b, int g, int bg,
                            int split, int nsplit, int gen0, int (*hw)[256], int (*hc)[256],
                            int *s_last) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int U = min(max(pool.n_cand[b], 0), pool.unit_cap);
  uint4 qv[8];
  score_query_load<uint16_t, D>(q, hq, b, g, st.group, lane, qv);
  float qs[8];
  score_query_sum<uint16_t, D>(qv, st.group, qs);
  const uint16_t *idx = static_cast<const uint16_t *>(pool.unit_index) + (size_t)bg * pool.unit_cap * D;
  float *sc = st.scores + (size_t)bg * pool.unit_cap;
  const int ups = ((pool.unit_cap + nsplit - 1) / nsplit + 63) / 64 * 64;  // units per workgroup
  const int u_hi = min(U, (split + 1) * ups);
  for (int u0 = split * ups + wave * 64; u0 < u_hi; u0 += NW * 64)
    score_units64<uint16_t, D>(idx, sc, qs, u0, u_hi, lane);
  int sz[KPT], ust[KPT];
  select_sizes<KPT>(pool, bg, U, sz, ust);
  if (last_block_arrives(&st.sel_counters[bg], nsplit, s_last)) {
    select_prefix_block<NT, KPT, true>(pool, bg, st.budget, sc, sz, ust, st.sel_units, st.sel_cap,
                                       st.sel_n, st.sel_rows, st.sel_spans, hw, hc);
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's coherent stores are acknowledged
    __syncthreads();
    if (tid == 0) {
      __hip_atomic_store(&st.sel_counters[bg], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&st.gen[bg], gen0 + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  } else if (tid == 0) {
    int spins = 0;
    while (__hip_atomic_load(&st.gen[bg], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen0) {
      __builtin_amdgcn_s_sleep(2);
      if (++spins >= kStepSpinLimit) {
        __hip_atomic_store(st.status, (int)KV_ERR_HIP, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}

// Rows [r_lo, r_hi) of the concatenated selection (n units, r_sel rows, in
// s_psum / s_start) from the pool to the same positions of the working set,
// kCopyUnroll 16-byte pieces in flight per thread, in passes of
// kAttendMfmaPiece rows through the row table. Ends with a barrier.
constexpr int kCopyUnroll = 8;

template <int NT, int D>
__device__ void attend_copy_rows(const kv_pool &pool, int bg, const AttendFetch &fx, int r_lo,
                                 int r_hi, int n, int r_sel, const int *s_psum,
                                 const int *s_start, int *s_rowtab) {
  constexpr int LPR = D / 8;  // 16-byte pieces per bf16 row
  const int tid = threadIdx.x;
  const uint4 *ks = static_cast<const uint4 *>(pool.k) + (size_t)bg * pool.row_cap * LPR;
  const uint4 *vs = static_cast<const uint4 *>(pool.v) + (size_t)bg * pool.row_cap * LPR;
  uint4 *kd = static_cast<uint4 *>(fx.k) + (size_t)bg * fx.cap * LPR;
  uint4 *vd = static_cast<uint4 *>(fx.v) + (size_t)bg * fx.cap * LPR;
  for (int p0 = r_lo; p0 < r_hi; p0 += kAttendMfmaPiece) {
    const int plen = min(kAttendMfmaPiece, r_hi - p0);
    __syncthreads();  // the previous pass is done with the row table
    for (int i = tid; i < plen; i += NT)
      s_rowtab[i] = attend_row_of(p0 + i, n, r_sel, 0, s_psum, s_start, pool.row_cap);
    __syncthreads();
    const int pieces = plen * LPR;  // of K, and as many of V
    for (int base = 0; base < 2 * pieces; base += NT * kCopyUnroll) {
      u32x4_t buf[kCopyUnroll];
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) {
        int p = base + tid + u * NT;
        p = p < 2 * pieces ? p : 0;
        const bool is_v = p >= pieces;
        const int q = is_v ? p - pieces : p;
        const u32x4_t *src = reinterpret_cast<const u32x4_t *>(is_v ? vs : ks);
        buf[u] = src[(size_t)s_rowtab[q / LPR] * LPR + q % LPR];
      }
#pragma unroll
      for (int u = 0; u < kCopyUnroll; ++u) {
        const int p = base + tid + u * NT;
        u32x4_t *d = reinterpret_cast<u32x4_t *>(p < pieces ? kd + (size_t)p0 * LPR + p
                                                            : vd + (size_t)p0 * LPR + (p - pieces));
        if (p < 2 * pieces) *d = buf[u];
      }
    }
  }
  __syncthreads();
}

// Fold one chunk into the wave's online-softmax state (m_run, l_run per
// query head `col`, identical in the four lanes col + 16 q; acc as described
// at AttendAcc). VALU path: probabilities and the rescale factor move to the V
// lanes by row broadcasts, no LDS round trip. MFMA path: each probability is
// split into two bf16 parts (hi = RNE(p), lo = RNE(p - hi)), so the products
// carry about 16 significant bits of p, and both parts go through the tile.
template <int D, int G>
__device__ __forceinline__ void attend_chunk_fold(AttendChunk<D> &c, const bf16x8a_t *qf,
                                                  int it, int plen, float scale_log2,
                                                  float &m_run, float &l_run,
                                                  AttendAcc<D, G> &acc, int lane) {
  using C = AttendChunk<D>;
  const int quad = lane >> 4, sub = (lane & 15) / C::LPR;
  if (it + kAttendChunk > plen) {
    // rows past the piece: whatever was loaded for them, their p = 0 must
    // meet v = 0 so that they add exactly nothing
#pragma unroll
    for (int i = 0; i < C::VU; ++i) {
      const int k = i * C::RPL + sub;
      if (it + 16 * (k >> 2) + 4 * quad + (k & 3) >= plen) c.vv[i] = uint4{0u, 0u, 0u, 0u};
    }
  }
  f32x4_t sc[2];
#pragma unroll
  for (int tk = 0; tk < 2; ++tk) {
    sc[tk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      sc[tk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(c.kf[tk][s], qf[s], sc[tk], 0, 0, 0);
  }
  float sv[8];
  float mt = -INFINITY;
#pragma unroll
  for (int tk = 0; tk < 2; ++tk)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int li = it + tk * 16 + 4 * quad + r;
      const float v = li < plen ? sc[tk][r] * scale_log2 : -INFINITY;
      sv[tk * 4 + r] = v;
      mt = fmaxf(mt, v);
    }
  mt = max_xor32(max_xor16(mt));  // over the four lanes of query head `col`
  const float m_new = fmaxf(m_run, mt);
  const float alpha = safe_scale(m_run, m_new);
  float p[8];
  float ps = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    p[k] = sv[k] == -INFINITY ? 0.f : exp2f(sv[k] - m_new);
    ps += p[k];
  }
  ps = sum_xor32(sum_xor16(ps));
  l_run = l_run * alpha + ps;
  m_run = m_new;
  if constexpr (AttendAcc<D, G>::kMfma) {
    // this lane's head is col = l%16, so alpha needs no broadcast
#pragma unroll
    for (int j = 0; j < 8; ++j) acc.t[j] *= alpha;
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    u32x4_t ph, pl;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x2_t pp = {p[2 * k], p[2 * k + 1]};
      const bf16x2_t h = __builtin_convertvector(pp, bf16x2_t);
      const bf16x2_t l = __builtin_convertvector(pp - __builtin_convertvector(h, f32x2_t), bf16x2_t);
      ph[k] = __builtin_bit_cast(uint32_t, h);
      pl[k] = __builtin_bit_cast(uint32_t, l);
    }
    const bf16x8a_t bh = __builtin_bit_cast(bf16x8a_t, ph), bl = __builtin_bit_cast(bf16x8a_t, pl);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // A of tile j: element j of each of the eight rows, rows in k-slot order
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      u32x4_t a;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint4 lo = c.vv[2 * w], hi = c.vv[2 * w + 1];
        const uint32_t dl = (j >> 1) == 0 ? lo.x : (j >> 1) == 1 ? lo.y : (j >> 1) == 2 ? lo.z : lo.w;
        const uint32_t dh = (j >> 1) == 0 ? hi.x : (j >> 1) == 1 ? hi.y : (j >> 1) == 2 ? hi.z : hi.w;
        a[w] = __builtin_amdgcn_perm(dh, dl, sel);
      }
      const bf16x8a_t av = __builtin_bit_cast(bf16x8a_t, a);
      acc.t[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bh, acc.t[j], 0, 0, 0);
      acc.t[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bl, acc.t[j], 0, 0, 0);
    }
  } else {
    static_for<G>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      const float al = row_bcast<h>(alpha);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc.a[h][e] *= al;
    });
#pragma unroll
    for (int i = 0; i < C::VU; ++i) {
      float vf[8];
      unpack16<uint16_t>(c.vv[i], vf);
      static_for<G>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        float pu;
        if constexpr (C::RPL == 1) {
          pu = row_bcast<h>(p[i]);
        } else {
          const float b0 = row_bcast<h>(p[i * C::RPL]), b1 = row_bcast<h>(p[i * C::RPL + 1]);
          pu = sub ? b1 : b0;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc.a[h][e] = fmaf(pu, vf[e], acc.a[h][e]);
      });
    }
  }
}

// The register budget at 8 waves per workgroup is 256 VGPRs: G = 8 (p.v
// accumulators) and G = 1 do not fit a second chunk in flight without
// spilling, so they fold one chunk at a time.
template <int G> constexpr bool kAttendPipelined = G == 2 || G == 4;

// Bytes of k_gather_attend_mfma's explicit arguments.
constexpr int kAttendArgBytes = 456;

// STEP_KPT > 0 (working-set mode, no local buffer): the whole decode step, see
// DecodeStep; the selection lists and flag of fx / sel_* are then outputs.
template <int D, int G, bool BUF, int STEP_KPT = 0, bool STEP_W47 = true>
__global__ void __launch_bounds__(kAttendThreads)
    k_gather_attend_mfma(const uint16_t *__restrict__ ws_k, const uint16_t *__restrict__ ws_v,
                         const uint16_t *__restrict__ q, const uint16_t *__restrict__ q_prev,
                         int geo, int rcap, int ws_cap, int hq,
                         const int32_t *__restrict__ ws_spans, const int32_t *__restrict__ ws_count,
                         kv_pool pool, float scale_log2,
                         const int32_t *__restrict__ sel_units,
                         const int32_t *__restrict__ sel_spans, int sel_cap,
                         const int32_t *__restrict__ sel_n, float *__restrict__ out,
                         float *__restrict__ partials, int32_t *counters, AttendFetch fx,
                         DecodeStep st = DecodeStep{}) {
  static_assert(G <= 16, "query columns of one MFMA tile");
  constexpr bool DSTEP = STEP_KPT > 0;
  // kv_decode_step: the rest of its arguments in one round trip, requested
  // now and waited for once the rows and the boundary test's loads are out
  KernargLines<kAttendArgBytes> kargs;
  if constexpr (DSTEP) kargs.issue();

  static_assert(!(DSTEP && BUF), "a decode step in one launch has no local buffer");
  constexpr int NT = kAttendThreads, NW = kAttendWaves;
  constexpr int KS = D / 32;
  constexpr int LPR = D / 8;
  constexpr int STEP = NW * kAttendChunk;
  __shared__ int s_psum[kMaxSel];
  __shared__ int s_start[kMaxSel];
  __shared__ int s_rowtab[kAttendMfmaPiece];
  __shared__ int s_wsum[NW];
  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ __align__(16) float s_acc[NW][G][D];
  __shared__ int s_last;

  const int H = geo & 0xffff;  // pool.n_kv_heads
  const int bg = blockIdx.y, b = bg / H, g = bg % H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nsplit = geo >> 16, split = blockIdx.x;  // nsplit == gridDim.x
  const int col = lane & 15, quad = lane >> 4;  // MFMA: column (query head) and k group
  const int vpart = lane % LPR;                   // V elements 8 vpart .. 8 vpart + 7

  // Query fragments (B operand, 32 k x 16 columns): lane holds column `col`
  // (query head col < G, else zero) and the same head-dimension entries as
  // the K fragments, so one K load instruction reads a contiguous 64-byte
  // span of each of 16 rows.
  // kv_decode_step: the boundary test runs on waves 4-7. When a workgroup's
  // chunk holds at most 128 rows (!STEP_W47) those waves request no rows, so
  // the test runs while waves 0-3 wait for theirs; otherwise its loads go
  // first and it waits with everything else.
  constexpr int BW0 = NW - 4;
  BoundaryFirst<uint16_t, D> bfirst;
  if constexpr (DSTEP && STEP_W47)
    if (q_prev != nullptr) boundary_prefetch<uint16_t, D, BW0>(q_prev, q, hq, b, bfirst);
  bf16x8a_t qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    uint4 v = {0u, 0u, 0u, 0u};
    if (col < G)
      v = *reinterpret_cast<const uint4 *>(q + ((size_t)b * hq + g * G + col) * D + 32 * s + 8 * quad);
    qf[s] = __builtin_bit_cast(bf16x8a_t, v);
  }

  // Rows come from the pool's selection, or (working-set mode on a step
  // without retrieval) from the working set's one span; on a retrieval step
  // of working-set mode they come from the pool and are stored to the
  // working set as they are loaded.
  // (always for kv_decode_step: a compile-time true keeps its span loads out of
  // a branch, whose merge would make the wave wait for them on the spot)
  const bool ws_mode = DSTEP || fx.flag != nullptr;
  // Working-set mode without a local buffer: the working set's rows are
  // contiguous from row 0 and this workgroup's chunk starts at
  // split * ceil(rcap / nsplit) whenever the span holds at most rcap rows, so
  // each wave requests its first 32 rows now, in the same memory round trip
  // as the flag and the span. A retrieval step (or any other span) discards
  // them and takes the general path.
  // The flag and the working set's one span (read as attend_load_selection
  // reads a one-entry list) are requested right behind the rows (and, in
  // kv_decode_step, the boundary test's loads); every value feeds the test
  // below, so none of the loads is deferred into a branch and all of them are
  // in flight at once. The rows and the test use only the leading, preloaded
  // kernel arguments, so they go out as the waves start.
  int ws_flag = 0, ws_cnt = 0;
  int2 ws_sp = {0, 0};
  int gen0 = 0;
  auto ws_loads = [&]() {
    if (ws_mode) {
      if (!DSTEP) ws_flag = fx.flag[b];
      if (!BUF) {
        // kv_decode_step: vector loads (see opaque_zero), so that the waits for
        // kernel arguments before the test and the rows do not wait for these
        const int z = DSTEP ? opaque_zero() : 0;
        ws_cnt = ws_count[bg + z];
        ws_sp = *reinterpret_cast<const int2 *>(ws_spans + 2 * (bg + z));
      }
    }
    if constexpr (DSTEP)
      if (tid == 0) gen0 = __hip_atomic_load(&st.gen[bg], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  AttendChunk<D> ca;
  const int spec_chunk = (max(rcap, 1) + nsplit - 1) / nsplit;
  const int spec_lo = split * spec_chunk;
  auto spec_rows = [&]() {
    if (!BUF && ws_mode && wave * kAttendChunk < spec_chunk)  // waves with rows in the chunk
      attend_chunk_load_direct<D>(
          ca, spec_lo + wave * kAttendChunk, ws_cap - 1, ws_k + (size_t)bg * ws_cap * D,
          ws_v + (size_t)bg * ws_cap * D, lane);
  };
  __shared__ float s_part[4];
  if constexpr (DSTEP && !STEP_W47) {
    if (wave >= BW0) {
      if (q_prev != nullptr) {
        boundary_prefetch<uint16_t, D, BW0>(q_prev, q, hq, b, bfirst);
        boundary_partial<uint16_t, D, BW0>(q_prev, q, hq, b, s_part, bfirst);
      }
    } else {
      spec_rows();
    }
  } else {
    spec_rows();
  }
  // the span and count need kernel arguments that are not preloaded: requested
  // after the rows and the boundary test's loads, which need only preloaded ones
  if constexpr (DSTEP) kargs.consume();
  ws_loads();
  if constexpr (DSTEP) {
    // the step's retrieval decision, taken here by every workgroup of the
    // sequence with the same function as k_boundary (so the same bits)
    float rv = __builtin_nanf("");
    ws_flag = 1;
    if (q_prev != nullptr) {
      if constexpr (!STEP_W47)
        rv = boundary_combine(s_part, hq);
      else
        rv = boundary_r_pre<uint16_t, D, BW0>(q_prev, q, hq, b, s_part, bfirst);
      ws_flag = rv < st.tau ? 1 : 0;
    }
    if (split == 0 && g == 0 && tid == 0) {
      st.flag[b] = (uint8_t)ws_flag;
      if (st.r) st.r[b] = rv;
    }
  }
  const int ws_n = min(max(ws_cnt, 0), 1);
  const int ws_size = max(ws_sp.y, 0) * ws_n, ws_start = ws_sp.x * ws_n;
  // uniform: a step without retrieval whose rows start at 0 and fit the bound,
  // i.e. `ca` holds this wave's first chunk
  const bool spec = !BUF && ws_mode && ws_flag == 0 && ws_start == 0 && ws_size <= rcap;
  const bool fetching = ws_mode && ws_flag != 0;  // uniform
  const bool from_ws = ws_mode && !fetching;
  int n, r_sel;
  if (!BUF && from_ws) {
    n = ws_n;
    r_sel = ws_size;
    if (tid == 0) {
      s_psum[0] = 0;
      s_start[0] = ws_start;
    }
    __syncthreads();
  } else {
    if constexpr (DSTEP) {
      // retrieval step: select now (the radix histograms borrow s_psum, free until
      // the selection is loaded into it below)
      int(*hw)[256] = reinterpret_cast<int(*)[256]>(s_psum);
      int(*hc)[256] = reinterpret_cast<int(*)[256]>(s_psum + NW * 256);
      static_assert(2 * NW * 256 <= kMaxSel, "histograms fit s_psum");
      step_select<NT, D, STEP_KPT>(pool, st, q, hq, b, g, bg, split, nsplit, gen0, hw, hc,
                                   &s_last);
    }
    const int scap = from_ws ? 1 : (DSTEP ? st.sel_cap : sel_cap);
    const int32_t *su = (from_ws || DSTEP) ? nullptr : sel_units;
    const int32_t *sp = from_ws ? fx.spans : (DSTEP ? st.sel_spans : sel_spans);
    r_sel = attend_load_selection<NT, DSTEP>(
        pool, bg, su ? su + (size_t)bg * scap : nullptr, sp ? sp + (size_t)bg * scap * 2 : nullptr,
        from_ws ? fx.count : (DSTEP ? st.sel_n : sel_n), scap, &n, s_psum, s_start, s_wsum);
  }
  const int r_all = r_sel;
  if (fetching) r_sel = min(r_sel, fx.cap);
  int r_buf = 0, buf_begin = 0;
  if (pool.buf_cap > 0) {
    buf_begin = pool.buf_begin[b];
    r_buf = max(pool.n_rows[b] - buf_begin, 0);
  }
  const int R = r_sel + r_buf;
  const int chunk = (max(R, rcap) + nsplit - 1) / nsplit;
  const int r_lo = min(R, split * chunk), r_hi = min(R, r_lo + chunk);

  // Retrieval step of working-set mode: the rows this workgroup attends,
  // [r_lo, r_hi) of the selection, also go to the same positions of the
  // working set. Without a local buffer each chunk is stored from the
  // registers the attention loads it into (every row crosses the host link,
  // for a pool in host memory, once); with one, a copy pass runs first and
  // the attention reads the pool rows it has brought into L2 (device memory)
  // or the working set (host memory).
  const bool store_ws = !BUF && fetching;  // uniform
  if (fetching) {
    if (split == 0 && tid == 0) {
      fx.spans[2 * bg] = 0;
      fx.spans[2 * bg + 1] = r_sel;
      fx.count[bg] = r_sel > 0 ? 1 : 0;
      if (r_all > fx.cap)
        __hip_atomic_store(pool.status, (int)KV_ERR_CAPACITY, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!store_ws)
      attend_copy_rows<NT, D>(pool, bg, fx, min(r_lo, r_sel), min(r_hi, r_sel), n, r_sel, s_psum,
                              s_start, s_rowtab);
    if (!store_ws && fx.reread) {
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the copies are written
      __syncthreads();
      if (tid == 0) {  // the selection is now the working set's one span
        s_start[0] = 0;
        s_psum[0] = 0;
      }
      n = 1;
      __syncthreads();
    }
  }
  const bool read_ws = ws_mode && (!fetching || (!store_ws && fx.reread));
  const int row_cap = read_ws ? fx.cap : pool.row_cap;
  uint16_t *wsk = nullptr, *wsv = nullptr;
  if (store_ws) {
    wsk = static_cast<uint16_t *>(fx.k) + (size_t)bg * fx.cap * D;
    wsv = static_cast<uint16_t *>(fx.v) + (size_t)bg * fx.cap * D;
  }

  // Online softmax state. m_run / l_run: per query head `col`, identical in
  // the four lanes col, col+16, col+32, col+48. acc: p.v partial sums of this
  // lane's V rows, elements 8 vpart .. 8 vpart + 7, relative to m_run.
  float m_run = -INFINITY, l_run = 0.f;
  AttendAcc<D, G> acc;
  if constexpr (AttendAcc<D, G>::kMfma) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc.t[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc.a[h][e] = 0.f;
  }

  const uint16_t *kbase =
      static_cast<const uint16_t *>(read_ws ? fx.k : pool.k) + (size_t)bg * row_cap * D;
  const uint16_t *vbase =
      static_cast<const uint16_t *>(read_ws ? fx.v : pool.v) + (size_t)bg * row_cap * D;
  const int ring = BUF ? pool.buf_ring : 0;
  const uint16_t *kbuf = nullptr, *vbuf = nullptr;
  if (BUF) {
    kbuf = static_cast<const uint16_t *>(pool.buf_k) + (size_t)bg * ring * D;
    vbuf = static_cast<const uint16_t *>(pool.buf_v) + (size_t)bg * ring * D;
  }

  // In the speculative case the rows are p0 + position (what the row table
  // would hold), read straight from the working set.
  bool preloaded = spec;
  for (int p0 = r_lo; p0 < r_hi; p0 += kAttendMfmaPiece) {
    const int plen = min(kAttendMfmaPiece, r_hi - p0);
    if (!spec) {
      for (int i = tid; i < plen; i += NT)
        s_rowtab[i] = attend_row_of(p0 + i, n, r_sel, buf_begin, s_psum, s_start, row_cap, ring);
      __syncthreads();
    }
    auto load = [&](AttendChunk<D> &c, int pos) {
      if (spec)
        attend_chunk_load_direct<D>(c, p0 + pos, row_cap - 1, kbase, vbase, lane);
      else
        attend_chunk_load<D, BUF>(c, s_rowtab, pos, plen, kbase, vbase, kbuf, vbuf, lane);
    };
    int it = wave * kAttendChunk;
    if constexpr (kAttendPipelined<G>) {
      // Two register sets: the next step's loads are in flight while this
      // step's scores and p.v run.
      AttendChunk<D> cb;
      if (it < plen && !preloaded) load(ca, it);
      while (it < plen) {
        if (it + STEP < plen) load(cb, it + STEP);
        if (store_ws) attend_chunk_store<D>(ca, it, plen, p0, wsk, wsv, lane);
        attend_chunk_fold<D, G>(ca, qf, it, plen, scale_log2, m_run, l_run, acc, lane);
        it += STEP;
        if (it >= plen) break;
        if (it + STEP < plen) load(ca, it + STEP);
        if (store_ws) attend_chunk_store<D>(cb, it, plen, p0, wsk, wsv, lane);
        attend_chunk_fold<D, G>(cb, qf, it, plen, scale_log2, m_run, l_run, acc, lane);
        it += STEP;
      }
    } else {
      for (; it < plen; it += STEP) {
        if (!preloaded) load(ca, it);
        preloaded = false;
        if (store_ws) attend_chunk_store<D>(ca, it, plen, p0, wsk, wsv, lane);
        attend_chunk_fold<D, G>(ca, qf, it, plen, scale_log2, m_run, l_run, acc, lane);
      }
    }
    preloaded = false;
    __syncthreads();
  }

  if constexpr (AttendAcc<D, G>::kMfma) {
    // the tiles already summed over the wave's rows
    if (col < G) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float *dst = &s_acc[wave][col][8 * (4 * quad + r)];
        *reinterpret_cast<float4 *>(dst) = float4{acc.t[0][r], acc.t[1][r], acc.t[2][r], acc.t[3][r]};
        *reinterpret_cast<float4 *>(dst + 4) =
            float4{acc.t[4][r], acc.t[5][r], acc.t[6][r], acc.t[7][r]};
      }
    }
  } else {
    // rows of one wave share m_run: lane groups combine by plain sums
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc.a[h][e] = sum_stride<LPR>(acc.a[h][e]);
    if (lane < LPR) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) s_acc[wave][h][8 * vpart + e] = acc.a[h][e];
    }
  }
  if (lane < G) {
    s_m[wave][lane] = m_run;
    s_l[wave][lane] = l_run;
  }
  __syncthreads();
  attend_finish<NT, G, D>(bg, b, g, hq, nsplit, split, s_m, s_l, s_acc, out, partials, counters,
                          &s_last);
}

// ---- fp32: all-VALU variant ------------------------------------------------------
constexpr int kAttendValuThreads = 512;

template <typename T, int D, int G>
__global__ void __launch_bounds__(kAttendValuThreads)
    k_gather_attend_valu(kv_pool pool, const T *__restrict__ q, int hq, float scale_log2,
                         const int32_t *__restrict__ sel_units,
                         const int32_t *__restrict__ sel_spans, int sel_cap,
                         const int32_t *__restrict__ sel_n, int rcap, float *__restrict__ out,
                         float *__restrict__ partials, int32_t *counters) {
  constexpr int NT = kAttendValuThreads, NW = NT / 64;
  constexpr int EPL = 16 / Elem<T>::kBytes;  // elements per lane (one 16-byte load)
  constexpr int LPR = D / EPL;               // lanes per row
  constexpr int RPI = 64 / LPR;              // rows per wave instruction
  constexpr int UNR = (G >= 4 ? 4 : 8);       // row pieces in flight per lane group
  __shared__ int s_psum[kMaxSel];
  __shared__ int s_start[kMaxSel];
  __shared__ int s_rowtab[NT];
  __shared__ int s_wsum[NW];
  __shared__ float s_m[NW][G], s_l[NW][G];
  __shared__ float s_acc[NW][G][D];
  __shared__ int s_last;

  const int H = pool.n_kv_heads;
  const int bg = blockIdx.y, b = bg / H, g = bg % H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int part = lane % LPR, slot = lane / LPR;
  const int nsplit = gridDim.x, split = blockIdx.x;

  float qf[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 v =
        *reinterpret_cast<const uint4 *>(q + ((size_t)b * hq + g * G + h) * D + part * EPL);
    unpack16<T>(v, qf[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[h][e] *= scale_log2;
  }
  int n;
  const int r_sel = attend_load_selection<NT>(
      pool, bg, sel_units ? sel_units + (size_t)bg * sel_cap : nullptr,
      sel_spans ? sel_spans + (size_t)bg * sel_cap * 2 : nullptr, sel_n, sel_cap, &n, s_psum,
      s_start, s_wsum);
  int r_buf = 0, buf_begin = 0;
  if (pool.buf_cap > 0) {
    buf_begin = pool.buf_begin[b];
    r_buf = max(pool.n_rows[b] - buf_begin, 0);
  }
  const int R = r_sel + r_buf;
  const int chunk = (max(R, rcap) + nsplit - 1) / nsplit;
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
  const int ring = pool.buf_k != nullptr ? pool.buf_ring : 0;
  const T *kbuf = kbase, *vbuf = vbase;  // local buffer's HBM copy (slots ~r of negative rows)
  if (ring > 0) {
    kbuf = static_cast<const T *>(pool.buf_k) + (size_t)bg * ring * D + part * EPL;
    vbuf = static_cast<const T *>(pool.buf_v) + (size_t)bg * ring * D + part * EPL;
  }

  for (int p0 = r_lo; p0 < r_hi; p0 += NT) {
    const int plen = min(NT, r_hi - p0);
    if (tid < plen)
      s_rowtab[tid] =
          attend_row_of(p0 + tid, n, r_sel, buf_begin, s_psum, s_start, pool.row_cap, ring);
    __syncthreads();
    for (int it = wave * UNR * RPI; it < plen; it += NW * UNR * RPI) {
      uint4 kv[UNR], vv[UNR];
      bool ok[UNR];
#pragma unroll
      for (int uu = 0; uu < UNR; ++uu) {
        const int li = it + uu * RPI + slot;
        ok[uu] = li < plen;
        const int r = ok[uu] ? s_rowtab[li] : 0;
        kv[uu] = *reinterpret_cast<const uint4 *>(r >= 0 ? kbase + (size_t)r * D
                                                         : kbuf + (size_t)(~r) * D);
        vv[uu] = *reinterpret_cast<const uint4 *>(r >= 0 ? vbase + (size_t)r * D
                                                         : vbuf + (size_t)(~r) * D);
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
          d0 = group_sum<LPR>(d0);
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
  attend_finish<NT, G, D>(bg, b, g, hq, nsplit, split, s_m, s_l, s_acc, out, partials, counters,
                          &s_last);
}

// Attended rows a call expects per (b, g) at most: max_rows selected rows
// plus a full local buffer. Rows are dealt to workgroups in chunks of
// ceil(max(R, bound) / nsplit), so calls with equal max_rows split equal rows
// identically, and a chunk's first row is known before R is.
int attend_row_bound(const kv_pool *pool, int max_rows) {
  return (max_rows > 0 ? max_rows : 0) + (pool->buf_cap > 0 ? pool->buf_cap : 0);
}

int attend_num_splits(const kv_pool *pool, int max_rows) {
  const long rows = attend_row_bound(pool, max_rows);
  const long bh = (long)pool->batch * pool->n_kv_heads;
  long by_rows = (rows + kAttendMinRowsPerSplit - 1) / kAttendMinRowsPerSplit;
  long by_grid = (kAttendTargetBlocks + bh - 1) / bh;
  long ns = by_rows < by_grid ? by_rows : by_grid;
  if (ns < 1) ns = 1;
  // at most one batch of shares for the merging workgroup (a second batch is
  // one more dependent round trip, which costs more than the split saves)
  if (ns > kMergeBatch) ns = kMergeBatch;
  return (int)ns;
}

// Kernel argument `geo` of k_gather_attend_mfma: n_kv_heads | nsplit << 16.
static int attend_geo(const kv_pool *pool, int nsplit) {
  return (pool->n_kv_heads & 0xffff) | (nsplit << 16);
}

template <typename T, int D>
static kv_status attend_dispatch(const kv_pool *pool, const void *q, int hq, float scale_log2,
                                 const int32_t *sel_units, const int32_t *sel_spans,
                                 int sel_cap, const int32_t *sel_n, int nsplit, int rcap,
                                 float *out, float *partials, int32_t *counters,
                                 const AttendFetch &fx, hipStream_t s) {
  const int G = hq / pool->n_kv_heads;
  const dim3 grid(nsplit, pool->batch * pool->n_kv_heads);
  const int geo = attend_geo(pool, nsplit);
  if (sizeof(T) != 2 && fx.flag != nullptr) return KV_ERR_UNSUPPORTED;
#define KVC_ATT(GG)                                                                           \
  do {                                                                                        \
    if constexpr (sizeof(T) == 2)                                                             \
      if (pool->buf_k != nullptr)                                                             \
        k_gather_attend_mfma<D, GG, true><<<grid, kAttendThreads, 0, s>>>(                    \
            (const uint16_t *)fx.k, (const uint16_t *)fx.v, (const uint16_t *)q, nullptr, geo,  \
            rcap, fx.cap, hq, fx.spans, fx.count, *pool, scale_log2, sel_units, sel_spans,      \
            sel_cap, sel_n, out, partials, counters, fx);                                     \
      else                                                                                    \
        k_gather_attend_mfma<D, GG, false><<<grid, kAttendThreads, 0, s>>>(                   \
            (const uint16_t *)fx.k, (const uint16_t *)fx.v, (const uint16_t *)q, nullptr, geo,  \
            rcap, fx.cap, hq, fx.spans, fx.count, *pool, scale_log2, sel_units, sel_spans,      \
            sel_cap, sel_n, out, partials, counters, fx);                                     \
    else                                                                                      \
      k_gather_attend_valu<T, D, GG><<<grid, kAttendValuThreads, 0, s>>>(                     \
          *pool, (const T *)q, hq, scale_log2, sel_units, sel_spans, sel_cap, sel_n, rcap,    \
          out, partials, counters);                                                           \
  } while (0)
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

static kv_status attend_launch(const kv_pool *pool, const void *q, int hq, float scale,
                               const int32_t *sel_units, const int32_t *sel_spans, int sel_cap,
                               const int32_t *sel_n, int nsplit, int rcap, float *out,
                               float *partials, int32_t *counters, const AttendFetch &fx,
                               hipStream_t s) {
  const float sl2 = scale * 1.4426950408889634f;  // log2(e): exp(x) = exp2(x log2 e)
#define KVC_AD(T, D)                                                                          \
  attend_dispatch<T, D>(pool, q, hq, sl2, sel_units, sel_spans, sel_cap, sel_n, nsplit, rcap, \
                        out, partials, counters, fx, s)
  kv_status st;
  if (pool->dtype == KV_BF16)
    st = pool->head_dim == 128 ? KVC_AD(uint16_t, 128) : KVC_AD(uint16_t, 64);
  else
    st = pool->head_dim == 128 ? KVC_AD(float, 128) : KVC_AD(float, 64);
#undef KVC_AD
  return st;
}

kv_status launch_gather_attend(const kv_pool *pool, const void *q, int hq, float scale,
                               const int32_t *sel_units, const int32_t *sel_spans, int sel_cap,
                               const int32_t *sel_n, int nsplit, int rcap, float *out,
                               float *partials, int32_t *counters, hipStream_t s) {
  const AttendFetch off{};
  return attend_launch(pool, q, hq, scale, sel_units, sel_spans, sel_cap, sel_n, nsplit, rcap, out,
                       partials, counters, off, s);
}


// ---------------------------------------------------------------- working-set fetch
// Rows of the selected units -> a device-resident working set, stored one
// after another in selection order, so that attention over the working set
// sees the same rows in the same order as attention over the pool. One (b, g)
// per blockIdx.y; blockIdx.x takes a range of RPB rows of the concatenated
// selection, so that a workgroup moves exactly kFetchBlockBytes (its K and V
// pieces) with every thread holding kFetchUnroll 16-byte reads in flight
// before it stores. Sequences whose flag is 0 return at once and keep the
// previous working set. The source pool may live in host memory mapped into
// the device's address space: then every piece is a read over the host link,
// and keeping many in flight is what sets the rate.
constexpr int kFetchThreads = 256;
constexpr int kFetchUnroll = 8;
constexpr int kFetchBlockBytes = kFetchThreads * kFetchUnroll * 16;

template <int RB>
__global__ void __launch_bounds__(kFetchThreads)
k_fetch_rows(kv_pool src, const uint8_t *__restrict__ flag, const int32_t *sel_units,
             const int32_t *sel_spans, int sel_cap, const int32_t *__restrict__ sel_n,
             kv_pool dst, int32_t *__restrict__ dst_spans, int32_t *__restrict__ dst_n) {
  constexpr int NT = kFetchThreads;
  constexpr int LPR = RB / 16;                        // 16-byte pieces per row
  constexpr int RPB = kFetchBlockBytes / (2 * RB);    // rows per workgroup
  static_assert(RPB * LPR * 2 == NT * kFetchUnroll, "one pass per workgroup");
  __shared__ int s_psum[kMaxSel];
  __shared__ int s_start[kMaxSel];
  __shared__ int s_wsum[NT / 64];
  __shared__ int s_row[RPB];
  const int tid = threadIdx.x;
  const int bg = blockIdx.y, b = bg / src.n_kv_heads;
  if (flag[b] == 0) return;  // uniform over the workgroup
  int n;
  const int r_all = attend_load_selection<NT>(
      src, bg, sel_units ? sel_units + (size_t)bg * sel_cap : nullptr,
      sel_spans ? sel_spans + (size_t)bg * sel_cap * 2 : nullptr, sel_n, sel_cap, &n, s_psum,
      s_start, s_wsum);
  const int R = min(r_all, dst.row_cap);
  if (blockIdx.x == 0 && tid == 0) {
    dst_spans[2 * bg] = 0;
    dst_spans[2 * bg + 1] = R;
    dst_n[bg] = R > 0 ? 1 : 0;
    if (r_all > dst.row_cap)
      __hip_atomic_store(src.status, (int)KV_ERR_CAPACITY, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  const int r_lo = blockIdx.x * RPB;
  if (r_lo >= R) return;  // uniform
  const int rows = min(RPB, R - r_lo);
  for (int i = tid; i < rows; i += NT)
    s_row[i] = attend_row_of(r_lo + i, n, r_all, 0, s_psum, s_start, src.row_cap);
  __syncthreads();
  const size_t src_head = (size_t)bg * src.row_cap * LPR;
  const size_t dst_head = ((size_t)bg * dst.row_cap + r_lo) * LPR;
  const u32x4_t *ks = static_cast<const u32x4_t *>(src.k) + src_head;
  const u32x4_t *vs = static_cast<const u32x4_t *>(src.v) + src_head;
  u32x4_t *kd = static_cast<u32x4_t *>(dst.k) + dst_head;
  u32x4_t *vd = static_cast<u32x4_t *>(dst.v) + dst_head;
  const int pieces = rows * LPR;  // of K, and as many of V
  // piece p < pieces: K piece p; else V piece p - pieces. Pieces past the
  // end re-read the block's first piece (in bounds) and are not stored.
  u32x4_t buf[kFetchUnroll];
#pragma unroll
  for (int u = 0; u < kFetchUnroll; ++u) {
    int p = tid + u * NT;
    p = p < 2 * pieces ? p : 0;
    const bool is_v = p >= pieces;
    const int q = is_v ? p - pieces : p;
    buf[u] = (is_v ? vs : ks)[(size_t)s_row[q / LPR] * LPR + q % LPR];
  }
#pragma unroll
  for (int u = 0; u < kFetchUnroll; ++u) {
    const int p = tid + u * NT;
    u32x4_t *d = p < pieces ? kd + p : vd + (p - pieces);
    if (p < 2 * pieces) *d = buf[u];
  }
}

int fetch_num_blocks(const kv_pool *dst) {
  const int rb = dst->head_dim * (dst->dtype == KV_BF16 ? 2 : 4);
  const int rpb = kFetchBlockBytes / (2 * rb);
  return (dst->row_cap + rpb - 1) / rpb;
}

kv_status launch_fetch_rows(const kv_pool *src, const uint8_t *flag, const int32_t *sel_units,
                            const int32_t *sel_spans, int sel_cap, const int32_t *sel_n,
                            const kv_pool *dst, int32_t *dst_spans, int32_t *dst_n,
                            hipStream_t s) {
  const dim3 grid(fetch_num_blocks(dst), src->batch * src->n_kv_heads);
  const int rb = src->head_dim * (src->dtype == KV_BF16 ? 2 : 4);
#define KVC_FETCH(RB)                                                                          \
  k_fetch_rows<RB><<<grid, kFetchThreads, 0, s>>>(*src, flag, sel_units, sel_spans, sel_cap,  \
                                                  sel_n, *dst, dst_spans, dst_n)
  switch (rb) {
    case 128: KVC_FETCH(128); break;
    case 256: KVC_FETCH(256); break;
    case 512: KVC_FETCH(512); break;
    default: return KV_ERR_UNSUPPORTED;
  }
#undef KVC_FETCH
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

// Working-set fetch and attention in one launch (bf16): on a retrieval step
// every attention workgroup stores the rows it loads from the pool into the
// working set; otherwise it reads them from there. fp32 pools run the two
// launches kv_fetch_selected and kv_gather_attend compose.
kv_status launch_fetch_attend(const kv_pool *pool, const void *q, int hq, float scale,
                              const uint8_t *flag, const int32_t *sel_units,
                              const int32_t *sel_spans, int sel_cap, const int32_t *sel_n,
                              int nsplit, int rcap, const kv_pool *dst, int32_t *dst_spans,
                              int32_t *dst_n, float *out, float *partials, int32_t *counters,
                              hipStream_t s) {
  if (pool->dtype != KV_BF16) {
    kv_status st = launch_fetch_rows(pool, flag, sel_units, sel_spans, sel_cap, sel_n, dst,
                                     dst_spans, dst_n, s);
    if (st != KV_OK) return st;
    return launch_gather_attend(dst, q, hq, scale, nullptr, dst_spans, 1, dst_n, nsplit, rcap,
                                out, partials, counters, s);
  }
  // Where the pool's rows live decides how a retrieval step reads them back.
  hipPointerAttribute_t attr;
  int reread = 1;
  if (hipPointerGetAttributes(&attr, pool->k) == hipSuccess)
    reread = attr.type == hipMemoryTypeDevice ? 0 : 1;
  else
    (void)hipGetLastError();
  AttendFetch fx{flag, dst->k, dst->v, dst->row_cap, dst_spans, dst_n, reread};
  return attend_launch(pool, q, hq, scale, sel_units, sel_spans, sel_cap, sel_n, nsplit, rcap, out,
                       partials, counters, fx, s);
}

// The whole decode step in one launch (bf16 pool without a local buffer):
// boundary test, on retrieval steps scoring + selection, working-set fetch
// and attention. The split over workgroups is kv_fetch_attend's for
// max_rows = budget, so the outputs equal kv_boundary_select followed by
// kv_fetch_attend bit for bit.
template <int D>
static kv_status decode_step_dispatch(const kv_pool *pool, const void *q, int hq,
                                      float scale_log2, int nsplit, int rcap, float *out,
                                      float *partials, int32_t *counters, const AttendFetch &fx,
                                      const DecodeStep &st, hipStream_t s) {
  const int G = hq / pool->n_kv_heads;
  const dim3 grid(nsplit, pool->batch * pool->n_kv_heads);
  // do waves 4-7 get rows of the first pass (a chunk of more than 4 x 32 rows)?
  const bool w47 = (std::max(rcap, 1) + nsplit - 1) / nsplit > (kAttendWaves - 4) * kAttendChunk;
  const bool small = pool->unit_cap <= kAttendThreads * 4;  // 4 selection keys per thread
  const int geo = attend_geo(pool, nsplit);
#define KVC_STEP(GG, KPT, W47)                                                                \
  k_gather_attend_mfma<D, GG, false, KPT, W47><<<grid, kAttendThreads, 0, s>>>(              \
      (const uint16_t *)fx.k, (const uint16_t *)fx.v, (const uint16_t *)q,                     \
      (const uint16_t *)st.q_prev, geo, rcap, fx.cap, hq, fx.spans, fx.count, *pool, scale_log2, \
      nullptr, nullptr, 1, nullptr, out, partials, counters, fx, st)
#define KVC_STEP2(GG)                                  \
  do {                                                 \
    if (small) {                                       \
      if (w47) KVC_STEP(GG, 4, true);                  \
      else KVC_STEP(GG, 4, false);                     \
    } else {                                           \
      if (w47) KVC_STEP(GG, 16, true);                 \
      else KVC_STEP(GG, 16, false);                    \
    }                                                  \
  } while (0)
  switch (G) {
    case 1: KVC_STEP2(1); break;
    case 2: KVC_STEP2(2); break;
    case 4: KVC_STEP2(4); break;
    case 8: KVC_STEP2(8); break;
    default: return KV_ERR_UNSUPPORTED;
  }
#undef KVC_STEP2
#undef KVC_STEP
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

kv_status launch_decode_step(const kv_pool *pool, const void *q_prev, const void *q, int hq,
                             float tau, float scale, int budget, uint8_t *flag, float *r,
                             int32_t *sel_units, int32_t *sel_spans, int sel_cap, int32_t *sel_n,
                             int32_t *sel_rows, int nsplit, int rcap, const kv_pool *dst,
                             int32_t *dst_spans, int32_t *dst_n, float *out, float *partials,
                             int32_t *counters, float *scores, int32_t *sel_counters,
                             int32_t *gen, hipStream_t s) {
  static_assert(kAttendThreads * 16 >= 8192, "16 selection keys per thread cover 8192 units");
  if (pool->dtype != KV_BF16 || pool->buf_cap > 0) return KV_ERR_UNSUPPORTED;
  hipPointerAttribute_t attr;
  int reread = 1;
  if (hipPointerGetAttributes(&attr, pool->k) == hipSuccess)
    reread = attr.type == hipMemoryTypeDevice ? 0 : 1;
  else
    (void)hipGetLastError();
  AttendFetch fx{flag, dst->k, dst->v, dst->row_cap, dst_spans, dst_n, reread};
  DecodeStep st{(const uint16_t *)q_prev, tau, budget, hq / pool->n_kv_heads, flag, r, sel_units,
                sel_n, sel_rows, sel_spans, sel_cap, scores, sel_counters, gen, pool->status};
  const float sl2 = scale * 1.4426950408889634f;  // log2(e): exp(x) = exp2(x log2 e)
  return pool->head_dim == 128
             ? decode_step_dispatch<128>(pool, q, hq, sl2, nsplit, rcap, out, partials,
                                         counters, fx, st, s)
             : decode_step_dispatch<64>(pool, q, hq, sl2, nsplit, rcap, out, partials, counters,
                                        fx, st, s);
}

}  // namespace kvc

// Internal helpers shared by the HIP translation units of libkvc (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

constexpr int kWave = 64;     // CDNA wavefront width
constexpr int kNumXcd = 8;    // MI355X: 8 XCDs, workgroups dispatched round-robin
constexpr int kMaxSel = 4096; // selected units staged in LDS by the attend kernel
constexpr int kSelectBlockThreads = 512;     // threads of a selection workgroup
constexpr int kSelectMaxKeysPerThread = 16;  // selection keys held per thread
constexpr int kMaxClusters = 8192;  // one counting-sort chunk's label counts fit 64 KB of LDS

// bf16 is carried as raw uint16_t bits.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float to_f32(float x) { return x; }
  __device__ __forceinline__ static float from_f32(float x) { return x; }
};
template <> struct Elem<uint16_t> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float to_f32(uint16_t x) { return bf16_bits_to_f32(x); }
  __device__ __forceinline__ static uint16_t from_f32(float x) { return f32_to_bf16_rne(x); }
};

// Unpack one 16-byte vector of elements into fp32 values.
template <typename T> __device__ __forceinline__ void unpack16(const uint4 &v, float *out);
template <> __device__ __forceinline__ void unpack16<float>(const uint4 &v, float *out) {
  out[0] = __uint_as_float(v.x);
  out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z);
  out[3] = __uint_as_float(v.w);
}
template <> __device__ __forceinline__ void unpack16<uint16_t>(const uint4 &v, float *out) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// DPP lane moves (gfx9 encodings): mirror a 16-lane row, mirror each 8-lane
// half row, rotate a row by 8 lanes (= lane ^ 8 within the row), broadcast
// one lane of each row to the row, and permute within quads.
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppRowBcast0 = 0x150;  // + n: lane n of each row to the whole row (gfx90a+)
constexpr int kDppQuadSwap2 = 0x4e;  // quad_perm [2, 3, 0, 1]
constexpr int kDppQuadSwap1 = 0xb1;  // quad_perm [1, 0, 3, 2]

template <int CTRL> __device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Exchanges across 16- and 32-lane distance with gfx950's lane-swap
// instructions (VALU, no LDS permute). Swapping v with itself leaves, in
// every lane l, the pair {v[l], v[l ^ 16]} (resp. v[l ^ 32]) in some order;
// + and max are commutative, so the results equal v op shfl_xor(v, 16 / 32)
// bit for bit.
__device__ __forceinline__ void swap_pair16(float v, float &a, float &b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap_pair32(float v, float &a, float &b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor16(float v) {
  float a, b;
  swap_pair16(v, a, b);
  return a + b;
}
__device__ __forceinline__ float sum_xor32(float v) {
  float a, b;
  swap_pair32(v, a, b);
  return a + b;
}
__device__ __forceinline__ float max_xor16(float v) {
  float a, b;
  swap_pair16(v, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float max_xor32(float v) {
  float a, b;
  swap_pair32(v, a, b);
  return fmaxf(a, b);
}

// Sum over aligned groups of N lanes (N = 2, 4, 8, 16, 32, 64); every lane of a
// group receives the group total. Within a 16-lane row the pairing is
// mirror -> half mirror -> quad swaps: after the row-mirror step lane i holds
// x_i + x_15-i, after the half-mirror step it holds the four lanes
// {j, 7-j, 8+j, 15-j} (j = i mod 8), and the two quad swaps combine the four
// such sets of a row. Wider groups add the 16- and 32-lane exchanges. All
// lanes must be active.
template <int N> __device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group size");
  if constexpr (N >= 16) v += dpp_mov<kDppRowMirror>(v);
  if constexpr (N >= 8) v += dpp_mov<kDppRowHalfMirror>(v);
  if constexpr (N >= 4) v += dpp_mov<kDppQuadSwap2>(v);
  v += dpp_mov<kDppQuadSwap1>(v);
  if constexpr (N >= 32) v = sum_xor16(v);
  if constexpr (N >= 64) v = sum_xor32(v);
  return v;
}

// Bitwise OR / AND over the whole wave, in every lane (row exchanges, then the
// 16- and 32-lane swaps; no LDS permute).
template <bool OR> __device__ __forceinline__ uint32_t wave_bits32(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return OR ? (a | b) : (a & b); };
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowMirror, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowHalfMirror, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadSwap2, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadSwap1, 0xf, 0xf, false));
  const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(r16[0], r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(r32[0], r32[1]);
}
// Unsigned maximum / minimum over the whole wave, in every lane (same pairing).
template <bool MAX> __device__ __forceinline__ uint32_t wave_ext_u32(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowMirror, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppRowHalfMirror, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadSwap2, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppQuadSwap1, 0xf, 0xf, false));
  const auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(r16[0], r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(r32[0], r32[1]);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_ext_u32<true>(v); }
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return wave_ext_u32<false>(v); }

template <bool OR> __device__ __forceinline__ unsigned long long wave_bits64(unsigned long long v) {
  return (unsigned long long)wave_bits32<OR>((uint32_t)v) |
         ((unsigned long long)wave_bits32<OR>((uint32_t)(v >> 32)) << 32);
}

// Integer sum over the whole wave, in every lane (same pairing as group_sum;
// exact, so the pairing does not matter).
__device__ __forceinline__ int wave_sum_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowMirror, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowHalfMirror, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppQuadSwap2, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppQuadSwap1, 0xf, 0xf, false);
  const auto r16 = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  v = (int)r16[0] + (int)r16[1];
  const auto r32 = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return (int)r32[0] + (int)r32[1];
}

// Inclusive prefix sums over the wave in lane order, by DPP lane moves only:
// shifts by 1, 2, 4 and 8 within each 16-lane row (lanes shifted in from
// outside the row read 0), then the last lane of row 0 and of row 2 added to
// rows 1 and 3, and the last lane of row 1 added to rows 2 and 3.
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowShr2 = 0x112;
constexpr int kDppRowShr4 = 0x114;
constexpr int kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

__device__ __forceinline__ int wave_incl_scan_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr1, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr2, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr4, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr8, 0xf, 0xf, true);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast15, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowBcast31, 0xc, 0xf, false);
  return v;
}

template <int CTRL, int ROWS, bool BOUND>
__device__ __forceinline__ long long dpp_mov_i64(long long v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWS, 0xf, BOUND);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)((unsigned long long)v >> 32), CTRL,
                                             ROWS, 0xf, BOUND);
  return (long long)(((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo);
}

__device__ __forceinline__ long long wave_incl_scan_i64(long long v) {
  v += dpp_mov_i64<kDppRowShr1, 0xf, true>(v);
  v += dpp_mov_i64<kDppRowShr2, 0xf, true>(v);
  v += dpp_mov_i64<kDppRowShr4, 0xf, true>(v);
  v += dpp_mov_i64<kDppRowShr8, 0xf, true>(v);
  v += dpp_mov_i64<kDppRowBcast15, 0xa, false>(v);
  v += dpp_mov_i64<kDppRowBcast31, 0xc, false>(v);
  return v;
}

// The value of lane `src` (the same in every lane) in every lane.
__device__ __forceinline__ int lane_value(int v, int src) {
  return __builtin_amdgcn_readlane(v, src);
}
__device__ __forceinline__ long long lane_value_i64(long long v, int src) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, src);
  const uint32_t hi =
      (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((unsigned long long)v >> 32), src);
  return (long long)(((unsigned long long)hi << 32) | lo);
}

// Maximum over the whole wave, in every lane (same pairing as group_sum).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<kDppRowMirror>(v));
  v = fmaxf(v, dpp_mov<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_mov<kDppQuadSwap2>(v));
  v = fmaxf(v, dpp_mov<kDppQuadSwap1>(v));
  v = max_xor16(v);
  return max_xor32(v);
}

// Sum over the lanes l' with l' % L == l % L (L = 8, 16, 32): lane groups that
// hold the same elements of different rows.
template <int L> __device__ __forceinline__ float sum_stride(float v) {
  static_assert(L == 8 || L == 16 || L == 32 || L == 64, "stride");
  if constexpr (L <= 8) v += dpp_mov<kDppRowRor8>(v);
  if constexpr (L <= 16) v = sum_xor16(v);
  if constexpr (L <= 32) v = sum_xor32(v);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

// Every 64-byte line of the first BYTES of the kernel's argument segment,
// requested at once by issue() and waited for by consume(). Left to itself
// the compiler loads an argument where it is first needed, so each new line
// is a scalar-cache miss and a wait of its own, one after another. Only the
// first dword of each line below BYTES is read, so BYTES up to the size of
// the explicit arguments keeps every load inside the segment.
template <int BYTES> struct KernargLines {
  static constexpr int N = (BYTES + 63) / 64;
  uint32_t w[N];
  __device__ __forceinline__ void issue() {
    typedef const uint32_t __attribute__((address_space(4))) karg_u32;
    karg_u32 *ka = (karg_u32 *)__builtin_amdgcn_kernarg_segment_ptr();
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = ka[16 * i];
    __builtin_amdgcn_sched_barrier(0);  // every request goes out here
  }
  __device__ __forceinline__ void consume() const {
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) x ^= w[i];
    asm volatile("" ::"s"(x));
  }
};

// Map a hardware workgroup id to a logical one so that each XCD (which
// receives ids x, x+8, x+16, ...) processes one contiguous range of logical
// work; neighbouring logical blocks then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int hw_id, int total) {
  const int per = total / kNumXcd, rem = total % kNumXcd;
  const int xcd = hw_id % kNumXcd, j = hw_id / kNumXcd;
  return (xcd < rem) ? xcd * (per + 1) + j : rem * (per + 1) + (xcd - rem) * per + j;
}

// Orderable key of a float: larger float -> larger unsigned (-0 folded to +0).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The float whose float_order_key is k (-0 comes back as +0).
__device__ __forceinline__ float order_key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace kvc

// Host-side launchers (defined in the .hip files, used by api.hip).
namespace kvc {

// K-means
// A head whose assignment in some round gives back the previous round's
// labels has reached a fixed point of Lloyd's iteration: the update then
// reproduces the centroids bit for bit, so every later round gives the same
// labels and centroids. kv_cluster_build tracks this per head and lets the
// kernels of the later rounds return at once for such heads:
//   conv[bh]: once the head has reached its fixed point, the number of
//             rounds whose assignment ran (the last of them changed nothing);
//   chg[bh]:  1 when this round's assignment changed a label of the head.
// Both are zeroed with the initial centroids. A null pointer disables it.
struct LloydSkip {
  int32_t *conv = nullptr;
  int32_t *chg = nullptr;
  int round = 0;  // 1-based number of the round the launch belongs to
  // [bh][c] or null: the clusters this round's label changes touched; the
  // member sums of an untouched cluster are those of the last round, so its
  // centroid and tile stay as they are
  const int32_t *touched = nullptr;
};
// Incremental assignment of kv_cluster_build (bf16): a round sweeps every
// centroid only for the keys whose own cluster moved in the last update; the
// other keys compare their recorded score with the moved centroids alone.
// Kernel-side view (per head; null members disable the part that uses them):
struct AssignInc {
  int32_t *own = nullptr;                // [bh][n]  winning score bits (upper 28) of each key
  float *koff = nullptr;                 // [bh][ceil(n/64)]  K_w of each 64-key wave
  const int32_t *fprev = nullptr;        // [bh][c]  clusters the last round's changes touched
  int32_t *fcur = nullptr;               // [bh][c]  ... this round's
  int32_t *mlist = nullptr;              // [bh][c]  moved clusters, ascending
  int32_t *hstate = nullptr;             // [bh][4]  moved count, mode, queued keys, -
  uint16_t *cfrags = nullptr;            // the moved clusters' tiles, in mlist order
  int32_t *glist = nullptr;              // [bh][n]  queued keys
  unsigned long long *gbest = nullptr;   // [bh][n]  (score bits << 32 | label) per queued key
  unsigned long long *work = nullptr;    // [bh]     (key, centroid) pairs scored after round 1
};
// Its workspace (carved from kv_cluster_build's).
struct AssignIncWs {
  int32_t *own, *flags[2], *mlist, *hstate, *glist;
  float *koff;
  uint16_t *cfrags;
  unsigned long long *gbest;
  unsigned long long *work;  // zeroed with the fixed-point flags
};
size_t assign_inc_ws_bytes(int bh, int n, int c, int d);
void assign_inc_ws_carve(void *base, int bh, int n, int c, int d, AssignIncWs *w);
// One assignment round (1-based `round`) of kv_cluster_build, bf16, with the
// fixed-point skip active from round 2 on: round 1 sweeps every centroid and
// records the scores; round 2 as well (every centroid moved in round 1's
// update); from round 3 on, heads where at most a third of the centroids
// moved run incrementally. The labels equal those of a whole sweep bit for
// bit. `frags` holds the current centroids' tiles.
kv_status launch_assign_round(const void *keys, int bh, int n, int d, int c, int32_t *labels,
                              const void *frags, const AssignIncWs &w, int round, LloydSkip skip,
                              hipStream_t s);
// rounds[i] = conv[i] if set, else iters (conv null: iters for every head);
// sweeps[i] (when given) = the assignment work in whole sweeps of n x c
// pairs: 1 + work[i] / (n c) with the incremental work counter, else the
// rounds.
kv_status launch_rounds_out(const int32_t *conv, const unsigned long long *work, int32_t *rounds,
                            float *sweeps, int bh, int iters, int n, int c, hipStream_t s);
kv_status launch_init_centroids(const void *keys, const int32_t *init_idx, float *cent, int bh,
                                int n, int c, int d, kv_dtype dt, int32_t *status, hipStream_t s,
                                int32_t *zero = nullptr, int nzero = 0);
size_t assign_ws_bytes(int bh, int c, int d, kv_dtype dt);
kv_status launch_prep_frags(const float *cent, int bh, int d, int c, void *ws, hipStream_t s);
kv_status launch_assign_prepare(const float *cent, int bh, int d, int c, kv_dtype dt, void *ws,
                                hipStream_t s);
// skip (bf16 only): heads with conv set return at once; the others compare
// their new labels with the ones in `labels` and set chg when one differs.
kv_status launch_assign_prepared(const void *keys, const float *cent, int bh, int n, int d, int c,
                                 kv_dtype dt, int32_t *labels, const void *ws, hipStream_t s,
                                 LloydSkip skip = {});
kv_status launch_assign(const void *keys, const float *cent, int bh, int n, int d, int c,
                        kv_dtype dt, int32_t *labels, void *ws, hipStream_t s,
                        bool frags_ready = false, LloydSkip skip = {});
size_t update_ws_bytes(int bh, int n, int c);
kv_status launch_update(const void *keys, const int32_t *labels, const float *cent_in,
                        float *cent_out, int32_t *counts, int bh, int n, int d, int c,
                        kv_dtype dt, void *ws, hipStream_t s,
                        const int32_t **perm_out, const int32_t **start_out,
                        const int32_t **tot_out, void *frags_out = nullptr,
                        int32_t *status = nullptr, LloydSkip skip = {});
// The update of a round whose permutation, starts and counts nobody reads
// (centroids and next tiles only; the same bits as launch_update), in two
// launches, where that is the faster way (update_local_ok).
bool update_local_ok(int bh, int n, int c);
// skip: the first kernel marks conv for heads whose chg is 0 (and every
// kernel returns at once for heads with conv set); the last clears chg.
kv_status launch_update_local(const void *keys, const int32_t *labels, const float *cent_in,
                              float *cent_out, int bh, int n, int d, int c, kv_dtype dt,
                              void *ws, hipStream_t s, void *frags_out, LloydSkip skip = {});
kv_status launch_pack(const kv_pool *pool, const void *keys, const void *values,
                      const float *cent, const int32_t *perm, const int32_t *start,
                      const int32_t *tot, int n, int c, hipStream_t s);

// Decode
kv_status launch_boundary(const void *q_prev, const void *q_cur, int batch, int hq, int d,
                          kv_dtype dt, float tau, uint8_t *flag, float *r, hipStream_t s);
// fused: run the boundary test on (q_prev, q_cur) inside the append kernel and
// write flag_out / r_out instead of reading flag.
kv_status launch_segment_append(const kv_pool *pool, const void *k_t, const void *v_t,
                                const uint8_t *flag, bool fused, const void *q_prev,
                                const void *q_cur, int hq, float tau, uint8_t *flag_out,
                                float *r_out, hipStream_t s);
int select_num_blocks(const kv_pool *pool);
// fused: run the boundary test on (q_prev, q) inside the select kernel and
// write flag_out / r_out instead of reading flag.
kv_status launch_select(const kv_pool *pool, const void *q, int hq, int budget,
                        const uint8_t *flag, int32_t *sel_units, int sel_cap, int32_t *sel_n,
                        int32_t *sel_rows, int32_t *sel_spans, float *scores, int32_t *counters,
                        bool fused,
                        const void *q_prev, float tau, uint8_t *flag_out, float *r_out,
                        hipStream_t s);
int attend_num_splits(const kv_pool *pool, int max_rows);
kv_status launch_decode_step(const kv_pool *pool, const void *q_prev, const void *q, int hq,
                             float tau, float scale, int budget, uint8_t *flag, float *r,
                             int32_t *sel_units, int32_t *sel_spans, int sel_cap, int32_t *sel_n,
                             int32_t *sel_rows, int nsplit, int rcap, const kv_pool *dst,
                             int32_t *dst_spans, int32_t *dst_n, float *out, float *partials,
                             int32_t *counters, float *scores, int32_t *sel_counters,
                             int32_t *gen, hipStream_t s);
int attend_row_bound(const kv_pool *pool, int max_rows);
kv_status launch_gather_attend(const kv_pool *pool, const void *q, int hq, float scale,
                               const int32_t *sel_units, const int32_t *sel_spans, int sel_cap,
                               const int32_t *sel_n, int nsplit, int rcap, float *out,
                               float *partials, int32_t *counters, hipStream_t s);
int fetch_num_blocks(const kv_pool *dst);
kv_status launch_fetch_rows(const kv_pool *src, const uint8_t *flag, const int32_t *sel_units,
                            const int32_t *sel_spans, int sel_cap, const int32_t *sel_n,
                            const kv_pool *dst, int32_t *dst_spans, int32_t *dst_n,
                            hipStream_t s);
kv_status launch_fetch_attend(const kv_pool *pool, const void *q, int hq, float scale,
                              const uint8_t *flag, const int32_t *sel_units,
                              const int32_t *sel_spans, int sel_cap, const int32_t *sel_n,
                              int nsplit, int rcap, const kv_pool *dst, int32_t *dst_spans,
                              int32_t *dst_n, float *out, float *partials, int32_t *counters,
                              hipStream_t s);

}  // namespace kvc

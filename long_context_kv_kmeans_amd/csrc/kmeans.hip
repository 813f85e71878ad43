// Prefill K-means for centroid-indexed KV retrieval, gfx950.
//
// LouisKV note (papernotes.org), "Key designs" item 2: each KV head's prefill
// keys are grouped with K-means; a cluster's centroid, the mean of its keys,
// is its retrieval index. One Lloyd round here is
//   assign  -- a(x) = argmax_k (x . c^_k - |c^_k|^2 / 2) == argmin_k |x - c^_k|^2,
//              c^ = bf16(fp32 master), fp32 accumulation on the matrix cores,
//              ties to the lowest k;
//   update  -- stable counting sort of keys by label, then each centroid is
//              the in-order fp32 sum of its members divided by their count
//              (empty clusters keep their value). No float atomics, so the
//              result is bitwise reproducible.
#include "kvc_internal.hpp"

namespace kvc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kAssignColBlocks = 2;                      // 32-key MFMA column blocks per wave
constexpr int kAssignMinWaves = 4;                       // waves per SIMD the register budget targets
constexpr int kTilesPerStage = 2;                        // 64 centroids per LDS stage
constexpr int kAssignWaves = 8;                          // waves per workgroup

// ---------------------------------------------------------------- init
// An index outside [0, n) is clamped into it (so no read leaves the head's
// keys) and reported as KV_ERR_INVALID_ARG through *status when given.
template <typename T>
__global__ void k_init_centroids(const T *__restrict__ keys, const int32_t *__restrict__ init_idx,
                                 float *__restrict__ cent, int n, int c, int d, long total,
                                 int32_t *status, int32_t *__restrict__ zero, int nzero) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total;
       i += (long)gridDim.x * blockDim.x) {
    if (i < nzero) zero[i] = 0;  // (total >= nzero: every entry is reached)
    const long bh = i / ((long)c * d);
    const int k = (int)((i / d) % c), e = (int)(i % d);
    int src = init_idx[bh * c + k];
    if (src < 0 || src >= n) {
      if (status && e == 0)
        __hip_atomic_store(status, (int)KV_ERR_INVALID_ARG, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      src = src < 0 ? 0 : n - 1;
    }
    cent[i] = Elem<T>::to_f32(keys[(bh * n + src) * d + e]);
  }
}

kv_status launch_init_centroids(const void *keys, const int32_t *init_idx, float *cent, int bh,
                                int n, int c, int d, kv_dtype dt, int32_t *status, hipStream_t s,
                                int32_t *zero, int nzero) {
  const long total = (long)bh * c * d;
  if (nzero > total) return KV_ERR_INVALID_ARG;
  const int blocks = (int)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  if (dt == KV_BF16)
    k_init_centroids<uint16_t><<<blocks, 256, 0, s>>>((const uint16_t *)keys, init_idx, cent, n,
                                                      c, d, total, status, zero, nzero);
  else
    k_init_centroids<float><<<blocks, 256, 0, s>>>((const float *)keys, init_idx, cent, n, c, d,
                                                   total, status, zero, nzero);
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

// ---------------------------------------------------------------- bf16 assign
// Centroid tiles for v_mfma_f32_32x32x16_bf16 with centroids as the A operand
// (32 rows x 16 k per instruction). A tile of 32 centroids is KS = D / 16
// fragment blocks followed by one norm block:
//   fragment block s, lane l (16 bytes): row m = l % 32 and
//     k = 16 s + 8 (l / 32) + j, j = 0..7;
//   norm block (32 fp32): entry m = -|c^_m|^2 / 2 of the bf16-rounded row;
//     padding rows (m >= C) hold kPadNorm and never win.
// The norm block is the accumulator's initial value, so the matrix cores
// produce x . c^ - |c^|^2 / 2 with no extra k-step.
constexpr int kNormU4 = 8;  // 16-byte units of a tile's norm block
constexpr float kPadNorm = -3.0e38f;

template <int D> struct AssignTile {
  static constexpr int KS = D / 16;             // k-steps per tile
  static constexpr int U4 = KS * 64 + kNormU4;  // 16-byte units per tile
};

__device__ __forceinline__ void write_centroid_norm(uint4 *tile, int ks, int m, float neg_halfsq) {
  reinterpret_cast<float *>(tile + ks * 64)[m] = neg_halfsq;
}

// fp32 centroids -> tiles; D/8 lanes per centroid row, 8 consecutive
// elements each: the lane layout, the in-lane order of the squared-norm sum
// and the pairing across lanes of segsum_finish, which writes the tiles of
// the later rounds, so both give the same tile bits for the same centroid.
template <int D>
__global__ void __launch_bounds__(256) k_prep_frags(const float *__restrict__ cent,
                                                    uint16_t *__restrict__ frags, int c, int ntile) {
  using TL = AssignTile<D>;
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const int bh = blockIdx.y;
  const int row = blockIdx.x * RPB + threadIdx.x / LPR;
  const int e0 = (threadIdx.x % LPR) * 8;
  if (row >= ntile * 32) return;  // uniform per row group (LPR divides 64)
  const bool real = row < c;
  float v[8];
  const float4 *src = reinterpret_cast<const float4 *>(cent + ((size_t)bh * c + (real ? row : 0)) * D + e0);
  const float4 lo = real ? src[0] : float4{0.f, 0.f, 0.f, 0.f};
  const float4 hi = real ? src[1] : float4{0.f, 0.f, 0.f, 0.f};
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  uint16_t b[8];
  float sq = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    b[e] = f32_to_bf16_rne(v[e]);
    const float r = bf16_bits_to_f32(b[e]);
    sq = fmaf(r, r, sq);
  }
  sq = group_sum<LPR>(sq);
  const int t = row / 32, m = row % 32;
  uint4 *tile = reinterpret_cast<uint4 *>(frags) + ((size_t)bh * ntile + t) * TL::U4;
  uint4 pk;
  pk.x = b[0] | ((uint32_t)b[1] << 16);
  pk.y = b[2] | ((uint32_t)b[3] << 16);
  pk.z = b[4] | ((uint32_t)b[5] << 16);
  pk.w = b[6] | ((uint32_t)b[7] << 16);
  tile[(e0 / 16) * 64 + m + 32 * ((e0 % 16) / 8)] = pk;
  if (e0 == 0) write_centroid_norm(tile, TL::KS, m, real ? -0.5f * sq : kPadNorm);
}

// Heads whose blocks a launch serves, spread over the whole grid: with A such
// heads, blocks i < A * bph take work item w = xcd_remap(i, A * bph) (so every
// XCD still gets a contiguous range), i.e. key block w % bph of the
// (w / bph)-th served head in index order; the other blocks have nothing to
// do. Without this a converged head's blocks would leave its XCD idle while
// the others' XCDs still work through theirs. A head is served when its conv
// flag is 0 and, with a state table, its sweep mode is `want`. Returns that
// head (wave-uniform, the same in every wave) or -1.
__device__ __forceinline__ bool head_served(const int32_t *__restrict__ conv,
                                            const int32_t *__restrict__ hstate, int want, int i) {
  return conv[i] == 0 && (hstate == nullptr || hstate[4 * i + 1] == want);
}

__device__ __forceinline__ int active_head_block(const int32_t *__restrict__ conv,
                                                 const int32_t *__restrict__ hstate, int want,
                                                 int nbh, int bph, int *bid) {
  const int lane = threadIdx.x & 63;
  int na = 0;
  for (int b0 = 0; b0 < nbh; b0 += 64) {
    const int i = b0 + lane;
    na += __popcll(__ballot(i < nbh && head_served(conv, hstate, want, i)));
  }
  const int work = na * bph;
  if ((int)blockIdx.x >= work) return -1;
  *bid = xcd_remap(blockIdx.x, work);
  int r = *bid / bph;
  for (int b0 = 0; b0 < nbh; b0 += 64) {
    const int i = b0 + lane;
    const bool act = i < nbh && head_served(conv, hstate, want, i);
    const uint64_t m = __ballot(act);
    const int cnt = __popcll(m);
    if (r < cnt) {
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      return b0 + __builtin_ctzll(__ballot(act && below == r));
    }
    r -= cnt;
  }
  return -1;
}

// Key groups of the full sweep over gathered keys (kAssignGather): head i
// holds ceil(gathered_i / keys per workgroup) of them when it is served in
// incremental mode. Sets *total to their sum over the heads; for group g <
// total also the head (return value) and the group's index within the head.
__device__ __forceinline__ int gathered_groups(const int32_t *__restrict__ conv,
                                               const int32_t *__restrict__ hstate, int nbh,
                                               int kpb, int g, int *total, int *gin) {
  const int lane = threadIdx.x & 63;
  int sum = 0, head = -1;
  for (int b0 = 0; b0 < nbh; b0 += 64) {
    const int i = b0 + lane;
    const int gi = (i < nbh && head_served(conv, hstate, 0, i)) ? (hstate[4 * i + 2] + kpb - 1) / kpb
                                                                : 0;
    const int incl = wave_incl_scan_i32(gi);
    const int tot = lane_value(incl, 63);
    if (head < 0 && g >= sum && g < sum + tot) {
      const int l = __builtin_ctzll(__ballot(sum + incl > g));
      head = b0 + l;
      *gin = g - (sum + lane_value(incl, l) - lane_value(gi, l));
    }
    sum += tot;
  }
  *total = sum;
  return head;
}

// One workgroup = 8 waves x 64 keys. Keys are the B operand (column n = key),
// resident in VGPRs for the whole centroid sweep. Centroid tiles stream into
// two LDS stage buffers with direct global->LDS loads (each wave instruction
// moves one 1 KB block of the stage's flat copy), so staging costs neither
// VGPRs nor LDS write instructions; the two buffers are separate objects and
// are selected statically, which lets the compiler keep the next stage's
// loads in flight while the current stage is read. A wave folds tile t into
// its argmin before issuing tile t+1's MFMAs into the same accumulators (no
// copies); the matrix cores and the VALU overlap across the 4 waves each SIMD
// holds (128 VGPRs), and a stage's barrier is shared by 8 waves.
//
// Scores: the accumulators start from the tile's norm block minus K_w, the
// largest |x|^2 / 2 among the wave's keys (plus 0.1%), so every score
// x . c^ - |c^|^2 / 2 - K_w = -|x - c^|^2 / 2 - (K_w - |x|^2 / 2) is <= 0 and
// orders a key's centroids exactly as the distance does.
//
// Argmin: every lane sees one key and 16 centroid rows per tile. A score
// (<= 0; negative floats order inversely to their bit patterns) is packed as
// (bits & ~15) | r, so among packed values the unsigned minimum is the
// largest score (nearest centroid) and, on equal upper 28 bits, the lowest
// row r: one v_and_or and half a v_min3 per score. A score that rounding
// leaves slightly above 0 packs below every negative one, i.e. it still
// ranks as nearest.
// Across tiles a new minimum must be strictly smaller in the upper 28 bits,
// so earlier (lower-index) tiles win ties. Comparing 28 of 32 bits moves a
// decision only where two scores agree to about 2^-19 relative, the size of
// the fp32 accumulation error of the 128-term dot product.
// The label is therefore the minimum of (upper 28 score bits, index) in
// lexicographic order over the centroids swept, whatever their order: a
// sweep may be split over centroid ranges or restricted to a subset and
// still give the same label as the whole sweep. Each (key, centroid) score
// depends only on the key, K_w of the key's 64-key wave and the centroid's
// tile row, which the incremental modes below rely on.
//
// MODE (the incremental assignment of kv_cluster_build, exact: the labels of
// a whole sweep):
//   kAssignFull    -- every centroid for the keys of the served heads; with
//                     `inc` also records each key's winning score bits, each
//                     wave's K_w and the clusters its label changes touch;
//   kAssignMoved   -- only the moved centroids (compact tiles): a key whose
//                     own cluster did not move keeps the lexicographic
//                     minimum of its recorded score and the moved ones; a key
//                     whose own cluster moved is queued for kAssignGather;
//   kAssignGather  -- every centroid for the queued keys, the centroid range
//                     split over workgroups (a loop over work items); the
//                     splits meet in a 64-bit atomic minimum of
//                     (score bits << 32 | label) per queued key.
constexpr int kAssignFull = 0, kAssignMoved = 1, kAssignGather = 2;

template <int D, int NCB, int MINW, int MODE>
__global__ void __launch_bounds__(64 * kAssignWaves, MINW)
    k_assign_mfma(const uint16_t *__restrict__ keys, const uint16_t *__restrict__ frags,
                  int32_t *__restrict__ labels, int n, int c, int ntile, int blocks_per_head,
                  int total_blocks, const int32_t *__restrict__ conv, int32_t *__restrict__ chg,
                  AssignInc inc) {
  using TL = AssignTile<D>;
  constexpr int KS = TL::KS;
  constexpr int TILE_U4 = TL::U4;
  constexpr int STAGE_U4 = kTilesPerStage * TILE_U4;   // 16-byte units per stage
  constexpr int STAGE_BLOCKS = (STAGE_U4 + 63) / 64;  // 1 KB DMA blocks (the last partial)
  __shared__ uint4 lds0[STAGE_BLOCKS * 64];
  __shared__ uint4 lds1[STAGE_BLOCKS * 64];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int KPW = 32 * NCB;  // keys per wave
  constexpr int KPB = kAssignWaves * KPW;
  const int half = lane >> 5;
  const int nbh = total_blocks / blocks_per_head;
  const int nw = (n + KPW - 1) / KPW;  // 64-key waves per head
  const int nstage_all = (ntile + kTilesPerStage - 1) / kTilesPerStage;

  // kAssignGather: work items (key group, centroid split), S splits per group
  int item = blockIdx.x, nitems = 1, nsplit = 1;
  if constexpr (MODE == kAssignGather) {
    int total = 0, gin = 0;
    (void)gathered_groups(conv, inc.hstate, nbh, KPB, -1, &total, &gin);
    nsplit = total >= (int)gridDim.x ? 1 : min(nstage_all, (int)gridDim.x / max(total, 1));
    nitems = total * nsplit;
    if (item >= nitems) return;
  }
  for (;;) {
    int bh = 0, key0 = 0, t0 = 0, ntl = ntile, cl = c, gcount = 0, gpos0 = 0;
    const uint16_t *src = frags;
    bool work = true;
    if constexpr (MODE == kAssignGather) {
      int total = 0, gin = 0;
      bh = gathered_groups(conv, inc.hstate, nbh, KPB, item / nsplit, &total, &gin);
      const int sps = (nstage_all + nsplit - 1) / nsplit;  // stages per split
      const int st0 = (item % nsplit) * sps, st1 = min(st0 + sps, nstage_all);
      work = bh >= 0 && st0 < st1;
      t0 = st0 * kTilesPerStage;
      ntl = min(st1 * kTilesPerStage, ntile) - t0;
      cl = c - t0 * 32;
      gcount = bh >= 0 ? inc.hstate[4 * bh + 2] : 0;
      gpos0 = gin * KPB + wave * KPW;
    } else {
      int bid = xcd_remap(blockIdx.x, total_blocks);
      bh = bid / blocks_per_head;
      if (conv != nullptr) {  // only heads still iterating (in this mode) get blocks
        bh = active_head_block(conv, inc.hstate, MODE == kAssignMoved ? 0 : 1, nbh,
                               blocks_per_head, &bid);
        if (bh < 0) return;
      }
      key0 = (bid % blocks_per_head) * KPB + wave * KPW;
      if constexpr (MODE == kAssignMoved) {
        src = inc.cfrags;
        cl = inc.hstate[4 * bh + 0];
        ntl = (cl + 31) / 32;
        if (ntl == 0) return;  // nothing moved: every label stands
      }
    }
    if (work) {
      // Key fragments (B operand): lane holds key n = lane % 32, k = 16 s + 8 half + j.
      bf16x8_t bfrag[NCB][KS];
      float kmax = 0.f;
      int gkey[NCB];   // kAssignGather: the lane's key (valid when < n)
      float kofs[NCB];  // kAssignGather: K_w of that key's wave
      // kAssignMoved: the key's label (requested now, used after the sweep)
      int oldl[NCB];
      if constexpr (MODE == kAssignMoved) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          oldl[cb] = labels[(size_t)bh * n + min(key0 + cb * 32 + (lane & 31), n - 1)];
      }
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        int key = key0 + cb * 32 + (lane & 31);
        if constexpr (MODE == kAssignGather) {
          const int p = gpos0 + cb * 32 + (lane & 31);
          key = p < gcount ? inc.glist[(size_t)bh * n + p] : n;
          gkey[cb] = key;
          kofs[cb] = key < n ? inc.koff[(size_t)bh * nw + key / KPW] : 0.f;
        }
        const uint16_t *krow = keys + ((size_t)bh * n + (key < n ? key : 0)) * D;
        float sq = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          uint4 v = {0u, 0u, 0u, 0u};
          if (key < n) v = *reinterpret_cast<const uint4 *>(krow + 16 * s + 8 * half);
          bfrag[cb][s] = __builtin_bit_cast(bf16x8_t, v);
          if constexpr (MODE != kAssignGather) {
            float f[8];
            unpack16<uint16_t>(v, f);
#pragma unroll
            for (int j = 0; j < 8; ++j) sq = fmaf(f[j], f[j], sq);
          }
        }
        if constexpr (MODE != kAssignGather) kmax = fmaxf(kmax, sum_xor32(sq));
      }
      // The empty asm makes the product opaque, so the compiler cannot fuse it
      // into the per-tile subtractions below in some tiles and not in others:
      // every tile's accumulator start must be the same function of its norms
      // bit for bit (identical centroids must score identically in every tile
      // for the lowest-index tie rule).
      float koff = 0.5f * wave_max(kmax) * 1.001f;
      asm volatile("" : "+v"(koff));
      if (MODE != kAssignGather && inc.koff != nullptr && lane == 0 && key0 < n)
        inc.koff[(size_t)bh * nw + key0 / KPW] = koff;

      uint32_t bestp[NCB];
      int btile[NCB];
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        bestp[cb] = 0xffffffffu;
        btile[cb] = 0;
      }

      const uint4 *gfr = reinterpret_cast<const uint4 *>(src) + ((size_t)bh * ntile + t0) * TILE_U4;
      const int nstage = (ntl + kTilesPerStage - 1) / kTilesPerStage;

      // Stage st -> LDS as one flat copy of its tiles: wave w moves 1 KB blocks
      // w, w + 8, ...; units past the range's last tile are not loaded (and never read).
      auto dma_stage = [&](int st, uint4 *dst) {
        const int lim = min(ntl - st * kTilesPerStage, kTilesPerStage) * TILE_U4;
#pragma unroll
        for (int i = wave; i < STAGE_BLOCKS; i += kAssignWaves) {
          if (i * 64 + lane < lim)
            __builtin_amdgcn_global_load_lds(gfr + (size_t)st * STAGE_U4 + i * 64 + lane,
                                             dst + i * 64, 16, 0, 0);
        }
      };
      // D layout: lane holds column n = lane % 32 and rows 8 (r / 4) + 4 half + r % 4,
      // whose norms are entries 8 j + 4 half .. + 3 (unit 2 j + half) of the norm block.
      // The next k-step's A fragment is requested before this k-step's MFMAs issue.
      // kAssignGather: the columns' keys come from different waves, so each
      // column block starts from its own K_w (per lane).
      auto mfma_tile = [&](const uint4 *buf, int tt, f32x16_t *o) {
        const uint4 *tb = buf + tt * TILE_U4;
        bf16x8_t a[2];
        a[0] = __builtin_bit_cast(bf16x8_t, tb[lane]);
        f32x16_t ci;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 u = tb[KS * 64 + 2 * j + half];
          ci[4 * j + 0] = __uint_as_float(u.x);
          ci[4 * j + 1] = __uint_as_float(u.y);
          ci[4 * j + 2] = __uint_as_float(u.z);
          ci[4 * j + 3] = __uint_as_float(u.w);
        }
        if constexpr (MODE == kAssignGather) {
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[cb][r] = ci[r] - kofs[cb];
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) ci[r] -= koff;
        }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          if (s + 1 < KS) a[(s + 1) & 1] = __builtin_bit_cast(bf16x8_t, tb[(s + 1) * 64 + lane]);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb) {
            if constexpr (MODE == kAssignGather)
              o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s & 1], bfrag[cb][s], o[cb], 0, 0, 0);
            else
              o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s & 1], bfrag[cb][s],
                                                              s == 0 ? ci : o[cb], 0, 0, 0);
          }
        }
      };
      auto argmin_tile = [&](const f32x16_t &acc, int cb, int t, bool last) {
        uint32_t p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          p[r] = (__float_as_uint(acc[r]) & 0xfffffff0u) | (uint32_t)r;
        if (last && t * 32 + 32 > cl) {  // ragged last tile: padding rows never take part
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (t * 32 + 8 * (r >> 2) + 4 * half + (r & 3) >= cl) p[r] = 0xffffffffu;
        }
        const uint32_t m0 = min(min(p[0], p[1]), p[2]);
        const uint32_t m1 = min(min(p[3], p[4]), p[5]);
        const uint32_t m2 = min(min(p[6], p[7]), p[8]);
        const uint32_t m3 = min(min(p[9], p[10]), p[11]);
        const uint32_t m4 = min(min(p[12], p[13]), p[14]);
        const uint32_t q0 = min(min(m0, m1), m2);
        const uint32_t q1 = min(min(m3, m4), p[15]);
        const uint32_t m = min(q0, q1);
        if ((m | 15u) < (bestp[cb] & 0xfffffff0u)) {
          bestp[cb] = m;
          btile[cb] = t;
        }
      };

      f32x16_t acc[NCB];
      int t = 0;  // tile whose scores sit in acc
      auto argmin_all = [&](bool last) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) argmin_tile(acc[cb], cb, t, last);
      };
      auto advance = [&](const uint4 *buf, int tt, int nt) {
        argmin_all(false);
        mfma_tile(buf, tt, acc);
        t = nt;
      };
      // Tiles [st * TPS + 1, (st + 1) * TPS) of stage st (in `cur`), then the first
      // tile of stage st + 1 (in `nxt`) once that stage has landed.
      auto run_stage = [&](int st, const uint4 *cur, uint4 *cur_w, const uint4 *nxt) {
#pragma unroll
        for (int tt = 1; tt < kTilesPerStage; ++tt) {
          const int nt = st * kTilesPerStage + tt;
          if (nt >= ntl) return;
          advance(cur, tt, nt);
        }
        const int nt = (st + 1) * kTilesPerStage;
        if (nt >= ntl) return;
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): stage st + 1 has landed
        __syncthreads();                     // ... for every wave; `cur` is free again
        if (st + 2 < nstage) dma_stage(st + 2, cur_w);
        advance(nxt, 0, nt);
      };

      dma_stage(0, lds0);
      __builtin_amdgcn_s_waitcnt(0x0f70);
      __syncthreads();
      if (nstage > 1) dma_stage(1, lds1);
      mfma_tile(lds0, 0, acc);
      for (int st = 0; st < nstage; st += 2) {
        run_stage(st, lds0, lds0, lds1);
        if (st + 1 < nstage) run_stage(st + 1, lds1, lds1, lds0);
      }
      argmin_all(true);

      bool diff = false;  // a label of this wave differs from the previous round's
      bool queue[NCB];    // kAssignMoved: the key's own cluster moved
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb) {
        queue[cb] = false;
        const uint32_t r = bestp[cb] & 15u;
        uint32_t kt = bestp[cb] & 0xfffffff0u;
        int idx = btile[cb] * 32 + 8 * (int)(r >> 2) + (int)(r & 3u) + 4 * half;
        const uint32_t ok = __shfl_xor(kt, 32);
        const int oi = __shfl_xor(idx, 32);
        if (ok < kt || (ok == kt && oi < idx)) {
          idx = oi;
          kt = ok;
        }
        if constexpr (MODE == kAssignGather) {
          const int p = gpos0 + cb * 32 + (lane & 31);
          if (half == 0 && gkey[cb] < n)
            atomicMin(inc.gbest + (size_t)bh * n + p,
                      ((unsigned long long)kt << 32) | (uint32_t)(t0 * 32 + idx));
          continue;
        }
        const int key = key0 + cb * 32 + (lane & 31);
        if (half != 0 || key >= n) continue;
        int32_t *lp = labels + (size_t)bh * n + key;
        if constexpr (MODE == kAssignMoved) {
          const int old = oldl[cb];
          if (inc.fprev[(size_t)bh * c + old] != 0) {
            queue[cb] = true;
            continue;
          }
          const int j = inc.mlist[(size_t)bh * c + min(idx, cl - 1)];
          const uint32_t own = (uint32_t)inc.own[(size_t)bh * n + key];
          if (kt < own || (kt == own && j < old)) {
            *lp = j;
            inc.own[(size_t)bh * n + key] = (int32_t)kt;
            inc.fcur[(size_t)bh * c + old] = 1;
            inc.fcur[(size_t)bh * c + j] = 1;
            diff = true;
          }
        } else {
          if (chg != nullptr) {
            const int old = *lp;
            if (old != idx) {
              diff = true;
              if (inc.fcur != nullptr) {
                inc.fcur[(size_t)bh * c + old] = 1;
                inc.fcur[(size_t)bh * c + idx] = 1;
              }
            }
          }
          *lp = idx;
          if (inc.own != nullptr) inc.own[(size_t)bh * n + key] = (int32_t)kt;
        }
      }
      if constexpr (MODE == kAssignMoved) {
        // queue the keys whose own cluster moved: a slot per key, one atomic
        // per workgroup (the head's counter is shared by all its workgroups)
        __shared__ int s_q[kAssignWaves + 1];
        uint64_t qm[NCB];
        int wq = 0;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          qm[cb] = __ballot(queue[cb]);
          wq += __popcll(qm[cb]);
        }
        if (lane == 0) s_q[wave] = wq;
        __syncthreads();
        if (threadIdx.x == 0) {
          int tq = 0;
          for (int w = 0; w < kAssignWaves; ++w) tq += s_q[w];
          s_q[kAssignWaves] = tq > 0 ? atomicAdd(inc.hstate + 4 * bh + 2, tq) : 0;
        }
        __syncthreads();
        int base = s_q[kAssignWaves];
        for (int w = 0; w < wave; ++w) base += s_q[w];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          if (queue[cb]) {
            const int p = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(qm[cb] >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)qm[cb], 0u));
            inc.glist[(size_t)bh * n + p] = key0 + cb * 32 + (lane & 31);
            inc.gbest[(size_t)bh * n + p] = ~0ull;
          }
          base += __popcll(qm[cb]);
        }
      }
      // the head's change flag: stored by the first waves that see it clear
      // (every wave storing to one line would queue thousands of writes there)
      if (MODE != kAssignGather && chg != nullptr && __ballot(diff) != 0ull && lane == 0 &&
          chg[bh] == 0)
        chg[bh] = 1;
    }
    if constexpr (MODE != kAssignGather) break;
    item += gridDim.x;
    if (item >= nitems) break;
    __syncthreads();  // the stage buffers are filled again for the next item
  }
}

// After kAssignGather: the queued keys take the labels the splits agreed on.
__global__ void __launch_bounds__(256) k_assign_gathered_finish(int32_t *__restrict__ labels,
                                                                int n, int c,
                                                                const int32_t *__restrict__ conv,
                                                                int32_t *__restrict__ chg,
                                                                AssignInc inc) {
  const int bh = blockIdx.y;
  if (!head_served(conv, inc.hstate, 0, bh)) return;
  const int g = inc.hstate[4 * bh + 2];
  if (inc.work != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
    inc.work[bh] += (unsigned long long)g * c;
  bool diff = false;
  for (int p = blockIdx.x * 256 + threadIdx.x; p < g; p += gridDim.x * 256) {
    const int key = inc.glist[(size_t)bh * n + p];
    const unsigned long long b = inc.gbest[(size_t)bh * n + p];
    const int j = (int)(uint32_t)b;
    if (key < 0 || key >= n || j < 0 || j >= c) continue;  // every split wrote a label
    int32_t *lp = labels + (size_t)bh * n + key;
    const int old = *lp;
    inc.own[(size_t)bh * n + key] = (int32_t)(uint32_t)(b >> 32);
    if (j != old) {
      *lp = j;
      inc.fcur[(size_t)bh * c + old] = 1;
      inc.fcur[(size_t)bh * c + j] = 1;
      diff = true;
    }
  }
  if (__ballot(diff) != 0ull && (threadIdx.x & 63) == 0 && chg[bh] == 0) chg[bh] = 1;
}

// Before a round's assignment: the clusters the previous round's label
// changes touched (fprev) are the only ones whose centroid can have moved.
// Lists them in index order with their tiles copied into compact tiles, and
// sets the head's state: [0] moved count, [1] mode (1: sweep every centroid,
// when more than a third moved or on force_full; 0: incremental; 2: head
// converged), [2] queued keys = 0. Clears fcur for this round's assignment.
template <int D>
__global__ void __launch_bounds__(256) k_moved_list(const uint16_t *__restrict__ frags, int n,
                                                    int c, int ntile,
                                                    const int32_t *__restrict__ conv,
                                                    int force_full, AssignInc inc) {
  using TL = AssignTile<D>;
  __shared__ int s_w[2][4];
  const int bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = blockIdx.x * 256 + tid;
  int32_t *hs = inc.hstate + 4 * bh;
  if (conv[bh] != 0) {
    if (blockIdx.x == 0 && tid == 0) {
      hs[0] = 0;
      hs[1] = 2;
      hs[2] = 0;
    }
    return;
  }
  if (k < c) inc.fcur[(size_t)bh * c + k] = 0;
  if (force_full) {
    if (blockIdx.x == 0 && tid == 0) {
      hs[0] = c;
      hs[1] = 1;
      hs[2] = 0;
      if (inc.work != nullptr) inc.work[bh] += (unsigned long long)n * c;
    }
    return;
  }
  const int32_t *fp = inc.fprev + (size_t)bh * c;
  const int lo = blockIdx.x * 256;
  int before = 0, tot = 0;
  for (int i = tid; i < c; i += 256) {
    const int f = fp[i] != 0;
    tot += f;
    before += (i < lo) ? f : 0;
  }
  before = wave_sum_i32(before);
  tot = wave_sum_i32(tot);
  if (lane == 0) {
    s_w[0][wave] = before;
    s_w[1][wave] = tot;
  }
  __syncthreads();
  before = s_w[0][0] + s_w[0][1] + s_w[0][2] + s_w[0][3];
  tot = s_w[1][0] + s_w[1][1] + s_w[1][2] + s_w[1][3];
  const int mode = 3 * tot > c ? 1 : 0;
  if (blockIdx.x == 0 && tid == 0) {
    hs[0] = tot;
    hs[1] = mode;
    hs[2] = 0;
    if (inc.work != nullptr) inc.work[bh] += (unsigned long long)n * (mode != 0 ? c : tot);
  }
  if (mode != 0) return;
  __syncthreads();  // s_w is reused
  const int f = (k < c && fp[k] != 0) ? 1 : 0;
  const int incl = wave_incl_scan_i32(f);
  if (lane == 63) s_w[0][wave] = incl;
  __syncthreads();
  int q = before + incl - f;
  for (int w = 0; w < wave; ++w) q += s_w[0][w];
  if (f) {
    inc.mlist[(size_t)bh * c + q] = k;
    const uint4 *st = reinterpret_cast<const uint4 *>(frags) + ((size_t)bh * ntile + k / 32) * TL::U4;
    uint4 *dt = reinterpret_cast<uint4 *>(inc.cfrags) +
                ((size_t)bh * ntile + q / 32) * TL::U4;
    const int ms = k % 32, md = q % 32;
#pragma unroll
    for (int s = 0; s < TL::KS; ++s) {
      dt[s * 64 + md] = st[s * 64 + ms];
      dt[s * 64 + md + 32] = st[s * 64 + ms + 32];
    }
    reinterpret_cast<float *>(dt + TL::KS * 64)[md] =
        reinterpret_cast<const float *>(st + TL::KS * 64)[ms];
  }
}

// ---------------------------------------------------------------- fp32 assign
// fp32 keys: plain VALU, one key per thread, centroids broadcast from LDS.
template <int D>
__global__ void k_halfnorm_f32(const float *__restrict__ cent, float *__restrict__ hn, long total) {
  const long i = blockIdx.x * (long)blockDim.x + threadIdx.x;
  if (i >= total) return;
  const float *row = cent + i * D;
  float s = 0.f;
  for (int e = 0; e < D; ++e) s = fmaf(row[e], row[e], s);
  hn[i] = 0.5f * s;
}

template <int D>
__global__ void __launch_bounds__(256) k_assign_f32(const float *__restrict__ keys,
                                                    const float *__restrict__ cent,
                                                    const float *__restrict__ hn,
                                                    int32_t *__restrict__ labels, int n, int c) {
  constexpr int CB = 32;
  __shared__ float sc[CB][D];
  __shared__ float sh[CB];
  const int bh = blockIdx.y;
  const int key = blockIdx.x * 256 + threadIdx.x;
  float x[D];
  const float *krow = keys + ((size_t)bh * n + (key < n ? key : 0)) * D;
#pragma unroll
  for (int e = 0; e < D; ++e) x[e] = krow[e];
  float best = -INFINITY;
  int bi = 0;
  for (int c0 = 0; c0 < c; c0 += CB) {
    __syncthreads();
    for (int i = threadIdx.x; i < CB * D; i += 256) {
      const int k = c0 + i / D;
      sc[i / D][i % D] = k < c ? cent[((size_t)bh * c + k) * D + i % D] : 0.f;
    }
    for (int i = threadIdx.x; i < CB; i += 256) sh[i] = c0 + i < c ? hn[(size_t)bh * c + c0 + i] : 0.f;
    __syncthreads();
    const int lim = c - c0 < CB ? c - c0 : CB;
    for (int j = 0; j < lim; ++j) {
      float s = -sh[j];
#pragma unroll
      for (int e = 0; e < D; ++e) s = fmaf(x[e], sc[j][e], s);
      if (s > best) { best = s; bi = c0 + j; }
    }
  }
  if (key < n) labels[(size_t)bh * n + key] = bi;
}

size_t assign_ws_bytes(int bh, int c, int d, kv_dtype dt) {
  if (dt == KV_BF16) {
    const size_t ntile = (size_t)(c + 31) / 32;
    return align_up((size_t)bh * ntile * ((size_t)(d / 16) * 64 + kNormU4) * 16, 256);
  }
  return align_up((size_t)bh * c * sizeof(float), 256);
}

kv_status launch_prep_frags(const float *cent, int bh, int d, int c, void *ws, hipStream_t s) {
  const int ntile = (c + 31) / 32;
  uint16_t *frags = static_cast<uint16_t *>(ws);
  if (d == 128)
    k_prep_frags<128><<<dim3((ntile * 32 + 15) / 16, bh), 256, 0, s>>>(cent, frags, c, ntile);
  else
    k_prep_frags<64><<<dim3((ntile * 32 + 31) / 32, bh), 256, 0, s>>>(cent, frags, c, ntile);
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

kv_status launch_assign_prepare(const float *cent, int bh, int d, int c, kv_dtype dt, void *ws,
                                hipStream_t s) {
  if (dt == KV_BF16) return launch_prep_frags(cent, bh, d, c, ws, s);
  float *hn = static_cast<float *>(ws);
  const long tot = (long)bh * c;
  if (d == 128)
    k_halfnorm_f32<128><<<(unsigned)((tot + 255) / 256), 256, 0, s>>>(cent, hn, tot);
  else
    k_halfnorm_f32<64><<<(unsigned)((tot + 255) / 256), 256, 0, s>>>(cent, hn, tot);
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

kv_status launch_assign_prepared(const void *keys, const float *cent, int bh, int n, int d, int c,
                                 kv_dtype dt, int32_t *labels, const void *ws, hipStream_t s,
                                 LloydSkip skip) {
  if (dt == KV_BF16) {
    const int ntile = (c + 31) / 32;
    const uint16_t *frags = static_cast<const uint16_t *>(ws);
    constexpr int NCB = kAssignColBlocks;
    constexpr int KPB = kAssignWaves * 32 * NCB;  // keys per workgroup
    const int bph = (n + KPB - 1) / KPB;
    const int total = bph * bh;
    if (d == 128)
      k_assign_mfma<128, NCB, kAssignMinWaves, kAssignFull><<<total, 64 * kAssignWaves, 0, s>>>(
          (const uint16_t *)keys, frags, labels, n, c, ntile, bph, total, skip.conv, skip.chg,
          AssignInc{});
    else
      k_assign_mfma<64, NCB, kAssignMinWaves, kAssignFull><<<total, 64 * kAssignWaves, 0, s>>>(
          (const uint16_t *)keys, frags, labels, n, c, ntile, bph, total, skip.conv, skip.chg,
          AssignInc{});
  } else {
    const float *hn = static_cast<const float *>(ws);
    const dim3 grid((n + 255) / 256, bh);
    if (d == 128)
      k_assign_f32<128><<<grid, 256, 0, s>>>((const float *)keys, cent, hn, labels, n, c);
    else
      k_assign_f32<64><<<grid, 256, 0, s>>>((const float *)keys, cent, hn, labels, n, c);
  }
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

size_t assign_inc_ws_bytes(int bh, int n, int c, int d) {
  const size_t ntile = (size_t)(c + 31) / 32, nw = (size_t)(n + 63) / 64;
  size_t b = 0;
  b += align_up((size_t)bh * n * 4, 256);                                        // own
  b += align_up((size_t)bh * nw * 4, 256);                                       // koff
  b += 2 * align_up((size_t)bh * c * 4, 256);                                    // flags
  b += align_up((size_t)bh * c * 4, 256);                                        // mlist
  b += align_up((size_t)bh * 4 * 4, 256);                                        // hstate
  b += align_up((size_t)bh * ntile * ((size_t)(d / 16) * 64 + kNormU4) * 16, 256);  // cfrags
  b += align_up((size_t)bh * n * 4, 256);                                        // glist
  b += align_up((size_t)bh * n * 8, 256);                                        // gbest
  return b;
}

void assign_inc_ws_carve(void *base, int bh, int n, int c, int d, AssignIncWs *w) {
  const size_t ntile = (size_t)(c + 31) / 32, nw = (size_t)(n + 63) / 64;
  char *p = static_cast<char *>(base);
  auto take = [&](size_t bytes) {
    char *q = p;
    p += align_up(bytes, 256);
    return q;
  };
  w->own = reinterpret_cast<int32_t *>(take((size_t)bh * n * 4));
  w->koff = reinterpret_cast<float *>(take((size_t)bh * nw * 4));
  w->flags[0] = reinterpret_cast<int32_t *>(take((size_t)bh * c * 4));
  w->flags[1] = reinterpret_cast<int32_t *>(take((size_t)bh * c * 4));
  w->mlist = reinterpret_cast<int32_t *>(take((size_t)bh * c * 4));
  w->hstate = reinterpret_cast<int32_t *>(take((size_t)bh * 4 * 4));
  w->cfrags = reinterpret_cast<uint16_t *>(
      take((size_t)bh * ntile * ((size_t)(d / 16) * 64 + kNormU4) * 16));
  w->glist = reinterpret_cast<int32_t *>(take((size_t)bh * n * 4));
  w->gbest = reinterpret_cast<unsigned long long *>(take((size_t)bh * n * 8));
}

// Workgroups of the gathered sweep: one full residency of the chip (one
// 8-wave workgroup per CU: the per-column offsets need more than 128
// registers), looping over the (key group, split) items.
constexpr int kGatherGrid = 256;
constexpr int kGatherMinWaves = 2;

template <int D>
static void assign_round_kernels(const uint16_t *keys, int bh, int n, int c, int32_t *labels,
                                 const uint16_t *frags, const AssignInc &ia, int round,
                                 LloydSkip skip, hipStream_t s) {
  constexpr int NCB = kAssignColBlocks;
  constexpr int KPB = kAssignWaves * 32 * NCB;
  const int ntile = (c + 31) / 32, bph = (n + KPB - 1) / KPB, total = bph * bh;
  if (round >= 2)
    k_moved_list<D><<<dim3((c + 255) / 256, bh), 256, 0, s>>>(frags, n, c, ntile, skip.conv,
                                                               round == 2 ? 1 : 0, ia);
  k_assign_mfma<D, NCB, kAssignMinWaves, kAssignFull><<<total, 64 * kAssignWaves, 0, s>>>(
      keys, frags, labels, n, c, ntile, bph, total, skip.conv, skip.chg, ia);
  if (round >= 3) {
    k_assign_mfma<D, NCB, kAssignMinWaves, kAssignMoved><<<total, 64 * kAssignWaves, 0, s>>>(
        keys, frags, labels, n, c, ntile, bph, total, skip.conv, skip.chg, ia);
    k_assign_mfma<D, NCB, kGatherMinWaves, kAssignGather>
        <<<kGatherGrid, 64 * kAssignWaves, 0, s>>>(keys, frags, labels, n, c, ntile, bph, total,
                                                    skip.conv, skip.chg, ia);
    k_assign_gathered_finish<<<dim3(16, bh), 256, 0, s>>>(labels, n, c, skip.conv, skip.chg, ia);
  }
}

kv_status launch_assign_round(const void *keys, int bh, int n, int d, int c, int32_t *labels,
                              const void *frags, const AssignIncWs &w, int round, LloydSkip skip,
                              hipStream_t s) {
  if (round >= 2 && (skip.conv == nullptr || skip.chg == nullptr)) return KV_ERR_INVALID_ARG;
  AssignInc ia;
  ia.own = w.own;
  ia.koff = w.koff;
  ia.work = w.work;
  if (round >= 2) {
    ia.fprev = w.flags[(round - 1) & 1];
    ia.fcur = w.flags[round & 1];
    ia.mlist = w.mlist;
    ia.hstate = w.hstate;
    ia.cfrags = w.cfrags;
    ia.glist = w.glist;
    ia.gbest = w.gbest;
  }
  const uint16_t *k = static_cast<const uint16_t *>(keys);
  const uint16_t *f = static_cast<const uint16_t *>(frags);
  if (d == 128)
    assign_round_kernels<128>(k, bh, n, c, labels, f, ia, round, skip, s);
  else if (d == 64)
    assign_round_kernels<64>(k, bh, n, c, labels, f, ia, round, skip, s);
  else
    return KV_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

kv_status launch_assign(const void *keys, const float *cent, int bh, int n, int d, int c,
                        kv_dtype dt, int32_t *labels, void *ws, hipStream_t s, bool frags_ready,
                        LloydSkip skip) {
  if (!(frags_ready && dt == KV_BF16)) {
    const kv_status st = launch_assign_prepare(cent, bh, d, c, dt, ws, s);
    if (st != KV_OK) return st;
  }
  return launch_assign_prepared(keys, cent, bh, n, d, c, dt, labels, ws, s, skip);
}

// ---------------------------------------------------------------- update
// Stable counting sort of keys by label, in three passes:
//  k_rank_hist -- one workgroup per chunk of CHUNK keys, its NW waves taking
//                 consecutive parts: the rank of each key among earlier keys
//                 of the chunk with the same label (within a part, label
//                 equality found with one ballot per label bit; then the
//                 label's counts in the earlier parts, added in part order)
//                 and the chunk's label histogram;
//  k_colscan   -- per label, exclusive prefix of the histograms over chunks
//                 and the label's total; per block of 256 labels, each
//                 label's exclusive prefix of totals within the block and
//                 the block's total (cluster start = the sum of the earlier
//                 blocks' totals + the in-block prefix: at most 32 blocks up
//                 to 8192 labels, so every consumer adds them up itself and
//                 no separate scan over labels is launched);
//  k_scatter   -- perm[start[a] + chunk_prefix[a] + rank] = key.
// A label outside [0, c) takes no part: its key gets no rank, no histogram
// count and no place in the permutation (reported through *status when given).
// First kernel of an update round under the fixed-point skip: true when the
// workgroup has nothing to do because head bh has reached its fixed point
// (conv set earlier, or no label changed in this round's assignment, which
// then records the round in conv).
__device__ __forceinline__ bool update_head_done(const int32_t *chg, int32_t *conv, int bh,
                                                 int round) {
  if (chg == nullptr) return false;
  if (conv[bh] != 0) return true;
  if (chg[bh] != 0) return false;
  if (blockIdx.x == 0 && threadIdx.x == 0) conv[bh] = round;
  return true;
}

__global__ void k_rounds_out(const int32_t *__restrict__ conv,
                             const unsigned long long *__restrict__ work,
                             int32_t *__restrict__ rounds, float *__restrict__ sweeps, int bh,
                             int iters, int n, int c) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= bh) return;
  const int r = (conv != nullptr && conv[i] != 0) ? conv[i] : iters;
  if (rounds != nullptr) rounds[i] = r;
  if (sweeps != nullptr)
    sweeps[i] = (work != nullptr && iters > 0)
                    ? (float)(1.0 + (double)work[i] / ((double)n * (double)c))
                    : (float)r;
}

kv_status launch_rounds_out(const int32_t *conv, const unsigned long long *work, int32_t *rounds,
                            float *sweeps, int bh, int iters, int n, int c, hipStream_t s) {
  k_rounds_out<<<(bh + 255) / 256, 256, 0, s>>>(conv, work, rounds, sweeps, bh, iters, n, c);
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

template <int NW, int CHUNK>
__global__ void __launch_bounds__(64 * NW) k_rank_hist(const int32_t *__restrict__ labels,
                                                       int32_t *__restrict__ rank,
                                                       int32_t *__restrict__ hist, int n, int c,
                                                       int nbits, int nchunk, int32_t *status,
                                                       const int32_t *chg, int32_t *conv,
                                                       int round) {
  constexpr int KPW = CHUNK / NW;  // keys per wave: wave w takes the w-th part of the chunk
  constexpr int SUB = KPW / 64;
  extern __shared__ int32_t cnt[];      // [NW][c]: label counts of each wave's part
  const int bh = blockIdx.y, ch = blockIdx.x;
  if (update_head_done(chg, conv, bh, round)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int32_t *lab = labels + (size_t)bh * n;
  const int base = ch * CHUNK + wave * KPW;
  // all label loads in flight at once (clamped index, masked below; n >= 1)
  int a[SUB];
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub) a[sub] = lab[min(base + sub * 64 + lane, n - 1)];
  bool bad = false;
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub) {
    const int i = base + sub * 64 + lane;
    const int v = i < n ? a[sub] : -1;
    a[sub] = (v >= 0 && v < c) ? v : -1;
    bad |= i < n && a[sub] < 0;
  }
  if (status && bad)
    __hip_atomic_store(status, (int)KV_ERR_INVALID_ARG, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  for (int k = threadIdx.x; k < NW * c; k += 64 * NW) cnt[k] = 0;
  __syncthreads();
  // rank within the wave's part: earlier keys of the part with the same label
  int32_t *mine = cnt + wave * c;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int lr[SUB];
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub) {
    const bool valid = a[sub] >= 0;
    const int v = valid ? a[sub] : 0;
    uint64_t mask = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (v >> b) & 1;
      const uint64_t m = __ballot(bit);
      mask &= bit ? m : ~m;
    }
    lr[sub] = 0;
    if (valid) {
      lr[sub] = mine[v] + __popcll(mask & below);
      if ((mask >> lane) == 1ull) mine[v] += __popcll(mask);
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  // + the same label's keys in the chunk's earlier parts; the chunk histogram
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub) {
    const int i = base + sub * 64 + lane;
    if (a[sub] >= 0) {
      int r = lr[sub];
      for (int w = 0; w < wave; ++w) r += cnt[w * c + a[sub]];
      rank[(size_t)bh * n + i] = r;
    }
  }
  int32_t *hrow = hist + ((size_t)bh * nchunk + ch) * c;
  for (int k = threadIdx.x; k < c; k += 64 * NW) {
    int t = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += cnt[w * c + k];
    hrow[k] = t;
  }
}

constexpr int kLabelBlock = 256;  // labels per k_colscan workgroup

// Start of label blocks: the sum of the totals of blocks 0 .. blk - 1 of
// head bh (one wave; blk <= 64).
__device__ __forceinline__ int label_block_base(const int32_t *__restrict__ agg, int nblk,
                                                int bh, int blk) {
  const int lane = threadIdx.x & 63;
  return wave_sum_i32(lane < blk ? agg[(size_t)bh * nblk + lane] : 0);
}

__global__ void __launch_bounds__(kLabelBlock)
    k_colscan(int32_t *__restrict__ hist, int32_t *__restrict__ tot, int32_t *__restrict__ ipre,
              int32_t *__restrict__ agg, int32_t *__restrict__ counts, int c, int nchunk,
              const int32_t *conv) {
  __shared__ int wsum[kLabelBlock / 64];
  const int bh = blockIdx.y, k = blockIdx.x * kLabelBlock + threadIdx.x;
  if (conv != nullptr && conv[bh] != 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t run = 0;
  if (k < c) {
    // 32 chunks per memory round trip (clamped loads, masked stores)
    int32_t *col = hist + (size_t)bh * nchunk * c + k;
    for (int ch = 0; ch < nchunk; ch += 32) {
      int32_t h[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) h[i] = col[(size_t)min(ch + i, nchunk - 1) * c];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if (ch + i < nchunk) {
          col[(size_t)(ch + i) * c] = run;
          run += h[i];
        }
      }
    }
  }
  // exclusive prefix of the totals within the block of 256 labels
  const int incl = wave_incl_scan_i32(run);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int off = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kLabelBlock / 64; ++w) {
    if (w < wave) off += wsum[w];
    all += wsum[w];
  }
  if (k < c) {
    tot[(size_t)bh * c + k] = run;
    ipre[(size_t)bh * c + k] = off + incl - run;
    if (counts) counts[(size_t)bh * c + k] = run;
  }
  if (threadIdx.x == 0) agg[(size_t)bh * gridDim.x + blockIdx.x] = all;
}

__global__ void __launch_bounds__(256)
    k_scatter(const int32_t *__restrict__ labels, const int32_t *__restrict__ rank,
              const int32_t *__restrict__ hist, const int32_t *__restrict__ ipre,
              const int32_t *__restrict__ agg, int32_t *__restrict__ perm, int n, int c,
              int nchunk, int chunk_shift, const int32_t *conv) {
  __shared__ int s_base[64];  // start of each block of 256 labels
  const int bh = blockIdx.y, i = blockIdx.x * 256 + threadIdx.x;
  if (conv != nullptr && conv[bh] != 0) return;
  const int nblk = (c + kLabelBlock - 1) / kLabelBlock;
  // the key's label and rank in one round trip (clamped index; n >= 1)
  const int ic = min(i, n - 1);
  const int lab_i = labels[(size_t)bh * n + ic], rank_i = rank[(size_t)bh * n + ic];
  const int a = i < n ? lab_i : -1;
  if (threadIdx.x < 64) {  // wave 0: exclusive scan of the block totals
    const int lane = threadIdx.x;
    const int v = lane < nblk ? agg[(size_t)bh * nblk + lane] : 0;
    s_base[lane] = wave_incl_scan_i32(v) - v;
  }
  __syncthreads();
  if (i >= n || a < 0 || a >= c) return;  // labels out of range: left out by k_rank_hist too
  const int ch = i >> chunk_shift;
  const int dest = s_base[a / kLabelBlock] + ipre[(size_t)bh * c + a] +
                   hist[((size_t)bh * nchunk + ch) * c + a] + rank_i;
  perm[(size_t)bh * n + dest] = i;
}

// The cluster's member sums (this lane's part of the row, summed over its
// row slot) -> the mean, which replaces the centroid (an empty cluster keeps
// its value), and for bf16 keys the next round's MFMA tiles (fragments and
// norm block).
template <typename T, int D>
__device__ __forceinline__ void segsum_finish(float (&acc)[16 / Elem<T>::kBytes], int cnt, int bh,
                                              int c, int k, int ntile, const float *cent_in,
                                              float *cent_out, uint16_t *__restrict__ frags) {
  constexpr int EPL = 16 / Elem<T>::kBytes;
  constexpr int LPR = D / EPL;
  const int lane = threadIdx.x & 63;
  const int part = lane % LPR, slot = lane / LPR;
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = sum_stride<LPR>(acc[e]);
  float mean[EPL];
  const float *in = cent_in + ((size_t)bh * c + k) * D + part * EPL;
#pragma unroll
  for (int e = 0; e < EPL; ++e) mean[e] = cnt > 0 ? acc[e] / (float)cnt : in[e];
  if (slot == 0) {
    float *out = cent_out + ((size_t)bh * c + k) * D + part * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[e] = mean[e];
  }
  if (frags != nullptr && EPL == 8) {
    // element e0 = 8 part lives in k-step e0 / 16, lane half (e0 % 16) / 8
    uint16_t b[8];
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      b[e] = f32_to_bf16_rne(mean[e % EPL]);
      const float r = bf16_bits_to_f32(b[e]);
      sq = fmaf(r, r, sq);
    }
    sq = group_sum<LPR>(sq);
    const int t = k / 32, m = k % 32, e0 = part * 8;
    uint4 *tile = reinterpret_cast<uint4 *>(frags) + ((size_t)bh * ntile + t) * AssignTile<D>::U4;
    if (slot == 0) {
      uint4 pk;
      pk.x = b[0] | ((uint32_t)b[1] << 16);
      pk.y = b[2] | ((uint32_t)b[3] << 16);
      pk.z = b[4] | ((uint32_t)b[5] << 16);
      pk.w = b[6] | ((uint32_t)b[7] << 16);
      tile[(e0 / 16) * 64 + m + 32 * ((e0 % 16) / 8)] = pk;
    }
    if (lane == 0) write_centroid_norm(tile, AssignTile<D>::KS, m, -0.5f * sq);
  }
}

// One wave per cluster. Lanes split a key row into 16-byte pieces, so one
// wave instruction reads RPI member rows; members are dealt round-robin to
// the RPI row slots, each slot sums its members in key order, and the slots
// are combined in a fixed order (fp32 throughout, so the result is
// reproducible bit for bit). The mean replaces the centroid (an empty
// cluster keeps its value). For bf16 keys the same pass writes the next
// round's MFMA tiles (fragments and norm block), so no separate prep is needed.
// start: the in-block label prefixes of k_colscan on entry; each wave adds
// its block's base and writes the cluster's start back (the pack reads it).
template <typename T, int D>
__global__ void __launch_bounds__(256) k_segsum(int n, int c, int ntile,
                                                const int32_t *__restrict__ tot,
                                                int32_t *__restrict__ start,
                                                const int32_t *__restrict__ agg,
                                                const int32_t *__restrict__ perm,
                                                const T *__restrict__ keys,
                                                const float *cent_in, float *cent_out,
                                                uint16_t *__restrict__ frags,
                                                const int32_t *conv, int32_t *chg,
                                                const int32_t *__restrict__ touched) {
  constexpr int EPL = 16 / Elem<T>::kBytes;  // elements per lane
  constexpr int LPR = D / EPL;               // lanes per row
  constexpr int RPI = 64 / LPR;              // member rows per wave instruction
  constexpr int UNR = 4;
  const int bh = blockIdx.y;
  if (chg != nullptr && blockIdx.x == 0 && threadIdx.x == 0) chg[bh] = 0;  // for the next round
  if (conv != nullptr && conv[bh] != 0) return;
  const int k = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int part = lane % LPR, slot = lane / LPR;
  if (k >= c) return;
  if (touched != nullptr && touched[(size_t)bh * c + k] == 0) return;  // same members as before
  const int cnt = tot[(size_t)bh * c + k];
  const int st = label_block_base(agg, (c + kLabelBlock - 1) / kLabelBlock, bh, k / kLabelBlock) +
                 start[(size_t)bh * c + k];
  if (lane == 0) start[(size_t)bh * c + k] = st;
  const int32_t *p = perm + (size_t)bh * n + st;
  const T *kb = keys + (size_t)bh * n * D + part * EPL;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int j0 = 0; j0 < cnt; j0 += RPI * UNR) {
    uint4 v[UNR];
    bool ok[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int j = j0 + u * RPI + slot;
      ok[u] = j < cnt;
      // clamped (cnt >= 1 here) rather than conditional: the member indices
      // of the step are requested together instead of one wait each
      const int row = p[min(j, cnt - 1)];
      v[u] = *reinterpret_cast<const uint4 *>(kb + (size_t)row * D);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      float f[EPL];
      unpack16<T>(v[u], f);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += ok[u] ? f[e] : 0.f;
    }
  }
  segsum_finish<T, D>(acc, cnt, bh, c, k, ntile, cent_in, cent_out, frags);
}

// ---- two-launch update for the rounds whose permutation nobody reads
// (every Lloyd round but the last of kv_cluster_build): no global scan.
//  k_rank_local   -- per chunk of 1024 keys, the ranks of k_rank_hist, then
//                    the chunk's own exclusive prefix of its label counts and
//                    a stable local sort: local[chunk base + prefix[a] + rank]
//                    = key; per (chunk, label) the entry prefix << 16 | count;
//  k_segsum_local -- per cluster, the chunks' entries in chunk order give its
//                    members in key order (the order the global sort gives),
//                    64 at a time into LDS; then the sums of k_segsum, in the
//                    same order and grouping, so the centroids and tiles are
//                    the same bits.
constexpr int kLocalChunk = 1024;
// A cluster's entries are read one per chunk (a line each), so the two
// launches do not move less data than the four; they save two launches,
// which is what counts when the launches are short: at most 64 chunks per
// head, 4096 labels and 1024 chunks in all (measured: 29 against 35 us per
// round at 8 heads x 32768 keys x 2048 clusters; 352 against 357 us at 128
// heads of that size; 169 against 131 us at 8 heads x 131072 keys x 8192
// clusters).
constexpr int kLocalMaxChunks = 64;  // n <= 65536 keys per head
constexpr int kSegWindow = 64;        // members placed in LDS at a time

template <int NW>
__global__ void __launch_bounds__(64 * NW) k_rank_local(const int32_t *__restrict__ labels,
                                                        int32_t *__restrict__ local,
                                                        int32_t *__restrict__ ltab, int n, int c,
                                                        int nbits, int nchunk, const int32_t *chg,
                                                        int32_t *conv, int round) {
  constexpr int KPW = kLocalChunk / NW;
  constexpr int SUB = KPW / 64;
  extern __shared__ int32_t cnt[];  // [NW][c]: label counts of each wave's part
  const int bh = blockIdx.y, ch = blockIdx.x;
  if (update_head_done(chg, conv, bh, round)) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int32_t *lab = labels + (size_t)bh * n;
  const int base = ch * kLocalChunk + wave * KPW;
  int a[SUB];
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub) a[sub] = lab[min(base + sub * 64 + lane, n - 1)];
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub) {
    const int i = base + sub * 64 + lane;
    const int v = i < n ? a[sub] : -1;
    a[sub] = (v >= 0 && v < c) ? v : -1;
  }
  for (int k = threadIdx.x; k < NW * c; k += 64 * NW) cnt[k] = 0;
  __syncthreads();
  int32_t *mine = cnt + wave * c;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int r[SUB];
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub) {
    const bool valid = a[sub] >= 0;
    const int v = valid ? a[sub] : 0;
    uint64_t mask = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (v >> b) & 1;
      const uint64_t m = __ballot(bit);
      mask &= bit ? m : ~m;
    }
    r[sub] = 0;
    if (valid) {
      r[sub] = mine[v] + __popcll(mask & below);
      if ((mask >> lane) == 1ull) mine[v] += __popcll(mask);
    }
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub)
    if (a[sub] >= 0)
      for (int w = 0; w < wave; ++w) r[sub] += cnt[w * c + a[sub]];
  __syncthreads();  // every rank read before row 0 is overwritten
  // exclusive prefix of the chunk's label counts: wave w takes the labels
  // [w span, (w + 1) span) in tiles of 64 and leaves prefix-within-its-span
  // << 16 | count in row 0; the spans' offsets are added on the way out
  const int span = ((c + NW - 1) / NW + 63) / 64 * 64;
  int carry = 0;
  for (int k0 = wave * span; k0 < min((wave + 1) * span, c); k0 += 64) {
    const int k = k0 + lane;
    int t = 0;
    if (k < c)
      for (int w = 0; w < NW; ++w) t += cnt[w * c + k];
    const int incl = wave_incl_scan_i32(t);
    if (k < c) cnt[k] = ((carry + incl - t) << 16) | t;
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  __syncthreads();
  // where each span starts in the chunk's order: the earlier spans' totals
  // (a span's total is its last label's prefix + count)
  int soff[NW];
  soff[0] = 0;
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    const int last = min(w * span, c) - 1;
    const int e = last >= (w - 1) * span ? cnt[last] : 0;
    soff[w] = soff[w - 1] + (e >> 16) + (e & 0xffff);
  }
  auto span_off = [&](int k) {
    int o = 0;
#pragma unroll
    for (int w = 1; w < NW; ++w) o = k >= w * span ? soff[w] : o;
    return o;
  };
  int32_t *trow = ltab + ((size_t)bh * nchunk + ch) * c;
  for (int k = threadIdx.x; k < c; k += 64 * NW) trow[k] = cnt[k] + (span_off(k) << 16);
  int32_t *lrow = local + (size_t)bh * n + (size_t)ch * kLocalChunk;
#pragma unroll
  for (int sub = 0; sub < SUB; ++sub)
    if (a[sub] >= 0)
      lrow[(cnt[a[sub]] >> 16) + span_off(a[sub]) + r[sub]] = base + sub * 64 + lane;
}

template <typename T, int D>
__global__ void __launch_bounds__(256) k_segsum_local(int n, int c, int ntile, int nchunk,
                                                      const int32_t *__restrict__ ltab,
                                                      const int32_t *__restrict__ local,
                                                      const T *__restrict__ keys,
                                                      const float *cent_in, float *cent_out,
                                                      uint16_t *__restrict__ frags,
                                                      const int32_t *conv, int32_t *chg,
                                                      const int32_t *__restrict__ touched) {
  constexpr int EPL = 16 / Elem<T>::kBytes;
  constexpr int LPR = D / EPL;
  constexpr int RPI = 64 / LPR;
  constexpr int UNR = 4;
  static_assert(kSegWindow % (RPI * UNR) == 0, "window holds whole steps");
  if (chg != nullptr && blockIdx.x == 0 && threadIdx.x == 0) chg[blockIdx.y] = 0;  // next round
  if (conv != nullptr && conv[blockIdx.y] != 0) return;
  static_assert(kLocalMaxChunks <= 64, "one chunk per lane");
  __shared__ int s_at[4][kSegWindow];   // positions in `local` of the window's members
  __shared__ int s_mem[4][kSegWindow];  // the window's members
  const int bh = blockIdx.y, wave = threadIdx.x >> 6;
  const int k = blockIdx.x * 4 + wave;
  const int lane = threadIdx.x & 63;
  const int part = lane % LPR, slot = lane / LPR;
  if (k >= c) return;
  if (touched != nullptr && touched[(size_t)bh * c + k] == 0) return;  // same members as before
  // lane = chunk: label k's (prefix, count) entry there; the members of the
  // earlier chunks; where its members start in `local`
  const int chn = min(lane, nchunk - 1);
  const int e = ltab[((size_t)bh * nchunk + chn) * c + k];
  const int m = lane < nchunk ? (e & 0xffff) : 0;
  const int incl = wave_incl_scan_i32(m);
  const int pre = incl - m, at = chn * kLocalChunk + (e >> 16);
  const int cnt = __builtin_amdgcn_readlane(incl, 63);
  const int32_t *lrow = local + (size_t)bh * n;
  const T *kb = keys + (size_t)bh * n * D + part * EPL;
  float acc[EPL];
#pragma unroll
  for (int q = 0; q < EPL; ++q) acc[q] = 0.f;
  for (int w0 = 0; w0 < cnt; w0 += kSegWindow) {
    // each chunk places the positions of its members that fall in the window
    // (LDS only), then every lane loads one member
    const int i1 = min(pre + m, w0 + kSegWindow);
    for (int i = max(pre, w0); i < i1; ++i) s_at[wave][i - w0] = at + (i - pre);
    __builtin_amdgcn_wave_barrier();
    const int id = lrow[s_at[wave][min(w0 + lane, cnt - 1) - w0]];
    __builtin_amdgcn_wave_barrier();
    s_mem[wave][lane] = id;
    __builtin_amdgcn_wave_barrier();
    const int wend = min(w0 + kSegWindow, cnt);
    for (int j0 = w0; j0 < wend; j0 += RPI * UNR) {
      uint4 v[UNR];
      bool ok[UNR];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const int j = j0 + u * RPI + slot;
        ok[u] = j < cnt;
        const int row = s_mem[wave][min(j, cnt - 1) - w0];
        v[u] = *reinterpret_cast<const uint4 *>(kb + (size_t)row * D);
      }
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        float f[EPL];
        unpack16<T>(v[u], f);
#pragma unroll
        for (int q = 0; q < EPL; ++q) acc[q] += ok[u] ? f[q] : 0.f;
      }
    }
  }
  segsum_finish<T, D>(acc, cnt, bh, c, k, ntile, cent_in, cent_out, frags);
}

static int ceil_log2(int c) {
  int b = 0;
  while ((1 << b) < c) ++b;
  return b;
}

// Keys per counting-sort chunk. A chunk's waves rank their parts one 64-key
// step after another, so longer chunks rank more slowly per key; they pay
// only where the chunk histograms (chunks x labels counts per head) dominate
// the traffic and there are enough keys for >= 1024 workgroups of 4096:
// 4096 keys for 1024 < c <= 4096 (4 waves), else 1024.
static int rank_chunk(int bh, int n, int c) {
  return (c > 1024 && c <= 4096 && (long)bh * n >= 4096L * 1024) ? 4096 : 1024;
}

size_t update_ws_bytes(int bh, int n, int c) {
  const size_t nchunk = (size_t)(n + 1023) / 1024;  // the smallest chunk: an upper bound
  size_t b = 0;
  b += align_up((size_t)bh * n * 4, 256);           // rank
  b += align_up((size_t)bh * nchunk * c * 4, 256);  // hist
  b += align_up((size_t)bh * c * 4, 256);           // tot
  b += align_up((size_t)bh * c * 4, 256);           // start
  b += align_up((size_t)bh * n * 4, 256);           // perm
  b += align_up((size_t)bh * ((c + kLabelBlock - 1) / kLabelBlock) * 4, 256);  // block totals
  return b;
}

kv_status launch_update(const void *keys, const int32_t *labels, const float *cent_in,
                        float *cent_out, int32_t *counts, int bh, int n, int d, int c,
                        kv_dtype dt, void *ws, hipStream_t s, const int32_t **perm_out,
                        const int32_t **start_out, const int32_t **tot_out, void *frags_out,
                        int32_t *status, LloydSkip skip) {
  const int chunk = rank_chunk(bh, n, c), nchunk = (n + chunk - 1) / chunk;
  char *w = static_cast<char *>(ws);
  int32_t *rank = reinterpret_cast<int32_t *>(w);
  w += align_up((size_t)bh * n * 4, 256);
  int32_t *hist = reinterpret_cast<int32_t *>(w);
  w += align_up((size_t)bh * ((n + 1023) / 1024) * c * 4, 256);
  int32_t *tot = reinterpret_cast<int32_t *>(w);
  w += align_up((size_t)bh * c * 4, 256);
  int32_t *start = reinterpret_cast<int32_t *>(w);
  w += align_up((size_t)bh * c * 4, 256);
  int32_t *perm = reinterpret_cast<int32_t *>(w);
  w += align_up((size_t)bh * n * 4, 256);
  int32_t *agg = reinterpret_cast<int32_t *>(w);
  const int nblk = (c + kLabelBlock - 1) / kLabelBlock;

  // a chunk's label counts ([waves][c] int32) stay within 64 KB of LDS: 4 waves
  // per chunk up to 4096 labels, 2 up to kMaxClusters = 8192
  if (c > kMaxClusters) return KV_ERR_UNSUPPORTED;
  const dim3 rg(nchunk, bh);
  if (chunk == 1024 && c <= 4096)
    k_rank_hist<4, 1024><<<rg, 256, (size_t)4 * c * 4, s>>>(labels, rank, hist, n, c,
                                                            ceil_log2(c), nchunk, status, skip.chg,
                                                            skip.conv, skip.round);
  else if (c <= 4096)
    k_rank_hist<4, 4096><<<rg, 256, (size_t)4 * c * 4, s>>>(labels, rank, hist, n, c,
                                                            ceil_log2(c), nchunk, status, skip.chg,
                                                            skip.conv, skip.round);
  else
    k_rank_hist<2, 1024><<<rg, 128, (size_t)2 * c * 4, s>>>(labels, rank, hist, n, c,
                                                            ceil_log2(c), nchunk, status, skip.chg,
                                                            skip.conv, skip.round);
  k_colscan<<<dim3(nblk, bh), kLabelBlock, 0, s>>>(hist, tot, start, agg, counts, c, nchunk,
                                                    skip.conv);
  k_scatter<<<dim3((n + 255) / 256, bh), 256, 0, s>>>(labels, rank, hist, start, agg, perm, n, c,
                                                      nchunk, ceil_log2(chunk), skip.conv);
  const dim3 g((c + 3) / 4, bh);
  uint16_t *fr = static_cast<uint16_t *>(frags_out);
  const int ntile = (c + 31) / 32;
  if (dt == KV_BF16) {
    if (d == 128)
      k_segsum<uint16_t, 128><<<g, 256, 0, s>>>(n, c, ntile, tot, start, agg, perm, (const uint16_t *)keys,
                                                cent_in, cent_out, fr, skip.conv, skip.chg, skip.touched);
    else
      k_segsum<uint16_t, 64><<<g, 256, 0, s>>>(n, c, ntile, tot, start, agg, perm, (const uint16_t *)keys,
                                               cent_in, cent_out, fr, skip.conv, skip.chg, skip.touched);
  } else {
    if (d == 128)
      k_segsum<float, 128><<<g, 256, 0, s>>>(n, c, ntile, tot, start, agg, perm, (const float *)keys,
                                             cent_in, cent_out, nullptr, skip.conv, skip.chg, skip.touched);
    else
      k_segsum<float, 64><<<g, 256, 0, s>>>(n, c, ntile, tot, start, agg, perm, (const float *)keys,
                                            cent_in, cent_out, nullptr, skip.conv, skip.chg, skip.touched);
  }
  if (perm_out) *perm_out = perm;
  if (start_out) *start_out = start;
  if (tot_out) *tot_out = tot;
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

bool update_local_ok(int bh, int n, int c) {
  const long nchunk = (n + kLocalChunk - 1) / kLocalChunk;
  return nchunk <= kLocalMaxChunks && c <= 4096 && (long)bh * nchunk <= 1024;
}

kv_status launch_update_local(const void *keys, const int32_t *labels, const float *cent_in,
                              float *cent_out, int bh, int n, int d, int c, kv_dtype dt,
                              void *ws, hipStream_t s, void *frags_out, LloydSkip skip) {
  if (!update_local_ok(bh, n, c)) return KV_ERR_UNSUPPORTED;
  const int nchunk = (n + kLocalChunk - 1) / kLocalChunk;
  // the update workspace's rank and histogram regions hold the local order
  // and the (prefix, count) table
  char *w = static_cast<char *>(ws);
  int32_t *local = reinterpret_cast<int32_t *>(w);
  w += align_up((size_t)bh * n * 4, 256);
  int32_t *ltab = reinterpret_cast<int32_t *>(w);
  const dim3 rg(nchunk, bh);
  k_rank_local<4><<<rg, 256, (size_t)4 * c * 4, s>>>(labels, local, ltab, n, c, ceil_log2(c),
                                                      nchunk, skip.chg, skip.conv, skip.round);
  const dim3 g((c + 3) / 4, bh);
  uint16_t *fr = static_cast<uint16_t *>(frags_out);
  const int ntile = (c + 31) / 32;
  if (dt == KV_BF16) {
    if (d == 128)
      k_segsum_local<uint16_t, 128><<<g, 256, 0, s>>>(n, c, ntile, nchunk, ltab, local,
                                                      (const uint16_t *)keys, cent_in, cent_out, fr, skip.conv, skip.chg, skip.touched);
    else
      k_segsum_local<uint16_t, 64><<<g, 256, 0, s>>>(n, c, ntile, nchunk, ltab, local,
                                                     (const uint16_t *)keys, cent_in, cent_out, fr, skip.conv, skip.chg, skip.touched);
  } else {
    if (d == 128)
      k_segsum_local<float, 128><<<g, 256, 0, s>>>(n, c, ntile, nchunk, ltab, local,
                                                    (const float *)keys, cent_in, cent_out, nullptr, skip.conv, skip.chg, skip.touched);
    else
      k_segsum_local<float, 64><<<g, 256, 0, s>>>(n, c, ntile, nchunk, ltab, local,
                                                   (const float *)keys, cent_in, cent_out, nullptr, skip.conv, skip.chg, skip.touched);
  }
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

// ---------------------------------------------------------------- pack
// Pool row j of head bh takes key perm[j] (K and V), 16 bytes per lane.
template <int ROW_BYTES>
__global__ void __launch_bounds__(256) k_pack_rows(const char *__restrict__ ksrc,
                                                   const char *__restrict__ vsrc,
                                                   const int32_t *__restrict__ perm,
                                                   char *__restrict__ kdst, char *__restrict__ vdst,
                                                   int n, int row_cap) {
  constexpr int LPR = ROW_BYTES / 16;
  constexpr int RPB = 256 / LPR;
  const int bh = blockIdx.y;
  const int j = blockIdx.x * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  if (j >= n) return;
  // rows past the clustered keys (keys whose label was out of range) have no
  // permutation entry; an entry outside [0, n) is never followed
  const int from = perm[(size_t)bh * n + j];
  if (from < 0 || from >= n) return;
  const size_t src = ((size_t)bh * n + from) * ROW_BYTES + part * 16;
  const size_t dst = ((size_t)bh * row_cap + j) * ROW_BYTES + part * 16;
  *reinterpret_cast<uint4 *>(kdst + dst) = *reinterpret_cast<const uint4 *>(ksrc + src);
  *reinterpret_cast<uint4 *>(vdst + dst) = *reinterpret_cast<const uint4 *>(vsrc + src);
}

template <typename T>
__global__ void k_pack_units(const float *__restrict__ cent, const int32_t *__restrict__ start,
                             const int32_t *__restrict__ tot, float *__restrict__ unit_mean,
                             T *__restrict__ unit_index, int32_t *__restrict__ unit_start,
                             int32_t *__restrict__ unit_size, int c, int d, int unit_cap) {
  const int bh = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= c * d) return;
  const int k = i / d, e = i % d;
  const float m = cent[(size_t)bh * c * d + i];
  const size_t o = ((size_t)bh * unit_cap + k) * d + e;
  unit_mean[o] = m;
  unit_index[o] = Elem<T>::from_f32(m);
  if (e == 0) {
    unit_start[(size_t)bh * unit_cap + k] = start[(size_t)bh * c + k];
    unit_size[(size_t)bh * unit_cap + k] = tot[(size_t)bh * c + k];
  }
}

__global__ void k_pack_counters(kv_pool pool, int n, int c) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < pool.batch) {
    pool.n_rows[i] = n;
    pool.n_units[i] = c;
    pool.n_cand[i] = c;
    pool.buf_begin[i] = n;
    pool.seg_begin[i] = n;
  }
  if (pool.seg_sum) {
    const int tot = pool.batch * pool.n_kv_heads * pool.head_dim;
    for (int j = i; j < tot; j += gridDim.x * 256) pool.seg_sum[j] = 0.f;
  }
}

kv_status launch_pack(const kv_pool *pool, const void *keys, const void *values,
                      const float *cent, const int32_t *perm, const int32_t *start,
                      const int32_t *tot, int n, int c, hipStream_t s) {
  const int bh = pool->batch * pool->n_kv_heads;
  const int d = pool->head_dim;
  const int row_bytes = d * (pool->dtype == KV_BF16 ? 2 : 4);
  const int rpb = 256 / (row_bytes / 16);
  const dim3 gr((n + rpb - 1) / rpb, bh);
  const char *ks = (const char *)keys, *vs = (const char *)values;
  char *kd = (char *)pool->k, *vd = (char *)pool->v;
  switch (row_bytes) {
    case 128: k_pack_rows<128><<<gr, 256, 0, s>>>(ks, vs, perm, kd, vd, n, pool->row_cap); break;
    case 256: k_pack_rows<256><<<gr, 256, 0, s>>>(ks, vs, perm, kd, vd, n, pool->row_cap); break;
    case 512: k_pack_rows<512><<<gr, 256, 0, s>>>(ks, vs, perm, kd, vd, n, pool->row_cap); break;
    default: return KV_ERR_UNSUPPORTED;
  }
  const dim3 gu((c * d + 255) / 256, bh);
  if (pool->dtype == KV_BF16)
    k_pack_units<uint16_t><<<gu, 256, 0, s>>>(cent, start, tot, pool->unit_mean,
                                              (uint16_t *)pool->unit_index, pool->unit_start,
                                              pool->unit_size, c, d, pool->unit_cap);
  else
    k_pack_units<float><<<gu, 256, 0, s>>>(cent, start, tot, pool->unit_mean,
                                           (float *)pool->unit_index, pool->unit_start,
                                           pool->unit_size, c, d, pool->unit_cap);
  const int seg_elems = pool->seg_sum ? pool->batch * pool->n_kv_heads * d : 0;
  const int nb = ((pool->batch > seg_elems ? pool->batch : seg_elems) + 255) / 256;
  k_pack_counters<<<nb > 0 ? nb : 1, 256, 0, s>>>(*pool, n, c);
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

}  // namespace kvc

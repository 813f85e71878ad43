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

constexpr int kAssignKeysPerWave = 64;                   // two 32-key MFMA column blocks
constexpr int kAssignWaves = 4;
constexpr int kAssignKeysPerBlock = kAssignKeysPerWave * kAssignWaves;
constexpr int kTilesPerStage = 2;                        // 64 centroids per LDS stage
constexpr int kRankChunk = 1024;                         // keys per counting-sort chunk

// ---------------------------------------------------------------- init
template <typename T>
__global__ void k_init_centroids(const T *__restrict__ keys, const int32_t *__restrict__ init_idx,
                                 float *__restrict__ cent, int n, int c, int d, long total) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total;
       i += (long)gridDim.x * blockDim.x) {
    const long bh = i / ((long)c * d);
    const int k = (int)((i / d) % c), e = (int)(i % d);
    const int src = init_idx[bh * c + k];
    cent[i] = Elem<T>::to_f32(keys[(bh * n + src) * d + e]);
  }
}

kv_status launch_init_centroids(const void *keys, const int32_t *init_idx, float *cent, int bh,
                                int n, int c, int d, kv_dtype dt, hipStream_t s) {
  const long total = (long)bh * c * d;
  const int blocks = (int)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  if (dt == KV_BF16)
    k_init_centroids<uint16_t><<<blocks, 256, 0, s>>>((const uint16_t *)keys, init_idx, cent, n,
                                                      c, d, total);
  else
    k_init_centroids<float><<<blocks, 256, 0, s>>>((const float *)keys, init_idx, cent, n, c, d,
                                                   total);
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

// ---------------------------------------------------------------- bf16 assign
// Centroid fragments for v_mfma_f32_32x32x16_bf16 with centroids as the A
// operand (32 rows x 16 k per instruction): for tile t, k-step s and lane l,
// the lane holds row m = l % 32 and k = 16 s + 8 (l / 32) + j, j = 0..7.
// The last k-step carries the bias: for lanes l < 32, k = D..D+2 hold
// -(hi, mid, lo) with hi + mid + lo = |c^|^2 / 2 split into three bf16 parts
// (about 24 significant bits), while the keys' matching entries are 1.0, so
// the MFMA accumulates x . c^ - |c^|^2 / 2 directly. Padding rows (k >= C)
// get a bias of -3.39e38 and never win.
template <int D>
__global__ void __launch_bounds__(64) k_prep_frags(const float *__restrict__ cent,
                                                   uint16_t *__restrict__ frags, int c, int ntile) {
  constexpr int KS = D / 16 + 1;
  const int bh = blockIdx.y, t = blockIdx.x, l = threadIdx.x;
  const int m = l & 31, half = l >> 5, k = t * 32 + m;
  const bool real = k < c;
  const float *row = cent + ((size_t)bh * c + (real ? k : 0)) * D;
  uint16_t *out = frags + ((size_t)bh * ntile + t) * KS * 64 * 8;
  float sq = 0.f;
#pragma unroll
  for (int s = 0; s < KS - 1; ++s) {
    uint16_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = real ? row[16 * s + 8 * half + j] : 0.f;
      v[j] = f32_to_bf16_rne(x);
      const float xr = bf16_bits_to_f32(v[j]);
      sq = fmaf(xr, xr, sq);
    }
    uint4 pk;
    pk.x = v[0] | ((uint32_t)v[1] << 16);
    pk.y = v[2] | ((uint32_t)v[3] << 16);
    pk.z = v[4] | ((uint32_t)v[5] << 16);
    pk.w = v[6] | ((uint32_t)v[7] << 16);
    *reinterpret_cast<uint4 *>(out + ((size_t)s * 64 + l) * 8) = pk;
  }
  sq += __shfl_xor(sq, 32);
  const float halfsq = 0.5f * sq;
  const uint16_t hi = f32_to_bf16_rne(halfsq);
  const float r1 = halfsq - bf16_bits_to_f32(hi);
  const uint16_t mid = f32_to_bf16_rne(r1);
  const float r2 = r1 - bf16_bits_to_f32(mid);
  const uint16_t lo = f32_to_bf16_rne(r2);
  uint4 pk = {0u, 0u, 0u, 0u};
  if (half == 0) {
    if (real) {
      pk.x = (uint32_t)(hi ^ 0x8000u) | ((uint32_t)(mid ^ 0x8000u) << 16);
      pk.y = (uint32_t)(lo ^ 0x8000u);
    } else {
      pk.x = 0xff7fu;  // bf16 -3.39e38
    }
  }
  *reinterpret_cast<uint4 *>(out + ((size_t)(KS - 1) * 64 + l) * 8) = pk;
}

// One workgroup = 4 waves x 64 keys. Keys are the B operand (column n = key),
// resident in VGPRs for the whole centroid sweep; centroid tiles stream
// through double-buffered LDS. Each lane sees one key and 16 centroid rows
// per tile, so the running argmax is two registers per column block and the
// final merge is one exchange with lane ^ 32.
template <int D>
__global__ void __launch_bounds__(256, 2)
    k_assign_mfma(const uint16_t *__restrict__ keys, const uint16_t *__restrict__ frags,
                  int32_t *__restrict__ labels, int n, int c, int ntile, int blocks_per_head,
                  int total_blocks) {
  constexpr int KS = D / 16 + 1;
  constexpr int STAGE_U4 = kTilesPerStage * KS * 64;  // 16-byte units per stage
  constexpr int PF = (STAGE_U4 + 255) / 256;          // prefetch registers per thread
  __shared__ uint4 lds[2][STAGE_U4];

  const int bid = xcd_remap(blockIdx.x, total_blocks);
  const int bh = bid / blocks_per_head;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int key0 = (bid % blocks_per_head) * kAssignKeysPerBlock + wave * kAssignKeysPerWave;
  const int half = lane >> 5;

  // Key fragments (B operand): lane holds key n = lane % 32, k = 16 s + 8 half + j.
  bf16x8_t bfrag[2][KS];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int key = key0 + cb * 32 + (lane & 31);
    const uint16_t *krow = keys + ((size_t)bh * n + (key < n ? key : 0)) * D;
#pragma unroll
    for (int s = 0; s < KS - 1; ++s) {
      uint4 v = {0u, 0u, 0u, 0u};
      if (key < n) v = *reinterpret_cast<const uint4 *>(krow + 16 * s + 8 * half);
      bfrag[cb][s] = __builtin_bit_cast(bf16x8_t, v);
    }
    uint4 aug = {0u, 0u, 0u, 0u};
    if (half == 0) {
      aug.x = 0x3f803f80u;  // 1.0, 1.0
      aug.y = 0x00003f80u;  // 1.0, 0
    }
    bfrag[cb][KS - 1] = __builtin_bit_cast(bf16x8_t, aug);
  }

  float best[2] = {-INFINITY, -INFINITY};
  int bidx[2] = {0, 0};

  const uint4 *gfr = reinterpret_cast<const uint4 *>(frags) + (size_t)bh * ntile * KS * 64;
  const int nstage = (ntile + kTilesPerStage - 1) / kTilesPerStage;
  const int tile_u4 = KS * 64;

  uint4 pf[PF];
  auto fetch = [&](int st) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int u = threadIdx.x + i * 256;
      const int t = st * kTilesPerStage + u / tile_u4;
      if (u < STAGE_U4 && t < ntile) pf[i] = gfr[(size_t)st * STAGE_U4 + u];
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int u = threadIdx.x + i * 256;
      if (u < STAGE_U4) lds[buf][u] = pf[i];
    }
  };

  fetch(0);
  stash(0);
  __syncthreads();
  for (int st = 0; st < nstage; ++st) {
    const int buf = st & 1;
    if (st + 1 < nstage) fetch(st + 1);
#pragma unroll
    for (int tt = 0; tt < kTilesPerStage; ++tt) {
      const int t = st * kTilesPerStage + tt;
      if (t >= ntile) break;
      f32x16_t acc0 = {}, acc1 = {};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, lds[buf][(tt * KS + s) * 64 + lane]);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bfrag[0][s], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bfrag[1][s], acc1, 0, 0, 0);
      }
      // D layout: lane holds column n = lane % 32 and rows 8 (r / 4) + 4 half + r % 4.
      if (t * 32 + 32 <= c) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int idx = t * 32 + 8 * (r >> 2) + (r & 3);
          if (acc0[r] > best[0]) { best[0] = acc0[r]; bidx[0] = idx; }
          if (acc1[r] > best[1]) { best[1] = acc1[r]; bidx[1] = idx; }
        }
      } else {  // ragged last tile: padding rows never take part
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int idx = t * 32 + 8 * (r >> 2) + (r & 3);
          const bool real = idx + 4 * half < c;
          if (real && acc0[r] > best[0]) { best[0] = acc0[r]; bidx[0] = idx; }
          if (real && acc1[r] > best[1]) { best[1] = acc1[r]; bidx[1] = idx; }
        }
      }
    }
    if (st + 1 < nstage) stash(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    int idx = bidx[cb] + 4 * half;
    float v = best[cb];
    const float ov = __shfl_xor(v, 32);
    const int oi = __shfl_xor(idx, 32);
    if (ov > v || (ov == v && oi < idx)) { v = ov; idx = oi; }
    const int key = key0 + cb * 32 + (lane & 31);
    if (half == 0 && key < n) labels[(size_t)bh * n + key] = idx;
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
    return align_up((size_t)bh * ntile * (d / 16 + 1) * 64 * 8 * sizeof(uint16_t), 256);
  }
  return align_up((size_t)bh * c * sizeof(float), 256);
}

kv_status launch_assign(const void *keys, const float *cent, int bh, int n, int d, int c,
                        kv_dtype dt, int32_t *labels, void *ws, hipStream_t s) {
  if (dt == KV_BF16) {
    const int ntile = (c + 31) / 32;
    uint16_t *frags = static_cast<uint16_t *>(ws);
    const int bph = (n + kAssignKeysPerBlock - 1) / kAssignKeysPerBlock;
    const int total = bph * bh;
    if (d == 128) {
      k_prep_frags<128><<<dim3(ntile, bh), 64, 0, s>>>(cent, frags, c, ntile);
      k_assign_mfma<128><<<total, 256, 0, s>>>((const uint16_t *)keys, frags, labels, n, c, ntile,
                                              bph, total);
    } else {
      k_prep_frags<64><<<dim3(ntile, bh), 64, 0, s>>>(cent, frags, c, ntile);
      k_assign_mfma<64><<<total, 256, 0, s>>>((const uint16_t *)keys, frags, labels, n, c, ntile,
                                             bph, total);
    }
  } else {
    float *hn = static_cast<float *>(ws);
    const long tot = (long)bh * c;
    const dim3 grid((n + 255) / 256, bh);
    if (d == 128) {
      k_halfnorm_f32<128><<<(unsigned)((tot + 255) / 256), 256, 0, s>>>(cent, hn, tot);
      k_assign_f32<128><<<grid, 256, 0, s>>>((const float *)keys, cent, hn, labels, n, c);
    } else {
      k_halfnorm_f32<64><<<(unsigned)((tot + 255) / 256), 256, 0, s>>>(cent, hn, tot);
      k_assign_f32<64><<<grid, 256, 0, s>>>((const float *)keys, cent, hn, labels, n, c);
    }
  }
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_HIP;
}

// ---------------------------------------------------------------- update
// Stable counting sort of keys by label, in three passes:
//  k_rank_hist -- one wave per chunk of 1024 keys: the rank of each key
//                 among earlier keys of the chunk with the same label (label
//                 equality found with one ballot per label bit) and the
//                 chunk's label histogram;
//  k_colscan   -- per label, exclusive prefix of the histograms over chunks
//                 and the label's total;
//  k_startscan -- exclusive scan of totals over labels (cluster starts);
//  k_scatter   -- perm[start[a] + chunk_prefix[a] + rank] = key.
__global__ void __launch_bounds__(64) k_rank_hist(const int32_t *__restrict__ labels,
                                                  int32_t *__restrict__ rank,
                                                  int32_t *__restrict__ hist, int n, int c,
                                                  int nbits, int nchunk) {
  extern __shared__ int32_t cnt[];
  const int bh = blockIdx.y, ch = blockIdx.x, lane = threadIdx.x;
  for (int k = lane; k < c; k += 64) cnt[k] = 0;
  __syncthreads();
  const int32_t *lab = labels + (size_t)bh * n;
  const int base = ch * kRankChunk;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int sub = 0; sub < kRankChunk; sub += 64) {
    const int i = base + sub + lane;
    const bool valid = i < n;
    const int a = valid ? lab[i] : 0;
    uint64_t mask = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (a >> b) & 1;
      const uint64_t m = __ballot(bit);
      mask &= bit ? m : ~m;
    }
    if (valid) {
      const int r = cnt[a] + __popcll(mask & below);
      rank[(size_t)bh * n + i] = r;
      if ((mask >> lane) == 1ull) cnt[a] += __popcll(mask);
    }
    __syncthreads();
  }
  int32_t *hrow = hist + ((size_t)bh * nchunk + ch) * c;
  for (int k = lane; k < c; k += 64) hrow[k] = cnt[k];
}

__global__ void k_colscan(int32_t *__restrict__ hist, int32_t *__restrict__ tot, int c,
                          int nchunk) {
  const int bh = blockIdx.y, k = blockIdx.x * 256 + threadIdx.x;
  if (k >= c) return;
  int32_t run = 0;
  int32_t *col = hist + (size_t)bh * nchunk * c + k;
  for (int ch = 0; ch < nchunk; ++ch) {
    const int32_t h = col[(size_t)ch * c];
    col[(size_t)ch * c] = run;
    run += h;
  }
  tot[(size_t)bh * c + k] = run;
}

// Block-wide exclusive scan of one int per thread (1024 threads); returns the
// exclusive prefix and writes the block total to *total.
__device__ int block_exclusive_scan_1024(int v, int *total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int off = 0, all = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    if (w < wave) off += wsum[w];
    all += wsum[w];
  }
  __syncthreads();
  *total = all;
  return off + incl - v;
}

__global__ void __launch_bounds__(1024) k_startscan(const int32_t *__restrict__ tot,
                                                    int32_t *__restrict__ start,
                                                    int32_t *__restrict__ counts, int c) {
  const int bh = blockIdx.x;
  const int per = (c + 1023) / 1024;
  const int lo = threadIdx.x * per;
  const int hi = lo + per < c ? lo + per : c;
  const int32_t *t = tot + (size_t)bh * c;
  int local = 0;
  for (int k = lo; k < hi; ++k) local += t[k];
  int total;
  int run = block_exclusive_scan_1024(local, &total);
  for (int k = lo; k < hi; ++k) {
    start[(size_t)bh * c + k] = run;
    if (counts) counts[(size_t)bh * c + k] = t[k];
    run += t[k];
  }
}

__global__ void k_scatter(const int32_t *__restrict__ labels, const int32_t *__restrict__ rank,
                          const int32_t *__restrict__ hist, const int32_t *__restrict__ start,
                          int32_t *__restrict__ perm, int n, int c, int nchunk) {
  const int bh = blockIdx.y, i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int a = labels[(size_t)bh * n + i];
  const int ch = i / kRankChunk;
  const int dest = start[(size_t)bh * c + a] + hist[((size_t)bh * nchunk + ch) * c + a] +
                   rank[(size_t)bh * n + i];
  perm[(size_t)bh * n + dest] = i;
}

// One wave per cluster: members summed in key order (fp32), then divided.
template <typename T, int D>
__global__ void __launch_bounds__(256) k_segsum(const T *__restrict__ keys,
                                                const int32_t *__restrict__ perm,
                                                const int32_t *__restrict__ start,
                                                const int32_t *__restrict__ tot,
                                                const float *cent_in, float *cent_out, int n,
                                                int c) {
  constexpr int EPL = D / 64;
  const int bh = blockIdx.y;
  const int k = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (k >= c) return;
  const int cnt = tot[(size_t)bh * c + k];
  const int st = start[(size_t)bh * c + k];
  const int32_t *p = perm + (size_t)bh * n + st;
  const T *kb = keys + (size_t)bh * n * D + lane * EPL;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  int j = 0;
  for (; j + 4 <= cnt; j += 4) {
    T v[4][EPL];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const T *row = kb + (size_t)p[j + u] * D;
#pragma unroll
      for (int e = 0; e < EPL; ++e) v[u][e] = row[e];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] += Elem<T>::to_f32(v[u][e]);
  }
  for (; j < cnt; ++j) {
    const T *row = kb + (size_t)p[j] * D;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += Elem<T>::to_f32(row[e]);
  }
  float *out = cent_out + ((size_t)bh * c + k) * D + lane * EPL;
  const float *in = cent_in + ((size_t)bh * c + k) * D + lane * EPL;
#pragma unroll
  for (int e = 0; e < EPL; ++e) out[e] = cnt > 0 ? acc[e] / (float)cnt : in[e];
}

static int ceil_log2(int c) {
  int b = 0;
  while ((1 << b) < c) ++b;
  return b;
}

size_t update_ws_bytes(int bh, int n, int c) {
  const size_t nchunk = (size_t)(n + kRankChunk - 1) / kRankChunk;
  size_t b = 0;
  b += align_up((size_t)bh * n * 4, 256);           // rank
  b += align_up((size_t)bh * nchunk * c * 4, 256);  // hist
  b += align_up((size_t)bh * c * 4, 256);           // tot
  b += align_up((size_t)bh * c * 4, 256);           // start
  b += align_up((size_t)bh * n * 4, 256);           // perm
  return b;
}

kv_status launch_update(const void *keys, const int32_t *labels, const float *cent_in,
                        float *cent_out, int32_t *counts, int bh, int n, int d, int c,
                        kv_dtype dt, void *ws, hipStream_t s, const int32_t **perm_out,
                        const int32_t **start_out, const int32_t **tot_out) {
  const int nchunk = (n + kRankChunk - 1) / kRankChunk;
  char *w = static_cast<char *>(ws);
  int32_t *rank = reinterpret_cast<int32_t *>(w);
  w += align_up((size_t)bh * n * 4, 256);
  int32_t *hist = reinterpret_cast<int32_t *>(w);
  w += align_up((size_t)bh * nchunk * c * 4, 256);
  int32_t *tot = reinterpret_cast<int32_t *>(w);
  w += align_up((size_t)bh * c * 4, 256);
  int32_t *start = reinterpret_cast<int32_t *>(w);
  w += align_up((size_t)bh * c * 4, 256);
  int32_t *perm = reinterpret_cast<int32_t *>(w);

  k_rank_hist<<<dim3(nchunk, bh), 64, (size_t)c * 4, s>>>(labels, rank, hist, n, c,
                                                          ceil_log2(c), nchunk);
  k_colscan<<<dim3((c + 255) / 256, bh), 256, 0, s>>>(hist, tot, c, nchunk);
  k_startscan<<<bh, 1024, 0, s>>>(tot, start, counts, c);
  k_scatter<<<dim3((n + 255) / 256, bh), 256, 0, s>>>(labels, rank, hist, start, perm, n, c,
                                                      nchunk);
  const dim3 g((c + 3) / 4, bh);
  if (dt == KV_BF16) {
    if (d == 128)
      k_segsum<uint16_t, 128><<<g, 256, 0, s>>>((const uint16_t *)keys, perm, start, tot, cent_in,
                                                cent_out, n, c);
    else
      k_segsum<uint16_t, 64><<<g, 256, 0, s>>>((const uint16_t *)keys, perm, start, tot, cent_in,
                                               cent_out, n, c);
  } else {
    if (d == 128)
      k_segsum<float, 128><<<g, 256, 0, s>>>((const float *)keys, perm, start, tot, cent_in,
                                             cent_out, n, c);
    else
      k_segsum<float, 64><<<g, 256, 0, s>>>((const float *)keys, perm, start, tot, cent_in,
                                            cent_out, n, c);
  }
  if (perm_out) *perm_out = perm;
  if (start_out) *start_out = start;
  if (tot_out) *tot_out = tot;
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
  const size_t src = ((size_t)bh * n + perm[(size_t)bh * n + j]) * ROW_BYTES + part * 16;
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

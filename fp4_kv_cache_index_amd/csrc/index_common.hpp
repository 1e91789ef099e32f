// Pieces shared by the indexer kernels: query positions and visibility, the
// E4M3 query quantisation, raw buffer loads, the scoring core that turns a
// batch of indexer keys into u32 order keys, and the ascending-order writers
// of a selection.
//
// Index score of entry e for one query (the pages name index scores but give
// no formula; the reading taken is the multi-head ReLU-gated dot product):
//   score = s_k(e) * sum_h (w_h * s_qh) * relu(q8_h . k8(e))
// E4M3 key bytes widen exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8, scale 1)
// and are dotted with the four E4M3 query heads on v_mfma_f32_16x16x32_bf16:
// the products are exact and the matrix core sums them in fp32 to within
// about one ulp of the exact dot (the FP8 matrix paths sum far more coarsely,
// which would move entries across the Top-512 boundary).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "block_ops.hpp"
#include "codec.hpp"
#include "kernels.hpp"

namespace csa2 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kScoreThreads = 512;
constexpr int kScoreWaves = kScoreThreads / 64;
constexpr int kBatch = 4;                              // 16-key groups per wave and batch
constexpr int kBatchKeys = kScoreWaves * kBatch * 16;  // 512 keys scored per batch
constexpr int kBins = 4096;                            // coarse histogram: the top 12 bits of a score key
constexpr int kBinShift = 20;

// ---------------------------------------------------------- query handling
__device__ __forceinline__ int32_t query_pos(const int32_t* q_pos, const int32_t* length, int32_t ratio, int b, int q,
                                             int Q) {
  return q_pos ? q_pos[(int64_t)b * Q + q] : length[b] * ratio - Q + q;
}

// number of entries visible to a query at token p: e < length and (e+1)r-1 <= p
__device__ __forceinline__ int32_t visible_count(int32_t len, int32_t cap, int32_t ratio, int32_t p) {
  if (len > cap) len = cap;
  if (p < 0) return 0;
  const int64_t by_pos = ((int64_t)p + 1) / ratio;
  return (int32_t)(by_pos < len ? by_pos : len);
}

// Quantise the query's four 64-dim heads to E4M3 with s = amax/448 and keep
// c_h = w_h * s_h; one wave per head.  Needs 256 threads, t = 0..255, each
// passing its own query element v = iq[t] and its head's weight wh.
__device__ __forceinline__ void prep_query(float v, float wh, uint8_t* s_q8, float* s_c, int t) {
  const int h = t >> 6;
  const float a = wave_max(fabsf(v));
  const float s = a / 448.0f;
  s_q8[t] = (uint8_t)(s == 0.0f ? 0u : e4m3_encode(v / s));
  if ((t & 63) == 0) s_c[h] = wh * s;
}

// Eight E4M3 bytes (two dwords) widened exactly to eight bf16 values.
__device__ __forceinline__ v8bf widen8(uint32_t w0, uint32_t w1) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  v8bf r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// A raw buffer of `bytes` bytes at p.  A load at an offset past the end
// returns zeros without a memory access, so a load that may not be wanted is
// issued anyway, with no branch around it (the compiler waits for a load under
// a branch before the branch ends, which would serialise a thread's loads).
using BufRsrc = __amdgpu_buffer_rsrc_t;
constexpr int kNT = 2;  // buffer load cache policy: non-temporal (streamed once)

__device__ __forceinline__ BufRsrc make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(BufRsrc r, uint32_t offset) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 0));
}

// ---------------------------------------------------------- scoring core
// One 512-lane workgroup scoring batches of 512 keys for one query.  Batch key
// k (0..511) is entry (Full) or pool slot (Reindex) base + k; wave w scores
// groups 8j + w (j = 0..3) of 16 keys, lane l loading 16 code bytes of key
// l%16 of each and finishing key `row` = l%16 of group jl = l/16: batch key
// own() = 16 (8 jl + w) + row.  Every user of this core gets the same keys for
// the same entries, bit for bit.
struct BatchLoad {
  v4i bytes[kBatch];  // 16 code bytes of key `row` of each of the wave's groups
  float sk;           // the indexer scale of the key this lane finishes
};

template <bool Reindex>
struct Scorer {
  BufRsrc kr, sr;  // the sequence's key codes and scales, bounded at n_vis entries
  int32_t n_vis;
  int lane, wave, row, grp, jl;
  v8bf qa0, qa1;
  float ch0, ch1, ch2, ch3;

  __device__ __forceinline__ void init(const uint8_t* ik_codes, const float* ik_scales, int64_t row_base,
                                       int32_t nv) {
    n_vis = nv;
    lane = threadIdx.x & 63;
    wave = threadIdx.x >> 6;
    row = lane & 15;
    grp = lane >> 4;
    jl = lane >> 4;
    kr = make_rsrc(ik_codes + row_base * 64, (uint32_t)nv * 64u);
    sr = make_rsrc(ik_scales + row_base, (uint32_t)nv * 4u);
  }
  __device__ __forceinline__ int own() const { return 16 * (jl * kScoreWaves + wave) + row; }
  __device__ __forceinline__ int key_of(int j) const { return 16 * (j * kScoreWaves + wave) + row; }

  // A operands from the quantised query (prep_query's s_q8, s_c): lane l holds
  // head l%16 (rows 0-3 used), virtual k = 8(l/16) + i <-> dim 16(l/16) + 8kk + i,
  // the same map the keys use.
  __device__ __forceinline__ void load_query(const uint8_t* s_q8, const float* s_c) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (row < 4) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(s_q8 + row * 64 + 16 * grp);
      w[0] = src[0]; w[1] = src[1]; w[2] = src[2]; w[3] = src[3];
    }
    qa0 = widen8(w[0], w[1]);
    qa1 = widen8(w[2], w[3]);
    ch0 = s_c[0]; ch1 = s_c[1]; ch2 = s_c[2]; ch3 = s_c[3];
  }

  // entry whose key `row` of group j is loaded (n_vis, a zero read, if none)
  __device__ __forceinline__ uint32_t entry(int64_t base, int j, const int32_t (&pe)[kBatch]) const {
    if constexpr (Reindex) {
      return (pe[j] >= 0 && pe[j] < n_vis) ? (uint32_t)pe[j] : (uint32_t)n_vis;
    } else {
      return (uint32_t)(base + key_of(j));
    }
  }

  // Issue the loads of the batch at `base`.  Reindex: pe are the pool entries
  // of the lane's four keys (pool[base + key_of(j)]).  Full: keys past n_vis read
  // zeros without a memory access.
  __device__ __forceinline__ void issue(int64_t base, const int32_t (&pe)[kBatch], BatchLoad& L) const {
    uint32_t es[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; j++) {
      es[j] = entry(base, j, pe);
      L.bytes[j] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(kr, es[j] * 64u + 16u * grp, 0, kNT));
    }
    const uint32_t e_own = jl == 0 ? es[0] : jl == 1 ? es[1] : jl == 2 ? es[2] : es[3];
    L.sk = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, e_own * 4u, 0, 0));
  }

  // The order key of the key this lane finishes (0 when `valid` is false): the
  // four groups' head dots land in lanes 0-15 of d[j]; permlane16/32 swaps
  // gather row 0 of d[j] into row j, so lane 16j + c holds key c of group j.
  __device__ __forceinline__ uint32_t compute(const BatchLoad& L, bool valid) const {
    v4f d[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; j++) {
      d[j] = (v4f){0.f, 0.f, 0.f, 0.f};
      d[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa0, widen8((uint32_t)L.bytes[j][0], (uint32_t)L.bytes[j][1]),
                                                     d[j], 0, 0, 0);
      d[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa1, widen8((uint32_t)L.bytes[j][2], (uint32_t)L.bytes[j][3]),
                                                     d[j], 0, 0, 0);
    }
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t x01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(d[0][i]), __float_as_uint(d[1][i]),
                                                            false, false)[0];
      const uint32_t x23 = __builtin_amdgcn_permlane16_swap(__float_as_uint(d[2][i]), __float_as_uint(d[3][i]),
                                                            false, false)[0];
      x[i] = __uint_as_float(__builtin_amdgcn_permlane32_swap(x01, x23, false, false)[0]);
    }
    float acc = 0.0f;
    acc = __builtin_fmaf(ch0, x[0] > 0.0f ? x[0] : 0.0f, acc);
    acc = __builtin_fmaf(ch1, x[1] > 0.0f ? x[1] : 0.0f, acc);
    acc = __builtin_fmaf(ch2, x[2] > 0.0f ? x[2] : 0.0f, acc);
    acc = __builtin_fmaf(ch3, x[3] > 0.0f ? x[3] : 0.0f, acc);
    return valid ? order_key(L.sk * acc) : 0u;
  }
};

// maximum over each aligned group of 8 lanes (an 8-entry block), in all 8
__device__ __forceinline__ uint32_t block_max8(uint32_t m) {
  m = max(m, dpp<kDppXor1>(m));
  m = max(m, dpp<kDppXor2>(m));
  m = max(m, dpp<kDppHalfMirror>(m));
  return m;
}

// ---------------------------------------------------------- ascending output
constexpr uint32_t kNoId = 0xFFFFFFFFu;
constexpr int kRankWords = 8192;  // rank bitmap words: ids below 262,144

// Rank of each selected id among all of them (ids unique and below `universe`
// <= 32 * kRankWords): one bit per id in an LDS bitmap, each word's offset by a
// prefix count over the words, and an id's rank is its word's offset plus the
// set bits below it in the word.  Thread t holds ids in id[] (kNoId: none).
// `bits` is 2 * kRankWords words of free LDS; `tmp` one int per wave.
template <int kPer>
__device__ void rank_ids(const uint32_t (&id)[kPer], int64_t universe, int (&rank)[kPer], uint32_t* bits, int* tmp) {
  const int tid = threadIdx.x;
  int* woff = reinterpret_cast<int*>(bits + kRankWords);
  const int nw = (int)((universe + 31) >> 5);
  for (int w = tid; w < nw; w += blockDim.x) bits[w] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; j++)
    if (id[j] != kNoId) atomicOr(&bits[id[j] >> 5], 1u << (id[j] & 31u));
  __syncthreads();
  const int wpt = (nw + (int)blockDim.x - 1) / (int)blockDim.x;  // words per thread, contiguous
  const int w0 = tid * wpt, w1 = min(nw, w0 + wpt);
  int cnt = 0;
  for (int w = w0; w < w1; w++) cnt += __popc(bits[w]);
  int tot;
  int pos = block_scan_excl(cnt, tmp, &tot);
  for (int w = w0; w < w1; w++) {
    woff[w] = pos;
    pos += __popc(bits[w]);
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; j++) {
    rank[j] = -1;
    if (id[j] != kNoId) {
      const uint32_t w = id[j] >> 5;
      rank[j] = woff[w] + __popc(bits[w] & ((1u << (id[j] & 31u)) - 1u));
    }
  }
}

// Write the n unique values x[0..n) in ascending order to out[0..n), for id
// ranges too wide for the rank bitmap: values are bucketed by x >> shift (at
// most nb_max buckets, take/off/ge arrays of that many ints), scattered to tmp,
// and placed by their rank inside the bucket.
__device__ inline void order_ascending(const uint32_t* x, int n, int shift, uint32_t* out, uint32_t* tmp, int* take,
                                       int* off, int* ge, int* wtmp) {
  const int tid = threadIdx.x;
  int nbk = 0;
  for (int i = tid; i < n; i += blockDim.x) nbk = max(nbk, (int)(x[i] >> shift) + 1);
  nbk = wave_max(nbk);
  if ((tid & 63) == 0) wtmp[tid >> 6] = nbk;
  __syncthreads();
  nbk = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); w++) nbk = max(nbk, wtmp[w]);
  __syncthreads();
  for (int b = tid; b < nbk; b += blockDim.x) {
    take[b] = 0;
    ge[b] = 0;
  }
  __syncthreads();
  for (int i = tid; i < n; i += blockDim.x) atomicAdd(&take[x[i] >> shift], 1);
  __syncthreads();
  (void)block_offsets(take, off, nbk, wtmp);
  for (int i = tid; i < n; i += blockDim.x) {
    const int b = (int)(x[i] >> shift);
    tmp[off[b] + atomicAdd(&ge[b], 1)] = x[i];
  }
  __syncthreads();
  for (int p = tid; p < n; p += blockDim.x) {
    const uint32_t v = tmp[p];
    const int b = (int)(v >> shift);
    const int lo = off[b], hi = lo + take[b];
    int rank = 0;
    for (int q = lo; q < hi; q++) rank += tmp[q] < v;
    out[lo + rank] = v;
  }
  __syncthreads();
}

}  // namespace csa2

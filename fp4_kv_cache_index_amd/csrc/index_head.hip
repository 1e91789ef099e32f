// Top-512 and candidate-pool selection of the CSA2 Full and Reindex layer
// modes with the score keys kept on chip (DeepSeek-V4.1-Flash report:
// technologiesdigest "CSA2" for the modes and Top-512; ai.info "Methodology in
// Plain English" for the hierarchical pool: the first Full layer keeps the
// 2,048 aligned 8-entry blocks whose largest index score ranks highest).
// Used for one to three queries per sequence and for Reindex; four or more
// queries of a sequence without a pool (prefill chunks) share each key load in
// index_shared_head, which writes heads of the same form; four or more with a
// pool go through the shared-load scorer in index.hip.
//
// Two kernels per call.
//  1. index_head: W workgroups per query each score one share of the keys
//     (Full: batches of 512 entries j, j + W, j + 2W, ... so that the query's
//     workgroups stream one region together; Reindex: pool slots).  Each key
//     becomes a u32 order key held in registers and counted in an LDS
//     histogram of its top 12 bits.  At the end the workgroup finds in its
//     histogram the bin that holds its own T-th largest key and writes every
//     key in a higher bin (and the keys of that bin, unless they would pass the
//     share's cap) to its own stretch of the query's candidate list as u64
//     keys (score << 32 | ~id), with their count and the largest u64 key it
//     did not write (its floor).  With a pool it does the same for the 8-entry
//     block maxima.  With a fused append the workgroup whose batch holds a new
//     entry first writes it to the cache.
//  2. index_select: one workgroup per query and kind gathers the stretches
//     and takes the K-th largest candidate S* (a histogram over the
//     candidates' score range, then an exact rank inside the boundary bin).
//     Every key any workgroup did not write is at most its floor, so when
//     every floor is below S* the candidates at or above S* are the exact
//     Top-K.  Otherwise (a share holding more of the Top-K than it wrote,
//     e.g. clustered scores or wide ties) it re-scores that share with the
//     same scoring core, adds its unwritten keys above S*, and selects again,
//     until no floor is above S*.  The result is written in ascending order
//     (the pool expanded to its entries) from a bitmap of the selected ids.
//     Nothing in the workspace carries over from one call to the next.
// Ties go to the lower index through the u64 key; the order is exact for any
// input.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "block_ops.hpp"
#include "codec.hpp"
#include "dev_check.hpp"
#include "index_common.hpp"
#include "kernels.hpp"
#include "quant_entry.hpp"

namespace csa2 {

constexpr int kFullIters = 9;     // most batches per workgroup, Full (their keys stay in registers)
constexpr int kReindexIters = 2;  // batches per workgroup, Reindex (1,024 pool slots)
constexpr int kResident = 512;    // head workgroups resident at once (two per compute unit)
constexpr int kHeadCap = 8192;    // candidates per query and kind, summed over its workgroups

// Workspace of the head path.  Workgroup j of a query writes its candidates
// of each kind to its own stretch of the query's list, slots [j Tc, j Tc + n)
// with Tc = kHeadCap / W, and n to count; nothing carries over between calls.
struct HeadWs {
  uint32_t* count;  // [BQ][2][wstride] candidates each workgroup wrote (entries or slots, blocks)
  uint64_t* cand;   // [BQ][2][kHeadCap] u64 keys (score << 32 | ~id)
  uint64_t* floor;  // [BQ][2][wstride] largest key a workgroup did not write (0: none)
  uint32_t* cut;    // [BQ][2][wstride] its cut bin << 1 | whether that bin was written
  uint32_t* top;    // [BQ][2][wstride] its largest key (every key it wrote is at most this)
  uint32_t* bot;    // [BQ][2][wstride] the smallest key it wrote (all ones: none)
  int32_t* nvis;    // [BQ][2] entries visible to the query; length to store after a fused append (-1: none)
  int32_t wstride;
};

// ------------------------------------------------------------------ geometry
static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workgroups per query.  Reindex: 16 of 1,024 pool slots.  Full: every share
// gets the same number of batches (at most kFullIters, whose keys stay in
// registers), so the grid should fill whole rounds of the resident slots: the
// fewest rounds that hold the shares needed, and as many shares as those
// rounds hold.
int head_workgroups(bool reindex, int32_t capacity, int64_t bq) {
  if (reindex) return kPool / (kReindexIters * kBatchKeys);
  const int64_t batches = ((int64_t)capacity + kBatchKeys - 1) / kBatchKeys;
  const int64_t w_min = (batches + kFullIters - 1) / kFullIters;
  if (bq < 1) bq = 1;
  const int64_t rounds = (bq * w_min + kResident - 1) / kResident;
  int64_t w = rounds * kResident / bq;
  if (w < w_min) w = w_min;
  if (w > batches) w = batches;
  return (int)(w > 0 ? w : 1);
}

// Workgroups per query of the shared-load heads (four or more queries per
// sequence, no pool): every share holds at most kSharedIters batches.
constexpr int kSharedIters = 8;
int shared_head_workgroups(int32_t capacity) {
  const int64_t batches = ((int64_t)capacity + kBatchKeys - 1) / kBatchKeys;
  const int64_t w = (batches + kSharedIters - 1) / kSharedIters;
  return (int)(w > 0 ? w : 1);
}

static inline int head_wmax(int32_t capacity, int64_t bq) {
  const int a = head_workgroups(false, capacity, bq), b = head_workgroups(true, capacity, bq);
  const int c = shared_head_workgroups(capacity);
  return a > b ? (a > c ? a : c) : (b > c ? b : c);
}

size_t head_ws_bytes(int64_t bq, int32_t capacity) {
  const int64_t W = head_wmax(capacity, bq);
  return 256 + align256(bq * 2 * W * 4) + align256(bq * 2 * kHeadCap * 8) + align256(bq * 2 * W * 8) +
         3 * align256(bq * 2 * W * 4) + align256(bq * 2 * 4);
}

HeadWs head_ws_carve(void* ws, int64_t bq, int32_t capacity) {
  const int64_t W = head_wmax(capacity, bq);
  HeadWs w;
  uint8_t* p = (uint8_t*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  w.count = (uint32_t*)p;
  p += align256(bq * 2 * W * 4);
  w.cand = (uint64_t*)p;
  p += align256(bq * 2 * kHeadCap * 8);
  w.floor = (uint64_t*)p;
  p += align256(bq * 2 * W * 8);
  w.cut = (uint32_t*)p;
  p += align256(bq * 2 * W * 4);
  w.top = (uint32_t*)p;
  p += align256(bq * 2 * W * 4);
  w.bot = (uint32_t*)p;
  p += align256(bq * 2 * W * 4);
  w.nvis = (int32_t*)p;
  w.wstride = (int32_t)W;
  return w;
}

__device__ __forceinline__ uint64_t key64(uint32_t key, uint32_t id) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ uint32_t key_id(uint64_t k) { return 0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull); }

// a key of a share is written to the candidates iff it is nonzero and its bin
// is above the share's cut bin, or equal to it when that bin was written
// max(x, 0) for a finite x, as one integer max on its bits (a negative float
// is a negative integer; -0 gives +0)
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ bool head_written(uint32_t x, uint32_t cut) {
  const uint32_t bn = x >> kBinShift, bt = cut >> 1;
  return x != 0u && (bn > bt || (bn == bt && (cut & 1u)));
}
// head_written as one compare: a key x is written iff x >= the threshold (the
// cut bin's lowest key when that bin is written, else the next bin's, and at
// least 1) and `any` (false when that is past the top bin)
__device__ __forceinline__ uint32_t head_threshold(uint32_t cut, bool& any) {
  const uint64_t thr64 = (uint64_t)((cut >> 1) + ((cut & 1u) ? 0u : 1u)) << kBinShift;
  any = thr64 <= 0xFFFFFFFFull;
  return thr64 > 1ull ? (uint32_t)thr64 : 1u;
}

// Keys a share wants of a kind: 1.25 K live / total + 16, rounded up (0 when
// the query has no key of the kind), through an fp32 reciprocal rather than an
// integer division: K live and total are below 2^24, so exact in fp32, and
// the target needs no exact rounding (the floors keep the selection exact
// whatever a share writes).
__device__ __forceinline__ int share_want(int K, uint32_t live, int64_t total) {
  if (total <= 0) return 0;
  const float x = 1.25f * (float)K * (float)live * __builtin_amdgcn_rcpf((float)total);
  return (int)ceilf(x) + 16;
}

struct HeadLds {
  uint32_t wmax[2][kScoreWaves];    // largest key of each wave, per kind
  uint32_t cut[2], top[2];
  int n[2];                         // keys written, per kind (zero before write_heads)
  uint32_t wlive[2][kScoreWaves];   // each wave's nonzero keys, per kind
  uint64_t wfloor[2][kScoreWaves];  // largest key each wave does not write, per kind
  uint32_t wbot[2][kScoreWaves];    // smallest key each wave writes, per kind
};

// One wave walks a kind's histogram down from the bin of the share's largest
// key mx, 64 bins a step, to the bin bt where the count of keys at or above it
// reaches T.  Returns the cut: bt << 1 | whether bin bt is written too (when
// the keys above it and in it fit in T_cap; otherwise only the keys above it,
// fewer than T, are written).  With fewer than T keys in all, every key is
// written (cut = 0 << 1 | 1).
template <typename CountF>
__device__ uint32_t head_cut(CountF count_of, uint32_t mx, int T, int T_cap) {
  const int lane = threadIdx.x & 63;
  int b_hi = mx ? (int)(mx >> kBinShift) : -1;
  uint32_t above = 0u;
  while (b_hi >= 0) {
    const int bn = b_hi - lane;
    const uint32_t cnt = bn >= 0 ? count_of(bn) : 0u;
    const uint32_t incl = wave_incl_scan(cnt);
    const uint32_t tot = readlane(incl, 63);
    if (above + tot >= (uint32_t)T) {
      const uint64_t m = __ballot(above + incl >= (uint32_t)T);
      const int l = __ffsll((unsigned long long)m) - 1;
      const uint32_t il = __builtin_amdgcn_readlane(incl, l), cl = __builtin_amdgcn_readlane(cnt, l);
      const uint32_t a = above + il - cl;  // keys in higher bins, fewer than T
      return ((uint32_t)(b_hi - l) << 1) | ((a + cl <= (uint32_t)T_cap) ? 1u : 0u);
    }
    above += tot;
    b_hi -= 64;
  }
  return 1u;
}

// Write a share's heads of `kinds` kinds (0: entries or pool slots, 1: block
// maxima) to its own stretch of the query's candidate list (slots
// [j T_cap, j T_cap + count) of each kind), with the count, the cut, the
// share's largest key, the smallest key it wrote and the floor: the largest
// key it did not write.
// ks[kind][it]: this lane's key of batch it (0 = none; a block key is held by
// lane 8b of its block only); idf(kind, it): the key's id.  H.wmax and H.wlive
// hold every wave's largest key and count of keys, and H.n is zero (the caller
// has synchronised after the histograms).  The share wants T = 1.25 K live /
// total + 16 keys of a kind (share_want): a quarter more than its share of the
// K selected, in proportion to its keys among the query's `total` (a Reindex
// pool shorter than its slots leaves most shares empty); T_cap: most keys a
// share may write.  Out-pointers are kind 0's; kind 1's follow at `stride`.
template <int kIters, typename IdF>
__device__ void write_heads(const uint32_t (&ks)[2][kIters], int kinds, IdF idf, const uint32_t* hist0,
                            const uint32_t* hist1, const int64_t (&total)[2], const int32_t (&T_cap)[2], int j,
                            uint64_t* cand, uint32_t* count_out, uint64_t* floor_out, uint32_t* cut_out,
                            uint32_t* top_out, uint32_t* bot_out, int32_t stride, HeadLds& H) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int kind = 0; kind < 2; kind++) {
    if (kind >= kinds) break;  // uniform
    // every wave finds the same cut
    uint32_t mx = 0u, live = 0u;
#pragma unroll
    for (int w = 0; w < kScoreWaves; w++) {
      mx = max(mx, H.wmax[kind][w]);
      live += H.wlive[kind][w];
    }
    const int T = min(share_want(kind ? kPoolBlocks : kTopK, live, total[kind]), T_cap[kind]);
    const uint32_t* hist = kind ? hist1 : hist0;
    // a share with no more keys than it wants writes them all (no histogram walk)
    const uint32_t cut = live <= (uint32_t)T ? 1u : head_cut([&](int bn) { return hist[bn]; }, mx, T, T_cap[kind]);
    bool any;
    const uint32_t thr = head_threshold(cut, any);
    // this lane's written keys and the largest unwritten one (the lowest id
    // among equal keys), kept as a 32-bit key and its id
    uint32_t mine = 0u, fx = 0u, fid = 0xFFFFFFFFu, mn = 0xFFFFFFFFu;
#pragma unroll
    for (int it = 0; it < kIters; it++) {
      const uint32_t x = ks[kind][it];
      const bool w = any && x >= thr;
      mine += w ? 1u : 0u;
      mn = w ? min(mn, x) : mn;
      const uint32_t xu = w ? 0u : x;
      const uint32_t id = idf(kind, it);
      const bool up = xu > fx || (xu == fx && id < fid);
      fx = up ? xu : fx;
      fid = up ? id : fid;
    }
    uint64_t fl = fx ? key64(fx, fid) : 0ull;
    // one LDS atomic per wave reserves its slots in the share's stretch
    uint32_t slot = (uint32_t)wave_alloc((int)mine, &H.n[kind]);
    uint64_t* dst = cand + kind * kHeadCap + (int64_t)j * T_cap[kind];
#pragma unroll
    for (int it = 0; it < kIters; it++) {
      const uint32_t x = ks[kind][it];
      const bool w = any && x >= thr;
      if (w && slot < (uint32_t)T_cap[kind]) dst[slot] = key64(x, idf(kind, it));  // the cap always holds
      slot += w ? 1u : 0u;
    }
    fl = wave_max(fl);
    mn = wave_min(mn);
    if (lane == 0) {
      H.wfloor[kind][wave] = fl;
      H.wbot[kind][wave] = mn;
    }
    if (tid == 0) {
      H.cut[kind] = cut;
      H.top[kind] = mx;
    }
  }
  __syncthreads();
  if (tid < kinds) {
    const int kind = tid;
    uint64_t f = 0ull;
    uint32_t bt = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < kScoreWaves; w++) {
      f = max(f, H.wfloor[kind][w]);
      bt = min(bt, H.wbot[kind][w]);
    }
    floor_out[kind * stride] = f;
    cut_out[kind * stride] = H.cut[kind];
    top_out[kind * stride] = H.top[kind];
    bot_out[kind * stride] = bt;
    count_out[kind * stride] = min((uint32_t)H.n[kind], (uint32_t)T_cap[kind]);
  }
}

// ------------------------------------------------------------------ head kernel
// Batch slot `it` of workgroup j of a query: the query's W x iters batch slots
// are dealt to its workgroups round-robin (j, j + W, ...), starting from a
// per-query rotation so that the queries of a call read different relative
// offsets of their sequences at any moment (Full only; Reindex has none).
// Slots past the query's keys are skipped.
__device__ __forceinline__ int head_rot(int64_t bq, int W, int iters, bool reindex) {
  return reindex ? 0 : (int)(((bq & 15) * (int64_t)W * iters) >> 4);
}
__device__ __forceinline__ int64_t head_batch(int j, int it, int W, int iters, int rot) {
  const int m = W * iters;
  int x = j + it * W + rot;  // below 2m
  if (x >= m) x -= m;
  return x;
}

struct HeadArgs {
  const uint8_t* ik_codes;
  const float* ik_scales;
  uint8_t* kv_codes_w;  // fused append: the cache planes it writes
  uint8_t* kv_scales_w;
  uint8_t* ik_codes_w;
  float* ik_scales_w;
  const int32_t* length;
  int32_t cap, ratio;
  const float* iq;
  const float* iw;
  const int32_t* q_pos;
  const int32_t* pool_in;
  int32_t Q;
  int32_t W;          // workgroups per query
  int32_t iters;      // batches per workgroup (at most kFullIters / kReindexIters)
  int32_t blocks;     // Full: also the pool's block keys
  int32_t T[2], T_cap[2];  // keys a share wants with evenly spread keys (the select's speculative loads); most it writes
  const float* app_kv;  // fused append: [B][app_T][512] f32 new entries (ratio 1), or null
  const float* app_ik;  // [B][app_T][64] f32
  int32_t app_T;
  HeadWs ws;
};

template <bool Reindex>
__global__ void __launch_bounds__(kScoreThreads) index_head_kernel(HeadArgs a) {
  constexpr int kIters = Reindex ? kReindexIters : kFullIters;
  __shared__ uint32_t s_hist[kBins];
  __shared__ uint32_t s_bhist[Reindex ? 1 : kBins];
  __shared__ __attribute__((aligned(16))) uint8_t s_q8[256];
  __shared__ float s_c[4];
  __shared__ HeadLds H;

  const int Q = a.Q, W = a.W;
  int64_t bq = blockIdx.x;
  int j = blockIdx.y;
  if (Q > 1) {  // uniform
    // the queries of one sequence's share j read the same keys (Full) or
    // overlapping ones (Reindex over the pools of consecutive tokens): they
    // take consecutive ranks of one XCD, so that they run side by side over
    // its L2 (placement only)
    const int64_t r = xcd_rank((int64_t)blockIdx.y * gridDim.x + blockIdx.x, (int64_t)gridDim.x * gridDim.y);
    const int64_t u = r / Q;  // (sequence, share)
    j = (int)(u % W);
    bq = (u / W) * Q + r % Q;
  }
  const int b = (int)(bq / Q), q = (int)(bq % Q);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the query element and head weight this thread quantises (threads 0-255),
  // loaded first
  const bool qthr = tid < 256;
  const float iq_v = a.iq[bq * 256 + (tid & 255)];
  const float iw_v = (a.iw && qthr) ? a.iw[bq * 4 + (tid >> 6)] : 1.0f;
  // a fused append makes the new entries visible: the length in memory is the
  // one before it (the select kernel advances it)
  const int32_t len0 = a.length[b];
  const bool fits = a.app_T > 0 && len0 >= 0 && (int64_t)len0 + a.app_T <= a.cap;
  if (kDebug && j == 0 && q == 0 && tid == 0) {
    if (len0 < 0 || len0 > a.cap)
      dev_flag(kErrLength);
    else if (a.app_T > 0 && !fits)
      dev_flag(kErrCapacity);
  }
  const int32_t len = fits ? len0 + a.app_T : len0;
  const int32_t p = a.q_pos ? a.q_pos[bq] : len * a.ratio - Q + q;
  const int32_t n_vis = __builtin_amdgcn_readfirstlane(visible_count(len, a.cap, a.ratio, p));
  if (j == 0 && tid == 0) {
    a.ws.nvis[bq * 2] = n_vis;
    a.ws.nvis[bq * 2 + 1] = fits ? len : -1;  // the length the select kernel stores
  }
  const int64_t row_base = (int64_t)b * a.cap;
  const int32_t* pool = Reindex ? a.pool_in + bq * kPool : nullptr;
  const int rot = head_rot(bq, W, a.iters, Reindex);

  // ---- fused append: the new entries in this workgroup's batches, one wave each
  if (!Reindex && fits) {
    for (int t = wave; t < a.app_T; t += kScoreWaves) {  // wave-uniform
      const int64_t e = (int64_t)len0 + t;
      const int owner = (int)((((e / kBatchKeys) - rot) % W + W) % W);  // the workgroup holding e's batch slot
      if (owner != j || q != 0) continue;  // the first query's workgroup of that batch writes it
      const float4* src = reinterpret_cast<const float4*>(a.app_kv + ((int64_t)b * a.app_T + t) * 512 + 8 * lane);
      const float4 v0 = src[0], v1 = src[1];
      const float x[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      const float k = a.app_ik[((int64_t)b * a.app_T + t) * 64 + lane];
      quantize_store_entry(a.kv_codes_w, a.kv_scales_w, a.ik_codes_w, a.ik_scales_w, row_base + e, x, k, lane);
    }
    // the stores are complete before any wave of this workgroup loads those keys
    // (__syncthreads waits for every store a thread has in flight)
    __syncthreads();
  }
  // Every query's workgroups read a new entry: the other queries' workgroups of
  // its batch are not the writer.  Decode calls have one query per sequence;
  // with more, the queries after the first read the new entry only after the
  // first query's workgroup has written it, which a launch does not order, so
  // the host fuses the append only when Q == 1.

  Scorer<Reindex> sc;
  sc.init(a.ik_codes, a.ik_scales, row_base, n_vis);
  int32_t pe[kIters][kBatch];
  if constexpr (Reindex) {
#pragma unroll
    for (int it = 0; it < kIters; it++)
#pragma unroll
      for (int jj = 0; jj < kBatch; jj++) pe[it][jj] = pool[head_batch(j, it, W, a.iters, rot) * kBatchKeys + sc.key_of(jj)];
    if (kDebug)
      for (int it = 0; it < kIters; it++)
        for (int jj = 0; jj < kBatch; jj++)
          if (pe[it][jj] < -1 || pe[it][jj] >= n_vis) dev_flag(kErrPoolId);  // scored as absent
  } else {
#pragma unroll
    for (int it = 0; it < kIters; it++)
#pragma unroll
      for (int jj = 0; jj < kBatch; jj++) pe[it][jj] = 0;
  }
  const int64_t n_keys = Reindex ? (int64_t)kPool : (int64_t)n_vis;  // keys of the query
  auto base_of = [&](int it) -> int64_t { return head_batch(j, it, W, a.iters, rot) * kBatchKeys; };
  auto live = [&](int it) -> bool { return it < a.iters && base_of(it) < n_keys; };  // uniform
  BatchLoad ld[2];
  if (live(0)) sc.issue(base_of(0), pe[0], ld[0]);
  if (kIters > 1 && live(1)) sc.issue(base_of(1), pe[1], ld[1]);

  for (int i = tid; i < kBins; i += kScoreThreads) {
    s_hist[i] = 0u;
    if (!Reindex && a.blocks) s_bhist[i] = 0u;
  }
  if (tid < 2) H.n[tid] = 0;
  if (qthr) prep_query(iq_v, iw_v, s_q8, s_c, tid);
  lds_barrier();  // LDS only: the first batch stays in flight
  sc.load_query(s_q8, s_c);

  uint32_t ks[2][kIters];  // this lane's entry (or slot) keys and block keys, per batch
  uint32_t kmax = 0u;
#pragma unroll
  for (int it = 0; it < kIters; it++) {
    ks[0][it] = 0u;
    ks[1][it] = 0u;
    // the next live batch's loads, issued before this batch's liveness is known:
    // with the rotation a dead slot can sit between two live ones
    if (it >= 1 && it + 1 < kIters && live(it + 1)) sc.issue(base_of(it + 1), pe[it + 1], ld[(it + 1) & 1]);
    if (!live(it)) continue;  // uniform
    const int64_t k_own = base_of(it) + sc.own();
    bool valid;
    if constexpr (Reindex) {
      const int32_t pj = sc.jl == 0 ? pe[it][0] : sc.jl == 1 ? pe[it][1] : sc.jl == 2 ? pe[it][2] : pe[it][3];
      valid = pj >= 0 && pj < n_vis;
    } else {
      valid = k_own < n_vis;
    }
    const uint32_t key = sc.compute(ld[it & 1], valid);
    ks[0][it] = key;
    kmax = max(kmax, key);
    if (key) atomicAdd(&s_hist[key >> kBinShift], 1u);
    if (!Reindex && a.blocks) {
      const uint32_t m = block_max8(key);
      ks[1][it] = (lane & 7) == 0 ? m : 0u;  // held by the block's first lane
      if ((lane & 7) == 0 && m) atomicAdd(&s_bhist[m >> kBinShift], 1u);
    }
  }
  kmax = wave_max(kmax);  // the block keys' maximum is the same key
  uint32_t live0 = 0u, live1 = 0u;
#pragma unroll
  for (int it = 0; it < kIters; it++) {
    live0 += ks[0][it] != 0u ? 1u : 0u;
    live1 += ks[1][it] != 0u ? 1u : 0u;
  }
  live0 = wave_sum(live0);
  live1 = wave_sum(live1);
  if (lane == 0) {
    H.wmax[0][wave] = kmax;
    H.wmax[1][wave] = kmax;
    H.wlive[0][wave] = live0;
    H.wlive[1][wave] = live1;
  }
  __syncthreads();  // the histograms, maxima and counts are complete

  const int64_t sl = (bq * 2) * a.ws.wstride + j;  // this share's floor and cut, kind 0
  auto idf = [&](int kind, int it) -> uint32_t {  // entry or pool slot; block
    const int64_t k = base_of(it) + sc.own();
    return (uint32_t)(kind ? (k >> 3) : k);
  };
  const int kinds = (!Reindex && a.blocks) ? 2 : 1;
  // keys of each kind over all the query's shares: its visible entries and their
  // blocks, or the entries of its pool (every visible one while they are fewer
  // than the pool's slots)
  const int64_t total[2] = {Reindex ? min((int64_t)n_vis, (int64_t)kPool) : (int64_t)n_vis,
                            ((int64_t)n_vis + kBlock - 1) / kBlock};
  write_heads<kIters>(ks, kinds, idf, s_hist, s_bhist, total, a.T_cap, j, a.ws.cand + (bq * 2) * kHeadCap,
                      a.ws.count + sl, a.ws.floor + sl, a.ws.cut + sl, a.ws.top + sl, a.ws.bot + sl, a.ws.wstride, H);
}

// ------------------------------------------------------------------ shared-load heads
// Four or more queries per sequence and no pool (prefill chunks, multi-token
// decode without a pool): 4G queries of one sequence share every key load, and
// each query's keys stay in registers, as at one query.  Workgroup (group, j)
// scores batches j, j + W, ... (no rotation: the group's queries share them),
// counts every query's keys in its own LDS histogram (two 16-bit counts per
// word: a share holds at most 4,096 keys), and writes each query's heads,
// count, floor and cut to that query's stretch j as index_head does.  The
// select kernel then completes the call unchanged: its repair re-scores a
// share with the one-query scoring core, whose keys are bit for bit these
// (the same two MFMAs per 16 keys, head sum and scale, in the same order).
struct SharedHeadArgs {
  const uint8_t* ik_codes;
  const float* ik_scales;
  const int32_t* length;
  int32_t cap, ratio;
  const float* iq;
  const float* iw;
  const int32_t* q_pos;
  int32_t Q, W, iters, T_cap;
  HeadWs ws;
};

template <int G, bool Blocks>
__global__ void __launch_bounds__(kScoreThreads) index_shared_head_kernel(SharedHeadArgs a) {
  constexpr int kQ = 4 * G;                 // queries per workgroup
  constexpr int kJ = kScoreThreads / 256;  // queries whose elements one pass of the workgroup loads
  constexpr int kKinds = Blocks ? 2 : 1;    // entries; the pool's 8-entry block maxima
  constexpr int kSlots = kSharedIters * kBatch;  // (batch, group) pairs of a lane
  static_assert(kQ % kJ == 0 && kQ <= kScoreWaves, "whole passes; one wave per query's cut");
  __shared__ uint32_t s_hist[kKinds][kQ][kBins / 2];
  __shared__ __attribute__((aligned(16))) uint8_t s_q8[kQ][256];
  __shared__ float s_c[kQ][4];
  __shared__ uint32_t s_max[kQ], s_cut[kKinds][kQ], s_bot[kKinds][kQ];
  __shared__ uint32_t s_n[kKinds][kQ];
  __shared__ unsigned long long s_floor[kKinds][kQ];

  const int W = a.W, Q = a.Q;
  const int groups_per_seq = (Q + kQ - 1) / kQ;
  // The query groups of one (sequence, share) read the same keys: they take
  // consecutive ranks of one XCD, so that they run side by side and the later
  // ones find the lines in that XCD's L2 (placement only)
  const int64_t r = xcd_rank(blockIdx.x, gridDim.x);
  const int64_t u = r / groups_per_seq;
  const int j = (int)(u % W), b = (int)(u / W), q0 = (int)(r % groups_per_seq) * kQ;
  const int nq = min(kQ, Q - q0);
  const int64_t bq0 = (int64_t)b * Q + q0;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane & 15, grp = lane >> 4, jq = lane >> 4;
  // query elements first (thread 256 jh + t quantises element t of queries
  // jh, jh + kJ, ...; a missing query reloads the last one, unused)
  const int t = tid & 255, jh = tid >> 8;
  float iq_v[kQ / kJ], iw_v[kQ / kJ];
#pragma unroll
  for (int k = 0; k < kQ / kJ; k++) {
    const int64_t jj = bq0 + min(jh + kJ * k, nq - 1);
    iq_v[k] = a.iq[jj * 256 + t];
    iw_v[k] = a.iw ? a.iw[jj * 4 + (t >> 6)] : 1.0f;
  }
  const int32_t len = a.length[b];
  if (kDebug && j == 0 && q0 == 0 && tid == 0 && (len < 0 || len > a.cap)) dev_flag(kErrLength);
  int32_t nv[kQ];
  int32_t nv_max = 0;
#pragma unroll
  for (int u = 0; u < kQ; u++) {
    nv[u] = u < nq ? visible_count(len, a.cap, a.ratio, query_pos(a.q_pos, a.length, a.ratio, b, q0 + u, Q)) : 0;
    nv_max = max(nv_max, nv[u]);
  }
  nv_max = __builtin_amdgcn_readfirstlane(nv_max);
  if (j == 0 && tid < nq) {
    int32_t v = 0;
#pragma unroll
    for (int u = 0; u < kQ; u++) v = u == tid ? nv[u] : v;
    a.ws.nvis[(bq0 + tid) * 2] = v;
    a.ws.nvis[(bq0 + tid) * 2 + 1] = -1;  // no length to store
  }

  const int64_t row_base = (int64_t)b * a.cap;
  // a lane's key of group jj in a batch is entry base + loff[jj]
  uint32_t loff[kBatch];
#pragma unroll
  for (int jj = 0; jj < kBatch; jj++) loff[jj] = (uint32_t)(16 * (jj * kScoreWaves + wave) + row);
  auto base_of = [&](int it) -> int64_t { return head_batch(j, it, W, a.iters, 0) * kBatchKeys; };
  // batches ascend with it, so the live ones come first
  auto live = [&](int it) -> bool { return it < a.iters && base_of(it) < nv_max; };  // uniform
  // a live batch's loads: its base goes into the buffer descriptors (bounded
  // at the largest visible count), so the per-lane offsets stay fixed
  auto issue = [&](int it, v4i (&bytes)[kBatch], float (&sk)[kBatch]) {
    const int64_t base = base_of(it);
    const int64_t left = (int64_t)nv_max - base;
    const uint32_t nrec = left < kBatchKeys ? (uint32_t)left : (uint32_t)kBatchKeys;
    const BufRsrc kb = make_rsrc(a.ik_codes + (row_base + base) * 64, nrec * 64u);
    const BufRsrc sb = make_rsrc(a.ik_scales + (row_base + base), nrec * 4u);
#pragma unroll
    for (int jj = 0; jj < kBatch; jj++) {
      bytes[jj] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(kb, loff[jj] * 64u + 16u * grp, 0, kNT));
      sk[jj] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sb, loff[jj] * 4u, 0, 0));
    }
  };
  v4i bytes[2][kBatch];
  float sk[2][kBatch];
  if (live(0)) issue(0, bytes[0], sk[0]);
  if (live(1)) issue(1, bytes[1], sk[1]);

  for (int i = tid; i < kKinds * kQ * kBins / 2; i += kScoreThreads) (&s_hist[0][0][0])[i] = 0u;
  if (tid < kQ) {
    s_max[tid] = 0u;
#pragma unroll
    for (int kind = 0; kind < kKinds; kind++) {
      s_n[kind][tid] = 0u;
      s_floor[kind][tid] = 0ull;
      s_bot[kind][tid] = 0xFFFFFFFFu;
    }
  }
#pragma unroll
  for (int k = 0; k < kQ / kJ; k++) {
    const int jx = jh + kJ * k;
    if (jx < nq) {
      prep_query(iq_v[k], iw_v[k], s_q8[jx], s_c[jx], t);
    } else {
      s_q8[jx][t] = 0;
      if (t < 4) s_c[jx][t] = 0.0f;
    }
  }
  lds_barrier();  // LDS only: the first batches stay in flight

  // A operands: in group g, row r = lane%16 is query 4g + r/4, head r%4;
  // lanes 16jq..16jq+15 finish query 4g + jq's keys
  v8bf qa0[G], qa1[G];
  float ch[G][4];
  int32_t my_nv[G];
#pragma unroll
  for (int g = 0; g < G; g++) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(&s_q8[4 * g + (row >> 2)][(row & 3) * 64 + 16 * grp]);
    qa0[g] = widen8(src[0], src[1]);
    qa1[g] = widen8(src[2], src[3]);
    const int jx = 4 * g + jq;
#pragma unroll
    for (int h = 0; h < 4; h++) ch[g][h] = s_c[jx][h];
    int32_t v = 0;
#pragma unroll
    for (int u = 0; u < kQ; u++) v = u == jx ? nv[u] : v;
    my_nv[g] = jx < nq ? v : 0;  // a missing query has no keys
  }

  uint32_t ks[kSharedIters][kBatch][G];  // this lane's keys: batch, group, query 4g + jq
  // block keys: the maximum of (batch it, group jj)'s 8-entry block of this
  // lane's row is kept by the lane of the block with row % 8 == s % 8, s = 4 it
  // + jj, in kb[g][s / 8] (four registers for 32 blocks)
  uint32_t kb[G][Blocks ? kSlots / 8 : 1];
  uint32_t kmax[G];  // the largest entry key, also the largest block key
#pragma unroll
  for (int g = 0; g < G; g++) {
    kmax[g] = 0u;
#pragma unroll
    for (int s8 = 0; s8 < (Blocks ? kSlots / 8 : 1); s8++) kb[g][s8] = 0u;
  }
#pragma unroll
  for (int it = 0; it < kSharedIters; it++) {
#pragma unroll
    for (int jj = 0; jj < kBatch; jj++)
#pragma unroll
      for (int g = 0; g < G; g++) ks[it][jj][g] = 0u;
    if (it >= 1 && it + 1 < kSharedIters && live(it + 1)) issue(it + 1, bytes[(it + 1) & 1], sk[(it + 1) & 1]);
    if (!live(it)) continue;  // uniform
    const int32_t sbase = (int32_t)base_of(it);
    const v4i(&by)[kBatch] = bytes[it & 1];
#pragma unroll
    for (int jj = 0; jj < kBatch; jj++) {
      const v8bf k0 = widen8((uint32_t)by[jj][0], (uint32_t)by[jj][1]);
      const v8bf k1 = widen8((uint32_t)by[jj][2], (uint32_t)by[jj][3]);
      const int32_t e = sbase + (int32_t)loff[jj];
#pragma unroll
      for (int g = 0; g < G; g++) {
        v4f d = {0.f, 0.f, 0.f, 0.f};
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa0[g], k0, d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa1[g], k1, d, 0, 0, 0);
        // the one-query core's arithmetic, in fewer instructions: ReLU as an
        // integer max (finite inputs: d > 0 keeps d, else +0), and the scale
        // as an fma with +0, which turns a -0 product into +0 so that the
        // order key needs no -0 case (order_key maps both zeros alike)
        float acc = 0.0f;
        acc = __builtin_fmaf(ch[g][0], relu_bits(d[0]), acc);
        acc = __builtin_fmaf(ch[g][1], relu_bits(d[1]), acc);
        acc = __builtin_fmaf(ch[g][2], relu_bits(d[2]), acc);
        acc = __builtin_fmaf(ch[g][3], relu_bits(d[3]), acc);
        const uint32_t u = __float_as_uint(__builtin_fmaf(sk[it & 1][jj], acc, 0.0f));
        const uint32_t key = e < my_nv[g] ? (u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u)) : 0u;
        ks[it][jj][g] = key;
        kmax[g] = max(kmax[g], key);
        const uint32_t bin = key >> kBinShift;
        atomicAdd(&s_hist[0][4 * g + jq][bin >> 1], key ? 1u << (16 * (bin & 1u)) : 0u);  // 0: no key, adds nothing
        if constexpr (Blocks) {
          const uint32_t m = block_max8(key);  // every lane of the block's 8
          const int sl = it * kBatch + jj;  // a constant once the loops unroll
          if ((row & 7) == (sl & 7)) kb[g][sl >> 3] = m;
          const uint32_t bb = m >> kBinShift;
          if ((row & 7) == 0 && m) atomicAdd(&s_hist[1][4 * g + jq][bb >> 1], 1u << (16 * (bb & 1u)));
        }
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; g++) {
    if (4 * g + jq < nq) atomicMax(&s_max[4 * g + jq], kmax[g]);
  }
  __syncthreads();  // the histograms, maxima and counts are complete

  // wave u finds query u's cuts: the bin holding the share's T-th key of each
  // kind, with T in proportion to the share's keys among the query's (its
  // visible entries, or their blocks, among the share's batches)
  if (wave < nq) {  // uniform
    int32_t total = 0;
#pragma unroll
    for (int u = 0; u < kQ; u++) total = u == wave ? nv[u] : total;
#pragma unroll
    for (int kind = 0; kind < kKinds; kind++) {
      uint32_t lv = 0u;
      for (int it = 0; it < a.iters; it++) {
        const int64_t left = (int64_t)total - base_of(it);
        const uint32_t ne = left <= 0 ? 0u : (left < kBatchKeys ? (uint32_t)left : (uint32_t)kBatchKeys);
        lv += kind ? (ne + kBlock - 1) / kBlock : ne;
      }
      const int64_t tot = kind ? ((int64_t)total + kBlock - 1) / kBlock : (int64_t)total;
      const int T = min(share_want(kind ? kPoolBlocks : kTopK, lv, tot), (int)a.T_cap);
      const uint32_t* h = s_hist[kind][wave];
      // no more keys than it wants (lv counts the visible ones): all written
      const uint32_t cut =
          lv <= (uint32_t)T
              ? 1u
              : head_cut([&](int bn) { return (h[bn >> 1] >> (16 * (bn & 1))) & 0xFFFFu; }, s_max[wave], T, a.T_cap);
      if (lane == 0) s_cut[kind][wave] = cut;
    }
  }
  __syncthreads();

  // each query's keys above its cut to its stretch j; the largest other key is
  // its floor.  A key x is written iff x >= head_threshold(cut); ids ascend
  // with a lane's (it, jj), so the first unwritten key of the largest value has
  // the lowest id.
#pragma unroll
  for (int g = 0; g < G; g++) {
    const int jx = 4 * g + jq;
    if (jx >= nq) continue;
    uint64_t* cand = a.ws.cand + ((bq0 + jx) * 2) * kHeadCap + (int64_t)j * a.T_cap;
    {  // entries
      bool any;
      const uint32_t thr = head_threshold(s_cut[0][jx], any);
      uint32_t mine = 0u, fx = 0u, fid = 0u, mn = 0xFFFFFFFFu;
#pragma unroll
      for (int it = 0; it < kSharedIters; it++) {
        const uint32_t sb = (uint32_t)base_of(it);
#pragma unroll
        for (int jj = 0; jj < kBatch; jj++) {
          const uint32_t x = ks[it][jj][g];
          const bool w = any && x >= thr;
          mine += w ? 1u : 0u;
          const uint32_t xu = w ? 0u : x;
          const bool up = xu > fx;
          fx = up ? xu : fx;
          fid = up ? sb + loff[jj] : fid;
        }
      }
      uint32_t slot = atomicAdd(&s_n[0][jx], mine);
#pragma unroll
      for (int it = 0; it < kSharedIters; it++) {
        const uint32_t sb = (uint32_t)base_of(it);
#pragma unroll
        for (int jj = 0; jj < kBatch; jj++) {
          const uint32_t x = ks[it][jj][g];
          if (any && x >= thr) {
            if (slot < (uint32_t)a.T_cap) cand[slot] = key64(x, sb + loff[jj]);  // the cap always holds
            slot++;
            mn = min(mn, x);  // tracked here, not while counting: fewer registers live across the loops
          }
        }
      }
      if (fx) atomicMax(&s_floor[0][jx], (unsigned long long)key64(fx, fid));
      if (mine) atomicMin(&s_bot[0][jx], mn);
    }
    if constexpr (Blocks) {  // block maxima: this lane's kb[g][s8] is block slot s = 8 s8 + row % 8
      bool any;
      const uint32_t thr = head_threshold(s_cut[1][jx], any);
      uint32_t bid[kSlots / 8];
#pragma unroll
      for (int s8 = 0; s8 < kSlots / 8; s8++) {
        const int sl = 8 * s8 + (row & 7);
        const int it = sl / kBatch, jj = sl % kBatch;
        const int64_t x = head_batch(j, it, W, a.iters, 0);  // below 2^23 / 512
        bid[s8] = (uint32_t)((x * kBatchKeys + 16 * (jj * kScoreWaves + wave) + (row & 8)) >> 3);
      }
      uint32_t mine = 0u, fx = 0u, fid = 0u, mn = 0xFFFFFFFFu;
#pragma unroll
      for (int s8 = 0; s8 < kSlots / 8; s8++) {
        const uint32_t x = kb[g][s8];
        const bool w = any && x >= thr;
        mine += w ? 1u : 0u;
        const uint32_t xu = w ? 0u : x;
        const bool up = xu > fx;
        fx = up ? xu : fx;
        fid = up ? bid[s8] : fid;
      }
      uint32_t slot = atomicAdd(&s_n[1][jx], mine);
      uint64_t* cb = cand + kHeadCap;
#pragma unroll
      for (int s8 = 0; s8 < kSlots / 8; s8++) {
        const uint32_t x = kb[g][s8];
        if (any && x >= thr) {
          if (slot < (uint32_t)a.T_cap) cb[slot] = key64(x, bid[s8]);
          slot++;
          mn = min(mn, x);
        }
      }
      if (fx) atomicMax(&s_floor[1][jx], (unsigned long long)key64(fx, fid));
      if (mine) atomicMin(&s_bot[1][jx], mn);
    }
  }
  __syncthreads();
  if (tid < nq) {
#pragma unroll
    for (int kind = 0; kind < kKinds; kind++) {
      const int64_t sl = ((bq0 + tid) * 2 + kind) * a.ws.wstride + j;
      a.ws.floor[sl] = s_floor[kind][tid];
      a.ws.cut[sl] = s_cut[kind][tid];
      a.ws.top[sl] = s_max[tid];  // the block keys' largest is the same key
      a.ws.bot[sl] = s_bot[kind][tid];
      a.ws.count[sl] = min(s_n[kind][tid], (uint32_t)a.T_cap);
    }
  }
}

// ------------------------------------------------------------------ select kernel
struct SelectArgs {
  const uint8_t* ik_codes;
  const float* ik_scales;
  int32_t* length;  // advanced here after a fused append
  int32_t cap, ratio;
  const float* iq;
  const float* iw;
  const int32_t* pool_in;
  int32_t Q, W, iters, app_T;
  int32_t rotate;  // the head kernel's per-query batch rotation (0: the shared-load heads, none)
  int32_t tc;  // each workgroup's stretch of the candidate list (even, W tc <= kHeadCap)
  // per kind: the slots of each stretch loaded before the counts are known (R,
  // even, <= tc) and floor(2^32 / (R / 2)) + 1, so that p / (R / 2) ==
  // umulhi(p, magic) for every p < kHeadCap / 2
  int32_t spec[2];
  uint32_t spec_magic[2];
  HeadWs ws;
  int32_t* topk_out;
  int32_t* pool_out;
};

constexpr int kBitWords = 10240;  // the Full output bitmap: ids below 327,680

// Sizes of a select kernel instance.  SelAll serves every call.  SelLean
// serves the Full calls of the shared-load heads with no pool and at most
// 65,536 visible entries (shares of at most 8 batches): about 71 KB of LDS
// instead of 150, so that two workgroups share a compute unit when thousands
// of queries select at once.
struct SelAll {
  static constexpr int kSet = kHeadCap;     // candidates held (and the largest key batch)
  static constexpr int kOut = kPoolBlocks;  // selected keys; boundary-bin keys
  static constexpr int kIdx = kPoolBlocks;  // share counts (W <= kIdx); wide-range ids
  static constexpr int kBitW = kBitWords;   // output bitmap words
  static constexpr int kTake = kBins / 2;   // wide-range buckets
  static constexpr bool kWide = true;       // the pool kind and ids past the bitmap
};
struct SelLean {
  static constexpr int kSet = 9 * kScoreThreads;  // K kept plus one repaired share of 8 batches
  static constexpr int kOut = kTopK;
  static constexpr int kIdx = kScoreThreads;
  static constexpr int kBitW = 2048;  // ids below 65,536
  static constexpr int kTake = 1;
  static constexpr bool kWide = false;
};

template <class C>
struct SelectLdsT {
  using Cfg = C;
  uint64_t set[C::kSet];  // candidates (then the rank bitmap and its offsets)
  union {
    struct {
      uint64_t out[C::kOut];  // the selected keys; the boundary bin's keys during a selection
      uint32_t idx[C::kIdx];  // each share's count while loading; ids in the wide-range output
      uint32_t hist[kBins];   // candidates per bin of their score keys' range
    };
    uint32_t woff[C::kBitW + C::kBitW / 8];  // Full Top-K output: the selected ids before each bitmap word (padded)
  };
  union {
    uint32_t bits[C::kBitW + C::kBitW / 8];  // one bit per selected id (Full; padded words)
    struct {
      int take[C::kTake], off[C::kTake], ge[C::kTake];  // the wide-range output's buckets
    };
  };
  SelShared sel;
  uint8_t q8[256];
  float c[4];
  uint64_t wfl[kScoreWaves];
  uint64_t wfm[kScoreWaves];  // largest floor of each wave's shares
  int wj[kScoreWaves];
  uint32_t wmx[kScoreWaves], wmn[kScoreWaves];
  int wov[kScoreWaves];  // whether a wave's shares wrote more than the speculative slots
  int tmp[16];
  int n, n_out, n_tie, bt, above;
  uint64_t kth;
};

// This thread's keys of L.set[0, n), i = tid + 512 r, loaded together (a load
// and its use one after another would wait out the LDS latency per key); 0
// past n (candidate keys are never 0).
template <int N>
struct KeyBatch {
  static constexpr int kN = N;
  uint64_t x[N];
  __device__ __forceinline__ void load(const uint64_t* set, int n) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int r = 0; r < N; r++) {
      const uint64_t v = set[tid + r * kScoreThreads];  // inside L.set: N * 512 <= its size
      x[r] = tid + r * kScoreThreads < n ? v : 0ull;
    }
  }
};
template <int kMaxN, typename F>
__device__ __forceinline__ void with_keys(const uint64_t* set, int n, F&& f) {
  static_assert(kMaxN > 8, "the largest batch");
  const int nr = (n + kScoreThreads - 1) / kScoreThreads;  // uniform
  if (nr <= 4) {
    KeyBatch<4> b;
    b.load(set, n);
    f(b);
  } else if (nr <= 8) {
    KeyBatch<8> b;
    b.load(set, n);
    f(b);
  } else {
    KeyBatch<kMaxN> b;
    b.load(set, n);
    f(b);
  }
}

template <int N>
struct IntC {
  static constexpr int value = N;
};

// Output bitmaps hold word w at w + w / 8: a thread that owns eight
// consecutive words then reads and writes them without LDS bank conflicts
// (lanes 9 words apart instead of 8).
__device__ __forceinline__ int bw(int w) { return w + (w >> 3); }
__device__ __forceinline__ void set_bit(uint32_t* bits, uint32_t id) {
  atomicOr(&bits[bw((int)(id >> 5))], 1u << (id & 31u));
}

// The range [lo, hi] of the score keys (top 32 bits) of the n keys in L.set.
// Every thread gets it.
template <class Lds>
__device__ __forceinline__ void key_range(Lds& L, int n, uint32_t& lo, uint32_t& hi) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  lo = ~0u;
  hi = 0u;
  with_keys<std::remove_reference_t<decltype(L)>::Cfg::kSet / kScoreThreads>(L.set, n, [&](auto& b) {
#pragma unroll
    for (int r = 0; r < b.kN; r++) {
      const uint32_t x = (uint32_t)(b.x[r] >> 32);
      lo = b.x[r] ? min(lo, x) : lo;
      hi = max(hi, x);
    }
  });
  lo = wave_min(lo);
  hi = wave_max(hi);
  if (lane == 0) {
    L.wmx[wave] = hi;
    L.wmn[wave] = lo;
  }
  __syncthreads();
  lo = ~0u;
  hi = 0u;
#pragma unroll
  for (int w = 0; w < kScoreWaves; w++) {
    lo = min(lo, L.wmn[w]);
    hi = max(hi, L.wmx[w]);
  }
  __syncthreads();
}

// Bin of a score key x in [lo, hi]: (x - lo) >> bin_shift(lo, hi), below kBins.
__device__ __forceinline__ int bin_shift(uint32_t lo, uint32_t hi) {
  const uint32_t span = hi - lo;
  return span < (uint32_t)kBins ? 0 : 32 - __clz((int)(span >> 12));
}

// The K-th largest S* of the n unique nonzero u64 keys in L.set (n > K),
// whose score keys lie in [lo, hi]; with `mark`, also the bit of every key at
// or above S* in L.bits (the key's id).  On entry L.n_tie is zero, and L.hist
// is zero or, with `counted`, already holds the keys' counts per bin (and
// L.bits is zero with `mark`); the call leaves them dirty.  The keys are counted
// in 4,096 bins spanning [lo, hi]; a count over the bins from the top finds the
// bin holding the K-th key; the keys of higher bins are taken, and that bin's
// keys (typically one or two) are gathered and ranked exactly (by one wave when
// there are at most 64 of them, else by the radix select).  Every thread gets
// S*.
template <class Lds>
__device__ __forceinline__ uint64_t select_kth(Lds& L, int n, int K, uint32_t lo, uint32_t hi, bool mark,
                                              bool counted = false) {
  using C = typename Lds::Cfg;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int kThr = kScoreThreads;
  const int shift = bin_shift(lo, hi);
  if (!counted) {  // uniform
    with_keys<std::remove_reference_t<decltype(L)>::Cfg::kSet / kScoreThreads>(L.set, n, [&](auto& b) {
#pragma unroll
      for (int r = 0; r < b.kN; r++)
        if (b.x[r]) atomicAdd(&L.hist[(((uint32_t)(b.x[r] >> 32)) - lo) >> shift], 1u);
    });
    __syncthreads();
  }
  {
    // thread t counts bins [8c, 8c + 8) with c = kThr - 1 - t, so a prefix over
    // the threads is a count from the top bin down; the thread whose range
    // holds the K-th key finds its bin
    constexpr int kPerT = kBins / kThr;
    const int c = kThr - 1 - tid;
    uint32_t h[kPerT];
    uint32_t s = 0u;
#pragma unroll
    for (int u = 0; u < kPerT; u++) {
      h[u] = L.hist[c * kPerT + u];
      s += h[u];
    }
    int tot;
    uint32_t acc = (uint32_t)block_scan_excl1((int)s, L.tmp, &tot);  // keys in higher bins
    if (acc < (uint32_t)K && acc + s >= (uint32_t)K) {
#pragma unroll
      for (int u = kPerT - 1; u >= 0; u--) {
        if (acc + h[u] >= (uint32_t)K) {
          L.bt = c * kPerT + u;
          L.above = (int)acc;
          break;
        }
        acc += h[u];
      }
    }
  }
  __syncthreads();
  const uint32_t bt = (uint32_t)L.bt;
  const int need = K - L.above;  // keys to take from the boundary bin, >= 1
  // the keys of higher bins are taken; the boundary bin's are gathered
  with_keys<std::remove_reference_t<decltype(L)>::Cfg::kSet / kScoreThreads>(L.set, n, [&](auto& b) {
    int nt = 0;
#pragma unroll
    for (int r = 0; r < b.kN; r++) {
      const uint32_t bn = (((uint32_t)(b.x[r] >> 32)) - lo) >> shift;
      if (mark && b.x[r] && bn > bt) set_bit(L.bits, key_id(b.x[r]));
      nt += (b.x[r] && bn == bt) ? 1 : 0;
    }
    int slot = wave_alloc(nt, &L.n_tie);
#pragma unroll
    for (int r = 0; r < b.kN; r++) {
      const uint32_t bn = (((uint32_t)(b.x[r] >> 32)) - lo) >> shift;
      if (b.x[r] && bn == bt) {
        if (slot < C::kOut) L.out[slot] = b.x[r];
        slot++;
      }
    }
  });
  __syncthreads();
  const int n_tie = L.n_tie;
  if (n_tie <= 64) {
    if (wave == 0) {  // rank by comparing every pair across the lanes
      const uint64_t v = lane < n_tie ? L.out[lane] : 0ull;
      int greater = 0;
      for (int j = 0; j < n_tie; j++) greater += readlane(v, j) > v ? 1 : 0;
      if (lane < n_tie && greater < need) {
        if (mark) set_bit(L.bits, key_id(v));
        if (greater == need - 1) L.kth = v;
      }
    }
  } else {
    if (n_tie <= C::kOut && need < n_tie) {
      int cnt;
      const uint64_t t = topk_threshold<uint64_t>([&](int i) { return L.out[i]; }, n_tie, need, L.sel, &cnt);
      if (tid == 0) L.kth = t;
    } else if (n_tie <= C::kOut) {  // the whole bin is taken: its smallest key
      uint64_t m = ~0ull;
      for (int i = tid; i < n_tie; i += kThr) m = min(m, L.out[i]);
      m = wave_min(m);
      if (lane == 0) L.wfl[wave] = m;
      __syncthreads();
      if (tid == 0) {
        uint64_t g = ~0ull;
        for (int w = 0; w < kThr / 64; w++) g = min(g, L.wfl[w]);
        L.kth = g;
      }
    } else {  // very wide ties: select over all keys
      int cnt;
      const uint64_t t = topk_threshold<uint64_t>([&](int i) { return L.set[i]; }, n, K, L.sel, &cnt);
      if (tid == 0) L.kth = t;
    }
    if (mark) {  // the boundary bin's keys at or above S*
      __syncthreads();
      const uint64_t kth = L.kth;
      with_keys<std::remove_reference_t<decltype(L)>::Cfg::kSet / kScoreThreads>(L.set, n, [&](auto& b) {
#pragma unroll
        for (int r = 0; r < b.kN; r++) {
          const uint32_t bn = (((uint32_t)(b.x[r] >> 32)) - lo) >> shift;
          if (b.x[r] && bn == bt && b.x[r] >= kth) set_bit(L.bits, key_id(b.x[r]));
        }
      });
    }
  }
  __syncthreads();
  return L.kth;  // not written again before two more barriers
}

// Re-score share j of query bq exactly as index_head did and append to L.set
// every key of the kind that the share did not write and that is above s_star.
template <bool Reindex, class Lds>
__device__ __forceinline__ void repair_share(const SelectArgs& a, int64_t bq, int kind, int j, uint32_t cut, uint64_t s_star,
                             int32_t n_vis, Lds& L) {
  const int b = (int)(bq / a.Q);
  const int W = a.W;
  const int lane = threadIdx.x & 63;
  Scorer<Reindex> sc;
  sc.init(a.ik_codes, a.ik_scales, (int64_t)b * a.cap, n_vis);
  sc.load_query(L.q8, L.c);
  const int32_t* pool = Reindex ? a.pool_in + bq * kPool : nullptr;
  const int64_t n_keys = Reindex ? (int64_t)kPool : (int64_t)n_vis;
  const int rot = a.rotate ? head_rot(bq, W, a.iters, Reindex) : 0;
  for (int it = 0; it < a.iters; it++) {
    const int64_t base = head_batch(j, it, W, a.iters, rot) * kBatchKeys;
    if (base >= n_keys) continue;  // uniform
    int32_t pe[kBatch];
#pragma unroll
    for (int jj = 0; jj < kBatch; jj++) pe[jj] = Reindex ? pool[base + sc.key_of(jj)] : 0;
    BatchLoad ld;
    sc.issue(base, pe, ld);
    const int64_t k_own = base + sc.own();
    bool valid;
    if constexpr (Reindex) {
      const int32_t pj = pe[sc.jl];
      valid = pj >= 0 && pj < n_vis;
    } else {
      valid = k_own < n_vis;
    }
    uint32_t key = sc.compute(ld, valid);
    uint32_t id = (uint32_t)k_own;
    bool own = true;
    if (kind == 1) {
      key = block_max8(key);
      id = (uint32_t)(k_own >> 3);
      own = (lane & 7) == 0;
    }
    const uint64_t k64 = key64(key, id);
    const bool add = own && key != 0u && !head_written(key, cut) && k64 > s_star;
    const int slot = wave_slot(add, &L.n);
    if (add && slot < Lds::Cfg::kSet) L.set[slot] = k64;
  }
  __syncthreads();
}

// grid (BQ, kinds): kind 0 writes the Top-512, kind 1 the candidate pool
// (SelAll only; SelLean serves kind 0 with ids below 32 C::kBitW)
template <bool Reindex, class C>
__global__ void __launch_bounds__(kScoreThreads) index_select_kernel(SelectArgs a) {
  __shared__ SelectLdsT<C> L;
  constexpr int kThr = kScoreThreads;
  const int64_t bq = blockIdx.x;
  const int kind = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int W = a.W, tc = a.tc;
  const int K = kind ? kPoolBlocks : kTopK;
  const int32_t n_vis = a.ws.nvis[bq * 2];
  const uint64_t* cand = a.ws.cand + (bq * 2 + kind) * kHeadCap;
  const uint32_t* counts = a.ws.count + (bq * 2 + kind) * a.ws.wstride;
  const uint64_t* floors = a.ws.floor + (bq * 2 + kind) * a.ws.wstride;
  const uint32_t* cuts = a.ws.cut + (bq * 2 + kind) * a.ws.wstride;
  const uint32_t* tops = a.ws.top + (bq * 2 + kind) * a.ws.wstride;
  const uint32_t* bots = a.ws.bot + (bq * 2 + kind) * a.ws.wstride;
  // ids of the output: entries or blocks (Full), pool slots (Reindex)
  const int64_t universe = Reindex ? (int64_t)kPool : (kind == 0 ? (int64_t)n_vis : ((int64_t)n_vis + kBlock - 1) / kBlock);
  const bool direct = !C::kWide || universe <= 32 * (int64_t)C::kBitW;  // uniform: the bitmap output
  const int nw = direct ? (int)((universe + 31) >> 5) : 0;

  // ---- the first R slots of every stretch (speculatively), the counts, floors,
  // bottoms and tops, all at once: thread t holds slot pairs p = t + 512 u
  // (pair p is slots 2 (p mod R/2) and one more of stretch p div R/2), and the
  // figures of shares t + 512 f (W <= C::kIdx).  The written keys lie between
  // the smallest bottom and the largest top of the shares that wrote, so they
  // are counted in the histogram as they go to L.set.
  constexpr int kPairs = (C::kSet / 2 + kThr - 1) / kThr;  // W tc <= C::kSet
  static_assert(kPairs >= 4, "the gather's instances");
  constexpr int kFl = C::kIdx / kThr;
  const int R = a.spec[kind], rh = R >> 1;
  const uint32_t rh_magic = a.spec_magic[kind];
  const uint32_t npairs = (uint32_t)W * (uint32_t)rh;
  uint64_t fl[kFl];
  // NP slot pairs per thread: the least of 2, 4, 6 and kPairs that covers the
  // speculative slots (uniform), so the loop does no work past them
  auto gather = [&](auto np_tag) {
    constexpr int NP = decltype(np_tag)::value;
    const BufRsrc cand_r = make_rsrc(cand, (uint32_t)W * (uint32_t)tc * 8u);
    uint4 cv[NP];
#pragma unroll
    for (int u = 0; u < NP; u++) {
      const uint32_t pp = (uint32_t)(tid + u * kThr);
      const uint32_t sh = __umulhi(pp, rh_magic);
      const uint32_t s0 = sh * (uint32_t)tc + 2u * (pp - sh * (uint32_t)rh);
      cv[u] = buf_load16(cand_r, pp < npairs ? 8u * s0 : 0x80000000u);  // past the end: zeros, no access
    }
    const BufRsrc cn_r = make_rsrc(counts, (uint32_t)W * 4u);
    const BufRsrc fl_r = make_rsrc(floors, (uint32_t)W * 8u);
    const BufRsrc bt_r = make_rsrc(bots, (uint32_t)W * 4u);
    const BufRsrc tp_r = make_rsrc(tops, (uint32_t)W * 4u);
    uint32_t cn[kFl], bt[kFl], tp[kFl];
#pragma unroll
    for (int f = 0; f < kFl; f++) {
      const uint32_t sj = (uint32_t)(tid + f * kThr);
      cn[f] = __builtin_amdgcn_raw_buffer_load_b32(cn_r, 4u * sj, 0, 0);
      fl[f] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(fl_r, 8u * sj, 0, 0));
      bt[f] = __builtin_amdgcn_raw_buffer_load_b32(bt_r, 4u * sj, 0, 0);
      tp[f] = __builtin_amdgcn_raw_buffer_load_b32(tp_r, 4u * sj, 0, 0);
    }
    // the histogram and the bitmap start clear
    for (int i = tid; i < kBins; i += kThr) L.hist[i] = 0u;
    for (int i = tid; i < bw(nw); i += kThr) L.bits[i] = 0u;
    uint64_t fmax = 0ull;
    bool over = false;
    uint32_t lo = ~0u, hi = 0u;
#pragma unroll
    for (int f = 0; f < kFl; f++) {
      if (tid + f * kThr < W) L.idx[tid + f * kThr] = cn[f];
      fmax = max(fmax, fl[f]);
      over = over || (int)cn[f] > R;  // zero past W
      lo = cn[f] ? min(lo, bt[f]) : lo;
      hi = cn[f] ? max(hi, tp[f]) : hi;
    }
    fmax = wave_max(fmax);
    const bool wover = __ballot(over) != 0ull;
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) {
      L.wfm[wave] = fmax;
      L.wov[wave] = wover ? 1 : 0;
      L.wmx[wave] = hi;
      L.wmn[wave] = lo;
    }
    if (tid == 0) {
      L.n = 0;
      L.n_tie = 0;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kScoreWaves; w++) {
      lo = min(lo, L.wmn[w]);
      hi = max(hi, L.wmx[w]);
    }
    const int shift = bin_shift(lo, hi);
    // ---- the written slots into L.set, each counted in its bin
    uint64_t k[2 * NP];
    bool v[2 * NP];
    int nv = 0;
#pragma unroll
    for (int u = 0; u < NP; u++) {
      const uint32_t pp = (uint32_t)(tid + u * kThr);
      const uint32_t sh = __umulhi(pp, rh_magic);
      const int o = 2 * (int)(pp - sh * (uint32_t)rh);  // the pair's first slot in its stretch
      const int c = sh < (uint32_t)W ? (int)L.idx[sh] : 0;
      v[2 * u] = o < c;
      v[2 * u + 1] = o + 1 < c;
      k[2 * u] = ((uint64_t)cv[u].y << 32) | cv[u].x;
      k[2 * u + 1] = ((uint64_t)cv[u].w << 32) | cv[u].z;
      nv += (v[2 * u] ? 1 : 0) + (v[2 * u + 1] ? 1 : 0);
    }
    // every lane stores every key, the unwritten ones to its own spare slot in
    // L.out (free until the selection); the written ones are counted
    int slot = wave_alloc(nv, &L.n);
#pragma unroll
    for (int i = 0; i < 2 * NP; i++) {
      uint64_t* dst = v[i] ? &L.set[slot] : &L.out[lane];
      *dst = k[i];
      slot += v[i] ? 1 : 0;
      if (v[i]) atomicAdd(&L.hist[(((uint32_t)(k[i] >> 32)) - lo) >> shift], 1u);
    }
    // stretches holding more than R keys: the rest, one wave per stretch
    bool any_over = false;
#pragma unroll
    for (int w = 0; w < kScoreWaves; w++) any_over = any_over || L.wov[w] != 0;
    if (any_over) {  // uniform
      for (int j = wave; j < W; j += kScoreWaves) {
        const int c = (int)L.idx[j];
        for (int o = R + lane; o - lane < c; o += 64) {  // wave-uniform trip count
          const bool has = o < c;
          const uint64_t x = has ? cand[(int64_t)j * tc + o] : 0ull;
          const int so = wave_slot(has, &L.n);
          if (has) {
            L.set[so] = x;
            atomicAdd(&L.hist[(((uint32_t)(x >> 32)) - lo) >> shift], 1u);
          }
        }
      }
    }
    __syncthreads();
  };
  const uint32_t np = (npairs + kThr - 1) / kThr;  // uniform
  if (np <= 2)
    gather(IntC<2>{});
  else if (np <= 4)
    gather(IntC<4>{});
  else if (kPairs > 6 && np <= 6)
    gather(IntC<6>{});
  else
    gather(IntC<kPairs>{});
  int n = L.n;
  uint32_t lo = ~0u, hi = 0u;
  uint64_t gfmax = 0ull;
#pragma unroll
  for (int w = 0; w < kScoreWaves; w++) {
    lo = min(lo, L.wmn[w]);
    hi = max(hi, L.wmx[w]);
    gfmax = max(gfmax, L.wfm[w]);
  }
  // Reindex: the entries of this thread's candidate slots load during the
  // selection (the same L.set positions are read at the output unless a repair
  // changes the set)
  constexpr int kPf = 4;
  int32_t pe[kPf];
  bool pf_ok = Reindex && n <= kPf * kThr;  // uniform
  if (pf_ok) {
    const int32_t* pool = a.pool_in + bq * kPool;
#pragma unroll
    for (int r = 0; r < kPf; r++) {
      const int i = tid + r * kThr;
      const uint64_t x = L.set[i];
      pe[r] = pool[i < n ? key_id(x) : 0u];  // a slot below kPool
    }
  }
  // S* = 0 when every candidate is taken
  uint64_t s_star = n > K ? select_kth(L, n, K, lo, hi, direct, true) : 0ull;
  bool marked = n > K;  // the bitmap holds the selection

  // ---- while a floor is above S*, repair the share with the largest and select again
  if (gfmax > s_star) {
    marked = false;
    pf_ok = false;
    bool query_ready = false;
    for (int round = 0; round < W; round++) {  // every round clears one share's floor
      // the share with the largest floor above S* (lowest index on ties)
      uint64_t best = 0ull;
      int bj = -1;
#pragma unroll
      for (int f = 0; f < kFl; f++) {
        const int jj = tid + f * kThr;
        if (jj < W && fl[f] > s_star && fl[f] > best) {
          best = fl[f];
          bj = jj;
        }
      }
      const uint64_t wbest = wave_max(best);
      const uint64_t m = __ballot(best == wbest && bj >= 0);
      int wj = -1;
      if (m) wj = __builtin_amdgcn_readlane(bj, __ffsll((unsigned long long)m) - 1);
      if (lane == 0) {
        L.wfl[wave] = wbest;
        L.wj[wave] = wj;
      }
      __syncthreads();
      uint64_t gbest = 0ull;
      int gj = -1;
      for (int w = 0; w < kScoreWaves; w++)
        if (L.wj[w] >= 0 && (L.wfl[w] > gbest || (L.wfl[w] == gbest && L.wj[w] < gj))) {
          gbest = L.wfl[w];
          gj = L.wj[w];
        }
      __syncthreads();
      if (gj < 0) break;  // uniform: every floor is below S*
      if (!query_ready) {
        const int t = tid & 255;
        const float qv = a.iq[bq * 256 + t];
        const float wh = a.iw ? a.iw[bq * 4 + (t >> 6)] : 1.0f;
        if (tid < 256) prep_query(qv, wh, L.q8, L.c, t);
        __syncthreads();
        query_ready = true;
      }
      // keep only the candidates at or above S*, then add share gj's unwritten keys above S*
      if (n > K) {
        if (tid == 0) L.n_out = 0;
        __syncthreads();
        for (int i0 = 0; i0 < n; i0 += kThr) {
          const int i = i0 + tid;
          const uint64_t x = i < n ? L.set[i] : 0ull;
          const bool keep = i < n && x >= s_star;
          const int so = wave_slot(keep, &L.n_out);
          if (keep) L.out[so] = x;  // at most K kept
        }
        __syncthreads();
        const int nk = L.n_out;
        for (int i = tid; i < nk; i += kThr) L.set[i] = L.out[i];
        if (tid == 0) L.n = nk;
        __syncthreads();
      }
      repair_share<Reindex>(a, bq, kind, gj, cuts[gj], s_star, n_vis, L);
      if (tid == 0 && L.n > C::kSet) L.n = C::kSet;  // never reached: at most K kept plus one share's keys
      __syncthreads();
#pragma unroll
      for (int f = 0; f < kFl; f++)
        if (tid + f * kThr == gj) fl[f] = 0ull;
      n = L.n;
      if (n > K) {
        for (int i = tid; i < kBins; i += kThr) L.hist[i] = 0u;
        if (tid == 0) L.n_tie = 0;
        key_range(L, n, lo, hi);  // synchronises after the clears
        s_star = select_kth(L, n, K, lo, hi, false);
      } else {
        s_star = 0ull;
      }
    }
    if (direct) {
      for (int i = tid; i < bw(nw); i += kThr) L.bits[i] = 0u;
      __syncthreads();
    }
  }

  constexpr int kR = C::kSet / kThr;  // candidates per thread at most
  if (direct) {
    // ---- Full: one bit per selected id, then each thread writes the ids of its
    // words in ascending order from its offset
    if (!marked) {  // uniform
      with_keys<std::remove_reference_t<decltype(L)>::Cfg::kSet / kScoreThreads>(L.set, n, [&](auto& b) {
#pragma unroll
        for (int r = 0; r < b.kN; r++)
          if (b.x[r] && b.x[r] >= s_star) set_bit(L.bits, key_id(b.x[r]));  // ids below universe
      });
      __syncthreads();
    }
    // thread t owns words [N t, N t + N), contiguous so that its ids are one run
    // of the ascending order, with N the least of 1, 2, 4, 8, 16, 20 that covers
    // the bitmap; its words load together
    auto emit = [&](auto tag) {
      constexpr int N = decltype(tag)::value;
      const int w0 = tid * N;
      uint32_t wd[N];
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < N; i++) {
        const uint32_t v = L.bits[bw(w0 + i)];  // inside L.bits: 512 N <= C::kBitW
        wd[i] = w0 + i < nw ? v : 0u;
        cnt += __popc(wd[i]);
      }
      int nsel;
      int pos = block_scan_excl1(cnt, L.tmp, &nsel);  // at most K set
      if (kind == 0) {
        // sparse: each selected id's rank is the selected ids before its word
        // plus the set bits below it in the word
#pragma unroll
        for (int i = 0; i < N; i++) {
          if (w0 + i < nw) L.woff[bw(w0 + i)] = (uint32_t)pos;
          pos += __popc(wd[i]);
        }
        __syncthreads();
        // (Reindex: an id is a pool slot; the pool is ascending, so slot order
        // is entry order, and the slot's entry is written)
        int32_t* dst = a.topk_out + bq * kTopK;
        const int32_t* pool = Reindex ? a.pool_in + bq * kPool : nullptr;
        with_keys<std::remove_reference_t<decltype(L)>::Cfg::kSet / kScoreThreads>(L.set, n, [&](auto& b) {
#pragma unroll
          for (int r = 0; r < b.kN; r++) {
            if (b.x[r] && b.x[r] >= s_star) {
              const uint32_t id = key_id(b.x[r]);
              const uint32_t w = id >> 5;
              const int rank = (int)L.woff[bw((int)w)] + __popc(L.bits[bw((int)w)] & ((1u << (id & 31u)) - 1u));
              int32_t v = (int32_t)id;
              if (Reindex) v = (pf_ok && r < kPf) ? pe[r < kPf ? r : 0] : pool[id];
              if (rank < kTopK) dst[rank] = v;
            }
          }
        });
        for (int i = nsel + tid; i < kTopK; i += kThr) dst[i] = -1;
      } else if constexpr (C::kWide) {
        // the chosen blocks in ascending order into L.idx, then each expanded to
        // its visible entries (every chosen block is full except possibly the one
        // holding the last visible entry, so block r of the order fills slots
        // 8r .. 8r+7): thread t writes the int4 chunks t + 512 k
        if (bw(nw) <= 2 * C::kOut) {  // uniform: the word offsets fit in L.out, below L.idx
          // as the Top-512: each chosen block's rank is the chosen blocks
          // before its word plus the set bits below it in the word (no loop
          // over the bits of a word, whose length differs from lane to lane)
#pragma unroll
          for (int i = 0; i < N; i++) {
            if (w0 + i < nw) L.woff[bw(w0 + i)] = (uint32_t)pos;
            pos += __popc(wd[i]);
          }
          __syncthreads();
          with_keys<std::remove_reference_t<decltype(L)>::Cfg::kSet / kScoreThreads>(L.set, n, [&](auto& b) {
#pragma unroll
            for (int r = 0; r < b.kN; r++) {
              if (b.x[r] && b.x[r] >= s_star) {
                const uint32_t id = key_id(b.x[r]);
                const int w = (int)(id >> 5);
                const int rank = (int)L.woff[bw(w)] + __popc(L.bits[bw(w)] & ((1u << (id & 31u)) - 1u));
                if (rank < kPoolBlocks) L.idx[rank] = id;
              }
            }
          });
        } else {
#pragma unroll
          for (int i = 0; i < N; i++) {
            uint32_t m = wd[i];
            while (m) {
              const int b = __ffs(m) - 1;
              m &= m - 1u;
              if (pos < kPoolBlocks) L.idx[pos] = (uint32_t)(32 * (w0 + i) + b);
              pos++;
            }
          }
        }
        __syncthreads();
        int4* po = reinterpret_cast<int4*>(a.pool_out + bq * kPool);
#pragma unroll
        for (int k = 0; k < 2 * kPoolBlocks / kThr; k++) {
          const int c = tid + k * kThr;
          const int p = c >> 1;
          int4 v = make_int4(-1, -1, -1, -1);
          if (p < nsel) {
            const int e0 = (int)L.idx[p] * kBlock + 4 * (c & 1);
            v = make_int4(e0 < n_vis ? e0 : -1, e0 + 1 < n_vis ? e0 + 1 : -1, e0 + 2 < n_vis ? e0 + 2 : -1,
                          e0 + 3 < n_vis ? e0 + 3 : -1);
          }
          po[c] = v;
        }
      }
    };
    const int wpt = (nw + kThr - 1) / kThr;  // uniform, at most C::kBitW / kThr
    if (wpt <= 1) {
      emit(IntC<1>{});
    } else if (wpt <= 2) {
      emit(IntC<2>{});
    } else if (wpt <= 4) {
      emit(IntC<4>{});
    } else {
      if constexpr (C::kBitW / kScoreThreads > 4) {
        if (wpt <= 8)
          emit(IntC<8>{});
        else if (wpt <= 16)
          emit(IntC<16>{});
        else
          emit(IntC<C::kBitW / kScoreThreads>{});
      }
    }
  } else if constexpr (C::kWide) {
    // ---- the selected keys: every candidate at or above S*, one LDS atomic per wave
    if (tid == 0) L.n_out = 0;
    __syncthreads();
    {
      int nt = 0;
#pragma unroll
      for (int r = 0; r < kR; r++) {
        const int i = tid + r * kThr;
        const uint64_t x = i < n ? L.set[i] : 0ull;
        nt += (x != 0ull && x >= s_star) ? 1 : 0;
      }
      int so = wave_alloc(nt, &L.n_out);
#pragma unroll
      for (int r = 0; r < kR; r++) {
        const int i = tid + r * kThr;
        const uint64_t x = i < n ? L.set[i] : 0ull;
        if (x != 0ull && x >= s_star && so < kPoolBlocks) L.out[so++] = x;  // at most K taken
      }
    }
    __syncthreads();
    const int nsel = min(L.n_out, K);

    // ---- ascending output.  Thread t holds the selected ids t + 512 j.  A
    // Reindex id is a pool slot: the pool is ascending, so slot order is entry
    // order, and the entry loads while the slots are ranked.
    constexpr int kPer = kPoolBlocks / kThr;
    const int per = K / kThr;
    uint32_t id[kPer];
    int32_t ent[kPer];
#pragma unroll
    for (int jj = 0; jj < kPer; jj++) {
      const int i = tid + jj * kThr;
      id[jj] = (jj < per && i < nsel) ? key_id(L.out[i]) : kNoId;
    }
    if (Reindex) {
      const int32_t* pool = a.pool_in + bq * kPool;
#pragma unroll
      for (int jj = 0; jj < kPer; jj++) ent[jj] = pool[id[jj] != kNoId ? id[jj] : 0u];
    }
    uint32_t* bits = reinterpret_cast<uint32_t*>(L.set);  // the candidates are no longer needed
    if (universe <= 32 * (int64_t)kRankWords) {
      int rank[kPer];
      rank_ids(id, universe, rank, bits, L.tmp);
      if (kind == 0) {
        int32_t* dst = a.topk_out + bq * kTopK;
        if (id[0] != kNoId) dst[rank[0]] = Reindex ? ent[0] : (int32_t)id[0];
        if (tid >= nsel) dst[tid] = -1;
      } else {
        int4* po = reinterpret_cast<int4*>(a.pool_out + bq * kPool);
#pragma unroll
        for (int jj = 0; jj < kPer; jj++) {
          if (id[jj] == kNoId) continue;
          int e[8];
          const int base = (int)id[jj] * kBlock;
#pragma unroll
          for (int t = 0; t < 8; t++) e[t] = base + t < n_vis ? base + t : -1;
          po[2 * rank[jj]] = make_int4(e[0], e[1], e[2], e[3]);
          po[2 * rank[jj] + 1] = make_int4(e[4], e[5], e[6], e[7]);
        }
        for (int i = nsel + tid; i < kPoolBlocks; i += kThr) {
          po[2 * i] = make_int4(-1, -1, -1, -1);
          po[2 * i + 1] = make_int4(-1, -1, -1, -1);
        }
      }
    } else {
      // wide id ranges (Full only): bucketed ordering through LDS
#pragma unroll
      for (int jj = 0; jj < kPer; jj++)
        if (id[jj] != kNoId) L.idx[tid + jj * kThr] = id[jj];
      __syncthreads();
      uint32_t* s_ord = reinterpret_cast<uint32_t*>(L.out);  // free once idx holds the ids
      // entries of one 4,096-entry stretch share idx >> 12; blocks of one, idx >> 9
      order_ascending(L.idx, nsel, kind ? 9 : 12, s_ord, bits, L.take, L.off, L.ge, L.tmp);
      if (kind == 0) {
        int4* dst = reinterpret_cast<int4*>(a.topk_out + bq * kTopK);
        for (int i = tid; i < kTopK / 4; i += kThr) {
          int4 v;
          v.x = 4 * i + 0 < nsel ? (int)s_ord[4 * i + 0] : -1;
          v.y = 4 * i + 1 < nsel ? (int)s_ord[4 * i + 1] : -1;
          v.z = 4 * i + 2 < nsel ? (int)s_ord[4 * i + 2] : -1;
          v.w = 4 * i + 3 < nsel ? (int)s_ord[4 * i + 3] : -1;
          dst[i] = v;
        }
      } else {
        int4* po = reinterpret_cast<int4*>(a.pool_out + bq * kPool);
        for (int i = tid; i < kPoolBlocks; i += kThr) {
          int e[8];
          if (i < nsel) {
            const int base = (int)s_ord[i] * kBlock;
#pragma unroll
            for (int t = 0; t < 8; t++) e[t] = base + t < n_vis ? base + t : -1;
          } else {
#pragma unroll
            for (int t = 0; t < 8; t++) e[t] = -1;
          }
          po[2 * i] = make_int4(e[0], e[1], e[2], e[3]);
          po[2 * i + 1] = make_int4(e[4], e[5], e[6], e[7]);
        }
      }
    }
  }
  // ---- a fused append's length, once every kernel of the call that reads the old one is done
  if (!Reindex && a.app_T > 0 && kind == 0 && (bq % a.Q) == 0 && tid == 0) {
    const int32_t nl = a.ws.nvis[bq * 2 + 1];
    if (nl >= 0) a.length[bq / a.Q] = nl;
  }
}

// ------------------------------------------------------------------ launch
CSA2_DEV_ERROR_TAKER(take_head_dev_error)

// per share: the keys wanted when every share holds as many keys (1.25 times
// its even share of K, plus 16; each share scales this by its own
// keys in the kernel) and the most it may write (the query's kHeadCap split
// evenly).  A share holding more of the Top-K than it wrote is re-scored by
// the select kernel.
static void head_targets(int W, int K, int32_t& T, int32_t& T_cap, int cap_total = kHeadCap) {
  T_cap = (cap_total / W) & ~1;  // even: the select kernel loads slot pairs
  const int want = (5 * K + 4 * W - 1) / (4 * W) + 16;
  T = want < T_cap ? want : T_cap;
}

// The select kernel over the heads of W shares per query (iters batches each);
// `lean`: the SelLean instance (kind 0, ids below 65,536, at most 8 batches a
// share), whose stretches hold SelLean::kSet / W keys.
static hipError_t launch_select(const LaunchCache& c, bool reindex, const float* iq, const float* iw,
                                const int32_t* pool_in, int32_t* topk_out, int32_t* pool_out, int32_t Q, int W,
                                int iters, int32_t app_T, int rotate, int kinds, const HeadWs& ws, bool lean,
                                hipStream_t stream) {
  const int64_t bq = (int64_t)c.batch * Q;
  int32_t T[2], T_cap[2];
  const int cap_total = lean ? SelLean::kSet : kHeadCap;
  head_targets(W, kTopK, T[0], T_cap[0], cap_total);
  head_targets(W, kPoolBlocks, T[1], T_cap[1], cap_total);
  SelectArgs s;
  s.ik_codes = c.ik_codes;
  s.ik_scales = c.ik_scales;
  s.length = c.length;
  s.cap = c.capacity;
  s.ratio = c.ratio;
  s.iq = iq;
  s.iw = iw;
  s.pool_in = pool_in;
  s.Q = Q;
  s.W = W;
  s.iters = iters;
  s.app_T = app_T;
  s.rotate = rotate;
  s.tc = T_cap[0];
  for (int k = 0; k < 2; k++) {
    // twice the keys wanted covers a share's count but for a wide boundary bin
    const int r = 2 * T[k] < s.tc ? 2 * T[k] : s.tc;
    s.spec[k] = (r + 1) & ~1;
    s.spec_magic[k] = (uint32_t)((1ull << 32) / (uint64_t)(s.spec[k] / 2) + 1ull);
  }
  s.ws = ws;
  s.topk_out = topk_out;
  s.pool_out = reindex ? nullptr : pool_out;
  const dim3 sgrid((unsigned)bq, (unsigned)kinds);
  if (reindex)
    hipLaunchKernelGGL((index_select_kernel<true, SelAll>), sgrid, dim3(kScoreThreads), 0, stream, s);
  else if (lean)
    hipLaunchKernelGGL((index_select_kernel<false, SelLean>), sgrid, dim3(kScoreThreads), 0, stream, s);
  else
    hipLaunchKernelGGL((index_select_kernel<false, SelAll>), sgrid, dim3(kScoreThreads), 0, stream, s);
  return hipGetLastError();
}

hipError_t launch_index_head(const LaunchCache& c, bool reindex, const float* iq, const float* iw,
                             const int32_t* q_pos, const int32_t* pool_in, int32_t* topk_out, int32_t* pool_out,
                             int32_t Q, const float* app_kv, const float* app_ik, int32_t app_T, void* ws_head,
                             hipStream_t stream) {
  const int64_t bq = (int64_t)c.batch * Q;
  if (bq == 0) return hipSuccess;
  const int kinds = (!reindex && pool_out) ? 2 : 1;
  HeadArgs h;
  h.ik_codes = c.ik_codes;
  h.ik_scales = c.ik_scales;
  h.kv_codes_w = c.kv_codes;
  h.kv_scales_w = c.kv_scales;
  h.ik_codes_w = c.ik_codes;
  h.ik_scales_w = c.ik_scales;
  h.length = c.length;
  h.cap = c.capacity;
  h.ratio = c.ratio;
  h.iq = iq;
  h.iw = iw;
  h.q_pos = q_pos;
  h.pool_in = pool_in;
  h.Q = Q;
  h.W = head_workgroups(reindex, c.capacity, bq);
  if (reindex) {
    h.iters = kReindexIters;
  } else {
    const int64_t batches = ((int64_t)c.capacity + kBatchKeys - 1) / kBatchKeys;
    h.iters = (int32_t)((batches + h.W - 1) / h.W);
  }
  h.blocks = kinds == 2 ? 1 : 0;
  head_targets(h.W, kTopK, h.T[0], h.T_cap[0]);
  head_targets(h.W, kPoolBlocks, h.T[1], h.T_cap[1]);
  h.app_kv = app_kv;
  h.app_ik = app_ik;
  h.app_T = app_T;
  h.ws = head_ws_carve(ws_head, bq, c.capacity);
  const dim3 grid((unsigned)bq, (unsigned)h.W);
  if (reindex)
    hipLaunchKernelGGL(index_head_kernel<true>, grid, dim3(kScoreThreads), 0, stream, h);
  else
    hipLaunchKernelGGL(index_head_kernel<false>, grid, dim3(kScoreThreads), 0, stream, h);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_select(c, reindex, iq, iw, pool_in, topk_out, pool_out, Q, h.W, h.iters, app_T, 1, kinds, h.ws,
                       false, stream);
}

// Full with four or more queries per sequence and no pool: the shared-load
// heads, four queries per workgroup, then the select kernel.  (Eight per
// workgroup share each load twice as widely, but their 64 keys per lane leave
// room for one workgroup per compute unit, not two: slower at the
// 2,048-query prefill.)
hipError_t launch_index_shared_heads(const LaunchCache& c, const float* iq, const float* iw, const int32_t* q_pos,
                                     int32_t* topk_out, int32_t* pool_out, int32_t Q, void* ws_head,
                                     hipStream_t stream) {
  const int64_t bq = (int64_t)c.batch * Q;
  if (bq == 0) return hipSuccess;
  const int qpw = 4;
  SharedHeadArgs h;
  h.ik_codes = c.ik_codes;
  h.ik_scales = c.ik_scales;
  h.length = c.length;
  h.cap = c.capacity;
  h.ratio = c.ratio;
  h.iq = iq;
  h.iw = iw;
  h.q_pos = q_pos;
  h.Q = Q;
  h.W = shared_head_workgroups(c.capacity);
  const int64_t batches = ((int64_t)c.capacity + kBatchKeys - 1) / kBatchKeys;
  h.iters = (int32_t)((batches + h.W - 1) / h.W);  // at most kSharedIters
  // the lean select serves ids below 65,536 (every query's visible entries
  // are at most the capacity)
  const bool lean = !pool_out && c.capacity <= 32 * SelLean::kBitW;
  int32_t T;
  head_targets(h.W, kTopK, T, h.T_cap, lean ? SelLean::kSet : kHeadCap);
  h.ws = head_ws_carve(ws_head, bq, c.capacity);
  const dim3 grid((unsigned)((int64_t)c.batch * ((Q + qpw - 1) / qpw) * h.W));
  if (pool_out)
    hipLaunchKernelGGL((index_shared_head_kernel<1, true>), grid, dim3(kScoreThreads), 0, stream, h);
  else
    hipLaunchKernelGGL((index_shared_head_kernel<1, false>), grid, dim3(kScoreThreads), 0, stream, h);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_select(c, false, iq, iw, nullptr, topk_out, pool_out, Q, h.W, h.iters, 0, 0, pool_out ? 2 : 1, h.ws,
                       lean, stream);
}

}  // namespace csa2

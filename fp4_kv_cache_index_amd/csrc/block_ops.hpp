// Workgroup-wide building blocks for the selection kernels: reductions,
// exclusive scan and exact top-k thresholds.  All operate on
// LDS data and must be called by every thread of the workgroup (blockDim a
// multiple of 64, at most 1024).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

// ---- wave-wide primitives on DPP (cross-lane moves inside the VALU; the
// __shfl family goes through the LDS crossbar with its latency)
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside each 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i inside each row of 16
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;  // row_shr:n

template <int Ctrl>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, Ctrl, 0xF, 0xF, true);
}
template <int Ctrl>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
  return (uint64_t)dpp32<Ctrl>((uint32_t)v) | ((uint64_t)dpp32<Ctrl>((uint32_t)(v >> 32)) << 32);
}
template <int Ctrl, typename T>
__device__ __forceinline__ T dpp(T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 8) return __builtin_bit_cast(T, dpp64<Ctrl>(__builtin_bit_cast(uint64_t, v)));
  else return __builtin_bit_cast(T, dpp32<Ctrl>(__builtin_bit_cast(uint32_t, v)));
}
template <typename T>
__device__ __forceinline__ T readlane(T v, int l) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 8) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(T, (uint64_t)lo | ((uint64_t)hi << 32));
  } else {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
  }
}

// Reduce over the wave with a commutative, associative op; every lane gets the result.
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = op(v, dpp<kDppXor1>(v));
  v = op(v, dpp<kDppXor2>(v));
  v = op(v, dpp<kDppHalfMirror>(v));
  v = op(v, dpp<kDppMirror>(v));  // every lane holds its row's result
  return op(op(readlane(v, 0), readlane(v, 16)), op(readlane(v, 32), readlane(v, 48)));
}
// Reduce over each DPP row of 16 lanes; every lane gets its row's result.
template <typename T, typename Op>
__device__ __forceinline__ T wave_row_reduce(T v, Op op) {
  v = op(v, dpp<kDppXor1>(v));
  v = op(v, dpp<kDppXor2>(v));
  v = op(v, dpp<kDppHalfMirror>(v));
  return op(v, dpp<kDppMirror>(v));
}
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  return wave_reduce(v, [](T x, T y) { return x + y; });
}
template <typename T>
__device__ __forceinline__ T wave_min(T v) {
  return wave_reduce(v, [](T x, T y) { return y < x ? y : x; });
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
  return wave_reduce(v, [](T x, T y) { return y > x ? y : x; });
}

// Inclusive prefix sum over the 64 lanes (lane 0 first), 32-bit.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += dpp32<kDppShr1>(x);  // out-of-row sources read 0
  x += dpp32<kDppShr2>(x);
  x += dpp32<kDppShr4>(x);
  x += dpp32<kDppShr8>(x);  // inclusive scan inside each row of 16
  const uint32_t r0 = readlane(x, 15), r1 = readlane(x, 31), r2 = readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// Slot from an LDS counter for every lane whose `pred` holds, with one atomic
// per wave; the lanes get consecutive slots in lane order.  Every lane of the
// wave must call it (returns -1 where pred is false).
__device__ __forceinline__ int wave_slot(bool pred, int* counter) {
  const uint64_t mask = __ballot(pred);
  if (mask == 0ull) return -1;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((unsigned long long)mask) - 1;
  int base = 0;
  if (lane == leader) base = atomicAdd(counter, __popcll(mask));
  base = __builtin_amdgcn_readlane(base, leader);
  return pred ? base + __popcll(mask & ((1ull << lane) - 1ull)) : -1;
}

// Reserve `count` consecutive slots per lane from an LDS counter with one
// atomic per wave; returns this lane's first slot (lanes in order).  Every lane
// of the wave must call it.
__device__ __forceinline__ int wave_alloc(int count, int* counter) {
  const uint32_t incl = wave_incl_scan((uint32_t)count);
  const uint32_t total = readlane(incl, 63);
  int base = 0;
  if ((threadIdx.x & 63) == 0 && total) base = atomicAdd(counter, (int)total);
  base = __builtin_amdgcn_readlane(base, 0);
  return base + (int)incl - count;
}

// Workgroup order aware of the 8 XCDs: the dispatcher deals workgroups to the
// XCDs round-robin (workgroup L to XCD L mod 8), and each XCD has its own L2.
// Rank r = (L mod 8) * (n / 8) + L / 8 gives XCD x the consecutive ranks
// [x n/8, (x+1) n/8), so workgroups of consecutive rank (one query's
// attention splits or merge heads, a sequence's index query groups) share an
// XCD and its L2.
// Identity when n is not a multiple of 8.  Placement only: no result depends
// on it.
__device__ __forceinline__ int64_t xcd_rank(int64_t L, int64_t n) {
  return (n & 7) == 0 ? (L & 7) * (n >> 3) + (L >> 3) : L;
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also makes
// the thread's global stores visible to the workgroup, and on gfx9 that means
// waiting for every global load, store and atomic the thread has in flight
// (they all count in vmcnt), prefetches included; this barrier leaves them in
// flight.  Use it where the threads exchange data through LDS alone.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Exclusive prefix sum of one int per thread over the workgroup; `tmp` holds
// one int per wave.  Returns the exclusive prefix, writes the total to *total.
__device__ __forceinline__ int block_scan_excl(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  const int x = (int)wave_incl_scan((uint32_t)v);
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < nw; w++) {
    const int t = tmp[w];
    if (w < wave) before += t;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// block_scan_excl with one barrier: the caller writes tmp again only after
// another barrier.
__device__ __forceinline__ int block_scan_excl1(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  const int x = (int)wave_incl_scan((uint32_t)v);
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < nw; w++) {
    const int t = tmp[w];
    if (w < wave) before += t;
    all += t;
  }
  *total = all;
  return before + x - v;
}

// Exclusive offsets of v[0..n) (LDS) into off[] (LDS); returns the total.
__device__ __forceinline__ int block_offsets(const int* v, int* off, int n, int* tmp) {
  int carry = 0;
  for (int base = 0; base < n; base += blockDim.x) {
    const int c = base + threadIdx.x;
    const int x = c < n ? v[c] : 0;
    int tot;
    const int ex = block_scan_excl(x, tmp, &tot);
    if (c < n) off[c] = carry + ex;
    carry += tot;
  }
  __syncthreads();
  return carry;
}

struct SelShared {
  uint32_t hist[256];
  uint64_t wmin[16], wmax[16];
  uint32_t wcnt[16];
  uint64_t small[64];
  uint64_t kbc[2];
  int ibc[6];
};

// Threshold of the top k among unique keys get(0) .. get(n-1), where a key of 0
// marks "no key": returns T such that exactly min(k, number of nonzero keys)
// keys are >= T (T = 1 when there are at most k).  *n_keys receives the number
// of nonzero keys.  `get` reads LDS (or registers) and is called many times.
//
// Most-significant-digit radix select.  The bits above the highest bit in which
// the keys differ are fixed at once; each pass then counts the next 8 bits of
// the keys still in the running into a 256-bin LDS histogram (atomic adds), and
// one wave finds the digit that holds the k-th key.  Once that bucket has at
// most 64 keys, one wave ranks them and the key of rank k is the answer.
template <typename Key, typename Get>
__device__ Key topk_threshold(Get get, int n, int k, SelShared& S, int* n_keys) {
  constexpr int kBits = (int)sizeof(Key) * 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  // ---- common prefix and count of the keys
  Key lo = ~(Key)0, hi = 0;
  int cnt = 0;
  for (int i = tid; i < n; i += blockDim.x) {
    const Key x = get(i);
    if (x == 0) continue;
    lo = x < lo ? x : lo;
    hi = x > hi ? x : hi;
    cnt++;
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  cnt = wave_sum(cnt);
  if (lane == 0) {
    S.wmin[wave] = (uint64_t)lo;
    S.wmax[wave] = (uint64_t)hi;
    S.wcnt[wave] = (uint32_t)cnt;
  }
  for (int i = tid; i < 256; i += blockDim.x) S.hist[i] = 0u;
  __syncthreads();
  {
    Key l = ~(Key)0, h = 0;
    int c = 0;
    for (int w = 0; w < nw; w++) {
      l = (Key)S.wmin[w] < l ? (Key)S.wmin[w] : l;
      h = (Key)S.wmax[w] > h ? (Key)S.wmax[w] : h;
      c += (int)S.wcnt[w];
    }
    lo = l;
    hi = h;
    cnt = c;
  }
  __syncthreads();  // every thread has read S.wmin/wmax/wcnt
  *n_keys = cnt;
  if (cnt <= k) return (Key)1;
  const Key diff = lo ^ hi;  // nonzero: the keys are unique and there are more than k >= 1
  int top = kBits - (kBits == 64 ? __clzll((long long)diff) : __clz((int)diff));  // bits [0, top) differ
  Key mask = top >= kBits ? (Key)0 : (Key)(~(Key)0 << top);
  Key prefix = hi & mask;
  int bucket = cnt;  // keys under the current prefix
  while (bucket > 64 && top > 0) {
    const int width = top < 8 ? top : 8;
    const int shift = top - width;
    const uint32_t dmask = (1u << width) - 1u;
    // the histogram is zero here: cleared before the first pass, and by its
    // reader after each pass
    for (int i = tid; i < n; i += blockDim.x) {
      const Key x = get(i);
      if (x == 0 || (x & mask) != prefix) continue;
      atomicAdd(&S.hist[(uint32_t)(x >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns digits 255-4l .. 252-4l, so a prefix sum over the lanes
      // counts the keys in all digits above a lane's four
      uint32_t c[4];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        c[j] = S.hist[255 - 4 * lane - j];
        S.hist[255 - 4 * lane - j] = 0u;
      }
      const uint32_t own = c[0] + c[1] + c[2] + c[3];
      uint32_t above = wave_incl_scan(own) - own;
#pragma unroll
      for (int j = 0; j < 4; j++) {  // this lane's digits, descending
        if ((int)above < k && (int)(above + c[j]) >= k) {
          S.ibc[0] = 255 - 4 * lane - j;
          S.ibc[1] = k - (int)above;
          S.ibc[2] = (int)c[j];
        }
        above += c[j];
      }
    }
    __syncthreads();
    const int d = S.ibc[0];
    k = S.ibc[1];
    bucket = S.ibc[2];
    prefix |= (Key)d << shift;
    mask |= (Key)dmask << shift;
    top = shift;
    __syncthreads();
  }
  if (top == 0) return prefix;  // every bit fixed (only unique keys reach here with bucket <= 1)
  // ---- small bucket: gather it and let one wave rank it
  if (tid == 0) S.ibc[3] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += blockDim.x) {
    const Key x = get(i);
    if (x == 0 || (x & mask) != prefix) continue;
    const int slot = atomicAdd(&S.ibc[3], 1);
    if (slot < 64) S.small[slot] = (uint64_t)x;
  }
  __syncthreads();
  if (wave == 0) {
    // rank each key of the bucket against all of them (broadcast LDS reads)
    const Key v = lane < bucket ? (Key)S.small[lane] : (Key)0;
    int greater = 0;
    for (int j = 0; j < bucket; j++) greater += (Key)S.small[j] > v;
    if (lane < bucket && greater == k - 1) S.kbc[0] = (uint64_t)v;
  }
  __syncthreads();
  const Key t = (Key)S.kbc[0];
  __syncthreads();
  return t;
}

}  // namespace csa2

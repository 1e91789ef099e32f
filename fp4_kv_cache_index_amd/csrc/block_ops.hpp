// Workgroup-wide building blocks for the selection kernels: reductions,
// exclusive scan, exact K-th-largest selection and bitonic sort.  All operate on
// LDS data and must be called by every thread of the workgroup (blockDim a
// multiple of 64, at most 1024).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_min(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const T y = __shfl_xor(v, o);
    v = y < v ? y : v;
  }
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const T y = __shfl_xor(v, o);
    v = y > v ? y : v;
  }
  return v;
}

// Exclusive prefix sum of one int per thread over the workgroup; `tmp` holds
// one int per wave.  Returns the exclusive prefix, writes the total to *total.
__device__ __forceinline__ int block_scan_excl(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
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

struct SelShared {
  uint32_t red[16][8];
  uint64_t wmin[16], wmax[16];
  uint64_t kbc[2];
  int ibc[4];
};

// Exact K-th largest of the eligible keys among a[0..n) (1 <= k <= number of
// eligible keys; keys equal to 0 are not eligible when skip_zero).  Returns the
// key value T; *rem receives how many keys equal to T complete the top k
// (the keys greater than T are k - *rem).
//
// Most-significant-digit radix select with 4-bit digits.  Each thread counts
// its keys into 16 counters held in registers (two 16-bit counters per word),
// the counts are summed across the workgroup, and the digit holding the k-th
// key fixes 4 more bits.  Leading bits common to all eligible keys are skipped,
// and the search stops as soon as every key left under the prefix is needed.
template <typename Key>
__device__ Key select_kth_largest(const Key* a, int n, int k, bool skip_zero, SelShared& S, int* rem) {
  constexpr int kBits = (int)sizeof(Key) * 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  // ---- common prefix of all eligible keys
  Key lo = ~(Key)0, hi = 0;
  for (int i = tid; i < n; i += blockDim.x) {
    const Key x = a[i];
    if (skip_zero && x == 0) continue;
    lo = x < lo ? x : lo;
    hi = x > hi ? x : hi;
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  if (lane == 0) {
    S.wmin[wave] = (uint64_t)lo;
    S.wmax[wave] = (uint64_t)hi;
  }
  __syncthreads();
  if (tid == 0) {
    Key l = ~(Key)0, h = 0;
    for (int w = 0; w < nw; w++) {
      l = (Key)S.wmin[w] < l ? (Key)S.wmin[w] : l;
      h = (Key)S.wmax[w] > h ? (Key)S.wmax[w] : h;
    }
    S.kbc[0] = (uint64_t)l;
    S.kbc[1] = (uint64_t)h;
  }
  __syncthreads();
  lo = (Key)S.kbc[0];
  hi = (Key)S.kbc[1];
  __syncthreads();
  const Key diff = lo ^ hi;
  if (diff == 0) {
    *rem = k;
    return hi;
  }
  const int lead = kBits == 64 ? __clzll((long long)diff) : __clz((int)diff);
  const int top = kBits - (lead / 4) * 4;  // bits [0, top) may differ
  Key mask = top >= kBits ? (Key)0 : (Key)(~(Key)0 << top);
  Key prefix = hi & mask;
  for (int shift = top - 4; shift >= 0; shift -= 4) {
    uint32_t c0 = 0, c1 = 0, c2 = 0, c3 = 0, c4 = 0, c5 = 0, c6 = 0, c7 = 0;
    for (int i = tid; i < n; i += blockDim.x) {
      const Key x = a[i];
      if ((skip_zero && x == 0) || (x & mask) != prefix) continue;
      const uint32_t d = (uint32_t)(x >> shift) & 15u;
      const uint32_t inc = 1u << ((d & 1u) * 16);
      const uint32_t w = d >> 1;
      c0 += w == 0 ? inc : 0u;
      c1 += w == 1 ? inc : 0u;
      c2 += w == 2 ? inc : 0u;
      c3 += w == 3 ? inc : 0u;
      c4 += w == 4 ? inc : 0u;
      c5 += w == 5 ? inc : 0u;
      c6 += w == 6 ? inc : 0u;
      c7 += w == 7 ? inc : 0u;
    }
    c0 = wave_sum(c0); c1 = wave_sum(c1); c2 = wave_sum(c2); c3 = wave_sum(c3);
    c4 = wave_sum(c4); c5 = wave_sum(c5); c6 = wave_sum(c6); c7 = wave_sum(c7);
    if (lane == 0) {
      S.red[wave][0] = c0; S.red[wave][1] = c1; S.red[wave][2] = c2; S.red[wave][3] = c3;
      S.red[wave][4] = c4; S.red[wave][5] = c5; S.red[wave][6] = c6; S.red[wave][7] = c7;
    }
    __syncthreads();
    if (wave == 0) {
      // lane j (< 16) owns digit j: its count, then the count of all larger digits
      uint32_t cnt = 0;
      if (lane < 16) {
        uint32_t s = 0;
        for (int w = 0; w < nw; w++) s += S.red[w][lane >> 1];  // per-lane counts stay below 2^16 / 64
        cnt = (lane & 1) ? (s >> 16) : (s & 0xFFFFu);
      }
      uint32_t incl = cnt;  // sum over digits >= lane
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const uint32_t y = __shfl_down(incl, o, 16);
        if (lane + o < 16) incl += y;
      }
      const int above = (int)(incl - cnt);
      if (lane < 16 && above < k && (int)incl >= k) {
        S.ibc[0] = lane;
        S.ibc[1] = k - above;
        S.ibc[2] = (int)cnt;
      }
    }
    __syncthreads();
    const int d = S.ibc[0];
    k = S.ibc[1];
    const int cd = S.ibc[2];
    prefix |= (Key)d << shift;
    mask |= (Key)15 << shift;
    if (cd == k && shift > 0) {
      // every key under this prefix is needed: the K-th is their minimum
      Key m = ~(Key)0;
      for (int i = tid; i < n; i += blockDim.x) {
        const Key x = a[i];
        if ((skip_zero && x == 0) || (x & mask) != prefix) continue;
        m = x < m ? x : m;
      }
      m = wave_min(m);
      if (lane == 0) S.wmin[wave] = (uint64_t)m;
      __syncthreads();
      Key mm = ~(Key)0;
      for (int w = 0; w < nw; w++) mm = (Key)S.wmin[w] < mm ? (Key)S.wmin[w] : mm;
      int eq = 0;
      for (int i = tid; i < n; i += blockDim.x) eq += (a[i] == mm) && !(skip_zero && mm == 0);
      eq = wave_sum(eq);
      __syncthreads();
      if (lane == 0) S.red[wave][0] = (uint32_t)eq;
      __syncthreads();
      int tot = 0;
      for (int w = 0; w < nw; w++) tot += (int)S.red[w][0];
      __syncthreads();
      *rem = tot;
      return mm;
    }
  }
  *rem = k;
  return prefix;
}

// Bitonic sort of n (power of two) keys in LDS, descending or ascending.
template <typename Key, bool Descending>
__device__ void bitonic_sort(Key* a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n / 2; i += blockDim.x) {
        const int lo = 2 * i - (i & (j - 1));
        const int hi = lo + j;
        const Key x = a[lo], y = a[hi];
        const bool up = (lo & k) == 0;  // this segment's target direction
        const bool swap = Descending ? (up ? x < y : x > y) : (up ? x > y : x < y);
        if (swap) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

}  // namespace csa2

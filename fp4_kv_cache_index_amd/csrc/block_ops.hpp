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
  uint32_t red[16][8];
  uint64_t wmin[16], wmax[16];
  uint64_t small[64];
  uint64_t kbc[2];
  int ibc[6];
};

// Sum each of eight per-lane words over the wave by reduce-scatter (10
// shuffles): lane l ends up with the total of word (l >> 3) & 7.
__device__ __forceinline__ uint32_t wave_reduce8(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t c4,
                                                 uint32_t c5, uint32_t c6, uint32_t c7) {
  const int lane = threadIdx.x & 63;
  const bool h32 = lane & 32, h16 = lane & 16, h8 = lane & 8;
  const uint32_t v0 = (h32 ? c4 : c0) + __shfl_xor(h32 ? c0 : c4, 32);
  const uint32_t v1 = (h32 ? c5 : c1) + __shfl_xor(h32 ? c1 : c5, 32);
  const uint32_t v2 = (h32 ? c6 : c2) + __shfl_xor(h32 ? c2 : c6, 32);
  const uint32_t v3 = (h32 ? c7 : c3) + __shfl_xor(h32 ? c3 : c7, 32);
  const uint32_t w0 = (h16 ? v2 : v0) + __shfl_xor(h16 ? v0 : v2, 16);
  const uint32_t w1 = (h16 ? v3 : v1) + __shfl_xor(h16 ? v1 : v3, 16);
  uint32_t u = (h8 ? w1 : w0) + __shfl_xor(h8 ? w0 : w1, 8);
  u += __shfl_xor(u, 4);
  u += __shfl_xor(u, 2);
  u += __shfl_xor(u, 1);
  return u;
}

// Descending bitonic sort of one value per lane across the wave.
template <typename Key>
__device__ __forceinline__ Key wave_sort_desc(Key v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const Key y = __shfl_xor(v, j);
      const bool lower = (lane & j) == 0;
      const bool desc = (lane & k) == 0;  // this k-block sorts descending
      const bool take_max = (lower == desc);
      v = take_max ? (y > v ? y : v) : (y < v ? y : v);
    }
  }
  return v;
}

// Exact K-th largest of the eligible keys among a[0..n) (1 <= k <= number of
// eligible keys, n < 65536; keys equal to 0 are not eligible when skip_zero).
// Returns the key value T; *rem receives how many keys equal to T complete the
// top k (the keys greater than T are k - *rem).
//
// Most-significant-digit radix select with 4-bit digits.  Each thread counts
// its keys into 16 counters held in registers (two 16-bit counters per word),
// a reduce-scatter sums them over the wave and LDS over the workgroup, and the
// digit holding the k-th key fixes 4 more bits.  Leading bits common to all
// eligible keys are skipped; once the bucket holding the k-th key has at most
// 64 keys, one wave sorts it and reads the answer off directly.
template <typename Key>
__device__ Key select_kth_largest(const Key* a, int n, int k, bool skip_zero, SelShared& S, int* rem) {
  constexpr int kBits = (int)sizeof(Key) * 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  // ---- common prefix and count of all eligible keys
  Key lo = ~(Key)0, hi = 0;
  int cnt_el = 0;
  for (int i = tid; i < n; i += blockDim.x) {
    const Key x = a[i];
    if (skip_zero && x == 0) continue;
    lo = x < lo ? x : lo;
    hi = x > hi ? x : hi;
    cnt_el++;
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  cnt_el = wave_sum(cnt_el);
  if (lane == 0) {
    S.wmin[wave] = (uint64_t)lo;
    S.wmax[wave] = (uint64_t)hi;
    S.red[wave][0] = (uint32_t)cnt_el;
  }
  __syncthreads();
  {
    Key l = ~(Key)0, h = 0;
    int c = 0;
    for (int w = 0; w < nw; w++) {
      l = (Key)S.wmin[w] < l ? (Key)S.wmin[w] : l;
      h = (Key)S.wmax[w] > h ? (Key)S.wmax[w] : h;
      c += (int)S.red[w][0];
    }
    lo = l;
    hi = h;
    cnt_el = c;
  }
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
  int bucket = cnt_el;  // keys under the current prefix
  int shift = top;
  while (bucket > 64 && shift > 0) {
    shift -= 4;
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
    const uint32_t tot = wave_reduce8(c0, c1, c2, c3, c4, c5, c6, c7);
    if ((lane & 7) == 0) S.red[wave][lane >> 3] = tot;
    __syncthreads();
    if (wave == 0) {
      // lane j (< 16) owns digit j: its count, then the count of all larger digits
      uint32_t cnt = 0;
      if (lane < 16) {
        uint32_t s = 0;
        for (int w = 0; w < nw; w++) s += S.red[w][lane >> 1];
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
    bucket = S.ibc[2];
    prefix |= (Key)d << shift;
    mask |= (Key)15 << shift;
    __syncthreads();
  }
  if (shift == 0) {  // the prefix is the whole key
    *rem = k;
    return prefix;
  }
  // ---- small bucket: gather it and let one wave sort it
  if (tid == 0) S.ibc[3] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += blockDim.x) {
    const Key x = a[i];
    if ((skip_zero && x == 0) || (x & mask) != prefix) continue;
    S.small[atomicAdd(&S.ibc[3], 1)] = (uint64_t)x;
  }
  __syncthreads();
  if (wave == 0) {
    Key v = lane < bucket ? (Key)S.small[lane] : (Key)0;
    v = wave_sort_desc<Key>(v);
    const Key t = __shfl(v, k - 1);
    const uint64_t gt = __ballot(lane < bucket && v > t);
    if (lane == 0) {
      S.kbc[0] = (uint64_t)t;
      S.ibc[4] = k - __popcll(gt);
    }
  }
  __syncthreads();
  const Key t = (Key)S.kbc[0];
  *rem = S.ibc[4];
  __syncthreads();
  return t;
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

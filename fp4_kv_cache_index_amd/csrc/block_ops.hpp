// Workgroup-wide building blocks for the selection kernels: exclusive scan,
// radix select of the K-th largest key, bitonic sort.  All operate on LDS and
// must be called by every thread of the workgroup.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

// Exclusive prefix sum of one int per thread over the workgroup; `tmp` holds
// one int per wave (up to 16 waves).  Returns the exclusive prefix, writes the
// total to *total.
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

// K-th largest (1-based k <= count of eligible keys) of n keys in LDS, by
// most-significant-digit radix select over `bits` bits (8-bit digits).  Keys
// equal to 0 are ignored when skip_zero.  Returns the exact key value; *rem
// receives how many keys equal to it are needed to complete the top k.
template <typename Key>
__device__ Key radix_kth_largest(const Key* a, int n, int k, int bits, bool skip_zero, uint32_t* hist,
                                 int* tmp, int* bcast, int* rem) {
  Key prefix = 0, mask = 0;
  for (int shift = bits - 8; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
      const Key x = a[i];
      if ((x & mask) == prefix && !(skip_zero && x == 0)) atomicAdd(&hist[(uint32_t)(x >> shift) & 255u], 1u);
    }
    __syncthreads();
    // suffix counts: thread t looks at digit 255 - t
    const int t = threadIdx.x;
    const int v = t < 256 ? (int)hist[255 - t] : 0;
    int total;
    const int ex = block_scan_excl(v, tmp, &total);
    if (t < 256 && ex < k && ex + v >= k) {
      bcast[0] = 255 - t;
      bcast[1] = k - ex;
    }
    __syncthreads();
    const int d = bcast[0];
    k = bcast[1];
    prefix |= (Key)d << shift;
    mask |= (Key)255 << shift;
    __syncthreads();
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

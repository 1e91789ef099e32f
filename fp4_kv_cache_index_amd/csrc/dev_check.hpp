// Device-side precondition checks of the debug library.
//
// A debug build (CSA2_DEBUG defined) checks the caller's device data that the
// host cannot see: cache lengths against the capacity, Top-K entry ids and
// Reindex pool entries against the entries visible to their query, window
// lengths against the tokens being appended.  A kernel that finds one out of
// range sets that kind's bit in its translation unit's error word, on its
// device, and treats the item as absent (an id as -1, an append that would
// pass the capacity as not made).  take_*_dev_error read and clear the word;
// the C-ABI turns a nonzero word into CSA2_EDEVICE on the next call.
//
// A release build compiles every check out (kDebug is false, dev_flag does
// nothing) and its take_*_dev_error return 0 without touching the GPU.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"

namespace csa2 {

#ifdef CSA2_DEBUG
constexpr bool kDebug = true;
// one word per translation unit (each .hip file includes this once) and device
static __device__ uint32_t g_dev_error;
__device__ __forceinline__ void dev_flag(uint32_t bit) { atomicOr(&g_dev_error, bit); }
// Reads the word after the stream's earlier work, then clears it.
#define CSA2_DEV_ERROR_TAKER(fn)                                                                              \
  uint32_t fn(hipStream_t s) {                                                                                \
    uint32_t v = 0;                                                                                           \
    if (hipMemcpyFromSymbolAsync(&v, HIP_SYMBOL(g_dev_error), 4, 0, hipMemcpyDeviceToHost, s) != hipSuccess || \
        hipStreamSynchronize(s) != hipSuccess)                                                                \
      return kErrUnreadable;                                                                                  \
    if (v) {                                                                                                  \
      const uint32_t zero = 0;                                                                                \
      if (hipMemcpyToSymbolAsync(HIP_SYMBOL(g_dev_error), &zero, 4, 0, hipMemcpyHostToDevice, s) != hipSuccess || \
          hipStreamSynchronize(s) != hipSuccess)                                                              \
        return v | kErrUnreadable;                                                                            \
    }                                                                                                         \
    return v;                                                                                                 \
  }
#else
constexpr bool kDebug = false;
__device__ __forceinline__ void dev_flag(uint32_t) {}
#define CSA2_DEV_ERROR_TAKER(fn) \
  uint32_t fn(hipStream_t) { return 0u; }
#endif

}  // namespace csa2

// Streaming-read ceiling of the GPU: the rate a plain read kernel reaches over
// a given span of HBM, the practical upper bound for any kernel that streams
// those bytes once (the indexer scan).  Each lane reads 16 bytes per load with
// the non-temporal hint, four loads in flight, grid-stride over the span, and
// folds the words into one value that is stored only if it matches a sentinel
// (never in practice), so that the loads cannot be removed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa2_roofline.h"

namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) stream_read_kernel(const v4u* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const v4u a = __builtin_nontemporal_load(src + i);
    const v4u b = __builtin_nontemporal_load(src + i + stride);
    const v4u c = __builtin_nontemporal_load(src + i + 2 * stride);
    const v4u d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a[0] ^ b[1] ^ c[2] ^ d[3] ^ a[3] ^ b[0] ^ c[1] ^ d[2];
  }
  for (; i < n16; i += stride) {
    const v4u a = src[i];
    acc ^= a[0] ^ a[3];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

extern "C" int csa2roof_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks, void* stream) {
  if (!src || !sink || bytes % 16 != 0 || ((uintptr_t)src & 15) != 0 || blocks < 1) return -1;
  if (bytes == 0) return 0;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const v4u*)src, (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Quantising one cache entry with one wave (ai.info "Main Findings": E2M1
// codes, an E4M3 scale for every 16 channels, no global scale).  Shared by the
// append kernel and the Full scorer's fused append, so both write the same
// bytes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec.hpp"

namespace csa2 {

// Lane l holds channels 8l .. 8l+7 of the entry's fp32 latent in x and
// element l of its fp32 indexer key in k.  Writes row `row` of the cache: the
// 256-byte FP4 code row (one dword per lane; a 16-channel group spans the lane
// pair 2g, 2g+1), the 32 group scales E4M3(amax / 6), the 64 E4M3 indexer
// codes and the fp32 indexer scale amax / 448 (a zero row stores 0).  Every
// lane of the wave must call it.
__device__ __forceinline__ void quantize_store_entry(uint8_t* __restrict__ kv_codes, uint8_t* __restrict__ kv_scales,
                                                     uint8_t* __restrict__ ik_codes, float* __restrict__ ik_scales,
                                                     int64_t row, const float (&x)[8], float k, int lane) {
  // ---- group amax over the lane pair, E4M3 scale of amax / 6
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 8; c++) amax = fmaxf(amax, fabsf(x[c]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  const uint32_t sc = e4m3_encode(amax / 6.0f);
  const float s = e4m3_decode(sc);
  uint32_t packed = 0;
#pragma unroll
  for (int c = 0; c < 8; c++) {
    const uint32_t nib = (s == 0.0f) ? ((__float_as_uint(x[c]) >> 28) & 8u) : e2m1_encode(x[c] / s);
    packed |= nib << (4 * c);
  }
  reinterpret_cast<uint32_t*>(kv_codes + row * 256)[lane] = packed;
  if ((lane & 1) == 0) kv_scales[row * 32 + (lane >> 1)] = (uint8_t)sc;

  // ---- indexer K: lane l owns dim l; one fp32 scale per row
  float kmax = fabsf(k);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) kmax = fmaxf(kmax, __shfl_xor(kmax, o));
  const float sk = kmax / 448.0f;
  ik_codes[row * 64 + lane] = (uint8_t)(sk == 0.0f ? 0u : e4m3_encode(k / sk));
  if (lane == 0) ik_scales[row] = sk;
}

}  // namespace csa2

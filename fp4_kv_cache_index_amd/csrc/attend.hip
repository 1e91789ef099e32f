// Sparse attention of one CSA2 layer: its own 16-head query over the selected
// global entries (FP4 main KV, dequantised on the fly) merged with its own
// 128-token FP8 sliding window, one softmax over both, key = value (the report
// stores one 512-channel latent per entry; ai.info "Main Findings";
// technologiesdigest "CSA2": every layer keeps its own query and window KV).
//
// Key slots per query: 0..511 = the Top-512 list, 512..639 = window positions
// p-127..p.  A workgroup (4 waves) walks a range of slots in tiles of 32:
//   gather + dequantise: E2M1 code * E4M3 scale (and plain E4M3 for the window)
//     is exact in both bf16 and fp16, so the tile lands in LDS twice: bf16
//     [key][dim] for Q.K^T and fp16 [dim][key] for P.V;
//   S = Q K^T on v_mfma_f32_16x16x32_bf16 (16 heads = the 16 MFMA rows; wave w
//     covers dims 128w..128w+127 and the four partial S are summed in LDS);
//   online softmax in fp32 (running max and sum per head);
//   O += P V on v_mfma_f32_16x16x32_f16, wave w owning output dims 128w.. .
// With several splits per query the unnormalised partials (O, max, sum) go to
// the workspace and a merge kernel combines them by log-sum-exp weights.
#include <hip/hip_runtime.h>

#include "codec.hpp"
#include "kernels.hpp"

namespace csa2 {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kKbStride = 520;  // bf16 elements per key row (512 + pad)
constexpr int kKtStride = 40;   // fp16 elements per dim row (32 keys + pad)
constexpr int kPStride = 40;
constexpr int kTilesPerQuery = kAttnKeys / kAttnTile;  // 20

int attend_splits(int64_t bq) {
  int64_t s = (256 + bq - 1) / bq;
  if (s < 1) s = 1;
  if (s > 10) s = 10;
  const int tps = (int)((kTilesPerQuery + s - 1) / s);
  return (kTilesPerQuery + tps - 1) / tps;
}

static inline int tiles_per_split(int splits) { return (kTilesPerQuery + splits - 1) / splits; }

size_t attend_ws_bytes(int64_t bq) {
  const int s = attend_splits(bq);
  if (s == 1) return 0;
  return (size_t)s * bq * (16 * 512 * 4 + 16 * 2 * 4) + 256;
}

__device__ __forceinline__ int32_t attn_query_pos(const int32_t* q_pos, const int32_t* length, int32_t ratio, int b,
                                                  int q, int Q) {
  return q_pos ? q_pos[(int64_t)b * Q + q] : length[b] * ratio - Q + q;
}

__device__ __forceinline__ uint16_t f32_to_bf16_exact(float v) { return (uint16_t)(__float_as_uint(v) >> 16); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ void __launch_bounds__(kThreads)
    attend_kernel(const uint8_t* __restrict__ kv_codes, const uint8_t* __restrict__ kv_scales,
                  const int32_t* __restrict__ length, int32_t cap, int32_t ratio, const int32_t* __restrict__ topk,
                  const uint8_t* __restrict__ swa, int32_t S, const uint16_t* __restrict__ q,
                  const int32_t* __restrict__ q_pos, float sm_scale, int32_t Q, int tps,
                  uint16_t* __restrict__ out, float* __restrict__ lse, float* __restrict__ part_o,
                  float* __restrict__ part_ml, int64_t bq_total) {
  __shared__ __attribute__((aligned(16))) uint16_t s_kb[kAttnTile * kKbStride];
  __shared__ __attribute__((aligned(16))) _Float16 s_kt[512 * kKtStride];
  __shared__ float s_red[4][2][256];
  __shared__ float s_sfull[16][kAttnTile];
  __shared__ __attribute__((aligned(16))) _Float16 s_p[16 * kPStride];
  __shared__ float s_m[16], s_l[16], s_alpha[16];
  __shared__ int s_valid[kAttnTile];
  __shared__ int32_t s_ent[kTilesPerQuery * kAttnTile];

  const int split = blockIdx.x;
  const int64_t bq = blockIdx.y;
  const int b = (int)(bq / Q), qi = (int)(bq % Q);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t p = attn_query_pos(q_pos, length, ratio, b, qi, Q);

  // Q operand of Q.K^T: lane l holds head l%16, dims 128*wave + 32*kk + 8*(l/16) .. +7
  v8bf qa[4];
  {
    const uint16_t* qrow = q + (bq * 16 + (lane & 15)) * 512 + 128 * wave + 8 * (lane >> 4);
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      const uint4 x = *reinterpret_cast<const uint4*>(qrow + 32 * kk);
      qa[kk] = __builtin_bit_cast(v8bf, x);
    }
  }
  v4f acc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ct++) acc[ct] = (v4f){0.f, 0.f, 0.f, 0.f};
  if (tid < 16) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.0f;
  }

  const int t_begin = split * tps;
  const int t_end = min(kTilesPerQuery, t_begin + tps);
  // this split's Top-K entries (main-KV slots only), staged once
  for (int i = tid; i < tps * kAttnTile; i += kThreads) {
    const int slot = t_begin * kAttnTile + i;
    s_ent[i] = (slot < 512 && cap > 0) ? topk[bq * 512 + slot] : -1;
  }
  __syncthreads();

  // thread -> (key j of the tile, 64-channel part)
  const int j = tid & 31, part = tid >> 5;
  // raw bytes of one tile for this thread: main rows use w[0..1] (32 code
  // bytes) and sc (4 scale bytes); window rows use w[0..3] (64 E4M3 bytes).
  // Loads are unconditional from a clamped address (masked later), so that a
  // tile's loads and the next tile's prefetch all stay in flight together.
  auto load_tile = [&](int tile, uint4* w, uint32_t& sc, bool& valid) {
    const int slot = tile * kAttnTile + j;
    if (tile * kAttnTile < 512) {  // uniform per tile: 512 is a multiple of the tile
      const int32_t e = s_ent[(tile - t_begin) * kAttnTile + j];
      valid = e >= 0;
      if (cap > 0) {  // uniform; an empty cache has no row to stand in
        const int64_t row = (int64_t)b * cap + (valid ? e : 0);
        const uint4* cp = reinterpret_cast<const uint4*>(kv_codes + row * 256 + 32 * part);
        w[0] = cp[0];
        w[1] = cp[1];
        sc = *reinterpret_cast<const uint32_t*>(kv_scales + row * 32 + 4 * part);
      }
    } else {
      const int64_t pos = (int64_t)p - 127 + (slot - 512);
      valid = pos >= 0;
      const uint4* sp = reinterpret_cast<const uint4*>(swa + ((int64_t)b * S + (valid ? pos % S : 0)) * 512 + 64 * part);
      w[0] = sp[0];
      w[1] = sp[1];
      w[2] = sp[2];
      w[3] = sp[3];
    }
  };
  uint4 wc[4] = {}, wn[4] = {};
  uint32_t scc = 0, scn = 0;
  bool vc = false, vn = false;
  load_tile(t_begin, wc, scc, vc);
  for (int tile = t_begin; tile < t_end; tile++) {
    load_tile(min(tile + 1, t_end - 1), wn, scn, vn);  // prefetch (the last tile reloads itself)
    // ---------------- dequantise this tile's 32 keys into LDS
    {
      float v[64];
      if (tile * kAttnTile < 512) {
        const uint32_t cw[8] = {wc[0].x, wc[0].y, wc[0].z, wc[0].w, wc[1].x, wc[1].y, wc[1].z, wc[1].w};
#pragma unroll
        for (int g = 0; g < 4; g++) {
          const float s = e4m3_decode((scc >> (8 * g)) & 0xFFu);
#pragma unroll
          for (int w = 0; w < 2; w++) {
            const uint32_t word = cw[2 * g + w];
#pragma unroll
            for (int n = 0; n < 8; n++) v[16 * g + 8 * w + n] = e2m1_decode((word >> (4 * n)) & 15u) * s;
          }
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; w++) {
          const uint32_t xw[4] = {wc[w].x, wc[w].y, wc[w].z, wc[w].w};
#pragma unroll
          for (int k = 0; k < 4; k++)
#pragma unroll
            for (int n = 0; n < 4; n++) v[16 * w + 4 * k + n] = e4m3_decode((xw[k] >> (8 * n)) & 0xFFu);
        }
      }
      if (!vc) {
#pragma unroll
        for (int c = 0; c < 64; c++) v[c] = 0.0f;
      }
      // bf16 [key][dim]
      uint32_t* kb = reinterpret_cast<uint32_t*>(s_kb + j * kKbStride + 64 * part);
#pragma unroll
      for (int c = 0; c < 32; c++)
        kb[c] = (uint32_t)f32_to_bf16_exact(v[2 * c]) | ((uint32_t)f32_to_bf16_exact(v[2 * c + 1]) << 16);
      // fp16 [dim][key]
#pragma unroll
      for (int c = 0; c < 64; c++) s_kt[(64 * part + c) * kKtStride + j] = (_Float16)v[c];
      if (part == 0) s_valid[j] = vc;
    }
    __syncthreads();

    // ---------------- partial S over this wave's 128 dims
#pragma unroll
    for (int th = 0; th < 2; th++) {
      v4f sacc = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = s_kb + (16 * th + (lane & 15)) * kKbStride + 128 * wave + 8 * (lane >> 4);
#pragma unroll
      for (int kk = 0; kk < 4; kk++) {
        const uint4 x = *reinterpret_cast<const uint4*>(krow + 32 * kk);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], __builtin_bit_cast(v8bf, x), sacc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; i++) s_red[wave][th][i * 64 + lane] = sacc[i];
    }
    __syncthreads();
    // reduce the four waves: element (th, i, lane) is head 4*(lane/16)+i, key 16*th + lane%16
    for (int x = tid; x < 512; x += kThreads) {
      const int th = x >> 8, i = (x >> 6) & 3, l = x & 63;
      const float sv = s_red[0][th][i * 64 + l] + s_red[1][th][i * 64 + l] + s_red[2][th][i * 64 + l] +
                       s_red[3][th][i * 64 + l];
      const int head = 4 * (l >> 4) + i, key = 16 * th + (l & 15);
      s_sfull[head][key] = s_valid[key] ? sv * sm_scale : -INFINITY;
    }
    __syncthreads();
    // ---------------- online softmax: 16 threads per head, 2 keys each
    {
      const int h = tid >> 4, k0 = 2 * (tid & 15);
      const float a0 = s_sfull[h][k0], a1 = s_sfull[h][k0 + 1];
      float mt = fmaxf(a0, a1);
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) mt = fmaxf(mt, __shfl_xor(mt, o, 16));
      const float m_old = s_m[h];
      const float m_new = fmaxf(m_old, mt);
      const float alpha = (m_new == -INFINITY) ? 1.0f : __expf(m_old - m_new);
      const float p0 = (a0 == -INFINITY) ? 0.0f : __expf(a0 - m_new);
      const float p1 = (a1 == -INFINITY) ? 0.0f : __expf(a1 - m_new);
      float ps = p0 + p1;
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) ps += __shfl_xor(ps, o, 16);
      s_p[h * kPStride + k0] = (_Float16)p0;
      s_p[h * kPStride + k0 + 1] = (_Float16)p1;
      __syncthreads();  // every thread has read s_m before it changes
      if ((tid & 15) == 0) {
        s_m[h] = m_new;
        s_l[h] = alpha * s_l[h] + ps;
        s_alpha[h] = alpha;
      }
    }
    __syncthreads();
    // ---------------- O = alpha * O + P V
    {
      const uint4 pa = *reinterpret_cast<const uint4*>(s_p + (lane & 15) * kPStride + 8 * (lane >> 4));
      const v8h pv = __builtin_bit_cast(v8h, pa);
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; i++) al[i] = s_alpha[4 * (lane >> 4) + i];
#pragma unroll
      for (int ct = 0; ct < 8; ct++) {
#pragma unroll
        for (int i = 0; i < 4; i++) acc[ct][i] *= al[i];
        const int dim = 128 * wave + 16 * ct + (lane & 15);
        const uint4 kx = *reinterpret_cast<const uint4*>(s_kt + dim * kKtStride + 8 * (lane >> 4));
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pv, __builtin_bit_cast(v8h, kx), acc[ct], 0, 0, 0);
      }
    }
    __syncthreads();
    wc[0] = wn[0];
    wc[1] = wn[1];
    wc[2] = wn[2];
    wc[3] = wn[3];
    scc = scn;
    vc = vn;
  }

  // ---------------- epilogue: rows 4*(lane/16)+i are heads, column lane%16 a dim
  if (part_o == nullptr) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int h = 4 * (lane >> 4) + i;
      const float l = s_l[h];
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
      for (int ct = 0; ct < 8; ct++) {
        const int dim = 128 * wave + 16 * ct + (lane & 15);
        out[(bq * 16 + h) * 512 + dim] = f32_to_bf16_rne(acc[ct][i] * inv);
      }
    }
    if (lse && tid < 16) lse[bq * 16 + tid] = s_l[tid] > 0.0f ? s_m[tid] + __logf(s_l[tid]) : -INFINITY;
  } else {
    float* po = part_o + ((int64_t)split * bq_total + bq) * 16 * 512;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int h = 4 * (lane >> 4) + i;
#pragma unroll
      for (int ct = 0; ct < 8; ct++) po[h * 512 + 128 * wave + 16 * ct + (lane & 15)] = acc[ct][i];
    }
    if (tid < 16) {
      float* pm = part_ml + ((int64_t)split * bq_total + bq) * 32;
      pm[2 * tid] = s_m[tid];
      pm[2 * tid + 1] = s_l[tid];
    }
  }
}

// One workgroup per (query, head): combine the splits' unnormalised partials by
// their log-sum-exp weights; each thread owns two of the 512 output channels.
__global__ void __launch_bounds__(kThreads)
    attend_merge_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml, int splits,
                        int64_t bq_total, uint16_t* __restrict__ out, float* __restrict__ lse) {
  __shared__ float s_m[16], s_l[16];
  const int64_t bq = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  if (tid < splits) {
    const float* pm = part_ml + ((int64_t)tid * bq_total + bq) * 32 + 2 * h;
    s_m[tid] = pm[0];
    s_l[tid] = pm[1];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int s = 0; s < splits; s++) M = fmaxf(M, s_m[s]);
  float L = 0.0f;
  float w[10];
#pragma unroll
  for (int s = 0; s < 10; s++) {
    w[s] = (s < splits && s_m[s] != -INFINITY) ? __expf(s_m[s] - M) : 0.0f;
    L += s < splits ? w[s] * s_l[s] : 0.0f;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
  for (int s = 0; s < 10; s++) {
    if (s < splits) {
      const float2 v = *reinterpret_cast<const float2*>(part_o + (((int64_t)s * bq_total + bq) * 16 + h) * 512 + 2 * tid);
      o0 += w[s] * v.x;
      o1 += w[s] * v.y;
    }
  }
  const uint32_t packed = (uint32_t)f32_to_bf16_rne(o0 * inv) | ((uint32_t)f32_to_bf16_rne(o1 * inv) << 16);
  reinterpret_cast<uint32_t*>(out + (bq * 16 + h) * 512)[tid] = packed;
  if (lse && tid == 0) lse[bq * 16 + h] = L > 0.0f ? M + __logf(L) : -INFINITY;
}

hipError_t launch_attend(const LaunchCache& c, const int32_t* topk, const uint8_t* swa, int32_t S,
                         const uint16_t* q, const int32_t* q_pos, float sm_scale, uint16_t* out, float* lse,
                         int32_t Q, void* ws, hipStream_t stream) {
  const int64_t bq = (int64_t)c.batch * Q;
  if (bq == 0) return hipSuccess;
  const int splits = attend_splits(bq);
  const int tps = tiles_per_split(splits);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (splits > 1) {
    uint8_t* base = (uint8_t*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
    part_o = (float*)base;
    part_ml = part_o + (int64_t)splits * bq * 16 * 512;
  }
  hipLaunchKernelGGL(attend_kernel, dim3(splits, (unsigned)bq), dim3(kThreads), 0, stream, c.kv_codes, c.kv_scales,
                     c.length, c.capacity, c.ratio, topk, swa, S, q, q_pos, sm_scale, Q, tps, out, lse, part_o,
                     part_ml, bq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  hipLaunchKernelGGL(attend_merge_kernel, dim3((unsigned)bq, 16), dim3(kThreads), 0, stream, part_o, part_ml, splits,
                     bq, out, lse);
  return hipGetLastError();
}

}  // namespace csa2

// Sparse attention of one CSA2 layer: its own 16-head query over the selected
// global entries (FP4 main KV, dequantised on the fly) merged with its own
// 128-token FP8 sliding window, one softmax over both, key = value (the report
// stores one 512-channel latent per entry; ai.info "Main Findings";
// technologiesdigest "CSA2": every layer keeps its own query and window KV).
// Optionally the same launch first appends the layer's new window tokens.
//
// Key slots per query: 0..511 = the Top-512 list, 512..639 = window positions
// p-127..p.  A workgroup (4 waves) walks a range of slots in tiles of 32:
//   gather: thread (kg, grp) owns keys 4kg..4kg+3 of the tile and channels
//     16grp..16grp+15, i.e. one E4M3 scale group per key (8 code bytes + 1
//     scale byte, or 16 window bytes);
//   dequantise: v_cvt_scalef32_pk_f16_fp4 with scale 1.0 gives the E2M1 values
//     exactly and one v_pk_mul_f16 by the group scale gives x = code * scale,
//     exact in fp16 (at most 6 significant bits, |x| in [2^-10, 2688]); window
//     bytes widen exactly with v_cvt_scalef32_pk_f16_fp8.  The tile lands in
//     LDS once, as fp16 [key][dim];
//   S = Q K^T on v_mfma_f32_16x16x32_f16: the bf16 query is scaled per head by
//     a power of two that puts its largest element in [2^14, 2^15), which makes
//     the fp16 copy exact for every element within 2^-28 of the head's largest,
//     and the scores are scaled back exactly (16 heads = the 16 MFMA rows; wave
//     w covers dims 128w..128w+127 and the four partial S are summed in LDS);
//   online softmax in fp32 (running max and sum per head);
//   O += P V on v_mfma_f32_16x16x32_f16, wave w owning output dims 128w..; the
//     V operand (8 keys of one dim per lane) comes straight from the [key][dim]
//     tile through the LDS transpose read ds_read_b64_tr_b16.
// With several splits per query the unnormalised partials (O, max, sum) go to
// the workspace and a second kernel merges them by log-sum-exp weights, one
// workgroup per (query, head).  (Merging in the last workgroup of each query
// needs a device-scope release per workgroup, an L2 write-back that costs more
// on gfx950 than the second launch.)
#include <hip/hip_runtime.h>

#include "block_ops.hpp"
#include "codec.hpp"
#include "dev_check.hpp"
#include "kernels.hpp"

namespace csa2 {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

// LDS transpose read: in each 16-lane group, lane 4j+q names 4 consecutive fp16
// of row j; lane i receives element i%4 of lanes i/4, i/4+4, i/4+8, i/4+12,
// i.e. column i of the 4-row block.
typedef short v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4h lds_read_tr16(const _Float16* p) {
  return __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p)));
}

constexpr int kThreads = 256;
constexpr int kKStride = 528;  // fp16 per key row of the [key][dim] tile (512 + pad)
constexpr int kPStride = 40;
constexpr int kRedStride = 80;  // 64 lanes + pad: the four row groups start 16 banks apart
constexpr int kTilesPerQuery = kAttnKeys / kAttnTile;  // 20
constexpr int kMaxSplits = 10;
constexpr int kFusedAppendMax = 8;  // new window tokens per sequence appended inside the attention launch

// Splits per query, at most kMaxSplits, rounded so every split holds as many
// tiles.  At most one workgroup per compute unit while that still gives four
// or more splits: workgroups sharing a compute unit mostly queue behind each
// other (measured: 32 queries run best as 7 splits, not 10).  Fewer queries
// than that get about two workgroups per compute unit instead (96 queries: 5
// splits beat 2, 3 and 10).
int attend_splits(int64_t bq) {
  int64_t s = 256 / bq;
  if (s < 4) s = (512 + bq - 1) / bq;
  if (s < 1) s = 1;
  if (s > kMaxSplits) s = kMaxSplits;
  const int tps = (int)((kTilesPerQuery + s - 1) / s);
  return (kTilesPerQuery + tps - 1) / tps;
}

static inline int tiles_per_split(int splits) { return (kTilesPerQuery + splits - 1) / splits; }

// [partial O, normalised by its own sum: splits x bq x 16 x 512 fp16]
// [partial (max, sum): splits x bq x 16 x 2 f32]
size_t attend_ws_bytes(int64_t bq) {
  const int s = attend_splits(bq);
  if (s == 1) return 0;
  return 256 + (size_t)s * bq * (16 * 512 * 2 + 16 * 2 * 4);
}

struct AttnArgs {
  const uint8_t* kv_codes;
  const uint8_t* kv_scales;
  const int32_t* length;
  int32_t cap, ratio;
  const int32_t* topk;
  uint8_t* swa;
  int32_t S;
  const float* swa_x;      // [B][swa_T][512] new window tokens, or null
  const int32_t* swa_len;  // [B] tokens after the append
  int32_t swa_T;
  const uint16_t* q;
  const int32_t* q_pos;
  float sm_scale;
  int32_t Q;
  int32_t tps, splits;
  uint16_t* out;
  float* lse;
  _Float16* part_o;
  float* part_ml;
  int64_t bq_total;
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t h2_bits(v2h h) { return __builtin_bit_cast(uint32_t, h); }

// A raw buffer of `bytes` bytes at p: a load past the end returns zeros without
// a memory access, so a load that may not be wanted needs no branch around it
// (the compiler waits for a load under a branch before the branch ends).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// 8 E2M1 codes (low nibble first) times a group scale, as four fp16x2 words
__device__ __forceinline__ void fp4_group(uint32_t w, v2h s2, uint32_t* o) {
  o[0] = h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2);
  o[1] = h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2);
  o[2] = h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2);
  o[3] = h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2);
}

template <bool kRefill>
__global__ void __launch_bounds__(kThreads) attend_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 s_k[kAttnTile * kKStride];
  __shared__ float s_red[4][2][4][kRedStride];  // [wave][key block][row group i][lane]
  __shared__ __attribute__((aligned(16))) _Float16 s_p[16 * kPStride];
  __shared__ float s_m[16], s_l[16], s_alpha[16];
  __shared__ float s_qmax[4][16];
  __shared__ float s_qfac[16];
  __shared__ int s_valid[kAttnTile];
  __shared__ __attribute__((aligned(16))) uint8_t s_new[kFusedAppendMax * 512];  // new window tokens, E4M3
  __shared__ __attribute__((aligned(16))) int32_t s_ids[512];                     // the query's Top-K row

  const int64_t wr = xcd_rank(blockIdx.x, (int64_t)a.splits * a.bq_total);
  const int split = (int)(wr % a.splits);
  const int64_t bq = wr / a.splits;
  const int Q = a.Q;
  const int b = (int)(bq / Q), qi = (int)(bq % Q);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t p = a.q_pos ? a.q_pos[bq] : a.length[b] * a.ratio - Q + qi;
  // new window tokens are positions new_lo .. new_hi-1
  const int32_t new_hi = a.swa_x ? a.swa_len[b] : 0;
  const int32_t new_lo = a.swa_x ? new_hi - a.swa_T : 0;
  // debug builds: the entries this query may list; a listed id at or past them
  // is flagged and skipped
  int32_t n_vis_dbg = 0;
  if (kDebug) {
    const int32_t len = a.length[b];
    if (tid == 0 && split == 0 && (len < 0 || len > a.cap)) dev_flag(kErrLength);
    if (tid == 0 && split == 0 && new_lo < 0) dev_flag(kErrSeqLen);
    const int64_t by_pos = p < 0 ? 0 : ((int64_t)p + 1) / a.ratio;
    n_vis_dbg = (int32_t)min((int64_t)min(len, a.cap), by_pos);
  }

  const int t_begin = split * a.tps;
  const int t_end = min(kTilesPerQuery, t_begin + a.tps);
  const int kg = tid & 7, grp = tid >> 3;  // keys 4kg..4kg+3, channels 16grp..16grp+15
  const int32_t* tk = a.topk + bq * 512 + 4 * kg;

  // the tile's Top-K ids for this thread's four keys, as loaded (from a clamped
  // tile): load_tile decides whether they count, since any arithmetic on them
  // here would wait for the load
  auto load_idx = [&](int tile) -> int4 {
    return *reinterpret_cast<const int4*>(tk + min(tile, 512 / kAttnTile - 1) * kAttnTile);
  };
  // Raw bytes of a tile for this thread, left as loaded until the tile is
  // dequantised (arithmetic on them here would wait for the loads): w[i] is the
  // aligned 16 bytes holding a main row's 16 codes of this thread (half grp & 1)
  // or a window row's 16 bytes, sc[i] a main row's scale byte.  Both tile kinds
  // issue the same loads, only their addresses differ, so no branch ends with a
  // wait: a missing entry reads row 0 (masked through vmask), and a load a tile
  // does not need (the scale of a window row, any row of an empty cache, a tile past
  // the split's) reads
  // this query's Top-K row instead.
  const uint8_t* stand_in = reinterpret_cast<const uint8_t*>(a.topk + bq * 512);
  auto load_tile = [&](int tile, int4 e4, uint4* w, uint32_t* sc, uint32_t& vmask) {
    const bool mine = tile < t_end;                 // uniform: tiles past the split hold nothing
    const bool main_tile = tile * kAttnTile < 512;  // uniform: 512 is a multiple of the tile
    const bool rows = main_tile && a.cap > 0 && mine;  // uniform
    int32_t es[4] = {mine ? e4.x : -1, mine ? e4.y : -1, mine ? e4.z : -1, mine ? e4.w : -1};
    if (kDebug && main_tile && mine)
#pragma unroll
      for (int i = 0; i < 4; i++)
        if (es[i] < -1 || es[i] >= n_vis_dbg) {
          dev_flag(kErrEntryId);
          es[i] = -1;
        }
    vmask = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int32_t pos = p - 127 + (tile * kAttnTile + 4 * kg + i - 512);  // window tiles
      vmask |= (uint32_t)(main_tile ? es[i] >= 0 : pos >= 0) << i;
      const int64_t row = (int64_t)b * a.cap + (es[i] >= 0 ? es[i] : 0);
      const int32_t slot = main_tile ? 0 : (pos >= 0 ? pos : 0) % a.S;
      const uint8_t* src = rows                ? a.kv_codes + row * 256 + 16 * (grp >> 1)
                           : main_tile || !mine ? stand_in
                                                : a.swa + ((int64_t)b * a.S + slot) * 512 + 16 * grp;
      w[i] = *reinterpret_cast<const uint4*>(src);
      sc[i] = *(rows ? a.kv_scales + row * 32 + grp : stand_in);
    }
  };

  uint4 wc[4] = {}, wn[4] = {};
  uint32_t sc_c[4] = {}, sc_n[4] = {};
  uint32_t vc = 0, vn = 0;
  int4 ec = load_idx(t_begin);
  int4 en = load_idx(t_begin + 1);
  // the whole Top-K row, for the later tiles' ids (kept in LDS, so that the
  // tile loop reads no ids from global memory)
  const int2 idv = *reinterpret_cast<const int2*>(a.topk + bq * 512 + 2 * tid);

  // ---------------- new window tokens (fused append): the workgroups whose
  // tiles reach the window load all of the sequence's new tokens (at most
  // kFusedAppendMax), two channels per thread; they are encoded into s_new
  // once the query is in, and these workgroups also write them to the ring
  const int first_win = 512 / (a.tps * kAttnTile);  // first split holding window tiles
  const bool has_win = t_end * kAttnTile > 512;
  const bool stage = a.swa_x != nullptr && has_win;
  float2 xv[kFusedAppendMax];
  {
    const __amdgpu_buffer_rsrc_t xr =
        make_rsrc(a.swa_x + (stage ? (int64_t)b * a.swa_T * 512 : 0), stage ? (uint32_t)a.swa_T * 2048u : 0u);
#pragma unroll
    for (int j = 0; j < kFusedAppendMax; j++)
      xv[j] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(xr, (uint32_t)(j * 2048 + 8 * tid), 0, 0));
  }

  // ---------------- query: lane holds head lane%16, dims 128*wave + 32*kk + 8*(lane/16) .. +7
  v8h qa[4];
  {
    const uint16_t* qrow = a.q + (bq * 16 + (lane & 15)) * 512 + 128 * wave + 8 * (lane >> 4);
    uint4 qraw[4];
#pragma unroll
    for (int kk = 0; kk < 4; kk++) qraw[kk] = *reinterpret_cast<const uint4*>(qrow + 32 * kk);
    // the first two tiles' rows load while the query is scaled
    load_tile(t_begin, ec, wc, sc_c, vc);
    load_tile(t_begin + 1, en, wn, sc_n, vn);  // past t_end: harmless loads, never used
    float qf[4][8];
    float amax = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      const uint32_t xw[4] = {qraw[kk].x, qraw[kk].y, qraw[kk].z, qraw[kk].w};
#pragma unroll
      for (int n = 0; n < 4; n++) {
        qf[kk][2 * n] = __uint_as_float(xw[n] << 16);
        qf[kk][2 * n + 1] = __uint_as_float(xw[n] & 0xFFFF0000u);
        amax = fmaxf(amax, fmaxf(fabsf(qf[kk][2 * n]), fabsf(qf[kk][2 * n + 1])));
      }
    }
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    if (lane < 16) s_qmax[wave][lane] = amax;
    *reinterpret_cast<int2*>(s_ids + 2 * tid) = idv;
    if (stage) {
      // new token j: into s_new, and into the ring by the (query, window split)
      // of rank j mod (Q * window splits)
      const int n_w = Q * (a.splits - first_win), rank = qi * (a.splits - first_win) + (split - first_win);
#pragma unroll
      for (int j = 0; j < kFusedAppendMax; j++) {
        if (j < a.swa_T) {
          const uint16_t c = (uint16_t)(e4m3_encode(xv[j].x) | (e4m3_encode(xv[j].y) << 8));
          reinterpret_cast<uint16_t*>(s_new + j * 512)[tid] = c;
          if (j % n_w == rank && new_lo + j >= 0)  // a window shorter than the append has no slot for it
            reinterpret_cast<uint16_t*>(a.swa + ((int64_t)b * a.S + (new_lo + j) % a.S) * 512)[tid] = c;
        }
      }
    }
    lds_barrier();
    const int h = lane & 15;
    const float hmax = fmaxf(fmaxf(s_qmax[0][h], s_qmax[1][h]), fmaxf(s_qmax[2][h], s_qmax[3][h]));
    int ex;
    frexpf(hmax, &ex);  // hmax = f * 2^ex, f in [0.5, 1); ex = 0 for a zero head
    const int sh = min(127, max(-126, 15 - ex));
    const float up = ldexpf(1.0f, sh);
    if (tid < 16) s_qfac[tid] = ldexpf(a.sm_scale, -sh);
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
#pragma unroll
      for (int n = 0; n < 8; n++) qa[kk][n] = (_Float16)(qf[kk][n] * up);
    }
  }
  v4f acc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ct++) acc[ct] = (v4f){0.f, 0.f, 0.f, 0.f};
  // online softmax state: thread tid serves head tid/16 (its 16 threads are one
  // DPP row and all hold the head's running max and sum)
  const int sm_h = tid >> 4;
  float m_run = -INFINITY, l_run = 0.0f;
  lds_barrier();  // s_qfac is written
  const float qfac = s_qfac[sm_h];

  // One tile: dequantise the rows held in (w, sc, vm) into LDS, refill those
  // registers with the tile two ahead (kRefill: so a tile's rows are in flight
  // while the two before it are processed; past the split they read a
  // stand-in), then S, the online softmax and O += PV.  Tiles alternate between
  // two register sets, and no load is under a branch.  Splits of at most two
  // tiles load both at entry and need no refill.
  auto tile_step = [&](int tile, uint4(&w)[4], uint32_t(&sc)[4], uint32_t& vm) {
    // ---------------- dequantise this tile's keys into LDS (fp16 [key][dim])
    {
      uint32_t hv[4][8];  // key i: channel pairs (2m, 2m+1) of the group, as fp16x2
      if (tile * kAttnTile < 512) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const uint32_t sb = ((vm >> i) & 1u) ? (sc[i] & 0xFFu) : 0u;
          const v2h s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb * 0x0101u, 1.0f, false);
          // this thread's half of the 16 bytes, by mask (a select here is
          // compiled as an index into the row, which moves the rows to scratch)
          const uint32_t odd = 0u - (uint32_t)(grp & 1);
          fp4_group((w[i].x & ~odd) | (w[i].z & odd), s2, hv[i]);
          fp4_group((w[i].y & ~odd) | (w[i].w & odd), s2, hv[i] + 4);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const bool valid = (vm >> i) & 1u;
          const int32_t pos = p - 127 + (tile * kAttnTile + 4 * kg + i - 512);
          uint4 raw = w[i];
          if (pos >= new_lo && pos < new_hi) raw = *reinterpret_cast<const uint4*>(s_new + (pos - new_lo) * 512 + 16 * grp);
          const uint32_t xw[4] = {valid ? raw.x : 0u, valid ? raw.y : 0u, valid ? raw.z : 0u, valid ? raw.w : 0u};
#pragma unroll
          for (int k = 0; k < 4; k++) {
            hv[i][2 * k] = h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(xw[k], 1.0f, false));
            hv[i][2 * k + 1] = h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(xw[k], 1.0f, true));
          }
        }
      }
      // [key][dim]: key 4kg+i, channels 16grp .. +15
#pragma unroll
      for (int i = 0; i < 4; i++) {
        uint4* dst = reinterpret_cast<uint4*>(s_k + (4 * kg + i) * kKStride + 16 * grp);
        dst[0] = make_uint4(hv[i][0], hv[i][1], hv[i][2], hv[i][3]);
        dst[1] = make_uint4(hv[i][4], hv[i][5], hv[i][6], hv[i][7]);
      }
    }
    if (grp == 0) {
#pragma unroll
      for (int i = 0; i < 4; i++) s_valid[4 * kg + i] = (vm >> i) & 1u;
    }
    if constexpr (kRefill) {
      const int4 e = *reinterpret_cast<const int4*>(s_ids + min(tile + 2, 512 / kAttnTile - 1) * kAttnTile + 4 * kg);
      load_tile(tile + 2, e, w, sc, vm);
    }
    lds_barrier();

    // ---------------- partial S over this wave's 128 dims
#pragma unroll
    for (int th = 0; th < 2; th++) {
      v4f sacc = {0.f, 0.f, 0.f, 0.f};
      const _Float16* krow = s_k + (16 * th + (lane & 15)) * kKStride + 128 * wave + 8 * (lane >> 4);
#pragma unroll
      for (int kk = 0; kk < 4; kk++) {
        const uint4 x = *reinterpret_cast<const uint4*>(krow + 32 * kk);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[kk], __builtin_bit_cast(v8h, x), sacc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; i++) s_red[wave][th][i][lane] = sacc[i];
    }
    lds_barrier();
    // ---------------- scores (the four waves' partial sums) and online softmax:
    // thread (head h, keys 2j, 2j+1); partial element (th, i, lane) is head
    // 4*(lane/16)+i, key 16*th + lane%16
    {
      const int h = sm_h, k0 = 2 * (tid & 15);
      const int th = k0 >> 4, l = 16 * (h >> 2) + (k0 & 15), i = h & 3;
      const float s0 = s_red[0][th][i][l] + s_red[1][th][i][l] + s_red[2][th][i][l] + s_red[3][th][i][l];
      const float s1 = s_red[0][th][i][l + 1] + s_red[1][th][i][l + 1] + s_red[2][th][i][l + 1] + s_red[3][th][i][l + 1];
      // the head's factor undoes its query scale exactly and applies sm_scale
      const float a0 = s_valid[k0] ? s0 * qfac : -INFINITY;
      const float a1 = s_valid[k0 + 1] ? s1 * qfac : -INFINITY;
      const float mt = wave_row_reduce(fmaxf(a0, a1), [](float x, float y) { return fmaxf(x, y); });
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_new == -INFINITY) ? 1.0f : __expf(m_run - m_new);
      const float p0 = (a0 == -INFINITY) ? 0.0f : __expf(a0 - m_new);
      const float p1 = (a1 == -INFINITY) ? 0.0f : __expf(a1 - m_new);
      const float ps = wave_row_reduce(p0 + p1, [](float x, float y) { return x + y; });
      s_p[h * kPStride + k0] = (_Float16)p0;
      s_p[h * kPStride + k0 + 1] = (_Float16)p1;
      m_run = m_new;
      l_run = alpha * l_run + ps;
      if ((tid & 15) == 0) s_alpha[h] = alpha;
    }
    lds_barrier();
    // ---------------- O = alpha * O + P V
    {
      const uint4 pa = *reinterpret_cast<const uint4*>(s_p + (lane & 15) * kPStride + 8 * (lane >> 4));
      const v8h pv = __builtin_bit_cast(v8h, pa);
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; i++) al[i] = s_alpha[4 * (lane >> 4) + i];
      // V operand of lane (group G = lane/16, column i = lane%16): keys 8G..8G+7 of
      // dim 128*wave + 16*ct + i; lane 4j+q of the group names row 8G+j (then
      // 8G+4+j), dims 4q..4q+3 of the block
      const _Float16* vsrc =
          s_k + (8 * (lane >> 4) + ((lane & 15) >> 2)) * kKStride + 128 * wave + 4 * (lane & 3);
#pragma unroll
      for (int ct = 0; ct < 8; ct++) {
#pragma unroll
        for (int i = 0; i < 4; i++) acc[ct][i] *= al[i];
        const v4h lo = lds_read_tr16(vsrc + 16 * ct);
        const v4h hi = lds_read_tr16(vsrc + 4 * kKStride + 16 * ct);
        const v8h vb = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pv, vb, acc[ct], 0, 0, 0);
      }
    }
    lds_barrier();
  };
  int tile = t_begin;
  for (; tile + 1 < t_end; tile += 2) {
    tile_step(tile, wc, sc_c, vc);
    tile_step(tile + 1, wn, sc_n, vn);
  }
  if (tile < t_end) tile_step(tile, wc, sc_c, vc);

  // ---------------- epilogue: rows 4*(lane/16)+i are heads, column lane%16 a dim
  if ((tid & 15) == 0) {
    s_m[sm_h] = m_run;
    s_l[sm_h] = l_run;
  }
  lds_barrier();
  if (a.splits == 1) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int h = 4 * (lane >> 4) + i;
      const float l = s_l[h];
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
      for (int ct = 0; ct < 8; ct++) {
        const int dim = 128 * wave + 16 * ct + (lane & 15);
        a.out[(bq * 16 + h) * 512 + dim] = f32_to_bf16_rne(acc[ct][i] * inv);
      }
    }
    if (a.lse && tid < 16) a.lse[bq * 16 + tid] = s_l[tid] > 0.0f ? s_m[tid] + __logf(s_l[tid]) : -INFINITY;
    return;
  }
  {
    // the split's output normalised by its own sum: |value| <= the largest key
    // value (2688), so fp16 holds it to 2^-12 relative
    _Float16* po = a.part_o + ((int64_t)split * a.bq_total + bq) * 16 * 512;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int h = 4 * (lane >> 4) + i;
      const float l = s_l[h];
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
      for (int ct = 0; ct < 8; ct++) po[h * 512 + 128 * wave + 16 * ct + (lane & 15)] = (_Float16)(acc[ct][i] * inv);
    }
    if (tid < 16) {
      float* pm = a.part_ml + ((int64_t)split * a.bq_total + bq) * 32;
      pm[2 * tid] = s_m[tid];
      pm[2 * tid + 1] = s_l[tid];
    }
  }
}

// One workgroup per (query, head): combine the splits' normalised partials,
// each weighted by its sum times exp(its max - the overall max); each thread
// owns two of the 512 output channels.
__global__ void __launch_bounds__(kThreads)
    attend_merge_kernel(const _Float16* __restrict__ part_o, const float* __restrict__ part_ml, int splits,
                        int64_t bq_total, uint16_t* __restrict__ out, float* __restrict__ lse) {
  const int64_t wr = xcd_rank(blockIdx.x, bq_total * 16);  // the XCD of the query's attention splits
  const int64_t bq = wr >> 4;
  const int h = (int)(wr & 15);
  const int tid = threadIdx.x;
  // every load is issued from a clamped split so they all stay in flight together
  float ms[kMaxSplits], ls[kMaxSplits];
  v2h v[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; s++) {
    const int sc = min(s, splits - 1);
    const float2 ml = *reinterpret_cast<const float2*>(part_ml + ((int64_t)sc * bq_total + bq) * 32 + 2 * h);
    ms[s] = ml.x;
    ls[s] = ml.y;
    v[s] = *reinterpret_cast<const v2h*>(part_o + (((int64_t)sc * bq_total + bq) * 16 + h) * 512 + 2 * tid);
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxSplits; s++)
    if (s < splits) M = fmaxf(M, ms[s]);
  float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
  for (int s = 0; s < kMaxSplits; s++) {
    const float w = (s < splits && ms[s] != -INFINITY) ? __expf(ms[s] - M) * ls[s] : 0.0f;
    L += w;
    o0 += w * (float)v[s][0];
    o1 += w * (float)v[s][1];
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const uint32_t packed = (uint32_t)f32_to_bf16_rne(o0 * inv) | ((uint32_t)f32_to_bf16_rne(o1 * inv) << 16);
  reinterpret_cast<uint32_t*>(out + (bq * 16 + h) * 512)[tid] = packed;
  if (lse && tid == 0) lse[bq * 16 + h] = L > 0.0f ? M + __logf(L) : -INFINITY;
}

CSA2_DEV_ERROR_TAKER(take_attend_dev_error)

hipError_t launch_attend(const LaunchCache& c, const int32_t* topk, uint8_t* swa, int32_t S, const float* swa_x,
                         const int32_t* swa_len, int32_t swa_T, const uint16_t* q, const int32_t* q_pos,
                         float sm_scale, uint16_t* out, float* lse, int32_t Q, void* ws, hipStream_t stream) {
  const int64_t bq = (int64_t)c.batch * Q;
  if (bq == 0) return hipSuccess;
  // A long append (a prefill chunk) goes first as its own launch: inside the
  // attention kernel every new token would be re-encoded by each of the up to
  // 128 queries whose window holds it.  The result is the same either way.
  if (swa_x && swa_T > kFusedAppendMax) {
    const hipError_t e = launch_swa_append(swa, S, swa_x, swa_len, c.batch, swa_T, stream);
    if (e != hipSuccess) return e;
    swa_x = nullptr;
    swa_len = nullptr;
    swa_T = 0;
  }
  AttnArgs a;
  a.kv_codes = c.kv_codes;
  a.kv_scales = c.kv_scales;
  a.length = c.length;
  a.cap = c.capacity;
  a.ratio = c.ratio;
  a.topk = topk;
  a.swa = swa;
  a.S = S;
  a.swa_x = swa_x;
  a.swa_len = swa_len;
  a.swa_T = swa_x ? swa_T : 0;
  a.q = q;
  a.q_pos = q_pos;
  a.sm_scale = sm_scale;
  a.Q = Q;
  a.splits = attend_splits(bq);
  a.tps = tiles_per_split(a.splits);
  a.out = out;
  a.lse = lse;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  a.bq_total = bq;
  if (a.splits > 1) {
    uint8_t* base = (uint8_t*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
    a.part_o = (_Float16*)base;
    a.part_ml = (float*)(a.part_o + (int64_t)a.splits * bq * 16 * 512);
  }
  const unsigned n_wg = (unsigned)(a.splits * bq);  // (split, query) pairs in XCD-aware order
  if (a.tps > 2)
    hipLaunchKernelGGL(attend_kernel<true>, dim3(n_wg), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attend_kernel<false>, dim3(n_wg), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL(attend_merge_kernel, dim3((unsigned)(bq * 16)), dim3(kThreads), 0, stream, a.part_o, a.part_ml,
                     a.splits, bq, out, lse);
  return hipGetLastError();
}

}  // namespace csa2

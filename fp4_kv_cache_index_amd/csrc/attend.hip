// Sparse attention of one CSA2 layer: its own 16-head query over the selected
// global entries (FP4 main KV, dequantised on the fly) merged with its own
// 128-token FP8 sliding window, one softmax over both, key = value (the report
// stores one 512-channel latent per entry; ai.info "Main Findings";
// technologiesdigest "CSA2": every layer keeps its own query and window KV).
// Optionally the same launch first appends the layer's new window tokens.
//
// Key slots per query: 0..511 = the Top-512 list, 512..639 = window positions
// p-127..p, taken in groups of 16.  A workgroup of four waves owns a range of
// groups (a split) and takes them in blocks of four, one group per wave:
//   gather: lane l holds key l%16 of its wave's group, channels 128(l/16)..+127
//     (64 FP4 code bytes and 8 E4M3 scale bytes of a main row, or 128 bytes of
//     a window row), as raw buffer loads issued one block ahead;
//   dequantise in registers, half a lane's channels at a time:
//     v_cvt_scalef32_pk_f16_fp4 with scale 1.0 gives the E2M1 values exactly
//     and one fp16 multiply by the group scale gives x = code * scale, exact
//     in fp16 (at most 6 significant bits, |x| in [2^-10, 2688]); window bytes
//     widen exactly with v_cvt_scalef32_pk_f16_fp8;
//   S^T = K Q^T on v_mfma_f32_16x16x32_f16 straight from those registers (key
//     rows are the matrix rows, the 16 heads its columns; the contraction
//     order of the 512 channels is permuted identically on both operands)
//     against the query held in registers.  The bf16 query is scaled per head
//     by a power of two that puts its largest element in [2^14, 2^15), which
//     makes its fp16 copy exact for every element within 2^-28 of the head's
//     largest; the scores are scaled back exactly;
//   the four waves' scores (16 heads x 64 keys) and dequantised keys go to
//     LDS; every wave takes the block's softmax for all 16 heads in fp32 (lane
//     l holds head l%16 for 16 of the keys, the layout of the P^T operand of
//     the next product), so all waves keep the same running max and sum;
//   O^T = alpha O^T + V^T P^T on v_mfma_f32_16x16x32_f16 for the wave's own 128
//     output channels, the keys coming back channel-major from the [key]
//     [channel] tile through the transposing read ds_read_b64_tr_b16.
// No combine across waves is needed at the end.  With one split the workgroup
// writes the bf16 output; with several it writes its unnormalised fp32 partial
// and a second kernel merges the splits by their maxima.  (Merging inside the
// launch, the last split of a query merging, costs a counting atomic's round
// trip and one compute unit reading every split's partial: measured slower
// than the 1.9 us of a dependent launch on gfx950.)
#include <hip/hip_runtime.h>

#include "block_ops.hpp"
#include "codec.hpp"
#include "dev_check.hpp"
#include "kernels.hpp"

namespace csa2 {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKeyGroup = 16;                      // keys per group (one MFMA tile of keys)
constexpr int kMainGroups = 512 / kKeyGroup;       // groups 0..31 hold Top-K slots, 32..39 the window
constexpr int kVStride = 528;                      // fp16 per key row of a wave's V tile (512 + pad)
constexpr int kQStride = 520;                      // fp16 per head row of the scaled query (512 + pad)
constexpr int kFusedAppendMax = 8;  // new window tokens per sequence appended inside the attention launch

// Splits per query (each a workgroup of four waves taking 10 / splits blocks
// of 64 keys).  Few queries spread every query over 10 workgroups of one
// block, so that each workgroup gathers only 64 rows: a gather's time grows with
// the rows one compute unit fetches (measured on gfx950, 10,240 rows: 2.8 us at
// 16 rows per workgroup, 4.0 at 64, 6.2 at 128).  Many queries fill the chip
// with fewer splits and need no merge at all from 1,024 queries on.
int attend_splits(int64_t bq) {
  if (bq <= 64) return 10;
  if (bq <= 256) return 5;
  if (bq <= 1024) return 2;
  return 1;
}

// [partial O, unnormalised fp32: splits x bq x 16 x 512] [partial (max, sum): splits x bq x 16 x 2 f32]
size_t attend_ws_bytes(int64_t bq) {
  const int s = attend_splits(bq);
  if (s == 1) return 0;
  return 256 + (size_t)s * bq * (16 * 512 * 4 + 16 * 2 * 4);
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
  int32_t splits;
  uint16_t* out;
  float* lse;
  float* part_o;
  float* part_ml;
  int64_t bq_total;
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t h2_bits(v2h h) { return __builtin_bit_cast(uint32_t, h); }

using BufRsrc = __amdgpu_buffer_rsrc_t;
// A raw buffer of `bytes` bytes at p: a load at an offset past the end returns
// zeros without a memory access, so a load that may not be wanted is issued
// anyway, with no branch around it (the compiler waits for a load under a
// branch before the branch ends).
__device__ __forceinline__ BufRsrc make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOff = 0x80000000u;  // an offset past every buffer here

__device__ __forceinline__ uint4 buf16(BufRsrc r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// LDS transpose read: in each 16-lane group, lane 4j+q names 4 consecutive fp16
// of row j; lane i receives element i%4 of lanes i/4, i/4+4, i/4+8, i/4+12,
// i.e. column i of the 4-row block.
__device__ __forceinline__ v4h lds_read_tr16(const _Float16* p) {
  return __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p)));
}

// LDS ordering inside one wave: the wave's earlier LDS stores are complete and
// visible to all of its lanes, and the compiler moves no LDS access across.
__device__ __forceinline__ void lds_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// max / sum of one value per lane over the four lanes l%16 + 16j (the four
// rows of a wave), every lane getting the result
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// 8 E2M1 codes (low nibble first) times a group scale, as four fp16x2 words
__device__ __forceinline__ void fp4_word(uint32_t w, v2h s2, uint32_t* o) {
  o[0] = h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2);
  o[1] = h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2);
  o[2] = h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2);
  o[3] = h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2);
}

// One group's raw bytes for this lane, as loaded: w[0..7] 128 bytes (a main row
// uses w[0..3], its 64 code bytes), sc the 8 scale bytes of a main row.
struct Raw {
  uint4 w[8];
  uint2 sc;
};

// What a workgroup knows about its (query, split).
struct Wg {
  int64_t bq;
  int split, b, qi, tid, wave, n, g;  // n = lane % 16 (key row of S^T, head column), g = lane / 16
  int32_t p;                          // the query's token position
  int32_t new_lo, new_hi;             // new window tokens: positions new_lo .. new_hi-1
  int32_t n_vis_dbg;                  // debug builds: entries the query may list
  bool stage;                         // stages the new window tokens (holds window groups)
  int first_win_split;
  BufRsrc ids_r, codes_r, scales_r, swa_r, none_r;
};

__device__ __forceinline__ Wg make_wg(const AttnArgs& a, int gpw) {
  Wg w;
  const int64_t wr = xcd_rank(blockIdx.x, (int64_t)a.splits * a.bq_total);
  w.split = (int)(wr % a.splits);
  w.bq = wr / a.splits;
  w.b = (int)(w.bq / a.Q);
  w.qi = (int)(w.bq % a.Q);
  w.tid = threadIdx.x;
  w.wave = __builtin_amdgcn_readfirstlane(w.tid >> 6);  // uniform in the wave: the buffer descriptors it selects stay scalar
  w.n = w.tid & 15;
  w.g = (w.tid & 63) >> 4;
  w.p = a.q_pos ? a.q_pos[w.bq] : a.length[w.b] * a.ratio - a.Q + w.qi;
  w.new_hi = a.swa_x ? a.swa_len[w.b] : 0;
  w.new_lo = a.swa_x ? w.new_hi - a.swa_T : 0;
  w.n_vis_dbg = 0;
  if (kDebug) {
    const int32_t len = a.length[w.b];
    if (w.tid == 0 && w.split == 0 && (len < 0 || len > a.cap)) dev_flag(kErrLength);
    if (w.tid == 0 && w.split == 0 && w.new_lo < 0) dev_flag(kErrSeqLen);
    const int64_t by_pos = w.p < 0 ? 0 : ((int64_t)w.p + 1) / a.ratio;
    w.n_vis_dbg = (int32_t)min((int64_t)min(len, a.cap), by_pos);
  }
  w.first_win_split = kMainGroups / (kWaves * gpw);
  w.stage = a.swa_x != nullptr && (w.split + 1) * kWaves * gpw > kMainGroups;
  w.ids_r = make_rsrc(a.topk + w.bq * 512, 2048u);
  w.codes_r = make_rsrc(a.kv_codes + (int64_t)w.b * a.cap * 256, (uint32_t)a.cap * 256u);
  w.scales_r = make_rsrc(a.kv_scales + (int64_t)w.b * a.cap * 32, (uint32_t)a.cap * 32u);
  w.swa_r = make_rsrc(a.swa + (int64_t)w.b * a.S * 512, (uint32_t)a.S * 512u);
  w.none_r = make_rsrc(a.swa, 0u);
  return w;
}

// the window position of key n of window group grp
__device__ __forceinline__ int32_t win_pos(const Wg& w, int grp) { return w.p - 127 + (grp * kKeyGroup + w.n - 512); }

// the Top-K id of key n of group grp (a window group reads nothing: 0)
__device__ __forceinline__ int32_t load_id(const Wg& w, int grp) {
  const uint32_t off = grp < kMainGroups ? (uint32_t)(grp * kKeyGroup + w.n) * 4u : kOff;
  return (int32_t)__builtin_amdgcn_raw_buffer_load_b32(w.ids_r, off, 0, 0);
}

// whether key n of group grp exists: a listed id (debug builds: flagged and
// dropped when past the visible entries), or a window position >= 0
__device__ __forceinline__ bool key_valid(const Wg& w, int grp, int32_t& id) {
  if (grp < kMainGroups) {
    if (kDebug && (id < -1 || (id >= 0 && id >= w.n_vis_dbg))) {
      dev_flag(kErrEntryId);
      id = -1;
    }
    return id >= 0;
  }
  return win_pos(w, grp) >= 0;
}

// issue the loads of group grp (wave-uniform kind; no branch around a load)
__device__ __forceinline__ void issue(const Wg& w, const AttnArgs& a, int grp, int32_t id, Raw& r,
                                      bool live = true) {
  const bool is_main = grp < kMainGroups;
  const bool ok = live && key_valid(w, grp, id);
  const int32_t pos = win_pos(w, grp);
  const uint32_t slot = (uint32_t)((pos >= 0 ? pos : 0) % a.S);
  const BufRsrc rr = is_main ? w.codes_r : w.swa_r;
  const BufRsrc sr = is_main ? w.scales_r : w.none_r;
  const uint32_t base = !ok ? kOff : is_main ? (uint32_t)id * 256u + 64u * w.g : slot * 512u + 128u * w.g;
#pragma unroll
  for (int j = 0; j < 8; j++) r.w[j] = buf16(rr, (is_main && j >= 4) ? kOff : base + 16u * j);
  r.sc = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(sr, ok ? (uint32_t)id * 32u + 8u * w.g : kOff, 0, 0));
}

// query: thread t holds head t/16, channels 32(t%16) .. +31 (bf16)
__device__ __forceinline__ void load_query(const Wg& w, const AttnArgs& a, uint4 (&qraw)[4]) {
  const uint16_t* qrow = a.q + (w.bq * 16 + (w.tid >> 4)) * 512 + 32 * (w.tid & 15);
#pragma unroll
  for (int k = 0; k < 4; k++) qraw[k] = *reinterpret_cast<const uint4*>(qrow + 8 * k);
}

// the new window tokens (fp32), channels 2t, 2t+1 of each, when this workgroup stages them
__device__ __forceinline__ void load_new(const Wg& w, const AttnArgs& a, float2 (&xv)[kFusedAppendMax]) {
  const BufRsrc xr = make_rsrc(a.swa_x + (w.stage ? (int64_t)w.b * a.swa_T * 512 : 0),
                               w.stage ? (uint32_t)a.swa_T * 2048u : 0u);
#pragma unroll
  for (int j = 0; j < kFusedAppendMax; j++)
    xv[j] = __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(xr, (uint32_t)(j * 2048 + 8 * w.tid), 0, 0));
}

// The query scaled per head into fp16 (s_q [head][kQStride]) with the factor
// that undoes the scale and applies sm_scale (s_qfac); the new window tokens
// encoded into s_new and, by the (query, window split) of rank j mod
// (Q * window splits), into the ring.
__device__ __forceinline__ void stage_inputs(const Wg& w, const AttnArgs& a, const uint4 (&qraw)[4],
                                             const float2 (&xv)[kFusedAppendMax], _Float16* s_q, float* s_qfac,
                                             uint8_t* s_new) {
  const int qh = w.tid >> 4, qc = 32 * (w.tid & 15);
  float qf[32];
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const uint32_t xw[4] = {qraw[k].x, qraw[k].y, qraw[k].z, qraw[k].w};
#pragma unroll
    for (int m = 0; m < 4; m++) {
      qf[8 * k + 2 * m] = __uint_as_float(xw[m] << 16);
      qf[8 * k + 2 * m + 1] = __uint_as_float(xw[m] & 0xFFFF0000u);
      amax = fmaxf(amax, fmaxf(fabsf(qf[8 * k + 2 * m]), fabsf(qf[8 * k + 2 * m + 1])));
    }
  }
  amax = wave_row_reduce(amax, [](float x, float y) { return fmaxf(x, y); });  // the 16 threads of head qh
  int ex;
  frexpf(amax, &ex);  // amax = f * 2^ex, f in [0.5, 1); ex = 0 for a zero head
  const int sh = min(127, max(-126, 15 - ex));
  const float up = ldexpf(1.0f, sh);
  if ((w.tid & 15) == 0) s_qfac[qh] = ldexpf(a.sm_scale, -sh);
#pragma unroll
  for (int k = 0; k < 4; k++) {
    v8h h;
#pragma unroll
    for (int m = 0; m < 8; m++) h[m] = (_Float16)(qf[8 * k + m] * up);
    *reinterpret_cast<v8h*>(s_q + qh * kQStride + qc + 8 * k) = h;
  }
  if (w.stage) {
    const int n_ws = a.splits - w.first_win_split;
    const int n_w = a.Q * n_ws, rank = w.qi * n_ws + (w.split - w.first_win_split);
#pragma unroll
    for (int j = 0; j < kFusedAppendMax; j++) {
      if (j < a.swa_T) {
        const uint16_t c = (uint16_t)(e4m3_encode(xv[j].x) | (e4m3_encode(xv[j].y) << 8));
        reinterpret_cast<uint16_t*>(s_new + j * 512)[w.tid] = c;
        if (j % n_w == rank && w.new_lo + j >= 0)  // a window shorter than the append has no slot for it
          reinterpret_cast<uint16_t*>(a.swa + ((int64_t)w.b * a.S + (w.new_lo + j) % a.S) * 512)[w.tid] = c;
      }
    }
  }
}

// Half h of this lane's quarter of key n of group grp as fp16 pairs: kh[c]
// holds channels 128g + 64h + 2c, 2c + 1 (c < 32).  A window token appended by
// this call comes from s_new.
__device__ __forceinline__ void dequant(const Wg& w, int grp, const Raw& r, const uint8_t* s_new, int h,
                                             uint32_t (&kh)[32]) {
  if (grp < kMainGroups) {
    const uint32_t scw = h ? r.sc.y : r.sc.x;
#pragma unroll
    for (int s4 = 0; s4 < 4; s4++) {  // scale group 4h + s4: channels 128g + 16(4h + s4) .. +15
      const uint32_t sb = (scw >> (8 * s4)) & 0xFFu;
      const v2h s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb * 0x0101u, 1.0f, false);
      const uint4 w4 = r.w[2 * h + (s4 >> 1)];
      const uint32_t c0 = (s4 & 1) ? w4.z : w4.x, c1 = (s4 & 1) ? w4.w : w4.y;
      fp4_word(c0, s2, kh + 8 * s4);
      fp4_word(c1, s2, kh + 8 * s4 + 4);
    }
  } else {
    const int32_t pos = win_pos(w, grp);
    const bool fresh = pos >= w.new_lo && pos < w.new_hi;
#pragma unroll
    for (int j4 = 0; j4 < 4; j4++) {
      const int j = 4 * h + j4;
      uint4 x = r.w[j];
      if (fresh) x = *reinterpret_cast<const uint4*>(s_new + (pos - w.new_lo) * 512 + 128 * w.g + 16 * j);
      const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int k = 0; k < 4; k++) {
        kh[8 * j4 + 2 * k] = h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(xw[k], 1.0f, false));
        kh[8 * j4 + 2 * k + 1] = h2_bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(xw[k], 1.0f, true));
      }
    }
  }
}

constexpr int kSStride = 68;  // fp32 per head row of the shared scores (64 keys + pad)

// One block of a split for this wave: group grp (rows in cur, id id_c) is
// dequantised and scored against the query operand qb, the four waves' scores
// and keys meet in LDS (s_s, s_v), and the wave folds the block's softmax into
// its running (m_run, l_run) and P V into its 128 output channels (acc).
// Block j > 0 first waits until every wave is past block j - 1.
__device__ __forceinline__ void attend_block(const Wg& w, int j, int grp, const Raw& cur, int32_t id_c,
                                             const v8h (&qb)[16], float qfac, const uint8_t* s_new, _Float16* s_v,
                                             float* s_s, v4f (&acc)[8], float& m_run, float& l_run) {
  const int n = w.n, g = w.g, wave = w.wave;
  const uint32_t vmask = (uint32_t)__ballot(key_valid(w, grp, id_c)) & 0xFFFFu;  // bit k: key k exists
  // the group's keys in two halves of each lane's 128 channels: dequantise,
  // score and store each half into the tile (free once every wave is past
  // the previous block), so only one half is held in registers
  if (j > 0) lds_barrier();  // every wave is done with the previous block's tile and scores
  v4f st = {0.f, 0.f, 0.f, 0.f};
  _Float16* rows = s_v + wave * 16 * kVStride + n * kVStride + 128 * g;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    uint32_t kh[32];
    dequant(w, grp, cur, s_new, h, kh);
#pragma unroll
    for (int kb = 0; kb < 8; kb++) {
      const v8h ka = __builtin_bit_cast(v8h, make_uint4(kh[4 * kb], kh[4 * kb + 1], kh[4 * kb + 2], kh[4 * kb + 3]));
      st = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[8 * h + kb], st, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < 8; c++)
      *reinterpret_cast<uint4*>(rows + 64 * h + 8 * c) = make_uint4(kh[4 * c], kh[4 * c + 1], kh[4 * c + 2], kh[4 * c + 3]);
  }
  {
    v4f sc;
#pragma unroll
    for (int i = 0; i < 4; i++) sc[i] = ((vmask >> (4 * g + i)) & 1u) ? st[i] * qfac : -INFINITY;
    *reinterpret_cast<v4f*>(s_s + n * kSStride + 16 * wave + 4 * g) = sc;
  }
  lds_barrier();  // every wave's scores and keys are in

  // ---- softmax of head n over the block: this lane holds keys 32kb + 8g .. +7
  float sv[2][8];
#pragma unroll
  for (int kb = 0; kb < 2; kb++) {
    const v4f lo = *reinterpret_cast<const v4f*>(s_s + n * kSStride + 32 * kb + 8 * g);
    const v4f hi = *reinterpret_cast<const v4f*>(s_s + n * kSStride + 32 * kb + 8 * g + 4);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      sv[kb][i] = lo[i];
      sv[kb][4 + i] = hi[i];
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; kb++)
#pragma unroll
    for (int i = 0; i < 8; i++) mx = fmaxf(mx, sv[kb][i]);
  mx = rows_max(mx);
  const float m_new = fmaxf(m_run, mx);
  const float alpha = (m_new == -INFINITY) ? 1.0f : __expf(m_run - m_new);
  float ps = 0.0f;
  v8h pb[2], pr[2];  // P as its fp16 rounding and the residual (P_hi + P_lo)
#pragma unroll
  for (int kb = 0; kb < 2; kb++)
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float pv = sv[kb][i] == -INFINITY ? 0.0f : __expf(sv[kb][i] - m_new);
      ps += pv;
      const _Float16 ph = (_Float16)pv;
      pb[kb][i] = ph;
      pr[kb][i] = (_Float16)(pv - (float)ph);  // the difference is exact in fp32
    }
  ps = rows_sum(ps);
  m_run = m_new;
  l_run = alpha * l_run + ps;

  // ---- O^T = alpha O^T + V^T P^T for channels 128 wave .. +127 (alpha = 1 before the first block)
#pragma unroll
  for (int c = 0; c < 8; c++) acc[c] *= alpha;
#pragma unroll
  for (int kb = 0; kb < 2; kb++) {
    const _Float16* vsrc = s_v + (32 * kb + 8 * g + (n >> 2)) * kVStride + 128 * wave + 4 * (n & 3);
#pragma unroll
    for (int c = 0; c < 8; c++) {
      const v4h lo = lds_read_tr16(vsrc + 16 * c);
      const v4h hi = lds_read_tr16(vsrc + 4 * kVStride + 16 * c);
      const v8h va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[kb], acc[c], 0, 0, 0);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pr[kb], acc[c], 0, 0, 0);
    }
  }
}

constexpr int kPStride = 72;  // fp16 per head row of the shared P tile (64 keys + pad)
constexpr float kLazyMax = 8.0f;  // most a logit may exceed its head's running max (attend_block_sp)

// attend_block with the block's softmax split over the waves (many queries:
// two workgroups per compute unit, where VALU work, not a barrier, sets the
// pace): wave w takes heads 4w .. 4w+3, four keys per lane, and shares P (fp16)
// and each head's rescale factor through LDS (s_p, s_alpha).  This wave's
// running (m_run, l_run) are those of head 4 wave + lane / 16; the output
// rows of this lane's accumulators are head n = lane % 16.  A head's running
// max moves only when a block's maximum exceeds it by more than kLazyMax, so
// P stays below e^kLazyMax (about 2,981, well inside fp16) and after the
// first blocks the rescale of the accumulators is mostly skipped; every
// quantity stays relative to the same m_run, so the softmax is unchanged but
// for rounding.
__device__ __forceinline__ void attend_block_sp(const Wg& w, int j, int grp, const Raw& cur, int32_t id_c,
                                                const v8h (&qb)[16], float qfac, const uint8_t* s_new, _Float16* s_v,
                                                float* s_s, _Float16* s_p, float* s_alpha, v4f (&acc)[8], float& m_run,
                                                float& l_run) {
  const int n = w.n, g = w.g, wave = w.wave;
  const int lane = w.tid & 63;
  const uint32_t vmask = (uint32_t)__ballot(key_valid(w, grp, id_c)) & 0xFFFFu;  // bit k: key k exists
  if (j > 0) lds_barrier();  // every wave is done with the previous block's tile, scores and P
  v4f st = {0.f, 0.f, 0.f, 0.f};
  _Float16* rows = s_v + wave * 16 * kVStride + n * kVStride + 128 * g;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    uint32_t kh[32];
    dequant(w, grp, cur, s_new, h, kh);
#pragma unroll
    for (int kb = 0; kb < 8; kb++) {
      const v8h ka = __builtin_bit_cast(v8h, make_uint4(kh[4 * kb], kh[4 * kb + 1], kh[4 * kb + 2], kh[4 * kb + 3]));
      st = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka, qb[8 * h + kb], st, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < 8; c++)
      *reinterpret_cast<uint4*>(rows + 64 * h + 8 * c) = make_uint4(kh[4 * c], kh[4 * c + 1], kh[4 * c + 2], kh[4 * c + 3]);
  }
  {
    v4f sc;
#pragma unroll
    for (int i = 0; i < 4; i++) sc[i] = ((vmask >> (4 * g + i)) & 1u) ? st[i] * qfac : -INFINITY;
    *reinterpret_cast<v4f*>(s_s + n * kSStride + 16 * wave + 4 * g) = sc;
  }
  lds_barrier();  // every wave's scores and keys are in

  // ---- softmax of head hs = 4 wave + lane / 16 over the block: keys 4 (lane % 16) .. +3
  {
    const int hs = 4 * wave + (lane >> 4), k0 = 4 * (lane & 15);
    const v4f sv = *reinterpret_cast<const v4f*>(s_s + hs * kSStride + k0);
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = wave_row_reduce(mx, [](float x, float y) { return fmaxf(x, y); });
    // m_run stays unless this block's maximum is more than kLazyMax above it
    // (a first finite maximum always moves it off -inf)
    const float m_new = mx > m_run + kLazyMax ? mx : m_run;
    const float alpha = m_new == m_run ? 1.0f : __expf(m_run - m_new);
    float ps = 0.0f;
    v4h pv, pl;  // P as its fp16 rounding and the residual (P_hi + P_lo)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float e = sv[i] == -INFINITY ? 0.0f : __expf(sv[i] - m_new);
      ps += e;
      pv[i] = (_Float16)e;
      pl[i] = (_Float16)(e - (float)pv[i]);  // the difference is exact in fp32
    }
    ps = wave_row_reduce(ps, [](float x, float y) { return x + y; });
    m_run = m_new;
    l_run = alpha * l_run + ps;
    *reinterpret_cast<v4h*>(s_p + hs * kPStride + k0) = pv;
    *reinterpret_cast<v4h*>(s_p + (16 + hs) * kPStride + k0) = pl;
    if ((lane & 15) == 0) s_alpha[hs] = alpha;
  }
  lds_barrier();  // P and every head's rescale factor are in

  // ---- O^T = alpha O^T + V^T P^T for channels 128 wave .. +127, head n
  const float alpha_n = s_alpha[n];
  v8h pb[2], pr[2];
#pragma unroll
  for (int kb = 0; kb < 2; kb++) {
    pb[kb] = *reinterpret_cast<const v8h*>(s_p + n * kPStride + 32 * kb + 8 * g);
    pr[kb] = *reinterpret_cast<const v8h*>(s_p + (16 + n) * kPStride + 32 * kb + 8 * g);
  }
  if (__ballot(alpha_n != 1.0f)) {  // uniform: some head's running max moved
#pragma unroll
    for (int c = 0; c < 8; c++) acc[c] *= alpha_n;
  }
#pragma unroll
  for (int kb = 0; kb < 2; kb++) {
    const _Float16* vsrc = s_v + (32 * kb + 8 * g + (n >> 2)) * kVStride + 128 * wave + 4 * (n & 3);
#pragma unroll
    for (int c = 0; c < 8; c++) {
      const v4h lo = lds_read_tr16(vsrc + 16 * c);
      const v4h hi = lds_read_tr16(vsrc + 4 * kVStride + 16 * c);
      const v8h va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[kb], acc[c], 0, 0, 0);
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pr[kb], acc[c], 0, 0, 0);
    }
  }
}

// The query staged in LDS (s_q, s_qfac) and the new window tokens (s_new);
// returns the query operand of S^T = K Q^T in qb: head n, channels 128g + 8kb .. +7.
__device__ __forceinline__ void attend_setup(const Wg& w, const AttnArgs& a, const uint4 (&qraw)[4],
                                             const float2 (&xv)[kFusedAppendMax], _Float16* s_q, float* s_qfac,
                                             uint8_t* s_new, v8h (&qb)[16], float& qfac) {
  stage_inputs(w, a, qraw, xv, s_q, s_qfac, s_new);
  lds_barrier();  // s_q, s_qfac, s_new written; the rows stay in flight
  qfac = s_qfac[w.n];
#pragma unroll
  for (int kb = 0; kb < 16; kb++) qb[kb] = *reinterpret_cast<const v8h*>(s_q + w.n * kQStride + 128 * w.g + 8 * kb);
  lds_barrier();  // every wave holds its query operand: the staging area becomes the key tile
}

// The wave's 128 channels of the result: the bf16 output (one split) or the
// unnormalised fp32 partial with (max, sum) per head.
__device__ __forceinline__ void attend_finish(const Wg& w, const AttnArgs& a, const v4f (&acc)[8], float m_run,
                                              float l_run) {
  const int n = w.n, g = w.g, wave = w.wave;
  // every wave holds the same (m_run, l_run) for head n
  if (a.splits == 1) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    uint16_t* dst = a.out + (w.bq * 16 + n) * 512 + 128 * wave + 4 * g;
#pragma unroll
    for (int c = 0; c < 8; c++) {
      const uint2 v = make_uint2((uint32_t)f32_to_bf16_rne(acc[c][0] * inv) | ((uint32_t)f32_to_bf16_rne(acc[c][1] * inv) << 16),
                                 (uint32_t)f32_to_bf16_rne(acc[c][2] * inv) | ((uint32_t)f32_to_bf16_rne(acc[c][3] * inv) << 16));
      *reinterpret_cast<uint2*>(dst + 16 * c) = v;
    }
    if (wave == 0 && g == 0 && a.lse) a.lse[w.bq * 16 + n] = l_run > 0.0f ? m_run + __logf(l_run) : -INFINITY;
  } else {
    float* po = a.part_o + ((int64_t)w.split * a.bq_total + w.bq) * 16 * 512 + n * 512 + 128 * wave + 4 * g;
#pragma unroll
    for (int c = 0; c < 8; c++) *reinterpret_cast<v4f*>(po + 16 * c) = acc[c];
    if (wave == 0 && g == 0) {
      float* pm = a.part_ml + ((int64_t)w.split * a.bq_total + w.bq) * 32;
      pm[2 * n] = m_run;
      pm[2 * n + 1] = l_run;
    }
  }
}

// More queries, fewer splits: a workgroup takes its split's groups in blocks
// of four (64 keys), one group per wave, with an online softmax across the
// blocks.  Per block every wave scores its group against the query (held in
// registers), shares the scores and its dequantised keys through LDS, takes
// the softmax of the block for all 16 heads (so every wave holds the same
// running max and sum), and accumulates P V for its own 128 output channels:
// 32 accumulator registers per lane, no combine at the end.  The query staging
// area and the key tile share LDS, which keeps the kernel at 76 KB.
//
// attend_block_kernel: two workgroups per compute unit (244 VGPRs); the next
// block's rows load while one is processed.  Blocks go in pairs through a loop
// that is not unrolled; the loads past the last block are issued to offsets
// that read nothing, so no load sits under a branch.
template <int kGpw>  // blocks per workgroup
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) attend_block_kernel(AttnArgs a) {
  static_assert(16 * kQStride <= kWaves * 16 * kVStride, "the query staging fits in the key tile");
  // the softmax split over the waves where a workgroup takes every block of its query
  constexpr bool kShareP = kGpw == 10;
  __shared__ __attribute__((aligned(16))) _Float16 s_v[kWaves * 16 * kVStride];  // query staging, then keys
  __shared__ __attribute__((aligned(16))) float s_s[16 * kSStride];              // scores [head][key]
  __shared__ __attribute__((aligned(16))) uint8_t s_new[kFusedAppendMax * 512];
  __shared__ float s_qfac[16];
  __shared__ __attribute__((aligned(16))) _Float16 s_p[kShareP ? 32 * kPStride : 8];  // P [head][key], then its residuals
  __shared__ float s_alpha[16];
  __shared__ float2 s_ml[16];
  const Wg w = make_wg(a, kGpw);
  const int grp0 = w.split * kWaves * kGpw + w.wave;  // block j: group grp0 + 4j

  int32_t id_a = load_id(w, grp0);
  int32_t id_b = load_id(w, kGpw > 1 ? grp0 + kWaves : kMainGroups);
  uint4 qraw[4];
  load_query(w, a, qraw);
  float2 xv[kFusedAppendMax];
  load_new(w, a, xv);
  Raw ra, rb;
  issue(w, a, grp0, id_a, ra);
  v8h qb[16];
  float qfac;
  attend_setup(w, a, qraw, xv, s_v, s_qfac, s_new, qb, qfac);
  v4f acc[8];  // O^T: acc[c][i] = O[head n][channel 128 wave + 16c + 4g + i], relative to m_run
#pragma unroll
  for (int c = 0; c < 8; c++) acc[c] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  // block j: its rows in cur (id id_c); block j + 1's rows (id id_n) load into
  // nxt, and block j + 2's id is returned
  auto step = [&](int j, Raw& cur, Raw& nxt, int32_t id_c, int32_t id_n) -> int32_t {
    const int grp = grp0 + kWaves * j;
    const int32_t id_n2 = load_id(w, j + 2 < kGpw ? grp + 2 * kWaves : kMainGroups);
    issue(w, a, grp + kWaves, id_n, nxt, j + 1 < kGpw);
    if constexpr (kShareP)
      attend_block_sp(w, j, grp, cur, id_c, qb, qfac, s_new, s_v, s_s, s_p, s_alpha, acc, m_run, l_run);
    else
      attend_block(w, j, grp, cur, id_c, qb, qfac, s_new, s_v, s_s, acc, m_run, l_run);
    return id_n2;
  };
#pragma unroll 1
  for (int j = 0; j < kGpw; j += 2) {
    const int32_t id_c = step(j, ra, rb, id_a, id_b);  // block j + 2's id
    if (kGpw % 2 == 0 || j + 1 < kGpw) {  // always, for an even block count
      const int32_t id_d = step(j + 1, rb, ra, id_b, id_c);
      id_a = id_c;
      id_b = id_d;
    }
  }
  if constexpr (kShareP) {  // head n's (max, sum) from the wave that took its softmax
    if (((w.tid & 63) & 15) == 0) s_ml[4 * w.wave + ((w.tid & 63) >> 4)] = make_float2(m_run, l_run);
    lds_barrier();
    const float2 ml = s_ml[w.n];
    m_run = ml.x;
    l_run = ml.y;
  }
  attend_finish(w, a, acc, m_run, l_run);
}

// One workgroup per (query, head): combine the splits' unnormalised partials,
// each weighted by exp(its max - the overall max); each thread owns four of the
// 512 output channels.
constexpr int kMergeThreads = 128;
__global__ void __launch_bounds__(kMergeThreads)
    attend_merge_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml, int splits,
                        int64_t bq_total, uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int kMax = 10;
  const int64_t wr = xcd_rank(blockIdx.x, bq_total * 16);  // the XCD of the query's attention splits
  const int64_t bq = wr >> 4;
  const int h = (int)(wr & 15);
  const int tid = threadIdx.x;
  // every load is issued from a clamped split so they all stay in flight together
  float ms[kMax], ls[kMax];
  float4 v[kMax];
#pragma unroll
  for (int s = 0; s < kMax; s++) {
    const int sc = min(s, splits - 1);
    const float2 ml = *reinterpret_cast<const float2*>(part_ml + ((int64_t)sc * bq_total + bq) * 32 + 2 * h);
    ms[s] = ml.x;
    ls[s] = ml.y;
    v[s] = *reinterpret_cast<const float4*>(part_o + (((int64_t)sc * bq_total + bq) * 16 + h) * 512 + 4 * tid);
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMax; s++)
    if (s < splits) M = fmaxf(M, ms[s]);
  float L = 0.0f, o0 = 0.0f, o1 = 0.0f, o2 = 0.0f, o3 = 0.0f;
#pragma unroll
  for (int s = 0; s < kMax; s++) {
    const float w = (s < splits && ms[s] != -INFINITY) ? __expf(ms[s] - M) : 0.0f;
    L += w * ls[s];
    o0 += w * v[s].x;
    o1 += w * v[s].y;
    o2 += w * v[s].z;
    o3 += w * v[s].w;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const uint2 packed = make_uint2(
      (uint32_t)f32_to_bf16_rne(o0 * inv) | ((uint32_t)f32_to_bf16_rne(o1 * inv) << 16),
      (uint32_t)f32_to_bf16_rne(o2 * inv) | ((uint32_t)f32_to_bf16_rne(o3 * inv) << 16));
  reinterpret_cast<uint2*>(out + (bq * 16 + h) * 512)[tid] = packed;
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
  a.out = out;
  a.lse = lse;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  a.bq_total = bq;
  if (a.splits > 1) {
    uint8_t* base = (uint8_t*)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
    a.part_o = (float*)base;
    a.part_ml = a.part_o + (int64_t)a.splits * bq * 16 * 512;
  }
  const unsigned n_wg = (unsigned)(a.splits * bq);  // (split, query) pairs in XCD-aware order
  switch (a.splits) {
    case 10: hipLaunchKernelGGL(attend_block_kernel<1>, dim3(n_wg), dim3(kThreads), 0, stream, a); break;
    case 5: hipLaunchKernelGGL(attend_block_kernel<2>, dim3(n_wg), dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(attend_block_kernel<5>, dim3(n_wg), dim3(kThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL(attend_block_kernel<10>, dim3(n_wg), dim3(kThreads), 0, stream, a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL(attend_merge_kernel, dim3((unsigned)(bq * 16)), dim3(kMergeThreads), 0, stream, a.part_o,
                     a.part_ml, a.splits, bq, out, lse);
  return hipGetLastError();
}

}  // namespace csa2

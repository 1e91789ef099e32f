// Host side of the C-ABI declared in include/csa2.h: argument validation,
// workspace sizing and dispatch to the gfx950 kernels.  Every check here runs
// before anything is enqueued, so a call that fails enqueues nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "csa2.h"
#include "kernels.hpp"

// Device scratch of csa2_sparse_attend_noalloc: one array per GPU the library
// runs on, held until the process ends.  Host code never passes `scratch`
// itself to a kernel (on the host it only names the symbol); it looks up each
// device's address once with hipGetSymbolAddress and passes that.
static __device__ __align__(256) uint8_t scratch[CSA2_NOALLOC_SCRATCH_BYTES];

namespace {

using csa2::kMaxCapacity;
constexpr int32_t kMaxRatio = 16;                              // tokens per compressed entry

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_cache(const csa2_cache* c, bool need_index, bool need_main) {
  if (!c) return CSA2_EINVAL;
  if (c->batch < 0 || c->capacity < 0) return CSA2_EINVAL;
  if (c->ratio < 1 || c->ratio > kMaxRatio) return CSA2_EINVAL;
  if (c->capacity > kMaxCapacity) return CSA2_EUNSUPPORTED;
  if (c->batch == 0) return CSA2_OK;
  if (!c->length || !aligned(c->length, 4)) return CSA2_EINVAL;
  if (need_index && (!c->ik_codes || !c->ik_scales || !aligned(c->ik_codes, 16) || !aligned(c->ik_scales, 4)))
    return CSA2_EINVAL;
  if (need_main && (!c->kv_codes || !c->kv_scales || !aligned(c->kv_codes, 16) || !aligned(c->kv_scales, 4)))
    return CSA2_EINVAL;
  return CSA2_OK;
}

csa2::LaunchCache to_launch(const csa2_cache* c) {
  csa2::LaunchCache l;
  l.kv_codes = c->kv_codes;
  l.kv_scales = c->kv_scales;
  l.ik_codes = c->ik_codes;
  l.ik_scales = c->ik_scales;
  l.length = c->length;
  l.batch = c->batch;
  l.capacity = c->capacity;
  l.ratio = c->ratio;
  return l;
}

int from_hip(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_EHIP; }

// This device's address of `scratch`, looked up on the first call that needs it
// on the device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int device_scratch(void* stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return CSA2_EHIP;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return CSA2_EHIP;
    if (sdev != dev) return CSA2_EINVAL;  // the stream must belong to the current device
  }
  if (dev < 0 || dev >= kMaxDevices) return CSA2_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CSA2_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSA2_OK;
}

// Debug library: a precondition violation that an earlier call's kernels
// recorded on this device (read once the stream's earlier work is done) is
// reported as CSA2_EDEVICE, and the record cleared, by the next call that has
// work to enqueue.  The release library returns CSA2_OK without touching the
// GPU.
int device_status(void* stream) {
  const hipStream_t s = (hipStream_t)stream;
  const uint32_t e = csa2::take_append_dev_error(s) | csa2::take_attend_dev_error(s) | csa2::take_head_dev_error(s);
  return e ? CSA2_EDEVICE : CSA2_OK;
}

}  // namespace

extern "C" {

// the shared body of the two append calls: exactly one of ik and w_ik is given
static int quantize_append_impl(const csa2_cache* cache, const float* kv, const float* logits, const float* ik,
                                const float* w_ik, int32_t T, int32_t host_len_bound, void* stream) {
  int rc = check_cache(cache, true, true);
  if (rc != CSA2_OK) return rc;
  if (T < 0 || host_len_bound < 0) return CSA2_EINVAL;
  if (T % cache->ratio != 0) return CSA2_EINVAL;
  if ((cache->ratio >= 2) != (logits != nullptr)) return CSA2_EINVAL;
  const int64_t n_new = T / cache->ratio;
  if ((int64_t)host_len_bound + n_new > cache->capacity) return CSA2_ECAPACITY;
  if (cache->batch == 0 || T == 0) return CSA2_OK;
  if (!kv || !aligned(kv, 16)) return CSA2_EINVAL;
  if ((ik == nullptr) == (w_ik == nullptr)) return CSA2_EINVAL;
  if ((ik && !aligned(ik, 4)) || (w_ik && !aligned(w_ik, 4))) return CSA2_EINVAL;
  if (logits && !aligned(logits, 4)) return CSA2_EINVAL;
  if ((rc = device_status(stream)) != CSA2_OK) return rc;
  return from_hip(csa2::launch_quant_append(to_launch(cache), kv, logits, ik, w_ik, T, (hipStream_t)stream));
}

int csa2_quantize_append(const csa2_cache* cache, const float* kv, const float* logits, const float* ik, int32_t T,
                         int32_t host_len_bound, void* stream) {
  if (!ik && cache && cache->batch > 0 && T > 0) return CSA2_EINVAL;
  return quantize_append_impl(cache, kv, logits, ik, nullptr, T, host_len_bound, stream);
}

int csa2_quantize_append_proj(const csa2_cache* cache, const float* kv, const float* logits, const float* w_ik,
                              int32_t T, int32_t host_len_bound, void* stream) {
  if (!w_ik && cache && cache->batch > 0 && T > 0) return CSA2_EINVAL;
  return quantize_append_impl(cache, kv, logits, nullptr, w_ik, T, host_len_bound, stream);
}

int csa2_compress(const float* kv, const float* logits, int32_t B, int32_t T, int32_t ratio, float* out,
                  void* stream) {
  if (B < 0 || T < 0 || ratio < 1 || ratio > kMaxRatio || T % ratio != 0) return CSA2_EINVAL;
  if ((ratio >= 2) != (logits != nullptr)) return CSA2_EINVAL;
  if (B == 0 || T == 0) return CSA2_OK;
  if (!kv || !out || !aligned(kv, 4) || !aligned(out, 4) || (logits && !aligned(logits, 4))) return CSA2_EINVAL;
  const int rc = device_status(stream);
  if (rc != CSA2_OK) return rc;
  return from_hip(csa2::launch_compress(kv, logits, B, T, ratio, out, (hipStream_t)stream));
}

int csa2_swa_append(uint8_t* swa, int32_t S, const float* x, const int32_t* seq_len, int32_t B, int32_t T,
                    void* stream) {
  if (S < 1 || B < 0 || T < 0 || T > S) return CSA2_EINVAL;
  if (B == 0 || T == 0) return CSA2_OK;
  if (!swa || !x || !seq_len || !aligned(swa, 4) || !aligned(x, 16) || !aligned(seq_len, 4)) return CSA2_EINVAL;
  const int rc = device_status(stream);
  if (rc != CSA2_OK) return rc;
  return from_hip(csa2::launch_swa_append(swa, S, x, seq_len, B, T, (hipStream_t)stream));
}

int csa2_index_score_topk(const csa2_cache* cache, int mode, const float* iq, const float* iw, const int32_t* q_pos,
                          const int32_t* pool_in, int32_t* topk_out, int32_t* pool_out, int32_t Q, void* ws,
                          size_t ws_bytes, void* stream) {
  int rc = check_cache(cache, true, false);
  if (rc != CSA2_OK) return rc;
  if (Q < 0) return CSA2_EINVAL;
  if (mode == CSA2_FULL) {
    if (pool_in) return CSA2_EINVAL;
  } else if (mode == CSA2_REINDEX) {
    if (pool_out) return CSA2_EINVAL;
  } else {
    return CSA2_EINVAL;
  }
  if (cache->batch == 0 || Q == 0) return CSA2_OK;
  if (mode == CSA2_REINDEX && (!pool_in || !aligned(pool_in, 4))) return CSA2_EINVAL;
  if (!iq || !topk_out || !aligned(iq, 4) || !aligned(topk_out, 4)) return CSA2_EINVAL;
  if ((iw && !aligned(iw, 4)) || (q_pos && !aligned(q_pos, 4)) || (pool_out && !aligned(pool_out, 4)))
    return CSA2_EINVAL;
  const size_t need = csa2_workspace_bytes(CSA2_OP_INDEX, cache->batch, Q, cache->capacity);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA2_EWORKSPACE;
  if ((rc = device_status(stream)) != CSA2_OK) return rc;
  return from_hip(csa2::launch_index(to_launch(cache), mode, iq, iw, q_pos, pool_in, topk_out, pool_out, Q, ws,
                                     (hipStream_t)stream));
}

int csa2_append_index_score_topk(const csa2_cache* cache, const float* kv, const float* ik, int32_t T,
                                  int32_t host_len_bound, const float* iq, const float* iw, const int32_t* q_pos,
                                  int32_t* topk_out, int32_t* pool_out, int32_t Q, void* ws, size_t ws_bytes,
                                  void* stream) {
  // the append's checks (ratio 1: no logits), then the Full call's
  int rc = check_cache(cache, true, true);
  if (rc != CSA2_OK) return rc;
  if (cache->ratio != 1) return CSA2_EINVAL;
  if (T < 0 || host_len_bound < 0 || Q < 0) return CSA2_EINVAL;
  if ((int64_t)host_len_bound + T > cache->capacity) return CSA2_ECAPACITY;
  if (cache->batch == 0 || (T == 0 && Q == 0)) return CSA2_OK;
  if (T > 0 && (!kv || !ik || !aligned(kv, 16) || !aligned(ik, 4))) return CSA2_EINVAL;
  if (Q > 0) {
    if (!iq || !topk_out || !aligned(iq, 4) || !aligned(topk_out, 4)) return CSA2_EINVAL;
    if ((iw && !aligned(iw, 4)) || (q_pos && !aligned(q_pos, 4)) || (pool_out && !aligned(pool_out, 4)))
      return CSA2_EINVAL;
    const size_t need = csa2_workspace_bytes(CSA2_OP_INDEX, cache->batch, Q, cache->capacity);
    if (need > 0 && (!ws || ws_bytes < need)) return CSA2_EWORKSPACE;
  }
  if ((rc = device_status(stream)) != CSA2_OK) return rc;
  const csa2::LaunchCache c = to_launch(cache);
  if (Q == 0) return from_hip(csa2::launch_quant_append(c, kv, nullptr, ik, nullptr, T, (hipStream_t)stream));
  if (T == 0)
    return from_hip(csa2::launch_index(c, CSA2_FULL, iq, iw, q_pos, nullptr, topk_out, pool_out, Q, ws,
                                       (hipStream_t)stream));
  return from_hip(csa2::launch_append_index(c, kv, ik, T, iq, iw, q_pos, topk_out, pool_out, Q, ws,
                                            (hipStream_t)stream));
}

int csa2_sparse_attend(const csa2_cache* cache, const int32_t* topk, uint8_t* swa, int32_t S, const float* swa_x,
                       const int32_t* swa_len, int32_t swa_T, const uint16_t* q, const int32_t* q_pos, float sm_scale,
                       uint16_t* out, float* lse, int32_t Q, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_cache(cache, false, true);
  if (rc != CSA2_OK) return rc;
  if (Q < 0 || S < 1) return CSA2_EINVAL;
  if (swa_x ? (swa_T < 1 || swa_T > S || !swa_len) : (swa_T != 0 || swa_len)) return CSA2_EINVAL;
  if (cache->batch == 0) return CSA2_OK;
  if (swa_x && (!swa || !aligned(swa, 16) || !aligned(swa_x, 16) || !aligned(swa_len, 4))) return CSA2_EINVAL;
  if (Q == 0) {  // no query: only the window append, if any
    if (!swa_x) return CSA2_OK;
    if ((rc = device_status(stream)) != CSA2_OK) return rc;
    return from_hip(csa2::launch_swa_append(swa, S, swa_x, swa_len, cache->batch, swa_T, (hipStream_t)stream));
  }
  if (!topk || !swa || !q || !out) return CSA2_EINVAL;
  if (!aligned(topk, 16) || !aligned(swa, 16) || !aligned(q, 16) || !aligned(out, 16)) return CSA2_EINVAL;
  if ((lse && !aligned(lse, 4)) || (q_pos && !aligned(q_pos, 4))) return CSA2_EINVAL;
  const size_t need = csa2_workspace_bytes(CSA2_OP_ATTEND, cache->batch, Q, cache->capacity);
  if (need > 0 && (!ws || ws_bytes < need)) return CSA2_EWORKSPACE;
  if ((rc = device_status(stream)) != CSA2_OK) return rc;
  return from_hip(csa2::launch_attend(to_launch(cache), topk, swa, S, swa_x, swa_len, swa_T, q, q_pos, sm_scale, out,
                                      lse, Q, ws, (hipStream_t)stream));
}

int csa2_sparse_attend_noalloc(const csa2_cache* cache, const int32_t* topk, uint8_t* swa, int32_t S,
                               const float* swa_x, const int32_t* swa_len, int32_t swa_T, const uint16_t* q,
                               const int32_t* q_pos, float sm_scale, uint16_t* out, float* lse, int32_t Q,
                               void* stream) {
  // every host check first: a call that fails them touches no device
  int rc = check_cache(cache, false, true);
  if (rc != CSA2_OK) return rc;
  if (Q < 0 || S < 1) return CSA2_EINVAL;
  if (swa_x ? (swa_T < 1 || swa_T > S || !swa_len) : (swa_T != 0 || swa_len)) return CSA2_EINVAL;
  if (cache->batch == 0 || (Q == 0 && !swa_x)) return CSA2_OK;
  if (swa_x && (!swa || !aligned(swa, 16) || !aligned(swa_x, 16) || !aligned(swa_len, 4))) return CSA2_EINVAL;
  const size_t need = Q > 0 ? csa2_workspace_bytes(CSA2_OP_ATTEND, cache->batch, Q, cache->capacity) : 0;
  if (need > CSA2_NOALLOC_SCRATCH_BYTES) return CSA2_EWORKSPACE;
  void* ws = nullptr;
  if ((rc = device_scratch(stream, &ws)) != CSA2_OK) return rc;
  return csa2_sparse_attend(cache, topk, swa, S, swa_x, swa_len, swa_T, q, q_pos, sm_scale, out, lse, Q, ws,
                            CSA2_NOALLOC_SCRATCH_BYTES, stream);
}

size_t csa2_workspace_bytes(int op, int32_t B, int32_t Q, int32_t capacity) {
  if (B <= 0 || Q <= 0 || capacity < 0) return 0;
  const int64_t bq = (int64_t)B * Q;
  if (op == CSA2_OP_INDEX) return csa2::index_total_ws_bytes(bq, capacity);
  if (op == CSA2_OP_ATTEND) return csa2::attend_ws_bytes(bq);
  return 0;
}

const char* csa2_status_string(int status) {
  switch (status) {
    case CSA2_OK: return "ok";
    case CSA2_EINVAL: return "invalid argument";
    case CSA2_ECAPACITY: return "append exceeds cache capacity";
    case CSA2_EWORKSPACE: return "workspace missing or too small";
    case CSA2_EUNSUPPORTED: return "unsupported request";
    case CSA2_EHIP: return "HIP launch failed";
    case CSA2_EDEVICE: return "an earlier call found a device precondition violated (debug library)";
    default: return "unknown status";
  }
}

#ifdef CSA2_DEBUG
const char* csa2_version(void) { return "csa2-gfx950 0.1 debug"; }
#else
const char* csa2_version(void) { return "csa2-gfx950 0.1"; }
#endif

}  // extern "C"

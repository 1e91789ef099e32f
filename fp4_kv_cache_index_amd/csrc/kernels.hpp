// Launch entry points of the gfx950 kernels behind the C-ABI.  Host-side
// validation lives in csa2_abi.cpp; these functions only size grids and launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

struct LaunchCache {
  uint8_t* kv_codes;
  uint8_t* kv_scales;
  uint8_t* ik_codes;
  float* ik_scales;
  int32_t* length;
  int32_t batch;
  int32_t capacity;
  int32_t ratio;
};

// ---- indexer geometry
// entries per sequence at most: 2,048 shares of 8 batches of 512 keys, the most
// shares the select kernel takes
constexpr int64_t kMaxCapacity = 2048LL * 8 * 512;
constexpr int kTopK = 512;
constexpr int kPoolBlocks = 2048;
constexpr int kBlock = 8;
constexpr int kPool = kPoolBlocks * kBlock;

// workspace of an index call (index_head.hip's candidate stretches, counts,
// floors and cuts); nothing in it carries over between calls
size_t head_ws_bytes(int64_t bq, int32_t capacity);
int head_workgroups(bool reindex, int32_t capacity, int64_t bq);
size_t index_total_ws_bytes(int64_t bq, int32_t capacity);

// ---- attention geometry
constexpr int kAttnKeys = 640;  // 512 selected + 128 window
int attend_splits(int64_t bq);
size_t attend_ws_bytes(int64_t bq);

// ---- device precondition violations a debug build records (dev_check.hpp)
enum : uint32_t {
  kErrLength = 1u,       // length[b] above the capacity, or negative
  kErrEntryId = 2u,      // a Top-K id at or past the entries visible to its query
  kErrPoolId = 4u,       // a Reindex pool entry at or past the entries visible to its query
  kErrSeqLen = 8u,       // a window length smaller than the tokens appended
  kErrCapacity = 16u,    // an append that would pass the capacity (not made)
  kErrUnreadable = 1u << 31,  // the word itself could not be read or cleared
};
uint32_t take_append_dev_error(hipStream_t stream);
uint32_t take_attend_dev_error(hipStream_t stream);
uint32_t take_head_dev_error(hipStream_t stream);

hipError_t launch_quant_append(const LaunchCache& c, const float* kv, const float* logits, const float* ik,
                               const float* w_ik, int32_t T, hipStream_t stream);
hipError_t launch_swa_append(uint8_t* swa, int32_t S, const float* x, const int32_t* seq_len, int32_t B, int32_t T,
                             hipStream_t stream);
hipError_t launch_compress(const float* kv, const float* logits, int32_t B, int32_t T, int32_t ratio, float* out,
                           hipStream_t stream);
hipError_t launch_index(const LaunchCache& c, int mode, const float* iq, const float* iw, const int32_t* q_pos,
                        const int32_t* pool_in, int32_t* topk_out, int32_t* pool_out, int32_t Q, void* ws,
                        hipStream_t stream);
// One to three queries per sequence (Full) or Reindex: scoring with on-chip
// candidates, then the exact selection.  With app_T > 0 (Full, ratio 1, one
// query per sequence) the scoring launch first appends app_T new entries per
// sequence (app_kv [B][app_T][512], app_ik [B][app_T][64]) and the selection
// launch advances the lengths.
hipError_t launch_index_head(const LaunchCache& c, bool reindex, const float* iq, const float* iw,
                             const int32_t* q_pos, const int32_t* pool_in, int32_t* topk_out, int32_t* pool_out,
                             int32_t Q, const float* app_kv, const float* app_ik, int32_t app_T, void* ws_head,
                             hipStream_t stream);
// Full with four or more queries per sequence: the shared-load scoring with
// on-chip candidates (and, with pool_out, the pool's block maxima), then the
// same exact selection.
hipError_t launch_index_shared_heads(const LaunchCache& c, const float* iq, const float* iw, const int32_t* q_pos,
                                     int32_t* topk_out, int32_t* pool_out, int32_t Q, void* ws_head,
                                     hipStream_t stream);
constexpr int kMaxFusedAppend = 8;  // new entries per sequence an indexing launch appends itself
hipError_t launch_append_index(const LaunchCache& c, const float* kv, const float* ik, int32_t T, const float* iq,
                               const float* iw, const int32_t* q_pos, int32_t* topk_out, int32_t* pool_out,
                               int32_t Q, void* ws, hipStream_t stream);
hipError_t launch_attend(const LaunchCache& c, const int32_t* topk, uint8_t* swa, int32_t S, const float* swa_x,
                         const int32_t* swa_len, int32_t swa_T, const uint16_t* q, const int32_t* q_pos,
                         float sm_scale, uint16_t* out, float* lse, int32_t Q, void* ws, hipStream_t stream);

}  // namespace csa2

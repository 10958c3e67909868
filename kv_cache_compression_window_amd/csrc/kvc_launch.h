// Launchers of the gfx950 kernels (host functions defined in the .hip files).
// Arguments have been validated by the C-ABI layer before these are called.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "kvc_plan.h"

namespace kvc {

struct WsArgs {
  int bf16;  // 1: bfloat16 storage, 0: float32
  int B, H, Hkv, S, D, w;
  const void* q;
  const void* k;
  const uint8_t* valid;
  const int32_t* chan_idx;
  int d_keep;
  int reduce;  // 0 group, 1 all heads
  int causal;
  float* scores;
  void* ws;
};
hipError_t launch_window_scores(const WsArgs& a, const WsPlan& plan, hipStream_t st);

// Device address of the current device's fixed scratch (kNoAllocScratchBytes),
// looked up once per device (noalloc.hip).
hipError_t noalloc_scratch(void** ptr);

struct CsArgs {
  int bf16;
  int B, H, Hkv, S, D, w;
  const void* q;
  const void* k;
  float* out;
  void* ws;
};
hipError_t launch_channel_scores(const CsArgs& a, const CsPlan& plan, hipStream_t st);

hipError_t launch_topk(const float* scores, int rows, int n, int k, int n_tail, int32_t* idx, void* ws,
                       hipStream_t st);

struct GatherArgs {
  int bf16;
  int B, Hkv, S, D;
  const void* k;
  const void* v;
  const int32_t* idx;
  int n_keep;
  const int32_t* chan_idx;
  int d_keep;
  void* k_out;
  void* v_out;
};
hipError_t launch_gather(const GatherArgs& a, hipStream_t st);  // k may be NULL (V only)

// Row-wise channel gathers of ThinK's compressed key cache (channels.hip).
struct ChanRowsArgs {
  int esz;              // element bytes: 2 (bf16) or 4 (f32)
  int groups;           // (b, KV head) pairs, or (b, query head) pairs when H > 0
  int H, Hkv;           // H > 0: group g is query head g % H of batch g / H and uses its KV head's channels
  const void* in;
  void* out;
  const int32_t* idx;   // [groups][n_rows] source rows, or NULL (output row r reads input row r)
  const int32_t* chan;  // [channel rows][d_keep]
  int n_rows, in_rows;  // output rows and input rows per group
  int in_ch, out_ch;    // channels per input and per output row
  int d_keep;
  int expand;           // 0: out[j] = in[chan[j]];  1: out[chan[j]] = in[j], other channels +0.0
};
hipError_t launch_chan_rows(const ChanRowsArgs& a, hipStream_t st);

struct ScissorArgs {
  int B, Hkv, C, hist_len;
  int64_t step;
  const float* probs;
  uint8_t* valid;
  uint32_t* hist;
  uint16_t* counts;
  const int64_t* since;  // [B, Hkv, C] recordings before each slot's token, or NULL (all 0)
  float* frac_out;
  const int32_t* evict_idx;
  int n_evict;
};
hipError_t launch_scissor(const ScissorArgs& a, hipStream_t st);

// Scissorhands with insertion: the eviction queue's refill and the insertion.
struct ScissorRefillArgs {
  int B, Hkv, C, hist_len;
  long long step;
  const uint8_t* valid;
  const uint16_t* counts;
  const int64_t* since;  // or NULL (all 0)
  int n_protect, m;
  float* frac;    // [B*Hkv*C] workspace
  void* topk_ws;  // top-k workspace
  int32_t* queue; // [B, Hkv, m] out
};
hipError_t launch_scissor_refill(const ScissorRefillArgs& a, hipStream_t st);

struct ScissorInsertArgs {
  int B, Hkv, C, hist_len, row_bytes;
  const int32_t* queue;  // [B, Hkv, m] or NULL (fill_pos for every row)
  int m, j, fill_pos;
  const void* k_new;     // [B, Hkv, D]
  const void* v_new;     // [B, Hkv, D] or NULL
  void* k_cache;         // [B, Hkv, C, D]
  void* v_cache;
  uint8_t* valid;
  uint32_t* hist;
  uint16_t* counts;
  long long rec;    // recordings made before the new token
  int64_t* since;   // [B, Hkv, C]
};
hipError_t launch_scissor_insert(const ScissorInsertArgs& a, hipStream_t st);

}  // namespace kvc

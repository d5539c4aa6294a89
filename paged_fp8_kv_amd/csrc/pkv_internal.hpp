// Internal launch interfaces between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kHeadDimSupported = 64;   // the only head size the kernels are built for
constexpr int kMaxWorkers = 4096;          // waves of one attention launch (16 per CU on 256 CUs)
// 32-token sub-tiles per worker at least: smaller shares only add partials
// (an 8-sequence batch of 1024-4096 tokens, full-attention launch: 18.7-18.9 us
// with 10, 18.1-18.3 us with 12, 18.3-18.6 us with 14, 18.5-18.8 us with 16,
// 20.0 us with 20, 20.8 us with 24)
constexpr int kMinSubtilesPerWorker = 12;
constexpr int kMaxBatch = 8192;            // per-sequence prefix scan lives in LDS

struct AttnLaunch {
  const uint16_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const int32_t* table;
  const int32_t* frame_pos;
  uint16_t* out;
  void* workspace;
  int64_t nb;
  int32_t B, Hq, Hkv, block;
  int32_t bt_stride, table_width, window;
  float k_scale, v_scale, sm_scale;
  int32_t n_workers;
  int32_t k_packed;  // 1: K half in the packed (token-pair interleaved) arrangement
  // Optional write of each sequence's new token (null k_new: none).  The new
  // token sits at the sequence's frame position; its K/V rows
  // (bf16 [B, Hkv, 64]) are quantised with k_scale / v_scale, stored in the
  // slot the table gives for that position, and attended from registers.
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint8_t* k_w;
  uint8_t* v_w;
  // Write slots of the fused write (int64 [B], block_id*block + offset): -1
  // skips the write; any other value must be the slot the table gives for
  // the frame position, else the row is NaN and nothing is written.
  const int64_t* upd;
  // Optional rotary cos/sin, fp32 [B, 32] (null: no rotation): every query
  // head, and the new K before it is quantised, are turned half-split.
  const float* rope_cos;
  const float* rope_sin;
};

int attn_max_subtiles(int block, int table_width, int window);
int attn_workers(int64_t batch, int kv_heads, int max_subtiles);
int64_t attn_workspace_bytes(int64_t batch, int kv_heads, int n_workers);
hipError_t launch_decode_attn(const AttnLaunch& L, hipStream_t stream);

// Bytes of the library's own device workspace (one per GPU), used by
// launch_decode_attn_scratch in place of L.workspace: launches needing more
// are refused.  attn_scratch gives the current device's copy.
constexpr int64_t kScratchBytes = int64_t{24} << 20;
hipError_t attn_scratch(void** ptr);
hipError_t launch_decode_attn_scratch(const AttnLaunch& L, hipStream_t stream);

struct SetupLaunch {
  int32_t B, block, window;
  int32_t anchor_lag;  // 0, or 1: the window frame is anchored at p - 1
  const int32_t* seq_lens;
  const uint8_t* active;
  const int64_t* positions;
  const int32_t* bt_full;
  int32_t bt_full_stride;
  const int32_t* bt_swa;
  int32_t bt_swa_stride, bt_width;
  int32_t* pos_full;
  int32_t* pos_swa;
  int32_t* trim;
  int32_t trim_width;
  int64_t* upd_full;
  int64_t* upd_swa;
  int64_t* pos_abs;
};
hipError_t launch_setup(const SetupLaunch& L, hipStream_t stream);

// Compressed page lists for launch_setup_csr; the padded full table and the
// token counts are outputs (SetupLaunch::bt_full / seq_lens unused).
struct CsrInput {
  const int32_t* kv_indptr;      // [B + 1]
  const int32_t* full_indices;
  const int32_t* swa_indices;    // null when window == 0
  const int32_t* last_page_len;  // [B]
  int32_t* bt_full_out;          // [B, bt_full_stride]
  int32_t* seq_lens_out;         // [B]
};
hipError_t launch_setup_csr(const SetupLaunch& L, const CsrInput& C, hipStream_t stream);

struct UpdateLaunch {
  int32_t B, Hkv, block;
  int64_t nb;
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint8_t* k;
  uint8_t* v;
  int32_t k_packed;
  const int64_t* slot;
  float k_scale, v_scale;
  const float* rope_cos;  // fp32 [B, 32] or null: K rotated before quantising
  const float* rope_sin;
};
hipError_t launch_kv_update(const UpdateLaunch& L, hipStream_t stream);

}  // namespace pkv

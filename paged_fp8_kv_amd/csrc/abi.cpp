// C ABI of libpkv: host-side argument checks, error text and dispatch to the
// gfx950 kernels.  Declarations and the meaning of every argument are in
// include/pkv.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/pkv.h"
#include "pkv_internal.hpp"

namespace {

thread_local std::string g_err;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return status;
}

int ok() {
  g_err.clear();
  return PKV_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool block_supported(int block) {
  return block == 16 || block == 32 || block == 64 || block == 128;
}

// shape checks shared by update and attention
int check_kv_shape(int32_t kv_heads, int32_t head_dim, int32_t block, int64_t num_blocks) {
  if (kv_heads < 1) return fail(PKV_ERR_ARG, "kv_heads must be >= 1 (got %d)", kv_heads);
  if (num_blocks < 1) return fail(PKV_ERR_ARG, "num_blocks must be >= 1 (got %lld)", (long long)num_blocks);
  if (head_dim != pkv::kHeadDimSupported)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d unsupported (only 64)", head_dim);
  if (!block_supported(block))
    return fail(PKV_ERR_UNSUPPORTED, "block %d unsupported (16, 32, 64 or 128)", block);
  // half bytes must fit int64
  if (num_blocks > (INT64_MAX / 2) / (static_cast<int64_t>(kv_heads) * block * head_dim))
    return fail(PKV_ERR_ARG, "buffer size overflows int64");
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_last_error(void) { return g_err.c_str(); }

int pkv_kv_buffer_bytes(int64_t num_blocks, int32_t kv_heads, int32_t block, int32_t head_dim,
                        int64_t* half_bytes, int64_t* total_bytes) {
  if (!half_bytes || !total_bytes) return fail(PKV_ERR_ARG, "null output pointer");
  if (num_blocks < 0 || kv_heads < 1 || block < 1 || head_dim < 1)
    return fail(PKV_ERR_ARG, "sizes must be positive");
  const int64_t per = static_cast<int64_t>(kv_heads) * block * head_dim;
  if (num_blocks > (INT64_MAX / 2) / per) return fail(PKV_ERR_ARG, "buffer size overflows int64");
  *half_bytes = num_blocks * per;
  *total_bytes = 2 * num_blocks * per;
  return ok();
}

int pkv_kv_budget(int64_t total_hbm_bytes, int64_t bytes_used, double gmu, double cap_fraction,
                  double min_kv_gib, int64_t* available_bytes) {
  if (!available_bytes) return fail(PKV_ERR_ARG, "null output pointer");
  if (total_hbm_bytes < 0 || bytes_used < 0 || total_hbm_bytes > (int64_t{1} << 52))
    return fail(PKV_ERR_ARG, "byte counts must be in [0, 2^52]");
  if (!(gmu >= 0.0 && gmu <= 1.0) || !(cap_fraction >= 0.0 && cap_fraction <= 1.0) ||
      !(min_kv_gib >= 0.0 && min_kv_gib < 1e9))
    return fail(PKV_ERR_ARG, "gmu and cap_fraction must be in [0, 1], min_kv_gib >= 0");
  // The engine's share of the device, and the resident bytes taken out of
  // it, clamped into [0, cap * share].  int(x) of a double truncates toward
  // zero; byte counts below 2^53 convert exactly.
  const int64_t share = static_cast<int64_t>(static_cast<double>(total_hbm_bytes) * gmu);
  const int64_t cap = static_cast<int64_t>(static_cast<double>(share) * cap_fraction);
  const int64_t available = std::clamp<int64_t>(share - bytes_used, 0, cap);
  *available_bytes = available;
  if (static_cast<double>(available) < min_kv_gib * 1073741824.0)
    return fail(PKV_ERR_DATA, "KV budget of %lld bytes is below the minimum of %g GiB",
                static_cast<long long>(available), min_kv_gib);
  return ok();
}

int pkv_kv_num_blocks(int64_t available_bytes, int32_t n_buffers, int32_t kv_heads, int32_t block,
                      int32_t head_dim, int64_t* num_blocks) {
  if (!num_blocks) return fail(PKV_ERR_ARG, "null output pointer");
  if (available_bytes < 0 || n_buffers < 1 || kv_heads < 1 || block < 1 || head_dim < 1)
    return fail(PKV_ERR_ARG, "sizes must be positive");
  const int64_t per = int64_t{2} * n_buffers * kv_heads * block * head_dim;
  const int64_t n = available_bytes / per;
  *num_blocks = std::min<int64_t>(n, INT32_MAX);  // block ids are int32
  return ok();
}

int pkv_trimmed_width(int32_t window, int32_t block, int32_t anchor_lag) {
  if (window < 1 || block < 1) return fail(PKV_ERR_ARG, "window and block must be >= 1");
  if (anchor_lag != 0 && anchor_lag != 1) return fail(PKV_ERR_ARG, "anchor_lag must be 0 or 1");
  if (window > INT32_MAX / 2) return fail(PKV_ERR_ARG, "window too large");
  g_err.clear();
  return (window - 1 + anchor_lag + block - 1) / block + 1;
}

int pkv_setup_attn_control(int32_t batch, int32_t block, int32_t window, int32_t anchor_lag,
                           const int32_t* seq_lens,
                           const uint8_t* active, const int64_t* positions, const int32_t* bt_full,
                           int32_t bt_full_stride, const int32_t* bt_swa, int32_t bt_swa_stride,
                           int32_t bt_width, int32_t* pos_full, int32_t* pos_swa,
                           int32_t* bt_swa_trim, int32_t trim_width, int64_t* upd_full,
                           int64_t* upd_swa, int64_t* pos_abs, void* stream) {
  if (batch < 0) return fail(PKV_ERR_ARG, "batch must be >= 0");
  if (batch == 0) return ok();
  if (block < 1 || block % 2) return fail(PKV_ERR_ARG, "block must be a positive even number");
  if (window < 0) return fail(PKV_ERR_ARG, "window must be >= 0");
  if (bt_width < 1 || bt_full_stride < bt_width)
    return fail(PKV_ERR_ARG, "need 1 <= bt_width <= bt_full_stride");
  if (!seq_lens || !active || !bt_full || !pos_full || !upd_full)
    return fail(PKV_ERR_ARG, "null device pointer");
  if (anchor_lag != 0 && anchor_lag != 1) return fail(PKV_ERR_ARG, "anchor_lag must be 0 or 1");
  if (window > 0) {
    if (!bt_swa || !pos_swa || !bt_swa_trim || !upd_swa)
      return fail(PKV_ERR_ARG, "window > 0 needs bt_swa, pos_swa, bt_swa_trim and upd_swa");
    if (bt_swa_stride < bt_width) return fail(PKV_ERR_ARG, "bt_swa_stride < bt_width");
    const int need = pkv_trimmed_width(window, block, anchor_lag);
    if (need < 0) return need;
    if (trim_width != need)
      return fail(PKV_ERR_ARG, "trim_width must be %d for window %d, block %d, lag %d (got %d)",
                  need, window, block, anchor_lag, trim_width);
  }
  pkv::SetupLaunch L{};
  L.B = batch;
  L.block = block;
  L.window = window;
  L.anchor_lag = anchor_lag;
  L.seq_lens = seq_lens;
  L.active = active;
  L.positions = positions;
  L.bt_full = bt_full;
  L.bt_full_stride = bt_full_stride;
  L.bt_swa = bt_swa;
  L.bt_swa_stride = bt_swa_stride;
  L.bt_width = bt_width;
  L.pos_full = pos_full;
  L.pos_swa = pos_swa;
  L.trim = window > 0 ? bt_swa_trim : nullptr;
  L.trim_width = window > 0 ? trim_width : 0;
  L.upd_full = upd_full;
  L.upd_swa = upd_swa;
  L.pos_abs = pos_abs;
  return hip_status(pkv::launch_setup(L, static_cast<hipStream_t>(stream)), "setup launch");
}

int pkv_setup_attn_control_csr(int32_t batch, int32_t block, int32_t window,
                               int32_t anchor_lag, const int32_t* kv_indptr, const int32_t* full_indices,
                               const int32_t* swa_indices, const int32_t* last_page_len,
                               const uint8_t* active, const int64_t* positions, int32_t* bt_full,
                               int32_t bt_stride, int32_t bt_width, int32_t* seq_lens,
                               int32_t* pos_full, int32_t* pos_swa, int32_t* bt_swa_trim,
                               int32_t trim_width, int64_t* upd_full, int64_t* upd_swa,
                               int64_t* pos_abs, void* stream) {
  if (batch < 0) return fail(PKV_ERR_ARG, "batch must be >= 0");
  if (batch == 0) return ok();
  if (batch > INT32_MAX / 2) return fail(PKV_ERR_ARG, "batch too large");
  if (block < 1 || block % 2) return fail(PKV_ERR_ARG, "block must be a positive even number");
  if (window < 0) return fail(PKV_ERR_ARG, "window must be >= 0");
  if (bt_width < 1 || bt_stride < bt_width) return fail(PKV_ERR_ARG, "need 1 <= bt_width <= bt_stride");
  if (!kv_indptr || !full_indices || !last_page_len || !active || !bt_full || !seq_lens ||
      !pos_full || !upd_full)
    return fail(PKV_ERR_ARG, "null device pointer");
  if (anchor_lag != 0 && anchor_lag != 1) return fail(PKV_ERR_ARG, "anchor_lag must be 0 or 1");
  if (window > 0) {
    if (!swa_indices || !pos_swa || !bt_swa_trim || !upd_swa)
      return fail(PKV_ERR_ARG, "window > 0 needs swa_indices, pos_swa, bt_swa_trim and upd_swa");
    const int need = pkv_trimmed_width(window, block, anchor_lag);
    if (need < 0) return need;
    if (trim_width != need)
      return fail(PKV_ERR_ARG, "trim_width must be %d for window %d, block %d, lag %d (got %d)",
                  need, window, block, anchor_lag, trim_width);
  }
  pkv::SetupLaunch L{};
  L.B = batch;
  L.block = block;
  L.window = window;
  L.anchor_lag = anchor_lag;
  L.active = active;
  L.positions = positions;
  L.bt_full_stride = bt_stride;
  L.bt_width = bt_width;
  L.pos_full = pos_full;
  L.pos_swa = pos_swa;
  L.trim = window > 0 ? bt_swa_trim : nullptr;
  L.trim_width = window > 0 ? trim_width : 0;
  L.upd_full = upd_full;
  L.upd_swa = upd_swa;
  L.pos_abs = pos_abs;
  pkv::CsrInput C{};
  C.kv_indptr = kv_indptr;
  C.full_indices = full_indices;
  C.swa_indices = window > 0 ? swa_indices : nullptr;
  C.last_page_len = last_page_len;
  C.bt_full_out = bt_full;
  C.seq_lens_out = seq_lens;
  return hip_status(pkv::launch_setup_csr(L, C, static_cast<hipStream_t>(stream)), "setup launch");
}

int pkv_kv_cache_update(int32_t batch, int32_t kv_heads, int32_t head_dim, int32_t block,
                        int64_t num_blocks, const uint16_t* k_new, const uint16_t* v_new,
                        uint8_t* k_half, int32_t k_packed, uint8_t* v_half,
                        const int64_t* slot_idx, const float* rope_cos, const float* rope_sin,
                        float k_scale, float v_scale, void* stream) {
  if (batch < 0) return fail(PKV_ERR_ARG, "batch must be >= 0");
  if (batch == 0) return ok();
  int st = check_kv_shape(kv_heads, head_dim, block, num_blocks);
  if (st) return st;
  if (!k_new || !v_new || !k_half || !v_half || !slot_idx)
    return fail(PKV_ERR_ARG, "null device pointer");
  if (!aligned(k_half, 16) || !aligned(v_half, 16))
    return fail(PKV_ERR_ARG, "K/V halves must be 16-byte aligned");
  if (k_packed != 0 && k_packed != 1) return fail(PKV_ERR_ARG, "k_packed must be 0 or 1");
  if ((rope_cos == nullptr) != (rope_sin == nullptr))
    return fail(PKV_ERR_ARG, "rope_cos and rope_sin must both be given or both be null");
  if (rope_cos && (!aligned(rope_cos, 4) || !aligned(rope_sin, 4)))
    return fail(PKV_ERR_ARG, "rope_cos / rope_sin must be 4-byte aligned");
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || k_scale == INFINITY || v_scale == INFINITY)
    return fail(PKV_ERR_ARG, "scales must be finite and > 0");
  pkv::UpdateLaunch L{};
  L.B = batch;
  L.Hkv = kv_heads;
  L.block = block;
  L.nb = num_blocks;
  L.k_new = k_new;
  L.v_new = v_new;
  L.k = k_half;
  L.v = v_half;
  L.k_packed = k_packed;
  L.slot = slot_idx;
  L.k_scale = k_scale;
  L.v_scale = v_scale;
  L.rope_cos = rope_cos;
  L.rope_sin = rope_sin;
  return hip_status(pkv::launch_kv_update(L, static_cast<hipStream_t>(stream)), "kv update launch");
}

int64_t pkv_decode_workspace_bytes(int32_t batch, int32_t q_heads, int32_t kv_heads,
                                   int32_t head_dim, int32_t block, int32_t table_width,
                                   int32_t window) {
  if (batch < 0 || q_heads < 1 || kv_heads < 1 || table_width < 1 || window < 0)
    return fail(PKV_ERR_ARG, "bad sizes");
  if (head_dim != pkv::kHeadDimSupported) return fail(PKV_ERR_UNSUPPORTED, "head_dim must be 64");
  if (!block_supported(block)) return fail(PKV_ERR_UNSUPPORTED, "unsupported block");
  g_err.clear();
  if (batch == 0) return 0;
  const int ms = pkv::attn_max_subtiles(block, table_width, window);
  const int w = pkv::attn_workers(batch, kv_heads, ms);
  return pkv::attn_workspace_bytes(batch, kv_heads, w);
}

// Attention, optionally with the fused write of each sequence's new token
// (k_new / v_new rows into the writable halves k_w / v_w; see pkv_decode_layer).
static int attn_impl(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                     int32_t block, int64_t num_blocks, int32_t window, const uint16_t* q,
                     const uint8_t* k_half, int32_t k_packed, const uint8_t* v_half,
                     const int32_t* block_table, int32_t bt_stride, int32_t table_width,
                     const int32_t* frame_pos, float k_scale, float v_scale, float sm_scale,
                     uint16_t* out, void* workspace, int64_t workspace_bytes, void* stream,
                     const uint16_t* k_new, const uint16_t* v_new, uint8_t* k_w, uint8_t* v_w,
                     const int64_t* upd, const float* rope_cos, const float* rope_sin,
                     bool use_scratch = false) {
  if (batch < 0) return fail(PKV_ERR_ARG, "batch must be >= 0");
  if (batch == 0) return ok();
  if (batch > pkv::kMaxBatch)
    return fail(PKV_ERR_UNSUPPORTED, "batch %d above the supported %d", batch, pkv::kMaxBatch);
  int st = check_kv_shape(kv_heads, head_dim, block, num_blocks);
  if (st) return st;
  if (q_heads < 1 || q_heads % kv_heads)
    return fail(PKV_ERR_ARG, "q_heads (%d) must be a positive multiple of kv_heads (%d)", q_heads,
                kv_heads);
  if (q_heads / kv_heads > 8)
    return fail(PKV_ERR_UNSUPPORTED, "query group of %d heads above 8", q_heads / kv_heads);
  if (window < 0) return fail(PKV_ERR_ARG, "window must be >= 0");
  if (table_width < 1 || bt_stride < table_width)
    return fail(PKV_ERR_ARG, "need 1 <= table_width <= bt_stride");
  if (static_cast<int64_t>(table_width) * block > INT32_MAX / 2)
    return fail(PKV_ERR_UNSUPPORTED, "table covers too many tokens");
  if (!q || !k_half || !v_half || !block_table || !frame_pos || !out)
    return fail(PKV_ERR_ARG, "null device pointer");
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_half, 16) || !aligned(v_half, 16))
    return fail(PKV_ERR_ARG, "q, out and the K/V halves must be 16-byte aligned");
  if (!aligned(block_table, 4) || !aligned(frame_pos, 4))
    return fail(PKV_ERR_ARG, "tables must be 4-byte aligned");
  if (k_packed != 0 && k_packed != 1) return fail(PKV_ERR_ARG, "k_packed must be 0 or 1");
  if ((rope_cos == nullptr) != (rope_sin == nullptr))
    return fail(PKV_ERR_ARG, "rope_cos and rope_sin must both be given or both be null");
  if (rope_cos && (!aligned(rope_cos, 16) || !aligned(rope_sin, 16)))
    return fail(PKV_ERR_ARG, "rope_cos / rope_sin must be 16-byte aligned");
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || !(sm_scale > 0.f) || k_scale == INFINITY ||
      v_scale == INFINITY || sm_scale == INFINITY)
    return fail(PKV_ERR_ARG, "scales must be finite and > 0");
  {
    // the kernel scales scores by this product (log2 domain): it must be a
    // finite positive float for the softmax to be defined
    const float ss = sm_scale * k_scale * 1.4426950408889634f;
    if (!(ss > 0.f) || ss == INFINITY)
      return fail(PKV_ERR_ARG, "sm_scale * k_scale must be a finite positive float");
  }
  const int ms = pkv::attn_max_subtiles(block, table_width, window);
  const int w = pkv::attn_workers(batch, kv_heads, ms);
  const int64_t need = pkv::attn_workspace_bytes(batch, kv_heads, w);
  if (use_scratch) {
    if (need > pkv::kScratchBytes)
      return fail(PKV_ERR_WORKSPACE,
                  "these shapes need %lld bytes of workspace; the library's own holds %lld",
                  (long long)need, (long long)pkv::kScratchBytes);
  } else {
    if (!workspace || workspace_bytes < need)
      return fail(PKV_ERR_WORKSPACE, "workspace of %lld bytes needed (got %lld)", (long long)need,
                  (long long)workspace_bytes);
    if (!aligned(workspace, 256)) return fail(PKV_ERR_ARG, "workspace must be 256-byte aligned");
  }
  pkv::AttnLaunch L{};
  L.q = q;
  L.k = k_half;
  L.v = v_half;
  L.table = block_table;
  L.frame_pos = frame_pos;
  L.out = out;
  L.workspace = workspace;
  L.nb = num_blocks;
  L.B = batch;
  L.Hq = q_heads;
  L.Hkv = kv_heads;
  L.block = block;
  L.bt_stride = bt_stride;
  L.table_width = table_width;
  L.window = window;
  L.k_scale = k_scale;
  L.v_scale = v_scale;
  L.sm_scale = sm_scale;
  L.n_workers = w;
  L.k_packed = k_packed;
  L.k_new = k_new;
  L.v_new = v_new;
  L.k_w = k_w;
  L.v_w = v_w;
  L.upd = upd;
  L.rope_cos = rope_cos;
  L.rope_sin = rope_sin;
  if (use_scratch)
    return hip_status(pkv::launch_decode_attn_scratch(L, static_cast<hipStream_t>(stream)),
                      "attention launch");
  return hip_status(pkv::launch_decode_attn(L, static_cast<hipStream_t>(stream)), "attention launch");
}

int pkv_paged_decode_attn(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                          int32_t block, int64_t num_blocks, int32_t window, const uint16_t* q,
                          const uint8_t* k_half, int32_t k_packed, const uint8_t* v_half,
                          const int32_t* block_table, int32_t bt_stride, int32_t table_width,
                          const int32_t* frame_pos, const float* rope_cos,
                          const float* rope_sin, float k_scale, float v_scale, float sm_scale,
                          uint16_t* out, void* workspace, int64_t workspace_bytes, void* stream) {
  return attn_impl(batch, q_heads, kv_heads, head_dim, block, num_blocks, window, q, k_half,
                   k_packed, v_half, block_table, bt_stride, table_width, frame_pos, k_scale,
                   v_scale, sm_scale, out, workspace, workspace_bytes, stream, nullptr, nullptr,
                   nullptr, nullptr, nullptr, rope_cos, rope_sin);
}

static int decode_layer_impl(const pkv_step* s, int32_t layer, const uint16_t* q,
                             const uint16_t* k_new, const uint16_t* v_new, float k_scale,
                             float v_scale, float sm_scale, uint16_t* out, void* workspace,
                             int64_t workspace_bytes, void* stream, bool use_scratch) {
  if (!s) return fail(PKV_ERR_ARG, "null step");
  if (layer < 0 || layer / 2 >= s->n_buffers)
    return fail(PKV_ERR_ARG, "layer %d has no buffer (n_buffers %d)", layer, s->n_buffers);
  const bool per_buffer = s->k_bufs != nullptr || s->v_bufs != nullptr;
  const bool stacked = s->stacked != nullptr;
  if (per_buffer == stacked)
    return fail(PKV_ERR_ARG, "exactly one KV form (per-buffer or stacked) must be given");
  int64_t half = 0, total = 0;
  int st = pkv_kv_buffer_bytes(s->num_blocks, s->kv_heads, s->block, s->head_dim, &half, &total);
  if (st) return st;
  uint8_t* kh;
  uint8_t* vh;
  const int j = layer / 2;
  if (per_buffer) {
    if (!s->k_bufs || !s->v_bufs) return fail(PKV_ERR_ARG, "per-buffer form needs k_bufs and v_bufs");
    kh = s->k_bufs[j];
    vh = s->v_bufs[j];
  } else {
    kh = s->stacked + static_cast<int64_t>(j) * total;
    vh = kh + half;
  }
  const bool swa = (layer % 2) == 0;
  if (swa && s->window < 1) return fail(PKV_ERR_ARG, "even layers need window >= 1");
  // One launch: the attention writes each sequence's new token itself
  // through the layer's update index (upd_swa / upd_full) and attends to it
  // from registers.
  if (!k_new || !v_new) return fail(PKV_ERR_ARG, "null k_new / v_new");
  if (!aligned(k_new, 2) || !aligned(v_new, 2)) return fail(PKV_ERR_ARG, "k_new / v_new must be 2-byte aligned");
  const int64_t* upd = swa ? s->upd_swa : s->upd_full;
  if (!upd) return fail(PKV_ERR_ARG, "the step needs upd_swa and upd_full");
  if (!aligned(upd, 8)) return fail(PKV_ERR_ARG, "update indices must be 8-byte aligned");
  if (swa)
    return attn_impl(s->batch, s->q_heads, s->kv_heads, s->head_dim, s->block, s->num_blocks,
                     s->window, q, kh, s->k_packed, vh, s->bt_swa_trim, s->trim_width,
                     s->trim_width, s->pos_swa, k_scale, v_scale, sm_scale, out, workspace,
                     workspace_bytes, stream, k_new, v_new, kh, vh, upd, s->rope_cos, s->rope_sin,
                     use_scratch);
  return attn_impl(s->batch, s->q_heads, s->kv_heads, s->head_dim, s->block, s->num_blocks, 0, q,
                   kh, s->k_packed, vh, s->bt_full, s->bt_full_stride, s->bt_full_width,
                   s->pos_full, k_scale, v_scale, sm_scale, out, workspace, workspace_bytes, stream,
                   k_new, v_new, kh, vh, upd, s->rope_cos, s->rope_sin, use_scratch);
}

int pkv_decode_layer(const pkv_step* s, int32_t layer, const uint16_t* q, const uint16_t* k_new,
                     const uint16_t* v_new, float k_scale, float v_scale, float sm_scale,
                     uint16_t* out, void* workspace, int64_t workspace_bytes, void* stream) {
  return decode_layer_impl(s, layer, q, k_new, v_new, k_scale, v_scale, sm_scale, out, workspace,
                           workspace_bytes, stream, false);
}

int pkv_decode_layer_noalloc(const pkv_step* s, int32_t layer, const uint16_t* q,
                             const uint16_t* k_new, const uint16_t* v_new, float k_scale,
                             float v_scale, float sm_scale, uint16_t* out, void* stream) {
  return decode_layer_impl(s, layer, q, k_new, v_new, k_scale, v_scale, sm_scale, out, nullptr, 0,
                           stream, true);
}

int pkv_validate_attn_control(int32_t batch, int32_t block, int32_t window, int64_t num_blocks,
                              const int32_t* seq_lens, const uint8_t* active,
                              const int32_t* bt_full, int32_t bt_full_stride,
                              const int32_t* bt_swa, int32_t bt_swa_stride, int32_t bt_width,
                              void* stream) {
  if (batch < 0 || block < 1 || window < 0 || num_blocks < 1 || bt_width < 1 ||
      bt_full_stride < bt_width)
    return fail(PKV_ERR_ARG, "bad sizes");
  if (batch == 0) return ok();
  if (!seq_lens || !active || !bt_full || (window > 0 && (!bt_swa || bt_swa_stride < bt_width)))
    return fail(PKV_ERR_ARG, "null pointer or bad stride");
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<int32_t> len(batch), full(static_cast<size_t>(batch) * bt_full_stride);
  std::vector<uint8_t> act(batch);
  std::vector<int32_t> swa(window > 0 ? static_cast<size_t>(batch) * bt_swa_stride : 0);
  hipError_t e = hipMemcpyAsync(len.data(), seq_lens, batch * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(act.data(), active, batch, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(full.data(), bt_full, full.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && window > 0)
    e = hipMemcpyAsync(swa.data(), bt_swa, swa.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_status(e, "validate copy");
  std::vector<uint8_t> owner(static_cast<size_t>(num_blocks), 0);  // 1 full, 2 window
  for (int b = 0; b < batch; ++b) {
    if (!act[b] || len[b] <= 0) continue;
    const int p = len[b] - 1, cp = p / block;
    if (cp >= bt_width)
      return fail(PKV_ERR_DATA, "sequence %d: token %d needs column %d >= bt_width %d", b, p, cp,
                  bt_width);
    for (int c = 0; c <= cp; ++c) {
      const int id = full[static_cast<size_t>(b) * bt_full_stride + c];
      if (id < 0 || id >= num_blocks)
        return fail(PKV_ERR_DATA, "full table (%d, %d): block id %d outside [0, %lld)", b, c, id,
                    (long long)num_blocks);
      if (owner[id] == 2)
        return fail(PKV_ERR_DATA, "full table (%d, %d): block %d is also a window block", b, c, id);
      owner[id] = 1;
    }
  }
  if (window > 0) {
    for (int b = 0; b < batch; ++b) {
      if (!act[b] || len[b] <= 0) continue;
      const int p = len[b] - 1, cp = p / block;
      const int first = std::max(0, p - window + 1) / block;
      for (int c = first; c <= cp; ++c) {
        const int id = swa[static_cast<size_t>(b) * bt_swa_stride + c];
        if (id < 0 || id >= num_blocks)
          return fail(PKV_ERR_DATA, "window table (%d, %d): block id %d outside [0, %lld)", b, c,
                      id, (long long)num_blocks);
        if (owner[id] == 1)
          return fail(PKV_ERR_DATA, "window table (%d, %d): block %d is also a full block", b, c,
                      id);
        owner[id] = 2;
      }
    }
  }
  return ok();
}

}  // extern "C"

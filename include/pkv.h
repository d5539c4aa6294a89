/*
 * pkv.h -- C ABI of libpkv: one decode step of paged attention over a
 * packed-FP8 KV cache on AMD Instinct MI355X (gfx950).
 *
 * What the calls compute is defined on the page "GPT-OSS-120B giga-kernel
 * decode" (AWS Neuron vllm-neuron design documentation):
 *   - section "Kernel contract": the layer-invariant attention control (a full
 *     block table, a trimmed sliding-window table, the active mask, absolute
 *     and window-frame positions, two KV-update indices), the alternating
 *     sliding-window (window 128, even layers) / full (odd layers) schedule,
 *     buffer i/2 for layer i, and the rule that exactly one KV form is given;
 *   - section "KV-cache layout (per-buffer, HMA-preserving)": one allocation
 *     [2, num_blocks, kv_heads, block, head_dim] per shared buffer, K half then
 *     V half, 1 byte per element, K optionally stored through the packed view
 *     [..., block/2, head_dim, 2] (token pairs interleaved per dimension), V
 *     never packed, and per-buffer base-0 addressing.
 * The FP8 element type is OCP E4M3 ("e4m3fn") with one per-tensor
 * dequantisation multiplier for K and one for V.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns all
 *     memory; the library allocates nothing and keeps no pointer after a call
 *     returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     device work is enqueued asynchronously on it; no call synchronises
 *     except pkv_validate_attn_control.
 *   - bf16 tensors are passed as uint16_t bit patterns.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     failure nothing is enqueued, a negative pkv_status is returned and
 *     pkv_last_error() describes it (thread-local text).
 *   - Table contents live on the device and are not checked on the fast path.
 *     The kernels never touch memory outside the buffers they are given: a
 *     block id outside [0, num_blocks) or a position beyond the table makes the
 *     affected output rows NaN (attention) or skips the write (update).
 *     pkv_validate_attn_control checks tables on the host side.
 *   - Supported shapes: head_dim == 64; block in {16, 32, 64, 128};
 *     1 <= q_heads / kv_heads <= 8 with q_heads % kv_heads == 0;
 *     window == 0 (full attention) or 1 <= window.
 *   - Reentrant; calls on different streams may overlap as long as they do not
 *     share output or workspace memory.
 */
#ifndef PKV_H
#define PKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 3

typedef enum {
  PKV_OK = 0,
  PKV_ERR_ARG = -1,         /* null/misaligned pointer, negative or inconsistent size */
  PKV_ERR_UNSUPPORTED = -2, /* well-formed but outside the supported shapes */
  PKV_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  PKV_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  PKV_ERR_DATA = -5         /* pkv_validate_attn_control found bad table data */
} pkv_status;

/* Version of this ABI (PKV_ABI_VERSION of the built library). */
int pkv_abi_version(void);

/* Text of the last non-OK status returned on this thread ("" if none). */
const char* pkv_last_error(void);

/* Host only.  Bytes the KV cache may take on a device ("determine_available_
 * memory design": "How GMU works", "Heuristic formula", "Minimum KV guard").
 * The engine's share of the device is int(total_hbm_bytes * gmu); the cache
 * gets that share less bytes_used, clamped into [0, int(share * cap_fraction)]
 * (int() truncating toward zero, doubles as in Python; the page's defaults
 * are cap_fraction 0.30 and min_kv_gib 1.0).  *available_bytes (host) is
 * written in every non-ARG case; a budget below min_kv_gib GiB returns
 * PKV_ERR_DATA.  Byte counts must lie in [0, 2^52], gmu and cap_fraction in
 * [0, 1]. */
int pkv_kv_budget(int64_t total_hbm_bytes, int64_t bytes_used, double gmu,
                  double cap_fraction, double min_kv_gib, int64_t* available_bytes);

/* Host only.  Blocks per buffer a budget buys ("GPT-OSS-120B giga-kernel
 * decode", "KV budget (no cap)"): one block id costs both halves of each of
 * n_buffers shared buffers, 2 * kv_heads * block * head_dim bytes apiece;
 * rounded down and capped at INT32_MAX (block ids are int32). */
int pkv_kv_num_blocks(int64_t available_bytes, int32_t n_buffers, int32_t kv_heads,
                      int32_t block, int32_t head_dim, int64_t* num_blocks);

/* Host only.  Bytes of one half (K or V) and of a whole shared buffer
 * [2, num_blocks, kv_heads, block, head_dim] (section "KV-cache layout"); the
 * packed K view covers the same bytes.  Outputs are host pointers. */
int pkv_kv_buffer_bytes(int64_t num_blocks, int32_t kv_heads, int32_t block,
                        int32_t head_dim, int64_t* half_bytes, int64_t* total_bytes);

/* Host only.  Width of the trimmed sliding-window table: the most logical
 * blocks the window frame can touch, ceil((window-1+anchor_lag)/block) + 1
 * (anchor_lag 0 or 1, as in pkv_setup_attn_control). */
int pkv_trimmed_width(int32_t window, int32_t block, int32_t anchor_lag);

/* Layer-invariant attention control, built once per step ("Kernel contract").
 *
 * Inputs (device): seq_lens int32 [batch] = tokens of each sequence including
 * the new one (the new token's index is p = seq_lens-1); active uint8 [batch];
 * positions int64 [batch] absolute position of the new token (may be NULL);
 * bt_full / bt_swa int32 [batch, *] tables indexed by logical block with row
 * strides bt_full_stride / bt_swa_stride (elements) and `bt_width` valid
 * columns each.
 * anchor_lag (host, 0 or 1): 1 anchors the window frame one token back, at
 * p - 1, so that the window's oldest block stays in the trimmed table one
 * step past the boundary p % block == block-1 -- the reading taken here of
 * the sliding-window DI truncation of "DI wiring (NIXL)" (both nodes operate
 * at N-1).  The attended keys do not change.
 * Outputs (device): pos_full int32 [batch] = p; pos_swa int32 [batch] = the
 * window-frame position p - f*block with
 * f = max(0, p-anchor_lag-window+1)/block;
 * bt_swa_trim int32 [batch, trim_width] = bt_swa[b, f .. p/block] padded with
 * -1 (trim_width must equal pkv_trimmed_width(window, block, anchor_lag));
 * upd_full / upd_swa int64 [batch] = cache slots block_id*block + offset of
 * the new token in the full / sliding-window table; pos_abs int64 [batch]
 * (may be NULL) = positions, carried for the rotary stage.
 * Inactive sequences get -1 in every output.  A sequence whose p/block is
 * beyond bt_width keeps pos_full = p (so attention reports it as NaN) but gets
 * update slots of -1.  A table entry < 0 at the new token gives slot -1. */
int pkv_setup_attn_control(int32_t batch, int32_t block, int32_t window,
                           int32_t anchor_lag, const int32_t* seq_lens, const uint8_t* active,
                           const int64_t* positions,
                           const int32_t* bt_full, int32_t bt_full_stride,
                           const int32_t* bt_swa, int32_t bt_swa_stride, int32_t bt_width,
                           int32_t* pos_full, int32_t* pos_swa,
                           int32_t* bt_swa_trim, int32_t trim_width,
                           int64_t* upd_full, int64_t* upd_swa, int64_t* pos_abs,
                           void* stream);

/* The same control from compressed page lists instead of padded tables
 * ("MPK Internals: Compilation-to-Runtime Pipeline", "Phase 4": the
 * paged_kv_indptr / paged_kv_indices / paged_kv_last_page_len meta-tensors).
 * Sequence b's pages are full_indices[kv_indptr[b] .. kv_indptr[b+1]) in
 * logical order; it holds (pages-1)*block + last_page_len[b] tokens (0 pages:
 * none); swa_indices shares kv_indptr and holds -1 where the window's blocks
 * were freed (needed when window > 0).  A decode step has one query per
 * sequence, so no query index array is taken.  Outputs, besides those of
 * pkv_setup_attn_control: seq_lens int32 [batch] and the padded full table
 * bt_full int32 [batch, bt_stride] (bt_width columns written, -1 past a
 * sequence's pages; pages past bt_width are dropped) for
 * pkv_paged_decode_attn / pkv_step.  All arrays are device arrays; kv_indptr
 * has batch+1 entries and must be non-decreasing (not checked here). */
int pkv_setup_attn_control_csr(int32_t batch, int32_t block, int32_t window,
                               int32_t anchor_lag, const int32_t* kv_indptr,
                               const int32_t* full_indices,
                               const int32_t* swa_indices, const int32_t* last_page_len,
                               const uint8_t* active, const int64_t* positions, int32_t* bt_full,
                               int32_t bt_stride, int32_t bt_width, int32_t* seq_lens,
                               int32_t* pos_full, int32_t* pos_swa, int32_t* bt_swa_trim,
                               int32_t trim_width, int64_t* upd_full, int64_t* upd_swa,
                               int64_t* pos_abs, void* stream);

/* Quantise and scatter the new token's K and V into one shared buffer
 * ("Kernel contract": the write through an update index; "KV-cache layout":
 * packed K, plain V).
 *
 * k_new, v_new: bf16 [batch, kv_heads, head_dim].  k_half / v_half: the K and
 * V halves of the buffer (num_blocks*kv_heads*block*head_dim bytes each,
 * 16-byte aligned).  k_packed != 0 selects the packed K arrangement.
 * slot_idx int64 [batch]: block_id*block + offset, -1 = no write; slots outside
 * [0, num_blocks*block) are skipped.  Stored code = E4M3(fp32(x) / scale)
 * rounded to nearest even, saturating to +-448, NaN -> 0x7F|sign.
 * rope_cos, rope_sin: fp32 [batch, head_dim/2] (4-byte aligned) or both NULL.
 * Given, K is first turned by the attention control's rotary cos/sin
 * ("Kernel contract"), half-split: with h = head_dim/2 and i < h,
 * x_i' = x_i*c_i - x_{i+h}*s_i and x_{i+h}' = x_{i+h}*c_i + x_i*s_i, each
 * product rounded to fp32 before the sum (no fused multiply-add); x' is then
 * quantised as above.  V is never turned. */
int pkv_kv_cache_update(int32_t batch, int32_t kv_heads, int32_t head_dim, int32_t block,
                        int64_t num_blocks, const uint16_t* k_new, const uint16_t* v_new,
                        uint8_t* k_half, int32_t k_packed, uint8_t* v_half,
                        const int64_t* slot_idx, const float* rope_cos, const float* rope_sin,
                        float k_scale, float v_scale, void* stream);

/* Device bytes of the workspace pkv_paged_decode_attn needs for these shapes
 * (split-KV partial results and per-(sequence, KV head) arrival counters).
 * `table_width` is the number of valid table columns the call will get.
 * Returns a negative pkv_status on bad arguments.  The workspace must be
 * zero-filled once before its first use; every call leaves its counters at
 * zero again, so it can be reused by later calls on the same stream. */
int64_t pkv_decode_workspace_bytes(int32_t batch, int32_t q_heads, int32_t kv_heads,
                                   int32_t head_dim, int32_t block, int32_t table_width,
                                   int32_t window);

/* Paged decode attention for one layer (one query token per sequence).
 *
 * q bf16 [batch, q_heads, head_dim]; query head g reads KV head
 * g / (q_heads/kv_heads).  block_table int32 [batch, bt_stride] with
 * `table_width` valid columns: the full table (window == 0) or the trimmed
 * sliding-window table (window > 0).  frame_pos int32 [batch]: the newest key's
 * position in the table's frame (p for full, the window-frame position for
 * the trimmed table); < 0 = inactive (output row is +0).
 * Keys are frame positions [lo, frame_pos] with lo = 0 (full) or
 * max(0, frame_pos-window+1); key t lives in block block_table[b, t/block] at
 * slot t%block.  out bf16 [batch, q_heads, head_dim] =
 * softmax(sm_scale * q.K^) V^ with K^ = decode(K)*k_scale, V^ = decode(V)*v_scale,
 * accumulated in fp32 and rounded to bf16.  k_scale, v_scale and sm_scale are
 * finite and > 0, and so is the fp32 product sm_scale * k_scale * log2(e)
 * (else PKV_ERR_ARG).
 * k_packed: 1 = the K half in the packed view [nb, Hkv, block/2, head_dim, 2]
 * (two tokens interleaved per dimension), 0 = token-major rows
 * [nb, Hkv, block, head_dim] like V ("KV-cache layout"); same bytes, same speed.
 * rope_cos, rope_sin: fp32 [batch, head_dim/2] (16-byte aligned) or both NULL;
 * given, every query head of sequence b is first turned half-split by row b
 * (as in pkv_kv_cache_update), in fp32; the turned query enters the scores
 * as two bf16 parts (its bf16 rounding and the remainder of that rounding),
 * about 16 significant bits.
 * The cached keys are used as stored (a writer turned them before caching).
 * workspace: at least pkv_decode_workspace_bytes(...) bytes, 256-byte aligned,
 * zero-filled before first use. */
int pkv_paged_decode_attn(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                          int32_t block, int64_t num_blocks, int32_t window,
                          const uint16_t* q, const uint8_t* k_half, int32_t k_packed,
                          const uint8_t* v_half, const int32_t* block_table, int32_t bt_stride,
                          int32_t table_width, const int32_t* frame_pos,
                          const float* rope_cos, const float* rope_sin,
                          float k_scale, float v_scale, float sm_scale, uint16_t* out,
                          void* workspace, int64_t workspace_bytes, void* stream);

/* The per-step state the layer schedule needs: the shared buffers and the
 * control produced by pkv_setup_attn_control.  Host struct; the pointer
 * members are device pointers except the two buffer arrays, which are host
 * arrays of n_buffers device pointers.  Exactly one KV form must be given:
 * the per-buffer form (k_bufs/v_bufs) or the stacked form (`stacked`: one
 * allocation of n_buffers consecutive shared buffers, K half then V half
 * each) -- "Kernel contract". */
typedef struct pkv_step {
  int32_t batch, q_heads, kv_heads, head_dim, block, window;
  int64_t num_blocks;
  int32_t n_buffers;
  int32_t k_packed;
  uint8_t* const* k_bufs;       /* host array [n_buffers] of K halves, or NULL */
  uint8_t* const* v_bufs;       /* host array [n_buffers] of V halves, or NULL */
  uint8_t* stacked;             /* stacked form base, or NULL */
  const int32_t* bt_full;
  int32_t bt_full_stride, bt_full_width;
  const int32_t* bt_swa_trim;
  int32_t trim_width;
  const int32_t* pos_full;
  const int32_t* pos_swa;
  const int64_t* upd_full;
  const int64_t* upd_swa;
  const float* rope_cos;        /* fp32 [batch, head_dim/2] rotary cos/sin of the */
  const float* rope_sin;        /* step (16-byte aligned), or both NULL          */
} pkv_step;

/* One layer of the alternating schedule ("Kernel contract"): layer i writes
 * its new K/V into buffer i/2 through update index upd_swa (i even) or
 * upd_full (i odd) and attends with the trimmed table, window-frame
 * positions and window `step->window` (i even) or the full table, p and no
 * window (i odd).  Shapes as in pkv_kv_cache_update / pkv_paged_decode_attn.
 *
 * Both happen in one launch: the attention quantises each active sequence's
 * new token (code = E4M3(fp32(x) / fp32(scale))), stores it through the
 * layer's update index and attends to it.  Buffer bytes and outputs are
 * identical to pkv_kv_cache_update with that index followed by
 * pkv_paged_decode_attn (with the step's rope_cos / rope_sin passed to both
 * when given: the new K is turned before it is quantised, every query head
 * before the scores) whenever each update index is -1 (no write: the
 * attention reads the cache as it is) or the slot the layer's table gives for
 * the sequence's frame position, as pkv_setup_attn_control produces.  Any
 * other index makes that sequence's output row NaN and writes nothing for
 * it.  No id outside [0, num_blocks) is written.  The block holding a
 * sequence's new token must not appear in another sequence's table of the
 * same layer (its old bytes could be read there). */
int pkv_decode_layer(const pkv_step* step, int32_t layer, const uint16_t* q,
                     const uint16_t* k_new, const uint16_t* v_new, float k_scale,
                     float v_scale, float sm_scale, uint16_t* out, void* workspace,
                     int64_t workspace_bytes, void* stream);

/* pkv_decode_layer without a workspace argument, for callers that cannot
 * allocate device memory (work under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and bytes as
 * pkv_decode_layer; the split-KV workspace is instead a 24 MiB array the
 * library holds on each GPU it runs on, from its first use there until the
 * process ends.  Shapes whose pkv_decode_workspace_bytes exceeds 24 MiB are
 * refused with PKV_ERR_WORKSPACE before anything is enqueued.  Each call
 * clears the part of the array that must start at zero (one small extra
 * kernel on `stream`) and allocates nothing.  Every call on a GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller. */
int pkv_decode_layer_noalloc(const pkv_step* step, int32_t layer, const uint16_t* q,
                             const uint16_t* k_new, const uint16_t* v_new, float k_scale,
                             float v_scale, float sm_scale, uint16_t* out, void* stream);

/* Debug check of the control tables (synchronous: copies them to the host).
 * Checks every table entry a step would read: ids in [0, num_blocks) for the
 * keys of each active sequence in both tables, full and sliding-window ids
 * disjoint, p/block < bt_width.  Returns PKV_ERR_DATA with the first bad
 * (sequence, column) in pkv_last_error(), PKV_OK if clean. */
int pkv_validate_attn_control(int32_t batch, int32_t block, int32_t window,
                              int64_t num_blocks, const int32_t* seq_lens,
                              const uint8_t* active, const int32_t* bt_full,
                              int32_t bt_full_stride, const int32_t* bt_swa,
                              int32_t bt_swa_stride, int32_t bt_width, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */

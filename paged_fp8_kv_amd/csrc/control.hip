// Attention-control setup and the quantising KV write, gfx950.
//
// Setup builds, once per step, the layer-invariant control the page
// "GPT-OSS-120B giga-kernel decode" lists under "Kernel contract": the
// trimmed sliding-window table, the absolute and window-frame positions and
// the two KV-update indices.  The KV write quantises the new token's K/V to
// OCP E4M3 and scatters them through an update index, K through the packed
// view and V plain ("KV-cache layout"); with the control's rotary cos/sin it
// turns K (half-split) in fp32 first.
#include <algorithm>
#include <climits>

#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

namespace {

// The control of sequence b from its token count and an accessor for its
// table rows: full(c) / swa(c) give the block id of logical block c, or -1.
template <class Full, class Swa>
__device__ __forceinline__ void setup_one(const SetupLaunch& a, int b, int len, Full full, Swa swa) {
  const int BK = a.block;
  const bool act = a.active[b] != 0 && len > 0;
  int32_t* trow = a.trim ? a.trim + static_cast<int64_t>(b) * a.trim_width : nullptr;
  if (!act) {
    a.pos_full[b] = -1;
    a.upd_full[b] = -1;
    if (a.window > 0) {
      a.pos_swa[b] = -1;
      a.upd_swa[b] = -1;
      for (int i = 0; i < a.trim_width; ++i) trow[i] = -1;
    }
    if (a.pos_abs) a.pos_abs[b] = -1;
    return;
  }
  const int p = len - 1;
  const int cp = p / BK;
  const bool in_table = cp < a.bt_width;
  a.pos_full[b] = p;
  {
    const int blk = in_table ? full(cp) : -1;
    a.upd_full[b] = blk >= 0 ? static_cast<int64_t>(blk) * BK + p % BK : -1;
  }
  if (a.window > 0) {
    // anchor_lag 1 keeps the window's oldest block one step longer
    // ("DI wiring (NIXL)": both nodes operate at N - 1)
    const int first = max(0, p - a.anchor_lag - a.window + 1) / BK;
    for (int i = 0; i < a.trim_width; ++i) {
      const int c = first + i;
      trow[i] = (c <= cp && c < a.bt_width) ? swa(c) : -1;
    }
    a.pos_swa[b] = p - first * BK;
    const int blk = in_table ? swa(cp) : -1;
    a.upd_swa[b] = blk >= 0 ? static_cast<int64_t>(blk) * BK + p % BK : -1;
  }
  if (a.pos_abs) a.pos_abs[b] = a.positions ? a.positions[b] : -1;
}

// One thread per (sequence, trimmed-table column): column i of every
// sequence's trimmed row is filled by its own thread, column 0's thread also
// writing the sequence's positions and update indices, so that no thread
// runs a loop of dependent-address loads (measured at batch 256: 7.0 us with
// a thread per sequence looping over its row, in one workgroup).
constexpr int kSetupThreads = 64;
__global__ void __launch_bounds__(kSetupThreads) setup_kernel(SetupLaunch a) {
  const int cols = a.window > 0 ? max(a.trim_width, 1) : 1;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kSetupThreads + threadIdx.x;
  if (gid >= static_cast<int64_t>(a.B) * cols) return;
  const int b = static_cast<int>(gid / cols);
  const int i = static_cast<int>(gid - static_cast<int64_t>(b) * cols);
  const int32_t* frow = a.bt_full + static_cast<int64_t>(b) * a.bt_full_stride;
  const int32_t* srow = a.bt_swa ? a.bt_swa + static_cast<int64_t>(b) * a.bt_swa_stride : nullptr;
  const int len = a.seq_lens[b];
  if (i == 0) {
    SetupLaunch one = a;
    one.trim_width = 0;  // the row's columns are written below, by their own threads
    setup_one(one, b, len, [&](int c) { return frow[c]; }, [&](int c) { return srow[c]; });
  }
  if (a.window > 0 && i < a.trim_width) {
    const int BK = a.block;
    const bool act = a.active[b] != 0 && len > 0;
    int32_t v = -1;
    if (act) {
      const int p = len - 1;
      const int cp = p / BK;
      const int first = max(0, p - a.anchor_lag - a.window + 1) / BK;
      const int c = first + i;
      v = (c <= cp && c < a.bt_width) ? srow[c] : -1;
    }
    a.trim[static_cast<int64_t>(b) * a.trim_width + i] = v;
  }
}

// Compressed page lists ("MPK Internals", "Phase 4": paged_kv_indptr,
// paged_kv_indices, paged_kv_last_page_len): one workgroup per sequence
// writes its token count and its padded full-table row, and its thread 0
// builds the same control as setup_kernel.
__global__ void __launch_bounds__(256) setup_csr_kernel(SetupLaunch a, CsrInput c) {
  const int b = blockIdx.x;
  const int lo = c.kv_indptr[b];
  const int n = c.kv_indptr[b + 1] - lo;
  const int len = n > 0 ? (n - 1) * a.block + c.last_page_len[b] : 0;
  int32_t* frow = c.bt_full_out + static_cast<int64_t>(b) * a.bt_full_stride;
  for (int i = threadIdx.x; i < a.bt_width; i += 256) frow[i] = i < n ? c.full_indices[lo + i] : -1;
  if (threadIdx.x != 0) return;
  c.seq_lens_out[b] = len;
  setup_one(a, b, len, [&](int i) { return i < n ? c.full_indices[lo + i] : -1; },
            [&](int i) { return i < n ? c.swa_indices[lo + i] : -1; });
}

__global__ void __launch_bounds__(256) kv_update_kernel(UpdateLaunch a) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n = static_cast<int64_t>(a.B) * a.Hkv * kHeadDim;
  if (idx >= n) return;
  const int j = static_cast<int>(idx % kHeadDim);
  const int64_t bh = idx / kHeadDim;
  const int h = static_cast<int>(bh % a.Hkv);
  const int b = static_cast<int>(bh / a.Hkv);
  const int64_t slot = a.slot[b];
  const int BK = a.block;
  if (slot < 0 || slot >= a.nb * BK) return;
  const int64_t blk = slot / BK;
  const int t = static_cast<int>(slot % BK);
  float kf = bf16_bits_to_f32(a.k_new[idx]);
  if (a.rope_cos != nullptr) {
    // partner dimension j ^ 32 of the same row (rows are 64-aligned)
    const int i = b * (kHeadDim / 2) + (j & (kHeadDim / 2 - 1));
    kf = rope_turn(kf, bf16_bits_to_f32(a.k_new[idx ^ (kHeadDim / 2)]), a.rope_cos[i],
                   a.rope_sin[i], j >= kHeadDim / 2);
  }
  const float kx = __fdiv_rn(kf, a.k_scale);
  const float vx = __fdiv_rn(bf16_bits_to_f32(a.v_new[idx]), a.v_scale);
  const int64_t tile = (blk * a.Hkv + h) * static_cast<int64_t>(BK) * kHeadDim;
  const int64_t koff = a.k_packed ? tile + (static_cast<int64_t>(t / 2) * kHeadDim + j) * 2 + (t & 1)
                                  : tile + static_cast<int64_t>(t) * kHeadDim + j;
  a.k[koff] = f32_to_e4m3_rne_sat(kx);
  a.v[tile + static_cast<int64_t>(t) * kHeadDim + j] = f32_to_e4m3_rne_sat(vx);
}

}  // namespace

hipError_t launch_setup(const SetupLaunch& L, hipStream_t stream) {
  const int64_t cols = L.window > 0 ? std::max(L.trim_width, 1) : 1;
  const int64_t n_wg = (static_cast<int64_t>(L.B) * cols + kSetupThreads - 1) / kSetupThreads;
  if (n_wg > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(setup_kernel, dim3(static_cast<unsigned>(n_wg)), dim3(kSetupThreads), 0, stream, L);
  return hipGetLastError();
}

hipError_t launch_setup_csr(const SetupLaunch& L, const CsrInput& C, hipStream_t stream) {
  hipLaunchKernelGGL(setup_csr_kernel, dim3(L.B), dim3(256), 0, stream, L, C);
  return hipGetLastError();
}

hipError_t launch_kv_update(const UpdateLaunch& L, hipStream_t stream) {
  const int64_t n = static_cast<int64_t>(L.B) * L.Hkv * kHeadDim;
  const int64_t n_wg = (n + 255) / 256;
  hipLaunchKernelGGL(kv_update_kernel, dim3(static_cast<unsigned>(n_wg)), dim3(256), 0, stream, L);
  return hipGetLastError();
}

}  // namespace pkv

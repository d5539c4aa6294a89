// Paged decode attention over the packed-FP8 cache, gfx950.
//
// What it computes is decode attention read through the paged layout of the
// page "GPT-OSS-120B giga-kernel decode": keys of sequence b are frame
// positions [lo, hi] (hi = frame_pos[b]; lo = 0 for full layers and
// hi - window + 1 for sliding-window layers, section "Kernel contract"), key t
// sits in block table[b, t / BK] at slot t % BK, K stored through the packed
// view [.., BK/2, 64, 2] and V plain [.., BK, 64] (section "KV-cache layout").
//
// Work decomposition (MI355X design, not from the pages):
//  * The unit of work is a 32-token sub-tile of one (sequence, KV head) item.
//    All items' sub-tiles are laid end to end; each wave takes one contiguous,
//    equal share of that line (stream-K style), so ragged batches balance
//    without any host-side knowledge of the lengths.
//  * A wave works through its share item by item with its own online-softmax
//    state.  An item that lies wholly in one wave is written out directly; an
//    item cut by share boundaries leaves an fp32 partial (m, l, o) per piece,
//    and the last piece to arrive (device-scope counter) merges them.
//  * QK^T runs on v_mfma_f32_16x16x32_bf16 as S^T = Kp * Qx: the A operand is
//    16 packed K rows of 64 token-pair bytes each (two tokens interleaved per
//    dimension), B is the group's 8 queries expanded by token parity (column
//    (g, e) holds q_g in the lanes of parity e and zeros in the other), so one
//    16x16 tile yields the scores of 8 queries x 32 tokens with no byte
//    shuffling of K.  The E4M3 -> bf16 conversion is exact.
//  * PV runs on v_mfma_f32_16x16x32_f16 as O'^T = V'^T * P'^T: the scores
//    stay in the lanes that produced them (column (g, e), tokens 8q+2r+e), and
//    the V operand (8 consecutive tokens x one dimension per lane) is built
//    from per-token dwords with v_perm_b32 + the packed fp8 -> fp16 convert.
//    The two parity columns of a query are summed once at the end.
//  * Online softmax in the log2 domain (k_scale, 1/sqrt(d) and log2(e) folded
//    into one multiplier); the running maximum is only raised when some lane
//    beats it by more than 2^8, so rescaling is rare and the PV weights stay
//    below 256 (exact bookkeeping: numerator and denominator share the
//    reference maximum).
#include <algorithm>
#include <atomic>

#include "pkv_device.hpp"
#include "pkv_internal.hpp"

namespace pkv {

namespace {

constexpr int kSub = 32;              // tokens per MFMA sub-tile
#ifndef PKV_WAVES_PER_WG
#define PKV_WAVES_PER_WG 4
#endif
constexpr int kWavesPerWG = PKV_WAVES_PER_WG;
constexpr int kThreads = 64 * kWavesPerWG;
constexpr float kRescaleSlack = 8.0f; // log2 units
#ifndef PKV_DEPTH
#define PKV_DEPTH 4
#endif
// Sub-tiles in flight per wave.  Measured with the accumulators in VGPRs:
// 4 beats 6 by 1-1.5 us per full layer of the batch-64 x 8192 step (less
// queueing in the memory system for the same rate), 8 is 1 us slower, 2
// starves the stream (134 us).
constexpr int kDepth = PKV_DEPTH;
constexpr int kTinyItem = 8;          // items this short (sub-tiles) are never split
// Fixed cost of starting a short item (shorter than a share), in sub-tiles:
// the wait for its set-up loads and first K/V loads plus the fill and drain
// of the ring.  Per-wave timelines of a ragged batch (128 sequences, 128 to
// 32768 tokens) fit 0.63 us per streamed sub-tile and 3.5-3.8 us per item,
// about 6 sub-tiles; with 4, the waves given 10-13 short items finished
// 10-15 us after the median one.  The static split of full-attention
// launches counts it on top of the item's sub-tiles (window items are all
// short and alike: they are not weighted).
constexpr int kItemCost = 6;
// Waves per SIMD the kernel is compiled for (= workgroups per CU, 4 waves
// each); the stream-K shares assume every worker is resident at once.
#ifndef PKV_WG_PER_CU
#define PKV_WG_PER_CU 1
#endif
constexpr int kWGPerCU = PKV_WG_PER_CU;

struct AttnArgs {
  const uint16_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const int32_t* table;
  const int32_t* frame_pos;
  uint16_t* out;
  float* partial;
  int32_t* counters;  // [B * Hkv] arrival counters of split items
  int32_t partial_bytes;
  int64_t nb;
  int32_t B, Hq, Hkv, G;
  int32_t bt_stride, table_width, window;
  float score_scale;  // sm_scale * k_scale * log2(e)
  float v_scale;
  int32_t n_workers;
  // fused write of the new tokens (k_new null: none)
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint8_t* k_w;
  uint8_t* v_w;
  const int64_t* upd;  // write slot of each sequence's new token (-1: none)
  float k_scale;
  // rotary cos/sin fp32 [B, 32] (null: none) for the queries and the new K
  const float* rope_cos;
  const float* rope_sin;
};

// frame range [lo, hi] of sequence b; returns the number of sub-tiles
// (0 = no work: inactive, or invalid when *invalid is set).
template <int BK, bool WINDOWED>
__device__ __forceinline__ int seq_subtiles(const AttnArgs& a, int fp, int* lo_out,
                                            bool* invalid) {
  *invalid = false;
  if (fp < 0) return 0;
  if (fp >= a.table_width * BK) {
    *invalid = true;
    return 0;
  }
  const int lo = WINDOWED ? max(0, fp - a.window + 1) : 0;
  *lo_out = lo;
  return fp / kSub - lo / kSub + 1;
}

// Integer prefix and reductions over a wave's 64 lanes on the VALU (DPP row
// shifts and rotations, the gfx950 row-pair and half-wave swaps, lane reads)
// instead of LDS-crossbar permutes; integer sums and maxima are exact, so the
// order of the combining steps does not matter.  Every lane of the wave must
// be active.
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int x) {
  // lanes whose source lies outside their row of 16 read 0
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += dpp_i32<0x111>(x);  // row_shr:1 -- lane i adds lane i-1 of its row
  x += dpp_i32<0x112>(x);  // row_shr:2
  x += dpp_i32<0x114>(x);  // row_shr:4
  x += dpp_i32<0x118>(x);  // row_shr:8 -- now the prefix within the row
  const int r = lane_id() >> 4;
  const int t0 = __builtin_amdgcn_readlane(x, 15), t1 = __builtin_amdgcn_readlane(x, 31),
            t2 = __builtin_amdgcn_readlane(x, 47);
  return x + (r > 0 ? t0 : 0) + (r > 1 ? t1 : 0) + (r > 2 ? t2 : 0);
}
__device__ __forceinline__ int wave_max_i32(int x) {
  x = max(x, dpp_i32<0x121>(x));  // row_ror:1
  x = max(x, dpp_i32<0x122>(x));  // row_ror:2
  x = max(x, dpp_i32<0x124>(x));  // row_ror:4
  x = max(x, dpp_i32<0x128>(x));  // row_ror:8 -- the row's maximum in every lane
  const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max(static_cast<int>(p[0]), static_cast<int>(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max(static_cast<int>(q[0]), static_cast<int>(q[1]));
}
__device__ __forceinline__ int wave_sum_i32(int x) {
  x += dpp_i32<0x121>(x);
  x += dpp_i32<0x122>(x);
  x += dpp_i32<0x124>(x);
  x += dpp_i32<0x128>(x);
  const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = static_cast<int>(p[0]) + static_cast<int>(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return static_cast<int>(q[0]) + static_cast<int>(q[1]);
}

__device__ __forceinline__ void block_exclusive_scan(int* s, int n) {
  __shared__ int wsum[kWavesPerWG];
  const int tid = threadIdx.x;
  const int per = (n + kThreads - 1) / kThreads;
  const int beg = min(tid * per, n);
  const int end = min(beg + per, n);
  int local = 0;
  for (int i = beg; i < end; ++i) local += s[i];
  const int lane = tid & 63;
  const int x = wave_inclusive_sum(local);
  if (lane == 63) wsum[tid >> 6] = x;
  __syncthreads();
  int wave_off = 0;
  for (int w = 0; w < (tid >> 6); ++w) wave_off += wsum[w];
  int run = wave_off + x - local;
  for (int i = beg; i < end; ++i) {
    const int v = s[i];
    s[i] = run;
    run += v;
  }
  if (tid == kThreads - 1) s[n] = wave_off + x;
  __syncthreads();
}

// Cross-workgroup hand-off of split-KV partials.  Partials are written and
// read with device-coherent buffer accesses (write-through stores, loads that
// miss a stale L2 line; see write_partial and SlotPieces), and the writer
// waits for its stores to complete before it bumps the arrival counter.  This
// avoids agent-scope release/acquire fences, which on this target write back
// and invalidate the whole L2 of the issuing XCD.
__device__ __forceinline__ void wait_vm_stores() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): every issued store has completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Lane exchanges for the reductions over the lanes of one query (lanes
// i, i^8, i^16, i^32), done on the VALU instead of through the LDS crossbar
// (ds_bpermute): xor 8 is a rotation by 8 inside each row of 16 lanes (DPP
// row_ror:8); for xor 16 and xor 32, v_permlane16_swap / v_permlane32_swap of
// a value with itself leave each lane its own value in one result and its
// partner's in the other, so combining the two results is the same
// commutative max or sum a lane would form with its partner's value.
__device__ __forceinline__ float dpp_xor8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));
}
__device__ __forceinline__ float max_with_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_with_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float sum_with_xor16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_with_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ float wave_max_same_g(float v) {
  v = fmaxf(v, dpp_xor8(v));
  v = max_with_xor16(v);
  return max_with_xor32(v);
}
__device__ __forceinline__ float wave_sum_same_g(float v) {
  v += dpp_xor8(v);
  v = sum_with_xor16(v);
  return sum_with_xor32(v);
}

// Running state of one wave for one item (per lane: query g = m%8, parity e = m/8).
struct State {
  f32x4_t acc[4];  // acc[tau][r] = O'[(g,e)][dim 16q + 4r + tau] (unnormalised)
  float m;         // reference maximum (log2 domain), identical in all lanes of g
  float l;         // this lane's share of the denominator
  bool bad;        // a table entry outside [0, nb) was met
};

// dword 3 of a raw (untyped, unswizzled) buffer resource on this target
constexpr int kRsrcWord3 = 0x00020000;

struct Stage {
  u32x4_t k0, k1;   // 32 bytes of packed K row (pair m), bytes [32q, 32q+32)
  uint32_t v[8];    // V dwords: tokens 8q..8q+7, dims 4m..4m+3
};

// ---- LDS staging of K/V sub-tiles ------------------------------------------
// Each wave owns a ring of kDepth slots of 4 KiB (K 2 KiB, V 2 KiB).  A slot is
// filled by four 1 KiB direct-to-LDS buffer loads (16 bytes per lane, whole
// 128-byte lines per instruction); lane L's 16 bytes land at slot + 16*L.  The
// global chunk each lane fetches is chosen so that the slot holds a swizzled
// image from which the MFMA operands are read without bank conflicts:
//  * K: pair row r (128 B = 8 chunks) keeps chunk c at position
//    8r + (c ^ fk(r)), fk(r) = (r & 7) ^ (r >> 3);
//  * V: token t (64 B = 4 chunks) sits in row slot
//    s(t) = (t & ~3) | ((t + (t >> 3)) & 3), so the four tokens 8q+i read
//    together by the four lane groups fall in different banks.
constexpr int kSlotBytes = 4096;
constexpr int kWinRegs = 4;                  // table window: 64 entries per register
constexpr int kWinEntries = 64 * kWinRegs;
typedef __attribute__((address_space(3))) uint8_t* lds_ptr_t;
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer resource of `bytes` bytes at p, as four SGPRs.
__device__ __forceinline__ i32x4_t tile_desc(const uint8_t* p, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return i32x4_t{static_cast<int32_t>(static_cast<uint32_t>(a)),
                 static_cast<int32_t>(static_cast<uint32_t>(a >> 32) & 0xffffu), bytes, kRsrcWord3};
}

// One 16-byte-per-lane load from a buffer resource into LDS at
// lds_addr + 16 * lane.  Issued as inline assembly on purpose: the compiler
// cannot tell ring slots apart and would otherwise drain every outstanding
// direct-to-LDS load before each LDS read.  Completion is tracked by the
// explicit vmcnt waits below; the compiler's own waits for other loads only
// become stricter.
// NT marks the load non-temporal: the K/V bytes are read exactly once, and
// full-attention layers stream their whole context through the caches.
template <bool NT>
__device__ __forceinline__ void dma16(i32x4_t desc, uint32_t voff, uint32_t soff,
                                      uint32_t lds_addr) {
  if constexpr (NT)
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen nt lds"
                 :
                 : "v"(voff), "s"(desc), "s"(soff), "{m0}"(lds_addr)
                 : "memory");
  else
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voff), "s"(desc), "s"(soff), "{m0}"(lds_addr)
                 : "memory");
}
__device__ __forceinline__ uint32_t lds_addr_of(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)(const_cast<uint8_t*>(p))));
}

__device__ __forceinline__ int fk_swz(int r) { return (r & 7) ^ (r >> 3); }
__device__ __forceinline__ int v_row_slot(int t) { return (t & ~3) | ((t + (t >> 3)) & 3); }
__device__ __forceinline__ int v_row_token(int s) { return (s & ~3) | ((s - (s >> 3)) & 3); }

// s_waitcnt vmcnt(N) (expcnt / lgkmcnt left alone), fenced against compiler
// reordering of LDS accesses: direct-to-LDS loads are not tracked by the
// compiler's own wait insertion, so every read of a slot follows one of these.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until at most n sub-tiles' loads (four instructions each) are
// outstanding, 0 <= n < kDepth.
__device__ __forceinline__ void wait_vmcnt_slots(int n) {
  static_assert(kDepth <= 8, "wait table below");
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<4>(); break;
    case 2: wait_vmcnt<8>(); break;
    case 3: wait_vmcnt<12>(); break;
    case 4: wait_vmcnt<16>(); break;
    case 5: wait_vmcnt<20>(); break;
    case 6: wait_vmcnt<24>(); break;
    default: wait_vmcnt<28>(); break;
  }
}

template <int BK, bool WINDOWED, bool KP, int NREG = kWinRegs>
struct Item {
  // non-temporal K/V loads for full attention (measured: faster there, and
  // no gain for the short window reads)
  static constexpr bool kStreamNT = !WINDOWED;
  static constexpr int kEntries = 64 * NREG;  // table entries held in registers
  static constexpr int kBK = BK;
  const uint8_t* kbase;
  const uint8_t* vbase;
  uint8_t* kw;          // writable halves, for the fused new-token write
  uint8_t* vw;
  const int32_t* trow;
  int nb32;             // num_blocks clamped to int32 (block ids are int32)
  int width;            // table entries per row
  int hkv, h;
  int clo, chi;         // first / last logical block holding keys
  int tab_base;         // logical block held by lane 0 of tab[0]
  int tab[NREG];        // table entries for logical blocks tab_base + 64 r + lane
  bool bad;

  __device__ Item(const AttnArgs& a, int b, int h_)
      : kbase(a.k), vbase(a.v), kw(a.k_w), vw(a.v_w), hkv(a.Hkv), h(h_), bad(false) {
    nb32 = a.nb > 0x7fffffff ? 0x7fffffff : static_cast<int>(a.nb);
    width = a.table_width;
    clo = 0;
    chi = 0;
    trow = a.table + static_cast<int64_t>(b) * a.bt_stride;
    tab_base = -1000000;
#pragma unroll
    for (int r = 0; r < NREG; ++r) tab[r] = 0;
  }

  // Keys lo .. hi: logical blocks lo/BK .. hi/BK.
  __device__ __forceinline__ void set_range(int lo, int hi) {
    clo = lo / BK;
    chi = hi / BK;
  }

  // Load the table entries of logical blocks c0 .. c0+kEntries-1 (entries
  // past the row's width read as 0; only blocks clo .. chi are ever used).
  // Done between pipelined runs only, so no table load is ever pending while
  // K/V loads are in flight.
  __device__ __forceinline__ void load_window(int c0) {
    tab_base = c0;
#pragma unroll
    for (int r = 0; r < NREG; ++r) {
      const int cc = c0 + 64 * r + lane_id();
      tab[r] = (cc < width) ? trow[cc] : 0;
    }
  }

  // Block id of logical block c (uniform, inside the loaded window).
  // Out-of-range ids are replaced by 0 and flagged.
  __device__ __forceinline__ int block_of(int c) {
    const int i = c - tab_base;
    const int sel = i >> 6;
    int blk = __builtin_amdgcn_readlane(tab[0], i & 63);
#pragma unroll
    for (int r = 1; r < NREG; ++r) {
      const int br = __builtin_amdgcn_readlane(tab[r], i & 63);
      blk = (sel == r) ? br : blk;
    }
    if (blk < 0 || blk >= nb32) {
      bad = true;
      blk = 0;
    }
    return blk;
  }

  __device__ __forceinline__ int clampc(int c) const { return min(max(c, clo), chi); }

  // Fill ring slot `slot` with sub-tile t32 (four direct-to-LDS loads through
  // per-tile buffer resources; the resource range check keeps every access
  // inside its tile).
  __device__ __forceinline__ void issue(uint8_t* ring, int slot, int t32) {
    const int lane = lane_id();
    const int base = t32 * kSub;
    const uint32_t dst = lds_addr_of(ring + slot * kSlotBytes);
    if constexpr (BK >= kSub) {
      const int blk = block_of(clampc(base / BK));
      const int64_t tile = (static_cast<int64_t>(blk) * hkv + h) * (BK * kHeadDim);
      const i32x4_t rk = tile_desc(kbase + tile, BK * kHeadDim);
      const i32x4_t rv = tile_desc(vbase + tile, BK * kHeadDim);
      const uint32_t so = static_cast<uint32_t>((base % BK) * kHeadDim);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t kof = KP ? static_cast<uint32_t>((8 * j + (lane >> 3)) * 128 +
                                                        (((lane & 7) ^ (lane >> 3) ^ j) * 16))
                                : static_cast<uint32_t>(v_row_token(16 * j + (lane >> 2)) * kHeadDim +
                                                        (lane & 3) * 16);
        dma16<kStreamNT>(rk, kof, so, dst + 1024 * j);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int t = v_row_token(16 * j + (lane >> 2));
        const uint32_t vof = static_cast<uint32_t>(t * kHeadDim + (lane & 3) * 16);
        dma16<kStreamNT>(rv, vof, so, dst + 2048 + 1024 * j);
      }
    } else {
      // BK == 16: each load instruction covers one of the two blocks of the
      // sub-tile (K pair rows 8j.., V tokens 16j..)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int blk = block_of(clampc(base / BK + j));
        const int64_t tile = (static_cast<int64_t>(blk) * hkv + h) * (BK * kHeadDim);
        const i32x4_t rk = tile_desc(kbase + tile, BK * kHeadDim);
        const i32x4_t rv = tile_desc(vbase + tile, BK * kHeadDim);
        const int t = v_row_token(16 * j + (lane >> 2)) - 16 * j;
        const uint32_t kof = KP ? static_cast<uint32_t>((lane >> 3) * 128 + (((lane & 7) ^ (lane >> 3) ^ j) * 16))
                                : static_cast<uint32_t>(t * kHeadDim + (lane & 3) * 16);
        dma16<kStreamNT>(rk, kof, 0u, dst + 1024 * j);
        const uint32_t vof = static_cast<uint32_t>(t * kHeadDim + (lane & 3) * 16);
        dma16<kStreamNT>(rv, vof, 0u, dst + 2048 + 1024 * j);
      }
    }
  }
};

// Read a filled slot into the MFMA lane layout: K pair row m, bytes
// [32q, 32q+32); V dwords of tokens 8q..8q+7 at dims 4m..4m+3.
template <bool KP>
__device__ __forceinline__ void read_slot(const uint8_t* ring, int slot, Stage& st) {
  const int lane = lane_id();
  const int m = lane & 15, q = lane >> 4;
  const uint8_t* src = ring + slot * kSlotBytes;
  if constexpr (KP) {
    const int fk = fk_swz(m);
    st.k0 = *reinterpret_cast<const u32x4_t*>(src + (8 * m + ((2 * q) ^ fk)) * 16);
    st.k1 = *reinterpret_cast<const u32x4_t*>(src + (8 * m + ((2 * q + 1) ^ fk)) * 16);
  } else {
    // token-major K rows (placed like V): build the packed operand -- pair row
    // m, bytes [32q, 32q+32) = dims 16q .. 16q+15 of tokens 2m, 2m+1
    // interleaved -- from 16 bytes of each token's row
    const u32x4_t t0 = *reinterpret_cast<const u32x4_t*>(src + v_row_slot(2 * m) * kHeadDim + 16 * q);
    const u32x4_t t1 = *reinterpret_cast<const u32x4_t*>(src + v_row_slot(2 * m + 1) * kHeadDim + 16 * q);
    st.k0 = u32x4_t{__builtin_amdgcn_perm(t1[0], t0[0], 0x05010400u), __builtin_amdgcn_perm(t1[0], t0[0], 0x07030602u),
                    __builtin_amdgcn_perm(t1[1], t0[1], 0x05010400u), __builtin_amdgcn_perm(t1[1], t0[1], 0x07030602u)};
    st.k1 = u32x4_t{__builtin_amdgcn_perm(t1[2], t0[2], 0x05010400u), __builtin_amdgcn_perm(t1[2], t0[2], 0x07030602u),
                    __builtin_amdgcn_perm(t1[3], t0[3], 0x05010400u), __builtin_amdgcn_perm(t1[3], t0[3], 0x07030602u)};
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
    st.v[i] = *reinterpret_cast<const uint32_t*>(src + 2048 + v_row_slot(8 * q + i) * kHeadDim +
                                                 (m >> 2) * 16 + (m & 3) * 4);
}

// Put the new token's codes (lane j: dim j) into a filled slot, at token
// `tok` (0..31) of the sub-tile, in the slot's own arrangement: K pair row
// tok/2, byte 2j + tok%2 of the row, rows chunk-swizzled; V row of token tok.
template <bool KP>
__device__ __forceinline__ void patch_slot(uint8_t* ring, int slot, int tok, uint32_t kcode,
                                           uint32_t vcode) {
  const int j = lane_id();
  uint8_t* dst = ring + slot * kSlotBytes;
  if constexpr (KP) {
    const int r = tok >> 1;
    const int kb = 2 * j + (tok & 1);
    dst[r * 128 + (((kb >> 4) ^ fk_swz(r)) << 4) + (kb & 15)] = static_cast<uint8_t>(kcode);
  } else {
    dst[v_row_slot(tok) * kHeadDim + j] = static_cast<uint8_t>(kcode);
  }
  dst[2048 + v_row_slot(tok) * kHeadDim + j] = static_cast<uint8_t>(vcode);
}

// One 32-token sub-tile: scores, online-softmax update and PV accumulation.
// MASKED selects the edge path (keys outside [lo, hi] removed); the stage
// registers are never written here, so the interior path carries no copies.
// LO: the queries are carried as bf16 pairs hi + lo (rotated queries): the
// scores take a second pass of MFMAs over the low parts, with the same K.
template <bool MASKED, bool LO = false>
__device__ __forceinline__ void compute_subtile(const Stage& st, int t32, int lo, int hi,
                                                float score_scale, const uint32_t (&qx)[4][4],
                                                const uint32_t (&qxl)[4][4], State& s) {
  const int lane = lane_id();
  const int m = lane & 15, q = lane >> 4, e = m >> 3;
  const int base = t32 * kSub;
  uint32_t kd[8] = {st.k0[0], st.k0[1], st.k0[2], st.k0[3], st.k1[0], st.k1[1], st.k1[2], st.k1[3]};
  uint32_t vd[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) vd[i] = st.v[i];
  if constexpr (MASKED) {
    // zero the bytes of out-of-range tokens so 0 * NaN never reaches a score
    const int t_even = base + 2 * m;
    const bool ok0 = (t_even >= lo) && (t_even <= hi);
    const bool ok1 = (t_even + 1 >= lo) && (t_even + 1 <= hi);
    const uint32_t keep = (ok0 ? 0x00ff00ffu : 0u) | (ok1 ? 0xff00ff00u : 0u);
#pragma unroll
    for (int i = 0; i < 8; ++i) kd[i] &= keep;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = base + 8 * q + i;
      vd[i] = (t < lo || t > hi) ? 0u : vd[i];
    }
  }
  // ---- S^T = Kp * Qx
  f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t av[4] = {e4m3x2_to_bf16x2<false>(kd[2 * i]), e4m3x2_to_bf16x2<true>(kd[2 * i]),
                      e4m3x2_to_bf16x2<false>(kd[2 * i + 1]), e4m3x2_to_bf16x2<true>(kd[2 * i + 1])};
    bf16x8_t A = __builtin_bit_cast(bf16x8_t, av);
    bf16x8_t Bq = __builtin_bit_cast(bf16x8_t, qx[i]);
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bq, sacc, 0, 0, 0);
    if constexpr (LO) {
      bf16x8_t Bl = __builtin_bit_cast(bf16x8_t, qxl[i]);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bl, sacc, 0, 0, 0);
    }
  }
  // lane holds scores of query g for tokens base + 8q + 2r + e
  float x[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x[r] = sacc[r] * score_scale;
    if constexpr (MASKED) {
      const int t = base + 8 * q + 2 * r + e;
      if (t < lo || t > hi) x[r] = -INFINITY;
    }
  }
  const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  if (__any(mx > s.m + kRescaleSlack)) {
    const float mnew = fmaxf(s.m, wave_max_same_g(mx));
    const float alpha = __builtin_amdgcn_exp2f(s.m - mnew);
#pragma unroll
    for (int t = 0; t < 4; ++t) s.acc[t] *= alpha;
    s.l *= alpha;
    s.m = mnew;
  }
  uint32_t pv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float p = __builtin_amdgcn_exp2f(x[r] - s.m);
    s.l += p;
    const _Float16 ph = static_cast<_Float16>(p);
    pv[r] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, ph)) << (16 * e);
  }
  f16x8_t Bp = __builtin_bit_cast(f16x8_t, pv);
  // ---- V operands: dims 4m+tau, tokens 8q .. 8q+7 in slot order
  uint32_t vop[4][4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo2 = __builtin_amdgcn_perm(vd[2 * k + 1], vd[2 * k], 0x05010400u);
    const uint32_t hi2 = __builtin_amdgcn_perm(vd[2 * k + 1], vd[2 * k], 0x07030602u);
    vop[0][k] = e4m3x2_to_f16x2<false>(lo2);
    vop[1][k] = e4m3x2_to_f16x2<true>(lo2);
    vop[2][k] = e4m3x2_to_f16x2<false>(hi2);
    vop[3][k] = e4m3x2_to_f16x2<true>(hi2);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f16x8_t Av = __builtin_bit_cast(f16x8_t, vop[t]);
    s.acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Av, Bp, s.acc[t], 0, 0, 0);
  }
}

__device__ __forceinline__ void store_bf16x16(uint16_t* dst, const float* v) {
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    w[i] = static_cast<uint32_t>(f32_to_bf16_bits(v[2 * i])) |
           (static_cast<uint32_t>(f32_to_bf16_bits(v[2 * i + 1])) << 16);
  u32x4_t* d = reinterpret_cast<u32x4_t*>(dst);
  d[0] = u32x4_t{w[0], w[1], w[2], w[3]};
  d[1] = u32x4_t{w[4], w[5], w[6], w[7]};
}

// Fused cache write of the new token at frame position hi of the item
// (lane j: dim j) through the sequence's update index `upd`: when it is the
// slot the table gives for hi, patch the LDS slot holding the token's
// sub-tile and store the codes there; when it is -1, write nothing and read
// the cache as it is (as the separate update would); any other value, or a
// table id outside the pool, flags the item bad (NaN row) and writes nothing.
template <int BK, bool WINDOWED, bool KP, int NREG>
__device__ __forceinline__ void write_new_token(Item<BK, WINDOWED, KP, NREG>& it, uint8_t* ring,
                                                int slot, int hi, int64_t upd, uint32_t kcode,
                                                uint32_t vcode) {
  if (upd < 0) return;
  const bool was_bad = it.bad;
  it.bad = false;
  const int blk = it.block_of(it.clampc(hi / BK));
  const bool valid = !it.bad && upd == static_cast<int64_t>(blk) * BK + hi % BK;
  it.bad = was_bad || !valid;
  if (valid) {
    patch_slot<KP>(ring, slot, hi % kSub, kcode, vcode);
    const int j = lane_id();
    const int tok = hi % BK;
    const int64_t tile = (static_cast<int64_t>(blk) * it.hkv + it.h) * (BK * kHeadDim);
    it.kw[KP ? tile + ((tok >> 1) * kHeadDim + j) * 2 + (tok & 1) : tile + tok * kHeadDim + j] =
        static_cast<uint8_t>(kcode);
    it.vw[tile + tok * kHeadDim + j] = static_cast<uint8_t>(vcode);
  }
}

constexpr int kSlotFloats = 8 * kHeadDim + 16;  // o[8][64], m[8], l[8]
constexpr int kSlotBytesF = kSlotFloats * 4;

// Chunks of the item line [0, total): chunk c covers [c*C, (c+1)*C).  The
// pieces of one item are in consecutive chunks and use partial slots 2c (the
// piece continues an item begun in an earlier chunk) or 2c+1 (the piece
// begins an item that goes on).
struct Sched {
  int64_t C;
  __device__ __forceinline__ int of(int64_t x) const { return static_cast<int>(x / C); }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(const AttnArgs& a) {
  return __builtin_amdgcn_make_buffer_rsrc(a.partial, 0, a.partial_bytes, kRsrcWord3);
}
constexpr int kCoherent = 16;  // sc1: device-coherent access (write-through / no stale L2 hit)

// Write one piece's partial (o unnormalised, running max m, sum l) to a slot.
// Lane (m, q) with e == 0 holds o of head g = m, dims 16q .. 16q+15.
__device__ __forceinline__ void write_partial(const AttnArgs& a, int slot, const float (&o)[16],
                                              float mx, float lsum, int lane) {
  const int m = lane & 15, q = lane >> 4;
  const __amdgpu_buffer_rsrc_t r = partial_rsrc(a);
  const int base = slot * kSlotBytesF;
  if (m < 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4_t w = {__float_as_uint(o[4 * i]), __float_as_uint(o[4 * i + 1]),
                         __float_as_uint(o[4 * i + 2]), __float_as_uint(o[4 * i + 3])};
      __builtin_amdgcn_raw_buffer_store_b128(w, r, base + (m * kHeadDim + 16 * q + 4 * i) * 4, 0,
                                             kCoherent);
    }
    if (q == 0) {
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(mx), r, base + (8 * kHeadDim + m) * 4, 0,
                                            kCoherent);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lsum), r,
                                            base + (8 * kHeadDim + 8 + m) * 4, 0, kCoherent);
    }
  }
}

// Write one piece's partial into workgroup LDS, same layout as a workspace slot.
__device__ __forceinline__ void write_partial_lds(float* dst, const float (&o)[16], float mx,
                                                  float lsum, int lane) {
  const int m = lane & 15, q = lane >> 4;
  if (m < 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<f32x4_t*>(dst + m * kHeadDim + 16 * q + 4 * i) =
          f32x4_t{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
    if (q == 0) {
      dst[8 * kHeadDim + m] = mx;
      dst[8 * kHeadDim + 8 + m] = lsum;
    }
  }
}

// Pieces of an item in workspace slots: chunk cf's tail slot, then the head
// slots of chunks cf+1 .. (device-coherent loads).
struct SlotPieces {
  __amdgpu_buffer_rsrc_t r;
  int cf;
  __device__ __forceinline__ void load(int k, int g, int part, float& m, float& l, u32x4_t& o0,
                                       u32x4_t& o1) const {
    const int sl = (k == 0) ? 2 * cf + 1 : 2 * (cf + k);
    const int base = sl * kSlotBytesF;
    m = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, base + (8 * kHeadDim + g) * 4, 0, kCoherent));
    l = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, base + (8 * kHeadDim + 8 + g) * 4, 0, kCoherent));
    o0 = __builtin_amdgcn_raw_buffer_load_b128(r, base + (g * kHeadDim + 8 * part) * 4, 0, kCoherent);
    o1 = __builtin_amdgcn_raw_buffer_load_b128(r, base + (g * kHeadDim + 8 * part + 4) * 4, 0, kCoherent);
  }
};

// Consecutive LDS slots holding pieces 0, 1, ... of one item.
struct LdsSlots {
  const float* base;
  __device__ __forceinline__ void load(int k, int g, int part, float& m, float& l, u32x4_t& o0,
                                       u32x4_t& o1) const {
    const float* p = base + k * kSlotFloats;
    m = p[8 * kHeadDim + g];
    l = p[8 * kHeadDim + 8 + g];
    o0 = *reinterpret_cast<const u32x4_t*>(p + g * kHeadDim + 8 * part);
    o1 = *reinterpret_cast<const u32x4_t*>(p + g * kHeadDim + 8 * part + 4);
  }
};

// The two pieces of an item cut once inside one workgroup, in LDS.
struct LdsPieces {
  const float* p0;
  const float* p1;
  __device__ __forceinline__ void load(int k, int g, int part, float& m, float& l, u32x4_t& o0,
                                       u32x4_t& o1) const {
    const float* p = k == 0 ? p0 : p1;
    m = p[8 * kHeadDim + g];
    l = p[8 * kHeadDim + 8 + g];
    o0 = *reinterpret_cast<const u32x4_t*>(p + g * kHeadDim + 8 * part);
    o1 = *reinterpret_cast<const u32x4_t*>(p + g * kHeadDim + 8 * part + 4);
  }
};

// Combine the P pieces of item (b, h), in piece order, and write the output
// row.  ROUND pieces are fetched per round (8 from the workspace; the two LDS
// pieces of an item cut inside one workgroup in a single round of 2); lane
// (g = lane & 7, part = lane >> 3) owns dims 8*part .. 8*part+7 of head g.
// Rounds combine with a running maximum.
template <int ROUND, class Src>
__device__ __forceinline__ void merge_item(const AttnArgs& a, int b, int h, int P, int lane,
                                           const Src& src) {
  const int g = lane & 7, part = lane >> 3;
  float mrun = -INFINITY, lrun = 0.f;
  float acc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) acc[d] = 0.f;
  for (int k0 = 0; k0 < P; k0 += ROUND) {
    float mk[ROUND], lk[ROUND];
    u32x4_t o0[ROUND], o1[ROUND];
#pragma unroll
    for (int i = 0; i < ROUND; ++i) src.load(min(k0 + i, P - 1), g, part, mk[i], lk[i], o0[i], o1[i]);
    float mx = mrun;
#pragma unroll
    for (int i = 0; i < ROUND; ++i)
      if (k0 + i < P) mx = fmaxf(mx, mk[i]);
    const float sc = __builtin_amdgcn_exp2f(mrun - mx);
    lrun *= sc;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] *= sc;
#pragma unroll
    for (int i = 0; i < ROUND; ++i) {
      if (k0 + i < P) {
        const float w = __builtin_amdgcn_exp2f(mk[i] - mx);
        lrun += w * lk[i];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          acc[d] += w * __uint_as_float(o0[i][d]);
          acc[4 + d] += w * __uint_as_float(o1[i][d]);
        }
      }
    }
    mrun = mx;
  }
  if (g < a.G) {
    const float f = a.v_scale / lrun;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16_bits(acc[2 * i] * f)) |
             (static_cast<uint32_t>(f32_to_bf16_bits(acc[2 * i + 1] * f)) << 16);
    *reinterpret_cast<u32x4_t*>(a.out + (static_cast<int64_t>(b) * a.Hq + h * a.G + g) * kHeadDim +
                                8 * part) = u32x4_t{w[0], w[1], w[2], w[3]};
  }
}

// Exclusive prefix of the per-sequence sub-tile counts, pre(b) for
// 0 <= b <= B (pre(B) = the total), held in LDS by the workgroup ...
struct PreLds {
  const int* s;
  __device__ __forceinline__ int operator()(int i) const { return s[i]; }
  // frame position of sequence b (a load)
  __device__ __forceinline__ int pos(const AttnArgs& a, int b) const { return a.frame_pos[b]; }
  // the last b in [0, B) with pre(b) * hkv <= x (uniform)
  __device__ __forceinline__ int last_at_or_below(int B, int hkv, int64_t x) const {
    int lo_i = 0, hi_i = B - 1;
    while (lo_i < hi_i) {
      const int mid = (lo_i + hi_i + 1) >> 1;
      if (static_cast<int64_t>(s[mid]) * hkv <= x) lo_i = mid; else hi_i = mid - 1;
    }
    return __builtin_amdgcn_readfirstlane(lo_i);
  }
};

// ... or, for B <= 64, in one register of every wave: lane b holds pre(b)
// (lanes b >= B hold the total).
struct PreReg {
  int v;
  int total;
  int p;  // lane b: frame position of sequence b, as loaded for the prefix
  __device__ __forceinline__ int operator()(int i) const {
    return i < kWave ? __builtin_amdgcn_readlane(v, i) : total;
  }
  __device__ __forceinline__ int pos(const AttnArgs&, int b) const {
    return __builtin_amdgcn_readlane(p, b);
  }
  __device__ __forceinline__ int last_at_or_below(int B, int hkv, int64_t x) const {
    // pre is non-decreasing, so the lanes that qualify are a prefix of [0, B)
    const uint64_t m = __ballot(lane_id() < B && static_cast<int64_t>(v) * hkv <= x);
    return __builtin_amdgcn_readfirstlane(__popcll(m) - 1);
  }
};

// Offset (in the item line) of the first item that starts at or after x;
// `total` when there is none.  Items are (b, h) in order, sequence b holding
// Hkv items of pre(b+1)-pre(b) sub-tiles each.
template <class Pre>
__device__ __forceinline__ int64_t first_item_start_at_or_after(const Pre& pre, int B, int hkv,
                                                                int64_t x) {
  const int64_t total = static_cast<int64_t>(pre(B)) * hkv;
  if (x >= total) return total;
  const int lo_i = pre.last_at_or_below(B, hkv, x);
  const int64_t base = static_cast<int64_t>(pre(lo_i)) * hkv;
  const int n = pre(lo_i + 1) - pre(lo_i);
  const int64_t h = (x - base + n - 1) / n;  // first item of b at or after x
  if (h < hkv) return base + h * n;
  return static_cast<int64_t>(pre(lo_i + 1)) * hkv;  // first item of the next sequence with work
}

// Half-split rotation of the lane's 16 query dims (16q .. 16q+15, packed bf16
// in q0, q1); the partner dims 16(q^2) .. live in lane ^ 32.  In fp32, then
// carried as two bf16 parts: q0, q1 get the rounded value and l0, l1 what
// that rounding left out (exact in fp32, rounded to bf16 in turn), so that
// the scores see about 16 significant bits of each rotated dim.
__device__ __forceinline__ void rotate_queries(u32x4_t& q0, u32x4_t& q1, u32x4_t& l0, u32x4_t& l1,
                                               const f32x4_t (&c)[4], const f32x4_t (&s)[4],
                                               bool upper) {
  uint32_t w[8] = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
  uint32_t p[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) p[k] = static_cast<uint32_t>(__shfl_xor(static_cast<int>(w[k]), 32));
  uint32_t r[8], rl[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint32_t hh[2], ll[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int d = 2 * k + e;
      const float x = __uint_as_float((e ? w[k] & 0xffff0000u : w[k] << 16));
      const float xp = __uint_as_float((e ? p[k] & 0xffff0000u : p[k] << 16));
      const float y = rope_turn(x, xp, c[d >> 2][d & 3], s[d >> 2][d & 3], upper);
      hh[e] = f32_to_bf16_bits(y);
      ll[e] = f32_to_bf16_bits(y - bf16_bits_to_f32(static_cast<uint16_t>(hh[e])));
    }
    r[k] = hh[0] | (hh[1] << 16);
    rl[k] = ll[0] | (ll[1] << 16);
  }
  q0 = u32x4_t{r[0], r[1], r[2], r[3]};
  q1 = u32x4_t{r[4], r[5], r[6], r[7]};
  l0 = u32x4_t{rl[0], rl[1], rl[2], rl[3]};
  l1 = u32x4_t{rl[4], rl[5], rl[6], rl[7]};
}

// Expanded queries for the score MFMA: qx[i][k] holds q[g][16q + 4i + k]
// (lane: g = m & 7, q = lane >> 4) in the 16-bit half of parity e = m >> 3,
// zeros in the other half.
__device__ __forceinline__ void expand_queries(const u32x4_t& q0, const u32x4_t& q1, int e,
                                               uint32_t (&qx)[4][4]) {
  const uint32_t qw[8] = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = 4 * i + k;  // dim 16q + d
      const uint32_t bits = (qw[d >> 1] >> (16 * (d & 1))) & 0xffffu;
      qx[i][k] = bits << (16 * e);
    }
}

// FP8 codes of the new token's K and V at dimension `lane` (K turned first
// when rotary cos/sin are given: the partner dimension lives in lane ^ 32,
// so every lane of the wave must be here).
template <bool ROPE>
__device__ __forceinline__ void new_token_codes(const AttnArgs& a, uint16_t kn_bits,
                                                uint16_t vn_bits, float kn_c, float kn_s,
                                                uint32_t& kcode, uint32_t& vcode) {
  const int lane = lane_id();
  float kf = bf16_bits_to_f32(kn_bits);
  if (ROPE)
    kf = rope_turn(kf, bf16_bits_to_f32(static_cast<uint16_t>(__shfl_xor(static_cast<int>(kn_bits), 32))),
                   kn_c, kn_s, lane >= kHeadDim / 2);
  kcode = f32_to_e4m3_rne_sat(__fdiv_rn(kf, a.k_scale));
  vcode = f32_to_e4m3_rne_sat(__fdiv_rn(bf16_bits_to_f32(vn_bits), a.v_scale));
}

__device__ __forceinline__ void reset_state(State& s) {
#pragma unroll
  for (int t = 0; t < 4; ++t) s.acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  s.m = -INFINITY;
  s.l = 0.f;
}

// Two-stage software pipeline over the sub-tiles t0 .. tlast of one piece,
// run per window of the item's table entries held in registers.  Ring of
// kDepth slots: sub-tile k lives in slot (k - tw) % kDepth.  While sub-tile k
// is computed from registers, sub-tile k+1 is read from its slot into the
// other register stage and up to kDepth-1 later sub-tiles are in flight; slot
// k is refilled once k has been consumed.  start_run() issues a run's first
// loads; stream() consumes every sub-tile, starting further runs as needed.
static_assert(kDepth % 2 == 0, "register stages alternate with the slot index");
template <class It>
struct Segment {
  It& it;
  uint8_t* ring;
  int tw, twl, tlast, span;

  __device__ __forceinline__ Segment(It& it_, uint8_t* ring_, int t0, int tlast_, int span0)
      : it(it_), ring(ring_), tw(t0), twl(t0), tlast(tlast_), span(span0) {}

  __device__ __forceinline__ void start_run() {
    const int cw0 = it.clampc((tw * kSub) / It::kBK);
    if (cw0 < it.tab_base || cw0 >= it.tab_base + It::kEntries) it.load_window(cw0);
    const int cend = min(it.tab_base + It::kEntries, cw0 + span);  // first column past the run
    twl = max(tw, min(tlast, (cend * It::kBK) / kSub - 1));
    span = It::kEntries;
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
      if (tw + d <= twl) it.issue(ring, d, tw + d);
  }

  // The first run must have been started.  t_new: the sub-tile holding the
  // new token (its codes patched into the slot before it is read), or -1.
  template <bool KP, bool LO = false>
  __device__ __forceinline__ void stream(float score_scale, int lo, int hi, int t_new,
                                         int64_t upd, uint32_t kcode, uint32_t vcode,
                                         const uint32_t (&qx)[4][4], const uint32_t (&qxl)[4][4],
                                         State& s) {
    for (bool first = true; tw <= tlast; first = false) {
      if (!first) start_run();
      Stage st[2];
      wait_vmcnt_slots(min(twl - tw, kDepth - 1));
      if (tw == t_new) write_new_token(it, ring, 0, hi, upd, kcode, vcode);
      read_slot<KP>(ring, 0, st[0]);
      for (int i = tw; i <= twl; i += kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
          const int t32 = i + d;
          if (t32 > twl) break;
          // sub-tile t32+1 is complete once at most the sub-tiles issued after
          // it (t32+2 .. min(twl, t32+kDepth-1)) are outstanding
          if (t32 < twl) {
            wait_vmcnt_slots(min(twl - t32 - 1, kDepth - 2));
            if (t32 + 1 == t_new)
              write_new_token(it, ring, (d + 1) % kDepth, hi, upd, kcode, vcode);
            read_slot<KP>(ring, (d + 1) % kDepth, st[(d + 1) & 1]);
          }
          if (t32 * kSub >= lo && t32 * kSub + kSub - 1 <= hi)
            compute_subtile<false, LO>(st[d & 1], t32, lo, hi, score_scale, qx, qxl, s);
          else
            compute_subtile<true, LO>(st[d & 1], t32, lo, hi, score_scale, qx, qxl, s);
          if (t32 + kDepth <= twl) it.issue(ring, d, t32 + kDepth);
        }
      }
      tw = twl + 1;
    }
    s.bad = it.bad;
  }
};

// Reduce a piece's state across the parity halves of the wave: o[4r + tau] =
// dim 16q + 4r + tau of query g (valid in the lanes with e == 0), the
// denominator and whether a bad table entry was met.
__device__ __forceinline__ void finish_piece(State& s, float (&o)[16], float& lsum, bool& bad) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) s.acc[t][r] += dpp_xor8(s.acc[t][r]);
  lsum = wave_sum_same_g(s.l);
  bad = __any(s.bad);
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < 4; ++t) o[4 * r + t] = s.acc[t][r];
}

// Normalise and store a whole item's output rows (lanes with e == 0, g < G).
__device__ __forceinline__ void store_whole(const AttnArgs& a, int b, int h, float (&o)[16],
                                            float lsum, bool bad) {
  const int lane = lane_id();
  const int m = lane & 15, q = lane >> 4, e = m >> 3, g = m & 7;
  if (e == 0 && g < a.G) {
    const float f = bad ? NAN : a.v_scale / lsum;
#pragma unroll
    for (int i = 0; i < 16; ++i) o[i] *= f;
    store_bf16x16(a.out + (static_cast<int64_t>(b) * a.Hq + h * a.G + g) * kHeadDim + 16 * q, o);
  }
}

// Workgroup LDS for partials of items cut once inside the workgroup: two
// piece slots per wave (head piece, tail piece) and one arrival counter per
// chunk of the workgroup.
struct WgLocal {
  float* part;  // [kWavesPerWG][2][kSlotFloats]
  int* cnt;     // [kWavesPerWG]
};

// Process the sub-tiles [cur, wend) of the item line, chunk `cid` of the
// schedule.  Items that lie wholly inside are written out; pieces of items
// cut by chunk boundaries go through partial slots 2*cid / 2*cid+1 and are
// merged by the last piece to arrive.
template <int BK, bool WINDOWED, bool KP, bool ROPE, class Pre>
__device__ __forceinline__ void process_chunk(const AttnArgs& a, const Pre& s_pre, int B, int cid,
                                              const Sched sc, int64_t cur, int64_t wend,
                                              uint8_t* ring, const WgLocal wg, int64_t per_r,
                                              int half) {
  const int lane = lane_id();
  const int m = lane & 15, q = lane >> 4, e = m >> 3, g = m & 7;
  const int64_t wbeg = cur;
  // locate the first item: the last b with pre(b) * Hkv <= cur (uniform)
  int b = s_pre.last_at_or_below(B, a.Hkv, cur);
  int n = s_pre(b + 1) - s_pre(b);
  int64_t rel = cur - static_cast<int64_t>(s_pre(b)) * a.Hkv;
  int h = __builtin_amdgcn_readfirstlane(static_cast<int>(rel / n));
  int j = __builtin_amdgcn_readfirstlane(static_cast<int>(rel % n));

  while (cur < wend && b < B) {
    n = __builtin_amdgcn_readfirstlane(s_pre(b + 1) - s_pre(b));
    const int pre_b = __builtin_amdgcn_readfirstlane(s_pre(b));
    const int seg = static_cast<int>(min(static_cast<int64_t>(n - j), wend - cur));
    const int64_t item_beg = static_cast<int64_t>(pre_b) * a.Hkv + static_cast<int64_t>(h) * n;
    // The item's frame position (from the prefix's registers when it has
    // them), its first table window and its queries are loaded together.
    // Without a window the keys start at 0, so the first sub-tile (j) and its
    // table window do not depend on the position.
    const int fp_raw = s_pre.pos(a, b);
    Item<BK, WINDOWED, KP> it(a, b, h);
    // without a window: the window must hold column jr*kSub/BK; only an item
    // shorter than a share can carry a start cost (jr = j - kItemCost)
    // (in halves mode the whole item, at most kTinyItem sub-tiles, is inside a
    // window from column 0)
    if (!WINDOWED)
      it.load_window(half > 0 ? 0 : ((n < per_r + kItemCost ? max(j - kItemCost, 0) : j) * kSub) / BK);
    u32x4_t q0 = {0u, 0u, 0u, 0u}, q1 = {0u, 0u, 0u, 0u};
    if (g < a.G) {
      const uint16_t* qp = a.q + (static_cast<int64_t>(b) * a.Hq + h * a.G + g) * kHeadDim + 16 * q;
      q0 = *reinterpret_cast<const u32x4_t*>(qp);
      q1 = *reinterpret_cast<const u32x4_t*>(qp + 8);
    }
    // rotary cos/sin of the lane's dims 16q .. 16q+15 (frequencies 16(q&1) ..)
    f32x4_t rc[4], rs[4];
    constexpr bool rope = ROPE;
    if (rope) {
      const int64_t ro = static_cast<int64_t>(b) * (kHeadDim / 2) + 16 * (q & 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rc[i] = *reinterpret_cast<const f32x4_t*>(a.rope_cos + ro + 4 * i);
        rs[i] = *reinterpret_cast<const f32x4_t*>(a.rope_sin + ro + 4 * i);
      }
    }
    // the new token's K/V rows (fused write), fetched with the queries; used
    // only by the segment holding the token
    uint16_t kn_bits = 0, vn_bits = 0;
    float kn_c = 1.f, kn_s = 0.f;
    int64_t upd_b = -1;
    if (a.k_new != nullptr) {
      const int64_t row = (static_cast<int64_t>(b) * a.Hkv + h) * kHeadDim + lane;
      kn_bits = a.k_new[row];
      vn_bits = a.v_new[row];
      upd_b = a.upd[b];
      if (rope) {
        const int64_t ci = static_cast<int64_t>(b) * (kHeadDim / 2) + (lane & (kHeadDim / 2 - 1));
        kn_c = a.rope_cos[ci];
        kn_s = a.rope_sin[ci];
      }
    }
    const int hi = __builtin_amdgcn_readfirstlane(fp_raw);
    const int lo = WINDOWED ? max(0, hi - a.window + 1) : 0;
    it.set_range(lo, hi);
    // On the line the item holds c0 virtual sub-tiles (a start cost of 0 or
    // kItemCost, or in halves mode the padding that centres its sub-tiles on
    // the boundary of its two shares), then its nr sub-tiles, then (halves
    // mode only) trailing padding: this piece's sub-tiles are [jr, jr + segr).
    const int nr = hi / kSub - lo / kSub + 1;
    const int c0 = half > 0 ? half - (nr + 1) / 2 : n - nr;
    const int jr = max(j - c0, 0);
    const int segr = min(max(0, j + seg - c0 - jr), nr - jr);
    const int64_t real_beg = item_beg + c0;  // where the item's sub-tiles start on the line
    const int64_t real_end = real_beg + nr;  // ... and end
    if (segr <= 0) {
      // the piece covers only virtual sub-tiles: no keys, no partial
      cur += seg;
      j = 0;
      if (++h == a.Hkv) {
        h = 0;
        do {
          ++b;
        } while (b < B && s_pre(b + 1) == s_pre(b));
        b = __builtin_amdgcn_readfirstlane(b);
      }
      continue;
    }
    if (WINDOWED) it.load_window(it.clampc(((lo / kSub + jr) * kSub) / BK));

    const int t0 = lo / kSub + jr;
    const int tlast = t0 + segr - 1;
    // The first run of a segment is shortened by a per-wave amount so that the
    // waves of a workgroup reach their run boundaries (where the ring drains
    // and refills) at different times and cover each other's bubbles.
    Segment<Item<BK, WINDOWED, KP>> seg_run(
        it, ring, t0, tlast,
        __builtin_amdgcn_readfirstlane(kWinEntries - 16 * ((threadIdx.x >> 6) & 3)));
    // the first run's K/V loads go out before anything waits for the queries
    // or the new token's rows, so those loads overlap the ring fill
    seg_run.start_run();

    uint32_t qx[4][4], qxl[4][4];
    if (rope) {
      u32x4_t l0, l1;
      rotate_queries(q0, q1, l0, l1, rc, rs, q >= 2);
      expand_queries(l0, l1, e, qxl);
    }
    expand_queries(q0, q1, e, qx);

    // The new token (frame position hi) is in sub-tile t_new; with a fused
    // write, the segment holding it quantises the token's K/V (lane j: dim j),
    // patches them into that sub-tile's slot before it is read, and stores
    // them into the cache slot of position hi.
    const int t_new = (a.k_new != nullptr && hi / kSub >= lo / kSub + jr &&
                       hi / kSub < lo / kSub + jr + segr) ? hi / kSub : -1;
    uint32_t kcode = 0, vcode = 0;
    if (t_new >= 0) new_token_codes<ROPE>(a, kn_bits, vn_bits, kn_c, kn_s, kcode, vcode);
    State s;
    reset_state(s);
    if constexpr (ROPE)
      seg_run.template stream<KP, true>(a.score_scale, lo, hi, t_new, upd_b, kcode, vcode, qx, qxl, s);
    else
      seg_run.template stream<KP>(a.score_scale, lo, hi, t_new, upd_b, kcode, vcode, qx, qx, s);

    // ---- finish the piece
    float o[16];
    float lsum;
    bool bad;
    finish_piece(s, o, lsum, bad);

    const bool whole = (real_beg >= wbeg) && (real_end <= wend);
    if (whole) {
      store_whole(a, b, h, o, lsum, bad);
    } else if (sc.of(real_end - 1) == sc.of(real_beg) + 1 &&
               sc.of(real_beg) / kWavesPerWG == sc.of(real_end - 1) / kWavesPerWG) {
      // cut once, both pieces in this workgroup: hand off through LDS
      const int cf = sc.of(real_beg), cl = cf + 1;
      const int slot = (real_beg >= wbeg) ? 1 : 0;
      write_partial_lds(wg.part + (2 * (cid % kWavesPerWG) + slot) * kSlotFloats, o, s.m,
                        bad ? NAN : lsum, lane);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      int old = 0;
      if (lane == 0)
        old = __hip_atomic_fetch_add(wg.cnt + cf % kWavesPerWG, 1, __ATOMIC_ACQ_REL,
                                     __HIP_MEMORY_SCOPE_WORKGROUP);
      old = __builtin_amdgcn_readlane(old, 0);
      if (old == 1) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        merge_item<2>(a, b, h, 2, lane,
                      LdsPieces{wg.part + (2 * (cf % kWavesPerWG) + 1) * kSlotFloats,
                                wg.part + (2 * (cl % kWavesPerWG) + 0) * kSlotFloats});
      }
    } else {
      const int cf = sc.of(real_beg), cl = sc.of(real_end - 1);
      const int slot = (real_beg >= wbeg) ? 2 * cid + 1 : 2 * cid;
      write_partial(a, slot, o, s.m, bad ? NAN : lsum, lane);
      wait_vm_stores();
      int old = 0;
      int32_t* ctr = a.counters + static_cast<int64_t>(b) * a.Hkv + h;
      if (lane == 0) old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      old = __builtin_amdgcn_readlane(old, 0);
      const int ncontrib = cl - cf + 1;
      if (old == ncontrib - 1) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        merge_item<8>(a, b, h, ncontrib, lane, SlotPieces{partial_rsrc(a), cf});
        if (lane == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }

    cur += seg;
    j = 0;
    if (++h == a.Hkv) {
      h = 0;
      do {
        ++b;
      } while (b < B && s_pre(b + 1) == s_pre(b));
      b = __builtin_amdgcn_readfirstlane(b);
    }
  }
}

// Items of at most kTinyItem sub-tiles are split between two waves of one
// workgroup (two shares of `half` sub-tiles each, the item's sub-tiles centred
// on their boundary, the two pieces merged through LDS) when the launch has
// two waves per item: each wave's dependent chain of set-up loads, K/V loads
// and sub-tiles is then about half as long.  Full and window launches decide
// alike, so a window launch over contexts that fit the window reproduces the
// full launch bit for bit.
__device__ __forceinline__ bool halves_fit(int longest, int64_t items, int workers) {
  return longest >= 2 && longest <= kTinyItem && 2 * items <= workers;
}

// Everything after the prefix: rows without work, the static split of the
// item line over the W waves, and the wave's share.
template <int BK, bool WINDOWED, bool KP, bool ROPE, class Pre>
__device__ __forceinline__ void run_shares(const AttnArgs& a, const Pre& pre, int B, int longest,
                                           uint8_t* ring, const WgLocal wg, int64_t per_r,
                                           int half) {
  const int tid = threadIdx.x;
  // rows with no work: +0 for inactive sequences, NaN for invalid positions
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    if (pre(b + 1) != pre(b)) continue;
    int lo = 0;
    bool inv;
    seq_subtiles<BK, WINDOWED>(a, a.frame_pos[b], &lo, &inv);
    const uint16_t fill = inv ? 0x7fc0u : 0u;
    const uint32_t f2 = static_cast<uint32_t>(fill) * 0x10001u;
    u32x4_t* row = reinterpret_cast<u32x4_t*>(a.out + static_cast<int64_t>(b) * a.Hq * kHeadDim);
    for (int i = tid; i < a.Hq * kHeadDim / 8; i += kThreads) row[i] = u32x4_t{f2, f2, f2, f2};
  }

  // Static split of the item line over the W waves: wave w's share is the
  // sub-tile range [w*per, (w+1)*per).  Short items are never cut: when every
  // item is tiny or at most half a share, wave w takes the whole items whose
  // first sub-tile falls in its share (no partials, no merge); otherwise
  // shares are exact and cut items are merged through the workspace.
  const int64_t total = static_cast<int64_t>(__builtin_amdgcn_readfirstlane(pre(B))) * a.Hkv;
  if (total == 0) return;
  const int W = a.n_workers;
  const int wid = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerWG + (tid >> 6));
  // halves mode: every item is exactly two shares of `half` sub-tiles
  const int64_t per = half > 0 ? half : (total + W - 1) / W;
  const int64_t cb = static_cast<int64_t>(wid) * per;
  const bool whole_items =
      half == 0 && (longest <= kTinyItem || 2 * static_cast<int64_t>(longest) <= per);
  if (!whole_items) {
    // items may be cut: clear the workgroup's LDS arrival counters (every
    // wave of the workgroup gets here; the decision is the same for all)
    if (tid < kWavesPerWG) wg.cnt[tid] = 0;
    __syncthreads();
  }
  if (cb >= total) return;
  const Sched sc{per};
  if (whole_items) {
    const int64_t lo_w = first_item_start_at_or_after(pre, B, a.Hkv, cb);
    const int64_t hi_w = first_item_start_at_or_after(pre, B, a.Hkv, min(cb + per, total));
    if (lo_w < hi_w)
      process_chunk<BK, WINDOWED, KP, ROPE>(a, pre, B, wid, sc, lo_w, hi_w, ring, wg, per_r, 0);
  } else {
    process_chunk<BK, WINDOWED, KP, ROPE>(a, pre, B, wid, sc, cb, min(cb + per, total), ring, wg,
                                          per_r, half);
  }
}

template <int BK, bool WINDOWED, bool KP, bool ROPE>
__global__ void __launch_bounds__(kThreads, kWGPerCU * kWavesPerWG / 4) decode_attn_kernel(AttnArgs a) {
  extern __shared__ int s_pre[];  // [B + 1] prefix of per-sequence sub-tile counts
  __shared__ int s_longest;       // longest item, in sub-tiles
  __shared__ int s_active;        // sequences with work (window launches)
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[kWavesPerWG * kDepth * kSlotBytes];
  __shared__ __attribute__((aligned(16))) float s_part[kWavesPerWG * 2 * kSlotFloats];
  __shared__ int s_cnt[kWavesPerWG];
  uint8_t* ring = s_ring + (threadIdx.x >> 6) * (kDepth * kSlotBytes);
  const int tid = threadIdx.x;
  const int B = a.B;
  const WgLocal wg{s_part, s_cnt};
  if (B <= kWave) {
    // Every wave scans the (at most 64) positions in registers: no LDS, no
    // barrier between the position load and the wave's first item.
    const int lane = tid & (kWave - 1);
    int n = 0, posv = 0;
    if (lane < B) {
      int lo = 0;
      bool inv;
      posv = a.frame_pos[lane];
      n = seq_subtiles<BK, WINDOWED>(a, posv, &lo, &inv);
    }
    const int x = wave_inclusive_sum(n);  // inclusive prefix over the lanes
    // in real sub-tiles: decides whether items may be cut
    const int longest = __builtin_amdgcn_readfirstlane(wave_max_i32(n));
    const uint64_t am = __ballot(n > 0);  // sequences with work
    const int64_t items = static_cast<int64_t>(__popcll(am)) * a.Hkv;
    int64_t per_r = 0;
    int half = 0;
    int v = n, xv = x;
    bool rescan = false;
    if (halves_fit(longest, items, a.n_workers)) {
      // every item with work is 2*half long on the line: the prefix is that
      // times the number of such sequences before this lane
      half = (longest + 1) / 2;
      const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(am >> 32),
                                                  __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(am), 0));
      v = n > 0 ? 2 * half : 0;
      xv = 2 * half * below + v;
    } else if constexpr (!WINDOWED) {
      // each short item also counts its start cost (kItemCost)
      per_r = (static_cast<int64_t>(__builtin_amdgcn_readlane(x, kWave - 1)) * a.Hkv +
               a.n_workers - 1) / a.n_workers;
      if (__ballot(n > 0 && n < per_r) != 0) {  // some item is short: redo the prefix
        v = (n > 0 && n < per_r) ? n + kItemCost : n;
        rescan = true;
      }
    }
    if (rescan) xv = wave_inclusive_sum(v);
    const PreReg pre{xv - v, __builtin_amdgcn_readlane(xv, kWave - 1), posv};
    run_shares<BK, WINDOWED, KP, ROPE>(a, pre, B, longest, ring, wg, per_r, half);
  } else {
    if (tid == 0) {
      s_longest = 0;
      s_active = 0;
    }
    __syncthreads();
    int longest = 0;  // in real sub-tiles: decides whether items may be cut
    int active = 0;   // sequences with work
    constexpr int kPerThread = WINDOWED ? 1 : (kMaxBatch + kThreads - 1) / kThreads;
    int nl[kPerThread];  // full launches keep their counts for the rewrites below
    if constexpr (WINDOWED) {
      for (int b = tid; b < B; b += kThreads) {
        int lo = 0;
        bool inv;
        const int n = seq_subtiles<BK, WINDOWED>(a, a.frame_pos[b], &lo, &inv);
        s_pre[b] = n;
        longest = max(longest, n);
        active += n > 0;
      }
    } else {
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) {
        const int b = tid + k * kThreads;
        nl[k] = 0;
        if (b < B) {
          int lo = 0;
          bool inv;
          nl[k] = seq_subtiles<BK, WINDOWED>(a, a.frame_pos[b], &lo, &inv);
          s_pre[b] = nl[k];
          longest = max(longest, nl[k]);
          active += nl[k] > 0;
        }
      }
    }
    // one LDS atomic per wave and quantity (64 lanes on one address would
    // serialise)
    longest = wave_max_i32(longest);
    active = wave_sum_i32(active);
    if ((tid & 63) == 0) {
      atomicMax(&s_longest, longest);
      atomicAdd(&s_active, active);
    }
    __syncthreads();
    const int lg = __builtin_amdgcn_readfirstlane(s_longest);
    const int64_t items = static_cast<int64_t>(s_active) * a.Hkv;
    int64_t per_r = 0;
    int half = 0;
    if (halves_fit(lg, items, a.n_workers)) {
      half = (lg + 1) / 2;
      for (int b = tid; b < B; b += kThreads) s_pre[b] = s_pre[b] > 0 ? 2 * half : 0;
      __syncthreads();
    } else if constexpr (!WINDOWED) {
      // each short item also counts its start cost (kItemCost): redo the prefix
      block_exclusive_scan(s_pre, B);
      per_r = (static_cast<int64_t>(s_pre[B]) * a.Hkv + a.n_workers - 1) / a.n_workers;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k) {
        const int b = tid + k * kThreads;
        if (b < B) s_pre[b] = (nl[k] > 0 && nl[k] < per_r) ? nl[k] + kItemCost : nl[k];
      }
      __syncthreads();
    }
    block_exclusive_scan(s_pre, B);
    run_shares<BK, WINDOWED, KP, ROPE>(a, PreLds{s_pre}, B, lg, ring, wg, per_r, half);
  }
  wait_vmcnt<0>();  // no direct-to-LDS load outlives the wave
}

// ---- direct launches ----------------------------------------------------------
// When the items of a launch are short enough not to need balancing -- every
// sliding-window launch (a window of up to 224 keys spans at most 8
// sub-tiles), full launches whose tables cover at most 8 sub-tiles, and
// launches of items up to 32 sub-tiles with enough of them to fill the GPU
// -- item (b, h) = (i / Hkv, i % Hkv) gets `pieces` waves (1, 2 or 4) of one
// workgroup straight from its index.  No position scan, no item search: the
// item's position, its first table window, its queries and its new token's
// rows are fetched in one round trip, and the K/V loads go out as soon as the
// position is known.  With several pieces the item's nr sub-tiles are split
// into consecutive parts of nr / pieces (the first nr % pieces parts one
// more) and the parts merge, in order, through LDS; a two-piece split is the
// same as the stream-K kernel's two-waves-per-item mode, so both kernels give
// identical bits for the same items.
constexpr int kDirectMax = 8;        // longest item (sub-tiles) always run directly
constexpr int kDirectMaxWide = 32;   // ... and when the items fill the resident waves
constexpr int kDirectWGPerCU = 2;    // workgroups per CU the direct kernel is compiled for
constexpr int kDirectRegs = 1;       // table entries in registers: 64 per window

template <int BK, bool WINDOWED, bool KP, bool ROPE>
__global__ void __launch_bounds__(kThreads, kDirectWGPerCU * kWavesPerWG / 4)
    decode_attn_direct_kernel(AttnArgs a, int pieces_log2) {
  __shared__ __attribute__((aligned(16))) uint8_t s_ring[kWavesPerWG * kDepth * kSlotBytes];
  __shared__ __attribute__((aligned(16))) float s_part[kWavesPerWG * kSlotFloats];
  __shared__ int s_cnt[kWavesPerWG];
  // wave-uniform indices (readfirstlane: the compiler cannot tell that
  // threadIdx.x >> 6 is uniform, and the buffer descriptors need SGPRs)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int m = lane & 15, q = lane >> 4, e = m >> 3, g = m & 7;
  uint8_t* ring = s_ring + wave * (kDepth * kSlotBytes);
  // 32-bit indices (the host launches at most INT32_MAX waves): a 64-bit
  // division by the head count took ~280 scalar instructions ahead of the
  // first load
  const uint32_t wid = blockIdx.x * static_cast<uint32_t>(kWavesPerWG) + wave;
  const int pieces = 1 << pieces_log2;  // 1, 2 or 4
  const uint32_t item = wid >> pieces_log2;
  const int piece = __builtin_amdgcn_readfirstlane(static_cast<int>(wid & (pieces - 1)));
  const uint32_t hkv = static_cast<uint32_t>(a.Hkv);
  const bool live = item < static_cast<uint32_t>(a.B) * hkv;
  const int b = __builtin_amdgcn_readfirstlane(live ? static_cast<int>(item / hkv) : 0);
  const int h = __builtin_amdgcn_readfirstlane(live ? static_cast<int>(item - b * hkv) : 0);

  // ---- set-up loads, none of which depends on the position
  const int fp = __builtin_amdgcn_readfirstlane(live ? a.frame_pos[b] : -1);
  Item<BK, WINDOWED, KP, kDirectRegs> it(a, b, h);
  it.load_window(0);
  u32x4_t q0 = {0u, 0u, 0u, 0u}, q1 = {0u, 0u, 0u, 0u};
  if (live && g < a.G) {
    const uint16_t* qp = a.q + (static_cast<int64_t>(b) * a.Hq + h * a.G + g) * kHeadDim + 16 * q;
    q0 = *reinterpret_cast<const u32x4_t*>(qp);
    q1 = *reinterpret_cast<const u32x4_t*>(qp + 8);
  }
  f32x4_t rc[4], rs[4];
  if (ROPE) {
    const int64_t ro = static_cast<int64_t>(b) * (kHeadDim / 2) + 16 * (q & 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rc[i] = *reinterpret_cast<const f32x4_t*>(a.rope_cos + ro + 4 * i);
      rs[i] = *reinterpret_cast<const f32x4_t*>(a.rope_sin + ro + 4 * i);
    }
  }
  uint16_t kn_bits = 0, vn_bits = 0;
  float kn_c = 1.f, kn_s = 0.f;
  int64_t upd_b = -1;
  if (a.k_new != nullptr && live) {
    const int64_t row = (static_cast<int64_t>(b) * a.Hkv + h) * kHeadDim + lane;
    kn_bits = a.k_new[row];
    vn_bits = a.v_new[row];
    upd_b = a.upd[b];
    if (ROPE) {
      const int64_t ci = static_cast<int64_t>(b) * (kHeadDim / 2) + (lane & (kHeadDim / 2 - 1));
      kn_c = a.rope_cos[ci];
      kn_s = a.rope_sin[ci];
    }
  }
  if (pieces > 1) {
    // the items' LDS arrival counters start at zero (every wave gets here)
    if (threadIdx.x < kWavesPerWG) s_cnt[threadIdx.x] = 0;
    __syncthreads();
  }
  if (!live) return;

  int lo = 0;
  bool invalid;
  const int nr = seq_subtiles<BK, WINDOWED>(a, fp, &lo, &invalid);
  if (nr == 0) {
    // no work: +0 rows for an inactive sequence, NaN for a position beyond
    // the table; the first piece writes the item's G rows
    if (piece == 0) {
      const uint32_t f2 = invalid ? 0x7fc07fc0u : 0u;
      const int gg = lane >> 3, part = lane & 7;
      if (gg < a.G)
        *reinterpret_cast<u32x4_t*>(a.out + (static_cast<int64_t>(b) * a.Hq + h * a.G + gg) *
                                                kHeadDim + 8 * part) = u32x4_t{f2, f2, f2, f2};
    }
    return;
  }
  const int hi = fp;
  it.set_range(lo, hi);
  // this piece's part of the nr sub-tiles; only the first min(pieces, nr)
  // parts hold any
  const int each = nr >> pieces_log2, extra = nr & (pieces - 1);
  const int segr = each + (piece < extra ? 1 : 0);
  if (segr <= 0) return;
  const int npieces = min(pieces, nr);
  const int t0 = lo / kSub + piece * each + min(piece, extra);
  const int tlast = t0 + segr - 1;

  Segment<Item<BK, WINDOWED, KP, kDirectRegs>> sg(it, ring, t0, tlast, it.kEntries);
  sg.start_run();
  uint32_t qx[4][4], qxl[4][4];
  if (ROPE) {
    u32x4_t l0, l1;
    rotate_queries(q0, q1, l0, l1, rc, rs, q >= 2);
    expand_queries(l0, l1, e, qxl);
  }
  expand_queries(q0, q1, e, qx);
  const int t_new = (a.k_new != nullptr && hi / kSub >= t0 && hi / kSub <= tlast) ? hi / kSub : -1;
  uint32_t kcode = 0, vcode = 0;
  if (t_new >= 0) new_token_codes<ROPE>(a, kn_bits, vn_bits, kn_c, kn_s, kcode, vcode);
  State s;
  reset_state(s);
  if constexpr (ROPE)
    sg.template stream<KP, true>(a.score_scale, lo, hi, t_new, upd_b, kcode, vcode, qx, qxl, s);
  else
    sg.template stream<KP>(a.score_scale, lo, hi, t_new, upd_b, kcode, vcode, qx, qx, s);
  wait_vmcnt<0>();

  float o[16];
  float lsum;
  bool bad;
  finish_piece(s, o, lsum, bad);
  if (npieces == 1) {
    store_whole(a, b, h, o, lsum, bad);
    return;
  }
  // several pieces: each writes its partial to its wave's LDS slot; the last
  // to arrive merges them in piece order (the item's waves are consecutive)
  write_partial_lds(s_part + wave * kSlotFloats, o, s.m, bad ? NAN : lsum, lane);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  int old = 0;
  const int slot0 = wave - piece;
  if (lane == 0)
    old = __hip_atomic_fetch_add(s_cnt + slot0, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
  old = __builtin_amdgcn_readlane(old, 0);
  if (old == npieces - 1) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    // two pieces in one round of two (the same operations, in the same order,
    // as a round of four over two pieces)
    if (npieces == 2)
      merge_item<2>(a, b, h, 2, lane, LdsSlots{s_part + slot0 * kSlotFloats});
    else
      merge_item<kWavesPerWG>(a, b, h, npieces, lane, LdsSlots{s_part + slot0 * kSlotFloats});
  }
}

// Grid of a launch: `pieces` > 0 selects the direct kernel (n_wg workgroups,
// `pieces` waves per item), 0 the stream-K kernel (n_wg workgroups, `lds`
// bytes of dynamic LDS for the prefix).
struct Grid {
  int n_wg;
  int pieces;
  size_t lds;
};

template <int BK, bool WINDOWED, bool KP, bool ROPE>
hipError_t launch(const AttnArgs& a, const Grid& gr, hipStream_t stream) {
  if (gr.pieces > 0)
    hipLaunchKernelGGL((decode_attn_direct_kernel<BK, WINDOWED, KP, ROPE>), dim3(gr.n_wg),
                       dim3(kThreads), 0, stream, a, gr.pieces == 4 ? 2 : gr.pieces == 2 ? 1 : 0);
  else
    hipLaunchKernelGGL((decode_attn_kernel<BK, WINDOWED, KP, ROPE>), dim3(gr.n_wg), dim3(kThreads),
                       gr.lds, stream, a);
  return hipGetLastError();
}

template <int BK, bool ROPE>
hipError_t launch_kp(const AttnArgs& a, bool win, bool kp, const Grid& gr, hipStream_t stream) {
  if (kp)
    return win ? launch<BK, true, true, ROPE>(a, gr, stream)
               : launch<BK, false, true, ROPE>(a, gr, stream);
  return win ? launch<BK, true, false, ROPE>(a, gr, stream)
             : launch<BK, false, false, ROPE>(a, gr, stream);
}

// The rotary variant is a separate instantiation so that calls without it run
// the kernel without its code.
template <int BK>
hipError_t launch_bk(const AttnArgs& a, bool win, bool kp, const Grid& gr, hipStream_t stream) {
  return a.rope_cos != nullptr ? launch_kp<BK, true>(a, win, kp, gr, stream)
                               : launch_kp<BK, false>(a, win, kp, gr, stream);
}

// Waves per item of a direct launch (0: run the stream-K kernel).  Items of
// at most kDirectMax sub-tiles always run directly, longer ones up to
// kDirectMaxWide when the items alone fill at least half the resident waves.
// An item gets as many pieces (4, 2, 1) as the resident waves hold for every
// item, but no more than half its sub-tiles -- or, while the launch stays at
// one wave per SIMD, no more than its sub-tiles (a window item of 4-5
// sub-tiles in four pieces: an 8-sequence window launch 5.93 -> 5.41 us; at
// two waves per SIMD the same split was slower, 6.31 -> 6.46 us for 64
// sequences).
int direct_pieces(int64_t batch, int kv_heads, int64_t longest, int cus) {
  const int64_t items = batch * kv_heads;
  const int64_t one_per_simd = static_cast<int64_t>(cus > 0 ? cus : 256) * 4;  // four SIMDs per CU
  const int64_t resident = static_cast<int64_t>(cus > 0 ? cus : 256) * kDirectWGPerCU * kWavesPerWG;
  if (longest > kDirectMaxWide || (longest > kDirectMax && 2 * items < resident)) return 0;
  for (int p = kWavesPerWG; p > 1; p /= 2)
    if (p * items <= resident && (2 * p <= longest || (p <= longest && p * items <= one_per_simd))) return p;
  return 1;
}

// The most sub-tiles one item of a launch can span: keys lie in frame
// positions [lo, hi] with hi < table_width * block; a window of W keys can
// start anywhere inside a sub-tile.
int64_t longest_item(int block, int table_width, int window) {
  const int64_t full = (static_cast<int64_t>(table_width) * block + kSub - 1) / kSub;
  if (window <= 0) return full;
  return std::min<int64_t>(full, (static_cast<int64_t>(window) + 2 * kSub - 2) / kSub);
}

}  // namespace

int attn_workers(int64_t batch, int kv_heads, int max_subtiles) {
  const int64_t total = batch * kv_heads * static_cast<int64_t>(max_subtiles);
  int64_t w = (total + kMinSubtilesPerWorker - 1) / kMinSubtilesPerWorker;
  // short items: up to two waves each (window launches split each item
  // between two waves of one workgroup when the launch has them)
  if (w < 2 * batch * kv_heads) w = 2 * batch * kv_heads;
  w = (w + kWavesPerWG - 1) / kWavesPerWG * kWavesPerWG;
  if (w < kWavesPerWG) w = kWavesPerWG;
  if (w > kMaxWorkers) w = kMaxWorkers / kWavesPerWG * kWavesPerWG;
  return static_cast<int>(w);
}

int attn_max_subtiles(int block, int table_width, int window) {
  int64_t keys = static_cast<int64_t>(table_width) * block;
  if (window > 0 && window < keys) keys = window;
  return static_cast<int>((keys + kSub - 1) / kSub + 1);
}

// Workspace layout: [arrival counters, B*Hkv int32][reserved][partial slots,
// 2 per chunk, one chunk per worker], each region 256-byte aligned.
static int64_t counters_bytes(int64_t batch, int kv_heads) {
  return (batch * kv_heads * 4 + 255) / 256 * 256;
}
constexpr int64_t kQueueBytes = 256;

int64_t attn_workspace_bytes(int64_t batch, int kv_heads, int n_workers) {
  return counters_bytes(batch, kv_heads) + kQueueBytes +
         static_cast<int64_t>(2) * n_workers * kSlotBytesF;
}

hipError_t launch_decode_attn(const AttnLaunch& L, hipStream_t stream) {
  AttnArgs a;
  a.q = L.q;
  a.k = L.k;
  a.v = L.v;
  a.table = L.table;
  a.frame_pos = L.frame_pos;
  a.out = L.out;
  const int64_t ctr = counters_bytes(L.B, L.Hkv);
  a.counters = reinterpret_cast<int32_t*>(L.workspace);
  a.partial = reinterpret_cast<float*>(reinterpret_cast<char*>(L.workspace) + ctr + kQueueBytes);
  a.nb = L.nb;
  a.B = L.B;
  a.Hq = L.Hq;
  a.Hkv = L.Hkv;
  a.G = L.Hq / L.Hkv;
  a.bt_stride = L.bt_stride;
  a.table_width = L.table_width;
  a.window = L.window;
  a.score_scale = L.sm_scale * L.k_scale * 1.4426950408889634f;
  a.v_scale = L.v_scale;
  a.k_scale = L.k_scale;
  a.k_new = L.k_new;
  a.v_new = L.v_new;
  a.rope_cos = L.rope_cos;
  a.rope_sin = L.rope_sin;
  a.k_w = L.k_w;
  a.v_w = L.v_w;
  a.upd = L.upd;
  a.n_workers = L.n_workers;
  a.partial_bytes = static_cast<int32_t>(static_cast<int64_t>(2) * L.n_workers * kSlotBytesF);
  // the workspace holds partial slots for at most this many workers
  if (a.n_workers < kWavesPerWG || a.n_workers > kMaxWorkers || a.n_workers % kWavesPerWG)
    return hipErrorInvalidValue;
  // never launch more workers than can be resident together (the CU count
  // of each device is cached; concurrent callers may both query it)
  static std::atomic<int> cu_count[64];
  int dev = 0;
  int cus = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    cus = cu_count[dev].load(std::memory_order_relaxed);
    if (!cus && hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      cu_count[dev].store(cus, std::memory_order_relaxed);
    const int resident = cus * kWGPerCU * kWavesPerWG;
    if (resident >= kWavesPerWG && a.n_workers > resident) a.n_workers = resident;
  }
  Grid gr{a.n_workers / kWavesPerWG, 0, static_cast<size_t>(L.B + 1) * sizeof(int)};
  gr.pieces = direct_pieces(L.B, L.Hkv, longest_item(L.block, L.table_width, L.window), cus);
  if (gr.pieces > 0) {
    const int64_t items = static_cast<int64_t>(L.B) * L.Hkv;
    // the kernel indexes waves in 32 bits
    if (items * gr.pieces > INT32_MAX) return hipErrorInvalidValue;
    gr.n_wg = static_cast<int>((items * gr.pieces + kWavesPerWG - 1) / kWavesPerWG);
  }
  const bool win = L.window > 0;
  switch (L.block) {
    case 16: return launch_bk<16>(a, win, L.k_packed != 0, gr, stream);
    case 32: return launch_bk<32>(a, win, L.k_packed != 0, gr, stream);
    case 64: return launch_bk<64>(a, win, L.k_packed != 0, gr, stream);
    case 128: return launch_bk<128>(a, win, L.k_packed != 0, gr, stream);
    default: return hipErrorInvalidValue;
  }
}

// ---- the library's own workspace, for pkv_decode_layer_noalloc -------------
// Callers that cannot allocate device memory (work under HIP graph capture,
// tight serving loops) get the split-KV workspace from this array instead of
// an argument.  Each GPU the library runs on holds its own copy until the
// process ends; every call on a GPU shares it, so calls that overlap on one
// GPU race.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t attn_scratch(void** ptr) {
  // The array's name is a host-side stand-in: its device address is looked
  // up once per device, with that device current, and kept.
  static std::atomic<void*> addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  void* p = (dev >= 0 && dev < 64) ? addr[dev].load(std::memory_order_acquire) : nullptr;
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    if (dev >= 0 && dev < 64) addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_decode_attn_scratch(const AttnLaunch& L0, hipStream_t stream) {
  if (attn_workspace_bytes(L0.B, L0.Hkv, L0.n_workers) > kScratchBytes) return hipErrorInvalidValue;
  void* p = nullptr;
  hipError_t e = attn_scratch(&p);
  if (e != hipSuccess) return e;
  AttnLaunch L = L0;
  L.workspace = p;
  // the arrival counters must start at zero: clear them on every call (a
  // fill kernel rather than a memset node, so the call can be captured)
  const int64_t words = counters_bytes(L.B, L.Hkv) / 4;
  hipLaunchKernelGGL(zero_words_kernel, dim3(static_cast<unsigned>((words + 255) / 256)), dim3(256),
                     0, stream, static_cast<uint32_t*>(p), words);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_attn(L, stream);
}

}  // namespace pkv

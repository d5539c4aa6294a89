// Read-bandwidth probes for the HBM ceiling the attention kernel is measured
// against (C ABI declared in include/pkv_probe.h).
//
// The attention kernel's traffic is whole K and V tiles (block * head_dim
// bytes each, 2 KiB at block 32) at table-chosen places in a pool far larger
// than the 256 MB Infinity Cache.  Two probes bound what any kernel can do
// with that traffic on this part:
//   - stream: every 16-byte word of a buffer read once, consecutive lanes on
//     consecutive words (the best case for the memory system);
//   - tiles: whole tiles of a given size, each read once, in an order that a
//     bijective scramble of the tile index makes look random (the gather the
//     paged layout makes).
// Both read with plain or non-temporal loads, and fold everything they read
// into one XOR per workgroup (stored to its own word: no atomics, whose
// serialisation on one address would add ~10 ns per wave to the launch), so
// the loads stay live and the host can check that every byte was read exactly
// once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pkv_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // four waves
constexpr int kWaves = kThreads / 64;
constexpr int kStreamUnroll = 8;  // 16-byte loads in flight per lane (stream)
constexpr int kTileKiBInFlight = 16;  // KiB in flight per wave (tiles)

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

__device__ __forceinline__ uint32_t fold(u32x4 r) { return r.x ^ r.y ^ r.z ^ r.w; }

// The workgroup's XOR into sink[blockIdx.x]: a butterfly over each wave's
// 64 lanes, then the four waves through LDS.
__device__ __forceinline__ void publish(uint32_t acc, uint32_t* sink) {
  __shared__ uint32_t s_acc[kWaves];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) s_acc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) x ^= s_acc[w];
    sink[blockIdx.x] = x;
  }
}

// Word i of n16 is read by thread i mod (grid * 256).
template <bool NT>
__global__ void __launch_bounds__(kThreads) stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                               uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
    u32x4 r[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) r[u] = load16<NT>(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= fold(r[u]);
  }
  for (; i < n16; i += stride) acc ^= fold(load16<NT>(src + i));
  publish(acc, sink);
}

// A bijection of [0, 2^bits): xor-shifts and odd multipliers modulo 2^bits
// are each invertible on that range.
__device__ __forceinline__ uint64_t scramble(uint64_t x, uint64_t mask, int sh) {
  x ^= x >> sh;
  x = (x * 0x9E3779B97F4A7C15ull) & mask;
  x ^= x >> sh;
  x = (x * 0xBF58476D1CE4E5B9ull) & mask;
  x ^= x >> sh;
  return x;
}

// Wave w reads tiles scramble(w * per_wave + j), j < per_wave; lane l reads
// bytes [16 l, 16 l + 16) of every KiB of a tile.  per_wave is a multiple of
// the tiles in one group, and waves * per_wave <= 2^bits.
template <int TKB, bool NT>
__global__ void __launch_bounds__(kThreads) tile_read_kernel(const u32x4* __restrict__ src, int bits,
                                                             int64_t per_wave, uint32_t* sink) {
  constexpr int kGroup = kTileKiBInFlight / TKB;  // tiles per group
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const uint64_t mask = (bits >= 64) ? ~0ull : ((1ull << bits) - 1);
  const int sh = (bits + 1) / 2;
  uint32_t acc = 0;
  for (int64_t j = 0; j < per_wave; j += kGroup) {
    u32x4 r[kTileKiBInFlight];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const uint64_t t = scramble((uint64_t)(wave * per_wave + j + g), mask, sh);
      const u32x4* tile = src + t * (TKB * 64);  // 64 words of 16 B per KiB
#pragma unroll
      for (int k = 0; k < TKB; ++k) r[g * TKB + k] = load16<NT>(tile + k * 64 + lane);
    }
#pragma unroll
    for (int u = 0; u < kTileKiBInFlight; ++u) acc ^= fold(r[u]);
  }
  publish(acc, sink);
}

bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int log2i(int64_t x) {
  int b = 0;
  while ((int64_t)1 << b < x) ++b;
  return b;
}

int64_t launched(hipError_t e) { return e == hipSuccess ? 0 : PKV_PROBE_ERR_HIP; }

template <int TKB>
int64_t launch_tiles(const void* src, int bits, int64_t per_wave, int32_t grid, int nt, uint32_t* sink,
                     hipStream_t s) {
  const u32x4* p = (const u32x4*)src;
  if (nt) hipLaunchKernelGGL((tile_read_kernel<TKB, true>), dim3(grid), dim3(kThreads), 0, s, p, bits, per_wave, sink);
  else hipLaunchKernelGGL((tile_read_kernel<TKB, false>), dim3(grid), dim3(kThreads), 0, s, p, bits, per_wave, sink);
  return launched(hipGetLastError());
}

}  // namespace

extern "C" int64_t pkv_probe_stream_read(const void* src, int64_t bytes, int32_t grid, int32_t nontemporal,
                                         uint32_t* sink, void* stream) {
  if (!src || !sink || ((uintptr_t)src & 15) || bytes <= 0 || (bytes & 15) || grid < 1 || grid > (1 << 20))
    return PKV_PROBE_ERR_ARG;
  hipStream_t s = (hipStream_t)stream;
  const u32x4* p = (const u32x4*)src;
  if (nontemporal) hipLaunchKernelGGL((stream_read_kernel<true>), dim3(grid), dim3(kThreads), 0, s, p, bytes / 16, sink);
  else hipLaunchKernelGGL((stream_read_kernel<false>), dim3(grid), dim3(kThreads), 0, s, p, bytes / 16, sink);
  const int64_t rc = launched(hipGetLastError());
  return rc ? rc : bytes;
}

extern "C" int64_t pkv_probe_tile_read_bytes(int64_t bytes, int32_t tile_bytes, int32_t grid) {
  if (bytes <= 0 || !pow2(bytes) || grid < 1 || grid > (1 << 20)) return PKV_PROBE_ERR_ARG;
  if (tile_bytes < 1024 || tile_bytes > kTileKiBInFlight * 1024 || !pow2(tile_bytes) || tile_bytes > bytes)
    return PKV_PROBE_ERR_ARG;
  const int64_t tiles = bytes / tile_bytes;
  const int64_t group = kTileKiBInFlight * 1024 / tile_bytes;
  const int64_t waves = (int64_t)grid * kWaves;
  const int64_t per_wave = tiles / waves / group * group;
  return per_wave * waves * tile_bytes;
}

extern "C" int64_t pkv_probe_tile_read(const void* src, int64_t bytes, int32_t tile_bytes, int32_t grid,
                                       int32_t nontemporal, uint32_t* sink, void* stream) {
  const int64_t total = pkv_probe_tile_read_bytes(bytes, tile_bytes, grid);
  if (total < 0 || !src || !sink || ((uintptr_t)src & 15)) return PKV_PROBE_ERR_ARG;
  if (total == 0) return 0;
  const int64_t waves = (int64_t)grid * kWaves;
  const int64_t per_wave = total / waves / tile_bytes;
  const int bits = log2i(bytes / tile_bytes);
  hipStream_t s = (hipStream_t)stream;
  int64_t rc;
  switch (tile_bytes) {
    case 1024: rc = launch_tiles<1>(src, bits, per_wave, grid, nontemporal, sink, s); break;
    case 2048: rc = launch_tiles<2>(src, bits, per_wave, grid, nontemporal, sink, s); break;
    case 4096: rc = launch_tiles<4>(src, bits, per_wave, grid, nontemporal, sink, s); break;
    case 8192: rc = launch_tiles<8>(src, bits, per_wave, grid, nontemporal, sink, s); break;
    default: rc = launch_tiles<16>(src, bits, per_wave, grid, nontemporal, sink, s); break;
  }
  return rc ? rc : total;
}

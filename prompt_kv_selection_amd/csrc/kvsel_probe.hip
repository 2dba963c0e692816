// Streaming-read probes: what HBM delivers to the access patterns of the
// scoring kernels, measured on a plain buffer (a ceiling for the roofline
// fraction, not part of the selection).
//
//  * tile modes: one workgroup per CU of 8 or 4 waves, each wave moving
//    32-row tiles of 256-byte rows (8 KB) into LDS with direct-to-LDS loads
//    (global_load_lds_dwordx4, 1 KB contiguous per instruction), 1, 2 or 4
//    tiles in flight per wave (64 or 128 KB per CU).  A workgroup owns 128 KB blocks in turn, the
//    blocks of a round being consecutive across the grid: the order in which
//    the single-read scoring kernel streams a head's keys.
//  * vector mode: a grid-stride loop of 16-byte loads into registers,
//    four per lane in flight, eight 256-thread workgroups per CU.
// Each wave folds what it read into a checksum (so no load is dead) and
// stores it to sink[wave of the grid].

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvsel_internal.h"

namespace kvsel {
namespace {

constexpr int kTileBytes = 8192;                 // 32 rows of 256 bytes
constexpr int kBlockBytes = 128 * 1024;          // a workgroup's block per round

template <int kWaves, int kDepth, bool kNT = false>
__global__ __launch_bounds__(kWaves * 64, 1) void probe_tiles_kernel(const uint8_t* __restrict__ src,
                                                                     long long blocks, unsigned* __restrict__ sink) {
  constexpr int kTilesPerWave = kBlockBytes / kTileBytes / kWaves;
  static_assert(kWaves * kDepth * kTileBytes <= 128 * 1024, "the ring fits the LDS");
  static_assert(kDepth <= 4, "wait counts below cover four tiles");
  __shared__ uint4 ring[kWaves][kDepth][kTileBytes / 16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long nwg = gridDim.x;
  unsigned acc = 0u;
  // The wave's tiles in order: block b = round * nwg + blockIdx.x, tile t of
  // the wave's kTilesPerWave in that block.
  const long long my_blocks = blocks > blockIdx.x ? (blocks - blockIdx.x + nwg - 1) / nwg : 0;
  const long long tiles = my_blocks * kTilesPerWave;
  auto tile_addr = [&](long long i) {
    const long long b = (i / kTilesPerWave) * nwg + blockIdx.x;
    const int t = (int)(i % kTilesPerWave);
    return src + b * kBlockBytes + (long long)(wave * kTilesPerWave + t) * kTileBytes;
  };
  auto issue = [&](long long i) {
    const uint8_t* g = tile_addr(i);
    const unsigned long long fa = (unsigned long long)(uintptr_t)g;
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(fa >> 32));
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)fa);
    const uint8_t* first = (const uint8_t*)(((unsigned long long)hi << 32) | (unsigned long long)lo);
    const unsigned base = (unsigned)(uintptr_t)ring[wave][i % kDepth];
#pragma unroll
    for (int k = 0; k < kTileBytes / 1024; ++k) {
      const unsigned off = (unsigned)(k * 1024 + lane * 16);
      if constexpr (kNT)  // non-temporal, as the scoring kernels load a K larger than the cache
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                     :
                     : "s"(__builtin_amdgcn_readfirstlane(base + k * 1024)), "v"(off), "s"(first)
                     : "memory", "m0");
      else
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :
                     : "s"(__builtin_amdgcn_readfirstlane(base + k * 1024)), "v"(off), "s"(first)
                     : "memory", "m0");
    }
  };
  long long issued = 0;
  for (; issued < kDepth && issued < tiles; ++issued) issue(issued);
  for (long long i = 0; i < tiles; ++i) {
    // Tile i has landed once at most (issued - i - 1) tiles' loads remain.
    const long long after = issued - i - 1;
    if (after >= 3) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
    else if (after == 2) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if (after == 1) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const uint4 v = ring[wave][i % kDepth][lane * 8 + (int)(i & 7)];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (issued < tiles) {
      issue(issued);
      ++issued;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // Every lane's value: a reduction would cost nothing measurable either.
  if (lane == 0) sink[blockIdx.x * kWaves + wave] = acc;
}

__global__ __launch_bounds__(256) void probe_vector_kernel(const uint4* __restrict__ src, long long n16,
                                                           unsigned* __restrict__ sink) {
  const long long stride = (long long)gridDim.x * blockDim.x;
  long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  unsigned acc = 0u;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ b.y ^ c.z ^ d.w;
  }
  for (; i < n16; i += stride) acc ^= src[i].x;
  if ((threadIdx.x & 63) == 0) sink[(blockIdx.x * (long long)blockDim.x + threadIdx.x) / 64] = acc;
}

}  // namespace

// Sink words the probes write: a word per wave of the grid.
int probe_sink_words(int cus) { return cus * 8 * 256 / 64; }

hipError_t launch_probe(int mode, const void* src, long long bytes, unsigned* sink, int cus, hipStream_t st) {
  if (mode == 0 || mode == 1 || mode == 2 || mode == 4) {
    if (bytes % kBlockBytes != 0) return hipErrorInvalidValue;
    const long long blocks = bytes / kBlockBytes;
    const uint8_t* p = (const uint8_t*)src;
    if (mode == 0) hipLaunchKernelGGL((probe_tiles_kernel<8, 1>), dim3(cus), dim3(8 * 64), 0, st, p, blocks, sink);
    if (mode == 1) hipLaunchKernelGGL((probe_tiles_kernel<8, 2>), dim3(cus), dim3(8 * 64), 0, st, p, blocks, sink);
    if (mode == 2) hipLaunchKernelGGL((probe_tiles_kernel<4, 4>), dim3(cus), dim3(4 * 64), 0, st, p, blocks, sink);
    if (mode == 4)
      hipLaunchKernelGGL((probe_tiles_kernel<8, 1, true>), dim3(cus), dim3(8 * 64), 0, st, p, blocks, sink);
    return hipGetLastError();
  }
  if (mode == 3) {
    if (bytes % 16 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_vector_kernel, dim3(cus * 8), dim3(256), 0, st, (const uint4*)src, bytes / 16, sink);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace kvsel

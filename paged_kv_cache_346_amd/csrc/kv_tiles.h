// KV tile machinery shared by the attention kernels: the block-table window,
// pool loads with a cache policy, and the two-buffer tile pipeline.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace pkv {

// Physical block ids of up to 128 consecutive logical blocks, two per lane
// (lane l holds blocks base + l and base + 64 + l): each table entry is read
// from memory once per wave and taken as a scalar with readlane when its block
// is loaded.  A partition spans at most 128 blocks.
struct TableWindow {
  int base, v0, v1;
  __device__ __forceinline__ void load(const int* row, int b, int limit) {
    base = b;
    const int i = b + (int)(threadIdx.x & (kWave - 1));
    v0 = i < limit ? row[i] : 0;
    v1 = i + kWave < limit ? row[i + kWave] : 0;
  }
  // Block of logical block lb (wave-uniform, base <= lb < base + 128), clamped
  // into the pool so a corrupt entry can never address outside it.
  __device__ __forceinline__ int at(int lb, int num_blocks) const {
    const int d = lb - base;
    const int pb = d < kWave ? __builtin_amdgcn_readlane(v0, d)
                             : __builtin_amdgcn_readlane(v1, d - kWave);
    return min(max(pb, 0), num_blocks - 1);
  }
};

// A 16- or 8-byte vector load of pool data: nontemporal when the step streams
// the pool (every block read once), ordinary when blocks are shared by several
// sequences of the batch and a second read can hit in L2 or the last-level cache.
template <bool NT, typename V>
__device__ __forceinline__ V pool_load(const uint16_t* p) {
  const V* v = reinterpret_cast<const V*>(p);
  if constexpr (NT)
    return __builtin_nontemporal_load(v);
  else
    return *v;
}
template <bool NT, typename V>
__device__ __forceinline__ V pool_load(const uint8_t* p) {
  const V* v = reinterpret_cast<const V*>(p);
  if constexpr (NT)
    return __builtin_nontemporal_load(v);
  else
    return *v;
}
template <bool NT, typename V>
__device__ __forceinline__ V pool_load(const float* p) {
  const V* v = reinterpret_cast<const V*>(p);
  if constexpr (NT)
    return __builtin_nontemporal_load(v);
  else
    return *v;
}

// Run `compute(k, tile)` over a wave's n tiles with the loads of tile k+1 issued
// before tile k is computed.  Two register buffers alternate; every load in the
// steady loop is unconditional, so the compiler's wait before each compute only
// covers the tile it needs.  Two hooks that the steady loop never runs (so they
// add no code to it): `first()` once the first tile's loads are issued, and
// `last(k, tile)` in place of compute for the final tile.
struct NoHook {
  __device__ void operator()() const {}
};
template <typename Tile, typename Load, typename Compute, typename First, typename Last>
__device__ __forceinline__ void pipelined(int n, Load&& load, Compute&& compute, First&& first,
                                          Last&& last) {
  if (n <= 0) return;
  Tile ta, tb;
  load(0, ta);
  first();
  int k = 0;
  for (; k + 2 < n; k += 2) {
    load(k + 1, tb);
    compute(k, ta);
    load(k + 2, ta);
    compute(k + 1, tb);
  }
  if (k + 1 < n) {
    load(k + 1, tb);
    compute(k, ta);
    last(k + 1, tb);
  } else {
    last(k, ta);
  }
}
template <typename Tile, typename Load, typename Compute>
__device__ __forceinline__ void pipelined(int n, Load&& load, Compute&& compute) {
  pipelined<Tile>(n, load, compute, NoHook{}, compute);
}

// The same two-buffer pipeline, but the K half of tile k+2 is issued inside
// compute(k) for every other tile, through compute's `mid` hook, as soon as
// tile k's K registers have been consumed, and the V half after compute(k):
// more bytes are in flight while the rest of tile k is computed.  `load(k,
// tile)` loads both halves, `load_k` and `load_v` one each; `compute(k, tile,
// mid)` calls mid() exactly once.  Every load in the steady loop is
// unconditional.
template <typename Tile, typename Load, typename LoadK, typename LoadV, typename Compute,
          typename First, typename Last>
__device__ __forceinline__ void pipelined_split(int n, Load&& load, LoadK&& load_k,
                                                LoadV&& load_v, Compute&& compute,
                                                First&& first, Last&& last) {
  if (n <= 0) return;
  Tile ta, tb;
  load(0, ta);
  first();
  int k = 0;
  for (; k + 2 < n; k += 2) {
    load(k + 1, tb);
    compute(k, ta, [&] { load_k(k + 2, ta); });
    load_v(k + 2, ta);
    compute(k + 1, tb, NoHook{});
  }
  if (k + 1 < n) {
    load(k + 1, tb);
    compute(k, ta, NoHook{});
    last(k + 1, tb);
  } else {
    last(k, ta);
  }
}

}  // namespace pkv

// reshape_and_cache and copy_blocks for gfx950.
//
// Both are bit copies bound by HBM bandwidth: every thread moves one 16-byte
// vector (dwordx4), so a wave moves 1 KiB per instruction.
//   reshape_and_cache: each new token's K/V goes into its slot (PagedAttention:
//     The vLLM Paper, "Background and Motivation": every generated token adds
//     K/V vectors to the cache).  K keeps 16-byte groups of dims, so the K write
//     is one 16-byte store; V stores each dim's element into the dim's row of B
//     tokens (x scalar stores of 2 or 4 bytes).
//   copy_blocks: copy-on-write of whole blocks (PagedAttention and Continuous
//     Batching, "Pages, from operating systems": a shared block is copied only
//     when one sequence needs to modify it).  A (block, all heads) run is
//     contiguous in both pools, so a pair is two straight 16-byte-vector copies.
//   swap_blocks: the same copy between two pools, one of them in pinned host
//     memory that the GPU reads or writes over the host link (PagedAttention:
//     The vLLM Paper, "The Core Idea", analogy table, "Swapping": KV blocks
//     moved to CPU memory and back).
#include "../../include/pkv.h"
#include "device_common.h"
#include "launch_check.h"

namespace pkv {

template <typename E>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const E* __restrict__ key, const E* __restrict__ value, E* __restrict__ k_pool,
    E* __restrict__ v_pool, const int64_t* __restrict__ slot_mapping, int64_t total, int Hkv,
    int D, int B, int64_t num_slots) {
  constexpr int X = 16 / sizeof(E);
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int nch = D / X;
  const int c = (int)(gid % nch);
  const int64_t ih = gid / nch;  // token * Hkv + head
  const int h = (int)(ih % Hkv);
  const int64_t i = ih / Hkv;
  const int64_t slot = slot_mapping[i];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t pb = slot / B;
  const int off = (int)(slot % B);
  const int64_t src = ih * D + (int64_t)c * X;
  const u32x4 kv = *reinterpret_cast<const u32x4*>(key + src);
  const u32x4 vv = *reinterpret_cast<const u32x4*>(value + src);
  const int64_t kb = ((pb * Hkv + h) * nch + c) * B * X + (int64_t)off * X;
  *reinterpret_cast<u32x4*>(k_pool + kb) = kv;
  E* vrow = v_pool + ((pb * Hkv + h) * D + (int64_t)c * X) * B + off;
  if constexpr (sizeof(E) == 2) {
#pragma unroll
    for (int e = 0; e < X; ++e) {
      const uint32_t w = vv[e >> 1];
      reinterpret_cast<uint16_t*>(vrow)[(int64_t)e * B] = (uint16_t)((e & 1) ? (w >> 16) : w);
    }
  } else {
#pragma unroll
    for (int e = 0; e < X; ++e) reinterpret_cast<uint32_t*>(vrow)[(int64_t)e * B] = vv[e];
  }
}

// fp8 pools: token i's K/V (bf16) divided by its KV head's scale and encoded
// as E4M3 (f32_to_e4m3).  One thread per 4 dims, so a decode step's few
// tokens still spread over the whole chip: K is one 4-byte store into the
// token's 16-byte vector of its 16-dim chunk, V 4 byte stores into the dims'
// rows.
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
    const int64_t* __restrict__ slot_mapping, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale, int64_t total, int Hkv, int D, int B, int64_t num_slots) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int nq = D / 4;
  const int q = (int)(gid % nq);  // dims 4q .. 4q+3
  const int64_t ih = gid / nq;    // token * Hkv + head
  const int h = (int)(ih % Hkv);
  const int64_t i = ih / Hkv;
  const int64_t slot = slot_mapping[i];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t pb = slot / B;
  const int off = (int)(slot % B);
  const int64_t src = ih * D + (int64_t)q * 4;
  const float ks = k_scale[h], vs = v_scale[h];
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 kx = *reinterpret_cast<const u32x2*>(key + src);
  const u32x2 vx = *reinterpret_cast<const u32x2*>(value + src);
  uint32_t kw = 0u;
  uint8_t vb[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t kbits = (e & 1) ? (kx[e >> 1] & 0xffff0000u) : (kx[e >> 1] << 16);
    const uint32_t vbits = (e & 1) ? (vx[e >> 1] & 0xffff0000u) : (vx[e >> 1] << 16);
    kw |= f32_to_e4m3(__uint_as_float(kbits) / ks) << (8 * e);
    vb[e] = (uint8_t)f32_to_e4m3(__uint_as_float(vbits) / vs);
  }
  const int nch = D / 16;
  const int64_t kb = ((pb * Hkv + h) * nch + q / 4) * B * 16 + (int64_t)off * 16 + (q & 3) * 4;
  *reinterpret_cast<uint32_t*>(k_pool + kb) = kw;
  uint8_t* vrow = v_pool + ((pb * Hkv + h) * D + (int64_t)q * 4) * B + off;
#pragma unroll
  for (int e = 0; e < 4; ++e) vrow[(int64_t)e * B] = vb[e];
}

// dst_pool[dst] = src_pool[src] for each pair (src, dst), K and V; `units`
// 16-byte vectors per block.  A pair naming a block outside its pool is
// skipped.  src and dst may be the same pool (copy-on-write: within one call
// no block is both a source and a destination).
__global__ __launch_bounds__(256) void copy_blocks_kernel(
    const u32x4* src_k, const u32x4* src_v, int src_blocks, u32x4* dst_k, u32x4* dst_v,
    int dst_blocks, const int32_t* __restrict__ pairs, int64_t total, int64_t units) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int64_t k = gid / units;
  const int64_t u = gid % units;
  const int src = pairs[2 * k];
  const int dst = pairs[2 * k + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const u32x4 a = src_k[(int64_t)src * units + u];
  const u32x4 b = src_v[(int64_t)src * units + u];
  dst_k[(int64_t)dst * units + u] = a;
  dst_v[(int64_t)dst * units + u] = b;
}

}  // namespace pkv

using namespace pkv;

// bytes per pool element
static int elem_size(pkv_dtype dtype) {
  return dtype == PKV_F32 ? 4 : dtype == PKV_BF16 ? 2 : dtype == PKV_FP8_E4M3 ? 1 : 0;
}

extern "C" pkv_status pkv_reshape_and_cache(const void* key, const void* value, void* k_pool,
                                            void* v_pool, const int64_t* slot_mapping,
                                            int32_t T, int32_t Hkv, int32_t D, int32_t B,
                                            int32_t num_blocks, pkv_dtype dtype,
                                            const float* k_scale, const float* v_scale,
                                            void* hip_stream) {
  if (T < 0 || Hkv <= 0 || D <= 0 || B <= 0 || num_blocks <= 0) return PKV_EINVAL;
  const int es = elem_size(dtype);
  if (es == 0) return PKV_EINVAL;
  if ((D * es) % 16 != 0) return PKV_EINVAL;
  if (dtype == PKV_FP8_E4M3 && (!k_scale || !v_scale)) return PKV_EINVAL;
  if (T == 0) return PKV_OK;
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !slot_mapping)
    return PKV_EINVAL;
  // threads: one per 16-byte vector of a token's row; fp8, one per 4 dims
  const int64_t total = (int64_t)T * Hkv * (dtype == PKV_FP8_E4M3 ? D / 4 : D * es / 16);
  const dim3 grid((unsigned)((total + 255) / 256));
  hipStream_t st = (hipStream_t)hip_stream;
  const int64_t slots = (int64_t)num_blocks * B;
  if (dtype == PKV_FP8_E4M3)
    reshape_and_cache_fp8_kernel<<<grid, 256, 0, st>>>(
        (const uint16_t*)key, (const uint16_t*)value, (uint8_t*)k_pool, (uint8_t*)v_pool,
        slot_mapping, k_scale, v_scale, total, Hkv, D, B, slots);
  else if (dtype == PKV_F32)
    reshape_and_cache_kernel<float><<<grid, 256, 0, st>>>(
        (const float*)key, (const float*)value, (float*)k_pool, (float*)v_pool, slot_mapping,
        total, Hkv, D, B, slots);
  else
    reshape_and_cache_kernel<uint16_t><<<grid, 256, 0, st>>>(
        (const uint16_t*)key, (const uint16_t*)value, (uint16_t*)k_pool, (uint16_t*)v_pool,
        slot_mapping, total, Hkv, D, B, slots);
  return launch_status();
}

extern "C" pkv_status pkv_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs,
                                      int32_t n, int32_t Hkv, int32_t D, int32_t B,
                                      int32_t num_blocks, pkv_dtype dtype, void* hip_stream) {
  if (n < 0 || Hkv <= 0 || D <= 0 || B <= 0 || num_blocks <= 0) return PKV_EINVAL;
  const int es = elem_size(dtype);
  if (es == 0) return PKV_EINVAL;
  const int64_t block_bytes = (int64_t)Hkv * D * B * es;
  if (block_bytes % 16 != 0) return PKV_EINVAL;
  if (n == 0) return PKV_OK;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !pairs) return PKV_EINVAL;
  const int64_t units = block_bytes / 16;
  const int64_t total = units * n;
  const dim3 grid((unsigned)((total + 255) / 256));
  copy_blocks_kernel<<<grid, 256, 0, (hipStream_t)hip_stream>>>(
      (const u32x4*)k_pool, (const u32x4*)v_pool, num_blocks, (u32x4*)k_pool, (u32x4*)v_pool,
      num_blocks, pairs, total, units);
  return launch_status();
}

// The address at which the GPU reaches `p`: device memory as is, pinned host
// memory through its device mapping; nullptr for memory the GPU cannot reach
// (pageable host memory), so such a pool is rejected before any launch.
static void* device_view(const void* p) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();  // the query leaves its error behind for pageable memory
    return nullptr;
  }
  if (at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeHost) return nullptr;
  return at.devicePointer;
}

extern "C" pkv_status pkv_swap_blocks(void* dst_k, void* dst_v, int32_t dst_blocks,
                                      const void* src_k, const void* src_v, int32_t src_blocks,
                                      const int32_t* pairs, int32_t n, int32_t Hkv, int32_t D,
                                      int32_t B, pkv_dtype dtype, void* hip_stream) {
  if (n < 0 || Hkv <= 0 || D <= 0 || B <= 0 || dst_blocks <= 0 || src_blocks <= 0)
    return PKV_EINVAL;
  const int es = elem_size(dtype);
  if (es == 0) return PKV_EINVAL;
  const int64_t block_bytes = (int64_t)Hkv * D * B * es;
  if (block_bytes % 16 != 0) return PKV_EINVAL;
  if (n == 0) return PKV_OK;
  if (!pairs || !aligned16(dst_k) || !aligned16(dst_v) || !aligned16(src_k) || !aligned16(src_v))
    return PKV_EINVAL;
  void* dk = device_view(dst_k);
  void* dv = device_view(dst_v);
  void* sk = device_view(src_k);
  void* sv = device_view(src_v);
  if (!dk || !dv || !sk || !sv) return PKV_EINVAL;
  if (!aligned16(dk) || !aligned16(dv) || !aligned16(sk) || !aligned16(sv)) return PKV_EINVAL;
  const int64_t units = block_bytes / 16;
  const int64_t total = units * n;
  const dim3 grid((unsigned)((total + 255) / 256));
  copy_blocks_kernel<<<grid, 256, 0, (hipStream_t)hip_stream>>>(
      (const u32x4*)sk, (const u32x4*)sv, src_blocks, (u32x4*)dk, (u32x4*)dv, dst_blocks, pairs,
      total, units);
  return launch_status();
}

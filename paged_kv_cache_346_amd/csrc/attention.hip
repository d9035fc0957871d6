// PagedAttention decode for gfx950 (CDNA4): main kernel + log-sum-exp reduce.
//
// What is computed: for every running sequence s and query head h,
//   out[s, h] = softmax(q[s, h] . K_s^T * scale) V_s
// where K_s, V_s are the sequence's cached tokens, found through its block table
// (vLLM: PagedAttention and continuous batching, "Direct answer": attention
// follows the logical-to-physical block mapping; PagedAttention: The vLLM Paper,
// "The Core Idea": attention computed through block-table indirection, reading
// KV non-contiguously; "Background and Motivation": each new token attends over
// all previous tokens).  Query head h reads KV head h / G, G = Hq / Hkv (GQA,
// named in "Impact and Follow-Ups" as a way to shrink KV size).
//
// Work decomposition (not on the pages).  A work item is one (sequence, KV
// head, partition of P tokens); ONE wave64 owns an item from start to finish, so
// there is no cross-wave merge, no LDS tile staging and no workgroup barrier
// (LDS holds only an appended token, staged within its wave).  The whole GQA group of a
// KV head lives in that wave, so each K/V byte is fetched from HBM once.
// Items are numbered partition-major, with the partition counted from the END
// of its sequence and the farthest-from-the-end slice dispatched first:
//   * the dispatcher deals consecutive workgroups round-robin to the 8 XCDs, so
//     every XCD gets a like share of each slice (with the partition index
//     fastest, the first partitions -- most of the work when sequences are
//     short -- would pile onto a few XCDs);
//   * every slice but the last holds only full partitions, and the last slice
//     holds each sequence's final, partial one, so large items start first and
//     small ones fill the tail of a ragged batch.
// K/V tiles are read with nontemporal loads: the pool is streamed once per step
// and nothing in it is reused by the step, so it should not displace other data
// in the caches (measured 7-10% faster than ordinary loads on every workload).
//
// Each wave
//   * reads the partition's slice of the block table once, one entry per lane,
//     and takes each physical block id with readlane (a scalar) when needed;
//   * keeps two tiles of K/V in registers: the loads of tile k+1 are issued
//     before tile k is computed, so HBM traffic overlaps the arithmetic;
//   * keeps an online-softmax state: a reference m (the running maximum in the
//     VALU kernel; in the MFMA kernel a reference that trails it by at most 8
//     in log2 units and moves only when a score passes it by more), the sum l
//     of the weights exp2(score - m) and the unnormalised accumulator; any
//     reference gives the same acc / l, and the partials merge the same way.
// An item that covers its whole sequence writes the output rows; otherwise it
// writes its (m, l, acc) partial and the partitions are merged (log-sum-exp
// combine): by the item of the (sequence, KV head) that finishes last, inside
// the same launch, when no sequence has more than kMergeInLaunchMax partitions
// (and the batch fits the workspace's counters), else by pa_reduce_kernel in a
// second launch.  Scores are kept in
// base 2 (scale * log2 e folded in) so exp is one v_exp_f32.
//
// Two main kernels:
//   pa_valu_kernel  fp32 pools, and bf16 with G < 4.  Tile = one KV block.  Lanes
//                   (token, dim-chunk) for q.k with a cross-lane sum; lanes own
//                   output dims for p.v with the token weights read back as
//                   scalars.
//   pa_mfma_kernel  bf16 with G in {4, 8}: the GQA group x KV tile contraction is
//                   a small dense GEMM, run on v_mfma_f32_16x16x32_bf16 (group
//                   padded to 16).  Tile = 32 tokens.  S^T = K Q^T takes K
//                   straight from HBM as the A operand; O^T = V^T P^T takes V
//                   straight from HBM as the A operand.  P is split into bf16 hi +
//                   lo parts (two MFMAs) so the weights keep ~16 bits.
// Masking: tokens at or past the partition end get score -inf by selection and
// their V elements are zeroed before the product, so NaN in unused slots never
// reaches the output.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "../../include/pkv.h"
#include "decode_config.h"
#include "device_common.h"
#include "kv_tiles.h"
#include "launch_check.h"

namespace pkv {

// One wave per workgroup: the dispatcher then balances the ragged items wave by
// wave (measured faster than four-item workgroups on ragged batches).
constexpr int kWavesPerGroup = 1;           // items per workgroup
// Partitions per sequence up to which the main launch merges them itself; a
// longer split is merged by the reduce launch, whose many threads per row
// finish it sooner than one wave would.  Also the reduce launch merges when the
// batch has more (sequence, KV head) pairs than the workspace has counters.
constexpr int kMergeInLaunchMax = 16;
static_assert(kMaxPartitionBlocks == 2 * kWave, "two table entries per lane");

struct DecodeArgs {
  float* out;
  float* part_acc;   // [S, Hq, nparts, D]
  float* part_ml;    // [S, Hq, nparts, 2]
  int* counters;     // [S * Hkv] arrivals per (sequence, KV head) for the merge
                     // inside the launch, or nullptr (the reduce launch merges)
  const int* block_tables;
  const int* context_lens;
  const void* new_k;  // [S, Hkv, D]: each sequence's token of this step, or nullptr
  const void* new_v;
  const int4* plan;  // host-built work list {s, g, p, L} per item, or nullptr
  const float* k_scale;  // fp8 pools: per-KV-head scales of K and V, else nullptr
  const float* v_scale;
  int S;
  int SG;            // S * Hkv: items per partition index
  int items;         // attention work items in the grid
  int store_items;   // appending launch: S store items after them, else 0
  int Hkv, max_blocks, num_blocks, nparts, P;
  float scale_log2e;
};

// One wave's share: sequence s, KV head g, partition p, tokens [start, end).
// item_ids() stores the partition counted from the sequence's end in p;
// item_extent() turns it into the partition index once the length is known.
struct WorkItem {
  int s, g, p, start, end, nps;
  bool tail;  // the item ends at the sequence's own last token (no clamping cut it)
};

// Item of this wave and its sequence length; false past the last item.
// Without a plan: partition-major numbering of every (sequence, KV head,
// partition), the partition counted from the sequence's end (item_extent turns
// it into the index).  With a plan: item i is the plan's record i, whose
// partition index and length come from the host (no length load here), and a
// record naming a sequence or head outside the batch is skipped.
template <int NW>
__device__ __forceinline__ bool item_ids(const DecodeArgs& a, WorkItem& it, int& L) {
  const int item = (int)blockIdx.x * NW + uniform((int)threadIdx.x / kWave);
  if (item >= a.items) return false;
  if (a.plan) {
    const int4 rec = a.plan[item];
    it.s = rec.x;
    it.g = rec.y;
    const int p = rec.z;
    L = rec.w;
    if (it.s < 0 || it.s >= a.S || it.g < 0 || it.g >= a.Hkv || p < 0 || p >= a.nparts)
      return false;
    it.p = p;
    return true;
  }
  const int k = item / a.SG;
  it.p = a.nparts - 1 - k;   // partitions counted from the sequence's end
  const int sg = item - k * a.SG;
  it.g = sg % a.Hkv;
  it.s = sg / a.Hkv;
  L = a.context_lens[it.s];
  return true;
}

// Token extent of the item given the sequence length; false when the wave has
// nothing to do (a zero-length sequence gets zero output rows).
template <int D, int B, int G>
__device__ __forceinline__ bool item_extent(const DecodeArgs& a, WorkItem& it, int L) {
  const int L0 = L;
  L = min(L, a.max_blocks * B);
  const int np = L <= 0 ? 0 : min((L + a.P - 1) / a.P, a.nparts);
  int p = it.p;
  if (!a.plan) p = np - 1 - p;  // unplanned ids count the partition from the sequence's end
  if (L <= 0) {
    // a sequence with no tokens gets zero rows, written by its first item only
    if (a.plan ? p == 0 : p == -1) {
      float* o = a.out + ((size_t)it.s * a.Hkv * G + (size_t)it.g * G) * D;
      for (int i = threadIdx.x & (kWave - 1); i < G * D; i += kWave) o[i] = 0.f;
    }
    return false;
  }
  if (p < 0 || p >= np) return false;
  it.p = p;
  it.start = p * a.P;
  it.end = min(L, it.start + a.P);
  it.nps = np;
  it.tail = it.end == L0;
  return true;
}

// Where an item's result row for query head h goes: the output (the item covers
// the whole sequence) or its partition's partial slot.
struct RowSink {
  float* acc;  // D floats
  float* ml;   // (m, l) or nullptr for a final row
};

template <int D, int G>
__device__ __forceinline__ RowSink row_sink(const DecodeArgs& a, const WorkItem& it, int gi) {
  const int Hq = a.Hkv * G;
  const size_t h = (size_t)it.s * Hq + it.g * G + gi;
  if (it.nps == 1) return RowSink{a.out + h * D, nullptr};
  const size_t row = h * a.nparts + it.p;
  return RowSink{a.part_acc + row * D, a.part_ml + 2 * row};
}

// Store item of an appending launch: sequence s's token of this step (row s of
// new_k / new_v, every KV head) written into its slot at position L-1, when
// the launch covers that position (the rule that gives the sequence an
// attention item ending there).  The attention wave that ends at L-1 takes the
// token from new_k / new_v, never from the pool, so these stores need no
// ordering with it; the store items follow every attention item in the grid
// and run in the launch's tail, so no attention wave waits for a store to be
// acknowledged.  fp8 pools: each bf16 value is encoded with its head's scale,
// as the cache write does.
template <typename E, int D, int B>
__device__ __forceinline__ void store_new_token(const DecodeArgs& a, int s, E* __restrict__ k_pool,
                                                E* __restrict__ v_pool) {
  constexpr bool F8 = sizeof(E) == 1;
  using RE = std::conditional_t<F8, uint16_t, E>;  // element of the new rows
  constexpr int X = 16 / sizeof(E);                // elements per 16-byte K vector
  constexpr int NCH = D / X;                       // K vectors per head
  const int L0 = a.context_lens[s];
  if (L0 <= 0 || L0 > a.max_blocks * B || L0 > a.nparts * a.P) return;
  const int t = L0 - 1, off = t % B;
  const int pb =
      min(max(a.block_tables[(size_t)s * a.max_blocks + t / B], 0), a.num_blocks - 1);
  const int lane = threadIdx.x & (kWave - 1);
  const RE* kn = reinterpret_cast<const RE*>(a.new_k) + (size_t)s * a.Hkv * D;
  const RE* vn = reinterpret_cast<const RE*>(a.new_v) + (size_t)s * a.Hkv * D;
  E* kb = k_pool + (size_t)pb * a.Hkv * (D * B);
  E* vb = v_pool + (size_t)pb * a.Hkv * (D * B);
  for (int i = lane; i < a.Hkv * NCH; i += kWave) {
    const int g = i / NCH, ch = i - g * NCH;
    u32x4 w = {0u, 0u, 0u, 0u};
    if constexpr (F8) {
      const float ks = a.k_scale[g];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 src = *reinterpret_cast<const u32x4*>(kn + (size_t)g * D + ch * X + 8 * h);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t bits = (e & 1) ? (src[e >> 1] & 0xffff0000u) : (src[e >> 1] << 16);
          const int d = 8 * h + e;
          w[d >> 2] |= f32_to_e4m3(__uint_as_float(bits) / ks) << (8 * (d & 3));
        }
      }
    } else {
      w = *reinterpret_cast<const u32x4*>(kn + (size_t)g * D + ch * X);
    }
    *reinterpret_cast<u32x4*>(kb + (size_t)g * (D * B) + ((size_t)ch * B + off) * X) = w;
  }
  for (int i = lane; i < a.Hkv * D; i += kWave) {
    const int g = i / D, d = i - g * D;
    E v;
    if constexpr (F8)
      v = (E)f32_to_e4m3(__uint_as_float((uint32_t)vn[i] << 16) / a.v_scale[g]);
    else
      v = vn[i];
    vb[(size_t)g * (D * B) + (size_t)d * B + off] = v;
  }
}

// Grid position of this wave: a store item of an appending launch is handled
// here (true: the wave is done); attention items return false.
template <typename E, int D, int B, int NW, bool AP>
__device__ __forceinline__ bool store_item(const DecodeArgs& a, E* k_pool, E* v_pool) {
  if constexpr (!AP) return false;
  const int item = (int)blockIdx.x * NW + uniform((int)threadIdx.x / kWave);
  if (item < a.items) return false;
  const int s = item - a.items;
  if (s < a.store_items) store_new_token<E, D, B>(a, s, k_pool, v_pool);
  return true;
}

// ---------------------------------------------------------------------------
// Partition merge inside the main launch.  A split item writes its partial
// rows with device-scope stores (sc1: written through to the point where every
// XCD sees them), waits until they are acknowledged, then counts itself on its
// (sequence, KV head)'s counter with a device-scope atomic.  The item that
// finds every other one counted merges all partials, read back with
// device-scope loads, and resets the counter for the next launch.  Nothing
// waits on another wave, and no fence is needed: the partials never go
// through an XCD's L2 as ordinary (write-back) data, so there is nothing for a
// release to write back or for an acquire to invalidate (an agent-scope
// release or acquire on gfx950 is exactly the L2 write-back or invalidate plus
// the counter wait used here).
// ---------------------------------------------------------------------------
constexpr int kSc1 = 16;                        // cache-policy bit: device scope
constexpr int kNtPol = 2;                       // cache-policy bit: nontemporal
constexpr int kRsrcWord3 = 0x00020000;          // raw 32-bit buffer, gfx9 layout
constexpr int kWaitVm0 = 0x0F70;                // s_waitcnt vmcnt(0)
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// A buffer resource over `bytes` bytes at `base` (wave-uniform).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

// The partial rows of (sequence s, KV head g): acc [G, nparts, D] and
// (m, l) [G, nparts, 2], contiguous for the G query heads of the KV head.
template <int D, int G>
struct PartialRows {
  __amdgpu_buffer_rsrc_t acc, ml;
  int nparts;
  __device__ __forceinline__ PartialRows(const DecodeArgs& a, int s, int g) {
    const size_t row0 = ((size_t)s * a.Hkv + g) * G * a.nparts;
    acc = raw_rsrc(a.part_acc + row0 * D, (uint32_t)(G * a.nparts * D * 4));
    ml = raw_rsrc(a.part_ml + row0 * 2, (uint32_t)(G * a.nparts * 8));
    nparts = a.nparts;
  }
  // byte offsets of row (gi, p): its acc element e, its (m, l) pair
  __device__ __forceinline__ int acc_off(int gi, int p, int e) const {
    return ((gi * nparts + p) * D + e) * 4;
  }
  __device__ __forceinline__ int ml_off(int gi, int p) const { return (gi * nparts + p) * 8; }
  __device__ __forceinline__ void store4(const f32x4& v, int off) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), acc, off, 0, kSc1);
  }
  __device__ __forceinline__ void store1(float v, int off) const {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), acc, off, 0, kSc1);
  }
  // the same rows for the reduce launch: nontemporal stores (a wave holds its
  // slot until its stores are acknowledged, and under the launch's read
  // traffic nontemporal ones are acknowledged sooner: 5% on the 70B-shaped
  // batch, whose every item ends with a partial)
  __device__ __forceinline__ void store4_nt(const f32x4& v, int off) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), acc, off, 0, kNtPol);
  }
  __device__ __forceinline__ void store1_nt(float v, int off) const {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), acc, off, 0, kNtPol);
  }
  __device__ __forceinline__ void store_ml(float m, float l, int off) const {
    __builtin_amdgcn_raw_buffer_store_b64(u32x2v{__float_as_uint(m), __float_as_uint(l)}, ml,
                                          off, 0, kSc1);
  }
  __device__ __forceinline__ f32x4 load4(int off) const {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(acc, off, 0, kSc1));
  }
  __device__ __forceinline__ u32x2v load_ml(int off) const {
    return __builtin_amdgcn_raw_buffer_load_b64(ml, off, 0, kSc1);
  }
};

// After this wave's partial stores: true for the (sequence, KV head)'s last
// item to finish, which then owns the merge (its counter is reset to zero).
__device__ __forceinline__ bool arrive_last(const DecodeArgs& a, int s, int g, int nps) {
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's partial stores are acknowledged
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  int* cnt = a.counters + (size_t)s * a.Hkv + g;
  int old = 0;
  if ((threadIdx.x & (kWave - 1)) == 0)
    old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0, kWave);
  if (old != nps - 1) return false;
  if ((threadIdx.x & (kWave - 1)) == 0)
    __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// The merge by the last item: output rows of the G query heads of (s, g) from
// their nps partials.  Each lane takes float4 columns of the G x D block and
// folds the partitions U at a time (indices past the end re-read the last one
// with weight 0), as pa_reduce_kernel does for a row.
template <int D, int G>
__device__ __forceinline__ void merge_partials(const DecodeArgs& a, int s, int g, int nps) {
  constexpr int C4 = D / 4;
  constexpr int NCOL = G * C4;
  constexpr int PER = (NCOL + kWave - 1) / kWave;
  constexpr int U = 4;
  const PartialRows<D, G> pr(a, s, g);
  const int lane = threadIdx.x & (kWave - 1);
  const size_t out0 = ((size_t)s * a.Hkv + g) * G * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int col = lane + kWave * i;
    if (NCOL % kWave != 0 && col >= NCOL) break;
    const int gi = col / C4, c4 = col - gi * C4;
    float M = -INFINITY, den = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int p0 = 0; p0 < nps; p0 += U) {
      float mi[U], li[U];
      f32x4 ai[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int p = min(p0 + u, nps - 1);
        const u32x2v w = pr.load_ml(pr.ml_off(gi, p));
        mi[u] = p0 + u < nps ? __uint_as_float(w[0]) : -INFINITY;
        li[u] = __uint_as_float(w[1]);
        ai[u] = pr.load4(pr.acc_off(gi, p, 4 * c4));
      }
      float mn = M;
#pragma unroll
      for (int u = 0; u < U; ++u) mn = fmaxf(mn, mi[u]);
      const float fo = fast_exp2(M - mn);  // M = -inf gives 0
      den *= fo;
      acc *= fo;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float f = fast_exp2(mi[u] - mn);  // past the end: 0
        den = fmaf(f, li[u], den);
        acc += f * ai[u];
      }
      M = mn;
    }
    *reinterpret_cast<f32x4*>(a.out + out0 + (size_t)gi * D + 4 * c4) = acc * (1.f / den);
  }
}

// ---------------------------------------------------------------------------
// VALU main kernel.  E = float, uint16_t (bf16 bits) or uint8_t (fp8 E4M3 codes,
// bf16 queries: each 16-dim K chunk pairs with two 16-byte q vectors, codes are
// widened to fp32 exactly, the K scale joins the score scale and the V scale
// the output).  Tile = one KV block.
// ---------------------------------------------------------------------------
template <typename E, int D, int B, int G, int NW, bool NT, bool AP>
__global__ __launch_bounds__(NW* kWave) void pa_valu_kernel(
    DecodeArgs a, const std::conditional_t<sizeof(E) == 1, uint16_t, E>* __restrict__ q,
    E* __restrict__ k_pool, E* __restrict__ v_pool) {
  constexpr bool F8 = sizeof(E) == 1;
  using QE = std::conditional_t<F8, uint16_t, E>;
  constexpr int QV = F8 ? 2 : 1;     // 16-byte q vectors per K chunk
  constexpr int X = 16 / sizeof(E);  // elements per 16-byte vector
  constexpr int NCG = kWave / B;     // lanes sharing one token in q.k
  constexpr int NCH = D / X;         // 16-byte chunks per token
  constexpr int CPL = NCH / NCG;     // chunks per lane
  constexpr int NVT = B / X;         // 16-byte token runs in a V row
  constexpr int ND = D / kWave;      // output dims per lane
  static_assert(NCH % NCG == 0 && D % kWave == 0 && B % X == 0, "unsupported shape");

  const int lane = threadIdx.x & (kWave - 1);
  const int t = lane % B;   // token of this lane in q.k
  const int cg = lane / B;  // its chunk group
  if (store_item<E, D, B, NW, AP>(a, k_pool, v_pool)) return;
  WorkItem it;
  int L;
  if (!item_ids<NW>(a, it, L)) return;
  const int Hq = a.Hkv * G;

  // the length decides whether the item is empty (most of an unplanned grid when
  // the batch is ragged); then the partition's table slice and the queries load
  // together
  if (!item_extent<D, B, G>(a, it, L)) return;
  TableWindow tw;
  tw.load(a.block_tables + (size_t)it.s * a.max_blocks, it.start / B, a.max_blocks);
  u32x4 qv[G][CPL][QV];
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
      for (int h = 0; h < QV; ++h)
        qv[gi][j][h] = *reinterpret_cast<const u32x4*>(
            q + ((size_t)it.s * Hq + it.g * G + gi) * D + (cg + NCG * j) * X + 8 * h);
  const float score_scale = F8 ? a.scale_log2e * a.k_scale[it.g] : a.scale_log2e;
  const float out_scale = F8 ? a.v_scale[it.g] : 1.f;

  float m[G], ls[G], acc[G][ND];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    m[gi] = -INFINITY;
    ls[gi] = 0.f;
#pragma unroll
    for (int k = 0; k < ND; ++k) acc[gi][k] = 0.f;
  }

  struct Tile {
    u32x4 k[CPL];
    u32x4 v[NVT][ND];
  };
  const int lb_first = it.start / B;
  const int n = (it.end + B - 1) / B - lb_first;
  const size_t head_off = (size_t)it.g * (D * B);
  const size_t blk_stride = (size_t)a.Hkv * (D * B);

  // Append (decode step with new_k/new_v): the sequence's token of this step is
  // its last, at position L-1 in this item's final block.  The wave owning that
  // partition loads it before its first tile and puts it into the final tile's
  // registers in place of what the pool held there; a store item at the end of
  // the grid writes it into its slot (store_new_token).
  const bool appends = AP && it.tail;
  const int tnew = it.end - 1;
  u32x4 nk[CPL];
  E nv[ND];
  if (appends) {
    const size_t row = ((size_t)it.s * a.Hkv + it.g) * D;
    const QE* kn = reinterpret_cast<const QE*>(a.new_k) + row;
    const QE* vn = reinterpret_cast<const QE*>(a.new_v) + row;
    if constexpr (F8) {
      // the token's bf16 rows encoded with the head's scales, as the cache write does
      const float ks = a.k_scale[it.g], vs = a.v_scale[it.g];
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        nk[j] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(kn + (cg + NCG * j) * X + 8 * h);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t bits = (e & 1) ? (w[e >> 1] & 0xffff0000u) : (w[e >> 1] << 16);
            const int d = 8 * h + e;
            nk[j][d >> 2] |= f32_to_e4m3(__uint_as_float(bits) / ks) << (8 * (d & 3));
          }
        }
      }
#pragma unroll
      for (int k2 = 0; k2 < ND; ++k2)
        nv[k2] = (E)f32_to_e4m3(__uint_as_float((uint32_t)vn[lane + kWave * k2] << 16) / vs);
    } else {
#pragma unroll
      for (int j = 0; j < CPL; ++j)
        nk[j] = *reinterpret_cast<const u32x4*>(kn + (cg + NCG * j) * X);
#pragma unroll
      for (int k2 = 0; k2 < ND; ++k2) nv[k2] = vn[lane + kWave * k2];
    }
  }
  auto load = [&](int k, Tile& tl) {
    const int pb = tw.at(lb_first + k, a.num_blocks);
    const E* kb = k_pool + pb * blk_stride + head_off;
    const E* vb = v_pool + pb * blk_stride + head_off;
#pragma unroll
    for (int j = 0; j < CPL; ++j)
      tl.k[j] = pool_load<NT, u32x4>(kb + ((cg + NCG * j) * B + t) * X);
#pragma unroll
    for (int tc = 0; tc < NVT; ++tc)
#pragma unroll
      for (int k2 = 0; k2 < ND; ++k2)
        tl.v[tc][k2] = pool_load<NT, u32x4>(vb + (lane + kWave * k2) * B + tc * X);
  };

  // the final block: the appended token (its place tn in the block is
  // wave-uniform) replaces what the pool held there
  auto substitute = [&](int k, Tile& tl) {
    const int tn = tnew - (lb_first + k) * B;
    if (t == tn) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) tl.k[j] = nk[j];
    }
#pragma unroll
    for (int tc = 0; tc < NVT; ++tc)
#pragma unroll
      for (int e = 0; e < X; ++e)
        if (tc * X + e == tn) {
#pragma unroll
          for (int k2 = 0; k2 < ND; ++k2) vec_set<E>(tl.v[tc][k2], e, nv[k2]);
        }
  };

  auto compute = [&](int k, Tile& tl) {
    const int tok0 = (lb_first + k) * B;
    const bool valid = tok0 + t < it.end;
    float pr[G];
    // fp8: the K codes widened once for all heads of the group
    float kf[F8 ? CPL : 1][16];
    if constexpr (F8) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) fp8x16_to_f32(tl.k[j], kf[j]);
    }
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      float sc = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int e = 0; e < X; ++e) {
          if constexpr (F8)
            sc = fmaf(vec_elem<uint16_t>(qv[gi][j][e >> 3], e & 7), kf[j][e], sc);
          else
            sc = fmaf(vec_elem<E>(qv[gi][j][0], e), vec_elem<E>(tl.k[j], e), sc);
        }
      if (NCG >= 4) sc += shfl_xor_f(sc, 16);
      if (NCG >= 2) sc += shfl_xor_f(sc, 32);
      sc = valid ? sc * score_scale : -INFINITY;
      float mx = sc;
#pragma unroll
      for (int o = 1; o < B; o <<= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
      const float mn = fmaxf(m[gi], mx);  // finite: the block holds a valid token
      const float alpha = fast_exp2(m[gi] - mn);
      pr[gi] = fast_exp2(sc - mn);
      ls[gi] = ls[gi] * alpha + (cg == 0 ? pr[gi] : 0.f);
#pragma unroll
      for (int k2 = 0; k2 < ND; ++k2) acc[gi][k2] *= alpha;
      m[gi] = mn;
    }
#pragma unroll
    for (int tc = 0; tc < NVT; ++tc) {
      float vf[F8 ? ND : 1][16];
      if constexpr (F8) {
#pragma unroll
        for (int k2 = 0; k2 < ND; ++k2) fp8x16_to_f32(tl.v[tc][k2], vf[k2]);
      }
#pragma unroll
      for (int e = 0; e < X; ++e) {
        const int tt = tc * X + e;
        if (tok0 + tt < it.end) {
#pragma unroll
          for (int gi = 0; gi < G; ++gi) {
            const float pt = read_lane(pr[gi], tt);
#pragma unroll
            for (int k2 = 0; k2 < ND; ++k2) {
              if constexpr (F8)
                acc[gi][k2] = fmaf(pt, vf[k2][e], acc[gi][k2]);
              else
                acc[gi][k2] = fmaf(pt, vec_elem<E>(tl.v[tc][k2], e), acc[gi][k2]);
            }
          }
        }
      }
    }
  };

  if constexpr (AP) {
    pipelined<Tile>(n, load, compute, NoHook{}, [&](int k, Tile& tl) {
      if (appends) substitute(k, tl);
      compute(k, tl);
    });
  } else {
    pipelined<Tile>(n, load, compute);
  }

  if (it.nps > 1 && a.counters) {
    // partial rows at device scope, then the merge by the last item
    const PartialRows<D, G> pr(a, it.s, it.g);
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const float l = wave_sum(ls[gi]);
#pragma unroll
      for (int k = 0; k < ND; ++k)
        pr.store1(acc[gi][k] * out_scale, pr.acc_off(gi, it.p, lane + kWave * k));
      if (lane == 0) pr.store_ml(m[gi], l, pr.ml_off(gi, it.p));
    }
    if (arrive_last(a, it.s, it.g, it.nps)) merge_partials<D, G>(a, it.s, it.g, it.nps);
    return;
  }
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const float l = wave_sum(ls[gi]);
    const RowSink dst = row_sink<D, G>(a, it, gi);
    const float scl = (dst.ml ? 1.f : 1.f / l) * out_scale;
    if (dst.ml) {
      const PartialRows<D, G> pr(a, it.s, it.g);
#pragma unroll
      for (int k = 0; k < ND; ++k)
        pr.store1_nt(acc[gi][k] * scl, pr.acc_off(gi, it.p, lane + kWave * k));
    } else {
#pragma unroll
      for (int k = 0; k < ND; ++k) dst.acc[lane + kWave * k] = acc[gi][k] * scl;
    }
    if (dst.ml && lane == 0) {
      dst.ml[0] = m[gi];
      dst.ml[1] = l;
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA main kernel (bf16, G <= 16).  Tile = 32 tokens, as two 16-token halves
// th = 0, 1 (for B = 16, one KV block each).
// v_mfma_f32_16x16x32_bf16 operand layout (lane l, c = l / 16, r = l % 16):
//   A[16 x 32]: lane holds row r, k = 8c .. 8c+7;  B[32 x 16]: col r, k = 8c .. 8c+7;
//   C[16 x 16]: lane holds col r, rows 4c .. 4c+3.
// q.k:  C_th[m][n] = sum_d K[16th + m][d] Q[n][d]: the A operand of lane (c, r)
//       is token 16th + r, dims 32j + 8c .. +7 -- one 16-byte K vector; for a
//       fixed c the 16 lanes r read 16 consecutive tokens, 256 contiguous bytes.
//       Lane (c, r) ends with the scores of head r at tokens 16th + 4c + i.
// p.v:  O^T = V^T P^T with the MFMA k index 8c + 4th + i standing for tile token
//       16th + 4c + i -- exactly the eight scores lane (c, r) holds, so P needs
//       no shuffle.  The A operand of lane (c, r) is dim 16dt + r at those
//       tokens: two 8-byte runs of the V row (tokens 4c .. 4c+3 of each half).
// fp8 tiles are 64 tokens, two 32-token steps s of two quarters th each, and
// take the same number of load instructions per byte as bf16 (gfx9 lets a wave
// have at most 63 vector loads outstanding, so narrower loads would cap the
// bytes in flight):
//   K: one 16-byte load per lane is one whole 16-dim chunk of the layout and
//      feeds two q.k k-steps: k-step j of lane c takes dims 16(4(j/2) + c) +
//      8(j%2) .. +7 (q is read with the same mapping);
//   V: one 8-byte load per lane: tokens 8c .. 8c+7 of step s, dim 16dt + r.
//      For that, row r of quarter th stands for step token 8(r/4) + 4th + r%4,
//      so the scores lane (c, r) holds -- rows 4c .. 4c+3 of both quarters --
//      are exactly tokens 8c .. 8c+7, the p.v k index 8c + e is token 8c + e.
//   Those K rows read half of each 128-byte line per instruction.  At B = 16
//   the K loads instead read whole lines (lane r: token 8h + r%8 of block r/8,
//   h = 0, 1), nontemporal, and the operand moves the rows into MFMA order
//   with two DPP row shifts; at B = 32 the half-line loads stay, with ordinary
//   loads so the other half is served from L2.
// ---------------------------------------------------------------------------
template <int D, int B, int G, int NW, bool NT, bool AP, bool F8>
__global__ __launch_bounds__(NW* kWave, 2) void pa_mfma_kernel(
    DecodeArgs a, const uint16_t* __restrict__ q,
    std::conditional_t<F8, uint8_t, uint16_t>* __restrict__ k_pool,
    std::conditional_t<F8, uint8_t, uint16_t>* __restrict__ v_pool) {
  // bf16 tiles are 32 tokens (two 16-token quarters); fp8 tiles are 64 (four
  // quarters, two MFMA steps) so that one tile's loads move the same 16 KiB
  // per wave and keep as many bytes in flight
  constexpr int NQ = F8 ? 4 : 2;
  constexpr int TILE = 16 * NQ;
  constexpr int NJ = D / 32;   // q.k k-steps
  constexpr int NDT = D / 16;  // p.v output dim tiles
  static_assert(G >= 1 && G <= 16 && (B == 16 || B == 32) && D % 32 == 0, "unsupported shape");
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  // bf16 at B = 32: one V load instruction covers half of each 64-byte dim row
  // and the other half follows in the next instruction; a nontemporal first
  // read lets the line go before the second arrives (measured 17% slower), so
  // bf16 V streams only at B = 16, where every V instruction reads whole lines.
  // fp8 V instructions read whole lines at both block sizes; fp8 K loads read
  // 64-byte runs whose other halves come with the next quarter's load.
  constexpr bool kNtV = NT && (B == 16 || F8);
  constexpr bool kNtK = NT && !F8;

  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane >> 4, r = lane & 15;
  if (store_item<std::conditional_t<F8, uint8_t, uint16_t>, D, B, NW, AP>(a, k_pool, v_pool))
    return;
  WorkItem it;
  int L;
  if (!item_ids<NW>(a, it, L)) return;
  const int Hq = a.Hkv * G;

  // the length decides whether the item is empty (most of an unplanned grid when
  // the batch is ragged); then the partition's table slice and the queries load
  // together
  if (!item_extent<D, B, G>(a, it, L)) return;
  TableWindow tw;
  tw.load(a.block_tables + (size_t)it.s * a.max_blocks, it.start / B, a.max_blocks);
  bf16x8 qb[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    // the dims of k-step j in lane c (bf16: 32j + 8c; fp8: see above)
    const int d0 = F8 ? 16 * (4 * (j >> 1) + c) + 8 * (j & 1) : 8 * (4 * j + c);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < G)
      v = *reinterpret_cast<const u32x4*>(q + ((size_t)it.s * Hq + it.g * G + r) * D + d0);
    qb[j] = __builtin_bit_cast(bf16x8, v);
  }

  // running state of the lane's column (reference m, threshold thr in raw
  // score units, the lane's share of the weight sum)
  float m = -INFINITY, thr = -INFINITY, ls = 0.f;
  f32x4 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // bf16: K of quarter th, k-step j; V runs of quarter th, dim tile dt.
  // fp8 (raw codes; the MFMA operands are widened to bf16 where they are used):
  // K of quarter 2s + th, chunk 4i + c; V runs of step s, dim tile dt
  struct Tile16 {
    u32x4 k[NQ][NJ];
    u32x2 v[NQ][NDT];
  };
  struct Tile8 {
    u32x4 k[NQ][NJ / 2];
    u32x2 v[NQ / 2][NDT];
  };
  using Tile = std::conditional_t<F8, Tile8, Tile16>;
  // fp8: the K scale joins the score scale, the V scale the output
  // (positive: the host rejects scale <= 0, the fp8 scales are positive)
  const float score_scale = F8 ? a.scale_log2e * a.k_scale[it.g] : a.scale_log2e;
  const float inv_scale = 1.f / score_scale;
  const float out_scale = F8 ? a.v_scale[it.g] : 1.f;
  // tile k covers tokens it.start + TILE*k .. +TILE-1 (partitions start at
  // multiples of 32 and of B)
  const int n = (it.end - it.start + TILE - 1) / TILE;
  const int nb_last = (it.end + B - 1) / B - 1;  // last logical block of the partition
  const size_t head_off = (size_t)it.g * (D * B);
  const size_t blk_stride = (size_t)a.Hkv * (D * B);

  // Append (decode step with new_k/new_v): the sequence's token of this step is
  // its last, at position L-1 in this item's final tile.  The wave owning that
  // partition loads it before its first tile and stages it in LDS once that
  // tile's loads are out; when the final tile arrives the staged values replace
  // what the pool held there.  A store item at the end of the grid writes the
  // token into its slot (store_new_token).  fp8 pools: the token (bf16) is
  // encoded with its head's scales as the cache write does, and its codes are
  // staged and substituted.
  __shared__ __align__(16) uint16_t s_new[kWavesPerGroup][2][D];
  uint16_t* lds_k = s_new[threadIdx.x / kWave][0];
  uint16_t* lds_v = s_new[threadIdx.x / kWave][1];
  uint8_t* lds_k8 = reinterpret_cast<uint8_t*>(lds_k);
  uint8_t* lds_v8 = reinterpret_cast<uint8_t*>(lds_v);
  const bool appends = AP && it.tail;
  const int tnew = it.end - 1;
  // lanes < D/8 hold K dims 8*lane .. +7 (bf16: one chunk of the K layout;
  // fp8: half of one); every lane holds V dims lane + 64i, so four lanes share
  // each V line it writes
  constexpr int NVD = D / kWave;
  u32x4 nk = {0u, 0u, 0u, 0u};
  uint16_t nv[NVD];
  u32x2 nk8 = {0u, 0u};
  uint8_t nv8[NVD];
  if (appends) {
    const size_t row = ((size_t)it.s * a.Hkv + it.g) * D;
    if (lane < D / 8)
      nk = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.new_k) + row +
                                           8 * lane);
#pragma unroll
    for (int i = 0; i < NVD; ++i)
      nv[i] = reinterpret_cast<const uint16_t*>(a.new_v)[row + lane + kWave * i];
    if constexpr (F8) {
      const float ks = a.k_scale[it.g], vs = a.v_scale[it.g];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = nk[e >> 1];
        const uint32_t bits = (e & 1) ? (w & 0xffff0000u) : (w << 16);
        nk8[e >> 2] |= f32_to_e4m3(__uint_as_float(bits) / ks) << (8 * (e & 3));
      }
#pragma unroll
      for (int i = 0; i < NVD; ++i)
        nv8[i] = (uint8_t)f32_to_e4m3(__uint_as_float((uint32_t)nv[i] << 16) / vs);
    }
  }
  auto stage_new = [&]() {
    if constexpr (AP) {
      if (appends) {
        if constexpr (F8) {
          if (lane < D / 8) *reinterpret_cast<u32x2*>(lds_k8 + 8 * lane) = nk8;
#pragma unroll
          for (int i = 0; i < NVD; ++i) lds_v8[lane + kWave * i] = nv8[i];
        } else {
          if (lane < D / 8) *reinterpret_cast<u32x4*>(lds_k + 8 * lane) = nk;
#pragma unroll
          for (int i = 0; i < NVD; ++i) lds_v[lane + kWave * i] = nv[i];
        }
      }
      // other lanes of the wave read the staged token back: order the LDS
      // writes before those reads
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  };

  // the K and/or V half of tile k (WK, WV: std::bool_constant)
  auto load_part = [&](int k, Tile& tl, auto WK, auto WV) {
    const int lb0 = (it.start + k * TILE) / B;
    // the tile's blocks (B / 16 quarters each); a block past the partition end
    // repeats the last one (its tokens are masked)
    constexpr int NBT = TILE / B;
    int pbs[NBT];
#pragma unroll
    for (int i = 0; i < NBT; ++i) pbs[i] = tw.at(min(lb0 + i, nb_last), a.num_blocks);
    if constexpr (F8) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        // K row r of quarter th: step token 8(r/4) + 4th + r%4; V lane c: step
        // tokens 8c .. 8c+7.  At B = 16 a step spans two blocks, so the block
        // depends on the lane: K rows r >= 8 and V lanes c >= 2 are in the second
        const size_t bk = B == 16 ? (r >= 8 ? pbs[2 * st + 1] : pbs[2 * st]) : pbs[st];
        const size_t bv = B == 16 ? (c >= 2 ? pbs[2 * st + 1] : pbs[2 * st]) : pbs[st];
        const int vtok = (8 * c) % B;
        const auto* kb = k_pool + bk * blk_stride + head_off;
        const auto* vb = v_pool + bv * blk_stride + head_off;
        if constexpr (decltype(WK)::value) {
          if constexpr (B == 16) {
            // whole lines, nontemporal: register 2st + h holds, in lane r,
            // token 8h + r%8 of its block (k_operand moves the rows into MFMA
            // order)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int i = 0; i < NJ / 2; ++i)
                tl.k[2 * st + h][i] = pool_load<NT, u32x4>(
                    kb + ((size_t)(4 * i + c) * B + (r & 7) + 8 * h) * 16);
          } else {
            const int ktok = 8 * (r >> 2) + (r & 3);  // + 4th
#pragma unroll
            for (int th = 0; th < 2; ++th)
#pragma unroll
              for (int i = 0; i < NJ / 2; ++i)
                tl.k[2 * st + th][i] =
                    pool_load<kNtK, u32x4>(kb + ((size_t)(4 * i + c) * B + ktok + 4 * th) * 16);
          }
        }
        if constexpr (decltype(WV)::value) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            tl.v[st][dt] = pool_load<kNtV, u32x2>(vb + (size_t)(16 * dt + r) * B + vtok);
        }
      }
    } else {
#pragma unroll
      for (int th = 0; th < NQ; ++th) {
        const size_t blk = pbs[th * 16 / B];
        const int tok = (16 * th) % B;  // token offset of this quarter in its block
        const auto* kb = k_pool + blk * blk_stride + head_off;
        const auto* vb = v_pool + blk * blk_stride + head_off;
        if constexpr (decltype(WK)::value) {
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            tl.k[th][j] = pool_load<kNtK, u32x4>(kb + ((size_t)(4 * j + c) * B + tok + r) * 8);
        }
        if constexpr (decltype(WV)::value) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            tl.v[th][dt] = pool_load<kNtV, u32x2>(vb + (size_t)(16 * dt + r) * B + tok + 4 * c);
        }
      }
    }
  };
  using Yes = std::true_type;
  using No = std::false_type;
  auto load = [&](int k, Tile& tl) { load_part(k, tl, Yes{}, Yes{}); };
  auto load_k = [&](int k, Tile& tl) { load_part(k, tl, Yes{}, No{}); };
  auto load_v = [&](int k, Tile& tl) { load_part(k, tl, No{}, Yes{}); };

  // put the appended token (tile-relative index tn, wave-uniform) into half TH
  // of the final tile:
  // lane (c, r) holds K chunks 4j + c of token 16TH + r and V dims 16dt + r of
  // tokens 16TH + 4c .. +3
  auto substitute = [&](auto& tl, auto half, int tn) {  // bf16 tiles
    constexpr int TH = decltype(half)::value;
    if (r == (tn & 15)) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) tl.k[TH][j] = *reinterpret_cast<const u32x4*>(lds_k + 8 * (4 * j + c));
    }
    if (c == ((tn & 15) >> 2)) {
      const int e = tn & 3;  // element of this lane's 4-token V run
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint32_t nv = lds_v[16 * dt + r];
        uint32_t w = e < 2 ? tl.v[TH][dt][0] : tl.v[TH][dt][1];
        w = (e & 1) ? ((w & 0x0000ffffu) | (nv << 16)) : ((w & 0xffff0000u) | nv);
        if (e < 2)
          tl.v[TH][dt][0] = w;
        else
          tl.v[TH][dt][1] = w;
      }
    }
  };

  // fp8: put the appended token's codes (tile token tn = 32 ST + t) into step
  // ST of the final tile.  Row 4(t/8) + t%4 of quarter (t/4) % 2 holds its K
  // chunks; lanes c = t/8 hold its V codes at byte t%8 of their 8-token runs
  // At B = 16 the K registers hold whole-line rows (see load_part): token t
  // of step ST is in register 2ST + (t/8)%2 at lane 8(t/16) + t%8; TH is that
  // register's half.
  auto substitute8 = [&](auto& tl, auto stc, auto thc, int t) {
    constexpr int ST = decltype(stc)::value, TH = decltype(thc)::value;
    if (B == 16 ? r == 8 * (t >> 4) + (t & 7) : r == 4 * (t >> 3) + (t & 3)) {
#pragma unroll
      for (int i = 0; i < NJ / 2; ++i)
        tl.k[2 * ST + TH][i] = *reinterpret_cast<const u32x4*>(lds_k8 + 16 * (4 * i + c));
    }
    if (c == (t >> 3)) {
      const int e = t & 7;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const uint32_t code = lds_v8[16 * dt + r];
        const uint32_t sh = 8 * (e & 3), keep = ~(0xffu << sh);
        if (e < 4)
          tl.v[ST][dt][0] = (tl.v[ST][dt][0] & keep) | (code << sh);
        else
          tl.v[ST][dt][1] = (tl.v[ST][dt][1] & keep) | (code << sh);
      }
    }
  };

  // MFMA operands: the K vector of quarter th at k-step j, and the V runs of dim
  // tile dt over quarters q0, q0 + 1.  fp8 codes are widened to bf16 here, one
  // operand at a time, so no widened tile is ever held in registers
  auto k_operand = [&](Tile& tl, int th, int j) {
    if constexpr (F8 && B == 16) {
      // quarter th = 2 st + q of the tile.  Row r of quarter q is step token
      // 8(r/4) + 4q + r%4: block r/8, token 8(r%8/4) + 4q + r%4.  Registers 2st
      // (tokens 0..7 of each block) and 2st + 1 (tokens 8..15) hold block r/8's
      // token 8h + r%8 in lane r, so lanes with r%8 < 4 take their row from
      // register 2st (q = 0: lane r; q = 1: lane r + 4) and the others from
      // register 2st + 1 (q = 0: lane r - 4; q = 1: lane r), moved along the
      // 16-lane row by DPP
      const int st = th >> 1, q = th & 1;
      const u32x4 wx = tl.k[2 * st][j >> 1], wy = tl.k[2 * st + 1][j >> 1];
      const uint32_t x0 = (j & 1) ? wx[2] : wx[0], x1 = (j & 1) ? wx[3] : wx[1];
      const uint32_t y0 = (j & 1) ? wy[2] : wy[0], y1 = (j & 1) ? wy[3] : wy[1];
      const bool low = (r & 7) < 4;
      // the DPP moves run on every lane (a lane takes its value from another
      // one, which must be active), then each lane selects
      u32x2 w;
      if (q == 0) {
        const u32x2 sy = {dpp_row_shr4(y0), dpp_row_shr4(y1)};
        w = low ? u32x2{x0, x1} : sy;
      } else {
        const u32x2 sx = {dpp_row_shl4(x0), dpp_row_shl4(x1)};
        w = low ? sx : u32x2{y0, y1};
      }
      return __builtin_bit_cast(bf16x8, fp8x8_to_bf16(w));
    } else if constexpr (F8) {
      const u32x4 w = tl.k[th][j >> 1];
      return __builtin_bit_cast(bf16x8, fp8x8_to_bf16((j & 1) ? u32x2{w[2], w[3]}
                                                              : u32x2{w[0], w[1]}));
    } else {
      return __builtin_bit_cast(bf16x8, tl.k[th][j]);
    }
  };
  auto v_operand = [&](Tile& tl, int q0, int dt) {
    if constexpr (F8) {
      return __builtin_bit_cast(bf16x8, fp8x8_to_bf16(tl.v[q0 / 2][dt]));
    } else {
      return __builtin_bit_cast(bf16x8, u32x4{tl.v[q0][dt][0], tl.v[q0][dt][1],
                                              tl.v[q0 + 1][dt][0], tl.v[q0 + 1][dt][1]});
    }
  };
  // Tokens past the partition end: their scores become -inf and their V
  // elements zero (the pool may hold anything there, NaN included, and a zero
  // weight times NaN would still reach the output).  bf16: this lane's 4-token
  // run in quarter th keeps its first nv elements; fp8: its 8-token run of
  // step q0 / 2 keeps its first nv.
  auto mask_v = [&](Tile& tl, int th, int nv) {
    if constexpr (F8) {
      const uint32_t m0 = nv >= 4 ? 0xffffffffu : (1u << (8 * nv)) - 1u;
      const uint32_t m1 = nv >= 8 ? 0xffffffffu : nv <= 4 ? 0u : (1u << (8 * (nv - 4))) - 1u;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        tl.v[th / 2][dt][0] &= m0;
        tl.v[th / 2][dt][1] &= m1;
      }
    } else {
#pragma unroll
      for (int wd = 0; wd < 2; ++wd) {
        const uint32_t mk =
            (2 * wd < nv ? 0x0000ffffu : 0u) | (2 * wd + 1 < nv ? 0xffff0000u : 0u);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) tl.v[th][dt][wd] &= mk;
      }
    }
  };

  // one 32-token MFMA step over quarters q0, q0 + 1 of a tile: tokens T0 ..
  // T0 + 31, of which T0 is valid
  // `mid()` runs once the step's q.k products have taken their K operands
  auto step32 = [&](Tile& tl, auto q0c, int T0, auto&& mid) {
    constexpr int q0 = decltype(q0c)::value;
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int th = 0; th < 2; ++th)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        sacc[th] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand(tl, q0 + th, j), qb[j],
                                                           sacc[th], 0, 0, 0);
    if constexpr (!std::is_same_v<std::decay_t<decltype(mid)>, NoHook>) {
      // keep the next loads after the products that read these K registers
      // (hoisted above them, old and new K would both be live and spill)
      __builtin_amdgcn_sched_barrier(0);
      mid();
    }
    // sv[4th + i]: raw score of token T0 + 16th + 4c + i (bf16), T0 + 8c + 4th
    // + i (fp8); the score scale joins the exponent's argument
    float sv[8];
#pragma unroll
    for (int th = 0; th < 2; ++th)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[4 * th + i] = sacc[th][i];
    if (T0 + 32 > it.end) {  // the partition's last, partial step
      if constexpr (F8) {
        const int nv = min(max(it.end - (T0 + 8 * c), 0), 8);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= nv) sv[e] = -INFINITY;
        mask_v(tl, q0, nv);
      } else {
#pragma unroll
        for (int th = 0; th < 2; ++th) {
          const int nv = min(max(it.end - (T0 + 16 * th + 4 * c), 0), 4);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i >= nv) sv[4 * th + i] = -INFINITY;
          mask_v(tl, q0 + th, nv);
        }
      }
    }
    // a column moves its reference only when one of its scores passes
    // thr = (m + kLazyMax) / scale (raw units); compares, not a max, find out
    // (the compiler spaces them after the MFMA writes of sacc, and a max of
    // MFMA results would first be made canonical)
    bool hit = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) hit |= sv[i] > thr;
    if (__builtin_amdgcn_ballot_w64(hit) != 0) {
      // the column's largest score (finite: token T0 is valid); the scale is
      // positive, so scaling it gives the largest scaled score
      float lm = sv[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) lm = fmaxf(lm, sv[i]);
      float cm = fmaxf(lm, shfl_xor_f(lm, 16));
      cm = fmaxf(cm, shfl_xor_f(cm, 32));
      const float mn = cm > thr ? cm * score_scale : m;
      const float alpha = fast_exp2(m - mn);  // 1 where unchanged, 0 at the first step
      m = mn;
      thr = (mn + kLazyMax) * inv_scale;
      ls *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
    }
    u32x4 phw, plw;
    float psum = 0.f;
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      const float p0 = fast_exp2(__builtin_fmaf(sv[2 * wd], score_scale, -m));
      const float p1 = fast_exp2(__builtin_fmaf(sv[2 * wd + 1], score_scale, -m));
      psum += p0 + p1;
      // hi: truncated to bf16; lo: the exact remainder rounded to nearest even
      const uint32_t h0 = __float_as_uint(p0) & 0xffff0000u;
      const uint32_t h1 = __float_as_uint(p1) & 0xffff0000u;
      phw[wd] = (h0 >> 16) | h1;
      plw[wd] = __builtin_bit_cast(
          uint32_t, __builtin_convertvector(
                        f32x2v{p0 - __uint_as_float(h0), p1 - __uint_as_float(h1)}, bf16x2v));
    }
    ls += psum;
    const bf16x8 ph = __builtin_bit_cast(bf16x8, phw);
    const bf16x8 pl = __builtin_bit_cast(bf16x8, plw);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const bf16x8 va = v_operand(tl, q0, dt);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, ph, acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pl, acc[dt], 0, 0, 0);
    }
  };
  // tile k; `mid()` runs once the tile's K registers are free (after the last
  // q.k products), so the next loads into them can be issued before the p.v half
  auto compute_mid = [&](int k, Tile& tl, auto&& mid) {
    const int T0 = it.start + k * TILE;
    if constexpr (F8) {
      step32(tl, std::integral_constant<int, 0>{}, T0, NoHook{});
      if (T0 + 32 < it.end)
        step32(tl, std::integral_constant<int, 2>{}, T0 + 32, mid);
      else
        mid();
    } else {
      step32(tl, std::integral_constant<int, 0>{}, T0, mid);
    }
  };
  auto compute = [&](int k, Tile& tl) { compute_mid(k, tl, NoHook{}); };

  if constexpr (AP) {
    pipelined_split<Tile>(n, load, load_k, load_v, compute_mid, stage_new, [&](int k, Tile& tl) {
      const int tn = tnew - (it.start + k * TILE);  // in this tile when appending
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      if (appends) {
        if constexpr (F8) {
          const int t = tn & 31, th = B == 16 ? (t >> 3) & 1 : (t >> 2) & 1;
          if (tn < 32) {
            if (th == 0) substitute8(tl, I0{}, I0{}, t); else substitute8(tl, I0{}, I1{}, t);
          } else {
            if (th == 0) substitute8(tl, I1{}, I0{}, t); else substitute8(tl, I1{}, I1{}, t);
          }
        } else {
          if (tn < 16)
            substitute(tl, I0{}, tn);
          else
            substitute(tl, I1{}, tn);
        }
      }
      compute(k, tl);
    });
  } else {
    pipelined_split<Tile>(n, load, load_k, load_v, compute_mid, NoHook{}, compute);
  }

  ls += shfl_xor_f(ls, 16);
  ls += shfl_xor_f(ls, 32);
  if (it.nps > 1 && a.counters) {
    // partial rows at device scope, then the merge by the last item
    const PartialRows<D, G> pr(a, it.s, it.g);
    if (r < G) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        pr.store4(acc[dt] * out_scale, pr.acc_off(r, it.p, 16 * dt + 4 * c));
      if (c == 0) pr.store_ml(m, ls, pr.ml_off(r, it.p));
    }
    if (arrive_last(a, it.s, it.g, it.nps)) merge_partials<D, G>(a, it.s, it.g, it.nps);
    return;
  }
  if (r < G) {
    const RowSink dst = row_sink<D, G>(a, it, r);
    const float scl = (dst.ml ? 1.f : 1.f / ls) * out_scale;
    if (dst.ml) {
      const PartialRows<D, G> pr(a, it.s, it.g);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        pr.store4_nt(acc[dt] * scl, pr.acc_off(r, it.p, 16 * dt + 4 * c));
    } else {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4*>(dst.acc + 16 * dt + 4 * c) = acc[dt] * scl;
    }
    if (dst.ml && c == 0) {
      dst.ml[0] = m;
      dst.ml[1] = ls;
    }
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of partition partials: one TPR-thread workgroup per
// (sequence, query head) row (TPR = 64 when a row has at most 16 partitions,
// 256 for long contexts).  Thread (pg, col) folds partitions pg, pg + PG, ... of
// float4 column col into a local (max, sum, acc) state; U partitions per thread
// are loaded at once (indices past the end re-read the last partition with
// weight 0), so one round trip covers U * PG partitions (16 or 64).  The PG
// local states are then merged through LDS.
// ---------------------------------------------------------------------------
template <int D, int TPR>
__global__ __launch_bounds__(TPR) void pa_reduce_kernel(float* __restrict__ out,
                                                        const float* __restrict__ part_acc,
                                                        const float* __restrict__ part_ml,
                                                        const int* __restrict__ context_lens,
                                                        const int* __restrict__ merge_rows, int S,
                                                        int Hq, int G, int max_blocks, int B,
                                                        int nparts, int P) {
  constexpr int C4 = D / 4;                       // float4 columns of a row
  constexpr int PG = TPR / C4;                    // partition groups
  constexpr int U = (TPR == 64 ? 16 : 64) / PG;   // partitions per thread per round
  static_assert(PG >= 1 && U >= 1, "unsupported reduce shape");
  __shared__ float sm_m[PG], sm_l[PG];
  __shared__ f32x4 sm_acc[PG][C4];

  // row = s * Hq + h: every row of the batch, or (planned) the G query heads of
  // each listed (sequence, KV head) = s * Hkv + g, whose rows are (s*Hkv + g)*G + gi
  int row = blockIdx.x;
  if (merge_rows) {
    const int sg = merge_rows[blockIdx.x / G];
    if (sg < 0 || sg >= S * (Hq / G)) return;
    row = sg * G + (int)(blockIdx.x % G);
  }
  const int s = row / Hq;
  const int L = min(context_lens[s], max_blocks * B);
  const int n = L <= 0 ? 0 : min((L + P - 1) / P, nparts);
  if (n <= 1) return;  // the main kernel wrote this row
  const int col = threadIdx.x % C4, pg = threadIdx.x / C4;
  const float* ml = part_ml + (size_t)row * nparts * 2;
  const f32x4* pa = reinterpret_cast<const f32x4*>(part_acc + (size_t)row * nparts * D);

  float M = -INFINITY, den = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = pg; i0 < n; i0 += PG * U) {
    float mi[U], li[U];
    f32x4 ai[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = min(i0 + u * PG, n - 1);
      mi[u] = ml[2 * i];
      li[u] = ml[2 * i + 1];
      ai[u] = pa[(size_t)i * C4 + col];
    }
    float mn = M;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + u * PG >= n) mi[u] = -INFINITY;
      mn = fmaxf(mn, mi[u]);
    }
    const float fo = fast_exp2(M - mn);  // M = -inf gives 0
    den *= fo;
    acc *= fo;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float f = fast_exp2(mi[u] - mn);  // -inf (past the end) gives 0
      den = fmaf(f, li[u], den);
      acc += f * ai[u];
    }
    M = mn;
  }
  if (col == 0) {
    sm_m[pg] = M;
    sm_l[pg] = den;
  }
  sm_acc[pg][col] = acc;
  __syncthreads();
  if (threadIdx.x < C4) {
    float Mg = -INFINITY;
#pragma unroll
    for (int j = 0; j < PG; ++j) Mg = fmaxf(Mg, sm_m[j]);
    float dg = 0.f;
    f32x4 ag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < PG; ++j) {
      const float mj = sm_m[j];
      const float f = (mj == -INFINITY) ? 0.f : fast_exp2(mj - Mg);
      dg = fmaf(f, sm_l[j], dg);
      ag += f * sm_acc[j][threadIdx.x];
    }
    const float inv = 1.f / dg;
    reinterpret_cast<f32x4*>(out + (size_t)row * D)[threadIdx.x] = ag * inv;
  }
}

// ---------------------------------------------------------------------------
// Host dispatch.
// ---------------------------------------------------------------------------
// E is the pool element: float, uint16_t (bf16) or uint8_t (fp8 E4M3, whose
// queries and appended tokens are bf16): the MFMA kernel for G >= 4, else VALU.
template <typename E, int D, int B, int G, bool NT>
static void launch_main_nt(const DecodeArgs& a, unsigned grid, const void* q, void* kp, void* vp,
                           hipStream_t st) {
  constexpr bool kMfma = sizeof(E) <= 2 && G >= 4;
  // the append variants hold more registers and a longer epilogue; plain
  // launches compile without them
  using QE = std::conditional_t<sizeof(E) == 1, uint16_t, E>;
  if constexpr (sizeof(E) == 1 && G >= 4) {
    {
      if (a.new_k)
        pa_mfma_kernel<D, B, G, kWavesPerGroup, NT, true, true>
            <<<grid, kWavesPerGroup * kWave, 0, st>>>(a, (const uint16_t*)q, (uint8_t*)kp,
                                                       (uint8_t*)vp);
      else
        pa_mfma_kernel<D, B, G, kWavesPerGroup, NT, false, true>
            <<<grid, kWavesPerGroup * kWave, 0, st>>>(a, (const uint16_t*)q, (uint8_t*)kp,
                                                       (uint8_t*)vp);
    }
  } else if constexpr (kMfma) {
    if (a.new_k)
      pa_mfma_kernel<D, B, G, kWavesPerGroup, NT, true, false>
          <<<grid, kWavesPerGroup * kWave, 0, st>>>(a, (const uint16_t*)q, (uint16_t*)kp,
                                                     (uint16_t*)vp);
    else
      pa_mfma_kernel<D, B, G, kWavesPerGroup, NT, false, false>
          <<<grid, kWavesPerGroup * kWave, 0, st>>>(a, (const uint16_t*)q, (uint16_t*)kp,
                                                     (uint16_t*)vp);
  } else {
    if (a.new_k)
      pa_valu_kernel<E, D, B, G, kWavesPerGroup, NT, true><<<grid, kWavesPerGroup * kWave, 0, st>>>(
          a, (const QE*)q, (E*)kp, (E*)vp);
    else
      pa_valu_kernel<E, D, B, G, kWavesPerGroup, NT, false><<<grid, kWavesPerGroup * kWave, 0, st>>>(
          a, (const QE*)q, (E*)kp, (E*)vp);
  }
}

template <typename E, int D, int B, int G>
static void launch_main(bool stream, const DecodeArgs& a, unsigned grid, const void* q,
                        void* kp, void* vp, hipStream_t st) {
  if (stream)
    launch_main_nt<E, D, B, G, true>(a, grid, q, kp, vp, st);
  else
    launch_main_nt<E, D, B, G, false>(a, grid, q, kp, vp, st);
}

template <typename E, int D, int B>
static bool dispatch_g(int G, bool stream, const DecodeArgs& a, unsigned grid, const void* q,
                       void* kp, void* vp, hipStream_t st) {
  switch (G) {
    case 1: launch_main<E, D, B, 1>(stream, a, grid, q, kp, vp, st); return true;
    case 2: launch_main<E, D, B, 2>(stream, a, grid, q, kp, vp, st); return true;
    case 4: launch_main<E, D, B, 4>(stream, a, grid, q, kp, vp, st); return true;
    case 8: launch_main<E, D, B, 8>(stream, a, grid, q, kp, vp, st); return true;
    default: return false;
  }
}

template <typename E, int D>
static bool dispatch_b(int B, int G, bool stream, const DecodeArgs& a, unsigned grid,
                       const void* q, void* kp, void* vp, hipStream_t st) {
  if (B == 16) return dispatch_g<E, D, 16>(G, stream, a, grid, q, kp, vp, st);
  if (B == 32) return dispatch_g<E, D, 32>(G, stream, a, grid, q, kp, vp, st);
  return false;
}

template <typename E>
static bool dispatch_d(int D, int B, int G, bool stream, const DecodeArgs& a, unsigned grid,
                       const void* q, void* kp, void* vp, hipStream_t st) {
  if (D == 64) return dispatch_b<E, 64>(B, G, stream, a, grid, q, kp, vp, st);
  if (D == 128) return dispatch_b<E, 128>(B, G, stream, a, grid, q, kp, vp, st);
  return false;
}

static bool shape_supported(int D, int B, int G) {
  return (D == 64 || D == 128) && (B == 16 || B == 32) && (G == 1 || G == 2 || G == 4 || G == 8);
}

static int64_t num_partitions(int64_t max_context_len, int P) {
  return max_context_len <= 0 ? 1 : (max_context_len + P - 1) / P;
}

// Workspace of a split launch: kMergeCounters int32 merge counters, one per
// (sequence, KV head), at a fixed place whatever the batch, so a workspace can
// serve calls of any size without a counter ever landing on bytes another call
// used for partials; then the partials acc [S, Hq, nparts, D] and (m, l)
// [S, Hq, nparts, 2].
constexpr int64_t kMergeCounters = 16384;
constexpr size_t kCounterBytes = kMergeCounters * 4;
static size_t split_workspace_bytes(int64_t S, int64_t Hq, int64_t D, int64_t nparts) {
  return kCounterBytes + (size_t)S * Hq * nparts * (D + 2) * sizeof(float);
}
// The main launch merges the partitions itself (else the reduce launch does).
static bool merge_in_launch(int64_t S, int64_t Hkv, int64_t nparts) {
  return nparts <= kMergeInLaunchMax && S * Hkv <= kMergeCounters;
}

// The optional host-built plan: n_items records of 4 int32, then n_merge rows.
struct PlanArg {
  const int32_t* ptr;
  int32_t n_items, n_merge;
};

static bool plan_ok(const PlanArg& pl) {
  if (!pl.ptr) return true;
  return aligned16(pl.ptr) && pl.n_items >= 0 && pl.n_merge >= 0;
}

// Host validation and argument set-up shared by the attention entry points.
// On PKV_OK, *a and *groups describe the main launch (groups == 0: nothing to
// launch).
static pkv_status prepare_decode(DecodeArgs* a, int64_t* groups, float* out, const void* q,
                                 const void* k_pool, const void* v_pool, const void* new_key,
                                 const void* new_value, const int32_t* block_tables,
                                 const int32_t* context_lens,
                                 int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                 int32_t max_blocks, int32_t num_blocks, int32_t max_context_len,
                                 float scale, int32_t partition_size, const PlanArg& plan,
                                 void* workspace, size_t workspace_bytes, pkv_dtype dtype,
                                 uint32_t flags, const float* k_scale, const float* v_scale) {
  *groups = 0;
  if (flags & ~(uint32_t)PKV_ATTN_SHARED_KV) return PKV_EINVAL;
  if (S < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_blocks <= 0 || num_blocks <= 0 ||
      max_context_len < 0 || partition_size < 0 || !(scale > 0.f) || !std::isfinite(scale) ||
      !plan_ok(plan))
    return PKV_EINVAL;
  if (dtype != PKV_F32 && dtype != PKV_BF16 && dtype != PKV_FP8_E4M3) return PKV_EINVAL;
  const int G = Hq / Hkv;
  if (!shape_supported(D, B, G)) return PKV_EUNSUPPORTED;
  if (dtype == PKV_FP8_E4M3) {
    if (!k_scale || !v_scale) return PKV_EINVAL;
  }
  const int P = resolve_partition(partition_size, B);
  if (P == 0) return PKV_EINVAL;
  if (S == 0) return PKV_OK;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !block_tables || !context_lens)
    return PKV_EINVAL;
  if ((new_key == nullptr) != (new_value == nullptr)) return PKV_EINVAL;
  if (new_key && (!aligned16(new_key) || !aligned16(new_value))) return PKV_EINVAL;
  const int64_t mcl = std::min<int64_t>(max_context_len, (int64_t)max_blocks * B);
  const int64_t nparts = num_partitions(mcl, P);
  const int64_t items = plan.ptr ? (int64_t)plan.n_items : (int64_t)S * Hkv * nparts;
  const int64_t store_items = new_key ? S : 0;
  if (items + store_items > 0x7fffffffLL || (int64_t)S * Hq > 0x7fffffffLL) return PKV_EINVAL;
  *a = DecodeArgs{};
  a->out = out;
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->new_k = new_key;
  a->new_v = new_value;
  a->plan = reinterpret_cast<const int4*>(plan.ptr);
  a->k_scale = k_scale;
  a->v_scale = v_scale;
  a->S = S;
  a->SG = S * Hkv;
  a->items = (int)items;
  a->store_items = (int)store_items;
  a->Hkv = Hkv;
  a->max_blocks = max_blocks;
  a->num_blocks = num_blocks;
  a->nparts = (int)nparts;
  a->P = P;
  a->scale_log2e = scale * 1.4426950408889634f;
  if (nparts > 1) {
    if (!aligned16(workspace) || workspace_bytes < split_workspace_bytes(S, Hq, D, nparts))
      return PKV_EINVAL;
    a->counters = merge_in_launch(S, Hkv, nparts) ? (int*)workspace : nullptr;
    a->part_acc = (float*)((char*)workspace + kCounterBytes);
    a->part_ml = a->part_acc + (size_t)S * Hq * nparts * D;
  }
  // attention items, then (appending) one store item per sequence
  *groups = (items + store_items + kWavesPerGroup - 1) / kWavesPerGroup;
  return PKV_OK;
}

static pkv_status launch_main_kernel(const DecodeArgs& a, int64_t groups, const void* q,
                                     void* k_pool, void* v_pool, int D, int B, int G,
                                     pkv_dtype dtype, uint32_t flags, hipStream_t st) {
  const bool stream = (flags & PKV_ATTN_SHARED_KV) == 0;
  const unsigned g = (unsigned)groups;
  const bool ok =
      dtype == PKV_F32    ? dispatch_d<float>(D, B, G, stream, a, g, q, k_pool, v_pool, st)
      : dtype == PKV_BF16 ? dispatch_d<uint16_t>(D, B, G, stream, a, g, q, k_pool, v_pool, st)
                          : dispatch_d<uint8_t>(D, B, G, stream, a, g, q, k_pool, v_pool, st);
  if (!ok) return PKV_EUNSUPPORTED;
  return launch_status();
}

// The merge launch: every row of the batch, or only the plan's merge rows.
static pkv_status launch_reduce_kernel(const DecodeArgs& a, const PlanArg& plan, int S, int Hq,
                                       int G, int D, int B, hipStream_t st) {
  if (a.counters) return PKV_OK;  // merged by the main launch
  const int* rows = plan.ptr ? plan.ptr + 4 * (size_t)plan.n_items : nullptr;
  const int64_t grid = plan.ptr ? (int64_t)plan.n_merge * G : (int64_t)S * Hq;
  if (grid == 0) return PKV_OK;
  if (grid > 0x7fffffffLL) return PKV_EINVAL;
  const bool small = a.nparts <= 16;  // one round of a 64-thread row covers it
#define PKV_REDUCE(DD, TT)                                                                \
  pa_reduce_kernel<DD, TT><<<(unsigned)grid, TT, 0, st>>>(a.out, a.part_acc, a.part_ml,   \
                                                          a.context_lens, rows, S, Hq, G, \
                                                          a.max_blocks, B, a.nparts, a.P)
  if (D == 64) {
    if (small) PKV_REDUCE(64, 64); else PKV_REDUCE(64, 256);
  } else {
    if (small) PKV_REDUCE(128, 64); else PKV_REDUCE(128, 256);
  }
#undef PKV_REDUCE
  return launch_status();
}

}  // namespace pkv

using namespace pkv;

extern "C" size_t pkv_attention_workspace_bytes(int32_t S, int32_t Hq, int32_t D,
                                                int32_t max_context_len, int32_t partition_size) {
  if (S <= 0 || Hq <= 0 || D <= 0 || partition_size < 0) return 0;
  const int P = partition_size > 0 ? partition_size : kDefaultPartition;
  const int64_t np = num_partitions(max_context_len, P);
  if (np <= 1) return 0;
  return split_workspace_bytes(S, Hq, D, np);
}

extern "C" pkv_status pkv_paged_attention_decode(
    float* out, const void* q, void* k_pool, void* v_pool, const void* new_key,
    const void* new_value, const int32_t* block_tables, const int32_t* context_lens, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
    int32_t max_blocks, int32_t num_blocks, int32_t max_context_len, float scale,
    int32_t partition_size, const int32_t* plan, int32_t plan_items, int32_t plan_merge,
    void* workspace, size_t workspace_bytes, pkv_dtype dtype, uint32_t flags,
    const float* k_scale, const float* v_scale, void* hip_stream) {
  DecodeArgs a;
  int64_t groups;
  const PlanArg pl{plan, plan_items, plan_merge};
  pkv_status st = prepare_decode(&a, &groups, out, q, k_pool, v_pool, new_key, new_value,
                                 block_tables, context_lens,
                                 S, Hq, Hkv, D, B, max_blocks, num_blocks, max_context_len, scale,
                                 partition_size, pl, workspace, workspace_bytes, dtype, flags,
                                 k_scale, v_scale);
  if (st != PKV_OK || groups == 0) return st;
  hipStream_t hs = (hipStream_t)hip_stream;
  st = launch_main_kernel(a, groups, q, k_pool, v_pool, D, B, Hq / Hkv, dtype, flags, hs);
  if (st != PKV_OK) return st;
  return launch_reduce_kernel(a, pl, S, Hq, Hq / Hkv, D, B, hs);
}

extern "C" pkv_status pkv_paged_attention_main(
    float* out, const void* q, void* k_pool, void* v_pool, const void* new_key,
    const void* new_value, const int32_t* block_tables, const int32_t* context_lens, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
    int32_t max_blocks, int32_t num_blocks, int32_t max_context_len, float scale,
    int32_t partition_size, const int32_t* plan, int32_t plan_items, int32_t plan_merge,
    void* workspace, size_t workspace_bytes, pkv_dtype dtype, uint32_t flags,
    const float* k_scale, const float* v_scale, void* hip_stream) {
  DecodeArgs a;
  int64_t groups;
  const PlanArg pl{plan, plan_items, plan_merge};
  pkv_status st = prepare_decode(&a, &groups, out, q, k_pool, v_pool, new_key, new_value,
                                 block_tables, context_lens,
                                 S, Hq, Hkv, D, B, max_blocks, num_blocks, max_context_len, scale,
                                 partition_size, pl, workspace, workspace_bytes, dtype, flags,
                                 k_scale, v_scale);
  if (st != PKV_OK || groups == 0) return st;
  return launch_main_kernel(a, groups, q, k_pool, v_pool, D, B, Hq / Hkv, dtype, flags,
                            (hipStream_t)hip_stream);
}

extern "C" pkv_status pkv_paged_attention_reduce(
    float* out, const int32_t* context_lens, int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
    int32_t B, int32_t max_blocks, int32_t max_context_len, int32_t partition_size,
    const int32_t* plan, int32_t plan_items, int32_t plan_merge, const void* workspace,
    size_t workspace_bytes, void* hip_stream) {
  const PlanArg pl{plan, plan_items, plan_merge};
  if (S < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_blocks <= 0 || max_context_len < 0 ||
      partition_size < 0 || !plan_ok(pl))
    return PKV_EINVAL;
  if (!(D == 64 || D == 128) || !(B == 16 || B == 32)) return PKV_EUNSUPPORTED;
  const int P = resolve_partition(partition_size, B);
  if (P == 0) return PKV_EINVAL;
  if (S == 0) return PKV_OK;
  if (!aligned16(out) || !context_lens) return PKV_EINVAL;
  const int64_t mcl = std::min<int64_t>(max_context_len, (int64_t)max_blocks * B);
  const int64_t nparts = num_partitions(mcl, P);
  if ((int64_t)S * Hq > 0x7fffffffLL) return PKV_EINVAL;
  if (merge_in_launch(S, Hkv, nparts)) return PKV_OK;  // merged by the main launch
  if (!aligned16(workspace) || workspace_bytes < split_workspace_bytes(S, Hq, D, nparts))
    return PKV_EINVAL;
  DecodeArgs a{};
  a.out = out;
  a.context_lens = context_lens;
  a.max_blocks = max_blocks;
  a.nparts = (int)nparts;
  a.P = P;
  a.part_acc = (float*)((const char*)workspace + kCounterBytes);
  a.part_ml = a.part_acc + (size_t)S * Hq * nparts * D;
  return launch_reduce_kernel(a, pl, S, Hq, Hq / Hkv, D, B, (hipStream_t)hip_stream);
}

// ---------------------------------------------------------------------------
// The decode call without a workspace argument, for callers that cannot
// allocate.  Its partials and merge counters live in `scratch`, one array per
// GPU the library runs on.  In host code `scratch` only names the symbol: its
// device address on the current GPU comes from hipGetSymbolAddress, taken once
// per device at the first call there and kept; only that address is passed to
// kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[PKV_SCRATCH_BYTES];

namespace pkv {

constexpr int kMaxScratchDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxScratchDevices];

// Device address of `scratch` on the device of `st`, which must be current.
static pkv_status scratch_address(hipStream_t st, void** out) {
  int cur = -1, dev = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur < 0) return PKV_EHIP;
  if (hipStreamGetDevice(st, &dev) != hipSuccess || dev < 0) return PKV_EHIP;
  if (dev != cur) return PKV_EINVAL;
  if (dev >= kMaxScratchDevices) return PKV_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PKV_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

__global__ void clear_words_kernel(int* __restrict__ w, int n) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) w[i] = 0;
}

}  // namespace pkv

extern "C" pkv_status pkv_paged_attention_decode_noalloc(
    float* out, const void* q, void* k_pool, void* v_pool, const void* new_key,
    const void* new_value, const int32_t* block_tables, const int32_t* context_lens, int32_t S,
    int32_t Hq, int32_t Hkv, int32_t D, int32_t B, int32_t max_blocks, int32_t num_blocks,
    int32_t max_context_len, float scale, int32_t partition_size, const int32_t* plan,
    int32_t plan_items, int32_t plan_merge, pkv_dtype dtype, uint32_t flags,
    const float* k_scale, const float* v_scale, void* hip_stream) {
  if (S < 0 || Hq <= 0 || D <= 0 || max_context_len < 0 || partition_size < 0)
    return PKV_EINVAL;
  const size_t need = pkv_attention_workspace_bytes(S, Hq, D,
                                                    std::min<int64_t>(max_context_len,
                                                                      (int64_t)std::max(max_blocks, 0) * B),
                                                    partition_size);
  if (need > PKV_SCRATCH_BYTES) return PKV_ENOSCRATCH;
  hipStream_t hs = (hipStream_t)hip_stream;
  void* ws = nullptr;
  pkv_status st = scratch_address(hs, &ws);
  if (st != PKV_OK) return st;
  DecodeArgs a;
  int64_t groups;
  const PlanArg pl{plan, plan_items, plan_merge};
  st = prepare_decode(&a, &groups, out, q, k_pool, v_pool, new_key, new_value, block_tables,
                      context_lens, S, Hq, Hkv, D, B, max_blocks, num_blocks, max_context_len,
                      scale, partition_size, pl, ws, PKV_SCRATCH_BYTES, dtype, flags, k_scale,
                      v_scale);
  if (st != PKV_OK || groups == 0) return st;
  if (a.counters) {
    // the merge counters must start at zero: a call is not trusted to have
    // left them so (it may have been cut short)
    const int n = S * Hkv;
    clear_words_kernel<<<(unsigned)((n + 255) / 256), 256, 0, hs>>>(a.counters, n);
    st = launch_status();
    if (st != PKV_OK) return st;
  }
  st = launch_main_kernel(a, groups, q, k_pool, v_pool, D, B, Hq / Hkv, dtype, flags, hs);
  if (st != PKV_OK) return st;
  return launch_reduce_kernel(a, pl, S, Hq, Hq / Hkv, D, B, hs);
}

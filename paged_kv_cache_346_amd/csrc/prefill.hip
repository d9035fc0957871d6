// Multi-token queries over the paged KV cache for gfx950 (CDNA4): chunked
// prefill, and the uncached rest of a prompt after a prefix-cache hit
// (PagedAttention: The vLLM Paper, "Impact and Follow-Ups": prefix caching
// reuses the KV of a shared prompt prefix so only the rest is prefilled;
// chunked prefill splits a long prompt into chunks interleaved with decode).
//
// What is computed: sequence s holds L_s cached tokens, the last Q_s of which
// are this call's queries (their K/V are already in the cache).  The query at
// position p = L_s - Q_s + i attends causally to tokens 0..p ("Background and
// Motivation": each token attends over itself and every earlier token):
//   out[row, h] = softmax(q[row, h] . K_s[0..p]^T * scale) V_s[0..p]
// with query head h reading KV head h / G.  Rows are packed sequence by
// sequence: sequence s owns rows query_start[s] .. query_start[s+1]-1.
//
// Work decomposition (not on the pages).  A query group is 16/G consecutive
// query tokens: the 16 columns of v_mfma_f32_16x16x32_bf16 hold (token, head)
// pairs, 16/G tokens times the G heads of the KV head, so the matrix core is
// full for every G.  A workgroup of PW waves owns a (sequence, KV head, PW * NGQ
// consecutive query groups) item, NGQ groups per wave, and walks the sequence's
// KV from token 0 to the item's last position in 32-token tiles.  Each tile is
// copied once per workgroup straight from the pool into LDS (buffer loads that
// write LDS, no registers on the way) and each wave reads its MFMA operands from
// there, so a tile feeds PW * NGQ * 16 query columns.  Tiles move through a
// ring of three LDS slots: tile k + 2 lands while tile k is computed, with one
// barrier per tile; the small ring lets three workgroups share a CU.  The
// products are the decode kernel's operand layouts (bf16 hi + lo split of P,
// base-2 softmax), with one softmax state and accumulator per group; each
// column masks the tokens after its own position (causal) on the tiles that
// cross it.  The softmax keeps, per column, a reference m that may trail the
// column's running maximum by at most 8 (log2 units): the accumulator and the
// weight sum are rescaled only when a score passes m + 8, which after the first
// tiles is rare, and out = acc / sum holds for any reference.  Items are
// numbered from the end of each sequence's chunk, so the items with the longest
// KV range are dispatched first; every item of a sequence reads the same
// prefix, so the pool copies are ordinary cached loads.
// fp8 E4M3 pools: the tiles hold the raw codes (half the bytes) and each MFMA
// operand is widened to bf16 where it is used (exact: an E4M3 value fits bf16);
// the K scale joins the score scale and the V scale the output.
#include <cmath>
#include <type_traits>

#include "../../include/pkv.h"
#include "device_common.h"
#include "kv_tiles.h"
#include "launch_check.h"

namespace pkv {

struct PrefillArgs {
  float* out;                 // [T, Hq, D]
  const int* block_tables;    // [S, max_blocks]
  const int* context_lens;    // [S]
  const int* query_start;     // [S + 1]
  const float* k_scale;       // fp8 pools: per-KV-head scales, else nullptr
  const float* v_scale;
  int S, Hkv, T, max_blocks, num_blocks;
  float scale_log2e;
};

// Four waves of two groups each: 128 query columns per tile (measured on 16 x
// (1,536 cached + 512 new) tokens against four waves of one group and eight of
// one), at most 168 VGPRs so that three workgroups fit a CU.
constexpr int kPrefillSharedWaves = 4;
constexpr int kPrefillSharedGroups = 2;
constexpr int kPrefillOcc = 3;  // workgroups per CU (waves per SIMD)

// Max over lanes r, r + 16, r + 32, r + 48 (a score column's four row groups)
// with gfx950's lane-swap instructions instead of LDS permutes: swapping halves
// (rows) between two copies of x leaves each lane its own value in one register
// and that of lane ^ 32 (lane ^ 16) in the other.  The max is exact, so the
// order of the two steps does not matter.
__device__ __forceinline__ float max_over_rows(float x) {
  const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// Direct pool -> LDS copies of 16-byte chunks; the destination of lane i of a
// copy is the copy's LDS base + 16 i, so the lane's choice of source chunk lays
// the tile out in LDS.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
constexpr int kWaitVmem0 = 0x0F70;  // s_waitcnt vmcnt(0), other counters unwaited
// Buffer resource word 3 of a raw byte buffer on gfx9 parts (32-bit data
// format, no swizzle, no index stride)
constexpr int kBufferRsrcWord3 = 0x00020000;

// One copy: lane i moves the 16 bytes at byte offset off of the n-byte region
// at base (scalar) to LDS byte lds + 16 i.  A buffer load takes the scalar
// base and a 32-bit lane offset as they are, so no lane forms a 64-bit
// address, and its range check keeps every lane inside the region (the
// offsets used here always fall inside it).
__device__ __forceinline__ void copy16_to_lds(const uint8_t* base, int n, uint32_t off,
                                              uint8_t* lds) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, n, kBufferRsrcWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)lds, 16, off, 0, 0, 0);
}

// LDS layout of one 32-token tile (K, then V), CE = 16 / sizeof(element),
// CPT = D / CE:
//   K chunk (h, cc, sl) at 16 (16 (CPT h + cc) + sl): dims [CE cc, CE cc + CE) of
//     token 16h + (sl ^ 4h) (the second half's slots are swapped in fours);
//   V chunk (qv, d) at KB + 16 (D qv + d): tokens [CE qv, CE qv + CE) of dim d.
// Token order in the MFMAs: row 4c + i of quarter th of a score tile is token
// 8c + 4th + i, so lane (c, r) holds the scores of tokens 8c .. 8c + 7 of its
// column, which are also the eight consecutive V tokens of its P.V operand.  The
// slot swap spreads a K operand read over all LDS banks.
template <int D, int B, int G, int PW, int NGQ, bool F8>
__global__ __launch_bounds__(PW* kWave, kPrefillOcc) void pa_prefill_shared_kernel(
    PrefillArgs a, const uint16_t* __restrict__ q,
    const std::conditional_t<F8, uint8_t, uint16_t>* __restrict__ k_pool,
    const std::conditional_t<F8, uint8_t, uint16_t>* __restrict__ v_pool) {
  using E = std::conditional_t<F8, uint8_t, uint16_t>;
  constexpr int ES = (int)sizeof(E);
  constexpr int TILE = 32;
  constexpr int NJ = D / 32;         // q.k k-steps
  constexpr int NDT = D / 16;        // p.v output dim tiles
  constexpr int QT = 16 / G;         // query tokens per group
  constexpr int GPS = PW * NGQ;      // query groups per workgroup item
  constexpr int CE = 16 / ES;        // elements per 16-byte chunk
  constexpr int CPT = D / CE;        // chunks of one token's K
  constexpr int KCH = TILE * CPT;    // chunks of a tile's K (and of its V)
  constexpr int KB = 16 * KCH;
  constexpr int RUNS = 2 * KCH / kWave;  // 64-chunk copies per tile
  constexpr int RPW = RUNS / PW;         // per wave
  // s_waitcnt with at most RPW vector memory operations outstanding
  constexpr int kWaitVmemRPW = (RPW & 0xF) | ((RPW >> 4) << 14) | (0x7 << 4) | (0xF << 8);
  constexpr int NBUF = 3;                // tile ring: tile k + 2 lands while k is computed
  static_assert(16 % G == 0 && (B == 16 || B == 32) && D % kWave == 0, "unsupported shape");
  static_assert(KCH % kWave == 0 && RUNS % PW == 0, "a tile's copies split evenly over the waves");
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  __shared__ __align__(16) uint8_t smem[NBUF][2 * KB];

  // wave-uniform (scalar) values: the wave's index and all its tile bounds
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int c = lane >> 4, r = lane & 15;
  const int SG = a.S * a.Hkv;
  const int k_end = (int)blockIdx.x / SG;  // item counted from the chunk's end
  const int sg = (int)blockIdx.x - k_end * SG;
  const int s = sg / a.Hkv, g = sg - s * a.Hkv;
  const int Hq = a.Hkv * G;

  // workgroup-uniform exits only (before the first barrier)
  const int row0 = a.query_start[s];
  const int row1 = a.query_start[s + 1];
  const int L = min(a.context_lens[s], a.max_blocks * B);
  if (row0 < 0 || row1 > a.T || row1 < row0) return;  // a malformed offset: no rows
  const int Q = min(row1 - row0, L);
  if (Q <= 0) return;
  const int rbase = row1 - Q;  // row of query 0 (rows past L_s leave the first ones out)
  const int nsets = ((Q + QT - 1) / QT + GPS - 1) / GPS;
  const int set = nsets - 1 - k_end;
  if (set < 0) return;
  // one past the item's last position: the tiles the workgroup loads
  const int end = L - Q + min((set + 1) * GPS * QT, Q);

  // this wave's groups; a wave whose groups all lie past the chunk still copies
  // its share of every tile and takes every barrier
  const int qg0 = set * GPS + wave * NGQ;
  const bool active = qg0 * QT < Q;
  const int gi = r % G;
  int qi[NGQ], pos[NGQ];
  bool col_valid[NGQ];
#pragma unroll
  for (int u = 0; u < NGQ; ++u) {
    const int qi_raw = (qg0 + u) * QT + r / G;
    col_valid[u] = qi_raw < Q;
    qi[u] = min(qi_raw, Q - 1);
    pos[u] = L - Q + qi[u];
  }
  const int wend = L - Q + min((qg0 + NGQ) * QT, Q);  // one past the wave's last position
  const int first_pos = L - Q + qg0 * QT;

  bf16x8 qb[NGQ][NJ];
#pragma unroll
  for (int u = 0; u < NGQ; ++u) {
    const uint16_t* qrow = q + ((size_t)(rbase + qi[u]) * Hq + g * G + gi) * D;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      qb[u][j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 8 * (4 * j + c)));
  }
  // Running state per column, relative to a reference m that trails the true
  // maximum by at most kLazyMax: out = acc / ls exactly as with the maximum.
  float m[NGQ], ls[NGQ], thr[NGQ];
  f32x4 acc[NGQ][NDT];
#pragma unroll
  for (int u = 0; u < NGQ; ++u) {
    m[u] = -INFINITY;
    thr[u] = -INFINITY;
    ls[u] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // fp8: the K scale joins the score scale, the V scale the output
  const float score_scale = F8 ? a.scale_log2e * a.k_scale[g] : a.scale_log2e;
  const float out_scale = F8 ? a.v_scale[g] : 1.f;
  const float inv_scale = 1.f / score_scale;
  const int n = (end + TILE - 1) / TILE;
  const int nb_last = (end + B - 1) / B - 1;  // a block past it repeats it (masked tokens)
  const int* table = a.block_tables + (size_t)s * a.max_blocks;
  const size_t head_off = (size_t)g * (D * B) * ES;
  const size_t blk_stride = (size_t)a.Hkv * (D * B) * ES;

  // this wave's copies: copy rj = wave + PW i moves chunks 64 rj .. 64 rj + 63 of
  // the tile (K chunks, then V chunks), all from one of the tile's blocks
  // (B = 16: two); per lane, the chunk's byte offset inside its (block, head)
  // region -- the same for every tile
  static_assert((PW & (PW - 1)) == 0, "a power-of-two count of waves");
  const int wv = wave & (PW - 1);  // == wave; the mask lets the compiler fold each copy's block
  uint32_t src_off[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int p = kWave * (wv + PW * i) + lane;
    if (p < KCH) {
      const int h = p / (16 * CPT), cc = (p / 16) % CPT, sl = p % 16;
      const int t = 16 * h + (sl ^ (4 * h));
      src_off[i] = (uint32_t)((cc * B + t % B) * 16);
    } else {
      const int pv = p - KCH;
      const int t0 = (pv / D) * CE, d = pv % D;
      src_off[i] = (uint32_t)((d * B + t0 % B) * ES);
    }
  }
  // block of the tile each copy reads (0 or 1) and whether it is V
  auto run_v = [&](int i) { return kWave * (wv + PW * i) >= KCH; };
  auto run_blk = [&](int i) {
    const int p0 = kWave * (wv + PW * i);
    if (B == 32) return 0;
    return p0 < KCH ? p0 / (16 * CPT) : ((p0 - KCH) / D) * CE / B;
  };
  TableWindow tw;
  tw.load(table, 0, a.max_blocks);
  const uint8_t* kp8 = reinterpret_cast<const uint8_t*>(k_pool) + head_off;
  const uint8_t* vp8 = reinterpret_cast<const uint8_t*>(v_pool) + head_off;
  // copies of tile k into its ring slot; block ids are read before any copy
  auto issue = [&](int k) {
    size_t pb_off[TILE / B];  // byte offset of each of the tile's blocks in a pool (ids >= 0)
    const int lbl = min(k * (TILE / B) + TILE / B - 1, nb_last);
    if (lbl >= tw.base + 2 * kWave) tw.load(table, min(k * (TILE / B), nb_last), a.max_blocks);
#pragma unroll
    for (int b = 0; b < TILE / B; ++b)
      pb_off[b] = (size_t)(uint32_t)tw.at(min(k * (TILE / B) + b, nb_last), a.num_blocks) * blk_stride;
    uint8_t* dst = &smem[k % NBUF][0];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const uint8_t* base = (run_v(i) ? vp8 : kp8) + pb_off[run_blk(i)];
      copy16_to_lds(base, D * B * ES, src_off[i], dst + 16 * kWave * (wv + PW * i));
    }
  };

  // per-lane LDS offsets of the operands: K of quarter th (slot of token
  // 8 (r / 4) + 4 th + r % 4, dims 32 j + 8c .. + 7), V of dim tile 0 (tokens
  // 8c .. 8c + 7 of dim r)
  int kofs[2];
#pragma unroll
  for (int th = 0; th < 2; ++th) {
    const int t = 8 * (r >> 2) + 4 * th + (r & 3);
    const int h = t >> 4, sl = (t & 15) ^ (4 * h);
    kofs[th] = F8 ? (((h * CPT + (c >> 1)) * 16 + sl) * 16 + 8 * (c & 1))
                  : (((h * CPT + c) * 16 + sl) * 16);
  }
  const int vofs = KB + (F8 ? (((c >> 1) * D + r) * 16 + 8 * (c & 1)) : ((c * D + r) * 16));
  auto k_operand = [&](const uint8_t* t, int th, int j) {
    if constexpr (F8) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(t + kofs[th] + j * 512);
      return __builtin_bit_cast(bf16x8, fp8x8_to_bf16(w));
    } else {
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(t + kofs[th] + j * 1024));
    }
  };
  using VOp = std::conditional_t<F8, u32x2, u32x4>;
  auto compute = [&](int k, const uint8_t* t) {
    const int T0 = k * TILE;
    f32x4 sacc[NGQ][2];
#pragma unroll
    for (int u = 0; u < NGQ; ++u) sacc[u][0] = sacc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // fp8 pools: the wave raises its priority while it issues a block of
    // MFMAs, so that the SIMD's arbiter keeps the matrix core fed from it and
    // fills the gaps with the other waves' VALU work, here heavier by the
    // widening (2% faster on 512-token chunks, level on 128; over bf16 pools
    // the same cost 5% on 128-token chunks)
    if constexpr (F8) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int x = 0; x < 2 * NJ; ++x) {  // (quarter, k-step) = (x % 2, x / 2)
      const bf16x8 kop = k_operand(t, x % 2, x / 2);
#pragma unroll
      for (int u = 0; u < NGQ; ++u)
        sacc[u][x % 2] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qb[u][x / 2], sacc[u][x % 2], 0, 0, 0);
    }
    if constexpr (F8) __builtin_amdgcn_s_setprio(0);
    bf16x8 ph[NGQ], pl[NGQ];
#pragma unroll
    for (int u = 0; u < NGQ; ++u) {
      // sv[4th + i]: raw score of token T0 + 8c + 4th + i, column r
      float sv[8];
#pragma unroll
      for (int th = 0; th < 2; ++th)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[4 * th + i] = sacc[u][th][i];
      if (T0 + TILE > first_pos + u * QT + 1) {  // a tile some column cannot see all of
        const int nv = min(max(pos[u] + 1 - (T0 + 8 * c), 0), 8);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (i >= nv) sv[i] = -INFINITY;
      }
      // a column moves its reference only when one of its scores passes
      // thr = (m + kLazyMax) / scale (raw units); compares, not a max, find
      // out (the compiler spaces them after the MFMA writes of sacc, and a max
      // of MFMA results would first be made canonical)
      bool hit = false;
#pragma unroll
      for (int i = 0; i < 8; ++i) hit |= sv[i] > thr[u];
      if (__builtin_amdgcn_ballot_w64(hit) != 0) {
        // the column's largest score (finite: token 0 is visible to every
        // column); the scale is positive, so scaling it gives the largest
        // scaled score
        float lm = sv[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) lm = fmaxf(lm, sv[i]);
        const float cm = max_over_rows(lm);
        const float mn = cm > thr[u] ? cm * score_scale : m[u];
        const float alpha = fast_exp2(m[u] - mn);  // 1 where unchanged, 0 at the first tile
        m[u] = mn;
        thr[u] = (mn + kLazyMax) * inv_scale;
        ls[u] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[u][dt] *= alpha;
      }
      u32x4 phw, plw;
      float psum = 0.f;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const float p0 = fast_exp2(__builtin_fmaf(sv[2 * wd], score_scale, -m[u]));
        const float p1 = fast_exp2(__builtin_fmaf(sv[2 * wd + 1], score_scale, -m[u]));
        psum += p0 + p1;
        // hi: truncated to bf16; lo: the exact remainder rounded to nearest even
        const uint32_t h0 = __float_as_uint(p0) & 0xffff0000u;
        const uint32_t h1 = __float_as_uint(p1) & 0xffff0000u;
        phw[wd] = (h0 >> 16) | h1;
        plw[wd] = __builtin_bit_cast(
            uint32_t, __builtin_convertvector(
                          f32x2{p0 - __uint_as_float(h0), p1 - __uint_as_float(h1)}, bf16x2));
      }
      ls[u] += psum;
      ph[u] = __builtin_bit_cast(bf16x8, phw);
      pl[u] = __builtin_bit_cast(bf16x8, plw);
    }
    // P.V, one dim tile at a time (V of tokens past the item's end was zeroed
    // in LDS; past this wave's last position the weights are 0)
    // (each V operand is read two dim tiles ahead of its products)
    if constexpr (F8) __builtin_amdgcn_s_setprio(1);
    VOp vq[NDT];
    vq[0] = *reinterpret_cast<const VOp*>(t + vofs);
    vq[1] = *reinterpret_cast<const VOp*>(t + vofs + 256);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      if (dt + 2 < NDT) vq[dt + 2] = *reinterpret_cast<const VOp*>(t + vofs + (dt + 2) * 256);
      bf16x8 va;
      if constexpr (F8)
        va = __builtin_bit_cast(bf16x8, fp8x8_to_bf16(vq[dt]));
      else
        va = __builtin_bit_cast(bf16x8, vq[dt]);
#pragma unroll
      for (int u = 0; u < NGQ; ++u) {
        acc[u][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, ph[u], acc[u][dt], 0, 0, 0);
        acc[u][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pl[u], acc[u][dt], 0, 0, 0);
      }
    }
    if constexpr (F8) __builtin_amdgcn_s_setprio(0);
  };

  // the ring: tile k is copied at iteration k - 2 (tiles 0 and 1 before the
  // loop); at iteration k each wave waits for its own copies of tile k (those
  // of tile k + 1 may still be in flight), the barrier makes every wave's copies
  // visible and ends every read of the slot tile k + 2 takes (tile k - 1's),
  // then tile k + 2's copies are issued.  Only the item's last tile can hold
  // tokens that are not in the sequence (slots past its length, a repeated
  // last block); their V is zeroed in LDS before that tile is computed, so
  // that zero weights never meet NaN (their scores are masked).
  issue(0);
  if (n > 1) issue(1);
  for (int k = 0; k < n; ++k) {
    if (k + 1 < n)
      __builtin_amdgcn_s_waitcnt(kWaitVmemRPW);
    else
      __builtin_amdgcn_s_waitcnt(kWaitVmem0);
    __syncthreads();
    if (k + 2 < n) issue(k + 2);
    if (k == n - 1) {
      // V chunk (qv, d) holds tokens CE qv .. CE qv + CE - 1 of the tile
      const int e0 = end - k * TILE;  // first token to clear
      uint8_t* vz = &smem[k % NBUF][KB];
      for (int o = 16 * (int)threadIdx.x; o < KB; o += 16 * PW * kWave) {
        const int t0 = (o / 16 / D) * CE;
        if (t0 + CE > e0) {
          u32x4 w = *reinterpret_cast<u32x4*>(vz + o);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            uint32_t mk = 0;
#pragma unroll
            for (int y = 0; y < 4 / ES; ++y)
              if (t0 + (4 / ES) * x + y < e0) mk |= (ES == 2 ? 0xffffu : 0xffu) << (8 * ES * y);
            w[x] &= mk;
          }
          *reinterpret_cast<u32x4*>(vz + o) = w;
        }
      }
      __syncthreads();
    }
    if (active && k * TILE < wend) compute(k, &smem[k % NBUF][0]);
  }

#pragma unroll
  for (int u = 0; u < NGQ; ++u) {
    float l = ls[u];
    l += shfl_xor_f(l, 16);
    l += shfl_xor_f(l, 32);
    if (col_valid[u]) {
      float* dst = a.out + ((size_t)(rbase + qi[u]) * Hq + g * G + gi) * D;
      const float scl = out_scale / l;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4*>(dst + 16 * dt + 4 * c) = acc[u][dt] * scl;
    }
  }
}

template <int D, int B, bool F8>
static bool launch_prefill_shared(int G, const PrefillArgs& a, unsigned grid, const void* q,
                                  const void* kp, const void* vp, hipStream_t st) {
  constexpr int PW = kPrefillSharedWaves, NGQ = kPrefillSharedGroups;
  using E = std::conditional_t<F8, uint8_t, uint16_t>;
  const uint16_t* qq = (const uint16_t*)q;
  const E* kk = (const E*)kp;
  const E* vv = (const E*)vp;
  const dim3 blk(PW * kWave);
  switch (G) {
    case 1: pa_prefill_shared_kernel<D, B, 1, PW, NGQ, F8><<<grid, blk, 0, st>>>(a, qq, kk, vv); return true;
    case 2: pa_prefill_shared_kernel<D, B, 2, PW, NGQ, F8><<<grid, blk, 0, st>>>(a, qq, kk, vv); return true;
    case 4: pa_prefill_shared_kernel<D, B, 4, PW, NGQ, F8><<<grid, blk, 0, st>>>(a, qq, kk, vv); return true;
    case 8: pa_prefill_shared_kernel<D, B, 8, PW, NGQ, F8><<<grid, blk, 0, st>>>(a, qq, kk, vv); return true;
    default: return false;
  }
}

template <bool F8>
static bool launch_prefill_shared(int D, int B, int G, const PrefillArgs& a, unsigned grid,
                                  const void* q, const void* kp, const void* vp, hipStream_t st) {
  if (D == 64)
    return B == 16 ? launch_prefill_shared<64, 16, F8>(G, a, grid, q, kp, vp, st)
                   : launch_prefill_shared<64, 32, F8>(G, a, grid, q, kp, vp, st);
  return B == 16 ? launch_prefill_shared<128, 16, F8>(G, a, grid, q, kp, vp, st)
                 : launch_prefill_shared<128, 32, F8>(G, a, grid, q, kp, vp, st);
}

}  // namespace pkv

using namespace pkv;

extern "C" pkv_status pkv_paged_attention_prefill(
    float* out, const void* q, const void* k_pool, const void* v_pool,
    const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
    int32_t S, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t B, int32_t max_blocks,
    int32_t num_blocks, int32_t max_query_len, float scale, pkv_dtype dtype,
    const float* k_scale, const float* v_scale, void* hip_stream) {
  if (S < 0 || T < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || B <= 0 || max_blocks <= 0 ||
      num_blocks <= 0 || max_query_len < 0 || !(scale > 0.f) || Hq % Hkv != 0)
    return PKV_EINVAL;
  if (dtype != PKV_BF16 && dtype != PKV_F32 && dtype != PKV_FP8_E4M3) return PKV_EINVAL;
  const int G = Hq / Hkv;
  if (dtype == PKV_FP8_E4M3 && (!k_scale || !v_scale)) return PKV_EINVAL;
  if (dtype == PKV_F32 || (D != 64 && D != 128) || (B != 16 && B != 32) ||
      (G != 1 && G != 2 && G != 4 && G != 8))
    return PKV_EUNSUPPORTED;
  if (S == 0 || T == 0 || max_query_len == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start ||
      !aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return PKV_EINVAL;
  const int QT = 16 / G;
  const int64_t groups = (max_query_len + QT - 1) / QT;
  const bool f8 = dtype == PKV_FP8_E4M3;
  constexpr int ngq = kPrefillSharedWaves * kPrefillSharedGroups;  // query groups per item
  const int64_t sets = (groups + ngq - 1) / ngq;
  const int64_t items = sets * S * Hkv;
  if (items > 0x7fffffffLL) return PKV_EINVAL;
  PrefillArgs a;
  a.out = out;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.k_scale = dtype == PKV_FP8_E4M3 ? k_scale : nullptr;
  a.v_scale = dtype == PKV_FP8_E4M3 ? v_scale : nullptr;
  a.S = S;
  a.Hkv = Hkv;
  a.T = T;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.scale_log2e = scale * 1.4426950408889634f;
  hipStream_t st = (hipStream_t)hip_stream;
  const unsigned grid = (unsigned)items;
  const bool ok = f8 ? launch_prefill_shared<true>(D, B, G, a, grid, q, k_pool, v_pool, st)
                     : launch_prefill_shared<false>(D, B, G, a, grid, q, k_pool, v_pool, st);
  if (!ok) return PKV_EUNSUPPORTED;
  return launch_status();
}

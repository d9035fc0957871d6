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
// fetched once per workgroup -- every thread moves a few 16-byte vectors of it
// into LDS -- and each wave reads its MFMA operands from there, so a tile feeds
// PW * NGQ * 16 query columns.  The products are the
// decode kernel's (same operand layouts, same base-2 online softmax, same bf16
// hi + lo split of P), with one softmax state and accumulator per group; each
// column masks the tokens after its own position (causal).  Items are numbered
// from the end of each sequence's chunk, so the items with the longest KV range
// are dispatched first; every item of a sequence reads the same prefix, so the
// pool loads are ordinary cached loads.
// fp8 E4M3 pools: the tiles hold the raw codes (half the bytes) and each MFMA
// operand is widened to bf16 where it is used (exact: an E4M3 value fits bf16);
// the K scale joins the score scale and the V scale the output.
#include <cmath>
#include <type_traits>

#include "../../include/pkv.h"
#include "device_common.h"
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

// The LDS tile is a byte copy of the tile's K pool regions followed by its V in
// MFMA operand order, so a K operand is read contiguously by the wave and a V
// operand is one read per lane.  Tiles are staged two at a time, one barrier
// per pair: the buffer a pair is written into was last read two stages
// earlier, before every wave passed the previous barrier, and the loads of the
// next pair are issued after the barrier and land while this pair is computed.
// The stage count and every early exit depend only on the workgroup's item, so
// all its waves reach every barrier.  Each wave computes the tiles up to its
// own last position (V past it is zeroed) and skips the rest.  Four waves of two groups each: 128 query columns per tile (measured
// on 16 x (1,536 cached + 512 new) tokens against four waves of one group and
// eight of one; a wave of two groups keeps two per SIMD at D = 128).
constexpr int kPrefillSharedWaves = 4;
constexpr int kPrefillSharedGroups = 2;

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

template <int D, int B, int G, int PW, int NGQ, bool F8>
__global__ __launch_bounds__(PW* kWave, 2) void pa_prefill_shared_kernel(
    PrefillArgs a, const uint16_t* __restrict__ q,
    const std::conditional_t<F8, uint8_t, uint16_t>* __restrict__ k_pool,
    const std::conditional_t<F8, uint8_t, uint16_t>* __restrict__ v_pool) {
  using E = std::conditional_t<F8, uint8_t, uint16_t>;
  constexpr int ES = (int)sizeof(E);
  constexpr int TILE = 32;
  constexpr int NJ = D / 32;   // q.k k-steps
  constexpr int NDT = D / 16;  // p.v output dim tiles
  constexpr int QT = 16 / G;   // query tokens per group
  constexpr int GPS = PW * NGQ;     // query groups per workgroup item
  constexpr int KB = TILE * D * ES;  // bytes of a tile's K (and of its V)
  constexpr int RB = B * D * ES;     // bytes of one (block, head) K or V region
  constexpr int OPB = 8 * ES;        // bytes of one lane's V operand (8 tokens)
  constexpr int NTH = PW * kWave;
  constexpr int VPT = 2 * KB / (16 * NTH);  // 16-byte vectors per thread per tile
  static_assert(16 % G == 0 && (B == 16 || B == 32) && D % 32 == 0, "unsupported shape");
  static_assert(VPT >= 1 && VPT * 16 * NTH == 2 * KB, "a tile splits evenly over the threads");
  static_assert(RB % (16 * kWave) == 0, "a wave's run of a tile lies in one pool region");
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  constexpr int TPS = 2;  // tiles per LDS stage (one barrier each)
  __shared__ __align__(16) uint8_t smem[2][TPS][2 * KB];

  const int wave = (int)threadIdx.x / kWave;
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

  // this wave's groups; a wave whose groups all lie past the chunk still loads
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
  float m[NGQ], ls[NGQ];
  f32x4 acc[NGQ][NDT];
#pragma unroll
  for (int u = 0; u < NGQ; ++u) {
    m[u] = -INFINITY;
    ls[u] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // fp8: the K scale joins the score scale, the V scale the output
  const float score_scale = F8 ? a.scale_log2e * a.k_scale[g] : a.scale_log2e;
  const float out_scale = F8 ? a.v_scale[g] : 1.f;
  const int n = (end + TILE - 1) / TILE;
  const int nb_last = (end + B - 1) / B - 1;  // a block past it repeats it (masked tokens)
  const int* table = a.block_tables + (size_t)s * a.max_blocks;
  const size_t head_off = (size_t)g * (D * B);
  const size_t blk_stride = (size_t)a.Hkv * (D * B);

  // thread t moves bytes 16(t + NTH i) of the tile's pool regions (K of its
  // blocks, then V of its blocks); a wave's 1 KiB run lies in one region, so its
  // block id is wave-uniform and read once per wave.  K lands in LDS in the pool
  // layout.  V lands in MFMA operand order: OPB bytes per (dim tile dt, lane (c,
  // r)) at (64 dt + lane) * OPB -- dim 16dt + r, tokens 4c .. 4c+3 of quarter 0
  // and then of quarter 1 -- so each V operand is one contiguous read; a staged V
  // vector (dim d, tokens T .. T + 16/ES - 1 of the tile) splits into 4-token
  // runs of lanes (c0 + i, d % 16), c0 = (T % 16) / 4
  u32x4 stg[TPS][VPT];
  auto sstore = [&](int h, uint8_t* t) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int byte = 16 * ((int)threadIdx.x + NTH * i);
      if (byte < KB) {
        *reinterpret_cast<u32x4*>(t + byte) = stg[h][i];
      } else {
        const int o = byte - KB;
        const int bt = o / RB;
        const int e = (o - bt * RB) / ES;  // element of the (block, head) V region
        const int d = e / B, tt = bt * B + e % B;
        const int at =
            KB + ((d / 16) * kWave + ((tt % 16) / 4) * 16 + d % 16) * OPB + (tt / 16) * (4 * ES);
        if constexpr (F8) {
#pragma unroll
          for (int w = 0; w < 4; ++w)
            *reinterpret_cast<uint32_t*>(t + at + 16 * OPB * w) = stg[h][i][w];
        } else {
          *reinterpret_cast<u32x2*>(t + at) = u32x2{stg[h][i][0], stg[h][i][1]};
          *reinterpret_cast<u32x2*>(t + at + 16 * OPB) = u32x2{stg[h][i][2], stg[h][i][3]};
        }
      }
    }
  };
  auto gload = [&](int k, int h) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int byte = 16 * ((int)threadIdx.x + NTH * i);
      const int part = byte / KB;  // 0: K, 1: V
      const int o = byte - part * KB;
      const int bt = o / RB;       // block of the tile
      const int lb = __builtin_amdgcn_readfirstlane(min(k * (TILE / B) + bt, nb_last));
      const int pb = min(max(table[lb], 0), a.num_blocks - 1);
      const E* base = (part ? v_pool : k_pool) + (size_t)pb * blk_stride + head_off;
      stg[h][i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(base) +
                                                  (o - bt * RB));
    }
  };

  // tile k from LDS: K of quarter th at k-step j (lane (c, r): dims 32j + 8c ..
  // +7 of token 16th + r, in the pool layout: bf16 chunk 4j + c, fp8 half c % 2
  // of 16-dim chunk 2j + c / 2) and the V operand of dim tile dt.  fp8 codes are
  // widened to bf16 per operand (exact)
  auto k_operand = [&](const uint8_t* t, int th, int j) {
    const int rq = (16 * th) / B * RB, tq = (16 * th) % B;
    if constexpr (F8) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(
          t + rq + ((2 * j + (c >> 1)) * B + tq + r) * 16 + 8 * (c & 1));
      return __builtin_bit_cast(bf16x8, fp8x8_to_bf16(w));
    } else {
      return __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(t + rq + ((4 * j + c) * B + tq + r) * 16));
    }
  };
  using VOp = std::conditional_t<F8, u32x2, u32x4>;
  auto compute = [&](int k, const uint8_t* t) {
    const int T0 = k * TILE;
    VOp v[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      v[dt] = *reinterpret_cast<const VOp*>(t + KB + (dt * kWave + lane) * OPB);
    // V past the wave's last position may hold anything (NaN): zero it.  bf16:
    // words 2th + wd hold tokens 16th + 4c + 2wd, +1; fp8: word th holds tokens
    // 16th + 4c .. +3
    if (T0 + TILE > wend) {
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        const int ne = min(max(wend - (T0 + 16 * th + 4 * c), 0), 4);
        if constexpr (F8) {
          const uint32_t mk = ne >= 4 ? 0xffffffffu : (1u << (8 * ne)) - 1u;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) v[dt][th] &= mk;
        } else {
#pragma unroll
          for (int wd = 0; wd < 2; ++wd) {
            const uint32_t mk =
                (2 * wd < ne ? 0x0000ffffu : 0u) | (2 * wd + 1 < ne ? 0xffff0000u : 0u);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) v[dt][2 * th + wd] &= mk;
          }
        }
      }
    }
    f32x4 sacc[NGQ][2];
#pragma unroll
    for (int u = 0; u < NGQ; ++u) sacc[u][0] = sacc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int th = 0; th < 2; ++th) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bf16x8 kop = k_operand(t, th, j);
#pragma unroll
        for (int u = 0; u < NGQ; ++u)
          sacc[u][th] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qb[u][j], sacc[u][th], 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < NGQ; ++u) {
      // sv[4th + i]: token T0 + 16th + 4c + i of column r
      float sv[8];
#pragma unroll
      for (int th = 0; th < 2; ++th)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[4 * th + i] = sacc[u][th][i] * score_scale;
      if (T0 + TILE > first_pos + u * QT + 1) {  // a tile some column cannot see all of
#pragma unroll
        for (int th = 0; th < 2; ++th) {
          const int nv = min(max(pos[u] + 1 - (T0 + 16 * th + 4 * c), 0), 4);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i >= nv) sv[4 * th + i] = -INFINITY;
        }
      }
      float mx = sv[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
      mx = max_over_rows(mx);
      // finite: token 0 is visible to every column
      const float mn = fmaxf(m[u], mx);
      const float alpha = fast_exp2(m[u] - mn);
      // no column's max moved: alpha is exactly 1 everywhere, skip the rescale
      const bool rescale = __builtin_amdgcn_ballot_w64(mn != m[u]) != 0;
      m[u] = mn;
      u32x4 phw, plw;
      float psum = 0.f;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const float p0 = fast_exp2(sv[2 * wd] - mn);
        const float p1 = fast_exp2(sv[2 * wd + 1] - mn);
        psum += p0 + p1;
        // hi: truncated to bf16; lo: the exact remainder rounded to nearest even
        const uint32_t h0 = __float_as_uint(p0) & 0xffff0000u;
        const uint32_t h1 = __float_as_uint(p1) & 0xffff0000u;
        phw[wd] = (h0 >> 16) | h1;
        plw[wd] = __builtin_bit_cast(
            uint32_t, __builtin_convertvector(
                          f32x2{p0 - __uint_as_float(h0), p1 - __uint_as_float(h1)}, bf16x2));
      }
      ls[u] = ls[u] * alpha + psum;
      const bf16x8 ph = __builtin_bit_cast(bf16x8, phw);
      const bf16x8 pl = __builtin_bit_cast(bf16x8, plw);
      if (rescale) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[u][dt] *= alpha;
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        bf16x8 va;
        if constexpr (F8)
          va = __builtin_bit_cast(bf16x8, fp8x8_to_bf16(v[dt]));
        else
          va = __builtin_bit_cast(bf16x8, v[dt]);
        acc[u][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, ph, acc[u][dt], 0, 0, 0);
        acc[u][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pl, acc[u][dt], 0, 0, 0);
      }
    }
  };

  // stages of TPS tiles; a tile past the last (odd n) loads the clamped last
  // block and is not computed
  const int ns = (n + TPS - 1) / TPS;
#pragma unroll
  for (int h = 0; h < TPS; ++h) gload(h, h);
  for (int st = 0; st < ns; ++st) {
#pragma unroll
    for (int h = 0; h < TPS; ++h) sstore(h, smem[st & 1][h]);
    __syncthreads();
    if (st + 1 < ns) {
#pragma unroll
      for (int h = 0; h < TPS; ++h) gload((st + 1) * TPS + h, h);
    }
#pragma unroll
    for (int h = 0; h < TPS; ++h) {
      const int k = st * TPS + h;
      if (active && k * TILE < wend) compute(k, smem[st & 1][h]);
    }
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

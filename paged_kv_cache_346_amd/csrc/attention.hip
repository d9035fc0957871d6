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
// Work decomposition (not on the pages): one workgroup of NW wave64s per
// (sequence, KV head, partition of P tokens).  The whole GQA group of a KV head
// lives in one workgroup, so each K/V byte is fetched from HBM once.  Waves take
// the partition's tiles round-robin, each keeping an online-softmax state
// (running max m, running sum l, unnormalised accumulator), merged in LDS at the
// end.  A sequence with one partition writes its output directly; longer ones
// write (m, l, acc) partials that pa_reduce_kernel combines (log-sum-exp merge).
// Scores are kept in base 2 (scale * log2 e folded in) so exp is one v_exp_f32.
//
// Two main kernels:
//   pa_valu_kernel  fp32 pools, and bf16 with G < 4.  Lanes (token, dim-chunk)
//                   for q.k with a 2-step cross-lane sum; lanes own output dims
//                   for p.v with the token weights read back as scalars.
//   pa_mfma_kernel  bf16 with G in {4, 8}: the GQA group x KV tile contraction is
//                   a small dense GEMM, run on v_mfma_f32_16x16x32_bf16 (group
//                   padded to 16).  S^T = K Q^T takes K straight from HBM as the
//                   A operand (16 tokens x 8 dims per lane-row); O^T = V^T P^T
//                   takes V straight from HBM as the A operand (the V layout keeps
//                   8 consecutive tokens of one dim in 16 bytes).  P is split into
//                   bf16 hi + lo parts (two MFMAs) so the weights keep ~16 bits.
// Masking: tokens at or past the partition end get score -inf by selection and
// their V elements are zeroed before the product, so NaN in unused slots never
// reaches the output.
#include <algorithm>
#include <cmath>

#include "../../include/pkv.h"
#include "device_common.h"
#include "launch_check.h"

namespace pkv {

constexpr int kDefaultPartition = 512;
constexpr int kWavesPerGroup = 4;

struct DecodeArgs {
  float* out;
  float* part_acc;   // [S, Hq, nparts, D]
  float* part_ml;    // [S, Hq, nparts, 2]
  const int* block_tables;
  const int* context_lens;
  int Hkv, max_blocks, num_blocks, nparts, P;
  float scale_log2e;
};

// Sequence geometry shared by both main kernels.  Returns false when the
// workgroup has nothing to do.
template <int D, int B, int G, int NW>
__device__ __forceinline__ bool decode_setup(const DecodeArgs& a, int& s, int& g, int& p,
                                             int& start, int& end, int& nps) {
  const int bid = blockIdx.x;
  p = bid % a.nparts;
  const int sg = bid / a.nparts;
  g = sg % a.Hkv;
  s = sg / a.Hkv;
  int L = a.context_lens[s];
  L = min(L, a.max_blocks * B);
  if (L <= 0) {
    if (p == 0) {
      float* o = a.out + ((size_t)s * a.Hkv * G + (size_t)g * G) * D;
      for (int i = threadIdx.x; i < G * D; i += NW * kWave) o[i] = 0.f;
    }
    return false;
  }
  start = p * a.P;
  if (start >= L) return false;
  end = min(L, start + a.P);
  nps = min((L + a.P - 1) / a.P, a.nparts);
  return true;
}

// Merge the per-wave (m, l, acc) states held in LDS and write the output row or
// the partition's partial.
template <int D, int G, int NW>
__device__ __forceinline__ void merge_and_store(const DecodeArgs& a, int s, int g, int p, int nps,
                                                const float (*sm_m)[16], const float (*sm_l)[16],
                                                const float (*sm_acc)[G][D]) {
  const int Hq = a.Hkv * G;
  for (int i = threadIdx.x; i < G * D; i += NW * kWave) {
    const int gi = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][gi]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = sm_m[w][gi];
      const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
      num = fmaf(f, sm_acc[w][gi][d], num);
      den = fmaf(f, sm_l[w][gi], den);
    }
    const int h = g * G + gi;
    if (nps == 1) {
      a.out[((size_t)s * Hq + h) * D + d] = num / den;
    } else {
      const size_t row = ((size_t)s * Hq + h) * a.nparts + p;
      a.part_acc[row * D + d] = num;
      if (d == 0) {
        a.part_ml[2 * row] = M;
        a.part_ml[2 * row + 1] = den;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// VALU main kernel.  E = float or uint16_t (bf16 bits).
// ---------------------------------------------------------------------------
template <typename E, int D, int B, int G, int NW>
__global__ __launch_bounds__(NW* kWave) void pa_valu_kernel(DecodeArgs a,
                                                             const E* __restrict__ q,
                                                             const E* __restrict__ k_pool,
                                                             const E* __restrict__ v_pool) {
  constexpr int X = 16 / sizeof(E);  // elements per 16-byte vector
  constexpr int NCG = kWave / B;     // lanes sharing one token in q.k
  constexpr int NCH = D / X;         // 16-byte chunks per token
  constexpr int CPL = NCH / NCG;     // chunks per lane
  constexpr int NVT = B / X;         // 16-byte token runs in a V row
  constexpr int ND = D / kWave;      // output dims per lane
  static_assert(NCH % NCG == 0 && D % kWave == 0 && B % X == 0, "unsupported shape");

  __shared__ float sm_m[NW][16], sm_l[NW][16];
  __shared__ float sm_acc[NW][G][D];

  int s, g, p, start, end, nps;
  if (!decode_setup<D, B, G, NW>(a, s, g, p, start, end, nps)) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = uniform(threadIdx.x / kWave);
  const int Hq = a.Hkv * G;
  const int t = lane % B;   // token of this lane in q.k
  const int cg = lane / B;  // its chunk group

  float qr[G][CPL][X];
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(
          q + ((size_t)s * Hq + g * G + gi) * D + (cg + NCG * j) * X);
#pragma unroll
      for (int e = 0; e < X; ++e) qr[gi][j][e] = vec_elem<E>(v, e);
    }

  float m[G], ls[G], acc[G][ND];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    m[gi] = -INFINITY;
    ls[gi] = 0.f;
#pragma unroll
    for (int k = 0; k < ND; ++k) acc[gi][k] = 0.f;
  }

  const int* table = a.block_tables + (size_t)s * a.max_blocks;
  const int lb_end = (end + B - 1) / B;
  for (int lb = start / B + w; lb < lb_end; lb += NW) {
    const int pb = min(max(table[lb], 0), a.num_blocks - 1);
    const size_t base = ((size_t)pb * a.Hkv + g) * (size_t)(D * B);
    const E* kb = k_pool + base;
    const E* vb = v_pool + base;
    u32x4 kr[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j)
      kr[j] = *reinterpret_cast<const u32x4*>(kb + ((cg + NCG * j) * B + t) * X);
    u32x4 vr[NVT][ND];
#pragma unroll
    for (int tc = 0; tc < NVT; ++tc)
#pragma unroll
      for (int k = 0; k < ND; ++k)
        vr[tc][k] = *reinterpret_cast<const u32x4*>(vb + (lane + kWave * k) * B + tc * X);

    const bool valid = lb * B + t < end;
    float pr[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      float sc = 0.f;
#pragma unroll
      for (int j = 0; j < CPL; ++j)
#pragma unroll
        for (int e = 0; e < X; ++e) sc = fmaf(qr[gi][j][e], vec_elem<E>(kr[j], e), sc);
      if (NCG >= 4) sc += shfl_xor_f(sc, 16);
      if (NCG >= 2) sc += shfl_xor_f(sc, 32);
      sc = valid ? sc * a.scale_log2e : -INFINITY;
      float mx = sc;
#pragma unroll
      for (int o = 1; o < B; o <<= 1) mx = fmaxf(mx, shfl_xor_f(mx, o));
      const float mn = fmaxf(m[gi], mx);  // finite: the block holds a valid token
      const float alpha = fast_exp2(m[gi] - mn);
      pr[gi] = fast_exp2(sc - mn);
      ls[gi] = ls[gi] * alpha + (cg == 0 ? pr[gi] : 0.f);
#pragma unroll
      for (int k = 0; k < ND; ++k) acc[gi][k] *= alpha;
      m[gi] = mn;
    }
    const int tok0 = lb * B;
#pragma unroll
    for (int tc = 0; tc < NVT; ++tc)
#pragma unroll
      for (int e = 0; e < X; ++e) {
        const int tt = tc * X + e;
        if (tok0 + tt < end) {
#pragma unroll
          for (int gi = 0; gi < G; ++gi) {
            const float pt = read_lane(pr[gi], tt);
#pragma unroll
            for (int k = 0; k < ND; ++k) acc[gi][k] = fmaf(pt, vec_elem<E>(vr[tc][k], e), acc[gi][k]);
          }
        }
      }
  }

#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const float l = wave_sum(ls[gi]);
    if (lane == 0) {
      sm_m[w][gi] = m[gi];
      sm_l[w][gi] = l;
    }
#pragma unroll
    for (int k = 0; k < ND; ++k) sm_acc[w][gi][lane + kWave * k] = acc[gi][k];
  }
  __syncthreads();
  merge_and_store<D, G, NW>(a, s, g, p, nps, sm_m, sm_l, sm_acc);
}

// ---------------------------------------------------------------------------
// MFMA main kernel (bf16, G <= 16).  Tile = 32 tokens.
// v_mfma_f32_16x16x32_bf16 operand layout (lane l, c = l / 16, r = l % 16):
//   A[16 x 32]: lane holds row r, k = 8c .. 8c+7;  B[32 x 16]: col r, k = 8c .. 8c+7;
//   C[16 x 16]: lane holds col r, rows 4c .. 4c+3.
// q.k:  C_th[m][n] = sum_d K[tok_th(m)][d] Q[n][d], tok_th(m) = 8(m/4) + 4th + m%4,
//       so lane (c, r) ends with scores of head r for tile tokens 8c + 4th + i:
//       eight consecutive tokens 8c .. 8c+7 over th = 0, 1.
// p.v:  C_dt[m][n] = sum_t V[t][16dt + m] P[n][t] with the k index = tile token
//       8c + i, which is exactly the eight scores the lane already holds, and
//       exactly the 16 bytes V stores for dim 16dt + r at tokens 8c .. 8c+7.
// ---------------------------------------------------------------------------
template <int D, int B, int G, int NW>
__global__ __launch_bounds__(NW* kWave) void pa_mfma_kernel(DecodeArgs a,
                                                             const uint16_t* __restrict__ q,
                                                             const uint16_t* __restrict__ k_pool,
                                                             const uint16_t* __restrict__ v_pool) {
  constexpr int TILE = 32;
  constexpr int NJ = D / 32;   // q.k k-steps
  constexpr int NDT = D / 16;  // p.v output dim tiles
  static_assert(G >= 1 && G <= 16 && (B == 16 || B == 32) && D % 32 == 0, "unsupported shape");

  __shared__ float sm_m[NW][16], sm_l[NW][16];
  __shared__ float sm_acc[NW][G][D];

  int s, g, p, start, end, nps;
  if (!decode_setup<D, B, G, NW>(a, s, g, p, start, end, nps)) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int w = uniform(threadIdx.x / kWave);
  const int Hq = a.Hkv * G;
  const int c = lane >> 4, r = lane & 15;

  bf16x8 qb[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < G)
      v = *reinterpret_cast<const u32x4*>(q + ((size_t)s * Hq + g * G + r) * D + 8 * (4 * j + c));
    qb[j] = __builtin_bit_cast(bf16x8, v);
  }
  // tile tokens this lane loads: K rows for th = 0, 1 and its V run 8c .. 8c+7
  int ktok[2];
#pragma unroll
  for (int th = 0; th < 2; ++th) ktok[th] = 8 * (r >> 2) + 4 * th + (r & 3);
  const int vtok = 8 * c;

  float m = -INFINITY, ls = 0.f;
  f32x4 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int* table = a.block_tables + (size_t)s * a.max_blocks;
  const int t_end = (end + TILE - 1) / TILE;
  const int nb_end = (end + B - 1) / B;
  const size_t head_off = (size_t)g * (D * B);
  const size_t blk_stride = (size_t)a.Hkv * (D * B);
  for (int ti = start / TILE + w; ti < t_end; ti += NW) {
    const int T0 = ti * TILE;
    const int lb0 = T0 / B;
    const int pb0 = min(max(table[lb0], 0), a.num_blocks - 1);
    int pb1 = pb0;
    if (B == 16 && lb0 + 1 < nb_end) pb1 = min(max(table[lb0 + 1], 0), a.num_blocks - 1);
    const uint16_t* kb0 = k_pool + pb0 * blk_stride + head_off;
    const uint16_t* kb1 = k_pool + pb1 * blk_stride + head_off;
    const uint16_t* vb0 = v_pool + pb0 * blk_stride + head_off;
    const uint16_t* vb1 = v_pool + pb1 * blk_stride + head_off;

    u32x4 ka[2][NJ];
#pragma unroll
    for (int th = 0; th < 2; ++th) {
      const uint16_t* kb = (B == 16 && ktok[th] >= 16) ? kb1 : kb0;
      const int off = ktok[th] % B;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        ka[th][j] = *reinterpret_cast<const u32x4*>(kb + ((size_t)(4 * j + c) * B + off) * 8);
    }
    u32x4 va[NDT];
    {
      const uint16_t* vb = (B == 16 && vtok >= 16) ? vb1 : vb0;
      const int off = vtok % B;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        va[dt] = *reinterpret_cast<const u32x4*>(vb + (size_t)(16 * dt + r) * B + off);
    }

    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int th = 0; th < 2; ++th)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        sacc[th] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[th][j]),
                                                           qb[j], sacc[th], 0, 0, 0);

    float sv[8];
#pragma unroll
    for (int th = 0; th < 2; ++th)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[4 * th + i] = sacc[th][i] * a.scale_log2e;
    const bool partial = T0 + TILE > end;
    if (partial) {
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (T0 + vtok + k >= end) sv[k] = -INFINITY;
      const int nv = min(max(end - (T0 + vtok), 0), 8);
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const uint32_t mk = (2 * wd < nv ? 0x0000ffffu : 0u) | (2 * wd + 1 < nv ? 0xffff0000u : 0u);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) va[dt][wd] &= mk;
      }
    }
    float mx = sv[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) mx = fmaxf(mx, sv[k]);
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float mn = fmaxf(m, mx);  // finite: tile token T0 is valid
    const float alpha = fast_exp2(m - mn);
    m = mn;
    u32x4 phw, plw;
    float psum = 0.f;
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      const float p0 = fast_exp2(sv[2 * wd] - mn);
      const float p1 = fast_exp2(sv[2 * wd + 1] - mn);
      psum += p0 + p1;
      const uint32_t h0 = __float_as_uint(p0) & 0xffff0000u;
      const uint32_t h1 = __float_as_uint(p1) & 0xffff0000u;
      const uint32_t l0 = f32_to_bf16_rne(p0 - __uint_as_float(h0));
      const uint32_t l1 = f32_to_bf16_rne(p1 - __uint_as_float(h1));
      phw[wd] = (h0 >> 16) | h1;
      plw[wd] = l0 | (l1 << 16);
    }
    ls = ls * alpha + psum;
    const bf16x8 ph = __builtin_bit_cast(bf16x8, phw);
    const bf16x8 pl = __builtin_bit_cast(bf16x8, plw);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      acc[dt] *= alpha;
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va[dt]), ph,
                                                        acc[dt], 0, 0, 0);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va[dt]), pl,
                                                        acc[dt], 0, 0, 0);
    }
  }

  ls += shfl_xor_f(ls, 16);
  ls += shfl_xor_f(ls, 32);
  if (c == 0 && r < G) {
    sm_m[w][r] = m;
    sm_l[w][r] = ls;
  }
  if (r < G) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      *reinterpret_cast<f32x4*>(&sm_acc[w][r][16 * dt + 4 * c]) = acc[dt];
  }
  __syncthreads();
  merge_and_store<D, G, NW>(a, s, g, p, nps, sm_m, sm_l, sm_acc);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of partition partials: one wave per (sequence, query head).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kWave) void pa_reduce_kernel(float* __restrict__ out,
                                                          const float* __restrict__ part_acc,
                                                          const float* __restrict__ part_ml,
                                                          const int* __restrict__ context_lens,
                                                          int Hq, int max_blocks, int B, int nparts,
                                                          int P) {
  constexpr int ND = D / kWave;
  const int lane = threadIdx.x;
  const int row = blockIdx.x;  // s * Hq + h
  const int s = row / Hq;
  const int L = min(context_lens[s], max_blocks * B);
  const int n = L <= 0 ? 0 : min((L + P - 1) / P, nparts);
  if (n <= 1) return;  // the main kernel wrote this row
  const float* ml = part_ml + (size_t)row * nparts * 2;
  const float* pa = part_acc + (size_t)row * nparts * D;
  float M = -INFINITY;
  for (int i = lane; i < n; i += kWave) M = fmaxf(M, ml[2 * i]);
  M = wave_max(M);
  float den = 0.f;
  for (int i = lane; i < n; i += kWave) den += fast_exp2(ml[2 * i] - M) * ml[2 * i + 1];
  den = wave_sum(den);
  float num[ND];
#pragma unroll
  for (int k = 0; k < ND; ++k) num[k] = 0.f;
  for (int i = 0; i < n; ++i) {
    const float f = fast_exp2(ml[2 * i] - M);
#pragma unroll
    for (int k = 0; k < ND; ++k) num[k] = fmaf(f, pa[(size_t)i * D + lane + kWave * k], num[k]);
  }
  const float inv = 1.f / den;
#pragma unroll
  for (int k = 0; k < ND; ++k) out[(size_t)row * D + lane + kWave * k] = num[k] * inv;
}

// ---------------------------------------------------------------------------
// Host dispatch.
// ---------------------------------------------------------------------------
template <typename E, int D, int B, int G>
static void launch_main(const DecodeArgs& a, unsigned grid, const void* q, const void* kp,
                        const void* vp, hipStream_t st) {
  constexpr bool kMfma = sizeof(E) == 2 && G >= 4;
  if constexpr (kMfma)
    pa_mfma_kernel<D, B, G, kWavesPerGroup><<<grid, kWavesPerGroup * kWave, 0, st>>>(
        a, (const uint16_t*)q, (const uint16_t*)kp, (const uint16_t*)vp);
  else
    pa_valu_kernel<E, D, B, G, kWavesPerGroup><<<grid, kWavesPerGroup * kWave, 0, st>>>(
        a, (const E*)q, (const E*)kp, (const E*)vp);
}

template <typename E, int D, int B>
static bool dispatch_g(int G, const DecodeArgs& a, unsigned grid, const void* q, const void* kp,
                       const void* vp, hipStream_t st) {
  switch (G) {
    case 1: launch_main<E, D, B, 1>(a, grid, q, kp, vp, st); return true;
    case 2: launch_main<E, D, B, 2>(a, grid, q, kp, vp, st); return true;
    case 4: launch_main<E, D, B, 4>(a, grid, q, kp, vp, st); return true;
    case 8: launch_main<E, D, B, 8>(a, grid, q, kp, vp, st); return true;
    default: return false;
  }
}

template <typename E, int D>
static bool dispatch_b(int B, int G, const DecodeArgs& a, unsigned grid, const void* q,
                       const void* kp, const void* vp, hipStream_t st) {
  if (B == 16) return dispatch_g<E, D, 16>(G, a, grid, q, kp, vp, st);
  if (B == 32) return dispatch_g<E, D, 32>(G, a, grid, q, kp, vp, st);
  return false;
}

template <typename E>
static bool dispatch_d(int D, int B, int G, const DecodeArgs& a, unsigned grid, const void* q,
                       const void* kp, const void* vp, hipStream_t st) {
  if (D == 64) return dispatch_b<E, 64>(B, G, a, grid, q, kp, vp, st);
  if (D == 128) return dispatch_b<E, 128>(B, G, a, grid, q, kp, vp, st);
  return false;
}

static bool shape_supported(int D, int B, int G) {
  return (D == 64 || D == 128) && (B == 16 || B == 32) && (G == 1 || G == 2 || G == 4 || G == 8);
}

static int64_t num_partitions(int64_t max_context_len, int P) {
  return max_context_len <= 0 ? 1 : (max_context_len + P - 1) / P;
}

}  // namespace pkv

using namespace pkv;

extern "C" size_t pkv_attention_workspace_bytes(int32_t S, int32_t Hq, int32_t D,
                                                int32_t max_context_len, int32_t partition_size) {
  if (S <= 0 || Hq <= 0 || D <= 0 || partition_size < 0) return 0;
  const int P = partition_size > 0 ? partition_size : kDefaultPartition;
  const int64_t np = num_partitions(max_context_len, P);
  if (np <= 1) return 0;
  return (size_t)S * Hq * np * (D + 2) * sizeof(float);
}

namespace pkv {

// Host validation and argument set-up shared by the three attention entry
// points.  On PKV_OK, *a and *groups describe the main launch (groups == 0 when
// S == 0: nothing to launch).
static pkv_status prepare_decode(DecodeArgs* a, int64_t* groups, float* out, const void* q,
                                 const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                 int32_t max_blocks, int32_t num_blocks, int32_t max_context_len,
                                 float scale, int32_t partition_size, void* workspace,
                                 size_t workspace_bytes, pkv_dtype dtype) {
  *groups = 0;
  if (S < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || max_blocks <= 0 || num_blocks <= 0 ||
      max_context_len < 0 || partition_size < 0 || !std::isfinite(scale))
    return PKV_EINVAL;
  if (dtype != PKV_F32 && dtype != PKV_BF16) return PKV_EINVAL;
  const int G = Hq / Hkv;
  if (!shape_supported(D, B, G)) return PKV_EUNSUPPORTED;
  const int P = partition_size > 0 ? partition_size : kDefaultPartition;
  if (P % 32 != 0 || P % B != 0) return PKV_EINVAL;
  if (S == 0) return PKV_OK;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !block_tables || !context_lens)
    return PKV_EINVAL;
  const int64_t mcl = std::min<int64_t>(max_context_len, (int64_t)max_blocks * B);
  const int64_t nparts = num_partitions(mcl, P);
  const int64_t g = (int64_t)S * Hkv * nparts;
  if (g > 0x7fffffffLL || (int64_t)S * Hq > 0x7fffffffLL) return PKV_EINVAL;
  *a = DecodeArgs{};
  a->out = out;
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->Hkv = Hkv;
  a->max_blocks = max_blocks;
  a->num_blocks = num_blocks;
  a->nparts = (int)nparts;
  a->P = P;
  a->scale_log2e = scale * 1.4426950408889634f;
  if (nparts > 1) {
    const size_t need = (size_t)S * Hq * nparts * (D + 2) * sizeof(float);
    if (!aligned16(workspace) || workspace_bytes < need) return PKV_EINVAL;
    a->part_acc = (float*)workspace;
    a->part_ml = a->part_acc + (size_t)S * Hq * nparts * D;
  }
  *groups = g;
  return PKV_OK;
}

static pkv_status launch_main_kernel(const DecodeArgs& a, int64_t groups, const void* q,
                                     const void* k_pool, const void* v_pool, int D, int B, int G,
                                     pkv_dtype dtype, hipStream_t st) {
  const bool ok = dtype == PKV_F32
                      ? dispatch_d<float>(D, B, G, a, (unsigned)groups, q, k_pool, v_pool, st)
                      : dispatch_d<uint16_t>(D, B, G, a, (unsigned)groups, q, k_pool, v_pool, st);
  if (!ok) return PKV_EUNSUPPORTED;
  return launch_status();
}

static pkv_status launch_reduce_kernel(const DecodeArgs& a, int S, int Hq, int D, int B,
                                       hipStream_t st) {
  if (a.nparts <= 1) return PKV_OK;
  if (D == 64)
    pa_reduce_kernel<64><<<(unsigned)(S * Hq), kWave, 0, st>>>(
        a.out, a.part_acc, a.part_ml, a.context_lens, Hq, a.max_blocks, B, a.nparts, a.P);
  else
    pa_reduce_kernel<128><<<(unsigned)(S * Hq), kWave, 0, st>>>(
        a.out, a.part_acc, a.part_ml, a.context_lens, Hq, a.max_blocks, B, a.nparts, a.P);
  return launch_status();
}

}  // namespace pkv

extern "C" pkv_status pkv_paged_attention_decode(
    float* out, const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
    const int32_t* context_lens, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
    int32_t max_blocks, int32_t num_blocks, int32_t max_context_len, float scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, pkv_dtype dtype,
    void* hip_stream) {
  DecodeArgs a;
  int64_t groups;
  pkv_status st = prepare_decode(&a, &groups, out, q, k_pool, v_pool, block_tables, context_lens,
                                 S, Hq, Hkv, D, B, max_blocks, num_blocks, max_context_len, scale,
                                 partition_size, workspace, workspace_bytes, dtype);
  if (st != PKV_OK || groups == 0) return st;
  hipStream_t hs = (hipStream_t)hip_stream;
  st = launch_main_kernel(a, groups, q, k_pool, v_pool, D, B, Hq / Hkv, dtype, hs);
  if (st != PKV_OK) return st;
  return launch_reduce_kernel(a, S, Hq, D, B, hs);
}

extern "C" pkv_status pkv_paged_attention_main(
    float* out, const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
    const int32_t* context_lens, int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
    int32_t max_blocks, int32_t num_blocks, int32_t max_context_len, float scale,
    int32_t partition_size, void* workspace, size_t workspace_bytes, pkv_dtype dtype,
    void* hip_stream) {
  DecodeArgs a;
  int64_t groups;
  pkv_status st = prepare_decode(&a, &groups, out, q, k_pool, v_pool, block_tables, context_lens,
                                 S, Hq, Hkv, D, B, max_blocks, num_blocks, max_context_len, scale,
                                 partition_size, workspace, workspace_bytes, dtype);
  if (st != PKV_OK || groups == 0) return st;
  return launch_main_kernel(a, groups, q, k_pool, v_pool, D, B, Hq / Hkv, dtype,
                            (hipStream_t)hip_stream);
}

extern "C" pkv_status pkv_paged_attention_reduce(
    float* out, const int32_t* context_lens, int32_t S, int32_t Hq, int32_t D, int32_t B,
    int32_t max_blocks, int32_t max_context_len, int32_t partition_size, const void* workspace,
    size_t workspace_bytes, void* hip_stream) {
  if (S < 0 || Hq <= 0 || max_blocks <= 0 || max_context_len < 0 || partition_size < 0)
    return PKV_EINVAL;
  if (!(D == 64 || D == 128) || !(B == 16 || B == 32)) return PKV_EUNSUPPORTED;
  const int P = partition_size > 0 ? partition_size : kDefaultPartition;
  if (P % 32 != 0 || P % B != 0) return PKV_EINVAL;
  if (S == 0) return PKV_OK;
  if (!aligned16(out) || !context_lens) return PKV_EINVAL;
  const int64_t mcl = std::min<int64_t>(max_context_len, (int64_t)max_blocks * B);
  const int64_t nparts = num_partitions(mcl, P);
  if ((int64_t)S * Hq > 0x7fffffffLL) return PKV_EINVAL;
  if (nparts <= 1) return PKV_OK;
  const size_t need = (size_t)S * Hq * nparts * (D + 2) * sizeof(float);
  if (!aligned16(workspace) || workspace_bytes < need) return PKV_EINVAL;
  DecodeArgs a{};
  a.out = out;
  a.context_lens = context_lens;
  a.max_blocks = max_blocks;
  a.nparts = (int)nparts;
  a.P = P;
  a.part_acc = (float*)workspace;
  a.part_ml = a.part_acc + (size_t)S * Hq * nparts * D;
  return launch_reduce_kernel(a, S, Hq, D, B, (hipStream_t)hip_stream);
}

// A continuous-batching serving step in one native call (pkv_loop_step).
//
// The step is the one the pages describe ([RTI] "Batch by step, not by
// request"; [ZENO] "Continuous Batching" and "Implementation Essentials"): the
// scheduler decides which requests run (admissions with prefix reuse, prefill
// chunks, one new token per running request, preemption by dropping or
// swapping), the block manager hands the kernels the block tables, the block
// copies run (swap-in, swap-out, copy-on-write), the prefill chunks' K/V are
// written and attended, then paged decode attention runs over the batch and
// writes each new token's K/V into its slot, and the finished requests give
// their blocks back.
//
// Everything between two steps happens here: the scheduler call, packing of
// the step's device metadata into a pinned buffer (two alternate, so packing
// step t + 1 overlaps the copy of step t), one asynchronous copy, and every
// launch.  The loop computes no model: the step's query and K/V rows come from
// caller-filled device banks (row (request * mul + position) mod rows), so a
// step costs the host one call and the device the kernels the step needs.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <vector>

#include "../../include/pkv.h"
#include "device_common.h"
#include "launch_check.h"

namespace pkv {

// The step's rows from the banks: task 0 query rows (Hq heads), 1 K rows,
// 2 V rows (Hkv heads); row r of the step is bank row (id * mul + pos) mod n
// of its pair (id, pos).  One 16-byte vector per thread.
__global__ void gather_rows_kernel(const int64_t* __restrict__ pairs, int64_t rows,
                                   const u32x4* __restrict__ qb, const u32x4* __restrict__ kb,
                                   const u32x4* __restrict__ vb, int64_t bank_rows, int64_t q_mul,
                                   int64_t kv_mul, int q_vecs, int kv_vecs, u32x4* __restrict__ qo,
                                   u32x4* __restrict__ ko, u32x4* __restrict__ vo) {
  const int task = (int)blockIdx.y;
  const int vecs = task == 0 ? q_vecs : kv_vecs;
  const u32x4* src = task == 0 ? qb : (task == 1 ? kb : vb);
  u32x4* dst = task == 0 ? qo : (task == 1 ? ko : vo);
  const int64_t mul = task == 0 ? q_mul : kv_mul;
  const int64_t total = rows * vecs;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / vecs, e = i - r * vecs;
    const int64_t id = pairs[2 * r], pos = pairs[2 * r + 1];
    int64_t b = (id * mul + pos) % bank_rows;
    if (b < 0) b += bank_rows;
    dst[i] = src[b * vecs + e];
  }
}

}  // namespace pkv

using namespace pkv;

struct pkv_loop {
  pkv_bm* bm = nullptr;
  pkv_sched* sched = nullptr;
  int32_t num_blocks = 0, B = 0, Hq = 0, Hkv = 0, D = 0, max_running = 0, max_blocks = 0;
  int32_t P = 0, host_blocks = 0;
  pkv_dtype dtype = PKV_BF16;
  float scale = 0.f;
  void *k_pool = nullptr, *v_pool = nullptr, *host_k = nullptr, *host_v = nullptr;
  const float *k_scale = nullptr, *v_scale = nullptr;
  hipStream_t stream = nullptr;
  // the scheduler's step arrays
  std::vector<int64_t> ids, slots, adm, pf_ids, pre, fin, swin_ids, swout_ids;
  std::vector<int32_t> cow, adm_ctx, adm_cached, pf_start, pf_len, swin, swout;
  pkv_sched_step st{};
  // pinned staging, two alternating buffers, each with the event of its copy
  int32_t* host[2] = {nullptr, nullptr};
  size_t host_words[2] = {0, 0};
  hipEvent_t done[2] = {nullptr, nullptr};
  bool pending[2] = {false, false};
  int turn = 0;
  // device buffers, grown when a step needs more
  int32_t* dev = nullptr;
  size_t dev_words = 0;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  float* out = nullptr;         // [max_running, Hq, D]
  float* out_pf = nullptr;      // [out_pf_rows, Hq, D]
  int64_t out_pf_rows = 0;
  int64_t last_batch = 0, last_pf_rows = 0;  // the last step's output rows
  uint16_t *q_rows = nullptr, *k_rows = nullptr, *v_rows = nullptr;
  int64_t rows_cap = 0;
};

namespace {

// grow a device buffer: work queued on the stream may still read the old one
pkv_status grow_device(pkv_loop* L, void** p, size_t bytes) {
  if (*p) {
    if (hipStreamSynchronize(L->stream) != hipSuccess) return PKV_EHIP;
    if (hipFree(*p) != hipSuccess) return PKV_EHIP;
    *p = nullptr;
  }
  return hipMalloc(p, bytes) == hipSuccess ? PKV_OK : PKV_EHIP;
}

void free_all(pkv_loop* L) {
  if (L->stream) (void)hipStreamSynchronize(L->stream);
  for (int i = 0; i < 2; ++i) {
    if (L->host[i]) (void)hipHostFree(L->host[i]);
    if (L->done[i]) (void)hipEventDestroy(L->done[i]);
  }
  void* dv[] = {L->dev, L->ws, L->out, L->out_pf, L->q_rows, L->k_rows, L->v_rows};
  for (void* p : dv)
    if (p) (void)hipFree(p);
}

}  // namespace

extern "C" pkv_status pkv_loop_create(const pkv_loop_config* cfg, pkv_bm* bm, pkv_sched* sched,
                                      void* k_pool, void* v_pool, void* host_k, void* host_v,
                                      const float* k_scale, const float* v_scale,
                                      void* hip_stream, pkv_loop** out) {
  if (!out) return PKV_EINVAL;
  *out = nullptr;
  if (!cfg || !bm || !sched || !k_pool || !v_pool) return PKV_EINVAL;
  int32_t nb = 0, B = 0;
  if (pkv_bm_geometry(bm, &nb, &B) != PKV_OK) return PKV_EINVAL;
  if (cfg->block_size != B || cfg->num_blocks != nb || cfg->q_heads <= 0 ||
      cfg->kv_heads <= 0 || cfg->q_heads % cfg->kv_heads != 0 || cfg->head_dim <= 0 ||
      cfg->max_running <= 0 || cfg->max_len <= 0 || cfg->partition_size < 0 ||
      cfg->host_blocks < 0)
    return PKV_EINVAL;
  if (cfg->dtype != PKV_BF16 && cfg->dtype != PKV_FP8_E4M3) return PKV_EUNSUPPORTED;
  if ((cfg->dtype == PKV_FP8_E4M3) != (k_scale && v_scale)) return PKV_EINVAL;
  if (cfg->host_blocks && (!host_k || !host_v)) return PKV_EINVAL;
  if (((cfg->q_heads * cfg->head_dim * 2) & 15) || ((cfg->kv_heads * cfg->head_dim * 2) & 15))
    return PKV_EUNSUPPORTED;
  pkv_loop* L = new pkv_loop;
  L->bm = bm;
  L->sched = sched;
  L->num_blocks = nb;
  L->B = B;
  L->Hq = cfg->q_heads;
  L->Hkv = cfg->kv_heads;
  L->D = cfg->head_dim;
  L->max_running = cfg->max_running;
  L->max_blocks = std::max(1, (cfg->max_len + B - 1) / B);
  L->P = cfg->partition_size;
  L->host_blocks = cfg->host_blocks;
  L->dtype = cfg->dtype;
  L->scale = 1.f / std::sqrt((float)cfg->head_dim);
  L->k_pool = k_pool;
  L->v_pool = v_pool;
  L->host_k = host_k;
  L->host_v = host_v;
  L->k_scale = k_scale;
  L->v_scale = v_scale;
  L->stream = (hipStream_t)hip_stream;
  const int32_t n = cfg->max_running;
  const int32_t npairs = nb;
  L->ids.resize(n);
  L->slots.resize(n);
  L->adm.resize(n);
  L->pf_ids.resize(n);
  L->pre.resize(n);
  L->fin.resize(n);
  L->swin_ids.resize(n);
  L->swout_ids.resize(n);
  L->cow.resize(2 * (size_t)n);
  L->adm_ctx.resize(n);
  L->adm_cached.resize(n);
  L->pf_start.resize(n);
  L->pf_len.resize(n);
  L->swin.resize(2 * (size_t)npairs);
  L->swout.resize(2 * (size_t)npairs);
  pkv_sched_step& s = L->st;
  s.capacity = n;
  s.batch_ids = L->ids.data();
  s.slots = L->slots.data();
  s.cow_pairs = L->cow.data();
  s.admitted_ids = L->adm.data();
  s.admitted_ctx = L->adm_ctx.data();
  s.admitted_cached = L->adm_cached.data();
  s.prefill_ids = L->pf_ids.data();
  s.prefill_start = L->pf_start.data();
  s.prefill_len = L->pf_len.data();
  s.preempted_ids = L->pre.data();
  s.finished_ids = L->fin.data();
  s.pair_capacity = npairs;
  s.swap_in_pairs = L->swin.data();
  s.swap_out_pairs = L->swout.data();
  s.swapped_in_ids = L->swin_ids.data();
  s.swapped_out_ids = L->swout_ids.data();
  pkv_status st = PKV_OK;
  for (int i = 0; i < 2 && st == PKV_OK; ++i)
    if (hipEventCreateWithFlags(&L->done[i], hipEventDisableTiming) != hipSuccess) st = PKV_EHIP;
  // decode workspace for the largest batch and context, zeroed once (its
  // merge counters return to zero after every launch)
  if (st == PKV_OK) {
    L->ws_bytes = pkv_attention_workspace_bytes(n, L->Hq, L->D, cfg->max_len, L->P);
    if (L->ws_bytes) {
      st = grow_device(L, &L->ws, L->ws_bytes);
      if (st == PKV_OK && hipMemsetAsync(L->ws, 0, L->ws_bytes, L->stream) != hipSuccess)
        st = PKV_EHIP;
    }
  }
  if (st == PKV_OK)
    st = grow_device(L, (void**)&L->out, sizeof(float) * (size_t)n * L->Hq * L->D);
  if (st != PKV_OK) {
    free_all(L);
    delete L;
    return st;
  }
  *out = L;
  return PKV_OK;
}

extern "C" void pkv_loop_destroy(pkv_loop* loop) {
  if (!loop) return;
  free_all(loop);
  delete loop;
}

extern "C" pkv_status pkv_loop_step(pkv_loop* L, const pkv_loop_source* src,
                                    pkv_loop_step_info* info) {
  using clk = std::chrono::steady_clock;
  const auto t0 = clk::now();
  double wait_us = 0.0;
  if (!L || !src || !info || !src->q_bank || !src->k_bank || !src->v_bank || src->bank_rows <= 0)
    return PKV_EINVAL;
  if (!aligned16(src->q_bank) || !aligned16(src->k_bank) || !aligned16(src->v_bank))
    return PKV_EINVAL;
  pkv_sched_step& st = L->st;
  pkv_status s = pkv_sched_begin_step(L->sched, &st);
  if (s != PKV_OK) return s;
  // From here on the scheduler is inside the step: any failure still ends it,
  // so that the loop stays usable, and reports the first error.
  pkv_status err = PKV_OK;
  auto fail = [&](pkv_status e) {
    if (err == PKV_OK) err = e;
  };

  // pack into the pinned buffer whose previous copy has finished
  const int i = L->turn;
  L->turn ^= 1;
  if (L->pending[i]) {
    const auto w0 = clk::now();
    if (hipEventSynchronize(L->done[i]) != hipSuccess) fail(PKV_EHIP);
    wait_us += std::chrono::duration<double, std::micro>(clk::now() - w0).count();
    L->pending[i] = false;
  }
  pkv_step_pack lay{};
  if (err == PKV_OK) {
    s = pkv_pack_step(L->bm, &st, L->max_blocks, L->Hkv, L->P, L->host[i], L->host_words[i], &lay);
    if (s == PKV_EINVAL && (size_t)lay.total_words > L->host_words[i]) {
      const size_t words = std::max<size_t>((size_t)lay.total_words * 2, 1u << 16);
      if (L->host[i]) (void)hipHostFree(L->host[i]);
      L->host[i] = nullptr;
      L->host_words[i] = 0;
      if (hipHostMalloc((void**)&L->host[i], words * sizeof(int32_t), hipHostMallocDefault) !=
          hipSuccess) {
        fail(PKV_EHIP);
      } else {
        L->host_words[i] = words;
        s = pkv_pack_step(L->bm, &st, L->max_blocks, L->Hkv, L->P, L->host[i], words, &lay);
      }
    }
    if (err == PKV_OK && s != PKV_OK) fail(s);
  }
  const int32_t* h = L->host[i];
  const int64_t n_pf = lay.n_prefill_rows, nb = st.n_batch, nc = st.n_prefill;
  const int64_t rows = n_pf + nb;
  // device buffers for this step
  if (err == PKV_OK && (size_t)lay.total_words > L->dev_words) {
    const size_t words = std::max<size_t>((size_t)lay.total_words * 2, 1u << 16);
    if (grow_device(L, (void**)&L->dev, words * sizeof(int32_t)) == PKV_OK)
      L->dev_words = words;
    else
      fail(PKV_EHIP);
  }
  if (err == PKV_OK && rows > L->rows_cap) {
    const int64_t cap = std::max<int64_t>(rows * 2, 1024);
    const bool ok = grow_device(L, (void**)&L->q_rows, 2 * (size_t)cap * L->Hq * L->D) == PKV_OK &&
                    grow_device(L, (void**)&L->k_rows, 2 * (size_t)cap * L->Hkv * L->D) == PKV_OK &&
                    grow_device(L, (void**)&L->v_rows, 2 * (size_t)cap * L->Hkv * L->D) == PKV_OK;
    if (ok)
      L->rows_cap = cap;
    else
      fail(PKV_EHIP);
  }
  if (err == PKV_OK && n_pf > L->out_pf_rows) {
    const int64_t cap = std::max<int64_t>(n_pf * 2, 1024);
    if (grow_device(L, (void**)&L->out_pf, sizeof(float) * (size_t)cap * L->Hq * L->D) == PKV_OK)
      L->out_pf_rows = cap;
    else
      fail(PKV_EHIP);
  }
  if (err == PKV_OK && lay.total_words) {
    if (hipMemcpyAsync(L->dev, h, sizeof(int32_t) * (size_t)lay.total_words,
                       hipMemcpyHostToDevice, L->stream) != hipSuccess ||
        hipEventRecord(L->done[i], L->stream) != hipSuccess)
      fail(PKV_EHIP);
    else
      L->pending[i] = true;
  }
  const int32_t* d = L->dev;
  void* stream = (void*)L->stream;
  // block copies in the scheduler's order: swap-ins, swap-outs, copy-on-write
  if (err == PKV_OK && st.n_swap_in)
    fail(pkv_swap_blocks(L->k_pool, L->v_pool, L->num_blocks, L->host_k, L->host_v,
                         L->host_blocks, d + lay.swap_in_off, st.n_swap_in, L->Hkv, L->D, L->B,
                         L->dtype, stream));
  if (err == PKV_OK && st.n_swap_out)
    fail(pkv_swap_blocks(L->host_k, L->host_v, L->host_blocks, L->k_pool, L->v_pool,
                         L->num_blocks, d + lay.swap_out_off, st.n_swap_out, L->Hkv, L->D, L->B,
                         L->dtype, stream));
  if (err == PKV_OK && st.n_cow)
    fail(pkv_copy_blocks(L->k_pool, L->v_pool, d + lay.cow_off, st.n_cow, L->Hkv, L->D, L->B,
                         L->num_blocks, L->dtype, stream));
  // the step's rows: the prefill chunks' tokens in order, then one token per
  // decoding request
  if (err == PKV_OK && rows) {
    const int q_vecs = L->Hq * L->D * 2 / 16, kv_vecs = L->Hkv * L->D * 2 / 16;
    const int64_t work = rows * q_vecs;
    const unsigned gx = (unsigned)std::min<int64_t>((work + 255) / 256, 4096);
    gather_rows_kernel<<<dim3(gx, 3), 256, 0, L->stream>>>(
        reinterpret_cast<const int64_t*>(d + lay.pairs_off), rows,
        (const u32x4*)src->q_bank, (const u32x4*)src->k_bank, (const u32x4*)src->v_bank,
        src->bank_rows, src->q_mul, src->kv_mul, q_vecs, kv_vecs, (u32x4*)L->q_rows,
        (u32x4*)L->k_rows, (u32x4*)L->v_rows);
    fail(launch_status());
  }
  if (err == PKV_OK && n_pf) {
    fail(pkv_reshape_and_cache(L->k_rows, L->v_rows, L->k_pool, L->v_pool,
                               reinterpret_cast<const int64_t*>(d + lay.slots_off), (int32_t)n_pf,
                               L->Hkv, L->D, L->B, L->num_blocks, L->dtype, L->k_scale,
                               L->v_scale, stream));
    if (err == PKV_OK)
      fail(pkv_paged_attention_prefill(
          L->out_pf, L->q_rows, L->k_pool, L->v_pool, d + lay.pf_tables_off, d + lay.pf_lens_off,
          d + lay.pf_start_off, (int32_t)nc, (int32_t)n_pf, L->Hq, L->Hkv, L->D, L->B,
          std::max(lay.pf_width, 1), L->num_blocks, lay.pf_max_rows, L->scale, L->dtype,
          L->k_scale, L->v_scale, stream));
  }
  if (err == PKV_OK && nb) {
    const size_t qoff = (size_t)n_pf * L->Hq * L->D, kvoff = (size_t)n_pf * L->Hkv * L->D;
    fail(pkv_paged_attention_decode(
        L->out, L->q_rows + qoff, L->k_pool, L->v_pool, L->k_rows + kvoff, L->v_rows + kvoff,
        d + lay.tables_off, d + lay.lens_off, (int32_t)nb, L->Hq, L->Hkv, L->D, L->B,
        std::max(lay.width, 1), L->num_blocks, lay.max_context, L->scale, L->P, d + lay.plan_off,
        lay.n_items, lay.n_merge, L->ws, L->ws_bytes, L->dtype, 0u, L->k_scale, L->v_scale,
        stream));
  }
  // the step's account, taken before the finished requests leave
  pkv_loop_step_info r{};
  r.n_batch = st.n_batch;
  r.n_prefill = st.n_prefill;
  r.n_prefill_rows = (int32_t)n_pf;
  r.n_admitted = st.n_admitted;
  r.n_preempted = st.n_preempted;
  r.n_finished = st.n_finished;
  r.n_swapped_out = st.n_swapped_out;
  r.n_swapped_in = st.n_swapped_in;
  r.n_swap_out_blocks = st.n_swap_out;
  r.n_swap_in_blocks = st.n_swap_in;
  r.n_cow = st.n_cow;
  for (int32_t a = 0; a < st.n_admitted; ++a) r.cached_tokens += st.admitted_cached[a];
  r.max_context = lay.max_context;
  r.lens_host = h ? h + lay.lens_off : nullptr;
  r.decode_out = L->out;
  r.prefill_out = L->out_pf;
  int32_t nw = 0, nr = 0, ns = 0;
  const pkv_status ss = pkv_sched_stats(L->sched, &r.tokens_held, &r.slots_committed, &nw, &nr, &ns);
  if (ss != PKV_OK) fail(ss);
  r.n_waiting = nw;
  r.n_running = nr;
  r.n_swapped = ns;
  L->last_batch = nb;
  L->last_pf_rows = n_pf;
  const pkv_status se = pkv_sched_end_step(L->sched);
  if (se != PKV_OK) fail(se);
  r.wait_us = wait_us;
  r.host_us = std::chrono::duration<double, std::micro>(clk::now() - t0).count();
  *info = r;
  return err;
}

extern "C" pkv_status pkv_loop_copy_outputs(const pkv_loop* L, float* decode_dst,
                                            float* prefill_dst) {
  if (!L) return PKV_EINVAL;
  const size_t row = sizeof(float) * (size_t)L->Hq * L->D;
  if (decode_dst && L->last_batch &&
      hipMemcpyAsync(decode_dst, L->out, row * (size_t)L->last_batch, hipMemcpyDeviceToDevice,
                     L->stream) != hipSuccess)
    return PKV_EHIP;
  if (prefill_dst && L->last_pf_rows &&
      hipMemcpyAsync(prefill_dst, L->out_pf, row * (size_t)L->last_pf_rows,
                     hipMemcpyDeviceToDevice, L->stream) != hipSuccess)
    return PKV_EHIP;
  return PKV_OK;
}

// Device metadata of one continuous-batching step, packed on the host
// (pkv_pack_step).
//
// After the scheduler has decided a step (which requests decode, which prefill
// chunks run, which blocks move), the kernels need: the slots of every chunk
// token, the chunk requests' block tables, the decode batch's block tables,
// lengths and work plan, the (request, position) list of the K/V rows the step
// writes, and the block copy pairs ([ZENO] "Implementation Essentials": the
// block manager hands the kernels block tables; [RTI] "Batch by step, not by
// request").  They are laid out here in one int32 buffer, each array on a
// 16-byte boundary, so that one asynchronous copy takes them to the device.
// Pure host work through the block manager's public calls.
#include <algorithm>
#include <cstring>
#include <vector>

#include "../../include/pkv.h"

namespace {

int64_t pad4(int64_t words) { return (words + 3) / 4 * 4; }

void put64(int32_t* buf, int64_t word_off, int64_t v) {
  std::memcpy(buf + word_off, &v, sizeof v);
}

}  // namespace

extern "C" pkv_status pkv_pack_step(const pkv_bm* bm, const pkv_sched_step* st,
                                    int32_t max_blocks, int32_t Hkv, int32_t partition_size,
                                    int32_t* buf, size_t buf_words, pkv_step_pack* out) {
  if (!bm || !st || !out || max_blocks <= 0 || Hkv <= 0 || partition_size < 0)
    return PKV_EINVAL;
  int32_t num_blocks = 0, B = 0;
  pkv_status s = pkv_bm_geometry(bm, &num_blocks, &B);
  if (s != PKV_OK) return s;
  const int32_t nc = st->n_prefill, nb = st->n_batch;
  if (nc < 0 || nb < 0 || st->n_swap_in < 0 || st->n_swap_out < 0 || st->n_cow < 0)
    return PKV_EINVAL;

  // prefill chunks: rows, the longest chunk, the farthest end position
  int64_t rows = 0;
  int32_t pf_max_rows = 0, pf_end = 0;
  for (int32_t i = 0; i < nc; ++i) {
    const int32_t a = st->prefill_start[i], n = st->prefill_len[i];
    if (a < 0 || n < 0) return PKV_EINVAL;
    rows += n;
    pf_max_rows = std::max(pf_max_rows, n);
    pf_end = std::max(pf_end, a + n);
  }
  const int32_t pf_width = nc ? std::max(1, (pf_end + B - 1) / B) : 0;
  if (pf_width > max_blocks) return PKV_EINVAL;

  // decode batch: full-width rows first, trimmed to the longest context below
  std::vector<int32_t> tables((size_t)nb * max_blocks), lens(nb);
  if (nb) {
    s = pkv_bm_fill_batch(bm, st->batch_ids, nb, max_blocks, tables.data(), lens.data());
    if (s != PKV_OK) return s;
  }
  int32_t mcl = 0;
  for (int32_t v : lens) mcl = std::max(mcl, v);
  const int32_t width = nb ? std::max(1, (mcl + B - 1) / B) : 0;
  const size_t plan_cap =
      nb ? pkv_attention_plan_words(nb, Hkv, B, width, mcl, partition_size) : 0;
  if (nb && plan_cap == 0) return PKV_EINVAL;

  // layout
  pkv_step_pack L{};
  int64_t off = 0;
  auto take = [&](int64_t words) {
    const int64_t at = off;
    off += pad4(words);
    return (int32_t)at;
  };
  L.n_prefill_rows = (int32_t)rows;
  L.slots_off = take(2 * rows);
  L.pf_tables_off = take((int64_t)nc * pf_width);
  L.pf_width = pf_width;
  L.pf_lens_off = take(nc);
  L.pf_start_off = take(nc + 1);
  L.pf_max_rows = pf_max_rows;
  L.tables_off = take((int64_t)nb * width);
  L.width = width;
  L.lens_off = take(nb);
  L.max_context = mcl;
  L.plan_off = take((int64_t)plan_cap);
  L.pairs_off = take(4 * (rows + nb));
  L.swap_in_off = take(2 * (int64_t)st->n_swap_in);
  L.swap_out_off = take(2 * (int64_t)st->n_swap_out);
  L.cow_off = take(2 * (int64_t)st->n_cow);
  if (off > 0x7fffffffLL) return PKV_EINVAL;
  L.total_words = (int32_t)off;
  *out = L;
  if (!buf || (size_t)off > buf_words) return PKV_EINVAL;

  // prefill chunks: slots, tables, lengths, row offsets, (id, position) rows
  int64_t r = 0;
  if (nc) {
    std::vector<int32_t> pft((size_t)nc * max_blocks), pfl(nc);
    s = pkv_bm_fill_batch(bm, st->prefill_ids, nc, max_blocks, pft.data(), pfl.data());
    if (s != PKV_OK) return s;
    std::vector<int64_t> slots;
    buf[L.pf_start_off] = 0;
    for (int32_t i = 0; i < nc; ++i) {
      const int64_t id = st->prefill_ids[i];
      const int32_t a = st->prefill_start[i], n = st->prefill_len[i];
      slots.resize(std::max(n, 1));
      s = pkv_bm_slots(bm, id, a, n, slots.data());
      if (s != PKV_OK) return s;
      std::memcpy(buf + L.slots_off + 2 * r, slots.data(), sizeof(int64_t) * (size_t)n);
      std::memcpy(buf + L.pf_tables_off + (size_t)i * pf_width, pft.data() + (size_t)i * max_blocks,
                  sizeof(int32_t) * (size_t)pf_width);
      buf[L.pf_lens_off + i] = a + n;
      for (int32_t t = 0; t < n; ++t, ++r) {
        put64(buf, L.pairs_off + 4 * r, id);
        put64(buf, L.pairs_off + 4 * r + 2, a + t);
      }
      buf[L.pf_start_off + i + 1] = (int32_t)r;
    }
  }
  // decode batch: trimmed tables, lengths, plan, one (id, position) row each
  if (nb) {
    for (int32_t i = 0; i < nb; ++i) {
      std::memcpy(buf + L.tables_off + (size_t)i * width, tables.data() + (size_t)i * max_blocks,
                  sizeof(int32_t) * (size_t)width);
      buf[L.lens_off + i] = lens[i];
      put64(buf, L.pairs_off + 4 * (r + i), st->batch_ids[i]);
      put64(buf, L.pairs_off + 4 * (r + i) + 2, (int64_t)lens[i] - 1);
    }
    int32_t n_items = 0, n_merge = 0;
    s = pkv_attention_plan(buf + L.lens_off, nb, Hkv, B, width, mcl, partition_size,
                           buf + L.plan_off, plan_cap, &n_items, &n_merge);
    if (s != PKV_OK) return s;
    out->n_items = n_items;
    out->n_merge = n_merge;
  }
  // block copies, in the scheduler's order of use
  auto pairs = [&](int32_t at, const int32_t* src, int32_t n) {
    if (n > 0) std::memcpy(buf + at, src, sizeof(int32_t) * 2 * (size_t)n);
  };
  pairs(L.swap_in_off, st->swap_in_pairs, st->n_swap_in);
  pairs(L.swap_out_off, st->swap_out_pairs, st->n_swap_out);
  pairs(L.cow_off, st->cow_pairs, st->n_cow);
  return PKV_OK;
}

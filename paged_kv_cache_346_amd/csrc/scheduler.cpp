// Iteration-level (continuous) batching scheduler behind the pkv_sched_* entry
// points: a host-side loop driver over one block manager.
//
// PagedAttention and Continuous Batching, "Batch by step, not by request": the
// batch is rebuilt after every decode step -- finished sequences leave, waiting
// ones join -- and with paging a newcomer needs only free blocks.
// PagedAttention: The vLLM Paper, "Continuous Batching" (A finishes, A dequeues,
// D enqueues, giving {B, C, D}) and "Implementation Essentials" (preemption
// swaps a request's blocks to CPU memory, or drops them for later
// recomputation, under memory pressure).
//
// Policy (readings of the pages, stated in include/pkv.h): first-come
// first-served admission with no skipping ahead; at most max_running requests;
// one token per running request per step, appended in admission order; the
// most recently admitted request is preempted when an append finds no free
// block -- swapped to the host pool under the swap policy when it holds KV and
// the host has room, else dropped.  The reserve policy simulates the
// max-length reservation of the systems before paging over the same pool.
// Prefix caching and chunked prefill ("Impact and Follow-Ups"): requests may
// carry prompt token ids (admission then reuses cached prefix blocks), and a
// per-step prefill budget splits long prompts into chunks, continuing
// admitted requests first.  Integer bookkeeping only.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/pkv.h"

struct pkv_sched {
  struct Req {
    int64_t id;
    int32_t prompt, max_new, generated, reserved;
    std::vector<int32_t> tokens;  // prompt token ids, when known
    bool has_tokens;
    int32_t target, prefilled;    // context to prefill since admission, and done so far
    int32_t ctx() const { return prompt + generated; }
  };
  pkv_bm* bm = nullptr;
  int32_t N = 0, B = 0, max_running = 0;
  int64_t max_prefill = 0;  // tokens per step, 0 = no limit
  bool reserve = false, swap = false;
  int64_t reserved_total = 0;
  bool in_step = false;
  std::unordered_map<int64_t, Req> reqs;  // every submitted, unfinished request
  std::deque<Req*> waiting;
  std::deque<Req*> swapped;  // preempted to the host, front resumes first
  std::vector<Req*> running;
  std::vector<Req*> finishing;

  int32_t blocks(int64_t tokens) const { return (int32_t)((tokens + B - 1) / B); }
};

extern "C" {

pkv_status pkv_sched_create(pkv_bm* bm, int32_t max_running, int32_t policy,
                            int32_t max_prefill_tokens, pkv_sched** out) {
  if (!out) return PKV_EINVAL;
  *out = nullptr;
  if (!bm || max_running <= 0 || max_prefill_tokens < 0) return PKV_EINVAL;
  if (policy & ~(PKV_SCHED_RESERVE_MAX | PKV_SCHED_SWAP)) return PKV_EINVAL;
  if ((policy & PKV_SCHED_RESERVE_MAX) && (policy & PKV_SCHED_SWAP)) return PKV_EINVAL;
  int32_t N = 0, B = 0;
  if (pkv_bm_geometry(bm, &N, &B) != PKV_OK) return PKV_EINVAL;
  pkv_sched* s = new (std::nothrow) pkv_sched();
  if (!s) return PKV_EINVAL;
  s->bm = bm;
  s->N = N;
  s->B = B;
  s->max_running = max_running;
  s->reserve = (policy & PKV_SCHED_RESERVE_MAX) != 0;
  s->swap = (policy & PKV_SCHED_SWAP) != 0;
  s->max_prefill = max_prefill_tokens;
  *out = s;
  return PKV_OK;
}

void pkv_sched_destroy(pkv_sched* s) { delete s; }

pkv_status pkv_sched_add_request(pkv_sched* s, int64_t req_id, int32_t prompt_len,
                                 int32_t max_new_tokens, const int32_t* tokens) {
  if (!s || prompt_len < 0 || max_new_tokens < 1) return PKV_EINVAL;
  if (s->reqs.count(req_id)) return PKV_EEXIST;
  if (s->blocks((int64_t)prompt_len + max_new_tokens) > s->N) return PKV_EINVAL;
  pkv_sched::Req r{req_id, prompt_len, max_new_tokens, 0, 0, {}, tokens != nullptr, 0, 0};
  if (tokens) r.tokens.assign(tokens, tokens + prompt_len);
  auto it = s->reqs.emplace(req_id, std::move(r));
  s->waiting.push_back(&it.first->second);
  return PKV_OK;
}

pkv_status pkv_sched_begin_step(pkv_sched* s, pkv_sched_step* o) {
  if (!s || !o || o->capacity < s->max_running) return PKV_EINVAL;
  if (!o->batch_ids || !o->slots || !o->cow_pairs || !o->admitted_ids || !o->admitted_ctx ||
      !o->admitted_cached || !o->prefill_ids || !o->prefill_start || !o->prefill_len ||
      !o->preempted_ids || !o->finished_ids)
    return PKV_EINVAL;
  if (s->swap && (o->pair_capacity < s->N || !o->swap_in_pairs || !o->swap_out_pairs ||
                  !o->swapped_in_ids || !o->swapped_out_ids))
    return PKV_EINVAL;
  if (s->in_step) return PKV_EINVAL;  // end_step() of the last step is due
  o->n_batch = o->n_cow = o->n_admitted = o->n_preempted = o->n_finished = 0;
  o->n_swap_in = o->n_swap_out = o->n_swapped_in = o->n_swapped_out = o->n_prefill = 0;
  s->in_step = true;

  // swapped requests come back first, in queue order, while the device has room
  while (!s->swapped.empty() && (int32_t)s->running.size() < s->max_running) {
    pkv_sched::Req* r = s->swapped.front();
    int32_t n = 0;
    // at most N device blocks are free, so the pairs fit pair_capacity
    const pkv_status st = pkv_bm_swap_in(s->bm, r->id, o->swap_in_pairs + 2 * o->n_swap_in,
                                         o->pair_capacity - o->n_swap_in, &n);
    if (st == PKV_ENOBLOCKS) break;
    if (st != PKV_OK) return st;
    o->n_swap_in += n;
    s->swapped.pop_front();
    s->running.push_back(r);
    o->swapped_in_ids[o->n_swapped_in++] = r->id;
  }

  // prefill chunks: admitted requests first, in admission order, within the budget
  int64_t budget = s->max_prefill > 0 ? s->max_prefill : INT64_MAX;
  struct Chunk {
    pkv_sched::Req* r;
    int32_t start, n;
  };
  std::vector<Chunk> chunks;
  auto give_chunk = [&](pkv_sched::Req* r) {
    const int32_t n = (int32_t)std::min<int64_t>(r->target - r->prefilled, budget);
    if (n > 0) {
      chunks.push_back({r, r->prefilled, n});
      r->prefilled += n;
      budget -= n;
      if (r->has_tokens)  // the chunk's full prompt blocks join the prefix cache
        pkv_bm_register_prefix(s->bm, r->id, r->tokens.data(), (int32_t)r->tokens.size(),
                               r->prefilled);
    }
  };
  for (pkv_sched::Req* r : s->running)
    if (r->prefilled < r->target && budget > 0) give_chunk(r);

  // admissions, first come first served, none while a request is swapped out
  struct Adm {
    pkv_sched::Req* r;
    int32_t ctx, cached;
  };
  std::vector<Adm> admitted;
  while (s->swapped.empty() && !s->waiting.empty() &&
         (int32_t)s->running.size() < s->max_running && budget > 0) {
    pkv_sched::Req* r = s->waiting.front();
    const int32_t need_max = s->blocks((int64_t)r->prompt + r->max_new);
    if (s->reserve && s->reserved_total + need_max > s->N) break;
    int32_t cached = 0;
    const pkv_status st =
        r->has_tokens ? pkv_bm_add_seq_prefix(s->bm, r->id, r->tokens.data(),
                                              (int32_t)r->tokens.size(), r->ctx(), &cached)
                      : pkv_bm_add_seq(s->bm, r->id, r->ctx());
    if (st == PKV_ENOBLOCKS) break;
    if (st != PKV_OK) return st;
    if (s->reserve) {
      r->reserved = need_max;
      s->reserved_total += need_max;
    }
    s->waiting.pop_front();
    s->running.push_back(r);
    r->target = r->ctx();
    r->prefilled = cached;
    admitted.push_back({r, r->ctx(), cached});
    give_chunk(r);
  }

  // one slot per request whose prefill is complete; preempt the youngest when
  // the pool is dry
  std::vector<pkv_sched::Req*> decoding;
  size_t i = 0;
  while (i < s->running.size()) {
    pkv_sched::Req* r = s->running[i];
    if (r->prefilled < r->target) {  // still prefilling: no token this step
      ++i;
      continue;
    }
    int64_t slot;
    int32_t src, dst;
    const pkv_status st = pkv_bm_append_slot(s->bm, r->id, &slot, &src, &dst);
    if (st == PKV_ENOBLOCKS) {
      pkv_sched::Req* victim = s->running.back();
      s->running.pop_back();
      size_t fresh = admitted.size();  // admitted this step: no KV written yet
      for (size_t k = 0; k < admitted.size(); ++k)
        if (admitted[k].r == victim) fresh = k;
      for (size_t k = 0; k < chunks.size(); ++k)  // its chunk of this step is not written
        if (chunks[k].r == victim) {
          victim->prefilled -= chunks[k].n;
          chunks.erase(chunks.begin() + k);
          pkv_bm_unregister_prefix(s->bm, victim->id, victim->prefilled);
          break;
        }
      if (s->swap && fresh == admitted.size()) {
        int32_t len = 0, nb = 0, host_free = 0;
        pkv_bm_seq_info(s->bm, victim->id, &len, &nb);
        pkv_bm_num_free_host(s->bm, &host_free);
        // the step's swap-outs never hold more blocks than the device has
        if (nb <= host_free && o->n_swap_out + nb <= o->pair_capacity) {
          int32_t n = 0;
          const pkv_status ss =
              pkv_bm_swap_out(s->bm, victim->id, o->swap_out_pairs + 2 * o->n_swap_out,
                              o->pair_capacity - o->n_swap_out, &n);
          if (ss != PKV_OK) return ss;
          o->n_swap_out += n;
          o->swapped_out_ids[o->n_swapped_out++] = victim->id;
          s->swapped.push_front(victim);
          continue;
        }
      }
      const pkv_status fs = pkv_bm_free_seq(s->bm, victim->id);
      if (fs != PKV_OK) return fs;
      if (fresh < admitted.size()) admitted.erase(admitted.begin() + fresh);
      o->preempted_ids[o->n_preempted++] = victim->id;
      s->waiting.push_front(victim);
      continue;
    }
    if (st != PKV_OK) return st;
    o->slots[decoding.size()] = slot;
    if (src >= 0) {
      o->cow_pairs[2 * o->n_cow] = src;
      o->cow_pairs[2 * o->n_cow + 1] = dst;
      ++o->n_cow;
    }
    decoding.push_back(r);
    ++i;
  }

  for (size_t k = 0; k < decoding.size(); ++k) {
    pkv_sched::Req* r = decoding[k];
    o->batch_ids[k] = r->id;
    r->generated += 1;
    if (r->generated == r->max_new) {
      o->finished_ids[o->n_finished++] = r->id;
      s->finishing.push_back(r);
    }
  }
  o->n_batch = (int32_t)decoding.size();
  for (const Adm& a : admitted) {
    o->admitted_ids[o->n_admitted] = a.r->id;
    o->admitted_ctx[o->n_admitted] = a.ctx;
    o->admitted_cached[o->n_admitted] = a.cached;
    ++o->n_admitted;
  }
  for (const Chunk& c : chunks) {
    o->prefill_ids[o->n_prefill] = c.r->id;
    o->prefill_start[o->n_prefill] = c.start;
    o->prefill_len[o->n_prefill] = c.n;
    ++o->n_prefill;
  }
  return PKV_OK;
}

pkv_status pkv_sched_end_step(pkv_sched* s) {
  if (!s || !s->in_step) return PKV_EINVAL;
  s->in_step = false;
  for (pkv_sched::Req* r : s->finishing) {
    const pkv_status st = pkv_bm_free_seq(s->bm, r->id);
    if (st != PKV_OK) return st;
    for (size_t k = 0; k < s->running.size(); ++k)
      if (s->running[k] == r) {
        s->running.erase(s->running.begin() + k);
        break;
      }
    s->reserved_total -= r->reserved;
    s->reqs.erase(r->id);
  }
  s->finishing.clear();
  return PKV_OK;
}

pkv_status pkv_sched_stats(const pkv_sched* s, int64_t* tokens_held, int64_t* slots_committed,
                           int32_t* n_waiting, int32_t* n_running, int32_t* n_swapped) {
  if (!s || !tokens_held || !slots_committed || !n_waiting || !n_running || !n_swapped)
    return PKV_EINVAL;
  int64_t held = 0;
  for (const pkv_sched::Req* r : s->running) held += r->ctx();
  *tokens_held = held;
  if (s->reserve) {
    *slots_committed = s->reserved_total * s->B;
  } else {
    int32_t nfree = 0;
    pkv_bm_num_free(s->bm, &nfree);
    *slots_committed = (int64_t)(s->N - nfree) * s->B;
  }
  *n_waiting = (int32_t)s->waiting.size();
  *n_running = (int32_t)s->running.size();
  *n_swapped = (int32_t)s->swapped.size();
  return PKV_OK;
}

}  // extern "C"

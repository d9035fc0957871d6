// Host block manager behind the pkv_bm_* entry points.
//
// Bookkeeping for a pool of fixed-size KV blocks (PagedAttention: The vLLM
// Paper, "Implementation Essentials": pre-allocated pool, block allocation and
// reclamation, refcounts for cross-sequence sharing; "The Core Idea": blocks
// claimed on demand and returned when done; PagedAttention and Continuous
// Batching, "Pages, from operating systems": block tables, allocation as tokens
// arrive, copy-on-write of shared blocks).
//
// All integer work, O(1) per token except fork/free/swap (O(blocks of the
// sequence)).  The free queue is a doubly linked list threaded through two
// arrays of num_blocks entries: a block id is in it exactly when its refcount
// is zero, and a prefix-cache hit can take a block out of the middle in O(1).
//
// Swapping (PagedAttention: The vLLM Paper, "The Core Idea", OS-paging analogy
// table, "Swapping"; "Implementation Essentials": preemption moves a request's
// blocks to CPU memory): an optional host pool with the device pool's geometry
// and its own FIFO free ring.  A swapped sequence keeps its length and holds
// host block ids in its table until it is swapped back in or freed.
//
// Prefix caching (PagedAttention: The vLLM Paper, "Impact and Follow-Ups": the
// KV of a shared prompt prefix is cached and reused across requests): a full
// block is registered under the exact token ids of the whole prefix up to its
// end, stays cached while in use and after it is freed, and loses its entry
// when the free queue hands it out for other content.
#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/pkv.h"

struct pkv_bm {
  struct Seq {
    std::vector<int32_t> table;  // device blocks, or host blocks while swapped
    int32_t len = 0;
    bool swapped = false;
  };
  int32_t N = 0, B = 0;
  std::vector<int32_t> ref;
  std::vector<int32_t> nxt, prv;  // free queue links (-1 = none), front at head
  int32_t head = -1, tail = -1, nfree = 0;
  std::unordered_map<std::string, int32_t> cache;  // prefix token ids -> block
  std::vector<std::string> cached_key;             // block -> its key ("" = none)
  int32_t NH = 0;             // host pool: FIFO ring of its free blocks
  std::vector<int32_t> hring;
  int32_t hhead = 0, hnfree = 0;
  std::unordered_map<int64_t, Seq> seqs;

  void unlink(int32_t b) {
    if (prv[b] >= 0) nxt[prv[b]] = nxt[b]; else head = nxt[b];
    if (nxt[b] >= 0) prv[nxt[b]] = prv[b]; else tail = prv[b];
    nxt[b] = prv[b] = -1;
    --nfree;
  }
  // the front block, for new content: its cached prefix (if any) is dropped
  int32_t pop_free() {
    const int32_t b = head;
    unlink(b);
    ref[b] = 1;
    if (!cached_key[b].empty()) {
      cache.erase(cached_key[b]);
      cached_key[b].clear();
    }
    return b;
  }
  void push_free(int32_t b) {
    prv[b] = tail;
    nxt[b] = -1;
    if (tail >= 0) nxt[tail] = b; else head = b;
    tail = b;
    ++nfree;
  }
  int32_t pop_host() {
    int32_t h = hring[hhead];
    hhead = (hhead + 1 == NH) ? 0 : hhead + 1;
    --hnfree;
    return h;
  }
  void push_host(int32_t h) {
    int32_t t = hhead + hnfree;
    if (t >= NH) t -= NH;
    hring[t] = h;
    ++hnfree;
  }
  void release(const std::vector<int32_t>& table) {
    for (int32_t b : table)
      if (--ref[b] == 0) push_free(b);
  }
  // a sequence on the device: PKV_ENOSEQ if unknown, PKV_EINVAL if swapped out
  pkv_status resident(int64_t id, Seq** out) {
    auto it = seqs.find(id);
    if (it == seqs.end()) return PKV_ENOSEQ;
    if (it->second.swapped) return PKV_EINVAL;
    *out = &it->second;
    return PKV_OK;
  }
  pkv_status resident(int64_t id, const Seq** out) const {
    auto it = seqs.find(id);
    if (it == seqs.end()) return PKV_ENOSEQ;
    if (it->second.swapped) return PKV_EINVAL;
    *out = &it->second;
    return PKV_OK;
  }
};

extern "C" {

pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* init_free_order,
                         pkv_bm** out) {
  if (!out || num_blocks <= 0 || block_size <= 0) return PKV_EINVAL;
  *out = nullptr;
  pkv_bm* bm = new (std::nothrow) pkv_bm();
  if (!bm) return PKV_EINVAL;
  bm->N = num_blocks;
  bm->B = block_size;
  bm->ref.assign(num_blocks, 0);
  bm->nxt.assign(num_blocks, -1);
  bm->prv.assign(num_blocks, -1);
  bm->cached_key.resize(num_blocks);
  if (init_free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = init_free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return PKV_EINVAL;
      }
      seen[b] = 1;
    }
    for (int32_t i = 0; i < num_blocks; ++i) bm->push_free(init_free_order[i]);
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) bm->push_free(i);
  }
  *out = bm;
  return PKV_OK;
}

void pkv_bm_destroy(pkv_bm* bm) { delete bm; }

pkv_status pkv_bm_add_seq(pkv_bm* bm, int64_t seq_id, int32_t num_tokens) {
  if (!bm || num_tokens < 0) return PKV_EINVAL;
  if (bm->seqs.count(seq_id)) return PKV_EEXIST;
  int32_t need = num_tokens / bm->B + (num_tokens % bm->B != 0);
  if (need > bm->nfree) return PKV_ENOBLOCKS;
  pkv_bm::Seq s;
  s.table.reserve(need + 1);
  for (int32_t i = 0; i < need; ++i) s.table.push_back(bm->pop_free());
  s.len = num_tokens;
  bm->seqs.emplace(seq_id, std::move(s));
  return PKV_OK;
}

pkv_status pkv_bm_add_seq_prefix(pkv_bm* bm, int64_t seq_id, const int32_t* tokens,
                                 int32_t n_ids, int32_t num_tokens, int32_t* cached) {
  if (!bm || !cached || n_ids < 0 || num_tokens < n_ids || (n_ids > 0 && !tokens))
    return PKV_EINVAL;
  if (bm->seqs.count(seq_id)) return PKV_EEXIST;
  const int32_t B = bm->B;
  const int32_t full = n_ids / B;                      // full blocks the ids cover
  const int32_t cap = (num_tokens > 0 ? num_tokens - 1 : 0) / B;  // leave a token to compute
  const char* bytes = reinterpret_cast<const char*>(tokens);
  auto key_of = [&](int32_t j) { return std::string(bytes, (size_t)(j + 1) * B * sizeof(int32_t)); };
  std::vector<int32_t> hits;
  for (int32_t j = 0; j < full && j < cap; ++j) {
    auto it = bm->cache.find(key_of(j));
    if (it == bm->cache.end()) break;
    hits.push_back(it->second);
  }
  const int32_t need = num_tokens / B + (num_tokens % B != 0) - (int32_t)hits.size();
  int32_t from_free = 0;
  for (int32_t b : hits) from_free += bm->ref[b] == 0;
  if (need > bm->nfree - from_free) return PKV_ENOBLOCKS;
  for (int32_t b : hits) {
    if (bm->ref[b] == 0) bm->unlink(b);
    bm->ref[b] += 1;
  }
  pkv_bm::Seq s;
  s.table = hits;
  s.table.reserve(hits.size() + need + 1);
  for (int32_t i = 0; i < need; ++i) s.table.push_back(bm->pop_free());
  s.len = num_tokens;
  bm->seqs.emplace(seq_id, std::move(s));
  *cached = (int32_t)hits.size() * B;
  return PKV_OK;
}

pkv_status pkv_bm_register_prefix(pkv_bm* bm, int64_t seq_id, const int32_t* tokens,
                                  int32_t n_ids, int32_t upto) {
  if (!bm || n_ids < 0 || (n_ids > 0 && !tokens)) return PKV_EINVAL;
  pkv_bm::Seq* s;
  if (pkv_status st = bm->resident(seq_id, &s)) return st;
  if (upto < 0 || upto > s->len || n_ids > s->len) return PKV_EINVAL;
  const int32_t B = bm->B;
  const int32_t nfull = std::min(upto, n_ids) / B;
  const char* bytes = reinterpret_cast<const char*>(tokens);
  for (int32_t j = 0; j < nfull; ++j) {
    std::string key(bytes, (size_t)(j + 1) * B * sizeof(int32_t));
    const int32_t b = s->table[j];
    if (bm->cache.count(key) || !bm->cached_key[b].empty()) continue;
    bm->cached_key[b] = key;
    bm->cache.emplace(std::move(key), b);
  }
  return PKV_OK;
}

pkv_status pkv_bm_unregister_prefix(pkv_bm* bm, int64_t seq_id, int32_t start) {
  if (!bm || start < 0) return PKV_EINVAL;
  pkv_bm::Seq* s;
  if (pkv_status st = bm->resident(seq_id, &s)) return st;
  for (size_t j = (size_t)(start / bm->B); j < s->table.size(); ++j) {
    const int32_t b = s->table[j];
    if (bm->cached_key[b].empty() || bm->ref[b] != 1) continue;  // not cached, or shared
    bm->cache.erase(bm->cached_key[b]);
    bm->cached_key[b].clear();
  }
  return PKV_OK;
}

pkv_status pkv_bm_cached_blocks(const pkv_bm* bm, int32_t* out) {
  if (!bm || !out) return PKV_EINVAL;
  *out = (int32_t)bm->cache.size();
  return PKV_OK;
}

static pkv_status append_one(pkv_bm* bm, pkv_bm::Seq& s, int64_t* slot, int32_t* src,
                             int32_t* dst) {
  const int32_t B = bm->B, L = s.len;
  *src = -1;
  *dst = -1;
  if (L % B == 0) {
    if (bm->nfree == 0) return PKV_ENOBLOCKS;
    s.table.push_back(bm->pop_free());
  } else {
    int32_t last = s.table.back();
    if (bm->ref[last] > 1) {
      if (bm->nfree == 0) return PKV_ENOBLOCKS;
      int32_t nb = bm->pop_free();
      bm->ref[last] -= 1;
      s.table.back() = nb;
      *src = last;
      *dst = nb;
    }
  }
  *slot = (int64_t)s.table[L / B] * B + L % B;
  s.len = L + 1;
  return PKV_OK;
}

pkv_status pkv_bm_append_slot(pkv_bm* bm, int64_t seq_id, int64_t* slot, int32_t* cow_src,
                              int32_t* cow_dst) {
  if (!bm || !slot || !cow_src || !cow_dst) return PKV_EINVAL;
  pkv_bm::Seq* s;
  if (pkv_status st = bm->resident(seq_id, &s)) return st;
  return append_one(bm, *s, slot, cow_src, cow_dst);
}

pkv_status pkv_bm_append_slots(pkv_bm* bm, const int64_t* seq_ids, int32_t n, int64_t* slots,
                               int32_t* cow_pairs, int32_t* n_cow, int32_t* n_done) {
  if (!bm || n < 0 || !n_cow || !n_done || (n > 0 && (!seq_ids || !slots || !cow_pairs)))
    return PKV_EINVAL;
  *n_cow = 0;
  *n_done = 0;
  for (int32_t i = 0; i < n; ++i) {
    pkv_bm::Seq* s;
    if (pkv_status st = bm->resident(seq_ids[i], &s)) return st;
    int32_t src, dst;
    pkv_status st = append_one(bm, *s, &slots[i], &src, &dst);
    if (st != PKV_OK) return st;
    if (src >= 0) {
      cow_pairs[2 * *n_cow] = src;
      cow_pairs[2 * *n_cow + 1] = dst;
      ++*n_cow;
    }
    ++*n_done;
  }
  return PKV_OK;
}

pkv_status pkv_bm_fork(pkv_bm* bm, int64_t parent_id, int64_t child_id) {
  if (!bm) return PKV_EINVAL;
  pkv_bm::Seq* parent;
  if (pkv_status st = bm->resident(parent_id, &parent)) return st;
  if (bm->seqs.count(child_id)) return PKV_EEXIST;
  pkv_bm::Seq child = *parent;  // copy before emplace may rehash
  for (int32_t b : child.table) bm->ref[b] += 1;
  bm->seqs.emplace(child_id, std::move(child));
  return PKV_OK;
}

pkv_status pkv_bm_truncate(pkv_bm* bm, int64_t seq_id, int32_t new_len) {
  if (!bm) return PKV_EINVAL;
  pkv_bm::Seq* s;
  if (pkv_status st = bm->resident(seq_id, &s)) return st;
  if (new_len < 0 || new_len > s->len) return PKV_EINVAL;
  const size_t keep = (size_t)((new_len + bm->B - 1) / bm->B);
  if (new_len % bm->B) {
    // the kept last block becomes partial: appends will rewrite it in place
    // unless it is shared, so its prefix-cache entry goes
    const int32_t b = s->table[keep - 1];
    if (bm->ref[b] == 1 && !bm->cached_key[b].empty()) {
      bm->cache.erase(bm->cached_key[b]);
      bm->cached_key[b].clear();
    }
  }
  for (size_t j = keep; j < s->table.size(); ++j)
    if (--bm->ref[s->table[j]] == 0) bm->push_free(s->table[j]);
  s->table.resize(keep);
  s->len = new_len;
  return PKV_OK;
}

pkv_status pkv_bm_free_seq(pkv_bm* bm, int64_t seq_id) {
  if (!bm) return PKV_EINVAL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PKV_ENOSEQ;
  if (it->second.swapped) {
    for (int32_t h : it->second.table) bm->push_host(h);
  } else {
    bm->release(it->second.table);
  }
  bm->seqs.erase(it);
  return PKV_OK;
}

pkv_status pkv_bm_set_host_pool(pkv_bm* bm, int32_t num_host_blocks) {
  if (!bm || num_host_blocks <= 0 || bm->NH) return PKV_EINVAL;
  bm->hring.resize(num_host_blocks);
  for (int32_t i = 0; i < num_host_blocks; ++i) bm->hring[i] = i;
  bm->NH = num_host_blocks;
  bm->hnfree = num_host_blocks;
  bm->hhead = 0;
  return PKV_OK;
}

pkv_status pkv_bm_num_free_host(const pkv_bm* bm, int32_t* out) {
  if (!bm || !out) return PKV_EINVAL;
  *out = bm->hnfree;
  return PKV_OK;
}

pkv_status pkv_bm_is_swapped(const pkv_bm* bm, int64_t seq_id, int32_t* out) {
  if (!bm || !out) return PKV_EINVAL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PKV_ENOSEQ;
  *out = it->second.swapped ? 1 : 0;
  return PKV_OK;
}

pkv_status pkv_bm_swap_out(pkv_bm* bm, int64_t seq_id, int32_t* pairs, int32_t cap,
                           int32_t* n_pairs) {
  if (!bm || !n_pairs || cap < 0 || (cap > 0 && !pairs)) return PKV_EINVAL;
  pkv_bm::Seq* s;
  if (pkv_status st = bm->resident(seq_id, &s)) return st;
  const int32_t n = (int32_t)s->table.size();
  if (n > bm->hnfree) return PKV_ENOBLOCKS;  // before the buffer check: a caller
  if (n > cap) return PKV_EINVAL;            // sizing pairs by free blocks sees ENOBLOCKS
  std::vector<int32_t> host(n);
  for (int32_t i = 0; i < n; ++i) {
    host[i] = bm->pop_host();
    pairs[2 * i] = s->table[i];
    pairs[2 * i + 1] = host[i];
  }
  bm->release(s->table);
  s->table.swap(host);
  s->swapped = true;
  *n_pairs = n;
  return PKV_OK;
}

pkv_status pkv_bm_swap_in(pkv_bm* bm, int64_t seq_id, int32_t* pairs, int32_t cap,
                          int32_t* n_pairs) {
  if (!bm || !n_pairs || cap < 0 || (cap > 0 && !pairs)) return PKV_EINVAL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PKV_ENOSEQ;
  pkv_bm::Seq& s = it->second;
  if (!s.swapped) return PKV_EINVAL;
  const int32_t n = (int32_t)s.table.size();
  if (n > bm->nfree) return PKV_ENOBLOCKS;
  if (n > cap) return PKV_EINVAL;
  std::vector<int32_t> dev(n);
  for (int32_t i = 0; i < n; ++i) {
    dev[i] = bm->pop_free();
    pairs[2 * i] = s.table[i];
    pairs[2 * i + 1] = dev[i];
  }
  for (int32_t h : s.table) bm->push_host(h);
  s.table.swap(dev);
  s.swapped = false;
  *n_pairs = n;
  return PKV_OK;
}

pkv_status pkv_bm_geometry(const pkv_bm* bm, int32_t* num_blocks, int32_t* block_size) {
  if (!bm || !num_blocks || !block_size) return PKV_EINVAL;
  *num_blocks = bm->N;
  *block_size = bm->B;
  return PKV_OK;
}

pkv_status pkv_bm_num_free(const pkv_bm* bm, int32_t* out) {
  if (!bm || !out) return PKV_EINVAL;
  *out = bm->nfree;
  return PKV_OK;
}

pkv_status pkv_bm_refcount(const pkv_bm* bm, int32_t block, int32_t* out) {
  if (!bm || !out || block < 0 || block >= bm->N) return PKV_EINVAL;
  *out = bm->ref[block];
  return PKV_OK;
}

pkv_status pkv_bm_seq_info(const pkv_bm* bm, int64_t seq_id, int32_t* len, int32_t* nblocks) {
  if (!bm || !len || !nblocks) return PKV_EINVAL;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PKV_ENOSEQ;
  *len = it->second.len;
  *nblocks = (int32_t)it->second.table.size();
  return PKV_OK;
}

pkv_status pkv_bm_block_table(const pkv_bm* bm, int64_t seq_id, int32_t* out, int32_t cap) {
  if (!bm || cap < 0 || (cap > 0 && !out)) return PKV_EINVAL;
  const pkv_bm::Seq* s;
  if (pkv_status st = bm->resident(seq_id, &s)) return st;
  const auto& t = s->table;
  if ((int32_t)t.size() > cap) return PKV_EINVAL;
  if (!t.empty()) std::memcpy(out, t.data(), t.size() * sizeof(int32_t));
  return PKV_OK;
}

pkv_status pkv_bm_slots(const pkv_bm* bm, int64_t seq_id, int32_t start, int32_t count,
                        int64_t* slots) {
  if (!bm || start < 0 || count < 0 || (count > 0 && !slots)) return PKV_EINVAL;
  const pkv_bm::Seq* sp;
  if (pkv_status st = bm->resident(seq_id, &sp)) return st;
  const auto& s = *sp;
  if ((int64_t)start + count > s.len) return PKV_EINVAL;
  const int32_t B = bm->B;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t t = start + i;
    slots[i] = (int64_t)s.table[t / B] * B + t % B;
  }
  return PKV_OK;
}

pkv_status pkv_bm_fill_batch(const pkv_bm* bm, const int64_t* seq_ids, int32_t n,
                             int32_t max_blocks, int32_t* block_tables, int32_t* context_lens) {
  if (!bm || n < 0 || max_blocks < 0) return PKV_EINVAL;
  if (n > 0 && (!seq_ids || !context_lens || (max_blocks > 0 && !block_tables)))
    return PKV_EINVAL;
  // validate everything first so a failing call writes nothing
  for (int32_t i = 0; i < n; ++i) {
    const pkv_bm::Seq* s;
    if (pkv_status st = bm->resident(seq_ids[i], &s)) return st;
    if ((int32_t)s->table.size() > max_blocks) return PKV_EINVAL;
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& s = bm->seqs.find(seq_ids[i])->second;
    int32_t* row = block_tables + (size_t)i * max_blocks;
    size_t nb = s.table.size();
    if (nb) std::memcpy(row, s.table.data(), nb * sizeof(int32_t));
    for (size_t j = nb; j < (size_t)max_blocks; ++j) row[j] = -1;
    context_lens[i] = s.len;
  }
  return PKV_OK;
}

pkv_status pkv_bm_count_shared(const pkv_bm* bm, const int64_t* seq_ids, int32_t n,
                               int64_t* out) {
  if (!bm || n < 0 || !out || (n > 0 && !seq_ids)) return PKV_EINVAL;
  int64_t shared = 0;
  for (int32_t i = 0; i < n; ++i) {
    const pkv_bm::Seq* s;
    if (pkv_status st = bm->resident(seq_ids[i], &s)) return st;
    for (int32_t b : s->table) shared += bm->ref[b] > 1;
  }
  *out = shared;
  return PKV_OK;
}

pkv_status pkv_bm_snapshot(const pkv_bm* bm, int32_t* refcounts, int32_t* free_queue,
                           int32_t* n_free) {
  if (!bm || !refcounts || !free_queue || !n_free) return PKV_EINVAL;
  std::memcpy(refcounts, bm->ref.data(), (size_t)bm->N * sizeof(int32_t));
  int32_t i = 0;
  for (int32_t b = bm->head; b >= 0; b = bm->nxt[b]) free_queue[i++] = b;
  *n_free = bm->nfree;
  return PKV_OK;
}

pkv_status pkv_bm_host_snapshot(const pkv_bm* bm, int32_t* free_queue, int32_t* n_free) {
  if (!bm || !n_free || (bm->NH > 0 && !free_queue)) return PKV_EINVAL;
  for (int32_t i = 0; i < bm->hnfree; ++i) {
    int32_t k = bm->hhead + i;
    if (k >= bm->NH) k -= bm->NH;
    free_queue[i] = bm->hring[k];
  }
  *n_free = bm->hnfree;
  return PKV_OK;
}

}  // extern "C"

// Host-side work plan for the decode attention launch (pkv_attention_plan).
//
// The caller's block manager holds every sequence's length on the host, so the
// host can list exactly the (sequence, KV head, partition) work items the batch
// has, instead of the device launching one wave per possible partition and
// letting the empty ones exit.  The list is ordered largest item first (a
// longest-processing-time order: full partitions, then each sequence's partial
// last partition by decreasing size), so the waves that start last carry the
// least work.  It is followed by the (sequence, KV head) rows whose partitions
// the reduce launch must merge.  Pure integer work; no device memory is touched.
#include <algorithm>
#include <cstddef>
#include <vector>

#include "../../include/pkv.h"
#include "decode_config.h"

using pkv::resolve_partition;

namespace {

int64_t num_parts(int64_t mcl, int P) { return mcl <= 0 ? 1 : (mcl + P - 1) / P; }

}  // namespace

extern "C" size_t pkv_attention_plan_words(int32_t S, int32_t Hkv, int32_t B, int32_t max_blocks,
                                           int32_t max_context_len, int32_t partition_size) {
  if (S <= 0 || Hkv <= 0 || max_blocks <= 0 || max_context_len < 0) return 0;
  const int P = resolve_partition(partition_size, B);
  if (P == 0) return 0;
  const int64_t mcl = std::min<int64_t>(max_context_len, (int64_t)max_blocks * B);
  return (size_t)S * Hkv * (4 * (size_t)num_parts(mcl, P) + 1);
}

extern "C" pkv_status pkv_attention_plan(const int32_t* context_lens, int32_t S, int32_t Hkv,
                                         int32_t B, int32_t max_blocks, int32_t max_context_len,
                                         int32_t partition_size, int32_t* plan, size_t plan_words,
                                         int32_t* n_items, int32_t* n_merge) {
  if (!n_items || !n_merge || S < 0 || Hkv <= 0 || max_blocks <= 0 || max_context_len < 0)
    return PKV_EINVAL;
  const int P = resolve_partition(partition_size, B);
  if (P == 0) return PKV_EINVAL;
  if (S > 0 && (!context_lens || !plan)) return PKV_EINVAL;
  const int64_t cap = (int64_t)max_blocks * B;
  const int64_t nparts = num_parts(std::min<int64_t>(max_context_len, cap), P);

  // partitions per sequence (a zero-length sequence keeps one empty item that
  // writes its zero output rows)
  std::vector<int32_t> L(S), np(S);
  int64_t items = 0, merge = 0;
  for (int32_t s = 0; s < S; ++s) {
    L[s] = (int32_t)std::min<int64_t>(context_lens[s], cap);
    np[s] = L[s] <= 0 ? 0 : (int32_t)std::min<int64_t>((L[s] + P - 1) / P, nparts);
    items += (int64_t)std::max(np[s], 1) * Hkv;
    merge += np[s] > 1 ? Hkv : 0;
  }
  if (items > 0x7fffffffLL) return PKV_EINVAL;
  *n_items = (int32_t)items;
  *n_merge = (int32_t)merge;
  if ((size_t)(4 * items + merge) > plan_words) return PKV_EINVAL;

  // counting sort of (sequence, partition) by token count, largest first; the
  // KV heads of one (sequence, partition) stay adjacent
  std::vector<int64_t> count(P + 2, 0);
  auto size_of = [&](int32_t s, int32_t p) -> int32_t {
    return L[s] <= 0 ? 0 : std::min<int32_t>(P, L[s] - p * P);
  };
  for (int32_t s = 0; s < S; ++s)
    for (int32_t p = 0; p < std::max(np[s], 1); ++p) count[P - size_of(s, p)] += 1;
  std::vector<int64_t> pos(P + 2, 0);  // first slot of each size, sizes descending
  for (int k = 1; k <= P + 1; ++k) pos[k] = pos[k - 1] + count[k - 1];
  int32_t* rec = plan;
  for (int32_t s = 0; s < S; ++s) {
    for (int32_t p = 0; p < std::max(np[s], 1); ++p) {
      const int64_t slot = pos[P - size_of(s, p)]++;
      for (int32_t g = 0; g < Hkv; ++g) {
        int32_t* r = rec + 4 * (slot * Hkv + g);
        r[0] = s;
        r[1] = g;
        r[2] = p;
        r[3] = context_lens[s];  // as given: the kernel clamps it the same way
      }
    }
  }
  int32_t* rows = plan + 4 * items;
  for (int32_t s = 0; s < S; ++s)
    if (np[s] > 1)
      for (int32_t g = 0; g < Hkv; ++g) *rows++ = s * Hkv + g;
  return PKV_OK;
}

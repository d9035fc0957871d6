/*
 * pkv.h -- C ABI of the PagedAttention decode library (libpkv.so, MI355X / gfx950).
 *
 * What the library does comes from three accounts of "Efficient Memory Management
 * for Large Language Model Serving with PagedAttention" (Kwon, Li et al., SOSP 2023):
 *   [RTI]  "PagedAttention and Continuous Batching" (roadtointelligence.com)
 *   [LLMS] "vLLM: PagedAttention and continuous batching" (llmstudy)
 *   [ZENO] "PagedAttention: The vLLM Paper" (zenoagi)
 * Each entry point below names the passage that defines its operation.
 *
 * Conventions shared by every call
 *   - Every call returns pkv_status (PKV_OK == 0); pkv_status_string() names it.
 *   - Host validation runs before any launch; a rejected call changes nothing.
 *   - The library never allocates device memory, except inside a pkv_loop
 *     (the serving loop below).  Pools, tables, outputs and workspace are
 *     owned by the caller (the pool is allocated once, up front: [ZENO]
 *     "Implementation Essentials", pre-allocated memory pool).  Otherwise the
 *     only memory the library owns is the host heap behind its handles.
 *   - Device calls take raw device pointers and a hipStream_t (passed as void*,
 *     NULL = the null stream); they are asynchronous with respect to the host and
 *     ordered on that stream.  Device pointers must be 16-byte aligned.
 *   - Device-side indices (block-table entries, slots, copy pairs) cannot be
 *     checked on the host without a sync.  The kernels never access memory
 *     outside the buffers described here: out-of-range block ids are clamped
 *     into [0, num_blocks) and out-of-range slots or pairs are skipped.  The
 *     numerical result of such a call is undefined.
 *
 * KV pool layout (a choice of this library; the pages do not fix one)
 *   x = 16 / sizeof(element): 8 for bf16, 4 for fp32.
 *   K pool: [num_blocks, Hkv, D/x, B, x]   element (b, h, t, d) at
 *           ((b*Hkv + h)*(D/x) + d/x)*B*x + t*x + d%x
 *   V pool: [num_blocks, Hkv, D, B]        element (b, h, t, d) at
 *           ((b*Hkv + h)*D + d)*B + t
 *   (b = physical block, h = KV head, t = slot within the block, d = dim.)
 *   One (block, head) is a contiguous B*D run in both pools.  The K layout keeps
 *   16 bytes of one token's dims together; the V layout keeps each dim's B
 *   tokens together, so both operands of the attention contraction load as
 *   whole 16-byte vectors.
 *   A token at logical position t of a sequence lives in physical block
 *   block_table[t / B], slot t % B; its slot number is block*B + t % B.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_EINVAL = -1,        /* bad argument (null pointer, size, alignment, bad id) */
  PKV_ENOBLOCKS = -2,     /* not enough free blocks; block-manager state unchanged */
  PKV_ENOSEQ = -3,        /* unknown sequence id */
  PKV_EEXIST = -4,        /* sequence id already in use */
  PKV_EUNSUPPORTED = -5,  /* shape or dtype without a compiled kernel */
  PKV_EHIP = -6,          /* a HIP runtime call or kernel launch failed */
  PKV_ENOSCRATCH = -7     /* the call needs more than the library's static scratch */
} pkv_status;

/* Pool element type.  PKV_FP8_E4M3: an fp8 KV cache ([ZENO] "Impact and
 * Follow-Ups" and "Limitations": KV-cache quantization shrinks KV bytes
 * further).  Reading of the format, which the pages leave open: OCP E4M3
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities, NaN
 * 0x7F/0xFF, largest finite 448), stored as the value divided by a per-KV-head
 * fp32 scale (separate scales for K and V; K chunks hold 16 dims, x = 16).
 * Writes encode x / scale (fp32, correctly rounded) to the nearest E4M3 value,
 * ties to an even mantissa, saturating at 448; reads use code value * scale.
 * With fp8 pools the queries and the K/V rows written are bf16. */
typedef enum pkv_dtype { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 } pkv_dtype;

/* Attention flags (bit set).
 * PKV_ATTN_SHARED_KV: sequences of the batch share KV blocks (forked parallel
 *   samples, shared prompt prefixes: [RTI] "Pages, from operating systems",
 *   [ZENO] "Implementation Essentials", prefix sharing).  K/V are then read
 *   with ordinary cached loads, so a block that several sequences read can be
 *   served from L2 or the last-level cache after the first read.  Without it,
 *   K/V are streamed with nontemporal loads, which is faster when every block
 *   is read once per step.  Only a performance hint: results are identical.
 *   pkv_bm_count_shared() tells whether a batch shares blocks. */
enum { PKV_ATTN_SHARED_KV = 1u };

const char* pkv_status_string(pkv_status s);

/* ---------------------------------------------------------------------------
 * Host block manager ([ZENO] "Implementation Essentials": a pre-allocated pool,
 * block allocation and reclamation, refcounts that let sequences share blocks;
 * [RTI] "The solution" and "Pages, from operating systems": fixed-size blocks,
 * a per-request block table, blocks allocated as tokens are generated, shared
 * blocks copied only when one sharer writes them; [ZENO] "The Core Idea":
 * blocks claimed on demand, returned when done, reusable by any request, and
 * only the last block of a sequence partially filled).
 *
 * Semantics fixed by this library where the pages are silent:
 *   - free blocks form a FIFO queue; its initial order is given at creation
 *     (NULL = ascending) and freed blocks are appended in release order;
 *   - add_seq is all-or-nothing; every failing call leaves the state unchanged;
 *   - append_slot: when the length is a multiple of B a new private block is
 *     taken; otherwise, if the last block is shared (refcount > 1), a new block
 *     dst is taken, the pair (src, dst) is returned for the device copy
 *     (pkv_copy_blocks, to be ordered before the token's cache write), src loses
 *     one reference and dst replaces it in the table; a private last block is
 *     written in place.
 * A handle is not thread-safe: one scheduler thread owns it.
 * ------------------------------------------------------------------------- */
typedef struct pkv_bm pkv_bm;

/* Create a manager for num_blocks blocks of block_size tokens.  init_free_order
 * (host, num_blocks entries, a permutation of 0..num_blocks-1) or NULL. */
pkv_status pkv_bm_create(int32_t num_blocks, int32_t block_size,
                         const int32_t* init_free_order, pkv_bm** out);
void pkv_bm_destroy(pkv_bm* bm);

/* Admit sequence seq_id holding num_tokens (>= 0) tokens: ceil(n/B) blocks. */
pkv_status pkv_bm_add_seq(pkv_bm* bm, int64_t seq_id, int32_t num_tokens);

/* Reserve the slot of the sequence's next token.  *slot = block*B + offset;
 * *cow_src / *cow_dst = the block pair to copy first, or -1 / -1. */
pkv_status pkv_bm_append_slot(pkv_bm* bm, int64_t seq_id, int64_t* slot,
                              int32_t* cow_src, int32_t* cow_dst);

/* append_slot for n sequences in order (one decode step).  slots[n] receives each
 * slot; cow_pairs[2*k], cow_pairs[2*k+1] the k-th copy (room for n pairs);
 * *n_cow the number of copies; *n_done the sequences processed.  Stops at the
 * first failure and returns its status (the first *n_done appends stand). */
pkv_status pkv_bm_append_slots(pkv_bm* bm, const int64_t* seq_ids, int32_t n,
                               int64_t* slots, int32_t* cow_pairs, int32_t* n_cow,
                               int32_t* n_done);

/* Share the parent's blocks with a new sequence (parallel sampling): the child
 * gets a copy of the table and every block gains one reference. */
pkv_status pkv_bm_fork(pkv_bm* bm, int64_t parent_id, int64_t child_id);

/* Finish a sequence: each block loses one reference; blocks reaching zero go to
 * the back of the free queue in logical order. */
pkv_status pkv_bm_free_seq(pkv_bm* bm, int64_t seq_id);

/* Give back a resident sequence's tokens past new_len, e.g. speculative draft
 * tokens a verification rejected ([ZENO] "Impact and Follow-Ups": multi-token
 * queries over paged KV also serve speculative decoding; drafts take their
 * slots through pkv_bm_append_slot like any token).  Blocks past
 * ceil(new_len/B) lose one reference each, in logical order, as in
 * pkv_bm_free_seq; if the kept last block becomes partial and is not shared,
 * its prefix-cache entry is withdrawn (its later slots will be rewritten).
 * PKV_EINVAL for new_len outside [0, length] or a swapped-out sequence,
 * PKV_ENOSEQ for an unknown one; no change on error. */
pkv_status pkv_bm_truncate(pkv_bm* bm, int64_t seq_id, int32_t new_len);

pkv_status pkv_bm_num_free(const pkv_bm* bm, int32_t* out);
/* Pool geometry given at creation: blocks and tokens per block. */
pkv_status pkv_bm_geometry(const pkv_bm* bm, int32_t* num_blocks, int32_t* block_size);
pkv_status pkv_bm_refcount(const pkv_bm* bm, int32_t block, int32_t* out);
pkv_status pkv_bm_seq_info(const pkv_bm* bm, int64_t seq_id, int32_t* len, int32_t* nblocks);
/* Copy the sequence's table into out[cap]; PKV_EINVAL if cap is too small. */
pkv_status pkv_bm_block_table(const pkv_bm* bm, int64_t seq_id, int32_t* out, int32_t cap);

/* Slot numbers (block*B + offset) of the sequence's tokens [start,
 * start+count) into slots[count] -- where a prefill writes its KV
 * ([RTI] "Pages, from operating systems": token t of a request lives in its
 * logical block t/B, mapped by the block table).  PKV_EINVAL past its length. */
pkv_status pkv_bm_slots(const pkv_bm* bm, int64_t seq_id, int32_t start, int32_t count,
                        int64_t* slots);

/* Host arrays for a decode batch: block_tables[n*max_blocks] (row i = seq_ids[i],
 * padded with -1) and context_lens[n]. */
pkv_status pkv_bm_fill_batch(const pkv_bm* bm, const int64_t* seq_ids, int32_t n,
                             int32_t max_blocks, int32_t* block_tables,
                             int32_t* context_lens);

/* Table entries of the listed sequences whose block has refcount > 1 (blocks
 * shared through fork), summed over the sequences, into *out.  Non-zero means
 * the batch should be attended with PKV_ATTN_SHARED_KV. */
pkv_status pkv_bm_count_shared(const pkv_bm* bm, const int64_t* seq_ids, int32_t n,
                               int64_t* out);

/* Whole-pool state for parity checks: refcounts[num_blocks] and the free queue
 * front to back in free_queue[0 .. *n_free) (room for num_blocks entries). */
pkv_status pkv_bm_snapshot(const pkv_bm* bm, int32_t* refcounts, int32_t* free_queue,
                           int32_t* n_free);

/* Prefix caching ([ZENO] "Impact and Follow-Ups": the KV of a shared prompt
 * prefix is cached and reused across requests, so on a hit that part of the
 * prefill is free; [ZENO] "Implementation Essentials": prefix sharing through
 * block refcounts).  Semantics fixed by this library where the pages are
 * silent:
 *   - a full block is identified by the token ids of the whole prefix up to
 *     its end (exact match, no hash collisions);
 *   - pkv_bm_add_seq_prefix admits seq_id with num_tokens tokens whose first
 *     n_ids ids are tokens[0..n_ids).  Walking its full blocks from logical
 *     block 0 it reuses the cached block of each prefix while one exists
 *     (refcount + 1; a cached block with refcount 0 leaves the free queue), at
 *     most (num_tokens - 1) / B blocks so at least one token is left to
 *     compute; the remaining blocks are taken as add_seq takes them.
 *     *cached = reused tokens (a multiple of B).  All-or-nothing:
 *     PKV_ENOBLOCKS when the free queue, less the hits taken out of it, is too
 *     short; PKV_EEXIST for a known id; PKV_EINVAL when num_tokens < n_ids;
 *   - pkv_bm_register_prefix registers each full block of the sequence that
 *     the ids cover and that ends at or before token `upto`, unless another
 *     block holds that prefix already.  Call it once that KV is written, or
 *     will be written before anything reads it (a prefill chunk of the same
 *     step); PKV_EINVAL when upto or n_ids exceeds the sequence's length;
 *   - pkv_bm_unregister_prefix withdraws the sequence's own entries (blocks it
 *     alone holds) for blocks ending after token `start`: KV that will not be
 *     written after all (a prefill chunk withdrawn by preemption);
 *   - a cached block stays cached while in use and after it is freed, until
 *     the free queue hands it out for other content (the least recently freed
 *     cached block goes first).
 * Token ids are only compared, never interpreted. */
pkv_status pkv_bm_add_seq_prefix(pkv_bm* bm, int64_t seq_id, const int32_t* tokens,
                                 int32_t n_ids, int32_t num_tokens, int32_t* cached);
pkv_status pkv_bm_register_prefix(pkv_bm* bm, int64_t seq_id, const int32_t* tokens,
                                  int32_t n_ids, int32_t upto);
pkv_status pkv_bm_unregister_prefix(pkv_bm* bm, int64_t seq_id, int32_t start);
/* Number of blocks currently registered in the prefix cache. */
pkv_status pkv_bm_cached_blocks(const pkv_bm* bm, int32_t* out);

/* Swapping ([ZENO] "The Core Idea", OS-paging analogy table, "Swapping": KV
 * blocks go to CPU memory; [ZENO] "Implementation Essentials": preemption
 * swaps a request's blocks to the CPU).  Semantics fixed by this library where
 * the pages are silent:
 *   - a host pool of num_host_blocks blocks with the device pool's geometry,
 *     set once (PKV_EINVAL on a second call or a size <= 0); its free blocks
 *     form a FIFO queue, initially ascending;
 *   - swap_out moves a resident sequence to the host: walking its table from
 *     logical block 0 it takes one host block per entry and writes the pair
 *     (device block, host block) into pairs[2i], pairs[2i+1]; then it releases
 *     its device blocks as free_seq does.  A block it shares keeps its other
 *     references on the device; the host copy is private;
 *   - swap_in brings a swapped sequence back: one new device block per host
 *     block, in table order, pairs (host block, device block); then the host
 *     blocks return to the host free queue in table order;
 *   - both are all-or-nothing: PKV_ENOBLOCKS when the destination side has
 *     fewer free blocks than the table has entries (checked first), else
 *     PKV_EINVAL when `cap` (pairs, i.e. 2*cap int32 entries) is too small, PKV_ENOSEQ for an unknown
 *     id, PKV_EINVAL for the wrong side (swap_out of a swapped sequence, swap_in
 *     of a resident one); a failing call changes nothing;
 *   - a swapped sequence keeps its id and length (pkv_bm_seq_info works) and
 *     can be freed (its host blocks return to the host queue); append_slot(s),
 *     fork (as parent), block_table, slots, fill_batch and count_shared give
 *     PKV_EINVAL for it.
 * The caller copies the data (pkv_swap_blocks): swap-out pairs before any
 * write to the released device blocks, swap-in pairs before the sequence's
 * blocks are read or written on the device. */
pkv_status pkv_bm_set_host_pool(pkv_bm* bm, int32_t num_host_blocks);
pkv_status pkv_bm_num_free_host(const pkv_bm* bm, int32_t* out);
pkv_status pkv_bm_is_swapped(const pkv_bm* bm, int64_t seq_id, int32_t* out);
pkv_status pkv_bm_swap_out(pkv_bm* bm, int64_t seq_id, int32_t* pairs, int32_t cap,
                           int32_t* n_pairs);
pkv_status pkv_bm_swap_in(pkv_bm* bm, int64_t seq_id, int32_t* pairs, int32_t cap,
                          int32_t* n_pairs);
/* The host free queue front to back in free_queue[0 .. *n_free) (room for
 * num_host_blocks entries; free_queue may be NULL before a host pool is set). */
pkv_status pkv_bm_host_snapshot(const pkv_bm* bm, int32_t* free_queue, int32_t* n_free);

/* ---------------------------------------------------------------------------
 * Continuous batching scheduler ([RTI] "Batch by step, not by request": the
 * batch is rebuilt after every decode step, finished sequences leave and
 * waiting ones join, and with paging a newcomer needs only free blocks;
 * [ZENO] "Continuous Batching" figure: A finishes, A dequeues, D enqueues, the
 * batch becomes {B, C, D}; [ZENO] "Implementation Essentials": under memory
 * pressure a request's blocks are swapped to CPU memory, or dropped and its KV
 * recomputed later).
 *
 * A host-side driver over one block manager (which it does not own; the
 * manager must outlive it and take no other sequence ids meanwhile).  Policy
 * (readings where the pages are silent):
 *   - requests are admitted first come first served; admission stops at the
 *     first waiting request that does not fit; at most max_running run;
 *   - paged policy: admission allocates blocks for the request's context (its
 *     prompt plus tokens generated before any preemption), whose KV the caller
 *     then writes (prefill);
 *   - reserve policy (PKV_SCHED_RESERVE_MAX): a simulation of the max-length
 *     reservation of the systems before paging ([ZENO] "Background and
 *     Motivation"): a request is admitted only if the blocks not yet reserved
 *     cover ceil((prompt + max_new) / B); they stay reserved until it finishes;
 *   - every running request produces one token per step; slots are appended
 *     in admission order;
 *   - when an append finds no free block, the most recently admitted running
 *     request is preempted: its blocks are freed, it returns to the front of
 *     the waiting queue keeping its generated tokens, and the append is retried;
 *   - swap policy (PKV_SCHED_SWAP; the block manager needs a host pool): a
 *     preempted request that holds KV (not admitted in this same step, whose
 *     prefill is not written yet) is swapped out (pkv_bm_swap_out) when the
 *     host has a block for each of its blocks, and goes to the front of a
 *     swapped queue; otherwise it is dropped as above.  Each step first swaps
 *     requests back in from the front of that queue (pkv_bm_swap_in) while
 *     fewer than max_running run and the device has room, no skipping ahead;
 *     a resumed request rejoins the running list at its end.  No waiting
 *     request is admitted while any request is swapped out.  The caller runs a
 *     step's copies in this order: swap_in_pairs (host to device), then
 *     swap_out_pairs (device to host; they may reuse host blocks the swap-ins
 *     released), then cow_pairs, then the prefill writes, then the token
 *     writes and attention;
 *   - prefix caching and chunked prefill ([ZENO] "Impact and Follow-Ups"): a
 *     request submitted with its prompt's token ids is admitted with
 *     pkv_bm_add_seq_prefix and its cached tokens are not prefilled again (a
 *     dropped request admitted again finds its prompt blocks the same way;
 *     generated tokens are always recomputed).  With max_prefill_tokens > 0
 *     each step first continues the prefills of admitted requests in admission
 *     order, then admits new requests while budget is left, each getting a
 *     chunk of at most the budget left; 0 means no limit (every prefill
 *     completes in its admission step).  A request produces a token only in
 *     steps where its prefill is complete, including the step of its last
 *     chunk.  A preempted request's chunk of that step is withdrawn;
 *   - a request finishes in the step that produces its max_new-th token and is
 *     freed by pkv_sched_end_step, after the caller has read the step's tables.
 * Not thread-safe; one scheduler thread owns a handle.
 * ------------------------------------------------------------------------- */
typedef struct pkv_sched pkv_sched;

enum { PKV_SCHED_RESERVE_MAX = 1, PKV_SCHED_SWAP = 2 };

/* Caller-owned host arrays one step fills; each holds `capacity` entries
 * (>= max_running), cow_pairs 2*capacity.  Under the swap policy the two pair
 * arrays hold 2*pair_capacity entries (pair_capacity >= the pool's
 * num_blocks) and the id arrays `capacity`; otherwise they may be NULL and
 * their counts are 0. */
typedef struct pkv_sched_step {
  int32_t capacity;
  int64_t* batch_ids;      /* requests that produced a token, admission order */
  int64_t* slots;          /* slot of each one's new token (block*B + offset) */
  int32_t n_batch;
  int32_t* cow_pairs;      /* (src, dst) block copies to run before the writes */
  int32_t n_cow;
  int64_t* admitted_ids;   /* admitted this step with context ctx, of which ... */
  int32_t* admitted_ctx;
  int32_t* admitted_cached;/* ... the first `cached` tokens are in the prefix cache */
  int32_t n_admitted;
  int64_t* prefill_ids;    /* prefill chunks: tokens [start, start + len) of the */
  int32_t* prefill_start;  /* request, whose KV the caller writes (and whose rows */
  int32_t* prefill_len;    /* it attends) before the step's token writes */
  int32_t n_prefill;
  int64_t* preempted_ids;  /* preempted this step (back in the waiting queue) */
  int32_t n_preempted;
  int64_t* finished_ids;   /* produced their last token this step */
  int32_t n_finished;
  int32_t pair_capacity;
  int32_t* swap_in_pairs;   /* (host block, device block) copies, run first */
  int32_t n_swap_in;
  int32_t* swap_out_pairs;  /* (device block, host block) copies, run second */
  int32_t n_swap_out;
  int64_t* swapped_in_ids;  /* resumed from the host this step */
  int32_t n_swapped_in;
  int64_t* swapped_out_ids; /* swapped out this step (not in preempted_ids) */
  int32_t n_swapped_out;
} pkv_sched_step;

/* policy: 0 (paged, preempt by dropping), PKV_SCHED_RESERVE_MAX, or
 * PKV_SCHED_SWAP; PKV_EINVAL for unknown bits or both.  max_prefill_tokens:
 * prefill budget per step, 0 = no limit. */
pkv_status pkv_sched_create(pkv_bm* bm, int32_t max_running, int32_t policy,
                            int32_t max_prefill_tokens, pkv_sched** out);
void pkv_sched_destroy(pkv_sched* sched);
/* Queue a request; tokens: NULL or its prompt's prompt_len token ids (copied;
 * enables the prefix cache).  PKV_EEXIST for a known id, PKV_EINVAL when
 * prompt_len < 0, max_new_tokens < 1 or its maximum length can never fit the
 * pool. */
pkv_status pkv_sched_add_request(pkv_sched* sched, int64_t req_id, int32_t prompt_len,
                                 int32_t max_new_tokens, const int32_t* tokens);
/* One iteration (admissions, then one slot per running request).  Steps
 * alternate with pkv_sched_end_step; either one out of turn is PKV_EINVAL. */
pkv_status pkv_sched_begin_step(pkv_sched* sched, pkv_sched_step* out);
/* Free the requests that finished in the step. */
pkv_status pkv_sched_end_step(pkv_sched* sched);
/* Tokens the running requests hold, slots the policy keeps for them (allocated
 * device blocks, or reserved blocks under the reserve policy, times B), and the
 * sizes of the waiting, running and swapped-out sets. */
pkv_status pkv_sched_stats(const pkv_sched* sched, int64_t* tokens_held,
                           int64_t* slots_committed, int32_t* n_waiting,
                           int32_t* n_running, int32_t* n_swapped);

/* One step's device metadata, packed by pkv_pack_step into one host int32
 * buffer so that a single copy takes it to the device.  Offsets count int32
 * words from the buffer's start and are multiples of 4 (16 bytes); int64
 * arrays take two words per entry.  n_prefill_rows = sum of the step's prefill
 * chunk lengths; n_prefill = step->n_prefill; n_batch = step->n_batch. */
typedef struct pkv_step_pack {
  int32_t total_words;     /* words used (set also when buf_words is too small) */
  int32_t n_prefill_rows;
  int32_t slots_off;       /* int64 [n_prefill_rows]: slot of every chunk token */
  int32_t pf_tables_off;   /* int32 [n_prefill, pf_width]: chunk requests' tables */
  int32_t pf_width;        /* blocks of the longest chunk's end position */
  int32_t pf_lens_off;     /* int32 [n_prefill]: start + len of each chunk */
  int32_t pf_start_off;    /* int32 [n_prefill + 1]: first row of each chunk */
  int32_t pf_max_rows;     /* longest chunk */
  int32_t tables_off;      /* int32 [n_batch, width]: decode batch tables */
  int32_t width;           /* blocks of the batch's longest context */
  int32_t lens_off;        /* int32 [n_batch]: context lengths (token of the step included) */
  int32_t max_context;
  int32_t plan_off;        /* the batch's pkv_attention_plan, built from lens_off */
  int32_t n_items, n_merge;
  int32_t pairs_off;       /* int64 [n_prefill_rows + n_batch, 2]: (request id,
                              position) of every K/V row the step writes: the
                              chunks' tokens in order, then each batch request's
                              new token */
  int32_t swap_in_off, swap_out_off, cow_off; /* int32 pairs, step->n_* of each */
} pkv_step_pack;

/* Pack the device metadata of the step pkv_sched_begin_step just returned in
 * `step` (before pkv_sched_end_step): the chunks' slots and tables, the decode
 * batch's tables, lengths and work plan, the K/V row list and the block copy
 * pairs ([ZENO] "Implementation Essentials": the block manager hands the
 * kernels block tables; [RTI] "Batch by step, not by request").
 *   bm            the scheduler's block manager
 *   max_blocks    table row capacity of the loop (blocks of its longest request)
 *   Hkv, partition_size   as for the attention call (for the plan)
 *   buf           HOST int32 buffer of buf_words words (pinned, for an
 *                 asynchronous copy)
 * PKV_EINVAL with out->total_words set when buf_words is too small (nothing
 * useful written); the caller grows the buffer and calls again. */
pkv_status pkv_pack_step(const pkv_bm* bm, const pkv_sched_step* step, int32_t max_blocks,
                         int32_t Hkv, int32_t partition_size, int32_t* buf, size_t buf_words,
                         pkv_step_pack* out);

/* ---------------------------------------------------------------------------
 * Serving loop: a continuous-batching step in one native call ([RTI] "Batch by
 * step, not by request"; [ZENO] "Continuous Batching" and "Implementation
 * Essentials").  pkv_loop_step runs one iteration of the scheduler above and
 * everything the device needs for it: pkv_pack_step into a pinned host buffer
 * (two alternate, so the host packs step t + 1 while step t's copy may still
 * run), one asynchronous copy of the metadata, then on the loop's stream the
 * swap-in, swap-out and copy-on-write block copies, the step's query and K/V
 * rows, pkv_reshape_and_cache of the prefill chunks' tokens,
 * pkv_paged_attention_prefill over the chunks and pkv_paged_attention_decode
 * over the batch (host work plan; the new tokens are written by the attention
 * launch), and finally pkv_sched_end_step.
 * The loop computes no model: the step's rows come from caller-filled device
 * banks, row r of the step (request id, position) reading bank row
 * (id * mul + position) mod bank_rows (q_mul for the query bank, kv_mul for the
 * K and V banks).
 * Unlike the other calls a pkv_loop owns device memory: its metadata buffer,
 * the step's row buffers, the decode workspace and the output buffers, grown
 * (after a stream synchronize) when a step needs more; and two pinned host
 * buffers.  The pools, the scheduler and its block manager stay the caller's
 * and must outlive the loop.  Not thread-safe.
 * ------------------------------------------------------------------------- */
typedef struct pkv_loop pkv_loop;

typedef struct pkv_loop_config {
  int32_t num_blocks, block_size;  /* must match the block manager */
  int32_t q_heads, kv_heads, head_dim;
  int32_t max_running;             /* the scheduler's max_running */
  int32_t max_len;                 /* longest request (prompt + new tokens) */
  int32_t partition_size;          /* decode partitions (0 = the library default) */
  int32_t host_blocks;             /* host pool blocks (swap policy), else 0 */
  pkv_dtype dtype;                 /* PKV_BF16 or PKV_FP8_E4M3 pools */
} pkv_loop_config;

/* Device banks of bf16 rows: q_bank [bank_rows, Hq, D], k_bank and v_bank
 * [bank_rows, Hkv, D]. */
typedef struct pkv_loop_source {
  const void* q_bank;
  const void* k_bank;
  const void* v_bank;
  int64_t bank_rows;
  int64_t q_mul, kv_mul;
} pkv_loop_source;

/* What a step did.  Pointers stay valid until the next step: decode_out is
 * float32 [n_batch, Hq, D] (device), prefill_out float32 [n_prefill_rows, Hq,
 * D] (device, the chunks' rows in order), lens_host the batch's context lengths
 * (pinned host).  tokens_held .. n_swapped are pkv_sched_stats taken before the
 * finished requests leave.  host_us: the call's time on the host; wait_us: the
 * part of it spent waiting for a pinned buffer's previous copy (the device
 * running behind). */
typedef struct pkv_loop_step_info {
  int32_t n_batch, n_prefill, n_prefill_rows, n_admitted, n_preempted, n_finished;
  int32_t n_swapped_out, n_swapped_in, n_swap_out_blocks, n_swap_in_blocks, n_cow;
  int32_t max_context;
  int64_t cached_tokens;           /* prompt tokens of this step's admissions found cached */
  int64_t tokens_held, slots_committed;
  int32_t n_waiting, n_running, n_swapped;
  const int32_t* lens_host;
  const float* decode_out;
  const float* prefill_out;
  double host_us, wait_us;
} pkv_loop_step_info;

/* k_pool / v_pool: the device pools ([num_blocks] blocks, layouts above);
 * host_k / host_v: pinned host pools of host_blocks blocks (swap policy) or
 * NULL; k_scale / v_scale: fp8 per-KV-head scales (device float32 [Hkv]) or
 * NULL for bf16.  PKV_EINVAL for a bad or mismatched configuration,
 * PKV_EHIP when an allocation fails. */
pkv_status pkv_loop_create(const pkv_loop_config* cfg, pkv_bm* bm, pkv_sched* sched,
                           void* k_pool, void* v_pool, void* host_k, void* host_v,
                           const float* k_scale, const float* v_scale, void* hip_stream,
                           pkv_loop** out);
void pkv_loop_destroy(pkv_loop* loop);
/* One step.  An error after the scheduler began the step still ends it (the
 * loop stays usable) and is returned; *info is filled either way. */
pkv_status pkv_loop_step(pkv_loop* loop, const pkv_loop_source* source, pkv_loop_step_info* info);
/* Copy the last step's outputs (decode [n_batch, Hq, D], prefill
 * [n_prefill_rows, Hq, D], float32) into caller device buffers, on the loop's
 * stream; either destination may be NULL. */
pkv_status pkv_loop_copy_outputs(const pkv_loop* loop, float* decode_dst, float* prefill_dst);

/* ---------------------------------------------------------------------------
 * Device operations.
 * ------------------------------------------------------------------------- */

/* Write each new token's K/V into its slot ([ZENO] "Background and Motivation":
 * every generated token adds K/V vectors to the cache; [RTI] "Pages, from
 * operating systems": blocks are allocated as tokens are generated).
 *   key, value    device [T, Hkv, D], pool dtype
 *   k_pool/v_pool device pools (layout above), updated in place
 *   slot_mapping  device int64 [T]; slot < 0 = skip; slot >= num_blocks*B skipped
 * A bit copy: no conversion, NaN payloads kept.  Two tokens with the same slot
 * in one call race (caller's responsibility).
 *   k_scale, v_scale  fp8 pools: device fp32 [Hkv], the per-KV-head scales
 *                 (key/value are then bf16 and are encoded, see pkv_dtype);
 *                 ignored (may be NULL) otherwise. */
pkv_status pkv_reshape_and_cache(const void* key, const void* value, void* k_pool,
                                 void* v_pool, const int64_t* slot_mapping, int32_t T,
                                 int32_t Hkv, int32_t D, int32_t B, int32_t num_blocks,
                                 pkv_dtype dtype, const float* k_scale, const float* v_scale,
                                 void* hip_stream);

/* Copy-on-write block copies ([RTI] "Pages, from operating systems": shared
 * blocks are copied only when one sequence needs to modify them; [ZENO] OS-paging
 * analogy table: page sharing with fork and copy-on-write).  For each pair k,
 * block pairs[2k+1] := block pairs[2k] in both pools (all heads, all slots).
 *   pairs  device int32 [n, 2] (src, dst); a pair with an id outside
 *          [0, num_blocks) is skipped.  dst ids must be distinct and must not
 *          appear as a src in the same call (the copies run concurrently). */
pkv_status pkv_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int32_t n,
                           int32_t Hkv, int32_t D, int32_t B, int32_t num_blocks,
                           pkv_dtype dtype, void* hip_stream);

/* Multi-token queries over the paged cache: chunked prefill, and the
 * uncached rest of a prompt after a prefix-cache hit ([ZENO] "Impact and
 * Follow-Ups": prefix caching reuses a cached prompt prefix so only the rest
 * is prefilled; chunked prefill splits long prompts into chunks interleaved
 * with decode).  Sequence s holds L_s = context_lens[s] cached tokens; the
 * last Q_s = query_start[s+1] - query_start[s] of them are this call's queries
 * (their K/V already written, e.g. by pkv_reshape_and_cache).  The query at
 * position p = L_s - Q_s + i attends causally to tokens 0..p ([ZENO]
 * "Background and Motivation"):
 *   out[row, h] = softmax(q[row, h] . K_s[0..p]^T * scale) V_s[0..p]
 *   out           device fp32 [T, Hq, D]; rows of sequence s are
 *                 query_start[s] .. query_start[s+1]-1
 *   q             device bf16 [T, Hq, D], same row packing
 *   query_start   device int32 [S+1], non-decreasing, query_start[S] <= T; a
 *                 sequence whose rows fall outside [0, T) gets none written
 *   context_lens  device int32 [S]; Q_s is clamped to L_s (a sequence with
 *                 more rows than tokens gets only its last L_s rows written)
 *   max_query_len host bound on every Q_s (sizes the grid).  It is not checked
 *                 against query_start, which stays on the device.  A
 *                 sequence's rows are taken in runs of R = 128 / G rows
 *                 counted from its first row, and a call covers the last
 *                 ceil(max_query_len / R) runs of each sequence: when some Q_s
 *                 exceeds the bound, the rows of that sequence's earlier runs
 *                 are not written and no error is returned.  The Python
 *                 binding checks the bound when given a host query_start.
 *   block_tables, max_blocks, num_blocks, Hq, Hkv, scale as for decode.
 *   k_scale, v_scale  fp8 pools: device fp32 [Hkv] per-KV-head scales (q stays
 *                 bf16); NULL otherwise
 * bf16 or fp8 E4M3 pools, D in {64, 128}, B in {16, 32}, Hq/Hkv in
 * {1, 2, 4, 8}; others PKV_EUNSUPPORTED.  A query of one token per sequence is
 * decode (with bf16 pools the result matches pkv_paged_attention_decode's rows
 * bit for bit). */
pkv_status pkv_paged_attention_prefill(float* out, const void* q, const void* k_pool,
                                       const void* v_pool, const int32_t* block_tables,
                                       const int32_t* context_lens, const int32_t* query_start,
                                       int32_t S, int32_t T, int32_t Hq, int32_t Hkv, int32_t D,
                                       int32_t B, int32_t max_blocks, int32_t num_blocks,
                                       int32_t max_query_len, float scale, pkv_dtype dtype,
                                       const float* k_scale, const float* v_scale,
                                       void* hip_stream);

/* Block copies between two pools of the same geometry, one of which is usually
 * a host pool ([ZENO] "The Core Idea", OS-paging analogy table, "Swapping": KV
 * blocks moved to CPU memory and back; [ZENO] "Implementation Essentials").
 * For each pair k, dst block pairs[2k+1] := src block pairs[2k], K and V, all
 * heads and slots; a bit copy.
 *   dst_k, dst_v, dst_blocks   destination pools and their block count
 *   src_k, src_v, src_blocks   source pools and their block count
 *     Each pool is device memory or pinned host memory (hipHostMalloc, or a
 *     pinned torch tensor) that the GPU reaches through its device mapping; the
 *     GPU reads or writes host pools over the host link.  Pageable host memory
 *     is rejected with PKV_EINVAL before any launch.  16-byte aligned.
 *   pairs  device int32 [n, 2] (src block, dst block); a pair with an id
 *          outside its pool is skipped; dst ids must be distinct.
 * Stream-ordered like every device call: a swap-out (device to host) must be
 * enqueued before any write to its released device blocks, a swap-in before
 * the blocks are read; a host pool read by the CPU needs the stream synced. */
pkv_status pkv_swap_blocks(void* dst_k, void* dst_v, int32_t dst_blocks, const void* src_k,
                           const void* src_v, int32_t src_blocks, const int32_t* pairs,
                           int32_t n, int32_t Hkv, int32_t D, int32_t B, pkv_dtype dtype,
                           void* hip_stream);

/* Bytes of workspace pkv_paged_attention_decode needs: 0 when every sequence
 * fits one partition, else 65536 + S*Hq*nparts*(D+2)*4 with
 * nparts = ceil(max_context_len / partition) (partition_size 0 = default 512).
 * The first 65536 bytes are 16384 int32 completion counters of the merge
 * inside the main launch, one per (sequence, KV head): they must be zero
 * before a workspace's first use (allocate it zeroed), and every call that
 * completes leaves them zero, so one workspace serves any later call whose
 * size it covers.  The rest holds the partition partials. */
size_t pkv_attention_workspace_bytes(int32_t S, int32_t Hq, int32_t D,
                                     int32_t max_context_len, int32_t partition_size);

/* Host-side work plan for one decode batch (optional).  The caller's block
 * manager already holds every length on the host (the batch tables are built
 * there, [ZENO] "Implementation Essentials": block manager), so the host can
 * list exactly the batch's work items -- one per (sequence, KV head, partition)
 * that holds tokens -- instead of the device launching one per possible
 * partition.  Items are ordered largest first; a zero-length sequence keeps one
 * empty item (it writes the zero rows).  After the items come the (sequence, KV
 * head) rows whose partitions the reduce launch merges.
 *   context_lens  HOST int32 [S], the same lengths the device copy holds
 *   plan          HOST int32 buffer of plan_words entries, filled with
 *                 *n_items records {s, g, p, L} (4 int32 each) followed by
 *                 *n_merge entries s*Hkv + g
 *   B, max_blocks, max_context_len, partition_size: as for the attention call
 * *n_items and *n_merge are set even when plan_words is too small (then
 * PKV_EINVAL and the plan is not written); pkv_attention_plan_words gives an
 * upper bound.  The caller copies the plan to the device and passes it, with
 * the two counts, to the attention calls below. */
size_t pkv_attention_plan_words(int32_t S, int32_t Hkv, int32_t B, int32_t max_blocks,
                                int32_t max_context_len, int32_t partition_size);
pkv_status pkv_attention_plan(const int32_t* context_lens, int32_t S, int32_t Hkv, int32_t B,
                              int32_t max_blocks, int32_t max_context_len,
                              int32_t partition_size, int32_t* plan, size_t plan_words,
                              int32_t* n_items, int32_t* n_merge);

/* Decode attention through the block table ([LLMS] "Direct answer":
 * PagedAttention follows the logical-to-physical block mapping while computing
 * attention; [ZENO] "The Core Idea": attention computed through block-table
 * indirection, reading KV non-contiguously; [ZENO] "Background and Motivation":
 * each new token attends over all previous tokens).
 *   out           device fp32 [S, Hq, D]: softmax(q K^T * scale) V per (s, h)
 *   q             device [S, Hq, D], pool dtype
 *   k_pool/v_pool device pools; written only when new_key is given
 *   new_key, new_value   NULL, or device [S, Hkv, D] in the pool dtype (bf16
 *                 for fp8 pools, encoded as pkv_reshape_and_cache does): the
 *                 token each sequence appends this step (a decode step).  The
 *                 token is the sequence's last, at position context_lens[s]-1;
 *                 it is written into that position's slot (block
 *                 block_tables[s][(L-1)/B], offset (L-1)%B) and attended to in
 *                 the same launch.  Pools and output are bit-identical to
 *                 pkv_reshape_and_cache with those slots followed by the call
 *                 without new_key.  Copy-on-write copies must run before, so
 *                 that no other sequence of the batch reads the written block.
 *                 A zero-length sequence appends nothing, and so does one whose
 *                 last position is not in the launch (see context_lens).
 *   block_tables  device int32 [S, max_blocks]
 *   context_lens  device int32 [S]: tokens of sequence s (the one written this
 *                 step included); 0 gives a zero row; at most
 *                 min(max_context_len, max_blocks*B).  A larger value is not
 *                 an error the device reports: the launch covers the first
 *                 min(L, max_blocks*B, nparts*P) tokens, with P the partition
 *                 size and nparts = ceil(min(max_context_len, max_blocks*B) / P),
 *                 and appends only when that is all L tokens
 *   Query head h reads KV head h / (Hq/Hkv).
 *   max_context_len  host-known bound on context_lens; sizes the grid (no sync)
 *   scale         score scale, usually 1/sqrt(D); positive and finite, else
 *                 PKV_EINVAL
 *   partition_size   tokens per work item: 0 = default (512), else a positive
 *                 multiple of 32 and of B spanning at most 128 blocks (<= 128*B
 *                 tokens).  Sequences longer than one partition are split and
 *                 their partitions merged (log-sum-exp combine): inside the
 *                 main launch, by the last of a (sequence, KV head)'s items to
 *                 finish, when nparts <= 16 and S*Hkv <= 16384; else by a
 *                 second, reduce launch.
 *   plan, plan_items, plan_merge   NULL, or a DEVICE copy of the plan that
 *                 pkv_attention_plan built for this batch (16-byte aligned) and
 *                 its two counts.  With a plan the main launch runs exactly the
 *                 listed items (taking each partition's length from the plan)
 *                 and a reduce launch merges exactly the listed rows; results are
 *                 bit-identical to the unplanned call.  A record naming a
 *                 sequence or head outside the batch is skipped.
 *   workspace     device buffer of workspace_bytes >= pkv_attention_workspace_bytes
 *                 (may be NULL when that is 0), its counters zero (see there).
 *                 Calls that overlap in time must not share a workspace.
 *                 With the merge inside the launch the plan must list every
 *                 (sequence, KV head, partition) that holds tokens exactly
 *                 once, as pkv_attention_plan's plans do: a missing item
 *                 leaves its rows unwritten and its counter non-zero.
 *   flags         0 or PKV_ATTN_SHARED_KV (other bits: PKV_EINVAL)
 *   k_scale, v_scale  fp8 pools: device fp32 [Hkv] per-KV-head scales (the
 *                 values read are code * scale), positive and finite (the
 *                 device does not check); NULL otherwise
 * Compiled shapes: D in {64, 128}, B in {16, 32}; bf16 with Hq/Hkv in
 * {1, 2, 4, 8}; fp32 with Hq/Hkv in {1, 2, 4, 8}; fp8 pools (bf16 queries)
 * with Hq/Hkv in {4, 8}.  Others: PKV_EUNSUPPORTED. */
pkv_status pkv_paged_attention_decode(float* out, const void* q, void* k_pool, void* v_pool,
                                      const void* new_key, const void* new_value,
                                      const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t S, int32_t Hq,
                                      int32_t Hkv, int32_t D, int32_t B, int32_t max_blocks,
                                      int32_t num_blocks, int32_t max_context_len,
                                      float scale, int32_t partition_size,
                                      const int32_t* plan, int32_t plan_items,
                                      int32_t plan_merge, void* workspace,
                                      size_t workspace_bytes, pkv_dtype dtype,
                                      uint32_t flags, const float* k_scale,
                                      const float* v_scale, void* hip_stream);

/* The two launches of pkv_paged_attention_decode, callable one at a time (for
 * per-kernel timing, or to put other work between them on the stream).
 * pkv_paged_attention_main takes exactly pkv_paged_attention_decode's arguments
 * and runs the main kernel.  When it merges the partitions itself (see
 * partition_size) every row is final in `out` when it completes.  Else rows of
 * sequences that fit
 * one partition are final and longer sequences leave per-partition
 * (max, sum, accumulator) partials in `workspace`, which
 * pkv_paged_attention_reduce then merges into `out` (log-sum-exp combine of the
 * partitions; the split itself is not on the pages, which only note that long
 * contexts are hard: [ZENO] "Limitations").  Its arguments must repeat the
 * values given to the main call (same S, Hq, Hkv, D, B, max_blocks,
 * max_context_len, partition_size, plan, context_lens, workspace); it reads
 * nothing else and is a no-op when the main launch merged. */
pkv_status pkv_paged_attention_main(float* out, const void* q, void* k_pool, void* v_pool,
                                    const void* new_key, const void* new_value,
                                    const int32_t* block_tables,
                                    const int32_t* context_lens, int32_t S, int32_t Hq,
                                    int32_t Hkv, int32_t D, int32_t B, int32_t max_blocks,
                                    int32_t num_blocks, int32_t max_context_len, float scale,
                                    int32_t partition_size, const int32_t* plan,
                                    int32_t plan_items, int32_t plan_merge, void* workspace,
                                    size_t workspace_bytes, pkv_dtype dtype, uint32_t flags,
                                    const float* k_scale, const float* v_scale,
                                    void* hip_stream);
pkv_status pkv_paged_attention_reduce(float* out, const int32_t* context_lens, int32_t S,
                                      int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                      int32_t max_blocks, int32_t max_context_len,
                                      int32_t partition_size, const int32_t* plan,
                                      int32_t plan_items, int32_t plan_merge,
                                      const void* workspace, size_t workspace_bytes,
                                      void* hip_stream);

/* pkv_paged_attention_decode for callers that cannot allocate device memory
 * or bring a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  Same arguments and results as
 * pkv_paged_attention_decode without workspace/workspace_bytes: the partition
 * partials and merge counters live in a 64 MiB array that the library holds
 * in each GPU's memory from its first call on that GPU until the process ends
 * (PKV_SCRATCH_BYTES).  The call allocates nothing; it launches a small kernel
 * that zeroes the merge counters, then the decode launches.
 *   - The stream's device must be the calling thread's current device
 *     (PKV_EINVAL otherwise).
 *   - A call whose pkv_attention_workspace_bytes(S, Hq, D, max_context_len,
 *     partition_size) exceeds PKV_SCRATCH_BYTES returns PKV_ENOSCRATCH before
 *     any launch.
 *   - Every call on a GPU shares that GPU's array and leaves its contents
 *     there: calls that overlap in time on one GPU (several streams, several
 *     threads) race and give wrong results; serialize them. */
#define PKV_SCRATCH_BYTES (64u << 20)
pkv_status pkv_paged_attention_decode_noalloc(float* out, const void* q, void* k_pool,
                                              void* v_pool, const void* new_key,
                                              const void* new_value,
                                              const int32_t* block_tables,
                                              const int32_t* context_lens, int32_t S,
                                              int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                                              int32_t max_blocks, int32_t num_blocks,
                                              int32_t max_context_len, float scale,
                                              int32_t partition_size, const int32_t* plan,
                                              int32_t plan_items, int32_t plan_merge,
                                              pkv_dtype dtype, uint32_t flags,
                                              const float* k_scale, const float* v_scale,
                                              void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* PKV_H */

"""CPU oracle for PagedAttention decode -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct fp64 NumPy code that states what the GPU path
must compute.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import it; the product library never does, and it imports nothing from
the product.

Sources (three web accounts of Kwon, Li et al., "Efficient Memory Management for
Large Language Model Serving with PagedAttention", SOSP 2023):
  * "PagedAttention and Continuous Batching" (roadtointelligence.com), sections
    "The solution" and "Pages, from operating systems";
  * "vLLM: PagedAttention and continuous batching" (llmstudy), "Direct answer";
  * "PagedAttention: The vLLM Paper" (zenoagi), sections "Background and
    Motivation", "The Core Idea" (block-pool figure, OS-paging analogy table,
    three wins), "Implementation Essentials".

Modules:
  attention     gather through the block table + fp64 softmax(q K^T * scale) V,
                and the per-partition log-sum-exp split used for long contexts
  cache_ops     reshape_and_cache (token K/V -> slot) and copy_blocks (CoW copy)
  block_manager allocation, reclamation, refcounts, fork and copy-on-write

Parity pins: every function is pinned by tests marked "not gpu" (worked facts
and the block-pool figure from the pages, brute force, closed forms, a library
attention routine, algebraic identities).  No function is parity-unpinned.
"""

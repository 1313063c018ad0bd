"""CPU oracle for paged decode and prefill attention, the paged KV write and
the block manager.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import or call anything in this package.  The
product path (the HIP library under ``paged_kv_cache_81_amd`` and its Python
binding) never touches it, and it never touches the product path: the two share
no code.  Only the seeded input generators in ``workloads`` serve both.

Every function states the passage it follows.  Page key for the citations:

  [review]       studying-code.tistory.com -- Korean review of the vLLM paper
  [explainer]    tech.blogsailing.com (?p=100) -- Korean PagedAttention explainer
  [notes]        garden.houmin.site /infra/paged-attention -- Chinese notes
  [walkthrough]  itan.pw -- walk-through of vLLM 0.17.1's KVCacheManager

Pins (what each function is checked against, other than itself) live in
``tests/oracle_pins.py``; every function here is pinned.
"""
from .paged_attention import (  # noqa: F401
    TABLE_PAD,
    attention_ref,
    blocks_needed,
    cache_shape_from_bytes,
    chunk_positions,
    gather_ref,
    kv_bytes_per_token,
    last_block_fill,
    merge_ref,
    num_blocks_for,
    page_bytes,
    paged_attention_ref,
    partition_stats_ref,
    prefill_attention_ref,
    slot_mapping_ref,
    slot_of,
    to_f64,
    write_ref,
)
from .block_manager import (  # noqa: F401,E402
    NONE_HASH,
    OutOfBlocks,
    RefBlockManager,
    block_hash,
    copy_blocks_ref,
)

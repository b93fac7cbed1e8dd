"""CPU oracle for paged-KV decode: test infrastructure, not product code.

This package is a plain, slow, obviously-correct restatement of what the
reference pages define.  It exists only to check the HIP path.  Only the
test suite (``tests/``), ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import it; the product package never does, and this
package imports nothing from the product package (they share no code).

Pages cited (titles as they appear, with their web addresses):

* "qaqbuyan.com article 130" (qaqbuyan.com:88/乔安文章/130.html): vLLM
  PagedAttention walk-through -- KV-cache size formula, block-size formula,
  ``BlockTable``, ``paged_attention``/``traditional_attention`` pseudocode,
  ``BlockAllocator``, ``PrefixCache``, scheduler and a simplified
  ``paged_attention_kernel`` listing.
* "day31" (blog.ans20xx.com/posts/ai/day31): memory-estimate script, toy block
  allocator (``KVBlockPool``/``SequenceKV``), toy COW append
  (``fork_sequence``/``ensure_private_last_block``/``append_with_cow``) and the
  block-count script.
* "P06 · BlockManager: paged KV + prefix cache" (kuanzhou.online,
  nano-vllm-omni drills, p06_overview): the block-manager specification --
  spec overview, operations table, invariants I1-I5, pitfalls, Examples 1-3,
  key-question answers, details, data-structure table, algorithm notes and
  the eviction trace.

Modules:

* :mod:`oracle.block_manager` -- ``RefBlockManager`` (P06 spec + day31 fork/COW).
* :mod:`oracle.kv_ops`        -- ``ref_write_kv``, ``ref_copy_blocks``,
  ``ref_swap_out``, ``ref_swap_in``.
* :mod:`oracle.scheduler`     -- ``RefScheduler`` (article-130 continuous
  batching with preemption over ``RefBlockManager``).
* :mod:`oracle.attention`     -- ``ref_decode`` (fp64 gather + softmax attention)
  and ``ref_prefill`` (causal attention of an uncached suffix).
* :mod:`oracle.arithmetic`    -- the pages' memory formulas.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against values the pages print, closed forms, a library routine or brute
force, except the internal prefix-key *values* (only their equality is
observable) -- parity unpinned for those values by design.
"""

from .arithmetic import (block_bytes, blocks_needed, contiguous_tables,
                         kv_bytes_per_token, kv_cache_bytes, tail_waste_tokens)
from .attention import ref_decode, ref_decode_one, ref_prefill
from .block_manager import OutOfBlocks, RefBlockManager
from .kv_ops import ref_copy_blocks, ref_swap_in, ref_swap_out, ref_write_kv
from .scheduler import RefScheduler

__all__ = [
    "OutOfBlocks", "RefBlockManager", "ref_write_kv", "ref_copy_blocks",
    "ref_swap_out", "ref_swap_in", "RefScheduler",
    "ref_decode", "ref_decode_one", "ref_prefill", "kv_cache_bytes",
    "kv_bytes_per_token", "block_bytes", "blocks_needed", "tail_waste_tokens",
    "contiguous_tables",
]

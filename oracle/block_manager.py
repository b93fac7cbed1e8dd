"""Reference block manager (test infrastructure; see oracle/__init__).

Follows the "P06 · BlockManager: paged KV + prefix cache" page: its
data-structure table (free deque, ref list, block_hash, hash_to_block,
evictable OrderedDict, per-sequence tables/tokens/hashes/cached), its
operations table (allocate / append_slot / free, with the read steps, the
ordered write steps and the single raise point of each), its algorithm notes
(``_take_block`` helper, append order, reverse free) and its details section
(fixed chain sentinel, contiguous matching that stops at the first miss,
coarse ``can_allocate``, prefix cache switchable off, duplicate-content rule).
Fork and copy-on-write append come from the "day31" page, toy COW append
(``fork_sequence``, ``ensure_private_last_block``, ``append_with_cow``).

Readings where the pages are silent or disagree (each also listed in the
design notes):

* The page's ``free`` deque is called ``free_list`` here (the name ``free``
  is the operation).
* Free-list order is FIFO (P06 Example 1 and its data-structure table use a
  deque with popleft/append); the LIFO ``pop()`` of the other two pages'
  toy allocators is superseded.
* Prefix identity: the page hashes ``(h_{i-1}, tuple(block tokens))`` with a
  fixed sentinel for h_{-1}.  Here the "hash" is an exact interned key: the
  pair (parent key, block tokens) is mapped to a small integer the first time
  it is seen, so two blocks get the same key iff their whole prefixes are
  identical.  This is the hash chain with collisions made impossible; key
  values themselves are never compared with the library's.
* Registering a key that is already mapped keeps the old mapping but still
  records the key on the new block (P06 details, duplicate-content rule, and
  the pitfall about deleting another block's mapping on eviction).
* COW (day31): when append_slot lands in a last block whose ref > 1, a new
  block is taken first (the raise point), the old block is decref'd, the
  table's last entry is replaced and the pair (old, new) is reported so the
  caller copies the block's bytes.  A fork copies the parent's table, tokens,
  chain and cached count and increfs every block.
* allocate of an existing sequence, or append/fork of an unknown one, raises
  ``KeyError``/``ValueError``; free of an unknown sequence is a no-op (as the
  article-130 ``BlockAllocator.free`` ignores unknown ids).  allocate with no
  tokens is allowed and yields an empty table.
* Preemption ("qaqbuyan.com article 130", continuous-batching scheduler,
  ``_preempt_request``): the victim's blocks are copied to host memory and
  freed.  ``swap_out`` returns the table whose blocks the caller copies and
  frees it exactly as ``free`` does, keeping the token list.  The page does
  not show the way back; ``swap_in`` is read as the P06 allocate over the
  saved tokens, so full prefix blocks that are still registered come back as
  hits (their KV never left the GPU) and only the blocks from the first
  non-hit on are restored from host memory.  A swapped sequence holds no
  blocks; its id cannot be allocated or forked onto, and ``free`` drops its
  saved tokens.
"""

from collections import OrderedDict, deque
import math


class OutOfBlocks(Exception):
    """Raised when no free or evictable block is left (P06 spec overview)."""


class RefBlockManager:
    """Block manager with refcounts, chained prefix keys and an LRU pool."""

    def __init__(self, num_blocks: int, block_size: int,
                 enable_prefix_cache: bool = True):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.bs = block_size
        self.enable_prefix_cache = bool(enable_prefix_cache)
        # P06 data-structure table.
        self.free_list = deque(range(num_blocks))  # no-hash free blocks, FIFO
        self.ref = [0] * num_blocks
        self.block_hash = [None] * num_blocks     # key registered on a block
        self.hash_to_block = {}
        self.evictable = OrderedDict()            # ref==0 with a key; LRU order
        self.tables = {}
        self.tokens = {}
        self.hashes = {}
        self.cached = {}
        # Preempted sequences: id -> token list (no blocks held).
        self.swapped = {}
        # Exact prefix keys: (parent key, block tokens) -> integer.
        self._intern = {}

    # ----- prefix keys ---------------------------------------------------
    def _key(self, parent, block_tokens):
        """Key of a full block given its parent's key (None for block 0)."""
        pair = (parent, tuple(block_tokens))
        key = self._intern.get(pair)
        if key is None:
            key = len(self._intern)
            self._intern[pair] = key
        return key

    def _chain(self, tokens):
        """Keys of the len//bs full blocks of a prompt, chained from None."""
        keys = []
        parent = None
        for i in range(len(tokens) // self.bs):
            parent = self._key(parent, tokens[i * self.bs:(i + 1) * self.bs])
            keys.append(parent)
        return keys

    # ----- helpers -------------------------------------------------------
    @property
    def num_free_blocks(self) -> int:
        """Free plus evictable blocks (P06 spec overview)."""
        return len(self.free_list) + len(self.evictable)

    def can_allocate(self, num_tokens: int) -> bool:
        """Coarse check ceil(n/bs) <= num_free_blocks (P06 details)."""
        return math.ceil(num_tokens / self.bs) <= self.num_free_blocks

    def _take_block(self) -> int:
        """Free list first (popleft); else evict the oldest evictable block
        and drop its registration in both places; else raise.  The taken
        block gets ref 1 (P06 algorithm notes)."""
        if self.free_list:
            b = self.free_list.popleft()
        elif self.evictable:
            b, _ = self.evictable.popitem(last=False)
            key = self.block_hash[b]
            if self.hash_to_block.get(key) == b:
                del self.hash_to_block[key]
            self.block_hash[b] = None
        else:
            raise OutOfBlocks("no free or evictable block")
        self.ref[b] = 1
        return b

    def _register(self, b, key):
        """Record key on block b; keep an existing mapping (P06 details)."""
        self.block_hash[b] = key
        self.hash_to_block.setdefault(key, b)

    # ----- operations ----------------------------------------------------
    def allocate(self, seq, tokens):
        """P06 operations table, allocate row: steps 1-3 read, 4-7 write."""
        if seq in self.tables or seq in self.swapped:
            raise ValueError(f"sequence {seq!r} already allocated")
        tokens = list(tokens)
        n = len(tokens)
        # (1) chain keys for the full blocks only.
        keys = self._chain(tokens) if self.enable_prefix_cache else []
        # (2) contiguous lookups over the first (len-1)//bs blocks.
        hits = []
        if self.enable_prefix_cache:
            for i in range(max(0, (n - 1) // self.bs)):
                b = self.hash_to_block.get(keys[i])
                if b is None:
                    break
                hits.append(b)
        # (3) exact capacity: hits that sit in the evictable pool are no
        #     longer available for new blocks.
        new_needed = math.ceil(n / self.bs) - len(hits)
        revived = sum(1 for b in hits if self.ref[b] == 0)
        if new_needed > self.num_free_blocks - revived:
            raise OutOfBlocks(
                f"need {new_needed} new blocks, {self.num_free_blocks - revived} usable")
        # (4) hits: leave the evictable pool if ref==0, then ref+1.
        table = []
        for b in hits:
            if self.ref[b] == 0:
                del self.evictable[b]
            self.ref[b] += 1
            table.append(b)
        # (5) remaining blocks, in logical order.
        for _ in range(new_needed):
            table.append(self._take_block())
        # (6) register the full blocks that were not hits.
        for i in range(len(hits), len(keys)):
            self._register(table[i], keys[i])
        # (7) save the sequence's four records.
        self.tables[seq] = table
        self.tokens[seq] = tokens
        self.hashes[seq] = keys
        self.cached[seq] = len(hits) * self.bs
        return list(table)

    def append_slot(self, seq, token):
        """P06 append_slot with day31 COW merged in.

        Returns (slot, cow) where cow is None or the pair (src, dst) whose
        bytes the caller must copy before writing the new token.
        """
        table = self.tables[seq]
        toks = self.tokens[seq]
        pos = len(toks)
        cow = None
        # (1) take a block first: the only step that may raise.
        if pos // self.bs == len(table):
            table.append(self._take_block())
        else:
            old = table[-1]
            if self.ref[old] > 1:
                new = self._take_block()
                self.ref[old] -= 1          # stays >= 1: no pool movement
                table[-1] = new
                cow = (old, new)
        # (2) then the token.
        toks.append(token)
        # (3) a block that just filled is keyed with the chain tail as parent.
        if self.enable_prefix_cache and (pos + 1) % self.bs == 0:
            chain = self.hashes[seq]
            parent = chain[-1] if chain else None
            key = self._key(parent, toks[pos + 1 - self.bs:pos + 1])
            chain.append(key)
            self._register(table[pos // self.bs], key)
        return self.slot(seq, pos), cow

    def fork(self, parent, child):
        """day31 fork_sequence: share every block of the parent (ref+1)."""
        if child in self.tables or child in self.swapped:
            raise ValueError(f"sequence {child!r} already exists")
        table = self.tables[parent]
        self.tables[child] = list(table)
        self.tokens[child] = list(self.tokens[parent])
        self.hashes[child] = list(self.hashes[parent])
        self.cached[child] = self.cached[parent]
        for b in table:
            self.ref[b] += 1

    def free(self, seq):
        """P06 free: reverse walk, ref-1; at 0 a keyed block goes to the
        newest end of the evictable pool, any other block to the free list."""
        self.swapped.pop(seq, None)
        if seq not in self.tables:
            return
        for b in reversed(self.tables[seq]):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                if self.block_hash[b] is not None:
                    self.evictable[b] = None
                else:
                    self.free_list.append(b)
        del self.tables[seq], self.tokens[seq], self.hashes[seq], self.cached[seq]

    # ----- preemption ----------------------------------------------------
    def swap_out(self, seq):
        """article-130 ``_preempt_request``: the caller copies the returned
        blocks (logical order) to host memory; they are then freed in the
        P06 reverse order and the sequence keeps only its tokens."""
        table = list(self.tables[seq])          # KeyError: unknown sequence
        tokens = list(self.tokens[seq])
        self.free(seq)
        self.swapped[seq] = tokens
        return table

    def swap_in(self, seq):
        """Bring a preempted sequence back through the P06 allocate (all or
        nothing: OutOfBlocks leaves it swapped and the state unchanged).
        Returns (table, first_restore): logical blocks before first_restore
        were prefix hits whose KV is still on the GPU; the caller restores
        the host copies of blocks first_restore.. into table[first_restore:]."""
        tokens = self.swapped.pop(seq)          # KeyError: not swapped out
        try:
            table = self.allocate(seq, tokens)
        except OutOfBlocks:
            self.swapped[seq] = tokens
            raise
        return table, self.cached[seq] // self.bs

    # ----- queries -------------------------------------------------------
    def slot(self, seq, pos) -> int:
        """slot = table[pos // bs] * bs + pos % bs (P06 spec overview)."""
        if not 0 <= pos < len(self.tokens[seq]):
            raise IndexError(f"pos {pos} out of range")
        return self.tables[seq][pos // self.bs] * self.bs + pos % self.bs

    def num_cached_tokens(self, seq) -> int:
        return self.cached[seq]

    def seq_len(self, seq) -> int:
        return len(self.tokens[seq])

    def get_table(self, seq):
        return list(self.tables[seq])

    def dump(self):
        """Observable state, for comparison with another implementation."""
        return {
            "ref": list(self.ref),
            "has_hash": [k is not None for k in self.block_hash],
            "free": list(self.free_list),
            "evictable": list(self.evictable),
            "num_free_blocks": self.num_free_blocks,
            "tables": {s: list(t) for s, t in self.tables.items()},
            "lens": {s: len(t) for s, t in self.tokens.items()},
            "cached": dict(self.cached),
            "swapped": {s: len(t) for s, t in self.swapped.items()},
        }

    def check_invariants(self):
        """P06 invariants I1-I5; raises AssertionError on a violation."""
        free_set, evict_set = set(self.free_list), set(self.evictable)
        # I1: disjoint, all ref==0, sizes sum to num_free_blocks.
        assert len(free_set) == len(self.free_list), "I1: duplicate in free list"
        assert not (free_set & evict_set), "I1: free and evictable overlap"
        assert all(self.ref[b] == 0 for b in free_set | evict_set), "I1: ref!=0"
        assert self.num_free_blocks == len(self.free_list) + len(self.evictable)
        # I2: evictable <=> ref==0 and keyed.
        for b in range(self.num_blocks):
            expect = self.ref[b] == 0 and self.block_hash[b] is not None
            assert (b in evict_set) == expect, f"I2: block {b}"
        # I3: hash_to_block[h] == b  =>  block_hash[b] == h.
        for key, b in self.hash_to_block.items():
            assert self.block_hash[b] == key, f"I3: key {key} block {b}"
        # I4: ref == number of tables holding the block; no block is lost.
        count = [0] * self.num_blocks
        for t in self.tables.values():
            assert len(set(t)) == len(t), "a table repeats a block"
            for b in t:
                count[b] += 1
        assert count == self.ref, "I4: ref != table count"
        held = sum(1 for c in count if c > 0)
        assert held + self.num_free_blocks == self.num_blocks, "I4: leak"
        # I5: cached is a multiple of bs and below len (for a non-empty seq).
        for s, c in self.cached.items():
            n = len(self.tokens[s])
            assert c % self.bs == 0, "I5: cached % bs"
            assert c < n or (n == 0 and c == 0), "I5: cached >= len"
        # A swapped-out sequence holds no blocks.
        assert not (set(self.swapped) & set(self.tables)), "swapped seq holds blocks"
        # Tables are tight: exactly ceil(len/bs) blocks.
        for s, t in self.tables.items():
            assert len(t) == math.ceil(len(self.tokens[s]) / self.bs)

"""Pins the oracle block manager to what the pages fix.

Sources: the "P06 · BlockManager: paged KV + prefix cache" page (Examples
1-3, the eviction trace, invariants I1-I5, the pitfalls list, key-question
answers, self-check) and the "day31" page (block-count script, fork/COW).
Each pitfall is planted in a subclass of the oracle (on the CPU) and must be
caught by at least one of these pins.
"""

import copy
import random

import pytest

from oracle import OutOfBlocks, RefBlockManager, contiguous_tables, tail_waste_tokens
from tests.bm_steps import run_steps

GOLDEN_SCRIPTS = ["bm_example1.json", "bm_example2.json", "bm_example3.json",
                  "bm_eviction_trace.json", "bm_swap_nocache.json", "bm_swap_prefix.json"]


def make(spec, cls=RefBlockManager):
    return cls(spec["num_blocks"], spec["block_size"], spec["enable_prefix_cache"])


@pytest.mark.parametrize("name", GOLDEN_SCRIPTS)
def test_golden_scripts(golden, name):
    spec = golden(name)
    run_steps(make(spec), spec, OutOfBlocks)


def test_block_count_script(golden):
    """day31 block-count script: consecutive allocation of [7,16,31,48,63]."""
    spec = golden("block_count_script.json")
    bm = RefBlockManager(64, spec["block_size"], enable_prefix_cache=False)
    tables = [bm.allocate(i, list(range(n))) for i, n in enumerate(spec["lengths"])]
    assert tables == spec["tables"]
    assert 64 - bm.num_free_blocks == spec["physical_blocks"]
    t2, used = contiguous_tables(spec["lengths"], spec["block_size"])
    assert t2 == spec["tables"] and used == spec["physical_blocks"]
    assert tail_waste_tokens(spec["lengths"], spec["block_size"]) == spec["tail_waste_tokens"]


def test_key_answer_partial_block_not_cached():
    """10 tokens at bs=4: 3 blocks, blocks 0 and 1 get keys, block 2 does not."""
    bm = RefBlockManager(8, 4)
    t = bm.allocate(1, list(range(10)))
    assert len(t) == 3
    has = bm.dump()["has_hash"]
    assert [has[b] for b in t] == [True, True, False]


def test_key_answer_last_token_never_hits():
    """8 tokens at bs=4 with both blocks cached: only (8-1)//4 = 1 hit."""
    bm = RefBlockManager(8, 4)
    bm.allocate(1, list(range(8)))
    bm.free(1)
    bm.allocate(2, list(range(8)))
    assert bm.num_cached_tokens(2) == 4


def test_key_answer_chain_depends_on_prefix():
    """Same block content after different prefixes must not hit."""
    bm = RefBlockManager(8, 2)
    bm.allocate(1, [1, 2, 7, 8, 0])
    bm.allocate(2, [5, 6, 7, 8, 0])
    assert bm.num_cached_tokens(2) == 0
    bm.allocate(3, [1, 2, 7, 8, 9])
    assert bm.num_cached_tokens(3) == 4


def test_key_answer_hit_ref_positive_vs_zero():
    """A ref>0 hit only increments; a ref==0 hit leaves the pool and lowers
    num_free_blocks by one."""
    bm = RefBlockManager(8, 2)
    bm.allocate(1, [1, 2, 3])
    nf = bm.num_free_blocks
    bm.allocate(2, [1, 2, 4])            # hit on block 0 with ref 1
    assert bm.ref[0] == 2 and bm.num_free_blocks == nf - 1   # only the new block
    bm.free(1)
    bm.free(2)
    assert 0 in bm.evictable
    nf = bm.num_free_blocks
    bm.allocate(3, [1, 2, 5])            # hit on block 0 with ref 0
    assert bm.ref[0] == 1 and 0 not in bm.evictable
    assert bm.num_free_blocks == nf - 2  # the revived hit + the new block


def test_key_answer_eviction_clears_both_records():
    bm = RefBlockManager(2, 2)
    bm.allocate(1, [1, 2, 3])
    bm.free(1)
    key = bm.block_hash[0]
    bm.allocate(2, [9, 9, 9, 9])         # evicts block 0
    assert bm.block_hash[0] != key and key not in bm.hash_to_block


def test_self_check_shared_free():
    """Share a block between two sequences and free one: num_free_blocks
    rises only by the unshared blocks."""
    bm = RefBlockManager(8, 2)
    bm.allocate(1, [1, 2, 3, 4, 5])      # blocks 0,1,2
    bm.allocate(2, [1, 2, 3, 4, 6])      # hits 0,1; new 3
    nf = bm.num_free_blocks
    bm.free(1)
    assert bm.num_free_blocks == nf + 1  # only block 2
    bm.free(2)
    assert bm.num_free_blocks == 8


def test_config1_prefix_cache_tables():
    """Five prompts that are prefixes of one 63-token stream, bs 16, 64
    blocks, allocated in order (derived from the P06 rules)."""
    stream = list(range(100, 163))
    bm = RefBlockManager(64, 16)
    tables = [bm.allocate(i, stream[:n]) for i, n in enumerate([7, 16, 31, 48, 63])]
    assert tables == [[0], [1], [1, 2], [1, 3, 4], [1, 3, 4, 5]]
    assert [bm.num_cached_tokens(i) for i in range(5)] == [0, 0, 16, 16, 48]
    assert bm.ref[:6] == [1, 4, 1, 2, 2, 1]
    assert bm.num_free_blocks == 58
    bm.check_invariants()


def test_prefix_cache_off():
    """enable_prefix_cache=False: nothing keyed, cached always 0, everything
    returns to the free list."""
    bm = RefBlockManager(8, 2, enable_prefix_cache=False)
    bm.allocate(1, [1, 2, 3, 4, 5])
    bm.free(1)
    bm.allocate(2, [1, 2, 3, 4, 5])
    assert bm.num_cached_tokens(2) == 0
    assert not any(bm.dump()["has_hash"]) and not bm.evictable


def test_append_registers_full_block_and_is_hit():
    """A block filled by append_slot is keyed with the chain tail as parent
    and hit by a later allocate (multi-turn reuse)."""
    bm = RefBlockManager(8, 2)
    bm.allocate(1, [1])
    bm.append_slot(1, 2)                 # fills block 0 via append
    bm.append_slot(1, 3)
    bm.append_slot(1, 4)                 # fills block 1
    bm.allocate(2, [1, 2, 3, 4, 5])
    assert bm.num_cached_tokens(2) == 4
    assert bm.get_table(2)[:2] == bm.get_table(1)


def test_fork_and_cow():
    """day31 fork + COW: a fork shares every block; appending into a shared,
    partly filled last block takes a new block first, decrefs the old one and
    reports (old, new); the last holder writes in place."""
    bm = RefBlockManager(16, 4)
    bm.allocate(1, [1, 2, 3, 4, 5, 6])   # blocks 0, 1 (1 partly filled)
    bm.fork(1, 2)
    bm.fork(1, 3)
    assert bm.ref[:2] == [3, 3]
    slot, cow = bm.append_slot(1, 7)
    assert cow == (1, 2) and slot == 2 * 4 + 2
    assert bm.ref[1] == 2 and bm.get_table(1) == [0, 2]
    slot, cow = bm.append_slot(2, 8)
    assert cow == (1, 3) and bm.ref[1] == 1
    slot, cow = bm.append_slot(3, 9)     # now the only holder: no copy
    assert cow is None and slot == 1 * 4 + 2
    bm.check_invariants()
    for s in (1, 2, 3):
        bm.free(s)
    assert bm.num_free_blocks == 16
    bm.check_invariants()


def test_fork_full_last_block_no_cow():
    bm = RefBlockManager(8, 2)
    bm.allocate(1, [1, 2, 3, 4])
    bm.fork(1, 2)
    _, cow = bm.append_slot(2, 5)
    assert cow is None and bm.get_table(2)[:2] == [0, 1] and len(bm.get_table(2)) == 3


def test_empty_allocate_and_unknown_ids():
    bm = RefBlockManager(4, 2)
    assert bm.allocate(1, []) == []
    assert bm.num_cached_tokens(1) == 0
    slot, _ = bm.append_slot(1, 5)
    assert slot == 0
    with pytest.raises(ValueError):
        bm.allocate(1, [1])
    with pytest.raises(KeyError):
        bm.append_slot(99, 1)
    bm.free(99)                          # no-op
    with pytest.raises(IndexError):
        bm.slot(1, 1)


def test_can_allocate_is_coarse():
    """can_allocate ignores hits; allocate's own check is exact (Example 3
    state: 3 usable blocks, but a 7-token prompt that hits two evictable
    blocks still fails)."""
    bm = RefBlockManager(3, 2)
    bm.allocate(1, [1, 2, 3, 4, 5])
    bm.free(1)
    assert bm.can_allocate(6) and not bm.can_allocate(7)
    with pytest.raises(OutOfBlocks):
        bm.allocate(2, [1, 2, 3, 4, 5, 6, 7])


def _state(bm):
    return copy.deepcopy({k: v for k, v in vars(bm).items() if k != "_intern"})


def random_stream(bm, rng, n_ops, alphabet=3, max_prompt=12, check=True):
    """Seeded random operation stream; checks I1-I5 after every op and that a
    failing operation leaves the state unchanged."""
    live, swapped, next_id = [], [], 1
    stats = {"oob": 0, "hits": 0, "cow": 0, "swap_hits": 0}
    for _ in range(n_ops):
        r = rng.random()
        before = _state(bm) if check else None
        try:
            if r < 0.25 or not live:
                n = rng.randrange(0, max_prompt)
                toks = [rng.randrange(alphabet) for _ in range(n)]
                bm.allocate(next_id, toks)
                stats["hits"] += bm.num_cached_tokens(next_id) > 0
                live.append(next_id)
                next_id += 1
            elif r < 0.55:
                s = rng.choice(live)
                _, cow = bm.append_slot(s, rng.randrange(alphabet))
                stats["cow"] += cow is not None
            elif r < 0.67:
                bm.fork(rng.choice(live), next_id)
                live.append(next_id)
                next_id += 1
            elif r < 0.75:
                s = live.pop(rng.randrange(len(live)))
                table = bm.swap_out(s)
                assert len(table) == -(-len(bm.swapped[s]) // bm.bs)
                swapped.append(s)
            elif r < 0.83 and swapped:
                s = swapped[rng.randrange(len(swapped))]
                table, first = bm.swap_in(s)
                swapped.remove(s)
                live.append(s)
                assert first * bm.bs == bm.num_cached_tokens(s)
                stats["swap_hits"] += first > 0
            else:
                s = live.pop(rng.randrange(len(live)))
                bm.free(s)
        except OutOfBlocks:
            stats["oob"] += 1
            if check:
                assert _state(bm) == before, "state changed by a failed op"
        if check:
            bm.check_invariants()
    for s in live + swapped:
        bm.free(s)
    bm.check_invariants()
    assert not bm.swapped
    assert bm.num_free_blocks == bm.num_blocks
    return stats


@pytest.mark.parametrize("seed,bs,nblocks", [(0, 2, 8), (1, 4, 12), (2, 2, 5), (3, 1, 6)])
def test_random_stream_invariants(seed, bs, nblocks):
    stats = random_stream(RefBlockManager(nblocks, bs), random.Random(seed), 3000)
    # The stream must actually reach the interesting cases (with bs == 1 no
    # block is ever partly filled, so no copy-on-write can happen).
    assert stats["oob"] > 0 and stats["hits"] > 0 and stats["swap_hits"] > 0
    assert (stats["cow"] > 0) == (bs > 1)


# ---- pitfalls planted in the oracle: each must be caught -----------------
# Each mutant is the oracle with exactly one pitfall of the P06 page planted.

def _allocate(bm, seq, tokens, limit, exact_check=True, remove_revived=True):
    """The oracle's allocate with switchable pitfalls (test-only copy)."""
    tokens = list(tokens)
    keys = bm._chain(tokens)
    hits = []
    for i in range(max(0, limit(len(tokens), bm.bs))):
        b = bm.hash_to_block.get(keys[i])
        if b is None:
            break
        hits.append(b)
    new_needed = -(-len(tokens) // bm.bs) - len(hits)
    usable = bm.num_free_blocks
    if exact_check:
        usable -= sum(bm.ref[b] == 0 for b in hits)
    if new_needed > usable:
        raise OutOfBlocks()
    table = []
    for b in hits:
        if bm.ref[b] == 0 and remove_revived:
            del bm.evictable[b]
        bm.ref[b] += 1
        table.append(b)
    table += [bm._take_block() for _ in range(new_needed)]
    for i in range(len(hits), len(keys)):
        bm._register(table[i], keys[i])
    bm.tables[seq], bm.tokens[seq] = table, tokens
    bm.hashes[seq], bm.cached[seq] = keys, len(hits) * bm.bs
    return list(table)


class HashPartialBlock(RefBlockManager):
    """Pitfall: the partly filled last block also gets a key."""
    def _chain(self, tokens):
        keys, parent = [], None
        for i in range(-(-len(tokens) // self.bs)):
            parent = self._key(parent, tokens[i * self.bs:(i + 1) * self.bs])
            keys.append(parent)
        return keys


class MatchLimitLenDivBs(RefBlockManager):
    """Pitfall: up to len//bs blocks may be matched."""
    def allocate(self, seq, tokens):
        return _allocate(self, seq, tokens, lambda n, bs: n // bs)


class CoarseCapacityCheck(RefBlockManager):
    """Pitfall: allocate uses the coarse check (ignores revived hits)."""
    def allocate(self, seq, tokens):
        return _allocate(self, seq, tokens, lambda n, bs: (n - 1) // bs, exact_check=False)


class ReviveWithoutRemoval(RefBlockManager):
    """Pitfall: a ref==0 hit is revived but left in the evictable pool."""
    def allocate(self, seq, tokens):
        return _allocate(self, seq, tokens, lambda n, bs: (n - 1) // bs, remove_revived=False)


class OtherSentinelOnAppend(RefBlockManager):
    """Pitfall: append_slot chains block 0 from a different sentinel."""
    def append_slot(self, seq, token):
        table, toks = self.tables[seq], self.tokens[seq]
        pos = len(toks)
        if pos // self.bs == len(table):
            table.append(self._take_block())
        toks.append(token)
        if (pos + 1) % self.bs == 0:
            chain = self.hashes[seq]
            parent = chain[-1] if chain else "other-sentinel"
            key = self._key(parent, toks[pos + 1 - self.bs:pos + 1])
            chain.append(key)
            self._register(table[pos // self.bs], key)
        return self.slot(seq, pos), None


class TokenBeforeBlock(RefBlockManager):
    """Pitfall: append_slot appends the token before taking the block."""
    def append_slot(self, seq, token):
        table, toks = self.tables[seq], self.tokens[seq]
        pos = len(toks)
        toks.append(token)
        if pos // self.bs == len(table):
            table.append(self._take_block())
        return self.slot(seq, pos), None


class UnconditionalUnregister(RefBlockManager):
    """Pitfall: eviction deletes hash_to_block[h] even if it maps elsewhere."""
    def _take_block(self):
        if not self.free_list and self.evictable:
            b, _ = self.evictable.popitem(last=False)
            self.hash_to_block.pop(self.block_hash[b], None)
            self.block_hash[b] = None
            self.ref[b] = 1
            return b
        return super()._take_block()


class ForwardFree(RefBlockManager):
    """Pitfall: free walks the table front to back."""
    def free(self, seq):
        if seq not in self.tables:
            return
        for b in self.tables[seq]:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                if self.block_hash[b] is not None:
                    self.evictable[b] = None
                else:
                    self.free_list.append(b)
        del self.tables[seq], self.tokens[seq], self.hashes[seq], self.cached[seq]


class SwapInWithoutHits(RefBlockManager):
    """Mistake: swap_in restores every block, ignoring still-cached prefix
    blocks (fresh blocks for all, nothing revived)."""
    def swap_in(self, seq):
        tokens = self.swapped.pop(seq)
        table = [self._take_block() for _ in range(-(-len(tokens) // self.bs))]
        self.tables[seq], self.tokens[seq] = table, tokens
        self.hashes[seq], self.cached[seq] = self._chain(tokens), 0
        return list(table), 0


class SwapOutForwardFree(RefBlockManager):
    """Mistake: swap_out releases the table front to back."""
    def swap_out(self, seq):
        table = list(self.tables[seq])
        self.swapped[seq] = list(self.tokens[seq])
        ForwardFree.free(self, seq)
        return table


class SwapInNotAtomic(RefBlockManager):
    """Mistake: a failed swap_in loses the saved tokens."""
    def swap_in(self, seq):
        tokens = self.swapped.pop(seq)
        table = self.allocate(seq, tokens)
        return table, self.cached[seq] // self.bs


def partial_block_pin(cls, golden):
    bm = cls(8, 4)
    t = bm.allocate(1, list(range(10)))
    has = bm.dump()["has_hash"]
    assert [has[b] for b in t] == [True, True, False]


def sentinel_pin(cls, golden):
    bm = cls(8, 2)
    bm.allocate(1, [1])
    bm.append_slot(1, 2)             # block 0 fills through append
    bm.allocate(2, [1, 2, 3])
    assert bm.num_cached_tokens(2) == 2, "append-filled block 0 must be hit"


def duplicate_unregister_pin(cls, golden):
    bm = cls(5, 2)
    bm.allocate(1, [1, 2, 3])        # blocks 0, 1; key (1,2) maps to block 0
    bm.allocate(2, [1, 2])           # no hit allowed; block 2 gets the same key
    bm.free(2)                       # block 2 -> evictable
    bm.allocate(3, [9, 9, 9])        # takes free blocks 3, 4
    bm.allocate(4, [8])              # evicts block 2 (the duplicate)
    bm.free(4)
    bm.allocate(5, [1, 2, 5])        # must still hit block 0
    assert bm.num_cached_tokens(5) == 2


def append_atomicity_pin(cls, golden):
    bm = cls(1, 2)
    bm.allocate(1, [1, 2])
    before = _state(bm)
    with pytest.raises(OutOfBlocks):
        bm.append_slot(1, 3)
    assert _state(bm) == before


def golden_pin(name):
    def pin(cls, golden):
        spec = golden(name)
        run_steps(make(spec, cls), spec, OutOfBlocks)
    return pin


PITFALLS = [
    (HashPartialBlock, partial_block_pin),
    (MatchLimitLenDivBs, golden_pin("bm_example2.json")),
    (OtherSentinelOnAppend, sentinel_pin),
    (UnconditionalUnregister, duplicate_unregister_pin),
    (ForwardFree, golden_pin("bm_example2.json")),
    (CoarseCapacityCheck, golden_pin("bm_example3.json")),
    (ReviveWithoutRemoval, golden_pin("bm_example3.json")),
    (TokenBeforeBlock, append_atomicity_pin),
    (SwapInWithoutHits, golden_pin("bm_swap_prefix.json")),
    (SwapOutForwardFree, golden_pin("bm_swap_nocache.json")),
    (SwapInNotAtomic, golden_pin("bm_swap_nocache.json")),
]


@pytest.mark.parametrize("mutant,pin", PITFALLS, ids=[m.__name__ for m, _ in PITFALLS])
def test_pitfall_is_caught(mutant, pin, golden):
    pin(RefBlockManager, golden)            # the oracle passes the pin ...
    with pytest.raises((AssertionError, OutOfBlocks, KeyError)):
        pin(mutant, golden)                 # ... the planted mistake fails it

"""Python view of the library's host block manager (pa_bm_* calls).

Argument marshalling only: every decision (matching, capacity, eviction,
copy-on-write) is made by the C++ block manager behind the C ABI.
"""

import ctypes

import numpy as np

from ._lib import P_i8, P_i32, P_i64, PagedKVError, check, lib


def _i32p(a):
    return a.ctypes.data_as(P_i32)


class BlockManager:
    """Refcounted paged-KV block manager with a prefix cache.

    Mirrors the "P06 · BlockManager" page's interface (allocate,
    append_slot, free, slot, num_free_blocks, can_allocate,
    num_cached_tokens), the "day31" fork, and swap-out/in of a preempted
    sequence ("qaqbuyan.com article 130", continuous-batching scheduler).
    """

    def __init__(self, num_blocks, block_size, enable_prefix_cache=True):
        self._h = lib().pa_bm_create(int(num_blocks), int(block_size), int(bool(enable_prefix_cache)))
        if not self._h:
            raise ValueError(lib().pa_last_error().decode())
        self.num_blocks = int(num_blocks)
        self.bs = int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            lib().pa_bm_destroy(h)
            self._h = None

    # ---- operations -----------------------------------------------------
    def allocate(self, seq, tokens):
        toks = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
        cap = -(-len(toks) // self.bs)
        table = np.empty(max(cap, 1), dtype=np.int32)
        n = ctypes.c_int32()
        check(lib().pa_bm_allocate(self._h, int(seq), _i32p(toks), len(toks), _i32p(table), cap,
                                   ctypes.byref(n)))
        return table[:n.value].tolist()

    def append_slot(self, seq, token):
        """Returns (slot, cow) with cow None or the (src, dst) block pair."""
        slot, src, dst = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        check(lib().pa_bm_append_slot(self._h, int(seq), int(token), ctypes.byref(slot),
                                      ctypes.byref(src), ctypes.byref(dst)))
        cow = None if src.value < 0 else (src.value, dst.value)
        return slot.value, cow

    def append_slots(self, seqs, tokens):
        """Batched append_slot.  Returns (slots int64 [B], cow pairs int32
        [n_cow, 2]).  On the first failing append it raises the library's
        error with the completed appends attached, since they stay done:
        ``err.n_done``, ``err.slots`` (their slots) and ``err.cow_pairs``
        (their copy-on-write pairs, which still have to be copied)."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        B = len(seqs)
        slots = np.empty(B, dtype=np.int64)
        pairs = np.empty((max(B, 1), 2), dtype=np.int32)
        ncow, ndone = ctypes.c_int32(), ctypes.c_int32()
        st = lib().pa_bm_append_slots(self._h, seqs.ctypes.data_as(P_i64), _i32p(tokens), B,
                                      slots.ctypes.data_as(P_i64), _i32p(pairs),
                                      ctypes.byref(ncow), ctypes.byref(ndone))
        try:
            check(st)
        except PagedKVError as err:
            err.n_done = ndone.value
            err.slots = slots[:ndone.value].copy()
            err.cow_pairs = pairs[:ncow.value].copy()
            raise
        return slots, pairs[:ncow.value].copy()

    def fork(self, parent, child):
        check(lib().pa_bm_fork(self._h, int(parent), int(child)))

    def free(self, seq):
        check(lib().pa_bm_free(self._h, int(seq)))

    def fork_batch(self, parents, children):
        """fork(parents[i], children[i]) in order under one lock."""
        p = np.ascontiguousarray(parents, dtype=np.int64)
        c = np.ascontiguousarray(children, dtype=np.int64)
        assert p.shape == c.shape
        check(lib().pa_bm_fork_batch(self._h, p.ctypes.data_as(P_i64), c.ctypes.data_as(P_i64),
                                     len(p), None))

    def free_batch(self, seqs):
        """free(s) for every s, in order, under one lock."""
        a = np.ascontiguousarray(seqs, dtype=np.int64)
        check(lib().pa_bm_free_batch(self._h, a.ctypes.data_as(P_i64), len(a)))

    def swap_out(self, seq):
        """Preempt ``seq``: returns its table (the blocks whose bytes go to
        host memory, logical order) and frees them; the tokens are kept."""
        cap = -(-self.seq_len(seq) // self.bs)
        table = np.empty(max(cap, 1), dtype=np.int32)
        n = ctypes.c_int32()
        check(lib().pa_bm_swap_out(self._h, int(seq), _i32p(table), cap, ctypes.byref(n)))
        return table[:n.value].tolist()

    def swap_in(self, seq):
        """Resume a swapped-out ``seq``.  Returns (table, first_restore):
        blocks table[first_restore:] need their host copies back."""
        cap = -(-dict(self.swapped()).get(int(seq), 0) // self.bs)
        table = np.empty(max(cap, 1), dtype=np.int32)
        n, first = ctypes.c_int32(), ctypes.c_int32()
        check(lib().pa_bm_swap_in(self._h, int(seq), _i32p(table), cap, ctypes.byref(n),
                                  ctypes.byref(first)))
        return table[:n.value].tolist(), first.value

    def is_swapped(self, seq):
        return lib().pa_bm_is_swapped(self._h, int(seq)) == 1

    def swapped(self):
        """[(seq, len)] of the swapped-out sequences, ascending ids."""
        n = ctypes.c_int32()
        check(lib().pa_bm_swapped(self._h, None, None, 0, ctypes.byref(n)))
        ids = np.empty(max(n.value, 1), dtype=np.int64)
        lens = np.empty(max(n.value, 1), dtype=np.int32)
        check(lib().pa_bm_swapped(self._h, ids.ctypes.data_as(P_i64), _i32p(lens), n.value,
                                  ctypes.byref(n)))
        return list(zip(ids[:n.value].tolist(), lens[:n.value].tolist()))

    # ---- queries --------------------------------------------------------
    def slot(self, seq, pos):
        out = ctypes.c_int64()
        check(lib().pa_bm_slot(self._h, int(seq), int(pos), ctypes.byref(out)))
        return out.value

    @property
    def num_free_blocks(self):
        return lib().pa_bm_num_free_blocks(self._h)

    def can_allocate(self, num_tokens):
        return bool(lib().pa_bm_can_allocate(self._h, int(num_tokens)))

    def num_cached_tokens(self, seq):
        out = ctypes.c_int32()
        check(lib().pa_bm_num_cached_tokens(self._h, int(seq), ctypes.byref(out)))
        return out.value

    def seq_len(self, seq):
        out = ctypes.c_int32()
        check(lib().pa_bm_seq_len(self._h, int(seq), ctypes.byref(out)))
        return out.value

    def get_table(self, seq):
        cap = -(-self.seq_len(seq) // self.bs)
        out = np.empty(max(cap, 1), dtype=np.int32)
        n = ctypes.c_int32()
        check(lib().pa_bm_get_table(self._h, int(seq), _i32p(out), cap, ctypes.byref(n)))
        return out[:n.value].tolist()

    def seq_ids(self):
        n = lib().pa_bm_num_seqs(self._h)
        out = np.empty(max(n, 1), dtype=np.int64)
        got = ctypes.c_int32()
        check(lib().pa_bm_seq_ids(self._h, out.ctypes.data_as(P_i64), n, ctypes.byref(got)))
        return out[:got.value].tolist()

    def export_batch(self, seqs, max_blocks, pad_block=0, tables_out=None, lens_out=None):
        """Decode inputs for ``seqs``: int32 tables [B, max_blocks] padded
        with ``pad_block`` and int32 context lengths [B].  Optional output
        arrays (e.g. pinned host buffers viewed as NumPy) are filled in place."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int64)
        B = len(seqs)
        tables = tables_out if tables_out is not None else np.empty((B, max_blocks), dtype=np.int32)
        lens = lens_out if lens_out is not None else np.empty(B, dtype=np.int32)
        assert tables.dtype == np.int32 and tables.flags.c_contiguous and tables.shape == (B, max_blocks)
        assert lens.dtype == np.int32 and lens.flags.c_contiguous and lens.shape == (B,)
        check(lib().pa_bm_export_batch(self._h, seqs.ctypes.data_as(P_i64), B, _i32p(tables),
                                       int(max_blocks), int(pad_block), _i32p(lens)))
        return tables, lens

    def check_invariants(self):
        st = lib().pa_bm_check_invariants(self._h)
        if st != 0:
            raise AssertionError(lib().pa_last_error().decode())

    def dump(self):
        nb = self.num_blocks
        ref = np.empty(nb, dtype=np.int32)
        has = np.empty(nb, dtype=np.int8)
        fr = np.empty(nb, dtype=np.int32)
        ev = np.empty(nb, dtype=np.int32)
        nf, ne = ctypes.c_int32(), ctypes.c_int32()
        check(lib().pa_bm_dump(self._h, _i32p(ref), has.ctypes.data_as(P_i8), _i32p(fr),
                               ctypes.byref(nf), _i32p(ev), ctypes.byref(ne)))
        seqs = self.seq_ids()
        return {
            "ref": ref.tolist(),
            "has_hash": [bool(x) for x in has],
            "free": fr[:nf.value].tolist(),
            "evictable": ev[:ne.value].tolist(),
            "num_free_blocks": self.num_free_blocks,
            "tables": {s: self.get_table(s) for s in seqs},
            "lens": {s: self.seq_len(s) for s in seqs},
            "cached": {s: self.num_cached_tokens(s) for s in seqs},
            "swapped": dict(self.swapped()),
        }

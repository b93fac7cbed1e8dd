"""Pins the oracle's paged decode, KV write and block copy.

What fixes them on the pages ("qaqbuyan.com article 130"):
* ``paged_attention`` = gather the physical blocks named by the block table,
  concatenate, then ``scaled_dot_product_attention`` -> pinned against
  torch's SDPA in float64 on the CPU (the library routine the page calls),
  over K/V gathered block by block with ``torch.cat``;
* ``traditional_attention`` over contiguous K/V must give the same result ->
  paged == contiguous;
* the kernel listing's scale 1/sqrt(head_dim) and layout
  ``[num_blocks, block_size, heads, head_dim]``.
Closed forms and placement invariance complete the pins; planted mistakes
(wrong slot index, wrong GQA mapping, missing scale, whole-last-block length)
must each fail one of them.
"""

import numpy as np
import pytest
import torch

from oracle import (RefBlockManager, ref_copy_blocks, ref_decode, ref_decode_one,
                    ref_swap_in, ref_swap_out,
                    ref_write_kv)


def make_case(seed, lens, hq, hkv, d, bs=16, num_blocks=None, poison=True):
    """Random cache with each sequence's blocks at random physical ids."""
    rng = np.random.default_rng(seed)
    need = [-(-n // bs) for n in lens]
    num_blocks = num_blocks or sum(need) + 3
    perm = rng.permutation(num_blocks)
    tables, o = [], 0
    maxb = max(need + [1])
    for k in need:
        t = np.full(maxb, -1, dtype=np.int64)
        t[:k] = perm[o:o + k]
        o += k
        tables.append(t)
    kc = rng.standard_normal((num_blocks, bs, hkv, d))
    vc = rng.standard_normal((num_blocks, bs, hkv, d))
    if poison:
        # Slots past each length and unreferenced blocks hold NaN.
        mask = np.ones((num_blocks, bs), dtype=bool)
        for t, n in zip(tables, lens):
            for i in range(n):
                mask[t[i // bs], i % bs] = False
        kc[mask] = np.nan
        vc[mask] = np.nan
    q = rng.standard_normal((len(lens), hq, d))
    return q, kc, vc, np.stack(tables), np.asarray(lens)


def sdpa_paged(q, kc, vc, tables, lens, scale=None):
    """The page's paged_attention: torch.cat of key_blocks[table[i]] per
    logical block, then SDPA (float64, CPU, GQA by repeat-interleave)."""
    B, hq, d = q.shape
    hkv = kc.shape[2]
    out = np.zeros((B, hq, d))
    K, V = torch.from_numpy(kc), torch.from_numpy(vc)
    for b in range(B):
        n = int(lens[b])
        nblk = -(-n // kc.shape[1])
        keys = torch.cat([K[int(tables[b][i])] for i in range(nblk)], dim=0)[:n]
        vals = torch.cat([V[int(tables[b][i])] for i in range(nblk)], dim=0)[:n]
        # [n, hkv, d] -> [1, hkv, n, d]
        keys = keys.permute(1, 0, 2).unsqueeze(0).contiguous()
        vals = vals.permute(1, 0, 2).unsqueeze(0).contiguous()
        qq = torch.from_numpy(q[b]).reshape(1, hq, 1, d)
        o = torch.nn.functional.scaled_dot_product_attention(
            qq, keys, vals, scale=scale, enable_gqa=(hq != hkv))
        out[b] = o.reshape(hq, d).numpy()
    return out


CASES = [
    # (lens, hq, hkv, d): the five-length tiny batch, MHA and GQA shapes,
    # partial and exact block boundaries, length 1.
    ([7, 16, 31, 48, 63], 4, 4, 64),
    ([1, 17, 33, 100], 8, 2, 32),
    ([64, 5], 6, 3, 16),
]


@pytest.mark.parametrize("lens,hq,hkv,d", CASES)
def test_matches_library_sdpa(lens, hq, hkv, d):
    q, kc, vc, tables, lens = make_case(0, lens, hq, hkv, d)
    got = ref_decode(q, kc, vc, tables, lens)
    want = sdpa_paged(q, kc, vc, tables, lens)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("lens,hq,hkv,d", CASES)
def test_paged_equals_contiguous(lens, hq, hkv, d):
    """traditional_attention over contiguous rows == paged over a random
    table holding the same rows (paged cache filled through BM slots)."""
    rng = np.random.default_rng(1)
    bs = 16
    bm = RefBlockManager(64, bs, enable_prefix_cache=False)
    # Scramble the free list so tables are not 0, 1, 2, ...
    for i in range(64):
        bm.allocate(1000 + i, [0])
    for i in rng.permutation(64):
        bm.free(1000 + int(i))
    kc = np.full((64, bs, hkv, d), np.nan)
    vc = np.full((64, bs, hkv, d), np.nan)
    q = rng.standard_normal((len(lens), hq, d))
    conts = []
    for b, n in enumerate(lens):
        keys = rng.standard_normal((n, hkv, d))
        vals = rng.standard_normal((n, hkv, d))
        conts.append((keys, vals))
        bm.allocate(b, [])
        slots = [bm.append_slot(b, 7)[0] for _ in range(n)]
        kc, vc = ref_write_kv(kc, vc, keys, vals, slots)
    maxb = max(len(bm.get_table(b)) for b in range(len(lens)))
    tables = np.array([bm.get_table(b) + [0] * (maxb - len(bm.get_table(b)))
                       for b in range(len(lens))])
    got = ref_decode(q, kc, vc, tables, np.array(lens))
    for b, (keys, vals) in enumerate(conts):
        K = torch.from_numpy(keys).permute(1, 0, 2).unsqueeze(0).contiguous()
        V = torch.from_numpy(vals).permute(1, 0, 2).unsqueeze(0).contiguous()
        Q = torch.from_numpy(q[b]).reshape(1, hq, 1, d)
        want = torch.nn.functional.scaled_dot_product_attention(
            Q, K, V, enable_gqa=(hq != hkv)).reshape(hq, d).numpy()
        np.testing.assert_allclose(got[b], want, rtol=1e-12, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(2)
    q, kc, vc, tables, _ = make_case(3, [40], 2, 2, 8, poison=False)
    # length 1: the output is v_0 exactly.
    o = ref_decode_one(q[0, 0], kc, vc, tables[0], 1, 0, 0.3)
    assert np.array_equal(o, vc[tables[0][0], 0, 0])
    # q = 0: uniform weights -> mean of V.
    o = ref_decode_one(np.zeros(8), kc, vc, tables[0], 40, 1, 0.3)
    idx = [tables[0][t // 16] * 16 + t % 16 for t in range(40)]
    mean_v = vc.reshape(-1, 2, 8)[idx, 1].mean(axis=0)
    np.testing.assert_allclose(o, mean_v, rtol=1e-13, atol=1e-13)
    # all keys equal -> mean of V.
    kc2 = kc.copy()
    kc2[...] = rng.standard_normal(8)
    o = ref_decode_one(q[0, 1], kc2, vc, tables[0], 40, 1, 0.3)
    np.testing.assert_allclose(o, mean_v, rtol=1e-13, atol=1e-13)
    # all V rows equal -> that row.
    vc2 = vc.copy()
    row = rng.standard_normal(8)
    vc2[...] = row
    o = ref_decode_one(q[0, 1], kc, vc2, tables[0], 40, 1, 0.3)
    np.testing.assert_allclose(o, row, rtol=1e-13, atol=1e-13)
    # empty sequence: zeros (reading for a degenerate case).
    assert not ref_decode_one(q[0, 0], kc, vc, tables[0], 0, 0, 0.3).any()


def test_placement_invariance():
    """Same logical rows under two different tables: bitwise-equal output."""
    q, kc, vc, tables, lens = make_case(4, [37, 5, 16], 4, 2, 16, poison=False)
    rng = np.random.default_rng(5)
    perm = rng.permutation(kc.shape[0])          # physical block b -> perm[b]
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    tables2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1)
    a = ref_decode(q, kc, vc, tables, lens)
    b = ref_decode(q, kc2, vc2, tables2, lens)
    assert np.array_equal(a, b)


def test_write_kv_definition():
    rng = np.random.default_rng(6)
    kc = rng.standard_normal((6, 4, 2, 8)).astype(np.float16)
    vc = rng.standard_normal((6, 4, 2, 8)).astype(np.float16)
    kn = rng.standard_normal((3, 2, 8)).astype(np.float16)
    vn = rng.standard_normal((3, 2, 8)).astype(np.float16)
    slots = [5, -1, 22]                      # -1: skipped (out of range)
    k2, v2 = ref_write_kv(kc, vc, kn, vn, slots)
    kf, k2f = kc.reshape(24, 2, 8), k2.reshape(24, 2, 8)
    assert np.array_equal(k2f[5], kn[0]) and np.array_equal(k2f[22], kn[2])
    assert np.array_equal(v2.reshape(24, 2, 8)[5], vn[0])
    others = [s for s in range(24) if s not in (5, 22)]
    assert np.array_equal(k2f[others], kf[others])
    assert np.array_equal(kc.reshape(24, 2, 8), kf)    # input untouched
    with pytest.raises(AssertionError):
        ref_write_kv(kc, vc, kn, vn, [3, 3, 4])


def test_copy_blocks_definition():
    rng = np.random.default_rng(7)
    ks = [rng.standard_normal((5, 4, 2, 3)) for _ in range(2)]
    vs = [rng.standard_normal((5, 4, 2, 3)) for _ in range(2)]
    k2, v2 = ref_copy_blocks(ks, vs, [(1, 3), (0, 4)])
    for layer in range(2):
        assert np.array_equal(k2[layer][3], ks[layer][1])
        assert np.array_equal(v2[layer][4], vs[layer][0])
        assert np.array_equal(k2[layer][:3], ks[layer][:3])
    with pytest.raises(AssertionError):
        ref_copy_blocks(ks, vs, [(1, 3), (2, 3)])
    with pytest.raises(AssertionError):
        ref_copy_blocks(ks, vs, [(1, 3), (3, 4)])


def test_swap_copies_definition():
    """Preemption copies (article 130, scheduler, _preempt_request): the host
    record of list entry i, layer l is K_l/V_l of block i, and restoring it
    into other blocks reproduces those bytes there and nowhere else."""
    rng = np.random.default_rng(8)
    ks = [rng.standard_normal((6, 4, 2, 3)) for _ in range(3)]
    vs = [rng.standard_normal((6, 4, 2, 3)) for _ in range(3)]
    host = ref_swap_out(ks, vs, [4, 1])
    assert host.shape == (2, 3, 2, 4, 2, 3)
    for layer in range(3):
        assert np.array_equal(host[0, layer, 0], ks[layer][4])
        assert np.array_equal(host[1, layer, 1], vs[layer][1])
    k2, v2 = ref_swap_in(ks, vs, [0, 5], host)
    for layer in range(3):
        assert np.array_equal(k2[layer][0], ks[layer][4]) and np.array_equal(k2[layer][5], ks[layer][1])
        assert np.array_equal(v2[layer][0], vs[layer][4]) and np.array_equal(v2[layer][5], vs[layer][1])
        assert np.array_equal(k2[layer][1:5], ks[layer][1:5])
    with pytest.raises(AssertionError):
        ref_swap_in(ks, vs, [2, 2], host)


@pytest.mark.parametrize("prefix", [False, True])
def test_swap_round_trip_keeps_attention(prefix):
    """A preempted sequence that comes back attends to exactly the same K/V:
    decode after swap-out, reuse of its blocks by another sequence, and
    swap-in (restoring only blocks from first_restore on) equals decode
    before.  Its own full prefix blocks are the hits when the cache is on."""
    rng = np.random.default_rng(9)
    bs, nb, H, D = 4, 8, 2, 8
    bm = RefBlockManager(nb, bs, prefix)
    k = rng.standard_normal((nb, bs, H, D))
    v = rng.standard_normal((nb, bs, H, D))
    toks = list(range(100, 114))                  # 14 tokens: blocks 0-3
    t0 = bm.allocate(1, toks)
    q = rng.standard_normal((1, H, D))
    before = ref_decode(q, k, v, np.array([t0]), np.array([14]))
    host = ref_swap_out([k], [v], bm.swap_out(1))
    # Another sequence takes six blocks: the four free ones, block 3 and
    # (prefix cache on: by evicting the oldest keyed block) block 2, and
    # overwrites them; then it finishes.
    t2 = bm.allocate(2, list(range(200, 224)))
    assert sorted(t2) == [2, 3, 4, 5, 6, 7]
    for b in t2:
        k[b] = rng.standard_normal((bs, H, D))
        v[b] = rng.standard_normal((bs, H, D))
    bm.free(2)
    t1, first = bm.swap_in(1)
    # Cache on: blocks 0 and 1 are still keyed (hits); block 2's key went
    # with its eviction.  Cache off: everything comes back from host.
    assert first == (2 if prefix else 0)
    assert t1[:first] == t0[:first]
    (k,), (v,) = ref_swap_in([k], [v], t1[first:], host[first:])
    after = ref_decode(q, k, v, np.array([t1]), np.array([14]))
    assert np.array_equal(after, before)


# ---- planted mistakes: each must fail a pin -------------------------------

def mutant_slot_index(q, kc, vc, tables, lens, scale=None):
    """Mistake: token t read from slot table[t % nblk] * bs + t // bs."""
    bs = kc.shape[1]
    out = np.zeros(q.shape)
    g = q.shape[1] // kc.shape[2]
    for b in range(q.shape[0]):
        n = int(lens[b])
        nblk = -(-n // bs)
        idx = [tables[b][t % nblk] * bs + (t // nblk) % bs for t in range(n)]
        for h in range(q.shape[1]):
            K = kc.reshape(-1, kc.shape[2], kc.shape[3])[idx, h // g]
            V = vc.reshape(-1, vc.shape[2], vc.shape[3])[idx, h // g]
            s = (K @ q[b, h]) / np.sqrt(q.shape[2])
            p = np.exp(s - s.max())
            out[b, h] = (p / p.sum()) @ V
    return out


def mutant_gqa_modulo(q, kc, vc, tables, lens, scale=None):
    """Mistake: query head h reads KV head h % Hkv."""
    hkv = kc.shape[2]
    out = np.zeros(q.shape)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            out[b, h] = ref_decode_one(q[b, h], kc, vc, tables[b], int(lens[b]),
                                       h % hkv, 1 / np.sqrt(q.shape[2]))
    return out


def mutant_no_scale(q, kc, vc, tables, lens, scale=None):
    return ref_decode(q, kc, vc, tables, lens, scale=1.0)


def mutant_whole_last_block(q, kc, vc, tables, lens, scale=None):
    """Mistake (as in the page's kernel listing): seq_len = blocks * bs."""
    bs = kc.shape[1]
    return ref_decode(q, kc, vc, tables, -(-np.asarray(lens) // bs) * bs, scale)


@pytest.mark.parametrize("mutant", [mutant_slot_index, mutant_gqa_modulo,
                                    mutant_no_scale, mutant_whole_last_block])
def test_planted_mistake_is_caught(mutant):
    lens, hq, hkv, d = CASES[1]
    q, kc, vc, tables, lens = make_case(0, lens, hq, hkv, d)
    want = sdpa_paged(q, kc, vc, tables, lens)
    got = mutant(q, kc, vc, tables, lens)
    assert not np.allclose(got, want, rtol=1e-6, atol=1e-6, equal_nan=False)

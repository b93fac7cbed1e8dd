"""The oracle's prefill of an uncached suffix against what the pages and
the mathematics fix.

* Library routine: torch's scaled_dot_product_attention in float64 on the
  CPU over K/V gathered block by block with torch.cat (the article-130
  paged_attention pseudocode), with an explicit causal mask aligned to the
  end of the sequence (suffix row i sits at position n - q + i) -- and
  is_causal=True when nothing is cached.
* The last suffix row equals paged decode at the full length; a one-token
  suffix is exactly decode.
* Closed form: the first token of an uncached prompt attends only to itself,
  so its output is its own V row exactly.
* Placement invariance: the same logical K/V under two random block
  tables gives bitwise-equal outputs.
Planted mistakes (a strict causal mask, a mask aligned to the start
instead of the end, a suffix that ignores the cached prefix) must fail.
"""

import numpy as np
import pytest
import torch

from oracle import ref_decode, ref_decode_one, ref_prefill
from tests.test_oracle_attention import make_case

CASES = [
    # (qlens, lens, hq, hkv, d, bs)
    ([7, 16, 31], [7, 40, 64], 4, 4, 32, 16),     # fully uncached, partial and exact blocks
    ([1, 5, 33], [17, 100, 33], 8, 2, 16, 16),    # GQA, one-token suffix, cached prefixes
    ([12, 3], [12, 50], 6, 3, 16, 4),             # small blocks
]


def sdpa_prefill(q, kc, vc, tables, qlens, lens, causal_flag=False):
    T, hq, d = q.shape
    hkv = kc.shape[2]
    out = np.zeros((T, hq, d))
    K, V = torch.from_numpy(kc), torch.from_numpy(vc)
    row = 0
    for b, (ql, n) in enumerate(zip(qlens, lens)):
        nblk = -(-n // kc.shape[1])
        keys = torch.cat([K[int(tables[b][i])] for i in range(nblk)], dim=0)[:n]
        vals = torch.cat([V[int(tables[b][i])] for i in range(nblk)], dim=0)[:n]
        keys = keys.permute(1, 0, 2).unsqueeze(0).contiguous()
        vals = vals.permute(1, 0, 2).unsqueeze(0).contiguous()
        qq = torch.from_numpy(q[row:row + ql]).permute(1, 0, 2).unsqueeze(0).contiguous()
        if causal_flag:
            assert ql == n
            o = torch.nn.functional.scaled_dot_product_attention(qq, keys, vals, is_causal=True,
                                                                 enable_gqa=(hq != hkv))
        else:
            pos = torch.arange(n - ql, n).unsqueeze(1)
            mask = torch.arange(n).unsqueeze(0) <= pos           # [ql, n], end-aligned
            o = torch.nn.functional.scaled_dot_product_attention(qq, keys, vals, attn_mask=mask,
                                                                 enable_gqa=(hq != hkv))
        out[row:row + ql] = o[0].permute(1, 0, 2).numpy()
        row += ql
    return out


def case(seed, qlens, lens, hq, hkv, d, bs, poison=True):
    _, kc, vc, tables, _ = make_case(seed, lens, hq, hkv, d, bs=bs, poison=poison)
    q = np.random.default_rng(seed + 1).standard_normal((sum(qlens), hq, d))
    return q, kc, vc, tables


@pytest.mark.parametrize("qlens,lens,hq,hkv,d,bs", CASES)
def test_matches_sdpa_with_end_aligned_causal_mask(qlens, lens, hq, hkv, d, bs):
    q, kc, vc, tables = case(0, qlens, lens, hq, hkv, d, bs)
    got = ref_prefill(q, kc, vc, tables, qlens, lens)
    want = sdpa_prefill(q, kc, vc, tables, qlens, lens)
    assert np.isfinite(got).all()
    assert np.abs(got - want).max() < 1e-12


def test_uncached_prompt_is_plain_causal_attention():
    qlens = lens = [9, 32, 45]
    q, kc, vc, tables = case(3, qlens, lens, 4, 2, 16, 16)
    got = ref_prefill(q, kc, vc, tables, qlens, lens)
    want = sdpa_prefill(q, kc, vc, tables, qlens, lens, causal_flag=True)
    assert np.abs(got - want).max() < 1e-12


def test_last_row_is_decode_and_one_token_suffix_is_decode():
    qlens, lens = [4, 1, 20], [30, 17, 20]
    q, kc, vc, tables = case(5, qlens, lens, 4, 4, 16, 16)
    got = ref_prefill(q, kc, vc, tables, qlens, lens)
    last = np.cumsum(qlens) - 1
    dec = ref_decode(q[last], kc, vc, tables, np.asarray(lens))
    assert np.array_equal(got[last], dec)


def test_first_prompt_token_is_its_own_value_row():
    qlens = lens = [5, 20]
    q, kc, vc, tables = case(7, qlens, lens, 2, 2, 8, 4)
    got = ref_prefill(q, kc, vc, tables, qlens, lens)
    for b, row in ((0, 0), (1, 5)):
        slot0 = int(tables[b][0]) * kc.shape[1]
        v0 = vc.reshape(-1, 2, 8)[slot0]
        assert np.array_equal(got[row], v0)


def test_placement_invariance():
    qlens, lens = [6, 11], [40, 11]
    q, kc, vc, tables = case(9, qlens, lens, 4, 2, 16, 8, poison=False)
    bs, nb = kc.shape[1], kc.shape[0]
    perm = np.random.default_rng(1).permutation(nb)       # move every block
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    tables2 = np.where(tables >= 0, perm[np.maximum(tables, 0)], -1)
    a = ref_prefill(q, kc, vc, tables, qlens, lens)
    b = ref_prefill(q, kc2, vc2, tables2, qlens, lens)
    assert np.array_equal(a, b)


# ---- planted mistakes -------------------------------------------------------

def strict_mask(q, kc, vc, tables, qlens, lens):
    """Mistake: a token does not attend to itself."""
    out, row = np.zeros(q.shape), 0
    for b, (ql, n) in enumerate(zip(qlens, lens)):
        for i in range(ql):
            for h in range(q.shape[1]):
                out[row + i, h] = ref_decode_one(q[row + i, h], kc, vc, tables[b], n - ql + i,
                                                 h // (q.shape[1] // kc.shape[2]), 1 / np.sqrt(q.shape[2]))
        row += ql
    return out


def start_aligned(q, kc, vc, tables, qlens, lens):
    """Mistake: suffix row i attends to tokens 0..i (mask aligned to the
    start, as if nothing were cached)."""
    out, row = np.zeros(q.shape), 0
    for b, (ql, n) in enumerate(zip(qlens, lens)):
        for i in range(ql):
            for h in range(q.shape[1]):
                out[row + i, h] = ref_decode_one(q[row + i, h], kc, vc, tables[b], i + 1,
                                                 h // (q.shape[1] // kc.shape[2]), 1 / np.sqrt(q.shape[2]))
        row += ql
    return out


def suffix_only(q, kc, vc, tables, qlens, lens):
    """Mistake: the suffix attends only to suffix tokens (cached prefix
    ignored)."""
    out, row = np.zeros(q.shape), 0
    bs = kc.shape[1]
    for b, (ql, n) in enumerate(zip(qlens, lens)):
        c = n - ql
        t = np.arange(n)
        slots = tables[b][t // bs] * bs + t % bs
        for i in range(ql):
            for h in range(q.shape[1]):
                g = h // (q.shape[1] // kc.shape[2])
                keys = kc.reshape(-1, kc.shape[2], kc.shape[3])[slots[c:c + i + 1], g]
                vals = vc.reshape(-1, vc.shape[2], vc.shape[3])[slots[c:c + i + 1], g]
                s = keys @ q[row + i, h] / np.sqrt(q.shape[2])
                p = np.exp(s - s.max())
                out[row + i, h] = (p / p.sum()) @ vals
        row += ql
    return out


@pytest.mark.parametrize("mistake", [strict_mask, start_aligned, suffix_only])
def test_mistake_fails_the_sdpa_pin(mistake):
    qlens, lens, hq, hkv, d, bs = CASES[1]
    q, kc, vc, tables = case(0, qlens, lens, hq, hkv, d, bs, poison=False)
    want = sdpa_prefill(q, kc, vc, tables, qlens, lens)
    assert np.abs(ref_prefill(q, kc, vc, tables, qlens, lens) - want).max() < 1e-12
    assert np.abs(mistake(q, kc, vc, tables, qlens, lens) - want).max() > 1e-3

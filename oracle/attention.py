"""Reference paged decode attention in float64 (test infrastructure; see
oracle/__init__).

Definition ("qaqbuyan.com article 130", ``paged_attention`` pseudocode): for
each logical block of a sequence, fetch physical block ``block_table[i]``,
concatenate the fetched K and V in logical order, and run scaled dot-product
attention of the query against them.  The kernel listing on the same page
fixes the cache layout ``[num_blocks, block_size, num_heads, head_dim]``, the
output ``[num_requests, num_heads, head_dim]`` in float, and the scale
``1/sqrt(head_dim)``.

Readings:

* Only the first ``context_len`` tokens are attended; slots past the length
  in the last block are never read (the listing's ``num_blocks*block_size``
  would also read the unused tail of the last block; "day31" says a 50-token
  request's last block holds 2 tokens).
* Grouped-query attention: query head h reads KV head h // (Hq // Hkv).
* A sequence with context length 0 has nothing to attend to; its output is 0.
* Inputs of any float dtype are converted exactly to float64; all arithmetic
  is float64.
"""

import numpy as np


def _gather_positions(table, n, bs):
    """Flat slot of token t: table[t // bs] * bs + t % bs (P06 spec overview)."""
    t = np.arange(n, dtype=np.int64)
    return np.asarray(table, dtype=np.int64)[t // bs] * bs + t % bs


def ref_decode_one(q_bh, k_cache, v_cache, table, n, kv_head, scale):
    """Attention of one query vector over one sequence's n tokens, float64."""
    d = k_cache.shape[-1]
    out = np.zeros(d, dtype=np.float64)
    if n == 0:
        return out
    bs = k_cache.shape[1]
    idx = _gather_positions(table, n, bs)
    keys = k_cache.reshape(-1, k_cache.shape[2], d)[idx, kv_head, :].astype(np.float64)
    vals = v_cache.reshape(-1, v_cache.shape[2], d)[idx, kv_head, :].astype(np.float64)
    s = scale * (keys @ np.asarray(q_bh, dtype=np.float64))
    p = np.exp(s - s.max())
    p /= p.sum()
    return p @ vals


def ref_decode(q, k_cache, v_cache, block_tables, context_lens, scale=None):
    """Paged decode attention for a batch.

    q:            [B, Hq, D]
    k_cache/v_cache: [num_blocks, block_size, Hkv, D]
    block_tables: [B, >= ceil(max_len / block_size)] physical block ids
    context_lens: [B] tokens to attend per sequence
    Returns float64 [B, Hq, D].
    """
    q = np.asarray(q)
    B, hq, d = q.shape
    hkv = k_cache.shape[2]
    assert hq % hkv == 0, "query heads must be a multiple of KV heads"
    group = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, hq, d), dtype=np.float64)
    for b in range(B):
        n = int(context_lens[b])
        for h in range(hq):
            out[b, h] = ref_decode_one(q[b, h], k_cache, v_cache, block_tables[b],
                                       n, h // group, scale)
    return out


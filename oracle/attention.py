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
* ``ref_prefill`` (the uncached suffix after a prefix hit) is the same
  attention once per suffix token, each over the tokens up to and including
  its own position.
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



def ref_prefill(q, k_cache, v_cache, block_tables, query_lens, context_lens, scale=None):
    """Attention of a sequence's uncached suffix over its paged K/V, float64.

    "P06 · BlockManager" spec overview and key-question answers: a prompt
    whose first ``num_cached_tokens`` tokens are prefix hits needs a forward
    pass only for the rest -- at least its last token, whose output yields
    the next token.  "qaqbuyan.com article 130", system-prompt section: a
    later request reuses the shared prompt's blocks and computes only what
    follows them.  Each suffix token attends to every earlier token and to
    itself (causal), through the block table, with the suffix's own K/V
    already in the cache.

    q:            [T, Hq, D], the suffix tokens of all sequences, sequence
                  after sequence (query_lens[b] rows each)
    query_lens:   [B] suffix length q_b of each sequence
    context_lens: [B] total length n_b (prefix + suffix); query row i of
                  sequence b is the token at position n_b - q_b + i
    Returns float64 [T, Hq, D].
    """
    q = np.asarray(q)
    T, hq, d = q.shape
    hkv = k_cache.shape[2]
    assert hq % hkv == 0
    group = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    assert int(np.sum(query_lens)) == T
    out = np.zeros((T, hq, d), dtype=np.float64)
    row = 0
    for b in range(len(query_lens)):
        qb, n = int(query_lens[b]), int(context_lens[b])
        assert 0 <= qb <= n
        for i in range(qb):
            pos = n - qb + i
            for h in range(hq):
                out[row + i, h] = ref_decode_one(q[row + i, h], k_cache, v_cache, block_tables[b],
                                                 pos + 1, h // group, scale)
        row += qb
    return out

"""Reference KV write and block copy (test infrastructure; see oracle/__init__).

Both are plain element copies on NumPy arrays in the pages' cache layout
``[num_blocks, block_size, num_heads, head_dim]`` ("qaqbuyan.com article 130",
``paged_attention`` pseudocode and kernel listing).
"""

import numpy as np


def ref_write_kv(k_cache, v_cache, k_new, v_new, slot_mapping, inplace=False):
    """Scatter token t's K/V rows into flat slot ``slot_mapping[t]``.

    "qaqbuyan.com article 130", KV-cache section (each step computes the new
    token's K and V and appends them to the cache) and "day31" (a new token
    goes into the last, partly filled block).  Slots outside
    ``[0, num_blocks*block_size)`` are skipped; valid slots must be unique.
    Returns new arrays (the inputs untouched), or with ``inplace`` writes
    into ``k_cache``/``v_cache`` and returns them.
    """
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    slots = np.asarray(slot_mapping, dtype=np.int64)
    valid = [(t, int(s)) for t, s in enumerate(slots) if 0 <= s < nb * bs]
    assert len({s for _, s in valid}) == len(valid), "duplicate slot"
    k_out, v_out = (k_cache, v_cache) if inplace else (k_cache.copy(), v_cache.copy())
    k_flat = k_out.reshape(nb * bs, *k_cache.shape[2:])
    v_flat = v_out.reshape(nb * bs, *v_cache.shape[2:])
    for t, s in valid:
        k_flat[s] = k_new[t]
        v_flat[s] = v_new[t]
    return k_out, v_out


def ref_copy_blocks(k_caches, v_caches, pairs, inplace=False):
    """For every layer and every (src, dst): K[dst] = K[src], V[dst] = V[src].

    "day31", toy COW append: the new private block receives the old block's
    KV bytes.  The whole block (all slots) is copied.  Destinations must be
    distinct and none may also be a source.  Returns new per-layer lists,
    or with ``inplace`` copies within the given arrays and returns them.
    """
    pairs = [(int(s), int(d)) for s, d in pairs]
    dsts = [d for _, d in pairs]
    assert len(set(dsts)) == len(dsts), "duplicate destination"
    assert not (set(dsts) & {s for s, _ in pairs}), "destination is a source"
    k_out = list(k_caches) if inplace else [k.copy() for k in k_caches]
    v_out = list(v_caches) if inplace else [v.copy() for v in v_caches]
    for layer in range(len(k_out)):
        for s, d in pairs:
            k_out[layer][d] = k_out[layer][s]
            v_out[layer][d] = v_out[layer][s]
    return k_out, v_out


def ref_swap_out(k_caches, v_caches, blocks):
    """Copy blocks to host memory: the preempted sequence's KV leaves the GPU.

    "qaqbuyan.com article 130", continuous-batching scheduler,
    ``_preempt_request``: each of the victim's physical blocks is copied to
    CPU memory before it is freed.  Returns one array
    ``[len(blocks), num_layers, 2, block_size, num_heads, head_dim]``: for
    list entry i and layer l, ``[i, l, 0]`` is ``K_l[blocks[i]]`` and
    ``[i, l, 1]`` is ``V_l[blocks[i]]``.
    """
    blocks = [int(b) for b in blocks]
    L = len(k_caches)
    shape = (len(blocks), L, 2) + tuple(k_caches[0].shape[1:])
    out = np.empty(shape, dtype=k_caches[0].dtype)
    for i, b in enumerate(blocks):
        for layer in range(L):
            out[i, layer, 0] = k_caches[layer][b]
            out[i, layer, 1] = v_caches[layer][b]
    return out


def ref_swap_in(k_caches, v_caches, blocks, host, inplace=False):
    """Restore host copies into (fresh) blocks: the inverse of ref_swap_out.

    For list entry i and every layer l: ``K_l[blocks[i]] = host[i, l, 0]``
    and ``V_l[blocks[i]] = host[i, l, 1]``.  Blocks must be distinct.
    Returns new per-layer lists, or with ``inplace`` writes into the given
    arrays and returns them.
    """
    blocks = [int(b) for b in blocks]
    assert len(set(blocks)) == len(blocks), "duplicate destination block"
    assert host.shape[0] == len(blocks) and host.shape[1] == len(k_caches)
    k_out = list(k_caches) if inplace else [k.copy() for k in k_caches]
    v_out = list(v_caches) if inplace else [v.copy() for v in v_caches]
    for i, b in enumerate(blocks):
        for layer in range(len(k_out)):
            k_out[layer][b] = host[i, layer, 0]
            v_out[layer][b] = host[i, layer, 1]
    return k_out, v_out

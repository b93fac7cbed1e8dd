"""Memory arithmetic from the pages (test infrastructure; see oracle/__init__).

Each function is the plain definition the pages print.
"""

import math


def kv_cache_bytes(layers: int, heads: int, head_dim: int, seq_len: int,
                   bytes_per_elem: int) -> int:
    """KV-cache bytes of one sequence: 2 (K and V) x L x H x D x S x B.

    "qaqbuyan.com article 130", KV-cache size formula (the worked
    Llama-2-13B examples at 1000 and 4096 tokens use it).
    """
    return 2 * layers * heads * head_dim * seq_len * bytes_per_elem


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int,
                       bytes_per_elem: int = 2) -> int:
    """Bytes of K and V for one token over all layers.

    "day31", memory-estimate script (``kv_bytes_per_token``).
    """
    return 2 * layers * kv_heads * head_dim * bytes_per_elem


def block_bytes(layers: int, heads: int, head_dim: int, bytes_per_elem: int,
                block_size: int = 16) -> int:
    """Bytes of one physical KV block, which spans every layer.

    "qaqbuyan.com article 130", block-size formula 2 x L x H x D x 16 x B.
    """
    return 2 * layers * heads * head_dim * block_size * bytes_per_elem


def blocks_needed(tokens: int, block_size: int) -> int:
    """ceil(tokens / block_size): "day31", block-count script."""
    return math.ceil(tokens / block_size)


def contiguous_tables(lengths, block_size):
    """Tables handed out consecutively from block 0 with no reuse.

    "day31", block-count script (``allocate_requests``): request i gets the
    next ``blocks_needed(len_i)`` block ids.  Returns (tables, blocks used).
    """
    next_block = 0
    tables = []
    for length in lengths:
        n = blocks_needed(length, block_size)
        tables.append(list(range(next_block, next_block + n)))
        next_block += n
    return tables, next_block


def tail_waste_tokens(lengths, block_size) -> int:
    """Unused token slots in each request's last block, summed.

    "day31", block-count script (``waste_tokens``).
    """
    return sum(blocks_needed(x, block_size) * block_size - x for x in lengths)

"""Seeded synthetic inputs shaped like the pages' workloads.

Shared by the tests, ``bench.py`` and the smoke check.  This module holds no
part of the method's arithmetic: it only draws lengths, token ids, block
orders and N(0, 1) values from fixed seeds.  Both the HIP path and the CPU
oracle consume what it returns; neither is imported here.

Workloads (sizes as the pages give them; see the design notes for sources):

* ``tiny``      -- lengths [7, 16, 31, 48, 63] ("day31" block-count script),
  1 layer, 4 heads x 64 dims, fp32, 64-block pool.
* ``13b_layer`` -- Llama-2-13B shape from "qaqbuyan.com article 130"
  (40 heads x 128, fp16), 10 sequences x 4096 tokens, 4096-block pool.
* ``mixed_7b``  -- shape of the "day31" memory-estimate script (32 layers x
  32 KV heads x 128, fp16), 128 sequences with lengths log-uniform in
  [50, 4096], 16384-block pool.
* ``fork_cow``  -- parallel sampling ("day31" fork + COW): 64 prompts of 2048
  tokens, each forked 8 ways, 256 appended tokens per fork, 32 heads x 128,
  fp16, 20480-block pool.
* ``gqa_long``  -- 32 query / 8 KV heads x 128, bf16, 32 sequences x 32768,
  131072-block pool, 512-token split-KV partitions.
* ``beam``      -- beam search ("day31" fork + COW at arbitrary positions):
  64 prompts with lengths log-uniform in [50, 2048], 8 beams each, every
  step each beam's continuation picks a parent beam; 32 heads x 128, fp16,
  20480-block pool.
"""

import numpy as np

CONFIGS = {
    "tiny": dict(layers=1, lens=[7, 16, 31, 48, 63], hq=4, hkv=4, d=64,
                 dtype="f32", bs=16, num_blocks=64, prefix_cache=True,
                 partition_tokens=512),
    "13b_layer": dict(layers=1, lens=[4096] * 10, hq=40, hkv=40, d=128,
                      dtype="f16", bs=16, num_blocks=4096, prefix_cache=False,
                      partition_tokens=512),
    "mixed_7b": dict(layers=32, B=128, len_lo=50, len_hi=4096, hq=32, hkv=32,
                     d=128, dtype="f16", bs=16, num_blocks=16384,
                     prefix_cache=False, partition_tokens=512),
    "fork_cow": dict(layers=1, prompts=64, forks=8, prompt_len=2048, extra=256,
                     hq=32, hkv=32, d=128, dtype="f16", bs=16,
                     num_blocks=20480, prefix_cache=True, partition_tokens=512),
    "gqa_long": dict(layers=1, lens=[32768] * 32, hq=32, hkv=8, d=128,
                     dtype="bf16", bs=16, num_blocks=131072,
                     prefix_cache=False, partition_tokens=512),
    "beam": dict(layers=1, groups=64, beams=8, len_lo=50, len_hi=2048, hq=32, hkv=32,
                 d=128, dtype="f16", bs=16, num_blocks=20480, prefix_cache=True,
                 partition_tokens=512),
}

ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


def mixed_lengths(B=128, lo=50, hi=4096, seed=0):
    """Lengths exp(U[ln lo, ln hi]) rounded and clipped, NumPy PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    u = rng.uniform(np.log(lo), np.log(hi), size=B)
    return np.clip(np.round(np.exp(u)), lo, hi).astype(np.int64)


def lengths(name, seed=0):
    cfg = CONFIGS[name]
    if "lens" in cfg:
        return np.asarray(cfg["lens"], dtype=np.int64)
    if name == "mixed_7b":
        return mixed_lengths(cfg["B"], cfg["len_lo"], cfg["len_hi"], seed)
    raise KeyError(name)


def block_order(num_blocks, seed):
    """A seeded permutation of the pool: the order blocks are handed out."""
    return np.random.Generator(np.random.PCG64(seed)).permutation(num_blocks)


def token_ids(n, seed, vocab=32000):
    """n seeded token ids in [0, vocab)."""
    return np.random.Generator(np.random.PCG64(seed)).integers(0, vocab, size=n).tolist()


def scramble_free_list(bm, order, first_seq=1 << 40):
    """Leave ``bm``'s free list in ``order`` using only allocate/free: one
    single-token sequence per block (the free list hands them out 0, 1, ...),
    then free them in ``order``.  Works on any manager with the block-manager
    API (the library's or the oracle's)."""
    n = len(order)
    for i in range(n):
        bm.allocate(first_seq + i, [0])
    for b in order:
        bm.free(first_seq + int(b))


def normal_np(shape, seed, dtype=np.float32):
    """N(0,1) values on the host (small cases), rounded to ``dtype``."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(shape).astype(dtype)


def normal_torch(shape, seed, dtype, device):
    """N(0,1) tensor drawn by torch's generator on ``device`` (large cases;
    the oracle reads the resulting bytes back)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=dtype)


def beam_parents(rng, beams):
    """Parents of the next ``beams`` beams of one group: a seeded draw with
    replacement, sorted (a stand-in for top-k selection; some beams get
    several children, some none)."""
    return np.sort(rng.integers(0, beams, size=beams))

"""Helpers for the GPU parity tests: seeded cases in device memory plus the
host copies the oracle reads (never anything the HIP path produced)."""

import sys

import numpy as np
import torch

import workloads

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
TOL = {"f32": 1e-4, "f16": 2e-3, "bf16": 2e-3}


REPORT = []


def say(*args):
    """Name the case before each GPU step (flushed, so a crash still shows it)."""
    print("[gpu-case]", *args, file=sys.stderr, flush=True)


def report(name, value):
    """Record a measured figure (a max abs error) for the end-of-run summary."""
    REPORT.append((name, value))


def host_f32(t):
    """Host float32 copy of a device tensor (exact for f32, f16 and bf16);
    the oracle widens to float64 itself."""
    return t.detach().float().cpu().numpy()


def random_tables(lens, bs, num_blocks, seed, pad=-1):
    """Each sequence's blocks drawn in order from a seeded permutation of
    the pool; rows padded with ``pad``."""
    need = [-(-int(n) // bs) for n in lens]
    assert sum(need) <= num_blocks
    order = workloads.block_order(num_blocks, seed)
    maxb = max(need + [1])
    tab = np.full((len(lens), maxb), pad, dtype=np.int32)
    o = 0
    for i, k in enumerate(need):
        tab[i, :k] = order[o:o + k]
        o += k
    return tab


def poison_mask(tables, lens, num_blocks, bs):
    """True for every slot that no sequence attends (unused tails, blocks
    outside every table)."""
    used = np.zeros((num_blocks, bs), dtype=bool)
    for row, n in zip(tables, lens):
        for i in range(int(n)):
            used[row[i // bs], i % bs] = True
    return ~used


def make_cache(num_blocks, bs, hkv, d, dtype, seed, device="cuda", poison=None):
    """Seeded N(0,1) K and V caches on the device; slots in ``poison`` (a
    [num_blocks, bs] bool mask) are set to NaN."""
    tdt = TORCH_DTYPES[dtype]
    k = workloads.normal_torch((num_blocks, bs, hkv, d), seed, tdt, device)
    v = workloads.normal_torch((num_blocks, bs, hkv, d), seed + 1, tdt, device)
    if poison is not None:
        m = torch.from_numpy(poison).to(device)
        k[m] = float("nan")
        v[m] = float("nan")
    return k, v

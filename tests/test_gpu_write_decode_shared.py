"""GPU parity of pa_write_decode_shared: each sequence's new token's K/V
written to its slot and the shared-prefix decode over it, in one call
("qaqbuyan.com article 130", decode loop: append the new K/V, then attend
over every cached token; "day31", fork and copy-on-write: forked sequences
share the parent's blocks, and an append copies a shared, partly filled
last block first, so every last block here is a sequence's own).

It must leave exactly the cache bytes pa_write_kv leaves at the slots of
position len - 1 ("P06 · BlockManager" spec overview) and return
pa_decode_shared's output after that write, with the plan the library's
planner makes: equal up to the last bit (the fused kernels are compiled
apart from the plain ones, and the compiler may fuse a multiply and an add
differently in each; bf16 with one query head per KV head in the
four-heads mapping differs by one ulp), and within the attention tolerance
of the oracle's write followed by its fp64 attention.  Slots no sequence
attends hold NaN.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.families import beam_family, fork_family
from tests.gpu_util import TOL, TORCH_DTYPES, host_f32, make_cache, poison_mask, say

pytestmark = pytest.mark.gpu

pkv = pytest.importorskip("paged_kv_cache_136_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


BS = 16


def _slots(tables, lens):
    return np.array([int(tables[b, (n - 1) // BS]) * BS + (n - 1) % BS
                     for b, n in enumerate(lens)], dtype=np.int64)


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _int_view(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


def _run(tables, lens, hq, hkv, d, dtype, pt, seed, heads, plan=None, with_oracle=True):
    """(fused output, separate output, caches equal, fused caches, the
    original caches, oracle output or None)."""
    lens = np.asarray(lens, dtype=np.int32)
    nb = int(tables.max()) + 1
    k, v = make_cache(nb, BS, hkv, d, dtype, seed, poison=poison_mask(tables, lens, nb, BS))
    tdt = TORCH_DTYPES[dtype]
    B = len(lens)
    q = workloads.normal_torch((B, hq, d), seed + 7, tdt, "cuda")
    kn = workloads.normal_torch((B, hkv, d), seed + 8, tdt, "cuda")
    vn = workloads.normal_torch((B, hkv, d), seed + 9, tdt, "cuda")
    if plan is None:
        plan = pkv.pa_shared_plan(tables, lens, BS, pt, hq // hkv)
    sg, groups, mx, mp = plan[:4]
    pargs = (_i32(sg), _i32(np.asarray(groups).reshape(-1, 17)), mx, mp)
    d_tab, d_len, max_len = _i32(tables), _i32(lens), int(lens.max())
    hint = 1 if heads else 0
    k1, v1 = k.clone(), v.clone()
    pkv.pa_write_kv(k1, v1, kn, vn, torch.from_numpy(_slots(tables, lens)).cuda())
    sep = pkv.pa_decode_shared(q, k1, v1, d_tab, d_len, max_len, *pargs, partition_tokens=pt,
                               max_private_blocks=hint)
    k2, v2 = k.clone(), v.clone()
    fused = pkv.pa_write_decode_shared(q, k2, v2, kn, vn, d_tab, d_len, max_len, *pargs,
                                       partition_tokens=pt, max_private_blocks=hint)
    torch.cuda.synchronize()
    same = (torch.equal(_int_view(k1), _int_view(k2)) and torch.equal(_int_view(v1), _int_view(v2)))
    want = None
    if with_oracle:
        kh, vh = oracle.ref_write_kv(host_f32(k), host_f32(v), host_f32(kn), host_f32(vn),
                                     _slots(tables, lens))
        want = oracle.ref_decode(host_f32(q), kh, vh, tables, lens)
    return (fused.cpu().numpy(), sep.cpu().numpy(), same, (k2, v2), (k, v, kn, vn), want)


def _same_output(a, b):
    """Equal, or apart by rounding in the last bits: |diff| at most
    2^-20 of the magnitude (8 ulp of float32), or 2^-23 near zero."""
    return np.array_equal(np.isnan(a), np.isnan(b)) and bool(
        (np.abs(a - b) <= np.maximum(np.abs(b) * 2.0 ** -20, 2.0 ** -23))[~np.isnan(b)].all())


@pytest.mark.parametrize("pt", [128, 512])
@pytest.mark.parametrize("heads", [False, True])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_write_decode_shared_fork_families(group, d, dtype, heads, pt):
    """Four fork families (16/group members, at most 4) with ragged appends
    and two unforked sequences; the private pass in either wave mapping;
    128-token partitions (the reduce merges) and 512 (the private pass
    finishes every sequence)."""
    hkv, forks = 4, min(4, 16 // group)
    prompts = [700, 1100, 530, 95]
    extra = np.random.default_rng(d + group).integers(1, 60, size=len(prompts) * forks)
    tables, lens = fork_family(prompts, forks, extra, singles=[300, 17], seed=group)
    say("write_decode_shared forks", group, d, dtype, "heads", heads, "pt", pt)
    fused, sep, same, _, _, want = _run(tables, lens, hkv * group, hkv, d, dtype, pt,
                                        seed=61 + d + group, heads=heads)
    assert same
    assert _same_output(fused, sep)
    assert np.isfinite(fused).all()
    assert np.abs(fused - want).max() <= TOL[dtype]


@pytest.mark.parametrize("group", [1, 4])
def test_write_decode_shared_beams(group):
    """Beam-search trees (seeded re-forks, the old beams freed, every beam
    appending): the mapping the beam batch uses (four heads per private
    workgroup, 512-token partitions)."""
    tables, lens = beam_family([300, 700, 150, 45], 16 // group, 30, seed=4)
    say("write_decode_shared beams", group)
    fused, sep, same, _, _, want = _run(tables, lens, 8 * group, 8, 128, "f16", 512, seed=17,
                                        heads=True)
    assert same
    assert _same_output(fused, sep)
    assert np.abs(fused - want).max() <= TOL["f16"]


def test_write_decode_shared_without_groups():
    """A plan with no groups: the call is pa_write_decode."""
    tables, lens = fork_family([200, 90], 1, [5, 9], singles=[40], seed=3)
    plan = (np.full(len(lens), -1, np.int32), np.zeros((0, 17), np.int32), 0, 0)
    say("write_decode_shared no groups")
    fused, sep, same, _, _, want = _run(tables, lens, 4, 4, 128, "f16", 64, seed=5, heads=False,
                                        plan=plan)
    assert same and _same_output(fused, sep)
    assert np.abs(fused - want).max() <= TOL["f16"]


def test_write_decode_shared_private_bound_too_small():
    """A private bound below what some sequences need (vector path, one
    head per workgroup): those sequences come out NaN and their new rows are
    not written (the private grid never reaches their last block); every
    other sequence is written and exact."""
    tables, lens = fork_family([700, 260], 2, [3, 150, 9, 40], singles=[500], seed=8)
    pt = 64
    sg, groups, mx, mp = pkv.pa_shared_plan(tables, lens, BS, pt, 1)
    assert mp > 1
    plan = (sg, groups, mx, 1)
    pb = pt // BS
    over = []
    for b, n in enumerate(lens):
        S = int(groups[sg[b], 0]) if sg[b] >= 0 else 0
        if -(-(-(-int(n) // BS) - S) // pb) > 1:
            over.append(b)
    ok = [b for b in range(len(lens)) if b not in over]
    assert over and ok
    say("write_decode_shared short private grid", over)
    fused, _, _, (k2, v2), (k0, v0, kn, vn), _ = _run(tables, lens, 4, 4, 128, "f16", pt, seed=23,
                                                     heads=False, plan=plan, with_oracle=False)
    assert np.isnan(fused[over]).all()
    slots = _slots(tables, lens)
    kh, vh = oracle.ref_write_kv(host_f32(k0), host_f32(v0), host_f32(kn)[ok], host_f32(vn)[ok],
                                 slots[ok])
    assert np.array_equal(host_f32(k2), kh, equal_nan=True)
    assert np.array_equal(host_f32(v2), vh, equal_nan=True)
    q_want = oracle.ref_decode(host_f32(workloads.normal_torch((len(lens), 4, 128), 23 + 7,
                                                               torch.float16, "cuda"))[ok],
                               kh, vh, tables[ok], lens[ok])
    assert np.abs(fused[ok] - q_want).max() <= TOL["f16"]

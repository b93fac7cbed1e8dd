"""GPU parity of pa_write_decode: each sequence's new token's K/V written to
its slot and the decode over it, in one call ("qaqbuyan.com article 130",
decode loop: append the new K/V, then attend over every cached token).

It must leave exactly the cache bytes pa_write_kv leaves, at the slots the
block table gives position len - 1 ("P06 · BlockManager" spec overview),
and return exactly pa_decode's output after that write: both are checked
bit for bit, and the output also against the oracle's write followed by
its fp64 attention.  Slots no sequence attends hold NaN.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import TOL, TORCH_DTYPES, host_f32, make_cache, poison_mask, random_tables, say

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
RAGGED = [1, 15, 16, 17, 31, 33, 64, 100, 511, 512, 513, 700]


def _slots(tables, lens):
    """The slot of each sequence's position len - 1 (-1 for an empty one)."""
    return np.array([int(tables[b, (n - 1) // BS]) * BS + (n - 1) % BS if n > 0 else -1
                     for b, n in enumerate(lens)], dtype=np.int64)


def _run(lens, hq, hkv, d, dtype, partition, seed, tables=None, num_blocks=None, with_oracle=True):
    """(fused output, separate output, caches equal, oracle output or None)."""
    lens = np.asarray(lens, dtype=np.int32)
    nb = num_blocks or sum(-(-int(n) // BS) for n in lens) + 5
    if tables is None:
        tables = random_tables(lens, BS, nb, seed, pad=0)
    k, v = make_cache(nb, BS, hkv, d, dtype, seed, poison=poison_mask(tables, lens, nb, BS))
    tdt = TORCH_DTYPES[dtype]
    B = len(lens)
    q = workloads.normal_torch((B, hq, d), seed + 7, tdt, "cuda")
    kn = workloads.normal_torch((B, hkv, d), seed + 8, tdt, "cuda")
    vn = workloads.normal_torch((B, hkv, d), seed + 9, tdt, "cuda")
    d_tab = torch.from_numpy(tables).cuda()
    d_len = torch.from_numpy(lens).cuda()
    max_len = int(lens.max())
    slots = _slots(tables, lens)
    k1, v1 = k.clone(), v.clone()
    pkv.pa_write_kv(k1, v1, kn, vn, torch.from_numpy(slots).cuda())
    sep = pkv.pa_decode(q, k1, v1, d_tab, d_len, max_len, partition_tokens=partition)
    k2, v2 = k.clone(), v.clone()
    fused = pkv.pa_write_decode(q, k2, v2, kn, vn, d_tab, d_len, max_len,
                                partition_tokens=partition)
    torch.cuda.synchronize()
    same_cache = (torch.equal(k1.view(torch.int16 if dtype != "f32" else torch.int32),
                              k2.view(torch.int16 if dtype != "f32" else torch.int32)) and
                  torch.equal(v1.view(torch.int16 if dtype != "f32" else torch.int32),
                              v2.view(torch.int16 if dtype != "f32" else torch.int32)))
    want = None
    if with_oracle:
        kh, vh = oracle.ref_write_kv(host_f32(k), host_f32(v), host_f32(kn), host_f32(vn), slots)
        want = oracle.ref_decode(host_f32(q), kh, vh, tables, lens)
    return fused.cpu().numpy(), sep.cpu().numpy(), same_cache, want


def _bits_equal(a, b):
    return np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_write_decode_ragged(dtype, d, group):
    """Every position of the new token within its block (first, middle,
    last row), every query group and dtype, against write + decode bit for
    bit and against the oracle."""
    say("write_decode ragged", dtype, d, group)
    fused, sep, same_cache, want = _run(RAGGED, 2 * group, 2, d, dtype, 128, seed=200 + d + group)
    assert same_cache
    assert _bits_equal(fused, sep)
    assert np.isfinite(fused).all()
    assert np.abs(fused - want).max() <= TOL[dtype]


@pytest.mark.parametrize("partition", [0, 16, 64, 512, 2048])
@pytest.mark.parametrize("dtype,group", [("f16", 1), ("bf16", 4), ("f16", 8)])
def test_write_decode_partition_sizes(partition, dtype, group):
    """Whole sequences in one partition (no reduce), split partitions, and on
    the matrix-core path one workgroup holding all of a sequence's
    partitions or not."""
    lens = [1, 300, 1000, 2049, 3001]
    say("write_decode partitions", partition, dtype, group)
    fused, sep, same_cache, want = _run(lens, 2 * group, 2, 128, dtype, partition, seed=31)
    assert same_cache
    assert _bits_equal(fused, sep)
    assert np.abs(fused - want).max() <= TOL[dtype]


@pytest.mark.parametrize("dtype,group", [("f16", 1), ("bf16", 2), ("bf16", 8), ("f32", 4)])
def test_write_decode_edge_cases(dtype, group):
    """An empty sequence writes nothing and returns zeros; a length past
    max_context_len writes nothing and returns NaN; a last block outside
    the pool writes nothing (NaN rows); a bad id in an earlier block still
    writes the new token (NaN rows); every other sequence is exact."""
    lens = np.array([0, 40, 90, 130, 64, 17], dtype=np.int32)
    nb = 40
    tables = random_tables(lens, BS, nb, seed=9, pad=0)
    tables[3, 8] = nb + 5                     # last block of the 130-token sequence: bad
    tables[4, 1] = -3                         # an earlier block of the 64-token sequence: bad
    hq, hkv, d = 2 * group, 2, 128
    k, v = make_cache(nb, BS, hkv, d, dtype, seed=10)
    tdt = TORCH_DTYPES[dtype]
    q = workloads.normal_torch((6, hq, d), 11, tdt, "cuda")
    kn = workloads.normal_torch((6, hkv, d), 12, tdt, "cuda")
    vn = workloads.normal_torch((6, hkv, d), 13, tdt, "cuda")
    max_len = 140
    lens_d = lens.copy()
    lens_d[5] = 141                           # past max_context_len: invalid
    say("write_decode edges", dtype, group)
    k2, v2 = k.clone(), v.clone()
    out = pkv.pa_write_decode(q, k2, v2, kn, vn, torch.from_numpy(tables).cuda(),
                              torch.from_numpy(lens_d).cuda(), max_len, partition_tokens=64)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert (got[0] == 0).all()
    assert np.isnan(got[3]).all() and np.isnan(got[4]).all() and np.isnan(got[5]).all()
    # the cache changes exactly at the new slots of the 40- and 90-token
    # sequences and of the 64-token one (bad earlier block, good last one)
    slots = _slots(tables, lens)
    written = [1, 2, 4]
    kh, vh = oracle.ref_write_kv(host_f32(k), host_f32(v), host_f32(kn)[written],
                                 host_f32(vn)[written], slots[written])
    assert np.array_equal(host_f32(k2), kh) and np.array_equal(host_f32(v2), vh)
    want = oracle.ref_decode(host_f32(q)[[1, 2]], kh, vh, tables[[1, 2]], lens[[1, 2]])
    assert np.abs(got[[1, 2]] - want).max() <= TOL[dtype]


def test_write_decode_mixed_7b_layer():
    """One layer of the mixed 7B batch (128 sequences, lengths log-uniform in
    [50, 4096], 32 heads x 128, fp16, 512-token partitions), the launch
    configuration the bench times: caches and output bit for bit against
    pa_write_kv + pa_decode (whose full-size output the parity suite checks
    against the oracle row by row)."""
    lens = workloads.lengths("mixed_7b")
    nb = sum(-(-int(n) // BS) for n in lens) + 8
    tables = random_tables(lens, BS, nb, seed=77, pad=0)
    say("write_decode mixed 7B layer")
    fused, sep, same_cache, _ = _run(lens, 32, 32, 128, "f16", 512, seed=77, tables=tables,
                                     num_blocks=nb, with_oracle=False)
    assert same_cache
    assert _bits_equal(fused, sep)
    assert np.isfinite(fused).all()

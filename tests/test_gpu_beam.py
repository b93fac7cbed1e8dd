"""GPU parity of beam search over the paged cache ("day31", fork and
copy-on-write append): every step each group's beams are re-forked from
seeded parents at arbitrary positions, the old beams are freed, and every
beam appends a token, so beams that share a partly filled last block copy
it (many small pa_copy_blocks pairs per step).  Mirrored step by step by
the oracle: identical slots and copy pairs, bit-exact caches after every
step, decode within the attention tolerance.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import TOL, make_cache, say

pytestmark = pytest.mark.gpu

pkv = pytest.importorskip("paged_kv_cache_136_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy()


def test_beam_search_flow():
    G, W, bs, nb, hkv, hq, d, steps = 4, 4, 16, 160, 4, 8, 64, 40
    say("beam search flow")
    bm = pkv.BlockManager(nb, bs, True)
    rbm = oracle.RefBlockManager(nb, bs, True)
    k, v = make_cache(nb, bs, hkv, d, "f16", seed=900)
    kb, vb = _bits(k), _bits(v)
    rng = np.random.default_rng(5)
    beams, nid = [], 1
    for g, n in enumerate([37, 50, 64, 100]):
        toks = workloads.token_ids(n, seed=950 + g)
        assert bm.allocate(nid, toks) == rbm.allocate(nid, toks)
        beams.append([nid] * W)
        nid += 1
    total_cow = 0
    for step in range(steps):
        par, kid, old, new = [], [], [], []
        for grp in beams:
            ks = []
            for p in workloads.beam_parents(rng, W):
                par.append(grp[p])
                kid.append(nid)
                ks.append(nid)
                nid += 1
            new.append(ks)
            old += sorted(set(grp))
        bm.fork_batch(par, kid)
        for p, c in zip(par, kid):
            rbm.fork(p, c)
        bm.free_batch(old)
        for s in old:
            rbm.free(s)
        beams = new
        flat = [s for g in beams for s in g]
        toks = rng.integers(0, 32000, len(flat))
        slots, pairs = bm.append_slots(flat, toks)
        want = [rbm.append_slot(s, int(t)) for s, t in zip(flat, toks)]
        assert slots.tolist() == [w[0] for w in want]
        want_pairs = [w[1] for w in want if w[1] is not None]
        assert [tuple(x) for x in pairs.tolist()] == want_pairs
        total_cow += len(pairs)
        if len(pairs):
            pkv.pa_copy_blocks([k], [v], torch.from_numpy(pairs).cuda())
            oracle.ref_copy_blocks([kb], [vb], want_pairs, inplace=True)
        kn = workloads.normal_torch((len(flat), hkv, d), 2000 + step, torch.float16, "cuda")
        vn = workloads.normal_torch((len(flat), hkv, d), 3000 + step, torch.float16, "cuda")
        pkv.pa_write_kv(k, v, kn, vn, torch.from_numpy(slots).cuda())
        oracle.ref_write_kv(kb, vb, _bits(kn), _bits(vn), slots, inplace=True)
        lens = [rbm.seq_len(s) for s in flat]
        width = max(-(-n // bs) for n in lens)
        tables, clens = bm.export_batch(flat, width, pad_block=0)
        q = workloads.normal_torch((len(flat), hq, d), 4000 + step, torch.float16, "cuda")
        out = pkv.pa_decode(q, k, v, torch.from_numpy(tables).cuda(), torch.from_numpy(clens).cuda(),
                            max(lens), partition_tokens=64)
        ref = oracle.ref_decode(_bits(q).view(np.float16), kb.view(np.float16), vb.view(np.float16),
                                tables, clens)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(k), kb) and np.array_equal(_bits(v), vb), step
        err = np.abs(out.cpu().numpy() - ref).max()
        assert err <= TOL["f16"], (step, err)
    assert total_cow > steps             # several small copies per step on average
    bm.free_batch([s for g in beams for s in g])
    assert bm.num_free_blocks == nb

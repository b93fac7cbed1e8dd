"""Block tables of sequence families built with the oracle's block manager
("day31" fork and copy-on-write append; "P06 · BlockManager" prefix cache),
for the shared-prefix planner and decode tests."""

import numpy as np

import oracle
import workloads


def _export(rbm, seqs, bs):
    lens = np.array([rbm.seq_len(s) for s in seqs], dtype=np.int32)
    mb = max(-(-int(n) // bs) for n in lens)
    tables = np.zeros((len(seqs), mb), dtype=np.int32)
    for i, s in enumerate(seqs):
        t = rbm.get_table(s)
        tables[i, :len(t)] = t
    return tables, lens


def fork_family(prompts, forks, extra, bs=16, nb=4096, seed=0, singles=()):
    """Each prompt allocated (prefix cache on), its parent appends one token
    and forks forks-1 children, then every sequence appends extra[i] tokens
    (copy-on-write where a partly filled block is shared).  ``singles``
    adds unforked sequences of those lengths after the families.  Returns
    (tables int32 [B, max_blocks] zero-padded, lens int32 [B])."""
    rbm = oracle.RefBlockManager(nb, bs, True)
    seqs, sid = [], 0
    for p, n in enumerate(prompts):
        rbm.allocate(sid, workloads.token_ids(n, seed=seed + p))
        rbm.append_slot(sid, 7)
        fam = [sid]
        for c in range(1, forks):
            rbm.fork(sid, sid + c)
            fam.append(sid + c)
        seqs += fam
        sid += forks
    for s, e in zip(seqs, extra):
        for t in range(int(e)):
            rbm.append_slot(s, 100 + t)
    for j, n in enumerate(singles):
        rbm.allocate(sid, workloads.token_ids(int(n), seed=seed + 500 + j))
        seqs.append(sid)
        sid += 1
    return _export(rbm, seqs, bs)


def beam_family(prompts, beams, steps, bs=16, nb=2048, seed=0):
    """Beam search: every step each group's beams are re-forked from seeded
    parents (workloads.beam_parents), the old beams freed, and every beam
    appends one token."""
    rng = np.random.default_rng(seed)
    rbm = oracle.RefBlockManager(nb, bs, True)
    groups, nid = [], 1
    for g, n in enumerate(prompts):
        rbm.allocate(nid, workloads.token_ids(n, seed=seed + 50 + g))
        groups.append([nid] * beams)
        nid += 1
    for _ in range(steps):
        new = []
        for grp in groups:
            ks = []
            for p in workloads.beam_parents(rng, beams):
                rbm.fork(grp[p], nid)
                ks.append(nid)
                nid += 1
            for old in set(grp):
                rbm.free(old)
            for s in ks:
                rbm.append_slot(s, int(rng.integers(0, 1000)))
            new.append(ks)
        groups = new
    return _export(rbm, [s for grp in groups for s in grp], bs)

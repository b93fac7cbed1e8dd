"""The oracle's continuous-batching scheduler against what the pages fix.

Pins: the step timeline printed in "qaqbuyan.com article 130" (who leaves
and who joins at which step, generated counts), three hand-derived
preemption traces (swap to host, recompute, and the page's most-generated
victim over every running request), and invariants over seeded random
request streams (every request finishes with exactly its token budget, the
batch never exceeds its size, host records and blocks are conserved, the
block manager's I1-I5 hold after every step, and the plans' device work,
played in plan order on a cache whose rows fingerprint each token's
prefix, leaves every decoded request reading exactly its own tokens).
Each planted mistake below must fail one of them.
"""

import random

import numpy as np
import pytest

from oracle import (RefBlockManager, RefScheduler, ref_copy_blocks, ref_swap_in, ref_swap_out,
                    ref_write_kv)
from oracle.block_manager import OutOfBlocks
from tests.sched_steps import commit_step, device_ops, run_script, run_timeline

SCRIPTS = ["cb_preempt_swap.json", "cb_preempt_recompute.json", "cb_victim.json"]


def make(spec, cls=RefScheduler):
    bm = RefBlockManager(spec["num_blocks"], spec["block_size"],
                         spec.get("enable_prefix_cache", True))
    return cls(bm, spec["max_batch"], spec["host_slots"])


def test_timeline(golden):
    spec = golden("cb_timeline.json")
    run_timeline(make(spec), spec)


@pytest.mark.parametrize("name", SCRIPTS)
def test_preemption_scripts(golden, name):
    spec = golden(name)
    run_script(make(spec), spec)


def _fp(tokens):
    """Fingerprint of the token at position len(tokens) - 1 of a request
    with these tokens: its position, its id and a hash of its prefix."""
    h = 0
    for t in tokens:
        h = (h * 1000003 + t + 1) % (1 << 31)
    return (len(tokens) - 1, tokens[-1], h)


class TokenCache:
    """One-layer cache whose K row of a token is its fingerprint (V the
    negation), driven through the oracle's copies in plan order."""

    def __init__(self, nb, bs, host):
        self.k = [np.full((nb, bs, 1, 3), -1, dtype=np.int64)]
        self.v = [np.full((nb, bs, 1, 3), -1, dtype=np.int64)]
        self.host = np.zeros((max(host, 1), 1, 2, bs, 1, 3), dtype=np.int64)

    def _write(self, slots, rows):
        rows = np.array(rows, dtype=np.int64).reshape(len(rows), 1, 3)
        ref_write_kv(self.k[0], self.v[0], rows, -rows, slots, inplace=True)

    def play(self, plan, reqs):
        for kind, a, b in device_ops(plan):
            if kind == "swap_in":
                recs, blocks = zip(*plan["swap_in"][a:b])
                ref_swap_in(self.k, self.v, blocks, self.host[list(recs)], inplace=True)
            elif kind == "prefill":
                for rid, slots in plan["prefill"][a:b]:
                    toks = reqs[rid].tokens
                    first = len(toks) - len(slots)
                    self._write(slots, [_fp(toks[:p + 1]) for p in range(first, len(toks))])
            elif kind == "cow":
                ref_copy_blocks(self.k, self.v, plan["cow"][a:b], inplace=True)
            elif kind == "writes":
                self._write(plan["slots"][a:b], [_fp(reqs[r].tokens) for r in plan["writes"][a:b]])
            else:
                blocks, recs = zip(*plan["swap_out"][a:b])
                self.host[list(recs)] = ref_swap_out(self.k, self.v, blocks)

    def check(self, bm, rid, tokens):
        for p in range(len(tokens)):
            s = bm.slot(rid, p)
            want = np.array(_fp(tokens[:p + 1]))
            assert np.array_equal(self.k[0].reshape(-1, 3)[s], want), (rid, p)
            assert np.array_equal(self.v[0].reshape(-1, 3)[s], -want), (rid, p)


def _requests(sc):
    return {r.id: r for r in list(sc.running) + list(sc.waiting) + list(sc.swapped)}


def random_run(cls, seed, nb, bs, batch, host, prefix, n_req=40, max_steps=4000):
    rng = random.Random(seed)
    bm = RefBlockManager(nb, bs, prefix)
    sc = cls(bm, batch, host)
    cache = TokenCache(nb, bs, host)
    budget, produced = {}, {}
    shared = [rng.randrange(50) for _ in range(3 * bs)]
    nxt, stats = 1, {"preempted": 0, "recomputed": 0, "swapped_in": 0, "hits": 0,
                     "appended_victim": 0, "decode_only": 0}
    for step in range(1, max_steps + 1):
        while nxt <= n_req and rng.random() < 0.3:
            n = rng.randrange(1, 3 * bs)
            prompt = (shared[:rng.randrange(0, 3 * bs)] + [rng.randrange(50) for _ in range(n)])
            budget[nxt] = rng.randrange(1, 4 * bs)
            sc.add_request(nxt, prompt, budget[nxt])
            nxt += 1
        plan = sc.step()
        reqs = _requests(sc)
        cache.play(plan, reqs)
        for rid in plan["batch"]:
            cache.check(bm, rid, reqs[rid].tokens)
        stats["appended_victim"] += len(set(plan["preempted"]) & set(plan["writes"]))
        stats["decode_only"] += len(set(plan["batch"]) - set(plan["writes"]))
        for rid in plan["finished"]:
            assert produced[rid] == budget[rid]
        stats["preempted"] += len(plan["preempted"])
        stats["recomputed"] += len(plan["recomputed"])
        stats["swapped_in"] += len(plan["resumed"])
        for rid, slots in plan["prefill"]:
            if rid not in plan["preempted"]:        # admitted, then preempted in the step
                stats["hits"] += bm.num_cached_tokens(rid) > 0
        st = sc.state()
        assert len(st["running"]) <= batch
        held = sum(len(h) for _, h in st["swapped"])
        assert held + len(st["host_free"]) == host
        assert sorted(st["host_free"] + [x for _, h in st["swapped"] for x in h]) == list(range(host))
        bm.check_invariants()
        for rid in sc.to_commit:
            produced[rid] = produced.get(rid, 0) + 1
        commit_step(sc, step)
        if nxt > n_req and not st["running"] and not st["waiting"] and not st["swapped"]:
            break
    else:
        raise AssertionError("requests did not drain")
    assert set(produced) == set(budget) and all(produced[r] == budget[r] for r in budget)
    assert bm.num_free_blocks == nb
    return stats


@pytest.mark.parametrize("seed,nb,bs,batch,host,prefix",
                         [(0, 12, 4, 4, 16, True), (1, 10, 2, 5, 6, True), (2, 16, 4, 6, 0, True),
                          (3, 9, 3, 4, 40, False)])
def test_random_streams_drain(seed, nb, bs, batch, host, prefix):
    stats = random_run(RefScheduler, seed, nb, bs, batch, host, prefix)
    assert stats["preempted"] > 0 and stats["appended_victim"] > 0
    if host:
        assert stats["swapped_in"] > 0 and stats["decode_only"] > 0
    if host < 16:
        assert stats["recomputed"] > 0
    if prefix:
        assert stats["hits"] > 0


# ---- planted mistakes ------------------------------------------------------

class AdmitBeforeFinish(RefScheduler):
    """Mistake: finished requests leave only after admission (the batch is
    one short for a step)."""
    def step(self):
        done = [r for r in self.running if r.generated >= r.max_new]
        for r in done:
            r.max_new += 10 ** 9            # hide them from the finish phase
        plan = super().step()
        for r in done:
            r.max_new -= 10 ** 9
        return plan


class LifoAdmission(RefScheduler):
    """Mistake: the newest waiting request is admitted first."""
    def add_request(self, rid, prompt, max_new_tokens):
        super().add_request(rid, prompt, max_new_tokens)
        self.waiting.rotate(1)


class FewestGeneratedVictim(RefScheduler):
    """Mistake: the victim is the request with the fewest generated tokens."""
    @staticmethod
    def _choose_victim(running, plan):
        return min(running, key=lambda x: x.generated)


class NotAppendedVictim(RefScheduler):
    """Mistake: the victim is taken only among running requests that have
    neither appended nor been admitted in this step (a narrower set than
    the page's max over every running request)."""
    @staticmethod
    def _choose_victim(running, plan):
        done = set(plan["writes"]) | set(plan["admitted"])
        return max((x for x in running if x.id not in done), key=lambda x: x.generated)


class SwapOutFirst(RefScheduler):
    """Mistake: every swap-out is ordered before the step's copies and
    writes (a victim's own write would then land after its blocks left,
    and a block it frees could be rewritten before it is copied out)."""
    def step(self):
        plan = super().step()
        plan["cuts"] = [[0, 0, c[2]] for c in plan["cuts"]]
        return plan


class NewBeforeSwapped(RefScheduler):
    """Mistake: waiting requests are admitted before swapped ones resume."""
    def step(self):
        keep, self.swapped = self.swapped, type(self.swapped)()
        admitted_first = []
        orig_running = len(self.running)
        plan = super().step()
        self.swapped = keep
        return plan if not keep else self._resume_late(plan, admitted_first, orig_running)

    def _resume_late(self, plan, *_):
        while self.swapped and len(self.running) < self.max_batch:
            r = self.swapped[0]
            try:
                table, first = self.bm.swap_in(r.id)
            except OutOfBlocks:
                break
            self.swapped.popleft()
            plan["swap_in"] += list(zip(r.host[first:], table[first:]))
            self.host_free.extend(r.host)
            r.host = []
            self.running.append(r)
            plan["resumed"].append(r.id)
        return plan


MISTAKES = [
    (AdmitBeforeFinish, "cb_timeline.json"),
    (LifoAdmission, "cb_timeline.json"),
    (FewestGeneratedVictim, "cb_victim.json"),
    (NotAppendedVictim, "cb_victim.json"),
    (NotAppendedVictim, "cb_preempt_swap.json"),
    (SwapOutFirst, "cb_victim.json"),
    (NewBeforeSwapped, "cb_preempt_swap.json"),
]


@pytest.mark.parametrize("mutant,name", MISTAKES, ids=[f"{m.__name__}-{n}" for m, n in MISTAKES])
def test_mistake_is_caught(mutant, name, golden):
    spec = golden(name)
    run = run_timeline if "timeline" in name else run_script
    run(make(spec), spec)                          # the oracle passes ...
    with pytest.raises((AssertionError, ValueError, KeyError, RuntimeError)):
        run(make(spec, mutant), spec)              # ... the planted mistake fails


def test_swap_out_first_breaks_the_token_cache():
    """The device-order mistake also fails the fingerprint check on a
    random stream (a victim's own write or a reused block lands out of
    order), not only the golden script's cut values."""
    with pytest.raises(AssertionError):
        random_run(SwapOutFirst, 0, 12, 4, 4, 16, True)

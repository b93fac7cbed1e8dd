"""Python view of the library's continuous-batching scheduler (pa_sched_*).

Argument marshalling only: every decision (finish, resume, admit, append,
preempt) is made by the C++ scheduler behind the C ABI.
"""

import ctypes

import numpy as np

from ._lib import P_i32, P_i64, check, lib


def plan_lists(a):
    """A plan from step_arrays() as plain lists (pairs and cuts as lists of
    lists, prompt slots grouped per admitted request)."""
    prefill, o = [], 0
    for rid, n in zip(a["admitted"].tolist(), a["prefill_counts"].tolist()):
        prefill.append((rid, a["prefill_slots"][o:o + n].tolist()))
        o += n
    return {
        "finished": a["finished"].tolist(), "resumed": a["resumed"].tolist(),
        "admitted": a["admitted"].tolist(), "preempted": a["preempted"].tolist(),
        "recomputed": a["recomputed"].tolist(),
        "swap_in": [tuple(x) for x in a["swap_in"].tolist()],
        "swap_out": [tuple(x) for x in a["swap_out"].tolist()], "prefill": prefill,
        "writes": a["writes"].tolist(), "slots": a["slots"].tolist(),
        "cow": [tuple(x) for x in a["cow"].tolist()], "cuts": a["cuts"].tolist(),
        "batch": a["batch"].tolist(),
    }


class Plan(ctypes.Structure):
    """Mirror of pa_sched_plan (field order and types as in pagedkv.h)."""
    _fields_ = [
        ("ids_cap", ctypes.c_int32), ("pairs_cap", ctypes.c_int32), ("prefill_cap", ctypes.c_int32),
        ("finished", P_i64), ("n_finished", ctypes.c_int32),
        ("resumed", P_i64), ("n_resumed", ctypes.c_int32),
        ("admitted", P_i64), ("n_admitted", ctypes.c_int32),
        ("preempted", P_i64), ("n_preempted", ctypes.c_int32),
        ("recomputed", P_i64), ("n_recomputed", ctypes.c_int32),
        ("swap_in", P_i32), ("n_swap_in", ctypes.c_int32),
        ("swap_out", P_i32), ("n_swap_out", ctypes.c_int32),
        ("prefill_slots", P_i64), ("n_prefill_slots", ctypes.c_int32),
        ("prefill_counts", P_i32),
        ("writes", P_i64), ("slots", P_i64), ("n_writes", ctypes.c_int32),
        ("cow_pairs", P_i32), ("n_cow", ctypes.c_int32),
        ("cuts", P_i32),
        ("batch", P_i64), ("n_batch", ctypes.c_int32),
    ]


class Scheduler:
    """Continuous batching with preemption over a :class:`BlockManager`
    ("qaqbuyan.com article 130", continuous-batching section).

    ``step()`` returns the plan as NumPy views of the scheduler's arrays
    (valid until the next step); ``commit`` hands in the step's tokens."""

    def __init__(self, bm, max_batch, host_slots):
        self.bm = bm                      # keeps the manager alive
        self._h = lib().pa_sched_create(bm._h, int(max_batch), int(host_slots))
        if not self._h:
            raise ValueError(lib().pa_last_error().decode())
        self.max_batch, self.host_slots = int(max_batch), int(host_slots)
        nb, bs = bm.num_blocks, bm.bs
        ids = max(self.max_batch, 1)
        pairs = max(self.host_slots, 1)
        self._arr = {
            "finished": np.empty(ids, np.int64), "resumed": np.empty(ids, np.int64),
            "admitted": np.empty(ids, np.int64), "preempted": np.empty(ids, np.int64),
            "recomputed": np.empty(ids, np.int64), "swap_in": np.empty((pairs, 2), np.int32),
            "swap_out": np.empty((pairs, 2), np.int32), "prefill_slots": np.empty(nb * bs, np.int64),
            "prefill_counts": np.empty(ids, np.int32), "writes": np.empty(ids, np.int64),
            "slots": np.empty(ids, np.int64), "cow_pairs": np.empty((ids, 2), np.int32),
            "cuts": np.empty((ids, 3), np.int32), "batch": np.empty(ids, np.int64),
        }
        p = Plan()
        p.ids_cap, p.pairs_cap, p.prefill_cap = ids, pairs, nb * bs
        for name, a in self._arr.items():
            setattr(p, name, a.ctypes.data_as(P_i64 if a.dtype == np.int64 else P_i32))
        self._plan = p
        self.to_commit = set()

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            lib().pa_sched_destroy(h)
            self._h = None

    def add_request(self, rid, prompt, max_new_tokens):
        toks = np.ascontiguousarray(prompt, dtype=np.int32)
        check(lib().pa_sched_add_request(self._h, int(rid), toks.ctypes.data_as(P_i32), len(toks),
                                         int(max_new_tokens)))

    def step_arrays(self):
        """Run one step; returns the plan as NumPy views (engine use)."""
        p = self._plan
        check(lib().pa_sched_step(self._h, ctypes.addressof(p)))
        a = self._arr
        out = {
            "finished": a["finished"][:p.n_finished], "resumed": a["resumed"][:p.n_resumed],
            "admitted": a["admitted"][:p.n_admitted], "preempted": a["preempted"][:p.n_preempted],
            "recomputed": a["recomputed"][:p.n_recomputed], "swap_in": a["swap_in"][:p.n_swap_in],
            "swap_out": a["swap_out"][:p.n_swap_out],
            "prefill_slots": a["prefill_slots"][:p.n_prefill_slots],
            "prefill_counts": a["prefill_counts"][:p.n_admitted],
            "writes": a["writes"][:p.n_writes], "slots": a["slots"][:p.n_writes],
            "cow": a["cow_pairs"][:p.n_cow], "cuts": a["cuts"][:p.n_preempted],
            "batch": a["batch"][:p.n_batch],
        }
        self.to_commit = (set(out["batch"].tolist())
                          | (set(out["admitted"].tolist()) - set(out["preempted"].tolist())))
        return out

    def step(self):
        """Run one step; returns the plan with the oracle scheduler's keys
        and list values (parity tests)."""
        return plan_lists(self.step_arrays())

    def commit(self, tokens):
        """{request id: token} for every request of the last step's decode
        batch and every admission still running."""
        ids = np.fromiter(tokens.keys(), dtype=np.int64, count=len(tokens))
        toks = np.fromiter(tokens.values(), dtype=np.int32, count=len(tokens))
        check(lib().pa_sched_commit(self._h, ids.ctypes.data_as(P_i64), toks.ctypes.data_as(P_i32),
                                    len(ids)))
        self.to_commit = set()

    def state(self):
        """Observable state in the oracle scheduler's format."""
        h, n = self._h, ctypes.c_int32()
        check(lib().pa_sched_running(h, None, None, 0, ctypes.byref(n)))
        rid, gen = np.empty(max(n.value, 1), np.int64), np.empty(max(n.value, 1), np.int32)
        check(lib().pa_sched_running(h, rid.ctypes.data_as(P_i64), gen.ctypes.data_as(P_i32),
                                     n.value, ctypes.byref(n)))
        running = list(zip(rid[:n.value].tolist(), gen[:n.value].tolist()))
        check(lib().pa_sched_waiting(h, None, 0, ctypes.byref(n)))
        wid = np.empty(max(n.value, 1), np.int64)
        check(lib().pa_sched_waiting(h, wid.ctypes.data_as(P_i64), n.value, ctypes.byref(n)))
        waiting = wid[:n.value].tolist()
        check(lib().pa_sched_swapped(h, None, None, 0, None, 0, ctypes.byref(n)))
        k = max(self.host_slots, 1)
        sid, cnt, rec = np.empty(max(n.value, 1), np.int64), np.empty(max(n.value, 1), np.int32), np.empty(k, np.int32)
        check(lib().pa_sched_swapped(h, sid.ctypes.data_as(P_i64), cnt.ctypes.data_as(P_i32), n.value,
                                     rec.ctypes.data_as(P_i32), k, ctypes.byref(n)))
        swapped, o = [], 0
        for i in range(n.value):
            swapped.append((int(sid[i]), rec[o:o + cnt[i]].tolist()))
            o += int(cnt[i])
        check(lib().pa_sched_host_free(h, None, 0, ctypes.byref(n)))
        hf = np.empty(k, np.int32)
        check(lib().pa_sched_host_free(h, hf.ctypes.data_as(P_i32), k, ctypes.byref(n)))
        return {"waiting": waiting, "running": running, "swapped": swapped,
                "host_free": hf[:n.value].tolist()}

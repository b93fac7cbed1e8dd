"""Runs golden continuous-batching scripts against any scheduler object.

The scheduler must offer add_request(id, prompt, max_new_tokens), step() ->
plan dict, commit({id: token}), state() -> dict and the pending commit set
``to_commit``, with the oracle's semantics.  Plans are compared on the keys
a script lists (pairs as 2-element lists).
"""


def _norm(v):
    if isinstance(v, (list, tuple)):
        return [_norm(x) for x in v]
    return v


def commit_step(sched, step):
    """Tokens of a step: 100 + step for every request owed one."""
    sched.commit({i: 100 + step for i in sched.to_commit})


def run_timeline(sched, spec):
    names = [n for n, _ in spec["requests"]]
    ids = {n: i + 1 for i, n in enumerate(names)}
    inv = {i: n for n, i in ids.items()}
    for n, need in spec["requests"]:
        sched.add_request(ids[n], [ids[n] * 1000 + j for j in range(spec["prompt_len"])], need)
    for step in range(1, spec["steps"] + 1):
        plan = sched.step()
        commit_step(sched, step)
        exp = spec["expect"].get(str(step))
        if exp is None:
            continue
        st = sched.state()
        got_running = [[inv[i], g] for i, g in st["running"]]
        assert got_running == exp["running"], (step, got_running)
        assert [inv[i] for i in plan["finished"]] == exp.get("finished", []), step
        assert [inv[i] for i in plan["admitted"]] == exp.get("admitted", []), step


def run_script(sched, spec):
    """Requests are [id, prompt, max_new_tokens] or [..., arrival step]
    (added just before that step; default 1)."""
    for step, exp in enumerate(spec["steps"], start=1):
        for req in spec["requests"]:
            if (req[3] if len(req) > 3 else 1) == step:
                sched.add_request(req[0], req[1], req[2])
        plan = sched.step()
        for key in ("finished", "resumed", "admitted", "preempted", "recomputed", "swap_in",
                    "swap_out", "prefill", "writes", "slots", "cow", "cuts", "batch"):
            assert _norm(plan[key]) == exp.get(key, []), (step, key, plan[key])
        st = sched.state()
        if "host_free" in exp:
            assert st["host_free"] == exp["host_free"], (step, st["host_free"])
        if "waiting" in exp:
            assert st["waiting"] == exp["waiting"], (step, st["waiting"])
        commit_step(sched, step)


def device_ops(plan):
    """The step's device work in the order its decisions require: swap-in
    copies, prompt writes, then per preemption the copy-on-write copies and
    K/V writes of the appends made before it followed by its swap-out
    copies, then the rest of the copies and writes.  Yields (kind, a, b):
    entries [a, b) of plan["swap_in"], plan["prefill"] (requests),
    plan["cow"], plan["writes"] or plan["swap_out"]."""
    if plan["swap_in"]:
        yield "swap_in", 0, len(plan["swap_in"])
    if plan["prefill"]:
        yield "prefill", 0, len(plan["prefill"])
    w = c = s = 0
    for nw, nc, ns in list(plan["cuts"]) + [(len(plan["writes"]), len(plan["cow"]), None)]:
        if nc > c:
            yield "cow", c, nc
        if nw > w:
            yield "writes", w, nw
        w, c = nw, nc
        if ns is not None and ns > s:
            yield "swap_out", s, ns
            s = ns

"""Reference continuous-batching scheduler (test infrastructure; see
oracle/__init__).

Follows "qaqbuyan.com article 130", continuous-batching section: the step
timeline (a finished request leaves and a waiting one joins in the next
step, so the batch stays full) and ``ContinuousBatchingScheduler.step``
(1. drop finished requests and free their blocks; 2. admit waiting
requests first-come first-served until the batch is full or memory runs
short, putting the one that does not fit back at the front; 3. run the
batch; 4. append each request's new token, and when no block is left,
preempt: ``_preempt_request`` takes the running request with the most
generated tokens, copies its KV to CPU memory and frees its blocks).
Blocks come from the P06 block manager (``RefBlockManager``).

Readings where the page stops short (each also in the design notes):

* Token accounting follows the timeline: the step that admits a request
  runs its prompt and yields its first generated token; each later step
  appends the previous token (its K/V is written) and decodes the next one.
  A request with ``generated == max_new_tokens`` leaves at the start of the
  next step.  Tokens are handed in after each step with ``commit``.
* The appends run in running order over the list as it stood when they
  began; a request preempted earlier in the loop is skipped.  When an
  append finds no block, the victim is the page's: the request with the
  most generated tokens among all running requests (the first such in
  running order, as ``max`` does on the page's list), whether or not it
  has appended or was admitted in this step.  The failing request then
  tries again, until its append succeeds or it is the victim itself.
* Nothing is undone.  A victim that already appended keeps that token: its
  K/V is written before its blocks are copied out, and it is not decoded in
  this step.  A request whose last token is in the cache but not yet
  decoded (preempted after its append or after its admission, then swapped
  back in) joins a later step's decode batch without appending.
* The step's device work follows the order of the decisions: each
  preemption closes an epoch, and the copies and writes of the appends made
  before it precede its swap-out copies, while blocks it frees are reused
  only by later epochs.  ``plan["cuts"]`` holds, per preemption, the number
  of writes and copy-on-write pairs before it and the number of swap-out
  pairs through it.
* Preempted requests (swapped out) come back before new ones are admitted,
  oldest preemption first, through ``RefBlockManager.swap_in``.
* Host swap space is a pool of ``host_slots`` block-sized records handed out
  first-in first-out.  A victim whose blocks do not fit is recomputed
  instead: its blocks are freed and it returns to the front of the waiting
  queue with every token it has produced so far as its prompt; the prompt
  run on re-admission yields its next token.
* A request admitted in a step does not append in that step (its forward is
  the prompt run).
"""

from collections import deque

from .block_manager import OutOfBlocks


class _Req:
    __slots__ = ("id", "tokens", "max_new", "generated", "pending", "host")

    def __init__(self, rid, prompt, max_new):
        self.id = rid
        self.tokens = list(prompt)      # tokens the block manager holds
        self.max_new = max_new
        self.generated = 0              # tokens produced (committed)
        self.pending = None             # produced, not yet appended
        self.host = []                  # host records while swapped out


class RefScheduler:
    """Continuous batching over a ``RefBlockManager``."""

    def __init__(self, bm, max_batch, host_slots):
        if max_batch <= 0 or host_slots < 0:
            raise ValueError("max_batch must be positive, host_slots >= 0")
        self.bm = bm
        self.max_batch = max_batch
        self.waiting = deque()
        self.running = []
        self.swapped = deque()
        self.host_free = deque(range(host_slots))
        self.ids = set()
        self.to_commit = set()

    def add_request(self, rid, prompt, max_new_tokens):
        if rid in self.ids or not prompt or max_new_tokens < 1:
            raise ValueError("bad request")
        self.ids.add(rid)
        self.waiting.append(_Req(rid, prompt, max_new_tokens))

    @staticmethod
    def _choose_victim(running, plan):
        """article 130 _preempt_request: the running request with the most
        generated tokens (the first such in running order, as max() on the
        page's list), whatever this step's ``plan`` holds so far."""
        return max(running, key=lambda x: x.generated)

    def _preempt(self, victim, plan):
        """article 130 _preempt_request: KV to host memory, blocks freed."""
        need = len(self.bm.get_table(victim.id))
        self.running.remove(victim)
        plan["preempted"].append(victim.id)
        if need <= len(self.host_free):
            table = self.bm.swap_out(victim.id)
            victim.host = [self.host_free.popleft() for _ in table]
            plan["swap_out"] += list(zip(table, victim.host))
            self.swapped.append(victim)
        else:
            self.bm.free(victim.id)
            if victim.pending is not None:      # its K/V was never computed
                victim.tokens.append(victim.pending)
                victim.pending = None
            self.waiting.appendleft(victim)
            plan["recomputed"].append(victim.id)
        plan["cuts"].append([len(plan["writes"]), len(plan["cow"]), len(plan["swap_out"])])

    def step(self):
        """One step; returns the plan of host decisions and device copies."""
        if self.to_commit:
            raise RuntimeError("commit the previous step's tokens first")
        plan = {"finished": [], "resumed": [], "admitted": [], "preempted": [],
                "recomputed": [], "swap_in": [], "swap_out": [], "prefill": [],
                "writes": [], "slots": [], "cow": [], "cuts": [], "batch": []}
        # 1. finished requests leave; their blocks are freed.
        for r in list(self.running):
            if r.generated >= r.max_new:
                self.running.remove(r)
                self.bm.free(r.id)
                self.ids.discard(r.id)
                plan["finished"].append(r.id)
        # 2. preempted requests come back first, oldest first.
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
        # 3. admit waiting requests, first come first served.
        admitted = set()
        while self.waiting and len(self.running) < self.max_batch:
            r = self.waiting[0]
            try:
                self.bm.allocate(r.id, r.tokens)
            except OutOfBlocks:
                break
            self.waiting.popleft()
            c = self.bm.num_cached_tokens(r.id)
            plan["prefill"].append((r.id, [self.bm.slot(r.id, p) for p in range(c, len(r.tokens))]))
            self.running.append(r)
            admitted.add(r.id)
            plan["admitted"].append(r.id)
        # 4. append each running request's pending token, preempting the
        #    most-generated running request whenever no block is left.
        for r in list(self.running):
            if r.id in admitted or r.pending is None or r not in self.running:
                continue
            while True:
                try:
                    slot, cow = self.bm.append_slot(r.id, r.pending)
                except OutOfBlocks:
                    victim = self._choose_victim(self.running, plan)
                    self._preempt(victim, plan)
                    if victim is r:
                        break
                    continue
                r.tokens.append(r.pending)
                r.pending = None
                plan["writes"].append(r.id)
                plan["slots"].append(slot)
                if cow is not None:
                    plan["cow"].append(cow)
                break
        # The decode batch: every running request not admitted in this step
        # (each has its last token in the cache, appended now or earlier).
        plan["batch"] = [r.id for r in self.running if r.id not in admitted]
        self.to_commit = set(plan["batch"]) | (admitted & {r.id for r in self.running})
        return plan

    def commit(self, tokens):
        """Tokens produced by this step: {request id: token} for every
        request in the decode batch and every request admitted."""
        if set(tokens) != self.to_commit:
            raise ValueError("commit must cover exactly this step's batch and admissions")
        for r in self.running:
            if r.id in tokens:
                r.pending = tokens[r.id]
                r.generated += 1
        self.to_commit = set()

    # ----- queries -------------------------------------------------------
    def state(self):
        """Observable state, for comparison with another implementation."""
        return {
            "waiting": [r.id for r in self.waiting],
            "running": [(r.id, r.generated) for r in self.running],
            "swapped": [(r.id, list(r.host)) for r in self.swapped],
            "host_free": list(self.host_free),
        }

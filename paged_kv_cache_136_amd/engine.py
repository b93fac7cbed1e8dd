"""Continuous-batching decode loop on one GPU (orchestration only).

Each step asks the library's scheduler for a plan and performs its device
work through the library's calls, in the order the plan's decisions
require:

  1. swap-in copies (pa_swap_in) of resumed requests;
  2. prompt K/V writes (pa_write_kv) of admitted requests' uncached tokens,
     then, for the admitted requests still running, the prompt's attention
     over the uncached suffix (pa_prefill): after prefix hits only that
     suffix needs a forward pass ("P06 · BlockManager" spec overview and
     key-question answers);
  3. for each preemption, in order: the copy-on-write copies
     (pa_copy_blocks) and K/V writes (pa_write_kv) of the appends made
     before it, then its swap-out copies (pa_swap_out) -- a victim's own
     write lands before its blocks are copied out, and blocks it frees are
     written again only afterwards; then the remaining copies and writes;
  4. decode (pa_decode) of the batch, every layer.  When no preemption
     split the step's writes and the batch is exactly the requests that
     appended, in the same order (the usual step), each layer's writes of
     the batch's new tokens happen inside its decode instead
     (pa_write_decode, or pa_write_decode_shared with a plan: the token at
     position len - 1 is the one each of them appended), and step 3 is only
     the copies.  With ``shared_prefix``
     the host plans shared-prefix groups once per step (pa_shared_plan) and
     every layer decodes with pa_decode_shared, reading blocks that several
     sequences share (a common system prompt, forks) once per group -- when
     the plan saves at least ``shared_min_saving`` of the batch's block
     reads; below that the shared pass costs more than it saves (the
     repeated reads of a short common prefix mostly hit in L2), and the
     step decodes with pa_decode.

There is no model here: the caller supplies the K/V rows to write, the
queries and the sampled tokens through functions, so every value the
device computes comes from the library's kernels.  The step ends with a
stream synchronization, as a sampler reading the outputs would.
"""

import time

import numpy as np
import torch

from .block_manager import BlockManager
from .ops import (pa_copy_blocks, pa_decode, pa_decode_shared, pa_decode_shared_workspace_bytes,
                  pa_decode_workspace_bytes, pa_prefill, pa_shared_plan, pa_swap_in, pa_swap_out,
                  pa_write_decode, pa_write_decode_shared, pa_write_kv, swap_record_bytes)
from .scheduler import Scheduler


_TORCH_INT = {np.dtype(np.int32): torch.int32, np.dtype(np.int64): torch.int64}


class _Uploads:
    """A step's small host arrays (slots, tables, lengths, plans) uploaded
    through one pinned buffer: each upload fills the next piece of it and
    starts an asynchronous copy on the current stream, so the host keeps
    queueing work instead of waiting for each pageable copy to drain the
    GPU.  reset() makes the whole buffer free again once every copy of the
    previous step is done; a step that needs more grows it there.  A CPU
    device (host-only tests) uploads directly."""

    def __init__(self, dev, nbytes=1 << 20):
        self.dev = dev
        self.cuda = dev.type == "cuda"
        self.want = nbytes
        self.pin = None
        self.off = 0
        self.used = False
        self.done = torch.cuda.Event() if self.cuda else None

    def reset(self):
        if self.used:
            self.done.record()                # after everything queued so far
            self.done.synchronize()
            self.used = False
        if self.cuda and (self.pin is None or self.pin.numel() < self.want):
            self.pin = torch.empty(self.want, dtype=torch.uint8, pin_memory=True)
            self.pin_np = self.pin.numpy()
        self.off = 0

    def __call__(self, a, dtype):
        a = np.ascontiguousarray(a, dtype=dtype)
        if not self.cuda:
            return torch.from_numpy(a.copy())
        n = (a.nbytes + 255) & ~255
        if self.pin is None or self.off + n > self.pin.numel():
            self.want = max(self.want, 2 * (self.off + n))
            return torch.from_numpy(a.copy()).to(self.dev)     # this step only
        self.pin_np[self.off:self.off + a.nbytes].view(a.dtype)[:] = a.reshape(-1)
        src = self.pin[self.off:self.off + a.nbytes].view(_TORCH_INT[a.dtype]).view(a.shape)
        dst = torch.empty(a.shape, dtype=src.dtype, device=self.dev)
        dst.copy_(src, non_blocking=True)
        self.off += n
        self.used = True
        return dst


class DecodeEngine:
    """Paged KV caches (one K and one V tensor per layer, [num_blocks, bs,
    Hkv, D]), a block manager, a scheduler and a pinned host swap pool of
    ``host_slots`` block records."""

    def __init__(self, num_layers, num_blocks, block_size, num_kv_heads, num_q_heads, head_dim,
                 dtype, max_batch, host_slots, enable_prefix_cache=True, partition_tokens=512,
                 device="cuda", caches=None, shared_prefix=False, prompt_attention=True,
                 timing=False, shared_min_saving=0.25):
        self.L, self.nb, self.bs = num_layers, num_blocks, block_size
        self.hkv, self.hq, self.d, self.dtype = num_kv_heads, num_q_heads, head_dim, dtype
        self.dev = torch.device(device)
        self.partition_tokens = partition_tokens
        if shared_prefix and (dtype == torch.float32 or partition_tokens <= 0):
            raise ValueError("shared_prefix needs 16-bit caches and partition_tokens > 0")
        if prompt_attention and dtype == torch.float32:
            raise ValueError("prompt attention (pa_prefill) needs 16-bit caches")
        self.shared_prefix = shared_prefix
        self.shared_min_saving = shared_min_saving
        self.prompt_attention = prompt_attention
        self.shared_groups = 0           # groups decoded through a plan, summed over steps
        self.bm = BlockManager(num_blocks, block_size, enable_prefix_cache)
        self.sched = Scheduler(self.bm, max_batch, host_slots)
        if caches is None:
            shape = (num_blocks, block_size, num_kv_heads, head_dim)
            caches = ([torch.zeros(shape, dtype=dtype, device=self.dev) for _ in range(num_layers)],
                      [torch.zeros(shape, dtype=dtype, device=self.dev) for _ in range(num_layers)])
        self.k, self.v = caches
        self.record_bytes = swap_record_bytes(self.k)
        # Pinned, so the swap kernels can reach it (a host pool for a CPU
        # device only serves tests that stand in for the device calls).
        self.host = torch.empty(max(host_slots, 1) * self.record_bytes, dtype=torch.uint8,
                                pin_memory=self.dev.type == "cuda")
        self.ws = None                   # decode workspace, grown on demand
        self.folded_steps = 0            # steps whose batch writes ran inside the decode
        # The last step's context lengths of the decode batch (after its
        # appends, plan["batch"] order) and of the prompt-attention requests
        # (prompt_ids order); empty when there were none.
        self.last_decode_lens = np.zeros(0, np.int32)
        self.last_prompt_lens = np.zeros(0, np.int32)
        self.up = _Uploads(self.dev)
        self.step_no = 0
        self.host_seconds = 0.0          # time in scheduler / block-manager calls
        # With ``timing``, HIP events on the launch stream bracket the prompt
        # phase (writes and attention) and the decode phase of every step.
        self.timing = timing
        self.prompt_ms = 0.0
        self.decode_ms = 0.0

    def add_request(self, rid, prompt, max_new_tokens):
        self.sched.add_request(rid, prompt, max_new_tokens)

    def _i32(self, a):
        return self.up(a, np.int32)

    def _event(self):
        if not self.timing or self.dev.type != "cuda":
            return None
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def step(self, kv_rows, q_rows, sample):
        """One step.  ``kv_rows(layer, kind, plan)`` returns device K and V
        rows [n, Hkv, D]: for kind "prompt" one per entry of
        plan["prefill_slots"] (the admitted requests' uncached prompt tokens,
        request after request, plan["prefill_counts"] each), for "append"
        one per entry of plan["writes"] (the tokens appended in this step).
        ``q_rows(layer, kind, n)`` returns n queries [n, Hq, D]: for
        "prompt" one per prompt row of the requests in ``prompt_ids`` (the
        admitted requests still running, in admission order; their rows are
        their entries of plan["prefill_slots"]), for "decode" one per entry
        of plan["batch"].  ``sample(owed, outs, prompt_outs)``
        returns {id: token} for ``owed`` (the decode batch, then
        ``prompt_ids``) given the per-layer float32 decode outputs [B, Hq, D]
        and prompt-attention outputs [rows, Hq, D] (the last row of each
        request yields its first token).
        Returns (plan, outs, prompt_outs, prompt_ids)."""
        self.step_no += 1
        self.up.reset()
        h0 = time.perf_counter()
        plan = self.sched.step_arrays()
        self.host_seconds += time.perf_counter() - h0
        # 1. swap-in copies
        if len(plan["swap_in"]):
            pa_swap_in(self.k, self.v, self._i32(plan["swap_in"][:, 1]), self.host,
                       host_slots=self._i32(plan["swap_in"][:, 0]))
        # 2. prompt K/V of admitted requests, then their prompt attention
        e_p0 = self._event()
        prompt_outs, prompt_ids = self._prompts(plan, kv_rows, q_rows)
        e_p1 = self._event()
        # The decode's host work (tables, plan, uploads) needs only the
        # block manager's state after this step's appends, so it runs here,
        # while the GPU works through the prompts, rather than after the
        # short writes below, where the GPU would wait for it.
        dec = self._decode_prep(plan)
        # 3. copy-on-write copies, the appended tokens' K/V and swap-outs,
        #    epoch by epoch
        writes = plan["writes"]
        rows = [kv_rows(layer, "append", plan) for layer in range(self.L)] if len(writes) else None
        # The batch's writes fold into its decode when nothing orders them
        # against a swap-out and every decoded request appended exactly once.
        fold = (dec is not None and len(writes) > 0 and not len(plan["cuts"])
                and np.array_equal(writes, plan["batch"]))
        slots = self.up(plan["slots"], np.int64) if len(writes) and not fold else None
        w = c = so = 0
        for nw, nc, ns in plan["cuts"].tolist():
            self._cow_and_writes(plan, rows, slots, c, nc, w, nw)
            if ns > so:
                sw = plan["swap_out"][so:ns]
                pa_swap_out(self.k, self.v, self._i32(sw[:, 0]), self.host,
                            host_slots=self._i32(sw[:, 1]))
            w, c, so = nw, nc, ns
        self._cow_and_writes(plan, rows, slots, c, len(plan["cow"]), w,
                             w if fold else len(writes))
        # 4. decode every layer
        e_d0 = self._event()
        self.folded_steps += fold
        outs = self._decode(dec, q_rows, rows if fold else None)
        e_d1 = self._event()
        if self.dev.type == "cuda":
            torch.cuda.current_stream().synchronize()
        if e_p0 is not None:
            self.prompt_ms += e_p0.elapsed_time(e_p1)
            self.decode_ms += e_d0.elapsed_time(e_d1)
        owed = plan["batch"].tolist() + prompt_ids
        toks = sample(owed, outs, prompt_outs)
        h0 = time.perf_counter()
        self.sched.commit(toks)
        self.host_seconds += time.perf_counter() - h0
        return plan, outs, prompt_outs, prompt_ids

    def _prompts(self, plan, kv_rows, q_rows):
        self.last_prompt_lens = np.zeros(0, np.int32)
        if not len(plan["prefill_slots"]):
            return [], []
        slots = self.up(plan["prefill_slots"], np.int64)
        for layer in range(self.L):
            k, v = kv_rows(layer, "prompt", plan)
            pa_write_kv(self.k[layer], self.v[layer], k, v, slots)
        preempted = set(plan["preempted"].tolist())
        ids, counts = [], []
        for rid, n in zip(plan["admitted"].tolist(), plan["prefill_counts"].tolist()):
            if rid not in preempted:
                ids.append(rid)
                counts.append(n)
        if not ids or not self.prompt_attention:
            return [], ids
        h0 = time.perf_counter()
        tables, lens = self.bm.export_batch(ids, self._table_width(ids), pad_block=0)
        self.host_seconds += time.perf_counter() - h0
        self.last_prompt_lens = lens
        qstart = np.zeros(len(ids) + 1, dtype=np.int32)
        qstart[1:] = np.cumsum(counts)
        d_tab, d_len, d_qs = self._i32(tables), self._i32(lens), self._i32(qstart)
        outs = []
        for layer in range(self.L):
            outs.append(pa_prefill(q_rows(layer, "prompt", int(qstart[-1])), self.k[layer],
                                   self.v[layer], d_tab, d_qs, d_len, max(counts)))
        return outs, ids

    def _cow_and_writes(self, plan, rows, slots, c0, c1, w0, w1):
        if c1 > c0:
            pa_copy_blocks(self.k, self.v, self._i32(plan["cow"][c0:c1]))
        if w1 > w0:
            for layer in range(self.L):
                k, v = rows[layer]
                pa_write_kv(self.k[layer], self.v[layer], k[w0:w1], v[w0:w1], slots[w0:w1])

    def _decode_prep(self, plan):
        """Host side of the decode: the batch's tables and lengths, the
        shared-prefix plan if one pays, their uploads and the workspace."""
        ids = plan["batch"]
        self.last_decode_lens = np.zeros(0, np.int32)
        if not len(ids):
            return None
        B = len(ids)
        h0 = time.perf_counter()
        tables, lens = self.bm.export_batch(ids, self._table_width(ids), pad_block=0)
        self.last_decode_lens = lens
        splan = None
        if self.shared_prefix:
            plan = pa_shared_plan(tables, lens, self.bs, self.partition_tokens,
                                  self.hq // self.hkv)
            sg, groups, mx, mp = plan
            # block reads the plan saves: (members - 1) x shared blocks per group
            saved = int(((groups[:, 1:] >= 0).sum(axis=1) - 1) @ groups[:, 0]) if len(groups) else 0
            total = int((-(-lens.astype(np.int64) // self.bs)).sum())
            if len(groups) and saved >= self.shared_min_saving * total:
                self.shared_groups += len(groups)
                splan = (self._i32(sg), self._i32(groups), mx, mp, plan.max_private_blocks)
        self.host_seconds += time.perf_counter() - h0
        max_len = int(lens.max())
        d_tab, d_len = self._i32(tables), self._i32(lens)
        need = (pa_decode_shared_workspace_bytes if splan is not None else pa_decode_workspace_bytes)(
            B, self.hq, self.d, max_len, self.partition_tokens)
        if need and (self.ws is None or self.ws.numel() < need):
            self.ws = torch.empty(2 * need, dtype=torch.uint8, device=self.dev)
        return B, d_tab, d_len, max_len, splan

    def _decode(self, dec, q_rows, rows=None):
        """Every layer's decode; ``rows`` (per layer, the batch's new K/V
        rows in batch order) makes it write them first."""
        outs = []
        if dec is None:
            return outs
        B, d_tab, d_len, max_len, splan = dec
        for layer in range(self.L):
            q = q_rows(layer, "decode", B)
            if rows is not None and splan is None:
                k, v = rows[layer]
                outs.append(pa_write_decode(q, self.k[layer], self.v[layer], k, v, d_tab, d_len,
                                            max_len, partition_tokens=self.partition_tokens,
                                            workspace=self.ws))
            elif rows is not None:
                k, v = rows[layer]
                outs.append(pa_write_decode_shared(
                    q, self.k[layer], self.v[layer], k, v, d_tab, d_len, max_len, *splan[:4],
                    max_private_blocks=splan[4], partition_tokens=self.partition_tokens,
                    workspace=self.ws))
            elif splan is None:
                outs.append(pa_decode(q, self.k[layer], self.v[layer], d_tab, d_len, max_len,
                                      partition_tokens=self.partition_tokens, workspace=self.ws))
            else:
                outs.append(pa_decode_shared(q, self.k[layer], self.v[layer], d_tab, d_len, max_len,
                                             *splan[:4], max_private_blocks=splan[4],
                                             partition_tokens=self.partition_tokens,
                                             workspace=self.ws))
        return outs

    def _table_width(self, ids):
        return max(-(-self.bm.seq_len(int(i)) // self.bs) for i in ids)

    def idle(self):
        st = self.sched.state()
        return not st["running"] and not st["waiting"] and not st["swapped"]

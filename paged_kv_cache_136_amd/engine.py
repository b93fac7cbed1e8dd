"""Continuous-batching decode loop on one GPU (orchestration only).

Each step asks the library's scheduler for a plan and performs its device
work through the library's calls, in the order the plan requires:

  1. swap-in copies (pa_swap_in) of resumed requests;
  2. prompt K/V writes (pa_write_kv) of admitted requests' uncached tokens;
  3. swap-out copies (pa_swap_out) of preempted requests;
  4. copy-on-write copies (pa_copy_blocks);
  5. the batch's K/V writes (pa_write_kv) at the appended slots;
  6. decode (pa_decode) of the batch, every layer; with ``shared_prefix``
     the host plans shared-prefix groups once per step (pa_shared_plan) and
     every layer decodes with pa_decode_shared, reading blocks that several
     sequences share (a common system prompt, forks) once per group.

There is no model here: the caller supplies the K/V rows to write, the
queries and the sampled tokens through functions, so every value the
device computes comes from the library's kernels.  The step ends with a
stream synchronization, as a sampler reading the outputs would.
"""

import time

import numpy as np
import torch

from .block_manager import BlockManager
from .ops import (pa_copy_blocks, pa_decode, pa_decode_shared, pa_decode_workspace_bytes,
                  pa_shared_plan, pa_swap_in, pa_swap_out, pa_write_kv, swap_record_bytes)
from .scheduler import Scheduler


class DecodeEngine:
    """Paged KV caches (one K and one V tensor per layer, [num_blocks, bs,
    Hkv, D]), a block manager, a scheduler and a pinned host swap pool of
    ``host_slots`` block records."""

    def __init__(self, num_layers, num_blocks, block_size, num_kv_heads, num_q_heads, head_dim,
                 dtype, max_batch, host_slots, enable_prefix_cache=True, partition_tokens=512,
                 device="cuda", caches=None, shared_prefix=False):
        self.L, self.nb, self.bs = num_layers, num_blocks, block_size
        self.hkv, self.hq, self.d, self.dtype = num_kv_heads, num_q_heads, head_dim, dtype
        self.dev = torch.device(device)
        self.partition_tokens = partition_tokens
        if shared_prefix and (dtype == torch.float32 or partition_tokens <= 0):
            raise ValueError("shared_prefix needs 16-bit caches and partition_tokens > 0")
        self.shared_prefix = shared_prefix
        self.shared_groups = 0           # groups planned, summed over steps
        self.bm = BlockManager(num_blocks, block_size, enable_prefix_cache)
        self.sched = Scheduler(self.bm, max_batch, host_slots)
        if caches is None:
            shape = (num_blocks, block_size, num_kv_heads, head_dim)
            caches = ([torch.zeros(shape, dtype=dtype, device=self.dev) for _ in range(num_layers)],
                      [torch.zeros(shape, dtype=dtype, device=self.dev) for _ in range(num_layers)])
        self.k, self.v = caches
        self.record_bytes = swap_record_bytes(self.k)
        self.host = torch.empty(max(host_slots, 1) * self.record_bytes, dtype=torch.uint8,
                                pin_memory=True)
        self.ws = None                   # decode workspace, grown on demand
        self.step_no = 0
        self.host_seconds = 0.0          # time in scheduler / block-manager calls

    def add_request(self, rid, prompt, max_new_tokens):
        self.sched.add_request(rid, prompt, max_new_tokens)

    def _i32(self, a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(self.dev)

    def step(self, kv_rows, q_rows, sample):
        """One step.  ``kv_rows(layer, kind, plan)`` returns device K and V
        rows [n, Hkv, D]: for kind "prefill" one per entry of
        plan["prefill_slots"] (the admitted requests' uncached prompt
        tokens, request after request, plan["prefill_counts"] each), for
        "decode" one per entry of plan["batch"].  ``q_rows(layer, plan)``
        returns the batch's queries [B, Hq, D].  ``sample(owed, outs)``
        returns {id: token} for ``owed`` (the batch, then the admitted
        requests) given the per-layer float32 decode outputs [B, Hq, D].
        Returns (plan, outs)."""
        self.step_no += 1
        h0 = time.perf_counter()
        plan = self.sched.step_arrays()
        self.host_seconds += time.perf_counter() - h0
        # 1. swap-in copies
        if len(plan["swap_in"]):
            pa_swap_in(self.k, self.v, self._i32(plan["swap_in"][:, 1]), self.host,
                       host_slots=self._i32(plan["swap_in"][:, 0]))
        # 2. prompt K/V of admitted requests
        if len(plan["prefill_slots"]):
            slots = torch.from_numpy(plan["prefill_slots"].copy()).to(self.dev)
            for layer in range(self.L):
                k, v = kv_rows(layer, "prefill", plan)
                pa_write_kv(self.k[layer], self.v[layer], k, v, slots)
        # 3. swap-out copies
        if len(plan["swap_out"]):
            pa_swap_out(self.k, self.v, self._i32(plan["swap_out"][:, 0]), self.host,
                        host_slots=self._i32(plan["swap_out"][:, 1]))
        # 4. copy-on-write
        if len(plan["cow"]):
            pa_copy_blocks(self.k, self.v, self._i32(plan["cow"]))
        # 5-6. the batch: new tokens' K/V, then decode every layer
        ids = plan["batch"].copy()
        outs = []
        if len(ids):
            B = len(ids)
            slots = torch.from_numpy(plan["slots"].copy()).to(self.dev)
            h0 = time.perf_counter()
            tables, lens = self.bm.export_batch(ids, self._table_width(ids), pad_block=0)
            splan = None
            if self.shared_prefix:
                sg, groups, mx, mp = pa_shared_plan(tables, lens, self.bs, self.partition_tokens,
                                                    self.hq // self.hkv)
                self.shared_groups += len(groups)
                if len(groups):
                    splan = (torch.from_numpy(sg).to(self.dev),
                             torch.from_numpy(groups).to(self.dev), mx, mp)
            self.host_seconds += time.perf_counter() - h0
            max_len = int(lens.max())
            d_tab = torch.from_numpy(tables).to(self.dev)
            d_len = torch.from_numpy(lens).to(self.dev)
            need = pa_decode_workspace_bytes(B, self.hq, self.d, max_len, self.partition_tokens)
            if need and (self.ws is None or self.ws.numel() < need):
                self.ws = torch.empty(2 * need, dtype=torch.uint8, device=self.dev)
            for layer in range(self.L):
                k, v = kv_rows(layer, "decode", plan)
                pa_write_kv(self.k[layer], self.v[layer], k, v, slots)
                if splan is None:
                    outs.append(pa_decode(q_rows(layer, plan), self.k[layer], self.v[layer], d_tab,
                                          d_len, max_len, partition_tokens=self.partition_tokens,
                                          workspace=self.ws))
                else:
                    outs.append(pa_decode_shared(q_rows(layer, plan), self.k[layer], self.v[layer],
                                                 d_tab, d_len, max_len, *splan,
                                                 partition_tokens=self.partition_tokens,
                                                 workspace=self.ws))
        torch.cuda.current_stream().synchronize()
        owed = ids.tolist() + plan["admitted"].tolist()
        toks = sample(owed, outs)
        h0 = time.perf_counter()
        self.sched.commit(toks)
        self.host_seconds += time.perf_counter() - h0
        return plan, outs

    def _table_width(self, ids):
        return max(-(-self.bm.seq_len(int(i)) // self.bs) for i in ids)

    def idle(self):
        st = self.sched.state()
        return not st["running"] and not st["waiting"] and not st["swapped"]

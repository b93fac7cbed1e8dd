#!/usr/bin/env python3
"""Paged decode step throughput on one MI355X.

Default workload: the mixed-length batch of the Llama-7B shape (32 layers x
32 KV heads x 128 dims, fp16, block size 16, 128 sequences with lengths
log-uniform in [50, 4096], a 16384-block pool scattered by a seeded
permutation).  One step is one pass of the whole hot path:

  host   pa_bm_append_slots (one new token per sequence: slot, table growth)
         pa_bm_export_batch into a pinned staging buffer, one async upload
         (the block tables only when they changed)
  device pa_copy_blocks when appends report copy-on-write pairs (none in
         this workload), then for each layer pa_write_decode: the new
         token's K/V written to its slot and the split-KV decode over it
         (phase 1 + reduce) in one call; --separate-write times pa_write_kv
         then pa_decode instead

Sequences grow by one token per step, as in real decoding; the KV bytes of
every step are counted exactly.  The metric is achieved KV GB/s (valid
tokens' K and V bytes read per second, whole job) with seqs/s beside it.

Prints one JSON line.  --gpus N with N > 1 exits: the library runs on one GPU.
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, published
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "paged_kv_cache_136_amd", "csrc")
DECODE_SRC = os.path.join(CSRC, "decode.hip")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="mixed_7b",
                   choices=["mixed_7b", "tiny", "13b_layer", "gqa_long", "fork_cow", "swap", "serve",
                            "beam", "prefill", "prefill_gqa"],
                   help="mixed_7b is the headline workload; the others are reported lines")
    p.add_argument("--shared-prefix", choices=["on", "off"], default=None,
                   help="serve: decode with pa_decode_shared (default: the workload's choice)")
    p.add_argument("--partition-tokens", type=int, default=-1,
                   help="split-KV partition size (default: the workload's, 512)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target CPU time of the oracle baseline sample (0 = skip)")
    p.add_argument("--calibrate", action="store_true",
                   help="instead of the step: run pa_copy_blocks over a known number of "
                        "bytes (3 launches of 8192 x 128 KiB blocks, K and V) and "
                        "pa_stream_read over 8 GiB (3 launches), for scaling rocprofv3 "
                        "FETCH_SIZE / WRITE_SIZE readings")
    p.add_argument("--read-gib", type=int, default=8,
                   help="size of the streaming-read ceiling measurement (0 = skip)")
    p.add_argument("--separate-write", action="store_true",
                   help="decode, fork and beam lines: pa_write_kv then pa_decode (or "
                        "pa_decode_shared) instead of pa_write_decode "
                        "(pa_write_decode_shared)")
    return p.parse_args()


def calibrate():
    """pa_copy_blocks over 8192 disjoint block pairs of 128 KiB in one layer's
    K and V: each launch reads and writes exactly 2 * 8192 * 128 KiB = 2 GiB.
    Then pa_stream_read over 8 GiB: each launch reads exactly 8 GiB and
    writes nothing."""
    import torch

    import paged_kv_cache_136_amd as pkv

    nb, block = 16384, (16, 32, 128)
    k = torch.zeros((nb, *block), dtype=torch.float16, device="cuda")
    v = torch.zeros_like(k)
    pairs = torch.stack([torch.arange(0, 8192), torch.arange(8192, 16384)], 1).int().cuda()
    for _ in range(3):
        pkv.pa_copy_blocks([k], [v], pairs)
    torch.cuda.synchronize()
    nbytes = 2 * 8192 * k[0].numel() * k.element_size()
    del k, v
    buf = torch.zeros(8 << 30, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    for _ in range(3):
        pkv.pa_stream_read(buf, 4096, sink)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": ["pa_copy_blocks", "pa_stream_read"], "launches": 3,
                      "copy_read_bytes_per_launch": nbytes, "copy_write_bytes_per_launch": nbytes,
                      "stream_read_bytes_per_launch": 8 << 30}))


def stream_read_ceiling(torch, pkv, gib):
    """HBM read rate reachable on this GPU: pa_stream_read over a ``gib``
    GiB buffer (far above the 256 MB Infinity Cache) with 1024, 4096 and
    16384 workgroups, 2 untimed then 5 timed launches each (HIP events);
    the best median.  Run after the timed steps, outside them."""
    if gib <= 0:
        return None
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(16384, dtype=torch.int32, device="cuda")
    T = torch.cuda.Event
    per = {}
    for wg in (1024, 4096, 16384):
        for _ in range(2):
            pkv.pa_stream_read(buf, wg, sink)
        ev = [(T(enable_timing=True), T(enable_timing=True)) for _ in range(5)]
        for a, b in ev:
            a.record()
            pkv.pa_stream_read(buf, wg, sink)
            b.record()
        torch.cuda.synchronize()
        per[wg] = nbytes / (float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    best = max(per, key=per.get)
    return {"gbs": round(per[best], 2), "bytes": nbytes, "workgroups": best,
            "by_workgroups": {str(k): round(v, 2) for k, v in per.items()},
            "kernel": "pa_stream_read (nontemporal 16-byte buffer loads, one contiguous "
                      "chunk per workgroup)"}


def with_ceiling(roofline, ceiling):
    """Adds the measured read ceiling and the achieved fraction of it."""
    if roofline is not None and ceiling is not None:
        roofline["measured_read_gbs"] = ceiling["gbs"]
        roofline["frac_of_measured_read"] = round(roofline["achieved"] / ceiling["gbs"], 4)
        roofline["measured_read"] = ceiling
    return roofline


def source_sha(path):
    """Fingerprint of a kernel source's code: its text without comments
    and blank lines, so that an edit to a comment does not mark the
    counters taken on the same code as stale."""
    with open(path, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def load_traffic(name):
    """HBM bytes per launch of a workload's dominant kernel from its
    committed rocprofv3 counter summary (profiles/<name>_pmc.json), or None
    if absent or taken on a different source of the kernel."""
    try:
        with open(os.path.join(PROFILES, name + "_pmc.json")) as f:
            pmc = json.load(f)
    except (OSError, ValueError):
        return None
    src = os.path.join(CSRC, pmc.get("source_file", "decode.hip"))
    sha = pmc.get("source_sha", pmc.get("decode_source_sha"))
    if not os.path.exists(src) or sha != source_sha(src):
        return None
    return pmc.get("traffic_bytes_per_launch")


TORCH_DTYPE_NAMES = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}


def cpu_baseline(lens, hq, hkv, D, bs, dtype, seconds, layers, workload):
    """The oracle timed on the host over one layer of the same workload
    shape (a prefix of the sequences, all heads), with fresh seeded inputs,
    repeated until about ``seconds``.  The sample's sequences are split
    over one thread per core this process may run on (at most 16), each
    calling the oracle on its share with BLAS limited to one thread."""
    import concurrent.futures

    import torch
    from threadpoolctl import threadpool_limits

    import oracle
    import workloads

    tdt = getattr(torch, TORCH_DTYPE_NAMES[dtype])
    # Bounded sample: the first sequences of the batch, up to ~150k tokens.
    cum = np.cumsum(lens)
    nseq = int(max(1, np.searchsorted(cum, 150_000, side="right")))
    lens = np.asarray(lens[:nseq])
    need = [-(-int(n) // bs) for n in lens]
    nblk = sum(need)
    order = workloads.block_order(nblk, seed=11)
    tables = np.zeros((len(lens), max(need)), dtype=np.int64)
    o = 0
    for i, k in enumerate(need):
        tables[i, :k] = order[o:o + k]
        o += k
    k = workloads.normal_torch((nblk, bs, hkv, D), 12, tdt, "cuda").float().cpu().numpy()
    v = workloads.normal_torch((nblk, bs, hkv, D), 13, tdt, "cuda").float().cpu().numpy()
    q = workloads.normal_torch((len(lens), hq, D), 14, tdt, "cuda").float().cpu().numpy()
    elem = workloads.ELEM_BYTES[dtype]
    sample_bytes = int(np.sum(lens)) * 2 * hkv * D * elem
    cores = max(1, min(16, len(os.sched_getaffinity(0)), len(lens)))

    def run_seq(b):
        oracle.ref_decode(q[b:b + 1], k, v, tables[b:b + 1], lens[b:b + 1])

    reps, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=1), concurrent.futures.ThreadPoolExecutor(cores) as ex:
        while True:
            list(ex.map(run_seq, range(len(lens))))
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": round(sample_bytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"one layer of the {workload} step restricted to its first {nseq} sequences "
                      f"({int(np.sum(lens))} tokens x {hq} query heads, fresh seeded {dtype} inputs), "
                      f"{reps} repetitions in {el:.1f} s, float64 NumPy, one sequence per task on "
                      f"{cores} threads, BLAS 1 thread each",
            "seqs_per_s": round(nseq * reps / el / layers, 4)}


class DecodeBench:
    """Device state and step of a decode workload (see the module doc)."""

    def __init__(self, name, args, torch, pkv, workloads):
        self.name, self.args, self.torch, self.pkv = name, args, torch, pkv
        cfg = workloads.CONFIGS[name]
        self.cfg = cfg
        dev = torch.device("cuda:0")
        self.L, self.hq, self.H, self.D = cfg["layers"], cfg["hq"], cfg["hkv"], cfg["d"]
        self.bs, self.NB, self.dtype = cfg["bs"], cfg["num_blocks"], cfg["dtype"]
        self.tdt = getattr(torch, TORCH_DTYPE_NAMES[self.dtype])
        self.elem = workloads.ELEM_BYTES[self.dtype]
        self.lens0 = workloads.lengths(name)                # include the step's new token
        B = self.B = len(self.lens0)
        S = args.warmup + args.steps
        self.max_len_final = int(self.lens0.max()) + S - 1
        self.max_blocks = -(-self.max_len_final // self.bs)
        self.partition = args.partition_tokens if args.partition_tokens >= 0 else cfg["partition_tokens"]

        # Host block manager: free list scrambled by a seeded permutation,
        # then each sequence admitted with its prompt (length - 1 tokens).
        self.bm = pkv.BlockManager(self.NB, self.bs, enable_prefix_cache=False)
        workloads.scramble_free_list(self.bm, workloads.block_order(self.NB, seed=1))
        toks = workloads.token_ids(int(self.lens0.max()), seed=2)
        for i in range(B):
            self.bm.allocate(i, toks[:int(self.lens0[i]) - 1])
        self.seqs = np.arange(B, dtype=np.int64)

        # Device inputs, resident in HBM: every layer's KV pool, and each
        # layer's query and new K/V rows.
        L, H, D, bs, NB = self.L, self.H, self.D, self.bs, self.NB
        self.pool = torch.empty((L, 2, NB, bs, H, D), dtype=self.tdt, device=dev)
        g = torch.Generator(device=dev)
        g.manual_seed(3)
        for layer in range(L):
            self.pool[layer].normal_(generator=g)
        self.q = workloads.normal_torch((L, B, self.hq, D), 4, self.tdt, dev)
        self.k_new = workloads.normal_torch((L, B, H, D), 5, self.tdt, dev)
        self.v_new = workloads.normal_torch((L, B, H, D), 6, self.tdt, dev)
        self.out = torch.empty((L, B, self.hq, D), dtype=torch.float32, device=dev)
        ws_bytes = pkv.pa_decode_workspace_bytes(B, self.hq, D, self.max_len_final, self.partition)
        self.ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        # The step's host outputs share one staging layout: [slots int64 B |
        # lens int32 B | pairs int32 B x 2 | tables int32 B x max_blocks].
        # One copy uploads the head of it every step, and the tables too
        # when they changed (a sequence crossed into a new block: once in
        # 16 steps per sequence), so the device keeps the last tables.  Two
        # pinned host buffers: the host fills one while the other's upload
        # may still be queued.
        self.stage_bytes = B * 8 + B * 4 + B * 2 * 4 + B * self.max_blocks * 4
        self.tab_off = self.stage_bytes - B * self.max_blocks * 4
        self.first_upload = True
        self.d_stage = torch.empty(self.stage_bytes, dtype=torch.uint8, device=dev)
        self.d_slot, self.d_tab, self.d_len, self.d_pairs = self._views(self.d_stage)
        self.pin = []
        for _ in range(2):
            buf = torch.empty(self.stage_bytes, dtype=torch.uint8).pin_memory()
            slot, tab, lens, pairs = self._views(buf)
            self.pin.append(dict(buf=buf, slot=slot, tab=tab, len=lens, pairs=pairs,
                                 ev=torch.cuda.Event()))
        for p in self.pin:
            p["ev"].record()
        self.new_tok = np.full(B, 7, dtype=np.int32)
        self.k_layers = [self.pool[layer, 0] for layer in range(L)]
        self.v_layers = [self.pool[layer, 1] for layer in range(L)]
        self.host_s = []
        torch.cuda.synchronize()

    def _views(self, buf):
        """(slots, tables, lens, pairs) views of one staging buffer."""
        torch, B, mb = self.torch, self.B, self.max_blocks
        o1 = B * 8
        o2 = o1 + B * 4
        o3 = o2 + B * 2 * 4
        return (buf[:o1].view(torch.int64), buf[o3:].view(torch.int32).view(B, mb),
                buf[o1:o2].view(torch.int32), buf[o2:o3].view(torch.int32).view(B, 2))

    def step(self, s, ev_pairs=None, ev_start=None, ev_end=None):
        """One step; ev_start, if given, is recorded after the host work,
        right before the step's first GPU operation (the upload), and ev_end
        after its last.  ev_pairs[layer] brackets that layer's pa_decode; the
        last layer's end is ev_end itself when given.  Every event record
        leaves the GPU idle for a few microseconds (the next dispatch waits
        for the marker), so the step records only these, and the staging
        buffer's reuse event goes at the end of the step rather than between
        the upload and the first kernel."""
        pkv, p = self.pkv, self.pin[s % 2]
        p["ev"].synchronize()                 # its previous upload has run
        h0 = time.perf_counter()
        slots, pairs = self.bm.append_slots(self.seqs, self.new_tok)
        p["slot"].numpy()[:] = slots
        self.bm.export_batch(self.seqs, self.max_blocks, 0, tables_out=p["tab"].numpy(),
                             lens_out=p["len"].numpy())
        self.host_s.append(time.perf_counter() - h0)
        if len(pairs):
            p["pairs"].numpy()[:len(pairs)] = pairs
        # A table changes only when a token opens a new block (its slot is
        # the block's first) or a copy-on-write replaces a block.
        changed = self.first_upload or len(pairs) > 0 or bool(np.any(slots % self.bs == 0))
        self.first_upload = False
        used = self.stage_bytes if changed else self.tab_off
        if ev_start is not None:
            ev_start.record()
        self.d_stage[:used].copy_(p["buf"][:used], non_blocking=True)
        if len(pairs):
            pkv.pa_copy_blocks(self.k_layers, self.v_layers, self.d_pairs[:len(pairs)])
        max_len = int(self.lens0.max()) + s
        for layer in range(self.L):
            if self.args.separate_write:
                pkv.pa_write_kv(self.k_layers[layer], self.v_layers[layer], self.k_new[layer],
                                self.v_new[layer], self.d_slot)
            if ev_pairs is not None:
                ev_pairs[layer][0].record()
            if self.args.separate_write:
                pkv.pa_decode(self.q[layer], self.k_layers[layer], self.v_layers[layer], self.d_tab,
                              self.d_len, max_len, partition_tokens=self.partition,
                              out=self.out[layer], workspace=self.ws)
            else:
                # the new token's slot is table[(len - 1) // 16] * 16 + (len - 1) % 16,
                # the one append_slots returned
                pkv.pa_write_decode(self.q[layer], self.k_layers[layer], self.v_layers[layer],
                                    self.k_new[layer], self.v_new[layer], self.d_tab, self.d_len,
                                    max_len, partition_tokens=self.partition,
                                    out=self.out[layer], workspace=self.ws)
            if ev_pairs is not None and not (layer == self.L - 1 and ev_end is not None):
                ev_pairs[layer][1].record()
        if ev_end is not None:
            ev_end.record()
        p["ev"].record()                      # the staging buffer may be refilled after this

    def run(self):
        """Time the steps.  Working sets under 4 GiB per step could be served
        partly from the 256 MB Infinity Cache across steps, so those steps
        are separated by a 1 GiB scratch write and timed with HIP events
        from the step's first to last GPU operation; larger ones are timed
        by the wall clock over all steps."""
        torch, args = self.torch, self.args
        per_token_layer = 2 * self.H * self.D * self.elem
        small = int(self.lens0.sum()) * per_token_layer * self.L < 4 * 2**30
        scratch = torch.empty(2**30, dtype=torch.uint8, device="cuda") if small else None
        for s in range(args.warmup):
            self.step(s)
        torch.cuda.synchronize()
        T = torch.cuda.Event
        # Per-launch events (two per layer) leave the GPU idle a few
        # microseconds each, so they ride on a few evenly spaced timed steps
        # only (all of their layers): about 64 launches, and at most every
        # fourth step.
        stride = max(4, args.steps // -(-64 // self.L))
        timed = [i for i in range(args.steps) if i % stride == stride - 1] or [args.steps - 1]
        step_ev = [(T(enable_timing=True), T(enable_timing=True)) for _ in range(args.steps)]
        events = {i: [(T(enable_timing=True), T(enable_timing=True)) for _ in range(self.L - 1)] +
                     [(T(enable_timing=True), step_ev[i][1])] for i in timed}
        self.host_s.clear()
        t0 = time.perf_counter()
        for i in range(args.steps):
            if small:
                scratch.fill_(i & 0xff)
            self.step(args.warmup + i, events.get(i), *step_ev[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        # The device's tables and lengths (uploaded only when changed) must
        # be the block manager's after the last step.
        tab_now, len_now = self.bm.export_batch(self.seqs, self.max_blocks, 0)
        if not (np.array_equal(self.d_tab.cpu().numpy(), tab_now) and
                np.array_equal(self.d_len.cpu().numpy(), len_now)):
            raise RuntimeError("device block tables differ from the block manager's")
        step_gpu_ms = np.array([a.elapsed_time(b) for a, b in step_ev])
        gpu_s = step_gpu_ms.sum() * 1e-3
        timed_s = gpu_s if small else wall
        step_tokens = [int(self.lens0.sum()) + self.B * (args.warmup + i) for i in range(args.steps)]
        kv_bytes = sum(step_tokens) * per_token_layer * self.L
        value = kv_bytes / timed_s / 1e9
        dec_ms = np.array([[a.elapsed_time(b) for a, b in events[i]] for i in timed])
        launch_bytes = np.array([step_tokens[i] for i in timed], dtype=np.float64) * per_token_layer
        achieved = float(launch_bytes.mean() / (dec_ms.mean() * 1e-3) / 1e9)
        cfg = self.cfg
        return {
            "metric": "paged decode attention: achieved KV GB/s (% of HBM peak) and seqs/s",
            "value": round(value, 2),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(timed_s / args.steps * 1e3, 4),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": self.dtype,
            "data": "synthetic",
            "config": {"workload": self.name, "layers": self.L, "batch": self.B,
                       "q_heads": self.hq, "kv_heads": self.H, "head_dim": self.D,
                       "block_size": self.bs, "num_blocks": self.NB,
                       "lengths": LENGTH_NOTES[self.name],
                       "mean_context": round(float(np.mean(step_tokens)) / self.B, 1),
                       "partition_tokens": self.partition,
                       "kv_write": "pa_write_kv, then pa_decode" if self.args.separate_write
                       else "in the decode call (pa_write_decode)",
                       "timing": "GPU events per step, 1 GiB cache flush between steps"
                                 if small else "wall clock over all steps"},
            "seqs_per_s": round(self.B * args.steps / timed_s, 1),
            "pct_hbm_peak": round(100 * value / PEAK_HBM_GBS, 2),
            "kv_bytes_per_step": int(kv_bytes // args.steps),
            "host_bm_ms_per_step": round(1e3 * float(np.mean(self.host_s)), 4),
            "gpu_step_ms_p10_p50_p90": [round(float(x), 4) for x in
                                        np.percentile(step_gpu_ms, [10, 50, 90])],
            "roofline": with_ceiling(
                {"kernel": "pa_decode (split-KV phase 1 + reduce), one layer" if self.args.separate_write
                 else "pa_write_decode (the new token's K/V write, split-KV phase 1 + reduce), one layer",
                 "bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                 "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                 "traffic": None if self.args.separate_write else load_traffic("pa_decode_" + self.name),
                 "avg_launch_ms": round(float(dec_ms.mean()), 5),
                 "algorithmic_bytes_per_launch": int(launch_bytes.mean())},
                stream_read_ceiling(torch, self.pkv, args.read_gib)),
        }


def run_fork_cow(args, torch, pkv, workloads):
    """Parallel sampling with copy-on-write: 64 prompts of 2048 tokens
    (prefix cache on), each parent appends one sampled token and forks 7
    children; every round all 512 sequences append one token.  The first
    round after the fork copies 7 shared, partly filled blocks per prompt
    (448 pa_copy_blocks pairs); rounds 2..255 are run untimed; the timed
    steps are then rounds of append + write + decode over 512 sequences of
    2305+ tokens.  Decode is pa_write_decode_shared (the appended tokens'
    K/V written in the same call; --separate-write: pa_write_kv, then
    pa_decode_shared) with a plan from pa_shared_plan made on the host every
    step (the 128 prompt blocks of a family are read once per family);
    plain pa_decode on the final batch is
    timed after the steps for comparison.  Reported: logical KV GB/s (every
    sequence's tokens) and GB/s over the unique blocks read, plus the COW
    round's copy kernel."""
    cfg = workloads.CONFIGS["fork_cow"]
    bs, NB, H, D = cfg["bs"], cfg["num_blocks"], cfg["hkv"], cfg["d"]
    P, F, L0, X = cfg["prompts"], cfg["forks"], cfg["prompt_len"], cfg["extra"]
    dev = torch.device("cuda:0")
    bm = pkv.BlockManager(NB, bs, True)
    k = workloads.normal_torch((NB, bs, H, D), 40, torch.float16, dev)
    v = workloads.normal_torch((NB, bs, H, D), 41, torch.float16, dev)
    for p in range(P):
        bm.allocate(p * F, workloads.token_ids(L0, seed=1000 + p))
    parents = np.arange(P, dtype=np.int64) * F
    seqs = np.array([p + c for p in parents for c in range(F)], dtype=np.int64)
    B = len(seqs)
    S = X + args.warmup + args.steps
    max_blocks = -(-(L0 + 1 + S) // bs)
    kn = workloads.normal_torch((B, H, D), 42, torch.float16, dev)
    vn = workloads.normal_torch((B, H, D), 43, torch.float16, dev)
    q = workloads.normal_torch((B, cfg["hq"], D), 44, torch.float16, dev)
    out = torch.empty((B, cfg["hq"], D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(pkv.pa_decode_shared_workspace_bytes(B, cfg["hq"], D, L0 + 1 + S, 512), 1),
                     dtype=torch.uint8, device=dev)
    tab_h = torch.empty((B, max_blocks), dtype=torch.int32).pin_memory()
    len_h = torch.empty(B, dtype=torch.int32).pin_memory()
    d_tab = torch.empty((B, max_blocks), dtype=torch.int32, device=dev)
    d_len = torch.empty(B, dtype=torch.int32, device=dev)

    def append(ids, toks):
        slots, pairs = bm.append_slots(ids, toks)
        d_slot = torch.from_numpy(slots).to(dev, non_blocking=False)
        d_pairs = torch.from_numpy(pairs).to(dev) if len(pairs) else None
        return d_slot, d_pairs, len(pairs)

    plan_s = []

    def prepare(shared=True):
        """Host part of a decode: tables and lengths exported and uploaded,
        and the shared-prefix plan made and uploaded.  Runs before a step's
        timed region, which holds GPU work only."""
        bm.export_batch(seqs, max_blocks, 0, tables_out=tab_h.numpy(), lens_out=len_h.numpy())
        d_tab.copy_(tab_h)
        d_len.copy_(len_h)
        if not shared:
            return None
        h0 = time.perf_counter()
        splan = pkv.pa_shared_plan(tab_h.numpy(), len_h.numpy(), bs, 512, 1)
        sg, groups, mx, mp = splan
        plan_s.append(time.perf_counter() - h0)
        return (torch.from_numpy(sg).to(dev), torch.from_numpy(groups).to(dev), mx, mp,
                splan.max_private_blocks)

    fold = not args.separate_write

    def decode(max_len, plan, ev=None, write=False):
        """The decode; with ``write``, the appended tokens' K/V written in
        the same call (their slots are the sequences' positions len - 1)."""
        if ev is not None:
            ev[0].record()
        if plan is not None and write:
            pkv.pa_write_decode_shared(q, k, v, kn, vn, d_tab, d_len, max_len, *plan[:4],
                                       max_private_blocks=plan[4], partition_tokens=512,
                                       out=out, workspace=ws)
        elif plan is not None:
            pkv.pa_decode_shared(q, k, v, d_tab, d_len, max_len, *plan[:4],
                                 max_private_blocks=plan[4], partition_tokens=512, out=out,
                                 workspace=ws)
        else:
            pkv.pa_decode(q, k, v, d_tab, d_len, max_len, partition_tokens=512, out=out,
                          workspace=ws)
        if ev is not None:
            ev[1].record()
        return 0 if plan is None else len(plan[1])

    T = torch.cuda.Event
    # Parent token, then the forks.
    d_slot, _, _ = append(parents, np.full(P, 7, dtype=np.int32))
    pkv.pa_write_kv(k, v, kn[:P], vn[:P], d_slot)
    for p in parents:
        for c in range(1, F):
            bm.fork(int(p), int(p) + c)
    torch.cuda.synchronize()
    # First append pass after the forks: the one with the copy-on-write copies, timed.
    toks = np.arange(B, dtype=np.int32)
    cow_ev, round_ev = (T(enable_timing=True), T(enable_timing=True)), (T(enable_timing=True), T(enable_timing=True))
    d_slot, d_pairs, npairs = append(seqs, toks)
    plan = prepare()
    # Untimed warm-up: as many copies between blocks at the top of the pool
    # (unused so far: the free list hands out ids in order), so the timed
    # round does not start on a GPU whose clock idled during the forks.
    assert NB - bm.num_free_blocks + 2 * npairs <= NB
    warm = torch.tensor([[NB - 2 * npairs + i, NB - npairs + i] for i in range(npairs)],
                        dtype=torch.int32, device=dev)
    pkv.pa_copy_blocks([k], [v], warm)
    torch.cuda.synchronize()
    round_ev[0].record()
    cow_ev[0].record()
    pkv.pa_copy_blocks([k], [v], d_pairs)
    cow_ev[1].record()
    if not fold:
        pkv.pa_write_kv(k, v, kn, vn, d_slot)
    decode(L0 + 2, plan, write=fold)
    round_ev[1].record()
    torch.cuda.synchronize()
    cow_ms, round_ms = cow_ev[0].elapsed_time(cow_ev[1]), round_ev[0].elapsed_time(round_ev[1])
    # The same copies again (idempotent: each destination gets its source's
    # bytes once more), each after a 1 GiB scratch write so its blocks come
    # from HBM as in the round itself: five more event-timed launches.
    scratch = torch.empty(2**30, dtype=torch.uint8, device=dev)
    rep_ev = [(T(enable_timing=True), T(enable_timing=True)) for _ in range(5)]
    for i, (a, b) in enumerate(rep_ev):
        scratch.fill_(i)
        a.record()
        pkv.pa_copy_blocks([k], [v], d_pairs)
        b.record()
    torch.cuda.synchronize()
    del scratch
    cow_rep_ms = np.array([a.elapsed_time(b) for a, b in rep_ev])
    # Rounds 2..X untimed (the flow up to 2305 tokens per sequence).
    for r in range(2, X + 1):
        d_slot, _, n = append(seqs, toks)
        assert n == 0
        pkv.pa_write_kv(k, v, kn, vn, d_slot)
    for w in range(args.warmup):
        d_slot, _, _ = append(seqs, toks)
        plan = prepare()
        if not fold:
            pkv.pa_write_kv(k, v, kn, vn, d_slot)
        decode(L0 + 1 + X + w + 1, plan, write=fold)
    torch.cuda.synchronize()
    evs = [(T(enable_timing=True), T(enable_timing=True)) for _ in range(args.steps)]
    dec = [(T(enable_timing=True), T(enable_timing=True)) for _ in range(args.steps)]
    lens, uniq = [], []
    plan_s.clear()
    t0 = time.perf_counter()
    for i in range(args.steps):
        n = L0 + 1 + X + args.warmup + i + 1
        d_slot, _, _ = append(seqs, toks)
        plan = prepare()
        evs[i][0].record()
        if fold:
            # one call: the step is the decode launch (no events inside)
            n_groups = decode(n, plan, write=True)
        else:
            pkv.pa_write_kv(k, v, kn, vn, d_slot)
            n_groups = decode(n, plan, dec[i])
        evs[i][1].record()
        lens.append(n)
        # unique blocks read: the shared prefix once per prompt plus every
        # sequence's private blocks (this step's exact table contents)
        uniq.append(len(np.unique(tab_h.numpy()[:, :-(-n // bs)])) * bs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = np.array([a.elapsed_time(b) for a, b in evs])
    dec_ms = step_ms if fold else np.array([a.elapsed_time(b) for a, b in dec])
    # plain pa_decode over the final batch, same tables, for comparison
    n_last = lens[-1]
    plain = [(T(enable_timing=True), T(enable_timing=True)) for _ in range(args.steps)]
    prepare(shared=False)
    for i in range(args.steps):
        decode(n_last, None, plain[i])
    torch.cuda.synchronize()
    plain_ms = np.array([a.elapsed_time(b) for a, b in plain])
    per_tok = 2 * H * D * 2
    logical = np.array(lens, dtype=np.float64) * B * per_tok
    unique = np.array(uniq, dtype=np.float64) * per_tok
    value = float(logical.sum() / (step_ms.sum() * 1e-3) / 1e9)
    achieved_u = float(unique.mean() / (dec_ms.mean() * 1e-3) / 1e9)
    cow_bytes = npairs * 2 * 2 * k[0].numel() * 2          # K and V, read + write
    cow_med = float(np.median(np.append(cow_rep_ms, cow_ms)))
    ceiling = stream_read_ceiling(torch, pkv, args.read_gib)
    cpu = (cpu_baseline([n_last] * B, cfg["hq"], H, D, bs, "f16", args.cpu_seconds, 1, "fork_cow")
           if args.cpu_seconds > 0 else None)
    if cpu is not None:
        cpu["sample"] += "; logical bytes (the oracle reads every sequence's blocks)"
    return {
        "metric": "paged decode attention: achieved KV GB/s (% of HBM peak) and seqs/s",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(float(step_ms.mean()), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "fork_cow", "prompts": P, "forks": F, "prompt_len": L0,
                   "appended": X, "q_heads": cfg["hq"], "kv_heads": H, "head_dim": D,
                   "block_size": bs, "num_blocks": NB, "partition_tokens": 512,
                   "timing": "GPU events per step (write + decode); value counts logical "
                             "KV bytes (shared prefix blocks once per sequence)",
                   "decode": "pa_decode_shared with a per-step host plan",
                   "kv_write": "pa_write_kv, then pa_decode_shared" if not fold
                   else "in the decode call (pa_write_decode_shared)"},
        "seqs_per_s": round(B * args.steps / (step_ms.sum() * 1e-3), 1),
        "gpu_step_ms_p10_p50_p90": [round(float(x), 4) for x in np.percentile(step_ms, [10, 50, 90])],
        "unique_kv_gbs": round(float(unique.sum() / (step_ms.sum() * 1e-3) / 1e9), 2),
        "used_blocks": int(NB - bm.num_free_blocks),
        "cow_round": {"pairs": npairs, "copy_ms": round(cow_ms, 4),
                      "copy_gbs": round(cow_bytes / (cow_ms * 1e-3) / 1e9, 2),
                      "round_ms": round(round_ms, 4),
                      "copy_ms_repeats": [round(float(x), 4) for x in cow_rep_ms],
                      "roofline": {"kernel": "copy_blocks_kernel (448 pairs, K and V, one layer)",
                                   "bound": "hbm", "unit": "GB/s",
                                   "achieved": round(cow_bytes / (cow_med * 1e-3) / 1e9, 2),
                                   "peak": PEAK_HBM_GBS,
                                   "frac": round(cow_bytes / (cow_med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                   "avg_launch_ms": round(cow_med, 5),
                                   "algorithmic_bytes_per_launch": cow_bytes,
                                   "traffic": load_traffic("copy_blocks_fork_cow")}},
        "shared_prefix": {"groups": n_groups, "host_plan_ms": round(1e3 * float(np.mean(plan_s)), 4),
                          "decode_ms": round(float(dec_ms.mean()), 5),
                          "plain_pa_decode_ms": round(float(plain_ms.mean()), 5),
                          "plain_unique_gbs": round(float(unique[-1] / (plain_ms.mean() * 1e-3) / 1e9), 2)},
        "roofline": with_ceiling(
            {"kernel": ("pa_write_decode_shared (the new tokens' write, shared pass + private pass, "
                        "which finishes each sequence), unique bytes" if fold else
                        "pa_decode_shared (shared pass + private pass, which finishes each "
                        "sequence), unique bytes"),
             "bound": "hbm", "achieved": round(achieved_u, 2), "peak": PEAK_HBM_GBS,
             "unit": "GB/s", "frac": round(achieved_u / PEAK_HBM_GBS, 4),
             "traffic": load_traffic("pa_decode_shared_fork_cow") if fold else None,
             "avg_launch_ms": round(float(dec_ms.mean()), 5),
             "algorithmic_bytes_per_launch": int(unique.mean())}, ceiling),
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
    }


def run_swap(args, torch, pkv, workloads):
    """Preemption traffic at the Llama-7B shape (32 layers x 32 KV heads x
    128 dims, fp16, block 16): the victim is one 4096-token sequence (256
    blocks scattered through a 1024-block pool).  A step swaps it out
    (every layer's K and V, 2 GiB, into one pinned host buffer) and back in
    (into 256 other scattered blocks).  Beside it, the same 2 GiB as one
    contiguous DMA copy each way: the host link's ceiling on this machine."""
    L, H, D, bs, NB, n = 32, 32, 128, 16, 1024, 256
    dev = torch.device("cuda:0")
    ks = [workloads.normal_torch((NB, bs, H, D), 60 + 2 * i, torch.float16, dev) for i in range(L)]
    vs = [workloads.normal_torch((NB, bs, H, D), 61 + 2 * i, torch.float16, dev) for i in range(L)]
    order = workloads.block_order(NB, 3)
    out_blocks = torch.from_numpy(np.ascontiguousarray(order[:n], dtype=np.int32)).to(dev)
    in_blocks = torch.from_numpy(np.ascontiguousarray(order[n:2 * n], dtype=np.int32)).to(dev)
    rec = pkv.swap_record_bytes(ks)
    total = n * rec
    host = torch.empty(total, dtype=torch.uint8, pin_memory=True)
    flat = torch.empty(total, dtype=torch.uint8, device=dev)
    T = torch.cuda.Event
    for _ in range(max(args.warmup, 1)):
        pkv.pa_swap_out(ks, vs, out_blocks, host)
        pkv.pa_swap_in(ks, vs, in_blocks, host)
    torch.cuda.synchronize()
    ev = [[T(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        pkv.pa_swap_out(ks, vs, out_blocks, host)
        e[1].record()
        pkv.pa_swap_in(ks, vs, in_blocks, host)
        e[2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    out_ms = np.array([a.elapsed_time(b) for a, b, _ in ev])
    in_ms = np.array([b.elapsed_time(c) for _, b, c in ev])
    dma = [[T(enable_timing=True) for _ in range(3)] for _ in range(3)]
    for e in dma:
        e[0].record()
        host.copy_(flat, non_blocking=True)
        e[1].record()
        flat.copy_(host, non_blocking=True)
        e[2].record()
    torch.cuda.synchronize()
    d2h = float(np.median([a.elapsed_time(b) for a, b, _ in dma]))
    h2d = float(np.median([b.elapsed_time(c) for _, b, c in dma]))
    gbs = lambda ms: total / (ms * 1e-3) / 1e9
    out_gbs, in_gbs = gbs(float(out_ms.mean())), gbs(float(in_ms.mean()))
    step_ms = out_ms + in_ms
    link_peak = 64.0        # PCIe 5.0 x16, per direction (published)
    return {
        "metric": "preemption swap: host-link GB/s (blocks out to pinned host memory and back)",
        "value": round(gbs(float(step_ms.mean()) / 2), 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(float(step_ms.mean()), 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "swap", "layers": L, "kv_heads": H, "head_dim": D, "block_size": bs,
                   "pool_blocks": NB, "victim_blocks": n, "bytes_each_way": total,
                   "timing": "GPU events around each call"},
        "swap_out_gbs": round(out_gbs, 2), "swap_in_gbs": round(in_gbs, 2),
        "dma_contiguous_gbs": {"d2h": round(gbs(d2h), 2), "h2d": round(gbs(h2d), 2)},
        "roofline": {"kernel": "pa_swap_out / pa_swap_in", "bound": "host-link",
                     "achieved": round(min(out_gbs, in_gbs), 2), "peak": link_peak, "unit": "GB/s",
                     "frac": round(min(out_gbs, in_gbs) / link_peak, 4), "traffic": None,
                     "avg_launch_ms": round(float(max(out_ms.mean(), in_ms.mean())), 5),
                     "algorithmic_bytes_per_launch": total},
        "cpu_baseline": None,
        "wall_s": round(wall, 3),
    }


def run_serve(args, torch, pkv, workloads):
    """Continuous batching at the Llama-7B shape (32 layers x 32 KV heads x
    128 dims, fp16, block 16, a 16384-block pool, batch 128): 1024 requests
    queued up front, prompts log-uniform in [50, 2048] tokens (every other
    one starting with a shared 256-token system prompt), output budgets
    log-uniform in [16, 512].  Each step is DecodeEngine.step: the
    scheduler's decisions, then swap copies, the admitted prompts' K/V
    writes and their attention over the uncached suffix (pa_prefill, 32
    layers), copy-on-write copies, the batch's K/V writes and 32 decode
    launches (the writes inside them, pa_write_decode, on steps without a
    preemption), and a stream sync.  Reported: sustained generated tokens/s,
    decode KV GB/s over the timed steps, and the GPU time of the prompt
    phase and of the decode phase (HIP events on the launch stream)."""
    from paged_kv_cache_136_amd.engine import DecodeEngine
    L, H, D, bs, NB, batch, host_slots, n_req = 32, 32, 128, 16, 16384, 128, 256, 1024
    dev = torch.device("cuda:0")
    pt = args.partition_tokens if args.partition_tokens >= 0 else 512
    shared = args.shared_prefix == "on"
    eng = DecodeEngine(L, NB, bs, H, H, D, torch.float16, batch, host_slots, True,
                       partition_tokens=pt, shared_prefix=shared, timing=True)
    rng = np.random.Generator(np.random.PCG64(11))
    system = workloads.token_ids(256, seed=12)
    lo, hi = math.log(50), math.log(2048)
    for rid in range(1, n_req + 1):
        n = int(round(math.exp(rng.uniform(lo, hi))))
        prompt = workloads.token_ids(n, seed=100000 + rid)
        if rid % 2 == 0:
            prompt = system + prompt
        budget = int(round(math.exp(rng.uniform(math.log(16), math.log(512)))))
        eng.add_request(rid, prompt, budget)
    # Rows come from preallocated random pools (their values do not matter
    # for the rate, and no RNG kernel runs inside the timed steps).
    pool = workloads.normal_torch((batch * (2048 + 256), H, D), 13, torch.float16, dev)

    def kv_rows(layer, kind, plan):
        n = len(plan["prefill_slots"]) if kind == "prompt" else len(plan["writes"])
        return pool[:n], pool[:n]

    def q_rows(layer, kind, n):
        return pool[:n]

    def sample(owed, outs, prompt_outs):
        return {i: (i * 131 + eng.step_no) % 32000 for i in owed}

    per_tok = 2 * H * D * 2 * L
    for _ in range(args.warmup):
        eng.step(kv_rows, q_rows, sample)
    torch.cuda.synchronize()
    tokens = kv_bytes = prompt_rows = prompt_flops = 0
    counts = {"admitted": 0, "finished": 0, "preempted": 0, "resumed": 0, "recomputed": 0}
    host0, pms0, dms0, fold0 = eng.host_seconds, eng.prompt_ms, eng.decode_ms, eng.folded_steps
    t0 = time.perf_counter()
    for _ in range(args.steps):
        plan, outs, prompt_outs, prompt_ids = eng.step(kv_rows, q_rows, sample)
        n_batch = len(plan["batch"])
        tokens += n_batch + len(prompt_ids)
        # the lengths the engine exported for its launches (no host calls
        # of the bench's own inside the timed steps)
        kv_bytes += int(eng.last_decode_lens.astype(np.int64).sum()) * per_tok
        plens = dict(zip(prompt_ids, eng.last_prompt_lens.tolist()))
        for rid, n in zip(plan["admitted"].tolist(), plan["prefill_counts"].tolist()):
            if rid in plens:
                total = plens[rid]
                prompt_rows += n
                # causal: row i of the suffix attends to total - n + i + 1 keys
                prompt_flops += 4 * D * H * L * (n * (total - n) + n * (n + 1) // 2)
        for k in counts:
            counts[k] += len(plan[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    tok_s = tokens / wall
    prompt_ms, decode_ms = eng.prompt_ms - pms0, eng.decode_ms - dms0
    return {
        "metric": "continuous-batching decode: sustained generated tokens/s (KV GB/s beside it)",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "serve", "layers": L, "kv_heads": H, "q_heads": H, "head_dim": D,
                   "block_size": bs, "num_blocks": NB, "max_batch": batch, "host_slots": host_slots,
                   "requests": n_req, "prompts": "log-uniform [50, 2048], half after a shared "
                   "256-token system prompt", "budgets": "log-uniform [16, 512]",
                   "timing": "wall clock over whole engine steps (host scheduling, copies, "
                             "prompt writes and attention, the batch's writes, 32 decode "
                             "launches, one sync per step)",
                   "kv_write": "inside the decode launches (pa_write_decode) on steps without "
                               "a preemption, else pa_write_kv",
                   "partition_tokens": pt, "shared_prefix_decode": shared},
        "shared_groups_per_step": round(eng.shared_groups / max(eng.step_no, 1), 2),
        "write_folded_steps": eng.folded_steps - fold0,
        "kv_gbs": round(kv_bytes / wall / 1e9, 2),
        "pct_hbm_peak": round(100 * kv_bytes / wall / 1e9 / PEAK_HBM_GBS, 2),
        "decode_phase_ms_per_step": round(decode_ms / args.steps, 4),
        "decode_phase_kv_gbs": round(kv_bytes / (decode_ms * 1e-3) / 1e9, 2) if decode_ms else None,
        "prompt_phase_ms_per_step": round(prompt_ms / args.steps, 4),
        "prompt_rows": prompt_rows,
        "prompt_attention_tflops": (round(prompt_flops / (prompt_ms * 1e-3) / 1e12, 2)
                                    if prompt_ms else None),
        "host_sched_ms_per_step": round((eng.host_seconds - host0) / args.steps * 1e3, 4),
        "events": counts,
        "roofline": with_ceiling(
            {"kernel": "decode phase of the engine step: 32 x pa_decode with table export and "
                       "upload, unique KV bytes of the batch",
             "bound": "hbm", "unit": "GB/s",
             "achieved": round(kv_bytes / (decode_ms * 1e-3) / 1e9, 2) if decode_ms else None,
             "peak": PEAK_HBM_GBS,
             "frac": round(kv_bytes / (decode_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4) if decode_ms else None,
             "traffic": None, "avg_launch_ms": round(decode_ms / args.steps / L, 5),
             "algorithmic_bytes_per_launch": int(kv_bytes / args.steps / L)},
            stream_read_ceiling(torch, pkv, args.read_gib)),
        "cpu_baseline": None,
        "wall_s": round(wall, 3),
    }


def run_beam(args, torch, pkv, workloads):
    """Beam search: 64 prompts (lengths log-uniform in [50, 2048], prefix
    cache on), 8 beams each, one layer of 32 KV heads x 128, fp16.  Every
    step each group's 8 beams are re-forked from seeded parents at their
    current (arbitrary) positions, the old beams freed, and all 512 beams
    append a token: beams sharing a partly filled last block copy it
    (pa_copy_blocks with many small pairs), then pa_write_decode_shared
    (the new tokens' K/V written inside the decode; --separate-write:
    pa_write_kv, then pa_decode_shared; host plan every step) over the 512
    beams.  Reported:
    step rate, copy pairs per step and the copy kernel's rate, decode KV
    GB/s (logical and over unique blocks), and plain pa_decode against
    pa_decode_shared on the final batch."""
    cfg = workloads.CONFIGS["beam"]
    bs, NB, H, D, G, W = cfg["bs"], cfg["num_blocks"], cfg["hkv"], cfg["d"], cfg["groups"], cfg["beams"]
    dev = torch.device("cuda:0")
    bm = pkv.BlockManager(NB, bs, True)
    k = workloads.normal_torch((NB, bs, H, D), 70, torch.float16, dev)
    v = workloads.normal_torch((NB, bs, H, D), 71, torch.float16, dev)
    lens0 = workloads.mixed_lengths(G, cfg["len_lo"], cfg["len_hi"], seed=7)
    beams, nid = [], 1
    for g in range(G):
        bm.allocate(nid, workloads.token_ids(int(lens0[g]), seed=5000 + g))
        beams.append([nid] * W)
        nid += 1
    B = G * W
    rng = np.random.default_rng(8)
    kn = workloads.normal_torch((B, H, D), 72, torch.float16, dev)
    vn = workloads.normal_torch((B, H, D), 73, torch.float16, dev)
    q = workloads.normal_torch((B, cfg["hq"], D), 74, torch.float16, dev)
    out = torch.empty((B, cfg["hq"], D), dtype=torch.float32, device=dev)
    maxlen = int(lens0.max()) + args.warmup + args.steps + 1
    ws = torch.empty(max(pkv.pa_decode_shared_workspace_bytes(B, cfg["hq"], D, maxlen, 512), 1),
                     dtype=torch.uint8, device=dev)
    width = -(-maxlen // bs)
    T = torch.cuda.Event

    def step(ev=None):
        nonlocal beams, nid
        h0 = time.perf_counter()
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
        bm.free_batch(old)
        beams = new
        flat = np.array([s for g in beams for s in g], dtype=np.int64)
        slots, pairs = bm.append_slots(flat, np.arange(B, dtype=np.int32))
        tables, lens = bm.export_batch(flat, width, pad_block=0)
        splan = pkv.pa_shared_plan(tables, lens, bs, 512, cfg["hq"] // H)
        sg, groups, mx, mp = splan
        host = time.perf_counter() - h0
        d_slot = torch.from_numpy(slots).to(dev) if not fold else None
        d_pairs = torch.from_numpy(pairs).to(dev) if len(pairs) else None
        d_tab = torch.from_numpy(tables).to(dev)
        d_len = torch.from_numpy(lens).to(dev)
        d_sg, d_gr = torch.from_numpy(sg).to(dev), torch.from_numpy(groups).to(dev)
        def mark(i):
            if ev is not None and ev[i] is not None:
                ev[i].record()
        mark(0)
        if d_pairs is not None:
            pkv.pa_copy_blocks([k], [v], d_pairs)
        if fold:
            # the copies, then one call (the decode phase is that call)
            mark(2)
            pkv.pa_write_decode_shared(q, k, v, kn, vn, d_tab, d_len, int(lens.max()), d_sg,
                                       d_gr, mx, mp, max_private_blocks=splan.max_private_blocks,
                                       partition_tokens=512, out=out, workspace=ws)
        else:
            mark(1)
            pkv.pa_write_kv(k, v, kn, vn, d_slot)
            mark(2)
            pkv.pa_decode_shared(q, k, v, d_tab, d_len, int(lens.max()), d_sg, d_gr, mx, mp,
                                 max_private_blocks=splan.max_private_blocks,
                                 partition_tokens=512, out=out, workspace=ws)
        mark(3)
        uniq = len(np.unique(np.concatenate([tables[i, :-(-int(n) // bs)] for i, n in enumerate(lens)])))
        last[:] = [d_tab, d_len, tables, lens]
        return len(pairs), int(lens.sum()), uniq, host

    last = [None] * 4
    fold = not args.separate_write

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Even steps record events around each phase (copy, write, decode);
    # odd steps only at their start and end, since every event record
    # leaves the GPU idle for a few microseconds: the step rate comes from
    # the odd steps (all steps if there is one), the phases from the even.
    # (With the write folded into the decode there is no event between
    # write and decode: copy = events 0 -> 2, decode = 2 -> 3.)
    evs = [[T(enable_timing=True) if (i % 2 == 0 and not (fold and j == 1)) or j in (0, 3)
            else None for j in range(4)]
           for i in range(args.steps)]
    info = []
    t0 = time.perf_counter()
    for e in evs:
        info.append(step(e))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    phase = np.arange(args.steps) % 2 == 0
    whole = ~phase if args.steps > 1 else phase
    copy_end = 2 if fold else 1
    copy_ms = np.array([e[0].elapsed_time(e[copy_end]) for e in evs if e[2] is not None])
    dec_ms = np.array([e[2].elapsed_time(e[3]) for e in evs if e[2] is not None])
    step_ms = np.array([e[0].elapsed_time(e[3]) for e in evs])
    # The final batch again: plain pa_decode against pa_decode_shared with a
    # host plan (beams of a group share their prefix up to the last fork).
    d_tab, d_len, tables, lens = last
    mlen = int(lens.max())

    def timed(fn, reps=10):
        ev = [(T(enable_timing=True), T(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev]))

    cmp = {"plain_pa_decode_ms": timed(lambda: pkv.pa_decode(
        q, k, v, d_tab, d_len, mlen, partition_tokens=512, out=out, workspace=ws))}
    for pt in (512, 128):
        splan = pkv.pa_shared_plan(tables, lens, bs, pt, cfg["hq"] // H)
        sg, groups, mx, mp = splan
        d_sg, d_gr = torch.from_numpy(sg).to(dev), torch.from_numpy(groups).to(dev)
        ws2 = torch.empty(max(pkv.pa_decode_shared_workspace_bytes(B, cfg["hq"], D, mlen, pt), 1),
                          dtype=torch.uint8, device=dev)
        cmp[f"shared_pt{pt}"] = {"groups": len(groups), "shared_blocks": int(groups[:, 0].sum()),
                                 "ms": timed(lambda: pkv.pa_decode_shared(
                                     q, k, v, d_tab, d_len, mlen, d_sg, d_gr, mx, mp,
                                     max_private_blocks=splan.max_private_blocks,
                                     partition_tokens=pt, out=out, workspace=ws2))}
    npairs = np.array([x[0] for x in info])
    toks = np.array([x[1] for x in info], dtype=np.float64)
    uniq_all = np.array([x[2] for x in info], dtype=np.float64)
    uniq = uniq_all[phase]
    per_tok = 2 * H * D * 2
    block_kv = 2 * k[0].numel() * 2
    copied = npairs[phase] * block_kv * 2       # read + write
    with_pairs = npairs[phase] > 0
    return {
        "metric": "beam search over the paged cache: decode KV GB/s and beams/s",
        "value": round(float(toks[whole].sum() * per_tok / (step_ms[whole].sum() * 1e-3) / 1e9), 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(float(step_ms[whole].mean()), 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "beam", "groups": G, "beams": W, "prompt_lengths": "log-uniform [50, 2048], seed 7",
                   "kv_heads": H, "q_heads": cfg["hq"], "head_dim": D, "block_size": bs, "num_blocks": NB,
                   "partition_tokens": 512,
                   "timing": "GPU events per step (COW copies + write + decode): odd steps at start and "
                             "end only (value, ms_per_step, beams/s), even steps around each phase (copy, "
                             "decode, roofline); value counts every beam's tokens (shared blocks once per beam)",
                   "decode": "pa_decode_shared with a per-step host plan",
                   "kv_write": "pa_write_kv, then pa_decode_shared" if not fold
                   else "in the decode call (pa_write_decode_shared)"},
        "beams_per_s": round(B * int(whole.sum()) / (step_ms[whole].sum() * 1e-3), 1),
        "unique_kv_gbs": round(float(uniq.sum() * bs * per_tok / (dec_ms.sum() * 1e-3) / 1e9), 2),
        "unique_kv_bytes_per_step": [int(u) * bs * per_tok for u in uniq_all],
        "cow_pairs_per_step": round(float(npairs.mean()), 1),
        "copy_ms_per_step": round(float(copy_ms.mean()), 4),
        "copy_gbs": round(float(copied[with_pairs].sum() / (copy_ms[with_pairs].sum() * 1e-3) / 1e9), 2)
        if with_pairs.any() else None,
        "decode_ms_per_step": round(float(dec_ms.mean()), 4),
        "host_ms_per_step": round(float(np.mean([x[3] for x in info]) * 1e3), 4),
        "final_batch_decode": cmp,
        "roofline": with_ceiling(
            {"kernel": ("pa_write_decode_shared (the new tokens' write, shared pass + private pass, "
                        "which finishes each sequence), unique bytes" if fold else
                        "pa_decode_shared (shared pass + private pass, which finishes each "
                        "sequence), unique bytes"),
             "bound": "hbm", "unit": "GB/s",
             "achieved": round(float(uniq.mean() * bs * per_tok / (dec_ms.mean() * 1e-3) / 1e9), 2),
             "peak": PEAK_HBM_GBS,
             "frac": round(float(uniq.mean() * bs * per_tok / (dec_ms.mean() * 1e-3) / 1e9)
                           / PEAK_HBM_GBS, 4),
             "traffic": load_traffic("pa_decode_shared_beam") if fold else None,
             "avg_launch_ms": round(float(dec_ms.mean()), 5),
             "algorithmic_bytes_per_launch": int(uniq.mean() * bs * per_tok)},
            stream_read_ceiling(torch, pkv, args.read_gib)),
        "cpu_baseline": None, "wall_s": round(wall, 3),
    }


PEAK_MFMA_F16_TFLOPS = 2500.0   # MI355X dense fp16 / bf16, published


def run_prefill(args, torch, pkv, workloads):
    """Prefill of uncached suffixes after a prefix hit: 16 sequences share a
    1024-token system prompt (prefix-cache hits) and each adds a 1024-token
    uncached suffix; one layer of 32 heads x 128, fp16, block 16.  The suffix
    K/V are written (pa_write_kv) and pa_prefill computes their causal
    attention over 2048-token contexts.  prefill_gqa is the same with 8
    KV heads for the 32 query heads.  Reported: the kernel's rate in
    TFLOP/s of algorithmic attention work (4 * head_dim flops per (query,
    key, head) with key <= query), and K/V bytes read per second."""
    B, sys_len, sfx, H, D, bs = 16, 1024, 1024, 32, 128, 16
    HKV = 8 if args.workload == "prefill_gqa" else H
    n = sys_len + sfx
    NB = B * (n // bs) + 64
    dev = torch.device("cuda:0")
    bm = pkv.BlockManager(NB, bs, True)
    system = workloads.token_ids(sys_len, seed=21)
    bm.allocate(0, system + [1])               # registers the shared prompt's blocks
    tables_l, cached = [], []
    for b in range(1, B + 1):
        toks = system + workloads.token_ids(sfx, seed=300 + b)
        bm.allocate(b, toks)
        cached.append(bm.num_cached_tokens(b))
    bm.free(0)
    seqs = list(range(1, B + 1))
    qlens = [n - c for c in cached]
    tables, lens = bm.export_batch(seqs, n // bs, pad_block=0)
    k = workloads.normal_torch((NB, bs, HKV, D), 80, torch.float16, dev)
    v = workloads.normal_torch((NB, bs, HKV, D), 81, torch.float16, dev)
    T = sum(qlens)
    q = workloads.normal_torch((T, H, D), 82, torch.float16, dev)
    qs = torch.tensor(np.concatenate([[0], np.cumsum(qlens)]), dtype=torch.int32, device=dev)
    d_tab = torch.from_numpy(tables).to(dev)
    d_len = torch.from_numpy(lens).to(dev)
    out = torch.empty((T, H, D), dtype=torch.float32, device=dev)
    mq = max(qlens)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for _ in range(args.warmup):
        pkv.pa_prefill(q, k, v, d_tab, qs, d_len, mq, out=out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in ev:
        e[0].record()
        pkv.pa_prefill(q, k, v, d_tab, qs, d_len, mq, out=out)
        e[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    pairs = sum(sum(c + i + 1 for i in range(ql)) for c, ql in zip(cached, qlens))
    flops = 4.0 * D * H * pairs
    kv_bytes = 2.0 * HKV * D * 2 * sum(lens)       # each sequence's K/V once
    tflops = flops / (ms.mean() * 1e-3) / 1e12
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        from threadpoolctl import threadpool_limits
        kh = k.float().cpu().numpy()
        vh = v.float().cpu().numpy()
        qh = q[:64].float().cpu().numpy()
        rows, t1 = 0, time.perf_counter()
        with threadpool_limits(limits=1):
            while True:
                oracle.ref_prefill(qh, kh, vh, tables[:1], [64], [cached[0] + 64])
                rows += 64
                if time.perf_counter() - t1 > min(args.cpu_seconds, 10):
                    break
        sec = time.perf_counter() - t1
        sample_pairs = rows // 64 * sum(cached[0] + i + 1 for i in range(64))
        cpu = {"value": round(4.0 * D * H * sample_pairs / sec / 1e12, 6), "unit": "TFLOP/s",
               "cores": 1, "kind": "oracle",
               "sample": f"the first 64 suffix rows of sequence 1 (after its {cached[0]} cached "
                         f"tokens), {rows // 64} repetitions in {sec:.1f} s, float64 NumPy, BLAS 1 thread"}
    return {
        "metric": "prefill of uncached suffixes: attention TFLOP/s",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(float(ms.mean()), 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": args.workload, "sequences": B, "cached_prefix": sys_len, "suffix": sfx,
                   "context": n, "q_heads": H, "kv_heads": HKV, "head_dim": D, "block_size": bs,
                   "cached_tokens": cached[:1], "timing": "GPU events per pa_prefill launch"},
        "kv_gbs": round(kv_bytes / (ms.mean() * 1e-3) / 1e9, 2),
        "roofline": {"kernel": "pa_prefill", "bound": "mfma", "achieved": round(tflops, 2),
                     "peak": PEAK_MFMA_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_MFMA_F16_TFLOPS, 4), "traffic": None,
                     "avg_launch_ms": round(float(ms.mean()), 5), "algorithmic_flops_per_launch": flops},
        "cpu_baseline": cpu, "wall_s": round(wall, 3),
    }


LENGTH_NOTES = {
    "tiny": "[7, 16, 31, 48, 63] (day31 block-count script), +1 token per step",
    "mixed_7b": "log-uniform [50, 4096], PCG64 seed 0, +1 token per step",
    "13b_layer": "10 x 4096, +1 token per step",
    "gqa_long": "32 x 32768, +1 token per step",
}


def main():
    args = parse_args()
    if args.calibrate:
        calibrate()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(decode would shard by sequence or by KV head, with no exchange inside attention).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_136_amd as pkv
    import workloads

    torch.cuda.set_device(0)
    if args.workload == "fork_cow":
        result = run_fork_cow(args, torch, pkv, workloads)
    elif args.workload == "swap":
        result = run_swap(args, torch, pkv, workloads)
    elif args.workload == "serve":
        result = run_serve(args, torch, pkv, workloads)
    elif args.workload == "beam":
        result = run_beam(args, torch, pkv, workloads)
    elif args.workload in ("prefill", "prefill_gqa"):
        result = run_prefill(args, torch, pkv, workloads)
    else:
        wb = DecodeBench(args.workload, args, torch, pkv, workloads)
        result = wb.run()
        if args.cpu_seconds > 0:
            result["cpu_baseline"] = cpu_baseline(wb.lens0, wb.hq, wb.H, wb.D, wb.bs, wb.dtype,
                                                  args.cpu_seconds, wb.L, args.workload)
        else:
            result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

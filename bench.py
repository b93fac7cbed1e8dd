#!/usr/bin/env python3
"""Paged decode step throughput on one MI355X.

Default workload: the mixed-length batch of the Llama-7B shape (32 layers x
32 KV heads x 128 dims, fp16, block size 16, 128 sequences with lengths
log-uniform in [50, 4096], a 16384-block pool scattered by a seeded
permutation).  One step is one pass of the whole hot path:

  host   pa_bm_append_slots (one new token per sequence: slot, table growth)
         pa_bm_export_batch into pinned buffers, async upload
  device for each layer: pa_write_kv (the new token's K/V), pa_decode
         (split-KV phase 1 + reduce); pa_copy_blocks when appends report
         copy-on-write pairs (none in this workload)

Sequences grow by one token per step, as in real decoding; the KV bytes of
every step are counted exactly.  The metric is achieved KV GB/s (valid
tokens' K and V bytes read per second, whole job) with seqs/s beside it.

Prints one JSON line.  --gpus N with N > 1 exits: this build runs on one GPU.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, published
PMC_FILE = os.path.join(ROOT, "profiles", "pa_decode_mixed_7b_pmc.json")
DECODE_SRC = os.path.join(ROOT, "paged_kv_cache_136_amd", "csrc", "decode.hip")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--partition-tokens", type=int, default=512)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="target CPU time of the oracle baseline sample (0 = skip)")
    p.add_argument("--calibrate", action="store_true",
                   help="instead of the step: run pa_copy_blocks over a known number of "
                        "bytes (3 launches of 8192 x 128 KiB blocks, K and V), for scaling "
                        "rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    return p.parse_args()


def calibrate():
    """pa_copy_blocks over 8192 disjoint block pairs of 128 KiB in one layer's
    K and V: each launch reads and writes exactly 2 * 8192 * 128 KiB = 2 GiB."""
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
    print(json.dumps({"calibration": "pa_copy_blocks", "launches": 3,
                      "read_bytes_per_launch": nbytes, "write_bytes_per_launch": nbytes}))


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter
    summary, or None if absent or taken on a different kernel source."""
    try:
        with open(PMC_FILE) as f:
            pmc = json.load(f)
    except (OSError, ValueError):
        return None
    if pmc.get("decode_source_sha") != source_sha(DECODE_SRC):
        return None
    return pmc.get("traffic_bytes_per_launch")


def cpu_baseline(lens, H, D, bs, seconds):
    """The oracle timed on the host over one layer of the same workload
    shape (all sequences, all heads), with fresh seeded inputs, repeated
    until about ``seconds`` of CPU time; BLAS limited to one thread."""
    import torch
    from threadpoolctl import threadpool_limits

    import oracle
    import workloads

    need = [-(-int(n) // bs) for n in lens]
    nblk = sum(need)
    order = workloads.block_order(nblk, seed=11)
    tables = np.zeros((len(lens), max(need)), dtype=np.int64)
    o = 0
    for i, k in enumerate(need):
        tables[i, :k] = order[o:o + k]
        o += k
    k = workloads.normal_torch((nblk, bs, H, D), 12, torch.float16, "cuda").cpu().numpy()
    v = workloads.normal_torch((nblk, bs, H, D), 13, torch.float16, "cuda").cpu().numpy()
    q = workloads.normal_torch((len(lens), H, D), 14, torch.float16, "cuda").cpu().numpy()
    layer_bytes = int(np.sum(lens)) * 2 * H * D * 2
    reps, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            oracle.ref_decode(q, k, v, tables, lens)
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    return {"value": round(layer_bytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"one layer of the mixed_7b step ({len(lens)} sequences x {H} heads, "
                      f"{int(np.sum(lens))} tokens, fresh seeded fp16 inputs), "
                      f"{reps} repetitions in {el:.1f} s, float64 NumPy, BLAS 1 thread",
            "seqs_per_s": round(len(lens) * reps / el / 32, 4)}


def main():
    args = parse_args()
    if args.calibrate:
        calibrate()
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(decode shards by sequence or KV head with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_136_amd as pkv
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = workloads.CONFIGS["mixed_7b"]
    L, H, D, bs, NB = cfg["layers"], cfg["hkv"], cfg["d"], cfg["bs"], cfg["num_blocks"]
    lens0 = workloads.lengths("mixed_7b")                 # includes the step's new token
    B = len(lens0)
    S = args.warmup + args.steps
    max_len_final = int(lens0.max()) + S - 1
    max_blocks = -(-max_len_final // bs)

    # Host block manager: free list scrambled by a seeded permutation, then
    # each sequence admitted with its prompt (length - 1 tokens).
    bm = pkv.BlockManager(NB, bs, enable_prefix_cache=False)
    workloads.scramble_free_list(bm, workloads.block_order(NB, seed=1))
    toks = workloads.token_ids(int(lens0.max()), seed=2)
    for i in range(B):
        bm.allocate(i, toks[:int(lens0[i]) - 1])
    seqs = np.arange(B, dtype=np.int64)

    # Device inputs, resident in HBM: the KV pool of every layer, and each
    # layer's query and new K/V rows.
    pool = torch.empty((L, 2, NB, bs, H, D), dtype=torch.float16, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    for layer in range(L):
        pool[layer].normal_(generator=g)
    q = workloads.normal_torch((L, B, cfg["hq"], D), 4, torch.float16, dev)
    k_new = workloads.normal_torch((L, B, H, D), 5, torch.float16, dev)
    v_new = workloads.normal_torch((L, B, H, D), 6, torch.float16, dev)
    out = torch.empty((L, B, cfg["hq"], D), dtype=torch.float32, device=dev)
    ws_bytes = pkv.pa_decode_workspace_bytes(B, cfg["hq"], D, max_len_final, args.partition_tokens)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    d_tab = torch.empty((B, max_blocks), dtype=torch.int32, device=dev)
    d_len = torch.empty(B, dtype=torch.int32, device=dev)
    d_slot = torch.empty(B, dtype=torch.int64, device=dev)
    d_pairs = torch.empty((B, 2), dtype=torch.int32, device=dev)
    # Two pinned host buffer sets: the host fills one while the other's
    # upload may still be queued.
    pin = [dict(tab=torch.empty((B, max_blocks), dtype=torch.int32).pin_memory(),
                len=torch.empty(B, dtype=torch.int32).pin_memory(),
                slot=torch.empty(B, dtype=torch.int64).pin_memory(),
                pairs=torch.empty((B, 2), dtype=torch.int32).pin_memory(),
                ev=torch.cuda.Event()) for _ in range(2)]
    for p in pin:
        p["ev"].record()
    new_tok = np.full(B, 7, dtype=np.int32)
    k_layers = [pool[layer, 0] for layer in range(L)]
    v_layers = [pool[layer, 1] for layer in range(L)]
    torch.cuda.synchronize()

    host_s = []

    def step(s, ev_pairs=None):
        p = pin[s % 2]
        p["ev"].synchronize()                 # its previous upload has run
        h0 = time.perf_counter()
        slots, pairs = bm.append_slots(seqs, new_tok)
        p["slot"].numpy()[:] = slots
        bm.export_batch(seqs, max_blocks, 0, tables_out=p["tab"].numpy(), lens_out=p["len"].numpy())
        host_s.append(time.perf_counter() - h0)
        d_tab.copy_(p["tab"], non_blocking=True)
        d_len.copy_(p["len"], non_blocking=True)
        d_slot.copy_(p["slot"], non_blocking=True)
        if len(pairs):
            p["pairs"].numpy()[:len(pairs)] = pairs
            d_pairs[:len(pairs)].copy_(p["pairs"][:len(pairs)], non_blocking=True)
        p["ev"].record()
        if len(pairs):
            pkv.pa_copy_blocks(k_layers, v_layers, d_pairs[:len(pairs)])
        max_len = int(lens0.max()) + s
        for layer in range(L):
            pkv.pa_write_kv(k_layers[layer], v_layers[layer], k_new[layer], v_new[layer], d_slot)
            if ev_pairs is not None:
                ev_pairs[layer][0].record()
            pkv.pa_decode(q[layer], k_layers[layer], v_layers[layer], d_tab, d_len, max_len,
                          partition_tokens=args.partition_tokens, out=out[layer], workspace=ws)
            if ev_pairs is not None:
                ev_pairs[layer][1].record()

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(L)] for _ in range(args.steps)]
    host_s.clear()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Algorithmic KV bytes: valid tokens' K and V rows, every layer.
    per_token_layer = 2 * H * D * 2
    step_tokens = [int(lens0.sum()) + B * (args.warmup + i) for i in range(args.steps)]
    kv_bytes = sum(step_tokens) * per_token_layer * L
    value = kv_bytes / wall / 1e9
    dec_ms = np.array([[a.elapsed_time(b) for a, b in row] for row in events])   # [steps, L]
    launch_bytes = np.array(step_tokens, dtype=np.float64) * per_token_layer   # per launch
    # Average algorithmic bytes per launch / average launch duration.
    achieved = float(launch_bytes.mean() / (dec_ms.mean() * 1e-3) / 1e9)
    traffic = load_traffic()

    result = {
        "metric": "paged decode attention: achieved KV GB/s (% of HBM peak) and seqs/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "mixed_7b", "layers": L, "batch": B, "q_heads": cfg["hq"],
                   "kv_heads": H, "head_dim": D, "block_size": bs, "num_blocks": NB,
                   "lengths": "log-uniform [50, 4096], PCG64 seed 0, +1 token per step",
                   "mean_context": round(float(np.mean(step_tokens)) / B, 1),
                   "partition_tokens": args.partition_tokens},
        "seqs_per_s": round(B * args.steps / wall, 1),
        "pct_hbm_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "kv_bytes_per_step": int(kv_bytes // args.steps),
        "host_bm_ms_per_step": round(1e3 * float(np.mean(host_s)), 4),
        "roofline": {"kernel": "pa_decode (split-KV phase 1 + reduce), one layer",
                     "bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic,
                     "avg_launch_ms": round(float(dec_ms.mean()), 5),
                     "algorithmic_bytes_per_launch": int(launch_bytes.mean())},
    }
    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(lens0, H, D, bs, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

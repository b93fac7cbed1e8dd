"""torch-tensor front end of the device calls (argument marshalling only).

Each function checks shapes, dtypes and devices (every tensor argument,
outputs and workspaces included, must be a contiguous GPU tensor), then
calls the C entry point of the same name on the current HIP stream, or on
``stream`` when one is given; temporaries a call allocates (a defaulted
output, a workspace) are then allocated on that stream.  Every step of the
path runs in the library's kernels; nothing here computes.
"""

import contextlib
import ctypes
import math

import numpy as np
import torch

from ._lib import (PA_DTYPE_BF16, PA_DTYPE_F16, PA_DTYPE_F32, c_vp, check, lib)

SHARED_ROW = 17          # PA_SHARED_ROW: shared partitions, then 16 member slots

_DTYPES = {torch.float32: PA_DTYPE_F32, torch.float16: PA_DTYPE_F16, torch.bfloat16: PA_DTYPE_BF16}


def _dtype_code(t):
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensor must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensor must be contiguous")


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream):
    """Handle of the HIP stream to launch on: ``stream``, else torch's
    current stream on the current device, read as a raw handle (building a
    Stream object costs a few microseconds per call)."""
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    if _raw_stream is not None:
        return ctypes.c_void_p(_raw_stream(torch.cuda.current_device()))
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _on(stream):
    """Context for allocating a call's temporaries on the stream the call
    is launched on: torch's caching allocator then hands their memory to
    the next allocation only in that stream's order, so a temporary freed
    when the call returns cannot be reused while the kernel is queued."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _check_workspace(workspace):
    _dev(workspace)
    if workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise ValueError("workspace must be a contiguous uint8 [bytes] GPU tensor")


def pa_write_kv(k_cache, v_cache, k_new, v_new, slot_mapping, stream=None):
    """Scatter k_new/v_new [T, Hkv, D] into caches [num_blocks, bs, Hkv, D]
    at int64 slot_mapping [T] (out-of-range slots are skipped)."""
    _dev(k_cache, v_cache, k_new, v_new, slot_mapping)
    nb, bs, hkv, d = k_cache.shape
    T = k_new.shape[0]
    if v_cache.shape != k_cache.shape or k_new.shape != (T, hkv, d) or v_new.shape != (T, hkv, d):
        raise ValueError("shape mismatch")
    if slot_mapping.dtype != torch.int64 or slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be int64 [T]")
    if not (k_cache.dtype == v_cache.dtype == k_new.dtype == v_new.dtype):
        raise ValueError("dtype mismatch")
    check(lib().pa_write_kv(k_cache.data_ptr(), v_cache.data_ptr(), k_new.data_ptr(),
                            v_new.data_ptr(), slot_mapping.data_ptr(), T, nb, bs, hkv, d,
                            _dtype_code(k_cache), _stream(stream)))


def pa_copy_blocks(k_caches, v_caches, pairs, stream=None):
    """For each layer's caches and each (src, dst) row of int32 ``pairs``
    [P, 2] on the GPU: K[dst] = K[src], V[dst] = V[src] (whole blocks)."""
    k_caches, v_caches = list(k_caches), list(v_caches)
    if len(k_caches) != len(v_caches):
        raise ValueError("K and V layer counts differ")
    _dev(pairs, *k_caches, *v_caches)
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be int32 [P, 2]")
    if not k_caches:
        return
    shape = k_caches[0].shape
    for t in k_caches + v_caches:
        if t.shape != shape or t.dtype != k_caches[0].dtype:
            raise ValueError("all caches must share shape and dtype")
    nb = shape[0]
    block_bytes = k_caches[0][0].numel() * k_caches[0].element_size()
    L = len(k_caches)
    kp = (c_vp * L)(*[t.data_ptr() for t in k_caches])
    vp = (c_vp * L)(*[t.data_ptr() for t in v_caches])
    check(lib().pa_copy_blocks(kp, vp, L, block_bytes, nb, pairs.data_ptr(), pairs.shape[0],
                               _stream(stream)))


def _layer_ptrs(k_caches, v_caches):
    k_caches, v_caches = list(k_caches), list(v_caches)
    if len(k_caches) != len(v_caches):
        raise ValueError("K and V layer counts differ")
    _dev(*k_caches, *v_caches)
    shape = k_caches[0].shape
    for t in k_caches + v_caches:
        if t.shape != shape or t.dtype != k_caches[0].dtype:
            raise ValueError("all caches must share shape and dtype")
    L = len(k_caches)
    kp = (c_vp * L)(*[t.data_ptr() for t in k_caches])
    vp = (c_vp * L)(*[t.data_ptr() for t in v_caches])
    block_bytes = k_caches[0][0].numel() * k_caches[0].element_size()
    return kp, vp, L, block_bytes, shape[0]


def swap_record_bytes(k_caches):
    """Host bytes one block takes in a swap record (every layer, K and V)."""
    k_caches = list(k_caches)
    return len(k_caches) * 2 * k_caches[0][0].numel() * k_caches[0].element_size()


def _swap(fn, k_caches, v_caches, blocks, host, host_slots, stream):
    if not k_caches:
        return
    _dev(blocks)
    if blocks.dtype != torch.int32 or blocks.dim() != 1:
        raise ValueError("blocks must be an int32 [n] device tensor")
    if host_slots is not None:
        _dev(host_slots)
        if host_slots.dtype != torch.int32 or host_slots.shape != blocks.shape:
            raise ValueError("host_slots must be an int32 [n] device tensor like blocks")
    if host.is_cuda or not host.is_contiguous():
        raise ValueError("host buffer must be a contiguous host tensor (pin_memory=True)")
    kp, vp, L, block_bytes, nb = _layer_ptrs(k_caches, v_caches)
    host_bytes = host.numel() * host.element_size()
    slots_ptr = host_slots.data_ptr() if host_slots is not None else None
    check(fn(kp, vp, L, block_bytes, nb, blocks.data_ptr(), slots_ptr, blocks.shape[0],
             host.data_ptr(), host_bytes, _stream(stream)))


def pa_swap_out(k_caches, v_caches, blocks, host, host_slots=None, stream=None):
    """Copy the listed blocks of every layer's K and V into records of the
    pinned host tensor ``host`` (R = swap_record_bytes(k_caches) bytes each,
    layer-major, K then V): entry i goes to record host_slots[i], or to
    record i without a slot list."""
    _swap(lib().pa_swap_out, list(k_caches), list(v_caches), blocks, host, host_slots, stream)


def pa_swap_in(k_caches, v_caches, blocks, host, host_slots=None, stream=None):
    """Restore host records (layout of pa_swap_out) into the listed blocks."""
    _swap(lib().pa_swap_in, list(k_caches), list(v_caches), blocks, host, host_slots, stream)


def pa_decode_shared_workspace_bytes(B, num_q_heads, head_dim, max_context_len, partition_tokens):
    """Workspace bytes of pa_decode_shared with a plan (one partition slot
    per (sequence, head) more than pa_decode's)."""
    return lib().pa_decode_shared_workspace_bytes(B, num_q_heads, head_dim, max_context_len,
                                                  partition_tokens)


def pa_decode_workspace_bytes(B, num_q_heads, head_dim, max_context_len, partition_tokens):
    return lib().pa_decode_workspace_bytes(B, num_q_heads, head_dim, max_context_len,
                                           partition_tokens)


def _decode_args(q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                 partition_tokens, out, workspace, stream, with_workspace=True,
                 need_fn=pa_decode_workspace_bytes):
    _dev(q, k_cache, v_cache, block_tables, context_lens)
    B, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    if v_cache.shape != k_cache.shape or d2 != d:
        raise ValueError("shape mismatch")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q and caches must share a dtype")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B, max_blocks]")
    if context_lens.dtype != torch.int32 or context_lens.shape != (B,):
        raise ValueError("context_lens must be int32 [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is not None:
        _dev(out)
        if out.dtype != torch.float32 or out.shape != (B, hq, d):
            raise ValueError("out must be contiguous float32 [B, Hq, D] on the GPU")
    if workspace is not None:
        _check_workspace(workspace)
    need = need_fn(B, hq, d, int(max_context_len), int(partition_tokens)) if with_workspace else 0
    with _on(stream):
        if out is None:
            out = torch.empty((B, hq, d), dtype=torch.float32, device=q.device)
        if need and (workspace is None or workspace.numel() < need):
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if (need and workspace is not None) else None
    ws_bytes = workspace.numel() if ws_ptr else 0
    head = (out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_tables.data_ptr(), block_tables.shape[1], context_lens.data_ptr(),
            int(max_context_len), B, hq, hkv, d, bs, nb, float(scale), int(partition_tokens),
            _dtype_code(q))
    return out, head, (ws_ptr, ws_bytes)


def pa_decode(q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale=None,
              partition_tokens=512, out=None, workspace=None, stream=None):
    """Paged decode attention; returns float32 out [B, Hq, D].

    q [B, Hq, D] and caches [num_blocks, 16, Hkv, D] share a dtype;
    block_tables int32 [B, max_blocks]; context_lens int32 [B];
    max_context_len is a host int bounding context_lens."""
    out, head, ws = _decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                 max_context_len, scale, partition_tokens, out, workspace, stream)
    check(lib().pa_decode(*head, *ws, _stream(stream)))
    return out


def pa_write_decode(q, k_cache, v_cache, k_new, v_new, block_tables, context_lens, max_context_len,
                    scale=None, partition_tokens=512, out=None, workspace=None, stream=None):
    """pa_write_kv of each sequence's new token followed by pa_decode, in
    one call: k_new / v_new [B, Hkv, D] (the caches' dtype) are the K/V rows
    of the token at position context_lens[b] - 1, written to its slot
    through the block table while the decode reads it.  Returns float32
    out [B, Hq, D]."""
    out, head, ws = _decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                 max_context_len, scale, partition_tokens, out, workspace, stream)
    _check_new_rows(q, k_cache, k_new, v_new)
    # head = (out, q, k, v, tables, max_blocks, lens, max_len, B, hq, hkv, d, bs, nb, scale, pt, dtype)
    check(lib().pa_write_decode(*head[:4], k_new.data_ptr(), v_new.data_ptr(), *head[4:], *ws,
                                _stream(stream)))
    return out


def _check_new_rows(q, k_cache, k_new, v_new):
    _dev(k_new, v_new)
    B, hkv, d = q.shape[0], k_cache.shape[2], k_cache.shape[3]
    if k_new.shape != (B, hkv, d) or v_new.shape != (B, hkv, d):
        raise ValueError("k_new and v_new must be [B, Hkv, D]")
    if not (k_new.dtype == v_new.dtype == k_cache.dtype):
        raise ValueError("k_new and v_new must share the caches' dtype")


def pa_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, max_context_len, out,
                      scale=None, partition_tokens=512, stream=None):
    """pa_decode whose split-KV partials live in the library's per-device
    scratch array (pa_decode_noalloc_max_bytes() bytes) instead of a
    workspace: the caller passes every buffer, ``out`` included, and the
    call allocates nothing.  Calls that overlap on one GPU race."""
    if out is None:
        raise ValueError("pa_decode_noalloc needs a caller-owned out")
    out, head, _ = _decode_args(q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                                scale, partition_tokens, out, None, stream, with_workspace=False)
    check(lib().pa_decode_noalloc(*head, _stream(stream)))
    return out


def pa_decode_noalloc_max_bytes():
    return lib().pa_decode_noalloc_max_bytes()


class SharedPlan(tuple):
    """(seq_group, groups, max_shared_parts, max_private_parts), with the
    planner's private-pass hint in ``max_private_blocks``."""
    max_private_blocks = 0


def pa_shared_plan(block_tables, context_lens, block_size, partition_tokens, query_group):
    """Shared-prefix plan from host int32 arrays tables [B, max_blocks] and
    lens [B].  Returns a SharedPlan: (seq_group int32 [B], groups int32
    [n, 17], max_shared_parts, max_private_parts), plus the hint
    ``.max_private_blocks`` for pa_decode_shared."""
    tab = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    if tab.ndim != 2 or lens.shape != (tab.shape[0],):
        raise ValueError("tables must be [B, max_blocks] and lens [B]")
    B = tab.shape[0]
    seq_group = np.empty(B, dtype=np.int32)
    groups = np.empty((max(B // 2, 1), SHARED_ROW), dtype=np.int32)
    n, mx, mp, mb = (ctypes.c_int32(0) for _ in range(4))
    p = ctypes.POINTER(ctypes.c_int32)
    check(lib().pa_shared_plan(tab.ctypes.data_as(p), tab.shape[1], lens.ctypes.data_as(p), B,
                               int(block_size), int(partition_tokens), int(query_group),
                               seq_group.ctypes.data_as(p), groups.ctypes.data_as(p),
                               ctypes.byref(n), ctypes.byref(mx), ctypes.byref(mp),
                               ctypes.byref(mb)))
    plan = SharedPlan((seq_group, groups[:n.value].copy(), mx.value, mp.value))
    plan.max_private_blocks = mb.value
    return plan


def pa_decode_shared(q, k_cache, v_cache, block_tables, context_lens, max_context_len, seq_group,
                     groups, max_shared_parts, max_private_parts=0, scale=None,
                     partition_tokens=512, out=None, workspace=None, stream=None,
                     max_private_blocks=0):
    """pa_decode with a shared-prefix plan: seq_group int32 [B] and groups
    int32 [n, 17] on the GPU (from pa_shared_plan; row = shared blocks, then
    the members); max_shared_parts and max_private_parts are the plan's
    host-side grid bounds (0 for the latter: no bound), max_private_blocks
    its private-pass hint (0: unknown).  A given workspace must hold
    pa_decode_shared_workspace_bytes(...) bytes when the plan has groups."""
    out, head, plan, ws = _shared_args(q, k_cache, v_cache, block_tables, context_lens,
                                       max_context_len, seq_group, groups, max_shared_parts,
                                       max_private_parts, max_private_blocks, scale,
                                       partition_tokens, out, workspace, stream)
    check(lib().pa_decode_shared(*head, *plan, *ws, _stream(stream)))
    return out


def pa_write_decode_shared(q, k_cache, v_cache, k_new, v_new, block_tables, context_lens,
                           max_context_len, seq_group, groups, max_shared_parts,
                           max_private_parts=0, scale=None, partition_tokens=512, out=None,
                           workspace=None, stream=None, max_private_blocks=0):
    """pa_write_decode's write of each sequence's new token (k_new / v_new
    [B, Hkv, D], at position context_lens[b] - 1) with pa_decode_shared's
    decode, in one call; the plan arguments as pa_decode_shared's."""
    out, head, plan, ws = _shared_args(q, k_cache, v_cache, block_tables, context_lens,
                                       max_context_len, seq_group, groups, max_shared_parts,
                                       max_private_parts, max_private_blocks, scale,
                                       partition_tokens, out, workspace, stream)
    _check_new_rows(q, k_cache, k_new, v_new)
    check(lib().pa_write_decode_shared(*head[:4], k_new.data_ptr(), v_new.data_ptr(), *head[4:],
                                       *plan, *ws, _stream(stream)))
    return out


def _shared_args(q, k_cache, v_cache, block_tables, context_lens, max_context_len, seq_group,
                 groups, max_shared_parts, max_private_parts, max_private_blocks, scale,
                 partition_tokens, out, workspace, stream):
    n = 0 if groups is None else groups.shape[0]
    need_fn = (pa_decode_shared_workspace_bytes if n and int(max_shared_parts) > 0
               else pa_decode_workspace_bytes)
    out, head, ws = _decode_args(q, k_cache, v_cache, block_tables, context_lens,
                                 max_context_len, scale, partition_tokens, out, workspace, stream,
                                 need_fn=need_fn)
    if n:
        _dev(seq_group, groups)
        if (seq_group.dtype != torch.int32 or seq_group.shape != (q.shape[0],)
                or groups.dtype != torch.int32 or groups.shape != (n, SHARED_ROW)
                or not groups.is_contiguous()):
            raise ValueError("seq_group must be int32 [B] and groups int32 [n, 17]")
    plan = (seq_group.data_ptr() if n else None, groups.data_ptr() if n else None, n,
            int(max_shared_parts), int(max_private_parts), int(max_private_blocks))
    return out, head, plan, ws


def pa_prefill(q, k_cache, v_cache, block_tables, query_start, context_lens, max_query_len,
               scale=None, out=None, stream=None):
    """Causal attention of uncached suffixes; returns float32 out [T, Hq, D].

    q [T, Hq, D] holds the suffix rows of every sequence, sequence after
    sequence (int32 query_start [B+1] on the GPU); context_lens int32 [B]
    are total lengths; max_query_len is a host int bounding every suffix."""
    _dev(q, k_cache, v_cache, block_tables, query_start, context_lens)
    T, hq, d = q.shape
    nb, bs, hkv, d2 = k_cache.shape
    B = context_lens.shape[0]
    if v_cache.shape != k_cache.shape or d2 != d:
        raise ValueError("shape mismatch")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q and caches must share a dtype")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B, max_blocks]")
    if query_start.dtype != torch.int32 or query_start.shape != (B + 1,):
        raise ValueError("query_start must be int32 [B + 1]")
    if context_lens.dtype != torch.int32:
        raise ValueError("context_lens must be int32 [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        with _on(stream):
            out = torch.empty((T, hq, d), dtype=torch.float32, device=q.device)
    else:
        _dev(out)
        if out.dtype != torch.float32 or out.shape != (T, hq, d):
            raise ValueError("out must be contiguous float32 [T, Hq, D] on the GPU")
    check(lib().pa_prefill(out.data_ptr(), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                           block_tables.data_ptr(), block_tables.shape[1], query_start.data_ptr(),
                           context_lens.data_ptr(), B, T, int(max_query_len), hq, hkv, d, bs, nb,
                           float(scale), _dtype_code(q), _stream(stream)))
    return out


def pa_stream_read(buf, workgroups, sink, stream=None):
    """Streaming read of every byte of the GPU tensor ``buf`` (a size that is
    a multiple of 16 bytes) by ``workgroups`` workgroups, each reading one
    contiguous chunk; ``sink`` is an int32 GPU tensor of >= workgroups
    entries (rarely written).  Measures the HBM read rate reachable on the
    GPU."""
    _dev(buf, sink)
    nbytes = buf.numel() * buf.element_size()
    if sink.dtype != torch.int32 or sink.numel() < workgroups:
        raise ValueError("sink must be an int32 GPU tensor of >= workgroups entries")
    check(lib().pa_stream_read(buf.data_ptr(), nbytes, int(workgroups), sink.data_ptr(),
                               _stream(stream)))

"""Stage a batch on the device through the library: block allocation
(kv_pool_alloc), table upload, and K/V scatter-write (kv_append_scatter).

This is how a caller prepares one step: every sequence first gets blocks for
its resident context, then for the tokens the step appends; resident K/V are
written once; the step's K/V are written by the step itself.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from . import (BLOCK_SIZE, empty_pools, kv_append_scatter, kv_pool_alloc, kv_pool_create,
               paged_attention_workspace_size)


@dataclass
class Staged:
    pool: object                 # host block manager
    tables_np: np.ndarray        # int32 [S, max_blocks]
    step_slots_np: np.ndarray    # int32 [n_step_total]
    k_pools: list                # device tensors, one per copy ("layer")
    v_pools: list
    q: object                    # device [rows, Hq, D]
    tables: object               # device int32 [S, max_blocks]
    context_lens: object         # device int32 [S]
    qsl: object                  # device int32 [S+1]
    k_step: object               # device [n_step_total, Hkv, D]
    v_step: object
    step_slots: object           # device int32 [n_step_total]
    sinks: Optional[object]
    out: object                  # device float32 [rows, Hq, D]
    workspace: object
    max_q_len: int
    max_context_len: int
    max_blocks: int
    unique_blocks: int           # physical blocks holding the batch's keys


def prefix_hint(tables, min_tokens: int = 256):
    """(prefix_seqs, prefix_tokens) for paged_attention_prefix_forward from
    the host block tables of a batch (int32 [S, max_blocks]): the run of
    sequences from 0 whose leading table entries name the same physical
    blocks as sequence 0's for at least min_tokens positions, and the
    positions all of them hold in those blocks. (0, 0) when there is none.
    This is what the block manager knows when it hands out shared blocks."""
    tables = np.asarray(tables)
    if tables.shape[0] < 2:
        return 0, 0
    first = tables[0]
    common = []
    for row in tables[1:]:
        same = (row == first) & (first >= 0)
        k = int(np.argmin(same)) if not same.all() else same.size
        if k * BLOCK_SIZE < min_tokens:
            break
        common.append(k)
    if not common:
        return 0, 0
    return len(common) + 1, min(common) * BLOCK_SIZE


def _torch_dtype(name):
    """Element type of the pools for a workload dtype ("fp8", "fp4": 8- and
    4-bit pools)."""
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": "fp8", "fp4": "fp4"}[name]


def _to_device(a, dtype_name, device):
    """Rows (queries, new K/V) to the device; "fp8" and "fp4" workloads carry
    bf16 rows."""
    import torch
    if dtype_name in ("bf16", "fp8", "fp4"):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)
        return t.view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def stage(w, device="cuda", copies: int = 1, poison: bool = True, scatter_step: bool = True) -> Staged:
    """w: a workload (synth.Workload). copies: independent pool copies sharing
    the tables (model layers). poison: fill pools with NaN first, so that any
    read of an unwritten slot shows up in the result."""
    import torch
    S = len(w.seqs)
    maxb = w.max_blocks_per_seq
    pool = kv_pool_create(w.num_blocks, BLOCK_SIZE, w.free_order)
    res_slots: List[np.ndarray] = []
    for s, seq in enumerate(w.seqs):
        n_res = seq.ctx - seq.n_step
        _, _, _, slots = kv_pool_alloc(pool, s, seq.tokens[:n_res], maxb)
        res_slots.append(slots)
    tables = np.full((S, maxb), -1, dtype=np.int32)
    step_slots = []
    for s, seq in enumerate(w.seqs):
        row, nb, ctx, slots = kv_pool_alloc(pool, s, seq.tokens[seq.ctx - seq.n_step:], maxb)
        assert ctx == seq.ctx
        tables[s] = row
        step_slots.append(slots)
    unique = len({int(b) for s, seq in enumerate(w.seqs) for b in tables[s, :-(-seq.ctx // BLOCK_SIZE)]})

    dt = _torch_dtype(w.dtype)
    Hkv, D = w.num_kv_heads, w.head_dim
    k0, v0 = empty_pools(w.num_blocks, Hkv, D, dt, device)
    if poison and w.dtype in ("fp8", "fp4"):
        k0.fill_(0xFF)   # code 0xFF is NaN in E4M3FN, four 0xFF bytes a NaN scale
        v0.fill_(0xFF)
    elif poison:
        k0.fill_(float("nan"))
        v0.fill_(float("nan"))
    else:
        k0.zero_()
        v0.zero_()
    # resident context
    kr = np.concatenate([seq.k[:seq.ctx - seq.n_step] for seq in w.seqs])
    vr = np.concatenate([seq.v[:seq.ctx - seq.n_step] for seq in w.seqs])
    sr = np.concatenate(res_slots).astype(np.int32)
    if sr.size:
        kv_append_scatter(_to_device(kr, w.dtype, device), _to_device(vr, w.dtype, device),
                          torch.from_numpy(sr).to(device), k0, v0)
    ks = np.concatenate([seq.k[seq.ctx - seq.n_step:] for seq in w.seqs])
    vs = np.concatenate([seq.v[seq.ctx - seq.n_step:] for seq in w.seqs])
    ss = np.concatenate(step_slots).astype(np.int32)
    k_step = _to_device(ks, w.dtype, device)
    v_step = _to_device(vs, w.dtype, device)
    step_dev = torch.from_numpy(ss).to(device)
    if scatter_step:
        kv_append_scatter(k_step, v_step, step_dev, k0, v0)
    k_pools, v_pools = [k0], [v0]
    for _ in range(1, copies):
        k_pools.append(k0.clone())
        v_pools.append(v0.clone())
    rows = w.total_rows
    max_ctx = int(max(seq.ctx for seq in w.seqs))
    ws = paged_attention_workspace_size(S, rows, w.num_q_heads, D, max_ctx)
    return Staged(
        pool=pool, tables_np=tables, step_slots_np=ss, k_pools=k_pools, v_pools=v_pools,
        q=_to_device(w.q, w.dtype, device), tables=torch.from_numpy(tables).to(device),
        context_lens=torch.from_numpy(w.context_lens).to(device), qsl=torch.from_numpy(w.qsl).to(device),
        k_step=k_step, v_step=v_step, step_slots=step_dev,
        sinks=None if w.sinks is None else torch.from_numpy(w.sinks).to(device),
        out=torch.empty((rows, w.num_q_heads, D), dtype=torch.float32, device=device),
        workspace=torch.zeros(max(ws, 1), dtype=torch.uint8, device=device),
        max_q_len=int(max(seq.q_len for seq in w.seqs)), max_context_len=max_ctx, max_blocks=maxb,
        unique_blocks=unique)

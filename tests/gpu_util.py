"""Shared helpers of the GPU tests: the oracle side of a workload and small
custom workloads. Importing this module needs no GPU."""
from __future__ import annotations

import numpy as np

import oracle
import synth

TOL = {"bf16": 2e-3, "f32": 1e-5, "fp8": 2e-3, "fp4": 2e-3}


def oracle_side(w, fill_nan=True, tree_mask=None, window=0, drop=None):
    """Oracle allocation (same call order as the device staging), oracle
    scatter into NaN-filled pools, oracle paged attention (with tree masks
    and a sliding window when given). drop: {sequence: first kept position}
    frees those sequences' blocks below it after the scatter."""
    a = oracle.Allocator(w.num_blocks, w.block_size, w.free_order)
    maxb = w.max_blocks_per_seq
    res, step = [], []
    for s, seq in enumerate(w.seqs):
        res.append(a.alloc(s, seq.tokens[:seq.ctx - seq.n_step], maxb)[3])
    tables = []
    for s, seq in enumerate(w.seqs):
        row, nb, ctx, slots = a.alloc(s, seq.tokens[seq.ctx - seq.n_step:], maxb)
        tables.append(row)
        step.append(slots)
    if w.dtype == "fp8":
        kp, vp = oracle.fp8_empty_pools(w.num_blocks, w.num_kv_heads, w.head_dim,
                                        fill=np.uint8(0xFF) if fill_nan else None)
        put = oracle.fp8_scatter
    elif w.dtype == "fp4":
        kp, vp = oracle.fp4_empty_pools(w.num_blocks, w.num_kv_heads, w.head_dim,
                                        fill=np.uint8(0xFF) if fill_nan else None)
        put = oracle.fp4_scatter
    else:
        nan = np.uint16(0x7FC0) if w.dtype == "bf16" else np.float32(np.nan)
        kp, vp = oracle.empty_pools(w.num_blocks, w.num_kv_heads, w.head_dim, w.block_size, w.dtype,
                                    fill=nan if fill_nan else None)
        put = oracle.scatter
    for s, seq in enumerate(w.seqs):
        n_res = seq.ctx - seq.n_step
        put(kp, vp, seq.k[:n_res], seq.v[:n_res], res[s])
        put(kp, vp, seq.k[n_res:], seq.v[n_res:], step[s])
    if drop:
        for s, first in drop.items():
            a.drop_prefix(s, first)
        tables = [a.table_row(s, maxb) for s in range(len(w.seqs))]
    tables = np.array(tables, dtype=np.int32)
    out = oracle.paged_attention(w.q, kp, vp, tables, w.context_lens, w.qsl, w.num_q_heads,
                                 w.num_kv_heads, w.scale, w.sinks, w.dtype, tree_mask=tree_mask, window=window)
    return tables, kp, vp, out


def _dense(rows, dtype):
    """Dense K or V rows as the attention sees them: for 8- and 4-bit pools
    the oracle's quantize-then-dequantize of each (token, KV head) row."""
    if dtype == "fp8":
        return oracle.fp8_dequantize(*oracle.fp8_quantize_rows(rows))
    if dtype == "fp4":
        return oracle.fp4_dequantize(*oracle.fp4_quantize_rows(rows))
    return rows


def oracle_rows(w, rows):
    """Oracle output for a subset of global query rows, from the dense K/V."""
    qsl = w.qsl
    ks, vs, qsel, qls = [], [], [], []
    for i in rows:
        s = int(np.searchsorted(qsl, i, side="right") - 1)
        seq = w.seqs[s]
        p = seq.ctx - seq.q_len + (i - int(qsl[s]))
        ks.append(_dense(seq.k[:p + 1], w.dtype))
        vs.append(_dense(seq.v[:p + 1], w.dtype))
        qsel.append(w.q[i])
    q = np.stack(qsel)
    return oracle.attention(q, ks, vs, np.arange(len(rows) + 1, dtype=np.int32), w.num_q_heads,
                            w.num_kv_heads, w.scale, w.sinks, w.dtype)


def custom(dtype, Hq, Hkv, D, ctxs, q_lens, seed, sinks=False, shared_prefix=0, n_shared=0, scale=None):
    return synth.build("custom", dtype, Hq, Hkv, D, ctxs, q_lens, seed, sinks=sinks,
                       shared_prefix=shared_prefix, n_shared=n_shared, scale=scale)


def run_forward(pk, st, w, k_pool=None, v_pool=None):
    return pk.paged_attention_forward(
        st.q, st.k_pools[0] if k_pool is None else k_pool, st.v_pools[0] if v_pool is None else v_pool,
        st.tables, st.context_lens, st.qsl, st.max_q_len, st.max_context_len, w.scale,
        sinks=st.sinks, out=st.out, workspace=st.workspace)


def max_err(got, want):
    return float(np.max(np.abs(got.astype(np.float64) - want))) if got.size else 0.0

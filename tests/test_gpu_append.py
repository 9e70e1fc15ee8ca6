"""paged_attention_append_forward (GPU): one call that appends each row's own
token and attends must equal kv_append_scatter followed by
paged_attention_forward, bit for bit in the output and in both pools, on
decode batches (where the new tokens are taken inside the attention launch)
and on other batches (scattered first). Both sides start from the same pools,
NaN-filled wherever nothing was written, so a new key read from the pool
before it was written would show up as NaN.
"""
import sys

import numpy as np
import pytest

import synth
from gpu_util import TOL, custom, max_err, oracle_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a device"
    import paged_kv_attention_block_amd as pk
    return pk


def _bits(t):
    import torch
    if t.dtype == torch.uint8:
        return t.cpu().numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy()
    return t.cpu().numpy().view(np.uint32)


def _both(pk, w, resident_slots=()):
    """Run the two-call path and the one-call path from identical pools;
    return both outputs and pools. Sequences listed in resident_slots get
    their new token written beforehand and slot -1 in both paths."""
    import torch
    from paged_kv_attention_block_amd.staging import stage
    print(f"\n[case] append {w.name} dtype={w.dtype} S={len(w.seqs)} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"D={w.head_dim} ctx={[s.ctx for s in w.seqs][:8]} q_len={[s.q_len for s in w.seqs][:8]}", flush=True)
    st = stage(w, copies=2, poison=True, scatter_step=False)
    slots = st.step_slots.clone()
    qsl = w.qsl
    for s in resident_slots:
        rows = slice(int(qsl[s]), int(qsl[s + 1]))
        for l in range(2):
            pk.kv_append_scatter(st.k_step[rows], st.v_step[rows], slots[rows], st.k_pools[l], st.v_pools[l])
        slots[rows] = -1
    torch.cuda.synchronize()
    outs = []
    pk.kv_append_scatter(st.k_step, st.v_step, slots, st.k_pools[0], st.v_pools[0])
    outs.append(pk.paged_attention_forward(st.q, st.k_pools[0], st.v_pools[0], st.tables, st.context_lens, st.qsl,
                                           st.max_q_len, st.max_context_len, w.scale, sinks=st.sinks).clone())
    outs.append(pk.paged_attention_append_forward(st.q, st.k_step, st.v_step, slots, st.k_pools[1], st.v_pools[1],
                                                  st.tables, st.context_lens, st.qsl, st.max_q_len,
                                                  st.max_context_len, w.scale, sinks=st.sinks).clone())
    torch.cuda.synchronize()
    return st, outs


def _check(pk, w, resident_slots=(), oracle_sample=None):
    st, (a, b) = _both(pk, w, resident_slots)
    np.testing.assert_array_equal(_bits(st.k_pools[0]), _bits(st.k_pools[1]))
    np.testing.assert_array_equal(_bits(st.v_pools[0]), _bits(st.v_pools[1]))
    ga, gb = a.cpu().numpy(), b.cpu().numpy()
    assert np.all(np.isfinite(gb))
    np.testing.assert_array_equal(ga.view(np.uint32), gb.view(np.uint32))
    rows = list(range(w.total_rows)) if oracle_sample is None else oracle_sample
    err = max_err(gb[rows], oracle_rows(w, rows))
    print(f"[case] append {w.name}: bitwise equal to scatter + forward; max abs err vs oracle {err:.3e}", flush=True)
    assert err <= TOL[w.dtype]


def test_mid_decode_small_grid(pk):
    _check(pk, synth.mid_decode())


def test_sink_decode_large_grid(pk):
    _check(pk, synth.sink_decode(), oracle_sample=[0, 7, 31])


@pytest.mark.parametrize("dtype", ["fp8", "fp4"])
def test_decode_into_quantized_pools(pk, dtype):
    """Decode rows into 8- and 4-bit pools: the new tokens are quantized by
    the scatter launch, then attended."""
    _check(pk, synth.sink_decode(dtype=dtype), oracle_sample=[0, 7, 31])


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 2, 64), (40, 2, 128), (4, 4, 128)])
def test_block_and_split_boundaries(pk, Hq, Hkv, D):
    """New tokens at every offset class in a block and next to split edges;
    40/2 heads take the two-tile rows, which scatter first."""
    ctxs = [1, 2, 15, 16, 17, 31, 32, 33, 255, 256, 257, 1023, 1024, 1025, 2047, 2048, 2049, 3072, 4097]
    w = custom("bf16", Hq, Hkv, D, ctxs, [1] * len(ctxs), seed=Hq * 100 + Hkv * 10 + D, sinks=(Hq % 8 == 0))
    _check(pk, w)


def test_resident_token_slot_minus_one(pk):
    """slot -1: the token is already in the pool; nothing is written and the
    one-call path still attends to it."""
    w = custom("bf16", 32, 8, 128, [100, 300, 17, 64], [1] * 4, seed=4321)
    _check(pk, w, resident_slots=(1, 3))


@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp8", "fp4"])
def test_other_batches_scatter_first(pk, dtype):
    """Verify windows, prefill chunks, fp32, 8- and 4-bit pools take the scatter
    launch first; the result is the same as two calls."""
    w = custom(dtype, 16, 4, 64, [300, 1100, 70, 40], [8, 130, 1, 40], seed=99)
    _check(pk, w)


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp4"])
@pytest.mark.parametrize("D", [64, 128])
def test_wide_query_groups_append(pk, dtype, D):
    """64 query heads on one KV head: the appending call scatters first and
    equals two calls."""
    w = custom(dtype, 64, 1, D, [3000, 700, 1025, 64, 1], [1] * 5, seed=320 + D, sinks=True)
    _check(pk, w)

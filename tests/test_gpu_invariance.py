"""Bitwise row invariance of the HIP path (GPU).

The speculative-decoding pages demand that a verify-window row uses exactly
the arithmetic of the serial step, so that a row computed alone and the same
row inside a window (or a batch) are bitwise identical. "Alone" here is the
plainest reading: the same query submitted by itself as a decode row
(q_len = 1) over the keys up to its position, through the same block table.
"""
import copy
import sys

import numpy as np
import pytest

from gpu_util import custom, run_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a device"
    import paged_kv_attention_block_amd as pk
    return pk


def announce(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def bits(t):
    import torch
    return t.contiguous().view(torch.int32).cpu().numpy()


def alone(pk, st, w, i):
    """Row i as a single decode row over keys 0..p."""
    import torch
    qsl = w.qsl
    s = int(np.searchsorted(qsl, i, side="right") - 1)
    seq = w.seqs[s]
    p = seq.ctx - seq.q_len + (i - int(qsl[s]))
    dev = st.q.device
    return pk.paged_attention_forward(
        st.q[i:i + 1].contiguous(), st.k_pools[0], st.v_pools[0], st.tables[s:s + 1].contiguous(),
        torch.tensor([p + 1], dtype=torch.int32, device=dev), torch.tensor([0, 1], dtype=torch.int32, device=dev),
        1, p + 1, w.scale, sinks=st.sinks)


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [("bf16", 32, 8, 128), ("bf16", 64, 8, 64), ("f32", 4, 2, 64),
                                             ("bf16", 8, 8, 64), ("fp8", 32, 8, 128), ("fp8", 64, 8, 64),
                                             ("fp4", 32, 8, 128), ("fp4", 64, 8, 64)])
def test_window_rows_equal_rows_alone(pk, dtype, Hq, Hkv, D):
    import torch
    from paged_kv_attention_block_amd.staging import stage
    w = custom(dtype, Hq, Hkv, D, [1000, 4100, 6000, 70], [8, 8, 8, 8], seed=90 + D + Hq, sinks=True)
    announce(f"window invariance {dtype} {Hq}/{Hkv} D{D}")
    st = stage(w)
    full = bits(run_forward(pk, st, w))
    for i in range(w.total_rows):
        got = bits(alone(pk, st, w, i))
        np.testing.assert_array_equal(got[0], full[i], err_msg=f"row {i}")


@pytest.mark.parametrize("dtype", ["fp8", "fp4"])
def test_quantized_mixed_batch_rows_equal_rows_alone(pk, dtype):
    """8- and 4-bit batches with a prefill chunk take a one-tile split launch
    that covers windows of 17-32 rows in two passes: those rows, the decode
    rows and the prefill rows each equal themselves alone."""
    from paged_kv_attention_block_amd.staging import stage
    # Hq/Hkv = 4: windows of 5 and 8 rows are 20 and 32 rows per KV head
    w = custom(dtype, 16, 4, 128, [2600, 1300, 900, 5000], [5, 300, 1, 8], seed=99, sinks=True)
    announce(f"quantized mixed-batch invariance {dtype}")
    st = stage(w)
    full = bits(run_forward(pk, st, w))
    for i in [0, 2, 4, 5, 6, 150, 304, 305, 306, 308, 312]:
        np.testing.assert_array_equal(bits(alone(pk, st, w, i))[0], full[i], err_msg=f"row {i}")


def test_prefill_rows_equal_rows_alone(pk):
    from paged_kv_attention_block_amd.staging import stage
    w = custom("bf16", 16, 4, 128, [1500, 300], [200, 300], seed=95, sinks=True)
    announce("prefill invariance")
    st = stage(w)
    full = bits(run_forward(pk, st, w))
    for i in [0, 1, 15, 16, 17, 63, 64, 199, 200, 201, 299, 350, 499]:
        np.testing.assert_array_equal(bits(alone(pk, st, w, i))[0], full[i], err_msg=f"row {i}")


def test_batch_invariance(pk):
    """A sequence alone and inside a batch of others gives the same bits."""
    from paged_kv_attention_block_amd.staging import stage
    ctxs = [800, 3000, 17, 5000, 1024]
    qls = [1, 8, 1, 1, 4]
    w = custom("bf16", 32, 8, 128, ctxs, qls, seed=96)
    announce("batch invariance")
    full = bits(run_forward(pk, stage(w), w))
    start = 0
    for s in range(len(ctxs)):
        ws = copy.deepcopy(w)
        ws.seqs = [w.seqs[s]]
        ws.q = w.q[start:start + qls[s]]
        one = bits(run_forward(pk, stage(ws), ws))
        np.testing.assert_array_equal(one, full[start:start + qls[s]], err_msg=f"seq {s}")
        start += qls[s]


def test_block_placement_invariance(pk):
    """Another physical placement of the same blocks gives the same bits."""
    from paged_kv_attention_block_amd.staging import stage
    w = custom("bf16", 64, 8, 64, [900, 2100, 33], [1, 3, 1], seed=97, sinks=True)
    announce("placement invariance")
    a = bits(run_forward(pk, stage(w), w))
    w2 = copy.deepcopy(w)
    w2.free_order = np.random.default_rng(5).permutation(w.num_blocks).astype(np.int32)
    b = bits(run_forward(pk, stage(w2), w2))
    np.testing.assert_array_equal(a, b)


def test_shared_prefix_equals_private_copies(pk):
    from paged_kv_attention_block_amd.staging import stage
    w = custom("bf16", 32, 8, 128, [700, 650, 901], [1, 1, 3], seed=98, shared_prefix=600, n_shared=3)
    announce("shared vs private prefix")
    st = stage(w)
    assert (st.tables_np[0, :37] == st.tables_np[1, :37]).all()
    a = bits(run_forward(pk, st, w))
    w2 = copy.deepcopy(w)
    rng = np.random.default_rng(6)
    for seq in w2.seqs:                      # distinct token ids, same K/V bytes: no sharing
        seq.tokens = rng.integers(0, 1 << 30, size=seq.ctx).astype(np.int32)
    w2.num_blocks = 3 * w.num_blocks         # private copies need room for every block
    w2.free_order = rng.permutation(w2.num_blocks).astype(np.int32)
    st2 = stage(w2)
    assert not (st2.tables_np[0, :37] == st2.tables_np[1, :37]).any()
    np.testing.assert_array_equal(a, bits(run_forward(pk, st2, w2)))


def test_run_to_run_determinism(pk):
    from paged_kv_attention_block_amd.staging import stage
    w = custom("bf16", 32, 8, 128, [4000, 12000, 100, 7000], [8, 1, 16, 3], seed=99, sinks=True)
    announce("determinism")
    st = stage(w)
    a = bits(run_forward(pk, st, w)).copy()
    for _ in range(3):
        np.testing.assert_array_equal(bits(run_forward(pk, st, w)), a)


@pytest.mark.parametrize("dtype,S,D,maxctx", [("bf16", 40, 128, 6000), ("bf16", 64, 64, 6000), ("bf16", 65, 64, 6000),
                                              ("fp8", 64, 64, 2500), ("fp4", 48, 64, 2500)])
def test_decode_batch_dispatch_orders(pk, dtype, S, D, maxctx):
    """Decode batches large enough that workgroups queue are dealt in an order
    computed from the context lengths (up to 64 sequences; 65 take the fixed
    slot order): split-aligned lengths, one-key last splits, contexts below
    one large split and long ones. Every row matches the oracle and equals
    itself alone (a grid too small to queue, in the fixed order)."""
    from gpu_util import TOL, max_err, oracle_side
    from paged_kv_attention_block_amd.staging import stage
    rng = np.random.default_rng(300 + S + D)
    edge = [c for c in [1, 2, 255, 256, 257, 1023, 1024, 1025, 2048, 2049, 3072, 4096, 5000] if c <= maxctx]
    ctxs = (edge + [int(x) for x in rng.integers(1, maxctx, size=S)])[:S]
    rng.shuffle(ctxs)
    w = custom(dtype, 32, 8, D, ctxs, [1] * S, seed=310 + S, sinks=True)
    announce(f"decode dispatch order {dtype} S={S} D={D}")
    st = stage(w)
    out = run_forward(pk, st, w)
    got = out.cpu().numpy()
    want = oracle_side(w)[3]
    err = max_err(got, want)
    print(f"[case] max abs err {err:.3e}", flush=True)
    assert np.all(np.isfinite(got)) and err <= TOL[dtype]
    full = bits(out)
    for i in sorted(set([0, S - 1] + [ctxs.index(c) for c in edge if c in ctxs] +
                        [int(x) for x in rng.integers(0, S, size=6)])):
        np.testing.assert_array_equal(bits(alone(pk, st, w, i))[0], full[i], err_msg=f"row {i} ctx {ctxs[i]}")


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [("bf16", 32, 8, 128), ("bf16", 64, 8, 64), ("bf16", 16, 8, 64),
                                             ("fp8", 32, 8, 128), ("fp4", 32, 8, 128)])
def test_shared_prefix_batch_rows(pk, dtype, Hq, Hkv, D):
    """A decode batch in which sequences 0-9 share a 2100-token prefix (five
    whole splits read through the same blocks) and 10-13 have private
    blocks. Every row matches the oracle, equals itself alone, and equals
    the same batch with private copies of the prefix blocks."""
    from gpu_util import TOL, max_err, oracle_side
    from paged_kv_attention_block_amd.staging import stage
    rng = np.random.default_rng(400 + D + Hq)
    ctxs = [2100 + int(x) for x in rng.integers(1, 900, size=12)] + [3000, 1500]
    w = custom(dtype, Hq, Hkv, D, ctxs, [1] * len(ctxs), seed=410 + Hq, sinks=True, shared_prefix=2100, n_shared=10)
    announce(f"shared-prefix batch {dtype} {Hq}/{Hkv} D{D}")
    st = stage(w)
    assert (st.tables_np[0, :131] == st.tables_np[9, :131]).all()
    out = run_forward(pk, st, w)
    got = out.cpu().numpy()
    err = max_err(got, oracle_side(w)[3])
    print(f"[case] max abs err {err:.3e}", flush=True)
    assert np.all(np.isfinite(got)) and err <= TOL[dtype]
    full = bits(out)
    for i in range(len(ctxs)):
        np.testing.assert_array_equal(bits(alone(pk, st, w, i))[0], full[i], err_msg=f"row {i}")
    w2 = copy.deepcopy(w)
    r2 = np.random.default_rng(7)
    for seq in w2.seqs:                      # distinct token ids, same K/V bytes: no sharing
        seq.tokens = r2.integers(0, 1 << 30, size=seq.ctx).astype(np.int32)
    w2.num_blocks = 4 * w.num_blocks
    w2.free_order = r2.permutation(w2.num_blocks).astype(np.int32)
    st2 = stage(w2)
    assert not (st2.tables_np[0, :131] == st2.tables_np[1, :131]).any()
    np.testing.assert_array_equal(full, bits(run_forward(pk, st2, w2)))


@pytest.mark.parametrize("name", ["verify_window", "verify_window_fp8", "verify_window_fp4"])
def test_verify_window_workload_every_row_equals_row_alone(pk, name):
    """The 8-row speculative verify windows of 16 sequences with contexts of
    4096-16384 keys (the TensorFold page's row-invariant wide-window rule):
    each of the 128 rows, computed alone as a decode row over the keys up to
    its position, gives the bits it has inside its window."""
    import synth
    from paged_kv_attention_block_amd.staging import stage
    w = synth.by_name(name)
    announce(f"{name}: all {w.total_rows} rows alone, contexts {min(s.ctx for s in w.seqs)}-"
             f"{max(s.ctx for s in w.seqs)}")
    st = stage(w)
    full = bits(run_forward(pk, st, w))
    for i in range(w.total_rows):
        np.testing.assert_array_equal(bits(alone(pk, st, w, i))[0], full[i], err_msg=f"row {i}")


@pytest.mark.parametrize("dtype", ["bf16", "fp4"])
def test_mixed_step_workload_rows_equal_rows_alone(pk, dtype):
    """The continuous-batching step: every decode row over the 181 hash-shared
    prefix blocks, and prefill rows 0, 15, 16, 63, 64 and 1023 of both
    1024-row chunks, each equal to itself computed alone (the ds4 glossary's
    rule that batched results equal per-session results)."""
    import synth
    from paged_kv_attention_block_amd.staging import stage
    w = synth.mixed_step(dtype=dtype)
    qsl = w.qsl
    n_dec = sum(1 for s in w.seqs if s.q_len == 1)
    rows = list(range(n_dec))
    for s in range(n_dec, len(w.seqs)):
        rows += [int(qsl[s]) + r for r in (0, 15, 16, 63, 64, 1023)]
    announce(f"mixed_step {dtype}: {len(rows)} rows alone ({n_dec} decode rows over the shared prefix)")
    st = stage(w)
    shared = set(st.tables_np[0, :181].tolist())
    assert all(set(st.tables_np[s, :181].tolist()) == shared for s in range(n_dec))
    full = bits(run_forward(pk, st, w))
    for i in rows:
        np.testing.assert_array_equal(bits(alone(pk, st, w, i))[0], full[i], err_msg=f"row {i}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp4"])
@pytest.mark.parametrize("D", [64, 128])
def test_wide_query_groups_rows_equal_rows_alone(pk, dtype, D):
    """64 query heads on one KV head (more rows per KV head than one split
    workgroup takes): decode rows and an 8-row window, each row equal to
    itself alone."""
    from paged_kv_attention_block_amd.staging import stage
    w = custom(dtype, 64, 1, D, [3000, 700, 1025, 64], [1, 8, 1, 1], seed=310 + D, sinks=True)
    announce(f"wide groups invariance {dtype} 64/1 D{D}")
    st = stage(w)
    full = bits(run_forward(pk, st, w))
    for i in range(w.total_rows):
        np.testing.assert_array_equal(bits(alone(pk, st, w, i))[0], full[i], err_msg=f"row {i}")

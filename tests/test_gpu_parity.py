"""Parity of the HIP path with the oracle (GPU).

Every test compares the library's output, produced through the C ABI
(kv_pool_alloc, kv_append_scatter, paged_attention_forward), with the fp64
oracle on the same seeded inputs: max-abs error <= 2e-3 for bf16 K/V and for
8- and 4-bit pools (against the oracle's attention over its own dequantized codes),
<= 1e-5 for fp32 K/V, and bit-exact pools after the scatter-write.
"""
import sys

import numpy as np
import pytest

import synth
from gpu_util import TOL, custom, max_err, oracle_rows, oracle_side, run_forward

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


def _bits(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint32)


def check_workload(pk, w, compare_pools=True, sample_rows=None):
    import torch
    from paged_kv_attention_block_amd.staging import stage
    announce(f"{w.name} dtype={w.dtype} S={len(w.seqs)} rows={w.total_rows} Hq={w.num_q_heads} "
             f"Hkv={w.num_kv_heads} D={w.head_dim} maxctx={max(s.ctx for s in w.seqs)}")
    st = stage(w)
    out = run_forward(pk, st, w)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    if sample_rows is None:
        tables_o, kp_o, vp_o, want = oracle_side(w)
        np.testing.assert_array_equal(st.tables_np, tables_o)
        if compare_pools:
            ok = w.dtype == "bf16" and np.uint16 or np.uint32
            np.testing.assert_array_equal(_bits(st.k_pools[0]), kp_o.view(ok))
            np.testing.assert_array_equal(_bits(st.v_pools[0]), vp_o.view(ok))
        err = max_err(got, want)
    else:
        want = oracle_rows(w, sample_rows)
        err = max_err(got[sample_rows], want)
    print(f"[case] {w.name}: max abs err {err:.3e} (tol {TOL[w.dtype]})", flush=True)
    assert np.all(np.isfinite(got))
    assert err <= TOL[w.dtype]
    return st, got


@pytest.mark.parametrize("name", ["tiny_decode", "mid_decode", "sink_decode", "verify_window",
                                  "mid_decode_fp8", "sink_decode_fp8", "verify_window_fp8",
                                  "mid_decode_fp4", "sink_decode_fp4", "verify_window_fp4"])
def test_named_workloads_full(pk, name):
    check_workload(pk, synth.by_name(name))


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp4"])
def test_mixed_step_full(pk, dtype):
    check_workload(pk, synth.mixed_step(dtype=dtype))


@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp8", "fp4"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (8, 8), (16, 2), (12, 4)])
def test_small_shapes(pk, dtype, D, Hq, Hkv):
    """Several tiles, ragged tails, every split segment boundary nearby."""
    rng = np.random.default_rng(D + Hq * 7 + Hkv + (dtype == "bf16"))
    ctxs = [1, 15, 16, 17, 63, 64, 65, 129, int(rng.integers(200, 900)), 1023, 1024, 1025, 4097]
    q_lens = [1] * len(ctxs)
    q_lens[2] = 16
    q_lens[5] = 3
    q_lens[8] = 37
    q_lens[11] = 9
    w = custom(dtype, Hq, Hkv, D, ctxs, q_lens, seed=int(rng.integers(1 << 30)), sinks=(Hq % 8 == 0))
    check_workload(pk, w)


@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp8", "fp4"])
def test_prefill_chunks_and_decode_mixed(pk, dtype):
    """Long prefill windows (multi-rowblock path) next to decode rows."""
    w = custom(dtype, 8, 2, 128, [300, 1100, 70, 2500, 5], [300, 130, 1, 1, 5], seed=77, sinks=True)
    check_workload(pk, w)


def test_prefill_from_zero_full_causal(pk):
    w = custom("bf16", 32, 8, 128, [1024], [1024], seed=78)
    check_workload(pk, w)


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp4"])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_chunk_on_long_context(pk, D, dtype):
    """Prefill chunks whose rows see thousands of keys: the prefill shape walks
    many 32-step windows of block ids, across both split sizes."""
    w = custom(dtype, 16, 4, D, [5000, 2300, 700], [200, 33, 9], seed=80 + D, sinks=True)
    check_workload(pk, w)


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp4"])
def test_long_context(pk, dtype):
    w = custom(dtype, 16, 2, 128, [20000, 9000], [1, 4], seed=79, sinks=True)
    check_workload(pk, w)


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp4"])
def test_shared_prefix_sequences(pk, dtype):
    w = custom(dtype, 16, 4, 64, [700, 650, 901, 64], [1, 1, 3, 1], seed=80, shared_prefix=600, n_shared=3)
    check_workload(pk, w)


def test_scale_zero_gives_mean(pk):
    """scale 0: every visible key weighs the same; output = mean of V."""
    w = custom("f32", 4, 2, 64, [37, 100], [1, 5], seed=81, scale=0.0)
    st, got = check_workload(pk, w)
    row = 0
    for seq in w.seqs:
        for r in range(seq.q_len):
            p = seq.ctx - seq.q_len + r
            mean = seq.v[:p + 1].astype(np.float64).mean(axis=0)     # [Hkv, D]
            want = np.repeat(mean, 2, axis=0)
            assert np.max(np.abs(got[row + r] - want)) < 1e-5
        row += seq.q_len


def test_empty_batch_is_noop(pk):
    import torch
    q = torch.zeros((0, 4, 64), dtype=torch.bfloat16, device="cuda")
    kp, vp = pk.empty_pools(4, 2, 64, torch.bfloat16)
    bt = torch.zeros((0, 4), dtype=torch.int32, device="cuda")
    cl = torch.zeros((0,), dtype=torch.int32, device="cuda")
    qsl = torch.zeros((1,), dtype=torch.int32, device="cuda")
    out = pk.paged_attention_forward(q, kp, vp, bt, cl, qsl, 1, 64, 0.125)
    torch.cuda.synchronize()
    assert out.shape == (0, 4, 64)


def test_workspace_reuse(pk):
    """One workspace, left as the previous call wrote it, serves consecutive
    calls of different shapes; each call matches the oracle (stale split
    states must never leak into a later call)."""
    import torch
    from paged_kv_attention_block_amd.staging import stage
    ws = None
    for i, (S, lo, hi, q_len) in enumerate([(24, 3000, 9000, 1), (6, 200, 900, 1), (12, 2500, 7000, 8)]):
        rng = np.random.default_rng(4242 + i)
        ctxs = [int(x) for x in rng.integers(lo, hi, size=S)]
        w = custom("bf16", 32, 8, 128, ctxs, [q_len] * S, seed=777 + i)
        announce(f"workspace reuse call {i}: S={S} q_len={q_len} maxctx={max(ctxs)}")
        st = stage(w)
        need = pk.paged_attention_workspace_size(len(ctxs), w.total_rows, 32, 128, st.max_context_len)
        if ws is None or ws.numel() < need:
            ws = torch.full((max(need, 1 << 24),), 0x7F, dtype=torch.uint8, device="cuda")
        out = pk.paged_attention_forward(st.q, st.k_pools[0], st.v_pools[0], st.tables, st.context_lens, st.qsl,
                                         st.max_q_len, st.max_context_len, w.scale, out=st.out, workspace=ws)
        torch.cuda.synchronize()
        want = oracle_rows(w, list(range(w.total_rows)))
        err = max_err(out.cpu().numpy(), want)
        print(f"[case] workspace reuse call {i}: max abs err {err:.3e}", flush=True)
        assert err <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [16, 48, 64, 128, 256])
def test_scatter_patterns_bit_exact(pk, dtype, D):
    """kv_append_scatter against the oracle scatter on slot patterns that mix
    whole blocks written in order (the 16-byte-piece path), runs shifted
    inside blocks, reversed runs, skipped slots (-1) and a ragged last group.
    Head sizes from 16 to 256 take one, two or four 16-byte pieces per lane,
    and rows that leave lanes without a piece of their own."""
    import torch
    import oracle
    rng = np.random.default_rng(31 + D + (dtype == "bf16"))
    nb, hkv = 96, 3
    perm = rng.permutation(nb)
    slots = []
    slots += list(range(perm[0] * 16, perm[0] * 16 + 16))            # group 0: whole block, in order
    slots += list(range(perm[2] * 16, perm[2] * 16 + 16))[::-1]       # group 1: whole block, reversed
    slots += list(range(perm[4] * 16, perm[4] * 16 + 16))             # group 2: whole block, in order
    slots += list(range(perm[1] * 16 + 5, perm[1] * 16 + 16))         # shifted run
    slots += [-1] * 3 + list(range(perm[3] * 16, perm[3] * 16 + 13))  # skipped slots
    slots += list(range(perm[5] * 16, perm[5] * 16 + 7))              # ragged end
    slots = np.array(slots, dtype=np.int32)
    n = slots.size
    announce(f"scatter patterns dtype={dtype} D={D} n={n}")
    if dtype == "bf16":
        kn = synth.f32_to_bf16_bits(rng.standard_normal((n, hkv, D), dtype=np.float32))
        vn = synth.f32_to_bf16_bits(rng.standard_normal((n, hkv, D), dtype=np.float32))
        tk = torch.from_numpy(kn.view(np.int16)).cuda().view(torch.bfloat16)
        tv = torch.from_numpy(vn.view(np.int16)).cuda().view(torch.bfloat16)
        nan = np.uint16(0x7FC0)
    else:
        kn = rng.standard_normal((n, hkv, D), dtype=np.float32)
        vn = rng.standard_normal((n, hkv, D), dtype=np.float32)
        tk, tv = torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda()
        nan = np.float32(np.nan)
    kp, vp = pk.empty_pools(nb, hkv, D, tk.dtype, "cuda")
    kp.fill_(float("nan"))
    vp.fill_(float("nan"))
    pk.kv_append_scatter(tk, tv, torch.from_numpy(slots).cuda(), kp, vp)
    torch.cuda.synchronize()
    ko, vo = oracle.empty_pools(nb, hkv, D, 16, dtype, fill=nan)
    oracle.scatter(ko, vo, kn, vn, slots)
    np.testing.assert_array_equal(_bits(kp), ko.view(np.uint16 if dtype == "bf16" else np.uint32))
    np.testing.assert_array_equal(_bits(vp), vo.view(np.uint16 if dtype == "bf16" else np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp4"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("q_lens", [[1, 1, 1, 1, 1], [1, 8, 1, 3, 1]])
def test_wide_query_groups(pk, dtype, D, q_lens):
    """64 query heads sharing one KV head: even a decode row brings 64 rows to
    its KV head, more than one split workgroup takes."""
    w = custom(dtype, 64, 1, D, [3000, 700, 1025, 64, 2049], q_lens, seed=300 + D + sum(q_lens), sinks=True)
    check_workload(pk, w)

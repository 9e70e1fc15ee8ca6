"""Tree verify windows, sliding windows, block copies, the accept walk and
rollback on the GPU, through the C ABI, against the oracle.

Tree windows and the accept walk follow the TensorFold page, section on the
GPU accept kernel (drafts as a chain or a tree of at most 16 rows; the
accepted path follows the first child whose draft equals the target's
choice; a rollback restores the KV cache after the path). Sliding windows
follow the TensorSharp "高级功能" page (SWA-1024 drafters in "MTP / NextN
推测解码"; sliding-window layers in "性能优化"). Tolerances are those of the unmasked parity tests (2e-3 bf16 and
8-bit pools, 1e-5 fp32); block copies, masks and accept paths are exact;
row invariance is bitwise.
"""
import sys

import numpy as np
import pytest

import oracle
from gpu_util import TOL, _dense, custom, max_err, oracle_side

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


def random_parents(rng, n):
    return ([-1] + [int(rng.integers(-1, r)) for r in range(1, n)]) if n else []


def masks_for(w, rng, chain=False):
    """One random tree (or a chain) per sequence's window; masks [rows]."""
    out = []
    for seq in w.seqs:
        parents = list(range(-1, seq.q_len - 1)) if chain else random_parents(rng, seq.q_len)
        out.append(oracle.tree_masks(parents))
    return np.concatenate(out).astype(np.uint32)


def dev_mask(m):
    import torch
    return torch.from_numpy(np.ascontiguousarray(m).view(np.int32)).cuda()


def masked(pk, st, w, tree_mask=None, window=0, tables=None):
    return pk.paged_attention_masked_forward(
        st.q, st.k_pools[0], st.v_pools[0], st.tables if tables is None else tables, st.context_lens, st.qsl,
        st.max_q_len, st.max_context_len, w.scale, sinks=st.sinks,
        tree_mask=None if tree_mask is None else dev_mask(tree_mask), sliding_window=window)


def check(pk, w, tree_mask=None, window=0, drop=None):
    import torch
    from paged_kv_attention_block_amd.staging import stage
    announce(f"masked {w.name} dtype={w.dtype} Hq={w.num_q_heads} Hkv={w.num_kv_heads} D={w.head_dim} "
             f"ctx={[s.ctx for s in w.seqs][:6]} q_len={[s.q_len for s in w.seqs][:6]} "
             f"tree={tree_mask is not None} window={window} drop={drop}")
    st = stage(w)
    tables = st.tables
    if drop:
        for s, first in drop.items():
            pk.kv_pool_drop_prefix(st.pool, s, first)
        rows = [pk.kv_pool_alloc(st.pool, s, [], st.max_blocks)[0] for s in range(len(w.seqs))]
        tables = torch.from_numpy(np.stack(rows).astype(np.int32)).cuda()
        # poison the freed blocks: any read of them would show as NaN
        freed = sorted(set(int(b) for b in st.tables_np.reshape(-1) if b >= 0) -
                       set(int(b) for r in rows for b in r if b >= 0))
        if freed:
            idx = torch.tensor(freed, dtype=torch.long, device="cuda")
            fill = 0xFF if w.dtype in ("fp8", "fp4") else float("nan")
            st.k_pools[0][idx] = fill
            st.v_pools[0][idx] = fill
    out = masked(pk, st, w, tree_mask, window, tables)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    tables_o, _, _, want = oracle_side(w, tree_mask=tree_mask, window=window, drop=drop)
    if not drop:
        np.testing.assert_array_equal(st.tables_np, tables_o)
    err = max_err(got, want)
    print(f"[case] {w.name}: max abs err {err:.3e} (tol {TOL[w.dtype]})", flush=True)
    assert np.all(np.isfinite(got))
    assert err <= TOL[w.dtype]
    return st, out


@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp8", "fp4"])
@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (16, 2, 64), (8, 8, 64)])
def test_tree_windows(pk, dtype, Hq, Hkv, D):
    """Tree windows of up to 16 rows (both tile counts), next to decode rows,
    on contexts crossing split edges; sinks on."""
    rng = np.random.default_rng(Hq * 10 + D + len(dtype))
    ctxs = [40, 300, 1030, 2061, 3000, 17, 4500]
    q_lens = [16, 5, 16, 9, 1, 16, 12]
    w = custom(dtype, Hq, Hkv, D, ctxs, q_lens, seed=int(rng.integers(1 << 30)), sinks=True)
    check(pk, w, tree_mask=masks_for(w, rng))


def test_chain_mask_equals_causal_bitwise(pk):
    import torch
    from paged_kv_attention_block_amd.staging import stage
    rng = np.random.default_rng(5)
    w = custom("bf16", 32, 8, 128, [3000, 700, 40], [16, 8, 16], seed=55, sinks=True)
    st = stage(w)
    a = masked(pk, st, w, tree_mask=masks_for(w, rng, chain=True)).clone()
    b = pk.paged_attention_forward(st.q, st.k_pools[0], st.v_pools[0], st.tables, st.context_lens, st.qsl,
                                   st.max_q_len, st.max_context_len, w.scale, sinks=st.sinks)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(a), bits(b))


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp4"])
def test_tree_row_equals_window_cut_after_it(pk, dtype):
    """Row r of a tree window gives the same bits as the last row of the same
    window cut after row r (context base + r + 1, masks of rows 0 .. r)."""
    import torch
    from paged_kv_attention_block_amd.staging import stage
    rng = np.random.default_rng(6)
    w = custom(dtype, 32, 8, 128, [2600], [16], seed=66, sinks=True)
    m = masks_for(w, rng)
    st = stage(w)
    full = bits(masked(pk, st, w, tree_mask=m))
    base = w.seqs[0].ctx - 16
    for r in [0, 3, 9, 15]:
        out = pk.paged_attention_masked_forward(
            st.q[:r + 1].contiguous(), st.k_pools[0], st.v_pools[0], st.tables,
            torch.tensor([base + r + 1], dtype=torch.int32, device="cuda"),
            torch.tensor([0, r + 1], dtype=torch.int32, device="cuda"), r + 1, base + r + 1, w.scale,
            sinks=st.sinks, tree_mask=dev_mask(m[:r + 1]))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(out)[r], full[r])


@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp8", "fp4"])
@pytest.mark.parametrize("window", [1, 100, 128, 1000, 4096])
def test_sliding_window_decode(pk, dtype, window):
    w = custom(dtype, 64, 8, 64, [1024, 5000, 8192, 3000, 130, 2049], [1] * 6, seed=700 + window, sinks=True)
    check(pk, w, window=window)


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp4"])
@pytest.mark.parametrize("window", [7, 128, 700])
def test_sliding_window_verify_and_prefill(pk, dtype, window):
    """Verify windows (8 rows), a long prefill chunk (the sequential shape)
    and decode rows under one sliding window."""
    w = custom(dtype, 16, 4, 128, [5000, 2300, 900, 3100], [8, 600, 1, 40], seed=800 + window, sinks=True)
    check(pk, w, window=window)


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp4"])
def test_sliding_window_with_freed_blocks(pk, dtype):
    """Blocks below every row's window freed on the host (table entries -1)
    and poisoned in the pool: nothing changes."""
    W = 256
    ctxs, q_lens = [4000, 2500, 600, 9000], [1, 8, 1, 300]
    w = custom(dtype, 32, 8, 128, ctxs, q_lens, seed=901, sinks=True)
    drop = {s: c - q - W + 1 for s, (c, q) in enumerate(zip(ctxs, q_lens)) if c - q - W + 1 > 16}
    check(pk, w, window=W, drop=drop)


def test_tree_and_window_together(pk):
    rng = np.random.default_rng(9)
    w = custom("bf16", 32, 8, 128, [3000, 40, 1500], [16, 16, 7], seed=909, sinks=True)
    check(pk, w, tree_mask=masks_for(w, rng), window=10)


def test_window_rows_invariant(pk):
    """A sliding-window row alone (a decode row at its position) and inside
    a verify window or a batch: the same bits."""
    import torch
    from paged_kv_attention_block_amd.staging import stage
    w = custom("bf16", 32, 8, 128, [4100, 2000], [8, 1], seed=910, sinks=True)
    st = stage(w)
    W = 300
    full = bits(masked(pk, st, w, window=W))
    for i in [0, 5, 7, 8]:
        s = 0 if i < 8 else 1
        seq = w.seqs[s]
        p = seq.ctx - seq.q_len + (i - int(w.qsl[s]))
        out = pk.paged_attention_masked_forward(
            st.q[i:i + 1].contiguous(), st.k_pools[0], st.v_pools[0], st.tables[s:s + 1].contiguous(),
            torch.tensor([p + 1], dtype=torch.int32, device="cuda"), torch.tensor([0, 1], dtype=torch.int32,
                                                                                  device="cuda"),
            1, p + 1, w.scale, sinks=st.sinks, sliding_window=W)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(out)[0], full[i])


def test_masked_rejects_bad_arguments(pk):
    import torch
    from paged_kv_attention_block_amd.staging import stage
    w = custom("bf16", 8, 2, 64, [100], [40], seed=911)
    st = stage(w)
    with pytest.raises(pk.KVError) as e:
        masked(pk, st, w, tree_mask=np.zeros(40, np.uint32))
    assert e.value.code == pk.KV_EINVAL and "32" in e.value.message
    with pytest.raises(pk.KVError) as e:
        masked(pk, st, w, window=-1)
    assert e.value.code == pk.KV_EINVAL


# ---------------------------------------------------------------------------
# block copies, accept walk, rollback
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp8", "fp4"])
def test_copy_blocks_bit_exact(pk, dtype):
    import torch
    rng = np.random.default_rng(12)
    nb, hkv, D = 40, 3, 128 if dtype != "f32" else 64
    announce(f"copy blocks {dtype}")
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": "fp8", "fp4": "fp4"}[dtype]
    kp, vp = pk.empty_pools(nb, hkv, D, tdt, "cuda")
    if dtype in ("fp8", "fp4"):
        kp.copy_(torch.randint(0, 256, kp.shape, dtype=torch.uint8))
        vp.copy_(torch.randint(0, 256, vp.shape, dtype=torch.uint8))
    else:
        kp.copy_(torch.randn(kp.shape).to(tdt))
        vp.copy_(torch.randn(vp.shape).to(tdt))
    perm = rng.permutation(nb)
    src, dst = perm[:10].astype(np.int32), perm[10:20].astype(np.int32)
    src_x = np.concatenate([src, [-1, 5]]).astype(np.int32)       # out-of-range pairs copy nothing
    dst_x = np.concatenate([dst, [7, nb]]).astype(np.int32)
    raw = lambda t: t.view(torch.uint8).cpu().numpy()          # bytes of each block, any element type
    ko, vo = raw(kp).copy(), raw(vp).copy()
    pk.kv_copy_blocks(kp, vp, torch.from_numpy(src_x).cuda(), torch.from_numpy(dst_x).cuda())
    torch.cuda.synchronize()
    oracle.copy_blocks(ko, vo, src, dst)
    np.testing.assert_array_equal(raw(kp), ko)
    np.testing.assert_array_equal(raw(vp), vo)


def test_accept_paths_match_oracle(pk):
    import torch
    rng = np.random.default_rng(13)
    S = 150
    q_lens = [int(rng.integers(0, 17)) for _ in range(S)]
    q_lens[:3] = [16, 1, 0]
    parents, drafts, choices, roots = [], [], [], []
    want = []
    for s, n in enumerate(q_lens):
        par = list(range(-1, n - 1)) if s % 3 == 0 else random_parents(rng, n)
        dr = [int(x) for x in rng.integers(0, 3, n)]
        ch = [int(x) for x in rng.integers(0, 3, n)]
        root = int(rng.integers(0, 3))
        parents += par
        drafts += dr
        choices += ch
        roots.append(root)
        want.append(oracle.accept_path(par, dr, ch, root))
    qsl = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.int32), device="cuda")
    announce(f"accept paths S={S} rows={qsl[-1]}")
    path, plen, bonus = pk.kv_accept_paths(t(parents), t(drafts), t(choices), t(roots), t(qsl))
    torch.cuda.synchronize()
    path, plen, bonus = path.cpu().numpy(), plen.cpu().numpy(), bonus.cpu().numpy()
    lens = []
    for s, (p_want, b_want) in enumerate(want):
        seg = path[qsl[s]:qsl[s + 1]]
        assert list(seg[:len(p_want)]) == p_want and (seg[len(p_want):] == -1).all()
        assert plen[s] == len(p_want) and bonus[s] == b_want
        lens.append(len(p_want))
    assert max(lens) >= 3


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp4"])
def test_rollback_round(pk, dtype):
    """One speculative round end to end on two sequences with a 12-row draft
    tree each. Sequence 1 allocates the prompt and its first 8 drafts (the
    same as sequence 0's) at once, so it shares sequence 0's first three
    blocks. The accept walk runs on the device; rollback truncates each
    sequence to the window base (the shared block the base ends in is copied
    for the first sequence that truncates), then appends the accepted tokens
    and scatters their rows. The next decode step's attention equals the
    oracle over the accepted sequences."""
    import torch
    import synth
    rng = np.random.default_rng(14 + len(dtype))
    B, Hq, Hkv, D, nb = 16, 32, 8, 128, 64
    tdt = dtype if dtype in ("fp8", "fp4") else torch.bfloat16
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.int32), device="cuda")

    def rows(*shape):
        return synth.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    def put(k, v, slots):
        pk.kv_append_scatter(dev(k), dev(v), torch.from_numpy(np.asarray(slots, np.int32)).cuda(), kp, vp)

    pool = pk.kv_pool_create(nb, B, rng.permutation(nb))
    kp, vp = pk.empty_pools(nb, Hkv, D, tdt, "cuda")
    kp.fill_(0xFF if dtype in ("fp8", "fp4") else float("nan"))
    vp.fill_(0xFF if dtype in ("fp8", "fp4") else float("nan"))
    prompt = [int(x) for x in rng.integers(0, 50, 40)]          # 2 full blocks + 8 tokens
    kr, vr = rows(40, Hkv, D), rows(40, Hkv, D)
    parents = [-1, 0, 0, 1, 2, 3, -1, 6, 4, 8, 9, 10]
    # root's children: rows 0 (2), 6 (3); row 0's: 1 (0), 2 (1); row 2's: 4;
    # row 4's: 8; row 8's: 9 (2)
    d0 = [2, 0, 1, 3, 2, 0, 3, 1, 3, 2, 0, 1]
    d1 = d0[:8] + [int(x) for x in rng.integers(0, 4, 4)]
    drafts = {0: d0, 1: d1}
    kw0, vw0 = rows(12, Hkv, D), rows(12, Hkv, D)
    kw = {0: kw0, 1: np.concatenate([kw0[:8], rows(4, Hkv, D)])}
    vw = {0: vw0, 1: np.concatenate([vw0[:8], rows(4, Hkv, D)])}
    _, _, _, sl = pk.kv_pool_alloc(pool, 0, prompt, 8)
    put(kr, vr, sl)
    _, _, _, sl = pk.kv_pool_alloc(pool, 0, d0, 8)
    put(kw[0], vw[0], sl)
    row1, _, _, sl = pk.kv_pool_alloc(pool, 1, prompt + d1[:8], 8)
    assert (sl == -1).all()                                      # three shared blocks
    _, _, _, sl = pk.kv_pool_alloc(pool, 1, d1[8:], 8)
    put(kw[1][8:], vw[1][8:], sl)
    # target choices: sequence 0 follows rows 0, 2, 4, 8; sequence 1 at random
    c0 = [0] * 12
    c0[0], c0[2], c0[4], c0[8] = d0[2], d0[4], d0[8], 3
    choices = {0: c0, 1: [int(x) for x in rng.integers(0, 4, 12)]}
    roots = [2, d1[0]]
    path, plen, _ = pk.kv_accept_paths(t(parents * 2), t(d0 + d1), t(choices[0] + choices[1]), t(roots),
                                       t([0, 12, 24]))
    torch.cuda.synchronize()
    path, plen = path.cpu().numpy(), plen.cpu().numpy()
    acc = {}
    for s in (0, 1):
        acc[s] = [int(x) for x in path[12 * s:12 * s + plen[s]]]
        assert acc[s] == oracle.accept_path(parents, drafts[s], choices[s], roots[s])[0]
    assert acc[0] == [0, 2, 4, 8]
    copies = []
    for s in (0, 1):
        src, dst = pk.kv_pool_truncate(pool, s, 40)
        if src >= 0:
            copies.append((src, dst))
            pk.kv_copy_blocks(kp, vp, t([src]), t([dst]))
        if acc[s]:
            _, _, _, sl = pk.kv_pool_alloc(pool, s, [drafts[s][r] for r in acc[s]], 8)
            put(kw[s][acc[s]], vw[s][acc[s]], sl)
    assert len(copies) == 1 and copies[0][0] == row1[2]
    # next decode step
    q = rows(2, Hq, D)
    kn, vn = rows(2, Hkv, D), rows(2, Hkv, D)
    tables, ctxs = [], []
    for s in (0, 1):
        row, _, ctx, sl = pk.kv_pool_alloc(pool, s, [7], 8)
        put(kn[s:s + 1], vn[s:s + 1], sl)
        tables.append(row)
        ctxs.append(ctx)
    announce(f"rollback round {dtype}: accepted {acc}, copies {copies}, ctx {ctxs}")
    out = pk.paged_attention_forward(dev(q), kp, vp, t(np.stack(tables)), t(ctxs), t([0, 1, 2]), 1, max(ctxs),
                                     1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    ks = [np.concatenate([kr, kw[s][acc[s]], kn[s:s + 1]]) for s in (0, 1)]
    vs = [np.concatenate([vr, vw[s][acc[s]], vn[s:s + 1]]) for s in (0, 1)]
    if dtype in ("fp8", "fp4"):
        ks = [_dense(k, dtype) for k in ks]
        vs = [_dense(v, dtype) for v in vs]
    want = oracle.attention(q, ks, vs, np.array([0, 1, 2], np.int32), Hq, Hkv, 1.0 / np.sqrt(D), None, dtype)
    err = max_err(out.cpu().numpy(), want)
    print(f"[case] rollback round {dtype}: max abs err {err:.3e}", flush=True)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("fp4", 128)])
def test_window_prefill_rows_invariant(pk, dtype, D):
    """Prefill chunks under a sliding window take the sequential shape, whose
    walk starts at the step of the lowest key any row of the workgroup sees;
    with window 600 that start falls inside a 256-key quarter past key 1024.
    Each sampled row equals itself computed alone (a decode row at its
    position)."""
    import torch
    from paged_kv_attention_block_amd.staging import stage
    w = custom(dtype, 16, 4, D, [3000, 1800, 900], [200, 40, 64], seed=911 + D, sinks=True)
    st = stage(w)
    W = 600
    print(f"\n[case] window prefill invariance {dtype} D={D} window={W}", flush=True)
    full = bits(masked(pk, st, w, window=W))
    qsl = [int(x) for x in w.qsl]
    rows = []
    for s in range(len(w.seqs)):
        rows += [qsl[s], qsl[s] + 15, qsl[s] + 16, qsl[s + 1] - 17, qsl[s + 1] - 1]
    for i in rows:
        s = max(k for k in range(len(w.seqs)) if qsl[k] <= i)
        seq = w.seqs[s]
        p = seq.ctx - seq.q_len + (i - qsl[s])
        out = pk.paged_attention_masked_forward(
            st.q[i:i + 1].contiguous(), st.k_pools[0], st.v_pools[0], st.tables[s:s + 1].contiguous(),
            torch.tensor([p + 1], dtype=torch.int32, device="cuda"), torch.tensor([0, 1], dtype=torch.int32,
                                                                                  device="cuda"),
            1, p + 1, w.scale, sinks=st.sinks, sliding_window=W)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(out)[0], full[i], err_msg=f"row {i}")

"""Pins of the oracle's tree windows, sliding windows, truncate and accept
walk (CPU only).

Tree windows and the accept walk follow the TensorFold page, section on the
GPU accept kernel (drafts laid out as a chain or a tree of at most 16 rows;
the accepted path follows the first child whose token equals the target's
choice; a rollback restores the KV cache after the accepted path). Sliding
windows follow the TensorSharp "高级功能" page (SWA-1024 drafters in
"MTP / NextN 推测解码"; sliding-window layers in "性能优化").

The masked attention is checked against a dense brute force whose mask matrix
is built by walking parent pointers (not from the mask words the oracle
reads), against closed forms (a one-key window returns that key's value), and
against the causal oracle on compacted sequences (a tree row sees exactly its
ancestors, so it equals a causal row over resident keys + ancestors + itself).
"""
import copy

import numpy as np
import pytest
from scipy.special import softmax

import oracle


def _ancestors(parents, r):
    out = {r}
    p = int(parents[r])
    while p >= 0:
        out.add(p)
        p = int(parents[p])
    return out


def brute_masked(q, ks, vs, q_lens, parents_list, window, Hq, Hkv, scale, sinks=None):
    """Dense attention with an explicit [q_len, ctx] visibility matrix: key t
    is visible to row r when t <= p, t > p - window (window > 0), and, inside
    the window of a tree, t - base is r or one of r's ancestors (walked from
    the parent pointers)."""
    outs, row = [], 0
    for k, v, ql, parents in zip(ks, vs, q_lens, parents_list):
        ctx = k.shape[0]
        base = ctx - ql
        vis = np.zeros((ql, ctx), dtype=bool)
        for r in range(ql):
            p = base + r
            anc = None if parents is None else _ancestors(parents, r)
            for t in range(ctx):
                ok = t <= p and (window == 0 or t > p - window)
                if ok and anc is not None and t >= base:
                    ok = (t - base) in anc
                vis[r, t] = ok
        kr = np.repeat(k.astype(np.float64), Hq // Hkv, axis=1)
        vr = np.repeat(v.astype(np.float64), Hq // Hkv, axis=1)
        qs = q[row:row + ql].astype(np.float64)
        scores = np.einsum("rhd,thd->hrt", qs, kr) * scale
        scores = np.where(vis[None], scores, -np.inf)
        if sinks is not None:
            col = np.broadcast_to(np.asarray(sinks, np.float64)[:, None, None], (Hq, ql, 1))
            scores = np.concatenate([scores, col], axis=2)
            vr = np.concatenate([vr, np.zeros((1,) + vr.shape[1:])], axis=0)
        w = softmax(scores, axis=2)
        outs.append(np.einsum("hrt,thd->rhd", w, vr))
        row += ql
    return np.concatenate(outs, axis=0)


def random_parents(rng, n):
    return [-1] + [int(rng.integers(-1, r)) for r in range(1, n)]


def case(rng, ctxs, q_lens, Hq=4, Hkv=2, D=8, sinks=False):
    q = rng.standard_normal((sum(q_lens), Hq, D)).astype(np.float32)
    ks = [rng.standard_normal((c, Hkv, D)).astype(np.float32) for c in ctxs]
    vs = [rng.standard_normal((c, Hkv, D)).astype(np.float32) for c in ctxs]
    sk = rng.standard_normal(Hq).astype(np.float32) * 2 if sinks else None
    qsl = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    return q, ks, vs, qsl, sk


@pytest.mark.parametrize("sinks", [False, True])
@pytest.mark.parametrize("window", [0, 1, 3, 17])
def test_tree_and_window_against_brute_force(sinks, window):
    rng = np.random.default_rng(11 + window + 100 * sinks)
    ctxs, q_lens = [9, 30, 16, 40], [3, 16, 1, 12]
    q, ks, vs, qsl, sk = case(rng, ctxs, q_lens, sinks=sinks)
    parents_list = [random_parents(rng, n) for n in q_lens]
    masks = np.concatenate([oracle.tree_masks(p) for p in parents_list])
    got = oracle.attention(q, ks, vs, qsl, 4, 2, 0.4, sk, "f32", tree_mask=masks, window=window)
    want = brute_masked(q, ks, vs, q_lens, parents_list, window, 4, 2, 0.4, sk)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [1, 5, 64])
def test_window_without_tree_against_brute_force(window):
    rng = np.random.default_rng(21 + window)
    ctxs, q_lens = [70, 33, 5], [1, 20, 5]
    q, ks, vs, qsl, sk = case(rng, ctxs, q_lens, sinks=True)
    got = oracle.attention(q, ks, vs, qsl, 4, 2, 0.3, sk, "f32", window=window)
    want = brute_masked(q, ks, vs, q_lens, [None] * 3, window, 4, 2, 0.3, sk)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_chain_mask_is_causal_exactly():
    rng = np.random.default_rng(31)
    ctxs, q_lens = [40, 17], [16, 8]
    q, ks, vs, qsl, sk = case(rng, ctxs, q_lens, sinks=True)
    chain = np.concatenate([oracle.tree_masks(list(range(-1, n - 1))) for n in q_lens])
    assert chain[3] == 0b1111
    a = oracle.attention(q, ks, vs, qsl, 4, 2, 0.5, sk, "f32")
    b = oracle.attention(q, ks, vs, qsl, 4, 2, 0.5, sk, "f32", tree_mask=chain)
    np.testing.assert_array_equal(a, b)


def test_window_covering_the_context_changes_nothing():
    rng = np.random.default_rng(32)
    ctxs, q_lens = [40, 17], [6, 17]
    q, ks, vs, qsl, sk = case(rng, ctxs, q_lens)
    a = oracle.attention(q, ks, vs, qsl, 4, 2, 0.5, None, "f32")
    b = oracle.attention(q, ks, vs, qsl, 4, 2, 0.5, None, "f32", window=40)
    np.testing.assert_array_equal(a, b)


def test_one_key_window_closed_form():
    """W = 1: the row sees only its own key: out = v_p, or with a sink
    v_p / (1 + exp(sigma - x_p)), x_p = scale * <q, k_p>."""
    rng = np.random.default_rng(33)
    ctxs, q_lens = [12, 7], [4, 1]
    q, ks, vs, qsl, sk = case(rng, ctxs, q_lens, Hq=2, Hkv=2, D=4, sinks=True)
    plain = oracle.attention(q, ks, vs, qsl, 2, 2, 0.7, None, "f32", window=1)
    sunk = oracle.attention(q, ks, vs, qsl, 2, 2, 0.7, sk, "f32", window=1)
    row = 0
    for k, v, ql in zip(ks, vs, q_lens):
        for r in range(ql):
            p = k.shape[0] - ql + r
            for h in range(2):
                vp = v[p, h].astype(np.float64)
                assert np.array_equal(plain[row + r, h], vp)
                x = 0.7 * float(np.dot(q[row + r, h].astype(np.float64), k[p, h].astype(np.float64)))
                np.testing.assert_allclose(sunk[row + r, h], vp / (1.0 + np.exp(float(sk[h]) - x)),
                                           rtol=1e-14, atol=1e-15)
        row += ql


def test_tree_row_equals_causal_row_over_its_ancestors():
    """A tree row attends to resident keys + its ancestors + itself: the same
    as the causal last row of a sequence made of exactly those keys."""
    rng = np.random.default_rng(34)
    base, W = 23, 12
    parents = [-1, 0, 0, 1, 1, 2, -1, 6, 3, 8, 4, 9]
    q, ks, vs, qsl, sk = case(rng, [base + W], [W], sinks=True)
    got = oracle.attention(q, ks, vs, qsl, 4, 2, 0.5, sk, "f32", tree_mask=oracle.tree_masks(parents))
    for r in range(W):
        keep = list(range(base)) + sorted(base + j for j in _ancestors(parents, r))
        kc, vc = ks[0][keep], vs[0][keep]
        want = oracle.attention(q[r:r + 1], [kc], [vc], np.array([0, 1], np.int32), 4, 2, 0.5, sk, "f32")
        np.testing.assert_allclose(got[r], want[0], rtol=0, atol=1e-15)


def test_mask_bits_outside_the_ancestry_rule():
    """Bits at or above the row's own index are ignored; the own key is
    visible even with an all-zero mask."""
    rng = np.random.default_rng(35)
    q, ks, vs, qsl, _ = case(rng, [20], [5])
    zeros = np.zeros(5, np.uint32)
    high = np.array([0xFFFFFFFE, 0xFFFFFFFC, 0xFFFFFFF8, 0xFFFFFFF0, 0xFFFFFFE0], np.uint32)
    a = oracle.attention(q, ks, vs, qsl, 4, 2, 0.5, None, "f32", tree_mask=zeros)
    b = oracle.attention(q, ks, vs, qsl, 4, 2, 0.5, None, "f32", tree_mask=high)
    np.testing.assert_array_equal(a, b)
    want = brute_masked(q, ks, vs, [5], [[-1] * 5], 0, 4, 2, 0.5)
    np.testing.assert_allclose(a, want, rtol=0, atol=1e-12)


def test_masked_oracle_rejects_long_windows():
    rng = np.random.default_rng(36)
    q, ks, vs, qsl, _ = case(rng, [40], [33])
    with pytest.raises(ValueError):
        oracle.attention(q, ks, vs, qsl, 4, 2, 0.5, None, "f32", tree_mask=np.zeros(33, np.uint32))


# ---------------------------------------------------------------------------
# accept walk
# ---------------------------------------------------------------------------

def test_accept_walk_by_hand():
    #        root
    #       /    \
    #     0(5)   4(5)
    #     /  \
    #   1(6) 2(7)
    #    |
    #   3(8)
    parents = [-1, 0, 0, 1, -1]
    drafts = [5, 6, 7, 8, 5]
    assert oracle.accept_path(parents, drafts, [6, 1, 9, 2, 0], 5) == ([0, 1], 1)
    assert oracle.accept_path(parents, drafts, [7, 8, 9, 4, 0], 5) == ([0, 2], 9)
    assert oracle.accept_path(parents, drafts, [6, 8, 9, 4, 0], 5) == ([0, 1, 3], 4)
    assert oracle.accept_path(parents, drafts, [6, 8, 9, 4, 0], 3) == ([], 3)


def test_accept_walk_on_a_chain_is_the_longest_matching_prefix():
    rng = np.random.default_rng(37)
    for _ in range(50):
        n = int(rng.integers(1, 17))
        drafts = rng.integers(0, 4, n)
        target = rng.integers(0, 4, n + 1)   # target[i]: the target's token at draft position i
        k = 0
        while k < n and drafts[k] == target[k]:
            k += 1
        path, bonus = oracle.accept_path(list(range(-1, n - 1)), drafts, target[1:], target[0])
        assert path == list(range(k)) and bonus == target[k]


# ---------------------------------------------------------------------------
# truncate (KV rollback on the host side)
# ---------------------------------------------------------------------------

def invariants(a):
    refs = [0] * a.n
    for st in a.seqs.values():
        assert len(st["blocks"]) == -(-len(st["tokens"]) // a.B)
        assert len(st["hashes"]) == len(st["tokens"]) // a.B
        for b in st["blocks"]:
            if b >= 0:                         # -1: freed by drop_prefix, no reference held
                refs[b] += 1
    assert refs == a.ref
    free = list(a.free)
    assert len(set(free)) == len(free)
    assert sorted(free) == [b for b in range(a.n) if refs[b] == 0]
    assert all(a.in_free[b] == (b in free) for b in range(a.n))
    for h, (b, _, _, _) in a.table.items():
        assert a.blk_hash[b] == h


def test_truncate_at_a_boundary_then_regrow_reuses_the_blocks():
    a = oracle.Allocator(16, 4, list(range(16))[::-1])
    toks = list(range(1, 15))                  # 3 full blocks + 2
    row0, _, _, _ = a.alloc(1, toks, 8)
    assert a.truncate(1, 4) == (-1, -1)
    invariants(a)
    assert a.table_row(1, 8)[:2] == [row0[0], -1]
    row1, nb, ctx, slots = a.alloc(1, toks[4:], 8)
    invariants(a)
    assert ctx == 14 and nb == 4
    assert row1[:3] == row0[:3]                # full blocks found again through their hashes
    assert slots[:8] == [-1] * 8               # already resident


def test_truncate_inside_own_full_block_unhashes_it():
    a = oracle.Allocator(16, 4)
    toks = list(range(1, 13))                  # 3 full blocks
    row0, _, _, _ = a.alloc(1, toks, 8)
    assert a.truncate(1, 6) == (-1, -1)        # block 1 keeps slots 0, 1
    invariants(a)
    assert a.table_row(1, 8)[:2] == row0[:2]
    assert a.blk_hash[row0[1]] is None
    # a new sequence with the old prefix shares block 0 only
    row2, _, _, slots = a.alloc(2, toks, 8)
    invariants(a)
    assert row2[0] == row0[0] and row2[1] != row0[1]
    assert slots[:4] == [-1] * 4 and -1 not in slots[4:]


def test_truncate_inside_a_shared_block_copies_it():
    a = oracle.Allocator(16, 4)
    toks = list(range(1, 13))
    row_a, _, _, _ = a.alloc(1, toks, 8)
    row_b, _, _, _ = a.alloc(2, toks, 8)
    assert row_a[:3] == row_b[:3]
    src, dst = a.truncate(2, 5)
    invariants(a)
    assert src == row_a[1] and dst not in row_a[:3]
    assert a.table_row(2, 8)[:2] == [row_a[0], dst]
    assert a.table_row(1, 8)[:3] == row_a[:3]  # the other sequence keeps its blocks
    assert a.ref[row_a[1]] == 1 and a.ref[dst] == 1
    assert a.blk_hash[row_a[1]] is not None    # still hashed: sequence 1 holds it full


def test_truncate_out_of_blocks_leaves_state_unchanged():
    a = oracle.Allocator(3, 4)
    toks = list(range(1, 13))
    a.alloc(1, toks, 8)
    a.alloc(2, toks, 8)
    assert len(a.free) == 0
    before = copy.deepcopy(a.__dict__)
    with pytest.raises(oracle.OutOfBlocks):
        a.truncate(2, 5)
    assert a.__dict__ == before


def test_truncate_edges():
    a = oracle.Allocator(8, 4)
    a.alloc(1, list(range(10)), 4)
    assert a.truncate(1, 10) == (-1, -1)
    assert a.table_row(1, 4)[:3] != [-1] * 3
    with pytest.raises(ValueError):
        a.truncate(1, 11)
    with pytest.raises(KeyError):
        a.truncate(9, 0)
    assert a.truncate(1, 0) == (-1, -1)
    invariants(a)
    assert a.table_row(1, 4) == [-1] * 4 and len(a.free) == 8


def test_rollback_after_a_tree_round_matches_serial_appends():
    """Window rows scattered at window positions; accept a tree path; roll
    back by truncating to the window base, allocating the accepted tokens and
    scattering their rows. The gathered cache then equals a cache built by
    appending the accepted tokens one by one."""
    rng = np.random.default_rng(38)
    B, Hkv, D = 16, 2, 16
    base = 37
    parents = [-1, 0, 0, 1, 2, 3, -1, 6]
    drafts = [3, 4, 5, 6, 7, 8, 3, 1]
    path, _ = oracle.accept_path(parents, drafts, [5, 0, 7, 0, 2, 0, 0, 0], 3)
    assert path == [0, 2, 4]
    ctx_tokens = list(rng.integers(0, 50, base))
    kr = oracle.to_f32(rng.standard_normal((base, Hkv, D)).astype(np.float32), "f32")
    vr = rng.standard_normal((base, Hkv, D)).astype(np.float32)
    kw = rng.standard_normal((len(parents), Hkv, D)).astype(np.float32)
    vw = rng.standard_normal((len(parents), Hkv, D)).astype(np.float32)

    a = oracle.Allocator(32, B, rng.permutation(32))
    kp, vp = oracle.empty_pools(32, Hkv, D, B, "f32", fill=np.float32(np.nan))
    _, _, _, s0 = a.alloc(1, ctx_tokens, 8)
    oracle.scatter(kp, vp, kr, vr, s0)
    _, _, _, s1 = a.alloc(1, drafts, 8)
    oracle.scatter(kp, vp, kw, vw, s1)
    src, dst = a.truncate(1, base)
    assert (src, dst) == (-1, -1)
    row, _, ctx, s2 = a.alloc(1, [drafts[r] for r in path], 8)
    oracle.scatter(kp, vp, kw[path], vw[path], s2)
    invariants(a)
    k_got, v_got = oracle.gather(kp, vp, row, ctx)
    np.testing.assert_array_equal(k_got, np.concatenate([kr, kw[path]]))
    np.testing.assert_array_equal(v_got, np.concatenate([vr, vw[path]]))


# ----------------------------------------------------------------------------
# Allocator.drop_prefix: freeing the blocks a sliding window has passed
# (TensorSharp "高级功能" page, "性能优化": sliding-window layers; prefix
# reuse bounded by the window). Every expectation below is worked out by hand
# from the rule "block j is freed when (j + 1) * B <= first_kept; freed blocks
# go to the back of the free list, highest j first, and keep their hash".
# ----------------------------------------------------------------------------

def _fresh_seq_of_14(B=4):
    """12 blocks in identity order; sequence 1 holds tokens 1..14 in blocks
    0, 1, 2 (full) and 3 (two slots)."""
    a = oracle.Allocator(12, B)
    row, nb, ctx, _ = a.alloc(1, list(range(1, 15)), 6)
    assert row == [0, 1, 2, 3, -1, -1] and nb == 4 and ctx == 14
    assert list(a.free) == list(range(4, 12))
    return a


@pytest.mark.parametrize("first_kept,freed", [(8, [1, 0]), (7, [0]), (9, [1, 0]), (3, []), (0, []),
                                              (12, [2, 1, 0]), (14, [2, 1, 0]), (100, [2, 1, 0])])
def test_drop_prefix_frees_whole_blocks_below_first_kept(first_kept, freed):
    a = _fresh_seq_of_14()
    a.drop_prefix(1, first_kept)
    invariants(a)
    # freed blocks join the back of the free list, the highest block index j first
    assert list(a.free) == list(range(4, 12)) + freed
    assert a.table_row(1, 6) == [-1 if b in freed else b for b in [0, 1, 2, 3]] + [-1, -1]
    for b in freed:
        assert a.ref[b] == 0 and a.in_free[b]
        assert a.blk_hash[b] is not None          # hash kept: LRU reuse stays possible
    assert a.seqs[1]["dropped"] == bool(freed)
    assert len(a.seqs[1]["tokens"]) == 14         # positions keep their meaning


def test_drop_prefix_of_a_shared_block_only_drops_a_reference():
    a = _fresh_seq_of_14()
    row2, _, _, slots = a.alloc(2, list(range(1, 9)), 6)   # shares blocks 0 and 1
    assert row2[:2] == [0, 1] and slots == [-1] * 8
    assert a.ref[0] == 2 and a.ref[1] == 2
    a.drop_prefix(1, 8)
    invariants(a)
    assert a.ref[0] == 1 and a.ref[1] == 1
    assert list(a.free) == list(range(4, 12))      # nothing went back to the pool
    assert a.table_row(1, 6)[:4] == [-1, -1, 2, 3]
    assert a.table_row(2, 6)[:2] == [0, 1]         # the other sequence keeps them


def test_dropped_blocks_stay_hash_addressable_for_other_sequences():
    a = _fresh_seq_of_14()
    a.drop_prefix(1, 8)
    assert list(a.free)[-2:] == [1, 0]
    row2, _, _, slots = a.alloc(2, list(range(1, 9)), 6)
    invariants(a)
    assert row2[:2] == [0, 1] and slots == [-1] * 8   # revived from the free list
    assert list(a.free) == list(range(4, 12))


def test_a_dropped_sequence_neither_registers_nor_looks_up():
    a = _fresh_seq_of_14()
    a.drop_prefix(1, 8)
    # block 3 fills up after the drop: it must not be registered ...
    _, _, _, s = a.alloc(1, [15, 16], 6)
    assert s == [14, 15]                            # block 3, slots 2 and 3
    assert a.blk_hash[3] is None
    # ... so a new sequence with the same 16 tokens shares blocks 0-2 only
    row3, _, _, slots3 = a.alloc(3, list(range(1, 17)), 6)
    invariants(a)
    assert row3[:3] == [0, 1, 2] and row3[3] not in (3, -1)
    assert slots3[:12] == [-1] * 12 and -1 not in slots3[12:]
    # and a full block that another sequence registered is not looked up by
    # the dropped sequence: it gets a fresh block for the same four tokens
    a.alloc(3, [17, 18, 19, 20], 6)
    ref4 = a.table_row(3, 6)[4]
    assert a.blk_hash[ref4] is not None
    row1, _, _, s1 = a.alloc(1, [17, 18, 19, 20], 6)
    invariants(a)
    assert row1[4] != ref4 and -1 not in s1


def test_drop_prefix_errors():
    a = _fresh_seq_of_14()
    with pytest.raises(KeyError):
        a.drop_prefix(7, 4)
    with pytest.raises(ValueError):
        a.drop_prefix(1, -1)
    a.drop_prefix(1, 8)
    a.drop_prefix(1, 8)                             # a second drop frees nothing more
    invariants(a)
    assert list(a.free) == list(range(4, 12)) + [1, 0]


# ----------------------------------------------------------------------------
# copy_blocks: the device copy a truncate into a shared block asks for
# (TensorFold page, section on the GPU accept kernel: a rollback restores the
# KV cache after the accepted path). Pinned on hand-built pools whose every
# element names its own (block, head, element) position.
# ----------------------------------------------------------------------------

def _labelled_pool(nb, Hkv, tile, offset):
    return (offset + np.arange(nb * Hkv * tile, dtype=np.int64).reshape(nb, Hkv, tile)).astype(np.float32)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "fp4"])
def test_copy_blocks_direction_and_whole_tiles(fmt):
    nb, Hkv, D = 6, 3, 64
    if fmt == "bf16":
        kp, vp = oracle.empty_pools(nb, Hkv, D, 16, "bf16")
        kp[...] = np.arange(kp.size, dtype=np.uint16).reshape(kp.shape)
        vp[...] = (np.arange(vp.size) + 40000).astype(np.uint16).reshape(vp.shape)
    else:
        mk = oracle.fp8_empty_pools if fmt == "fp8" else oracle.fp4_empty_pools
        kp, vp = mk(nb, Hkv, D)
        kp[...] = (np.arange(kp.size) % 251).astype(np.uint8).reshape(kp.shape)
        vp[...] = (np.arange(vp.size) % 241).astype(np.uint8).reshape(vp.shape)
    k0, v0 = kp.copy(), vp.copy()
    oracle.copy_blocks(kp, vp, [4, 0], [1, 5])
    # destination blocks hold the source blocks' full tiles, every head and slot
    np.testing.assert_array_equal(kp[1], k0[4])
    np.testing.assert_array_equal(vp[1], v0[4])
    np.testing.assert_array_equal(kp[5], k0[0])
    np.testing.assert_array_equal(vp[5], v0[0])
    # sources and all other blocks are untouched (direction: src -> dst)
    for b in (0, 2, 3, 4):
        np.testing.assert_array_equal(kp[b], k0[b])
        np.testing.assert_array_equal(vp[b], v0[b])
    # the tiles really differ, so a copy the other way would have shown
    assert not np.array_equal(k0[1], k0[4]) and not np.array_equal(v0[5], v0[0])


def test_copy_blocks_then_retarget_gathers_the_same_keys():
    """A truncate's copy-on-write: copy the shared block, point the table at
    the copy, and the sequence gathers exactly the keys it had."""
    rng = np.random.default_rng(44)
    B, Hkv, D = 16, 2, 8
    kp, vp = oracle.empty_pools(8, Hkv, D, B, "f32", fill=np.float32(np.nan))
    k = rng.standard_normal((40, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((40, Hkv, D)).astype(np.float32)
    row = [6, 2, 3]
    slots = [row[t // B] * B + t % B for t in range(40)]
    oracle.scatter(kp, vp, k, v, slots)
    oracle.copy_blocks(kp, vp, [2], [7])
    kg, vg = oracle.gather(kp, vp, [6, 7, 3], 40)
    np.testing.assert_array_equal(kg, k)
    np.testing.assert_array_equal(vg, v)

"""Pins of the oracle allocator (CPU only).

Block-hash prefix sharing (TensorSharp "高级功能" page, section
"连续批处理与分页 KV 缓存": full blocks are content-hashed and identical
prefixes are shared across concurrent and later requests; section "内存优化":
LRU eviction and cross-session reuse). The checks below follow from that
description and from counting, not from re-running the allocator's code.
"""
import numpy as np
import pytest

import oracle
import synth


def test_fifo_order_follows_initial_permutation():
    order = [5, 3, 7, 0, 1, 2, 4, 6]
    a = oracle.Allocator(8, 4, order)
    row, nb, ctx, slots = a.alloc(1, range(10), 8)
    assert row[:3] == [5, 3, 7] and row[3:] == [-1] * 5
    assert nb == 3 and ctx == 10
    assert slots == [5 * 4 + i for i in range(4)] + [3 * 4 + i for i in range(4)] + [28, 29]


def test_partial_block_filled_in_place():
    a = oracle.Allocator(4, 4)
    a.alloc(1, [1, 2, 3], 4)
    row, nb, ctx, slots = a.alloc(1, [4, 5], 4)
    assert row[:2] == [0, 1] and nb == 2 and ctx == 5
    assert slots == [3, 4]


def test_identical_prefix_shared_tail_private():
    B = 4
    a = oracle.Allocator(32, B)
    prefix = list(range(100, 110))             # 2 full blocks + 2 tokens
    r1, _, _, s1 = a.alloc(1, prefix + [1, 2, 3], 8)
    r2, _, _, s2 = a.alloc(2, prefix + [7, 8, 9], 8)
    assert r1[:2] == r2[:2]                   # two full prefix blocks shared
    assert r1[2] != r2[2]                     # block with diverging tokens private
    assert s2[:8] == [-1] * 8                 # shared tokens are not rewritten
    assert all(s >= 0 for s in s2[8:])
    free, cached, live = a.stats()
    assert live == 4 + 2 and free == 32 - 6     # 13 tokens = 4 blocks each, 2 shared


def test_no_share_after_divergence_even_if_later_tokens_match():
    B = 2
    a = oracle.Allocator(16, B)
    a.alloc(1, [1, 2, 3, 4], 8)
    r2, _, _, s2 = a.alloc(2, [9, 9, 3, 4], 8)   # block 1 content equal, parent differs
    r1 = a.seqs[1]["blocks"]
    assert r2[0] != r1[0] and r2[1] != r1[1]
    assert -1 not in s2


def test_mixed_step_sharing_counts():
    w = synth.mixed_step()
    a = oracle.Allocator(w.num_blocks, w.block_size, w.free_order)
    maxb = w.max_blocks_per_seq
    rows = []
    for s, seq in enumerate(w.seqs):
        row, nb, ctx, slots = a.alloc(s, seq.tokens, maxb)
        assert ctx == seq.ctx and nb == -(-seq.ctx // 16)
        rows.append(row)
        if 0 < s < 48:
            assert slots[:181 * 16] == [-1] * (181 * 16)
            assert all(x >= 0 for x in slots[181 * 16:])
    shared = rows[0][:181]
    for s in range(48):
        assert rows[s][:181] == shared
    for b in shared:
        assert a.ref[b] == 48
    # the block holding the prefix's last 4 tokens is private to each sequence
    assert len({rows[s][181] for s in range(48)}) == 48
    live = sum(-(-seq.ctx // 16) for seq in w.seqs) - 181 * 47
    assert a.stats()[2] == live
    used = set()
    for s, seq in enumerate(w.seqs):
        used.update(rows[s][:-(-seq.ctx // 16)])
    assert len(used) == live


def test_out_of_blocks_leaves_state_unchanged():
    a = oracle.Allocator(4, 4, [3, 2, 1, 0])
    a.alloc(1, range(8), 4)
    before = (list(a.free), list(a.ref), dict(a.table), a.stats())
    with pytest.raises(oracle.OutOfBlocks):
        a.alloc(2, range(50, 62), 4)           # needs 3 blocks, 2 free
    assert (list(a.free), list(a.ref), dict(a.table), a.stats()) == before
    assert 2 not in a.seqs


def test_release_lru_reuse_and_eviction():
    B = 2
    a = oracle.Allocator(6, B, [0, 1, 2, 3, 4, 5])
    a.alloc(1, [1, 2, 3, 4, 5], 8)            # blocks 0,1 (full) and 2 (partial)
    a.release(1)
    # freed to the back, last block first; full blocks keep their hash (cached)
    assert list(a.free) == [3, 4, 5, 2, 1, 0]
    assert a.stats() == (6, 2, 0)
    # same prefix comes back: revived from the free list, no new pops for it
    row, _, _, slots = a.alloc(2, [1, 2, 3, 4], 8)
    assert row[:2] == [0, 1] and slots == [-1] * 4
    assert list(a.free) == [3, 4, 5, 2]
    a.release(2)
    # fill the pool with other content: cached blocks get popped and evicted
    a.alloc(3, range(100, 112), 8)
    assert a.stats()[1] == 0
    a.release(3)
    row, _, _, slots = a.alloc(4, [1, 2], 8)   # prefix no longer cached
    assert -1 not in slots


def test_hash_collision_never_shares():
    a = oracle.Allocator(64, 4)
    a.hash_fn = lambda parent, toks: 42        # every block collides
    r1, _, _, _ = a.alloc(1, list(range(16)), 8)
    r2, _, _, s2 = a.alloc(2, list(range(100, 116)), 8)
    assert not set(r1[:4]) & set(r2[:4])
    assert -1 not in s2
    # identical first block still shares (same tokens, same empty parent)
    r3, _, _, s3 = a.alloc(3, list(range(4)) + [7, 7, 7, 7], 8)
    assert r3[0] == r1[0] and s3[:4] == [-1] * 4 and r3[1] != r1[1]


def test_block_hash_chains_parent():
    h0 = oracle.block_hash(0, [1, 2, 3, 4])
    assert oracle.block_hash(h0, [5, 6, 7, 8]) != oracle.block_hash(0, [5, 6, 7, 8])
    # little-endian layout of the hashed bytes: parent then tokens
    data = (0).to_bytes(8, "little") + b"".join(t.to_bytes(4, "little", signed=True) for t in [1, 2, 3, 4])
    assert h0 == oracle.fnv1a64(data)

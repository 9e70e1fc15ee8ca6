"""Product block manager (C++, host only) against the oracle allocator:
identical block tables, slot mappings and counters, bit for bit, over scripted
and random scenarios, including pool exhaustion, releases, LRU reuse, forced
hash collisions, rollbacks (truncate, with copy-on-write of shared blocks) and
freed prefixes below a sliding window."""
import numpy as np
import pytest

import oracle
import synth


@pytest.fixture(scope="module")
def pk():
    import paged_kv_attention_block_amd as pk
    return pk


class Pair:
    """Runs every operation on both allocators and compares the results."""

    def __init__(self, pk, num_blocks, B, order=None, collide=False):
        self.pk = pk
        self.c = pk.kv_pool_create(num_blocks, B, order)
        self.o = oracle.Allocator(num_blocks, B, order)
        if collide:
            pk.kv_pool_set_hash_mask(self.c, 0)
            self.o.hash_fn = lambda parent, toks: 0

    def alloc(self, seq, toks, maxb):
        try:
            want = self.o.alloc(seq, list(toks), maxb)
        except oracle.OutOfBlocks:
            with pytest.raises(self.pk.KVError) as e:
                self.pk.kv_pool_alloc(self.c, seq, toks, maxb)
            assert e.value.code == self.pk.KV_ENOMEM
            self.check_stats()
            return None
        row, nb, ctx, slots = self.pk.kv_pool_alloc(self.c, seq, toks, maxb)
        assert list(row) == want[0]
        assert (nb, ctx) == (want[1], want[2])
        assert list(slots) == want[3]
        self.check_stats()
        return want

    def release(self, seq):
        self.o.release(seq)
        self.pk.kv_pool_release(self.c, seq)
        self.check_stats()

    def truncate(self, seq, new_len, maxb=64):
        try:
            want = self.o.truncate(seq, new_len)
        except oracle.OutOfBlocks:
            with pytest.raises(self.pk.KVError) as e:
                self.pk.kv_pool_truncate(self.c, seq, new_len)
            assert e.value.code == self.pk.KV_ENOMEM
            self.check_stats()
            return None
        except ValueError:
            with pytest.raises(self.pk.KVError) as e:
                self.pk.kv_pool_truncate(self.c, seq, new_len)
            assert e.value.code == self.pk.KV_EINVAL
            return None
        got = self.pk.kv_pool_truncate(self.c, seq, new_len)
        assert got == tuple(want)
        self.check_row(seq, maxb)
        self.check_stats()
        return want

    def drop_prefix(self, seq, first_kept, maxb=64):
        self.o.drop_prefix(seq, first_kept)
        self.pk.kv_pool_drop_prefix(self.c, seq, first_kept)
        self.check_row(seq, maxb)
        self.check_stats()

    def check_row(self, seq, maxb):
        row, nb, ctx, _ = self.pk.kv_pool_alloc(self.c, seq, [], maxb)
        assert list(row) == self.o.table_row(seq, maxb)
        assert ctx == len(self.o.seqs[seq]["tokens"])

    def check_stats(self):
        assert self.pk.kv_pool_stats(self.c) == self.o.stats()


@pytest.mark.parametrize("name", ["tiny_decode", "mid_decode", "sink_decode", "mixed_step"])
def test_named_workload_tables_identical(pk, name):
    w = synth.by_name(name)
    pair = Pair(pk, w.num_blocks, 16, w.free_order)
    maxb = w.max_blocks_per_seq
    for s, seq in enumerate(w.seqs):
        pair.alloc(s, seq.tokens[:seq.ctx - seq.n_step], maxb)
    for s, seq in enumerate(w.seqs):
        pair.alloc(s, seq.tokens[seq.ctx - seq.n_step:], maxb)


def test_mixed_step_shares_prefix_in_product(pk):
    w = synth.mixed_step()
    p = pk.kv_pool_create(w.num_blocks, 16, w.free_order)
    rows = [pk.kv_pool_alloc(p, s, seq.tokens, w.max_blocks_per_seq)[0] for s, seq in enumerate(w.seqs)]
    for s in range(1, 48):
        assert (rows[s][:181] == rows[0][:181]).all()
    live = sum(-(-seq.ctx // 16) for seq in w.seqs) - 181 * 47
    assert pk.kv_pool_stats(p)[2] == live


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("collide", [False, True])
def test_random_scenarios_with_rollback_identical(pk, seed, collide):
    """Appends, releases, truncates (into own, shared and partial blocks,
    to block boundaries, to zero) and dropped prefixes, in random order."""
    rng = np.random.default_rng(100 + seed)
    B = int(rng.choice([2, 4, 16]))
    nb = int(rng.integers(10, 48))
    pair = Pair(pk, nb, B, rng.permutation(nb), collide)
    prefixes = [list(rng.integers(0, 4, size=int(rng.integers(B, 4 * B)))) for _ in range(2)]
    live = set()
    counts = {"truncate": 0, "copy": 0, "drop": 0}
    for step in range(200):
        op = rng.random()
        if op < 0.45 or not live:
            seq = int(rng.integers(0, 6))
            if seq not in live:
                toks = prefixes[int(rng.integers(0, 2))] + list(rng.integers(0, 4, size=int(rng.integers(0, 2 * B))))
            else:
                toks = list(rng.integers(0, 4, size=int(rng.integers(0, 3 * B + 1))))
            if pair.alloc(seq, toks, 64) is not None:
                live.add(seq)
        elif op < 0.75:
            seq = sorted(live)[int(rng.integers(0, len(live)))]
            n = len(pair.o.seqs[seq]["tokens"])
            new_len = int(rng.integers(0, n + 1)) if rng.random() < 0.8 else n + 1   # sometimes invalid
            got = pair.truncate(seq, new_len)
            counts["truncate"] += got is not None
            counts["copy"] += got is not None and got[0] >= 0
        elif op < 0.82:
            seq = sorted(live)[int(rng.integers(0, len(live)))]
            n = len(pair.o.seqs[seq]["tokens"])
            pair.drop_prefix(seq, int(rng.integers(0, n + 1)))
            counts["drop"] += 1
        else:
            seq = sorted(live)[int(rng.integers(0, len(live)))]
            pair.release(seq)
            live.discard(seq)
    assert counts["truncate"] > 10 and counts["drop"] > 3


def test_truncate_copy_on_write_in_product(pk):
    pair = Pair(pk, 16, 4)
    toks = list(range(1, 13))
    a = pair.alloc(1, toks, 8)
    pair.alloc(2, toks, 8)
    src, dst = pair.truncate(2, 5, 8)
    assert src == a[0][1] and dst >= 0
    row, _, _, _ = pk.kv_pool_alloc(pair.c, 2, [], 8)
    assert row[1] == dst and row[0] == a[0][0]


def test_truncate_enomem_is_atomic(pk):
    pair = Pair(pk, 3, 4)
    toks = list(range(1, 13))
    pair.alloc(1, toks, 8)
    pair.alloc(2, toks, 8)
    before = pk.kv_pool_stats(pair.c)
    assert pair.truncate(2, 5, 8) is None          # needs a copy, no block free
    assert pk.kv_pool_stats(pair.c) == before
    row, _, ctx, _ = pk.kv_pool_alloc(pair.c, 2, [], 8)
    assert ctx == 12


def test_tree_masks_match_oracle_and_reject_bad_parents(pk):
    rng = np.random.default_rng(7)
    for n in [0, 1, 5, 16, 32]:
        parents = [-1] + [int(rng.integers(-1, r)) for r in range(1, n)] if n else []
        np.testing.assert_array_equal(pk.kv_tree_masks(parents), oracle.tree_masks(parents))
    for bad in ([0], [-1, 1], [-2], [-1] * 33):
        with pytest.raises(pk.KVError) as e:
            pk.kv_tree_masks(bad)
        assert e.value.code == pk.KV_EINVAL


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("collide", [False, True])
def test_random_scenarios_identical(pk, seed, collide):
    rng = np.random.default_rng(seed)
    B = int(rng.choice([1, 2, 4, 16]))
    nb = int(rng.integers(8, 64))
    order = rng.permutation(nb)
    pair = Pair(pk, nb, B, order, collide)
    prefixes = [list(rng.integers(0, 5, size=int(rng.integers(0, 3 * B + 2)))) for _ in range(3)]
    live = set()
    for step in range(120):
        op = rng.random()
        if op < 0.55 or not live:
            seq = int(rng.integers(0, 8))
            if seq not in live:
                toks = prefixes[int(rng.integers(0, 3))] + list(rng.integers(0, 5, size=int(rng.integers(0, 2 * B))))
            else:
                toks = list(rng.integers(0, 5, size=int(rng.integers(0, 2 * B + 1))))
            if pair.alloc(seq, toks, 64) is not None:
                live.add(seq)
        else:
            seq = sorted(live)[int(rng.integers(0, len(live)))]
            pair.release(seq)
            live.discard(seq)


def test_collision_in_product_never_shares_different_tokens(pk):
    p = pk.kv_pool_create(64, 4)
    pk.kv_pool_set_hash_mask(p, 0)
    r1 = pk.kv_pool_alloc(p, 1, list(range(16)), 8)[0]
    r2, _, _, s2 = pk.kv_pool_alloc(p, 2, list(range(100, 116)), 8)
    assert not set(r1[:4]) & set(r2[:4])
    assert (s2 >= 0).all()


def test_enomem_is_atomic(pk):
    p = pk.kv_pool_create(4, 4, [3, 2, 1, 0])
    pk.kv_pool_alloc(p, 1, range(8), 4)
    before = pk.kv_pool_stats(p)
    with pytest.raises(pk.KVError) as e:
        pk.kv_pool_alloc(p, 2, range(50, 62), 4)
    assert e.value.code == pk.KV_ENOMEM
    assert "free" in e.value.message
    assert pk.kv_pool_stats(p) == before
    with pytest.raises(pk.KVError):
        pk.kv_pool_release(p, 2)                 # the failed sequence was not created


def test_prefix_hint_from_host_tables():
    """staging.prefix_hint reads the run of sequences sharing sequence 0's
    leading physical blocks off the host tables, and the positions they all
    hold in those blocks (by hand: 3 sequences share 20, 18 and 25 blocks)."""
    from paged_kv_attention_block_amd.staging import prefix_hint
    base = np.arange(100, 140, dtype=np.int32)
    t = np.full((5, 40), -1, dtype=np.int32)
    t[0] = base
    t[1, :20] = base[:20]
    t[1, 20:30] = np.arange(500, 510)
    t[2, :18] = base[:18]
    t[2, 18:25] = np.arange(600, 607)
    t[3, :25] = base[:25]
    t[4, :10] = np.arange(700, 710)          # shares nothing: ends the run
    assert prefix_hint(t) == (4, 18 * 16)
    assert prefix_hint(t[[0, 4]]) == (0, 0)
    assert prefix_hint(t[:1]) == (0, 0)
    t2 = t.copy()
    t2[1, :15] = base[:15]
    t2[1, 15:] = 900                          # 15 blocks = 240 tokens < 256: no run
    assert prefix_hint(t2[:2]) == (0, 0)

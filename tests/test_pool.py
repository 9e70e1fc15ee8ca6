"""Product block manager (C++, host only) against the oracle allocator:
identical block tables, slot mappings and counters, bit for bit, over scripted
and random scenarios, including pool exhaustion, releases, LRU reuse and forced
hash collisions."""
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

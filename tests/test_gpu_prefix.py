"""paged_attention_prefix_forward (GPU): a batch whose first sequences share a
prompt prefix in the same physical blocks computes the splits inside the
prefix once per group of sequences. Its output must be paged_attention_forward's
bit for bit, on the continuous-batching step with its 2900-token shared
prefix and on decode batches of every group size, and stay so when the hint
is wrong (a prefix longer than the blocks really shared, a member with more
than one row, sequences that share nothing): the groups check the block ids
and the rows themselves.
"""
import numpy as np
import pytest

import synth
from gpu_util import TOL, custom, max_err, oracle_rows, run_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a device"
    import paged_kv_attention_block_amd as pk
    return pk


def _bits(t):
    return t.contiguous().cpu().numpy().view(np.uint32)


def _prefix(pk, st, w, prefix_seqs, prefix_tokens):
    import torch
    return pk.paged_attention_prefix_forward(st.q, st.k_pools[0], st.v_pools[0], st.tables, st.context_lens, st.qsl,
                                             st.max_q_len, st.max_context_len, w.scale, prefix_seqs, prefix_tokens,
                                             sinks=st.sinks, out=torch.empty_like(st.out))


def _check(pk, w, prefix_seqs, prefix_tokens, oracle_sample=None):
    from paged_kv_attention_block_amd.staging import stage
    print(f"\n[case] prefix {w.name} dtype={w.dtype} S={len(w.seqs)} Hq={w.num_q_heads} Hkv={w.num_kv_heads} "
          f"D={w.head_dim} prefix_seqs={prefix_seqs} prefix_tokens={prefix_tokens}", flush=True)
    st = stage(w)
    want = _bits(run_forward(pk, st, w))
    got = _prefix(pk, st, w, prefix_seqs, prefix_tokens)
    np.testing.assert_array_equal(_bits(got), want)
    if oracle_sample is not None:
        err = max_err(got.cpu().numpy()[oracle_sample], oracle_rows(w, oracle_sample))
        print(f"[case] max abs err vs oracle {err:.3e}", flush=True)
        assert err <= TOL[w.dtype]
    return st


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp4"])
def test_mixed_step_shared_prompt(pk, dtype):
    """48 decode rows over a 2900-token prompt held in 181 shared blocks, two
    1024-row prefill chunks beside them: splits 0-4 lie in the shared blocks."""
    w = synth.mixed_step(dtype=dtype)
    _check(pk, w, 48, 181 * 16, oracle_sample=[0, 3, 4, 47, 48, 1071, 2095])


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (64, 8, 64), (16, 8, 128), (8, 8, 64), (4, 1, 64), (12, 4, 128)])
def test_decode_batch_group_sizes(pk, Hq, Hkv, D):
    """Decode batches (one tile per sequence): groups of 4 (G <= 4) or 2 (G = 8)
    sequences, a group count that does not divide the sequences, tails of
    different lengths past the prefix."""
    rng = np.random.default_rng(Hq * 10 + Hkv + D)
    n = 11
    ctxs = [2300 + int(x) for x in rng.integers(1, 700, size=n)] + [900, 4000]
    w = custom("bf16", Hq, Hkv, D, ctxs, [1] * len(ctxs), seed=int(rng.integers(1 << 30)), sinks=True,
               shared_prefix=2200, n_shared=n)
    _check(pk, w, n, (2200 // 16) * 16, oracle_sample=[0, 5, 10, 11, 12])


@pytest.mark.parametrize("Hq,Hkv,D", [(64, 8, 64), (16, 8, 128), (32, 8, 128), (12, 4, 128), (8, 8, 64)])
def test_decode_batch_group_sizes_at_the_prompt_end(pk, Hq, Hkv, D):
    """A 2900-token prompt: the split holding its end (2048-3071) is a group
    item too, its first three quarters shared and the members' last quarters
    computed member by member (G = 8: two members a group, G = 2, 4, 3, 1:
    four), contexts ending inside that split and past it, a last group of
    three sequences."""
    rng = np.random.default_rng(Hq * 100 + Hkv + D)
    n = 11
    ctxs = [2900 + int(x) for x in rng.integers(1, 700, size=n)] + [900, 4000]
    w = custom("bf16", Hq, Hkv, D, ctxs, [1] * len(ctxs), seed=int(rng.integers(1 << 30)), sinks=True,
               shared_prefix=2900, n_shared=n)
    _check(pk, w, n, (2900 // 16) * 16, oracle_sample=[0, 5, 10, 11, 12])


def test_more_heads_per_group_than_a_tile_shares(pk):
    """16 query heads per KV head: no groups (a member fills the tile), the plain grid."""
    w = custom("bf16", 32, 2, 64, [1500, 1700, 1600], [1, 1, 1], seed=401, shared_prefix=1300, n_shared=3)
    _check(pk, w, 3, 1296)


def test_hint_longer_than_the_shared_blocks(pk):
    """The sequences share 1100 tokens but the hint claims 3000: the splits
    past the real prefix hold different blocks and are computed per sequence."""
    w = custom("bf16", 32, 8, 128, [3300, 3500, 3100, 3900, 3200], [1] * 5, seed=402, shared_prefix=1100,
               n_shared=5)
    _check(pk, w, 5, 3000, oracle_sample=[0, 4])


def test_hint_over_unrelated_sequences(pk):
    """Nothing is shared, the hint says all of it is: every group falls back."""
    w = custom("bf16", 32, 8, 128, [2100, 2500, 2300, 2700, 2900, 2200], [1] * 6, seed=403)
    _check(pk, w, 6, 2048, oracle_sample=[0, 5])


@pytest.mark.parametrize("dtype", ["bf16", "fp4"])
def test_member_with_several_rows(pk, dtype):
    """A verify window (8 rows) and a prefill chunk among the prefix sequences:
    their groups compute the members one by one (the window in two passes of
    16 rows, the chunk in the prefill shape)."""
    w = custom(dtype, 16, 4, 128, [2500, 2600, 2700, 2550, 2800, 2650], [1, 8, 1, 300, 1, 1], seed=404,
               sinks=True, shared_prefix=2100, n_shared=6)
    _check(pk, w, 6, 2096, oracle_sample=[0, 1, 8, 9, 10, 309, 310, 311])


def test_short_prefix_and_zero_hint(pk):
    """A prefix shorter than the first split, and prefix_seqs 0 or 1: the plain grid."""
    w = custom("bf16", 32, 8, 128, [1200, 1300, 1250], [1, 1, 1], seed=405, shared_prefix=200, n_shared=3)
    _check(pk, w, 3, 192)
    _check(pk, w, 0, 2048)
    _check(pk, w, 1, 2048)


def test_rows_alone_through_the_prefix_path(pk):
    """Rows of the mixed step computed by the prefix path equal themselves
    computed alone (the row-invariance rule)."""
    import torch
    from paged_kv_attention_block_amd.staging import stage
    w = synth.mixed_step()
    st = stage(w)
    full = _bits(_prefix(pk, st, w, 48, 181 * 16))
    dev = st.q.device
    for i in [0, 1, 2, 3, 4, 17, 46, 47]:
        s = i
        p = w.seqs[s].ctx - 1
        one = pk.paged_attention_forward(
            st.q[i:i + 1].contiguous(), st.k_pools[0], st.v_pools[0], st.tables[s:s + 1].contiguous(),
            torch.tensor([p + 1], dtype=torch.int32, device=dev), torch.tensor([0, 1], dtype=torch.int32, device=dev),
            1, p + 1, w.scale, sinks=st.sinks)
        np.testing.assert_array_equal(_bits(one)[0], full[i], err_msg=f"row {i}")


def test_rejects_negative_hint(pk):
    from paged_kv_attention_block_amd import KVError
    from paged_kv_attention_block_amd.staging import stage
    w = custom("bf16", 32, 8, 128, [300, 400], [1, 1], seed=406)
    st = stage(w)
    with pytest.raises(KVError):
        _prefix(pk, st, w, -1, 100)
    with pytest.raises(KVError):
        _prefix(pk, st, w, 2, -5)


@pytest.mark.parametrize("dtype,shared", [("bf16", 1100), ("bf16", 1280), ("bf16", 1700), ("bf16", 2048),
                                          ("bf16", 600), ("bf16", 700), ("fp4", 1700), ("fp8", 1300),
                                          ("bf16", 1792), ("bf16", 1850), ("bf16", 2040), ("bf16", 740),
                                          ("fp4", 1850), ("fp8", 1900)])
def test_prefix_ending_inside_a_split(pk, dtype, shared):
    """Prompts ending inside a quarter and on a quarter edge, in 1024-key
    splits and in 256-key ones (600, 700, 740): the splits wholly inside the
    prompt are group items; the one holding its end is a group item too when
    the prompt covers its first three quarters (1792, 1850, 2040, 740, 1900:
    the members' last quarters are computed member by member, some contexts
    ending inside that quarter), otherwise each sequence's own, as are all
    later splits; groups of four sequences (G = 4, the last of one) with
    tails of different lengths. The output is the plain forward's, bit for
    bit."""
    rng = np.random.default_rng(shared + (dtype == "fp4"))
    n = 9
    ctxs = [shared + int(x) for x in rng.integers(1, 900, size=n)] + [1500]
    w = custom(dtype, 16, 4, 128, ctxs, [1] * len(ctxs), seed=int(rng.integers(1 << 30)), sinks=True,
               shared_prefix=shared, n_shared=n)
    _check(pk, w, n, (shared // 16) * 16, oracle_sample=[0, 4, 8, 9])

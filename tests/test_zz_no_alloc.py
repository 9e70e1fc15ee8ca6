"""paged_attention_forward_noalloc (GPU): the forward for callers that cannot
allocate, its split states in the library's own device scratch array. Through
the C ABI it must give the bits of paged_attention_forward with a caller
workspace, on two calls in a row (the second smaller, so it runs over the
first call's leftover states), and reject batches beyond the array's size."""
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


def _bits(t):
    return t.contiguous().cpu().numpy().view(np.uint32)


def _noalloc(pk, st, w, out):
    return pk.paged_attention_forward_noalloc(st.q, st.k_pools[0], st.v_pools[0], st.tables, st.context_lens,
                                              st.qsl, st.max_q_len, st.max_context_len, w.scale, sinks=st.sinks,
                                              out=out)


@pytest.mark.parametrize("dtype", ["bf16", "fp4"])
def test_noalloc_equals_forward_on_two_calls_second_smaller(pk, dtype):
    import torch
    from paged_kv_attention_block_amd.staging import stage
    cases = [
        # verify windows up to 16000 keys (about 13 MB of split states), then
        # a small decode batch of another head shape over the leftovers
        custom(dtype, 32, 8, 128, [9000, 4100, 16000, 700, 12000], [8, 8, 8, 8, 8], seed=601, sinks=True),
        custom(dtype, 64, 8, 64, [1500, 300, 2049], [1, 1, 1], seed=602, sinks=True),
    ]
    staged, want, outs = [], [], []
    for w in cases:
        st = stage(w)
        staged.append(st)
        want.append(_bits(run_forward(pk, st, w)))
        outs.append(torch.full_like(st.out, float("nan")))
    torch.cuda.synchronize()
    # cumulative count of torch's device allocations: frees of earlier
    # tests' garbage cannot move it, any allocation would
    before = torch.cuda.memory_stats()["allocation.all.allocated"]
    for w, st, out in zip(cases, staged, outs):
        print(f"\n[case] noalloc {dtype} S={len(w.seqs)} Hq={w.num_q_heads} D={w.head_dim} "
              f"ctx={[s.ctx for s in w.seqs]}", flush=True)
        _noalloc(pk, st, w, out)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats()["allocation.all.allocated"] == before
    for i, out in enumerate(outs):
        np.testing.assert_array_equal(_bits(out), want[i], err_msg=f"call {i}")


def test_noalloc_prefill_and_decode_batch(pk):
    """A batch with a prefill chunk (its rows need no split states) and
    decode rows, twice in a row with the second call smaller."""
    import torch
    from paged_kv_attention_block_amd.staging import stage
    cases = [custom("bf16", 16, 4, 128, [1500, 300, 5000], [200, 1, 8], seed=603, sinks=True),
             custom("bf16", 16, 4, 128, [900, 40], [1, 40], seed=604)]
    res = []
    for w in cases:
        st = stage(w)
        want = _bits(run_forward(pk, st, w))
        res.append((w, st, want))
    for w, st, want in res:
        got = _bits(_noalloc(pk, st, w, torch.empty_like(st.out)))
        np.testing.assert_array_equal(got, want)


def test_noalloc_rejects_batches_beyond_the_scratch_array(pk):
    """The mixed step's sizes (2096 rows x 32 heads x 7 splits x 520 bytes,
    about 244 MB) exceed the 64 MiB array: KV_EINVAL with the numbers, and
    nothing launched."""
    import torch
    from paged_kv_attention_block_amd import KVError, KV_EINVAL
    dev = torch.device("cuda:0")
    q = torch.zeros((2096, 32, 128), dtype=torch.bfloat16, device=dev)
    kp, vp = pk.empty_pools(64, 8, 128, torch.bfloat16, dev)
    bt = torch.zeros((50, 256), dtype=torch.int32, device=dev)
    ctx = torch.full((50,), 3925, dtype=torch.int32, device=dev)
    qsl = torch.arange(51, dtype=torch.int32, device=dev)
    need = pk.paged_attention_workspace_size(50, 2096, 32, 128, 3925)
    assert need > 64 << 20
    with pytest.raises(KVError) as ei:
        pk.paged_attention_forward_noalloc(q, kp, vp, bt, ctx, qsl, 1024, 3925, 0.1,
                                           out=torch.empty((2096, 32, 128), dtype=torch.float32, device=dev))
    assert ei.value.code == KV_EINVAL and str(need) in ei.value.message

"""Calls on a stream other than the current one (GPU).

Buffers a call allocates itself (the output and the split-state workspace)
must belong to the stream its kernels run on: torch's caching allocator hands
a freed block to later allocations on the stream it was allocated on, so a
workspace allocated on the current stream, and freed when the call returns,
could be handed to the next allocation there while the kernels on the side
stream still read it. These tests launch on a side stream, then allocate and
fill memory on the current stream before synchronizing.
"""
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


@pytest.mark.parametrize("kind", ["forward", "append", "masked"])
def test_side_stream_with_allocations_on_the_current_stream(pk, kind):
    import torch
    from paged_kv_attention_block_amd.staging import stage
    w = custom("bf16", 32, 8, 128, [5000, 3100, 9000, 700, 4000, 6100], [8, 8, 8, 8, 8, 8], seed=501, sinks=True)
    print(f"\n[case] side stream {kind}", flush=True)
    st = stage(w)
    want = _bits(run_forward(pk, st, w))
    ws_bytes = st.workspace.numel()
    side = torch.cuda.Stream()
    outs, junk = [], []
    for _ in range(4):
        side.wait_stream(torch.cuda.current_stream())
        if kind == "forward":
            o = pk.paged_attention_forward(st.q, st.k_pools[0], st.v_pools[0], st.tables, st.context_lens, st.qsl,
                                           st.max_q_len, st.max_context_len, w.scale, sinks=st.sinks, stream=side)
        elif kind == "append":
            # slot -1 everywhere: the tokens are resident, nothing is written
            none = torch.full_like(st.step_slots, -1)
            o = pk.paged_attention_append_forward(st.q, st.k_step, st.v_step, none, st.k_pools[0], st.v_pools[0],
                                                  st.tables, st.context_lens, st.qsl, st.max_q_len,
                                                  st.max_context_len, w.scale, sinks=st.sinks, stream=side)
        else:
            o = pk.paged_attention_masked_forward(st.q, st.k_pools[0], st.v_pools[0], st.tables, st.context_lens,
                                                  st.qsl, st.max_q_len, st.max_context_len, w.scale, sinks=st.sinks,
                                                  stream=side)
        outs.append(o)
        # the current stream allocates about a workspace's worth and fills it
        # while the side stream may still be running
        junk.append(torch.full((ws_bytes // 4 + 1024,), float("nan"), dtype=torch.float32, device=st.q.device))
    torch.cuda.synchronize()
    for o in outs:
        np.testing.assert_array_equal(_bits(o), want)

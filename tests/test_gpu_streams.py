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


def _mixed(dtype, seed):
    """Decode rows beside two prefill chunks: the chunks (more than 32 rows
    per KV head) take the sequential launch, the decode rows the split
    launch."""
    return custom(dtype, 32, 8, 128, [3000, 1100, 700, 2500, 1500, 900], [1, 300, 1, 64, 1, 1], seed=seed,
                  sinks=True)


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "fp4"])
def test_mixed_batch_on_two_streams(pk, dtype):
    """A batch with prefill chunks and decode rows, called eagerly (both
    launches on the caller's stream). Sampled rows of both shapes match the
    oracle; the whole output equals, bit for bit, the no-workspace entry
    point's; a call on a stream other than the current one, with the current
    stream allocating and filling memory meanwhile, gives the same bits."""
    import torch
    from gpu_util import TOL, max_err, oracle_rows
    from paged_kv_attention_block_amd.staging import stage
    w = _mixed(dtype, 511)
    print(f"\n[case] two streams {dtype}", flush=True)
    st = stage(w)
    got = run_forward(pk, st, w).cpu().numpy()
    qsl = [int(x) for x in w.qsl]
    rows = [qsl[0], qsl[2], qsl[4], qsl[5], qsl[1], qsl[1] + 137, qsl[2] - 1, qsl[3], qsl[4] - 1]
    want = oracle_rows(w, rows)
    assert max_err(got[rows], want) < TOL[dtype]
    serial = pk.paged_attention_forward_noalloc(st.q, st.k_pools[0], st.v_pools[0], st.tables, st.context_lens,
                                                st.qsl, st.max_q_len, st.max_context_len, w.scale, sinks=st.sinks,
                                                out=torch.empty_like(st.out))
    np.testing.assert_array_equal(_bits(serial), got.view(np.uint32))
    side = torch.cuda.Stream()
    outs, junk = [], []
    for _ in range(3):
        side.wait_stream(torch.cuda.current_stream())
        outs.append(pk.paged_attention_forward(st.q, st.k_pools[0], st.v_pools[0], st.tables, st.context_lens,
                                               st.qsl, st.max_q_len, st.max_context_len, w.scale, sinks=st.sinks,
                                               stream=side))
        junk.append(torch.full((st.out.numel() + 4096,), float("nan"), dtype=torch.float32, device=st.q.device))
    torch.cuda.synchronize()
    for o in outs:
        np.testing.assert_array_equal(_bits(o), got.view(np.uint32))


@pytest.mark.parametrize("dtype,window", [("bf16", 0), ("fp4", 0), ("bf16", 200), ("fp8", 700)])
def test_mixed_batch_in_a_graph(pk, dtype, window):
    """The same batch captured into a HIP graph, where the chunks' launch
    runs on the library's side stream beside the decode rows' launches (the
    side stream joins the capture through the fork event and rejoins the
    caller's stream through the join event). Every replay equals the eager
    call bit for bit, with eager calls and synchronizations between the
    replays. With a sliding window the masked instances take the same two
    streams."""
    import torch
    from paged_kv_attention_block_amd.staging import stage
    w = _mixed(dtype, 521 + window)
    print(f"\n[case] graph {dtype} window={window}", flush=True)
    st = stage(w)

    def call(out=None, ws=None):
        if window:
            return pk.paged_attention_masked_forward(st.q, st.k_pools[0], st.v_pools[0], st.tables,
                                                     st.context_lens, st.qsl, st.max_q_len, st.max_context_len,
                                                     w.scale, sinks=st.sinks, sliding_window=window,
                                                     out=out if out is not None else st.out,
                                                     workspace=ws if ws is not None else st.workspace)
        return pk.paged_attention_forward(st.q, st.k_pools[0], st.v_pools[0], st.tables, st.context_lens, st.qsl,
                                          st.max_q_len, st.max_context_len, w.scale, sinks=st.sinks,
                                          out=out if out is not None else st.out,
                                          workspace=ws if ws is not None else st.workspace)

    want = _bits(call())
    if window:
        # the window is real: the last row of the 300-row chunk differs from its unmasked value
        full = _bits(run_forward(pk, st, w))
        r = int(w.qsl[2]) - 1
        assert not np.array_equal(full[r], want[r])
    out = torch.empty_like(st.out)
    ws = torch.empty_like(st.workspace)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, ws)
    for i in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(_bits(out), want, err_msg=f"replay {i}")
        np.testing.assert_array_equal(_bits(call()), want, err_msg=f"eager after replay {i}")
        torch.cuda.synchronize()


def test_two_mixed_graphs_replayed_side_by_side(pk):
    """Two mixed batches, each captured into its own graph (both graphs hold
    branches on the library's side stream), replayed at the same time on two
    streams, several times: every replay equals its eager call bit for bit."""
    import torch
    from paged_kv_attention_block_amd.staging import stage
    cases = []
    for seed, dtype in ((531, "bf16"), (532, "fp4")):
        w = _mixed(dtype, seed)
        st = stage(w)
        want = _bits(run_forward(pk, st, w))
        out = torch.empty_like(st.out)
        ws = torch.empty_like(st.workspace)
        cases.append((w, st, want, out, ws))
    print("\n[case] two graphs side by side", flush=True)
    torch.cuda.synchronize()
    graphs = []
    for w, st, _, out, ws in cases:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            pk.paged_attention_forward(st.q, st.k_pools[0], st.v_pools[0], st.tables, st.context_lens, st.qsl,
                                       st.max_q_len, st.max_context_len, w.scale, sinks=st.sinks, out=out,
                                       workspace=ws)
        graphs.append(g)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for i in range(3):
        for _, _, _, out, _ in cases:
            out.fill_(float("nan"))
        torch.cuda.synchronize()
        for g, s in zip(graphs, streams):
            with torch.cuda.stream(s):
                g.replay()
        torch.cuda.synchronize()
        for k, (_, _, want, out, _) in enumerate(cases):
            np.testing.assert_array_equal(_bits(out), want, err_msg=f"graph {k} replay {i}")

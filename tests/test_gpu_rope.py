"""kv_qknorm_rope_scatter (GPU) against the oracle's QK-norm + NeoX RoPE +
scatter (TensorSharp "高级功能" page: the fused QK-Norm + NeoX RoPE kernel of
Qwen 3.5/3.6 and the batched forward's paged K/V scatter-write).

The oracle computes the exact value and rounds once to bf16; the kernel
computes in float32 (the angle in float64, reduced by multiples of pi/2 to
at most pi/4, then polynomials for the float32 sine and cosine) and rounds
once. Its float32 error before the rounding stays below 2^-20 of the row's
largest magnitude (a few float32 rounding steps in the norm, the angle and
the rotation; where a cos - b sin cancels, that error is large next to the
result). The bar per value: at most
one bf16 step of the oracle's value plus 2^-20 of the row's largest
magnitude, and at most 1 in 500 values differing at all. V is copied, so it
is bit-exact, and every pool slot that is not written keeps its NaN fill.
"""
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pk():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a device"
    import paged_kv_attention_block_amd as pk
    return pk


def within_bound(got, want, row_max, name):
    """got, want: bf16 bits; row_max: the largest |value| of each value's row."""
    g = oracle.to_f32(got, "bf16").astype(np.float64)
    w = oracle.to_f32(want, "bf16").astype(np.float64)
    _, e = np.frexp(w)
    step = np.ldexp(1.0, np.maximum(e - 8, -133))
    err = np.abs(g - w)
    bound = step + row_max * 2.0 ** -20
    frac = float(np.mean(got != want)) if got.size else 0.0
    worst = float(np.max(err / bound)) if got.size else 0.0
    print(f"[case] {name}: worst error / bound {worst:.3f}, differing fraction {frac:.2e}", flush=True)
    assert worst <= 1.0
    assert frac <= 2e-3


def row_max(bits):
    """Largest |value| of each row (last axis), broadcast back to the row."""
    a = np.abs(oracle.to_f32(bits, "bf16").astype(np.float64))
    return np.broadcast_to(a.max(axis=-1, keepdims=True), a.shape)


def slot_pattern(rng, n, nb):
    perm = rng.permutation(nb)
    s = []
    b = 0
    while len(s) < n:
        kind = len(s) // 16 % 3
        if kind == 0:                                   # a whole block in order
            s += list(range(perm[b] * 16, perm[b] * 16 + 16))
        elif kind == 1:                                 # a shifted run with a skipped slot
            s += [-1] + list(range(perm[b] * 16 + 3, perm[b] * 16 + 16)) + [-1, -1]
        else:                                           # a reversed whole block
            s += list(range(perm[b] * 16, perm[b] * 16 + 16))[::-1]
        b += 1
    return np.array(s[:n], dtype=np.int32)


CONFIGS = [
    # Hq, Hkv, D, rotary_dim, theta, weight offset, weights
    (32, 8, 128, 128, 1e6, 0.0, True),     # Qwen3-like
    (16, 2, 256, 64, 1e7, 1.0, True),      # partial rotary, zero-centred weights
    (64, 8, 64, 64, 150000.0, 0.0, False),  # no weights
    (8, 8, 128, 64, 10000.0, 0.0, True),
    (4, 2, 128, 0, 10000.0, 0.0, True),    # norm only
]


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: f"{c[0]}-{c[1]}-D{c[2]}-rd{c[3]}")
# n = 700 runs the workgroups of 4 heads, the smaller batches those of 2
@pytest.mark.parametrize("n", [1, 37, 130, 700])
def test_qknorm_rope_scatter_parity(pk, cfg, n):
    import torch
    Hq, Hkv, D, rd, theta, off, weights = cfg
    rng = np.random.default_rng(n * 1000 + Hq + D + rd)
    nb = 3 * ((n + 15) // 16) + 8
    bf = lambda *s: synth.f32_to_bf16_bits((rng.standard_normal(s) * 2.0).astype(np.float32))
    q, k, v = bf(n, Hq, D), bf(n, Hkv, D), bf(n, Hkv, D)
    qw = bf(D) if weights else None
    kw = bf(D) if weights else None
    pos = rng.integers(0, 131072, n).astype(np.int32)
    pos[: n // 2] = np.arange(n // 2) + 5000                   # consecutive positions, as in a prefill chunk
    slots = slot_pattern(rng, n, nb)
    print(f"\n[case] qknorm_rope Hq={Hq} Hkv={Hkv} D={D} rd={rd} theta={theta} off={off} w={weights} n={n}",
          flush=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    kp, vp = pk.empty_pools(nb, Hkv, D, torch.bfloat16, "cuda")
    kp.fill_(float("nan"))
    vp.fill_(float("nan"))
    q_out = pk.kv_qknorm_rope_scatter(dev(q), dev(k), dev(v), torch.from_numpy(pos).cuda(),
                                      torch.from_numpy(slots).cuda(), kp, vp,
                                      q_norm_weight=None if qw is None else dev(qw),
                                      k_norm_weight=None if kw is None else dev(kw), eps=1e-6, weight_offset=off,
                                      rope_theta=theta, rotary_dim=rd)
    torch.cuda.synchronize()
    ko, vo = oracle.empty_pools(nb, Hkv, D, 16, "bf16", fill=np.uint16(0x7FC0))
    q_want = oracle.qknorm_rope_scatter(ko, vo, q, k, v, pos, slots, qw, kw, 1e-6, theta, rd, off)
    within_bound(q_out.view(torch.int16).cpu().numpy().view(np.uint16), q_want, row_max(q_want), "q_out")
    kg = kp.view(torch.int16).cpu().numpy().view(np.uint16)
    vg = vp.view(torch.int16).cpu().numpy().view(np.uint16)
    mark_k = np.zeros(ko.shape, dtype=np.uint16)
    oracle.scatter(mark_k, np.zeros(vo.shape, np.uint16), np.ones((n, Hkv, D), np.uint16),
                   np.ones((n, Hkv, D), np.uint16), slots)
    written = mark_k == 1
    np.testing.assert_array_equal(kg[~written], ko[~written])         # untouched slots keep the NaN fill
    # K tiles [D/8][16][8]: a token's row is the D values of one slot
    kmax = np.abs(oracle.to_f32(np.where(written, ko, 0), "bf16").astype(np.float64))
    kmax = np.nan_to_num(kmax).max(axis=(2, 4), keepdims=True)
    within_bound(kg[written], ko[written], np.broadcast_to(kmax, ko.shape)[written], "K pool")
    np.testing.assert_array_equal(vg, vo)


def test_rejects_bad_rotary_dim_and_dtype(pk):
    import torch
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
    kp, vp = pk.empty_pools(4, 2, 128, torch.bfloat16, "cuda")
    args = (z(3, 4, 128), z(3, 2, 128), z(3, 2, 128), torch.zeros(3, dtype=torch.int32, device="cuda"),
            torch.zeros(3, dtype=torch.int32, device="cuda"), kp, vp)
    for rd in (3, 130, 36):
        with pytest.raises(pk.KVError) as e:
            pk.kv_qknorm_rope_scatter(*args, rotary_dim=rd)
        assert e.value.code == pk.KV_EINVAL
    kf, vf = pk.empty_pools(4, 2, 128, torch.float32, "cuda")
    with pytest.raises(pk.KVError):
        pk.kv_qknorm_rope_scatter(*args[:5], kf, vf)


def test_qknorm_rope_scatter_mixed_step_size(pk):
    """The launch the producer bench times: mixed_step's 2096 step tokens
    (48 decode tokens after a 2900-token prefix, two 1024-token chunks from
    position 0), 32 q / 8 KV heads, D 128, whole rotary, theta 1e6, norm
    weights, whole blocks (slots 16 ..): 131 x 12 workgroups of 4 heads.
    Every output against the oracle, to the same bar."""
    import torch
    w = synth.by_name("mixed_step")
    n, Hq, Hkv, D = w.total_rows, w.num_q_heads, w.num_kv_heads, w.head_dim
    rng = np.random.default_rng(2096)
    bf = lambda *s: synth.f32_to_bf16_bits(rng.standard_normal(s).astype(np.float32))
    q, k, v = bf(n, Hq, D), bf(n, Hkv, D), bf(n, Hkv, D)
    qw, kw = bf(D), bf(D)
    pos = np.concatenate([np.arange(s.ctx - s.q_len, s.ctx) for s in w.seqs]).astype(np.int32)
    slots = (np.arange(n) + 16).astype(np.int32)
    nb = -(-n // 16) + 2
    print(f"\n[case] qknorm_rope mixed_step size n={n} Hq={Hq} Hkv={Hkv} D={D}", flush=True)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    kp, vp = pk.empty_pools(nb, Hkv, D, torch.bfloat16, "cuda")
    kp.fill_(float("nan"))
    vp.fill_(float("nan"))
    q_out = pk.kv_qknorm_rope_scatter(dev(q), dev(k), dev(v), torch.from_numpy(pos).cuda(),
                                      torch.from_numpy(slots).cuda(), kp, vp, q_norm_weight=dev(qw),
                                      k_norm_weight=dev(kw), eps=1e-6, rope_theta=1e6, rotary_dim=D)
    torch.cuda.synchronize()
    ko, vo = oracle.empty_pools(nb, Hkv, D, 16, "bf16", fill=np.uint16(0x7FC0))
    q_want = oracle.qknorm_rope_scatter(ko, vo, q, k, v, pos, slots, qw, kw, 1e-6, 1e6, D)
    within_bound(q_out.view(torch.int16).cpu().numpy().view(np.uint16), q_want, row_max(q_want), "q_out")
    kg = kp.view(torch.int16).cpu().numpy().view(np.uint16)
    vg = vp.view(torch.int16).cpu().numpy().view(np.uint16)
    written = np.zeros(ko.shape, dtype=bool)
    written[1:1 + n // 16] = True
    np.testing.assert_array_equal(kg[~written], ko[~written])
    kmax = np.abs(oracle.to_f32(np.where(written, ko, 0), "bf16").astype(np.float64))
    kmax = np.nan_to_num(kmax).max(axis=(2, 4), keepdims=True)
    within_bound(kg[written], ko[written], np.broadcast_to(kmax, ko.shape)[written], "K pool")
    np.testing.assert_array_equal(vg, vo)

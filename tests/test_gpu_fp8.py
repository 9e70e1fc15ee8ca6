"""8-bit pools (GPU): kv_append_scatter quantizes each (token, KV head) row
into E4M3 codes with a float32 scale, and the pools it writes must equal the
oracle's (oracle.fp8_scatter) byte for byte, on slot patterns that take both
the whole-block path and the per-token path, and on rows chosen for the codec:
zero rows, exact ties between neighbouring codes (normal and subnormal),
signed zeros, a dominant value, huge and tiny magnitudes.
"""
import sys

import numpy as np
import pytest

import synth

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


def _bf16(x):
    return synth.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _slots(rng, nb):
    perm = rng.permutation(nb)
    s = []
    s += list(range(perm[0] * 16, perm[0] * 16 + 16))            # whole block, in order
    s += list(range(perm[2] * 16, perm[2] * 16 + 16))[::-1]       # whole block, reversed
    s += list(range(perm[4] * 16, perm[4] * 16 + 16))             # whole block, in order
    s += list(range(perm[1] * 16 + 5, perm[1] * 16 + 16))         # shifted run
    s += [-1] * 3 + list(range(perm[3] * 16, perm[3] * 16 + 13))  # skipped slots
    s += list(range(perm[5] * 16, perm[5] * 16 + 7))              # ragged end
    return np.array(s, dtype=np.int32)


def _run(pk, kn, vn, slots, nb):
    """Device scatter into 0xFF-filled pools and the oracle's; both as uint8."""
    import torch
    import oracle
    n, hkv, D = kn.shape
    tk = torch.from_numpy(kn.view(np.int16)).cuda().view(torch.bfloat16)
    tv = torch.from_numpy(vn.view(np.int16)).cuda().view(torch.bfloat16)
    kp, vp = pk.empty_pools(nb, hkv, D, torch.uint8, "cuda")
    kp.fill_(0xFF)
    vp.fill_(0xFF)
    pk.kv_append_scatter(tk, tv, torch.from_numpy(slots).cuda(), kp, vp)
    torch.cuda.synchronize()
    ko, vo = oracle.fp8_empty_pools(nb, hkv, D, fill=np.uint8(0xFF))
    oracle.fp8_scatter(ko, vo, kn, vn, slots)
    return kp.cpu().numpy(), vp.cpu().numpy(), ko, vo


def _assert_pools(got_k, got_v, want_k, want_v):
    for got, want, name in ((got_k, want_k, "K"), (got_v, want_v, "V")):
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{name} pool differs at {len(bad)} bytes, first {bad[:4].tolist()}: " \
                              f"got {got[tuple(bad[0])]:#04x} want {want[tuple(bad[0])]:#04x}"


@pytest.mark.parametrize("D", [64, 128])
def test_scatter_patterns_bit_exact(pk, D):
    rng = np.random.default_rng(500 + D)
    nb, hkv = 96, 3
    slots = _slots(rng, nb)
    n = slots.size
    announce(f"fp8 scatter patterns D={D} n={n}")
    kn = _bf16(rng.standard_normal((n, hkv, D), dtype=np.float32) * 3)
    vn = _bf16(rng.standard_normal((n, hkv, D), dtype=np.float32))
    _assert_pools(*_run(pk, kn, vn, slots, nb))


def _special_rows(rng, n, hkv, D):
    x = rng.standard_normal((n, hkv, D), dtype=np.float32)
    x[0, 0] = 0.0                                   # zero row: scale 0, codes 0
    x[1, 1] = -0.0
    row = rng.uniform(-1, 1, D).astype(np.float32)  # amax 448: scale 1, x / s = x
    row[:12] = [448.0, 1.0625, 1.1875, -1.0625, -1.1875, 2.0 ** -10, -(2.0 ** -10), 1.5 * 2.0 ** -9,
                -1.5 * 2.0 ** -9, 2.5 * 2.0 ** -9, 0.0, -0.0]
    x[2, 0] = row                                   # ties to the even code, signed zeros
    x[3, 1] = rng.uniform(-1e-3, 1e-3, D)
    x[3, 1, 7] = 1000.0                             # one dominant value; the rest mostly flush
    x[4, 0] = rng.standard_normal(D) * 1e37         # huge magnitudes
    x[5, 1] = -np.abs(rng.standard_normal(D)) - 1.0
    x[5, 1, 3] = -50.0                              # amax from a negative value
    x[6, 0] = 448.0 * np.sign(rng.standard_normal(D))  # every code at +-448
    return _bf16(x)


@pytest.mark.parametrize("D", [64, 128])
def test_scatter_special_rows(pk, D):
    rng = np.random.default_rng(600 + D)
    nb, hkv = 40, 2
    slots = _slots(rng, nb)
    n = slots.size
    announce(f"fp8 scatter special rows D={D} n={n}")
    kn = _special_rows(rng, n, hkv, D)
    vn = _special_rows(rng, n, hkv, D)[::-1].copy()
    # the special rows sit in the whole-block group (tokens 0..6) for K and in
    # the per-token groups for V (reversed order)
    _assert_pools(*_run(pk, kn, vn, slots, nb))


@pytest.mark.parametrize("D", [64, 128])
def test_scatter_tiny_rows(pk, D):
    """Rows near the smallest normal bf16: the scale 448 times smaller is a
    float32 subnormal and must be kept, as the oracle keeps it."""
    rng = np.random.default_rng(700 + D)
    nb, hkv = 8, 1
    slots = np.arange(32, dtype=np.int32) + 16
    x = rng.standard_normal((32, hkv, D), dtype=np.float32) * np.float32(2.0 ** -120)
    x[:4] *= np.float32(2.0 ** -6)                 # amax ~ 2^-126
    announce(f"fp8 scatter tiny rows D={D}")
    kn = _bf16(x)
    vn = _bf16(x[::-1].copy())
    _assert_pools(*_run(pk, kn, vn, slots, nb))

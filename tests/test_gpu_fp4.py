"""4-bit pools (GPU): kv_append_scatter quantizes each (token, KV head) row
into E2M1 codes with a float32 scale, and the pools it writes must equal the
oracle's (oracle.fp4_scatter) byte for byte, on slot patterns that take both
the whole-block path and the per-token path, including neighbouring tokens
that share V bytes and are written by different workgroups or different
calls, and on rows chosen for the codec: zero rows, exact ties between
neighbouring codes, signed zeros, values that flush to zero, a dominant
value, huge and tiny magnitudes.
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
    # tokens 0-15 (one workgroup): the odd slots of block A, then the first
    # half of block B; tokens 16-31 (the next workgroup): the even slots of
    # block A, then the second half of block B. Both workgroups write every
    # V byte of block A.
    s += [perm[6] * 16 + 2 * i + 1 for i in range(8)] + [perm[7] * 16 + i for i in range(8)]
    s += [perm[6] * 16 + 2 * i for i in range(8)] + [perm[7] * 16 + 8 + i for i in range(8)]
    s += list(range(perm[0] * 16, perm[0] * 16 + 16))            # whole block, in order
    s += list(range(perm[2] * 16, perm[2] * 16 + 16))[::-1]       # whole block, reversed
    s += list(range(perm[4] * 16, perm[4] * 16 + 16))             # whole block, in order
    s += list(range(perm[1] * 16 + 5, perm[1] * 16 + 16))         # shifted run
    s += [-1] * 3 + list(range(perm[3] * 16, perm[3] * 16 + 13))  # skipped slots
    s += list(range(perm[5] * 16, perm[5] * 16 + 7))              # ragged end
    return np.array(s, dtype=np.int32)


def _device_rows(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _run(pk, kn, vn, slots, nb, calls=1):
    """Device scatter into 0xFF-filled pools and the oracle's; both as uint8.
    calls > 1 splits the tokens into that many consecutive calls."""
    import torch
    import oracle
    n, hkv, D = kn.shape
    kp, vp = pk.empty_pools(nb, hkv, D, "fp4", "cuda")
    kp.fill_(0xFF)
    vp.fill_(0xFF)
    cuts = np.linspace(0, n, calls + 1).astype(int)
    for a, b in zip(cuts[:-1], cuts[1:]):
        pk.kv_append_scatter(_device_rows(kn[a:b]), _device_rows(vn[a:b]), torch.from_numpy(slots[a:b]).cuda(),
                             kp, vp)
    torch.cuda.synchronize()
    ko, vo = oracle.fp4_empty_pools(nb, hkv, D, fill=np.uint8(0xFF))
    oracle.fp4_scatter(ko, vo, kn, vn, slots)
    return kp.cpu().numpy(), vp.cpu().numpy(), ko, vo


def _assert_pools(got_k, got_v, want_k, want_v):
    for got, want, name in ((got_k, want_k, "K"), (got_v, want_v, "V")):
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{name} pool differs at {len(bad)} bytes, first {bad[:4].tolist()}: " \
                              f"got {got[tuple(bad[0])]:#04x} want {want[tuple(bad[0])]:#04x}"


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("calls", [1, 3])
def test_scatter_patterns_bit_exact(pk, D, calls):
    rng = np.random.default_rng(800 + D)
    nb, hkv = 96, 3
    slots = _slots(rng, nb)
    n = slots.size
    announce(f"fp4 scatter patterns D={D} n={n} calls={calls}")
    kn = _bf16(rng.standard_normal((n, hkv, D), dtype=np.float32) * 3)
    vn = _bf16(rng.standard_normal((n, hkv, D), dtype=np.float32))
    _assert_pools(*_run(pk, kn, vn, slots, nb, calls))


def test_scatter_one_token_at_a_time_in_random_order(pk):
    """Every token of four blocks in its own call, in a random order: each
    V byte is completed by a later call than the one that began it."""
    rng = np.random.default_rng(811)
    nb, hkv, D = 8, 2, 128
    slots = rng.permutation(np.arange(64) + 32).astype(np.int32)
    announce("fp4 scatter single tokens")
    kn = _bf16(rng.standard_normal((64, hkv, D), dtype=np.float32))
    vn = _bf16(rng.standard_normal((64, hkv, D), dtype=np.float32))
    _assert_pools(*_run(pk, kn, vn, slots, nb, calls=64))


def _special_rows(rng, n, hkv, D):
    x = rng.standard_normal((n, hkv, D), dtype=np.float32)
    x[0, 0] = 0.0                                   # zero row: scale 0, codes 0
    x[1, 1] = -0.0
    row = rng.uniform(-1, 1, D).astype(np.float32)  # amax 6: scale 1, x / s = x
    row[:20] = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0,
                0.0, -0.0, 0.2, -0.2, -6.0]
    x[2, 0] = row                                   # every tie goes to the even code; signed zeros
    x[3, 1] = rng.uniform(-1e-3, 1e-3, D)
    x[3, 1, 7] = 1000.0                             # one dominant value; the rest flush to +-0
    x[4, 0] = rng.standard_normal(D) * 1e37         # huge magnitudes
    x[5, 1] = -np.abs(rng.standard_normal(D)) - 1.0
    x[5, 1, 3] = -50.0                              # amax from a negative value
    x[6, 0] = 6.0 * np.sign(rng.standard_normal(D))  # every code at +-6
    return _bf16(x)


@pytest.mark.parametrize("D", [64, 128])
def test_scatter_special_rows(pk, D):
    rng = np.random.default_rng(900 + D)
    nb, hkv = 40, 2
    slots = _slots(rng, nb)
    n = slots.size
    announce(f"fp4 scatter special rows D={D} n={n}")
    kn = _special_rows(rng, n, hkv, D)
    vn = _special_rows(rng, n, hkv, D)[::-1].copy()
    _assert_pools(*_run(pk, kn, vn, slots, nb))


@pytest.mark.parametrize("D", [64, 128])
def test_scatter_tiny_rows(pk, D):
    """Rows near the smallest normal bf16: the scale 6 times smaller is a
    float32 subnormal and must be kept, as the oracle keeps it."""
    rng = np.random.default_rng(1000 + D)
    nb, hkv = 8, 1
    slots = np.arange(32, dtype=np.int32) + 16
    x = rng.standard_normal((32, hkv, D), dtype=np.float32) * np.float32(2.0 ** -120)
    x[:4] *= np.float32(2.0 ** -6)                 # amax ~ 2^-126
    announce(f"fp4 scatter tiny rows D={D}")
    kn = _bf16(x)
    vn = _bf16(x[::-1].copy())
    _assert_pools(*_run(pk, kn, vn, slots, nb))


@pytest.mark.parametrize("D", [64, 128])
def test_scatter_verify_windows(pk, D):
    """Verify-window writes: runs of 8 consecutive slots at random offsets
    (some crossing into the next block), two runs per group of 16 tokens, in
    blocks whose earlier slots an earlier call wrote. A run's tokens share V
    dwords (one channel of a half block) with each other and with the earlier
    tokens; where a run fills a half block the group writes the dword whole.
    Every pool byte equals the oracle's."""
    import torch
    import oracle
    rng = np.random.default_rng(1200 + D)
    nb, hkv, nwin = 40, 2, 12
    # run w starts in block 2w + 1 (and may end in block 2w + 2); one more
    # run fills the second half of block 25, whose first half came earlier
    starts = [(2 * w + 1) * 16 + int(rng.integers(0, 16)) for w in range(nwin)] + [25 * 16 + 8]
    before = np.concatenate([np.arange(st - st % 16, st) for st in starts]).astype(np.int32)
    wins = np.concatenate([np.arange(st, st + 8) for st in starts]).astype(np.int32)
    slots = np.concatenate([before, wins])
    n = slots.size
    announce(f"fp4 scatter verify windows D={D} n={n}")
    kn = _bf16(rng.standard_normal((n, hkv, D), dtype=np.float32) * 2)
    vn = _bf16(rng.standard_normal((n, hkv, D), dtype=np.float32))
    kp, vp = pk.empty_pools(nb, hkv, D, "fp4", "cuda")
    kp.fill_(0xFF)
    vp.fill_(0xFF)
    for a, b in ((0, before.size), (before.size, n)):
        if b > a:
            pk.kv_append_scatter(_device_rows(kn[a:b]), _device_rows(vn[a:b]), torch.from_numpy(slots[a:b]).cuda(),
                                 kp, vp)
    torch.cuda.synchronize()
    ko, vo = oracle.fp4_empty_pools(nb, hkv, D, fill=np.uint8(0xFF))
    oracle.fp4_scatter(ko, vo, kn, vn, slots)
    _assert_pools(kp.cpu().numpy(), vp.cpu().numpy(), ko, vo)

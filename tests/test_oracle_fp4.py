"""Pins of the oracle's 4-bit pools (FP4 E2M1 codes with per-token scales),
against the OCP E2M1 element definition, the arithmetic of the quantizer, and
an independent dense computation. CPU only."""
import numpy as np
import pytest

import oracle
import synth


def test_decode_matches_the_format_definition():
    # OCP microscaling formats, E2M1: bias 1, one mantissa bit, subnormal
    # value 0.5, largest value 6 = 1.5 * 2^2, no infinities or NaN
    dec = oracle.e2m1_decode
    assert dec(0x0) == 0.0 and np.signbit(dec(0x8))
    assert dec(0x1) == 0.5                              # the subnormal
    assert dec(0x2) == 1.0 and dec(0x3) == 1.5          # exponent field 1 is 2^0
    assert dec(0x4) == 2.0 and dec(0x5) == 3.0
    assert dec(0x6) == 4.0 and dec(0x7) == 6.0
    assert dec(0xF) == -6.0 and dec(0x9) == -0.5
    vals = dec(np.arange(8))
    assert np.all(np.diff(vals) > 0)
    np.testing.assert_array_equal(dec(np.arange(8, 16)), -vals)
    # only the low nibble counts
    np.testing.assert_array_equal(dec(np.arange(16) + 0x30), dec(np.arange(16)))


def test_encode_round_trips_every_code():
    codes = np.arange(16, dtype=np.uint8)
    np.testing.assert_array_equal(oracle.e2m1_encode(oracle.e2m1_decode(codes)), codes)


def test_encode_is_nearest_with_ties_to_the_even_code():
    vals = oracle.e2m1_decode(np.arange(8))
    mids = (vals[:-1] + vals[1:]) / 2                   # 0.25 0.75 1.25 1.75 2.5 3.5 5
    lo = np.arange(7)
    np.testing.assert_array_equal(oracle.e2m1_encode(mids).astype(int), np.where(lo % 2 == 0, lo, lo + 1))
    np.testing.assert_array_equal(oracle.e2m1_encode(-mids).astype(int), np.where(lo % 2 == 0, lo, lo + 1) | 8)
    rng = np.random.default_rng(15)
    x = rng.uniform(-6, 6, 20000)
    err = np.abs(oracle.e2m1_decode(oracle.e2m1_encode(x)) - x)
    allv = np.concatenate([vals, -vals])
    best = np.min(np.abs(allv[None, :] - x[:, None]), axis=1)   # no code is closer
    np.testing.assert_array_equal(err, best)
    # the sign bit follows the input, zero included
    assert oracle.e2m1_encode(np.array([-0.0]))[0] == 8 and oracle.e2m1_encode(np.array([-0.2]))[0] == 8
    with pytest.raises(ValueError):
        oracle.e2m1_encode(np.array([6.5]))


def test_quantize_rows_scale_error_bound_and_zero_rows():
    rng = np.random.default_rng(16)
    x = synth.f32_to_bf16_bits(rng.standard_normal((300, 128), dtype=np.float32) * 3)
    x[7] = 0
    codes, s = oracle.fp4_quantize_rows(x)
    assert codes.dtype == np.uint8 and codes.max() <= 15
    xf = oracle.to_f32(x, "bf16").astype(np.float64)
    amax = np.max(np.abs(xf), axis=1)
    np.testing.assert_array_equal(s, (amax.astype(np.float32) / np.float32(6)).astype(np.float32))
    assert s[7] == 0 and not codes[7].any()
    deq = oracle.fp4_dequantize(codes, s)
    # one mantissa bit: half a step is at most a quarter of the value, and a
    # quarter of s in the subnormal range
    bound = np.abs(xf) / 4 + s[:, None].astype(np.float64) / 4
    assert np.all(np.abs(deq - xf) <= bound * (1 + 1e-6))
    # each row's largest element lands on the largest code exactly
    big = np.argmax(np.abs(xf), axis=1)
    top = oracle.e2m1_decode(codes[np.arange(300), big])
    assert np.all((np.abs(top) == 6) | (s == 0))


def test_tile_layout_is_a_bijection_onto_the_code_nibbles():
    for D in (64, 128):
        for f in (oracle._fp4_k_nibbles, oracle._fp4_v_nibbles):
            off = f(D)
            assert off.shape == (16, D)
            assert np.array_equal(np.sort(off.ravel()), np.arange(16 * D))
    # a lane's 8 consecutive channels (K) or 8 consecutive tokens (V) share 4 bytes
    k = oracle._fp4_k_nibbles(128)
    assert np.array_equal(k[3, 40:48], k[3, 40] + np.arange(8)) and k[3, 40] % 8 == 0
    v = oracle._fp4_v_nibbles(128)
    assert np.array_equal(v[8:16, 37], v[8, 37] + np.arange(8)) and v[8, 37] % 8 == 0


@pytest.mark.parametrize("D", [64, 128])
def test_scatter_then_gather_gives_the_dequantized_rows(D):
    rng = np.random.default_rng(17 + D)
    nb, hkv, ctx = 12, 3, 70
    kp, vp = oracle.fp4_empty_pools(nb, hkv, D, fill=0xFF)
    assert kp.shape == (nb, hkv, 8 * D + 64)
    perm = rng.permutation(nb)
    table = perm[:5]
    slots = np.array([table[t // 16] * 16 + t % 16 for t in range(ctx)])
    k = synth.f32_to_bf16_bits(rng.standard_normal((ctx, hkv, D), dtype=np.float32))
    v = synth.f32_to_bf16_bits(rng.standard_normal((ctx, hkv, D), dtype=np.float32))
    oracle.fp4_scatter(kp, vp, k, v, slots)
    gk, gv = oracle.fp4_gather(kp, vp, table, ctx)
    kc, ks = oracle.fp4_quantize_rows(k)
    vc, vs = oracle.fp4_quantize_rows(v)
    np.testing.assert_array_equal(gk, oracle.fp4_dequantize(kc, ks))
    np.testing.assert_array_equal(gv, oracle.fp4_dequantize(vc, vs))
    assert np.all(kp[perm[5:]] == 0xFF)
    # the codes of one block, read back nibble by nibble by hand
    # every code and scale read back nibble by nibble, byte by byte, by hand
    nk, nv = oracle._fp4_k_nibbles(D), oracle._fp4_v_nibbles(D)
    for tok in range(0, ctx, 3):
        blk, off = int(table[tok // 16]), tok % 16
        for h in range(hkv):
            for pool, nib, codes, sc in ((kp, nk, kc, ks), (vp, nv, vc, vs)):
                for c in range(D):
                    n_ = int(nib[off, c])
                    byte = int(pool[blk, h, n_ // 2])
                    assert (byte >> 4 if n_ % 2 else byte & 0xF) == codes[tok, h, c]
                raw = bytes(int(x) for x in pool[blk, h, 8 * D + 4 * off:8 * D + 4 * off + 4])
                assert np.frombuffer(raw, np.float32)[0] == sc[tok, h]


def test_scatter_of_interleaved_tokens_keeps_both_nibbles():
    """Two tokens sharing V bytes, written by separate calls and in one call
    in either order, give the same tiles as one whole-block write."""
    rng = np.random.default_rng(21)
    D, hkv = 64, 2
    k = synth.f32_to_bf16_bits(rng.standard_normal((16, hkv, D), dtype=np.float32))
    v = synth.f32_to_bf16_bits(rng.standard_normal((16, hkv, D), dtype=np.float32))
    whole = oracle.fp4_empty_pools(2, hkv, D, fill=0xFF)
    oracle.fp4_scatter(*whole, k, v, np.arange(16) + 16)
    odd_even = oracle.fp4_empty_pools(2, hkv, D, fill=0xFF)
    order = np.r_[np.arange(1, 16, 2), np.arange(0, 16, 2)]
    for half in (order[:8], order[8:]):
        oracle.fp4_scatter(*odd_even, k[half], v[half], half + 16)
    mixed = oracle.fp4_empty_pools(2, hkv, D, fill=0xFF)
    perm = rng.permutation(16)
    oracle.fp4_scatter(*mixed, k[perm], v[perm], perm + 16)
    for got in (odd_even, mixed):
        np.testing.assert_array_equal(got[0][1], whole[0][1])
        np.testing.assert_array_equal(got[1][1], whole[1][1])


def test_paged_attention_on_4bit_pools_matches_dense_brute_force():
    from scipy.special import softmax
    rng = np.random.default_rng(18)
    Hq, Hkv, D, ctxs = 4, 2, 64, [5, 33, 17]
    nb = 8
    kp, vp = oracle.fp4_empty_pools(nb, Hkv, D)
    perm = rng.permutation(nb)
    tables = np.full((3, 3), -1)
    used = 0
    ks, vs = [], []
    for s, c in enumerate(ctxs):
        nbk = -(-c // 16)
        tables[s, :nbk] = perm[used:used + nbk]
        used += nbk
        k = synth.f32_to_bf16_bits(rng.standard_normal((c, Hkv, D), dtype=np.float32))
        v = synth.f32_to_bf16_bits(rng.standard_normal((c, Hkv, D), dtype=np.float32))
        oracle.fp4_scatter(kp, vp, k, v, [tables[s, t // 16] * 16 + t % 16 for t in range(c)])
        ks.append(oracle.fp4_dequantize(*oracle.fp4_quantize_rows(k)))
        vs.append(oracle.fp4_dequantize(*oracle.fp4_quantize_rows(v)))
    q = synth.f32_to_bf16_bits(rng.standard_normal((3, Hq, D), dtype=np.float32))
    qsl = np.array([0, 1, 2, 3], dtype=np.int32)
    got = oracle.paged_attention(q, kp, vp, tables, ctxs, qsl, Hq, Hkv, 0.125, None, "fp4")
    qf = oracle.to_f32(q, "bf16").astype(np.float64)
    for s in range(3):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            w = softmax(0.125 * ks[s][:, g] @ qf[s, h])
            np.testing.assert_allclose(got[s, h], w @ vs[s][:, g], rtol=1e-12, atol=1e-12)

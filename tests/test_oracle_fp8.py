"""Pins of the oracle's 8-bit pools (FP8 E4M3 codes with per-token scales),
against the OCP E4M3FN definition, the arithmetic of the quantizer, and an
independent dense computation. CPU only."""
import numpy as np
import pytest

import oracle
import synth


def test_decode_matches_the_format_definition():
    # OCP 8-bit floating point, E4M3: bias 7, subnormal step 2^-9, largest
    # normal 448 = 1.75 * 2^8, NaN at S.1111.111, no infinities
    dec = oracle.e4m3_decode
    assert dec(0x00) == 0.0 and np.signbit(dec(0x80))
    assert dec(0x01) == 2.0 ** -9                      # smallest subnormal
    assert dec(0x07) == 7 * 2.0 ** -9                  # largest subnormal
    assert dec(0x08) == 2.0 ** -6                      # smallest normal
    assert dec(0x38) == 1.0
    assert dec(0x3C) == 1.5
    assert dec(0x7E) == 448.0 and dec(0xFE) == -448.0
    assert np.isnan(dec(0x7F)) and np.isnan(dec(0xFF))
    vals = oracle.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(vals) > 0)                   # codes 0x00..0x7E ascend


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)


def test_encode_ties_go_to_the_even_code_and_rounding_is_nearest():
    vals = oracle.e4m3_decode(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2
    got = oracle.e4m3_encode(mids).astype(int)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    np.testing.assert_array_equal(got, want)
    rng = np.random.default_rng(5)
    x = rng.uniform(-448, 448, 20000)
    err = np.abs(oracle.e4m3_decode(oracle.e4m3_encode(x)) - x)
    # nearest: no finite code is closer
    allv = np.concatenate([vals, -vals])
    best = np.min(np.abs(allv[None, :] - x[:, None]), axis=1)
    np.testing.assert_array_equal(err, best)


def test_quantize_rows_scale_error_bound_and_zero_rows():
    rng = np.random.default_rng(6)
    x = synth.f32_to_bf16_bits(rng.standard_normal((300, 128), dtype=np.float32) * 3)
    x[7] = 0                                           # a row of zeros
    codes, s = oracle.fp8_quantize_rows(x)
    xf = oracle.to_f32(x, "bf16").astype(np.float64)
    amax = np.max(np.abs(xf), axis=1)
    np.testing.assert_array_equal(s, (amax.astype(np.float32) / np.float32(448)).astype(np.float32))
    assert s[7] == 0 and not codes[7].any()
    deq = oracle.fp8_dequantize(codes, s)
    # 3 mantissa bits: half a step is at most 2^-4 of the value (subnormals: half of 2^-9 * s)
    bound = np.abs(xf) * 2.0 ** -4 + s[:, None].astype(np.float64) * 2.0 ** -10
    assert np.all(np.abs(deq - xf) <= bound * (1 + 1e-6))
    # the largest element of each row lands on the largest code (or one step below it)
    big = np.argmax(np.abs(xf), axis=1)
    top = oracle.e4m3_decode(codes[np.arange(300), big])
    assert np.all((np.abs(top) >= 416) | (s == 0))


def test_tile_layout_is_a_bijection():
    for D in (64, 128):
        ok, ov = oracle._fp8_k_offsets(D), oracle._fp8_v_offsets(D)
        for off in (ok, ov):
            assert off.shape == (16, D)
            assert np.array_equal(np.sort(off.ravel()), np.arange(16 * D))


@pytest.mark.parametrize("D", [64, 128])
def test_scatter_then_gather_gives_the_dequantized_rows(D):
    rng = np.random.default_rng(7 + D)
    nb, hkv, ctx = 12, 3, 70
    kp, vp = oracle.fp8_empty_pools(nb, hkv, D, fill=0xFF)
    perm = rng.permutation(nb)
    table = perm[:5]
    slots = np.array([table[t // 16] * 16 + t % 16 for t in range(ctx)])
    k = synth.f32_to_bf16_bits(rng.standard_normal((ctx, hkv, D), dtype=np.float32))
    v = synth.f32_to_bf16_bits(rng.standard_normal((ctx, hkv, D), dtype=np.float32))
    oracle.fp8_scatter(kp, vp, k, v, slots)
    gk, gv = oracle.fp8_gather(kp, vp, table, ctx)
    kc, ks = oracle.fp8_quantize_rows(k)
    vc, vs = oracle.fp8_quantize_rows(v)
    np.testing.assert_array_equal(gk, oracle.fp8_dequantize(kc, ks))
    np.testing.assert_array_equal(gv, oracle.fp8_dequantize(vc, vs))
    # untouched blocks keep their fill
    assert np.all(kp[perm[5:]] == 0xFF)


def test_paged_attention_on_8bit_pools_matches_dense_brute_force():
    from scipy.special import softmax
    rng = np.random.default_rng(8)
    Hq, Hkv, D, ctxs = 4, 2, 64, [5, 33, 17]
    nb = 8
    kp, vp = oracle.fp8_empty_pools(nb, Hkv, D)
    perm = rng.permutation(nb)
    tables = np.full((3, 3), -1)
    used = 0
    ks, vs, qs = [], [], []
    for s, c in enumerate(ctxs):
        nbk = -(-c // 16)
        tables[s, :nbk] = perm[used:used + nbk]
        used += nbk
        k = synth.f32_to_bf16_bits(rng.standard_normal((c, Hkv, D), dtype=np.float32))
        v = synth.f32_to_bf16_bits(rng.standard_normal((c, Hkv, D), dtype=np.float32))
        oracle.fp8_scatter(kp, vp, k, v, [tables[s, t // 16] * 16 + t % 16 for t in range(c)])
        ks.append(oracle.fp8_dequantize(*oracle.fp8_quantize_rows(k)))
        vs.append(oracle.fp8_dequantize(*oracle.fp8_quantize_rows(v)))
    q = synth.f32_to_bf16_bits(rng.standard_normal((3, Hq, D), dtype=np.float32))
    qsl = np.array([0, 1, 2, 3], dtype=np.int32)
    got = oracle.paged_attention(q, kp, vp, tables, ctxs, qsl, Hq, Hkv, 0.125, None, "fp8")
    qf = oracle.to_f32(q, "bf16").astype(np.float64)
    for s in range(3):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            w = softmax(0.125 * ks[s][:, g] @ qf[s, h])
            np.testing.assert_allclose(got[s, h], w @ vs[s][:, g], rtol=1e-12, atol=1e-12)

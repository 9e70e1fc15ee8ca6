"""Pins of the oracle's QK-norm + NeoX RoPE producer step (CPU only).

TensorSharp "高级功能" page: one kernel applies QK-Norm and NeoX RoPE for
Qwen 3.5/3.6; the batched forward pairs the projection with the paged K/V
scatter-write. The checks use what the definitions fix: a hand-worked
rotation (which pairs turn, and which way), position 0 is the identity,
attention scores depend only on the distance between positions, pair norms
are kept, dimensions past rotary_dim pass through, RMSNorm's closed form, and
the single bf16 rounding against exact rational arithmetic.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


def test_bf16_rounding_matches_float32_path_and_rationals():
    rng = np.random.default_rng(1)
    f = rng.standard_normal(2000).astype(np.float32) * np.float32(37.0)
    # float32 inputs: the library's float32 -> bf16 rounding is an independent route
    np.testing.assert_array_equal(oracle.f64_to_bf16_bits(f.astype(np.float64)), synth.f32_to_bf16_bits(f))
    # float64 inputs between bf16 neighbours: exact rational nearest, ties to even
    for x in list(rng.standard_normal(300) * 5) + [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8 + 2 ** -40)]:
        got = float(oracle.to_f32(oracle.f64_to_bf16_bits(np.array([x])), "bf16")[0])
        e = math.frexp(x)[1]
        step = Fraction(2) ** (e - 8)
        fx = Fraction(x)
        lo = (fx / step).__floor__() * step
        hi = lo + step
        d_lo, d_hi = fx - lo, hi - fx
        if d_lo < d_hi:
            want = lo
        elif d_hi < d_lo:
            want = hi
        else:
            want = lo if (lo / step) % 2 == 0 else hi
        assert Fraction(got) == want, x


def test_rms_norm_closed_form():
    x = np.array([[3.0, 4.0]])
    np.testing.assert_allclose(oracle.rms_norm(x, None, 0.0), [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]],
                               rtol=1e-15)
    np.testing.assert_allclose(oracle.rms_norm(x, np.array([2.0, 0.5]), 0.5),
                               [[2 * 3 / math.sqrt(13.0), 0.5 * 4 / math.sqrt(13.0)]], rtol=1e-15)
    np.testing.assert_allclose(oracle.rms_norm(x, np.array([1.0, -0.5]), 0.0, weight_offset=1.0),
                               [[2 * 3 / math.sqrt(12.5), 0.5 * 4 / math.sqrt(12.5)]], rtol=1e-15)


def test_rope_hand_example():
    """D = rotary_dim = 4, theta 10000, position 1: pairs (0, 2) turn by 1
    radian and (1, 3) by 10000^(-1/2) = 0.01 radian."""
    x = np.array([[[1.0, 2.0, 3.0, 4.0]]])
    got = oracle.rope_neox(x, [1], 10000.0, 4)[0, 0]
    c0, s0, c1, s1 = math.cos(1.0), math.sin(1.0), math.cos(0.01), math.sin(0.01)
    want = [1 * c0 - 3 * s0, 2 * c1 - 4 * s1, 3 * c0 + 1 * s0, 4 * c1 + 2 * s1]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-15)


def test_rope_identity_at_zero_norms_kept_tail_passes():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 3, 128))
    np.testing.assert_array_equal(oracle.rope_neox(x, [0] * 5, 1e6, 128), x)
    y = oracle.rope_neox(x, [0, 7, 100, 5000, 131071], 1e6, 64)
    np.testing.assert_array_equal(y[..., 64:], x[..., 64:])
    pair = lambda a: a[..., :32] ** 2 + a[..., 32:64] ** 2
    np.testing.assert_allclose(pair(y), pair(x), rtol=1e-12)


@pytest.mark.parametrize("rd", [128, 64])
def test_rope_scores_depend_on_distance_only(rd):
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    def score(m, n):
        return float(np.sum(oracle.rope_neox(q, [m], 10000.0, rd) * oracle.rope_neox(k, [n], 10000.0, rd)))
    for m, n, d in [(5, 2, 40), (1000, 10, 777), (0, 3, 12345)]:
        assert abs(score(m, n) - score(m + d, n + d)) < 1e-9
    assert abs(score(5, 2) - score(6, 2)) > 1e-6


def test_qknorm_rope_scatter_writes_rotated_k_and_v():
    rng = np.random.default_rng(4)
    n, Hq, Hkv, D = 20, 4, 2, 64
    bf = lambda *s: synth.f32_to_bf16_bits(rng.standard_normal(s).astype(np.float32))
    q, k, v = bf(n, Hq, D), bf(n, Hkv, D), bf(n, Hkv, D)
    qw, kw = bf(D), bf(D)
    pos = rng.integers(0, 4000, n)
    slots = rng.permutation(64)[:n]
    kp, vp = oracle.empty_pools(4, Hkv, D, 16, "bf16", fill=np.uint16(0x7FC0))
    q_out = oracle.qknorm_rope_scatter(kp, vp, q, k, v, pos, slots, qw, kw, 1e-6, 1e6, D)
    q_want, k_want = oracle.qknorm_rope(q, k, pos, qw, kw, 1e-6, 1e6, D)
    np.testing.assert_array_equal(q_out, q_want)
    for i, s in enumerate(slots):
        kk, vv = oracle.gather(kp, vp, [s // 16] * 1, 16)
        np.testing.assert_array_equal(kk[s % 16], k_want[i])
        np.testing.assert_array_equal(vv[s % 16], v[i])
    # the stored K equals the rounded exact value of the definition
    x = oracle.to_f32(k[3, 1], "bf16").astype(np.float64)
    w = oracle.to_f32(kw, "bf16").astype(np.float64)
    y = x / math.sqrt(float(np.mean(x * x)) + 1e-6) * w
    np.testing.assert_array_equal(k_want[3, 1], oracle.f64_to_bf16_bits(oracle.rope_neox(y[None, None], [pos[3]],
                                                                                       1e6, D)[0, 0]))

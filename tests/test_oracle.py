"""Pins of the oracle (CPU only): closed forms, brute force, invariants.

The oracle is checked here against things other than itself: hand-derived
closed forms (tests/golden/closed_forms.json), a brute-force dense formulation
that uses a library softmax over an explicit mask matrix with repeated KV
heads, and properties that the textbook definition fixes (weights sum to one,
GQA equals MHA on repeated heads, block placement does not matter, a window
row equals the same row computed alone, the sink only rescales).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def brute_dense(q, ks, vs, q_lens, Hq, Hkv, scale, sinks=None):
    """Dense attention per sequence: repeat KV heads to Hq, build the full
    [q_len, ctx] causal mask (bottom-right aligned), library softmax over an
    optional extra sink column whose value vector is zero."""
    outs = []
    row = 0
    for k, v, ql in zip(ks, vs, q_lens):
        ctx = k.shape[0]
        kr = np.repeat(k.astype(np.float64), Hq // Hkv, axis=1)   # [ctx, Hq, D]
        vr = np.repeat(v.astype(np.float64), Hq // Hkv, axis=1)
        qs = q[row:row + ql].astype(np.float64)                   # [ql, Hq, D]
        scores = np.einsum("rhd,thd->hrt", qs, kr) * scale        # [Hq, ql, ctx]
        pos = np.arange(ctx)[None, :]
        last = (ctx - ql + np.arange(ql))[:, None]
        mask = pos <= last                                        # [ql, ctx]
        scores = np.where(mask[None], scores, -np.inf)
        if sinks is not None:
            col = np.broadcast_to(np.asarray(sinks, np.float64)[:, None, None], (Hq, ql, 1))
            scores = np.concatenate([scores, col], axis=2)
            vr = np.concatenate([vr, np.zeros((1,) + vr.shape[1:])], axis=0)
        w = softmax(scores, axis=2)
        outs.append(np.einsum("hrt,thd->rhd", w, vr))
        row += ql
    return np.concatenate(outs, axis=0)


def rand_case(rng, S, Hq, Hkv, D, max_ctx, sinks):
    ctxs = rng.integers(1, max_ctx, size=S, endpoint=True)
    qls = [int(rng.integers(1, c, endpoint=True)) for c in ctxs]
    q = rng.standard_normal((sum(qls), Hq, D)).astype(np.float32)
    ks = [rng.standard_normal((c, Hkv, D)).astype(np.float32) for c in ctxs]
    vs = [rng.standard_normal((c, Hkv, D)).astype(np.float32) for c in ctxs]
    sk = rng.standard_normal(Hq).astype(np.float32) * 2 if sinks else None
    qsl = np.concatenate([[0], np.cumsum(qls)]).astype(np.int32)
    return q, ks, vs, qls, qsl, sk


# --- closed forms -------------------------------------------------------------

def test_golden_attention_cases(oracle_lib):
    cases = json.load(open(GOLDEN))["attention"]
    for c in cases:
        q = np.array([[c["q"]]], np.float32)
        k = np.array(c["k"], np.float32)[:, None, :]
        v = np.array(c["v"], np.float32)[:, None, :]
        sinks = None if c["sink"] is None else np.array([c["sink"]], np.float32)
        out = oracle.attention(q, [k], [v], [0, 1], 1, 1, c["scale"], sinks)[0, 0]
        np.testing.assert_allclose(out, c["out"], rtol=0, atol=c["tol"], err_msg=c["name"])


def test_golden_fnv_vectors():
    for c in json.load(open(GOLDEN))["fnv1a64"]:
        assert oracle.fnv1a64(c["input_ascii"].encode()) == int(c["hash"], 16)


def test_uniform_scores_give_mean(oracle_lib):
    rng = np.random.default_rng(3)
    q, ks, vs, qls, qsl, _ = rand_case(rng, 3, 4, 2, 8, 30, False)
    out = oracle.attention(q, ks, vs, qsl, 4, 2, 0.0)
    row = 0
    for k, v, ql in zip(ks, vs, qls):
        ctx = k.shape[0]
        for r in range(ql):
            p = ctx - ql + r
            for h in range(4):
                want = v[:p + 1, h // 2, :].astype(np.float64).mean(axis=0)
                np.testing.assert_allclose(out[row + r, h], want, rtol=0, atol=1e-13)
        row += ql


def test_weights_sum_to_one_and_sink_share(oracle_lib):
    """With V = 1 the output is the total weight of the keys: 1 without a
    sink, Z0 / (Z0 + e^sigma) with one (Z0 = sum_t e^{x_t})."""
    rng = np.random.default_rng(4)
    q, ks, vs, qls, qsl, sk = rand_case(rng, 4, 2, 1, 4, 25, True)
    ones = [np.ones_like(v) for v in vs]
    out = oracle.attention(q, ks, ones, qsl, 2, 1, 0.5)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-13)
    outs = oracle.attention(q, ks, ones, qsl, 2, 1, 0.5, sk)
    row = 0
    for k, ql in zip(ks, qls):
        ctx = k.shape[0]
        for r in range(ql):
            p = ctx - ql + r
            for h in range(2):
                x = [0.5 * float(np.dot(q[row + r, h].astype(np.float64), k[t, 0].astype(np.float64)))
                     for t in range(p + 1)]
                z0 = sum(math.exp(xi) for xi in x)
                want = z0 / (z0 + math.exp(float(sk[h])))
                assert abs(outs[row + r, h, 0] - want) < 1e-12
        row += ql


def test_sink_rescales_only(oracle_lib):
    rng = np.random.default_rng(5)
    q, ks, vs, qls, qsl, sk = rand_case(rng, 3, 4, 4, 8, 20, True)
    plain = oracle.attention(q, ks, vs, qsl, 4, 4, 0.3)
    withs = oracle.attention(q, ks, vs, qsl, 4, 4, 0.3, sk)
    share = oracle.attention(q, ks, [np.ones_like(v) for v in vs], qsl, 4, 4, 0.3, sk)[:, :, :1]
    np.testing.assert_allclose(withs, plain * share, rtol=1e-12, atol=1e-14)
    very_neg = np.full_like(sk, -1e30)
    np.testing.assert_allclose(oracle.attention(q, ks, vs, qsl, 4, 4, 0.3, very_neg), plain,
                               rtol=0, atol=0)


# --- brute force --------------------------------------------------------------

@pytest.mark.parametrize("Hq,Hkv,D", [(1, 1, 1), (2, 1, 4), (4, 2, 8), (8, 2, 64), (8, 8, 4), (4, 1, 64)])
@pytest.mark.parametrize("sinks", [False, True])
def test_matches_brute_force(oracle_lib, Hq, Hkv, D, sinks):
    rng = np.random.default_rng(100 + Hq * 10 + Hkv + D + sinks)
    for _ in range(3):
        q, ks, vs, qls, qsl, sk = rand_case(rng, 3, Hq, Hkv, D, 40, sinks)
        scale = 1.0 / math.sqrt(D)
        got = oracle.attention(q, ks, vs, qsl, Hq, Hkv, scale, sk)
        want = brute_dense(q, ks, vs, qls, Hq, Hkv, scale, sk)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_large_logits_stable(oracle_lib):
    """Scores in the hundreds overflow a naive exp; the max shift keeps the
    result equal to the library softmax."""
    rng = np.random.default_rng(6)
    q, ks, vs, qls, qsl, sk = rand_case(rng, 2, 2, 1, 16, 30, True)
    got = oracle.attention(q, ks, vs, qsl, 2, 1, 40.0, sk * 100)
    want = brute_dense(q, ks, vs, qls, 2, 1, 40.0, sk * 100)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_gqa_equals_mha_on_repeated_heads(oracle_lib):
    rng = np.random.default_rng(7)
    q, ks, vs, qls, qsl, sk = rand_case(rng, 3, 8, 2, 8, 25, True)
    gqa = oracle.attention(q, ks, vs, qsl, 8, 2, 0.35, sk)
    rep = lambda a: np.repeat(a, 4, axis=1)
    mha = oracle.attention(q, [rep(k) for k in ks], [rep(v) for v in vs], qsl, 8, 8, 0.35, sk)
    np.testing.assert_array_equal(gqa, mha)


def test_window_row_equals_row_alone(oracle_lib):
    """Row r of a q_len-row window equals the same query as a single decode row
    on the first p + 1 keys."""
    rng = np.random.default_rng(8)
    q, ks, vs, qls, qsl, sk = rand_case(rng, 2, 4, 2, 8, 30, True)
    full = oracle.attention(q, ks, vs, qsl, 4, 2, 0.4, sk)
    row = 0
    for k, v, ql in zip(ks, vs, qls):
        ctx = k.shape[0]
        for r in range(ql):
            p = ctx - ql + r
            alone = oracle.attention(q[row + r:row + r + 1], [k[:p + 1]], [v[:p + 1]], [0, 1], 4, 2, 0.4, sk)
            np.testing.assert_array_equal(alone[0], full[row + r])
        row += ql


# --- gather / scatter ----------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scatter_gather_roundtrip_and_elementwise(dtype):
    rng = np.random.default_rng(9)
    Hkv, D, B, nb = 2, 16, 16, 12
    kp, vp = oracle.empty_pools(nb, Hkv, D, B, dtype)
    ctx = 37
    perm = rng.permutation(nb)[:3]
    k = rng.integers(0, 60000, size=(ctx, Hkv, D)).astype(oracle.storage_dtype(dtype))
    v = rng.integers(0, 60000, size=(ctx, Hkv, D)).astype(oracle.storage_dtype(dtype))
    slots = [int(perm[t // B]) * B + t % B for t in range(ctx)]
    oracle.scatter(kp, vp, k, v, slots)
    kg, vg = oracle.gather(kp, vp, perm, ctx)
    np.testing.assert_array_equal(kg, k)
    np.testing.assert_array_equal(vg, v)
    # element by element against the layout's definition
    X = oracle.chunk_elems(dtype)
    for t in range(ctx):
        b, o = int(perm[t // B]), t % B
        for h in range(Hkv):
            for d in range(D):
                assert kp[b, h, d // X, o, d % X] == k[t, h, d]
                assert vp[b, h, d, o] == v[t, h, d]


def test_scatter_skips_minus_one():
    kp, vp = oracle.empty_pools(2, 1, 8, 16, "f32", fill=np.nan)
    new = np.ones((2, 1, 8), np.float32)
    oracle.scatter(kp, vp, new, new, [-1, 17])
    assert np.isnan(kp[0]).all() and np.isnan(vp[0]).all()
    assert (kp[1, 0, :, 1, :] == 1).all() and (vp[1, 0, :, 1] == 1).all()
    assert np.isnan(kp[1, 0, :, 0, :]).all()


def test_paged_attention_permutation_invariant(oracle_lib):
    rng = np.random.default_rng(10)
    Hq, Hkv, D, B = 4, 2, 8, 16
    ctxs, qls = [37, 64, 5], [1, 3, 5]
    q = rng.standard_normal((sum(qls), Hq, D)).astype(np.float32)
    dense = [(rng.standard_normal((c, Hkv, D)).astype(np.float32),
              rng.standard_normal((c, Hkv, D)).astype(np.float32)) for c in ctxs]
    qsl = np.concatenate([[0], np.cumsum(qls)]).astype(np.int32)
    outs = []
    for trial in range(2):
        order = rng.permutation(16)
        kp, vp = oracle.empty_pools(16, Hkv, D, B, "f32", fill=np.nan)
        tables, pos = [], 0
        for (k, v), c in zip(dense, ctxs):
            nb = -(-c // B)
            row = list(order[pos:pos + nb]) + [-1] * (4 - nb)
            pos += nb
            oracle.scatter(kp, vp, k, v, [row[t // B] * B + t % B for t in range(c)])
            tables.append(row)
        outs.append(oracle.paged_attention(q, kp, vp, tables, ctxs, qsl, Hq, Hkv, 0.3))
    np.testing.assert_array_equal(outs[0], outs[1])
    want = brute_dense(q, [k for k, _ in dense], [v for _, v in dense], qls, Hq, Hkv, 0.3)
    np.testing.assert_allclose(outs[0], want, rtol=0, atol=1e-12)


def test_bf16_widening_exact():
    x = np.array([1.0, -2.5, 3.140625, 1e-3, 65504.0, -0.0], np.float32)
    bits = synth.f32_to_bf16_bits(x)
    back = oracle.to_f32(bits, "bf16")
    # every value that fits in 8 significant bits survives unchanged
    assert back[0] == 1.0 and back[1] == -2.5 and back[2] == 3.140625
    assert np.signbit(back[5])
    # round-to-nearest-even: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1)
    tie = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], np.float32)
    np.testing.assert_array_equal(oracle.to_f32(synth.f32_to_bf16_bits(tie), "bf16"),
                                  [1.0, 1.0 + 2.0 ** -6])

"""Pins for the oracle's attention over the 4-bit K/V cache (section 12).

gist.science/nl "Technische Samenvatting" §4 (W4A4KV4: keys and values kept
as 4-bit MXINT). The pages print no worked example; the pins below use K and
V built from exactly representable MXINT4 values (every 32-block a set of
codes in [-7, 7] with its maximum in [4, 7], times a power of two), so the
cache holds those values exactly and the expected outputs follow from the
definition of softmax attention.
"""
import numpy as np
import pytest

import oracle as orc


def representable(rng, shape):
    """float32 array whose 32-blocks along the last axis are MXINT4-exact."""
    *lead, D = shape
    c = rng.integers(-7, 8, size=(*lead, D // 32, 32))
    c[..., 0] = rng.choice([-7, -6, -5, -4, 4, 5, 6, 7], size=(*lead, D // 32))   # block maximum in [4, 7]
    e = rng.integers(-6, 3, size=(*lead, D // 32, 1)).astype(np.float64)
    return (c * np.exp2(e)).reshape(shape).astype(np.float32)


def cache(kv):
    codes, scales = orc.quantize_kv(kv)
    return codes, scales


def attention_np(q, K, V, scale, Hkv):
    Hq, D = q.shape
    G = Hq // Hkv
    out = np.zeros((Hq, D))
    for h in range(Hq):
        g = h // G
        s = scale * (K[:, g, :].astype(np.float64) @ q[h].astype(np.float64))
        p = np.exp(s - s.max())
        out[h] = (p[:, None] * V[:, g, :].astype(np.float64)).sum(0) / p.sum()
    return out


def test_cache_of_representable_values_is_exact():
    rng = np.random.default_rng(1)
    V = representable(rng, (3, 2, 64))
    codes, scales = cache(V)
    P = dict(q8=np.zeros((6, 0), np.int8), q6=np.zeros((6, 0), np.uint8), q4=codes.reshape(6, 32),
             sc=scales.reshape(6, 2), n8=0, n6=0, n4=2, K=64, rows=6)
    c = orc.unpack(P)
    deq = np.array([[orc.dequant(int(c[r, k]), int(P["sc"][r, k // 32])) for k in range(64)] for r in range(6)])
    assert np.array_equal(deq, V.reshape(6, 64).astype(np.float64))


def test_one_token_returns_its_value_row():
    rng = np.random.default_rng(2)
    K, V = representable(rng, (1, 2, 64)), representable(rng, (1, 2, 64))
    q = rng.standard_normal((6, 64)).astype(np.float32)
    out = orc.attend_kv4(q, *cache(K), *cache(V), 0.125)
    for h in range(6):
        assert np.array_equal(out[h], V[0, h // 3].astype(np.float64))


def test_equal_scores_average_the_values():
    rng = np.random.default_rng(3)
    T = 9
    K = np.repeat(representable(rng, (1, 1, 32)), T, axis=0)
    V = representable(rng, (T, 1, 32))
    q = rng.standard_normal((2, 32)).astype(np.float32)
    out = orc.attend_kv4(q, *cache(K), *cache(V), 1.0)
    mean = V[:, 0, :].astype(np.float64).mean(0)
    np.testing.assert_allclose(out, np.stack([mean, mean]), rtol=1e-13, atol=0)


def test_brute_force_and_grouping():
    rng = np.random.default_rng(4)
    for T, Hq, Hkv, D in ((5, 4, 2, 32), (17, 8, 2, 64), (3, 3, 3, 96)):
        K, V = representable(rng, (T, Hkv, D)), representable(rng, (T, Hkv, D))
        q = rng.standard_normal((Hq, D)).astype(np.float32)
        q[1] = q[0]                                           # two heads of one group, one query
        scale = 1.0 / np.sqrt(D)
        out = orc.attend_kv4(q, *cache(K), *cache(V), scale)
        np.testing.assert_allclose(out, attention_np(q, K, V, scale, Hkv), rtol=1e-12, atol=1e-300)
        if Hq // Hkv >= 2:
            assert np.array_equal(out[0], out[1])


def test_value_scaling_and_dominant_token():
    rng = np.random.default_rng(5)
    T, D = 6, 64
    K, V = representable(rng, (T, 1, D)), representable(rng, (T, 1, D))
    q = rng.standard_normal((1, D)).astype(np.float32)
    a = orc.attend_kv4(q, *cache(K), *cache(V), 0.3)
    b = orc.attend_kv4(q, *cache(K), *cache(V * 2), 0.3)
    assert np.array_equal(b, 2 * a)                           # powers of two scale exactly
    K2 = np.zeros((T, 1, D), np.float32)
    K2[3, 0, :32] = 4.0                                       # token 3 alone scores 4 * sum(q[:32]) * 1e4
    q2 = np.zeros((1, D), np.float32)
    q2[0, :32] = 1.0
    out = orc.attend_kv4(q2, *cache(K2), *cache(V), 1e4)
    assert np.array_equal(out[0], V[3, 0].astype(np.float64))


def test_quantized_random_cache_matches_dequantized_attention():
    # random K/V go through the quantizer; the oracle's attention equals plain
    # attention on the values the pinned unpack/dequant functions recover
    rng = np.random.default_rng(6)
    T, Hq, Hkv, D = 40, 8, 2, 64
    K = rng.standard_normal((T, Hkv, D)).astype(np.float32) * 3
    V = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((Hq, D)).astype(np.float32)

    def deq(x):
        codes, scales = cache(x)
        rows = T * Hkv
        P = dict(q8=np.zeros((rows, 0), np.int8), q6=np.zeros((rows, 0), np.uint8), q4=codes.reshape(rows, D // 2),
                 sc=scales.reshape(rows, D // 32), n8=0, n6=0, n4=D // 32, K=D, rows=rows)
        c = orc.unpack(P)
        e = P["sc"].astype(np.float64) - 127
        return (c * np.exp2(np.repeat(e, 32, axis=1))).reshape(T, Hkv, D)

    out = orc.attend_kv4(q, *cache(K), *cache(V), 0.125)
    np.testing.assert_allclose(out, attention_np(q, deq(K), deq(V), 0.125, Hkv), rtol=1e-12, atol=1e-14)
    with pytest.raises(ValueError):
        orc.attend_kv4(q[:3], *cache(K), *cache(V), 0.125)    # 3 heads over 2 KV heads

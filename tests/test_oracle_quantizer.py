"""Pins for the oracle's MXINT block quantizer (oracle section 1).

The pages give the format (one shared power-of-two scale per 32-value block,
4/6/8-bit mantissas: gist.science/nl technical summary §1, §2.2) but print no
worked example, so the expectations below are derived by hand from the
scale rule (comments show the arithmetic), by brute force over every
representable code, and from invariants that any correct MXINT quantizer has.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

f32 = np.float32


def q(orc, v, m):
    return orc.quantize_block(np.asarray(v, dtype=np.float32), m)


# ---------------------------------------------------------------- worked examples
def test_worked_example_all_widths(orc):
    v = [1.0, 0.3, -2.5, 0.75, 0.25, 1.25, -0.75, 3.0]
    # amax = 3 -> floor(log2 3) = 1.
    # m=4: s = 1-2 = -1, v*2 = [2, 0.6, -5, 1.5, 0.5, 2.5, -1.5, 6]; RNE sends
    #      0.6->1, 1.5->2, 0.5->0, 2.5->2, -1.5->-2.
    c, b = q(orc, v, 4)
    assert b == 127 - 1 and c.tolist() == [2, 1, -5, 2, 0, 2, -2, 6]
    # m=6: s = 1-4 = -3, v*8 = [8, 2.4, -20, 6, 2, 10, -6, 24].
    c, b = q(orc, v, 6)
    assert b == 127 - 3 and c.tolist() == [8, 2, -20, 6, 2, 10, -6, 24]
    # m=8: s = 1-6 = -5, v*32 = [32, 9.6, -80, 24, 8, 40, -24, 96].
    c, b = q(orc, v, 8)
    assert b == 127 - 5 and c.tolist() == [32, 10, -80, 24, 8, 40, -24, 96]


def test_worked_example_clamp_edge(orc):
    v = [3.9, 1.0, -0.1]
    # m=4: s=-1, v*2 = [7.8, 2, -0.2] -> 7.8 rounds to 8 which clamps to 7.
    c, b = q(orc, v, 4)
    assert b == 126 and c.tolist() == [7, 2, 0]
    # error of the clamped element: 3.9 - 7*0.5 = 0.4 = 0.8 * scale (> scale/2)
    assert abs(float(f32(3.9)) - 7 * 0.5) == pytest.approx(0.8 * 0.5, rel=1e-6)
    c, b = q(orc, v, 6)   # s=-3: [31.2, 8, -0.8]
    assert b == 124 and c.tolist() == [31, 8, -1]
    c, b = q(orc, v, 8)   # s=-5: [124.8, 32, -3.2]
    assert b == 122 and c.tolist() == [125, 32, -3]


def test_zero_block(orc):
    for m in (4, 6, 8):
        c, b = q(orc, np.zeros(32), m)
        assert b == 0 and not c.any()
        c, b = q(orc, [-0.0, 0.0], m)
        assert b == 0 and not c.any()


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_nonfinite_block(orc, bad):
    v = np.ones(32, np.float32)
    v[5] = bad
    for m in (4, 6, 8):
        c, b = q(orc, v, m)
        assert b == 0xFF and not c.any()
    assert math.isnan(orc.dequant(0, 0xFF))


def test_exponent_clamp_tiny(orc):
    # amax = 2^-140: s = -140-6 = -146 clamps to -127 (byte 0); v*2^127 = 2^-13 -> 0
    c, b = q(orc, [2.0 ** -140, -(2.0 ** -141)], 8)
    assert b == 0 and c.tolist() == [0, 0]


def test_subnormal_elements(orc):
    # amax = 2^-122 (normal): s = -122-6 = -128 clamps to -127; elements * 2^127:
    # 2^-122 -> 32, 2^-127 (fp32 subnormal) -> 1, 2^-149 (smallest subnormal) -> 2^-22 -> 0
    v = np.array([2.0 ** -122, 2.0 ** -127, 2.0 ** -149, -(2.0 ** -127)], np.float32)
    assert v[1] != 0 and v[2] != 0
    c, b = q(orc, v, 8)
    assert b == 0 and c.tolist() == [32, 1, 0, -1]


def test_largest_finite(orc):
    fmax = np.finfo(np.float32).max
    # E = 127, m=4: s = 125 (byte 252); fmax*2^-125 = 8 - 2^-21 rounds to 8, clamps to 7
    c, b = q(orc, [fmax, -fmax, 2.0 ** 125], 4)
    assert b == 252 and c.tolist() == [7, -7, 1]


# ---------------------------------------------------------------- brute force
def brute(v, m):
    """Search the scale byte and every code; independent of the oracle's rint/frexp."""
    v = [float(f32(x)) for x in v]
    amax = max(abs(x) for x in v)
    cmax = 2 ** (m - 1) - 1
    # the scale that puts amax in the top binade [2^(m-2), 2^(m-1)) of an m-bit
    # integer, found by search; below the E8M0 range it sticks at -127
    s = None
    for cand in range(-127, 128):
        r = Fraction(amax) / Fraction(2) ** cand
        if Fraction(2 ** (m - 2)) <= r < Fraction(2 ** (m - 1)):
            s = cand
            break
    if s is None:
        assert Fraction(amax) / Fraction(2) ** -127 < 2 ** (m - 2)
        s = -127
    codes = []
    for x in v:
        best = None
        for c in range(-cmax, cmax + 1):
            d = abs(Fraction(x) - c * Fraction(2) ** s)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        codes.append(best[1])
    return codes, s + 127


@pytest.mark.parametrize("m", [4, 6, 8])
def test_brute_force_small_blocks(orc, m):
    rng = np.random.default_rng(11 + m)
    for trial in range(60):
        n = int(rng.integers(1, 9))
        kind = trial % 4
        if kind == 0:
            v = rng.standard_normal(n)
        elif kind == 1:
            v = rng.standard_t(4, n) * 0.02
        elif kind == 2:   # exact ties: half-integers times a power of two
            v = (rng.integers(-2 ** m, 2 ** m, n) / 2.0) * 2.0 ** int(rng.integers(-10, 10))
        else:             # wide dynamic range inside one block
            v = rng.standard_normal(n) * 2.0 ** rng.integers(-30, 30, n)
        v = v.astype(np.float32)
        if not np.any(v):
            continue
        c, b = q(orc, v, m)
        bc, bb = brute(v, m)
        assert b == bb and c.tolist() == bc, (v, m)


# ---------------------------------------------------------------- invariants
def deq(codes, b):
    return codes.astype(np.float64) * 2.0 ** (b - 127)


@pytest.mark.parametrize("m", [4, 6, 8])
def test_invariants_random_blocks(orc, m):
    rng = np.random.default_rng(100 + m)
    cmax = 2 ** (m - 1) - 1
    clamped_blocks = 0
    nblocks = 3000
    for i in range(nblocks):
        v = (rng.standard_t(4, 32) * 0.02 if i % 2 else rng.standard_normal(32)).astype(np.float32)
        c, b = q(orc, v, m)
        scale = 2.0 ** (b - 127)
        # max code sits in the top binade (amax / scale in [2^(m-2), 2^(m-1)))
        assert 2 ** (m - 2) <= np.abs(v).max() / scale < 2 ** (m - 1)
        # per-element error: <= scale/2 unless clamped, < scale when clamped
        err = np.abs(v.astype(np.float64) - deq(c, b))
        cl = np.abs(c) == cmax
        assert np.all(err[~cl] <= scale / 2)
        assert np.all(err[cl] < scale)
        clamped_blocks += bool(np.any(err[cl] > scale / 2))
        # idempotence: re-quantising the dequantised block is a fixed point
        c2, b2 = q(orc, deq(c, b).astype(np.float32), m)
        if np.abs(c).max() >= 2 ** (m - 2):
            assert b2 == b and np.array_equal(c2, c)
        else:  # the max code rounded down out of the top binade: scale shrinks
            assert np.allclose(deq(c2, b2), deq(c, b))
        # sign symmetry
        c3, b3 = q(orc, -v, m)
        assert b3 == b and np.array_equal(c3, -c)
        # power-of-two equivariance
        j = int(rng.integers(-20, 20))
        c4, b4 = q(orc, (v * np.float32(2.0 ** j)).astype(np.float32), m)
        assert b4 == b + j and np.array_equal(c4, c)
    if m == 4:  # the clamp region is hit by a visible share of N(0,1)/t blocks
        assert 0.01 < clamped_blocks / nblocks < 0.3


@pytest.mark.parametrize("m", [4, 6, 8])
def test_representable_round_trip(orc, m):
    rng = np.random.default_rng(7 * m)
    cmax = 2 ** (m - 1) - 1
    for _ in range(500):
        c = rng.integers(-cmax, cmax + 1, 32)
        c[int(rng.integers(0, 32))] = int(rng.choice([-1, 1])) * int(rng.integers(2 ** (m - 2), cmax + 1))
        s = int(rng.integers(-100, 100))
        v = (c * 2.0 ** s).astype(np.float32)
        cc, b = q(orc, v, m)
        assert b == s + 127 and np.array_equal(cc, c)

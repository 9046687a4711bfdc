"""Pins for the oracle's 3D-RoPE and bf16 rounding (CPU).

Checked against: hand-worked values (tests/golden/rope_hand_examples.txt),
the identity at position 0, a complex-number formulation of the same
rotation, norm preservation and the relative-position identity of rotary
embeddings, and an exact rational implementation of round-to-nearest-even.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import bf16, rope
from wm_synth import to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def exact_rne_bf16(v: float) -> float:
    """RNE of a float64 to bf16 with exact rational arithmetic (independent check)."""
    if v == 0 or math.isinf(v) or math.isnan(v):
        return v
    fv = Fraction(v)
    a = abs(fv)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    # a in [1, 2), value = a * 2**e; bf16: 8 significant bits, min normal 2**-126
    q = Fraction(2) ** (max(e, -126) - 7)
    n = abs(fv) / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    out = fl * q
    if out >= Fraction(2) ** 128:
        return math.copysign(math.inf, v)
    return math.copysign(float(out), v)


def test_rne_against_exact_rationals():
    rng = np.random.default_rng(7)
    vals = list(rng.standard_normal(3000) * np.exp2(rng.integers(-140, 130, 3000)))
    # exact ties between bf16 neighbours, both parities, and boundary cases
    for base in (1.0, 1.0078125, 3.0, 2.0 ** -126, 2.0 ** -133, 2.0 ** 127):
        for frac in (0.5, 1.5, 0.25, 0.75):
            vals.append(base + frac * base * 2.0 ** -7)
    vals += [2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** 128 - 2.0 ** 119, 2.0 ** 128 - 2.0 ** 120,
             -0.0, 0.0, 1e-300, 65504.0, -1.7e38]
    got = bf16.bits_to_f64(bf16.f64_to_bits(np.array(vals)))
    for v, g in zip(vals, got):
        want = exact_rne_bf16(float(v))
        assert (g == want) or (math.isinf(g) and math.isinf(want)), (v, g, want)
        assert math.copysign(1, g) == math.copysign(1, v)


def test_rne_matches_torch_for_float32_inputs():
    """On fp32-representable inputs, direct RNE from fp64 equals PyTorch's fp32->bf16."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))).astype(np.float32)
    assert np.array_equal(bf16.f64_to_bits(x.astype(np.float64)), to_bf16_bits(x))


def read_hand_examples():
    out = []
    with open(os.path.join(GOLDEN, "rope_hand_examples.txt")) as fh:
        for line in fh:
            if line.startswith("#") or not line.strip():
                continue
            cols = [c.strip() for c in line.split("|")]
            case, d, bands, pos, x, y = cols[:6]
            theta = float(cols[6]) if len(cols) > 6 else 10000.0
            out.append((case, int(d), tuple(int(v) for v in bands.split(",")),
                        tuple(int(v) for v in pos.split(",")),
                        [float(v) for v in x.split(",")], [float(v) for v in y.split(",")], theta))
    return out


@pytest.mark.parametrize("ex", read_hand_examples(), ids=lambda e: e[0])
def test_hand_examples(ex):
    _, d, bands, (t, h, w), x, y, theta = ex
    xb = bf16.f64_to_bits(np.array(x)).reshape(1, 1, d)
    yb = rope.rotate(xb, np.array([t]), np.array([h]), np.array([w]), theta=theta, rope_dims=bands)
    assert list(bf16.bits_to_f64(yb).reshape(-1)) == y


def test_rne_is_one_rounding_from_fp64():
    """x just above a bf16 midpoint whose lower neighbour is even, closer to
    it than half an fp32 spacing: rounded once from fp64 it goes up; rounded
    to fp32 first it would land on the midpoint and tie down to even."""
    for e in (-20, -3, 0, 1, 7, 60):
        for k in (128, 130, 200, 254):                     # even 8-bit significands
            q = 2.0 ** (e - 8)                              # bf16 spacing for |x| in [2^(e-1), 2^e)
            x = (k + 0.5 + 2.0 ** -20) * q
            up = bf16.bits_to_f64(bf16.f64_to_bits(np.array([x, -x])))
            assert list(up) == [(k + 1) * q, -(k + 1) * q], (e, k)
            x = (k + 0.5 - 2.0 ** -20) * q
            assert bf16.bits_to_f64(bf16.f64_to_bits(np.array([x])))[0] == k * q, (e, k)


def test_tables_hold_fp32_values():
    """The (cos, sin) tables are libm fp64 values rounded once to fp32: every
    entry is an fp32 number, and it is the fp32 number nearest to libm's."""
    for pos in (0, 1, 7, 1234, 99991):
        for d_a in (2, 20, 44):
            c, s_ = rope.table_row(pos, 10000.0, d_a)
            assert np.array_equal(c.astype(np.float32).astype(np.float64), c)
            assert np.array_equal(s_.astype(np.float32).astype(np.float64), s_)
            j = d_a // 2 - 1
            ang = pos * math.pow(10000.0, -(2.0 * j) / d_a)
            assert c[j] == float(np.float32(math.cos(ang))) and s_[j] == float(np.float32(math.sin(ang)))


def test_default_band_split():
    assert rope.band_sizes(128) == (44, 42, 42)
    assert rope.band_sizes(64) == (24, 20, 20)
    with pytest.raises(ValueError):
        rope.band_sizes(128, (43, 43, 42))


def test_position_zero_is_identity():
    rng = np.random.default_rng(0)
    xb = to_bf16_bits(rng.standard_normal((64, 3, 128)).astype(np.float32))
    xb[xb == 0x8000] = 0                     # the -0 input is the one exception
    zeros = np.zeros(64, dtype=np.int64)
    assert np.array_equal(rope.rotate(xb, zeros, zeros, zeros), xb)


def test_complex_formulation_bit_identical():
    rng = np.random.default_rng(1)
    xb = to_bf16_bits(rng.standard_normal((200, 2, 128)).astype(np.float32))
    t = rng.integers(0, 10_001, 200)
    h = rng.integers(0, 44, 200)
    w = rng.integers(0, 80, 200)
    x = bf16.bits_to_f64(xb)
    y = rope.rotate_f64(x, t, h, w)
    cos, sin = rope.per_token_tables(t, h, w, 128)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * (cos + 1j * sin)[:, None, :]
    assert np.array_equal(z.real, y[..., 0::2])
    assert np.array_equal(z.imag, y[..., 1::2])


def test_norm_preserved_with_fp64_tables():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((50, 2, 128))
    t = rng.integers(0, 10_001, 50)
    h = rng.integers(0, 30, 50)
    w = rng.integers(0, 52, 50)
    y = rope.rotate_f64(x, t, h, w, round_fp32=False)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13, atol=0)


def test_relative_position_identity():
    """<R(p) q, R(p') k> == <q, R(p' - p) k> (fp64 tables)."""
    rng = np.random.default_rng(4)
    d = 128
    for _ in range(20):
        q = rng.standard_normal((1, 1, d))
        k = rng.standard_normal((1, 1, d))
        p = rng.integers(0, 500, 3)
        pp = p + rng.integers(0, 300, 3)
        a = rope.rotate_f64(q, *[np.array([v]) for v in p], round_fp32=False)
        b = rope.rotate_f64(k, *[np.array([v]) for v in pp], round_fp32=False)
        c = rope.rotate_f64(k, *[np.array([v]) for v in (pp - p)], round_fp32=False)
        assert abs(float(np.sum(a * b)) - float(np.sum(q * c))) < 1e-11


def test_bands_rotate_by_their_own_axis():
    """Moving only w leaves the t and h bands untouched, and vice versa."""
    rng = np.random.default_rng(5)
    xb = to_bf16_bits(rng.standard_normal((1, 1, 128)).astype(np.float32))
    base = rope.rotate(xb, np.array([7]), np.array([3]), np.array([5]))
    moved = rope.rotate(xb, np.array([7]), np.array([3]), np.array([9]))
    assert np.array_equal(base[..., :86], moved[..., :86])
    assert not np.array_equal(base[..., 86:], moved[..., 86:])
    moved_t = rope.rotate(xb, np.array([8]), np.array([3]), np.array([5]))
    assert np.array_equal(base[..., 44:], moved_t[..., 44:])
    assert not np.array_equal(base[..., :44], moved_t[..., :44])


def test_token_positions_layout():
    t, h, w = rope.token_positions(2, 3, 4, 10)
    assert list(t) == [10] * 12 + [11] * 12
    assert list(h[:12]) == [0] * 4 + [1] * 4 + [2] * 4
    assert list(w[:5]) == [0, 1, 2, 3, 0]


def test_token_positions_of_views_by_hand():
    """Two frames of 3 views of a 2x3 grid: views share t, each restarts its grid."""
    t, h, w = rope.token_positions(2, 2, 3, 5, n_views=3)
    grid_h = [0, 0, 0, 1, 1, 1]
    grid_w = [0, 1, 2, 0, 1, 2]
    assert list(t) == [5] * 18 + [6] * 18
    assert list(h) == grid_h * 6
    assert list(w) == grid_w * 6


def test_views_rotate_like_separate_single_view_frames():
    """A V-view frame, rotated, equals each view's tokens rotated as a one-view
    frame at the same t: views are independent grids that share the frame's t."""
    rng = np.random.default_rng(7)
    V, fh, fw, H, d = 4, 3, 5, 2, 64
    x = rng.integers(0, 1 << 16, size=(2 * V * fh * fw, H, d), dtype=np.uint32).astype(np.uint16)
    x[(x & 0x7F80) == 0x7F80] = 0x3F80          # no inf/NaN patterns
    got = rope.rotate_frames(x, fh, fw, 123, n_views=V)
    fv = fh * fw
    for f in range(2):
        for v in range(V):
            sl = slice((f * V + v) * fv, (f * V + v + 1) * fv)
            want = rope.rotate_frames(x[sl], fh, fw, 123 + f)
            assert np.array_equal(got[sl], want), (f, v)
    # and not like one tall grid: h of the second view does not continue the first's
    t, h, w = rope.token_positions(1, fh, fw, 0, n_views=V)
    assert h.max() == fh - 1

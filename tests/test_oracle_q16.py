"""Pins of the oracle's 16-bit state (oracle.q16_encode, q16_decode, step_q16).

The format: column d of a state holds int16 mantissas m[:, d] and one
exponent e[d]; the value is m * 2^e[d].  The exponent puts the column's
largest magnitude M at [2^14, 2^15) quanta (one step higher when it would
round up to 2^15), and mantissas are rounded half to even.

The pins do not reuse the oracle's formulas: two columns worked by hand;
states built from mantissas and exponents that satisfy the rule, valued with
exact rationals, must encode back to themselves; the rounding error bound and
the exponent range on random states; the NaN code; and step_q16 against
`forward` over one token (itself pinned by closed forms).  Broken copies of
the encoder (floor rounding, half-away rounding, an exponent one off, one
exponent per state instead of per column, no step-up at the top) must fail
at least one pin.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _exact(m, e):
    """m * 2^e as the nearest float64, through exact rationals."""
    return float(Fraction(int(m)) * (Fraction(2) ** int(e)))


def pin_hand_worked(enc):
    # column 0: M = 16385.5 = 0.50004.. 2^15, so e = 0; ties go to even
    # (16385.5 -> 16386, 16384.5 -> 16384, -2.5 -> -2, 3.5 -> 4, 0.25 -> 0,
    # -0.75 -> -1).
    # column 1: M = (2 - 2^-40) 2^-3 = (1 - 2^-41) 2^-2, so e = -2 - 15 = -17
    # first; M 2^17 = 32768 - 2^-26 would round to 2^15, so e = -16 and the
    # mantissas are 16384 - 2^-27 -> 16384, 2^-4 -> 0, -4096, 0, 0.75 -> 1, 8192.
    S = np.zeros((6, 2))
    S[:, 0] = [16385.5, 16384.5, -2.5, 3.5, 0.25, -0.75]
    S[:, 1] = [(2 - 2.0 ** -40) * 2.0 ** -3, 2.0 ** -20, -2.0 ** -4, 0.0, 3 * 2.0 ** -18, 2.0 ** -3]
    m, e = enc(S)
    np.testing.assert_array_equal(e, [0, -16])
    np.testing.assert_array_equal(m[:, 0], [16386, 16384, -2, 4, 0, -1])
    np.testing.assert_array_equal(m[:, 1], [16384, 0, -4096, 0, 1, 8192])


def pin_representable_round_trip(enc):
    """States whose columns already follow the rule encode to themselves."""
    r = np.random.default_rng(1)
    dk, dv = 96, 12
    m = r.integers(-32767, 32768, size=(dk, dv))
    top = r.integers(16384, 32768, size=dv)                 # the column maxima
    rows = r.integers(0, dk, size=dv)
    m = np.clip(m, -top + 1, top - 1)
    m[rows, np.arange(dv)] = top * r.choice([-1, 1], size=dv)
    m[:, 3] = 0
    m[5, 3] = 16384                                         # exactly 2^14 quanta
    e = r.integers(-60, 40, size=dv)
    e[7] = -130                                             # values down near fp64's normal range edge
    S = np.array([[_exact(m[c, d], e[d]) for d in range(dv)] for c in range(dk)])
    m2, e2 = enc(S)
    np.testing.assert_array_equal(e2, e)
    np.testing.assert_array_equal(m2, m)


def pin_error_bound_and_range(enc):
    r = np.random.default_rng(2)
    S = r.standard_normal((3, 4, 96, 192)) * np.exp(r.uniform(-20, 20, size=(3, 4, 1, 192)))
    S[0, 0, :, 5] = 0.0
    m, e = enc(S)
    assert m.dtype == np.int16 and e.dtype == np.int32
    assert m.shape == S.shape and e.shape == S.shape[:-2] + S.shape[-1:]
    q = np.ldexp(1.0, e)                                    # quantum per column
    M = np.abs(S).max(axis=-2)
    nz = M > 0
    ratio = M[nz] / q[nz]
    assert ratio.min() >= 2 ** 14 and ratio.max() < 32767.5
    assert np.all(np.abs(m) <= 32767)
    err = np.abs(m * q[..., None, :] - S)
    assert np.all(err <= 0.5 * q[..., None, :])
    assert np.all(m[0, 0, :, 5] == 0)


def pin_nan_column(enc):
    S = np.random.default_rng(3).standard_normal((8, 4))
    S[2, 1] = np.nan
    S[5, 3] = -np.inf
    m, e = enc(S)
    assert np.all(m[:, 1] == oracle.Q16_NAN) and np.all(m[:, 3] == oracle.Q16_NAN)
    assert e[1] == 0 and e[3] == 0
    d = oracle.q16_decode(m, e)
    assert np.isnan(d[:, 1]).all() and np.isnan(d[:, 3]).all()
    assert np.all(np.abs(d[:, [0, 2]] - S[:, [0, 2]]) <= 0.5 * np.ldexp(1.0, e[[0, 2]]))


PINS = [pin_hand_worked, pin_representable_round_trip, pin_error_bound_and_range, pin_nan_column]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_q16_encode_pins(pin):
    pin(oracle.q16_encode)


def test_decode_is_exact_scaling():
    m = np.array([[1, -32767], [16384, 0], [-3, 7]], dtype=np.int16)
    e = np.array([-149 + 20, 30], dtype=np.int32)
    d = oracle.q16_decode(m, e)
    want = np.array([[_exact(m[c, j], e[j]) for j in range(2)] for c in range(3)])
    np.testing.assert_array_equal(d, want)


def test_step_q16_reads_the_unrounded_state():
    """o of step_q16 equals one token of `forward` from the decoded state; the
    new state is that forward state rounded (within half a quantum)."""
    r = np.random.default_rng(4)
    N, H, dk, dv = 3, 2, 96, 192
    m0, e0 = oracle.q16_encode(r.standard_normal((N, H, dk, dv)) * 0.3)
    q, k = r.standard_normal((2, N, H, dk)) / np.sqrt(dk)
    v = r.standard_normal((N, H, dv))
    g = np.log(1 / (1 + np.exp(-(r.standard_normal((N, H)) + 4))))
    o, m1, e1 = oracle.step_q16(m0, e0, q, k, v, g)
    S0 = oracle.q16_decode(m0, e0)
    o_ref, S_ref = oracle.forward(q[:, None], k[:, None], v[:, None], g[:, None], S0)
    np.testing.assert_allclose(o, o_ref[:, 0], rtol=1e-13, atol=1e-15)
    quantum = np.ldexp(1.0, e1)[..., None, :]
    assert np.all(np.abs(oracle.q16_decode(m1, e1) - S_ref) <= 0.5 * quantum)
    # gamma = 1, k = v = 0: a representable state is a fixed point
    o2, m2, e2 = oracle.step_q16(m1, e1, q, np.zeros_like(k), np.zeros_like(v), np.zeros_like(g))
    np.testing.assert_array_equal(m2, m1)
    np.testing.assert_array_equal(e2, e1)


def _mutant(kind):
    def enc(S):
        S = np.asarray(S, np.float64)
        finite = np.isfinite(S).all(axis=-2)
        Sf = np.where(np.isfinite(S), S, 0.0)
        if kind == "one_exponent_per_state":
            M = np.broadcast_to(np.abs(Sf).max(axis=(-2, -1))[..., None], finite.shape)
        else:
            M = np.abs(Sf).max(axis=-2)
        _, x = np.frexp(M)
        e = x - {"exponent_low": 16, "exponent_high": 14}.get(kind, 15)
        if kind not in ("no_step_up", "exponent_low"):
            e = e + (np.ldexp(M, -e) >= 32767.5)
        y = np.ldexp(Sf, -e[..., None, :])
        if kind == "floor":
            m = np.floor(y)
        elif kind == "half_away":
            m = np.sign(y) * np.floor(np.abs(y) + 0.5)
        else:
            m = np.rint(y)
        m = np.clip(m, -32768, 32767)
        m = np.where(finite[..., None, :], m, -32768)
        return m.astype(np.int16), np.where(finite, e, 0).astype(np.int32)
    return enc


@pytest.mark.parametrize("kind", ["floor", "half_away", "exponent_low", "exponent_high",
                                  "one_exponent_per_state", "no_step_up"])
def test_pins_catch_planted_encoder_mistakes(kind):
    failures = 0
    for pin in PINS:
        try:
            pin(_mutant(kind))
        except AssertionError:
            failures += 1
    assert failures > 0, f"no pin rejects the '{kind}' mutant"

"""Pins for the fp64 rotary-embedding oracle (oracle/rope.py).

Each ``pin_*`` takes the oracle module and raises AssertionError when its
``rope`` disagrees with a fact that does not come from the oracle itself:
hand-derived closed forms at D = 2, 4 and 8, invariants of a rotation (pair
norms, identity at position 0, composition of angles), the relative-position
property that motivates the embedding (the score between a rotated query at
position m and a rotated key at position n depends on m - n only), and the
complex-number form of the same rotation.  ``tests/test_oracle_mutants.py``
plants mistakes in copies of the oracle and requires each to be caught.

Page short names as in the oracle package docstring; the operation is the one
[ATB-guide] §8.4 configures (base 10000, interleaved pairs).
"""

import math

import numpy as np


def _close(a, b, atol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.abs(a - b)
    assert np.all(err <= atol), f"{what}: max err {err.max()} at {np.argwhere(err > atol)[:3]}"


def _rng(seed):
    return np.random.default_rng(seed)


def pin_rope_position_zero_is_identity(orc):
    """cos 0 = 1, sin 0 = 0: row 0 (and any row given position 0) is unchanged."""
    x = _rng(1).standard_normal((2, 5, 3, 8))
    y = orc.rope(x)
    _close(y[:, 0], x[:, 0], 0.0, "default position of row 0")
    y = orc.rope(x, positions=np.zeros((2, 5), dtype=np.int64))
    _close(y, x, 0.0, "all positions 0")


def pin_rope_preserves_pair_norms(orc):
    """A rotation keeps the length of every (2i, 2i+1) pair."""
    x = _rng(2).standard_normal((2, 9, 2, 16)) * 3.0
    y = orc.rope(x)
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    _close(ny, nx, 1e-12 * max(1.0, nx.max()), "pair norms")


def pin_rope_d2_closed_form(orc):
    """D = 2: theta_0 = base^0 = 1, so the pair turns by exactly p radians.

    Rotating (x, y) by angle p counter-clockwise gives
    (x cos p - y sin p, x sin p + y cos p).
    """
    pos = np.array([[0, 1, 2, 7, 100, 12345]], dtype=np.int64)
    x = np.zeros((1, 6, 1, 2))
    x[..., 0] = 0.75
    x[..., 1] = -1.5
    y = orc.rope(x, positions=pos, base=777.0)
    for s, p in enumerate(pos[0]):
        ex = 0.75 * math.cos(p) - (-1.5) * math.sin(p)
        ey = 0.75 * math.sin(p) + (-1.5) * math.cos(p)
        _close(y[0, s, 0], np.array([ex, ey]), 1e-12, f"D=2 position {p}")


def pin_rope_frequency_closed_forms(orc):
    """D = 4 and D = 8 with unit vectors: the angle of pair i is p * base^(-2i/D).

    Worked by hand: D = 4, base 10000 -> theta_1 = 10000^(-1/2) = 0.01;
    D = 8, base 10000 -> theta_1 = 10000^(-1/4) = 0.1, theta_2 = 0.01,
    theta_3 = 10000^(-3/4) = 0.001.  A unit vector on the even slot of pair i
    lands on (cos a, sin a) in that pair and leaves the other pairs at zero.
    """
    cases = [(4, 1, 0.01), (8, 1, 0.1), (8, 2, 0.01), (8, 3, 0.001), (8, 0, 1.0)]
    for d, i, theta in cases:
        for p in (1, 3, 50, 1000):
            x = np.zeros((1, p + 1, 1, d))
            x[0, p, 0, 2 * i] = 1.0
            y = orc.rope(x)[0, p, 0]
            want = np.zeros(d)
            want[2 * i] = math.cos(p * theta)
            want[2 * i + 1] = math.sin(p * theta)
            _close(y, want, 1e-12, f"D={d} pair {i} position {p}")
            # the odd slot turns the same way: (0, 1) -> (-sin a, cos a)
            x = np.zeros((1, p + 1, 1, d))
            x[0, p, 0, 2 * i + 1] = 1.0
            y = orc.rope(x)[0, p, 0]
            want = np.zeros(d)
            want[2 * i] = -math.sin(p * theta)
            want[2 * i + 1] = math.cos(p * theta)
            _close(y, want, 1e-12, f"D={d} odd slot of pair {i} position {p}")


def pin_rope_composition(orc):
    """Rotations add: rotating by position a, then by b, equals rotating by a + b."""
    rng = _rng(3)
    x = rng.standard_normal((2, 4, 3, 16))
    a = rng.integers(0, 500, size=(2, 4))
    b = rng.integers(0, 500, size=(2, 4))
    _close(orc.rope(orc.rope(x, positions=a), positions=b), orc.rope(x, positions=a + b), 1e-10,
           "composition")


def pin_rope_relative_position(orc):
    """<R(q, m), R(k, n)> depends on m - n only: shifting both positions by c
    leaves every query-key dot product unchanged (and the scores differ from
    the unrotated ones, so the rotation is not the identity)."""
    rng = _rng(4)
    b, s, h, d = 1, 6, 2, 32
    q = rng.standard_normal((b, s, h, d))
    k = rng.standard_normal((b, s, h, d))
    base_pos = np.arange(s)[None, :]
    for c in (1, 17, 4000):
        s0 = np.einsum("bihd,bjhd->bhij", orc.rope(q), orc.rope(k))
        s1 = np.einsum("bihd,bjhd->bhij", orc.rope(q, positions=base_pos + c), orc.rope(k, positions=base_pos + c))
        _close(s1, s0, 1e-9, f"shift {c}")
    raw = np.einsum("bihd,bjhd->bhij", q, k)
    rot = np.einsum("bihd,bjhd->bhij", orc.rope(q), orc.rope(k))
    assert np.abs(rot - raw).max() > 1e-2, "rotation left the scores unchanged"
    # the diagonal (m = n) is unchanged by any rotation applied to both
    _close(np.diagonal(rot, axis1=2, axis2=3), np.diagonal(raw, axis1=2, axis2=3), 1e-10, "m = n")


def pin_rope_complex_form(orc):
    """Each pair as a complex number z = x_2i + j x_2i+1 is multiplied by
    exp(j p theta_i) (Euler's form of the same rotation), with the angles
    built here in Python floats."""
    rng = _rng(5)
    b, s, h, d = 2, 7, 3, 8
    x = rng.standard_normal((b, s, h, d))
    pos = rng.integers(-50, 3000, size=(b, s))
    base = 500.0
    y = orc.rope(x, positions=pos, base=base)
    for bb in range(b):
        for ss in range(s):
            for hh in range(h):
                for i in range(d // 2):
                    a = float(pos[bb, ss]) * base ** (-(2.0 * i) / d)
                    z = complex(x[bb, ss, hh, 2 * i], x[bb, ss, hh, 2 * i + 1]) * complex(math.cos(a), math.sin(a))
                    _close(y[bb, ss, hh, 2 * i:2 * i + 2], np.array([z.real, z.imag]), 1e-11,
                           f"complex form b{bb} s{ss} h{hh} i{i}")


def pin_rope_positions_per_batch(orc):
    """A position array applies per (batch, row) and to every head alike:
    batch 1 with positions shifted by 10 equals rotating the default by 10."""
    rng = _rng(6)
    x = rng.standard_normal((2, 5, 4, 8))
    pos = np.stack([np.arange(5), np.arange(5) + 10])
    y = orc.rope(x, positions=pos)
    _close(y[0], orc.rope(x)[0], 0.0, "batch 0 default positions")
    shifted = orc.rope(orc.rope(x), positions=np.full((2, 5), 10))
    _close(y[1], shifted[1], 1e-10, "batch 1 shifted by 10")
    for hh in range(1, 4):  # identical heads rotate identically
        xh = x.copy()
        xh[:, :, hh] = x[:, :, 0]
        _close(orc.rope(xh, positions=pos)[:, :, hh], y[:, :, 0], 0.0, f"head {hh}")


def pin_rope_default_base(orc):
    """The default base is 10000 ([ATB-guide] §8.4)."""
    x = _rng(7).standard_normal((1, 6, 1, 8))
    _close(orc.rope(x), orc.rope(x, base=10000.0), 0.0, "default base")
    _close(orc.rope_frequencies(8), np.array([1.0, 0.1, 0.01, 0.001]), 1e-15, "frequencies D=8")


ALL_PINS = [
    pin_rope_position_zero_is_identity,
    pin_rope_preserves_pair_norms,
    pin_rope_d2_closed_form,
    pin_rope_frequency_closed_forms,
    pin_rope_composition,
    pin_rope_relative_position,
    pin_rope_complex_form,
    pin_rope_positions_per_batch,
    pin_rope_default_base,
]

"""Rotary position embedding (RoPE) in float64 (the oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the
product path.

What is computed, and where the pages fix it
--------------------------------------------
[ATB-guide] §2.1 lists a RoPE operator that rotates Q and K without building
the rotated tensors explicitly; §4.1's fifth fusion pattern feeds RoPE(Q) and
RoPE(K) straight into the attention; §8.4 configures the operator with a
rotary base of 10000 and the interleaved pairing and checks it against a plain
rotation of each (even, odd) pair of head dimensions by the angle
position × frequency (bar: max error below 1e-3).  [graph-opt] Pattern 1 puts
the same rotation right after the Q/K projections.

Readings taken where the pages leave a step open (each is listed in the design doc):

* pairs are the interleaved dimensions (2i, 2i+1), i = 0 .. D/2-1;
* the frequency of pair i is theta_i = base^(-2i/D), the standard rotary
  frequency that the operator's parameters (base, head size, interleaved)
  describe.  §8.4's reference listing builds its exponent from an index that
  already steps over even numbers and then doubles it (base^(-4i/D)); that is
  read as a slip of the listing, since it would leave the upper half of the
  spectrum unused;
* pair i of a row at position p becomes
      x'_2i   = x_2i   cos(p theta_i) - x_2i+1 sin(p theta_i)
      x'_2i+1 = x_2i+1 cos(p theta_i) + x_2i   sin(p theta_i);
* the position of row s of batch b is positions[b, s] when a position array
  is given, else s;
* Q and K are rotated (every head with the same positions); V is not.

Arrays are (B, S, H, D); inputs are the values the GPU reads, as float64.
"""

import numpy as np

DEFAULT_BASE = 10000.0


def rope_frequencies(d, base=DEFAULT_BASE):
    """theta_i = base^(-2i/D) for i = 0 .. D/2-1 ([ATB-guide] §8.4: base 10000)."""
    if d % 2 != 0:
        raise ValueError("RoPE needs an even head size")
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d)


def rope_positions(b, s, positions=None):
    """(B, S) int64 positions: the given array, else 0 .. S-1 for every batch."""
    if positions is None:
        return np.broadcast_to(np.arange(s, dtype=np.int64), (b, s))
    pos = np.asarray(positions, dtype=np.int64)
    if pos.shape != (b, s):
        raise ValueError(f"positions must be (B, S) = {(b, s)}, got {pos.shape}")
    return pos


def rope(x, positions=None, base=DEFAULT_BASE):
    """Rotate every (2i, 2i+1) pair of x (B, S, H, D) by position x theta_i.

    [ATB-guide] §8.4: cos and sin of the angle, even and odd dimensions paired.
    Returns a new float64 array; x is not modified.
    """
    x = np.asarray(x, dtype=np.float64)
    b, s, h, d = x.shape
    theta = rope_frequencies(d, base)
    pos = rope_positions(b, s, positions).astype(np.float64)
    ang = pos[:, :, None] * theta[None, None, :]          # (B, S, D/2)
    c = np.cos(ang)[:, :, None, :]                         # broadcast over heads
    sn = np.sin(ang)[:, :, None, :]
    even = x[..., 0::2]
    odd = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = even * c - odd * sn
    out[..., 1::2] = odd * c + even * sn
    return out

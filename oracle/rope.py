"""Rotary position embedding for BlockAttention, fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[GEM-MFU, Detailed notes: BlockAttention item]: fixed 64-token blocks are
combined with a fused rotary position embedding.  The pages give no base,
pairing or positions; the reading taken:
  * rotary embedding with base 10000: dimension pair i of a head (i < d/2)
    turns by angle p * base^(-2i/d) at position p;
  * "rotate half" pairing: element i pairs with element i + d/2, i.e.
      x'_i       = x_i cos - x_{i+d/2} sin
      x'_{i+d/2} = x_{i+d/2} cos + x_i sin;
  * Q and K are rotated (V is not), each token at its position counted from
    its sequence's first token.
Block attention on rotated Q and K depends only on q and k positions through
their difference, so positions counted from each block's first token give
the same result (pinned in the tests).

Gradients: the rotation is linear and orthogonal per pair, so
dL/dx = R(p)^T dL/dx', a rotation by -p * theta.
"""

import numpy as np

DEFAULT_BASE = 10000.0


def rope_angles(positions, d, base=DEFAULT_BASE):
    """[n, d/2] angles p * base^(-2i/d) for every position p and pair i."""
    if d % 2:
        raise ValueError("head_dim must be even")
    i = np.arange(d // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / d)
    return np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]


def rope(x, positions, base=DEFAULT_BASE, inverse=False):
    """Rotate x [n, H, d] (fp64) by the angles of `positions` [n]; with
    inverse, by minus those angles (the transpose of the rotation)."""
    x = np.asarray(x, dtype=np.float64)
    n, H, d = x.shape
    ang = rope_angles(positions, d, base)
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    if inverse:
        s = -s
    h = d // 2
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def sequence_positions(offsets):
    """Position of every row within its sequence (offsets [B+1])."""
    off = np.asarray(offsets, dtype=np.int64)
    pos = np.zeros(int(off[-1]), dtype=np.int64)
    for b in range(len(off) - 1):
        pos[off[b]:off[b + 1]] = np.arange(off[b + 1] - off[b])
    return pos

"""Rotary position embedding at logical positions (oracle; test infrastructure only).

mlsanity.com page on WeDLM, "Builds on": RoFormer (rotary position
embedding). hyper.ai summary, "Method": logical position IDs are kept through
the reordering via RoPE, so attention scores reflect true positions rather than
physical indices.

Readings: rotate-half pairing, i.e. dimension j is paired with j + D/2 for
j < D/2, with angular frequency omega_j = theta^(-2j/D) (the form used by the
Qwen backbones the pages name). Queries and keys are rotated; values are not.
"""

import numpy as np


def rope_frequencies(D, theta):
    """omega_j = theta ** (-2 j / D), j = 0 .. D/2 - 1, in float64."""
    if D % 2:
        raise ValueError("head_dim must be even")
    j = np.arange(D // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * j / D)


def rope_rotate(x, positions, theta):
    """Rotate the last axis of x by the RoPE angle of each position.

    Args:
      x: float array [..., D]; the leading axes are broadcast against
         ``positions`` (positions has the shape of x without its last axis,
         or a shape that broadcasts to it).
      positions: integer (or float) logical positions.
      theta: RoPE base.

    Returns float64 [..., D]:
      y_j       = x_j cos(t w_j) - x_{j+D/2} sin(t w_j)
      y_{j+D/2} = x_{j+D/2} cos(t w_j) + x_j sin(t w_j)
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    omega = rope_frequencies(D, theta)
    t = np.asarray(positions, dtype=np.float64)[..., None]
    angle = t * omega
    c = np.cos(angle)
    s = np.sin(angle)
    lo = x[..., :half]
    hi = x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)

"""Oracle: per-sample axial 2D rotary position embedding.

Test infrastructure only (see the package docstring).

The pages name "per-sample 2D rotary embeddings" applied at each token's
native position (rcap.io post, "native-resolution packed step" pseudo-code;
ai.thesatyajit.com explainer, "A backbone that doesn't crop", Figure 5
caption; Mage-Flow paper section 3.2.1 as summarised on paperlayer.ai), but
give no formula.  Reading taken here:

* axial split: dims [0, D/2) rotate by the token's row, dims [D/2, D) by its
  column;
* within each half, adjacent pairs (2j, 2j+1), j < D/4, rotate as the
  original rotary embedding does (RoFormer, Su et al.): a planar rotation by
  angle p * theta^(-2j/(D/2));
* theta = 10000;
* the inverse rotation (angle negated) is the transpose, used to carry
  gradients from rotated Q/K back to the un-rotated inputs.
"""
from __future__ import annotations

import numpy as np


def inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """theta^(-2j/(D/2)) for j < D/4, float64."""
    if head_dim % 4 != 0:
        raise ValueError("head_dim must be a multiple of 4 for axial 2D RoPE")
    half = head_dim // 2
    return np.array([float(theta) ** (-(2.0 * j) / half) for j in range(head_dim // 4)],
                    dtype=np.float64)


def rope2d(x: np.ndarray, pos: np.ndarray, theta: float, inverse: bool = False) -> np.ndarray:
    """Rotate ``x`` [N][H][D] (float64) by per-token positions ``pos`` [N][2]."""
    x = np.asarray(x, dtype=np.float64)
    n, h, d = x.shape
    pos = np.asarray(pos).reshape(n, 2)
    freqs = inv_freq(d, theta)
    half = d // 2
    sign = -1.0 if inverse else 1.0
    out = np.empty_like(x)
    for axis in (0, 1):  # 0: row -> first half, 1: col -> second half
        base = axis * half
        angle = sign * pos[:, axis].astype(np.float64)[:, None] * freqs[None, :]  # [N][D/4]
        cos = np.cos(angle)[:, None, :]
        sin = np.sin(angle)[:, None, :]
        even = x[:, :, base:base + half:2]
        odd = x[:, :, base + 1:base + half:2]
        out[:, :, base:base + half:2] = even * cos - odd * sin
        out[:, :, base + 1:base + half:2] = even * sin + odd * cos
    return out


# ---------------------------------------------------------------------------
# Frame-aware 3D rotary embedding (editing)
# ---------------------------------------------------------------------------
#
# The pages extend the 2D rotary embedding with a frame axis, so that visual
# tokens carry (h, w, f) positions and a source image and its edited target
# differ only in frame while keeping spatial correspondence (Mage-Flow paper
# section 3.2.2 "Conditioning and rectified-flow training", hyper.ai
# summary; paperlayer.ai summary, "Method").  They do not say how the head
# dimension is shared among the three axes.  Reading taken here:
#
# * blocks of the head dimension: [0, 3D/8) rotate by the row, [3D/8, 3D/4)
#   by the column, [3D/4, D) by the frame (48/48/32 of 128, 24/24/16 of 64),
#   so every block is a whole number of 8-element chunks;
# * inside a block of d dims, adjacent pairs (2j, 2j+1), j < d/2, rotate by
#   p * theta^(-2j/d) -- the same rule as the 2D halves, where d = D/2.

def blocks3d(head_dim: int):
    """[(start, size, axis)] of the row, column and frame blocks."""
    if head_dim % 16 != 0:
        raise ValueError("head_dim must be a multiple of 16 for 3D RoPE")
    a = 3 * head_dim // 8
    return [(0, a, 0), (a, a, 1), (2 * a, head_dim - 2 * a, 2)]


def rope3d(x: np.ndarray, pos: np.ndarray, theta: float, inverse: bool = False) -> np.ndarray:
    """Rotate ``x`` [N][H][D] (float64) by per-token positions ``pos`` [N][3] = (row, col, frame)."""
    x = np.asarray(x, dtype=np.float64)
    n, h, d = x.shape
    pos = np.asarray(pos).reshape(n, 3)
    sign = -1.0 if inverse else 1.0
    out = np.empty_like(x)
    for start, size, axis in blocks3d(d):
        freqs = np.array([float(theta) ** (-(2.0 * j) / size) for j in range(size // 2)], dtype=np.float64)
        angle = sign * pos[:, axis].astype(np.float64)[:, None] * freqs[None, :]  # [N][size/2]
        cos = np.cos(angle)[:, None, :]
        sin = np.sin(angle)[:, None, :]
        even = x[:, :, start:start + size:2]
        odd = x[:, :, start + 1:start + size:2]
        out[:, :, start:start + size:2] = even * cos - odd * sin
        out[:, :, start + 1:start + size:2] = even * sin + odd * cos
    return out


def rope_axes(x: np.ndarray, pos: np.ndarray, theta: float, inverse: bool = False) -> np.ndarray:
    """2D or 3D rotation, chosen by the number of position components (2 or 3)."""
    width = np.asarray(pos).shape[-1]
    if width == 2:
        return rope2d(x, pos, theta, inverse)
    if width == 3:
        return rope3d(x, pos, theta, inverse)
    raise ValueError(f"positions must have 2 or 3 components, got {width}")

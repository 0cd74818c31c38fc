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

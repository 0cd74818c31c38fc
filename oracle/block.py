"""Oracle: the attention sub-block's fused operator chains around the packed
joint attention -- adaptive normalisation, the modality-specific QKV
projection with the rotary embedding, and the gated residual update.

Test infrastructure only (see the package docstring).

What the pages say:
* the backbone follows MMDiT: text and image tokens are concatenated for
  joint self-attention, with normalisation and projection layers specific
  to each modality (Mage-Flow paper section 3.2.1 "Model Architecture and
  Native Packing", paperlayer.ai summary; the ai.thesatyajit.com
  explainer's Figure 5 caption likewise shows each modality normalised on
  its own before the shared attention, with the rotary embedding applied
  per sample);
* the training system fuses the memory-bound chains of the transformer
  blocks; on the transformer side the fused chains combine adaptive
  normalisation, rotary embeddings and gated residual updates (paper
  section 3.3 "Training Infrastructure", paperlayer.ai summary).

Readings taken where the pages are silent:
* a token's modality: the first piece of a sample (its text) is text, every
  other piece (the image; for editing the source and the target grids) is
  image.  cu_pieces has frames + 1 pieces per sample (frames = image grids: 1 for
  generation, 2 for editing), as the packers write;
* adaptive normalisation: LayerNorm over the C channels without its own
  affine (population variance, eps = 1e-6, the DiT convention), then
  h = LN(x) (1 + scale) + shift with the sample's vectors for the token's
  modality; shift, scale and gate are inputs of shape [S][2][C] (the
  conditioning network that makes them is outside this path);
* projection: [q | k | v] = h W^T + b with the modality's W [3C][C] and b [3C];
  q, k, v are viewed as [N][H][D] with C = H D; q and k are rotated by the
  token's position exactly as the attention path rotates them, v is not;
* gated residual: y = x + gate (o W_o^T + b_o) with the modality's W_o [C][C],
  b_o [C] and the sample's gate for that modality.

The backward functions give the gradient of a scalar loss with respect to
every input of each chain from the gradient of its output (weights and
biases summed over the rows of their modality, modulation vectors over the
rows of their sample and modality).
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from .rope import rope_axes


def row_groups(cu_pieces: Sequence[int], n_samples: int, frames: int):
    """[(first_row, end_row, sample, modality)] for every piece (modality 0 = text, 1 = image)."""
    per = frames + 1
    cp = [int(c) for c in cu_pieces]
    out = []
    for s in range(n_samples):
        for p in range(per):
            out.append((cp[per * s + p], cp[per * s + p + 1], s, 0 if p == 0 else 1))
    return out


def layer_norm(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) over the last axis, population variance, float64."""
    x = np.asarray(x, dtype=np.float64)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps)


def adaln_modulate(x: np.ndarray, shift: np.ndarray, scale: np.ndarray, cu_pieces: Sequence[int],
                   n_samples: int, frames: int, eps: float = 1e-6) -> np.ndarray:
    """h [N][C] float64: LN(x) (1 + scale[s][m]) + shift[s][m] per token of sample s, modality m."""
    x = np.asarray(x, dtype=np.float64)
    shift = np.asarray(shift, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    h = np.zeros_like(x)
    for a, b, s, m in row_groups(cu_pieces, n_samples, frames):
        h[a:b] = layer_norm(x[a:b], eps) * (1.0 + scale[s, m]) + shift[s, m]
    return h


def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray]) -> np.ndarray:
    """x W^T + b in float64 (W is [out][in])."""
    y = np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T
    if b is not None:
        y = y + np.asarray(b, dtype=np.float64)
    return y


def qkv_rope(h: np.ndarray, w: Tuple[np.ndarray, np.ndarray], b: Tuple[Optional[np.ndarray], Optional[np.ndarray]],
             cu_pieces: Sequence[int], n_samples: int, frames: int, pos: Optional[np.ndarray], n_heads: int,
             head_dim: int, theta: float = 10000.0):
    """(q, k, v), each [N][H][D] float64: the modality's projection of h, q and k rotated by pos
    ([N][2] or [N][3]; None = no rotation)."""
    h = np.asarray(h, dtype=np.float64)
    n, c = h.shape
    if c != n_heads * head_dim:
        raise ValueError("channels must equal heads x head_dim")
    qkv = np.zeros((n, 3 * c), dtype=np.float64)
    for a, e, s, m in row_groups(cu_pieces, n_samples, frames):
        qkv[a:e] = linear(h[a:e], w[m], b[m])
    q = qkv[:, :c].reshape(n, n_heads, head_dim)
    k = qkv[:, c:2 * c].reshape(n, n_heads, head_dim)
    v = qkv[:, 2 * c:].reshape(n, n_heads, head_dim)
    if pos is not None:
        q = rope_axes(q, pos, theta)
        k = rope_axes(k, pos, theta)
    return q, k, v


def out_gated_residual(o: np.ndarray, x: np.ndarray, w: Tuple[np.ndarray, np.ndarray],
                       b: Tuple[Optional[np.ndarray], Optional[np.ndarray]], gate: np.ndarray,
                       cu_pieces: Sequence[int], n_samples: int, frames: int) -> np.ndarray:
    """y [N][C] float64: x + gate[s][m] (o W_o^T + b_o) with the modality's output projection."""
    o = np.asarray(o, dtype=np.float64).reshape(np.asarray(x).shape[0], -1)
    x = np.asarray(x, dtype=np.float64)
    gate = np.asarray(gate, dtype=np.float64)
    y = x.copy()
    for a, e, s, m in row_groups(cu_pieces, n_samples, frames):
        y[a:e] = x[a:e] + gate[s, m] * linear(o[a:e], w[m], b[m])
    return y


# ---------------------------------------------------------------------------
# Backward of the chains (gradients of a scalar loss with respect to every
# input, given the gradient of the chain's output).  The rotation is
# orthogonal, so its gradient is the inverse rotation.
# ---------------------------------------------------------------------------

def adaln_modulate_bwd(dh: np.ndarray, x: np.ndarray, shift: np.ndarray, scale: np.ndarray,
                       cu_pieces: Sequence[int], n_samples: int, frames: int, eps: float = 1e-6):
    """(dx [N][C], dshift [S][2][C], dscale [S][2][C]) for h = LN(x) (1 + scale[s][m]) + shift[s][m]."""
    dh = np.asarray(dh, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    dx = np.zeros_like(x)
    dshift = np.zeros(np.shape(shift), dtype=np.float64)
    dscale = np.zeros(np.shape(scale), dtype=np.float64)
    for a, b, s, m in row_groups(cu_pieces, n_samples, frames):
        if b == a:
            continue
        xs = x[a:b]
        mean = xs.mean(axis=-1, keepdims=True)
        var = ((xs - mean) ** 2).mean(axis=-1, keepdims=True)
        rstd = 1.0 / np.sqrt(var + eps)
        xhat = (xs - mean) * rstd
        g = dh[a:b]
        dshift[s, m] += g.sum(axis=0)
        dscale[s, m] += (g * xhat).sum(axis=0)
        dxhat = g * (1.0 + scale[s, m])
        dx[a:b] = rstd * (dxhat - dxhat.mean(axis=-1, keepdims=True)
                          - xhat * (dxhat * xhat).mean(axis=-1, keepdims=True))
    return dx, dshift, dscale


def qkv_rope_bwd(dq: np.ndarray, dk: np.ndarray, dv: np.ndarray, h: np.ndarray,
                 w: Tuple[np.ndarray, np.ndarray], cu_pieces: Sequence[int], n_samples: int, frames: int,
                 pos: Optional[np.ndarray], theta: float = 10000.0):
    """(dh [N][C], (dW_text, dW_image) [3C][C], (db_text, db_image) [3C]) given the gradients of the rotated
    q, k and of v ([N][H][D] each).  The output features may also be a subset of heads (w then holds their rows):
    dW and db of those rows come out exact, dh does not."""
    h = np.asarray(h, dtype=np.float64)
    n, c = h.shape
    dq = np.asarray(dq, dtype=np.float64)
    dk = np.asarray(dk, dtype=np.float64)
    if pos is not None:
        dq = rope_axes(dq, pos, theta, inverse=True)
        dk = rope_axes(dk, pos, theta, inverse=True)
    g = np.concatenate([dq.reshape(n, -1), dk.reshape(n, -1), np.asarray(dv, dtype=np.float64).reshape(n, -1)],
                       axis=1)
    f = g.shape[1]  # 3 C for the block's projection; any width for a slice of its output features
    dh = np.zeros_like(h)
    dw = [np.zeros((f, c)), np.zeros((f, c))]
    db = [np.zeros(f), np.zeros(f)]
    for a, e, s, m in row_groups(cu_pieces, n_samples, frames):
        dh[a:e] = g[a:e] @ np.asarray(w[m], dtype=np.float64)
        dw[m] += g[a:e].T @ h[a:e]
        db[m] += g[a:e].sum(axis=0)
    return dh, tuple(dw), tuple(db)


def out_gated_residual_bwd(dy: np.ndarray, o: np.ndarray, x: np.ndarray, w: Tuple[np.ndarray, np.ndarray],
                           b: Tuple[Optional[np.ndarray], Optional[np.ndarray]], gate: np.ndarray,
                           cu_pieces: Sequence[int], n_samples: int, frames: int):
    """(dx, do [N][C], (dW_text, dW_image) [C][C], (db_text, db_image) [C], dgate [S][2][C]) for
    y = x + gate[s][m] (o W_m^T + b_m)."""
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64).reshape(x.shape[0], -1)
    gate = np.asarray(gate, dtype=np.float64)
    c = x.shape[1]
    do = np.zeros_like(o)
    dw = [np.zeros((c, o.shape[1])), np.zeros((c, o.shape[1]))]
    db = [np.zeros(c), np.zeros(c)]
    dgate = np.zeros_like(gate)
    for a, e, s, m in row_groups(cu_pieces, n_samples, frames):
        u = gate[s, m] * dy[a:e]
        proj = linear(o[a:e], w[m], b[m])
        do[a:e] = u @ np.asarray(w[m], dtype=np.float64)
        dw[m] += u.T @ o[a:e]
        db[m] += u.sum(axis=0)
        dgate[s, m] += (dy[a:e] * proj).sum(axis=0)
    return dy.copy(), do, tuple(dw), tuple(db), dgate

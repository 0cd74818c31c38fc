"""Oracle: block-diagonal multi-head attention over a packed stream.

Test infrastructure only (see the package docstring).

The pages (Mage-Flow paper section 3.2.1 "Model Architecture and Native
Packing", paperlayer.ai summary; ai.thesatyajit.com explainer, Figure 5
caption; rcap.io post, "native-resolution packed step") state that the text
and image tokens of one sample attend jointly, that samples are packed into
one stream and run through variable-length attention kernels, and that packed
CFG branches do not change the result.  Packed attention is therefore exactly
per-segment dense softmax attention, and that definition is what this module
evaluates, one (segment, head) at a time, in float64.

Readings taken where the pages are silent:
* attention is non-causal inside a segment and absent across segments;
* RoPE (``oracle.rope``) is applied to Q and K before the scores; V is not
  rotated.  Positions with two components (row, col) take the 2D rotation,
  positions with three (row, col, frame) the frame-aware 3D rotation;
* softmax scale defaults to 1/sqrt(head_dim);
* LSE is the natural log of the row's sum of exp(scaled scores), laid out
  [H][N];
* the backward takes dO and returns gradients with respect to the
  un-rotated Q and K (the rotation's transpose applied to the rotated-space
  gradients) and to V.  It recomputes its own O from Q, K, V.

Query rows are processed in chunks (default 1024) only to bound memory; each
chunk still takes the full softmax over all keys of its segment.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

from .rope import rope_axes


def _segments(cu_seqlens: Sequence[int]):
    cu = [int(c) for c in cu_seqlens]
    for s in range(len(cu) - 1):
        yield s, cu[s], cu[s + 1]


def _rotated(x: np.ndarray, pos: Optional[np.ndarray], theta: float) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    if pos is None:
        return x
    return rope_axes(x, pos, theta)


def _scale(head_dim: int, scale: Optional[float]) -> float:
    return 1.0 / np.sqrt(head_dim) if scale is None or scale == 0 else float(scale)


def attn_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens: Sequence[int],
             pos: Optional[np.ndarray], theta: float = 10000.0,
             scale: Optional[float] = None, chunk: int = 1024) -> Tuple[np.ndarray, np.ndarray]:
    """O [N][H][D] and LSE [H][N] (float64) for packed segments ``cu_seqlens``.

    Tokens outside [0, cu_seqlens[-1]) are left at zero (O) and NaN (LSE).
    """
    v = np.asarray(v, dtype=np.float64)
    n, h_count, d = v.shape
    sc = _scale(d, scale)
    qr = _rotated(q, pos, theta)
    kr = _rotated(k, pos, theta)
    out = np.zeros((n, h_count, d), dtype=np.float64)
    lse = np.full((h_count, n), np.nan, dtype=np.float64)
    for _, a, b in _segments(cu_seqlens):
        if b <= a:
            continue
        for h in range(h_count):
            kk = kr[a:b, h, :]
            vv = v[a:b, h, :]
            for c0 in range(a, b, chunk):
                c1 = min(b, c0 + chunk)
                s = sc * (qr[c0:c1, h, :] @ kk.T)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                denom = e.sum(axis=1, keepdims=True)
                out[c0:c1, h, :] = (e / denom) @ vv
                lse[h, c0:c1] = (m + np.log(denom))[:, 0]
    return out, lse


def attn_fwd_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_seqlens: Sequence[int],
                  pos: Optional[np.ndarray], rows: Iterable[Tuple[int, int]],
                  theta: float = 10000.0, scale: Optional[float] = None):
    """O row and LSE for selected (token, head) pairs only.

    Returns (o [len(rows)][D], lse [len(rows)]) float64, in the order given.
    Each pair is evaluated with the same definition as :func:`attn_fwd`,
    against every key of the token's segment.
    """
    rows = [(int(t), int(h)) for t, h in rows]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    d = np.asarray(v).shape[2]
    sc = _scale(d, scale)
    o_out = np.zeros((len(rows), d), dtype=np.float64)
    l_out = np.zeros(len(rows), dtype=np.float64)
    groups = {}
    for i, (t, h) in enumerate(rows):
        s = int(np.searchsorted(cu, t, side="right") - 1)
        if s < 0 or s >= len(cu) - 1 or t >= cu[s + 1]:
            raise ValueError(f"token {t} is not inside a packed segment")
        groups.setdefault((s, h), []).append(i)
    for (s, h), idx in groups.items():
        a, b = int(cu[s]), int(cu[s + 1])
        pslice = None if pos is None else np.asarray(pos)[a:b]
        kk = _rotated(np.asarray(k)[a:b, h:h + 1, :], pslice, theta)[:, 0, :]
        vv = np.asarray(v, dtype=np.float64)[a:b, h, :]
        toks = [rows[i][0] for i in idx]
        qsel = np.asarray(q, dtype=np.float64)[toks, h:h + 1, :]
        psel = None if pos is None else np.asarray(pos)[toks]
        qq = _rotated(qsel, psel, theta)[:, 0, :]
        sco = sc * (qq @ kk.T)
        m = sco.max(axis=1, keepdims=True)
        e = np.exp(sco - m)
        denom = e.sum(axis=1, keepdims=True)
        o_out[idx] = (e / denom) @ vv
        l_out[idx] = (m + np.log(denom))[:, 0]
    return o_out, l_out


def attn_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray,
             cu_seqlens: Sequence[int], pos: Optional[np.ndarray], theta: float = 10000.0,
             scale: Optional[float] = None, chunk: int = 1024):
    """dQ, dK, dV [N][H][D] (float64) of loss = sum(dO * O) for packed segments.

    Per (segment, head), with P the row softmax of S = scale * Qr Kr^T:
      O = P V, Delta = rowsum(dO * O), dV = P^T dO, dP = dO V^T,
      dS = P * (dP - Delta), dQr = scale * dS Kr, dKr = scale * dS^T Qr,
    then dQ, dK are dQr, dKr rotated back by the inverse rotation.
    """
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    n, h_count, d = v.shape
    sc = _scale(d, scale)
    qr = _rotated(q, pos, theta)
    kr = _rotated(k, pos, theta)
    dqr = np.zeros_like(v)
    dkr = np.zeros_like(v)
    dv = np.zeros_like(v)
    for _, a, b in _segments(cu_seqlens):
        if b <= a:
            continue
        for h in range(h_count):
            kk = kr[a:b, h, :]
            vv = v[a:b, h, :]
            for c0 in range(a, b, chunk):
                c1 = min(b, c0 + chunk)
                qq = qr[c0:c1, h, :]
                dd = do[c0:c1, h, :]
                s = sc * (qq @ kk.T)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                p = e / e.sum(axis=1, keepdims=True)
                o = p @ vv
                delta = (dd * o).sum(axis=1, keepdims=True)
                dv[a:b, h, :] += p.T @ dd
                dp = dd @ vv.T
                ds = p * (dp - delta)
                dqr[c0:c1, h, :] = sc * (ds @ kk)
                dkr[a:b, h, :] += sc * (ds.T @ qq)
    if pos is None:
        return dqr, dkr, dv
    return rope_axes(dqr, pos, theta, inverse=True), rope_axes(dkr, pos, theta, inverse=True), dv


def attn_bwd_given(q: np.ndarray, k: np.ndarray, v: np.ndarray, o: np.ndarray, lse: np.ndarray,
                   dout: np.ndarray, cu_seqlens: Sequence[int], pos: Optional[np.ndarray],
                   theta: float = 10000.0, scale: Optional[float] = None, chunk: int = 1024):
    """dQ, dK, dV [N][H][D] (float64) of the backward step taken as a function
    of given forward outputs: O [N][H][D] and LSE [H][N] are inputs, as in the
    training shape of the workloads (Q, K, V, O, LSE and dO given).

    Per (segment, head): P = exp(scale * Qr Kr^T - LSE) row by row,
    Delta = rowsum(dO * O) from the given O, dV = P^T dO, dP = dO V^T,
    dS = P * (dP - Delta), dQr = scale * dS Kr, dKr = scale * dS^T Qr; dQ and
    dK are then rotated back.  With the exact O and LSE of ``attn_fwd`` this is
    ``attn_bwd``; with rounded O and LSE it is the exact gradient step on those
    rounded values, which separates a backward's own rounding error from the
    rounding its inputs already carry.
    """
    v = np.asarray(v, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    n, h_count, d = v.shape
    sc = _scale(d, scale)
    qr = _rotated(q, pos, theta)
    kr = _rotated(k, pos, theta)
    dqr = np.zeros_like(v)
    dkr = np.zeros_like(v)
    dv = np.zeros_like(v)
    for _, a, b in _segments(cu_seqlens):
        if b <= a:
            continue
        for h in range(h_count):
            kk = kr[a:b, h, :]
            vv = v[a:b, h, :]
            for c0 in range(a, b, chunk):
                c1 = min(b, c0 + chunk)
                qq = qr[c0:c1, h, :]
                dd = do[c0:c1, h, :]
                p = np.exp(sc * (qq @ kk.T) - lse[h, c0:c1, None])
                delta = (dd * o[c0:c1, h, :]).sum(axis=1, keepdims=True)
                dv[a:b, h, :] += p.T @ dd
                ds = p * (dd @ vv.T - delta)
                dqr[c0:c1, h, :] = sc * (ds @ kk)
                dkr[a:b, h, :] += sc * (ds.T @ qq)
    if pos is None:
        return dqr, dkr, dv
    return rope_axes(dqr, pos, theta, inverse=True), rope_axes(dkr, pos, theta, inverse=True), dv

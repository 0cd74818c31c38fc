"""Oracle: rectified-flow noising, target and loss over a packed stream, and
the packed classifier-free-guidance combine.

Test infrastructure only (see the package docstring).

What the pages say:
* training uses the rectified flow-matching objective: the squared L2 distance
  between the model's velocity v(z_t, t) and the target z - eps, where
  z_t = (1 - t) z + t eps and eps ~ N(0, I) (Mage-Flow paper section 3.2.1 as
  summarised on paperlayer.ai, "Method"; rcap.io post, the pseudo-code's
  `loss = mse(v_pred, (z - noise))`);
* for editing the loss is taken on the target tokens only; the source image's
  latents are conditioning (paper section 3.2.2 "Conditioning and
  rectified-flow training", hyper.ai summary);
* packed CFG runs each prompt's conditional and unconditional branches as two
  segments of one forward pass (paper section 3.2.1; hyper.ai summary,
  "Experiment") -- the pages give no combine formula.

Readings taken where the pages are silent:
* latents live in the packed layout [N][C] (one row per packed token; text
  rows carry no latent and are ignored);
* noised rows: the image rows of a generation sample (cu_pieces with two
  entries per sample), the target rows of an editing sample (three entries
  per sample: start, source start, target start); one timestep t per sample;
  rows that are not noised keep z (the source image stays clean);
* loss: per sample, the sum over its noised rows and channels of
  (v - (z - eps))^2; the batch loss the pseudo-code's `mse` names is the mean
  over all noised elements of the pack, i.e. sum / M, and its gradient with
  respect to v is 2 (v - (z - eps)) / M on noised rows and 0 elsewhere; the
  caller passes the scale (2 / M) because it knows M;
* CFG combine: the usual classifier-free guidance form (Ho and Salimans,
  "Classifier-Free Diffusion Guidance"): guided = v_u + s (v_c - v_u) over
  the image rows of each (cond, uncond) pair of consecutive samples, written
  to the cond sample's image rows; the two grids must have the same number of
  tokens.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np


def noised_ranges(cu_pieces: Sequence[int], n_samples: int, frames: int):
    """[(sample, first_row, end_row)] of the rows the flow objective covers."""
    per = frames + 1
    cp = [int(c) for c in cu_pieces]
    out = []
    for s in range(n_samples):
        start = cp[per * s + frames]          # image start (generation) or target start (editing)
        end = cp[per * (s + 1)]               # next sample's start (or N)
        out.append((s, start, end))
    return out


def rf_noise(z: np.ndarray, eps: np.ndarray, t: Sequence[float], cu_pieces: Sequence[int],
             n_samples: int, frames: int) -> np.ndarray:
    """z_t [N][C] (float64): (1 - t_s) z + t_s eps on sample s's noised rows, z elsewhere."""
    z = np.asarray(z, dtype=np.float64)
    eps = np.asarray(eps, dtype=np.float64)
    zt = z.copy()
    for s, a, b in noised_ranges(cu_pieces, n_samples, frames):
        ts = float(t[s])
        zt[a:b] = (1.0 - ts) * z[a:b] + ts * eps[a:b]
    return zt


def rf_loss(v: np.ndarray, z: np.ndarray, eps: np.ndarray, cu_pieces: Sequence[int], n_samples: int,
            frames: int, grad_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """(loss_sum [S], grad [N][C]) in float64: per-sample sums of (v - (z - eps))^2 over noised rows,
    and grad_scale * (v - (z - eps)) on noised rows, 0 elsewhere."""
    v = np.asarray(v, dtype=np.float64)
    target = np.asarray(z, dtype=np.float64) - np.asarray(eps, dtype=np.float64)
    loss = np.zeros(n_samples, dtype=np.float64)
    grad = np.zeros_like(v)
    for s, a, b in noised_ranges(cu_pieces, n_samples, frames):
        r = v[a:b] - target[a:b]
        loss[s] = float(np.sum(r * r))
        grad[a:b] = grad_scale * r
    return loss, grad


def cfg_combine(v: np.ndarray, cu_pieces: Sequence[int], n_pairs: int, scale: float) -> np.ndarray:
    """Copy of v (float64) whose cond image rows hold v_u + scale (v_c - v_u); pairs are
    samples (2p, 2p + 1) of a generation pack (two cu_pieces entries per sample)."""
    v = np.asarray(v, dtype=np.float64)
    out = v.copy()
    cp = [int(c) for c in cu_pieces]
    for p in range(n_pairs):
        c, u = 2 * p, 2 * p + 1
        ca, cb = cp[2 * c + 1], cp[2 * c + 2]
        ua, ub = cp[2 * u + 1], cp[2 * u + 2]
        if cb - ca != ub - ua:
            raise ValueError(f"pair {p}: cond and uncond images differ in size")
        out[ca:cb] = v[ua:ub] + scale * (v[ca:cb] - v[ua:ub])
    return out

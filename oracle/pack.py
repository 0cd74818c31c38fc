"""Oracle: native-resolution packing (offsets, positions, row gather).

Test infrastructure only (see the package docstring).

What the pages say (Mage-Flow paper section 3.2.1 "Model Architecture and
Native Packing", paperlayer.ai summary; rcap.io post, "native-resolution
packed step" pseudo-code; hyper.ai summary, "Method"): each image latent is
flattened into a variable-length token sequence and packed together with
variable-length text into one contiguous batch under a fixed token budget,
without text padding and keeping each image's native latent grid; text and
image tokens of a sample attend jointly.

Readings taken where the pages are silent:
* budget policy: the longest order-preserving prefix of the samples whose
  total length fits the budget; nothing is reordered, split or skipped;
* order inside a sample: the sample's text tokens, then its image tokens, as
  one contiguous joint segment;
* flatten order: row-major over the (grid_h rows, grid_w cols) latent grid;
* positions: text token u of a sample sits at (row, col) = (u, u); image token
  (r, c) sits at (text_len + r, text_len + c).
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np


def _lengths(samples: Sequence[Tuple[int, int, int]]) -> List[int]:
    out = []
    for (t, gh, gw) in samples:
        t, gh, gw = int(t), int(gh), int(gw)
        if t < 0 or gh < 0 or gw < 0:
            raise ValueError(f"negative sample descriptor {(t, gh, gw)}")
        out.append(t + gh * gw)
    return out


def pack(samples: Sequence[Tuple[int, int, int]], budget: int) -> Dict[str, object]:
    """Pack the longest prefix of ``samples`` that fits ``budget`` tokens.

    Returns a dict with
      n_packed    number of samples packed (segments),
      n_tokens    total packed tokens N,
      cu_seqlens  int32 [n_packed + 1], segment start offsets and N,
      cu_pieces   int32 [2 n_packed + 1], alternating segment start and
                  text/image boundary, ending with N,
      max_seqlen  longest packed segment (0 when nothing is packed),
      max_pos     1 + largest position coordinate (0 when nothing is packed).
    """
    lengths = _lengths(samples)
    n = 0
    total = 0
    for length in lengths:
        if total + length > budget:
            break
        total += length
        n += 1
    cu = [0]
    pieces = []
    for i in range(n):
        pieces.append(cu[i])
        pieces.append(cu[i] + int(samples[i][0]))
        cu.append(cu[i] + lengths[i])
    pieces.append(cu[n])
    max_pos = 0
    for i in range(n):
        t, gh, gw = (int(v) for v in samples[i])
        if t > 0:
            max_pos = max(max_pos, t)          # text positions 0..t-1
        if gh > 0 and gw > 0:
            max_pos = max(max_pos, t + max(gh, gw))  # image positions up to t+max-1
    return {
        "n_packed": n,
        "n_tokens": cu[n],
        "cu_seqlens": np.array(cu, dtype=np.int32),
        "cu_pieces": np.array(pieces, dtype=np.int32),
        "max_seqlen": max(lengths[:n], default=0),
        "max_pos": max_pos,
    }


def positions(samples: Sequence[Tuple[int, int, int]], n_packed: int) -> np.ndarray:
    """Per-token (row, col) of the first ``n_packed`` samples; int32 [N][2]."""
    rows = []
    for i in range(n_packed):
        t, gh, gw = (int(v) for v in samples[i])
        for u in range(t):
            rows.append((u, u))
        for r in range(gh):
            for c in range(gw):
                rows.append((t + r, t + c))
    return np.array(rows, dtype=np.int32).reshape(-1, 2)


def gather(text_rows: Sequence[np.ndarray], image_rows: Sequence[np.ndarray],
           n_packed: int) -> np.ndarray:
    """Concatenate each packed sample's text rows then its flattened image rows.

    ``text_rows[i]`` has shape [T_i, C]; ``image_rows[i]`` has shape
    [grid_h, grid_w, C] (or already [grid_h * grid_w, C]); rows are copied bit
    for bit.
    """
    parts = []
    for i in range(n_packed):
        t = np.asarray(text_rows[i])
        im = np.asarray(image_rows[i])
        parts.append(t.reshape(-1, t.shape[-1]))
        parts.append(im.reshape(-1, im.shape[-1]))
    if not parts:
        return np.zeros((0, 0), dtype=np.uint8)
    return np.concatenate(parts, axis=0)


# ---------------------------------------------------------------------------
# Editing samples: [text | source image | target image]
# ---------------------------------------------------------------------------
#
# For editing, the conditioning tokens are followed by the source image's
# latents and then the noisy target latents (Mage-Flow paper section 3.2.2
# "Conditioning and rectified-flow training", hyper.ai summary), and the
# visual tokens carry (h, w, f) positions whose frame tells source from
# target while the spatial positions correspond (same section).  Readings
# taken where the pages are silent:
# * one editing sample is one joint segment [text | source | target]; source
#   and target share the sample's latent grid (an edit keeps the image size);
# * positions (row, col, frame): text token u -> (u, u, u); source token
#   (r, c) -> (T + r, T + c, T); target token (r, c) -> (T + r, T + c, T + 1),
#   i.e. the 2D convention with the frame axis starting after the text too;
# * the budget policy is the same longest order-preserving prefix.

def _edit_lengths(samples: Sequence[Tuple[int, int, int]]) -> List[int]:
    return [t + 2 * (l - t) for t, l in zip((int(s[0]) for s in samples), _lengths(samples))]


def pack_edit(samples: Sequence[Tuple[int, int, int]], budget: int) -> Dict[str, object]:
    """Pack the longest prefix of editing ``samples`` (text_len, grid_h, grid_w) that fits ``budget``.

    Same fields as :func:`pack`, except
      cu_pieces   int32 [3 n_packed + 1]: per sample its start, the end of its
                  text and the end of its source image; then N;
      max_pos     1 + largest position coordinate over all three axes.
    """
    lengths = _edit_lengths(samples)
    n = 0
    total = 0
    for length in lengths:
        if total + length > budget:
            break
        total += length
        n += 1
    cu = [0]
    pieces = []
    max_pos = 0
    for i in range(n):
        t, gh, gw = (int(v) for v in samples[i])
        pieces += [cu[i], cu[i] + t, cu[i] + t + gh * gw]
        cu.append(cu[i] + lengths[i])
        if t > 0:
            max_pos = max(max_pos, t)                        # text positions 0..t-1
        if gh > 0 and gw > 0:
            max_pos = max(max_pos, t + max(gh, gw), t + 2)   # rows/cols up to t+max-1, frames t, t+1
    pieces.append(cu[n])
    return {
        "n_packed": n,
        "n_tokens": cu[n],
        "cu_seqlens": np.array(cu, dtype=np.int32),
        "cu_pieces": np.array(pieces, dtype=np.int32),
        "max_seqlen": max(lengths[:n], default=0),
        "max_pos": max_pos,
    }


def positions_edit(samples: Sequence[Tuple[int, int, int]], n_packed: int) -> np.ndarray:
    """Per-token (row, col, frame) of the first ``n_packed`` editing samples; int32 [N][3]."""
    rows = []
    for i in range(n_packed):
        t, gh, gw = (int(v) for v in samples[i])
        for u in range(t):
            rows.append((u, u, u))
        for f in (0, 1):  # source, then target
            for r in range(gh):
                for c in range(gw):
                    rows.append((t + r, t + c, t + f))
    return np.array(rows, dtype=np.int32).reshape(-1, 3)


def gather_edit(text_rows: Sequence[np.ndarray], source_rows: Sequence[np.ndarray],
                target_rows: Sequence[np.ndarray], n_packed: int) -> np.ndarray:
    """Concatenate each packed sample's text, source-image and target-image rows, bit for bit."""
    parts = []
    for i in range(n_packed):
        for a in (text_rows[i], source_rows[i], target_rows[i]):
            a = np.asarray(a)
            parts.append(a.reshape(-1, a.shape[-1]))
    if not parts:
        return np.zeros((0, 0), dtype=np.uint8)
    return np.concatenate(parts, axis=0)

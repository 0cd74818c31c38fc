"""Seeded synthetic inputs for packed 2D-RoPE varlen attention.

This module is shared by the oracle-side tests, the GPU parity tests and the
benchmark.  It only draws shapes and values: it holds none of the method's
arithmetic (no packing, no positions, no rotation, no attention).  The token
budget cut, the offsets and the positions are computed by whichever side
consumes the drawn sample descriptors.

Workload shapes follow what the Mage-Flow pages describe for native-resolution
training and packed-CFG inference:

* latents are 16x downsampled with the 2x2 patchify internalised, so an
  H x W image becomes an (H/16) x (W/16) token grid (Mage-Flow paper
  section 3.1, Mage-VAE, as summarised on paperlayer.ai);
* image sides run from 512 to 2048 with aspect ratios out to 4:1 in both
  orientations (paper section 3.2.1 "Model Architecture and Native Packing";
  czaidata model card, "Native resolution" highlight);
* packs are built under a 50 000-token budget (rcap.io post, the
  "native-resolution packed step" pseudo-code);
* classifier-free guidance packs each prompt's conditional and unconditional
  branch as separate samples of one pass (paper section 3.2.1; hyper.ai
  summary, "Experiment").

Every random draw uses ``numpy.random.default_rng`` (PCG64) seeded with a
``[seed, stream]`` pair, one stream per tensor, so each tensor is reproducible
on its own.  Normal draws are made in float32 and rounded to bfloat16 with
round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

# Stream tags for default_rng([seed, tag]).
STREAM_SHAPES = 0
STREAM_Q = 1
STREAM_K = 2
STREAM_V = 3
STREAM_DO = 4
# attention sub-block chains (adaptive norm, projections, gated residual)
STREAM_X = 20
STREAM_MOD = 21      # + 0 shift, + 1 scale, + 2 gate
STREAM_WQKV = 24     # + modality (0 text, 1 image)
STREAM_BQKV = 26     # + modality
STREAM_WO = 28       # + modality
STREAM_BO = 30       # + modality
STREAM_O = 32
STREAM_GRAD = 33    # + 0 dy / dh, + 1 dq, + 2 dk, + 3 dv

Sample = Tuple[int, int, int]  # (text_len, grid_h, grid_w)


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: sample descriptors plus tensor geometry.

    ``samples`` is the ordered candidate list handed to the packer; the packer
    keeps the longest prefix that fits ``budget``.
    """

    name: str
    samples: Tuple[Sample, ...]
    budget: int
    n_heads: int
    head_dim: int
    dtype: str  # "bf16" or "f32"
    seed: int
    theta: float = 10000.0
    backward: bool = False
    notes: str = ""
    editing: bool = False  # samples are [text | source | target] (two frames of one grid)


# ----------------------------------------------------------------------------
# bfloat16 helpers (value encoding only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# Sample descriptors
# ----------------------------------------------------------------------------

def tiny() -> Workload:
    """2 samples: text 7 + 4x6 grid, text 5 + 3x3 grid; 1 head, head_dim 64, fp32."""
    return Workload("tiny", ((7, 4, 6), (5, 3, 3)), budget=64, n_heads=1,
                    head_dim=64, dtype="f32", seed=1,
                    notes="2 joint segments of 31 and 14 tokens")


def cfg1024(seed: int = 2) -> Workload:
    """Packed-CFG inference at 1024^2: 4 prompts x {cond, uncond}.

    Each branch carries a 64x64 latent grid (1024/16).  The conditional text
    length is uniform in [64, 512]; the unconditional text is one token.
    Order: cond_0, uncond_0, cond_1, uncond_1, ...
    """
    rng = np.random.default_rng([seed, STREAM_SHAPES])
    samples: List[Sample] = []
    for _ in range(4):
        t = int(rng.integers(64, 513))
        samples.append((t, 64, 64))
        samples.append((1, 64, 64))
    return Workload("cfg1024", tuple(samples), budget=1 << 20, n_heads=24,
                    head_dim=128, dtype="bf16", seed=seed)


IMAGE_SIDES = tuple(range(512, 2048 + 1, 64))  # 25 sides, 512..2048


def mixed50k(seed: int = 3, n_candidates: int = 64, backward: bool = False) -> Workload:
    """Mixed native-resolution training pack under a 50 000-token budget.

    Candidates draw height and width independently from 512..2048 step 64
    (so aspect ratios span 1:1 to 4:1 in both orientations) and a text prefix
    uniform in [32, 512].  The packer keeps the longest prefix that fits.
    64 candidates always overflow the budget: the smallest candidate holds
    32 + 32*32 = 1056 tokens.
    """
    rng = np.random.default_rng([seed, STREAM_SHAPES])
    samples: List[Sample] = []
    for _ in range(n_candidates):
        h = IMAGE_SIDES[int(rng.integers(0, len(IMAGE_SIDES)))]
        w = IMAGE_SIDES[int(rng.integers(0, len(IMAGE_SIDES)))]
        t = int(rng.integers(32, 513))
        samples.append((t, h // 16, w // 16))
    return Workload("mixed50k_bwd" if backward else "mixed50k", tuple(samples),
                    budget=50_000, n_heads=24, head_dim=128, dtype="bf16",
                    seed=seed, backward=backward)


def edit50k(seed: int = 6, n_candidates: int = 32) -> Workload:
    """Editing training pack under a 50 000-token budget.

    Each candidate is an instruction (text uniform in [32, 512]) with a
    source image and its edited target on the same latent grid, height and
    width drawn independently from 512..2048 step 64 as in mixed50k; a
    sample holds text + 2 * grid tokens.  The packer keeps the longest prefix
    that fits.
    """
    rng = np.random.default_rng([seed, STREAM_SHAPES])
    samples: List[Sample] = []
    for _ in range(n_candidates):
        h = IMAGE_SIDES[int(rng.integers(0, len(IMAGE_SIDES)))]
        w = IMAGE_SIDES[int(rng.integers(0, len(IMAGE_SIDES)))]
        t = int(rng.integers(32, 513))
        samples.append((t, h // 16, w // 16))
    return Workload("edit50k", tuple(samples), budget=50_000, n_heads=24, head_dim=128, dtype="bf16",
                    seed=seed, editing=True)


def stress() -> Workload:
    """Long/ragged pack: a 2048^2 image, two 4:1 panoramas and 64 thumbnails.

    Grids are rows x cols: 2048x512 (height x width) is 128 rows x 32 cols.
    """
    samples: List[Sample] = [(512, 128, 128), (256, 128, 32), (256, 32, 128)]
    samples += [(16, 8, 8)] * 64
    return Workload("stress", tuple(samples), budget=1 << 20, n_heads=24,
                    head_dim=128, dtype="bf16", seed=4)


def captions(seed: int = 8, n: int = 1500) -> Workload:
    """A pack of short text segments only (the prompts of a training batch as
    the text side sees them): 1500 captions of 16-120 tokens, ~100k tokens.
    Tiny segments hold all of its work, the case for multi-segment tiles."""
    rng = np.random.default_rng([seed, STREAM_SHAPES])
    samples: List[Sample] = [(int(rng.integers(16, 121)), 0, 0) for _ in range(n)]
    return Workload("captions", tuple(samples), budget=1 << 20, n_heads=24, head_dim=128, dtype="bf16", seed=seed)


def all_workloads() -> List[Workload]:
    return [tiny(), cfg1024(), mixed50k(), stress(), mixed50k(backward=True)]


def random_samples(rng: np.random.Generator, n: int, max_text: int = 40,
                   max_side: int = 12, allow_empty: bool = True) -> List[Sample]:
    """Small random descriptors for parity tests (ragged, including empties)."""
    lo = 0 if allow_empty else 1
    out = []
    for _ in range(n):
        t = int(rng.integers(lo, max_text + 1))
        gh = int(rng.integers(0, max_side + 1))
        gw = int(rng.integers(0, max_side + 1))
        out.append((t, gh, gw))
    return out


# ----------------------------------------------------------------------------
# Tensor values
# ----------------------------------------------------------------------------

def normal(seed: int, stream: int, shape: Sequence[int], dtype: str,
           scale: float = 1.0) -> np.ndarray:
    """N(0, scale^2) draws of ``shape``.

    dtype "bf16" returns uint16 bfloat16 bit patterns (RNE from float32);
    dtype "f32" returns float32 values.
    """
    rng = np.random.default_rng([seed, stream])
    x = rng.standard_normal(size=tuple(int(s) for s in shape), dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of values produced by :func:`normal`."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def qkv(seed: int, n_tokens: int, n_heads: int, head_dim: int, dtype: str):
    shape = (n_tokens, n_heads, head_dim)
    return (normal(seed, STREAM_Q, shape, dtype),
            normal(seed, STREAM_K, shape, dtype),
            normal(seed, STREAM_V, shape, dtype))


def dout(seed: int, n_tokens: int, n_heads: int, head_dim: int, dtype: str):
    return normal(seed, STREAM_DO, (n_tokens, n_heads, head_dim), dtype)


def block_inputs(seed: int, n_tokens: int, n_samples: int, channels: int, dtype: str = "bf16"):
    """Seeded inputs of the attention sub-block chains.

    x [N][C] residual stream and o [N][C] attention output ~ N(0, 1);
    shift, scale, gate [S][2][C] float32 ~ N(0, 0.1^2) (modality 0 text,
    1 image); per modality W_qkv [3C][C] and W_o [C][C] ~ N(0, 1/C) (unit-
    variance outputs), biases b_qkv [3C] and b_o [C] float32 ~ N(0, 0.02^2).
    Matrices are bf16 bit patterns for dtype "bf16".
    """
    c = int(channels)
    w_scale = 1.0 / np.sqrt(c)
    out = {
        "x": normal(seed, STREAM_X, (n_tokens, c), dtype),
        "o": normal(seed, STREAM_O, (n_tokens, c), dtype),
        "shift": normal(seed, STREAM_MOD, (n_samples, 2, c), "f32", 0.1),
        "scale": normal(seed, STREAM_MOD + 1, (n_samples, 2, c), "f32", 0.1),
        "gate": normal(seed, STREAM_MOD + 2, (n_samples, 2, c), "f32", 0.1),
    }
    for m in range(2):
        out[f"w_qkv{m}"] = normal(seed, STREAM_WQKV + m, (3 * c, c), dtype, w_scale)
        out[f"b_qkv{m}"] = normal(seed, STREAM_BQKV + m, (3 * c,), "f32", 0.02)
        out[f"w_o{m}"] = normal(seed, STREAM_WO + m, (c, c), dtype, w_scale)
        out[f"b_o{m}"] = normal(seed, STREAM_BO + m, (c,), "f32", 0.02)
    return out


def block_grads(seed: int, n_tokens: int, channels: int, dtype: str = "bf16"):
    """Seeded output gradients for the sub-block chains' backward: dy (of the
    gated residual, also used as dh of the adaptive norm) and dq, dk, dv (of
    the QKV projection), each [N][C] ~ N(0, 1)."""
    c = int(channels)
    return {name: normal(seed, STREAM_GRAD + i, (n_tokens, c), dtype)
            for i, name in enumerate(("dy", "dq", "dk", "dv"))}


"""Pins of oracle.block (adaptive normalisation, QKV projection with the rotary
embedding, gated residual) against brute force, a library routine and closed
forms -- independent of the oracle's own vectorised code."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import block

EPS = 1e-6


def _ln_row_python(row, eps=EPS):
    n = len(row)
    mean = math.fsum(row) / n
    var = math.fsum((v - mean) ** 2 for v in row) / n
    return [(v - mean) / math.sqrt(var + eps) for v in row]


def test_layer_norm_matches_pure_python():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 24)) * 3.0 + 1.5
    got = block.layer_norm(x)
    for r in range(5):
        np.testing.assert_allclose(got[r], _ln_row_python(list(x[r])), rtol=0, atol=1e-13)


def test_layer_norm_matches_torch_float64():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((7, 64)) * 0.5 - 2.0
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (64,), eps=EPS).numpy()
    np.testing.assert_allclose(block.layer_norm(x), ref, rtol=0, atol=1e-12)


def test_layer_norm_closed_forms():
    # a constant row has zero variance: every output is 0
    np.testing.assert_array_equal(block.layer_norm(np.full((1, 16), 3.25)), np.zeros((1, 16)))
    # population variance: outputs have mean 0 and mean square var / (var + eps)
    rng = np.random.default_rng(13)
    x = rng.standard_normal((3, 32)) * 0.01  # small variance makes eps visible
    y = block.layer_norm(x)
    var = x.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose((y * y).mean(axis=1), var / (var + EPS), rtol=1e-12)


def test_row_groups_hand_typed_generation_and_editing():
    # generation (one image grid per sample): sample 0 = text 3 + image 4, sample 1 = text 2 + image 5
    assert block.row_groups([0, 3, 7, 9, 14], 2, 1) == [(0, 3, 0, 0), (3, 7, 0, 1), (7, 9, 1, 0), (9, 14, 1, 1)]
    # editing (two grids per sample): one sample = text 2, source 4, target 4; source and target are image rows
    assert block.row_groups([0, 2, 6, 10], 1, 2) == [(0, 2, 0, 0), (2, 6, 0, 1), (6, 10, 0, 1)]


@pytest.mark.parametrize("frames,cu", [(1, [0, 3, 7, 9, 14]), (2, [0, 2, 6, 10, 11, 14, 17])])
def test_adaln_modulate_brute_force(frames, cu):
    rng = np.random.default_rng(14 + frames)
    n_samples = (len(cu) - 1) // (frames + 1)
    n, c = cu[-1], 8
    x = rng.standard_normal((n, c))
    shift = rng.standard_normal((n_samples, 2, c))
    scale = rng.standard_normal((n_samples, 2, c))
    got = block.adaln_modulate(x, shift, scale, cu, n_samples, frames)
    per = frames + 1
    for t in range(n):
        piece = max(i for i in range(len(cu) - 1) if cu[i] <= t)
        s, m = piece // per, (0 if piece % per == 0 else 1)
        ln = _ln_row_python(list(x[t]))
        want = [ln[j] * (1.0 + scale[s, m, j]) + shift[s, m, j] for j in range(c)]
        np.testing.assert_allclose(got[t], want, rtol=0, atol=1e-12)


def test_adaln_zero_modulation_is_layer_norm():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((14, 16))
    z = np.zeros((2, 2, 16))
    np.testing.assert_array_equal(block.adaln_modulate(x, z, z, [0, 3, 7, 9, 14], 2, 1), block.layer_norm(x))


def test_linear_triple_loop():
    rng = np.random.default_rng(16)
    x, w, b = rng.standard_normal((3, 5)), rng.standard_normal((4, 5)), rng.standard_normal(4)
    got = block.linear(x, w, b)
    for i in range(3):
        for o in range(4):
            assert abs(got[i, o] - (math.fsum(x[i, k] * w[o, k] for k in range(5)) + b[o])) < 1e-12


def _tiny_layout():
    # two generation samples: text 3 + image 2x2, text 2 + image 1x5
    cu = [0, 3, 7, 9, 14]
    pos = np.array([[0, 0], [1, 1], [2, 2], [3, 3], [3, 4], [4, 3], [4, 4],
                    [0, 0], [1, 1], [2, 2], [2, 3], [2, 4], [2, 5], [2, 6]])
    return cu, pos


def test_qkv_rope_identity_weights_reduce_to_rotation():
    # W = [I; 2I; 3I] for text, [2I; 4I; 6I] for image: q = rope(h W_q^T), k = rope(h W_k^T), v = h W_v^T
    cu, pos = _tiny_layout()
    heads, d = 2, 8
    c = heads * d
    rng = np.random.default_rng(17)
    h = rng.standard_normal((14, c))
    eye = np.eye(c)
    w = (np.vstack([eye, 2 * eye, 3 * eye]), np.vstack([2 * eye, 4 * eye, 6 * eye]))
    q, k, v = block.qkv_rope(h, w, (None, None), cu, 2, 1, pos, heads, d)
    mult = np.array([1, 1, 1, 2, 2, 2, 2, 1, 1, 2, 2, 2, 2, 2], dtype=np.float64)[:, None]  # 1 text, 2 image
    hv = (h * mult).reshape(14, heads, d)
    np.testing.assert_allclose(q, oracle.rope2d(hv, pos, 10000.0), rtol=0, atol=1e-13)
    np.testing.assert_allclose(k, oracle.rope2d(2 * hv, pos, 10000.0), rtol=0, atol=1e-13)
    np.testing.assert_allclose(v, 3 * hv, rtol=0, atol=1e-13)


def test_qkv_rope_bias_and_no_rotation_brute_force():
    cu, _ = _tiny_layout()
    heads, d = 1, 4
    c = heads * d
    rng = np.random.default_rng(18)
    h = rng.standard_normal((14, c))
    w = (rng.standard_normal((3 * c, c)), rng.standard_normal((3 * c, c)))
    b = (rng.standard_normal(3 * c), None)
    q, k, v = block.qkv_rope(h, w, b, cu, 2, 1, None, heads, d)
    text = {0, 1, 2, 7, 8}
    for t in range(14):
        m = 0 if t in text else 1
        full = [math.fsum(h[t, j] * w[m][o, j] for j in range(c)) + (b[m][o] if b[m] is not None else 0.0)
                for o in range(3 * c)]
        np.testing.assert_allclose(np.concatenate([q[t, 0], k[t, 0], v[t, 0]]), full, rtol=0, atol=1e-12)


def test_qkv_rope_relative_position():
    # with W_q = W_k = I the per-head score q_i . k_j depends only on pos_j - pos_i: shifting every
    # position by the same 2D offset leaves all scores unchanged
    cu, pos = _tiny_layout()
    heads, d = 2, 8
    c = heads * d
    rng = np.random.default_rng(19)
    h = rng.standard_normal((14, c))
    eye = np.eye(c)
    w = (np.vstack([eye, eye, eye]),) * 2
    q0, k0, _ = block.qkv_rope(h, w, (None, None), cu, 2, 1, pos, heads, d)
    q1, k1, _ = block.qkv_rope(h, w, (None, None), cu, 2, 1, pos + np.array([5, 9]), heads, d)
    s0 = np.einsum("ihd,jhd->hij", q0, k0)
    s1 = np.einsum("ihd,jhd->hij", q1, k1)
    np.testing.assert_allclose(s0, s1, rtol=0, atol=1e-11)


def test_out_gated_residual_closed_forms_and_brute_force():
    cu, _ = _tiny_layout()
    c = 6
    rng = np.random.default_rng(20)
    o, x = rng.standard_normal((14, c)), rng.standard_normal((14, c))
    w = (rng.standard_normal((c, c)), rng.standard_normal((c, c)))
    b = (rng.standard_normal(c), rng.standard_normal(c))
    gate = rng.standard_normal((2, 2, c))
    # gate 0: the residual stream passes unchanged
    np.testing.assert_array_equal(block.out_gated_residual(o, x, w, b, np.zeros((2, 2, c)), cu, 2, 1), x)
    # identity projection, no bias, gate 1: y = x + o
    eye = (np.eye(c), np.eye(c))
    np.testing.assert_allclose(block.out_gated_residual(o, x, eye, (None, None), np.ones((2, 2, c)), cu, 2, 1),
                               x + o, rtol=0, atol=1e-15)
    got = block.out_gated_residual(o, x, w, b, gate, cu, 2, 1)
    text = {0, 1, 2, 7, 8}
    for t in range(14):
        m, s = (0 if t in text else 1), (0 if t < 7 else 1)
        for j in range(c):
            proj = math.fsum(o[t, i] * w[m][j, i] for i in range(c)) + b[m][j]
            assert abs(got[t, j] - (x[t, j] + gate[s, m, j] * proj)) < 1e-12

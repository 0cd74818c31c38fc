"""Pins for oracle.rope: closed forms and invariants of axial 2D rotary embedding.

A dropped term, a flipped sign, the wrong half for an axis, rotate-half
pairing instead of adjacent pairs, or a wrong frequency exponent each fail at
least one test here (the unit-vector tests fix all of them by value).
"""
import cmath
import math

import numpy as np
import pytest

import oracle

THETA = 10000.0


def _unit(d, i):
    x = np.zeros((1, 1, d))
    x[0, 0, i] = 1.0
    return x


@pytest.mark.parametrize("d", [64, 128])
def test_pair0_rotates_by_position_in_radians(d):
    row, col = 3, 5
    pos = np.array([[row, col]])
    y = oracle.rope2d(_unit(d, 0), pos, THETA)[0, 0]
    expect = np.zeros(d)
    expect[0], expect[1] = math.cos(3.0), math.sin(3.0)
    assert np.allclose(y, expect, atol=1e-15)
    # second half, pair 0: rotated by the column, in radians
    y = oracle.rope2d(_unit(d, d // 2 + 1), pos, THETA)[0, 0]
    expect = np.zeros(d)
    expect[d // 2], expect[d // 2 + 1] = -math.sin(5.0), math.cos(5.0)
    assert np.allclose(y, expect, atol=1e-15)


def test_frequencies_by_value_d64():
    # D = 64: per-axis half of 32 dims, 16 pairs; pair j turns at 10000^(-j/16).
    row, col = 7, 11
    pos = np.array([[row, col]])
    for j in (1, 5, 15):
        freq = 10.0 ** (-4.0 * j / 16.0)
        y = oracle.rope2d(_unit(64, 2 * j), pos, THETA)[0, 0]
        assert y[2 * j] == pytest.approx(math.cos(row * freq), abs=1e-14)
        assert y[2 * j + 1] == pytest.approx(math.sin(row * freq), abs=1e-14)
        assert np.count_nonzero(np.abs(y) > 1e-15) <= 2
        y = oracle.rope2d(_unit(64, 32 + 2 * j), pos, THETA)[0, 0]
        assert y[32 + 2 * j] == pytest.approx(math.cos(col * freq), abs=1e-14)
        assert y[32 + 2 * j + 1] == pytest.approx(math.sin(col * freq), abs=1e-14)


def test_inv_freq_values():
    f = oracle.inv_freq(128, THETA)
    assert f.shape == (32,)
    assert f[0] == 1.0
    assert f[16] == pytest.approx(0.01, rel=1e-14)       # 10000^(-32/64)
    assert f[31] == pytest.approx(10000.0 ** (-62 / 64), rel=1e-14)


def test_origin_is_identity_and_norm_preserved():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 3, 128))
    pos = rng.integers(0, 640, size=(50, 2))
    pos[0] = (0, 0)
    y = oracle.rope2d(x, pos, THETA)
    assert np.array_equal(y[0], x[0])
    assert np.allclose(np.linalg.norm(y, axis=2), np.linalg.norm(x, axis=2), rtol=1e-13)


def test_inverse_undoes_forward():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((40, 2, 64))
    pos = rng.integers(0, 640, size=(40, 2))
    y = oracle.rope2d(oracle.rope2d(x, pos, THETA), pos, THETA, inverse=True)
    assert np.allclose(y, x, atol=1e-12)


@pytest.mark.parametrize("d", [64, 128])
def test_scores_depend_only_on_2d_offset(d):
    rng = np.random.default_rng(2)
    q = rng.standard_normal((30, 1, d))
    k = rng.standard_normal((30, 1, d))
    pq = rng.integers(0, 300, size=(30, 2))
    pk = rng.integers(0, 300, size=(30, 2))
    base = np.einsum("nd,nd->n", oracle.rope2d(q, pq, THETA)[:, 0], oracle.rope2d(k, pk, THETA)[:, 0])
    for _ in range(3):
        delta = rng.integers(-200, 300, size=(1, 2))
        shifted = np.einsum("nd,nd->n", oracle.rope2d(q, pq + delta, THETA)[:, 0],
                            oracle.rope2d(k, pk + delta, THETA)[:, 0])
        assert np.allclose(shifted, base, atol=1e-10)
    # and a change of offset does change them
    other = np.einsum("nd,nd->n", oracle.rope2d(q, pq + [[1, 0]], THETA)[:, 0],
                      oracle.rope2d(k, pk, THETA)[:, 0])
    assert not np.allclose(other, base, atol=1e-3)


def test_text_tokens_match_1d_rope_in_complex_form():
    # A text token sits at (p, p): each half is the 1-D rotary embedding,
    # i.e. complex multiplication of (x_2j + i x_2j+1) by exp(i p f_j).
    rng = np.random.default_rng(3)
    d = 64
    x = rng.standard_normal((5, 1, d))
    p = np.array([0, 1, 9, 200, 511])
    y = oracle.rope2d(x, np.stack([p, p], axis=1), THETA)
    for n in range(5):
        for half in (0, 1):
            for j in range(d // 4):
                f = THETA ** (-2.0 * j / (d / 2))
                z = complex(x[n, 0, half * 32 + 2 * j], x[n, 0, half * 32 + 2 * j + 1])
                w = z * cmath.exp(1j * p[n] * f)
                assert y[n, 0, half * 32 + 2 * j] == pytest.approx(w.real, abs=1e-12)
                assert y[n, 0, half * 32 + 2 * j + 1] == pytest.approx(w.imag, abs=1e-12)


def test_heads_share_the_rotation():
    rng = np.random.default_rng(4)
    x1 = rng.standard_normal((6, 1, 64))
    x = np.concatenate([x1, 2 * x1, -x1], axis=1)
    pos = rng.integers(0, 100, size=(6, 2))
    y = oracle.rope2d(x, pos, THETA)
    y1 = oracle.rope2d(x1, pos, THETA)
    assert np.allclose(y[:, 0], y1[:, 0]) and np.allclose(y[:, 1], 2 * y1[:, 0]) and np.allclose(y[:, 2], -y1[:, 0])

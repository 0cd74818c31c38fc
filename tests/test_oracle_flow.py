"""Pins for oracle.flow: rectified-flow noising, target and loss over a packed
stream, and the packed-CFG combine.

A swapped (1 - t) / t, a target of eps - z instead of z - eps, a loss taken on
the wrong rows (text rows, editing source rows), a missing factor 2 or a
wrong scale in the gradient, or swapped cond/uncond in the combine each fail
at least one test here.
"""
import numpy as np
import pytest

import oracle
from oracle import flow

GEN = [(3, 2, 2), (0, 1, 3), (5, 0, 0), (2, 3, 1)]   # generation samples
EDIT = [(2, 1, 2), (0, 2, 1), (4, 1, 1)]             # editing samples


def _gen_case(seed=0, c=8):
    p = oracle.pack(GEN, 1 << 20)
    rng = np.random.default_rng(seed)
    n = p["n_tokens"]
    z, eps, v = (rng.standard_normal((n, c)) for _ in range(3))
    return p, z, eps, v


def test_noised_ranges_by_hand():
    # generation: cu_pieces [0,3, 7,7, 10,15, 15,17, 20]; image rows per sample
    p = oracle.pack(GEN, 1 << 20)
    assert p["cu_pieces"].tolist() == [0, 3, 7, 7, 10, 15, 15, 17, 20]
    assert flow.noised_ranges(p["cu_pieces"], 4, 1) == [(0, 3, 7), (1, 7, 10), (2, 15, 15), (3, 17, 20)]
    # editing: [start, source start, target start] per sample; only target rows
    e = oracle.pack_edit(EDIT, 1 << 20)
    assert e["cu_pieces"].tolist() == [0, 2, 4, 6, 6, 8, 10, 14, 15, 16]
    assert flow.noised_ranges(e["cu_pieces"], 3, 2) == [(0, 4, 6), (1, 8, 10), (2, 15, 16)]


def test_noise_closed_forms():
    p, z, eps, _ = _gen_case()
    cp = p["cu_pieces"]
    assert np.array_equal(flow.rf_noise(z, eps, [0.0] * 4, cp, 4, 1), z)
    zt1 = flow.rf_noise(z, eps, [1.0] * 4, cp, 4, 1)
    for s, a, b in flow.noised_ranges(cp, 4, 1):
        assert np.array_equal(zt1[a:b], eps[a:b])
    zt = flow.rf_noise(z, eps, [0.25, 0.5, 0.75, 1.0], cp, 4, 1)
    assert np.allclose(zt[3:7], 0.75 * z[3:7] + 0.25 * eps[3:7])
    assert np.allclose(zt[7:10], 0.5 * z[7:10] + 0.5 * eps[7:10])
    # text rows keep z
    for a, b in ((0, 3), (10, 15), (15, 17)):
        assert np.array_equal(zt[a:b], z[a:b])


def test_editing_source_rows_stay_clean():
    e = oracle.pack_edit(EDIT, 1 << 20)
    n = e["n_tokens"]
    rng = np.random.default_rng(1)
    z, eps = rng.standard_normal((n, 4)), rng.standard_normal((n, 4))
    zt = flow.rf_noise(z, eps, [0.5, 0.5, 0.5], e["cu_pieces"], 3, 2)
    noised = np.zeros(n, dtype=bool)
    for _, a, b in flow.noised_ranges(e["cu_pieces"], 3, 2):
        noised[a:b] = True
    assert np.array_equal(zt[~noised], z[~noised])
    assert np.allclose(zt[noised], 0.5 * (z[noised] + eps[noised]))


def test_target_is_minus_velocity_of_the_noise_path():
    # z_t moves from z (t = 0) to eps (t = 1) with constant speed eps - z;
    # the regression target z - eps is minus that derivative
    p, z, eps, _ = _gen_case(2)
    cp = p["cu_pieces"]
    h = 1e-3
    d = (flow.rf_noise(z, eps, [0.3 + h] * 4, cp, 4, 1) - flow.rf_noise(z, eps, [0.3] * 4, cp, 4, 1)) / h
    zero_v = np.zeros_like(z)
    _, g = flow.rf_loss(zero_v, z, eps, cp, 4, 1, grad_scale=1.0)   # g = 0 - (z - eps) on noised rows
    for _, a, b in flow.noised_ranges(cp, 4, 1):
        assert np.allclose(d[a:b], g[a:b], atol=1e-9)


def test_loss_closed_forms():
    p, z, eps, _ = _gen_case(3)
    cp = p["cu_pieces"]
    loss, grad = flow.rf_loss(z - eps, z, eps, cp, 4, 1, grad_scale=0.5)
    assert np.array_equal(loss, np.zeros(4)) and not grad.any()
    loss, grad = flow.rf_loss(z - eps + 0.5, z, eps, cp, 4, 1, grad_scale=2.0)
    rows = [4, 3, 0, 3]
    assert np.allclose(loss, [0.25 * r * 8 for r in rows])
    for _, a, b in flow.noised_ranges(cp, 4, 1):
        assert np.allclose(grad[a:b], 1.0)
    assert not grad[0:3].any() and not grad[10:17].any()


def test_gradient_of_pack_mean_matches_finite_differences():
    p, z, eps, v = _gen_case(4)
    cp = p["cu_pieces"]
    m = sum(b - a for _, a, b in flow.noised_ranges(cp, 4, 1)) * z.shape[1]

    def mean_loss(vv):
        return float(flow.rf_loss(vv, z, eps, cp, 4, 1, 1.0)[0].sum()) / m

    _, grad = flow.rf_loss(v, z, eps, cp, 4, 1, grad_scale=2.0 / m)
    rng = np.random.default_rng(5)
    direction = rng.standard_normal(v.shape)
    h = 1e-6
    fd = (mean_loss(v + h * direction) - mean_loss(v - h * direction)) / (2 * h)
    assert float(np.sum(grad * direction)) == pytest.approx(fd, rel=1e-7)


def test_cfg_combine():
    samples = [(4, 2, 3), (1, 2, 3), (2, 1, 2), (1, 1, 2)]   # [c0, u0, c1, u1]
    p = oracle.pack(samples, 1 << 20)
    cp = p["cu_pieces"]
    rng = np.random.default_rng(6)
    v = rng.standard_normal((p["n_tokens"], 5))
    c0, u0 = slice(4, 10), slice(11, 17)
    assert np.allclose(flow.cfg_combine(v, cp, 2, 1.0), v, atol=1e-15, rtol=0)
    out0 = flow.cfg_combine(v, cp, 2, 0.0)
    assert np.array_equal(out0[c0], v[u0])
    out2 = flow.cfg_combine(v, cp, 2, 2.0)
    assert np.allclose(out2[c0], 2 * v[c0] - v[u0])
    c1, u1 = slice(19, 21), slice(22, 24)
    assert np.allclose(out2[c1], 2 * v[c1] - v[u1])
    # uncond and text rows are untouched
    keep = np.ones(p["n_tokens"], dtype=bool)
    keep[c0] = keep[c1] = False
    assert np.array_equal(out2[keep], v[keep])
    with pytest.raises(ValueError):
        bad = oracle.pack([(1, 2, 2), (1, 2, 3)], 1 << 20)
        flow.cfg_combine(np.zeros((bad["n_tokens"], 2)), bad["cu_pieces"], 1, 2.0)

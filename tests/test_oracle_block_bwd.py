"""Pins of the block chains' backward in oracle.block: every gradient against
central finite differences (h = 1e-6, float64) of the scalar loss
sum(dy * output) on small inputs, and closed forms.  The finite differences
call only the forward functions, so a wrong term, sign, index or operand in
a gradient formula fails here."""
import numpy as np
import pytest

from oracle import block

CU = [0, 3, 7, 9, 14]  # generation: sample 0 = text 3 + image 4, sample 1 = text 2 + image 5
POS = np.array([[0, 0], [1, 1], [2, 2], [3, 3], [3, 4], [4, 3], [4, 4],
                [0, 0], [1, 1], [2, 2], [2, 3], [2, 4], [2, 5], [2, 6]])


def _fd(f, arr, h=1e-6):
    """Central-difference gradient of the scalar f() with respect to every element of arr (in place)."""
    g = np.zeros_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = arr[i]
        arr[i] = old + h
        fp = f()
        arr[i] = old - h
        fm = f()
        arr[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


def _close(a, b, tol=2e-6):
    scale = max(1.0, float(np.abs(b).max()))
    assert np.abs(a - b).max() <= tol * scale, float(np.abs(a - b).max())


@pytest.mark.parametrize("frames,cu", [(1, CU), (2, [0, 2, 6, 10, 11, 14, 17])])
def test_adaln_bwd_finite_differences(frames, cu):
    rng = np.random.default_rng(40 + frames)
    s = (len(cu) - 1) // (frames + 1)
    n, c = cu[-1], 8
    x = rng.standard_normal((n, c))
    shift = rng.standard_normal((s, 2, c))
    scale = rng.standard_normal((s, 2, c))
    dy = rng.standard_normal((n, c))
    loss = lambda: float(np.sum(dy * block.adaln_modulate(x, shift, scale, cu, s, frames)))  # noqa: E731
    dx, dsh, dsc = block.adaln_modulate_bwd(dy, x, shift, scale, cu, s, frames)
    _close(dx, _fd(loss, x))
    _close(dsh, _fd(loss, shift))
    _close(dsc, _fd(loss, scale))


def test_adaln_bwd_closed_forms():
    rng = np.random.default_rng(43)
    x = rng.standard_normal((14, 8))
    z = np.zeros((2, 2, 8))
    # LN is invariant to shifting its input row: a gradient constant along a row is removed exactly
    dy_const = np.repeat(rng.standard_normal((14, 1)), 8, axis=1)
    dx, dsh, _ = block.adaln_modulate_bwd(dy_const, x, z, z, CU, 2, 1)
    np.testing.assert_allclose(dx, 0.0, atol=1e-12)
    np.testing.assert_allclose(dsh[0, 0], dy_const[0:3].sum(axis=0), rtol=1e-12)
    xhat = block.layer_norm(x)
    dx2, _, dsc = block.adaln_modulate_bwd(xhat * 2.5, x, z, z, CU, 2, 1)
    # mean(xhat^2) = var / (var + eps), so the residue is exactly 2.5 rstd xhat eps / (var + eps)
    var = x.var(axis=1, keepdims=True)
    np.testing.assert_allclose(dx2, 2.5 * xhat * 1e-6 / (var + 1e-6) / np.sqrt(var + 1e-6), rtol=1e-6, atol=1e-15)
    np.testing.assert_allclose(dsc[1, 1], (2.5 * xhat[9:14] * xhat[9:14]).sum(axis=0), rtol=1e-12)


@pytest.mark.parametrize("rotate", [True, False])
def test_qkv_rope_bwd_finite_differences(rotate):
    rng = np.random.default_rng(44)
    heads, d = 2, 4
    c = heads * d
    h = rng.standard_normal((14, c))
    w = [rng.standard_normal((3 * c, c)) * 0.5, rng.standard_normal((3 * c, c)) * 0.5]
    b = [rng.standard_normal(3 * c), rng.standard_normal(3 * c)]
    dq, dk, dv = (rng.standard_normal((14, heads, d)) for _ in range(3))
    pos = POS if rotate else None

    def loss():
        q, k, v = block.qkv_rope(h, tuple(w), tuple(b), CU, 2, 1, pos, heads, d)
        return float(np.sum(dq * q) + np.sum(dk * k) + np.sum(dv * v))

    dh, dw, db = block.qkv_rope_bwd(dq, dk, dv, h, tuple(w), CU, 2, 1, pos)
    _close(dh, _fd(loss, h))
    for m in range(2):
        _close(dw[m], _fd(loss, w[m]))
        _close(db[m], _fd(loss, b[m]))


def test_out_gated_bwd_finite_differences():
    rng = np.random.default_rng(45)
    c = 8
    o, x = rng.standard_normal((14, c)), rng.standard_normal((14, c))
    w = [rng.standard_normal((c, c)), rng.standard_normal((c, c))]
    b = [rng.standard_normal(c), rng.standard_normal(c)]
    gate = rng.standard_normal((2, 2, c))
    dy = rng.standard_normal((14, c))
    loss = lambda: float(np.sum(dy * block.out_gated_residual(o, x, tuple(w), tuple(b), gate, CU, 2, 1)))  # noqa: E731
    dx, do, dw, db, dg = block.out_gated_residual_bwd(dy, o, x, tuple(w), tuple(b), gate, CU, 2, 1)
    _close(dx, _fd(loss, x))
    _close(do, _fd(loss, o))
    _close(dg, _fd(loss, gate))
    for m in range(2):
        _close(dw[m], _fd(loss, w[m]))
        _close(db[m], _fd(loss, b[m]))
    # gate 0: only the residual path carries gradient
    z = np.zeros_like(gate)
    _, do0, dw0, db0, _ = block.out_gated_residual_bwd(dy, o, x, tuple(w), tuple(b), z, CU, 2, 1)
    assert not do0.any() and not dw0[0].any() and not db0[1].any()

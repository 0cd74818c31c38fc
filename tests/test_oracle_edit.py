"""Pins for the editing extension of the oracle: the [text | source | target]
packer and the frame-aware 3D rotary embedding, and attention with 3D
positions.

A wrong block boundary, a swapped axis, a flipped sign, rotate-half pairing,
a wrong frequency exponent, a frame that does not advance from source to
target, or a 2D rotation used for 3D positions each fail at least one test.
"""
import cmath
import json
import math
import pathlib

import numpy as np
import pytest

import oracle

GOLD = pathlib.Path(__file__).parent / "golden"
THETA = 10000.0


# ---------------------------------------------------------------- packing

def test_tiny_edit_golden():
    g = json.loads((GOLD / "tiny_pack_edit.json").read_text())
    p = oracle.pack_edit(g["samples"], g["budget"])
    for key in ("n_packed", "n_tokens", "max_seqlen", "max_pos"):
        assert p[key] == g[key], key
    assert p["cu_seqlens"].tolist() == g["cu_seqlens"]
    assert p["cu_pieces"].tolist() == g["cu_pieces"]
    assert oracle.positions_edit(g["samples"], p["n_packed"]).tolist() == g["pos"]
    # one token less of budget drops the second sample whole
    assert oracle.pack_edit(g["samples"], g["budget"] - 1)["n_packed"] == 1


def _brute_force_edit(samples, budget):
    """Token-at-a-time walker over [text | source | target] samples."""
    stream = []  # (segment, piece, row, col, frame)
    seg = 0
    for (t, gh, gw) in samples:
        tokens = [(seg, 0, u, u, u) for u in range(t)]
        for f in (0, 1):
            idx = 0
            while idx < gh * gw:
                r, c = divmod(idx, gw)
                tokens.append((seg, 1 + f, t + r, t + c, t + f))
                idx += 1
        if len(stream) + len(tokens) > budget:
            break
        stream += tokens
        seg += 1
    return seg, stream


@pytest.mark.parametrize("seed", range(6))
def test_pack_edit_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    samples = [(int(rng.integers(0, 6)), int(rng.integers(0, 4)), int(rng.integers(0, 5))) for _ in range(7)]
    budget = int(rng.integers(0, 90))
    n, stream = _brute_force_edit(samples, budget)
    p = oracle.pack_edit(samples, budget)
    assert p["n_packed"] == n and p["n_tokens"] == len(stream)
    cu = p["cu_seqlens"].tolist()
    pieces = p["cu_pieces"].tolist()
    for i, (seg, piece, r, c, f) in enumerate(stream):
        assert cu[seg] <= i < cu[seg + 1]
        assert pieces[3 * seg + piece] <= i < (pieces[3 * seg + piece + 1])
    pos = oracle.positions_edit(samples, n)
    assert pos.tolist() == [[r, c, f] for (_, _, r, c, f) in stream]
    assert p["max_pos"] == (1 + max((max(r, c, f) for (*_, r, c, f) in stream), default=-1))


def test_pack_edit_edges():
    assert oracle.pack_edit([(3, 2, 2)], 11)["n_packed"] == 1      # exact fit: 3 + 2*4
    assert oracle.pack_edit([(3, 2, 2)], 10)["n_packed"] == 0
    assert oracle.pack_edit([(3, 2, 2)], 0)["n_tokens"] == 0
    p = oracle.pack_edit([(0, 0, 0), (2, 0, 5), (0, 1, 1)], 10)     # empty sample, text only, image only
    assert p["cu_seqlens"].tolist() == [0, 0, 2, 4]
    assert oracle.positions_edit([(0, 0, 0), (2, 0, 5), (0, 1, 1)], 3).tolist() == [
        [0, 0, 0], [1, 1, 1], [0, 0, 0], [0, 0, 1]]


def test_gather_edit_is_a_bitwise_concatenation():
    rng = np.random.default_rng(3)
    samples = [(2, 1, 3), (1, 2, 1)]
    txt = [rng.integers(0, 255, (t, 4), dtype=np.uint8) for t, _, _ in samples]
    src = [rng.integers(0, 255, (gh, gw, 4), dtype=np.uint8) for _, gh, gw in samples]
    tgt = [rng.integers(0, 255, (gh, gw, 4), dtype=np.uint8) for _, gh, gw in samples]
    out = oracle.gather_edit(txt, src, tgt, 2)
    expect = np.concatenate([txt[0], src[0].reshape(-1, 4), tgt[0].reshape(-1, 4),
                             txt[1], src[1].reshape(-1, 4), tgt[1].reshape(-1, 4)])
    assert np.array_equal(out, expect)


# ---------------------------------------------------------------- 3D rotation

def _unit(d, i):
    x = np.zeros((1, 1, d))
    x[0, 0, i] = 1.0
    return x


@pytest.mark.parametrize("d", [64, 128])
def test_block_boundaries_by_value(d):
    # pair 0 of each block turns by that block's coordinate, in radians:
    # row block at 0, column block at 3D/8, frame block at 3D/4.
    pos = np.array([[3, 5, 2]])
    for start, coord in ((0, 3.0), (3 * d // 8, 5.0), (3 * d // 4, 2.0)):
        y = oracle.rope3d(_unit(d, start), pos, THETA)[0, 0]
        expect = np.zeros(d)
        expect[start], expect[start + 1] = math.cos(coord), math.sin(coord)
        assert np.allclose(y, expect, atol=1e-15), start


def test_frequencies_by_value_d128():
    # D = 128: row/col blocks of 48 dims (pair j turns at 10^(-j/6)),
    # frame block of 32 dims (pair j turns at 10^(-j/4)).
    pos = np.array([[7, 11, 13]])
    for j in (1, 7, 23):
        freq = 10.0 ** (-j / 6.0)
        for start, coord in ((0, 7), (48, 11)):
            y = oracle.rope3d(_unit(128, start + 2 * j), pos, THETA)[0, 0]
            assert y[start + 2 * j] == pytest.approx(math.cos(coord * freq), abs=1e-14)
            assert y[start + 2 * j + 1] == pytest.approx(math.sin(coord * freq), abs=1e-14)
    for j in (1, 9, 15):
        freq = 10.0 ** (-j / 4.0)
        y = oracle.rope3d(_unit(128, 96 + 2 * j), pos, THETA)[0, 0]
        assert y[96 + 2 * j] == pytest.approx(math.cos(13 * freq), abs=1e-14)
        assert y[96 + 2 * j + 1] == pytest.approx(math.sin(13 * freq), abs=1e-14)


def _geometric_freqs(size):
    """Block frequencies by repeated multiplication (a different route from the oracle's powers)."""
    ratio = THETA ** (-2.0 / size)
    out, f = [], 1.0
    for _ in range(size // 2):
        out.append(f)
        f *= ratio
    return out


@pytest.mark.parametrize("d", [64, 128])
def test_complex_form(d):
    # Each block is 1D RoPE on complex pairs z_j -> z_j exp(i p w_j).
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 2, d))
    pos = rng.integers(0, 40, (4, 3))
    y = oracle.rope3d(x, pos, THETA)
    a = 3 * d // 8
    for n in range(4):
        for h in range(2):
            for start, size, axis in ((0, a, 0), (a, a, 1), (2 * a, d - 2 * a, 2)):
                for j, w in enumerate(_geometric_freqs(size)):
                    z = complex(x[n, h, start + 2 * j], x[n, h, start + 2 * j + 1])
                    zr = z * cmath.exp(1j * pos[n, axis] * w)
                    assert y[n, h, start + 2 * j] == pytest.approx(zr.real, abs=1e-9)
                    assert y[n, h, start + 2 * j + 1] == pytest.approx(zr.imag, abs=1e-9)


def test_norm_identity_inverse():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((16, 3, 128))
    pos = rng.integers(0, 200, (16, 3))
    y = oracle.rope3d(x, pos, THETA)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    assert np.array_equal(oracle.rope3d(x, np.zeros((16, 3), dtype=int), THETA), x)
    assert np.allclose(oracle.rope3d(y, pos, THETA, inverse=True), x, atol=1e-12)


def test_relative_offset_in_three_axes():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    p, pk = np.array([[3, 9, 4]]), np.array([[17, 2, 5]])
    base = float(np.sum(oracle.rope3d(q, p, THETA) * oracle.rope3d(k, pk, THETA)))
    for delta in ([5, 0, 0], [0, 7, 0], [0, 0, 1], [13, 21, 2]):
        dd = np.array([delta])
        shifted = float(np.sum(oracle.rope3d(q, p + dd, THETA) * oracle.rope3d(k, pk + dd, THETA)))
        assert shifted == pytest.approx(base, abs=1e-11)
    # and it does depend on each axis's offset
    for axis in range(3):
        dd = np.zeros((1, 3), dtype=int)
        dd[0, axis] = 1
        other = float(np.sum(oracle.rope3d(q, p + dd, THETA) * oracle.rope3d(k, pk, THETA)))
        assert abs(other - base) > 1e-6, axis


def test_source_and_target_differ_only_in_the_frame_block():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((1, 2, 128))
    src = oracle.rope3d(x, np.array([[9, 14, 6]]), THETA)
    tgt = oracle.rope3d(x, np.array([[9, 14, 7]]), THETA)
    assert np.array_equal(src[..., :96], tgt[..., :96])
    assert not np.allclose(src[..., 96:], tgt[..., 96:])
    # the target's frame block is the source's turned one frame further
    one = oracle.rope3d(src, np.array([[0, 0, 1]]), THETA)
    assert np.allclose(one, tgt, atol=1e-13)


def test_rope_axes_dispatch():
    rng = np.random.default_rng(17)
    x = rng.standard_normal((3, 1, 64))
    p2 = rng.integers(0, 9, (3, 2))
    p3 = rng.integers(0, 9, (3, 3))
    assert np.array_equal(oracle.rope_axes(x, p2, THETA), oracle.rope2d(x, p2, THETA))
    assert np.array_equal(oracle.rope_axes(x, p3, THETA), oracle.rope3d(x, p3, THETA))
    with pytest.raises(ValueError):
        oracle.rope_axes(x, rng.integers(0, 9, (3, 4)), THETA)


# ---------------------------------------------------------------- attention with 3D positions

def _edit_case(seed=2):
    samples = [(3, 2, 3), (2, 1, 2), (0, 2, 2)]
    p = oracle.pack_edit(samples, 64)
    pos = oracle.positions_edit(samples, p["n_packed"])
    n = p["n_tokens"]
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((n, 2, 16)) for _ in range(4))
    return p, pos, q, k, v, do


def test_attention_shift_invariance_3d():
    p, pos, q, k, v, _ = _edit_case()
    o, lse = oracle.attn_fwd(q, k, v, p["cu_seqlens"], pos)
    cu = p["cu_seqlens"].tolist()
    shifted = pos.copy()
    for s, delta in enumerate(([4, 1, 9], [0, 6, 2], [3, 3, 3])):
        shifted[cu[s]:cu[s + 1]] += np.array(delta)
    o2, lse2 = oracle.attn_fwd(q, k, v, p["cu_seqlens"], shifted)
    assert np.allclose(o, o2, atol=1e-12) and np.allclose(lse, lse2, atol=1e-12)
    # a frame swap between source and target changes the result
    swapped = pos.copy()
    a = cu[0]
    t = 3
    swapped[a + t:a + t + 6, 2], swapped[a + t + 6:a + t + 12, 2] = pos[a + t + 6:a + t + 12, 2], pos[a + t:a + t + 6, 2]
    o3, _ = oracle.attn_fwd(q, k, v, p["cu_seqlens"], swapped)
    assert not np.allclose(o[a:cu[1]], o3[a:cu[1]])


def test_attention_3d_equals_prerotated_2d_free_path():
    p, pos, q, k, v, do = _edit_case(4)
    o, lse = oracle.attn_fwd(q, k, v, p["cu_seqlens"], pos)
    qr, kr = oracle.rope3d(q, pos, THETA), oracle.rope3d(k, pos, THETA)
    o0, lse0 = oracle.attn_fwd(qr, kr, v, p["cu_seqlens"], None)
    assert np.allclose(o, o0, atol=1e-13) and np.allclose(lse, lse0, atol=1e-13)


def test_backward_3d_finite_differences():
    p, pos, q, k, v, do = _edit_case(6)
    cu = p["cu_seqlens"]
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, cu, pos)

    def loss(qq, kk, vv):
        return float(np.sum(do * oracle.attn_fwd(qq, kk, vv, cu, pos)[0]))

    rng = np.random.default_rng(8)
    h = 1e-6
    for grad, which in ((dq, 0), (dk, 1), (dv, 2)):
        direction = rng.standard_normal(q.shape)
        args_p = [q.copy(), k.copy(), v.copy()]
        args_m = [q.copy(), k.copy(), v.copy()]
        args_p[which] += h * direction
        args_m[which] -= h * direction
        fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert float(np.sum(grad * direction)) == pytest.approx(fd, rel=1e-6, abs=1e-8), which

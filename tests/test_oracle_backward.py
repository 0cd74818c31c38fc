"""Pins for oracle.attn_bwd: finite differences, autograd, special cases and
gradient invariants."""
import numpy as np
import pytest
import torch

import oracle
import workloads

THETA = 10000.0


def _loss(q, k, v, do, cu, pos):
    o, _ = oracle.attn_fwd(q, k, v, cu, pos, THETA)
    return float((o * do).sum())


def _tiny():
    w = workloads.tiny()
    p = oracle.pack(w.samples, w.budget)
    pos = oracle.positions(w.samples, p["n_packed"])
    q, k, v = (workloads.as_f64(x, "f32") for x in workloads.qkv(w.seed, p["n_tokens"], 1, 64, "f32"))
    do = workloads.as_f64(workloads.dout(w.seed, p["n_tokens"], 1, 64, "f32"), "f32")
    return p, pos, q, k, v, do


def test_tiny_finite_differences():
    p, pos, q, k, v, do = _tiny()
    cu = p["cu_seqlens"]
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, cu, pos, THETA)
    rng = np.random.default_rng(0)
    h = 1e-6
    grads = {"q": dq, "k": dk, "v": dv}
    base = {"q": q, "k": k, "v": v}
    for name in ("q", "k", "v"):
        # random directions over the whole tensor
        for _ in range(4):
            u = rng.standard_normal(q.shape)
            args_p = dict(base)
            args_m = dict(base)
            args_p[name] = base[name] + h * u
            args_m[name] = base[name] - h * u
            fd = (_loss(args_p["q"], args_p["k"], args_p["v"], do, cu, pos)
                  - _loss(args_m["q"], args_m["k"], args_m["v"], do, cu, pos)) / (2 * h)
            an = float((grads[name] * u).sum())
            assert fd == pytest.approx(an, rel=1e-6, abs=1e-7)
        # single elements, including first/last token of each segment
        for t in (0, 6, 7, 30, 31, 44):
            for dd in (0, 1, 33, 63):
                e = np.zeros(q.shape)
                e[t, 0, dd] = 1.0
                args_p = dict(base)
                args_m = dict(base)
                args_p[name] = base[name] + h * e
                args_m[name] = base[name] - h * e
                fd = (_loss(args_p["q"], args_p["k"], args_p["v"], do, cu, pos)
                      - _loss(args_m["q"], args_m["k"], args_m["v"], do, cu, pos)) / (2 * h)
                assert fd == pytest.approx(grads[name][t, 0, dd], rel=1e-5, abs=1e-8)


def test_matches_torch_autograd_in_rotated_space():
    rng = np.random.default_rng(1)
    samples = [(9, 4, 3), (1, 0, 0), (2, 5, 5)]
    p = oracle.pack(samples, 10_000)
    pos = oracle.positions(samples, p["n_packed"])
    n, h, d = p["n_tokens"], 3, 128
    q, k, v, do = (rng.standard_normal((n, h, d)) for _ in range(4))
    q *= 3.0
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, p["cu_seqlens"], pos, THETA)
    qr = torch.tensor(oracle.rope2d(q, pos, THETA), requires_grad=True)
    kr = torch.tensor(oracle.rope2d(k, pos, THETA), requires_grad=True)
    vt = torch.tensor(v, requires_grad=True)
    cu = p["cu_seqlens"]
    outs = []
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        qs, ks, vs = (x[a:b].transpose(0, 1) for x in (qr, kr, vt))
        sc = torch.softmax(qs @ ks.transpose(1, 2) / np.sqrt(d), dim=-1)
        outs.append((sc @ vs).transpose(0, 1))
    (torch.cat(outs) * torch.from_numpy(do)).sum().backward()
    # the oracle returns un-rotated gradients: rotate them forward to compare
    assert np.allclose(oracle.rope2d(dq, pos, THETA), qr.grad.numpy(), atol=1e-12)
    assert np.allclose(oracle.rope2d(dk, pos, THETA), kr.grad.numpy(), atol=1e-12)
    assert np.allclose(dv, vt.grad.numpy(), atol=1e-12)


def test_single_token_segment_gradients():
    rng = np.random.default_rng(2)
    samples = [(3, 2, 2), (1, 0, 0), (0, 1, 1)]
    p = oracle.pack(samples, 100)
    pos = oracle.positions(samples, p["n_packed"])
    n = p["n_tokens"]
    q, k, v, do = (rng.standard_normal((n, 2, 64)) for _ in range(4))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, p["cu_seqlens"], pos, THETA)
    for t in (7, 8):
        assert np.allclose(dq[t], 0.0, atol=1e-15) and np.allclose(dk[t], 0.0, atol=1e-15)
        assert np.allclose(dv[t], do[t], atol=1e-15)


def test_gradient_invariants_per_segment_and_head():
    rng = np.random.default_rng(3)
    samples = [(11, 3, 6), (4, 7, 2), (20, 0, 0)]
    p = oracle.pack(samples, 10_000)
    pos = oracle.positions(samples, p["n_packed"])
    n, h, d = p["n_tokens"], 2, 64
    q, k, v, do = (rng.standard_normal((n, h, d)) for _ in range(4))
    q *= 2.0
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, p["cu_seqlens"], pos, THETA, chunk=9)
    dkr = oracle.rope2d(dk, pos, THETA)
    cu = p["cu_seqlens"]
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for hh in range(h):
            # probabilities sum to one per row -> value gradients sum to the output gradients
            assert np.allclose(dv[a:b, hh].sum(0), do[a:b, hh].sum(0), atol=1e-12)
            # scores are invariant to Q -> aQ, K -> K/a
            assert np.sum(dq[a:b, hh] * q[a:b, hh]) == pytest.approx(np.sum(dk[a:b, hh] * k[a:b, hh]), abs=1e-10)
            # scores shift by a per-row constant when all rotated keys move together
            assert np.allclose(dkr[a:b, hh].sum(0), 0.0, atol=1e-12)


def test_chunking_is_invisible():
    rng = np.random.default_rng(4)
    samples = [(30, 4, 4)]
    p = oracle.pack(samples, 10_000)
    pos = oracle.positions(samples, 1)
    n = p["n_tokens"]
    q, k, v, do = (rng.standard_normal((n, 1, 64)) for _ in range(4))
    a = oracle.attn_bwd(q, k, v, do, p["cu_seqlens"], pos, THETA, chunk=5)
    b = oracle.attn_bwd(q, k, v, do, p["cu_seqlens"], pos, THETA, chunk=1000)
    for x, y in zip(a, b):
        assert np.allclose(x, y, atol=1e-13)


def _ragged(seed=5, heads=2, d=64):
    samples = [(7, 3, 5), (1, 0, 0), (20, 4, 4), (0, 2, 9)]
    p = oracle.pack(samples, 1 << 20)
    pos = oracle.positions(samples, p["n_packed"])
    n = p["n_tokens"]
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((n, heads, d)) for _ in range(4))
    return p["cu_seqlens"], pos, q, k, v, do


def test_given_forward_outputs_reduce_to_the_backward():
    """With the exact O and LSE of attn_fwd, the backward taken as a function
    of given outputs is attn_bwd (pinned above by finite differences)."""
    cu, pos, q, k, v, do = _ragged()
    o, lse = oracle.attn_fwd(q, k, v, cu, pos, THETA)
    for a, b in zip(oracle.attn_bwd_given(q, k, v, o, lse, do, cu, pos, THETA),
                    oracle.attn_bwd(q, k, v, do, cu, pos, THETA)):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_given_o_enters_only_through_delta():
    """Perturbing the given O by E changes Delta by rowsum(dO * E) = c per
    query and nothing else, so dS moves by -c P: dV is unchanged, dQr moves
    by -scale * c * (P Kr) (attention with Kr in place of V) and dKr by
    -scale * P^T (c Qr)."""
    cu, pos, q, k, v, do = _ragged(6)
    o, lse = oracle.attn_fwd(q, k, v, cu, pos, THETA)
    e = np.random.default_rng(7).standard_normal(o.shape) * 1e-3
    base = oracle.attn_bwd_given(q, k, v, o, lse, do, cu, pos, THETA)
    moved = oracle.attn_bwd_given(q, k, v, o + e, lse, do, cu, pos, THETA)
    assert np.allclose(moved[2], base[2], rtol=0, atol=1e-14)
    sc = 1.0 / np.sqrt(q.shape[2])
    c = (do * e).sum(axis=2)  # [N][H]
    qr = oracle.rope_axes(q, pos, THETA)
    kr = oracle.rope_axes(k, pos, THETA)
    p_kr, _ = oracle.attn_fwd(q, k, kr, cu, pos, THETA)  # P Kr per query
    want_dqr = -sc * c[:, :, None] * p_kr
    got_dqr = oracle.rope_axes(moved[0] - base[0], pos, THETA)  # back to rotated space
    assert np.allclose(got_dqr, want_dqr, rtol=1e-9, atol=1e-12)
    # dKr: -scale * sum_q P[q, key] c_q Qr[q]; P^T (c Qr) is attention of the
    # keys over the queries' weights, computed per segment from the softmax
    want_dkr = np.zeros_like(q)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        for h in range(q.shape[1]):
            sco = sc * qr[a:b, h] @ kr[a:b, h].T
            pm = np.exp(sco - sco.max(axis=1, keepdims=True))
            pm /= pm.sum(axis=1, keepdims=True)
            want_dkr[a:b, h] = -sc * pm.T @ (c[a:b, h, None] * qr[a:b, h])
    got_dkr = oracle.rope_axes(moved[1] - base[1], pos, THETA)
    assert np.allclose(got_dkr, want_dkr, rtol=1e-9, atol=1e-12)


def test_given_lse_scales_the_weights():
    """Adding a constant t to the given LSE multiplies every weight P by
    exp(-t); Delta comes from the given O and does not move, so dS, and with
    it dQ, dK and dV, scale by exactly exp(-t)."""
    cu, pos, q, k, v, do = _ragged(8)
    o, lse = oracle.attn_fwd(q, k, v, cu, pos, THETA)
    t = 0.37
    base = oracle.attn_bwd_given(q, k, v, o, lse, do, cu, pos, THETA)
    shifted = oracle.attn_bwd_given(q, k, v, o, lse + t, do, cu, pos, THETA)
    for a, b in zip(shifted, base):
        assert np.allclose(a, np.exp(-t) * b, rtol=1e-12, atol=1e-14)

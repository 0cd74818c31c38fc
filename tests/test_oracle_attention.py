"""Pins for oracle.attention (forward): special cases, brute force, a library
routine, and the invariants packing must preserve."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

THETA = 10000.0


def _rand_pack(rng, samples, h, d, qscale=1.0):
    p = oracle.pack(samples, 1 << 30)
    n = p["n_tokens"]
    pos = oracle.positions(samples, p["n_packed"])
    q = rng.standard_normal((n, h, d)) * qscale
    k = rng.standard_normal((n, h, d))
    v = rng.standard_normal((n, h, d))
    return p, pos, q, k, v


def test_single_token_segment_returns_its_value_row():
    rng = np.random.default_rng(0)
    samples = [(5, 2, 2), (1, 0, 0), (0, 1, 1), (3, 0, 0)]
    p, pos, q, k, v = _rand_pack(rng, samples, 2, 64)
    o, lse = oracle.attn_fwd(q, k, v, p["cu_seqlens"], pos, THETA)
    qr = oracle.rope2d(q, pos, THETA)
    kr = oracle.rope2d(k, pos, THETA)
    for t in (9, 10):  # the two 1-token segments
        assert np.allclose(o[t], v[t], atol=1e-15)
        for h in range(2):
            assert lse[h, t] == pytest.approx(np.dot(qr[t, h], kr[t, h]) / 8.0, abs=1e-12)


def test_zero_queries_give_mean_of_values_and_log_length():
    rng = np.random.default_rng(1)
    samples = [(3, 4, 5), (7, 2, 3)]
    p, pos, q, k, v = _rand_pack(rng, samples, 3, 128)
    q[:] = 0.0
    o, lse = oracle.attn_fwd(q, k, v, p["cu_seqlens"], pos, THETA)
    cu = p["cu_seqlens"]
    for s in range(2):
        a, b = cu[s], cu[s + 1]
        assert np.allclose(o[a:b], v[a:b].mean(axis=0, keepdims=True), atol=1e-14)
        assert np.allclose(lse[:, a:b], math.log(b - a), atol=1e-14)


def test_tiny_against_pure_python_loops():
    w = workloads.tiny()
    p = oracle.pack(w.samples, w.budget)
    pos = oracle.positions(w.samples, p["n_packed"])
    q, k, v = (workloads.as_f64(x, "f32") for x in workloads.qkv(w.seed, p["n_tokens"], 1, 64, "f32"))
    o, lse = oracle.attn_fwd(q, k, v, p["cu_seqlens"], pos, THETA)
    qr = oracle.rope2d(q, pos, THETA)
    kr = oracle.rope2d(k, pos, THETA)
    cu = p["cu_seqlens"].tolist()
    for s in range(len(cu) - 1):
        for i in range(cu[s], cu[s + 1]):
            scores = []
            for j in range(cu[s], cu[s + 1]):
                acc = 0.0
                for dd in range(64):
                    acc += qr[i, 0, dd] * kr[j, 0, dd]
                scores.append(acc / 8.0)
            m = max(scores)
            ex = [math.exp(x - m) for x in scores]
            tot = sum(ex)
            for dd in range(64):
                ref = sum(ex[j - cu[s]] * v[j, 0, dd] for j in range(cu[s], cu[s + 1])) / tot
                assert abs(o[i, 0, dd] - ref) < 1e-12
            assert abs(lse[0, i] - (m + math.log(tot))) < 1e-12


def test_matches_torch_sdpa_per_segment():
    rng = np.random.default_rng(2)
    samples = [(12, 5, 7), (1, 3, 3), (30, 0, 0), (4, 9, 2)]
    p, pos, q, k, v = _rand_pack(rng, samples, 4, 128, qscale=3.0)
    o, _ = oracle.attn_fwd(q, k, v, p["cu_seqlens"], pos, THETA, chunk=16)
    qr = torch.from_numpy(oracle.rope2d(q, pos, THETA))
    kr = torch.from_numpy(oracle.rope2d(k, pos, THETA))
    vt = torch.from_numpy(v)
    cu = p["cu_seqlens"]
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        ref = torch.nn.functional.scaled_dot_product_attention(
            qr[a:b].transpose(0, 1), kr[a:b].transpose(0, 1), vt[a:b].transpose(0, 1)).transpose(0, 1)
        assert np.allclose(o[a:b], ref.numpy(), atol=1e-12)


def test_packed_equals_unpacked_and_segments_do_not_leak():
    rng = np.random.default_rng(3)
    samples = [(5, 3, 4), (2, 6, 1), (9, 2, 2)]
    p, pos, q, k, v = _rand_pack(rng, samples, 2, 64)
    o, lse = oracle.attn_fwd(q, k, v, p["cu_seqlens"], pos, THETA)
    cu = p["cu_seqlens"]
    for s in range(3):
        a, b = int(cu[s]), int(cu[s + 1])
        ps = oracle.positions([samples[s]], 1)
        assert np.array_equal(ps, pos[a:b])
        o1, l1 = oracle.attn_fwd(q[a:b], k[a:b], v[a:b], [0, b - a], ps, THETA)
        assert np.allclose(o1, o[a:b], atol=1e-14) and np.allclose(l1, lse[:, a:b], atol=1e-14)
    # outliers in segment 0 leave segments 1 and 2 unchanged
    k2, v2 = k.copy(), v.copy()
    k2[: cu[1]] *= 30.0
    v2[: cu[1]] += 30.0
    o2, l2 = oracle.attn_fwd(q, k2, v2, cu, pos, THETA)
    assert np.array_equal(o2[cu[1]:], o[cu[1]:]) and np.array_equal(l2[:, cu[1]:], lse[:, cu[1]:])
    assert not np.allclose(o2[: cu[1]], o[: cu[1]])


def test_shift_of_a_samples_positions_changes_nothing():
    # RoPE on both Q and K makes attention depend only on 2-D offsets.
    rng = np.random.default_rng(4)
    samples = [(6, 4, 4), (3, 2, 5)]
    p, pos, q, k, v = _rand_pack(rng, samples, 2, 128, qscale=4.0)
    o, lse = oracle.attn_fwd(q, k, v, p["cu_seqlens"], pos, THETA)
    shifted = pos.copy()
    shifted[: p["cu_seqlens"][1]] += np.array([17, -5])
    o2, l2 = oracle.attn_fwd(q, k, v, p["cu_seqlens"], shifted, THETA)
    assert np.allclose(o2, o, atol=1e-11) and np.allclose(l2, lse, atol=1e-11)


def test_permuting_a_segment_permutes_outputs():
    rng = np.random.default_rng(5)
    samples = [(4, 3, 3)]
    p, pos, q, k, v = _rand_pack(rng, samples, 1, 64)
    o, lse = oracle.attn_fwd(q, k, v, p["cu_seqlens"], pos, THETA)
    perm = rng.permutation(p["n_tokens"])
    o2, l2 = oracle.attn_fwd(q[perm], k[perm], v[perm], p["cu_seqlens"], pos[perm], THETA)
    assert np.allclose(o2, o[perm], atol=1e-13) and np.allclose(l2, lse[:, perm], atol=1e-13)


def test_constant_values_reproduced_and_chunking_is_invisible():
    rng = np.random.default_rng(6)
    samples = [(40, 5, 6)]
    p, pos, q, k, v = _rand_pack(rng, samples, 1, 64, qscale=2.0)
    v[:] = 0.75  # rows of P sum to one
    o, _ = oracle.attn_fwd(q, k, v, p["cu_seqlens"], pos, THETA)
    assert np.allclose(o, 0.75, atol=1e-14)
    v = rng.standard_normal(v.shape)
    o1, l1 = oracle.attn_fwd(q, k, v, p["cu_seqlens"], pos, THETA, chunk=7)
    o2, l2 = oracle.attn_fwd(q, k, v, p["cu_seqlens"], pos, THETA, chunk=4096)
    assert np.allclose(o1, o2, atol=1e-14) and np.allclose(l1, l2, atol=1e-14)


def test_rows_helper_matches_full():
    rng = np.random.default_rng(7)
    samples = [(8, 5, 5), (2, 1, 9), (1, 0, 0)]
    p, pos, q, k, v = _rand_pack(rng, samples, 3, 128)
    o, lse = oracle.attn_fwd(q, k, v, p["cu_seqlens"], pos, THETA)
    rows = [(0, 0), (10, 2), (33, 1), (44, 0), (p["n_tokens"] - 1, 2)]
    orow, lrow = oracle.attn_fwd_rows(q, k, v, p["cu_seqlens"], pos, rows, THETA)
    for i, (t, h) in enumerate(rows):
        assert np.allclose(orow[i], o[t, h], atol=1e-13)
        assert lrow[i] == pytest.approx(lse[h, t], abs=1e-13)


def test_scale_argument():
    rng = np.random.default_rng(8)
    samples = [(3, 2, 2)]
    p, pos, q, k, v = _rand_pack(rng, samples, 1, 64)
    o1, l1 = oracle.attn_fwd(q, k, v, p["cu_seqlens"], pos, THETA, scale=0.25)
    o2, l2 = oracle.attn_fwd(2 * q, k, v, p["cu_seqlens"], pos, THETA)  # 2/8 = 0.25
    assert np.allclose(o1, o2, atol=1e-14) and np.allclose(l1, l2, atol=1e-14)

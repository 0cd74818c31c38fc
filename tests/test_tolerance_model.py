"""The GPU parity bars, pinned on the CPU against a model of the kernels'
rounding (no GPU needed).

The default bars (max-abs 2e-2, mean-abs 2e-3; LSE 1e-2) are written for
outputs of magnitude up to about 4.  Some GPU tests move the inputs away from
N(0, 1) on purpose (peaky scores, explicit scales, segments of a handful of
tokens) and use scaled bars instead.  Each scaled bar is derived here from the
arithmetic: ``emulate_fwd`` / ``emulate_bwd`` evaluate attention in float64
except at exactly the points where the kernels round to bf16 (the rotated Q
and K, the unnormalised softmax weights before P V, P before dV, dS before
dQ and dK, and every bf16 output) or keep fp32 (LSE).  For each scaled bar
the test checks two things:

* an implementation with those roundings and no other error stays inside the
  bar, with margin, on the GPU test's own inputs, for every admissible
  rounding outcome: the forward's running max may lag a row's true maximum
  by up to 8 in log2 units once a segment spans more than one 32-key tile,
  so the weights it rounds sit up to 2^8 above exp(S - max); the model draws
  that lag at random per row for such segments (``lag_seed``);
* a planted mistake (one key dropped from every segment's softmax) falls
  outside it, so the bar still catches a boundary error.

The model is test infrastructure beside the oracle (it imports ``oracle`` for
the rotation only) and shares nothing with the HIP path.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_close, assert_close_large_values, assert_close_scaled, assert_rel_rms

THETA = 10000.0
SMALL = [(7, 9, 13), (1, 0, 0), (300, 0, 0), (33, 10, 10), (0, 1, 1), (64, 8, 8), (0, 0, 0), (5, 17, 3),
         (2, 1, 62), (129, 0, 0)]


def bf(x) -> np.ndarray:
    """float64 -> float32 -> bf16 (round to nearest even), back to float64."""
    b = workloads.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    return workloads.bf16_bits_to_f32(b).astype(np.float64)


def _inputs(samples, heads, d, seed, qscale=1.0, with_dout=False):
    p = oracle.pack(samples, 1 << 20)
    n = p["n_tokens"]
    pos = oracle.positions(samples, p["n_packed"])
    q, k, v = (workloads.as_f64(x, "bf16") for x in workloads.qkv(seed, n, heads, d, "bf16"))
    if qscale != 1.0:
        q = workloads.as_f64(workloads.normal(seed, workloads.STREAM_Q, (n, heads, d), "bf16", scale=qscale), "bf16")
    do = workloads.as_f64(workloads.dout(seed, n, heads, d, "bf16"), "bf16") if with_dout else None
    return p["cu_seqlens"], pos, q, k, v, do


def _rot(x, pos, inverse=False):
    return x if pos is None else oracle.rope_axes(x, pos, THETA, inverse=inverse)


def _scores(qr, kr, sc, drop_last_key):
    s = sc * (qr @ kr.T)
    if drop_last_key and s.shape[1] > 1:
        s[:, -1] = -np.inf
    return s


KEY_TILE = 32  # keys per forward tile: the running max can lag from the second tile on
LAGS = (None, 1, 2, 3, 4)  # no lag, then four random lag draws


def emulate_fwd(q, k, v, cu, pos, scale=None, drop_last_key=False, lag_seed=None):
    n, h_count, d = q.shape
    sc = 1.0 / np.sqrt(d) if scale is None else scale
    qr, kr = bf(_rot(q, pos)), bf(_rot(k, pos))
    rng = np.random.default_rng(lag_seed) if lag_seed is not None else None
    o = np.zeros_like(q)
    lse = np.zeros((h_count, n))
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b <= a:
            continue
        for h in range(h_count):
            sco = _scores(qr[a:b, h], kr[a:b, h], sc, drop_last_key)
            m = sco.max(axis=1, keepdims=True)
            lag = 0.0
            if rng is not None and b - a > KEY_TILE:
                lag = rng.uniform(0.0, 8.0 * np.log(2.0), size=(b - a, 1))
            e = np.exp(sco - m + lag)
            ell = e.sum(axis=1, keepdims=True)
            o[a:b, h] = bf((bf(e) @ v[a:b, h]) / ell)
            lse[h, a:b] = np.float32(m - lag + np.log(ell))[:, 0]
    return o, lse


def emulate_bwd(q, k, v, o, lse, do, cu, pos, drop_last_key=False):
    """The backward's own roundings, given O and LSE."""
    n, h_count, d = q.shape
    sc = 1.0 / np.sqrt(d)
    qr, kr = bf(_rot(q, pos)), bf(_rot(k, pos))
    dqr, dkr, dv = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b <= a:
            continue
        for h in range(h_count):
            p = np.exp(_scores(qr[a:b, h], kr[a:b, h], sc, drop_last_key) - lse[h, a:b, None])
            dd = do[a:b, h]
            dv[a:b, h] = bf(p).T @ dd
            delta = (dd * o[a:b, h]).sum(axis=1, keepdims=True)
            ds = bf(p * (dd @ v[a:b, h].T - delta))
            dqr[a:b, h] = sc * (ds @ kr[a:b, h])
            dkr[a:b, h] = sc * (ds.T @ qr[a:b, h])
    return bf(_rot(dqr, pos, True)), bf(_rot(dkr, pos, True)), bf(dv)


def emulate_step(q, k, v, do, cu, pos, drop_last_key=False, lag_seed=None):
    o, lse = emulate_fwd(q, k, v, cu, pos, drop_last_key=drop_last_key, lag_seed=lag_seed)
    return emulate_bwd(q, k, v, o, lse, do, cu, pos, drop_last_key=drop_last_key)


def _count_failures(check, pairs):
    failures = 0
    for g, r, name in pairs:
        try:
            check(g, r, name)
        except AssertionError:
            failures += 1
    return failures


# -- peaky backward, Q x 4, no RoPE (tests/test_gpu_attn_bwd.py) --------------

def _bwd_case_peaky():
    cu, _, q, k, v, do = _inputs(SMALL[:6], 2, 128, 32, qscale=4.0, with_dout=True)
    return cu, q, k, v, do


def _given_outputs(q, k, v, cu, pos):
    """The forward outputs a backward test hands in: the oracle's O rounded to
    bf16 and its LSE rounded to fp32."""
    o, lse = oracle.attn_fwd(q, k, v, cu, pos, THETA)
    n = int(cu[-1])
    lse = np.where(np.isnan(lse), 0.0, lse)
    return bf(o), np.float32(lse).astype(np.float64), n


def test_peaky_backward_given_outputs_bar():
    """With O and LSE given, the backward's own roundings (P before dV, dS
    before dQ and dK, the bf16 outputs) stay under the max|ref|-scaled bar;
    logits reach ~12 and dK = scale dS^T Q grows with Q, which max|ref|
    tracks."""
    cu, q, k, v, do = _bwd_case_peaky()
    o, lse, _ = _given_outputs(q, k, v, cu, None)
    ref = oracle.attn_bwd_given(q, k, v, o, lse, do, cu, None, THETA)
    got = emulate_bwd(q, k, v, o, lse, do, cu, None)
    for g, r, name in zip(got, ref, ("dQ", "dK", "dV")):
        bar = 2e-2 * max(1.0, float(np.abs(r).max()) / 4.0)
        assert float(np.abs(g - r).max()) <= 0.8 * bar, name
        assert_close_scaled(g, r, f"model {name} given O, LSE")
    planted = emulate_bwd(q, k, v, o, lse, do, cu, None, drop_last_key=True)
    assert _count_failures(assert_close_scaled, zip(planted, ref, ("dQ", "dK", "dV"))) == 3


def test_peaky_backward_end_to_end_rel_rms():
    """Forward then backward: Delta now comes from the forward's own bf16 O,
    whose rounding reaches dS with weight P ~ 1 on a peaky row's winning key
    (and dK with a factor |Q|), so the largest element error moves with the
    rounding outcome by 2x or more; the relative RMS error does not."""
    cu, q, k, v, do = _bwd_case_peaky()
    ref = oracle.attn_bwd(q, k, v, do, cu, None, THETA)
    for lag in LAGS:
        got = emulate_step(q, k, v, do, cu, None, lag_seed=lag)
        for g, r, name in zip(got, ref, ("dQ", "dK", "dV")):
            rr = float(np.sqrt(np.mean((g - r) ** 2)) / np.sqrt(np.mean(r ** 2)))
            assert rr <= 0.75 * 8e-3, (name, lag, rr)
    planted = emulate_step(q, k, v, do, cu, None, drop_last_key=True)
    assert _count_failures(assert_rel_rms, zip(planted, ref, ("dQ", "dK", "dV"))) == 3


# -- peaky forward, Q x 8, RoPE (tests/test_gpu_attn_fwd.py) -------------------

def _fwd_case_peaky():
    cu, pos, q, k, v, _ = _inputs(SMALL, 2, 128, 24, qscale=8.0)
    return cu, pos, q, k, v


def test_peaky_forward_bar():
    """Logits reach ~28: the bf16 rounding of the rotated Q and K (2^-9
    relative each) moves a logit by up to ~0.1 and near-tied weights by
    ~10%, so O moves by a fraction of a V difference: max-abs 0.25,
    mean-abs 8e-3; LSE takes the max|ref|-scaled bar."""
    cu, pos, q, k, v = _fwd_case_peaky()
    ro, rl = oracle.attn_fwd(q, k, v, cu, pos, THETA)
    n = int(cu[-1])
    for lag in LAGS:
        go, gl = emulate_fwd(q, k, v, cu, pos, lag_seed=lag)
        err = np.abs(go[:n] - ro[:n])
        assert float(err.max()) <= 0.75 * 0.25 and float(err.mean()) <= 0.75 * 8e-3, lag
        assert_close(go[:n], ro[:n], 0.25, 8e-3, f"model O q*8 lag {lag}")
        assert_close_scaled(gl[:, :n], rl[:, :n], f"model LSE q*8 lag {lag}")
    go, _ = emulate_fwd(q, k, v, cu, pos, drop_last_key=True)
    with pytest.raises(AssertionError):
        assert_close(go[:n], ro[:n], 0.25, 8e-3, "planted O q*8")


# -- explicit softmax scale 0.3 at D = 64 (tests/test_gpu_attn_fwd.py) ---------

def test_explicit_scale_bars():
    """0.3 is 2.4x the default 1/8: the logit error the rotated-operand
    rounding leaves is linear in the score scale, and O and LSE errors follow
    it, so both default bars grow 2.4x."""
    cu, pos, q, k, v, _ = _inputs(SMALL[:4], 2, 64, 23)
    ro, rl = oracle.attn_fwd(q, k, v, cu, pos, THETA, scale=0.3)
    n = int(cu[-1])
    grow = 0.3 * np.sqrt(64)
    for lag in LAGS:
        go, gl = emulate_fwd(q, k, v, cu, pos, scale=0.3, lag_seed=lag)
        assert float(np.abs(go[:n] - ro[:n]).max()) <= 0.75 * 2e-2 * grow, lag
        assert float(np.abs(gl[:, :n] - rl[:, :n]).max()) <= 0.8 * 1e-2 * grow, lag


# -- 1300 segments of at most ~20 tokens (tests/test_gpu_attn_bwd.py) ----------

@pytest.fixture(scope="module")
def tiny_segments():
    rng = np.random.default_rng(78)
    samples = [(int(rng.integers(0, 12)), int(rng.integers(0, 4)), int(rng.integers(0, 4))) for _ in range(1300)]
    cu, pos, q, k, v, do = _inputs(samples, 2, 128, 35, with_dout=True)
    # every segment fits one key tile: the running max is each row's true max
    assert int(np.diff(cu).max()) <= KEY_TILE
    ref = oracle.attn_bwd(q, k, v, do, cu, pos, THETA)
    return cu, pos, q, k, v, do, ref


def test_few_key_bar(tiny_segments):
    cu, pos, q, k, v, do, ref = tiny_segments
    got = emulate_step(q, k, v, do, cu, pos)
    n = int(cu[-1])
    for g, r, name in zip(got, ref, ("dQ", "dK", "dV")):
        worst = float((np.abs(g[:n] - r[:n]) / (2e-2 + 1e-2 * np.abs(r[:n]))).max())
        assert worst <= 0.7, (name, worst)
        assert_close_large_values(g[:n], r[:n], f"model {name} 1300 segments")
    planted = emulate_step(q, k, v, do, cu, pos, drop_last_key=True)
    pairs = [(g[:n], r[:n], name) for g, r, name in zip(planted, ref, ("dQ", "dK", "dV"))]
    assert _count_failures(assert_close_large_values, pairs) == 3

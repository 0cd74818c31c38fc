"""GPU parity of the rectified-flow noising / loss and the packed CFG combine
against oracle.flow (float64).

Bars: float32 tensors within 1e-5 of the oracle (relative to the values'
scale); bf16 tensors within one bf16 rounding of the oracle's value
(|err| <= |ref| * 2^-8 + 1e-6); loss sums (float32 accumulation of up to
~6e6 terms of size ~2) within a relative 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import dev, host_f64, note
from oracle import flow

pytestmark = pytest.mark.gpu


def _mf():
    import packed_varlen_attention_amd as mf
    return mf


def _within_rounding(got, ref, dtype, label):
    err = np.abs(got - ref)
    bar = np.abs(ref) * 2.0 ** -8 + 1e-6 if dtype == "bf16" else np.abs(ref) * 1e-6 + 1e-6
    worst = float((err - bar).max()) if err.size else -1.0
    print(f"  {label}: max_abs={float(err.max()) if err.size else 0:.3e}", flush=True)
    assert worst <= 0, f"{label}: exceeds bar by {worst}"


def _case(samples, frames, c, dtype, seed):
    p = (oracle.pack_edit if frames == 2 else oracle.pack)(samples, 1 << 22)
    n, s = p["n_tokens"], len(samples)
    z, eps, v = (workloads.normal(seed, k, (n, c), dtype) for k in (11, 12, 13))
    t = np.random.default_rng([seed, 14]).uniform(0.0, 1.0, size=max(s, 1)).astype(np.float32)
    return p, z, eps, v, t


@pytest.mark.parametrize("frames", [1, 2])
@pytest.mark.parametrize("dtype,c", [("bf16", 128), ("f32", 128), ("bf16", 16), ("f32", 512)])
def test_noise_and_loss_small(frames, dtype, c):
    mf = _mf()
    rng = np.random.default_rng(frames * 10 + c)
    samples = workloads.random_samples(rng, 9, max_text=30, max_side=9)
    p, z, eps, v, t = _case(samples, frames, c, dtype, seed=50 + frames)
    n, s = p["n_tokens"], len(samples)
    cp = torch.from_numpy(p["cu_pieces"].astype(np.int32)).cuda()
    tz, te, tv = dev(z, dtype), dev(eps, dtype), dev(v, dtype)
    tt = torch.from_numpy(t).cuda()
    note(f"mf_rf_noise/mf_rf_loss N={n} C={c} {dtype} frames={frames}")
    zt = mf.rf_noise(tz, te, tt, cp, s, frames)
    m = max(1, sum(b - a for _, a, b in flow.noised_ranges(p["cu_pieces"], s, frames)) * c)
    loss, grad = mf.rf_loss(tv, tz, te, cp, s, frames, grad_scale=2.0 / m)
    torch.cuda.synchronize()
    zf, ef, vf = (workloads.as_f64(x, dtype) for x in (z, eps, v))
    ref_zt = flow.rf_noise(zf, ef, t.astype(np.float64), p["cu_pieces"], s, frames)
    # the kernel blends in float32 with t rounded to float32: compare at that precision
    _within_rounding(host_f64(zt), ref_zt, dtype, "z_t")
    ref_loss, ref_grad = flow.rf_loss(vf, zf, ef, p["cu_pieces"], s, frames, 2.0 / m)
    got = loss.cpu().numpy().astype(np.float64)
    assert np.allclose(got, ref_loss, rtol=1e-4, atol=1e-3), (got, ref_loss)
    _within_rounding(host_f64(grad), ref_grad, dtype, "grad")


def test_loss_full_size_mixed_pack_and_determinism():
    mf = _mf()
    w = workloads.mixed50k()
    p, z, eps, v, t = _case(list(w.samples), 1, 128, "bf16", seed=55)
    s = len(w.samples)
    cp = torch.from_numpy(p["cu_pieces"].astype(np.int32)).cuda()
    tz, te, tv = dev(z, "bf16"), dev(eps, "bf16"), dev(v, "bf16")
    note(f"mf_rf_loss mixed50k N={p['n_tokens']} C=128")
    loss1, grad1 = mf.rf_loss(tv, tz, te, cp, s, 1, grad_scale=1.0)
    loss2, grad2 = mf.rf_loss(tv, tz, te, cp, s, 1, grad_scale=1.0)
    torch.cuda.synchronize()
    assert torch.equal(loss1, loss2) and torch.equal(grad1.view(torch.int16), grad2.view(torch.int16))
    ref_loss, ref_grad = flow.rf_loss(*(workloads.as_f64(x, "bf16") for x in (v, z, eps)), p["cu_pieces"], s, 1, 1.0)
    got = loss1.cpu().numpy().astype(np.float64)
    assert np.allclose(got, ref_loss, rtol=1e-4), (got[:12], ref_loss[:12])
    rows = np.random.default_rng(0).integers(0, p["n_tokens"], size=3000)
    _within_rounding(host_f64(grad1[torch.from_numpy(rows).cuda()]), ref_grad[rows], "bf16", "grad sampled")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cfg_combine_packed_pairs(dtype):
    mf = _mf()
    w = workloads.cfg1024()
    samples = list(w.samples)
    p = oracle.pack(samples, w.budget)
    n = p["n_tokens"]
    v = workloads.normal(60, 1, (n, 128), dtype)
    cp = torch.from_numpy(p["cu_pieces"].astype(np.int32)).cuda()
    tv = dev(v, dtype)
    note(f"mf_cfg_combine cfg1024 N={n} {dtype}")
    out, bad = mf.cfg_combine(tv, cp, len(samples), 4, 4.5)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0
    ref = flow.cfg_combine(workloads.as_f64(v, dtype), p["cu_pieces"], 4, 4.5)
    _within_rounding(host_f64(out), ref, dtype, "guided")
    # in place gives the same values
    tv2 = tv.clone()
    mf.cfg_combine(tv2, cp, len(samples), 4, 4.5, out=tv2)
    torch.cuda.synchronize()
    assert torch.equal(tv2, out)


def test_cfg_mismatched_pair_is_counted_and_left_alone():
    mf = _mf()
    samples = [(3, 2, 2), (1, 2, 2), (2, 2, 3), (1, 3, 3)]   # second pair: 6 vs 9 image tokens
    p = oracle.pack(samples, 1 << 20)
    v = workloads.normal(61, 1, (p["n_tokens"], 16), "f32")
    cp = torch.from_numpy(p["cu_pieces"].astype(np.int32)).cuda()
    note("mf_cfg_combine mismatched pair")
    out, bad = mf.cfg_combine(dev(v, "f32"), cp, 4, 2, 3.0)
    torch.cuda.synchronize()
    assert int(bad.item()) == 1
    got = host_f64(out)
    # first pair: rows [0, 12) = cu_pieces[:5]; the second pair's rows stay copies
    assert p["cu_pieces"][:5].tolist() == [0, 3, 7, 8, 12]
    ref_first = flow.cfg_combine(v.astype(np.float64)[:12], p["cu_pieces"][:5], 1, 3.0)
    _within_rounding(got[:12], ref_first, "f32", "first pair")
    assert np.array_equal(got[12:], v[12:].astype(np.float64))

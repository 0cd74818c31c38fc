"""GPU parity of mf_rope2d_apply against oracle.rope2d."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import THETA, assert_close, dev, host_f64, note

pytestmark = pytest.mark.gpu


def _mf():
    import packed_varlen_attention_amd as mf
    return mf


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("inverse", [False, True])
def test_rope_matches_oracle(dtype, d, inverse):
    mf = _mf()
    samples = [(17, 12, 30), (1, 0, 0), (300, 2, 2), (5, 40, 9)]
    p = oracle.pack(samples, 1 << 20)
    pos = oracle.positions(samples, p["n_packed"])
    n, h = p["n_tokens"], 3
    x = workloads.normal(11, 1, (n, h, d), dtype)
    xf = workloads.as_f64(x, dtype)
    t = dev(x, dtype)
    tpos = torch.from_numpy(pos.astype(np.int32)).cuda()
    note(f"mf_rope2d_apply {dtype} D={d} inverse={inverse} N={n}")
    mf.rope2d_apply(t, tpos, THETA, p["max_pos"], inverse=inverse)
    torch.cuda.synchronize()
    ref = oracle.rope2d(xf, pos, THETA, inverse=inverse)
    if dtype == "f32":
        assert_close(host_f64(t), ref, 2e-5, 1e-6, "rope f32")
    else:
        assert_close(host_f64(t), ref, 2e-2, 2e-3, "rope bf16")
        # each output is the bf16 rounding of a value within ~1e-5 of the oracle
        assert np.all(np.abs(host_f64(t) - ref) <= np.abs(ref) * 2 ** -8 + 1e-4)


def test_rope_forward_then_inverse_roundtrip_f32():
    mf = _mf()
    samples = [(40, 20, 20)]
    p = oracle.pack(samples, 1 << 20)
    pos = oracle.positions(samples, 1)
    x = workloads.normal(12, 1, (p["n_tokens"], 2, 128), "f32")
    t = dev(x, "f32")
    tpos = torch.from_numpy(pos.astype(np.int32)).cuda()
    note("mf_rope2d_apply roundtrip")
    mf.rope2d_apply(t, tpos, THETA, p["max_pos"])
    mf.rope2d_apply(t, tpos, THETA, p["max_pos"], inverse=True)
    torch.cuda.synchronize()
    assert_close(host_f64(t), x.astype(np.float64), 1e-5, 1e-6, "roundtrip")


def test_rope_full_size_mixed_pack():
    """The standalone pass at the mixed 50k-token pack's full size."""
    mf = _mf()
    w = workloads.mixed50k()
    p = oracle.pack(w.samples, w.budget)
    pos = oracle.positions(w.samples, p["n_packed"])
    n = p["n_tokens"]
    x = workloads.normal(w.seed, workloads.STREAM_K, (n, w.n_heads, w.head_dim), "bf16")
    t = dev(x, "bf16")
    tpos = torch.from_numpy(pos.astype(np.int32)).cuda()
    note(f"mf_rope2d_apply mixed50k N={n}")
    mf.rope2d_apply(t, tpos, THETA, p["max_pos"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = rng.integers(0, n, size=2000)
    rows = np.concatenate([rows, [0, n - 1]])
    got = host_f64(t[torch.from_numpy(rows).cuda()])
    ref = oracle.rope2d(workloads.as_f64(x[rows], "bf16"), pos[rows], THETA)
    assert_close(got, ref, 2e-2, 2e-3, "rope mixed50k sampled rows")

"""GPU parity of mf_varlen_attn_bwd against the fp64 oracle backward.

The GPU backward consumes the GPU forward's O (bf16) and LSE; the oracle
recomputes its own in fp64.  Gradients: max-abs 2e-2, mean-abs 2e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (HEADS_PER_XCD, THETA, Case, assert_close, assert_close_large_values, assert_close_scaled,
                      assert_rel_rms, bench_step, dev, host_f64, merged_segments, note, oracle_per_head)

pytestmark = pytest.mark.gpu

G_MAX, G_MEAN = 2e-2, 2e-3

SMALL = [(7, 9, 13), (1, 0, 0), (300, 0, 0), (33, 10, 10), (0, 1, 1), (64, 8, 8), (0, 0, 0), (5, 17, 3),
         (2, 1, 62), (129, 0, 0)]


def _mf():
    import packed_varlen_attention_amd as mf
    return mf


def _run(c: Case, use_pos=True):
    mf = _mf()
    pos = c.tpos if use_pos else None
    note(f"mf_varlen_attn_fwd+bwd {c.describe()} rope={use_pos}")
    o, lse = mf.attn_fwd(c.tq, c.tk, c.tv, c.tcu, c.max_seqlen, pos, THETA, c.max_pos)
    dq, dk, dv = mf.attn_bwd(c.tq, c.tk, c.tv, o, lse, c.tdo, c.tcu, c.max_seqlen, pos, THETA, c.max_pos)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_small_packs_all_elements(dtype, d):
    c = Case(SMALL, 1 << 20, 3, d, dtype, seed=31, with_dout=True)
    dq, dk, dv = _run(c)
    rq, rk, rv = oracle.attn_bwd(c.q, c.k, c.v, c.do, c.cu, c.pos, THETA)
    n = c.n
    assert_close(host_f64(dq)[:n], rq[:n], G_MAX, G_MEAN, f"dQ {dtype} D{d}")
    assert_close(host_f64(dk)[:n], rk[:n], G_MAX, G_MEAN, f"dK {dtype} D{d}")
    assert_close(host_f64(dv)[:n], rv[:n], G_MAX, G_MEAN, f"dV {dtype} D{d}")


# Segment lengths around the tile sizes: a forward query tile holds 128 rows
# and a forward key tile 32 keys, a dq query tile 256 rows (64-key tiles), a
# dkdv workgroup 128 keys.  In a segment that fits one such tile, waves whose
# rows (keys) all lie past the end skip their products; in longer segments
# they do not.  Every element is checked either way.
TILE_EDGES = [(127, 0, 0), (128, 0, 0), (129, 0, 0), (224, 0, 0), (225, 0, 0), (31, 0, 0), (255, 0, 0),
              (256, 0, 0), (257, 0, 0), (288, 0, 0), (16, 15, 16), (1, 16, 16), (32, 0, 0), (33, 0, 0),
              (64, 0, 0), (65, 0, 0)]


@pytest.mark.parametrize("d", [128, 64])
def test_segments_at_tile_edges(d):
    c = Case(TILE_EDGES, 1 << 20, 3, d, "bf16", seed=37, with_dout=True)
    mf = _mf()
    note(f"mf_varlen_attn_fwd+bwd tile edges {c.describe()}")
    o, lse = mf.attn_fwd(c.tq, c.tk, c.tv, c.tcu, c.max_seqlen, c.tpos, THETA, c.max_pos)
    dq, dk, dv = mf.attn_bwd(c.tq, c.tk, c.tv, o, lse, c.tdo, c.tcu, c.max_seqlen, c.tpos, THETA, c.max_pos)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd(c.q, c.k, c.v, c.cu, c.pos, THETA)
    rq, rk, rv = oracle.attn_bwd(c.q, c.k, c.v, c.do, c.cu, c.pos, THETA)
    n = c.n
    assert_close(host_f64(o)[:n], ro[:n], 2e-2, 2e-3, f"O D{d}")
    assert_close(host_f64(lse)[:, :n], rl[:, :n], 1e-2, 1e-2, f"LSE D{d}")
    assert_close(host_f64(dq)[:n], rq[:n], G_MAX, G_MEAN, f"dQ D{d}")
    assert_close(host_f64(dk)[:n], rk[:n], G_MAX, G_MEAN, f"dK D{d}")
    assert_close(host_f64(dv)[:n], rv[:n], G_MAX, G_MEAN, f"dV D{d}")


def test_tiny_workload():
    w = workloads.tiny()
    c = Case(w.samples, w.budget, w.n_heads, w.head_dim, w.dtype, w.seed, with_dout=True)
    dq, dk, dv = _run(c)
    rq, rk, rv = oracle.attn_bwd(c.q, c.k, c.v, c.do, c.cu, c.pos, THETA)
    assert_close(host_f64(dq), rq, G_MAX, G_MEAN, "dQ tiny")
    assert_close(host_f64(dk), rk, G_MAX, G_MEAN, "dK tiny")
    assert_close(host_f64(dv), rv, G_MAX, G_MEAN, "dV tiny")


def test_peaky_backward_given_outputs():
    """Q x 4, no RoPE (logits reach ~12).  The backward is run on given
    forward outputs -- the oracle's O rounded to bf16 and its LSE rounded to
    fp32 -- and compared with the oracle's backward on those same O and LSE,
    so the bar measures the backward's own roundings (P before dV, dS before
    dQ and dK, the bf16 outputs): the default bar scaled by max|ref| / 4
    (pinned in test_tolerance_model.py::test_peaky_backward_given_outputs_bar)."""
    mf = _mf()
    c = Case(SMALL[:6], 1 << 20, 2, 128, "bf16", seed=32, qscale=4.0, with_dout=True)
    ro, rl = oracle.attn_fwd(c.q, c.k, c.v, c.cu, None, THETA)
    n = c.n
    o_bits = workloads.f32_to_bf16_bits(ro.astype(np.float32))
    o_in = dev(o_bits, "bf16")
    lse_in = torch.from_numpy(np.nan_to_num(rl, nan=0.0).astype(np.float32)).cuda()
    note(f"mf_varlen_attn_bwd on given O, LSE {c.describe()} rope=False")
    dq, dk, dv = mf.attn_bwd(c.tq, c.tk, c.tv, o_in, lse_in, c.tdo, c.tcu, c.max_seqlen, None, THETA, c.max_pos)
    torch.cuda.synchronize()
    o_given = workloads.bf16_bits_to_f32(o_bits).astype(np.float64)
    l_given = np.nan_to_num(rl, nan=0.0).astype(np.float32).astype(np.float64)
    rq, rk, rv = oracle.attn_bwd_given(c.q, c.k, c.v, o_given, l_given, c.do, c.cu, None, THETA)
    assert_close_scaled(host_f64(dq)[:n], rq[:n], "dQ no-rope q*4, given O, LSE")
    assert_close_scaled(host_f64(dk)[:n], rk[:n], "dK no-rope q*4, given O, LSE")
    assert_close_scaled(host_f64(dv)[:n], rv[:n], "dV no-rope q*4, given O, LSE")


def test_peaky_end_to_end_rel_rms():
    """The same peaky pack through forward and backward.  Delta then comes
    from the forward's own bf16 O; on a peaky row its rounding reaches dS with
    weight P ~ 1 and dK with a factor |Q|, so the largest element error moves
    with the rounding outcome; the relative RMS error stays at the bf16 level
    (pinned in test_tolerance_model.py::test_peaky_backward_end_to_end_rel_rms)."""
    c = Case(SMALL[:6], 1 << 20, 2, 128, "bf16", seed=32, qscale=4.0, with_dout=True)
    dq, dk, dv = _run(c, use_pos=False)
    rq, rk, rv = oracle.attn_bwd(c.q, c.k, c.v, c.do, c.cu, None, THETA)
    n = c.n
    assert_rel_rms(host_f64(dq)[:n], rq[:n], "dQ no-rope q*4")
    assert_rel_rms(host_f64(dk)[:n], rk[:n], "dK no-rope q*4")
    assert_rel_rms(host_f64(dv)[:n], rv[:n], "dV no-rope q*4")


def test_deterministic_and_segment_local():
    mf = _mf()
    c = Case(SMALL, 1 << 20, 2, 128, "bf16", seed=33, with_dout=True)
    a = _run(c)
    b = _run(c)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    # per-segment runs give bitwise the same gradients (a segment sharing a
    # multi-segment tile, see gpu_util.merged_segments, up to rounding)
    merged = merged_segments(c.cu)
    for s in (0, 2, 3):
        lo, hi = int(c.cu[s]), int(c.cu[s + 1])
        cu1 = torch.tensor([0, hi - lo], dtype=torch.int32).cuda()
        sl = [t[lo:hi].contiguous() for t in (c.tq, c.tk, c.tv, c.tdo)]
        p1 = c.tpos[lo:hi].contiguous()
        note(f"per-segment bwd s={s}")
        o1, l1 = mf.attn_fwd(sl[0], sl[1], sl[2], cu1, hi - lo, p1, THETA, c.max_pos)
        g = mf.attn_bwd(sl[0], sl[1], sl[2], o1, l1, sl[3], cu1, hi - lo, p1, THETA, c.max_pos)
        torch.cuda.synchronize()
        for x, y, name in zip(g, a, ("dQ", "dK", "dV")):
            if s in merged:
                assert_close_scaled(host_f64(x), host_f64(y[lo:hi]), f"{name} segment {s} (multi-segment tile)")
            else:
                assert torch.equal(x.view(torch.int16), y[lo:hi].view(torch.int16))


def test_gradient_sums_match_invariants():
    # sum over keys of dV equals sum over queries of dO, per (segment, head)
    c = Case(SMALL, 1 << 20, 2, 128, "bf16", seed=34, with_dout=True)
    _, _, dv = _run(c)
    g = host_f64(dv)
    for s in range(len(c.cu) - 1):
        a, b = int(c.cu[s]), int(c.cu[s + 1])
        if b > a:
            assert np.allclose(g[a:b].sum(0), c.do[a:b].astype(np.float64).sum(0), atol=5e-2 * np.sqrt(b - a))


def test_full_size_mixed_pack_eight_heads():
    """Backward on the mixed 50k-token pack (the training shape) through the
    benchmark's exact call (GPU pack, explicit workspaces, host segment
    count, the rotated buffer the forward fills and the backward reads); the
    oracle recomputes every element of dQ, dK and dV for one head of each
    XCD's group of heads."""
    w = workloads.mixed50k(backward=True)
    c = Case(w.samples, w.budget, w.n_heads, w.head_dim, w.dtype, w.seed, with_dout=True)
    _, _, dq, dk, dv = bench_step(c, backward=True)
    n = c.n

    def ref(h):
        sl = slice(h, h + 1)
        return oracle.attn_bwd(c.q[:, sl], c.k[:, sl], c.v[:, sl], c.do[:, sl], c.cu, c.pos, THETA)

    note(f"oracle backward, heads {HEADS_PER_XCD}")
    refs = oracle_per_head(ref, HEADS_PER_XCD)
    gq, gk, gv = host_f64(dq), host_f64(dk), host_f64(dv)
    for h, (rq, rk, rv) in zip(HEADS_PER_XCD, refs):
        assert_close(gq[:n, h:h + 1], rq[:n], G_MAX, G_MEAN, f"dQ mixed50k head {h}")
        assert_close(gk[:n, h:h + 1], rk[:n], G_MAX, G_MEAN, f"dK mixed50k head {h}")
        assert_close(gv[:n, h:h + 1], rv[:n], G_MAX, G_MEAN, f"dV mixed50k head {h}")


def test_full_size_kept_rotation_is_bit_identical():
    """At full size, the step with the rotated buffer (the benchmark's form)
    gives bit for bit the outputs and gradients of the calls without it."""
    mf = _mf()
    w = workloads.mixed50k(backward=True)
    c = Case(w.samples, w.budget, w.n_heads, w.head_dim, w.dtype, w.seed, with_dout=True)
    kept = bench_step(c, backward=True)
    note("mixed50k fwd+bwd without the rotated buffer")
    o, lse = mf.attn_fwd(c.tq, c.tk, c.tv, c.tcu, c.max_seqlen, c.tpos, THETA, c.max_pos)
    g = mf.attn_bwd(c.tq, c.tk, c.tv, o, lse, c.tdo, c.tcu, c.max_seqlen, c.tpos, THETA, c.max_pos)
    torch.cuda.synchronize()
    for a, b, name in zip(kept, (o, lse) + tuple(g), ("O", "LSE", "dQ", "dK", "dV")):
        assert torch.equal(a, b), f"{name} differs with the rotated buffer at full size"


def test_more_segments_than_the_scheduler_sorts():
    rng = np.random.default_rng(78)
    samples = [(int(rng.integers(0, 12)), int(rng.integers(0, 4)), int(rng.integers(0, 4))) for _ in range(1300)]
    c = Case(samples, 1 << 20, 2, 128, "bf16", seed=35, with_dout=True)
    assert len(c.cu) - 1 > 1024
    dq, dk, dv = _run(c)
    rq, rk, rv = oracle.attn_bwd(c.q, c.k, c.v, c.do, c.cu, c.pos, THETA)
    n = c.n
    # segments of at most ~20 tokens give gradients above |4|: see the helper
    # (pinned in test_tolerance_model.py::test_few_key_bar)
    assert_close_large_values(host_f64(dq)[:n], rq[:n], "dQ 1300 segments")
    assert_close_large_values(host_f64(dk)[:n], rk[:n], "dK 1300 segments")
    assert_close_large_values(host_f64(dv)[:n], rv[:n], "dV 1300 segments")


def test_rows_more_than_4gib_past_a_tile_base():
    """A segment whose rows reach more than 2^32 bytes past a tile's first
    row: 16384 heads of D = 128 make a token row 4 MiB, so the 1100-token
    segment spans 4.3 GiB.  The tile copies clamp rows past the segment end
    with a 32-bit byte offset, which must stay below 2^32 (a wrapped clamp
    would re-read the wrong rows of one K/V and one Q/dO tile).  Two heads
    are drawn and repeated across all heads on the device; the oracle
    recomputes the first and the last head, and heads with the same inputs
    must give identical gradients."""
    heads = 16384
    c = Case([(100, 40, 25)], 1 << 20, 2, 128, "bf16", seed=36, with_dout=True)
    assert c.n == 1100 and (c.n - 1) * heads * 128 * 2 >= 1 << 32

    def rep(t):
        return t.repeat(1, heads // 2, 1)

    mf = _mf()
    q, k, v, do = rep(c.tq), rep(c.tk), rep(c.tv), rep(c.tdo)
    note(f"mf_varlen_attn_fwd+bwd N={c.n} H={heads} D=128 bf16 (4.3 GiB per tensor)")
    o, lse = mf.attn_fwd(q, k, v, c.tcu, c.max_seqlen, c.tpos, THETA, c.max_pos)
    dq, dk, dv = mf.attn_bwd(q, k, v, o, lse, do, c.tcu, c.max_seqlen, c.tpos, THETA, c.max_pos)
    torch.cuda.synchronize()
    del q, k, v, do, o, lse
    for g, name in ((dq, "dQ"), (dk, "dK"), (dv, "dV")):
        assert torch.equal(g[:, 0], g[:, heads - 2]) and torch.equal(g[:, 1], g[:, heads - 1]), name
    for src, h in ((0, 0), (1, heads - 1)):
        sl = slice(src, src + 1)
        rq, rk, rv = oracle.attn_bwd(c.q[:, sl], c.k[:, sl], c.v[:, sl], c.do[:, sl], c.cu, c.pos, THETA)
        for g, r, name in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
            got = host_f64(g[:, h:h + 1])
            assert_close(got, r, G_MAX, G_MEAN, f"{name} 4 MiB rows head {h}")
            assert_close_scaled(got, r, f"{name} 4 MiB rows head {h}")
    del dq, dk, dv
    torch.cuda.empty_cache()

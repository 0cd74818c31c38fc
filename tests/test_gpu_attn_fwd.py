"""GPU parity of mf_varlen_attn_fwd against the fp64 oracle.

Tolerances: bf16 outputs within max-abs 2e-2 and mean-abs 2e-3 of the oracle;
LSE (float32) within max-abs 1e-2.  Because |O| is small for long segments,
structural gates (bitwise packed == per-segment, segment-leak, a peaky
Q x 8 run, determinism) catch boundary bugs the tolerances would not.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (HEADS_PER_XCD, THETA, Case, assert_close, assert_close_scaled, bench_step, host_f64,
                      merged_segments, note, oracle_per_head)

pytestmark = pytest.mark.gpu

O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-2

SMALL = [(7, 9, 13), (1, 0, 0), (300, 0, 0), (33, 10, 10), (0, 1, 1), (64, 8, 8), (0, 0, 0), (5, 17, 3),
         (2, 1, 62), (129, 0, 0)]


def _mf():
    import packed_varlen_attention_amd as mf
    return mf


def _run(c: Case, use_pos=True, scale=0.0):
    mf = _mf()
    note(f"mf_varlen_attn_fwd {c.describe()} rope={use_pos}")
    o, lse = mf.attn_fwd(c.tq, c.tk, c.tv, c.tcu, c.max_seqlen, c.tpos if use_pos else None, THETA, c.max_pos,
                         softmax_scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _full_ref(c: Case, use_pos=True, scale=None):
    return oracle.attn_fwd(c.q, c.k, c.v, c.cu, c.pos if use_pos else None, THETA, scale=scale)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_small_packs_all_elements(dtype, d):
    c = Case(SMALL, 1 << 20, 3, d, dtype, seed=21)
    o, lse = _run(c)
    ref_o, ref_l = _full_ref(c)
    n = c.n
    assert_close(host_f64(o)[:n], ref_o[:n], O_MAX, O_MEAN, f"O {dtype} D{d}")
    assert_close(host_f64(lse)[:, :n], ref_l[:, :n], LSE_MAX, LSE_MAX, f"LSE {dtype} D{d}")
    if dtype == "f32":
        # the inputs are rounded to bf16 for the products: errors stay at bf16 level
        assert_close(host_f64(o)[:n], ref_o[:n], 1e-2, 1e-3, "O f32 (tighter)")


def test_tiny_workload():
    w = workloads.tiny()
    c = Case(w.samples, w.budget, w.n_heads, w.head_dim, w.dtype, w.seed)
    o, lse = _run(c)
    ref_o, ref_l = _full_ref(c)
    assert_close(host_f64(o), ref_o, O_MAX, O_MEAN, "O tiny")
    assert_close(host_f64(lse), ref_l, LSE_MAX, LSE_MAX, "LSE tiny")


def test_without_rope():
    c = Case(SMALL[:6], 1 << 20, 2, 128, "bf16", seed=22)
    o, lse = _run(c, use_pos=False)
    ref_o, ref_l = _full_ref(c, use_pos=False)
    assert_close(host_f64(o), ref_o, O_MAX, O_MEAN, "O no-rope")
    assert_close(host_f64(lse), ref_l, LSE_MAX, LSE_MAX, "LSE no-rope")


def test_explicit_scale():
    c = Case(SMALL[:4], 1 << 20, 2, 64, "bf16", seed=23)
    o, lse = _run(c, scale=0.3)
    ref_o, ref_l = _full_ref(c, scale=0.3)
    # The logit error the bf16 rounding of the rotated Q and K leaves is
    # linear in the score scale, and the O and LSE errors follow it: 0.3 is
    # 2.4x the default 1/sqrt(64), so both default bars grow 2.4x (pinned in
    # test_tolerance_model.py::test_explicit_scale_bars).
    grow = 0.3 * np.sqrt(64)
    assert_close(host_f64(o), ref_o, O_MAX * grow, O_MEAN, "O scale 0.3")
    assert_close(host_f64(lse), ref_l, LSE_MAX * grow, LSE_MAX * grow, "LSE scale 0.3")


def test_peaky_scores_q_times_8():
    c = Case(SMALL, 1 << 20, 2, 128, "bf16", seed=24, qscale=8.0)
    o, lse = _run(c)
    ref_o, ref_l = _full_ref(c)
    # Logits reach ~28 here; the bf16 rounding of rotated Q and K moves them
    # by up to ~28 * 2^-8 = 0.11, which shifts near-tied softmax weights by
    # ~10%: O can move by up to ~0.3 of a V difference.  A dropped or extra
    # key would move peaky rows by O(|V|) ~ 1-3, far above this bar (both
    # pinned in test_tolerance_model.py::test_peaky_forward_bar).
    assert_close(host_f64(o), ref_o, 0.25, 8e-3, "O q*8")
    assert_close_scaled(host_f64(lse), ref_l, "LSE q*8")


def test_single_token_segments_return_value_row():
    c = Case([(1, 0, 0), (0, 1, 1), (3, 2, 2), (1, 0, 0)], 1 << 20, 4, 128, "bf16", seed=25)
    o, _ = _run(c)
    got = host_f64(o)
    for t in (0, 1, 9):
        assert np.array_equal(got[t], c.v[t].astype(np.float64))


def test_packed_equals_per_segment_bitwise_and_no_leak():
    mf = _mf()
    c = Case(SMALL, 1 << 20, 2, 128, "bf16", seed=26)
    o, lse = _run(c)
    merged = merged_segments(c.cu)  # none for this pack; multi-segment tiles: test_gpu_tiny_segments
    for s in range(len(c.cu) - 1):
        a, b = int(c.cu[s]), int(c.cu[s + 1])
        if b == a:
            continue
        note(f"per-segment fwd s={s} L={b - a}")
        cu1 = torch.tensor([0, b - a], dtype=torch.int32).cuda()
        o1, l1 = mf.attn_fwd(c.tq[a:b].contiguous(), c.tk[a:b].contiguous(), c.tv[a:b].contiguous(), cu1, b - a,
                             c.tpos[a:b].contiguous(), THETA, c.max_pos)
        torch.cuda.synchronize()
        if s in merged:
            assert_close(host_f64(o1), host_f64(o[a:b]), O_MAX, O_MEAN, f"segment {s} (multi-segment tile)")
            assert_close(host_f64(l1), host_f64(lse[:, a:b]), LSE_MAX, LSE_MAX, f"segment {s} LSE")
            continue
        assert torch.equal(o1.view(torch.int16), o[a:b].view(torch.int16)), f"segment {s} differs"
        assert torch.equal(l1, lse[:, a:b]), f"segment {s} LSE differs"
    # outliers in segment 2 must not change any other segment
    k2, v2 = c.tk.clone(), c.tv.clone()
    a, b = int(c.cu[2]), int(c.cu[3])
    k2[a:b] = 30.0
    v2[a:b] = -30.0
    note("segment leak run")
    o2, l2 = mf.attn_fwd(c.tq, k2, v2, c.tcu, c.max_seqlen, c.tpos, THETA, c.max_pos)
    torch.cuda.synchronize()
    assert torch.equal(o2[:a].view(torch.int16), o[:a].view(torch.int16))
    assert torch.equal(o2[b:c.n].view(torch.int16), o[b:c.n].view(torch.int16))
    assert torch.equal(l2[:, :a], lse[:, :a]) and torch.equal(l2[:, b:c.n], lse[:, b:c.n])
    assert not torch.equal(o2[a:b].view(torch.int16), o[a:b].view(torch.int16))


def test_deterministic():
    c = Case(SMALL, 1 << 20, 2, 128, "bf16", seed=27)
    o1, l1 = _run(c)
    o2, l2 = _run(c)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["cfg1024", "mixed50k", "stress"])
def test_full_size_eight_heads(name):
    """Full-size workloads through the benchmark's exact call (GPU pack,
    explicit workspace, host segment count, the kept rotated buffer); the
    oracle recomputes every element of O and LSE for one head of each XCD's
    group of heads."""
    w = getattr(workloads, name)()
    c = Case(w.samples, w.budget, w.n_heads, w.head_dim, w.dtype, w.seed)
    o, lse = bench_step(c, backward=False)
    n = c.n

    def ref(h):
        sl = slice(h, h + 1)
        return oracle.attn_fwd(c.q[:, sl], c.k[:, sl], c.v[:, sl], c.cu, c.pos, THETA)

    note(f"oracle forward, heads {HEADS_PER_XCD}")
    refs = oracle_per_head(ref, HEADS_PER_XCD)
    got_o, got_l = host_f64(o), host_f64(lse)
    for h, (ro, rl) in zip(HEADS_PER_XCD, refs):
        assert_close(got_o[:n, h:h + 1], ro[:n], O_MAX, O_MEAN, f"O {name} head {h}")
        assert_close(got_l[h:h + 1, :n], rl[:, :n], LSE_MAX, LSE_MAX, f"LSE {name} head {h}")
    # every head's rows are finite
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse[:, :n]).all()


@pytest.mark.parametrize("d", [128, 64])
def test_long_segments_take_the_256_row_shape(d):
    """A pack whose segments are all long (the longest at least 12288 tokens,
    the mean at least 8192) runs the forward's 256-row, 64-key form; both
    segments end mid-tile in either shape.  Every element of O and LSE."""
    c = Case([(12307, 0, 0), (13001, 0, 0)], 1 << 20, 1, d, "bf16", seed=29)
    assert c.max_seqlen >= 12288 and c.n >= 8192 * (len(c.cu) - 1)
    o, lse = _run(c)
    ref_o, ref_l = _full_ref(c)
    assert_close(host_f64(o)[: c.n], ref_o[: c.n], O_MAX, O_MEAN, f"O long segments D{d}")
    assert_close(host_f64(lse)[:, : c.n], ref_l[:, : c.n], LSE_MAX, LSE_MAX, f"LSE long segments D{d}")


def test_more_segments_than_the_scheduler_sorts():
    """Over 1024 segments the schedule keeps the given order instead of sorting
    by length: results must not depend on that."""
    rng = np.random.default_rng(77)
    samples = [(int(rng.integers(0, 12)), int(rng.integers(0, 4)), int(rng.integers(0, 4))) for _ in range(1500)]
    c = Case(samples, 1 << 20, 2, 64, "bf16", seed=28)
    assert len(c.cu) - 1 > 1024
    o, lse = _run(c)
    ref_o, ref_l = _full_ref(c)
    assert_close(host_f64(o)[: c.n], ref_o[: c.n], O_MAX, O_MEAN, "O 1500 segments")
    assert_close(host_f64(lse)[:, : c.n], ref_l[:, : c.n], LSE_MAX, LSE_MAX, "LSE 1500 segments")

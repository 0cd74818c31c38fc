"""GPU parity of the editing path (frame-aware 3D RoPE) against the oracle:
mf_pack_edit bit-exact, mf_rope3d_apply, and mf_varlen_attn3d_fwd/bwd within
the same bars as the 2D calls (O and gradients max-abs 2e-2, mean-abs 2e-3;
LSE 1e-2), on small ragged editing packs element by element and on the
edit50k pack at full size."""
import json
import pathlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import (HEADS_PER_XCD, THETA, Case, assert_close, bench_step, dev, host_f64, merged_segments, note,
                      oracle_per_head, samples_dev)

pytestmark = pytest.mark.gpu

GOLD = pathlib.Path(__file__).parent / "golden"
O_MAX, O_MEAN, LSE_MAX = 2e-2, 2e-3, 1e-2

SMALL_EDIT = [(7, 9, 13), (1, 0, 0), (40, 3, 3), (0, 5, 6), (2, 1, 30), (0, 0, 0), (64, 8, 8), (5, 11, 2)]


def _mf():
    import packed_varlen_attention_amd as mf
    return mf


# ---------------------------------------------------------------- packing

def _check_pack_edit(samples, budget, label, rows=None, row_bytes=0):
    mf = _mf()
    note(f"mf_pack_edit {label}: S={len(samples)} budget={budget}")
    args = rows if rows is not None else (None, None, None)
    r = mf.pack_edit(samples_dev(samples), budget, *args, row_bytes=row_bytes)
    torch.cuda.synchronize()
    ref = oracle.pack_edit(samples, budget)
    n, ntok = ref["n_packed"], ref["n_tokens"]
    assert r.counts.cpu().tolist() == [n, ntok, ref["max_seqlen"], ref["max_pos"]]
    cu = r.cu_seqlens.cpu().numpy()
    assert cu[: n + 1].tolist() == ref["cu_seqlens"].tolist() and (cu[n + 1:] == ntok).all()
    pieces = r.cu_pieces.cpu().numpy()
    assert pieces[: 3 * n + 1].tolist() == ref["cu_pieces"].tolist() and (pieces[3 * n + 1:] == ntok).all()
    assert np.array_equal(r.pos.cpu().numpy()[:ntok], oracle.positions_edit(samples, n).reshape(-1, 3))
    return r, ref


def test_tiny_edit_golden():
    g = json.loads((GOLD / "tiny_pack_edit.json").read_text())
    r, _ = _check_pack_edit(g["samples"], g["budget"], "golden")
    assert r.pos.cpu().numpy()[: g["n_tokens"]].tolist() == g["pos"]
    assert r.cu_pieces.cpu().tolist() == g["cu_pieces"]


@pytest.mark.parametrize("seed", range(12))
def test_random_edit_packs(seed):
    rng = np.random.default_rng(300 + seed)
    samples = workloads.random_samples(rng, int(rng.integers(1, 30)))
    _check_pack_edit(samples, int(rng.integers(0, 4000)), f"random seed={seed}")


def test_edit_workload_pack_and_errors():
    w = workloads.edit50k()
    _check_pack_edit(list(w.samples), w.budget, "edit50k")
    rng = np.random.default_rng(9)
    _check_pack_edit(workloads.random_samples(rng, 2100, max_text=10, max_side=3), 10 ** 9, "2100 samples")
    mf = _mf()
    note("mf_pack_edit negative descriptor")
    r = mf.pack_edit(samples_dev([(3, 2, 2), (1, 2, -2)]), 100)
    torch.cuda.synchronize()
    assert r.counts.cpu().tolist() == [-1, 0, 0, 0]


@pytest.mark.parametrize("row_bytes", [64, 20])
def test_edit_gather_bit_exact(row_bytes):
    rng = np.random.default_rng(row_bytes)
    samples = [(3, 2, 5), (0, 4, 4), (7, 0, 0), (2, 3, 3), (50, 10, 10)]
    budget = 23 + 32 + 7 + 20  # the last sample does not fit
    text = [rng.integers(0, 256, size=(t, row_bytes), dtype=np.uint8) for (t, _, _) in samples]
    src = [rng.integers(0, 256, size=(gh, gw, row_bytes), dtype=np.uint8) for (_, gh, gw) in samples]
    tgt = [rng.integers(0, 256, size=(gh, gw, row_bytes), dtype=np.uint8) for (_, gh, gw) in samples]
    keep = []

    def ptrs(parts):
        bufs = [torch.from_numpy(x.reshape(-1)).cuda() if x.size else None for x in parts]
        keep.extend(bufs)
        return torch.tensor([b.data_ptr() if b is not None else 0 for b in bufs], dtype=torch.int64).cuda()

    r, ref = _check_pack_edit(samples, budget, f"gather row_bytes={row_bytes}",
                              rows=(ptrs(text), ptrs(src), ptrs(tgt)), row_bytes=row_bytes)
    assert ref["n_packed"] == 4
    want = oracle.gather_edit(text, src, tgt, ref["n_packed"])
    assert np.array_equal(r.packed.cpu().numpy()[: ref["n_tokens"]], want)


# ---------------------------------------------------------------- 3D rotation

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("inverse", [False, True])
def test_rope3d_matches_oracle(dtype, d, inverse):
    mf = _mf()
    samples = [(17, 12, 30), (1, 0, 0), (300, 2, 2), (5, 40, 9)]
    p = oracle.pack_edit(samples, 1 << 20)
    pos = oracle.positions_edit(samples, p["n_packed"])
    n, h = p["n_tokens"], 3
    x = workloads.normal(13, 1, (n, h, d), dtype)
    t = dev(x, dtype)
    note(f"mf_rope3d_apply {dtype} D={d} inverse={inverse} N={n}")
    mf.rope3d_apply(t, torch.from_numpy(pos.astype(np.int32)).cuda(), THETA, p["max_pos"], inverse=inverse)
    torch.cuda.synchronize()
    ref = oracle.rope3d(workloads.as_f64(x, dtype), pos, THETA, inverse=inverse)
    if dtype == "f32":
        assert_close(host_f64(t), ref, 2e-5, 1e-6, "rope3d f32")
    else:
        assert_close(host_f64(t), ref, 2e-2, 2e-3, "rope3d bf16")
        assert np.all(np.abs(host_f64(t) - ref) <= np.abs(ref) * 2 ** -8 + 1e-4)


# ---------------------------------------------------------------- attention with 3D positions

def _fwd(c: Case, **kw):
    mf = _mf()
    note(f"mf_varlen_attn3d_fwd {c.describe()}")
    o, lse = mf.attn_fwd(c.tq, c.tk, c.tv, c.tcu, c.max_seqlen, kw.get("pos", c.tpos), THETA, c.max_pos)
    torch.cuda.synchronize()
    return o, lse


def _fwd_bwd(c: Case):
    mf = _mf()
    note(f"mf_varlen_attn3d_fwd+bwd {c.describe()}")
    o, lse = mf.attn_fwd(c.tq, c.tk, c.tv, c.tcu, c.max_seqlen, c.tpos, THETA, c.max_pos)
    g = mf.attn_bwd(c.tq, c.tk, c.tv, o, lse, c.tdo, c.tcu, c.max_seqlen, c.tpos, THETA, c.max_pos)
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_small_edit_packs_all_elements(dtype, d):
    c = Case(SMALL_EDIT, 1 << 20, 3, d, dtype, seed=41, with_dout=True, editing=True)
    o, lse = _fwd(c)
    ref_o, ref_l = oracle.attn_fwd(c.q, c.k, c.v, c.cu, c.pos, THETA)
    n = c.n
    assert_close(host_f64(o)[:n], ref_o[:n], O_MAX, O_MEAN, f"O 3D {dtype} D{d}")
    assert_close(host_f64(lse)[:, :n], ref_l[:, :n], LSE_MAX, LSE_MAX, f"LSE 3D {dtype} D{d}")
    dq, dk, dv = _fwd_bwd(c)
    rq, rk, rv = oracle.attn_bwd(c.q, c.k, c.v, c.do, c.cu, c.pos, THETA)
    assert_close(host_f64(dq)[:n], rq[:n], O_MAX, O_MEAN, f"dQ 3D {dtype} D{d}")
    assert_close(host_f64(dk)[:n], rk[:n], O_MAX, O_MEAN, f"dK 3D {dtype} D{d}")
    assert_close(host_f64(dv)[:n], rv[:n], O_MAX, O_MEAN, f"dV 3D {dtype} D{d}")


def test_frame_axis_changes_the_result_and_segments_stay_local():
    mf = _mf()
    c = Case(SMALL_EDIT, 1 << 20, 2, 128, "bf16", seed=42, editing=True)
    o, lse = _fwd(c)
    # every frame moved one step: relative frames are unchanged, so nothing changes
    shifted = c.tpos.clone()
    shifted[:, 2] += 1
    o1, l1 = _fwd(c, pos=shifted)
    assert_close(host_f64(o1), host_f64(o), O_MAX, O_MEAN, "O frame shift")
    # source and target frames swapped in segment 0: the result changes there only
    swapped = c.tpos.clone()
    a, b = int(c.cu[0]), int(c.cu[1])
    t, img = c.samples[0][0], c.samples[0][1] * c.samples[0][2]
    swapped[a + t:a + t + img, 2] += 1
    swapped[a + t + img:b, 2] -= 1
    o2, _ = _fwd(c, pos=swapped)
    assert torch.equal(o2[b:c.n].view(torch.int16), o[b:c.n].view(torch.int16))
    assert float((o2[a:b].float() - o[a:b].float()).abs().max()) > 2e-2
    # packed == per-segment, bitwise
    for s in range(len(c.cu) - 1):
        lo, hi = int(c.cu[s]), int(c.cu[s + 1])
        if hi == lo:
            continue
        cu1 = torch.tensor([0, hi - lo], dtype=torch.int32).cuda()
        note(f"per-segment 3D fwd s={s}")
        oo, ll = mf.attn_fwd(c.tq[lo:hi].contiguous(), c.tk[lo:hi].contiguous(), c.tv[lo:hi].contiguous(), cu1,
                             hi - lo, c.tpos[lo:hi].contiguous(), THETA, c.max_pos)
        torch.cuda.synchronize()
        if s in merged_segments(c.cu):
            assert_close(host_f64(oo), host_f64(o[lo:hi]), 2e-2, 2e-3, f"segment {s} (multi-segment tile)")
            continue
        assert torch.equal(oo.view(torch.int16), o[lo:hi].view(torch.int16)), s
        assert torch.equal(ll, lse[:, lo:hi]), s


def test_edit50k_full_size():
    """The edit50k pack at full size through the benchmark's exact call (GPU
    pack, explicit workspaces, host segment count, the rotated buffer the
    forward fills and the backward reads): every element of O and LSE for one
    head of each XCD's group of heads, and every element of dQ, dK and dV for
    the same heads."""
    w = workloads.edit50k()
    c = Case(w.samples, w.budget, w.n_heads, w.head_dim, w.dtype, w.seed, with_dout=True, editing=True)
    o, lse, dq, dk, dv = bench_step(c, backward=True)
    n = c.n

    def ref_fwd(h):
        sl = slice(h, h + 1)
        return oracle.attn_fwd(c.q[:, sl], c.k[:, sl], c.v[:, sl], c.cu, c.pos, THETA)

    note(f"oracle 3D forward, heads {HEADS_PER_XCD}")
    refs = oracle_per_head(ref_fwd, HEADS_PER_XCD)
    got_o, got_l = host_f64(o), host_f64(lse)
    for h, (ro, rl) in zip(HEADS_PER_XCD, refs):
        assert_close(got_o[:n, h:h + 1], ro[:n], O_MAX, O_MEAN, f"O edit50k head {h}")
        assert_close(got_l[h:h + 1, :n], rl[:, :n], LSE_MAX, LSE_MAX, f"LSE edit50k head {h}")

    bwd_heads = HEADS_PER_XCD

    def ref_bwd(h):
        sl = slice(h, h + 1)
        return oracle.attn_bwd(c.q[:, sl], c.k[:, sl], c.v[:, sl], c.do[:, sl], c.cu, c.pos, THETA)

    note(f"oracle 3D backward, heads {bwd_heads}")
    grefs = oracle_per_head(ref_bwd, bwd_heads)
    gq, gk, gv = host_f64(dq), host_f64(dk), host_f64(dv)
    for h, (rq, rk, rv) in zip(bwd_heads, grefs):
        assert_close(gq[:n, h:h + 1], rq[:n], O_MAX, O_MEAN, f"dQ edit50k head {h}")
        assert_close(gk[:n, h:h + 1], rk[:n], O_MAX, O_MEAN, f"dK edit50k head {h}")
        assert_close(gv[:n, h:h + 1], rv[:n], O_MAX, O_MEAN, f"dV edit50k head {h}")

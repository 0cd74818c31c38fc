"""GPU parity of the attention sub-block chains (adaptive norm, QKV projection
with the rotary embedding, output projection with the gated residual)
against oracle.block (float64), on the same bf16 / fp32 input values.

Bar: every bf16 output within one bf16 ulp of the oracle's value,
|err| <= |ref| 2^-7 + 1e-5.  The GPU rounds once, after fp32 arithmetic
(products of bf16 values are exact in fp32; the K <= 3072-term sums and the
LayerNorm statistics carry fp32 errors of order 1e-6 relative), so a value
either rounds to the nearest bf16 (half an ulp, <= 2^-8 relative) or, when
the fp32 error straddles a rounding boundary, to its neighbour (one ulp,
<= 2^-7 relative).  The chained case (norm -> projection -> attention ->
projection, each stage rounding to bf16) uses the attention tests' scaled
bars.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_close_scaled, dev, host_f64, note
from oracle import block

pytestmark = pytest.mark.gpu
THETA = 10000.0


def _mf():
    import packed_varlen_attention_amd as mf
    return mf


def _within_ulp(got, ref, label):
    err = np.abs(got - ref)
    bar = np.abs(ref) * 2.0 ** -7 + 1e-5
    worst = float((err - bar).max()) if err.size else -1.0
    print(f"  {label}: max_abs={float(err.max()) if err.size else 0:.3e} n={err.size}", flush=True)
    assert worst <= 0, f"{label}: exceeds the one-ulp bar by {worst:.3e}"


def _layout(samples, frames, budget=1 << 22):
    """(pack dict, positions [N][2 or 3]) from the oracle packer."""
    if frames == 2:
        p = oracle.pack_edit(samples, budget)
        pos = oracle.positions_edit(samples, p["n_packed"])
    else:
        p = oracle.pack(samples, budget)
        pos = oracle.positions(samples, p["n_packed"])
    return p, np.asarray(pos, dtype=np.int32)


def _i32(x):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.int32))).cuda()


def _f32(x):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32))).cuda()


def _bf(x):
    return workloads.as_f64(x, "bf16")


# ragged pieces: a text-only sample, a zero-text sample, pieces below, at and past one 256-row tile
SAMPLES = [(7, 4, 6), (1, 0, 0), (40, 9, 13), (0, 16, 16), (300, 3, 5), (5, 17, 31), (12, 1, 1)]
EDIT = [(9, 5, 7), (0, 16, 16), (33, 11, 3), (4, 1, 1)]


def _inputs(samples, frames, c, seed):
    p, pos = _layout(samples, frames)
    n, s = p["n_tokens"], p["n_packed"]
    d = workloads.block_inputs(seed, n, s, c)
    return p, pos, n, s, d


@pytest.mark.parametrize("frames,c", [(1, 512), (1, 3072), (2, 1024)])
def test_adaln_modulate(frames, c):
    mf = _mf()
    samples = EDIT if frames == 2 else SAMPLES
    p, _, n, s, d = _inputs(samples, frames, c, 31 + c)
    note(f"test_adaln_modulate frames={frames} C={c} N={n}")
    cu = _i32(p["cu_pieces"])
    x = dev(d["x"], "bf16")
    h = mf.adaln_modulate(x, _f32(d["shift"]), _f32(d["scale"]), cu, s, frames)
    torch.cuda.synchronize()
    ref = block.adaln_modulate(_bf(d["x"]), d["shift"], d["scale"], p["cu_pieces"], s, frames)
    _within_ulp(host_f64(h), ref, "h")
    # in place
    mf.adaln_modulate(x, _f32(d["shift"]), _f32(d["scale"]), cu, s, frames, out=x)
    torch.cuda.synchronize()
    _within_ulp(host_f64(x), ref, "h (in place)")


@pytest.mark.parametrize("frames,heads,hd,bias,rotate", [
    (1, 4, 128, True, True), (1, 8, 64, False, True), (1, 4, 128, True, False), (2, 2, 128, True, True),
    (2, 4, 64, True, True)])
def test_qkv_rope(frames, heads, hd, bias, rotate):
    mf = _mf()
    c = heads * hd
    samples = EDIT if frames == 2 else SAMPLES
    p, pos, n, s, d = _inputs(samples, frames, c, 41 + c + frames)
    note(f"test_qkv_rope frames={frames} H={heads} D={hd} bias={bias} rotate={rotate} N={n}")
    h = workloads.normal(43, 1, (n, c), "bf16")
    w = (dev(d["w_qkv0"], "bf16"), dev(d["w_qkv1"], "bf16"))
    b = (_f32(d["b_qkv0"]), _f32(d["b_qkv1"])) if bias else (None, None)
    max_pos = int(pos.max()) + 1
    q, k, v = mf.qkv_rope(dev(h, "bf16"), w, b, _i32(p["cu_pieces"]), s, frames, _i32(pos) if rotate else None,
                          heads, THETA, max_pos)
    torch.cuda.synchronize()
    rq, rk, rv = block.qkv_rope(_bf(h), (_bf(d["w_qkv0"]), _bf(d["w_qkv1"])),
                                (d["b_qkv0"], d["b_qkv1"]) if bias else (None, None), p["cu_pieces"], s, frames,
                                pos if rotate else None, heads, hd, THETA)
    _within_ulp(host_f64(q), rq, "q")
    _within_ulp(host_f64(k), rk, "k")
    _within_ulp(host_f64(v), rv, "v")


@pytest.mark.parametrize("frames,c,in_place", [(1, 512, False), (1, 1024, True), (2, 768, False)])
def test_out_gated_residual(frames, c, in_place):
    mf = _mf()
    samples = EDIT if frames == 2 else SAMPLES
    p, _, n, s, d = _inputs(samples, frames, c, 51 + c)
    note(f"test_out_gated_residual frames={frames} C={c} in_place={in_place} N={n}")
    x = dev(d["x"], "bf16")
    y = mf.out_gated_residual(dev(d["o"], "bf16"), x, (dev(d["w_o0"], "bf16"), dev(d["w_o1"], "bf16")),
                              (_f32(d["b_o0"]), _f32(d["b_o1"])), _f32(d["gate"]), _i32(p["cu_pieces"]), s, frames,
                              out=x if in_place else None)
    torch.cuda.synchronize()
    ref = block.out_gated_residual(_bf(d["o"]), _bf(d["x"]), (_bf(d["w_o0"]), _bf(d["w_o1"])),
                                   (d["b_o0"], d["b_o1"]), d["gate"], p["cu_pieces"], s, frames)
    _within_ulp(host_f64(y), ref, "y")


def test_chain_norm_projection_attention_projection():
    """x -> adaLN -> QKV + RoPE -> attention (q, k already rotated) -> gated residual, against the oracle's
    float64 chain from the same inputs (each GPU stage rounds to bf16)."""
    mf = _mf()
    heads, hd = 4, 128
    c = heads * hd
    p, pos, n, s, d = _inputs(SAMPLES, 1, c, 61)
    note(f"test_chain N={n} C={c}")
    cu = _i32(p["cu_pieces"])
    max_pos = int(pos.max()) + 1
    h = mf.adaln_modulate(dev(d["x"], "bf16"), _f32(d["shift"]), _f32(d["scale"]), cu, s, 1)
    q, k, v = mf.qkv_rope(h, (dev(d["w_qkv0"], "bf16"), dev(d["w_qkv1"], "bf16")),
                          (_f32(d["b_qkv0"]), _f32(d["b_qkv1"])), cu, s, 1, _i32(pos), heads, THETA, max_pos)
    cu_seq = _i32(p["cu_seqlens"])
    o, _ = mf.attn_fwd(q, k, v, cu_seq, int(p["max_seqlen"]), None, THETA, max_pos, n_segments=s)
    y = mf.out_gated_residual(o.reshape(n, c), dev(d["x"], "bf16"),
                              (dev(d["w_o0"], "bf16"), dev(d["w_o1"], "bf16")), (_f32(d["b_o0"]), _f32(d["b_o1"])),
                              _f32(d["gate"]), cu, s, 1)
    torch.cuda.synchronize()
    rh = block.adaln_modulate(_bf(d["x"]), d["shift"], d["scale"], p["cu_pieces"], s, 1)
    rq, rk, rv = block.qkv_rope(rh, (_bf(d["w_qkv0"]), _bf(d["w_qkv1"])), (d["b_qkv0"], d["b_qkv1"]),
                                p["cu_pieces"], s, 1, pos, heads, hd, THETA)
    ro, _ = oracle.attn_fwd(rq, rk, rv, p["cu_seqlens"], None, THETA)
    ry = block.out_gated_residual(ro.reshape(n, c), _bf(d["x"]), (_bf(d["w_o0"]), _bf(d["w_o1"])),
                                  (d["b_o0"], d["b_o1"]), d["gate"], p["cu_pieces"], s, 1)
    assert_close_scaled(host_f64(q), rq, "q")
    assert_close_scaled(host_f64(o).reshape(n, c), ro.reshape(n, c), "o")
    # y = x + gate * proj with gate ~ 0.1: its error is the projection's, scaled down
    err = np.abs(host_f64(y) - ry)
    print(f"  y: max_abs={err.max():.3e} rms={np.sqrt((err ** 2).mean()):.3e}", flush=True)
    assert err.max() < 2e-2 and np.sqrt((err ** 2).mean()) < 2e-3


def _sub_layout(cu_pieces, n_samples, per, rows):
    """cu_pieces of the sampled rows (sorted), with every row keeping its sample and modality."""
    cp = np.asarray(cu_pieces)
    counts = [int(np.sum((rows >= cp[i]) & (rows < cp[i + 1]))) for i in range(per * n_samples)]
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def test_full_size_mixed_pack_sampled_rows():
    """The mixed 50k-token training pack at the model width (24 heads x 128 = 3072 channels), in the launch
    configuration the benchmark times; 96 sampled rows per stage (first, last and middle rows of every piece
    plus random ones) against the oracle on those rows."""
    mf = _mf()
    w = workloads.mixed50k()
    heads, hd = w.n_heads, w.head_dim
    c = heads * hd
    p, pos = _layout(w.samples, 1, w.budget)
    n, s = p["n_tokens"], p["n_packed"]
    note(f"test_full_size N={n} S={s} C={c}")
    d = workloads.block_inputs(71, n, s, c)
    cu = _i32(p["cu_pieces"])
    max_pos = int(pos.max()) + 1
    h = mf.adaln_modulate(dev(d["x"], "bf16"), _f32(d["shift"]), _f32(d["scale"]), cu, s, 1)
    q, k, v = mf.qkv_rope(h, (dev(d["w_qkv0"], "bf16"), dev(d["w_qkv1"], "bf16")),
                          (_f32(d["b_qkv0"]), _f32(d["b_qkv1"])), cu, s, 1, _i32(pos), heads, THETA, max_pos)
    y = mf.out_gated_residual(dev(d["o"], "bf16"), dev(d["x"], "bf16"),
                              (dev(d["w_o0"], "bf16"), dev(d["w_o1"], "bf16")), (_f32(d["b_o0"]), _f32(d["b_o1"])),
                              _f32(d["gate"]), cu, s, 1)
    torch.cuda.synchronize()
    cp = np.asarray(p["cu_pieces"])
    rng = np.random.default_rng(72)
    pick = set()
    for i in range(len(cp) - 1):
        if cp[i + 1] > cp[i]:
            pick.update({int(cp[i]), int(cp[i + 1]) - 1, int((cp[i] + cp[i + 1]) // 2)})
    pick.update(int(r) for r in rng.integers(0, n, 96 - min(len(pick), 96)))
    rows = np.array(sorted(pick))
    sub = _sub_layout(cp, s, 2, rows)
    xs = _bf(d["x"][rows])
    rh = block.adaln_modulate(xs, d["shift"], d["scale"], sub, s, 1)
    _within_ulp(host_f64(h)[rows], rh, "h")
    hs = host_f64(h)[rows]  # the GPU's h feeds the projection's oracle
    rq, rk, rv = block.qkv_rope(hs, (_bf(d["w_qkv0"]), _bf(d["w_qkv1"])), (d["b_qkv0"], d["b_qkv1"]), sub, s, 1,
                                pos[rows], heads, hd, THETA)
    _within_ulp(host_f64(q)[rows], rq, "q")
    _within_ulp(host_f64(k)[rows], rk, "k")
    _within_ulp(host_f64(v)[rows], rv, "v")
    ry = block.out_gated_residual(_bf(d["o"][rows]), xs, (_bf(d["w_o0"]), _bf(d["w_o1"])), (d["b_o0"], d["b_o1"]),
                                  d["gate"], sub, s, 1)
    _within_ulp(host_f64(y)[rows], ry, "y")


def test_empty_and_malformed_pieces():
    mf = _mf()
    c = 512
    note("test_empty_and_malformed_pieces")
    d = workloads.block_inputs(81, 300, 2, c)
    w = (dev(d["w_o0"], "bf16"), dev(d["w_o1"], "bf16"))
    gate = _f32(d["gate"])
    # no tokens: nothing is launched
    e = torch.empty((0, c), dtype=torch.bfloat16, device="cuda")
    mf.out_gated_residual(e, e, w, (None, None), gate, _i32([0, 0, 0, 0, 0]), 2, 1)
    mf.adaln_modulate(e, gate, gate, _i32([0, 0, 0, 0, 0]), 2, 1)
    # cu_pieces running past n_tokens (device data the host cannot check): rows are clamped to the tensor,
    # the rows inside it are computed as if the last piece ended at n_tokens
    x = dev(d["x"], "bf16")
    o = dev(d["o"], "bf16")
    y = mf.out_gated_residual(o, x, w, (None, None), gate, _i32([0, 10, 200, 250, 900]), 2, 1)
    torch.cuda.synchronize()
    ref = block.out_gated_residual(_bf(d["o"]), _bf(d["x"]), (_bf(d["w_o0"]), _bf(d["w_o1"])), (None, None),
                                   d["gate"], [0, 10, 200, 250, 300], 2, 1)
    _within_ulp(host_f64(y), ref, "y (clamped)")

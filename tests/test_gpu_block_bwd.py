"""GPU parity of the sub-block chains' backward (adaptive norm, QKV projection
with the rotary embedding, output projection with the gated residual) against
oracle.block's backward (float64) on the same bf16 / fp32 input values.

Bars, derived from the arithmetic (u = 2^-24, the fp32 unit roundoff):
* bf16 outputs (dx, dh, d_o) round once after fp32 arithmetic: one bf16 ulp,
  |err| <= |ref| 2^-7, plus the fp32 error of a K-term dot product,
  <= K u sum|terms|, plus -- where the GPU rounds an operand to bf16 before
  its matrix product (u = gate dy of the output projection, the inverse-
  rotated dq, dk of the QKV projection) -- 2^-8 sum|terms| (half a bf16 ulp is
  at most 2^-8 of the operand: 8 significand bits).  sum|terms| is the
  oracle's own result on absolute values.
* fp32 sums over rows (weight, bias, modulation gradients): <= (K + 64) u
  sum|terms| (recursive summation over K rows plus the fixed-order block
  reduction), plus the 2^-8 term for a rounded operand, and for dgate the
  forward's bf16 rounding of proj (one ulp, 2^-8 |proj|).
* The worst-case bars leave single-term mistakes near their edge, so every
  output also meets a relative RMS bar (rms(err) / rms(ref)), set far above
  the random-walk error of fp32 sums (about u sqrt(K), 1e-5 here) and far
  below the effect of any dropped or misplaced term.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import dev, host_f64, note
from oracle import block

pytestmark = pytest.mark.gpu
THETA = 10000.0
U = 2.0 ** -24


def _mf():
    import packed_varlen_attention_amd as mf
    return mf


def _check(got, ref, bar, label, rms_rel):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    worst = float((err - bar).max()) if err.size else -1.0
    rref = float(np.sqrt((ref ** 2).mean())) if ref.size else 0.0
    rel = float(np.sqrt((err ** 2).mean())) / rref if rref > 0 else float(err.max(initial=0.0))
    print(f"  {label}: max_abs={float(err.max(initial=0.0)):.3e} rms_rel={rel:.2e} n={err.size}", flush=True)
    assert worst <= 0, f"{label}: exceeds its bar by {worst:.3e}"
    assert rel <= rms_rel, f"{label}: relative RMS error {rel:.2e} > {rms_rel:.1e}"


def _layout(samples, frames, budget=1 << 22):
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


def _host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _modality_rows(cu_pieces, n_samples, frames):
    """Token count of each modality (the K of its row sums)."""
    k = [0, 0]
    for a, e, _, m in block.row_groups(cu_pieces, n_samples, frames):
        k[m] += e - a
    return k


# ragged pieces: a text-only sample, a zero-text sample, pieces below, at and past one 256-row tile
SAMPLES = [(7, 4, 6), (1, 0, 0), (40, 9, 13), (0, 16, 16), (300, 3, 5), (5, 17, 31), (12, 1, 1)]
EDIT = [(9, 5, 7), (0, 16, 16), (33, 11, 3), (4, 1, 1)]


def _inputs(samples, frames, c, seed):
    p, pos = _layout(samples, frames)
    n, s = p["n_tokens"], p["n_packed"]
    return p, pos, n, s, workloads.block_inputs(seed, n, s, c), workloads.block_grads(seed + 1, n, c)


# ---------------------------------------------------------------------------
# adaptive norm

def _adaln_abs_sums(dh, x, cu, s, frames):
    """(sum |dh|, sum |dh| |xhat|) per (sample, modality): the magnitude of the modulation gradients' terms."""
    c = x.shape[1]
    a1 = np.zeros((s, 2, c))
    a2 = np.zeros((s, 2, c))
    xhat = block.layer_norm(x)
    for a, e, si, m in block.row_groups(cu, s, frames):
        a1[si, m] += np.abs(dh[a:e]).sum(axis=0)
        a2[si, m] += (np.abs(dh[a:e]) * np.abs(xhat[a:e])).sum(axis=0)
    return a1, a2


def _dx_bar(ref):
    # one ulp, plus a floor of 2^-14 of the row's RMS for elements where the three terms of dx cancel
    row = np.sqrt((ref ** 2).mean(axis=1, keepdims=True))
    return np.abs(ref) * 2.0 ** -7 + row * 2.0 ** -14 + 1e-6


@pytest.mark.parametrize("frames,c,with_dres", [(1, 512, False), (1, 3072, True), (2, 1024, True), (1, 4608, False)])
def test_adaln_modulate_bwd(frames, c, with_dres):
    mf = _mf()
    samples = EDIT if frames == 2 else SAMPLES
    p, _, n, s, d, g = _inputs(samples, frames, c, 101 + c)
    note(f"test_adaln_modulate_bwd frames={frames} C={c} dres={with_dres} N={n}")
    cu = p["cu_pieces"]
    dres = dev(g["dq"], "bf16") if with_dres else None
    dx, dsh, dsc = mf.adaln_modulate_bwd(dev(g["dy"], "bf16"), dev(d["x"], "bf16"), _f32(d["scale"]), _i32(cu), s,
                                         frames, dres=dres)
    torch.cuda.synchronize()
    x, dh = _bf(d["x"]), _bf(g["dy"])
    rdx, rsh, rsc = block.adaln_modulate_bwd(dh, x, d["shift"], d["scale"], cu, s, frames)
    if with_dres:
        rdx = rdx + _bf(g["dq"])
    _check(host_f64(dx), rdx, _dx_bar(rdx), "dx", 2.0 ** -8)
    k = max(_modality_rows(cu, s, frames))
    a1, a2 = _adaln_abs_sums(dh, x, cu, s, frames)
    _check(_host(dsh), rsh, (k + 64) * U * a1 + 1e-6, "dshift", 1e-4)
    # dscale: xhat from fp32 statistics (relative error ~1e-6 per element) on top of the summation
    _check(_host(dsc), rsc, ((k + 64) * U + 4e-6) * a2 + 1e-6, "dscale", 1e-4)
    if with_dres:  # dx written over dres: the same bits as out of place
        dx2, _, _ = mf.adaln_modulate_bwd(dev(g["dy"], "bf16"), dev(d["x"], "bf16"), _f32(d["scale"]), _i32(cu), s,
                                          frames, dres=dres, out=dres)
        torch.cuda.synchronize()
        assert dx2.data_ptr() == dres.data_ptr()
        assert torch.equal(dx2.view(torch.int16), dx.view(torch.int16))


# ---------------------------------------------------------------------------
# QKV projection with the rotary embedding

def _qkv_abs(dq, dk, dv, h, w, cu, s, frames, pos, heads, hd):
    """The oracle's backward on absolute values of the (inverse-rotated) gradients, inputs and weights."""
    n = h.shape[0]
    if pos is not None:
        dq = oracle.rope_axes(dq.reshape(n, heads, hd), pos, THETA, inverse=True)
        dk = oracle.rope_axes(dk.reshape(n, heads, hd), pos, THETA, inverse=True)
    sh = (n, heads, hd)
    return block.qkv_rope_bwd(np.abs(dq).reshape(sh), np.abs(dk).reshape(sh), np.abs(dv).reshape(sh), np.abs(h),
                              (np.abs(w[0]), np.abs(w[1])), cu, s, frames, None)


@pytest.mark.parametrize("frames,heads,hd,rotate,bias", [
    (1, 4, 128, True, True), (1, 8, 64, False, True), (1, 2, 128, False, False), (2, 2, 128, True, True),
    (2, 4, 64, True, False), (1, 24, 128, True, True)])
def test_qkv_rope_bwd(frames, heads, hd, rotate, bias):
    mf = _mf()
    c = heads * hd
    samples = EDIT if frames == 2 else SAMPLES
    p, pos, n, s, d, g = _inputs(samples, frames, c, 111 + c + frames)
    note(f"test_qkv_rope_bwd frames={frames} H={heads} D={hd} rotate={rotate} bias={bias} N={n}")
    cu = p["cu_pieces"]
    h = workloads.normal(113, 1, (n, c), "bf16")
    w = (d["w_qkv0"], d["w_qkv1"])
    max_pos = int(pos.max()) + 1
    dqkv = [dev(g[k], "bf16").view(n, heads, hd) for k in ("dq", "dk", "dv")]
    dh, dw, db = mf.qkv_rope_bwd(*dqkv, dev(h, "bf16"), (dev(w[0], "bf16"), dev(w[1], "bf16")), _i32(cu), s, frames,
                                 _i32(pos) if rotate else None, THETA, max_pos, bias=bias)
    torch.cuda.synchronize()
    sh = (n, heads, hd)
    gq, gk, gv = (_bf(g[k]).reshape(sh) for k in ("dq", "dk", "dv"))
    wf = (_bf(w[0]), _bf(w[1]))
    rdh, rdw, rdb = block.qkv_rope_bwd(gq, gk, gv, _bf(h), wf, cu, s, frames, pos if rotate else None, THETA)
    adh, adw, adb = _qkv_abs(gq, gk, gv, _bf(h), wf, cu, s, frames, pos if rotate else None, heads, hd)
    rnd = 2.0 ** -8 if rotate else 0.0  # the inverse-rotated dq, dk are rounded to bf16 for the products
    rms = 2.0 ** -8 if rotate else 1e-4
    _check(host_f64(dh), rdh, np.abs(rdh) * 2.0 ** -7 + (rnd + 3 * c * U) * adh + 1e-5, "dh", 2.0 ** -8)
    k = max(_modality_rows(cu, s, frames))
    for m in range(2):
        _check(_host(dw[m]), rdw[m], (rnd + (k + 64) * U) * adw[m] + 1e-6, f"dW[{m}]", rms)
        if bias:
            _check(_host(db[m]), rdb[m], (rnd + (k + 64) * U) * adb[m] + 1e-6, f"db[{m}]", rms)
        else:
            assert db[m] is None


# ---------------------------------------------------------------------------
# output projection with the gated residual

def _out_forward(mf, d, p, s, frames, c):
    """The forward with its pre-gate projection saved, checked against the oracle's projection."""
    n = p["n_tokens"]
    proj = torch.empty((n, c), dtype=torch.bfloat16, device="cuda")
    mf.out_gated_residual(dev(d["o"], "bf16"), dev(d["x"], "bf16"), (dev(d["w_o0"], "bf16"), dev(d["w_o1"], "bf16")),
                          (_f32(d["b_o0"]), _f32(d["b_o1"])), _f32(d["gate"]), _i32(p["cu_pieces"]), s, frames,
                          proj=proj)
    return proj


@pytest.mark.parametrize("frames,c", [(1, 512), (1, 3072), (2, 768)])
def test_out_gated_residual_bwd(frames, c):
    mf = _mf()
    samples = EDIT if frames == 2 else SAMPLES
    p, _, n, s, d, g = _inputs(samples, frames, c, 121 + c)
    note(f"test_out_gated_residual_bwd frames={frames} C={c} N={n}")
    cu = p["cu_pieces"]
    proj = _out_forward(mf, d, p, s, frames, c)
    torch.cuda.synchronize()
    o, x, dy = _bf(d["o"]), _bf(d["x"]), _bf(g["dy"])
    wf = (_bf(d["w_o0"]), _bf(d["w_o1"]))
    bf = (d["b_o0"], d["b_o1"])
    # the saved projection is the forward's pre-gate value: one bf16 ulp
    rproj = np.zeros((n, c))
    for a, e, _, m in block.row_groups(cu, s, frames):
        rproj[a:e] = block.linear(o[a:e], wf[m], bf[m])
    _check(host_f64(proj), rproj, np.abs(rproj) * 2.0 ** -7 + 1e-5, "proj", 2.0 ** -8)
    d_o, dw, db, dgate = mf.out_gated_residual_bwd(dev(g["dy"], "bf16"), dev(d["o"], "bf16"), proj,
                                                   (dev(d["w_o0"], "bf16"), dev(d["w_o1"], "bf16")),
                                                   _f32(d["gate"]), _i32(cu), s, frames)
    torch.cuda.synchronize()
    _, rdo, rdw, rdb, rdg = block.out_gated_residual_bwd(dy, o, x, wf, bf, d["gate"], cu, s, frames)
    _, ado, adw, adb, adg = block.out_gated_residual_bwd(np.abs(dy), np.abs(o), np.abs(x), (np.abs(wf[0]),
                                                         np.abs(wf[1])), (np.abs(bf[0]), np.abs(bf[1])),
                                                         np.abs(d["gate"]), cu, s, frames)
    rnd = 2.0 ** -8  # u = gate dy is rounded to bf16 for the products
    _check(host_f64(d_o), rdo, np.abs(rdo) * 2.0 ** -7 + (rnd + c * U) * ado + 1e-5, "d_o", 2.0 ** -8)
    k = max(_modality_rows(cu, s, frames))
    for m in range(2):
        _check(_host(dw[m]), rdw[m], (rnd + (k + 64) * U) * adw[m] + 1e-6, f"dW_o[{m}]", 2.0 ** -8)
        _check(_host(db[m]), rdb[m], (rnd + (k + 64) * U) * adb[m] + 1e-6, f"db_o[{m}]", 2.0 ** -8)
    # dgate = sum dy proj with the forward's bf16 proj (one ulp, 2^-8)
    _check(_host(dgate), rdg, (2.0 ** -8 + (k + 64) * U) * adg + 1e-6, "dgate", 2.0 ** -8)


# ---------------------------------------------------------------------------
# determinism, empty modalities, no tokens

def test_backward_is_deterministic():
    """Row sums run in a fixed order: two calls give identical bits."""
    mf = _mf()
    heads, hd, frames = 4, 128, 1
    c = heads * hd
    p, pos, n, s, d, g = _inputs(SAMPLES, frames, c, 131)
    note(f"test_backward_is_deterministic N={n}")
    cu = _i32(p["cu_pieces"])
    dqkv = [dev(g[k], "bf16").view(n, heads, hd) for k in ("dq", "dk", "dv")]
    w = (dev(d["w_qkv0"], "bf16"), dev(d["w_qkv1"], "bf16"))
    wo = (dev(d["w_o0"], "bf16"), dev(d["w_o1"], "bf16"))
    proj = _out_forward(mf, d, p, s, frames, c)

    def run():
        a = mf.qkv_rope_bwd(*dqkv, dev(d["x"], "bf16"), w, cu, s, frames, _i32(pos), THETA, int(pos.max()) + 1)
        b = mf.out_gated_residual_bwd(dev(g["dy"], "bf16"), dev(d["o"], "bf16"), proj, wo, _f32(d["gate"]), cu, s,
                                      frames)
        e = mf.adaln_modulate_bwd(dev(g["dy"], "bf16"), dev(d["x"], "bf16"), _f32(d["scale"]), cu, s, frames)
        torch.cuda.synchronize()
        flat = [a[0], *a[1], *a[2], b[0], *b[1], *b[2], b[3], *e]
        return [t.clone() for t in flat]

    r1, r2 = run(), run()
    for i, (x1, x2) in enumerate(zip(r1, r2)):
        assert torch.equal(x1.view(torch.int16) if x1.dtype == torch.bfloat16 else x1.view(torch.int32),
                           x2.view(torch.int16) if x2.dtype == torch.bfloat16 else x2.view(torch.int32)), i


def test_modality_without_tokens_and_empty_pack():
    """No text tokens anywhere: the text weights' and biases' gradients are exactly zero, the image ones match
    the oracle; no tokens at all: every gradient is zero."""
    mf = _mf()
    heads, hd, frames = 4, 128, 1
    c = heads * hd
    samples = [(0, 8, 9), (0, 16, 16), (0, 3, 30)]
    p, pos, n, s, d, g = _inputs(samples, frames, c, 141)
    note(f"test_modality_without_tokens N={n}")
    cu = p["cu_pieces"]
    dqkv = [dev(g[k], "bf16").view(n, heads, hd) for k in ("dq", "dk", "dv")]
    h = workloads.normal(142, 1, (n, c), "bf16")
    w = (d["w_qkv0"], d["w_qkv1"])
    _, dw, db = mf.qkv_rope_bwd(*dqkv, dev(h, "bf16"), (dev(w[0], "bf16"), dev(w[1], "bf16")), _i32(cu), s, frames,
                                None)
    proj = _out_forward(mf, d, p, s, frames, c)
    _, dwo, dbo, dgate = mf.out_gated_residual_bwd(dev(g["dy"], "bf16"), dev(d["o"], "bf16"), proj,
                                                   (dev(d["w_o0"], "bf16"), dev(d["w_o1"], "bf16")),
                                                   _f32(d["gate"]), _i32(cu), s, frames)
    _, dsh, dsc = mf.adaln_modulate_bwd(dev(g["dy"], "bf16"), dev(d["x"], "bf16"), _f32(d["scale"]), _i32(cu), s,
                                        frames)
    torch.cuda.synchronize()
    for t in (dw[0], db[0], dwo[0], dbo[0], dgate[:, 0], dsh[:, 0], dsc[:, 0]):
        assert not bool(t.any())
    sh = (n, heads, hd)
    _, rdw, rdb = block.qkv_rope_bwd(*(_bf(g[k]).reshape(sh) for k in ("dq", "dk", "dv")), _bf(h),
                                     (_bf(w[0]), _bf(w[1])), cu, s, frames, None)
    k = n
    _, adw, adb = _qkv_abs(*(_bf(g[q]) for q in ("dq", "dk", "dv")), _bf(h), (_bf(w[0]), _bf(w[1])), cu, s, frames,
                           None, heads, hd)
    _check(_host(dw[1]), rdw[1], (k + 64) * U * adw[1] + 1e-6, "dW[image]", 1e-4)
    _check(_host(db[1]), rdb[1], (k + 64) * U * adb[1] + 1e-6, "db[image]", 1e-4)
    # no tokens: zero gradients everywhere (the outputs start as garbage, so zeros are written)
    e = torch.empty((0, heads, hd), dtype=torch.bfloat16, device="cuda")
    z = _i32([0, 0, 0, 0, 0])
    _, dw0, db0 = mf.qkv_rope_bwd(e, e, e, e.view(0, c), (dev(w[0], "bf16"), dev(w[1], "bf16")), z, 2, 1, None)
    _, dsh0, dsc0 = mf.adaln_modulate_bwd(e.view(0, c), e.view(0, c), _f32(d["scale"][:2]), z, 2, 1)
    torch.cuda.synchronize()
    for t in (*dw0, *db0, dsh0, dsc0):
        assert not bool(t.any())


@pytest.mark.parametrize("kind", ["mixed", "image_only", "text_only"])
def test_weight_gradient_token_chunks(kind):
    """Packs of ~8k tokens, where the weight gradients cut each modality's tokens into chunks (8 work items for
    these tile counts) and add the chunk sums in a second pass; with a modality empty, its single chunk writes
    zeros.  Both projections' weight and bias gradients against the oracle."""
    mf = _mf()
    heads, hd, frames = 4, 128, 1
    c = heads * hd
    rng = np.random.default_rng(161)
    if kind == "mixed":
        samples = [(int(rng.integers(1, 200)), int(rng.integers(4, 40)), int(rng.integers(4, 40))) for _ in range(14)]
    elif kind == "image_only":
        samples = [(0, int(rng.integers(8, 50)), int(rng.integers(8, 50))) for _ in range(10)]
    else:
        samples = [(int(rng.integers(100, 900)), 0, 0) for _ in range(14)]
    p, pos, n, s, d, g = _inputs(samples, frames, c, 163)
    assert mf.mf_qkv_rope_bwd_workspace_size(s, frames, n, heads, hd, 0) > 0
    note(f"test_weight_gradient_token_chunks {kind} N={n} S={s}")
    cu = p["cu_pieces"]
    k = max(_modality_rows(cu, s, frames))
    dqkv = [dev(g[q], "bf16").view(n, heads, hd) for q in ("dq", "dk", "dv")]
    w = (d["w_qkv0"], d["w_qkv1"])
    _, dw, db = mf.qkv_rope_bwd(*dqkv, dev(d["x"], "bf16"), (dev(w[0], "bf16"), dev(w[1], "bf16")), _i32(cu), s,
                                frames, None)
    proj = _out_forward(mf, d, p, s, frames, c)
    _, dwo, dbo, _ = mf.out_gated_residual_bwd(dev(g["dy"], "bf16"), dev(d["o"], "bf16"), proj,
                                               (dev(d["w_o0"], "bf16"), dev(d["w_o1"], "bf16")), _f32(d["gate"]),
                                               _i32(cu), s, frames)
    torch.cuda.synchronize()
    sh = (n, heads, hd)
    gq, gk, gv = (_bf(g[q]).reshape(sh) for q in ("dq", "dk", "dv"))
    wf = (_bf(w[0]), _bf(w[1]))
    _, rdw, rdb = block.qkv_rope_bwd(gq, gk, gv, _bf(d["x"]), wf, cu, s, frames, None)
    _, adw, adb = _qkv_abs(gq, gk, gv, _bf(d["x"]), wf, cu, s, frames, None, heads, hd)
    for m in range(2):
        _check(_host(dw[m]), rdw[m], (k + 64) * U * adw[m] + 1e-6, f"dW[{m}]", 1e-4)
        _check(_host(db[m]), rdb[m], (k + 64) * U * adb[m] + 1e-6, f"db[{m}]", 1e-4)
    wo, bo = (_bf(d["w_o0"]), _bf(d["w_o1"])), (d["b_o0"], d["b_o1"])
    o, x, dy = _bf(d["o"]), _bf(d["x"]), _bf(g["dy"])
    _, _, rdw, rdb, _ = block.out_gated_residual_bwd(dy, o, x, wo, bo, d["gate"], cu, s, frames)
    _, _, adw, adb, _ = block.out_gated_residual_bwd(np.abs(dy), np.abs(o), np.abs(x), (np.abs(wo[0]), np.abs(wo[1])),
                                                     (np.abs(bo[0]), np.abs(bo[1])), np.abs(d["gate"]), cu, s, frames)
    for m in range(2):
        _check(_host(dwo[m]), rdw[m], (2.0 ** -8 + (k + 64) * U) * adw[m] + 1e-6, f"dW_o[{m}]", 2.0 ** -8)
        _check(_host(dbo[m]), rdb[m], (2.0 ** -8 + (k + 64) * U) * adb[m] + 1e-6, f"db_o[{m}]", 2.0 ** -8)
    empty = {"image_only": 0, "text_only": 1}.get(kind)
    if empty is not None:
        for t in (dw[empty], db[empty], dwo[empty], dbo[empty]):
            assert not bool(t.any())


def _chain_check(got, ref, label, rms_rel=2e-2):
    """Integration bar for gradients carried through several bf16-rounded stages (h, q, k, v, o, proj, u, d_o,
    dq, dk, dv): each rounding adds about 2^-8 / sqrt(3) relative RMS, so the composed error stays near 1%; a
    wrong or dropped term is off by O(100%).  The single chains' tests above carry the tight bars."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    rref = float(np.sqrt((ref ** 2).mean()))
    rel = float(np.sqrt((err ** 2).mean())) / rref
    print(f"  {label}: max_abs={float(err.max()):.3e} rms_rel={rel:.2e} max|ref|={float(np.abs(ref).max()):.3e}",
          flush=True)
    assert np.isfinite(got).all(), label
    assert rel <= rms_rel, f"{label}: relative RMS error {rel:.2e} > {rms_rel}"
    assert float(err.max()) <= 0.2 * float(np.abs(ref).max()), f"{label}: max error {float(err.max()):.3e}"


@pytest.mark.parametrize("frames", [1, 2])
def test_block_backward_chain(frames):
    """The attention sub-block's backward as a training step runs it: gated output projection -> attention
    (rotated q, k from the QKV epilogue, so pos = NULL there) -> QKV projection with the inverse rotation ->
    adaLN, adding the residual path's dy into dx; against the oracle's forward and backward composed in
    float64 from the same inputs."""
    mf = _mf()
    heads, hd = 4, 128
    c = heads * hd
    samples = EDIT if frames == 2 else SAMPLES
    p, pos, n, s, d, g = _inputs(samples, frames, c, 171 + frames)
    note(f"test_block_backward_chain frames={frames} N={n} C={c}")
    cu = p["cu_pieces"]
    tcu, tcs = _i32(cu), _i32(p["cu_seqlens"])
    max_pos = int(pos.max()) + 1
    x = dev(d["x"], "bf16")
    wq = (dev(d["w_qkv0"], "bf16"), dev(d["w_qkv1"], "bf16"))
    bq = (_f32(d["b_qkv0"]), _f32(d["b_qkv1"]))
    wo = (dev(d["w_o0"], "bf16"), dev(d["w_o1"], "bf16"))
    bo = (_f32(d["b_o0"]), _f32(d["b_o1"]))
    gate, shift, scale = _f32(d["gate"]), _f32(d["shift"]), _f32(d["scale"])
    # forward
    h = mf.adaln_modulate(x, shift, scale, tcu, s, frames)
    q, k, v = mf.qkv_rope(h, wq, bq, tcu, s, frames, _i32(pos), heads, THETA, max_pos)
    o, lse = mf.attn_fwd(q, k, v, tcs, int(p["max_seqlen"]), None, THETA, max_pos, n_segments=s)
    proj = torch.empty_like(x)
    mf.out_gated_residual(o.reshape(n, c), x, wo, bo, gate, tcu, s, frames, proj=proj)
    # backward
    dy = dev(g["dy"], "bf16")
    d_o, dwo, dbo, dgate = mf.out_gated_residual_bwd(dy, o.reshape(n, c), proj, wo, gate, tcu, s, frames)
    dq, dk, dv = mf.attn_bwd(q, k, v, o, lse, d_o.view(n, heads, hd), tcs, int(p["max_seqlen"]), None, THETA,
                             max_pos, n_segments=s)
    dh, dwq, dbq = mf.qkv_rope_bwd(dq, dk, dv, h, wq, tcu, s, frames, _i32(pos), THETA, max_pos)
    dx, dsh, dsc = mf.adaln_modulate_bwd(dh, x, scale, tcu, s, frames, dres=dy)
    torch.cuda.synchronize()
    # oracle, float64 end to end
    xf = _bf(d["x"])
    wqf = (_bf(d["w_qkv0"]), _bf(d["w_qkv1"]))
    wof = (_bf(d["w_o0"]), _bf(d["w_o1"]))
    bqf, bof = (d["b_qkv0"], d["b_qkv1"]), (d["b_o0"], d["b_o1"])
    rh = block.adaln_modulate(xf, d["shift"], d["scale"], cu, s, frames)
    rq, rk, rv = block.qkv_rope(rh, wqf, bqf, cu, s, frames, pos, heads, hd, THETA)
    ro, _ = oracle.attn_fwd(rq, rk, rv, p["cu_seqlens"], None, THETA)
    rdy = _bf(g["dy"])
    _, rdo, rdwo, rdbo, rdg = block.out_gated_residual_bwd(rdy, ro.reshape(n, c), xf, wof, bof, d["gate"], cu, s,
                                                           frames)
    rdq, rdk, rdv = oracle.attn_bwd(rq, rk, rv, rdo.reshape(n, heads, hd), p["cu_seqlens"], None, THETA)
    rdh, rdwq, rdbq = block.qkv_rope_bwd(rdq, rdk, rdv, rh, wqf, cu, s, frames, pos, THETA)
    rdx, rsh, rsc = block.adaln_modulate_bwd(rdh, xf, d["shift"], d["scale"], cu, s, frames)
    rdx = rdx + rdy
    _chain_check(host_f64(d_o), rdo, "d_o")
    _chain_check(host_f64(dq).reshape(n, c), rdq.reshape(n, c), "dq (rotated)")
    _chain_check(host_f64(dh), rdh, "dh")
    _chain_check(host_f64(dx), rdx, "dx")
    for m in range(2):
        _chain_check(_host(dwo[m]), rdwo[m], f"dW_o[{m}]")
        _chain_check(_host(dbo[m]), rdbo[m], f"db_o[{m}]")
        _chain_check(_host(dwq[m]), rdwq[m], f"dW_qkv[{m}]")
        _chain_check(_host(dbq[m]), rdbq[m], f"db_qkv[{m}]")
    _chain_check(_host(dgate), rdg, "dgate")
    _chain_check(_host(dsh), rsh, "dshift")
    _chain_check(_host(dsc), rsc, "dscale")


# ---------------------------------------------------------------------------
# full size, sampled

def _sub_layout(cu_pieces, n_samples, per, rows):
    """cu_pieces of the sampled rows (sorted), with every row keeping its sample and modality."""
    cp = np.asarray(cu_pieces)
    counts = [int(np.sum((rows >= cp[i]) & (rows < cp[i + 1]))) for i in range(per * n_samples)]
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)


def test_full_size_mixed_pack_sampled():
    """The mixed 50k-token training pack at the model width (24 heads x 128 = 3072 channels), the launch
    configuration the benchmark times.  Row outputs (dx, dh, d_o) on sampled rows; weight and bias gradients on
    sampled output features over all of a modality's tokens (the oracle's backward on column slices: dW[J][I]
    depends only on the gradient's columns J and the input's columns I); modulation gradients of sampled
    samples (the oracle on one sample's rows)."""
    mf = _mf()
    wl = workloads.mixed50k()
    heads, hd = wl.n_heads, wl.head_dim
    c = heads * hd
    p, pos = _layout(wl.samples, 1, wl.budget)
    n, s = p["n_tokens"], p["n_packed"]
    note(f"test_full_size_bwd N={n} S={s} C={c}")
    d = workloads.block_inputs(151, n, s, c)
    g = workloads.block_grads(152, n, c)
    cu = p["cu_pieces"]
    tcu = _i32(cu)
    max_pos = int(pos.max()) + 1
    dqkv = [dev(g[k], "bf16").view(n, heads, hd) for k in ("dq", "dk", "dv")]
    h = dev(d["x"], "bf16")  # any bf16 rows serve as the projection's input
    dh, dw, db = mf.qkv_rope_bwd(*dqkv, h, (dev(d["w_qkv0"], "bf16"), dev(d["w_qkv1"], "bf16")), tcu, s, 1,
                                 _i32(pos), THETA, max_pos)
    proj = _out_forward(mf, d, p, s, 1, c)
    d_o, dwo, dbo, dgate = mf.out_gated_residual_bwd(dev(g["dy"], "bf16"), dev(d["o"], "bf16"), proj,
                                                     (dev(d["w_o0"], "bf16"), dev(d["w_o1"], "bf16")),
                                                     _f32(d["gate"]), tcu, s, 1)
    dx, dsh, dsc = mf.adaln_modulate_bwd(dev(g["dy"], "bf16"), dev(d["x"], "bf16"), _f32(d["scale"]), tcu, s, 1)
    torch.cuda.synchronize()
    cp = np.asarray(cu)
    rng = np.random.default_rng(153)
    pick = set()
    for i in range(len(cp) - 1):
        if cp[i + 1] > cp[i]:
            pick.update({int(cp[i]), int(cp[i + 1]) - 1})
    pick.update(int(r) for r in rng.integers(0, n, 48))
    rows = np.array(sorted(pick))
    sub = _sub_layout(cp, s, 2, rows)
    sh = (len(rows), heads, hd)
    grads = {k: _bf(g[k][rows]) for k in g}
    wq = (_bf(d["w_qkv0"]), _bf(d["w_qkv1"]))
    # dh on the sampled rows
    rdh, _, _ = block.qkv_rope_bwd(grads["dq"].reshape(sh), grads["dk"].reshape(sh), grads["dv"].reshape(sh),
                                   _bf(d["x"][rows]), wq, sub, s, 1, pos[rows], THETA)
    adh, _, _ = _qkv_abs(grads["dq"], grads["dk"], grads["dv"], _bf(d["x"][rows]), wq, sub, s, 1, pos[rows], heads,
                         hd)
    _check(host_f64(dh)[rows], rdh, np.abs(rdh) * 2.0 ** -7 + (2.0 ** -8 + 3 * c * U) * adh + 1e-5, "dh rows",
           2.0 ** -8)
    # dW_qkv[J][I], db_qkv[J]: head 5's q, k and v features J against 64 input features I
    hsel = 5
    fj = np.concatenate([part * c + hsel * hd + np.arange(hd) for part in range(3)])
    fi = np.sort(rng.choice(c, 64, replace=False))
    gsl = {k: _bf(g[k][:, hsel * hd:(hsel + 1) * hd]).reshape(n, 1, hd) for k in ("dq", "dk", "dv")}
    xi = _bf(d["x"][:, fi])
    wsl = (wq[0][np.ix_(fj, fi)], wq[1][np.ix_(fj, fi)])
    possel = pos  # rotation of head hsel uses the full positions
    _, rdw, rdb = block.qkv_rope_bwd(gsl["dq"], gsl["dk"], gsl["dv"], xi, wsl, cu, s, 1, possel, THETA)
    _, adw, adb = _qkv_abs(gsl["dq"], gsl["dk"], gsl["dv"], xi, wsl, cu, s, 1, possel, 1, hd)
    k = max(_modality_rows(cu, s, 1))
    for m in range(2):
        got = _host(dw[m])[np.ix_(fj, fi)]
        _check(got, rdw[m], (2.0 ** -8 + (k + 64) * U) * adw[m] + 1e-6, f"dW_qkv[{m}] sampled", 2.0 ** -8)
        _check(_host(db[m])[fj], rdb[m], (2.0 ** -8 + (k + 64) * U) * adb[m] + 1e-6, f"db_qkv[{m}] sampled",
               2.0 ** -8)
    # output projection: d_o on the sampled rows
    wo = (_bf(d["w_o0"]), _bf(d["w_o1"]))
    bo = (d["b_o0"], d["b_o1"])
    _, rdo, _, _, _ = block.out_gated_residual_bwd(grads["dy"], _bf(d["o"][rows]), _bf(d["x"][rows]), wo, bo,
                                                   d["gate"], sub, s, 1)
    _, ado, _, _, _ = block.out_gated_residual_bwd(np.abs(grads["dy"]), np.abs(_bf(d["o"][rows])),
                                                   np.abs(_bf(d["x"][rows])), (np.abs(wo[0]), np.abs(wo[1])),
                                                   (np.abs(bo[0]), np.abs(bo[1])), np.abs(d["gate"]), sub, s, 1)
    _check(host_f64(d_o)[rows], rdo, np.abs(rdo) * 2.0 ** -7 + (2.0 ** -8 + c * U) * ado + 1e-5, "d_o rows",
           2.0 ** -8)
    # dW_o[J][:], db_o[J], dgate[:, :, J] for 32 output features J over all tokens
    fj = np.sort(rng.choice(c, 32, replace=False))
    wj = (wo[0][fj], wo[1][fj])
    bj = (bo[0][fj], bo[1][fj])
    dyj = _bf(g["dy"][:, fj])
    oall = _bf(d["o"])
    _, _, rdw, rdb, rdg = block.out_gated_residual_bwd(dyj, oall, dyj, wj, bj, d["gate"][:, :, fj], cu, s, 1)
    _, _, adw, adb, adg = block.out_gated_residual_bwd(np.abs(dyj), np.abs(oall), np.abs(dyj),
                                                       (np.abs(wj[0]), np.abs(wj[1])), (np.abs(bj[0]), np.abs(bj[1])),
                                                       np.abs(d["gate"][:, :, fj]), cu, s, 1)
    for m in range(2):
        _check(_host(dwo[m])[fj], rdw[m], (2.0 ** -8 + (k + 64) * U) * adw[m] + 1e-6, f"dW_o[{m}] sampled", 2.0 ** -8)
        _check(_host(dbo[m])[fj], rdb[m], (2.0 ** -8 + (k + 64) * U) * adb[m] + 1e-6, f"db_o[{m}] sampled", 2.0 ** -8)
    _check(_host(dgate)[:, :, fj], rdg, (2.0 ** -8 + (k + 64) * U) * adg + 1e-6, "dgate sampled", 2.0 ** -8)
    # adaptive norm: dx on the sampled rows, dshift / dscale of four samples
    rdx, _, _ = block.adaln_modulate_bwd(grads["dy"], _bf(d["x"][rows]), d["shift"], d["scale"], sub, s, 1)
    _check(host_f64(dx)[rows], rdx, _dx_bar(rdx), "dx rows", 2.0 ** -8)
    for si in sorted(set(rng.integers(0, s, 4).tolist())):
        a, b = int(cp[2 * si]), int(cp[2 * si + 2])
        one = [0, int(cp[2 * si + 1]) - a, b - a]
        xs, dys = _bf(d["x"][a:b]), _bf(g["dy"][a:b])
        _, rsh, rsc = block.adaln_modulate_bwd(dys, xs, d["shift"][si:si + 1], d["scale"][si:si + 1], one, 1, 1)
        a1, a2 = _adaln_abs_sums(dys, xs, one, 1, 1)
        kk = b - a
        _check(_host(dsh)[si:si + 1], rsh, (kk + 64) * U * a1 + 1e-6, f"dshift sample {si}", 1e-4)
        _check(_host(dsc)[si:si + 1], rsc, ((kk + 64) * U + 4e-6) * a2 + 1e-6, f"dscale sample {si}", 1e-4)

"""Write-side boundary of the attention calls (include/mf.h): o, lse, dq, dk
and dv rows outside every segment are not written, nothing past n_tokens is
written, and every element of every segment is.  The rotated buffer's Q half
follows the same rule; its K half is written for every row in [0, n_tokens).

The pack is placed inside a longer token range: rows before cu_seqlens[0]
and after cu_seqlens[-1] belong to no segment, and every buffer carries
guard rows past n_tokens.  All outputs start as a NaN bit pattern that no
computation produces; afterwards the untouched rows must hold it bit for bit,
the written ones must not, and the in-segment results must equal a run on
the pack alone, bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import THETA, dev, note

pytestmark = pytest.mark.gpu

RAGGED = [(7, 9, 13), (1, 0, 0), (300, 0, 0), (33, 10, 10), (0, 1, 1), (0, 0, 0), (5, 17, 3), (129, 0, 0)]
FRONT, TAIL, GUARD = 37, 29, 5
# Runs of tiny segments share a tile by the 128-token window of the stream
# their first tokens fall in; padding the front by a multiple of 128 keeps
# the same groups, so the padded run still equals the pack alone bit for bit.
FRONT_TINY = 128
NAN16 = 0x7FC1          # bf16 NaN with a payload no rounding produces
NAN32 = 0x7FC00ACE      # fp32 NaN, likewise


def _tiny():
    rng = np.random.default_rng(94)
    return [(int(rng.integers(0, 40)), int(rng.integers(0, 5)), int(rng.integers(0, 9))) for _ in range(70)]


def _mf():
    import packed_varlen_attention_amd as mf
    return mf


def _filled(shape, dtype):
    t = torch.empty(shape, dtype=dtype, device="cuda")
    if dtype == torch.float32:
        t.view(torch.int32).fill_(NAN32)
    else:
        t.view(torch.int16).fill_(NAN16)
    return t


def _is_pattern(t):
    if t.dtype == torch.float32:
        return t.view(torch.int32) == NAN32
    return t.view(torch.int16) == NAN16


@pytest.mark.parametrize("layout,dtype,d,editing", [
    ("ragged", "bf16", 128, False),
    ("ragged", "f32", 64, False),
    ("ragged", "bf16", 128, True),
    ("tiny", "bf16", 128, False),
])
def test_outputs_outside_segments_are_not_written(layout, dtype, d, editing):
    mf = _mf()
    samples = RAGGED if layout == "ragged" else _tiny()
    heads = 3
    p = (oracle.pack_edit if editing else oracle.pack)(samples, 1 << 20)
    pos_in = (oracle.positions_edit if editing else oracle.positions)(samples, p["n_packed"])
    nax = 3 if editing else 2
    n_pack, n_seg = p["n_tokens"], p["n_packed"]
    front = FRONT_TINY if layout == "tiny" else FRONT
    n = front + n_pack + TAIL
    rows = n + GUARD
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    # inputs over the whole range (padding rows hold ordinary values too)
    q, k, v = workloads.qkv(51, rows, heads, d, dtype)
    do = workloads.dout(51, rows, heads, d, dtype)
    tq, tk, tv, tdo = (dev(x, dtype) for x in (q, k, v, do))
    pos = np.zeros((rows, nax), dtype=np.int32)
    pos[front:front + n_pack] = pos_in.reshape(-1, nax)
    tpos = torch.from_numpy(pos).cuda()
    cu = torch.from_numpy((p["cu_seqlens"] + front).astype(np.int32)).cuda()
    max_pos = max(p["max_pos"], 1)
    # outputs with guard rows, all holding the pattern
    o = _filled((rows, heads, d), tdt)
    lse_flat = _filled((heads * n + GUARD * heads,), torch.float32)
    grads = tuple(_filled((rows, heads, d), tdt) for _ in range(3))
    half = n * heads * d
    rot_flat = _filled((2 * half + GUARD * heads * d,), torch.bfloat16)
    lse = lse_flat[:heads * n].view(heads, n)
    rot = rot_flat[:2 * half].view(2, n, heads, d)
    note(f"canary {layout} {dtype} D{d} editing={editing} n={n} segments={n_seg}")
    mf.attn_fwd(tq[:n], tk[:n], tv[:n], cu, p["max_seqlen"], tpos[:n], THETA, max_pos, out=o[:n], lse=lse,
                n_segments=n_seg, rotated=rot)
    mf.attn_bwd(tq[:n], tk[:n], tv[:n], o[:n], lse, tdo[:n], cu, p["max_seqlen"], tpos[:n], THETA, max_pos,
                grads=tuple(g[:n] for g in grads), n_segments=n_seg, rotated=rot)
    torch.cuda.synchronize()

    a, b = front, front + n_pack
    outside = torch.ones(rows, dtype=torch.bool, device="cuda")
    outside[a:b] = False
    for t, name in zip((o,) + grads, ("O", "dQ", "dK", "dV")):
        pat = _is_pattern(t)
        assert pat[outside].all(), f"{name}: a row outside every segment or past n_tokens was written"
        assert not pat[a:b].any(), f"{name}: an element inside a segment was not written"
        assert torch.isfinite(t[a:b].float()).all(), f"{name}: non-finite value inside a segment"
    pat = _is_pattern(lse_flat)
    assert pat[heads * n:].all(), "LSE: the guard past heads * n_tokens was written"
    lp = pat[:heads * n].view(heads, n)
    assert lp[:, :a].all() and lp[:, b:].all(), "LSE: a column outside every segment was written"
    assert not lp[:, a:b].any() and torch.isfinite(lse[:, a:b]).all(), "LSE: a segment column was not written"
    rp = _is_pattern(rot_flat)
    assert rp[2 * half:].all(), "rotated: the guard past 2 * n_tokens rows was written"
    qp = rp[:half].view(n, heads, d)
    assert qp[:a].all() and qp[b:].all(), "rotated Q half: a row outside every segment was written"
    assert not qp[a:b].any(), "rotated Q half: a segment row was not written"
    assert not rp[half:2 * half].any(), "rotated K half: a row in [0, n_tokens) was not written"

    # the in-segment results equal a run on the pack alone, bit for bit
    note("canary reference run on the pack alone")
    sl = slice(a, b)
    cu0 = torch.from_numpy(p["cu_seqlens"].astype(np.int32)).cuda()
    p0 = tpos[sl].contiguous()
    o0, l0 = mf.attn_fwd(tq[sl].contiguous(), tk[sl].contiguous(), tv[sl].contiguous(), cu0, p["max_seqlen"], p0,
                         THETA, max_pos, n_segments=n_seg)
    g0 = mf.attn_bwd(tq[sl].contiguous(), tk[sl].contiguous(), tv[sl].contiguous(), o0, l0, tdo[sl].contiguous(),
                     cu0, p["max_seqlen"], p0, THETA, max_pos, n_segments=n_seg)
    torch.cuda.synchronize()
    for x, y, name in zip((o0, l0) + tuple(g0), (o[sl], lse[:, sl]) + tuple(g[sl] for g in grads),
                          ("O", "LSE", "dQ", "dK", "dV")):
        assert torch.equal(x, y), f"{name}: padding the pack changed its results"

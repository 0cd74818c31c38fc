"""The optional `rotated` buffer of the attention calls: the forward keeps the
rotated bf16 Q and K in it, and the backward reads them instead of rotating
again.  Forward outputs and gradients must be bit-identical to the calls
without it, and the buffer must hold exactly what the rotation calls
produce (Q first, then K), on every row of every segment.  When the calls
neither rotate nor convert (no positions, bf16 inputs), the buffer is left
untouched.
"""
import numpy as np
import pytest
import torch

from gpu_util import THETA, Case, merged_segments, note

pytestmark = pytest.mark.gpu

RAGGED = [(7, 9, 13), (1, 0, 0), (300, 0, 0), (33, 10, 10), (0, 1, 1), (64, 8, 8), (5, 17, 3), (2, 1, 62), (129, 0, 0)]


def _tiny():
    rng = np.random.default_rng(93)
    return [(int(rng.integers(0, 40)), int(rng.integers(0, 5)), int(rng.integers(0, 9))) for _ in range(60)]


def _mf():
    import packed_varlen_attention_amd as mf
    return mf


def _both(mf, c, pos, rotated):
    o, lse = mf.attn_fwd(c.tq, c.tk, c.tv, c.tcu, c.max_seqlen, pos, THETA, c.max_pos, rotated=rotated)
    g = mf.attn_bwd(c.tq, c.tk, c.tv, o, lse, c.tdo, c.tcu, c.max_seqlen, pos, THETA, c.max_pos, rotated=rotated)
    torch.cuda.synchronize()
    return (o, lse) + tuple(g)


@pytest.mark.parametrize("layout,dtype,d,editing,use_pos", [
    ("ragged", "bf16", 128, False, True),
    ("ragged", "bf16", 64, False, True),
    ("ragged", "f32", 128, False, True),
    ("ragged", "f32", 64, False, False),
    ("ragged", "bf16", 128, True, True),
    ("tiny", "bf16", 128, False, True),
    ("ragged", "bf16", 128, False, False),
])
def test_kept_rotation_is_bit_identical(layout, dtype, d, editing, use_pos):
    mf = _mf()
    samples = RAGGED if layout == "ragged" else _tiny()
    c = Case(samples, 1 << 20, 3, d, dtype, seed=37, with_dout=True, editing=editing)
    if layout == "tiny":
        assert merged_segments(c.cu), "layout must produce multi-segment tiles"
    pos = c.tpos if use_pos else None
    note(f"rotated buffer {layout} {c.describe()} rope={use_pos}")
    ref = _both(mf, c, pos, None)
    rot = mf.rotated_buffer(c.tq)
    rot.view(torch.int16).fill_(0x7FC1)  # a NaN pattern no rotation produces
    fill = rot.clone()
    got = _both(mf, c, pos, rot)
    for r, g, name in zip(ref, got, ("O", "LSE", "dQ", "dK", "dV")):
        assert torch.equal(r, g), f"{name} differs with the rotated buffer"
    n = c.n
    if not use_pos and dtype == "bf16":
        assert torch.equal(rot.view(torch.int16), fill.view(torch.int16)), "buffer written without a rotation pass"
        return
    for half, x in ((0, c.tq), (1, c.tk)):
        y = x.clone()
        if use_pos:
            rope = mf.rope3d_apply if editing else mf.rope2d_apply
            rope(y, c.tpos, THETA, c.max_pos)
        want = y.to(torch.bfloat16)
        assert torch.equal(rot[half, :n].view(torch.int16), want[:n].view(torch.int16)), \
            f"{'QK'[half]} half differs from the rotation call"

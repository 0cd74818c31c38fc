"""mf_varlen_attn_fwd_noalloc: the forward for callers that cannot allocate,
with its scratch in the library's fixed device array.  It runs the kernels of
mf_varlen_attn_fwd, so its O, LSE and rotated buffer must equal that call's
bit for bit -- on consecutive calls that reuse the array, the second on a
smaller pack, and without rotation.
"""
import pytest
import torch

import oracle
import workloads
from gpu_util import THETA, Case, assert_close, host_f64, note

pytestmark = pytest.mark.gpu

RAGGED = [(7, 9, 13), (1, 0, 0), (300, 0, 0), (33, 10, 10), (0, 1, 1), (5, 17, 3), (129, 0, 0)]


def _mf():
    import packed_varlen_attention_amd as mf
    return mf


def _pair(c: Case, use_pos: bool):
    """(O, LSE, rotated) from the workspace call and from the no-allocation
    call on the same inputs; outputs start as different NaN patterns."""
    mf = _mf()
    nseg = len(c.cu) - 1
    pos = c.tpos if use_pos else None
    outs = []
    for fill in (0x7FC1, 0x7FC3):
        o = torch.empty_like(c.tq)
        o.view(torch.int16).fill_(fill)
        lse = torch.full((c.heads, c.n), float("nan"), dtype=torch.float32, device="cuda")
        rot = mf.rotated_buffer(c.tq)
        rot.view(torch.int16).fill_(fill)
        outs.append((o, lse, rot))
    o, lse, rot = outs[0]
    note(f"mf_varlen_attn_fwd (workspace) {c.describe()} rope={use_pos}")
    mf.attn_fwd(c.tq, c.tk, c.tv, c.tcu, c.max_seqlen, pos, THETA, c.max_pos, out=o, lse=lse, n_segments=nseg,
                rotated=rot if use_pos else None)
    o2, lse2, rot2 = outs[1]
    note(f"mf_varlen_attn_fwd_noalloc {c.describe()} rope={use_pos}")
    mf._binding.mf_varlen_attn_fwd_noalloc(c.tq, c.tk, c.tv, o2, lse2, c.tcu, nseg, c.max_seqlen, pos, THETA,
                                           c.max_pos, 0.0, rot2 if use_pos else None)
    torch.cuda.synchronize()
    return (o, lse, rot), (o2, lse2, rot2)


def _assert_same(a, b, n, use_pos, label):
    (o, lse, rot), (o2, lse2, rot2) = a, b
    assert torch.equal(o[:n].view(torch.int16), o2[:n].view(torch.int16)), f"O differs ({label})"
    assert torch.equal(lse[:, :n], lse2[:, :n]), f"LSE differs ({label})"
    if use_pos:
        half = rot[0].numel()
        got = rot2.view(-1)
        want = rot.view(-1)
        # Q half: rows of segments; K half: every row
        assert torch.equal(rot[0, :n].view(torch.int16), rot2[0, :n].view(torch.int16)), f"rotated Q ({label})"
        assert torch.equal(want[half:].view(torch.int16), got[half:].view(torch.int16)), f"rotated K ({label})"


def test_noalloc_matches_the_workspace_call_on_consecutive_calls():
    # first call: the mixed 50k-token pack (24 heads x 128, the benchmark's shape)
    w = workloads.mixed50k()
    big = Case(w.samples, w.budget, w.n_heads, w.head_dim, w.dtype, w.seed)
    a, b = _pair(big, True)
    _assert_same(a, b, big.n, True, "mixed50k")
    # its output is the forward: spot-check one head against the oracle
    ro, rl = oracle.attn_fwd(big.q[:, 5:6], big.k[:, 5:6], big.v[:, 5:6], big.cu, big.pos, THETA)
    assert_close(host_f64(b[0])[:big.n, 5:6], ro[:big.n], 2e-2, 2e-3, "O no-alloc mixed50k head 5")
    assert_close(host_f64(b[1])[5:6, :big.n], rl[:, :big.n], 1e-2, 1e-2, "LSE no-alloc mixed50k head 5")
    # second call, smaller: the array keeps the first call's table and schedule
    small = Case(RAGGED, 1 << 20, 3, 128, "bf16", seed=61)
    assert small.n < big.n and len(small.cu) < len(big.cu) + 8
    a, b = _pair(small, True)
    _assert_same(a, b, small.n, True, "ragged after mixed50k")
    # without rotation (no positions, no rotated buffer), D = 64
    plain = Case(RAGGED[:4], 1 << 20, 2, 64, "bf16", seed=62)
    a, b = _pair(plain, False)
    _assert_same(a, b, plain.n, False, "no rotation")
    # and a larger table again after the smaller one
    again = Case([(500, 20, 30), (3, 2, 2)], 1 << 20, 2, 128, "bf16", seed=63)
    assert again.max_pos > small.max_pos
    a, b = _pair(again, True)
    _assert_same(a, b, again.n, True, "larger table after smaller")


def test_noalloc_refuses_what_it_cannot_hold():
    mf = _mf()
    c = Case(RAGGED[:3], 1 << 20, 1, 128, "bf16", seed=64)
    nseg = len(c.cu) - 1
    o = torch.empty_like(c.tq)
    err = mf._binding.MFError
    with pytest.raises(err) as e:  # a rotation needs the caller's rotated buffer
        mf._binding.mf_varlen_attn_fwd_noalloc(c.tq, c.tk, c.tv, o, None, c.tcu, nseg, c.max_seqlen, c.tpos, THETA,
                                               c.max_pos, 0.0, None)
    assert e.value.status == -1
    with pytest.raises(err) as e:  # table beyond the fixed scratch
        mf._binding.mf_varlen_attn_fwd_noalloc(c.tq, c.tk, c.tv, o, None, c.tcu, nseg, c.max_seqlen, c.tpos, THETA,
                                               1 << 15, 0.0, mf.rotated_buffer(c.tq))
    assert e.value.status == -5
    f = Case(RAGGED[:3], 1 << 20, 1, 128, "f32", seed=65)
    with pytest.raises(err) as e:  # float32 input
        mf._binding.mf_varlen_attn_fwd_noalloc(f.tq, f.tk, f.tv, torch.empty_like(f.tq), None, f.tcu, nseg,
                                               f.max_seqlen, f.tpos, THETA, f.max_pos, 0.0, None)
    assert e.value.status == -2

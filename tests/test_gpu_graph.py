"""The hot path captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library makes no allocation, copy, memset or synchronisation inside its
calls, so pack (with the hidden-row gather), the forward with LSE and the
backward can be recorded once and replayed.  Every replay, with eager work
and synchronisations between replays, must reproduce the eager results bit
for bit, and a replay after the inputs change in place must match a fresh
eager run on the new inputs.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_util import THETA, note

pytestmark = pytest.mark.gpu

SAMPLES = [(37, 9, 14), (0, 16, 16), (120, 0, 0), (5, 3, 7), (64, 12, 10), (300, 20, 20)]
BUDGET = 1024
ROW_BYTES = 512
H, D = 4, 128


def _mf():
    import packed_varlen_attention_amd as mf
    return mf


def _bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


class _Step:
    """Preallocated outputs and workspaces, so a step allocates nothing."""

    def __init__(self, mf, seed: int):
        rng = np.random.default_rng(seed)
        self.samples = torch.tensor(np.asarray(SAMPLES, dtype=np.int32)).cuda()
        self.rows, ptrs = [], ([], [])
        for (t, gh, gw) in SAMPLES:
            for lst, n in zip(ptrs, (max(t, 1), max(gh * gw, 1))):
                b = torch.from_numpy(rng.integers(0, 256, (n, ROW_BYTES), dtype=np.uint8)).cuda()
                self.rows.append(b)
                lst.append(b.data_ptr())
        self.ptrs = [torch.tensor(x, dtype=torch.int64).cuda() for x in ptrs]
        self.pk = mf.pack(self.samples, BUDGET, *self.ptrs, ROW_BYTES)
        torch.cuda.synchronize()
        self.n_packed, self.n, self.max_seqlen, self.max_pos = (int(x) for x in self.pk.counts.cpu().tolist())
        q, k, v = workloads.qkv(seed, self.n, H, D, "bf16")
        self.q, self.k, self.v = _bf16(q), _bf16(k), _bf16(v)
        self.do = _bf16(workloads.dout(seed, self.n, H, D, "bf16"))
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((H, self.n), dtype=torch.float32, device="cuda")
        self.grads = (torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v))
        from packed_varlen_attention_amd.api import attn_workspace
        self.ws_f = attn_workspace(self.q, self.n_packed, self.max_pos, False)
        self.ws_b = attn_workspace(self.q, self.n_packed, self.max_pos, True)

    def run(self, mf):
        pk = self.pk
        mf.pack(self.samples, BUDGET, *self.ptrs, ROW_BYTES, out=pk)
        mf.attn_fwd(self.q, self.k, self.v, pk.cu_seqlens, self.max_seqlen, pk.pos, THETA, self.max_pos,
                    out=self.o, lse=self.lse, workspace=self.ws_f, n_segments=self.n_packed)
        mf.attn_bwd(self.q, self.k, self.v, self.o, self.lse, self.do, pk.cu_seqlens, self.max_seqlen, pk.pos,
                    THETA, self.max_pos, workspace=self.ws_b, grads=self.grads, n_segments=self.n_packed)

    def outputs(self):
        pk = self.pk
        return [t.clone() for t in (pk.cu_seqlens, pk.cu_pieces, pk.pos[: self.n], pk.counts, pk.packed[: self.n],
                                    self.o, self.lse, *self.grads)]

    def clear(self):
        pk = self.pk
        for t in (pk.cu_seqlens, pk.cu_pieces, pk.pos, pk.counts, pk.packed, self.o, self.lse, *self.grads):
            t.zero_()


NAMES = ("cu_seqlens", "cu_pieces", "pos", "counts", "packed rows", "O", "LSE", "dQ", "dK", "dV")


def _assert_same(got, ref, label):
    for g, r, name in zip(got, ref, NAMES):
        assert torch.equal(g, r), f"{label}: {name} differs from the eager result"


def test_pack_forward_backward_graph_replays_bit_exact():
    mf = _mf()
    st = _Step(mf, seed=41)
    assert 1 < st.n_packed < len(SAMPLES) and st.n > 512  # the budget drops the last sample
    note(f"graph capture: pack + fwd + bwd N={st.n} segments={st.n_packed} H={H} D={D}")
    st.run(mf)
    torch.cuda.synchronize()
    eager = st.outputs()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.run(mf)  # warm-up on the capture stream's side, as torch recommends
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run(mf)
    torch.cuda.synchronize()

    for i in range(3):
        st.clear()
        torch.cuda.synchronize()
        note(f"graph replay {i}")
        g.replay()
        torch.cuda.synchronize()
        _assert_same(st.outputs(), eager, f"replay {i}")
        # eager work between replays: an unrelated eager step on its own buffers
        other = torch.randn(1 << 16, device="cuda").sum()
        torch.cuda.synchronize()
        assert torch.isfinite(other)

    # new inputs written in place: the replay reads them, as a fresh eager run does
    q2, _, _ = workloads.qkv(42, st.n, H, D, "bf16")
    st.q.copy_(_bf16(q2))
    torch.cuda.synchronize()
    st.run(mf)
    torch.cuda.synchronize()
    eager2 = st.outputs()
    assert not torch.equal(eager2[5], eager[5])
    for i in range(2):
        st.clear()
        torch.cuda.synchronize()
        note(f"graph replay on new inputs {i}")
        g.replay()
        torch.cuda.synchronize()
        _assert_same(st.outputs(), eager2, f"replay on new inputs {i}")
    del g

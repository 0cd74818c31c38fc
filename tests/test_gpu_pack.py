"""GPU parity of mf_pack against the oracle: bit-exact offsets, positions,
counts and gathered rows."""
import json
import pathlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import note, samples_dev

pytestmark = pytest.mark.gpu

GOLD = pathlib.Path(__file__).parent / "golden"


def _mf():
    import packed_varlen_attention_amd as mf
    return mf


def _check_pack(samples, budget, label):
    mf = _mf()
    note(f"mf_pack {label}: S={len(samples)} budget={budget}")
    r = mf.pack(samples_dev(samples), budget)
    torch.cuda.synchronize()
    ref = oracle.pack(samples, budget)
    n, ntok = ref["n_packed"], ref["n_tokens"]
    counts = r.counts.cpu().numpy().tolist()
    assert counts == [n, ntok, ref["max_seqlen"], ref["max_pos"]], (counts, ref)
    cu = r.cu_seqlens.cpu().numpy()
    assert cu[: n + 1].tolist() == ref["cu_seqlens"].tolist()
    assert (cu[n + 1:] == ntok).all()
    pieces = r.cu_pieces.cpu().numpy()
    assert pieces[: 2 * n + 1].tolist() == ref["cu_pieces"].tolist()
    assert (pieces[2 * n + 1:] == ntok).all()
    pos = r.pos.cpu().numpy()[:ntok]
    assert np.array_equal(pos, oracle.positions(samples, n).reshape(-1, 2))
    return r


def test_tiny_golden():
    g = json.loads((GOLD / "tiny_pack.json").read_text())
    mf = _mf()
    note("mf_pack tiny golden")
    r = mf.pack(samples_dev(g["samples"]), g["budget"])
    torch.cuda.synchronize()
    assert r.cu_seqlens.cpu().tolist() == g["cu_seqlens"]
    assert r.cu_pieces.cpu().tolist() == g["cu_pieces"]
    assert r.counts.cpu().tolist() == [g["n_packed"], g["n_tokens"], g["max_seqlen"], g["max_pos"]]
    assert r.pos.cpu().numpy()[: g["n_tokens"]].tolist() == g["pos"]


@pytest.mark.parametrize("seed", range(24))
def test_random_packs(seed):
    rng = np.random.default_rng(100 + seed)
    samples = workloads.random_samples(rng, int(rng.integers(1, 40)))
    budget = int(rng.integers(0, 3000))
    _check_pack(samples, budget, f"random seed={seed}")


def test_many_samples_multi_chunk_scan():
    rng = np.random.default_rng(7)
    samples = workloads.random_samples(rng, 2500, max_text=20, max_side=4)
    _check_pack(samples, 10 ** 9, "2500 samples")
    _check_pack(samples, 20_000, "2500 samples budget cut")


@pytest.mark.parametrize("name", ["cfg1024", "mixed50k", "stress"])
def test_workload_packs(name):
    w = getattr(workloads, name)()
    _check_pack(list(w.samples), w.budget, name)


def test_zero_budget_and_empty():
    _check_pack([(3, 2, 2)], 0, "zero budget")
    _check_pack([(0, 0, 0), (0, 0, 0)], 10, "all empty")
    _check_pack([(5, 0, 0), (0, 3, 0), (0, 0, 4)], 100, "degenerate grids")


def test_negative_descriptor_flags_error():
    mf = _mf()
    note("mf_pack negative descriptor")
    r = mf.pack(samples_dev([(3, 2, 2), (1, -1, 2)]), 100)
    torch.cuda.synchronize()
    assert r.counts.cpu().tolist() == [-1, 0, 0, 0]
    assert (r.cu_seqlens.cpu().numpy() == 0).all()


@pytest.mark.parametrize("row_bytes", [48, 6144, 20])
def test_gather_rows_bit_exact(row_bytes):
    mf = _mf()
    rng = np.random.default_rng(row_bytes)
    samples = [(3, 2, 5), (0, 4, 4), (7, 0, 0), (2, 3, 3), (50, 10, 10)]
    budget = 3 + 10 + 16 + 7 + 2 + 9 + 5  # last sample does not fit
    text = [rng.integers(0, 256, size=(max(t, 0), row_bytes), dtype=np.uint8) for (t, _, _) in samples]
    img = [rng.integers(0, 256, size=(gh, gw, row_bytes), dtype=np.uint8) for (_, gh, gw) in samples]
    # device buffers; an empty part gets a null pointer
    tbuf = [torch.from_numpy(x.reshape(-1)).cuda() if x.size else None for x in text]
    ibuf = [torch.from_numpy(x.reshape(-1)).cuda() if x.size else None for x in img]
    tptr = torch.tensor([b.data_ptr() if b is not None else 0 for b in tbuf], dtype=torch.int64).cuda()
    iptr = torch.tensor([b.data_ptr() if b is not None else 0 for b in ibuf], dtype=torch.int64).cuda()
    note(f"mf_pack gather row_bytes={row_bytes}")
    r = mf.pack(samples_dev(samples), budget, tptr, iptr, row_bytes)
    torch.cuda.synchronize()
    ref = oracle.pack(samples, budget)
    assert ref["n_packed"] == 4
    want = oracle.gather(text, img, ref["n_packed"])
    got = r.packed.cpu().numpy()[: ref["n_tokens"]]
    assert np.array_equal(got, want)

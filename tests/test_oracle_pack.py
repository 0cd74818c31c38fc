"""Pins for oracle.pack: hand-typed golden values, brute force, budget edge cases."""
import json
import pathlib

import numpy as np
import pytest

import oracle
import workloads

GOLD = pathlib.Path(__file__).parent / "golden"


def test_tiny_golden():
    g = json.loads((GOLD / "tiny_pack.json").read_text())
    w = workloads.tiny()
    assert [list(s) for s in w.samples] == g["samples"]
    p = oracle.pack(w.samples, g["budget"])
    assert p["n_packed"] == g["n_packed"]
    assert p["n_tokens"] == g["n_tokens"]
    assert p["cu_seqlens"].tolist() == g["cu_seqlens"]
    assert p["cu_pieces"].tolist() == g["cu_pieces"]
    assert p["max_seqlen"] == g["max_seqlen"]
    assert p["max_pos"] == g["max_pos"]
    assert oracle.positions(w.samples, p["n_packed"]).tolist() == g["pos"]


def _brute_force(samples, budget):
    """Token-at-a-time walker: a sample is streamed token by token and rolled
    back whole if it would cross the budget; packing stops there."""
    stream = []  # (segment, is_text, row, col)
    seg = 0
    for (t, gh, gw) in samples:
        mark = len(stream)
        tokens = []
        u = 0
        while u < t:
            tokens.append((seg, True, u, u))
            u += 1
        for idx in range(gh * gw):
            r, c = divmod(idx, gw)
            tokens.append((seg, False, t + r, t + c))
        if mark + len(tokens) > budget:
            break
        stream.extend(tokens)
        seg += 1
    counts = [0] * seg
    text_counts = [0] * seg
    for (s, is_text, _, _) in stream:
        counts[s] += 1
        text_counts[s] += is_text
    cu = [0]
    pieces = []
    for s in range(seg):
        pieces += [cu[-1], cu[-1] + text_counts[s]]
        cu.append(cu[-1] + counts[s])
    pieces.append(cu[-1])
    pos = [[r, c] for (_, _, r, c) in stream]
    max_pos = 1 + max((max(r, c) for r, c in pos), default=-1)
    return seg, cu, pieces, pos, max_pos, max(counts, default=0)


@pytest.mark.parametrize("seed", range(40))
def test_against_brute_force(seed):
    rng = np.random.default_rng(seed)
    samples = workloads.random_samples(rng, int(rng.integers(0, 12)))
    budget = int(rng.integers(0, 600))
    p = oracle.pack(samples, budget)
    n, cu, pieces, pos, max_pos, max_len = _brute_force(samples, budget)
    assert p["n_packed"] == n
    assert p["cu_seqlens"].tolist() == cu
    assert p["cu_pieces"].tolist() == pieces
    assert p["n_tokens"] == cu[-1]
    assert p["max_seqlen"] == max_len
    assert p["max_pos"] == max_pos
    assert oracle.positions(samples, n).tolist() == pos


def test_budget_prefix_not_best_fit():
    samples = [(10, 0, 0), (5, 2, 2), (1, 0, 0)]  # lengths 10, 9, 1
    p = oracle.pack(samples, 15)
    assert p["n_packed"] == 1 and p["n_tokens"] == 10  # third would fit, but packing stops
    p = oracle.pack(samples, 20)  # exact fit
    assert p["n_packed"] == 3 and p["n_tokens"] == 20
    assert p["cu_seqlens"].tolist() == [0, 10, 19, 20]
    assert p["cu_pieces"].tolist() == [0, 10, 10, 15, 19, 20, 20]


def test_first_sample_too_big_and_empty():
    p = oracle.pack([(3, 4, 4)], 10)
    assert p["n_packed"] == 0 and p["n_tokens"] == 0
    assert p["cu_seqlens"].tolist() == [0] and p["cu_pieces"].tolist() == [0]
    assert p["max_pos"] == 0 and p["max_seqlen"] == 0
    p = oracle.pack([], 10)
    assert p["n_packed"] == 0 and p["cu_seqlens"].tolist() == [0]


def test_zero_length_segments_are_kept():
    p = oracle.pack([(0, 0, 0), (2, 0, 5), (0, 1, 1)], 100)
    assert p["cu_seqlens"].tolist() == [0, 0, 2, 3]
    assert p["cu_pieces"].tolist() == [0, 0, 0, 2, 2, 2, 3]
    assert oracle.positions([(0, 0, 0), (2, 0, 5), (0, 1, 1)], 3).tolist() == [[0, 0], [1, 1], [0, 0]]


def test_negative_descriptor_rejected():
    with pytest.raises(ValueError):
        oracle.pack([(1, -1, 2)], 100)


def test_workload_shapes():
    # mixed pack: a maximal prefix under 50k
    w = workloads.mixed50k()
    p = oracle.pack(w.samples, w.budget)
    n = p["n_packed"]
    assert 0 < n < len(w.samples)
    assert p["n_tokens"] <= 50_000
    t, gh, gw = w.samples[n]
    assert p["n_tokens"] + t + gh * gw > 50_000
    # stress pack: 2048^2 + two panoramas + 64 thumbnails
    s = workloads.stress()
    ps = oracle.pack(s.samples, s.budget)
    assert ps["n_packed"] == 67 and ps["n_tokens"] == 30720
    assert ps["max_seqlen"] == 16384 + 512
    # CFG pack: cond/uncond alternate; uncond text is one token
    c = workloads.cfg1024()
    pc = oracle.pack(c.samples, c.budget)
    assert pc["n_packed"] == 8
    lens = np.diff(pc["cu_seqlens"])
    assert all(lens[1::2] == 4097) and all((lens[0::2] >= 4160) & (lens[0::2] <= 4608))


def test_gather_row_major_bytes():
    rng = np.random.default_rng(5)
    samples = [(2, 2, 3), (1, 1, 2)]
    text = [rng.integers(0, 256, size=(t, 8), dtype=np.uint8) for (t, _, _) in samples]
    img = [rng.integers(0, 256, size=(gh, gw, 8), dtype=np.uint8) for (_, gh, gw) in samples]
    out = oracle.gather(text, img, 2)
    assert out.shape == (11, 8)
    assert (out[0:2] == text[0]).all()
    assert (out[2] == img[0][0, 0]).all() and (out[3] == img[0][0, 1]).all()
    assert (out[5] == img[0][1, 0]).all() and (out[7] == img[0][1, 2]).all()
    assert (out[8] == text[1][0]).all() and (out[10] == img[1][0, 1]).all()

"""Helpers shared by the GPU parity tests (host <-> device marshalling and
error metrics).  Expected values always come from ``oracle``."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads

THETA = 10000.0


def note(msg: str) -> None:
    """Name the case about to run on the GPU (flushed, so it survives a crash)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host_f64(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return workloads.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def samples_dev(samples) -> torch.Tensor:
    return torch.tensor(np.asarray(samples, dtype=np.int32).reshape(-1, 3)).cuda()


def errors(got: np.ndarray, ref: np.ndarray):
    diff = np.abs(np.asarray(got, dtype=np.float64) - np.asarray(ref, dtype=np.float64))
    return float(diff.max()) if diff.size else 0.0, float(diff.mean()) if diff.size else 0.0


def assert_close(got, ref, max_abs: float, mean_abs: float, label: str) -> None:
    mx, mn = errors(got, ref)
    ref = np.asarray(ref)
    rel = float(np.sqrt(np.mean((np.asarray(got) - ref) ** 2)) / max(np.sqrt(np.mean(ref ** 2)), 1e-30)) \
        if ref.size else 0.0
    print(f"  {label}: max_abs={mx:.3e} mean_abs={mn:.3e} rel_rms={rel:.3e} max|ref|={np.abs(ref).max() if ref.size else 0:.3e}",
          flush=True)
    assert np.isfinite(np.asarray(got)).all(), f"{label}: non-finite values"
    assert mx <= max_abs, f"{label}: max-abs {mx} > {max_abs}"
    assert mn <= mean_abs, f"{label}: mean-abs {mn} > {mean_abs}"


def assert_close_scaled(got, ref, label: str, rel_rms_max: float = 8e-3, qscale: float = 1.0) -> None:
    """Bar for inputs scaled away from N(0, 1) (the peaky gates): the fixed
    2e-2 max-abs bar holds for outputs up to |4|, so it grows with max|ref|
    beyond that, and with the Q scale, which multiplies the logits and so the
    logit error the bf16 rounding of rotated Q and K leaves; the relative RMS
    error must stay at the bf16 level."""
    ref = np.asarray(ref, dtype=np.float64)
    scale = qscale * (max(1.0, float(np.abs(ref).max()) / 4.0) if ref.size else 1.0)
    mx, mn = errors(got, ref)
    rel = float(np.sqrt(np.mean((np.asarray(got) - ref) ** 2)) / max(np.sqrt(np.mean(ref ** 2)), 1e-30))
    print(f"  {label}: max_abs={mx:.3e} (bar {2e-2 * scale:.3e}) rel_rms={rel:.3e} max|ref|={np.abs(ref).max():.3e}",
          flush=True)
    assert np.isfinite(np.asarray(got)).all(), f"{label}: non-finite values"
    assert mx <= 2e-2 * scale, f"{label}: max-abs {mx} > {2e-2 * scale}"
    assert rel <= rel_rms_max, f"{label}: relative rms {rel} > {rel_rms_max}"


def assert_close_large_values(got, ref, label: str, rel_large: float = 1.5e-2, rel_rms_max: float = 8e-3) -> None:
    """Bar for outputs whose magnitude exceeds the |x| <= 4 range the fixed
    2e-2 max-abs bar is written for (gradients of segments with only a few
    keys): elements with |ref| <= 4 keep max-abs 2e-2 (and the whole tensor
    mean-abs 2e-3); larger elements get a relative bound.  The bf16 rounding
    of the rotated Q and K moves a logit s by about |s| * 2^-8, i.e. the
    softmax weights, dS and the gradients by ~1% relative where |s| ~ 2-3,
    so 1.5% covers it; a wrong or missing term is off by O(100%)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    big = np.abs(ref) > 4.0
    small_max = float(err[~big].max()) if (~big).any() else 0.0
    big_rel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    rel = float(np.sqrt(np.mean((got - ref) ** 2)) / max(np.sqrt(np.mean(ref ** 2)), 1e-30))
    print(f"  {label}: max_abs(|ref|<=4)={small_max:.3e} max_rel(|ref|>4, n={int(big.sum())})={big_rel:.3e} "
          f"mean_abs={float(err.mean()):.3e} rel_rms={rel:.3e}", flush=True)
    assert np.isfinite(got).all(), f"{label}: non-finite values"
    assert small_max <= 2e-2, f"{label}: max-abs {small_max} > 2e-2 where |ref| <= 4"
    assert big_rel <= rel_large, f"{label}: relative error {big_rel} > {rel_large} where |ref| > 4"
    assert float(err.mean()) <= 2e-3, f"{label}: mean-abs {float(err.mean())} > 2e-3"
    assert rel <= rel_rms_max, f"{label}: relative rms {rel} > {rel_rms_max}"


# The attention kernels cover runs of tiny segments with one multi-segment
# tile (the library's stated rule): when tiny segments (at most TINY_LEN
# tokens) hold at least half of the pack's tokens, consecutive tiny segments
# whose first tokens lie in the same TINY_LEN-token window of the stream
# share a tile.  A merged segment meets its keys on other tile boundaries
# than when it runs alone, so its outputs equal a standalone run's only up to
# rounding; every other segment's outputs are bitwise the same.
TINY_LEN = 128


def merged_segments(cu) -> set:
    cu = [int(x) for x in cu]
    n = len(cu) - 1
    tokens = cu[-1] - cu[0] if n else 0
    tiny = sum(cu[s + 1] - cu[s] for s in range(n) if cu[s + 1] - cu[s] <= TINY_LEN)
    if n == 0 or 2 * tiny < tokens or tokens > 2 * TINY_LEN * n:
        return set()
    first = []  # index of the first segment of each group
    for s in range(n):
        if s > 0 and cu[s + 1] - cu[s] <= TINY_LEN and cu[s] - cu[s - 1] <= TINY_LEN and \
                cu[s] // TINY_LEN == cu[s - 1] // TINY_LEN:
            continue
        first.append(s)
    first.append(n)
    out = set()
    for a, b in zip(first[:-1], first[1:]):
        if b - a > 1:
            out.update(range(a, b))
    return out


class Case:
    """A packed workload with inputs on host (as exact float32 values) and GPU."""

    def __init__(self, samples, budget, heads, head_dim, dtype, seed, qscale=1.0, with_dout=False, editing=False):
        self.samples = [tuple(int(v) for v in s) for s in samples]
        self.budget = budget
        self.editing = editing
        p = (oracle.pack_edit if editing else oracle.pack)(self.samples, budget)
        self.pack = p
        self.n = p["n_tokens"]
        self.cu = p["cu_seqlens"]
        self.pos = (oracle.positions_edit if editing else oracle.positions)(self.samples, p["n_packed"])
        self.max_seqlen = p["max_seqlen"]
        self.max_pos = max(p["max_pos"], 1)
        self.heads, self.d, self.dtype = heads, head_dim, dtype
        q, k, v = workloads.qkv(seed, self.n, heads, head_dim, dtype)
        if qscale != 1.0:
            q = workloads.normal(seed, workloads.STREAM_Q, (self.n, heads, head_dim), dtype, scale=qscale)
        self.q_bits, self.k_bits, self.v_bits = q, k, v
        self.q = self._f32(q)
        self.k = self._f32(k)
        self.v = self._f32(v)
        self.dq_dev = None
        if with_dout:
            self.do_bits = workloads.dout(seed, self.n, heads, head_dim, dtype)
            self.do = self._f32(self.do_bits)
        self.tq = dev(q, dtype)
        self.tk = dev(k, dtype)
        self.tv = dev(v, dtype)
        self.tcu = torch.from_numpy(self.cu.astype(np.int32)).cuda()
        nax = 3 if editing else 2
        self.tpos = torch.from_numpy(self.pos.astype(np.int32).reshape(-1, nax)).cuda() if self.n else \
            torch.zeros((1, nax), dtype=torch.int32, device="cuda")
        if with_dout:
            self.tdo = dev(self.do_bits, dtype)

    def _f32(self, x):
        return workloads.bf16_bits_to_f32(x) if self.dtype == "bf16" else np.asarray(x, dtype=np.float32)

    def describe(self) -> str:
        return (f"N={self.n} segments={len(self.cu) - 1} H={self.heads} D={self.d} {self.dtype} "
                f"max_seqlen={self.max_seqlen}" + (" editing" if self.editing else ""))

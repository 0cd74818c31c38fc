#!/usr/bin/env python3
"""Benchmark of the packed 2D-RoPE variable-length attention hot path.

One step = one pass of the whole path over one synthetic batch:
  mf_pack             budget cut + offsets (scan), per-token (row, col) and the
                      gather of 3072-wide bf16 hidden rows into the packed buffer
  mf_varlen_attn_fwd  2D RoPE + block-diagonal attention, O and LSE
  mf_varlen_attn_bwd  dQ, dK, dV with the inverse rotation
on the mixed native-resolution training pack (50 000-token budget, 24 heads x
head_dim 128, bf16).  Inputs are resident in GPU memory before timing starts.

Prints ONE JSON line.  value = (forward + backward algorithmic FLOPs) / step
time (the median of the timed steps), with forward = 4 sum(L_i^2) D H and
backward = 10 sum(L_i^2) D H.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
ROW_BYTES = 3072 * 2        # one packed hidden row (hidden 3072, bf16)

# Algorithmic FLOPs per unit sum(L^2) * D * H, and algorithmic bytes per launch,
# for each kernel the library launches.
KERNEL_FLOP_FACTOR = {"attn_fwd": 4.0, "attn_bwd_dkdv": 8.0, "attn_bwd_dq": 2.0}
KERNEL_SOURCE = {
    "attn_fwd": "attn_fwd.hip", "attn_bwd_dkdv": "attn_bwd.hip", "attn_bwd_dq": "attn_bwd.hip",
    "attn_bwd_delta": "attn_bwd.hip", "rope_q": "rope.hip", "rope_k": "rope.hip", "rope_table": "rope.hip",
    "pack_scan": "pack.hip", "pack_fill": "pack.hip",
}


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixed50k", choices=["mixed50k", "cfg1024", "stress", "edit50k", "captions"],
                    help="bench line workload (mixed50k is the metric's; others for exploration; edit50k runs "
                         "the editing path with frame-aware 3D RoPE)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle CPU timing")
    ap.add_argument("--cpu-threads", type=int, default=16, help="BLAS threads for the oracle baseline")
    ap.add_argument("--flow", action="store_true",
                    help="after timing, also time the rectified-flow noising / loss passes on the pack's latents "
                         "(128 channels, bf16) and the CFG combine on the 1024^2 packed-CFG pack; reported under "
                         "'flow', not part of the step")
    ap.add_argument("--block", action="store_true",
                    help="after timing, also time the attention sub-block chains (adaLN, QKV projection with the "
                         "RoPE epilogue, output projection with the gated residual) on the pack at the model width "
                         "(24 heads x 128 = 3072 channels); reported under 'block', not part of the step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run a plain 1 GiB device copy (reference for HBM counters)")
    return ap.parse_args()


def source_digest(name: str) -> str:
    """Digest of a kernel's source file together with the device headers it includes."""
    h = hashlib.sha256()
    for part in (name, "mf_device.h", "mf_kernels.h"):
        with open(os.path.join(ROOT, "packed_varlen_attention_amd", "csrc", part), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_bytes(name: str, n: int, h: int, d: int, n_samples: int, pos_bytes: int = 8) -> float:
    """Algorithmic HBM bytes of the memory-bound kernels (per launch); pos_bytes
    is 8 for (row, col) positions, 12 for (row, col, frame)."""
    t = n * h * d * 2
    if name in ("rope_q", "rope_k"):
        return 2.0 * t + pos_bytes * n
    if name == "attn_bwd_delta":  # read O, dO, LSE; write Delta and log2-scaled LSE
        return 2.0 * t + 12.0 * n * h
    if name == "pack_fill":
        return 2.0 * n * ROW_BYTES + pos_bytes * n
    if name == "pack_scan":
        return 12.0 * n_samples + 4.0 * (3 * n_samples + 2) + 16
    return 0.0


def load_traffic(kernel: str):
    """HBM traffic per launch from the committed rocprofv3 counter summary, or
    None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(kernel)
    if not rec or rec.get("source_sha256_16") != source_digest(KERNEL_SOURCE[kernel]):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, samples, q, k, v, do, threads: int, min_seconds: float = 10.0):
    """Time the oracle (test infrastructure, never the product path) on a
    bounded sample: forward + backward of whole heads over every packed
    segment, adding heads until about ``min_seconds`` of CPU work."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    import workloads

    avail = len(os.sched_getaffinity(0))
    use = max(1, min(threads, avail))
    if w.editing:
        p = oracle.pack_edit(samples, w.budget)
        pos = oracle.positions_edit(samples, p["n_packed"])
    else:
        p = oracle.pack(samples, w.budget)
        pos = oracle.positions(samples, p["n_packed"])
    cu = p["cu_seqlens"]
    sum_l2 = float(np.sum(np.diff(cu).astype(np.float64) ** 2))
    secs = 0.0
    heads = 0
    with threadpool_limits(limits=use):
        info = threadpool_info()
        nthreads = max([i.get("num_threads", 1) for i in info] or [1])
        while heads < w.n_heads and secs < min_seconds:
            sl = slice(heads, heads + 1)
            qs, ks, vs, ds = (workloads.bf16_bits_to_f32(x[:, sl]) for x in (q, k, v, do))
            t0 = time.perf_counter()
            oracle.attn_fwd(qs, ks, vs, cu, pos, w.theta)
            oracle.attn_bwd(qs, ks, vs, ds, cu, pos, w.theta)
            secs += time.perf_counter() - t0
            heads += 1
    flops = 14.0 * sum_l2 * w.head_dim * heads  # forward 4 + backward 10 per head
    return {
        "value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": int(nthreads), "kind": "oracle",
        "blas_threads": int(nthreads), "host_affinity_cores": avail,
        "sample": f"fp64 numpy oracle, forward+backward of {heads} of {w.n_heads} heads over all "
                  f"{p['n_packed']} segments ({p['n_tokens']} tokens), {secs:.1f} s; "
                  f"{int(nthreads)} BLAS threads of the {avail} cores in the process's affinity mask",
    }


def flow_timing(mf, workloads, w, samples, packres, n_tokens: int, dev, reps: int = 20, cpu: bool = False) -> dict:
    """Mean per-launch time and algorithmic GB/s of the rectified-flow and CFG passes."""
    import numpy as np
    import torch

    c = 128  # latent channels
    frames = 2 if w.editing else 1
    s = len(samples)

    def bf16(stream):
        x = workloads.normal(w.seed, stream, (n_tokens, c), "bf16")
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    z, eps, v = bf16(20), bf16(21), bf16(22)
    t = torch.rand(s, generator=torch.Generator(device=dev).manual_seed(w.seed), device=dev)
    cp = packres.cu_pieces
    noised = int(sum(b - a for a, b in zip(
        cp.cpu().numpy()[frames::frames + 1][:s].tolist(), cp.cpu().numpy()[frames + 1::frames + 1][:s].tolist())))
    row = c * 2
    out = {}

    def timed(name, fn, nbytes):
        tr = mf.KernelTrace(4)
        fn(None)
        torch.cuda.synchronize()
        total = 0.0
        for _ in range(reps):
            fn(tr)
            torch.cuda.synchronize()
            total += sum(ms for _, ms in tr.results())
        ms = total / reps
        out[name] = {"ms": round(ms, 4), "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes}

    zt = torch.empty_like(z)
    grad = torch.empty_like(v)
    ws = torch.empty(mf._binding.mf_rf_loss_workspace_size(n_tokens), dtype=torch.uint8, device=dev)
    # noise: read z (all rows), eps (noised rows), write z_t (all rows)
    timed("rf_noise", lambda tr: mf.rf_noise(z, eps, t, cp, s, frames, out=zt, trace=tr),
          (2 * n_tokens + noised) * row)
    # loss: read v, z, eps (noised rows), write grad (all rows) and one float per row
    timed("rf_loss", lambda tr: mf.rf_loss(v, z, eps, cp, s, frames, 1.0, workspace=ws, trace=tr),
          3 * noised * row + n_tokens * row + 8 * n_tokens)
    g = workloads.cfg1024()
    gs = torch.tensor(np.asarray(g.samples, dtype=np.int32)).to(dev)
    gp = mf.pack(gs, g.budget)
    torch.cuda.synchronize()
    gn = int(gp.counts[1].item())
    gcp = gp.cu_pieces.cpu().numpy()
    cond_img = sum(int(gcp[2 * k + 2] - gcp[2 * k + 1]) for k in range(0, len(g.samples), 2))
    gv = torch.from_numpy(workloads.normal(g.seed, 23, (gn, c), "bf16").view(np.int16)).to(dev).view(torch.bfloat16)
    # combine in place: read cond and uncond image rows, write cond image rows
    timed("cfg_combine", lambda tr: mf.cfg_combine(gv, gp.cu_pieces, len(g.samples), len(g.samples) // 2, 4.5,
                                                   out=gv, trace=tr), 3 * cond_img * row)
    out["note"] = (f"latents [N][{c}] bf16 on the bench pack (N={n_tokens}, {noised} noised rows); CFG on the "
                   f"1024^2 packed-CFG pack ({gn} tokens, {len(g.samples) // 2} pairs)")
    for name in ("rf_noise", "rf_loss", "cfg_combine"):
        out[name]["roofline"] = {"bound": "hbm", "achieved": out[name]["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                 "frac": round(out[name]["gbs"] / PEAK_HBM_GBS, 4)}
    if cpu:
        # the oracle (test infrastructure, never the product path): the loss over the whole pack
        from oracle import flow as oflow
        f64 = lambda x: x.float().cpu().numpy().astype(np.float64)  # noqa: E731
        vz, zz, ez = f64(v), f64(z), f64(eps)
        cpn = cp.cpu().numpy()
        t0 = time.perf_counter()
        reps_cpu = 0
        while time.perf_counter() - t0 < 2.0:
            oflow.rf_loss(vz, zz, ez, cpn, s, frames, 1.0)
            reps_cpu += 1
        secs = (time.perf_counter() - t0) / reps_cpu
        nb = out["rf_loss"]["bytes"]
        out["cpu_baseline"] = {"value": round(nb / secs / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
                               "sample": f"fp64 numpy oracle rf_loss over the whole pack, {reps_cpu} runs in "
                                         f"{secs * reps_cpu:.1f} s (same algorithmic bytes as the kernel)"}
    return out


def block_timing(mf, workloads, w, packres, n_tokens: int, max_pos: int, dev, reps: int = 10,
                 cpu: bool = False) -> dict:
    """Per-launch time and rate of the sub-block chain kernels on the bench pack, plus (for context only) the
    library GEMM of the same shapes without an epilogue."""
    import numpy as np
    import torch

    heads, hd = w.n_heads, w.head_dim
    c = heads * hd
    frames = 2 if w.editing else 1
    s = int(packres.counts[0].item())
    d = workloads.block_inputs(w.seed + 100, n_tokens, s, c)

    def bf(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)

    def f32(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)

    x, o = bf(d["x"]), bf(d["o"])
    shift, scale, gate = f32(d["shift"]), f32(d["scale"]), f32(d["gate"])
    wq = (bf(d["w_qkv0"]), bf(d["w_qkv1"]))
    bq = (f32(d["b_qkv0"]), f32(d["b_qkv1"]))
    wo = (bf(d["w_o0"]), bf(d["w_o1"]))
    bo = (f32(d["b_o0"]), f32(d["b_o1"]))
    cp = packres.cu_pieces
    pos = packres.pos[:n_tokens]
    h = torch.empty_like(x)
    qkv = tuple(torch.empty((n_tokens, heads, hd), dtype=torch.bfloat16, device=dev) for _ in range(3))
    y = torch.empty_like(x)
    ws = mf.block_workspace(s, frames, hd, max_pos, dev)
    out = {}

    def timed(name, fn, kernel, flops, nbytes):
        tr = mf.KernelTrace(4)
        fn(None)
        torch.cuda.synchronize()
        total = 0.0
        for _ in range(reps):
            fn(tr)
            torch.cuda.synchronize()
            total += sum(ms for nm, ms in tr.results() if nm == kernel)
        ms = total / reps
        e = {"ms": round(ms, 4), "bytes": nbytes, "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}
        if flops:
            e["flops"] = flops
            e["tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
        out[name] = e

    row = 2 * c
    timed("adaln", lambda tr: mf.adaln_modulate(x, shift, scale, cp, s, frames, out=h, trace=tr), "adaln", 0,
          2 * n_tokens * row)
    timed("qkv_rope", lambda tr: mf.qkv_rope(h, wq, bq, cp, s, frames, pos, heads, 10000.0, max_pos, out=qkv,
                                             workspace=ws, trace=tr), "qkv_rope",
          2 * n_tokens * c * 3 * c, n_tokens * row + 3 * n_tokens * row + 3 * c * row)
    timed("out_gated", lambda tr: mf.out_gated_residual(o, x, wo, bo, gate, cp, s, frames, out=y, workspace=ws,
                                                        trace=tr), "out_gated",
          2 * n_tokens * c * c, 3 * n_tokens * row + c * row)

    # context: the library GEMM (hipBLASLt through torch.mm) of the same shapes, no epilogue, one weight
    def lib_ms(a, b_t):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.mm(a, b_t)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            torch.mm(a, b_t)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    wq_t = wq[1].t().contiguous()
    wo_t = wo[1].t().contiguous()
    mq, mo = lib_ms(h, wq_t), lib_ms(o, wo_t)
    for name, bound in (("adaln", "hbm"), ("qkv_rope", "mfma"), ("out_gated", "mfma")):
        e = out[name]
        if bound == "hbm":
            out[name]["roofline"] = {"bound": "hbm", "achieved": e["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                     "frac": round(e["gbs"] / PEAK_HBM_GBS, 4)}
        else:
            out[name]["roofline"] = {"bound": "mfma", "achieved": e["tflops"], "peak": PEAK_BF16_TFLOPS,
                                     "unit": "TFLOP/s", "frac": round(e["tflops"] / PEAK_BF16_TFLOPS, 4)}
    out["library_gemm_context"] = {
        "qkv_ms": round(mq, 4), "qkv_tflops": round(2 * n_tokens * c * 3 * c / (mq * 1e-3) / 1e12, 1),
        "out_ms": round(mo, 4), "out_tflops": round(2 * n_tokens * c * c / (mo * 1e-3) / 1e12, 1),
        "note": "torch.mm (hipBLASLt) on the same shapes with one weight, no bias, rotation or residual"}
    out["note"] = (f"bf16 [N][{c}] rows of the bench pack (N={n_tokens}, {s} samples), one weight matrix per "
                   f"modality; bytes = activations read and written once plus the weights of one modality")
    out["backward"] = block_bwd_timing(mf, workloads, w, d, packres, n_tokens, max_pos, dev, x, o, h, wq, bo, wo,
                                       gate, scale, reps)
    if cpu:
        out["cpu_baseline"] = block_cpu_baseline(w, d, packres, heads, hd, frames)
        out["backward"]["cpu_baseline"] = block_bwd_cpu_baseline(w, d, packres, heads, hd, frames)
    return out


def block_bwd_timing(mf, workloads, w, d, packres, n_tokens: int, max_pos: int, dev, x, o, h, wq, bo, wo, gate,
                     scale, reps: int) -> dict:
    """Per-stage time of the three backward calls on the bench pack.  FLOPs of a projection's backward:
    2 N F C for the activation gradient (dgrad) and again for the weight gradient (wgrad), F = 3C (QKV) or C
    (output); bytes of the memory-bound stages: operands read and written once."""
    import numpy as np
    import torch

    heads, hd = w.n_heads, w.head_dim
    c = heads * hd
    frames = 2 if w.editing else 1
    s = int(packres.counts[0].item())
    cp = packres.cu_pieces
    pos = packres.pos[:n_tokens]
    g = workloads.block_grads(w.seed + 101, n_tokens, c)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    dy = bf(g["dy"])
    dq, dk, dv = (bf(g[k]).view(n_tokens, heads, hd) for k in ("dq", "dk", "dv"))
    proj = torch.empty_like(x)
    mf.out_gated_residual(o, x, wo, bo, gate, cp, s, frames, proj=proj)
    ws_a = torch.empty(mf.mf_adaln_modulate_bwd_workspace_size(s, frames, n_tokens, c), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(mf.mf_qkv_rope_bwd_workspace_size(s, frames, n_tokens, heads, hd, max_pos), dtype=torch.uint8,
                       device=dev)
    ws_o = torch.empty(mf.mf_out_gated_residual_bwd_workspace_size(s, frames, n_tokens, c), dtype=torch.uint8,
                       device=dev)
    out = {}

    def staged(name, fn):
        tr = mf.KernelTrace(16)
        fn(None)
        torch.cuda.synchronize()
        acc = {}
        for _ in range(reps):
            fn(tr)
            torch.cuda.synchronize()
            for nm, ms in tr.results():
                acc[nm] = acc.get(nm, 0.0) + ms
        st = {nm: round(v / reps, 4) for nm, v in acc.items()}
        out[name] = {"ms": round(sum(st.values()), 4), "stages_ms": st}

    staged("adaln_bwd", lambda tr: mf.adaln_modulate_bwd(dy, x, scale, cp, s, frames, workspace=ws_a, trace=tr))
    staged("qkv_rope_bwd", lambda tr: mf.qkv_rope_bwd(dq, dk, dv, h, wq, cp, s, frames, pos, w.theta, max_pos,
                                                      workspace=ws_q, trace=tr))
    staged("out_gated_bwd", lambda tr: mf.out_gated_residual_bwd(dy, o, proj, wo, gate, cp, s, frames, workspace=ws_o,
                                                                 trace=tr))
    nc2 = n_tokens * c * 2  # bytes of one bf16 [N][C] tensor
    for name, f in (("qkv_rope_bwd", 3 * c), ("out_gated_bwd", c)):
        st = out[name]["stages_ms"]
        flops = 2.0 * n_tokens * f * c
        out[name]["flops_per_gemm"] = flops
        for stage in ("dgrad", "wgrad"):
            t = st[stage]
            tf = flops / (t * 1e-3) / 1e12
            out[name][stage] = {"ms": t, "tflops": round(tf, 1),
                                "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                                             "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}
        # the gather-transposes move the gradient and the layer input once each way
        t = st["gather_t"]
        gb = 2 * (f + c) * n_tokens * 2 / (t * 1e-3) / 1e9
        out[name]["gather_t"] = {"ms": t, "gbs": round(gb, 1), "frac_hbm": round(gb / PEAK_HBM_GBS, 4)}
    # adaLN backward: rows read x and dh and write dx; the column sums read x and dh again
    t = out["adaln_bwd"]["stages_ms"]["adaln_bwd"]
    gb = 5 * nc2 / (t * 1e-3) / 1e9
    out["adaln_bwd"]["roofline"] = {"bound": "hbm", "achieved": round(gb, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                    "frac": round(gb / PEAK_HBM_GBS, 4), "bytes": 5 * nc2}
    total = sum(out[k]["ms"] for k in ("adaln_bwd", "qkv_rope_bwd", "out_gated_bwd"))
    out["total_ms"] = round(total, 4)
    out["note"] = ("backward of the three chains on the bench pack, QKV with the inverse rotation; stage times from "
                   "HIP events around each launch (stages_ms), rates from the FLOPs and bytes stated in the fields")
    return out


def block_cpu_baseline(w, d, packres, heads: int, hd: int, frames: int, min_seconds: float = 8.0) -> dict:
    """Time the oracle (test infrastructure, never the product path) on a bounded sample of the block chain:
    adaLN, QKV projection with the rotation and the gated output projection over 128-row slices of the pack's
    image pieces (largest first) until about ``min_seconds`` of CPU work; reported as the projections' FLOP
    rate."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import block
    import workloads

    cp = packres.cu_pieces.cpu().numpy()
    s = int(packres.counts[0].item())
    per = frames + 1
    pieces = sorted(((int(cp[i + 1] - cp[i]), i) for i in range(per * s) if i % per != 0), reverse=True)
    pos = packres.pos.cpu().numpy()
    c = heads * hd
    f64 = lambda x: workloads.bf16_bits_to_f32(x).astype(np.float64)  # noqa: E731
    w_q = (f64(d["w_qkv0"]), f64(d["w_qkv1"]))
    w_o = (f64(d["w_o0"]), f64(d["w_o1"]))
    secs, rows = 0.0, 0
    with threadpool_limits(limits=max(1, min(16, len(os.sched_getaffinity(0))))):
        nthreads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        for length, piece in pieces:  # image pieces, largest first, in slices of 128 rows
            sample, a0 = piece // per, int(cp[piece])
            for r0 in range(0, length - 127, 128):
                if secs >= min_seconds:
                    break
                sl = slice(a0 + r0, a0 + r0 + 128)
                cu = [0, 0, 128]  # one sample: no text rows, 128 image rows
                x = f64(d["x"][sl])
                t0 = time.perf_counter()
                h = block.adaln_modulate(x, d["shift"][sample:sample + 1], d["scale"][sample:sample + 1], cu, 1, 1)
                block.qkv_rope(h, w_q, (d["b_qkv0"], d["b_qkv1"]), cu, 1, 1, pos[sl], heads, hd, w.theta)
                block.out_gated_residual(f64(d["o"][sl]), x, w_o, (d["b_o0"], d["b_o1"]),
                                         d["gate"][sample:sample + 1], cu, 1, 1)
                secs += time.perf_counter() - t0
                rows += 128
    flops = 2.0 * rows * c * 4 * c  # QKV (3C outputs) + output projection (C outputs)
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": int(nthreads), "kind": "oracle",
            "sample": f"fp64 numpy oracle: adaLN + QKV projection with RoPE + gated output projection over {rows} "
                      f"image rows (128-row slices, largest pieces first), {secs:.1f} s"}


def block_bwd_cpu_baseline(w, d, packres, heads: int, hd: int, frames: int, min_seconds: float = 8.0) -> dict:
    """Time the oracle's backward of the block chain (test infrastructure, never the product path) on a bounded
    sample: adaLN, QKV projection with the inverse rotation and gated output projection backward over 128-row
    slices of the pack's image pieces (largest first) until about ``min_seconds`` of CPU work; reported as the
    projections' FLOP rate (activation and weight gradients)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import block
    import workloads

    cp = packres.cu_pieces.cpu().numpy()
    s = int(packres.counts[0].item())
    per = frames + 1
    pieces = sorted(((int(cp[i + 1] - cp[i]), i) for i in range(per * s) if i % per != 0), reverse=True)
    pos = packres.pos.cpu().numpy()
    c = heads * hd
    f64 = lambda x: workloads.bf16_bits_to_f32(x).astype(np.float64)  # noqa: E731
    w_q = (f64(d["w_qkv0"]), f64(d["w_qkv1"]))
    w_o = (f64(d["w_o0"]), f64(d["w_o1"]))
    g = workloads.block_grads(w.seed + 102, 128, c)
    gq, gk, gv, gy = (f64(g[k]) for k in ("dq", "dk", "dv", "dy"))
    secs, rows = 0.0, 0
    with threadpool_limits(limits=max(1, min(16, len(os.sched_getaffinity(0))))):
        nthreads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        for length, piece in pieces:
            sample, a0 = piece // per, int(cp[piece])
            for r0 in range(0, length - 127, 128):
                if secs >= min_seconds:
                    break
                sl = slice(a0 + r0, a0 + r0 + 128)
                cu = [0, 0, 128]
                x, o = f64(d["x"][sl]), f64(d["o"][sl])
                sh = (128, heads, hd)
                t0 = time.perf_counter()
                block.out_gated_residual_bwd(gy, o, x, w_o, (d["b_o0"], d["b_o1"]), d["gate"][sample:sample + 1],
                                             cu, 1, 1)
                block.qkv_rope_bwd(gq.reshape(sh), gk.reshape(sh), gv.reshape(sh), x, w_q, cu, 1, 1, pos[sl],
                                   w.theta)
                block.adaln_modulate_bwd(gy, x, d["shift"][sample:sample + 1], d["scale"][sample:sample + 1], cu,
                                         1, 1)
                secs += time.perf_counter() - t0
                rows += 128
    flops = 2.0 * 2.0 * rows * c * 4 * c  # dgrad + wgrad of QKV (3C outputs) and output projection (C outputs)
    return {"value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": int(nthreads), "kind": "oracle",
            "sample": f"fp64 numpy oracle: gated output projection + QKV projection (inverse RoPE) + adaLN backward "
                      f"over {rows} image rows (128-row slices, largest pieces first), {secs:.1f} s"}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the packed segments are independent: data parallelism gives each GPU its own pack, and the "
              "attention path needs no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import packed_varlen_attention_amd as mf
    import workloads

    torch.cuda.set_device(0)
    w = {"mixed50k": lambda: workloads.mixed50k(backward=True), "cfg1024": workloads.cfg1024,
         "stress": workloads.stress, "edit50k": workloads.edit50k, "captions": workloads.captions}[args.workload]()
    samples = list(w.samples)
    H, D = w.n_heads, w.head_dim
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)

    # Per-sample hidden rows (text, then row-major image grid; for editing,
    # text, source grid, target grid) to gather.
    t_samples = torch.tensor(np.asarray(samples, dtype=np.int32)).to(dev)
    bufs, ptrs = [], ([], [], [])
    for (t, gh, gw) in samples:
        parts = [max(t, 1), max(gh * gw, 1)] + ([max(gh * gw, 1)] if w.editing else [])
        for lst, rows in zip(ptrs, parts):
            b = torch.randn((rows, ROW_BYTES // 2), generator=gen, device=dev, dtype=torch.bfloat16)
            bufs.append(b)
            lst.append(b.data_ptr())
    row_ptrs = [torch.tensor(x, dtype=torch.int64, device=dev) for x in ptrs if x]

    def do_pack(out=None, trace=None):
        if w.editing:
            return mf.pack_edit(t_samples, w.budget, *row_ptrs, row_bytes=ROW_BYTES, out=out, trace=trace)
        return mf.pack(t_samples, w.budget, *row_ptrs, ROW_BYTES, out=out, trace=trace)

    packres = do_pack()
    pos_bytes = 12 if w.editing else 8
    torch.cuda.synchronize()
    n_packed, N, max_seqlen, max_pos = (int(x) for x in packres.counts.cpu().tolist())
    cu_host = packres.cu_seqlens.cpu().numpy()[: n_packed + 1].astype(np.int64)
    sum_l2 = float(np.sum(np.diff(cu_host).astype(np.float64) ** 2))

    q, k, v = workloads.qkv(w.seed, N, H, D, "bf16")
    do = workloads.dout(w.seed, N, H, D, "bf16")

    def up(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    tq, tk, tv, tdo = up(q), up(k), up(v), up(do)
    o = torch.empty_like(tq)
    lse = torch.empty((H, N), dtype=torch.float32, device=dev)
    grads = (torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv))
    from packed_varlen_attention_amd.api import attn_workspace
    ws_f = attn_workspace(tq, n_packed, max_pos, False, rotated=True)
    ws_b = attn_workspace(tq, n_packed, max_pos, True, rotated=True)
    # the forward keeps its rotated bf16 Q and K here for the backward, as a
    # training step keeps activations
    rot = mf.rotated_buffer(tq)

    def step(traces=None):
        tp, tf, tb = traces if traces else (None, None, None)
        do_pack(out=packres, trace=tp)
        mf.attn_fwd(tq, tk, tv, packres.cu_seqlens, max_seqlen, packres.pos, w.theta, max_pos, out=o, lse=lse,
                    workspace=ws_f, trace=tf, n_segments=n_packed, rotated=rot)
        mf.attn_bwd(tq, tk, tv, o, lse, tdo, packres.cu_seqlens, max_seqlen, packres.pos, w.theta, max_pos,
                    workspace=ws_b, grads=grads, trace=tb, n_segments=n_packed, rotated=rot)

    for _ in range(args.warmup):
        step()
    traces = [(mf.KernelTrace(4), mf.KernelTrace(8), mf.KernelTrace(8)) for _ in range(args.steps)]
    stream = torch.cuda.current_stream()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for i in range(args.steps):
        step(traces[i])
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    ms_step = float(np.median(step_ms))
    ms_total = marks[0].elapsed_time(marks[-1])

    # per-kernel median duration over the timed steps (events on the launch
    # stream); each call's time is the median of its kernels' per-step sums
    per_step = [{} for _ in range(args.steps)]
    call_steps = {"pack": [0.0] * args.steps, "fwd": [0.0] * args.steps, "bwd": [0.0] * args.steps}
    for i, tr in enumerate(traces):
        for label, t in zip(("pack", "fwd", "bwd"), tr):
            for name, ms in t.results():
                key = name if label != "bwd" or name not in ("rope_table", "rope_k") else name + "@bwd"
                per_step[i][key] = per_step[i].get(key, 0.0) + ms
                call_steps[label][i] += ms
    kern = {key: float(np.median([d.get(key, 0.0) for d in per_step])) for key in per_step[0]}
    call_ms = {label: float(np.median(v)) for label, v in call_steps.items()}

    fwd_flops = 4.0 * sum_l2 * D * H
    bwd_flops = 10.0 * sum_l2 * D * H
    value = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12

    dominant = max(kern, key=kern.get)
    base = dominant.split("@")[0]
    if base in KERNEL_FLOP_FACTOR:
        algo = KERNEL_FLOP_FACTOR[base] * sum_l2 * D * H
        achieved = algo / (kern[dominant] * 1e-3) / 1e12
        roof = {"kernel": base, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "algorithmic_flops_per_launch": algo, "ms_per_launch": round(kern[dominant], 4)}
    else:
        algo = kernel_bytes(base, N, H, D, len(samples), pos_bytes)
        achieved = algo / (kern[dominant] * 1e-3) / 1e9
        roof = {"kernel": base, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "algorithmic_bytes_per_launch": algo, "ms_per_launch": round(kern[dominant], 4)}
    roof["traffic"] = load_traffic(base)

    per_kernel = {}
    for name, ms in sorted(kern.items(), key=lambda kv: -kv[1]):
        b = name.split("@")[0]
        entry = {"ms": round(ms, 4)}
        if b in KERNEL_FLOP_FACTOR:
            entry["tflops"] = round(KERNEL_FLOP_FACTOR[b] * sum_l2 * D * H / (ms * 1e-3) / 1e12, 1)
        elif kernel_bytes(b, N, H, D, len(samples), pos_bytes) > 0:
            entry["gbs"] = round(kernel_bytes(b, N, H, D, len(samples), pos_bytes) / (ms * 1e-3) / 1e9, 1)
        per_kernel[name] = entry

    result = {
        "metric": "packed 2D-RoPE varlen attention TFLOP/s (fwd, bwd) @50k tokens; % bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_mean": round(ms_total / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16 Q/K/V/dO (PCG64) on a seeded mixed native-resolution pack",
        "config": {
            "workload": {"mixed50k": "mixed native-resolution training pack, 50,000-token budget, seed 3: "
                                     "pack + fwd(LSE) + bwd",
                         "cfg1024": "1024^2 packed-CFG inference pack (4 prompts x cond/uncond): pack + fwd + bwd",
                         "stress": "long/ragged stress pack (2048^2 + two 4:1 panoramas + 64 thumbnails): "
                                   "pack + fwd + bwd",
                         "edit50k": "editing training pack [text | source | target], frame-aware 3D RoPE, "
                                    "50,000-token budget, seed 6: pack + fwd(LSE) + bwd",
                         "captions": "1500 text-only segments of 16-120 tokens (multi-segment tiles), seed 8: "
                                     "pack + fwd(LSE) + bwd"}[args.workload],
            "n_tokens": N, "segments": n_packed, "heads": H, "head_dim": D, "max_seqlen": max_seqlen,
            "sum_L2": sum_l2, "gather_row_bytes": ROW_BYTES,
        },
        "fwd_tflops": round(fwd_flops / (call_ms["fwd"] * 1e-3) / 1e12, 2),
        "fwd_frac_peak": round(fwd_flops / (call_ms["fwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "bwd_tflops": round(bwd_flops / (call_ms["bwd"] * 1e-3) / 1e12, 2),
        "bwd_frac_peak": round(bwd_flops / (call_ms["bwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "call_ms": {k2: round(v2, 4) for k2, v2 in call_ms.items()},
        "kernels": per_kernel,
        "roofline": roof,
        "cpu_baseline": None,
    }
    # Clock-limited ceiling: sustained matrix-instruction rate on operands with
    # the inputs' distribution, and the shader clock meanwhile (after timing).
    probe_ops = torch.from_numpy(
        workloads.normal(w.seed, 9, (mf.PROBE_VECTORS * 8,), "bf16").view(np.int16)).to(dev).view(torch.bfloat16)
    probe_blocks = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    mf.mfma_probe(probe_ops, probe_blocks, 20000)
    probe = mf.mfma_probe(probe_ops, probe_blocks, 400000)
    result["mfma_probe"] = {"tflops": round(probe["tflops"], 1), "sclk_mhz": round(probe["sclk_mhz"]),
                            "ms": round(probe["ms"], 2),
                            "operands": "seeded N(0,1) bf16; 32x32x16 bf16 MFMA, 2 waves per SIMD"}
    if roof["unit"] == "TFLOP/s":
        roof["peak_measured"] = round(probe["tflops"], 1)
        roof["frac_measured"] = round(roof["achieved"] / probe["tflops"], 4)
    if args.flow:
        result["flow"] = flow_timing(mf, workloads, w, samples, packres, N, dev, cpu=not args.no_cpu_baseline)
    if args.block:
        result["block"] = block_timing(mf, workloads, w, packres, N, max_pos, dev, cpu=not args.no_cpu_baseline)
    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(5):
            dst.copy_(src)
        c1.record()
        torch.cuda.synchronize()
        result["copy_1GiB_gbs"] = round(2 * (1 << 30) * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9, 1)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, samples, q, k, v, do, args.cpu_threads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

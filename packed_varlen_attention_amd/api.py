"""Allocation helpers over the C ABI wrappers.

Each helper allocates its outputs (and workspace, unless one is passed) with
PyTorch on the inputs' device and makes exactly one C ABI call.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import torch

from . import _binding as B


@dataclass
class PackResult:
    cu_seqlens: torch.Tensor  # int32 [S + 1]
    cu_pieces: torch.Tensor   # int32 [2 S + 1] ([3 S + 1] for editing packs)
    pos: torch.Tensor         # int32 [token_budget, 2] ([token_budget, 3] for editing packs)
    counts: torch.Tensor      # int32 [4]: n_packed, n_tokens, max_seqlen, max_pos
    packed: Optional[torch.Tensor]  # uint8 [token_budget, row_bytes] or None


def pack(samples: torch.Tensor, token_budget: int, text_rows: Optional[torch.Tensor] = None,
         image_rows: Optional[torch.Tensor] = None, row_bytes: int = 0, stream=None, trace=None,
         out: Optional[PackResult] = None) -> PackResult:
    if out is None:
        dev = samples.device
        s = int(samples.shape[0])
        packed = None
        if text_rows is not None:
            packed = torch.empty((max(int(token_budget), 1), int(row_bytes)), dtype=torch.uint8, device=dev)
        out = PackResult(torch.empty(s + 1, dtype=torch.int32, device=dev),
                         torch.empty(2 * s + 1, dtype=torch.int32, device=dev),
                         torch.empty((max(int(token_budget), 1), 2), dtype=torch.int32, device=dev),
                         torch.empty(4, dtype=torch.int32, device=dev), packed)
    B.mf_pack(samples, token_budget, out.cu_seqlens, out.cu_pieces, out.pos, out.counts, text_rows, image_rows,
              row_bytes, out.packed, stream, trace)
    return out


def pack_edit(samples: torch.Tensor, token_budget: int, text_rows: Optional[torch.Tensor] = None,
              source_rows: Optional[torch.Tensor] = None, target_rows: Optional[torch.Tensor] = None,
              row_bytes: int = 0, stream=None, trace=None, out: Optional[PackResult] = None) -> PackResult:
    """Editing pack [text | source | target]: cu_pieces [3 S + 1], pos [budget, 3]."""
    if out is None:
        dev = samples.device
        s = int(samples.shape[0])
        packed = None
        if text_rows is not None:
            packed = torch.empty((max(int(token_budget), 1), int(row_bytes)), dtype=torch.uint8, device=dev)
        out = PackResult(torch.empty(s + 1, dtype=torch.int32, device=dev),
                         torch.empty(3 * s + 1, dtype=torch.int32, device=dev),
                         torch.empty((max(int(token_budget), 1), 3), dtype=torch.int32, device=dev),
                         torch.empty(4, dtype=torch.int32, device=dev), packed)
    B.mf_pack_edit(samples, token_budget, out.cu_seqlens, out.cu_pieces, out.pos, out.counts, text_rows,
                   source_rows, target_rows, row_bytes, out.packed, stream, trace)
    return out


def rope3d_apply(x: torch.Tensor, pos: torch.Tensor, theta: float, max_pos: int, inverse: bool = False,
                 workspace: Optional[torch.Tensor] = None, stream=None, trace=None) -> torch.Tensor:
    if workspace is None:
        workspace = torch.empty(max(B.mf_rope3d_workspace_size(x.shape[2], max_pos), 1), dtype=torch.uint8,
                                device=x.device)
    B.mf_rope3d_apply(x, pos, theta, max_pos, inverse, workspace, stream, trace)
    return x


def rope2d_apply(x: torch.Tensor, pos: torch.Tensor, theta: float, max_pos: int, inverse: bool = False,
                 workspace: Optional[torch.Tensor] = None, stream=None, trace=None) -> torch.Tensor:
    if workspace is None:
        workspace = torch.empty(max(B.mf_rope2d_workspace_size(x.shape[2], max_pos), 1), dtype=torch.uint8,
                                device=x.device)
    B.mf_rope2d_apply(x, pos, theta, max_pos, inverse, workspace, stream, trace)
    return x


def attn_workspace(q: torch.Tensor, n_segments: int, max_pos: int, backward: bool,
                   rotated: bool = False) -> torch.Tensor:
    """Workspace for attn_fwd (backward=False) or attn_bwd; rotated=True when the
    call will be given a rotated buffer, which then holds the rotated Q and K
    (the workspace reserves no copies of them)."""
    n, h, d = q.shape
    size = B.mf_varlen_attn_workspace_size(n, h, d, n_segments, max_pos, B.dtype_code(q), backward, rotated)
    return torch.empty(max(size, 1), dtype=torch.uint8, device=q.device)


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
             pos: Optional[torch.Tensor] = None, theta: float = 10000.0, max_pos: int = 0,
             softmax_scale: float = 0.0, with_lse: bool = True, workspace: Optional[torch.Tensor] = None,
             out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
             stream=None, trace=None, n_segments: Optional[int] = None,
             rotated: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """rotated: an optional rotated_buffer(q) that keeps the rotated bf16 Q and K for attn_bwd."""
    n, h, _ = q.shape
    nseg = int(cu_seqlens.numel()) - 1 if n_segments is None else int(n_segments)
    o = torch.empty_like(q) if out is None else out
    if with_lse and lse is None:
        lse = torch.empty((h, n), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = attn_workspace(q, nseg, max_pos if pos is not None else 0, False, rotated is not None)
    B.mf_varlen_attn_fwd(q, k, v, o, lse if with_lse else None, cu_seqlens, nseg, max_seqlen, pos, theta,
                         max_pos, softmax_scale, workspace, stream, trace, rotated)
    return o, (lse if with_lse else None)


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
             dout: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int, pos: Optional[torch.Tensor] = None,
             theta: float = 10000.0, max_pos: int = 0, softmax_scale: float = 0.0,
             workspace: Optional[torch.Tensor] = None, grads=None,
             stream=None, trace=None, n_segments: Optional[int] = None,
             rotated: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """rotated: the buffer attn_fwd filled on the same q, k and positions; Q and K are then not rotated again."""
    nseg = int(cu_seqlens.numel()) - 1 if n_segments is None else int(n_segments)
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    dq, dk, dv = grads
    if workspace is None:
        workspace = attn_workspace(q, nseg, max_pos if pos is not None else 0, True, rotated is not None)
    B.mf_varlen_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens, nseg, max_seqlen, pos, theta, max_pos,
                         softmax_scale, workspace, stream, trace, rotated)
    return dq, dk, dv


def rotated_buffer(q: torch.Tensor) -> torch.Tensor:
    """A bf16 [2][n][H][D] buffer for the forward's rotated Q and K (see attn_fwd / attn_bwd)."""
    return torch.empty((2,) + tuple(q.shape), dtype=torch.bfloat16, device=q.device)


PROBE_VECTORS = 4096  # bf16x8 operand vectors mf_mfma_probe reads


def mfma_probe(operands: torch.Tensor, n_blocks: int, iters: int) -> dict:
    """Sustained bf16 matrix-instruction rate on ``operands`` and the shader clock.

    ``operands`` is a bf16 device tensor of PROBE_VECTORS * 8 elements.  One
    launch of ``n_blocks`` 256-thread workgroups, timed with events on the
    current stream (synchronises).  Returns flops, milliseconds, TFLOP/s and
    the mean shader clock in MHz over the workgroups.
    """
    if operands.dtype != torch.bfloat16 or operands.numel() != PROBE_VECTORS * 8:
        raise ValueError(f"operands must be {PROBE_VECTORS * 8} bf16 values")
    sink = torch.empty(n_blocks * 256, dtype=torch.float32, device=operands.device)
    clocks = torch.empty(2 * n_blocks, dtype=torch.int64, device=operands.device)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    khz = B.mf_mfma_probe(operands, n_blocks, iters, sink, clocks)
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1)
    c = clocks.view(n_blocks, 2).cpu().double()
    sclk_mhz = float(c[:, 0].sum() / c[:, 1].sum()) * khz / 1000.0
    flops = float(n_blocks) * 4 * 4 * iters * 32768
    return {"flops": flops, "ms": ms, "tflops": flops / ms / 1e9, "sclk_mhz": sclk_mhz}


def rf_noise(z: torch.Tensor, eps: torch.Tensor, t: torch.Tensor, cu_pieces: torch.Tensor, n_samples: int,
             frames: int = 1, out: Optional[torch.Tensor] = None, stream=None, trace=None) -> torch.Tensor:
    """Model input z_t of the rectified-flow objective on [N][C] packed latents."""
    zt = torch.empty_like(z) if out is None else out
    B.mf_rf_noise(z, eps, t, zt, cu_pieces, n_samples, frames, stream, trace)
    return zt


def rf_loss(v: torch.Tensor, z: torch.Tensor, eps: torch.Tensor, cu_pieces: torch.Tensor, n_samples: int,
            frames: int = 1, grad_scale: float = 1.0, with_grad: bool = True,
            workspace: Optional[torch.Tensor] = None, stream=None, trace=None):
    """(loss_sum [n_samples] float32, grad [N][C] or None)."""
    loss = torch.empty(max(int(n_samples), 1), dtype=torch.float32, device=v.device)
    grad = torch.empty_like(v) if with_grad else None
    if workspace is None:
        workspace = torch.empty(max(B.mf_rf_loss_workspace_size(v.shape[0]), 4), dtype=torch.uint8, device=v.device)
    B.mf_rf_loss(v, z, eps, grad, loss, cu_pieces, n_samples, frames, grad_scale, workspace, stream, trace)
    return loss[: int(n_samples)], grad


def cfg_combine(v: torch.Tensor, cu_pieces: torch.Tensor, n_samples: int, n_pairs: int, scale: float,
                out: Optional[torch.Tensor] = None, stream=None, trace=None):
    """(guided copy of v (or out), device int32 [1] count of mismatched pairs)."""
    o = torch.empty_like(v) if out is None else out
    mismatched = torch.zeros(1, dtype=torch.int32, device=v.device)
    B.mf_cfg_combine(v, o, mismatched, cu_pieces, n_samples, n_pairs, scale, stream, trace)
    return o, mismatched


def block_workspace(n_samples: int, frames: int, head_dim: int, max_pos: int, device) -> torch.Tensor:
    nbytes = max(B.mf_block_workspace_size(n_samples, frames, head_dim, max_pos), 256)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def adaln_modulate(x: torch.Tensor, shift: torch.Tensor, scale: torch.Tensor, cu_pieces: torch.Tensor,
                   n_samples: int, frames: int = 1, eps: float = 1e-6, out: Optional[torch.Tensor] = None,
                   stream=None, trace=None) -> torch.Tensor:
    """h = LN(x) (1 + scale[s][m]) + shift[s][m] over packed bf16 [N][C] rows."""
    h = torch.empty_like(x) if out is None else out
    B.mf_adaln_modulate(x, shift, scale, h, cu_pieces, n_samples, frames, eps, stream, trace)
    return h


def qkv_rope(h: torch.Tensor, w: Tuple[torch.Tensor, torch.Tensor],
             b: Tuple[Optional[torch.Tensor], Optional[torch.Tensor]], cu_pieces: torch.Tensor, n_samples: int,
             frames: int, pos: Optional[torch.Tensor], n_heads: int, theta: float = 10000.0, max_pos: int = 1,
             out=None, workspace: Optional[torch.Tensor] = None, stream=None, trace=None):
    """(q, k, v) bf16 [N][H][D]: the modality's projection of h, q and k rotated by pos."""
    n, c = h.shape
    d = c // n_heads
    if out is None:
        out = tuple(torch.empty((n, n_heads, d), dtype=h.dtype, device=h.device) for _ in range(3))
    if workspace is None:
        workspace = block_workspace(n_samples, frames, d, max_pos if pos is not None else 0, h.device)
    B.mf_qkv_rope(h, w[0], w[1], b[0], b[1], out[0], out[1], out[2], cu_pieces, n_samples, frames, pos, theta,
                  max_pos, workspace, stream, trace)
    return out


def out_gated_residual(o: torch.Tensor, x: torch.Tensor, w: Tuple[torch.Tensor, torch.Tensor],
                       b: Tuple[Optional[torch.Tensor], Optional[torch.Tensor]], gate: torch.Tensor,
                       cu_pieces: torch.Tensor, n_samples: int, frames: int = 1, out: Optional[torch.Tensor] = None,
                       proj: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None,
                       trace=None) -> torch.Tensor:
    """y = x + gate[s][m] (o W_o,m^T + b_o,m); out may be x.  proj, if given ([N][C] bf16), receives the
    pre-gate projection the backward needs."""
    y = torch.empty_like(x) if out is None else out
    if workspace is None:
        workspace = block_workspace(n_samples, frames, 64, 0, x.device)
    B.mf_out_gated_residual(o, x, w[0], w[1], b[0], b[1], gate, y, proj, cu_pieces, n_samples, frames, workspace,
                            stream, trace)
    return y


def _workspace(nbytes: int, device) -> torch.Tensor:
    if nbytes == 0:
        raise B.MFError(B.MF_ERR_UNSUPPORTED, "sizes not supported by the backward")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def adaln_modulate_bwd(dh: torch.Tensor, x: torch.Tensor, scale: torch.Tensor, cu_pieces: torch.Tensor,
                       n_samples: int, frames: int = 1, eps: float = 1e-6, dres: Optional[torch.Tensor] = None,
                       out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None,
                       trace=None):
    """(dx bf16 [N][C], dshift, dscale float [S][2][C]) for h = LN(x) (1 + scale) + shift; dres, if given, is
    added to dx.  out may be dres (in place), not dh or x."""
    n, c = x.shape
    dx = torch.empty_like(x) if out is None else out
    dshift = torch.empty((n_samples, 2, c), dtype=torch.float32, device=x.device)
    dscale = torch.empty_like(dshift)
    if workspace is None:
        workspace = _workspace(B.mf_adaln_modulate_bwd_workspace_size(n_samples, frames, n, c), x.device)
    B.mf_adaln_modulate_bwd(dh, x, scale, dres, dx, dshift, dscale, cu_pieces, n_samples, frames, eps, workspace,
                            stream, trace)
    return dx, dshift, dscale


def qkv_rope_bwd(dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor, h: torch.Tensor,
                 w: Tuple[torch.Tensor, torch.Tensor], cu_pieces: torch.Tensor, n_samples: int, frames: int,
                 pos: Optional[torch.Tensor], theta: float = 10000.0, max_pos: int = 1, bias: bool = True,
                 workspace: Optional[torch.Tensor] = None, stream=None, trace=None):
    """(dh bf16 [N][C], (dW_text, dW_image) float [3C][C], (db_text, db_image) float [3C] or None) given the
    gradients of the rotated q, k and of v."""
    n, heads, d = dq.shape
    c = heads * d
    dh = torch.empty((n, c), dtype=h.dtype, device=h.device)
    dw = tuple(torch.empty((3 * c, c), dtype=torch.float32, device=h.device) for _ in range(2))
    db = tuple(torch.empty(3 * c, dtype=torch.float32, device=h.device) for _ in range(2)) if bias else (None, None)
    if workspace is None:
        mp = max_pos if pos is not None else 0
        workspace = _workspace(B.mf_qkv_rope_bwd_workspace_size(n_samples, frames, n, heads, d, mp), h.device)
    B.mf_qkv_rope_bwd(dq, dk, dv, h, w[0], w[1], dh, dw[0], dw[1], db[0], db[1], cu_pieces, n_samples, frames, pos,
                      theta, max_pos, workspace, stream, trace)
    return dh, dw, db


def out_gated_residual_bwd(dy: torch.Tensor, o: torch.Tensor, proj: torch.Tensor,
                           w: Tuple[torch.Tensor, torch.Tensor], gate: torch.Tensor, cu_pieces: torch.Tensor,
                           n_samples: int, frames: int = 1, bias: bool = True,
                           workspace: Optional[torch.Tensor] = None, stream=None, trace=None):
    """(d_o bf16 [N][C], (dW_text, dW_image) float [C][C], (db_text, db_image) float [C] or None, dgate float
    [S][2][C]); the gradient with respect to x is dy itself."""
    n, c = dy.shape
    d_o = torch.empty_like(dy)
    dw = tuple(torch.empty((c, c), dtype=torch.float32, device=dy.device) for _ in range(2))
    db = tuple(torch.empty(c, dtype=torch.float32, device=dy.device) for _ in range(2)) if bias else (None, None)
    dgate = torch.empty((n_samples, 2, c), dtype=torch.float32, device=dy.device)
    if workspace is None:
        workspace = _workspace(B.mf_out_gated_residual_bwd_workspace_size(n_samples, frames, n, c), dy.device)
    B.mf_out_gated_residual_bwd(dy, o.reshape(n, c), proj, w[0], w[1], gate, d_o, dw[0], dw[1], db[0], db[1], dgate,
                                cu_pieces, n_samples, frames, workspace, stream, trace)
    return d_o, dw, db, dgate

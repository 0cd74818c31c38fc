"""ctypes binding of libmf.so (include/mf.h).

Argument marshalling only: every function here passes device pointers, sizes
and the current HIP stream to the C ABI call of the same name and raises
``MFError`` on a negative status.  All computation happens in the HIP
kernels; there is no fallback of any kind.  PyTorch supplies device memory and
the stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# MF_LIBRARY selects another build of the same library (e.g. the copy with
# host sanitizers that build.py --sanitize-host writes); there is no fallback.
LIB_PATH = os.environ.get("MF_LIBRARY") or os.path.join(_PKG, "libmf.so")

MF_OK = 0
MF_ERR_INVALID_ARG = -1
MF_ERR_UNSUPPORTED = -2
MF_ERR_WORKSPACE = -3
MF_ERR_HIP = -4
MF_BF16 = 0
MF_F32 = 1

EXPORTED = (
    "mf_status_string", "mf_abi_version", "mf_pack", "mf_rope2d_workspace_size",
    "mf_rope2d_apply", "mf_varlen_attn_workspace_size", "mf_varlen_attn_fwd",
    "mf_varlen_attn_bwd", "mf_mfma_probe", "mf_pack_edit", "mf_rope3d_workspace_size", "mf_rope3d_apply",
    "mf_varlen_attn3d_fwd", "mf_varlen_attn3d_bwd", "mf_rf_noise", "mf_rf_loss_workspace_size", "mf_rf_loss",
    "mf_cfg_combine", "mf_block_workspace_size", "mf_adaln_modulate", "mf_qkv_rope", "mf_out_gated_residual",
    "mf_adaln_modulate_bwd_workspace_size", "mf_adaln_modulate_bwd", "mf_qkv_rope_bwd_workspace_size",
    "mf_qkv_rope_bwd", "mf_out_gated_residual_bwd_workspace_size", "mf_out_gated_residual_bwd",
    "mf_varlen_attn_fwd_noalloc",
)


MF_TRACE_MAX = 16


class Trace(ctypes.Structure):
    """mf_trace: caller-owned HIP events recorded around each kernel launch."""
    _fields_ = [("capacity", ctypes.c_int32), ("count", ctypes.c_int32),
                ("start", ctypes.c_void_p * MF_TRACE_MAX), ("stop", ctypes.c_void_p * MF_TRACE_MAX),
                ("names", ctypes.c_char_p * MF_TRACE_MAX)]


class KernelTrace:
    """A Trace backed by torch timing events on the current device."""

    def __init__(self, capacity: int = MF_TRACE_MAX):
        self.capacity = int(capacity)
        self.starts = [torch.cuda.Event(enable_timing=True) for _ in range(self.capacity)]
        self.stops = [torch.cuda.Event(enable_timing=True) for _ in range(self.capacity)]
        for e in self.starts + self.stops:  # creates the underlying hipEvent_t
            e.record()
        self.struct = Trace()
        self.struct.capacity = self.capacity
        for i in range(self.capacity):
            self.struct.start[i] = self.starts[i].cuda_event
            self.struct.stop[i] = self.stops[i].cuda_event

    def results(self):
        """[(kernel name, milliseconds)] of the last traced call; synchronise first."""
        out = []
        for i in range(min(self.struct.count, self.capacity)):
            out.append((self.struct.names[i].decode(), self.starts[i].elapsed_time(self.stops[i])))
        return out


def _trace(t) -> Optional[object]:
    if t is None:
        return None
    if isinstance(t, KernelTrace):
        return ctypes.byref(t.struct)
    return ctypes.byref(t)


class MFError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call} failed with status {status}: {status_string(status)}")


_lib: Optional[ctypes.CDLL] = None

# MF_ABI_VERSION of include/mf.h that the argument lists below follow.
ABI_VERSION = 7

# Flags of mf_varlen_attn_workspace_size.
WS_BACKWARD = 1
WS_ROTATED = 2

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_dbl = ctypes.c_double
_f32 = ctypes.c_float


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmf.so (built in-tree by packed_varlen_attention_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m packed_varlen_attention_amd.build` "
            "(hipcc for gfx950); there is no fallback path")
    lib = ctypes.CDLL(path)
    lib.mf_status_string.restype = ctypes.c_char_p
    lib.mf_status_string.argtypes = [_i32]
    lib.mf_abi_version.restype = _i32
    lib.mf_abi_version.argtypes = []
    if lib.mf_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} has ABI version {lib.mf_abi_version()}, the binding expects {ABI_VERSION}: "
                          "rebuild it with `python -m packed_varlen_attention_amd.build`")
    lib.mf_pack.restype = _i32
    lib.mf_pack.argtypes = [_vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp]
    lib.mf_rope2d_workspace_size.restype = _sz
    lib.mf_rope2d_workspace_size.argtypes = [_i32, _i32]
    lib.mf_rope2d_apply.restype = _i32
    lib.mf_rope2d_apply.argtypes = [_vp, _i32, _vp, _i32, _i32, _i32, _dbl, _i32, _i32, _vp, _sz, _vp, _vp]
    lib.mf_varlen_attn_workspace_size.restype = _sz
    lib.mf_varlen_attn_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32]
    lib.mf_varlen_attn_fwd.restype = _i32
    lib.mf_varlen_attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _vp, _dbl, _i32,
                                       _i32, _i32, _i32, _f32, _vp, _vp, _sz, _vp, _vp]
    lib.mf_varlen_attn_fwd_noalloc.restype = _i32
    lib.mf_varlen_attn_fwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _vp, _dbl, _i32,
                                               _i32, _i32, _i32, _f32, _vp, _vp, _vp]
    lib.mf_varlen_attn_bwd.restype = _i32
    lib.mf_varlen_attn_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                                       _vp, _dbl, _i32, _i32, _i32, _i32, _f32, _vp, _vp, _sz, _vp, _vp]
    lib.mf_mfma_probe.restype = _i32
    lib.mf_mfma_probe.argtypes = [_vp, _i32, _i32, _vp, _vp, _vp, _vp]
    lib.mf_pack_edit.restype = _i32
    lib.mf_pack_edit.argtypes = [_vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _vp, _vp]
    lib.mf_rope3d_workspace_size.restype = _sz
    lib.mf_rope3d_workspace_size.argtypes = [_i32, _i32]
    lib.mf_rope3d_apply.restype = _i32
    lib.mf_rope3d_apply.argtypes = lib.mf_rope2d_apply.argtypes
    lib.mf_varlen_attn3d_fwd.restype = _i32
    lib.mf_varlen_attn3d_fwd.argtypes = lib.mf_varlen_attn_fwd.argtypes
    lib.mf_varlen_attn3d_bwd.restype = _i32
    lib.mf_varlen_attn3d_bwd.argtypes = lib.mf_varlen_attn_bwd.argtypes
    lib.mf_rf_noise.restype = _i32
    lib.mf_rf_noise.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _vp, _vp]
    lib.mf_rf_loss_workspace_size.restype = _sz
    lib.mf_rf_loss_workspace_size.argtypes = [_i32]
    lib.mf_rf_loss.restype = _i32
    lib.mf_rf_loss.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _f32, _vp, _sz, _vp,
                               _vp]
    lib.mf_cfg_combine.restype = _i32
    lib.mf_cfg_combine.argtypes = [_vp, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _f32, _vp, _vp]
    lib.mf_block_workspace_size.restype = _sz
    lib.mf_block_workspace_size.argtypes = [_i32, _i32, _i32, _i32]
    lib.mf_adaln_modulate.restype = _i32
    lib.mf_adaln_modulate.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _vp, _vp]
    lib.mf_qkv_rope.restype = _i32
    lib.mf_qkv_rope.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _i32, _dbl, _i32,
                                _i32, _i32, _i32, _vp, _sz, _vp, _vp]
    lib.mf_out_gated_residual.restype = _i32
    lib.mf_out_gated_residual.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                          _vp, _sz, _vp, _vp]
    lib.mf_adaln_modulate_bwd_workspace_size.restype = _sz
    lib.mf_adaln_modulate_bwd_workspace_size.argtypes = [_i32, _i32, _i32, _i32]
    lib.mf_adaln_modulate_bwd.restype = _i32
    lib.mf_adaln_modulate_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _f32, _vp,
                                          _sz, _vp, _vp]
    lib.mf_qkv_rope_bwd_workspace_size.restype = _sz
    lib.mf_qkv_rope_bwd_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32]
    lib.mf_qkv_rope_bwd.restype = _i32
    lib.mf_qkv_rope_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _i32,
                                    _dbl, _i32, _i32, _i32, _i32, _vp, _sz, _vp, _vp]
    lib.mf_out_gated_residual_bwd_workspace_size.restype = _sz
    lib.mf_out_gated_residual_bwd_workspace_size.argtypes = [_i32, _i32, _i32, _i32]
    lib.mf_out_gated_residual_bwd.restype = _i32
    lib.mf_out_gated_residual_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                              _i32, _i32, _i32, _vp, _sz, _vp, _vp]
    _lib = lib
    return lib


def lib() -> ctypes.CDLL:
    return _lib if _lib is not None else load_library()


def status_string(status: int) -> str:
    return lib().mf_status_string(int(status)).decode()


def abi_version() -> int:
    return int(lib().mf_abi_version())


def _check(status: int, call: str) -> None:
    if status != MF_OK:
        raise MFError(int(status), call)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MF_BF16
    if t.dtype == torch.float32:
        return MF_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


# ---------------------------------------------------------------------------
# 1:1 wrappers of the C ABI
# ---------------------------------------------------------------------------

def mf_pack(samples: torch.Tensor, token_budget: int, cu_seqlens: torch.Tensor,
            cu_pieces: Optional[torch.Tensor], pos: torch.Tensor, counts: torch.Tensor,
            text_rows: Optional[torch.Tensor] = None, image_rows: Optional[torch.Tensor] = None,
            row_bytes: int = 0, packed: Optional[torch.Tensor] = None, stream=None, trace=None) -> None:
    """samples: int32 [S, 3] on the GPU; text_rows/image_rows: int64 [S] device
    tensors holding row-buffer addresses."""
    if samples.dtype != torch.int32 or samples.dim() != 2 or samples.shape[1] != 3:
        raise ValueError("samples must be an int32 [S, 3] tensor")
    st = lib().mf_pack(_ptr(samples), int(samples.shape[0]), int(token_budget), _ptr(cu_seqlens),
                       _ptr(cu_pieces), _ptr(pos), _ptr(counts), _ptr(text_rows), _ptr(image_rows),
                       int(row_bytes), _ptr(packed), _stream(stream), _trace(trace))
    _check(st, "mf_pack")


def mf_pack_edit(samples: torch.Tensor, token_budget: int, cu_seqlens: torch.Tensor,
                 cu_pieces: Optional[torch.Tensor], pos: torch.Tensor, counts: torch.Tensor,
                 text_rows: Optional[torch.Tensor] = None, source_rows: Optional[torch.Tensor] = None,
                 target_rows: Optional[torch.Tensor] = None, row_bytes: int = 0,
                 packed: Optional[torch.Tensor] = None, stream=None, trace=None) -> None:
    """Editing samples [text | source | target]; pos is int32 [budget, 3]."""
    if samples.dtype != torch.int32 or samples.dim() != 2 or samples.shape[1] != 3:
        raise ValueError("samples must be an int32 [S, 3] tensor")
    st = lib().mf_pack_edit(_ptr(samples), int(samples.shape[0]), int(token_budget), _ptr(cu_seqlens),
                            _ptr(cu_pieces), _ptr(pos), _ptr(counts), _ptr(text_rows), _ptr(source_rows),
                            _ptr(target_rows), int(row_bytes), _ptr(packed), _stream(stream), _trace(trace))
    _check(st, "mf_pack_edit")


def mf_rope2d_workspace_size(head_dim: int, max_pos: int) -> int:
    return int(lib().mf_rope2d_workspace_size(int(head_dim), int(max_pos)))


def mf_rope2d_apply(x: torch.Tensor, pos: torch.Tensor, theta: float, max_pos: int,
                    inverse: bool, workspace: torch.Tensor, stream=None, trace=None) -> None:
    n, h, d = x.shape
    st = lib().mf_rope2d_apply(_ptr(x), dtype_code(x), _ptr(pos), int(n), int(h), int(d), float(theta),
                               int(max_pos), int(bool(inverse)), _ptr(workspace),
                               int(workspace.numel() * workspace.element_size()), _stream(stream),
                               _trace(trace))
    _check(st, "mf_rope2d_apply")


def mf_rope3d_workspace_size(head_dim: int, max_pos: int) -> int:
    return int(lib().mf_rope3d_workspace_size(int(head_dim), int(max_pos)))


def mf_rope3d_apply(x: torch.Tensor, pos: torch.Tensor, theta: float, max_pos: int,
                    inverse: bool, workspace: torch.Tensor, stream=None, trace=None) -> None:
    n, h, d = x.shape
    st = lib().mf_rope3d_apply(_ptr(x), dtype_code(x), _ptr(pos), int(n), int(h), int(d), float(theta),
                               int(max_pos), int(bool(inverse)), _ptr(workspace),
                               int(workspace.numel() * workspace.element_size()), _stream(stream),
                               _trace(trace))
    _check(st, "mf_rope3d_apply")


def mf_varlen_attn_workspace_size(n_tokens: int, n_heads: int, head_dim: int, n_segments: int,
                                  max_pos: int, dtype: int, backward: bool, rotated: bool = False) -> int:
    """rotated: the call will be given a rotated buffer (no rotation copies reserved)."""
    flags = (WS_BACKWARD if backward else 0) | (WS_ROTATED if rotated else 0)
    return int(lib().mf_varlen_attn_workspace_size(int(n_tokens), int(n_heads), int(head_dim),
                                                   int(n_segments), int(max_pos), int(dtype), flags))


def _entry(pos, which: str):
    """The 2D call for [n, 2] (or no) positions, the frame-aware 3D call for [n, 3]."""
    if pos is not None and pos.dim() == 2 and pos.shape[1] == 3:
        name = f"mf_varlen_attn3d_{which}"
    elif pos is None or (pos.dim() == 2 and pos.shape[1] == 2):
        name = f"mf_varlen_attn_{which}"
    else:
        raise ValueError("pos must be an int32 [n, 2] or [n, 3] tensor")
    return getattr(lib(), name), name


def _span(t: torch.Tensor):
    start = t.data_ptr()
    return start, start + t.numel() * t.element_size()


def _check_rotated(rotated, q, others) -> None:
    """The C ABI takes the rotated buffer as a bare pointer with no size: check
    here that it is a bf16 tensor of at least 2 * q.numel() elements that
    overlaps none of the call's other tensors."""
    if rotated is None:
        return
    if rotated.dtype != torch.bfloat16 or not rotated.is_contiguous():
        raise ValueError("rotated must be a contiguous bfloat16 tensor (see rotated_buffer)")
    if rotated.numel() < 2 * q.numel():
        raise ValueError(f"rotated holds {rotated.numel()} elements; the call needs 2 * {q.numel()}")
    if rotated.device != q.device:
        raise ValueError("rotated must be on the device of q")
    a0, a1 = _span(rotated)
    for t in others:
        if t is None or t.numel() == 0:
            continue
        b0, b1 = _span(t)
        if a0 < b1 and b0 < a1:
            raise ValueError("rotated overlaps another argument of the call")


def mf_varlen_attn_fwd(q, k, v, o, lse, cu_seqlens, n_segments: int, max_seqlen: int, pos,
                       theta: float, max_pos: int, softmax_scale: float, workspace, stream=None,
                       trace=None, rotated=None) -> None:
    n, h, d = q.shape
    _check_rotated(rotated, q, (q, k, v, o, lse, cu_seqlens, pos, workspace))
    call, name = _entry(pos, "fwd")
    st = call(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), dtype_code(q),
                                  _ptr(cu_seqlens), int(n_segments), int(max_seqlen), _ptr(pos),
                                  float(theta), int(max_pos), int(n), int(h), int(d), float(softmax_scale),
                                  _ptr(rotated), _ptr(workspace), int(workspace.numel() * workspace.element_size()),
                                  _stream(stream), _trace(trace))
    _check(st, name)


def mf_varlen_attn_fwd_noalloc(q, k, v, o, lse, cu_seqlens, n_segments: int, max_seqlen: int, pos,
                               theta: float, max_pos: int, softmax_scale: float, rotated, stream=None,
                               trace=None) -> None:
    """The forward without a workspace (2D positions or none; bf16 only)."""
    n, h, d = q.shape
    if pos is not None and not (pos.dim() == 2 and pos.shape[1] == 2):
        raise ValueError("pos must be an int32 [n, 2] tensor")
    _check_rotated(rotated, q, (q, k, v, o, lse, cu_seqlens, pos))
    st = lib().mf_varlen_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), dtype_code(q),
                                          _ptr(cu_seqlens), int(n_segments), int(max_seqlen), _ptr(pos),
                                          float(theta), int(max_pos), int(n), int(h), int(d), float(softmax_scale),
                                          _ptr(rotated), _stream(stream), _trace(trace))
    _check(st, "mf_varlen_attn_fwd_noalloc")


def mf_varlen_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens, n_segments: int, max_seqlen: int,
                       pos, theta: float, max_pos: int, softmax_scale: float, workspace,
                       stream=None, trace=None, rotated=None) -> None:
    n, h, d = q.shape
    _check_rotated(rotated, q, (q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens, pos, workspace))
    call, name = _entry(pos, "bwd")
    st = call(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                  _ptr(dk), _ptr(dv), dtype_code(q), _ptr(cu_seqlens), int(n_segments),
                                  int(max_seqlen), _ptr(pos), float(theta), int(max_pos), int(n), int(h),
                                  int(d), float(softmax_scale), _ptr(rotated), _ptr(workspace),
                                  int(workspace.numel() * workspace.element_size()), _stream(stream),
                                  _trace(trace))
    _check(st, name)


def mf_mfma_probe(operands: torch.Tensor, n_blocks: int, iters: int, sink: torch.Tensor, clocks: torch.Tensor,
                  stream=None) -> int:
    """Enqueue the matrix-instruction probe; returns the wall counter's rate in kHz."""
    khz = ctypes.c_int32(0)
    _check(lib().mf_mfma_probe(_ptr(operands), int(n_blocks), int(iters), _ptr(sink), _ptr(clocks),
                               ctypes.byref(khz), _stream(stream)), "mf_mfma_probe")
    return int(khz.value)


def mf_rf_noise(z, eps, t, zt, cu_pieces, n_samples: int, frames: int, stream=None, trace=None) -> None:
    n, c = z.shape
    _check(lib().mf_rf_noise(_ptr(z), _ptr(eps), _ptr(t), _ptr(zt), dtype_code(z), _ptr(cu_pieces), int(n_samples),
                             int(frames), int(n), int(c), _stream(stream), _trace(trace)), "mf_rf_noise")


def mf_rf_loss_workspace_size(n_tokens: int) -> int:
    return int(lib().mf_rf_loss_workspace_size(int(n_tokens)))


def mf_rf_loss(v, z, eps, grad, loss_sum, cu_pieces, n_samples: int, frames: int, grad_scale: float, workspace,
               stream=None, trace=None) -> None:
    n, c = v.shape
    _check(lib().mf_rf_loss(_ptr(v), _ptr(z), _ptr(eps), _ptr(grad), _ptr(loss_sum), dtype_code(v),
                            _ptr(cu_pieces), int(n_samples), int(frames), int(n), int(c), float(grad_scale),
                            _ptr(workspace), int(workspace.numel() * workspace.element_size()), _stream(stream),
                            _trace(trace)), "mf_rf_loss")


def mf_cfg_combine(v, out, mismatched, cu_pieces, n_samples: int, n_pairs: int, scale: float, stream=None,
                   trace=None) -> None:
    n, c = v.shape
    _check(lib().mf_cfg_combine(_ptr(v), _ptr(out), _ptr(mismatched), dtype_code(v), _ptr(cu_pieces),
                                int(n_samples), int(n_pairs), int(n), int(c), float(scale), _stream(stream),
                                _trace(trace)), "mf_cfg_combine")


def mf_block_workspace_size(n_samples: int, frames: int, head_dim: int, max_pos: int) -> int:
    return int(lib().mf_block_workspace_size(int(n_samples), int(frames), int(head_dim), int(max_pos)))


def mf_adaln_modulate(x, shift, scale, h, cu_pieces, n_samples: int, frames: int, eps: float = 1e-6, stream=None,
                      trace=None) -> None:
    n, c = x.shape
    _check(lib().mf_adaln_modulate(_ptr(x), _ptr(shift), _ptr(scale), _ptr(h), _ptr(cu_pieces), int(n_samples),
                                   int(frames), int(n), int(c), float(eps), _stream(stream), _trace(trace)),
           "mf_adaln_modulate")


def mf_qkv_rope(h, w_text, w_image, b_text, b_image, q, k, v, cu_pieces, n_samples: int, frames: int, pos,
                theta: float, max_pos: int, workspace, stream=None, trace=None) -> None:
    n, heads, d = q.shape
    nax = int(pos.shape[-1]) if pos is not None else 2
    _check(lib().mf_qkv_rope(_ptr(h), _ptr(w_text), _ptr(w_image), _ptr(b_text), _ptr(b_image), _ptr(q), _ptr(k),
                             _ptr(v), _ptr(cu_pieces), int(n_samples), int(frames), _ptr(pos), nax, float(theta),
                             int(max_pos), int(n), int(heads), int(d), _ptr(workspace),
                             int(workspace.numel() * workspace.element_size()), _stream(stream), _trace(trace)),
           "mf_qkv_rope")


def mf_out_gated_residual(o, x, w_text, w_image, b_text, b_image, gate, y, proj, cu_pieces, n_samples: int,
                          frames: int, workspace, stream=None, trace=None) -> None:
    n, c = x.shape
    _check(lib().mf_out_gated_residual(_ptr(o), _ptr(x), _ptr(w_text), _ptr(w_image), _ptr(b_text), _ptr(b_image),
                                       _ptr(gate), _ptr(y), _ptr(proj), _ptr(cu_pieces), int(n_samples), int(frames),
                                       int(n), int(c), _ptr(workspace),
                                       int(workspace.numel() * workspace.element_size()), _stream(stream),
                                       _trace(trace)), "mf_out_gated_residual")


def _nbytes(t) -> int:
    return int(t.numel() * t.element_size())


def mf_adaln_modulate_bwd_workspace_size(n_samples: int, frames: int, n_tokens: int, channels: int) -> int:
    return int(lib().mf_adaln_modulate_bwd_workspace_size(int(n_samples), int(frames), int(n_tokens), int(channels)))


def mf_adaln_modulate_bwd(dh, x, scale, dres, dx, dshift, dscale, cu_pieces, n_samples: int, frames: int, eps: float,
                          workspace, stream=None, trace=None) -> None:
    n, c = x.shape
    _check(lib().mf_adaln_modulate_bwd(_ptr(dh), _ptr(x), _ptr(scale), _ptr(dres), _ptr(dx), _ptr(dshift),
                                       _ptr(dscale), _ptr(cu_pieces), int(n_samples), int(frames), int(n), int(c),
                                       float(eps), _ptr(workspace), _nbytes(workspace), _stream(stream),
                                       _trace(trace)), "mf_adaln_modulate_bwd")


def mf_qkv_rope_bwd_workspace_size(n_samples: int, frames: int, n_tokens: int, n_heads: int, head_dim: int,
                                   max_pos: int) -> int:
    return int(lib().mf_qkv_rope_bwd_workspace_size(int(n_samples), int(frames), int(n_tokens), int(n_heads),
                                                    int(head_dim), int(max_pos)))


def mf_qkv_rope_bwd(dq, dk, dv, h, w_text, w_image, dh, dw_text, dw_image, db_text, db_image, cu_pieces,
                    n_samples: int, frames: int, pos, theta: float, max_pos: int, workspace, stream=None,
                    trace=None) -> None:
    n, heads, d = dq.shape
    nax = int(pos.shape[-1]) if pos is not None else 2
    _check(lib().mf_qkv_rope_bwd(_ptr(dq), _ptr(dk), _ptr(dv), _ptr(h), _ptr(w_text), _ptr(w_image), _ptr(dh),
                                 _ptr(dw_text), _ptr(dw_image), _ptr(db_text), _ptr(db_image), _ptr(cu_pieces),
                                 int(n_samples), int(frames), _ptr(pos), nax, float(theta), int(max_pos), int(n),
                                 int(heads), int(d), _ptr(workspace), _nbytes(workspace), _stream(stream),
                                 _trace(trace)), "mf_qkv_rope_bwd")


def mf_out_gated_residual_bwd_workspace_size(n_samples: int, frames: int, n_tokens: int, channels: int) -> int:
    return int(lib().mf_out_gated_residual_bwd_workspace_size(int(n_samples), int(frames), int(n_tokens),
                                                              int(channels)))


def mf_out_gated_residual_bwd(dy, o, proj, w_text, w_image, gate, d_o, dw_text, dw_image, db_text, db_image, dgate,
                              cu_pieces, n_samples: int, frames: int, workspace, stream=None, trace=None) -> None:
    n, c = dy.shape
    _check(lib().mf_out_gated_residual_bwd(_ptr(dy), _ptr(o), _ptr(proj), _ptr(w_text), _ptr(w_image), _ptr(gate),
                                           _ptr(d_o), _ptr(dw_text), _ptr(dw_image), _ptr(db_text), _ptr(db_image),
                                           _ptr(dgate), _ptr(cu_pieces), int(n_samples), int(frames), int(n), int(c),
                                           _ptr(workspace), _nbytes(workspace), _stream(stream), _trace(trace)),
           "mf_out_gated_residual_bwd")

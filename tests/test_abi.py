"""CPU checks of the C ABI library: it loads, exports every function that
include/mf.h declares, and rejects bad host arguments before launching
anything (these calls never reach a kernel, so no GPU is needed)."""
import ctypes
import os
import pathlib
import re

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "mf.h"
# MF_LIBRARY runs these checks against another build (the host-sanitized one).
LIB = pathlib.Path(os.environ.get("MF_LIBRARY") or ROOT / "packed_varlen_attention_amd" / "libmf.so")


def _declared():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mf_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not LIB.exists():
        pytest.fail(f"{LIB} not built: run `python -m packed_varlen_attention_amd.build`")
    import packed_varlen_attention_amd as m
    return m._binding.lib()


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("mf_pack", "mf_rope2d_apply", "mf_varlen_attn_fwd", "mf_varlen_attn_bwd"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(str(LIB))
    for name in _declared():
        assert hasattr(raw, name), name
    import packed_varlen_attention_amd as m
    assert set(m.EXPORTED) == set(_declared())


def test_status_strings_and_version(lib):
    import packed_varlen_attention_amd as m
    assert m.abi_version() == 7 == m._binding.ABI_VERSION
    for code in (0, -1, -2, -3, -4, -5):
        assert len(m.status_string(code)) > 0
    assert m.status_string(7) == "unknown status"


FAKE = 1 << 20  # a 256-byte-aligned non-null address; never dereferenced by these calls


def _fwd(lib, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dtype=0, cu=FAKE, nseg=1, maxlen=8, pos=FAKE,
                theta=10000.0, max_pos=16, n=8, h=1, d=128, scale=0.0, rot=None, ws=FAKE, wsb=1 << 30, stream=None)
    args.update(kw)
    return lib.mf_varlen_attn_fwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["dtype"],
                                  args["cu"], args["nseg"], args["maxlen"], args["pos"], args["theta"],
                                  args["max_pos"], args["n"], args["h"], args["d"], args["scale"], args["rot"],
                                  args["ws"], args["wsb"], args["stream"], args.get("trace"))


def test_forward_argument_errors(lib):
    assert _fwd(lib, d=96) == -2
    assert _fwd(lib, dtype=3) == -2
    assert _fwd(lib, q=None) == -1
    assert _fwd(lib, cu=None) == -1
    assert _fwd(lib, q=FAKE + 8) == -1       # misaligned
    assert _fwd(lib, h=0) == -1
    assert _fwd(lib, n=-1) == -1
    assert _fwd(lib, max_pos=0) == -1
    assert _fwd(lib, theta=-1.0) == -1
    assert _fwd(lib, scale=-1.0) == -1
    assert _fwd(lib, wsb=16) == -3
    assert _fwd(lib, ws=None) == -1
    assert _fwd(lib, rot=FAKE + 8) == -1    # the rotated-Q/K buffer misaligned
    assert _fwd(lib, rot=FAKE + 8, n=0) == -1
    # nothing to do is OK and launches nothing
    assert _fwd(lib, n=0) == 0
    assert _fwd(lib, nseg=0) == 0
    # a trace with null events or a bad capacity is rejected before launching
    import packed_varlen_attention_amd as m
    t = m.Trace()
    t.capacity = 2
    assert _fwd(lib, trace=ctypes.byref(t)) == -1
    t.capacity = 99
    assert _fwd(lib, trace=ctypes.byref(t)) == -1


def test_backward_argument_errors(lib):
    def bwd(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, dtype=0, cu=FAKE,
                 nseg=1, maxlen=8, pos=FAKE, theta=1e4, max_pos=16, n=8, h=2, d=64, scale=0.0, rot=None, ws=FAKE,
                 wsb=1 << 30)
        a.update(kw)
        return lib.mf_varlen_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                                      a["dv"], a["dtype"], a["cu"], a["nseg"], a["maxlen"], a["pos"], a["theta"],
                                      a["max_pos"], a["n"], a["h"], a["d"], a["scale"], a["rot"], a["ws"], a["wsb"],
                                      None, None)
    assert bwd(lse=None) == -1
    assert bwd(dq=None) == -1
    assert bwd(d=32) == -2
    assert bwd(wsb=1) == -3
    assert bwd(dk=FAKE + 4) == -1
    assert bwd(rot=FAKE + 4) == -1


def test_pack_and_rope_argument_errors(lib):
    assert lib.mf_pack(FAKE, -1, 10, FAKE, None, FAKE, FAKE, None, None, 0, None, None, None) == -1
    assert lib.mf_pack(FAKE, 2, -5, FAKE, None, FAKE, FAKE, None, None, 0, None, None, None) == -1
    assert lib.mf_pack(FAKE, 2, 10, None, None, FAKE, FAKE, None, None, 0, None, None, None) == -1
    assert lib.mf_pack(FAKE, 2, 10, FAKE, None, FAKE + 4, FAKE, None, None, 0, None, None, None) == -1
    assert lib.mf_pack(FAKE, 2, 10, FAKE, None, FAKE, FAKE, FAKE, None, 16, FAKE, None, None) == -1  # image_rows missing
    assert lib.mf_pack(FAKE, 2, 10, FAKE, None, FAKE, FAKE, FAKE, FAKE, 0, FAKE, None, None) == -1   # row_bytes 0
    assert lib.mf_rope2d_apply(FAKE, 0, FAKE, 8, 1, 48, 1e4, 16, 0, FAKE, 1 << 20, None, None) == -2
    assert lib.mf_rope2d_apply(FAKE, 0, FAKE, 8, 1, 64, 1e4, 16, 0, FAKE, 8, None, None) == -3
    assert lib.mf_rope2d_apply(FAKE, 0, None, 8, 1, 64, 1e4, 16, 0, FAKE, 1 << 20, None, None) == -1
    assert lib.mf_rope2d_apply(FAKE, 0, FAKE, 0, 1, 64, 1e4, 16, 0, FAKE, 1 << 20, None, None) == 0


def test_workspace_sizes(lib):
    n, h = 1000, 4
    fwd_bf16 = lib.mf_varlen_attn_workspace_size(n, h, 128, 3, 640, 0, 0)
    bwd_bf16 = lib.mf_varlen_attn_workspace_size(n, h, 128, 3, 640, 0, 1)
    fwd_f32 = lib.mf_varlen_attn_workspace_size(n, h, 128, 3, 640, 1, 0)
    table = 640 * 32 * 8
    tensor = n * h * 128 * 2
    assert fwd_bf16 >= table + tensor
    assert bwd_bf16 >= table + 2 * tensor + n * h * 4
    assert fwd_f32 >= fwd_bf16 + tensor
    assert fwd_bf16 % 256 == 0 and bwd_bf16 % 256 == 0
    assert lib.mf_varlen_attn_workspace_size(n, h, 96, 3, 640, 0, 0) == 0
    assert lib.mf_rope2d_workspace_size(128, 640) == table


def _align(x):
    return (x + 255) // 256 * 256


def test_workspace_without_rotation_copies(lib):
    # MF_WS_ROTATED (2) leaves out the rotated K (forward) and the rotated Q
    # and K (backward): the caller's `rotated` buffer holds them
    n, h, d = 1000, 4, 128
    tensor = _align(n * h * d * 2)
    for dtype in (0, 1):
        fwd = lib.mf_varlen_attn_workspace_size(n, h, d, 3, 640, dtype, 0)
        bwd = lib.mf_varlen_attn_workspace_size(n, h, d, 3, 640, dtype, 1)
        assert lib.mf_varlen_attn_workspace_size(n, h, d, 3, 640, dtype, 2) == fwd - tensor
        assert lib.mf_varlen_attn_workspace_size(n, h, d, 3, 640, dtype, 3) == bwd - 2 * tensor
    for bad in (4, 8, -1, 1 << 30):
        assert lib.mf_varlen_attn_workspace_size(n, h, d, 3, 640, 0, bad) == 0


def test_calls_accept_the_smaller_workspace_only_with_rotated(lib):
    # The size check comes before the null-workspace check, so ws=None tells
    # the two apart without launching: -3 = too small, -1 = size accepted.
    fa = dict(n=8, h=1, d=128, nseg=1, max_pos=16)
    fwd_full = lib.mf_varlen_attn_workspace_size(8, 1, 128, 1, 16, 0, 0)
    fwd_small = lib.mf_varlen_attn_workspace_size(8, 1, 128, 1, 16, 0, 2)
    assert fwd_small < fwd_full
    assert _fwd(lib, ws=None, wsb=fwd_small, rot=FAKE, **fa) == -1
    assert _fwd(lib, ws=None, wsb=fwd_small - 1, rot=FAKE, **fa) == -3
    assert _fwd(lib, ws=None, wsb=fwd_small, rot=None, **fa) == -3
    assert _fwd(lib, ws=None, wsb=fwd_full, rot=None, **fa) == -1

    def bwd(wsb, rot):
        return lib.mf_varlen_attn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1, 8, FAKE,
                                      1e4, 16, 8, 2, 64, 0.0, rot, None, wsb, None, None)
    bwd_full = lib.mf_varlen_attn_workspace_size(8, 2, 64, 1, 16, 0, 1)
    bwd_small = lib.mf_varlen_attn_workspace_size(8, 2, 64, 1, 16, 0, 3)
    assert bwd_small == bwd_full - 2 * _align(8 * 2 * 64 * 2)
    assert bwd(bwd_small, FAKE) == -1
    assert bwd(bwd_small - 1, FAKE) == -3
    assert bwd(bwd_small, None) == -3
    assert bwd(bwd_full, None) == -1


def test_probe_argument_errors(lib):
    khz = ctypes.c_int32(0)
    assert lib.mf_mfma_probe(None, 4, 10, FAKE, FAKE, ctypes.byref(khz), None) == -1
    assert lib.mf_mfma_probe(FAKE, 0, 10, FAKE, FAKE, ctypes.byref(khz), None) == -1
    assert lib.mf_mfma_probe(FAKE, 4, 0, FAKE, FAKE, ctypes.byref(khz), None) == -1
    assert lib.mf_mfma_probe(FAKE, (1 << 20) + 1, 10, FAKE, FAKE, ctypes.byref(khz), None) == -1
    assert lib.mf_mfma_probe(FAKE + 8, 4, 10, FAKE, FAKE, ctypes.byref(khz), None) == -1  # operands misaligned
    assert lib.mf_mfma_probe(FAKE, 4, 10, FAKE, FAKE + 4, ctypes.byref(khz), None) == -1  # clocks misaligned
    assert lib.mf_mfma_probe(FAKE, 4, 10, None, FAKE, ctypes.byref(khz), None) == -1


def test_editing_argument_errors(lib):
    # mf_pack_edit: positions are [n][3] int32 (4-byte aligned); target rows required when gathering
    assert lib.mf_pack_edit(FAKE, -1, 10, FAKE, None, FAKE, FAKE, None, None, None, 0, None, None, None) == -1
    assert lib.mf_pack_edit(FAKE, 2, 10, FAKE, None, FAKE + 2, FAKE, None, None, None, 0, None, None, None) == -1
    assert lib.mf_pack_edit(FAKE, 2, 10, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, 16, FAKE, None, None) == -1
    assert lib.mf_pack_edit(FAKE, 2, 10, FAKE, None, FAKE, FAKE, None, None, FAKE, 0, None, None, None) == -1
    # 3D rope: same checks as 2D, a 4-byte aligned [n][3] pos, the wider table
    assert lib.mf_rope3d_apply(FAKE, 0, FAKE, 8, 1, 48, 1e4, 16, 0, FAKE, 1 << 20, None, None) == -2
    assert lib.mf_rope3d_apply(FAKE, 0, FAKE, 8, 1, 64, 1e4, 16, 0, FAKE,
                               lib.mf_rope3d_workspace_size(64, 16) - 1, None, None) == -3
    assert lib.mf_rope3d_apply(FAKE, 0, FAKE + 2, 8, 1, 64, 1e4, 16, 0, FAKE, 1 << 20, None, None) == -1
    # 3D attention: positions are mandatory and 4-byte aligned
    def fwd3(**kw):
        a = dict(pos=FAKE, d=128)
        a.update(kw)
        return lib.mf_varlen_attn3d_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1, 8, a["pos"], 1e4, 16, 8, 1,
                                        a["d"], 0.0, None, FAKE, 1 << 30, None, None)
    assert fwd3(pos=None) == -1
    assert fwd3(pos=FAKE + 2) == -1
    assert fwd3(d=96) == -2
    assert lib.mf_varlen_attn3d_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1, 8, None,
                                    1e4, 16, 8, 1, 64, 0.0, None, FAKE, 1 << 30, None, None) == -1


def test_editing_workspace_sizes(lib):
    # 3D table: 3D/16 row/column pairs + D/8 frame pairs per position
    assert lib.mf_rope3d_workspace_size(128, 640) == 640 * 40 * 8
    assert lib.mf_rope3d_workspace_size(64, 10) == (10 * 20 * 8 + 255) // 256 * 256
    # the attention workspace holds the wider table for either call
    n, h = 1000, 4
    table3 = 640 * 40 * 8
    assert lib.mf_varlen_attn_workspace_size(n, h, 128, 3, 640, 0, 0) >= table3 + n * h * 128 * 2


def test_flow_argument_errors(lib):
    # mf_rf_noise(z, eps, t, zt, dtype, cu_pieces, n_samples, frames, n_tokens, channels, stream, trace)
    assert lib.mf_rf_noise(FAKE, FAKE, FAKE, FAKE, 0, FAKE, 2, 1, 8, 96, None, None) == -2     # channels
    assert lib.mf_rf_noise(FAKE, FAKE, FAKE, FAKE, 2, FAKE, 2, 1, 8, 128, None, None) == -2    # dtype
    assert lib.mf_rf_noise(FAKE, FAKE, FAKE, FAKE, 0, FAKE, 2, 3, 8, 128, None, None) == -1    # frames
    assert lib.mf_rf_noise(FAKE, FAKE, None, FAKE, 0, FAKE, 2, 1, 8, 128, None, None) == -1    # t
    assert lib.mf_rf_noise(FAKE + 8, FAKE, FAKE, FAKE, 0, FAKE, 2, 1, 8, 128, None, None) == -1
    assert lib.mf_rf_noise(FAKE, FAKE, FAKE, FAKE, 0, None, 2, 1, 8, 128, None, None) == -1
    assert lib.mf_rf_noise(FAKE, FAKE, FAKE, FAKE, 0, FAKE, 2, 1, 0, 128, None, None) == 0
    # mf_rf_loss(v, z, eps, grad, loss, dtype, cu, n_samples, frames, n, C, scale, ws, wsb, stream, trace)
    assert lib.mf_rf_loss(FAKE, FAKE, FAKE, None, FAKE, 0, FAKE, 2, 1, 8, 128, 1.0, FAKE, 4, None, None) == -3
    assert lib.mf_rf_loss(FAKE, FAKE, FAKE, None, None, 0, FAKE, 2, 1, 8, 128, 1.0, FAKE, 64, None, None) == -1
    assert lib.mf_rf_loss(FAKE, FAKE, FAKE, FAKE + 4, FAKE, 0, FAKE, 2, 1, 8, 128, 1.0, FAKE, 64, None, None) == -1
    assert lib.mf_rf_loss(FAKE, FAKE, FAKE, None, FAKE, 0, FAKE, 2, 1, 8, 128, float("nan"), FAKE, 64, None,
                          None) == -1
    assert lib.mf_rf_loss_workspace_size(1000) == 4096
    # mf_cfg_combine(v, out, mismatched, dtype, cu, n_samples, n_pairs, n, C, scale, stream, trace)
    assert lib.mf_cfg_combine(FAKE, FAKE, None, 0, FAKE, 3, 2, 8, 128, 3.0, None, None) == -1   # 2 pairs > 3 samples
    assert lib.mf_cfg_combine(FAKE, FAKE, FAKE + 2, 0, FAKE, 4, 2, 8, 128, 3.0, None, None) == -1
    assert lib.mf_cfg_combine(FAKE, FAKE, None, 0, FAKE, 4, 2, 8, 1000, 3.0, None, None) == -2


def test_block_workspace_sizes(lib):
    # tile table of (frames + 1) n_samples + 1 ints, then the 3-axis rotary table (5D/16 pairs per position)
    assert lib.mf_block_workspace_size(9, 1, 128, 0) == 256
    assert lib.mf_block_workspace_size(100, 2, 128, 0) == 1280               # 301 ints -> 1204 -> 1280
    assert lib.mf_block_workspace_size(9, 1, 128, 640) == 256 + 640 * 40 * 8  # 204 800, already aligned
    assert lib.mf_block_workspace_size(9, 3, 128, 0) == 0                    # bad frames
    assert lib.mf_block_workspace_size(-1, 1, 128, 0) == 0


def test_block_argument_errors(lib):
    ws = lib.mf_block_workspace_size(2, 1, 128, 64)
    # mf_adaln_modulate(x, shift, scale, h, cu, n_samples, frames, n, C, eps, stream, trace)
    assert lib.mf_adaln_modulate(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 1, 8, 768, 1e-6, None, None) == -2   # C % 512
    assert lib.mf_adaln_modulate(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 1, 8, 16384, 1e-6, None, None) == -2  # C > 8192
    assert lib.mf_adaln_modulate(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 1, 8, 3072, 0.0, None, None) == -1   # eps
    assert lib.mf_adaln_modulate(FAKE, None, FAKE, FAKE, FAKE, 2, 1, 8, 3072, 1e-6, None, None) == -1  # shift
    assert lib.mf_adaln_modulate(FAKE + 8, FAKE, FAKE, FAKE, FAKE, 2, 1, 8, 3072, 1e-6, None, None) == -1
    assert lib.mf_adaln_modulate(FAKE, FAKE, FAKE, FAKE, None, 2, 1, 8, 3072, 1e-6, None, None) == -1  # cu
    assert lib.mf_adaln_modulate(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 0, 8, 3072, 1e-6, None, None) == -1  # frames
    assert lib.mf_adaln_modulate(None, None, None, None, FAKE, 2, 1, 0, 3072, 1e-6, None, None) == 0  # empty
    # mf_qkv_rope(h, wt, wi, bt, bi, q, k, v, cu, n_samples, frames, pos, nax, theta, max_pos, n, H, D, ws, wsb, ...)
    def qkv(**kw):
        a = dict(h=FAKE, wt=FAKE, wi=FAKE, bt=None, bi=None, q=FAKE, k=FAKE, v=FAKE, cu=FAKE, ns=2, fr=1, pos=FAKE,
                 nax=2, theta=10000.0, max_pos=64, n=8, H=24, D=128, ws=FAKE, wsb=ws)
        a.update(kw)
        return lib.mf_qkv_rope(a["h"], a["wt"], a["wi"], a["bt"], a["bi"], a["q"], a["k"], a["v"], a["cu"], a["ns"],
                               a["fr"], a["pos"], a["nax"], a["theta"], a["max_pos"], a["n"], a["H"], a["D"], a["ws"],
                               a["wsb"], None, None)
    assert qkv(D=96) == -2
    assert qkv(H=3, D=64) == -2                 # channels 192 not a multiple of 256
    assert qkv(H=0) == -1
    assert qkv(nax=4) == -1
    assert qkv(theta=0.0) == -1
    assert qkv(max_pos=0) == -1
    assert qkv(pos=FAKE + 4) == -1              # 2D positions are 8-byte aligned
    assert qkv(wi=None) == -1
    assert qkv(bt=FAKE + 4) == -1
    assert qkv(q=FAKE + 8) == -1
    assert qkv(wsb=ws - 1) == -3
    assert qkv(ws=FAKE + 16) == -1
    assert qkv(n=0, h=None, q=None) == 0        # empty: nothing to launch
    # mf_out_gated_residual(o, x, wt, wi, bt, bi, gate, y, proj, cu, n_samples, frames, n, C, ws, wsb, stream, trace)
    wso = lib.mf_block_workspace_size(2, 1, 64, 0)
    assert lib.mf_out_gated_residual(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None, FAKE, 2, 1, 8, 3000, FAKE,
                                     wso, None, None) == -2
    assert lib.mf_out_gated_residual(FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, None, FAKE, 2, 1, 8, 3072, FAKE,
                                     wso, None, None) == -1  # gate
    assert lib.mf_out_gated_residual(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, None, FAKE, 2, 1, 8, 3072, FAKE,
                                     4, None, None) == -3
    assert lib.mf_out_gated_residual(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE + 2, None, FAKE, 2, 1, 8, 3072,
                                     FAKE, wso, None, None) == -1
    assert lib.mf_out_gated_residual(FAKE, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE + 8, FAKE, 2, 1, 8, 3072,
                                     FAKE, wso, None, None) == -1  # proj misaligned


def test_block_bwd_workspace_sizes(lib):
    # adaLN: tile table, (mean, rstd) per row, then 2 C floats per 64-row block (4 per projection tile bound)
    # S = 2, frames 1, N = 1000, C = 3072: 5 ints -> 256; 8000 -> 8192; 4 (4 + 4) blocks x 24 KiB = 786 432
    assert lib.mf_adaln_modulate_bwd_workspace_size(2, 1, 1000, 3072) == 256 + 8192 + 786432
    assert lib.mf_adaln_modulate_bwd_workspace_size(2, 1, 1000, 768) == 0      # C % 512
    assert lib.mf_adaln_modulate_bwd_workspace_size(2, 3, 1000, 3072) == 0     # frames
    # QKV projection, no rotation, N = 1000, 24 x 128: tile table, columns, counts (3 x 256), transposed
    # weights 2 x 9216 x 3072 bf16, gathered operands [9216][1280] and [3072][1280] bf16 (1280 = 1024 + 256
    # token columns), bias block sums 20 x 9216 floats; one split (no split partials)
    qkv = 768 + 2 * 9216 * 3072 * 2 + 9216 * 1280 * 2 + 3072 * 1280 * 2 + 20 * 9216 * 4
    assert lib.mf_qkv_rope_bwd_workspace_size(2, 1, 1000, 24, 128, 0) == qkv
    # with rotation: the 3-axis table (5 D / 16 pairs per position) and the inverse-rotated dq, dk
    assert lib.mf_qkv_rope_bwd_workspace_size(2, 1, 1000, 24, 128, 640) == qkv + 640 * 40 * 8 + 2 * 1000 * 3072 * 2
    assert lib.mf_qkv_rope_bwd_workspace_size(2, 1, 1000, 24, 96, 0) == 0      # head_dim
    assert lib.mf_qkv_rope_bwd_workspace_size(2, 1, 1 << 23, 24, 128, 0) == 0  # too many tokens for the pitch
    assert lib.mf_qkv_rope_bwd_workspace_size(2, 1, 1000, 256, 128, 0) == 0   # channels > 16384
    # output projection, N = 50000, C = 3072: u [N][C] bf16, 4 (196 + 4) dgate blocks x 3072 floats,
    # transposed weights, gathered operands of 50176 + 256 = 50432 columns, 788 bias blocks, and fp32 chunk
    # sums for 6 (chunk, modality) items [6][3072][3072]: 144 output tiles, 1 + 5 chunks (720 workgroups, 3
    # rounds of 256 CUs for 1/5 of the tokens each)
    out = (768 + 50000 * 3072 * 2 + 800 * 3072 * 4 + 2 * 3072 * 3072 * 2 + 2 * 3072 * 50432 * 2 + 788 * 3072 * 4
           + 6 * 3072 * 3072 * 4)
    assert lib.mf_out_gated_residual_bwd_workspace_size(2, 1, 50000, 3072) == out
    assert lib.mf_out_gated_residual_bwd_workspace_size(2, 1, 50000, 3000) == 0


def test_block_bwd_argument_errors(lib):
    ws = lib.mf_qkv_rope_bwd_workspace_size(2, 1, 8, 24, 128, 64)
    # mf_adaln_modulate_bwd(dh, x, scale, dres, dx, dshift, dscale, cu, S, frames, n, C, eps, ws, wsb, stream, trace)
    wsa = lib.mf_adaln_modulate_bwd_workspace_size(2, 1, 8, 3072)

    def ada(**kw):
        a = dict(dh=FAKE, x=FAKE, sc=FAKE, dres=None, dx=FAKE, dsh=FAKE, dsc=FAKE, cu=FAKE, ns=2, fr=1, n=8, C=3072,
                 eps=1e-6, ws=FAKE, wsb=wsa)
        a.update(kw)
        return lib.mf_adaln_modulate_bwd(a["dh"], a["x"], a["sc"], a["dres"], a["dx"], a["dsh"], a["dsc"], a["cu"],
                                         a["ns"], a["fr"], a["n"], a["C"], a["eps"], a["ws"], a["wsb"], None, None)
    assert ada(C=768) == -2
    assert ada(C=16384) == -2
    assert ada(eps=0.0) == -1
    assert ada(dsc=None) == -1
    assert ada(dres=FAKE + 8) == -1
    assert ada(dh=FAKE + 2) == -1
    assert ada(cu=None) == -1
    assert ada(wsb=wsa - 1) == -3
    assert ada(ws=FAKE + 16) == -1

    # mf_qkv_rope_bwd(dq, dk, dv, h, wt, wi, dh, dwt, dwi, dbt, dbi, cu, S, frames, pos, nax, theta, max_pos, n, H,
    #                 D, ws, wsb, stream, trace)
    def qkv(**kw):
        a = dict(dq=FAKE, dk=FAKE, dv=FAKE, h=FAKE, wt=FAKE, wi=FAKE, dh=FAKE, dwt=FAKE, dwi=FAKE, dbt=None, dbi=None,
                 cu=FAKE, ns=2, fr=1, pos=FAKE, nax=2, theta=10000.0, max_pos=64, n=8, H=24, D=128, ws=FAKE, wsb=ws)
        a.update(kw)
        return lib.mf_qkv_rope_bwd(a["dq"], a["dk"], a["dv"], a["h"], a["wt"], a["wi"], a["dh"], a["dwt"], a["dwi"],
                                   a["dbt"], a["dbi"], a["cu"], a["ns"], a["fr"], a["pos"], a["nax"], a["theta"],
                                   a["max_pos"], a["n"], a["H"], a["D"], a["ws"], a["wsb"], None, None)
    assert qkv(D=96) == -2
    assert qkv(H=256) == -2                     # channels 32768 > 16384
    assert qkv(H=0) == -1
    assert qkv(nax=4) == -1
    assert qkv(max_pos=0) == -1
    assert qkv(dwt=None) == -1
    assert qkv(dwi=FAKE + 4) == -1
    assert qkv(dbt=FAKE + 2) == -1              # float alignment
    assert qkv(dq=FAKE + 8) == -1
    assert qkv(wsb=ws - 1) == -3
    assert qkv(n=1 << 23) == -2                 # too many tokens
    # mf_out_gated_residual_bwd(dy, o, proj, wt, wi, gate, d_o, dwt, dwi, dbt, dbi, dgate, cu, S, frames, n, C, ws,
    #                           wsb, stream, trace)
    wso = lib.mf_out_gated_residual_bwd_workspace_size(2, 1, 8, 3072)

    def out(**kw):
        a = dict(dy=FAKE, o=FAKE, proj=FAKE, wt=FAKE, wi=FAKE, gate=FAKE, do=FAKE, dwt=FAKE, dwi=FAKE, dbt=None,
                 dbi=None, dg=FAKE, cu=FAKE, ns=2, fr=1, n=8, C=3072, ws=FAKE, wsb=wso)
        a.update(kw)
        return lib.mf_out_gated_residual_bwd(a["dy"], a["o"], a["proj"], a["wt"], a["wi"], a["gate"], a["do"],
                                             a["dwt"], a["dwi"], a["dbt"], a["dbi"], a["dg"], a["cu"], a["ns"],
                                             a["fr"], a["n"], a["C"], a["ws"], a["wsb"], None, None)
    assert out(C=3000) == -2
    assert out(proj=None) == -1                 # the forward's pre-gate projection is required
    assert out(dg=None) == -1
    assert out(gate=FAKE + 4) == -1
    assert out(fr=0) == -1
    assert out(wsb=wso - 1) == -3
    assert out(ws=FAKE + 16) == -1


def test_binding_refuses_another_abi_version(tmp_path):
    """The argument lists follow one ABI version; a library built from other
    sources is refused at load, before any call."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    src = tmp_path / "old.c"
    src.write_text('int mf_abi_version(void) { return 4; }\nconst char* mf_status_string(int s) { return "x"; }\n')
    so = tmp_path / "libold.so"
    subprocess.run(["gcc", "-shared", "-fPIC", str(src), "-o", str(so)], check=True)
    import packed_varlen_attention_amd._binding as B
    saved = B._lib
    B._lib = None
    try:
        with pytest.raises(ImportError, match="ABI version 4"):
            B.load_library(str(so))
    finally:
        B._lib = saved


def test_binding_checks_the_rotated_buffer():
    """The ABI passes the rotated buffer as a bare pointer; the binding refuses
    a wrong dtype, a buffer smaller than 2 * q.numel() elements and one that
    overlaps another argument, before any call."""
    import torch

    from packed_varlen_attention_amd import _binding as B

    q = torch.empty((10, 2, 64), dtype=torch.bfloat16)
    k = torch.empty_like(q)
    B._check_rotated(None, q, (q, k))
    B._check_rotated(torch.empty((2,) + tuple(q.shape), dtype=torch.bfloat16), q, (q, k))
    with pytest.raises(ValueError):
        B._check_rotated(torch.empty((2,) + tuple(q.shape), dtype=torch.float32), q, (q, k))
    with pytest.raises(ValueError):
        B._check_rotated(torch.empty(2 * q.numel() - 1, dtype=torch.bfloat16), q, (q, k))
    big = torch.empty(4 * q.numel(), dtype=torch.bfloat16)
    q2 = big[: q.numel()].view(q.shape)
    with pytest.raises(ValueError):
        B._check_rotated(big[q.numel() // 2: q.numel() // 2 + 2 * q.numel()], q2, (q2, k))
    B._check_rotated(big[q.numel(): 3 * q.numel()], q2, (q2, k))


def test_noalloc_forward_argument_errors(lib):
    """The no-allocation forward refuses, before any launch: float32 input,
    a rotation without the rotated buffer, and a table plus schedule beyond
    its fixed 4 MiB scratch (MF_ERR_SCRATCH)."""
    def call(**kw):
        a = dict(dtype=0, pos=FAKE, max_pos=16, nseg=1, d=128, rot=FAKE)
        a.update(kw)
        return lib.mf_varlen_attn_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, a["dtype"], FAKE, a["nseg"], 8, a["pos"],
                                              10000.0, a["max_pos"], 8, 1, a["d"], 0.0, a["rot"], None, None)
    assert call(dtype=1) == -2
    assert call(rot=None) == -1
    assert call(rot=FAKE + 8) == -1
    assert call(max_pos=16385) == -5          # 16385 x 256 B of table > 4 MiB
    assert call(d=96) == -2

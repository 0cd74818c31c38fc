"""Oracle for packed 2D-RoPE variable-length attention: TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct CPU implementation in float64 (numpy) of what
the GPU path computes.  It exists to check the HIP kernels and must never be
reached from the product path: only ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import it.  It shares no code
with the HIP library or its Python binding, and imports neither.

Sources (the Mage-Flow pages):
* native-resolution packing under a fixed token budget, text and image tokens
  of one sample forming one joint attention context -- Mage-Flow paper
  section 3.2.1 "Model Architecture and Native Packing" (paperlayer.ai
  summary); rcap.io post, "native-resolution packed step" pseudo-code;
* per-sample 2D rotary embeddings at native positions -- same pseudo-code
  ("per_sample_2d_rope"); ai.thesatyajit.com explainer, "A backbone that
  doesn't crop" and its Figure 5 caption;
* block-diagonal (per-segment) multi-head joint self-attention, as run by
  variable-length attention kernels -- same sections;
* packed classifier-free guidance: conditional and unconditional branches are
  independent segments of one pass -- paper section 3.2.1; hyper.ai summary,
  "Experiment";
* editing: text, source-image and target-image tokens of one sample in one
  segment, with a frame-aware 3D rotary embedding that tells source from
  target -- paper section 3.2.2 "Conditioning and rectified-flow training"
  (hyper.ai summary); paperlayer.ai summary, "Method";
* the rectified flow-matching objective on the packed latents and the packed
  CFG combine -- ``oracle.flow``;
* the attention sub-block's fused chains (adaptive normalisation, the
  modality-specific QKV projection with the rotary embedding, the gated
  residual) -- ``oracle.block``.

The pages fix no formula for the rotation, the position assignment, the
softmax scale or the log-sum-exp.  The readings taken here are listed in each
module's docstring.

Pins: every function is checked by ``tests/test_oracle_*.py`` against closed
forms, invariants, brute force and library routines (see those files).
"""
from .pack import pack, positions, gather, pack_edit, positions_edit, gather_edit  # noqa: F401
from .rope import inv_freq, rope2d, rope3d, rope_axes, blocks3d  # noqa: F401
from .attention import attn_fwd, attn_bwd, attn_bwd_given, attn_fwd_rows  # noqa: F401
from . import flow  # noqa: F401
from . import block  # noqa: F401

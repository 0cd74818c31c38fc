/*
 * mf.h -- C ABI of the packed 2D-RoPE variable-length attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The library implements the data-parallel hot path of native-resolution
 * packed joint self-attention as the Mage-Flow pages describe it:
 *   - variable-length text and image-latent token segments packed into one
 *     contiguous stream under a token budget, with per-sample (row, col)
 *     positions (Mage-Flow paper section 3.2.1 "Model Architecture and Native
 *     Packing", paperlayer.ai summary; rcap.io post, "native-resolution packed
 *     step" pseudo-code);
 *   - per-sample 2D rotary position embedding on Q and K (same pseudo-code;
 *     ai.thesatyajit.com explainer, "A backbone that doesn't crop");
 *   - block-diagonal, non-causal multi-head attention over the packed stream,
 *     forward with log-sum-exp and backward (paper section 3.2.1; the pages
 *     name variable-length attention kernels for this step).
 * Packed classifier-free guidance needs no call of its own: the conditional
 * and unconditional branches of a prompt are two consecutive samples
 * (paper section 3.2.1; hyper.ai summary, "Experiment").
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers owned by the caller.  Inputs are
 *     const; outputs are written only where documented.  The library never
 *     allocates device memory: scratch space comes from the caller's
 *     `workspace`.  Its only global state is the fixed scratch array of
 *     mf_varlen_attn_fwd_noalloc and that array's address on each device.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call only enqueues work on it and never synchronises.  Calls
 *     make no allocation, copy, memset or host synchronisation, so a
 *     sequence of them can be captured in a HIP graph and replayed; a replay
 *     reads the inputs' memory as it is at replay time.
 *   - Every call validates its host arguments first; on an error it returns a
 *     negative mf_status and launches nothing.  A launch failure reported by
 *     the HIP runtime returns MF_ERR_HIP.
 *   - The last argument of every compute call is an optional mf_trace*
 *     (NULL for none), see below.
 *   - Tensors q, k, v, o, dout, dq, dk, dv have layout [n_tokens][n_heads]
 *     [head_dim], contiguous, 16-byte aligned.  q and k hold UN-rotated
 *     values; the library applies the rotation.  lse is [n_heads][n_tokens]
 *     float32 (natural log).
 *   - dtype MF_BF16: bfloat16 tensors; MF_F32: float32 tensors, rounded to
 *     bfloat16 (round-to-nearest-even) for the matrix products, with float32
 *     outputs.  Accumulation and softmax are float32 in both cases.
 *   - Positions, offsets and counts are int32.  pos is [n_tokens][2] =
 *     (row, col).
 *
 * Readings taken where the pages give no formula
 *   - pack: the longest order-preserving prefix of the samples that fits the
 *     budget; each sample is [its text tokens | its image grid, row-major];
 *   - positions: text token u of a sample is at (u, u); image token (r, c)
 *     is at (text_len + r, text_len + c);
 *   - rotation: dims [0, D/2) turn by the row and [D/2, D) by the column;
 *     adjacent pairs (2j, 2j+1), j < D/4, turn by p * theta^(-2j/(D/2))
 *     (the original rotary pairing);
 *   - softmax scale 1/sqrt(head_dim) unless given.
 */
#ifndef MF_H_
#define MF_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mf_status;

#define MF_OK 0
#define MF_ERR_INVALID_ARG (-1)  /* null pointer, bad size, misaligned pointer */
#define MF_ERR_UNSUPPORTED (-2)  /* head_dim not 64/128, unknown dtype */
#define MF_ERR_WORKSPACE (-3)    /* workspace smaller than the size query returns */
#define MF_ERR_HIP (-4)          /* the HIP runtime reported a launch error */
#define MF_ERR_SCRATCH (-5)      /* sizes beyond the fixed scratch of mf_varlen_attn_fwd_noalloc */

#define MF_BF16 0
#define MF_F32 1

#define MF_ABI_VERSION 7

/* One sample descriptor: text tokens, then a grid_h x grid_w latent grid. */
typedef struct mf_sample {
  int32_t text_len;
  int32_t grid_h;
  int32_t grid_w;
} mf_sample;

/*
 * Optional per-kernel timing, owned by the caller.  When a call receives a
 * non-NULL trace, it records start[i] before and stop[i] after its i-th
 * kernel launch (i < capacity) on the call's stream and names the kernel in
 * names[i]; count receives the number of kernels the call launched.  The
 * events are hipEvent_t handles the caller created (passed as void*).  A
 * NULL trace records nothing.  Tracing never changes results.
 */
#define MF_TRACE_MAX 16
typedef struct mf_trace {
  int32_t capacity;               /* pairs available in start/stop, <= MF_TRACE_MAX */
  int32_t count;                  /* out: kernels launched by the call */
  void* start[MF_TRACE_MAX];      /* hipEvent_t */
  void* stop[MF_TRACE_MAX];       /* hipEvent_t */
  const char* names[MF_TRACE_MAX];  /* out: static kernel names */
} mf_trace;

/* Human-readable text for a status code (static storage, never NULL). */
const char* mf_status_string(mf_status status);

/* MF_ABI_VERSION of the built library. */
int32_t mf_abi_version(void);

/*
 * mf_pack -- native-resolution packing (Mage-Flow paper section 3.2.1
 * "Model Architecture and Native Packing": variable-length text and image
 * sequences packed under a fixed token budget without text padding, each
 * image keeping its native latent grid; rcap.io post, the `pack(...,
 * budget=50_000)` step of its pseudo-code).
 *
 * samples      [n_samples] device array of descriptors (n_samples >= 0).
 * token_budget maximum packed tokens (>= 0).  The longest prefix of samples
 *              whose lengths text_len + grid_h * grid_w sum to at most the
 *              budget is packed; nothing is reordered, split or skipped.
 * cu_seqlens   [n_samples + 1] out.  cu_seqlens[i] = start of sample i for
 *              i <= n_packed; entries past n_packed hold n_tokens, so the
 *              array can be handed to the attention calls with
 *              n_segments = n_samples (trailing segments are empty).
 * cu_pieces    [2 * n_samples + 1] out, or NULL.  cu_pieces[2i] = start of
 *              sample i, cu_pieces[2i+1] = start of its image tokens; entries
 *              past 2 * n_packed hold n_tokens.
 * pos          [token_budget][2] out: (row, col) of packed token t for
 *              t < n_tokens; later rows are not written.
 * counts       [4] out: {n_packed, n_tokens, max_seqlen, max_pos} where
 *              max_pos = 1 + the largest coordinate in pos (0 if empty).  A
 *              negative field in any descriptor, or a sample longer than
 *              2^31 - 1 tokens, gives counts = {-1, 0, 0, 0} and all-zero
 *              offsets.
 * text_rows, image_rows
 *              [n_samples] device arrays of device pointers, or both NULL.
 *              text_rows[i] holds text_len rows, image_rows[i] holds
 *              grid_h * grid_w rows in row-major grid order, row_bytes each.
 *              A pointer for an empty part may be NULL.
 * row_bytes    bytes per row (> 0 when gathering).
 * packed       [token_budget][row_bytes] out, or NULL: packed row t is a bit
 *              copy of its source row, for t < n_tokens.
 * Two kernels: a single-workgroup scan, then a fill of positions and rows.
 */
mf_status mf_pack(const mf_sample* samples, int32_t n_samples, int32_t token_budget,
                  int32_t* cu_seqlens, int32_t* cu_pieces, int32_t* pos, int32_t* counts,
                  const void* const* text_rows, const void* const* image_rows,
                  int64_t row_bytes, void* packed, void* stream, mf_trace* trace);

/* Bytes of workspace mf_rope2d_apply needs: the cos/sin table. */
size_t mf_rope2d_workspace_size(int32_t head_dim, int32_t max_pos);

/*
 * mf_rope2d_apply -- per-sample axial 2D rotary embedding, in place (rcap.io
 * post, `per_sample_2d_rope` in the "native-resolution packed step"
 * pseudo-code; Mage-Flow paper section 3.3 lists RoPE among the fused
 * memory-bound chains).
 *
 * x        [n_tokens][n_heads][head_dim] in/out, dtype MF_BF16 or MF_F32.
 * pos      [n_tokens][2] (row, col); every coordinate must lie in
 *          [0, max_pos) (coordinates outside are clamped into it).
 * theta    frequency base (> 0), 10000 in the workloads here.
 * inverse  0: rotate by +angle; 1: by -angle (the transpose).
 * workspace >= mf_rope2d_workspace_size(head_dim, max_pos) bytes, 256-byte
 *          aligned.
 */
mf_status mf_rope2d_apply(void* x, int32_t dtype, const int32_t* pos, int32_t n_tokens,
                          int32_t n_heads, int32_t head_dim, double theta, int32_t max_pos,
                          int32_t inverse, void* workspace, size_t workspace_bytes,
                          void* stream, mf_trace* trace);

/*
 * Bytes of workspace the attention calls need.  flags: MF_WS_BACKWARD for
 * the backward call (else the forward); MF_WS_ROTATED when the call will be
 * given a `rotated` buffer, which then holds the rotated Q and K and the
 * workspace reserves no copies of its own (2 * n_tokens * n_heads *
 * head_dim * 2 bytes less for the backward, half that for the forward).  A
 * call given `rotated` accepts either size; one given none needs the size
 * queried without MF_WS_ROTATED.  Any other flag bit returns 0.
 */
#define MF_WS_BACKWARD 1
#define MF_WS_ROTATED 2
size_t mf_varlen_attn_workspace_size(int32_t n_tokens, int32_t n_heads, int32_t head_dim,
                                     int32_t n_segments, int32_t max_pos, int32_t dtype,
                                     int32_t flags);

/*
 * mf_varlen_attn_fwd -- block-diagonal multi-head attention over packed
 * segments, with 2D RoPE on Q and K (Mage-Flow paper section 3.2.1: joint
 * self-attention over the concatenated text and image tokens of a sample;
 * packed samples never attend to each other).
 *
 * For every segment s = [cu_seqlens[s], cu_seqlens[s+1]) and head h:
 *   S = softmax_scale * R(pos) q . (R(pos) k)^T   (non-causal, inside s)
 *   o = softmax(S) v,  lse = log(sum(exp(S))) per row.
 * q, k, v      [n_tokens][n_heads][head_dim] in.
 * o            same shape, out; rows outside every segment are not written.
 * lse          [n_heads][n_tokens] float32 out, or NULL.
 * cu_seqlens   [n_segments + 1] non-decreasing offsets within [0, n_tokens].
 * max_seqlen   an upper bound on every segment length (host value).
 * pos          [n_tokens][2] positions in [0, max_pos), or NULL for no
 *              rotation (then theta and max_pos are ignored).
 * softmax_scale 0 selects 1/sqrt(head_dim).
 * head_dim     64 or 128.
 * rotated      NULL, or a caller-owned, 16-byte aligned bf16 buffer of
 *              2 * n_tokens * n_heads * head_dim elements that keeps the
 *              rotated Q and K for the backward.  It is used only when the
 *              call rotates or converts them (pos non-NULL, or dtype
 *              MF_F32), and is then filled with R(pos) q rounded to bf16
 *              ([n_tokens][n_heads][head_dim]), followed by R(pos) k
 *              rounded to bf16.  In the Q half, rows outside every segment
 *              are not written; the K half is written for every row in
 *              [0, n_tokens).  It must not overlap any other argument.
 * workspace    >= mf_varlen_attn_workspace_size(...) bytes for the forward
 *              (MF_WS_ROTATED may be set when `rotated` is non-NULL).
 */
mf_status mf_varlen_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                             int32_t dtype, const int32_t* cu_seqlens, int32_t n_segments,
                             int32_t max_seqlen, const int32_t* pos, double theta,
                             int32_t max_pos, int32_t n_tokens, int32_t n_heads,
                             int32_t head_dim, float softmax_scale, void* rotated,
                             void* workspace, size_t workspace_bytes, void* stream,
                             mf_trace* trace);

/*
 * mf_varlen_attn_fwd_noalloc -- mf_varlen_attn_fwd for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): it takes no workspace and calls no
 * allocator.  Its scratch -- the rotary table and the work schedule -- lives
 * in a fixed 4 MiB array in the library's device image (each GPU the library
 * runs on holds its own copy until the process ends); the rotated K goes to
 * the caller's `rotated` buffer.
 *
 * Arguments, layouts and results are those of mf_varlen_attn_fwd (2D RoPE),
 * bit for bit, with these limits:
 *   dtype     MF_BF16 only (MF_ERR_UNSUPPORTED otherwise: float32 input would
 *             need bf16 copies of K and V as large as the inputs);
 *   rotated   required when pos is non-NULL (MF_ERR_INVALID_ARG if NULL);
 *   sizes     the table, max_pos * head_dim / 4 (cos, sin) float pairs
 *             rounded up to 256 bytes, plus 4 * n_segments + 3 int32 of
 *             schedule must fit 4 MiB, else MF_ERR_SCRATCH before any launch
 *             (at head_dim 128: max_pos up to 8192 with any n_segments the
 *             ABI accepts).
 * The array's device address is looked up on the first call on each device,
 * with the caller's current device; the stream must belong to that device.
 * Every launch writes the scratch it reads first, so nothing needs clearing;
 * each call overwrites what the previous one left.  Calls that overlap on one
 * GPU (concurrent streams, or threads sharing a device) share the array and
 * race: serialise them.
 */
mf_status mf_varlen_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                     int32_t dtype, const int32_t* cu_seqlens, int32_t n_segments,
                                     int32_t max_seqlen, const int32_t* pos, double theta,
                                     int32_t max_pos, int32_t n_tokens, int32_t n_heads,
                                     int32_t head_dim, float softmax_scale, void* rotated,
                                     void* stream, mf_trace* trace);

/*
 * mf_varlen_attn_bwd -- gradients of the attention above with respect to
 * the un-rotated q and k and to v, given dout (the training step the pages
 * sketch runs backward through the packed blocks: rcap.io pseudo-code; paper
 * section 3.3 reports fused forward-and-backward steps).
 *
 * o, lse       the forward's outputs on the same q, k, v.
 * dout         [n_tokens][n_heads][head_dim] in.
 * dq, dk, dv   same shape, out; rows outside every segment are not written.
 * With P = softmax(S): dv = P^T dout, dS = P * (dout v^T - rowsum(dout*o)),
 * dq = R(pos)^T (scale dS kr), dk = R(pos)^T (scale dS^T qr).  Deterministic:
 * no atomics, the same inputs give bit-identical outputs.
 * rotated      NULL, or the buffer the forward call on the same q, k, pos,
 *              theta, dtype and cu_seqlens filled, unmodified since.  When
 *              the call would rotate or convert Q and K, it reads them from
 *              there instead, which skips two passes over Q and K; the
 *              results are bit-identical to those with NULL.  Otherwise
 *              it is ignored.
 * workspace    >= mf_varlen_attn_workspace_size(...) bytes for the backward
 *              (MF_WS_BACKWARD; MF_WS_ROTATED may be set when `rotated` is non-NULL).
 */
mf_status mf_varlen_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, void* dq, void* dk, void* dv,
                             int32_t dtype, const int32_t* cu_seqlens, int32_t n_segments,
                             int32_t max_seqlen, const int32_t* pos, double theta,
                             int32_t max_pos, int32_t n_tokens, int32_t n_heads,
                             int32_t head_dim, float softmax_scale, const void* rotated,
                             void* workspace, size_t workspace_bytes, void* stream,
                             mf_trace* trace);

/*
 * Editing (frame-aware 3D RoPE).  For instruction-based editing, a sample's
 * conditioning tokens are followed by the source image's latents and then
 * the noisy target latents, and visual tokens carry (h, w, f) positions: the
 * frame tells source from target while the spatial positions correspond
 * (Mage-Flow paper section 3.2.2 "Conditioning and rectified-flow training",
 * hyper.ai summary; paperlayer.ai summary, "Method").  The pages do not say
 * how the head dimension is shared among the axes.  Readings taken here:
 *   - one editing sample is one segment [text | source | target]; source and
 *     target have the sample's grid_h x grid_w grid;
 *   - positions (row, col, frame): text token u -> (u, u, u); source token
 *     (r, c) -> (T + r, T + c, T); target token (r, c) -> (T + r, T + c, T + 1);
 *   - rotation blocks: dims [0, 3D/8) turn by the row, [3D/8, 3D/4) by the
 *     column, [3D/4, D) by the frame; inside a block of d dims the pair
 *     (2j, 2j+1) turns by p * theta^(-2j/d).
 * Positions are [n][3] int32 (4-byte aligned) in these calls.
 */

/*
 * mf_pack_edit -- mf_pack for editing samples.  A sample's length is
 * text_len + 2 * grid_h * grid_w; the budget policy, cu_seqlens, counts,
 * errors and row gather are those of mf_pack, with:
 * cu_pieces    [3 * n_samples + 1] out, or NULL: per sample its start, the
 *              start of its source tokens and the start of its target
 *              tokens; entries past 3 * n_packed hold n_tokens.
 * pos          [token_budget][3] out: (row, col, frame) of packed token t.
 * counts[3]    1 + the largest coordinate over all three axes.
 * text_rows, source_rows, target_rows
 *              [n_samples] device arrays of device pointers, or all NULL;
 *              source_rows[i] and target_rows[i] hold grid_h * grid_w rows
 *              each, row-major.
 */
mf_status mf_pack_edit(const mf_sample* samples, int32_t n_samples, int32_t token_budget,
                       int32_t* cu_seqlens, int32_t* cu_pieces, int32_t* pos, int32_t* counts,
                       const void* const* text_rows, const void* const* source_rows,
                       const void* const* target_rows, int64_t row_bytes, void* packed,
                       void* stream, mf_trace* trace);

/* Bytes of workspace mf_rope3d_apply needs: the cos/sin table. */
size_t mf_rope3d_workspace_size(int32_t head_dim, int32_t max_pos);

/*
 * mf_rope3d_apply -- mf_rope2d_apply with the frame-aware 3D rotation:
 * pos is [n_tokens][3] (row, col, frame), every coordinate in [0, max_pos);
 * workspace >= mf_rope3d_workspace_size(head_dim, max_pos) bytes.
 */
mf_status mf_rope3d_apply(void* x, int32_t dtype, const int32_t* pos, int32_t n_tokens,
                          int32_t n_heads, int32_t head_dim, double theta, int32_t max_pos,
                          int32_t inverse, void* workspace, size_t workspace_bytes,
                          void* stream, mf_trace* trace);

/*
 * mf_varlen_attn3d_fwd, mf_varlen_attn3d_bwd -- mf_varlen_attn_fwd and
 * mf_varlen_attn_bwd with the frame-aware 3D rotation: pos is
 * [n_tokens][3] (row, col, frame) and must not be NULL.  Every other
 * argument, the workspace size (mf_varlen_attn_workspace_size) and the
 * error behaviour are those of the 2D calls.
 */
mf_status mf_varlen_attn3d_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                               int32_t dtype, const int32_t* cu_seqlens, int32_t n_segments,
                               int32_t max_seqlen, const int32_t* pos, double theta,
                               int32_t max_pos, int32_t n_tokens, int32_t n_heads,
                               int32_t head_dim, float softmax_scale, void* rotated,
                               void* workspace, size_t workspace_bytes, void* stream,
                               mf_trace* trace);

mf_status mf_varlen_attn3d_bwd(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               int32_t dtype, const int32_t* cu_seqlens, int32_t n_segments,
                               int32_t max_seqlen, const int32_t* pos, double theta,
                               int32_t max_pos, int32_t n_tokens, int32_t n_heads,
                               int32_t head_dim, float softmax_scale, const void* rotated,
                               void* workspace, size_t workspace_bytes, void* stream,
                               mf_trace* trace);

/*
 * Rectified-flow objective on the packed latents.  Training regresses the
 * model's velocity v(z_t, t) on the target z - eps, with model input
 * z_t = (1 - t) z + t eps and eps ~ N(0, I) (Mage-Flow paper section 3.2.1 as
 * summarised on paperlayer.ai, "Method"; rcap.io post, the pseudo-code's
 * `loss = mse(v_pred, (z - noise))`); for editing, only target tokens carry
 * the loss (paper section 3.2.2, hyper.ai summary).
 *
 * Latent tensors are [n_tokens][channels] rows in packed order, dtype MF_BF16
 * or MF_F32, 16-byte aligned; channels is a power of two in [8, 512] (the
 * latent space has 128 channels).  cu_pieces is the packer's output for the
 * same samples: frames = 1 for a generation pack (mf_pack: start, image
 * start per sample), frames = 2 for an editing pack (mf_pack_edit: start,
 * source start, target start).  The noised rows of sample s are its image
 * rows (frames = 1) or its target rows (frames = 2); text rows and editing
 * source rows are conditioning.
 */

/* mf_rf_noise -- zt = (1 - t[s]) z + t[s] eps on sample s's noised rows,
 * zt = z on every other row.  t: device float[n_samples]. */
mf_status mf_rf_noise(const void* z, const void* eps, const float* t, void* zt, int32_t dtype,
                      const int32_t* cu_pieces, int32_t n_samples, int32_t frames, int32_t n_tokens,
                      int32_t channels, void* stream, mf_trace* trace);

/* Bytes of workspace mf_rf_loss needs (one float per row). */
size_t mf_rf_loss_workspace_size(int32_t n_tokens);

/*
 * mf_rf_loss -- target, loss and gradient in one pass over v, z and eps.
 * loss_sum   device float[n_samples] out: per sample, the sum over its noised
 *            rows and channels of (v - (z - eps))^2, reduced in a fixed
 *            order (deterministic).  The pack's mean-squared error is
 *            sum(loss_sum) / M with M = channels x noised rows.
 * grad       [n_tokens][channels] out, or NULL: grad_scale * (v - (z - eps))
 *            on noised rows, 0 elsewhere (grad_scale = 2 / M gives the
 *            gradient of the mean).
 * workspace  >= mf_rf_loss_workspace_size(n_tokens) bytes, 4-byte aligned.
 */
mf_status mf_rf_loss(const void* v, const void* z, const void* eps, void* grad, float* loss_sum,
                     int32_t dtype, const int32_t* cu_pieces, int32_t n_samples, int32_t frames,
                     int32_t n_tokens, int32_t channels, float grad_scale, void* workspace,
                     size_t workspace_bytes, void* stream, mf_trace* trace);

/*
 * mf_cfg_combine -- packed classifier-free guidance: the conditional and
 * unconditional branches of each prompt run as consecutive samples of one
 * pack (paper section 3.2.1; hyper.ai summary, "Experiment").  The pages
 * give no combine formula; this is the usual guidance form (Ho and Salimans,
 * "Classifier-Free Diffusion Guidance"):
 *   out[cond image row r] = v_u[r] + scale * (v_c[r] - v_u[r])
 * for pairs (2p, 2p + 1), p < n_pairs, of a generation pack (cu_pieces of
 * mf_pack, n_samples samples, 2 * n_pairs <= n_samples).  Every other row of
 * out is a copy of v; out may be v (in place).  A pair whose two images
 * differ in token count is left as a copy; mismatched (device int32, or
 * NULL) receives the number of such pairs.
 */
mf_status mf_cfg_combine(const void* v, void* out, int32_t* mismatched, int32_t dtype,
                         const int32_t* cu_pieces, int32_t n_samples, int32_t n_pairs,
                         int32_t n_tokens, int32_t channels, float scale, void* stream,
                         mf_trace* trace);

/*
 * The attention sub-block's fused chains around the packed joint attention.
 * The backbone follows MMDiT: joint self-attention over the concatenated
 * text and image tokens, with normalisation and projection layers specific
 * to each modality (Mage-Flow paper section 3.2.1, paperlayer.ai summary;
 * ai.thesatyajit.com explainer, Figure 5 caption); the training system fuses
 * the blocks' chains of adaptive normalisation, rotary embeddings and gated
 * residual updates (paper section 3.3 "Training Infrastructure").
 *
 * Rows are tokens in packed order: activations are bf16 [n_tokens][channels]
 * (channels = n_heads x head_dim), 16-byte aligned.  cu_pieces is the
 * packer's output for the same samples (frames = 1: mf_pack, frames = 2:
 * mf_pack_edit); the first piece of a sample is its text (modality 0), the
 * other pieces are image grids (modality 1).  Per-sample modulation vectors
 * shift, scale, gate are device float [n_samples][2][channels] (16-byte
 * aligned), indexed by (sample, modality).  Weights are bf16 [out][in]
 * (row-major, 16-byte aligned), one matrix per modality; biases are device
 * float[out] or NULL.  Only dtype MF_BF16 exists here.
 *
 * Size limits: channels a multiple of 256 (mf_adaln_modulate: of 512, at most
 * 8192); head_dim 64 or 128; n_heads <= 65535.  Rows of cu_pieces outside
 * [0, n_tokens] are clamped away on the device (an inconsistent cu_pieces
 * yields unwritten rows, never an out-of-bounds access).
 */

/* Bytes of workspace mf_qkv_rope and mf_out_gated_residual need (tile table
 * of (frames + 1) n_samples + 1 ints, then, for mf_qkv_rope, the rotary table
 * of max_pos positions). */
size_t mf_block_workspace_size(int32_t n_samples, int32_t frames, int32_t head_dim, int32_t max_pos);

/*
 * mf_adaln_modulate -- h = LN(x) * (1 + scale[s][m]) + shift[s][m] per token
 * of sample s, modality m.  LN is LayerNorm over the channels without an
 * affine of its own: population variance, statistics in fp32, eps as given
 * (1e-6 is the DiT convention).  h may be x (in place).  Rows outside every
 * piece are normalised without modulation.
 */
mf_status mf_adaln_modulate(const void* x, const float* shift, const float* scale, void* h,
                            const int32_t* cu_pieces, int32_t n_samples, int32_t frames,
                            int32_t n_tokens, int32_t channels, float eps, void* stream,
                            mf_trace* trace);

/*
 * mf_qkv_rope -- [q | k | v] = h W_m^T + b_m with the token's modality m
 * (W_m bf16 [3 channels][channels], b_m float[3 channels] or NULL), q and k
 * rotated by the token's position, all three written bf16
 * [n_tokens][n_heads][head_dim] (q, k, v must not overlap h).  pos is the
 * packer's positions ([n_tokens][2] with nax = 2, [n_tokens][3] with nax = 3,
 * the same rotation as mf_rope2d_apply / mf_rope3d_apply with theta and
 * max_pos), or NULL for no rotation.  The rotated q and k feed
 * mf_varlen_attn_fwd with pos = NULL; its backward then returns gradients
 * with respect to the rotated q and k.
 * workspace  >= mf_block_workspace_size(n_samples, frames, head_dim, max_pos)
 *            bytes, 256-byte aligned.
 */
mf_status mf_qkv_rope(const void* h, const void* w_text, const void* w_image, const float* b_text,
                      const float* b_image, void* q, void* k, void* v, const int32_t* cu_pieces,
                      int32_t n_samples, int32_t frames, const int32_t* pos, int32_t nax,
                      double theta, int32_t max_pos, int32_t n_tokens, int32_t n_heads,
                      int32_t head_dim, void* workspace, size_t workspace_bytes, void* stream,
                      mf_trace* trace);

/*
 * mf_out_gated_residual -- y = x + gate[s][m] * (o W_o,m^T + b_o,m) with the
 * token's sample s and modality m (W_o,m bf16 [channels][channels], b_o,m
 * float[channels] or NULL).  o is the attention output ([N][H][D] is
 * [N][channels]); y may be x (in place) but must not overlap o.
 * proj       bf16 [n_tokens][channels], out, or NULL: o W_o,m^T + b_o,m
 *            before the gate, which mf_out_gated_residual_bwd needs for the
 *            gate's gradient.
 * workspace  >= mf_block_workspace_size(n_samples, frames, 64, 0) bytes,
 *            256-byte aligned.
 */
mf_status mf_out_gated_residual(const void* o, const void* x, const void* w_text, const void* w_image,
                                const float* b_text, const float* b_image, const float* gate, void* y, void* proj,
                                const int32_t* cu_pieces, int32_t n_samples, int32_t frames,
                                int32_t n_tokens, int32_t channels, void* workspace,
                                size_t workspace_bytes, void* stream, mf_trace* trace);

/*
 * Backward of the three chains: the gradient of a scalar loss with respect to
 * every input of a chain, given the gradient of its output (the chain rule
 * through the forward definitions above).  Sums over rows -- weight, bias and
 * modulation gradients -- are deterministic: partial sums over fixed blocks of
 * rows, then added in a fixed order, so repeated calls give identical bits.
 * Weight and bias gradients are float [out][in] / float[out] per modality and
 * are OVERWRITTEN (not accumulated); modulation gradients are float
 * [n_samples][2][channels].  A modality without tokens gets zero gradients.
 * Rows outside every piece take no part in the sums, and their rows of dh
 * and d_o are not written (the forward projections do not write them
 * either); the adaLN backward writes dx for every row.
 *
 * The weight gradient gathers each modality's rows into token-contiguous
 * operands in the workspace, so n_tokens is at most 2^23 - 512 for
 * mf_qkv_rope_bwd and mf_out_gated_residual_bwd, and channels at most 16384.
 */

/* Bytes of workspace of mf_adaln_modulate_bwd (0 for unsupported sizes). */
size_t mf_adaln_modulate_bwd_workspace_size(int32_t n_samples, int32_t frames, int32_t n_tokens,
                                            int32_t channels);

/*
 * mf_adaln_modulate_bwd -- backward of mf_adaln_modulate:
 *   dx = dres + rstd (g - mean(g) - xhat mean(g xhat)),  g = dh (1 + scale[s][m]),
 *   dshift[s][m] = sum of dh, dscale[s][m] = sum of dh xhat over the rows of
 *   sample s, modality m (xhat = LN(x), statistics recomputed from x as the
 *   forward computes them).
 * dh, x      bf16 [n_tokens][channels], in.
 * scale      the forward's float [n_samples][2][channels], in.
 * dres       bf16 [n_tokens][channels] or NULL: a gradient added to dx (the
 *            residual branch of x), in.  dx may alias dres, not dh or x.
 * dx         bf16 [n_tokens][channels], out.
 * dshift, dscale  float [n_samples][2][channels], out.
 * channels a multiple of 512, at most 8192.
 */
mf_status mf_adaln_modulate_bwd(const void* dh, const void* x, const float* scale, const void* dres, void* dx,
                                float* dshift, float* dscale, const int32_t* cu_pieces, int32_t n_samples,
                                int32_t frames, int32_t n_tokens, int32_t channels, float eps, void* workspace,
                                size_t workspace_bytes, void* stream, mf_trace* trace);

/* Bytes of workspace of mf_qkv_rope_bwd; max_pos 0 when pos will be NULL (0
 * for unsupported sizes). */
size_t mf_qkv_rope_bwd_workspace_size(int32_t n_samples, int32_t frames, int32_t n_tokens, int32_t n_heads,
                                      int32_t head_dim, int32_t max_pos);

/*
 * mf_qkv_rope_bwd -- backward of mf_qkv_rope.  With G = [dq' | dk' | dv]
 * ([n_tokens][3 channels], dq' and dk' the inverse rotation of dq and dk by
 * pos, or dq and dk themselves when pos is NULL):
 *   dh = G W_m per token of modality m, dW_m = G_m^T h_m, db_m = column sums
 *   of G_m, where _m takes modality m's rows.
 * dq, dk, dv bf16 [n_tokens][n_heads][head_dim], in: gradients of the
 *            projection's outputs as mf_qkv_rope wrote them (rotated q, k).
 * h          bf16 [n_tokens][channels], in: the forward's input.
 * w_text, w_image  the forward's weights, bf16 [3 channels][channels], in.
 * dh         bf16 [n_tokens][channels], out (must not overlap the inputs).
 * dw_text, dw_image  float [3 channels][channels], out.
 * db_text, db_image  float [3 channels], out, or NULL to skip.
 * pos, nax, theta, max_pos  as given to mf_qkv_rope.
 */
mf_status mf_qkv_rope_bwd(const void* dq, const void* dk, const void* dv, const void* h, const void* w_text,
                          const void* w_image, void* dh, float* dw_text, float* dw_image, float* db_text,
                          float* db_image, const int32_t* cu_pieces, int32_t n_samples, int32_t frames,
                          const int32_t* pos, int32_t nax, double theta, int32_t max_pos, int32_t n_tokens,
                          int32_t n_heads, int32_t head_dim, void* workspace, size_t workspace_bytes, void* stream,
                          mf_trace* trace);

/* Bytes of workspace of mf_out_gated_residual_bwd (0 for unsupported sizes). */
size_t mf_out_gated_residual_bwd_workspace_size(int32_t n_samples, int32_t frames, int32_t n_tokens,
                                                int32_t channels);

/*
 * mf_out_gated_residual_bwd -- backward of mf_out_gated_residual.  With
 * u = gate[s][m] dy per token of sample s, modality m:
 *   d_o = u W_o,m, dW_o,m = u_m^T o_m, db_o,m = column sums of u_m,
 *   dgate[s][m] = sum of dy proj over the rows of sample s, modality m.
 * The gradient with respect to x is dy itself (the residual path); no call
 * is needed for it.
 * dy         bf16 [n_tokens][channels], in.
 * o          the forward's attention output, bf16 [n_tokens][channels], in.
 * proj       the forward's pre-gate projection (mf_out_gated_residual's
 *            proj output), bf16 [n_tokens][channels], in.
 * w_text, w_image  the forward's weights, bf16 [channels][channels], in.
 * gate       float [n_samples][2][channels], in.
 * d_o        bf16 [n_tokens][channels], out (must not overlap the inputs).
 * dw_text, dw_image  float [channels][channels], out.
 * db_text, db_image  float [channels], out, or NULL to skip.
 * dgate      float [n_samples][2][channels], out.
 */
mf_status mf_out_gated_residual_bwd(const void* dy, const void* o, const void* proj, const void* w_text,
                                    const void* w_image, const float* gate, void* d_o, float* dw_text,
                                    float* dw_image, float* db_text, float* db_image, float* dgate,
                                    const int32_t* cu_pieces, int32_t n_samples, int32_t frames, int32_t n_tokens,
                                    int32_t channels, void* workspace, size_t workspace_bytes, void* stream,
                                    mf_trace* trace);

/*
 * mf_mfma_probe -- measurement helper, not a step of the path: the sustained
 * rate of the 32x32x16 bf16 matrix instruction on the caller's operand values
 * and the shader clock meanwhile.  Throughput figures of the attention
 * kernels are quoted against the datasheet peak, which assumes the top
 * clock; this call measures what the chip sustains under a full matrix load
 * with realistic data, where power limits lower the clock.
 *
 * operands     device, 4096 vectors of 8 bf16 (64 KiB), 16-byte aligned, in;
 *              wave lanes cycle through them as A and B fragments.
 * n_blocks     workgroups of 256 threads (4 waves), 1 .. 2^20.
 * iters        loop trips; each wave issues 4 * iters instructions of
 *              32 * 32 * 16 * 2 = 32768 flops each, so the launch performs
 *              n_blocks * 4 * 4 * iters * 32768 flops.
 * sink         device float[n_blocks * 256], out: accumulator sums (keeps
 *              the work observable; the values carry no meaning).
 * clocks       device uint64[2 * n_blocks], out: per workgroup, shader-clock
 *              ticks and wall-clock ticks between its first and last
 *              instruction.
 * wall_clock_khz  host int32*, out (may be NULL): the wall counter's rate,
 *              written before the call returns.
 * Returns MF_ERR_INVALID_ARG for a NULL or misaligned pointer or a size out
 * of range, MF_ERR_HIP if the launch fails.
 */
mf_status mf_mfma_probe(const void* operands, int32_t n_blocks, int32_t iters, float* sink,
                        uint64_t* clocks, int32_t* wall_clock_khz, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MF_H_ */

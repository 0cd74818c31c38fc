// Host-side launchers of the library's kernels (internal; the public C ABI
// lives in include/mf.h and csrc/api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace mf {

constexpr int kDtypeBf16 = 0;
constexpr int kDtypeF32 = 1;

// frames = 1: samples are [text | image], positions (row, col);
// frames = 2: editing samples [text | source | target], positions (row, col, frame).
hipError_t launch_pack_scan(const void* samples, int n, int budget, int frames, int* cu_seqlens, int* cu_pieces,
                            int* counts, hipStream_t stream);

hipError_t launch_pack_fill(const void* samples, int budget, int frames, const int* cu_seqlens, const int* counts,
                            int* pos, const void* const* text_rows, const void* const* image_rows,
                            const void* const* target_rows, long long row_bytes, void* packed, hipStream_t stream);

// (cos, sin) pairs per position of the rotary table: D/4 (2 axes) or 5D/16 (3 axes).
int rope_table_width(int head_dim, int nax);

hipError_t launch_rope_table(float2* tab, int max_pos, int head_dim, int nax, double theta, hipStream_t stream);

// dst = rotate(src) (or a plain copy/convert when rotate is false); pos is
// [n_tokens][nax] int32.
hipError_t launch_rope_apply(const void* src, int src_dtype, void* dst, int dst_dtype, const int* pos, int nax,
                             const float2* tab, int max_pos, int n_tokens, int heads, int head_dim,
                             bool rotate, bool inverse, hipStream_t stream);

// Longest-first schedule of (segment, tile) work; see sched.hip.
hipError_t launch_sched(const int* cu_seqlens, int n_segments, int n_tokens, int tile, int* order, int* pt,
                        hipStream_t stream);
// Virtual segments: runs of tiny segments (at most kTinySegment tokens)
// merged for multi-segment tiles (see sched.hip); vcu and vfirst hold
// n_segments + 1 ints each.
constexpr int kTinySegment = 128;
hipError_t launch_merge_tiny(const int* cu_seqlens, int n_segments, int n_tokens, int* vcu, int* vfirst,
                             hipStream_t stream);
// Blocks to launch for a schedule with the given tile size (an upper bound).
long long sched_grid(int n_tokens, int n_segments, int heads, int tile);

constexpr int kFwdTile = 256;   // query rows per forward workgroup (8 waves)
constexpr int kDqTile = 256;    // query rows per dq workgroup (8 waves)
constexpr int kDkdvTile = 128;  // keys per dkdv workgroup

struct AttnArgs {
  const int* cu_seqlens;
  int n_segments;
  int max_seqlen;
  int n_tokens;
  int n_heads;
  int head_dim;
  int dtype;  // of q/k/v/o/dout/dq/dk/dv
  const int* pos;  // [n_tokens][nax]; nullptr: no rotation
  int nax;         // 2: axial 2D rotation, 3: frame-aware 3D rotation
  const float2* tab;
  int max_pos;
  float scale;
  const int* order;  // schedule: segments longest first
  const int* pt;     // schedule: tile prefix in that order
  // Multi-segment tiles: cu_seqlens above holds the virtual segments; rcu is
  // the caller's cu_seqlens and vfirst[v] the first real segment of virtual
  // segment v (both nullptr: every virtual segment is one real segment).
  const int* rcu;
  const int* vfirst;
};

// q: caller's (rotated in-kernel), kr/vb: bf16 [N][H][D] (kr already rotated).
hipError_t launch_attn_fwd(const AttnArgs& a, const void* q, const void* kr, const void* vb, void* o,
                           float* lse, hipStream_t stream);

// qr/kr rotated bf16, vb/dob bf16, lse2 in log2 units; outputs in a.dtype.
hipError_t launch_attn_bwd_dkdv(const AttnArgs& a, const void* qr, const void* kr, const void* vb,
                                const void* dob, const float* lse, const float* delta, void* dk, void* dv,
                                hipStream_t stream);

// dq also writes the row statistics dkdv reads (so it runs first):
// delta = rowsum(dout * o), lse2 = lse * log2(e), both [H][N].  o and dout
// are the caller's tensors (a.dtype).
hipError_t launch_attn_bwd_dq(const AttnArgs& a, const void* qr, const void* kr, const void* vb,
                              const void* dob, const void* o, const void* dout, const float* lse, float* lse2,
                              float* delta, void* dq, hipStream_t stream);

// Rectified-flow noising / loss and the packed CFG combine over [N][C]
// latent rows (C / 8 a power of two <= 64); see flow.hip.
hipError_t launch_rf_noise(const void* z, const void* eps, const float* t, void* zt, int dtype, const int* cu_pieces,
                           int n_samples, int frames, int n_tokens, int channels, hipStream_t stream);
hipError_t launch_rf_loss(const void* v, const void* z, const void* eps, void* grad, float* row_sum,
                          float* loss_sum, int dtype, const int* cu_pieces, int n_samples, int frames, int n_tokens,
                          int channels, float grad_scale, hipStream_t stream);
hipError_t launch_cfg_combine(const void* v, void* out, int* mismatched, int dtype, const int* cu_pieces,
                              int n_pairs, int n_tokens, int channels, float scale, hipStream_t stream);

// The attention sub-block's fused chains (see block.hip).  Projections tile
// the token rows per piece: tstart (n_pieces + 1 ints) holds each piece's
// first tile, written by launch_piece_tiles.  bf16 [N][C] rows, C = H D, a
// multiple of 256 (512 for adaln); weights bf16 [out][in], biases and the
// modulation vectors ([S][2][C]) fp32.
int block_tile_rows();
// Row tiles of a projection over n_tokens rows in n_pieces pieces (an upper bound).
int block_mtiles_bound(int n_tokens, int n_pieces);
hipError_t launch_piece_tiles(const int* cu_pieces, int n_pieces, int n_tokens, int* tstart, hipStream_t stream);
hipError_t launch_adaln(const void* x, const float* shift, const float* scale, const int* cu_pieces, int n_samples,
                        int frames, int n_tokens, int channels, float eps, void* h, hipStream_t stream);
hipError_t launch_qkv_rope(const void* h, const void* w_text, const void* w_image, const float* b_text,
                           const float* b_image, const int* cu_pieces, const int* tstart, int n_samples, int frames,
                           int n_tokens, int n_heads, int head_dim, const int* pos, int nax, const float2* tab,
                           int max_pos, void* q, void* k, void* v, hipStream_t stream);
hipError_t launch_out_gated(const void* o, const void* x, const void* w_text, const void* w_image,
                            const float* b_text, const float* b_image, const float* gate, const int* cu_pieces,
                            const int* tstart, int n_samples, int frames, int n_tokens, int channels, void* y,
                            void* proj, hipStream_t stream);

// Backward of the chains (see block_bwd.hip).  Weight gradients gather each
// modality's rows into feature-major operands of block_bwd_cols(n_tokens)
// token columns (text first, then image, each run padded to 256); col0 and kr
// (n_samples (frames + 1) + 2 and 2 ints) describe that layout.  Partial sums
// run over blocks of 64 rows: 4 block_mtiles_bound(n_tokens, n_pieces) rows.
constexpr int kAdaBwdMaxC = 8192;
int block_bwd_cols(int n_tokens);
// (chunk, modality) work items of a weight gradient [n_rows][n_cols], >= 2.
int block_bwd_splits(int n_tokens, int n_rows, int n_cols);
hipError_t launch_modality_cols(const int* cu_pieces, int n_samples, int frames, int n_tokens, int* col0, int* kr,
                                hipStream_t stream);
// dst [cols][rows] = src [rows][cols]^T (bf16, rows and cols multiples of 64).
hipError_t launch_transpose(const void* src, int rows, int cols, void* dst, hipStream_t stream);
// dst [n_src seg][pitch]: the modality-gathered, transposed rows of the
// n_src sources [n_tokens][seg]; part [pitch / 64][n_src seg] column sums of
// 64-column blocks, or nullptr.
hipError_t launch_gather_t(const void* const* src, int n_src, int seg, const int* cu_pieces, const int* col0,
                           const int* kr, int n_samples, int frames, int n_tokens, void* dst, long long pitch,
                           float* part, hipStream_t stream);
hipError_t launch_gate_bwd(const void* dy, const void* proj, const float* gate, const int* cu_pieces,
                           const int* tstart, int n_samples, int frames, int n_tokens, int channels, void* u,
                           float* part, hipStream_t stream);
hipError_t launch_adaln_bwd(const void* dh, const void* x, const float* scale, const void* dres,
                            const int* cu_pieces, const int* tstart, int n_samples, int frames, int n_tokens,
                            int channels, float eps, void* dx, float2* stats, float* part, hipStream_t stream);
// out [n_samples][2][ncol] = sums of the partial rows (stride floats, from
// column col_off) of each (sample, modality).
hipError_t launch_group_sum(const float* part, long long stride, int col_off, int ncol, const int* tstart,
                            int n_samples, int frames, int n_tokens, float* out, hipStream_t stream);
hipError_t launch_bias_sum(const float* part, int n_feat, const int* kr, long long pitch, float* db0, float* db1,
                           hipStream_t stream);
// out [n_tokens][n_out] = [g0 | g1 | ...] W_m with W_m given transposed ([n_out][n_src kseg]).
hipError_t launch_dgrad(const void* const* g, int n_src, int kseg, const void* wt0, const void* wt1,
                        const int* cu_pieces, const int* tstart, int n_samples, int frames, int n_tokens, int n_out,
                        void* out, hipStream_t stream);
// dw_m [n_rows][n_cols] = at_m bt_m^T over modality m's token columns, cut
// into `pairs` (chunk, modality) items; chunk sums of a modality with several
// chunks go to part (pairs n_rows n_cols floats when pairs > 2) and
// launch_split_sum adds them into dw_m.
hipError_t launch_wgrad(const void* at, const void* bt, long long pitch, int n_rows, int n_cols, const int* kr,
                        int pairs, float* part, float* dw0, float* dw1, hipStream_t stream);
hipError_t launch_split_sum(const float* part, long long pitch, int n_rows, int n_cols, const int* kr, int pairs,
                            float* dw0, float* dw1, hipStream_t stream);
}  // namespace mf

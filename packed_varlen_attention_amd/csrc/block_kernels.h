// Host-side launchers of the attention sub-block's chain kernels (internal;
// the public C ABI lives in include/mf.h and csrc/api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace mf {

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
// Inverse rotation applied by launch_gather_t to its first two sources (dq,
// dk) on the way through; the rotated-back rows also go token-major to
// out_q and out_k ([n_tokens][seg], rows inside the pieces only).
struct GatherRotation {
  const int* pos;
  int nax, max_pos, head_dim;
  const float2* tab;
  void* out_q;
  void* out_k;
};
// dst [n_src seg][pitch]: the modality-gathered, transposed rows of the
// n_src sources [n_tokens][seg]; part [pitch / 64][n_src seg] column sums of
// 64-column blocks, or nullptr; rot, or nullptr.
hipError_t launch_gather_t(const void* const* src, int n_src, int seg, const int* cu_pieces, const int* col0,
                           const int* kr, int n_samples, int frames, int n_tokens, void* dst, long long pitch,
                           float* part, const GatherRotation* rot, hipStream_t stream);
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

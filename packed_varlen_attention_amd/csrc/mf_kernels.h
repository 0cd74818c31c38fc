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

constexpr int kFwdTile = 128;   // query rows per forward workgroup (4 waves, 32-key tiles)
constexpr int kFwdTileLong = 256;  // the same for packs of long segments (8 waves, 64-key tiles)
// The forward's shape for a call.  The 128-row form runs three workgroups per
// CU; the 256-row form shares each K/V tile among twice the rows and is
// faster once every sweep is long: by 2% on packs of 16k-token segments,
// while the 128-row form is faster by 1% at 8k, 5% at 4k and 7% at 2k.  So
// the 256-row form is taken when the longest segment has at least 12288
// tokens and the mean one at least 8192.
inline int fwd_tile(int max_seqlen, int n_tokens, int n_segments) {
  return max_seqlen >= 12288 && static_cast<long long>(n_tokens) >= 8192LL * n_segments ? kFwdTileLong : kFwdTile;
}
constexpr int kDqTile = 256;    // query rows per dq workgroup (8 waves)
constexpr int kDqTileMerged = 128;  // the same when tiny segments are merged (4 waves)
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
  // Forward only: if non-null, the rotated bf16 Q [n_tokens][n_heads][head_dim]
  // is written here for the backward.
  void* qr_out;
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
}  // namespace mf

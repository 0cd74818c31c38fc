// Public C ABI (include/mf.h): host-side argument checks, workspace layout and
// kernel launches.  Nothing here synchronises; every error is detected
// before the first launch of a call.
#include "mf.h"

#include <math.h>
#include <stdint.h>

#include <mutex>

#include "block_kernels.h"
#include "mf_kernels.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned16_or_null(const void* p) { return p == nullptr || aligned16(p); }

mf_status from_hip(hipError_t e) { return e == hipSuccess ? MF_OK : MF_ERR_HIP; }

// Records the caller's events around each kernel launch of one call.
class Tracer {
 public:
  Tracer(mf_trace* t, hipStream_t s) : t_(t), s_(s) {
    if (t_ != nullptr) t_->count = 0;
  }
  // Runs one launcher between the i-th (start, stop) event pair.
  template <typename F>
  hipError_t run(const char* name, F&& launch) {
    const bool rec = t_ != nullptr && i_ < t_->capacity && i_ < MF_TRACE_MAX;
    if (rec) {
      t_->names[i_] = name;
      if (hipEventRecord(static_cast<hipEvent_t>(t_->start[i_]), s_) != hipSuccess) return hipErrorInvalidValue;
    }
    const hipError_t e = launch();
    if (e != hipSuccess) return e;
    if (rec && hipEventRecord(static_cast<hipEvent_t>(t_->stop[i_]), s_) != hipSuccess) return hipErrorInvalidValue;
    ++i_;
    if (t_ != nullptr) t_->count = i_;
    return hipSuccess;
  }

 private:
  mf_trace* t_;
  hipStream_t s_;
  int i_ = 0;
};

bool trace_ok(const mf_trace* t) {
  if (t == nullptr) return true;
  if (t->capacity < 0 || t->capacity > MF_TRACE_MAX) return false;
  for (int i = 0; i < t->capacity; ++i)
    if (t->start[i] == nullptr || t->stop[i] == nullptr) return false;
  return true;
}

// Elements in one half of the caller's `rotated` buffer: one bf16 [n][H][D] tensor.
size_t rotated_half(int32_t n_tokens, int32_t n_heads, int32_t head_dim) {
  return static_cast<size_t>(n_tokens) * n_heads * head_dim;
}

// Workspace of the attention calls, in order; each part 256-byte aligned.
struct AttnWorkspace {
  size_t tab = 0, kr = 0, qr = 0, vb = 0, dob = 0, delta = 0, sched = 0, total = 0;
  size_t tab_off = 0, kr_off = 0, qr_off = 0, vb_off = 0, dob_off = 0, delta_off = 0, sched_off = 0;
};

AttnWorkspace attn_workspace(int32_t n_tokens, int32_t n_heads, int32_t head_dim, int32_t n_segments,
                             int32_t max_pos, int32_t dtype, bool backward, bool kept) {
  AttnWorkspace w;
  // schedules (order, tile prefix): one for the forward; dkdv's and dq's for
  // the backward; then the virtual segments (offsets, first segment) that
  // merge runs of tiny segments into multi-segment tiles
  const size_t nseg = static_cast<size_t>(n_segments > 0 ? n_segments : 0);
  w.sched = ((backward ? 2 : 1) * (2 * nseg + 1) + 2 * (nseg + 1)) * sizeof(int32_t);
  const size_t tensor_bf16 = static_cast<size_t>(n_tokens) * n_heads * head_dim * 2;
  // rotary table, sized for the wider (3-axis) layout so one size serves both
  w.tab = static_cast<size_t>(max_pos > 0 ? max_pos : 0) * mf::rope_table_width(head_dim, 3) * sizeof(float2);
  // rotated (or converted) K, and Q for the backward; none when the caller's
  // `rotated` buffer holds them
  w.kr = kept ? 0 : tensor_bf16;
  w.qr = (backward && !kept) ? tensor_bf16 : 0;
  w.vb = dtype == MF_F32 ? tensor_bf16 : 0;
  w.dob = (backward && dtype == MF_F32) ? tensor_bf16 : 0;
  w.delta = backward ? 2 * static_cast<size_t>(n_tokens) * n_heads * sizeof(float) : 0;  // delta, lse2
  size_t off = 0;
  w.tab_off = off;
  off += align_up(w.tab);
  w.kr_off = off;
  off += align_up(w.kr);
  w.qr_off = off;
  off += align_up(w.qr);
  w.vb_off = off;
  off += align_up(w.vb);
  w.dob_off = off;
  off += align_up(w.dob);
  w.delta_off = off;
  off += align_up(w.delta);
  w.sched_off = off;
  off += align_up(w.sched);
  w.total = off;
  return w;
}

mf_status check_attn_common(int32_t dtype, const int32_t* cu_seqlens, int32_t n_segments, int32_t max_seqlen,
                            const int32_t* pos, int nax, double theta, int32_t max_pos, int32_t n_tokens,
                            int32_t n_heads, int32_t head_dim, float softmax_scale) {
  if (dtype != MF_BF16 && dtype != MF_F32) return MF_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return MF_ERR_UNSUPPORTED;
  if (cu_seqlens == nullptr) return MF_ERR_INVALID_ARG;
  if (n_segments < 0 || n_segments > 65535 || max_seqlen < 0 || n_tokens < 0 || n_heads < 1 ||
      n_heads > 65535)
    return MF_ERR_INVALID_ARG;
  if (!(softmax_scale >= 0.0f) || isinf(softmax_scale)) return MF_ERR_INVALID_ARG;
  if (pos != nullptr) {
    if (max_pos < 1 || !(theta > 0.0) || isinf(theta)) return MF_ERR_INVALID_ARG;
    const uintptr_t align = nax == 3 ? 3u : 7u;  // [n][3] int32 or [n][2] int32 (read as int2)
    if ((reinterpret_cast<uintptr_t>(pos) & align) != 0) return MF_ERR_INVALID_ARG;
  }
  return MF_OK;
}

}  // namespace

extern "C" {

const char* mf_status_string(mf_status status) {
  switch (status) {
    case MF_OK:
      return "ok";
    case MF_ERR_INVALID_ARG:
      return "invalid argument (null pointer, bad size or misaligned pointer)";
    case MF_ERR_UNSUPPORTED:
      return "unsupported configuration (head_dim must be 64 or 128; dtype MF_BF16 or MF_F32)";
    case MF_ERR_WORKSPACE:
      return "workspace too small";
    case MF_ERR_HIP:
      return "HIP runtime error at launch";
    case MF_ERR_SCRATCH:
      return "sizes exceed the fixed scratch of the no-allocation call (max_pos or n_segments too large)";
    default:
      return "unknown status";
  }
}

int32_t mf_abi_version(void) { return MF_ABI_VERSION; }

}  // extern "C"

namespace {

mf_status pack_impl(int frames, const mf_sample* samples, int32_t n_samples, int32_t token_budget,
                    int32_t* cu_seqlens, int32_t* cu_pieces, int32_t* pos, int32_t* counts,
                    const void* const* text_rows, const void* const* image_rows, const void* const* target_rows,
                    int64_t row_bytes, void* packed, void* stream, mf_trace* trace) {
  if (n_samples < 0 || token_budget < 0) return MF_ERR_INVALID_ARG;
  if (n_samples > (0x7fffffff - 1) / (frames + 1)) return MF_ERR_INVALID_ARG;
  if (cu_seqlens == nullptr || counts == nullptr) return MF_ERR_INVALID_ARG;
  if (n_samples > 0 && samples == nullptr) return MF_ERR_INVALID_ARG;
  if (token_budget > 0 && pos == nullptr) return MF_ERR_INVALID_ARG;
  const uintptr_t pos_align = frames == 2 ? 3u : 7u;
  if (pos != nullptr && (reinterpret_cast<uintptr_t>(pos) & pos_align) != 0) return MF_ERR_INVALID_ARG;
  if (packed != nullptr) {
    if (row_bytes <= 0 || text_rows == nullptr || image_rows == nullptr) return MF_ERR_INVALID_ARG;
    if (frames == 2 && target_rows == nullptr) return MF_ERR_INVALID_ARG;
  } else if (text_rows != nullptr || image_rows != nullptr || target_rows != nullptr) {
    return MF_ERR_INVALID_ARG;
  }
  if (!trace_ok(trace)) return MF_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Tracer tr(trace, s);
  hipError_t e = tr.run("pack_scan", [&] {
    return mf::launch_pack_scan(samples, n_samples, token_budget, frames, cu_seqlens, cu_pieces, counts, s);
  });
  if (e != hipSuccess) return MF_ERR_HIP;
  if (token_budget == 0 || n_samples == 0) return MF_OK;
  e = tr.run("pack_fill", [&] {
    return mf::launch_pack_fill(samples, token_budget, frames, cu_seqlens, counts, pos, text_rows, image_rows,
                                target_rows, packed ? row_bytes : 0, packed, s);
  });
  return from_hip(e);
}

}  // namespace

extern "C" {

mf_status mf_pack(const mf_sample* samples, int32_t n_samples, int32_t token_budget, int32_t* cu_seqlens,
                  int32_t* cu_pieces, int32_t* pos, int32_t* counts, const void* const* text_rows,
                  const void* const* image_rows, int64_t row_bytes, void* packed, void* stream, mf_trace* trace) {
  return pack_impl(1, samples, n_samples, token_budget, cu_seqlens, cu_pieces, pos, counts, text_rows, image_rows,
                   nullptr, row_bytes, packed, stream, trace);
}

mf_status mf_pack_edit(const mf_sample* samples, int32_t n_samples, int32_t token_budget, int32_t* cu_seqlens,
                       int32_t* cu_pieces, int32_t* pos, int32_t* counts, const void* const* text_rows,
                       const void* const* source_rows, const void* const* target_rows, int64_t row_bytes,
                       void* packed, void* stream, mf_trace* trace) {
  return pack_impl(2, samples, n_samples, token_budget, cu_seqlens, cu_pieces, pos, counts, text_rows, source_rows,
                   target_rows, row_bytes, packed, stream, trace);
}

size_t mf_rope2d_workspace_size(int32_t head_dim, int32_t max_pos) {
  if (head_dim <= 0 || max_pos <= 0) return 0;
  return align_up(static_cast<size_t>(max_pos) * mf::rope_table_width(head_dim, 2) * sizeof(float2));
}

size_t mf_rope3d_workspace_size(int32_t head_dim, int32_t max_pos) {
  if (head_dim <= 0 || max_pos <= 0) return 0;
  return align_up(static_cast<size_t>(max_pos) * mf::rope_table_width(head_dim, 3) * sizeof(float2));
}

}  // extern "C"

namespace {

mf_status rope_impl(int nax, void* x, int32_t dtype, const int32_t* pos, int32_t n_tokens, int32_t n_heads,
                    int32_t head_dim, double theta, int32_t max_pos, int32_t inverse, void* workspace,
                    size_t workspace_bytes, void* stream, mf_trace* trace) {
  if (dtype != MF_BF16 && dtype != MF_F32) return MF_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return MF_ERR_UNSUPPORTED;
  if (n_tokens < 0 || n_heads < 1 || max_pos < 1 || !(theta > 0.0) || isinf(theta)) return MF_ERR_INVALID_ARG;
  if (!trace_ok(trace)) return MF_ERR_INVALID_ARG;
  if (n_tokens == 0) return MF_OK;
  if (x == nullptr || pos == nullptr || workspace == nullptr) return MF_ERR_INVALID_ARG;
  const uintptr_t pos_align = nax == 3 ? 3u : 7u;
  if (!aligned16(x) || (reinterpret_cast<uintptr_t>(pos) & pos_align) != 0 || !aligned16(workspace))
    return MF_ERR_INVALID_ARG;
  const size_t need = nax == 3 ? mf_rope3d_workspace_size(head_dim, max_pos)
                               : mf_rope2d_workspace_size(head_dim, max_pos);
  if (workspace_bytes < need) return MF_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Tracer tr(trace, s);
  float2* tab = static_cast<float2*>(workspace);
  hipError_t e =
      tr.run("rope_table", [&] { return mf::launch_rope_table(tab, max_pos, head_dim, nax, theta, s); });
  if (e != hipSuccess) return MF_ERR_HIP;
  e = tr.run("rope_apply", [&] {
    return mf::launch_rope_apply(x, dtype, x, dtype, pos, nax, tab, max_pos, n_tokens, n_heads, head_dim, true,
                                 inverse != 0, s);
  });
  return from_hip(e);
}

}  // namespace

extern "C" {

mf_status mf_rope2d_apply(void* x, int32_t dtype, const int32_t* pos, int32_t n_tokens, int32_t n_heads,
                          int32_t head_dim, double theta, int32_t max_pos, int32_t inverse, void* workspace,
                          size_t workspace_bytes, void* stream, mf_trace* trace) {
  return rope_impl(2, x, dtype, pos, n_tokens, n_heads, head_dim, theta, max_pos, inverse, workspace,
                   workspace_bytes, stream, trace);
}

mf_status mf_rope3d_apply(void* x, int32_t dtype, const int32_t* pos, int32_t n_tokens, int32_t n_heads,
                          int32_t head_dim, double theta, int32_t max_pos, int32_t inverse, void* workspace,
                          size_t workspace_bytes, void* stream, mf_trace* trace) {
  return rope_impl(3, x, dtype, pos, n_tokens, n_heads, head_dim, theta, max_pos, inverse, workspace,
                   workspace_bytes, stream, trace);
}

size_t mf_varlen_attn_workspace_size(int32_t n_tokens, int32_t n_heads, int32_t head_dim, int32_t n_segments,
                                     int32_t max_pos, int32_t dtype, int32_t flags) {
  if (n_tokens < 0 || n_heads < 1 || (head_dim != 64 && head_dim != 128)) return 0;
  if (n_segments < 0) return 0;
  if ((flags & ~(MF_WS_BACKWARD | MF_WS_ROTATED)) != 0) return 0;
  return attn_workspace(n_tokens, n_heads, head_dim, n_segments, max_pos, dtype, (flags & MF_WS_BACKWARD) != 0,
                        (flags & MF_WS_ROTATED) != 0)
      .total;
}

}  // extern "C"

namespace {

// The forward's launches, on scratch the caller has carved: tab (the rotary
// table, when pos is non-null), sched (the schedule, 2 n_segments + 1 ints,
// then the virtual-segment offsets, 2 (n_segments + 1) ints), kr_ws (a bf16 tensor for the
// rotated K, used only when the call rotates or converts and `rotated` is
// null) and vb_ws (a bf16 copy of v, float32 input only).
mf_status attn_fwd_run(int nax, const void* q, const void* k, const void* v, void* o, float* lse, int32_t dtype,
                       const int32_t* cu_seqlens, int32_t n_segments, int32_t max_pos, const int32_t* pos,
                       double theta, int32_t n_tokens, int32_t n_heads, int32_t head_dim, float softmax_scale,
                       int32_t max_seqlen, void* rotated, float2* tab, int* sched, void* kr_ws, void* vb_ws,
                       void* stream, mf_trace* trace) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  Tracer tr(trace, s);
  const void* kr = k;
  const void* vb = v;
  hipError_t e = hipSuccess;
  if (pos != nullptr) {
    e = tr.run("rope_table", [&] { return mf::launch_rope_table(tab, max_pos, head_dim, nax, theta, s); });
    if (e != hipSuccess) return MF_ERR_HIP;
  }
  // K rotated once into bf16 (also converts float32 input); Q is rotated
  // inside the attention kernel when it is loaded.  With `rotated`, K goes
  // to its second half and the kernel stores the rotated Q in its first.
  const bool rot_pass = pos != nullptr || dtype == MF_F32;
  uint16_t* keep = rot_pass ? static_cast<uint16_t*>(rotated) : nullptr;
  if (rot_pass) {
    void* kdst = keep != nullptr ? static_cast<void*>(keep + rotated_half(n_tokens, n_heads, head_dim)) : kr_ws;
    kr = kdst;
    e = tr.run("rope_k", [&] {
      return mf::launch_rope_apply(k, dtype, kdst, MF_BF16, pos, nax, tab, max_pos, n_tokens, n_heads, head_dim,
                                   pos != nullptr, false, s);
    });
    if (e != hipSuccess) return MF_ERR_HIP;
  }
  if (dtype == MF_F32) {
    vb = vb_ws;
    e = tr.run("convert_v", [&] {
      return mf::launch_rope_apply(v, dtype, vb_ws, MF_BF16, nullptr, 2, nullptr, 0, n_tokens, n_heads, head_dim,
                                   false, false, s);
    });
    if (e != hipSuccess) return MF_ERR_HIP;
  }
  mf::AttnArgs a = {};
  a.cu_seqlens = cu_seqlens;
  a.n_segments = n_segments;
  a.max_seqlen = max_seqlen;
  a.n_tokens = n_tokens;
  a.n_heads = n_heads;
  a.head_dim = head_dim;
  a.dtype = dtype;
  a.pos = pos;
  a.nax = nax;
  a.tab = tab;
  a.max_pos = max_pos;
  a.scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(head_dim));
  a.order = sched;
  a.pt = a.order + n_segments;
  // Multi-segment tiles for runs of tiny segments, when they can hold half of
  // the tokens at all (that needs a mean segment length of at most 256).
  const bool merge = static_cast<long long>(n_tokens) <= 2LL * mf::kTinySegment * n_segments;
  int* vcu = const_cast<int*>(a.pt) + n_segments + 1;
  int* vfirst = vcu + n_segments + 1;
  if (merge) {
    a.cu_seqlens = vcu;
    a.rcu = cu_seqlens;
    a.vfirst = vfirst;
  }
  a.qr_out = keep;
  e = tr.run("attn_sched", [&] {
    if (merge) {
      hipError_t r = mf::launch_merge_tiny(cu_seqlens, n_segments, n_tokens, vcu, vfirst, s);
      if (r != hipSuccess) return r;
    }
    return mf::launch_sched(a.cu_seqlens, n_segments, n_tokens, mf::fwd_tile(max_seqlen, n_tokens, n_segments),
                            const_cast<int*>(a.order), const_cast<int*>(a.pt), s);
  });
  if (e != hipSuccess) return MF_ERR_HIP;
  e = tr.run("attn_fwd", [&] { return mf::launch_attn_fwd(a, q, kr, vb, o, lse, s); });
  return from_hip(e);
}

mf_status attn_fwd_impl(int nax, const void* q, const void* k, const void* v, void* o, float* lse, int32_t dtype,
                        const int32_t* cu_seqlens, int32_t n_segments, int32_t max_seqlen, const int32_t* pos,
                        double theta, int32_t max_pos, int32_t n_tokens, int32_t n_heads, int32_t head_dim,
                        float softmax_scale, void* rotated, void* workspace, size_t workspace_bytes, void* stream,
                        mf_trace* trace) {
  mf_status st = check_attn_common(dtype, cu_seqlens, n_segments, max_seqlen, pos, nax, theta, max_pos, n_tokens,
                                   n_heads, head_dim, softmax_scale);
  if (st != MF_OK) return st;
  if (!trace_ok(trace)) return MF_ERR_INVALID_ARG;
  if (!aligned16_or_null(rotated)) return MF_ERR_INVALID_ARG;
  if (n_tokens == 0 || n_segments == 0 || max_seqlen == 0) return MF_OK;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return MF_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return MF_ERR_INVALID_ARG;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return MF_ERR_INVALID_ARG;
  const AttnWorkspace w =
      attn_workspace(n_tokens, n_heads, head_dim, n_segments, pos ? max_pos : 0, dtype, false, rotated != nullptr);
  if (workspace_bytes < w.total) return MF_ERR_WORKSPACE;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return MF_ERR_INVALID_ARG;
  char* ws = static_cast<char*>(workspace);
  return attn_fwd_run(nax, q, k, v, o, lse, dtype, cu_seqlens, n_segments, max_pos, pos, theta, n_tokens, n_heads,
                      head_dim, softmax_scale, max_seqlen, rotated, reinterpret_cast<float2*>(ws + w.tab_off),
                      reinterpret_cast<int*>(ws + w.sched_off), ws + w.kr_off, ws + w.vb_off, stream, trace);
}


mf_status attn_bwd_impl(int nax, const void* q, const void* k, const void* v, const void* o, const float* lse,
                        const void* dout, void* dq, void* dk, void* dv, int32_t dtype, const int32_t* cu_seqlens,
                        int32_t n_segments, int32_t max_seqlen, const int32_t* pos, double theta,
                        int32_t max_pos, int32_t n_tokens, int32_t n_heads, int32_t head_dim,
                        float softmax_scale, const void* rotated, void* workspace, size_t workspace_bytes,
                        void* stream, mf_trace* trace) {
  mf_status st = check_attn_common(dtype, cu_seqlens, n_segments, max_seqlen, pos, nax, theta, max_pos, n_tokens,
                                   n_heads, head_dim, softmax_scale);
  if (st != MF_OK) return st;
  if (!trace_ok(trace)) return MF_ERR_INVALID_ARG;
  if (!aligned16_or_null(rotated)) return MF_ERR_INVALID_ARG;
  if (n_tokens == 0 || n_segments == 0 || max_seqlen == 0) return MF_OK;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr || dout == nullptr ||
      dq == nullptr || dk == nullptr || dv == nullptr)
    return MF_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return MF_ERR_INVALID_ARG;
  const AttnWorkspace w =
      attn_workspace(n_tokens, n_heads, head_dim, n_segments, pos ? max_pos : 0, dtype, true, rotated != nullptr);
  if (workspace_bytes < w.total) return MF_ERR_WORKSPACE;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return MF_ERR_INVALID_ARG;

  hipStream_t s = static_cast<hipStream_t>(stream);
  Tracer tr(trace, s);
  char* ws = static_cast<char*>(workspace);
  float2* tab = reinterpret_cast<float2*>(ws + w.tab_off);
  const void* kr = k;
  const void* qr = q;
  float* delta = reinterpret_cast<float*>(ws + w.delta_off);
  float* lse2 = delta + static_cast<size_t>(n_tokens) * n_heads;
  const void* vb = v;
  const void* dob = dout;
  hipError_t e = hipSuccess;
  if (pos != nullptr) {
    e = tr.run("rope_table", [&] { return mf::launch_rope_table(tab, max_pos, head_dim, nax, theta, s); });
    if (e != hipSuccess) return MF_ERR_HIP;
  }
  if ((pos != nullptr || dtype == MF_F32) && rotated != nullptr) {
    // the forward's rotated bf16 Q and K
    qr = rotated;
    kr = static_cast<const uint16_t*>(rotated) + rotated_half(n_tokens, n_heads, head_dim);
  } else if (pos != nullptr || dtype == MF_F32) {
    qr = ws + w.qr_off;
    kr = ws + w.kr_off;
    e = tr.run("rope_q", [&] {
      return mf::launch_rope_apply(q, dtype, ws + w.qr_off, MF_BF16, pos, nax, tab, max_pos, n_tokens, n_heads,
                                   head_dim, pos != nullptr, false, s);
    });
    if (e != hipSuccess) return MF_ERR_HIP;
    e = tr.run("rope_k", [&] {
      return mf::launch_rope_apply(k, dtype, ws + w.kr_off, MF_BF16, pos, nax, tab, max_pos, n_tokens, n_heads,
                                   head_dim, pos != nullptr, false, s);
    });
    if (e != hipSuccess) return MF_ERR_HIP;
  }
  if (dtype == MF_F32) {
    vb = ws + w.vb_off;
    dob = ws + w.dob_off;
    e = tr.run("convert_v", [&] {
      return mf::launch_rope_apply(v, dtype, ws + w.vb_off, MF_BF16, nullptr, 2, nullptr, 0, n_tokens, n_heads,
                                   head_dim, false, false, s);
    });
    if (e != hipSuccess) return MF_ERR_HIP;
    e = tr.run("convert_do", [&] {
      return mf::launch_rope_apply(dout, dtype, ws + w.dob_off, MF_BF16, nullptr, 2, nullptr, 0, n_tokens, n_heads,
                                   head_dim, false, false, s);
    });
    if (e != hipSuccess) return MF_ERR_HIP;
  }
  mf::AttnArgs a = {};
  a.cu_seqlens = cu_seqlens;
  a.n_segments = n_segments;
  a.max_seqlen = max_seqlen;
  a.n_tokens = n_tokens;
  a.n_heads = n_heads;
  a.head_dim = head_dim;
  a.dtype = dtype;
  a.pos = pos;
  a.nax = nax;
  a.tab = tab;
  a.max_pos = max_pos;
  a.scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(head_dim));
  a.order = reinterpret_cast<int*>(ws + w.sched_off);
  a.pt = a.order + n_segments;
  // dkdv walks key tiles of kDkdvTile, dq query tiles of kDqTile (kDqTileMerged
  // when tiny segments are merged): one schedule each.
  mf::AttnArgs aq = a;
  aq.order = a.pt + n_segments + 1;
  aq.pt = aq.order + n_segments;
  // dq takes multi-segment tiles like the forward; dkdv keeps one tile per
  // segment (its 128-key x 32-query steps already fit tiny segments: a shared
  // tile measured slower).
  const bool merge = static_cast<long long>(n_tokens) <= 2LL * mf::kTinySegment * n_segments;
  int* vcu = const_cast<int*>(aq.pt) + n_segments + 1;
  int* vfirst = vcu + n_segments + 1;
  if (merge) {
    aq.cu_seqlens = vcu;
    aq.rcu = cu_seqlens;
    aq.vfirst = vfirst;
  }
  e = tr.run("attn_sched", [&] {
    hipError_t r = hipSuccess;
    if (merge) {
      r = mf::launch_merge_tiny(cu_seqlens, n_segments, n_tokens, vcu, vfirst, s);
      if (r != hipSuccess) return r;
    }
    r = mf::launch_sched(cu_seqlens, n_segments, n_tokens, mf::kDkdvTile, const_cast<int*>(a.order),
                         const_cast<int*>(a.pt), s);
    if (r != hipSuccess) return r;
    return mf::launch_sched(aq.cu_seqlens, n_segments, n_tokens, merge ? mf::kDqTileMerged : mf::kDqTile,
                            const_cast<int*>(aq.order), const_cast<int*>(aq.pt), s);
  });
  if (e != hipSuccess) return MF_ERR_HIP;
  // dq first: it also writes Delta and the log2-scaled LSE that dkdv reads.
  e = tr.run("attn_bwd_dq", [&] {
    return mf::launch_attn_bwd_dq(aq, qr, kr, vb, dob, o, dout, lse, lse2, delta, dq, s);
  });
  if (e != hipSuccess) return MF_ERR_HIP;
  e = tr.run("attn_bwd_dkdv",
             [&] { return mf::launch_attn_bwd_dkdv(a, qr, kr, vb, dob, lse2, delta, dk, dv, s); });
  return from_hip(e);
}

}  // namespace

extern "C" {

mf_status mf_varlen_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int32_t dtype,
                             const int32_t* cu_seqlens, int32_t n_segments, int32_t max_seqlen, const int32_t* pos,
                             double theta, int32_t max_pos, int32_t n_tokens, int32_t n_heads, int32_t head_dim,
                             float softmax_scale, void* rotated, void* workspace, size_t workspace_bytes,
                             void* stream, mf_trace* trace) {
  return attn_fwd_impl(2, q, k, v, o, lse, dtype, cu_seqlens, n_segments, max_seqlen, pos, theta, max_pos, n_tokens,
                       n_heads, head_dim, softmax_scale, rotated, workspace, workspace_bytes, stream, trace);
}

mf_status mf_varlen_attn3d_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int32_t dtype,
                               const int32_t* cu_seqlens, int32_t n_segments, int32_t max_seqlen,
                               const int32_t* pos, double theta, int32_t max_pos, int32_t n_tokens, int32_t n_heads,
                               int32_t head_dim, float softmax_scale, void* rotated, void* workspace,
                               size_t workspace_bytes, void* stream, mf_trace* trace) {
  if (pos == nullptr) return MF_ERR_INVALID_ARG;
  return attn_fwd_impl(3, q, k, v, o, lse, dtype, cu_seqlens, n_segments, max_seqlen, pos, theta, max_pos, n_tokens,
                       n_heads, head_dim, softmax_scale, rotated, workspace, workspace_bytes, stream, trace);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Forward without a workspace, for callers that cannot allocate device
// memory.  Its scratch (the rotary table and the schedule) lives in a fixed
// array in this library's device image; each GPU holds its own copy, whose
// address is looked up once per device, with that device current, on the
// first call there.  Every launch writes the scratch it reads before reading
// it, so nothing has to start at zero; the contents left by one call are
// overwritten by the next.  Calls that overlap on one GPU share the array and
// race.

namespace {

constexpr size_t kScratchBytes = size_t(4) << 20;
constexpr int kScratchDevices = 64;

static __device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kScratchDevices];  // device address of `scratch`, per device ordinal

// This device's address of `scratch` (host code may never use the array's
// name as a device address: it names a host-side stand-in).
mf_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return MF_ERR_HIP;
  }
  if (dev < 0 || dev >= kScratchDevices) return MF_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return MF_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MF_OK;
}

}  // namespace

extern "C" {

mf_status mf_varlen_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int32_t dtype,
                                     const int32_t* cu_seqlens, int32_t n_segments, int32_t max_seqlen,
                                     const int32_t* pos, double theta, int32_t max_pos, int32_t n_tokens,
                                     int32_t n_heads, int32_t head_dim, float softmax_scale, void* rotated,
                                     void* stream, mf_trace* trace) {
  mf_status st = check_attn_common(dtype, cu_seqlens, n_segments, max_seqlen, pos, 2, theta, max_pos, n_tokens,
                                   n_heads, head_dim, softmax_scale);
  if (st != MF_OK) return st;
  // float32 input would need bf16 copies of K and V as large as the inputs
  if (dtype != MF_BF16) return MF_ERR_UNSUPPORTED;
  if (!trace_ok(trace)) return MF_ERR_INVALID_ARG;
  if (!aligned16_or_null(rotated)) return MF_ERR_INVALID_ARG;
  // the rotated K goes to the caller's buffer, never to the scratch
  if (pos != nullptr && rotated == nullptr) return MF_ERR_INVALID_ARG;
  if (n_tokens == 0 || n_segments == 0 || max_seqlen == 0) return MF_OK;
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return MF_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return MF_ERR_INVALID_ARG;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return MF_ERR_INVALID_ARG;
  const size_t tab_bytes =
      pos != nullptr ? align_up(static_cast<size_t>(max_pos) * mf::rope_table_width(head_dim, 2) * sizeof(float2))
                     : 0;
  const size_t sched_bytes = (4 * static_cast<size_t>(n_segments) + 3) * sizeof(int32_t);
  if (tab_bytes + sched_bytes > kScratchBytes) return MF_ERR_SCRATCH;
  void* base = nullptr;
  st = scratch_address(&base);
  if (st != MF_OK) return st;
  char* sp = static_cast<char*>(base);
  return attn_fwd_run(2, q, k, v, o, lse, dtype, cu_seqlens, n_segments, max_pos, pos, theta, n_tokens, n_heads,
                      head_dim, softmax_scale, max_seqlen, rotated, reinterpret_cast<float2*>(sp),
                      reinterpret_cast<int*>(sp + tab_bytes), nullptr, nullptr, stream, trace);
}

mf_status mf_varlen_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, int32_t dtype, const int32_t* cu_seqlens,
                             int32_t n_segments, int32_t max_seqlen, const int32_t* pos, double theta,
                             int32_t max_pos, int32_t n_tokens, int32_t n_heads, int32_t head_dim,
                             float softmax_scale, const void* rotated, void* workspace, size_t workspace_bytes,
                             void* stream, mf_trace* trace) {
  return attn_bwd_impl(2, q, k, v, o, lse, dout, dq, dk, dv, dtype, cu_seqlens, n_segments, max_seqlen, pos, theta,
                       max_pos, n_tokens, n_heads, head_dim, softmax_scale, rotated, workspace, workspace_bytes,
                       stream, trace);
}

mf_status mf_varlen_attn3d_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                               const void* dout, void* dq, void* dk, void* dv, int32_t dtype,
                               const int32_t* cu_seqlens, int32_t n_segments, int32_t max_seqlen,
                               const int32_t* pos, double theta, int32_t max_pos, int32_t n_tokens, int32_t n_heads,
                               int32_t head_dim, float softmax_scale, const void* rotated, void* workspace,
                               size_t workspace_bytes, void* stream, mf_trace* trace) {
  if (pos == nullptr) return MF_ERR_INVALID_ARG;
  return attn_bwd_impl(3, q, k, v, o, lse, dout, dq, dk, dv, dtype, cu_seqlens, n_segments, max_seqlen, pos, theta,
                       max_pos, n_tokens, n_heads, head_dim, softmax_scale, rotated, workspace, workspace_bytes,
                       stream, trace);
}

// ---------------------------------------------------------------------------
// Rectified-flow objective and packed CFG combine on [n_tokens][channels] latents.

}  // extern "C"

namespace {

mf_status check_flow_common(int32_t dtype, const int32_t* cu_pieces, int32_t n_samples, int32_t frames,
                            int32_t n_tokens, int32_t channels) {
  if (dtype != MF_BF16 && dtype != MF_F32) return MF_ERR_UNSUPPORTED;
  // a row's channels / 8 vectors must be a power of two within one wave
  if (channels < 8 || channels > 512 || (channels & (channels - 1)) != 0) return MF_ERR_UNSUPPORTED;
  if (cu_pieces == nullptr || n_samples < 0 || n_tokens < 0 || (frames != 1 && frames != 2)) return MF_ERR_INVALID_ARG;
  if (static_cast<long long>(n_samples) * (frames + 1) >= 0x7fffffffLL) return MF_ERR_INVALID_ARG;
  return MF_OK;
}

bool aligned_for(const void* p, int32_t /*dtype*/) { return p != nullptr && aligned16(p); }

}  // namespace

extern "C" {

mf_status mf_rf_noise(const void* z, const void* eps, const float* t, void* zt, int32_t dtype,
                      const int32_t* cu_pieces, int32_t n_samples, int32_t frames, int32_t n_tokens,
                      int32_t channels, void* stream, mf_trace* trace) {
  mf_status st = check_flow_common(dtype, cu_pieces, n_samples, frames, n_tokens, channels);
  if (st != MF_OK) return st;
  if (!trace_ok(trace)) return MF_ERR_INVALID_ARG;
  if (n_tokens == 0) return MF_OK;
  if (!aligned_for(z, dtype) || !aligned_for(eps, dtype) || !aligned_for(zt, dtype)) return MF_ERR_INVALID_ARG;
  if (n_samples > 0 && (t == nullptr || (reinterpret_cast<uintptr_t>(t) & 3u) != 0)) return MF_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Tracer tr(trace, s);
  return from_hip(tr.run("rf_noise", [&] {
    return mf::launch_rf_noise(z, eps, t, zt, dtype, cu_pieces, n_samples, frames, n_tokens, channels, s);
  }));
}

size_t mf_rf_loss_workspace_size(int32_t n_tokens) {
  if (n_tokens <= 0) return 0;
  return align_up(static_cast<size_t>(n_tokens) * sizeof(float));
}

mf_status mf_rf_loss(const void* v, const void* z, const void* eps, void* grad, float* loss_sum, int32_t dtype,
                     const int32_t* cu_pieces, int32_t n_samples, int32_t frames, int32_t n_tokens, int32_t channels,
                     float grad_scale, void* workspace, size_t workspace_bytes, void* stream, mf_trace* trace) {
  mf_status st = check_flow_common(dtype, cu_pieces, n_samples, frames, n_tokens, channels);
  if (st != MF_OK) return st;
  if (!trace_ok(trace)) return MF_ERR_INVALID_ARG;
  if (isnan(grad_scale) || isinf(grad_scale)) return MF_ERR_INVALID_ARG;
  if (n_samples > 0 && (loss_sum == nullptr || (reinterpret_cast<uintptr_t>(loss_sum) & 3u) != 0))
    return MF_ERR_INVALID_ARG;
  if (n_tokens > 0) {
    if (!aligned_for(v, dtype) || !aligned_for(z, dtype) || !aligned_for(eps, dtype)) return MF_ERR_INVALID_ARG;
    if (grad != nullptr && !aligned_for(grad, dtype)) return MF_ERR_INVALID_ARG;
    if (workspace_bytes < mf_rf_loss_workspace_size(n_tokens)) return MF_ERR_WORKSPACE;
    if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 3u) != 0) return MF_ERR_INVALID_ARG;
  }
  if (n_samples == 0 && n_tokens == 0) return MF_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Tracer tr(trace, s);
  return from_hip(tr.run("rf_loss", [&] {
    return mf::launch_rf_loss(v, z, eps, grad, static_cast<float*>(workspace), loss_sum, dtype, cu_pieces, n_samples,
                              frames, n_tokens, channels, grad_scale, s);
  }));
}

mf_status mf_cfg_combine(const void* v, void* out, int32_t* mismatched, int32_t dtype, const int32_t* cu_pieces,
                         int32_t n_samples, int32_t n_pairs, int32_t n_tokens, int32_t channels, float scale,
                         void* stream, mf_trace* trace) {
  mf_status st = check_flow_common(dtype, cu_pieces, n_samples, 1, n_tokens, channels);
  if (st != MF_OK) return st;
  if (!trace_ok(trace)) return MF_ERR_INVALID_ARG;
  if (n_pairs < 0 || 2LL * n_pairs > n_samples || isnan(scale) || isinf(scale)) return MF_ERR_INVALID_ARG;
  if (mismatched != nullptr && (reinterpret_cast<uintptr_t>(mismatched) & 3u) != 0) return MF_ERR_INVALID_ARG;
  if (n_tokens > 0 && (!aligned_for(v, dtype) || !aligned_for(out, dtype))) return MF_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Tracer tr(trace, s);
  return from_hip(tr.run("cfg_combine", [&] {
    return mf::launch_cfg_combine(v, out, mismatched, dtype, cu_pieces, n_pairs, n_tokens, channels, scale, s);
  }));
}

}  // extern "C"

// The attention sub-block's fused chains (adaptive norm, QKV projection with
// the rotary embedding, output projection with the gated residual).

namespace {

size_t block_tiles_bytes(int32_t n_samples, int32_t frames) {
  return align_up((static_cast<size_t>(n_samples) * (frames + 1) + 1) * sizeof(int32_t));
}

mf_status check_block_sizes(int32_t n_samples, int32_t frames, int32_t n_tokens, int32_t channels) {
  if (n_samples < 0 || n_tokens < 0 || (frames != 1 && frames != 2)) return MF_ERR_INVALID_ARG;
  if (static_cast<long long>(n_samples) * (frames + 1) >= 0x7fffffffLL) return MF_ERR_INVALID_ARG;
  if (channels < 256 || channels % 256 != 0 || channels > 65535 * 128) return MF_ERR_UNSUPPORTED;
  return MF_OK;
}

mf_status check_block_common(const int32_t* cu_pieces, int32_t n_samples, int32_t frames, int32_t n_tokens,
                             int32_t channels) {
  if (cu_pieces == nullptr) return MF_ERR_INVALID_ARG;
  return check_block_sizes(n_samples, frames, n_tokens, channels);
}

}  // namespace

extern "C" {

size_t mf_block_workspace_size(int32_t n_samples, int32_t frames, int32_t head_dim, int32_t max_pos) {
  if (n_samples < 0 || (frames != 1 && frames != 2)) return 0;
  if (static_cast<long long>(n_samples) * (frames + 1) >= 0x7fffffffLL) return 0;
  size_t total = block_tiles_bytes(n_samples, frames);
  if (max_pos > 0 && (head_dim == 64 || head_dim == 128))
    total += align_up(static_cast<size_t>(max_pos) * mf::rope_table_width(head_dim, 3) * sizeof(float2));
  return total;
}

mf_status mf_adaln_modulate(const void* x, const float* shift, const float* scale, void* h,
                            const int32_t* cu_pieces, int32_t n_samples, int32_t frames, int32_t n_tokens,
                            int32_t channels, float eps, void* stream, mf_trace* trace) {
  mf_status st = check_block_common(cu_pieces, n_samples, frames, n_tokens, channels);
  if (st != MF_OK) return st;
  if (channels % 512 != 0 || channels > 8192) return MF_ERR_UNSUPPORTED;
  if (!trace_ok(trace)) return MF_ERR_INVALID_ARG;
  if (!(eps > 0.0f) || isinf(eps)) return MF_ERR_INVALID_ARG;
  if (n_tokens == 0) return MF_OK;
  if (x == nullptr || h == nullptr || !aligned16(x) || !aligned16(h)) return MF_ERR_INVALID_ARG;
  if (n_samples > 0 && (shift == nullptr || scale == nullptr || !aligned16(shift) || !aligned16(scale)))
    return MF_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Tracer tr(trace, s);
  return from_hip(tr.run("adaln", [&] {
    return mf::launch_adaln(x, shift, scale, cu_pieces, n_samples, frames, n_tokens, channels, eps, h, s);
  }));
}

mf_status mf_qkv_rope(const void* h, const void* w_text, const void* w_image, const float* b_text,
                      const float* b_image, void* q, void* k, void* v, const int32_t* cu_pieces, int32_t n_samples,
                      int32_t frames, const int32_t* pos, int32_t nax, double theta, int32_t max_pos,
                      int32_t n_tokens, int32_t n_heads, int32_t head_dim, void* workspace, size_t workspace_bytes,
                      void* stream, mf_trace* trace) {
  if (head_dim != 64 && head_dim != 128) return MF_ERR_UNSUPPORTED;
  if (n_heads < 1 || n_heads > 65535) return MF_ERR_INVALID_ARG;
  const int32_t channels = n_heads * head_dim;
  mf_status st = check_block_common(cu_pieces, n_samples, frames, n_tokens, channels);
  if (st != MF_OK) return st;
  if (!trace_ok(trace)) return MF_ERR_INVALID_ARG;
  if (pos != nullptr) {
    if (nax != 2 && nax != 3) return MF_ERR_INVALID_ARG;
    if (max_pos < 1 || !(theta > 0.0) || isinf(theta)) return MF_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(pos) & (nax == 2 ? 7u : 3u)) != 0) return MF_ERR_INVALID_ARG;
  }
  if (n_tokens == 0) return MF_OK;
  if (h == nullptr || q == nullptr || k == nullptr || v == nullptr || w_text == nullptr || w_image == nullptr)
    return MF_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(w_text) ||
      !aligned16(w_image) || !aligned16_or_null(b_text) || !aligned16_or_null(b_image))
    return MF_ERR_INVALID_ARG;
  const size_t need = mf_block_workspace_size(n_samples, frames, head_dim, pos != nullptr ? max_pos : 0);
  if (workspace_bytes < need) return MF_ERR_WORKSPACE;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return MF_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int* tstart = reinterpret_cast<int*>(ws);
  float2* tab = reinterpret_cast<float2*>(ws + block_tiles_bytes(n_samples, frames));
  const int n_pieces = (frames + 1) * n_samples;
  Tracer tr(trace, s);
  hipError_t e = tr.run("piece_tiles", [&] { return mf::launch_piece_tiles(cu_pieces, n_pieces, n_tokens, tstart, s); });
  if (e != hipSuccess) return MF_ERR_HIP;
  if (pos != nullptr) {
    e = tr.run("rope_table", [&] { return mf::launch_rope_table(tab, max_pos, head_dim, nax, theta, s); });
    if (e != hipSuccess) return MF_ERR_HIP;
  }
  return from_hip(tr.run("qkv_rope", [&] {
    return mf::launch_qkv_rope(h, w_text, w_image, b_text, b_image, cu_pieces, tstart, n_samples, frames, n_tokens,
                               n_heads, head_dim, pos, nax, tab, max_pos, q, k, v, s);
  }));
}

mf_status mf_out_gated_residual(const void* o, const void* x, const void* w_text, const void* w_image,
                                const float* b_text, const float* b_image, const float* gate, void* y, void* proj,
                                const int32_t* cu_pieces, int32_t n_samples, int32_t frames, int32_t n_tokens,
                                int32_t channels, void* workspace, size_t workspace_bytes, void* stream,
                                mf_trace* trace) {
  mf_status st = check_block_common(cu_pieces, n_samples, frames, n_tokens, channels);
  if (st != MF_OK) return st;
  if (!trace_ok(trace)) return MF_ERR_INVALID_ARG;
  if (n_tokens == 0) return MF_OK;
  if (o == nullptr || x == nullptr || y == nullptr || w_text == nullptr || w_image == nullptr)
    return MF_ERR_INVALID_ARG;
  if (!aligned16(o) || !aligned16(x) || !aligned16(y) || !aligned16(w_text) || !aligned16(w_image) ||
      !aligned16_or_null(b_text) || !aligned16_or_null(b_image) || !aligned16_or_null(proj))
    return MF_ERR_INVALID_ARG;
  if (n_samples > 0 && (gate == nullptr || !aligned16(gate))) return MF_ERR_INVALID_ARG;
  const size_t need = mf_block_workspace_size(n_samples, frames, 64, 0);
  if (workspace_bytes < need) return MF_ERR_WORKSPACE;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return MF_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int* tstart = static_cast<int*>(workspace);
  const int n_pieces = (frames + 1) * n_samples;
  Tracer tr(trace, s);
  hipError_t e = tr.run("piece_tiles", [&] { return mf::launch_piece_tiles(cu_pieces, n_pieces, n_tokens, tstart, s); });
  if (e != hipSuccess) return MF_ERR_HIP;
  return from_hip(tr.run("out_gated", [&] {
    return mf::launch_out_gated(o, x, w_text, w_image, b_text, b_image, gate, cu_pieces, tstart, n_samples, frames,
                                n_tokens, channels, y, proj, s);
  }));
}

}  // extern "C"

// Backward of the chains.  Workspace parts in order, each 256-byte aligned.

namespace {

struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  }
};

// Largest token count whose gathered operands keep a row pitch below 2^24 bytes.
constexpr int32_t kBwdMaxTokens = (1 << 23) - 512;
// Largest channel count of the projections' backward (transpose grids).
constexpr int32_t kBwdMaxChannels = 16384;

struct BlockBwdWorkspace {
  size_t tstart = 0, col0 = 0, kr = 0, stats = 0, part = 0;  // common
  size_t tab = 0, dqk = 0, u = 0, wt = 0, at = 0, bt = 0, bpart = 0, split = 0;
  long long pitch = 0;
  int splits = 2;
  size_t total = 0;
};

// kind 0: adaln; 1: qkv projection (rotation when max_pos > 0); 2: output projection.
BlockBwdWorkspace block_bwd_layout(int kind, int32_t n_samples, int32_t frames, int32_t n_tokens, int32_t channels,
                                   int32_t head_dim, int32_t max_pos) {
  BlockBwdWorkspace w;
  Carve c;
  const size_t n_pieces = static_cast<size_t>(n_samples) * (frames + 1);
  const size_t n = static_cast<size_t>(n_tokens), ch = static_cast<size_t>(channels);
  const size_t sub_rows = 4 * static_cast<size_t>(mf::block_mtiles_bound(n_tokens, static_cast<int>(n_pieces)));
  w.tstart = c.take((n_pieces + 1) * sizeof(int32_t));
  if (kind == 0) {
    w.stats = c.take(n * 2 * sizeof(float));
    w.part = c.take(sub_rows * 2 * ch * sizeof(float));
    w.total = c.off;
    return w;
  }
  const size_t out_rows = kind == 1 ? 3 * ch : ch;  // gradient features of the projection's output
  w.pitch = mf::block_bwd_cols(n_tokens);
  w.splits = mf::block_bwd_splits(n_tokens, static_cast<int>(out_rows), channels);
  w.col0 = c.take((n_pieces + 2) * sizeof(int32_t));
  w.kr = c.take(2 * sizeof(int32_t));
  if (kind == 1 && max_pos > 0) {
    w.tab = c.take(static_cast<size_t>(max_pos) * mf::rope_table_width(head_dim, 3) * sizeof(float2));
    w.dqk = c.take(2 * n * ch * 2);
  }
  if (kind == 2) {
    w.u = c.take(n * ch * 2);
    w.part = c.take(sub_rows * ch * sizeof(float));
  }
  w.wt = c.take(2 * out_rows * ch * 2);
  w.at = c.take(out_rows * static_cast<size_t>(w.pitch) * 2);
  w.bt = c.take(ch * static_cast<size_t>(w.pitch) * 2);
  w.bpart = c.take(static_cast<size_t>(w.pitch / 64) * out_rows * sizeof(float));
  if (w.splits > 2) w.split = c.take(static_cast<size_t>(w.splits) * out_rows * ch * sizeof(float));
  w.total = c.off;
  return w;
}

mf_status check_workspace(const void* workspace, size_t workspace_bytes, size_t need) {
  if (workspace_bytes < need) return MF_ERR_WORKSPACE;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0) return MF_ERR_INVALID_ARG;
  return MF_OK;
}

bool aligned4_or_null(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

}  // namespace

extern "C" {

size_t mf_adaln_modulate_bwd_workspace_size(int32_t n_samples, int32_t frames, int32_t n_tokens, int32_t channels) {
  if (check_block_sizes(n_samples, frames, n_tokens, channels) != MF_OK) return 0;
  if (channels % 512 != 0 || channels > mf::kAdaBwdMaxC) return 0;
  return block_bwd_layout(0, n_samples, frames, n_tokens, channels, 64, 0).total;
}

size_t mf_qkv_rope_bwd_workspace_size(int32_t n_samples, int32_t frames, int32_t n_tokens, int32_t n_heads,
                                      int32_t head_dim, int32_t max_pos) {
  if ((head_dim != 64 && head_dim != 128) || n_heads < 1 || n_heads > 65535 || n_tokens > kBwdMaxTokens) return 0;
  if (n_heads * head_dim > kBwdMaxChannels) return 0;
  if (check_block_sizes(n_samples, frames, n_tokens, n_heads * head_dim) != MF_OK) return 0;
  return block_bwd_layout(1, n_samples, frames, n_tokens, n_heads * head_dim, head_dim, max_pos > 0 ? max_pos : 0)
      .total;
}

size_t mf_out_gated_residual_bwd_workspace_size(int32_t n_samples, int32_t frames, int32_t n_tokens,
                                                int32_t channels) {
  if (n_tokens > kBwdMaxTokens || channels > kBwdMaxChannels) return 0;
  if (check_block_sizes(n_samples, frames, n_tokens, channels) != MF_OK) return 0;
  return block_bwd_layout(2, n_samples, frames, n_tokens, channels, 64, 0).total;
}

mf_status mf_adaln_modulate_bwd(const void* dh, const void* x, const float* scale, const void* dres, void* dx,
                                float* dshift, float* dscale, const int32_t* cu_pieces, int32_t n_samples,
                                int32_t frames, int32_t n_tokens, int32_t channels, float eps, void* workspace,
                                size_t workspace_bytes, void* stream, mf_trace* trace) {
  mf_status st = check_block_common(cu_pieces, n_samples, frames, n_tokens, channels);
  if (st != MF_OK) return st;
  if (channels % 512 != 0 || channels > mf::kAdaBwdMaxC) return MF_ERR_UNSUPPORTED;
  if (!trace_ok(trace)) return MF_ERR_INVALID_ARG;
  if (!(eps > 0.0f) || isinf(eps)) return MF_ERR_INVALID_ARG;
  if (n_samples > 0 && (scale == nullptr || dshift == nullptr || dscale == nullptr || !aligned16(scale) ||
                        !aligned16(dshift) || !aligned16(dscale)))
    return MF_ERR_INVALID_ARG;
  if (n_tokens > 0 && (dh == nullptr || x == nullptr || dx == nullptr || !aligned16(dh) || !aligned16(x) ||
                       !aligned16(dx) || !aligned16_or_null(dres)))
    return MF_ERR_INVALID_ARG;
  const BlockBwdWorkspace w = block_bwd_layout(0, n_samples, frames, n_tokens, channels, 64, 0);
  if ((st = check_workspace(workspace, workspace_bytes, w.total)) != MF_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int* tstart = reinterpret_cast<int*>(ws + w.tstart);
  float* part = reinterpret_cast<float*>(ws + w.part);
  const int n_pieces = (frames + 1) * n_samples;
  Tracer tr(trace, s);
  hipError_t e = tr.run("piece_tiles", [&] { return mf::launch_piece_tiles(cu_pieces, n_pieces, n_tokens, tstart, s); });
  if (e != hipSuccess) return MF_ERR_HIP;
  e = tr.run("adaln_bwd", [&] {
    return mf::launch_adaln_bwd(dh, x, scale, dres, cu_pieces, tstart, n_samples, frames, n_tokens, channels, eps, dx,
                                reinterpret_cast<float2*>(ws + w.stats), part, s);
  });
  if (e != hipSuccess) return MF_ERR_HIP;
  const long long stride = 2LL * channels;
  e = tr.run("group_sum", [&] {
    hipError_t r = mf::launch_group_sum(part, stride, 0, channels, tstart, n_samples, frames, n_tokens, dshift, s);
    if (r != hipSuccess) return r;
    return mf::launch_group_sum(part, stride, channels, channels, tstart, n_samples, frames, n_tokens, dscale, s);
  });
  return from_hip(e);
}

mf_status mf_qkv_rope_bwd(const void* dq, const void* dk, const void* dv, const void* h, const void* w_text,
                          const void* w_image, void* dh, float* dw_text, float* dw_image, float* db_text,
                          float* db_image, const int32_t* cu_pieces, int32_t n_samples, int32_t frames,
                          const int32_t* pos, int32_t nax, double theta, int32_t max_pos, int32_t n_tokens,
                          int32_t n_heads, int32_t head_dim, void* workspace, size_t workspace_bytes, void* stream,
                          mf_trace* trace) {
  if (head_dim != 64 && head_dim != 128) return MF_ERR_UNSUPPORTED;
  if (n_heads < 1 || n_heads > 65535) return MF_ERR_INVALID_ARG;
  const int32_t channels = n_heads * head_dim;
  mf_status st = check_block_common(cu_pieces, n_samples, frames, n_tokens, channels);
  if (st != MF_OK) return st;
  if (n_tokens > kBwdMaxTokens || channels > kBwdMaxChannels) return MF_ERR_UNSUPPORTED;
  if (!trace_ok(trace)) return MF_ERR_INVALID_ARG;
  if (pos != nullptr) {
    if (nax != 2 && nax != 3) return MF_ERR_INVALID_ARG;
    if (max_pos < 1 || !(theta > 0.0) || isinf(theta)) return MF_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(pos) & (nax == 2 ? 7u : 3u)) != 0) return MF_ERR_INVALID_ARG;
  }
  if (w_text == nullptr || w_image == nullptr || dw_text == nullptr || dw_image == nullptr || !aligned16(w_text) ||
      !aligned16(w_image) || !aligned16(dw_text) || !aligned16(dw_image) || !aligned4_or_null(db_text) ||
      !aligned4_or_null(db_image))
    return MF_ERR_INVALID_ARG;
  if (n_tokens > 0 && (dq == nullptr || dk == nullptr || dv == nullptr || h == nullptr || dh == nullptr ||
                       !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(h) || !aligned16(dh)))
    return MF_ERR_INVALID_ARG;
  const BlockBwdWorkspace w =
      block_bwd_layout(1, n_samples, frames, n_tokens, channels, head_dim, pos != nullptr ? max_pos : 0);
  if ((st = check_workspace(workspace, workspace_bytes, w.total)) != MF_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int* tstart = reinterpret_cast<int*>(ws + w.tstart);
  int* col0 = reinterpret_cast<int*>(ws + w.col0);
  int* kr = reinterpret_cast<int*>(ws + w.kr);
  const int n_pieces = (frames + 1) * n_samples;
  const size_t nc = static_cast<size_t>(n_tokens) * channels;
  Tracer tr(trace, s);
  hipError_t e = tr.run("piece_tiles", [&] { return mf::launch_piece_tiles(cu_pieces, n_pieces, n_tokens, tstart, s); });
  if (e != hipSuccess) return MF_ERR_HIP;
  e = tr.run("modality_cols",
             [&] { return mf::launch_modality_cols(cu_pieces, n_samples, frames, n_tokens, col0, kr, s); });
  if (e != hipSuccess) return MF_ERR_HIP;
  uint16_t* wt = reinterpret_cast<uint16_t*>(ws + w.wt);
  const size_t wsz = static_cast<size_t>(3) * channels * channels;
  e = tr.run("transpose_w", [&] {
    hipError_t r = mf::launch_transpose(w_text, 3 * channels, channels, wt, s);
    if (r != hipSuccess) return r;
    return mf::launch_transpose(w_image, 3 * channels, channels, wt + wsz, s);
  });
  if (e != hipSuccess) return MF_ERR_HIP;
  // The gather-transpose of G = [dq' | dk' | dv] applies the inverse rotation
  // on the way (gradients with respect to the un-rotated projections) and
  // leaves dq', dk' token-major in the workspace for the activation gradient.
  const void* g[3] = {dq, dk, dv};
  mf::GatherRotation rot = {};
  if (pos != nullptr) {
    float2* tab = reinterpret_cast<float2*>(ws + w.tab);
    uint16_t* dqk = reinterpret_cast<uint16_t*>(ws + w.dqk);
    e = tr.run("rope_table", [&] { return mf::launch_rope_table(tab, max_pos, head_dim, nax, theta, s); });
    if (e != hipSuccess) return MF_ERR_HIP;
    rot = {pos, nax, max_pos, head_dim, tab, dqk, dqk + nc};
  }
  float* bpart = reinterpret_cast<float*>(ws + w.bpart);
  e = tr.run("gather_t", [&] {
    hipError_t r = mf::launch_gather_t(g, 3, channels, cu_pieces, col0, kr, n_samples, frames, n_tokens, ws + w.at,
                                       w.pitch, bpart, pos != nullptr ? &rot : nullptr, s);
    if (r != hipSuccess) return r;
    const void* hs[1] = {h};
    return mf::launch_gather_t(hs, 1, channels, cu_pieces, col0, kr, n_samples, frames, n_tokens, ws + w.bt, w.pitch,
                               nullptr, nullptr, s);
  });
  if (e != hipSuccess) return MF_ERR_HIP;
  if (pos != nullptr) {
    g[0] = rot.out_q;
    g[1] = rot.out_k;
  }
  if (n_tokens > 0) {
    e = tr.run("dgrad", [&] {
      return mf::launch_dgrad(g, 3, channels, wt, wt + wsz, cu_pieces, tstart, n_samples, frames, n_tokens, channels,
                              dh, s);
    });
    if (e != hipSuccess) return MF_ERR_HIP;
  }
  e = tr.run("wgrad", [&] {
    return mf::launch_wgrad(ws + w.at, ws + w.bt, w.pitch, 3 * channels, channels, kr, w.splits,
                            reinterpret_cast<float*>(ws + w.split), dw_text, dw_image, s);
  });
  if (e != hipSuccess) return MF_ERR_HIP;
  if (w.splits > 2) {
    e = tr.run("split_sum", [&] {
      return mf::launch_split_sum(reinterpret_cast<float*>(ws + w.split), w.pitch, 3 * channels, channels, kr,
                                  w.splits, dw_text, dw_image, s);
    });
    if (e != hipSuccess) return MF_ERR_HIP;
  }
  return from_hip(tr.run("bias_sum", [&] { return mf::launch_bias_sum(bpart, 3 * channels, kr, w.pitch, db_text, db_image, s); }));
}

mf_status mf_out_gated_residual_bwd(const void* dy, const void* o, const void* proj, const void* w_text,
                                    const void* w_image, const float* gate, void* d_o, float* dw_text,
                                    float* dw_image, float* db_text, float* db_image, float* dgate,
                                    const int32_t* cu_pieces, int32_t n_samples, int32_t frames, int32_t n_tokens,
                                    int32_t channels, void* workspace, size_t workspace_bytes, void* stream,
                                    mf_trace* trace) {
  mf_status st = check_block_common(cu_pieces, n_samples, frames, n_tokens, channels);
  if (st != MF_OK) return st;
  if (n_tokens > kBwdMaxTokens || channels > kBwdMaxChannels) return MF_ERR_UNSUPPORTED;
  if (!trace_ok(trace)) return MF_ERR_INVALID_ARG;
  if (w_text == nullptr || w_image == nullptr || dw_text == nullptr || dw_image == nullptr || !aligned16(w_text) ||
      !aligned16(w_image) || !aligned16(dw_text) || !aligned16(dw_image) || !aligned4_or_null(db_text) ||
      !aligned4_or_null(db_image))
    return MF_ERR_INVALID_ARG;
  if (n_samples > 0 && (gate == nullptr || dgate == nullptr || !aligned16(gate) || !aligned16(dgate)))
    return MF_ERR_INVALID_ARG;
  if (n_tokens > 0 && (dy == nullptr || o == nullptr || proj == nullptr || d_o == nullptr || !aligned16(dy) ||
                       !aligned16(o) || !aligned16(proj) || !aligned16(d_o)))
    return MF_ERR_INVALID_ARG;
  const BlockBwdWorkspace w = block_bwd_layout(2, n_samples, frames, n_tokens, channels, 64, 0);
  if ((st = check_workspace(workspace, workspace_bytes, w.total)) != MF_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int* tstart = reinterpret_cast<int*>(ws + w.tstart);
  int* col0 = reinterpret_cast<int*>(ws + w.col0);
  int* kr = reinterpret_cast<int*>(ws + w.kr);
  void* u = ws + w.u;
  float* gpart = reinterpret_cast<float*>(ws + w.part);
  const int n_pieces = (frames + 1) * n_samples;
  Tracer tr(trace, s);
  hipError_t e = tr.run("piece_tiles", [&] { return mf::launch_piece_tiles(cu_pieces, n_pieces, n_tokens, tstart, s); });
  if (e != hipSuccess) return MF_ERR_HIP;
  e = tr.run("modality_cols",
             [&] { return mf::launch_modality_cols(cu_pieces, n_samples, frames, n_tokens, col0, kr, s); });
  if (e != hipSuccess) return MF_ERR_HIP;
  if (n_tokens > 0) {
    e = tr.run("gate_bwd", [&] {
      return mf::launch_gate_bwd(dy, proj, gate, cu_pieces, tstart, n_samples, frames, n_tokens, channels, u, gpart,
                                 s);
    });
    if (e != hipSuccess) return MF_ERR_HIP;
  }
  e = tr.run("group_sum",
             [&] { return mf::launch_group_sum(gpart, channels, 0, channels, tstart, n_samples, frames, n_tokens, dgate, s); });
  if (e != hipSuccess) return MF_ERR_HIP;
  uint16_t* wt = reinterpret_cast<uint16_t*>(ws + w.wt);
  const size_t wsz = static_cast<size_t>(channels) * channels;
  e = tr.run("transpose_w", [&] {
    hipError_t r = mf::launch_transpose(w_text, channels, channels, wt, s);
    if (r != hipSuccess) return r;
    return mf::launch_transpose(w_image, channels, channels, wt + wsz, s);
  });
  if (e != hipSuccess) return MF_ERR_HIP;
  const void* us[1] = {u};
  if (n_tokens > 0) {
    e = tr.run("dgrad", [&] {
      return mf::launch_dgrad(us, 1, channels, wt, wt + wsz, cu_pieces, tstart, n_samples, frames, n_tokens, channels,
                              d_o, s);
    });
    if (e != hipSuccess) return MF_ERR_HIP;
  }
  float* bpart = reinterpret_cast<float*>(ws + w.bpart);
  e = tr.run("gather_t", [&] {
    hipError_t r = mf::launch_gather_t(us, 1, channels, cu_pieces, col0, kr, n_samples, frames, n_tokens, ws + w.at,
                                       w.pitch, bpart, nullptr, s);
    if (r != hipSuccess) return r;
    const void* os[1] = {o};
    return mf::launch_gather_t(os, 1, channels, cu_pieces, col0, kr, n_samples, frames, n_tokens, ws + w.bt, w.pitch,
                               nullptr, nullptr, s);
  });
  if (e != hipSuccess) return MF_ERR_HIP;
  e = tr.run("wgrad", [&] {
    return mf::launch_wgrad(ws + w.at, ws + w.bt, w.pitch, channels, channels, kr, w.splits,
                            reinterpret_cast<float*>(ws + w.split), dw_text, dw_image, s);
  });
  if (e != hipSuccess) return MF_ERR_HIP;
  if (w.splits > 2) {
    e = tr.run("split_sum", [&] {
      return mf::launch_split_sum(reinterpret_cast<float*>(ws + w.split), w.pitch, channels, channels, kr, w.splits,
                                  dw_text, dw_image, s);
    });
    if (e != hipSuccess) return MF_ERR_HIP;
  }
  return from_hip(tr.run("bias_sum", [&] { return mf::launch_bias_sum(bpart, channels, kr, w.pitch, db_text, db_image, s); }));
}

}  // extern "C"

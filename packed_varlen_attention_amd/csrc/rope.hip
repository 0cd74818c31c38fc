// Rotary position embedding at native positions: axial 2D (rcap.io post,
// `per_sample_2d_rope` in the "native-resolution packed step" pseudo-code;
// ai.thesatyajit.com explainer, "A backbone that doesn't crop") and its
// frame-aware 3D extension for editing (Mage-Flow paper section 3.2.2,
// "Conditioning and rectified-flow training": visual tokens at (h, w, f)).
// Mage-Flow paper section 3.3 lists RoPE among the fused memory-bound chains.
//
// rope_table  cos/sin of the layout's angles (see rope_entry), computed in
//             float64, stored as float32, [max_pos][rope_tab_width] float2;
// rope_apply  streams a [N][H][D] tensor, 8 elements (one 16-byte bf16
//             vector) per thread, rotating each 8-element group by its
//             block's axis; optionally converts dtype on the way (the
//             attention calls use it to rotate K once and to convert float32
//             inputs to bf16).  HBM-bound.
#include "mf_device.h"
#include "mf_kernels.h"

namespace mf {

namespace {

// Entry j of a table row: pair j of a block of `block` dims turns at
// theta^(-2j/block).  2D rows are D/4 pairs of a D/2 block; 3D rows are the
// 3D/16 pairs of a 3D/8 block, then the D/8 pairs of the D/4 frame block.
__global__ __launch_bounds__(256) void rope_table_kernel(float2* __restrict__ tab, int max_pos, int head_dim,
                                                         int nax, double theta) {
  const int width = nax == 3 ? 3 * head_dim / 16 + head_dim / 8 : head_dim / 4;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= max_pos * width) return;
  const int p = idx / width;
  int j = idx % width;
  int block = head_dim / 2;
  if (nax == 3) {
    block = 3 * head_dim / 8;
    if (j >= block / 2) {
      j -= block / 2;
      block = head_dim / 4;
    }
  }
  const double freq = pow(theta, -(2.0 * j) / block);
  const double ang = static_cast<double>(p) * freq;
  tab[idx] = make_float2(static_cast<float>(cos(ang)), static_cast<float>(sin(ang)));
}

template <int D, typename TIn, typename TOut, bool kRotate>
__global__ __launch_bounds__(256) void rope_apply_kernel(const TIn* __restrict__ src, TOut* __restrict__ dst,
                                                         const int* __restrict__ pos, int nax,
                                                         const float2* __restrict__ tab, int max_pos,
                                                         long long n_vec, int heads, float sign) {
  constexpr int kVecPerRow = D / 8;
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  for (long long vi = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; vi < n_vec; vi += stride) {
    const long long row = vi / kVecPerRow;  // (token, head) row
    const int e0 = static_cast<int>(vi % kVecPerRow) * 8;
    float x[8];
    load8<TIn>(src + vi * 8, x);
    if constexpr (kRotate) {
      const long long t = row / heads;
      rotate_n<D, 8>(x, e0, load_pos(pos, t, nax), tab, max_pos, sign, nax);
    }
    store8<TOut>(dst + vi * 8, x);
  }
}

template <int D, typename TIn, typename TOut>
hipError_t launch_apply_d(const void* src, void* dst, const int* pos, int nax, const float2* tab, int max_pos,
                          int n_tokens, int heads, bool rotate, bool inverse, hipStream_t stream) {
  const long long n_vec = static_cast<long long>(n_tokens) * heads * (D / 8);
  if (n_vec == 0) return hipSuccess;
  long long blocks = (n_vec + 255) / 256;
  const long long max_blocks = 256LL * 16;
  if (blocks > max_blocks) blocks = max_blocks;
  const float sign = inverse ? -1.0f : 1.0f;
  if (rotate) {
    hipLaunchKernelGGL((rope_apply_kernel<D, TIn, TOut, true>), dim3(static_cast<int>(blocks)), dim3(256), 0,
                       stream, static_cast<const TIn*>(src), static_cast<TOut*>(dst), pos, nax, tab, max_pos,
                       n_vec, heads, sign);
  } else {
    hipLaunchKernelGGL((rope_apply_kernel<D, TIn, TOut, false>), dim3(static_cast<int>(blocks)), dim3(256), 0,
                       stream, static_cast<const TIn*>(src), static_cast<TOut*>(dst), pos, nax, tab, max_pos,
                       n_vec, heads, sign);
  }
  return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_apply_t(int head_dim, const void* src, void* dst, const int* pos, int nax, const float2* tab,
                          int max_pos, int n_tokens, int heads, bool rotate, bool inverse,
                          hipStream_t stream) {
  if (head_dim == 128)
    return launch_apply_d<128, TIn, TOut>(src, dst, pos, nax, tab, max_pos, n_tokens, heads, rotate, inverse,
                                          stream);
  return launch_apply_d<64, TIn, TOut>(src, dst, pos, nax, tab, max_pos, n_tokens, heads, rotate, inverse,
                                       stream);
}

}  // namespace

int rope_table_width(int head_dim, int nax) {
  return nax == 3 ? 3 * head_dim / 16 + head_dim / 8 : head_dim / 4;
}

hipError_t launch_rope_table(float2* tab, int max_pos, int head_dim, int nax, double theta, hipStream_t stream) {
  const long long total = static_cast<long long>(max_pos) * rope_table_width(head_dim, nax);
  if (total <= 0) return hipSuccess;
  if (total > 0x7fffffffLL - 255) return hipErrorInvalidValue;  // the grid's last index fits an int
  hipLaunchKernelGGL(rope_table_kernel, dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0, stream, tab,
                     max_pos, head_dim, nax, theta);
  return hipGetLastError();
}

hipError_t launch_rope_apply(const void* src, int src_dtype, void* dst, int dst_dtype, const int* pos, int nax,
                             const float2* tab, int max_pos, int n_tokens, int heads, int head_dim,
                             bool rotate, bool inverse, hipStream_t stream) {
  if (src_dtype == kDtypeBf16 && dst_dtype == kDtypeBf16)
    return launch_apply_t<uint16_t, uint16_t>(head_dim, src, dst, pos, nax, tab, max_pos, n_tokens, heads, rotate,
                                              inverse, stream);
  if (src_dtype == kDtypeF32 && dst_dtype == kDtypeF32)
    return launch_apply_t<float, float>(head_dim, src, dst, pos, nax, tab, max_pos, n_tokens, heads, rotate,
                                        inverse, stream);
  if (src_dtype == kDtypeF32 && dst_dtype == kDtypeBf16)
    return launch_apply_t<float, uint16_t>(head_dim, src, dst, pos, nax, tab, max_pos, n_tokens, heads, rotate,
                                           inverse, stream);
  return hipErrorInvalidValue;
}

}  // namespace mf

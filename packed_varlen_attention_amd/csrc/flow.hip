// Rectified-flow noising, target and loss over the packed latent stream, and
// the packed classifier-free-guidance combine.
//
// Training regresses the model's velocity on z - eps, where the model input
// is z_t = (1 - t) z + t eps (Mage-Flow paper section 3.2.1 as summarised on
// paperlayer.ai, "Method"; rcap.io post, `loss = mse(v_pred, (z - noise))`);
// for editing only the target tokens carry the loss (paper section 3.2.2,
// hyper.ai summary).  Packed CFG evaluates each prompt's conditional and
// unconditional branches as consecutive segments of one pass (paper section
// 3.2.1); the combine is the usual guidance form v_u + s (v_c - v_u).
//
// Latents are [N][C] rows in packed order (text rows carry none and are left
// alone).  A row's role comes from cu_pieces, which has frames + 1 entries
// per sample (start, image start for frames = 1; start, source start, target
// start for frames = 2): the noised rows of sample s are [cu_pieces[per*s +
// frames], cu_pieces[per*(s+1)]).  Every kernel is one HBM pass: one thread
// per 8 consecutive elements of a row, found by binary search in cu_pieces.
#include "mf_device.h"
#include "mf_kernels.h"

namespace mf {

namespace {

// Index i with cp[i] <= row < cp[i + 1] among cp[0..m], or -1.
__device__ __forceinline__ int piece_of(const int* __restrict__ cp, int m, int row) {
  if (m <= 0 || row < cp[0] || row >= cp[m]) return -1;
  int lo = 0, hi = m;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cp[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

template <typename T>
__global__ __launch_bounds__(256) void rf_noise_kernel(const T* __restrict__ z, const T* __restrict__ eps,
                                                       const float* __restrict__ t, T* __restrict__ zt,
                                                       const int* __restrict__ cp, int n_samples, int frames,
                                                       long long n_vec, int vec_per_row) {
  const int per = frames + 1;
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  for (long long vi = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; vi < n_vec; vi += stride) {
    const int row = static_cast<int>(vi / vec_per_row);
    const int i = piece_of(cp, per * n_samples, row);
    float a[8];
    load8<T>(z + vi * 8, a);
    if (i >= 0 && i % per == frames) {
      const float ts = t[i / per];
      float b[8];
      load8<T>(eps + vi * 8, b);
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = (1.0f - ts) * a[j] + ts * b[j];
    }
    store8<T>(zt + vi * 8, a);
  }
}

// grad = grad_scale * (v - (z - eps)) on noised rows (0 elsewhere); each
// row's sum of squares goes to row_sum[row] (0 for rows without loss).  The
// vec_per_row lanes of a row are consecutive in one wave (vec_per_row is a
// power of two <= 64), so the row sum is a shuffle reduction.
template <typename T>
__global__ __launch_bounds__(256) void rf_loss_rows_kernel(const T* __restrict__ v, const T* __restrict__ z,
                                                           const T* __restrict__ eps, T* __restrict__ grad,
                                                           float* __restrict__ row_sum, const int* __restrict__ cp,
                                                           int n_samples, int frames, long long n_vec,
                                                           int vec_per_row, float grad_scale) {
  const int per = frames + 1;
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  for (long long base = static_cast<long long>(blockIdx.x) * blockDim.x; base < n_vec; base += stride) {
    const long long vi = base + threadIdx.x;
    const bool in = vi < n_vec;
    const int row = in ? static_cast<int>(vi / vec_per_row) : 0;
    const int i = in ? piece_of(cp, per * n_samples, row) : -1;
    const bool noised = i >= 0 && i % per == frames;
    float r[8];
    float acc = 0.f;
    if (noised) {
      float a[8], b[8], c[8];
      load8<T>(v + vi * 8, a);
      load8<T>(z + vi * 8, b);
      load8<T>(eps + vi * 8, c);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        r[j] = a[j] - (b[j] - c[j]);
        acc += r[j] * r[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = 0.f;
    }
    if (in && grad != nullptr) {
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] *= grad_scale;
      store8<T>(grad + vi * 8, r);
    }
    for (int m = vec_per_row >> 1; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if (in && vi % vec_per_row == 0) row_sum[row] = acc;
  }
}

// loss_sum[s] = sum of row_sum over sample s's noised rows, one workgroup per
// sample, in a fixed order (deterministic).  Four independent loads per
// thread and trip keep the row sums streaming.
constexpr int kReduceThreads = 1024;

__global__ __launch_bounds__(kReduceThreads) void rf_loss_reduce_kernel(const float* __restrict__ row_sum,
                                                                        const int* __restrict__ cp, int frames,
                                                                        float* __restrict__ loss_sum) {
  __shared__ float s_part[kReduceThreads];
  const int per = frames + 1;
  const int s = blockIdx.x;
  const int a = cp[per * s + frames];
  const int b = cp[per * (s + 1)];
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int r = a + static_cast<int>(threadIdx.x); r < b; r += 4 * kReduceThreads) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (r + u * kReduceThreads < b) acc[u] += row_sum[r + u * kReduceThreads];
  }
  s_part[threadIdx.x] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  __syncthreads();
  for (int w = kReduceThreads / 2; w >= 1; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) s_part[threadIdx.x] += s_part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss_sum[s] = s_part[0];
}

// Number of (cond, uncond) pairs whose image sizes differ (one workgroup).
__global__ __launch_bounds__(256) void cfg_check_kernel(const int* __restrict__ cp, int n_pairs,
                                                        int* __restrict__ mismatched) {
  __shared__ int s_bad;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < n_pairs; p += 256) {
    const int c = 2 * p, u = c + 1;
    if (cp[2 * c + 2] - cp[2 * c + 1] != cp[2 * u + 2] - cp[2 * u + 1]) atomicAdd(&s_bad, 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) *mismatched = s_bad;
}

template <typename T>
__global__ __launch_bounds__(256) void cfg_combine_kernel(const T* v, T* out,  // may alias (in place)
                                                          const int* __restrict__ cp, int n_pairs, long long n_vec,
                                                          int vec_per_row, float scale) {
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  const bool in_place = static_cast<const void*>(out) == static_cast<const void*>(v);
  for (long long vi = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; vi < n_vec; vi += stride) {
    const int row = static_cast<int>(vi / vec_per_row);
    const int k = static_cast<int>(vi % vec_per_row);
    const int i = piece_of(cp, 4 * n_pairs, row);
    const int s = i >> 1;
    bool guided = i >= 0 && (i & 1) == 1 && (s & 1) == 0;  // image rows of a cond sample
    int urow = 0;
    if (guided) {
      const int u = s + 1;
      guided = cp[2 * s + 2] - cp[2 * s + 1] == cp[2 * u + 2] - cp[2 * u + 1];
      urow = cp[2 * u + 1] + (row - cp[2 * s + 1]);
    }
    if (guided) {
      float c[8], un[8];
      load8<T>(v + vi * 8, c);
      load8<T>(v + (static_cast<long long>(urow) * vec_per_row + k) * 8, un);
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = un[j] + scale * (c[j] - un[j]);
      store8<T>(out + vi * 8, c);
    } else if (!in_place) {
      float c[8];
      load8<T>(v + vi * 8, c);
      store8<T>(out + vi * 8, c);
    }
  }
}

int flow_blocks(long long n_vec) {
  long long blocks = (n_vec + 255) / 256;
  const long long max_blocks = 256LL * 16;
  return static_cast<int>(blocks > max_blocks ? max_blocks : (blocks < 1 ? 1 : blocks));
}

}  // namespace

hipError_t launch_rf_noise(const void* z, const void* eps, const float* t, void* zt, int dtype, const int* cu_pieces,
                           int n_samples, int frames, int n_tokens, int channels, hipStream_t stream) {
  const long long n_vec = static_cast<long long>(n_tokens) * (channels / 8);
  if (n_vec == 0) return hipSuccess;
  if (dtype == kDtypeBf16) {
    hipLaunchKernelGGL((rf_noise_kernel<uint16_t>), dim3(flow_blocks(n_vec)), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(z), static_cast<const uint16_t*>(eps), t,
                       static_cast<uint16_t*>(zt), cu_pieces, n_samples, frames, n_vec, channels / 8);
  } else {
    hipLaunchKernelGGL((rf_noise_kernel<float>), dim3(flow_blocks(n_vec)), dim3(256), 0, stream,
                       static_cast<const float*>(z), static_cast<const float*>(eps), t, static_cast<float*>(zt),
                       cu_pieces, n_samples, frames, n_vec, channels / 8);
  }
  return hipGetLastError();
}

hipError_t launch_rf_loss(const void* v, const void* z, const void* eps, void* grad, float* row_sum,
                          float* loss_sum, int dtype, const int* cu_pieces, int n_samples, int frames, int n_tokens,
                          int channels, float grad_scale, hipStream_t stream) {
  const long long n_vec = static_cast<long long>(n_tokens) * (channels / 8);
  if (n_vec > 0) {
    if (dtype == kDtypeBf16) {
      hipLaunchKernelGGL((rf_loss_rows_kernel<uint16_t>), dim3(flow_blocks(n_vec)), dim3(256), 0, stream,
                         static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(z),
                         static_cast<const uint16_t*>(eps), static_cast<uint16_t*>(grad), row_sum, cu_pieces,
                         n_samples, frames, n_vec, channels / 8, grad_scale);
    } else {
      hipLaunchKernelGGL((rf_loss_rows_kernel<float>), dim3(flow_blocks(n_vec)), dim3(256), 0, stream,
                         static_cast<const float*>(v), static_cast<const float*>(z), static_cast<const float*>(eps),
                         static_cast<float*>(grad), row_sum, cu_pieces, n_samples, frames, n_vec, channels / 8,
                         grad_scale);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_samples == 0) return hipSuccess;
  hipLaunchKernelGGL(rf_loss_reduce_kernel, dim3(n_samples), dim3(kReduceThreads), 0, stream, row_sum, cu_pieces,
                     frames, loss_sum);
  return hipGetLastError();
}

hipError_t launch_cfg_combine(const void* v, void* out, int* mismatched, int dtype, const int* cu_pieces,
                              int n_pairs, int n_tokens, int channels, float scale, hipStream_t stream) {
  if (mismatched != nullptr) {
    hipLaunchKernelGGL(cfg_check_kernel, dim3(1), dim3(256), 0, stream, cu_pieces, n_pairs, mismatched);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long n_vec = static_cast<long long>(n_tokens) * (channels / 8);
  if (n_vec == 0) return hipSuccess;
  if (dtype == kDtypeBf16) {
    hipLaunchKernelGGL((cfg_combine_kernel<uint16_t>), dim3(flow_blocks(n_vec)), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), cu_pieces, n_pairs, n_vec,
                       channels / 8, scale);
  } else {
    hipLaunchKernelGGL((cfg_combine_kernel<float>), dim3(flow_blocks(n_vec)), dim3(256), 0, stream,
                       static_cast<const float*>(v), static_cast<float*>(out), cu_pieces, n_pairs, n_vec,
                       channels / 8, scale);
  }
  return hipGetLastError();
}

}  // namespace mf

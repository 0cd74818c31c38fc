// Native-resolution packing on the device (Mage-Flow paper section 3.2.1
// "Model Architecture and Native Packing": variable-length text and image
// sequences packed under a fixed token budget, each image keeping its native
// latent grid; rcap.io post, `pack(..., budget=50_000)`).
//
// Editing samples (Mage-Flow paper section 3.2.2, "Conditioning and
// rectified-flow training": conditioning, then source-image latents, then
// noisy target latents; visual tokens at (h, w, f)) pack the same way with
// two frames per sample: [text | source | target].
//
// Two kernels, for frames = 1 ([text | image], positions (row, col)) or
// frames = 2 ([text | source | target], positions (row, col, frame)):
//   pack_scan  one workgroup: validates the descriptors, scans the sample
//              lengths T + frames * grid_h * grid_w, cuts the longest prefix
//              that fits the budget and writes cu_seqlens, cu_pieces and
//              counts;
//   pack_fill  one wave per packed token (grid-stride): finds the token's
//              segment by binary search in cu_seqlens, writes its position
//              and, when asked, copies its source row into the packed buffer.
#include "mf_device.h"
#include "mf_kernels.h"

namespace mf {

namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / 64;

struct Sample {
  int32_t text_len, grid_h, grid_w;
};

// Inclusive block-wide scan of one int64 per thread.
__device__ long long block_incl_scan(long long x, long long* s_wave) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const long long y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  if (wave == 0) {
    long long w = lane < kScanWaves ? s_wave[lane] : 0;
#pragma unroll
    for (int d = 1; d < kScanWaves; d <<= 1) {
      const long long y = __shfl_up(w, d, 64);
      if (lane >= d) w += y;
    }
    if (lane < kScanWaves) s_wave[lane] = w;
  }
  __syncthreads();
  if (wave > 0) x += s_wave[wave - 1];
  __syncthreads();
  return x;
}

__global__ __launch_bounds__(kScanThreads) void pack_scan_kernel(
    const Sample* __restrict__ samples, int n, int budget, int frames, int* __restrict__ cu_seqlens,
    int* __restrict__ cu_pieces, int* __restrict__ counts) {
  const int per = frames + 1;  // cu_pieces entries per sample
  __shared__ long long s_wave[kScanWaves];
  __shared__ int s_err;
  __shared__ int s_npacked;
  __shared__ long long s_total;
  __shared__ int s_maxlen;
  __shared__ int s_maxpos;
  if (threadIdx.x == 0) {
    s_err = 0;
    s_npacked = 0;
    s_total = 0;
    s_maxlen = 0;
    s_maxpos = 0;
  }
  __syncthreads();

  // Pass 1: every descriptor must be non-negative and its length fit int32.
  for (int i = threadIdx.x; i < n; i += kScanThreads) {
    const Sample s = samples[i];
    const long long len = static_cast<long long>(s.text_len) +
                          frames * static_cast<long long>(s.grid_h) * static_cast<long long>(s.grid_w);
    if (s.text_len < 0 || s.grid_h < 0 || s.grid_w < 0 || len > 0x7fffffffLL) s_err = 1;
  }
  __syncthreads();
  if (s_err) {
    for (int i = threadIdx.x; i <= n; i += kScanThreads) cu_seqlens[i] = 0;
    if (cu_pieces)
      for (int i = threadIdx.x; i <= per * n; i += kScanThreads) cu_pieces[i] = 0;
    if (threadIdx.x == 0) {
      counts[0] = -1;
      counts[1] = 0;
      counts[2] = 0;
      counts[3] = 0;
    }
    return;
  }

  // Pass 2: inclusive scan; a sample is packed iff its inclusive end fits
  // the budget (lengths are non-negative, so the packed set is a prefix).
  // cu_seqlens[i + 1] temporarily holds the end of sample i, or -1 if not
  // packed.
  long long carry = 0;
  for (int base = 0; base < n; base += kScanThreads) {
    const int i = base + threadIdx.x;
    long long len = 0;
    Sample s = {0, 0, 0};
    if (i < n) {
      s = samples[i];
      len = static_cast<long long>(s.text_len) + frames * static_cast<long long>(s.grid_h) * s.grid_w;
    }
    const long long incl = carry + block_incl_scan(len, s_wave);
    const bool packed = i < n && incl <= budget;
    if (i < n) cu_seqlens[i + 1] = packed ? static_cast<int>(incl) : -1;
    if (packed) {
      atomicAdd(&s_npacked, 1);
      atomicMax(&s_maxlen, static_cast<int>(len));
      int mp = 0;
      if (s.text_len > 0) mp = s.text_len;
      if (s.grid_h > 0 && s.grid_w > 0) {
        mp = max(mp, s.text_len + max(s.grid_h, s.grid_w));  // rows and columns up to T + max - 1
        if (frames == 2) mp = max(mp, s.text_len + 2);       // frames T (source) and T + 1 (target)
      }
      atomicMax(&s_maxpos, mp);
    }
    // The last thread's inclusive value is the running total.
    if (threadIdx.x == kScanThreads - 1) s_total = incl;
    __syncthreads();
    carry = s_total;
    __syncthreads();
  }
  const int npk = s_npacked;
  // Total of the packed prefix.
  __shared__ int s_ntok;
  if (threadIdx.x == 0) s_ntok = npk > 0 ? cu_seqlens[npk] : 0;
  __syncthreads();
  const int ntok = s_ntok;

  // Pass 3: final offsets.  Entries past the packed prefix hold ntok.
  for (int i = threadIdx.x; i <= n; i += kScanThreads) {
    int v;
    if (i == 0) {
      v = 0;
    } else if (i <= npk) {
      v = cu_seqlens[i];
    } else {
      v = ntok;
    }
    // Each thread rewrites only its own index, after reading it.
    cu_seqlens[i] = v;
    if (cu_pieces) {
      if (i < n) {
        const bool in = i < npk;
        const Sample si = samples[i];
        cu_pieces[per * i] = v;
        cu_pieces[per * i + 1] = in ? v + si.text_len : ntok;
        if (frames == 2) cu_pieces[per * i + 2] = in ? v + si.text_len + si.grid_h * si.grid_w : ntok;
      } else {
        cu_pieces[per * n] = ntok;
      }
    }
  }
  if (threadIdx.x == 0) {
    counts[0] = npk;
    counts[1] = ntok;
    counts[2] = s_maxlen;
    counts[3] = s_maxpos;
  }
}

__global__ __launch_bounds__(256) void pack_fill_kernel(
    const Sample* __restrict__ samples, const int* __restrict__ cu_seqlens, const int* __restrict__ counts,
    int frames, int* __restrict__ pos, const char* const* __restrict__ text_rows,
    const char* const* __restrict__ image_rows, const char* const* __restrict__ target_rows, long long row_bytes,
    char* __restrict__ packed) {
  const int npk = counts[0];
  const int ntok = counts[1];
  if (npk <= 0) return;
  const int lane = threadIdx.x & 63;
  const int waves_per_block = blockDim.x >> 6;
  const long long total_waves = static_cast<long long>(gridDim.x) * waves_per_block;
  for (long long t = static_cast<long long>(blockIdx.x) * waves_per_block + (threadIdx.x >> 6); t < ntok;
       t += total_waves) {
    // Segment s with cu[s] <= t < cu[s + 1] (empty segments are skipped).
    int lo = 0, hi = npk;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu_seqlens[mid] <= t) lo = mid; else hi = mid;
    }
    const Sample s = samples[lo];
    const int u = static_cast<int>(t) - cu_seqlens[lo];
    const bool text = u < s.text_len;
    // Image tokens: frame f (0 source, 1 target), index v inside the grid.
    int v = u - s.text_len;
    int f = 0;
    if (!text && frames == 2) {
      const int img = s.grid_h * s.grid_w;
      f = v >= img;
      v -= f * img;
    }
    if (lane == 0) {
      int r = u, c = u, fr = u;
      if (!text) {
        r = s.text_len + v / s.grid_w;
        c = s.text_len + v % s.grid_w;
        fr = s.text_len + f;
      }
      if (frames == 2) {
        pos[3 * t] = r;
        pos[3 * t + 1] = c;
        pos[3 * t + 2] = fr;
      } else {
        reinterpret_cast<int2*>(pos)[t] = make_int2(r, c);
      }
    }
    if (packed) {
      const char* src = text ? text_rows[lo] + static_cast<long long>(u) * row_bytes
                             : (f ? target_rows[lo] : image_rows[lo]) + static_cast<long long>(v) * row_bytes;
      char* dst = packed + t * row_bytes;
      if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) |
            static_cast<uintptr_t>(row_bytes)) & 15) == 0) {
        const long long n16 = row_bytes >> 4;
        for (long long c = lane; c < n16; c += 64)
          reinterpret_cast<u32x4*>(dst)[c] = reinterpret_cast<const u32x4*>(src)[c];
      } else {
        for (long long c = lane; c < row_bytes; c += 64) dst[c] = src[c];
      }
    }
  }
}

}  // namespace

hipError_t launch_pack_scan(const void* samples, int n, int budget, int frames, int* cu_seqlens, int* cu_pieces,
                            int* counts, hipStream_t stream) {
  hipLaunchKernelGGL(pack_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream,
                     static_cast<const Sample*>(samples), n, budget, frames, cu_seqlens, cu_pieces, counts);
  return hipGetLastError();
}

hipError_t launch_pack_fill(const void* samples, int budget, int frames, const int* cu_seqlens, const int* counts,
                            int* pos, const void* const* text_rows, const void* const* image_rows,
                            const void* const* target_rows, long long row_bytes, void* packed, hipStream_t stream) {
  // Enough waves to stream the rows at full bandwidth; each loops over tokens.
  long long waves = budget;
  const long long max_waves = 256LL * 8 * 4;  // 8 resident blocks of 4 waves on 256 CUs
  if (waves > max_waves) waves = max_waves;
  const int blocks = static_cast<int>((waves + 3) / 4);
  hipLaunchKernelGGL(pack_fill_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const Sample*>(samples), cu_seqlens, counts, frames, pos,
                     reinterpret_cast<const char* const*>(text_rows),
                     reinterpret_cast<const char* const*>(image_rows),
                     reinterpret_cast<const char* const*>(target_rows), row_bytes, static_cast<char*>(packed));
  return hipGetLastError();
}

}  // namespace mf

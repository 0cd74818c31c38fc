// Work schedule for the attention kernels: longest segment first, and every
// tile of one (segment, head) on the same XCD.
//
// sched_kernel (one workgroup) sorts the segments by length, longest first
// (ties by index; up to kMaxSortSegments, beyond that the given order), and
// writes order[r] = segment of rank r and the exclusive prefix pt[r] of the
// tile counts ceil(L / tile) in that order (pt[n] = total tiles).
//
// The attention kernels launch 8 * ceil(H/8) * bound blocks and decode block
// b with decode_item(): XCD x = b % 8 (the dispatcher hands consecutive block
// ids to the 8 XCDs in turn) owns heads x, x+8, ...; its i-th block (i = b/8)
// walks ranks in order, heads of the rank, then tiles, so the concurrently
// running blocks of one XCD share one (segment, head)'s K and V in that XCD's
// L2.  Blocks past the end of their XCD's list exit.
#include "mf_device.h"
#include "mf_kernels.h"

namespace mf {

namespace {

constexpr int kThreads = 1024;
constexpr int kMaxSortSegments = 1024;

__global__ __launch_bounds__(kThreads) void sched_kernel(const int* __restrict__ cu, int n_seg, int n_tokens,
                                                         int tile, int* __restrict__ order, int* __restrict__ pt) {
  __shared__ int sLen[kMaxSortSegments];
  __shared__ int sWave[kThreads / 64];
  __shared__ int sCarry;
  const bool sort = n_seg <= kMaxSortSegments;
  auto seg_len = [&](int s) {
    int a = cu[s], b = cu[s + 1];
    a = min(max(a, 0), n_tokens);
    b = min(max(b, a), n_tokens);
    return b - a;
  };
  if (sort) {
    for (int s = threadIdx.x; s < n_seg; s += kThreads) sLen[s] = seg_len(s);
    __syncthreads();
    for (int s = threadIdx.x; s < n_seg; s += kThreads) {
      const int l = sLen[s];
      int rank = 0;
      for (int t = 0; t < n_seg; ++t) {
        const int lt = sLen[t];
        rank += (lt > l) || (lt == l && t < s);
      }
      order[rank] = s;
    }
  } else {
    for (int s = threadIdx.x; s < n_seg; s += kThreads) order[s] = s;
  }
  __syncthreads();  // order[] (global) is read back by other threads below
  if (threadIdx.x == 0) sCarry = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int base = 0; base < n_seg; base += kThreads) {
    const int r = base + threadIdx.x;
    int t = 0;
    if (r < n_seg) {
      const int s = order[r];
      const int l = sort ? sLen[s] : seg_len(s);
      t = (l + tile - 1) / tile;
    }
    int x = t;  // inclusive scan
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane == 63) sWave[wave] = x;
    __syncthreads();
    if (wave == 0) {
      int w = lane < kThreads / 64 ? sWave[lane] : 0;
#pragma unroll
      for (int d = 1; d < kThreads / 64; d <<= 1) {
        const int y = __shfl_up(w, d, 64);
        if (lane >= d) w += y;
      }
      if (lane < kThreads / 64) sWave[lane] = w;
    }
    __syncthreads();
    const int incl = x + (wave > 0 ? sWave[wave - 1] : 0) + sCarry;
    if (r < n_seg) pt[r] = incl - t;
    __syncthreads();
    if (threadIdx.x == kThreads - 1) sCarry = incl;
    __syncthreads();
  }
  if (threadIdx.x == 0) pt[n_seg] = sCarry;
}

// Multi-segment tiles.  Tiny segments (at most kTinyLen tokens) that follow
// one another in the stream and start in the same kTinyLen-token window of it
// form one virtual segment, which the attention kernels cover with one or
// two query tiles and a per-lane block-diagonal mask.  Such a group spans at most
// 2 kTinyLen - 1 tokens (its last member starts inside the window and is at
// most kTinyLen long); every other segment is a virtual segment of its own.
// vcu[v] = first token of virtual segment v and vfirst[v] = its first
// segment; entries from the last virtual segment to n_seg hold the end and
// n_seg (zero-length virtual segments), so n_seg + 1 entries always suffice
// and the virtual count never exceeds n_seg.  Merging pays only when tiny
// segments carry most of the work: a shared tile runs in a launch of its own,
// while unmerged tiny tiles fill the idle tail of the long segments' launch.
// So groups form only when tiny segments hold at least half of the tokens;
// otherwise every segment is its own virtual segment.
constexpr int kTinyLen = kTinySegment;

__global__ __launch_bounds__(kThreads) void merge_kernel(const int* __restrict__ cu, int n_seg, int n_tokens,
                                                         int* __restrict__ vcu, int* __restrict__ vfirst) {
  __shared__ int sWave[kThreads / 64];
  __shared__ int sCarry;
  __shared__ int sTiny;
  if (threadIdx.x == 0) {
    sCarry = 0;
    sTiny = 0;
  }
  __syncthreads();
  auto start_of = [&](int s) { return min(max(cu[s], 0), n_tokens); };
  auto len_of = [&](int s) {
    const int a = start_of(s);
    return min(max(cu[s + 1], a), n_tokens) - a;
  };
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int tiny = 0;  // tokens in tiny segments
  for (int s = threadIdx.x; s < n_seg; s += kThreads) {
    const int l = len_of(s);
    if (l <= kTinyLen) tiny += l;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) tiny += __shfl_xor(tiny, d, 64);
  if (lane == 0) atomicAdd(&sTiny, tiny);
  __syncthreads();
  const bool merge = 2LL * sTiny >= n_tokens && n_tokens > 0;
  for (int base = 0; base < n_seg; base += kThreads) {
    const int s = base + threadIdx.x;
    int f = 0;  // 1: segment s starts a virtual segment
    if (s < n_seg) {
      f = 1;
      if (merge && s > 0 && len_of(s) <= kTinyLen && len_of(s - 1) <= kTinyLen && cu[s - 1] <= cu[s] &&
          start_of(s) / kTinyLen == start_of(s - 1) / kTinyLen)
        f = 0;
    }
    int x = f;  // inclusive scan over the block
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane == 63) sWave[wave] = x;
    __syncthreads();
    if (wave == 0) {
      int w = lane < kThreads / 64 ? sWave[lane] : 0;
#pragma unroll
      for (int d = 1; d < kThreads / 64; d <<= 1) {
        const int y = __shfl_up(w, d, 64);
        if (lane >= d) w += y;
      }
      if (lane < kThreads / 64) sWave[lane] = w;
    }
    __syncthreads();
    const int incl = x + (wave > 0 ? sWave[wave - 1] : 0) + sCarry;
    if (s < n_seg && f) {
      vcu[incl - 1] = start_of(s);
      vfirst[incl - 1] = s;
    }
    __syncthreads();
    if (threadIdx.x == kThreads - 1) sCarry = incl;
    __syncthreads();
  }
  const int n_v = sCarry;
  const int end = n_seg > 0 ? min(max(cu[n_seg], start_of(n_seg - 1)), n_tokens) : 0;
  for (int v = n_v + threadIdx.x; v <= n_seg; v += kThreads) {
    vcu[v] = end;
    vfirst[v] = n_seg;
  }
}

}  // namespace

hipError_t launch_sched(const int* cu_seqlens, int n_segments, int n_tokens, int tile, int* order, int* pt,
                        hipStream_t stream) {
  hipLaunchKernelGGL(sched_kernel, dim3(1), dim3(kThreads), 0, stream, cu_seqlens, n_segments, n_tokens, tile, order,
                     pt);
  return hipGetLastError();
}

long long sched_grid(int n_tokens, int n_segments, int heads, int tile) {
  const long long per_xcd_heads = (heads + 7) / 8;
  const long long tiles_bound = (static_cast<long long>(n_tokens) + tile - 1) / tile + n_segments;
  return 8LL * per_xcd_heads * tiles_bound;
}

hipError_t launch_merge_tiny(const int* cu_seqlens, int n_segments, int n_tokens, int* vcu, int* vfirst,
                             hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel, dim3(1), dim3(kThreads), 0, stream, cu_seqlens, n_segments, n_tokens, vcu, vfirst);
  return hipGetLastError();
}

}  // namespace mf

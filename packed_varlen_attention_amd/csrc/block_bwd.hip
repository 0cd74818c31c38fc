// Backward of the attention sub-block's fused chains: adaptive
// normalisation, the modality-specific QKV projection with the rotary
// embedding, and the output projection with the gated residual update
// (Mage-Flow paper section 3.2.1 "Model Architecture and Native Packing":
// normalisation and projection layers specific to each modality; paper
// section 3.3 "Training Infrastructure": fused chains of adaptive
// normalisation, rotary embeddings and gated residual updates).
//
// Gradients of a scalar loss, given the gradient of each chain's output:
//   adaln:  dx = rstd (g - mean(g) - xhat mean(g xhat)) with g = dh (1 + scale),
//           dshift[s][m] = sum of dh, dscale[s][m] = sum of dh xhat over the
//           rows of sample s, modality m;
//   proj:   d(act) = d(out) W_m, dW_m = d(out)^T act, db_m = column sums of
//           d(out), both summed over the rows of modality m;
//   gate:   u = gate[s][m] dy is d(out) of the output projection,
//           dgate[s][m] = sum of dy (o W^T + b) over sample s, modality m.
//
// Every sum over rows is deterministic: partial sums over fixed row blocks,
// then a reduction in a fixed order -- no atomics.
//
// Weight gradients need the reduction over tokens: both operands are gathered
// per modality and transposed to feature-major rows ([F][K], tokens
// contiguous; text tokens first, then image tokens, each run zero-padded to
// a multiple of 256), so the same 256 x 256 tile product as the forward runs
// over them with tokens as the reduction axis, split over token chunks when
// the output alone would not fill the chip.
#include "block_gemm.h"
#include "mf_device.h"
#include "block_kernels.h"
#include "mf_kernels.h"

namespace mf {

namespace {

constexpr int kSub = 64;  // rows per partial-sum block (a quarter of a projection tile)
// 64-feature tiles per transpose workgroup: the gathered form works out its
// column map once for eight; the plain weight transpose takes one
template <bool kGather>
constexpr int tr_feat_tiles() { return kGather ? 8 : 1; }

__device__ __forceinline__ int round256(int v) { return (v + 255) & ~255; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Largest i in [0, n) with arr[i] <= c, given arr[0] <= c < arr[n] (arr
// non-decreasing: the returned entry is non-empty and holds c).
__device__ __forceinline__ int search_le(const int* __restrict__ arr, int n, int c) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (arr[mid] <= c) lo = mid; else hi = mid;
  }
  return lo;
}

// Column layout of the per-modality gathered operands.  col0 holds the text
// pieces' first columns (n_samples + 1 entries, the last one = text token
// count K0), then the image pieces' (n_samples frames + 1 entries, the last =
// image token count K1); kr = {K0, K1}.  Text column c < K0 is text token
// c of the pack's text tokens in order; image column round256(K0) + r is
// image token r.
__global__ __launch_bounds__(1024) void modality_cols_kernel(const int* __restrict__ cp, int n_samples, int per,
                                                             int n_tokens, int* __restrict__ col0,
                                                             int* __restrict__ kr) {
  __shared__ int part_t[1024];
  __shared__ int part_i[1024];
  const int t = threadIdx.x;
  const int frames = per - 1;
  const int span = (n_samples + 1023) / 1024;
  const int s0 = min(t * span, n_samples), s1 = min(s0 + span, n_samples);
  int st = 0, si = 0;
  for (int s = s0; s < s1; ++s) {
    int a, e;
    piece_rows(cp, s * per, n_tokens, a, e);
    st += e - a;
    for (int f = 1; f < per; ++f) {
      piece_rows(cp, s * per + f, n_tokens, a, e);
      si += e - a;
    }
  }
  part_t[t] = st;
  part_i[t] = si;
  __syncthreads();
  if (t == 0) {
    int rt = 0, ri = 0;
    for (int i = 0; i < 1024; ++i) {
      const int vt = part_t[i], vi = part_i[i];
      part_t[i] = rt;
      part_i[i] = ri;
      rt += vt;
      ri += vi;
    }
    col0[n_samples] = rt;
    col0[n_samples + 1 + n_samples * frames] = ri;
    kr[0] = rt;
    kr[1] = ri;
  }
  __syncthreads();
  int rt = part_t[t], ri = part_i[t];
  int* col0_i = col0 + n_samples + 1;
  for (int s = s0; s < s1; ++s) {
    int a, e;
    piece_rows(cp, s * per, n_tokens, a, e);
    col0[s] = rt;
    rt += e - a;
    for (int f = 1; f < per; ++f) {
      piece_rows(cp, s * per + f, n_tokens, a, e);
      col0_i[s * frames + f - 1] = ri;
      ri += e - a;
    }
  }
}

// Source row (token) of gathered column c, or -1 for a padding column.
__device__ __forceinline__ int column_token(int c, const int* __restrict__ cp, const int* __restrict__ col0,
                                            const int* __restrict__ kr, int n_samples, int per, int n_tokens) {
  const int k0 = kr[0], k0p = round256(k0);
  int piece, local;
  if (c < k0p) {
    if (c >= k0) return -1;
    const int s = search_le(col0, n_samples, c);
    piece = s * per;
    local = c - col0[s];
  } else {
    const int r = c - k0p;
    if (r >= kr[1]) return -1;
    const int frames = per - 1;
    const int* col0_i = col0 + n_samples + 1;
    const int q = search_le(col0_i, n_samples * frames, r);
    piece = (q / frames) * per + 1 + q % frames;
    local = r - col0_i[q];
  }
  int a, e;
  piece_rows(cp, piece, n_tokens, a, e);
  return a + local;
}

struct TrArgs {
  const uint16_t* src[3];  // source rows [rows][seg]; feature f is column f % seg of src[f / seg]
  int seg, n_feat;
  int n_rows;              // plain transpose: source rows = destination columns
  uint16_t* dst;           // [n_feat][pitch]
  long long pitch;
  // gathered transpose
  const int* cp;
  const int* col0;
  const int* kr;
  int n_samples, per, n_tokens;
  float* part;  // [pitch / 64][n_feat] column sums of 64-column blocks, or nullptr
  // inverse rotation of sources 0 and 1 (dq, dk) on the way through, with
  // the rotated-back rows also written token-major to rot_out[0], rot_out[1]
  const int* pos;
  int nax, max_pos;
  const float2* tab;
  uint16_t* rot_out[2];
};

// dst[f][c] = src[row(c)][f] over one block of 64 columns x 64 features,
// staged through LDS; row(c) is c (plain) or the gathered column's token
// (zero for padding columns).  Optionally the sum of each feature over the
// block's 64 columns.
template <bool kGather, int kRotD>
__global__ __launch_bounds__(256) void transpose_kernel(TrArgs a) {
  __shared__ uint32_t tile[64][33];  // [column][feature pair], one dword of padding per row
  __shared__ int rows[64];
  const int t = threadIdx.x;
  const long long c0 = static_cast<long long>(blockIdx.x) * 64;
  long long n_cols;
  if constexpr (kGather) n_cols = min(static_cast<long long>(round256(a.kr[0])) + round256(a.kr[1]), a.pitch);
  else n_cols = a.n_rows;
  if (c0 >= n_cols) return;
  if (t < 64) {
    const long long c = c0 + t;
    int r = -1;
    if (c < n_cols) {
      if constexpr (kGather) r = column_token(static_cast<int>(c), a.cp, a.col0, a.kr, a.n_samples, a.per, a.n_tokens);
      else r = static_cast<int>(c);
    }
    rows[t] = r;
  }
  __syncthreads();
  const int chunk = t & 7;
  const int cc = t & 7;  // columns 8 cc .. 8 cc + 7
  constexpr int kTiles = tr_feat_tiles<kGather>();
  const int ft_end = min((blockIdx.y + 1) * kTiles, a.n_feat / 64);
  for (int ft = blockIdx.y * kTiles; ft < ft_end; ++ft) {
    const int f0 = ft * 64;
    const int si = f0 / a.seg;
    const uint16_t* src = a.src[si] + (f0 - si * a.seg);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = (t >> 3) + 32 * i;
      const int row = rows[r];
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row >= 0) {
        v = *reinterpret_cast<const u32x4*>(src + static_cast<size_t>(row) * a.seg + 8 * chunk);
        if constexpr (kRotD > 0) {
          if (si < 2) {  // dq or dk: back to the un-rotated projection's gradient
            const int c = f0 - si * a.seg + 8 * chunk;
            float x[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              x[2 * j] = bf16_bits_to_f32(static_cast<uint16_t>(v[j] & 0xffffu));
              x[2 * j + 1] = bf16_bits_to_f32(static_cast<uint16_t>(v[j] >> 16));
            }
            rotate_n<kRotD, 8>(x, c % kRotD, load_pos(a.pos, row, a.nax), a.tab, a.max_pos, -1.0f, a.nax);
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
            *reinterpret_cast<u32x4*>(a.rot_out[si] + static_cast<size_t>(row) * a.seg + c) = v;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) tile[r][4 * chunk + j] = v[j];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int f = (t >> 3) + 32 * i;
      float sum = 0.f;
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = (tile[8 * cc + 2 * j][f >> 1] >> (16 * (f & 1))) & 0xffffu;
        const uint32_t hi = (tile[8 * cc + 2 * j + 1][f >> 1] >> (16 * (f & 1))) & 0xffffu;
        w[j] = lo | (hi << 16);
        sum += bf16_bits_to_f32(static_cast<uint16_t>(lo));
        sum += bf16_bits_to_f32(static_cast<uint16_t>(hi));
      }
      if (c0 + 8 * cc < n_cols) {
        u32x4 o = {w[0], w[1], w[2], w[3]};
        *reinterpret_cast<u32x4*>(a.dst + static_cast<size_t>(f0 + f) * a.pitch + c0 + 8 * cc) = o;
      }
      if (a.part != nullptr) {
        sum += __shfl_xor(sum, 1, 64);
        sum += __shfl_xor(sum, 2, 64);
        sum += __shfl_xor(sum, 4, 64);
        if (cc == 0) a.part[static_cast<size_t>(blockIdx.x) * a.n_feat + f0 + f] = sum;
      }
    }
    __syncthreads();  // the tile is read before the next feature tile overwrites it
  }
}

// Rows of partial-sum block st (a quarter of projection tile st / 4):
// [r0, r1) in piece `piece`; false when the tile does not exist.
__device__ __forceinline__ bool sub_rows(const int* __restrict__ cp, const int* __restrict__ tstart, int n_pieces,
                                         int n_tokens, int st, int& piece, int& r0, int& r1) {
  const int mt = st / 4;
  if (mt >= tstart[n_pieces]) return false;
  piece = piece_of_tile(tstart, n_pieces, mt);
  int pa, pe;
  piece_rows(cp, piece, n_tokens, pa, pe);
  r0 = min(pa + (mt - tstart[piece]) * kPT + (st % 4) * kSub, pe);
  r1 = min(r0 + kSub, pe);
  return true;
}

// u = gate[s][m] dy and the partial sums of dy * proj (for dgate) over one
// block of 64 rows x 256 columns.  Wave w takes rows w, w + 4, ...; lane l
// columns 4 l .. 4 l + 3.
__global__ __launch_bounds__(256) void gate_bwd_kernel(const uint16_t* __restrict__ dy,
                                                       const uint16_t* __restrict__ proj,
                                                       const float* __restrict__ gate, const int* __restrict__ cp,
                                                       const int* __restrict__ tstart, int n_pieces, int per,
                                                       int n_tokens, int channels, uint16_t* __restrict__ u,
                                                       float* __restrict__ part) {
  __shared__ float4 red[4][64];
  const int st = blockIdx.x;
  int piece, r0, r1;
  if (!sub_rows(cp, tstart, n_pieces, n_tokens, st, piece, r0, r1)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = blockIdx.y * 256 + 4 * lane;
  const int g = (piece / per) * 2 + (piece % per == 0 ? 0 : 1);
  const float4 gv = *reinterpret_cast<const float4*>(gate + static_cast<size_t>(g) * channels + col);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int r = r0 + wave; r < r1; r += 4) {
    const size_t e = static_cast<size_t>(r) * channels + col;
    const u32x2 d = *reinterpret_cast<const u32x2*>(dy + e);
    const u32x2 p = *reinterpret_cast<const u32x2*>(proj + e);
    float dv[4], pv[4];
    dv[0] = bf16_bits_to_f32(static_cast<uint16_t>(d[0] & 0xffffu));
    dv[1] = bf16_bits_to_f32(static_cast<uint16_t>(d[0] >> 16));
    dv[2] = bf16_bits_to_f32(static_cast<uint16_t>(d[1] & 0xffffu));
    dv[3] = bf16_bits_to_f32(static_cast<uint16_t>(d[1] >> 16));
    pv[0] = bf16_bits_to_f32(static_cast<uint16_t>(p[0] & 0xffffu));
    pv[1] = bf16_bits_to_f32(static_cast<uint16_t>(p[0] >> 16));
    pv[2] = bf16_bits_to_f32(static_cast<uint16_t>(p[1] & 0xffffu));
    pv[3] = bf16_bits_to_f32(static_cast<uint16_t>(p[1] >> 16));
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += dv[j] * pv[j];
    store4<uint16_t>(u + e, gv.x * dv[0], gv.y * dv[1], gv.z * dv[2], gv.w * dv[3]);
  }
  red[wave][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  __syncthreads();
  if (wave == 0) {
    float4 s = red[0][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float4 o = red[w][lane];
      s.x += o.x;
      s.y += o.y;
      s.z += o.z;
      s.w += o.w;
    }
    *reinterpret_cast<float4*>(part + static_cast<size_t>(st) * channels + col) = s;
  }
}

// Index i with cp[i] <= row < cp[i + 1] among cp[0..m], or -1.
__device__ __forceinline__ int piece_of_row(const int* __restrict__ cp, int m, int row) {
  if (m <= 0 || row < cp[0] || row >= cp[m]) return -1;
  int lo = 0, hi = m;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cp[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

// adaLN backward, rows: one wave per token row, four rows per workgroup;
// lane l holds the 8-element chunks l, l + 64, ... of its row.  The row
// statistics are recomputed from x in the forward's order and saved
// (stats[row] = (mean, rstd)) for the column sums.  dh is read twice (the
// second time from cache): once for the row's two means, once for dx.
// (1 + scale) of the first row's (sample, modality) is staged in LDS.
// C = 512 cpl, cpl <= kMaxCpl.
template <int kMaxCpl>
__global__ __launch_bounds__(256) void adaln_bwd_rows_kernel(const uint16_t* __restrict__ dh,
                                                             const uint16_t* __restrict__ x,
                                                             const float* __restrict__ scale,
                                                             const uint16_t* __restrict__ dres,
                                                             const int* __restrict__ cp, int m, int per,
                                                             int n_tokens, int channels, float eps,
                                                             uint16_t* __restrict__ dx, float2* __restrict__ stats) {
  extern __shared__ float s1_lds[];  // [channels]: 1 + scale
  const int row0 = blockIdx.x * 4;
  const int row = row0 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int cpl = channels / 512;
  auto group_of = [&](int r) {
    const int i = piece_of_row(cp, m, r);
    return i < 0 ? -1 : (i / per) * 2 + (i % per == 0 ? 0 : 1);
  };
  const int g0 = group_of(row0);
  if (g0 >= 0) {
    const float* sc = scale + static_cast<size_t>(g0) * channels;
    for (int e = threadIdx.x * 4; e < channels; e += 256 * 4) {
      const float4 s4 = *reinterpret_cast<const float4*>(sc + e);
      *reinterpret_cast<float4*>(s1_lds + e) = make_float4(1.0f + s4.x, 1.0f + s4.y, 1.0f + s4.z, 1.0f + s4.w);
    }
  }
  __syncthreads();
  if (row >= n_tokens) return;
  const size_t rb = static_cast<size_t>(row) * channels;
  float v[kMaxCpl][8];
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxCpl; ++c)
    if (c < cpl) {
      load8<uint16_t>(x + rb + (c * 64 + lane) * 8, v[c]);
#pragma unroll
      for (int j = 0; j < 8; ++j) sum += v[c][j];
    }
  const float mean = wave_sum(sum) / static_cast<float>(channels);
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxCpl; ++c)
    if (c < cpl) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[c][j] -= mean;
        ss += v[c][j] * v[c][j];
      }
    }
  const float rstd = 1.0f / sqrtf(wave_sum(ss) / static_cast<float>(channels) + eps);
  const int g = group_of(row);  // wave-uniform
  // (1 + scale) for 8 elements from e
  auto mod8 = [&](int e, float (&s1)[8]) {
    if (g == g0 && g >= 0) {
      const float4* ls = reinterpret_cast<const float4*>(s1_lds + e);
      const float4 a = ls[0], b = ls[1];
      s1[0] = a.x; s1[1] = a.y; s1[2] = a.z; s1[3] = a.w;
      s1[4] = b.x; s1[5] = b.y; s1[6] = b.z; s1[7] = b.w;
    } else if (g >= 0) {
      const float* sc = scale + static_cast<size_t>(g) * channels + e;
      const float4 a = *reinterpret_cast<const float4*>(sc), b = *reinterpret_cast<const float4*>(sc + 4);
      s1[0] = 1.0f + a.x; s1[1] = 1.0f + a.y; s1[2] = 1.0f + a.z; s1[3] = 1.0f + a.w;
      s1[4] = 1.0f + b.x; s1[5] = 1.0f + b.y; s1[6] = 1.0f + b.z; s1[7] = 1.0f + b.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) s1[j] = 1.0f;
    }
  };
  float sa = 0.f, sb = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxCpl; ++c)
    if (c < cpl) {
      const int e = (c * 64 + lane) * 8;
      float d[8], s1[8];
      load8<uint16_t>(dh + rb + e, d);
      mod8(e, s1);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float gd = d[j] * s1[j];
        sa += gd;
        sb += gd * (v[c][j] * rstd);
      }
    }
  const float inv_c = 1.0f / static_cast<float>(channels);
  const float ma = wave_sum(sa) * inv_c, mb = wave_sum(sb) * inv_c;
#pragma unroll
  for (int c = 0; c < kMaxCpl; ++c)
    if (c < cpl) {
      const int e = (c * 64 + lane) * 8;
      float d[8], s1[8], o[8];
      load8<uint16_t>(dh + rb + e, d);
      mod8(e, s1);
      float r[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (dres != nullptr) load8<uint16_t>(dres + rb + e, r);
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = r[j] + rstd * (d[j] * s1[j] - ma - v[c][j] * rstd * mb);
      store8<uint16_t>(dx + rb + e, o);
    }
  if (lane == 0) stats[row] = make_float2(mean, rstd);
}

// adaLN backward, columns: partial sums of dh and dh xhat over one block of
// 64 rows x 256 columns (xhat from the saved row statistics): part[st][0][C],
// part[st][1][C].  Wave w takes rows w, w + 4, ...; lane l columns 4 l .. 4 l + 3.
__global__ __launch_bounds__(256) void adaln_bwd_cols_kernel(const uint16_t* __restrict__ dh,
                                                             const uint16_t* __restrict__ x,
                                                             const float2* __restrict__ stats,
                                                             const int* __restrict__ cp,
                                                             const int* __restrict__ tstart, int n_pieces,
                                                             int n_tokens, int channels, float* __restrict__ part) {
  __shared__ float4 red[2][4][64];
  const int st = blockIdx.x;
  int piece, r0, r1;
  if (!sub_rows(cp, tstart, n_pieces, n_tokens, st, piece, r0, r1)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = blockIdx.y * 256 + 4 * lane;
  float ps[4] = {0.f, 0.f, 0.f, 0.f}, pc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int r = r0 + wave; r < r1; r += 4) {
    const size_t e = static_cast<size_t>(r) * channels + col;
    const u32x2 d = *reinterpret_cast<const u32x2*>(dh + e);
    const u32x2 xv = *reinterpret_cast<const u32x2*>(x + e);
    const float2 mr = stats[r];
    float dv[4], xh[4];
    dv[0] = bf16_bits_to_f32(static_cast<uint16_t>(d[0] & 0xffffu));
    dv[1] = bf16_bits_to_f32(static_cast<uint16_t>(d[0] >> 16));
    dv[2] = bf16_bits_to_f32(static_cast<uint16_t>(d[1] & 0xffffu));
    dv[3] = bf16_bits_to_f32(static_cast<uint16_t>(d[1] >> 16));
    xh[0] = bf16_bits_to_f32(static_cast<uint16_t>(xv[0] & 0xffffu));
    xh[1] = bf16_bits_to_f32(static_cast<uint16_t>(xv[0] >> 16));
    xh[2] = bf16_bits_to_f32(static_cast<uint16_t>(xv[1] & 0xffffu));
    xh[3] = bf16_bits_to_f32(static_cast<uint16_t>(xv[1] >> 16));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ps[j] += dv[j];
      pc[j] += dv[j] * ((xh[j] - mr.x) * mr.y);
    }
  }
  red[0][wave][lane] = make_float4(ps[0], ps[1], ps[2], ps[3]);
  red[1][wave][lane] = make_float4(pc[0], pc[1], pc[2], pc[3]);
  __syncthreads();
  if (wave < 2) {  // wave 0: sums of dh, wave 1: sums of dh xhat
    float4 s = red[wave][0][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float4 o = red[wave][w][lane];
      s.x += o.x;
      s.y += o.y;
      s.z += o.z;
      s.w += o.w;
    }
    *reinterpret_cast<float4*>(part + (static_cast<size_t>(st) * 2 + wave) * channels + col) = s;
  }
}

// out[g][col] = sum over the partial-sum blocks of group g = (sample,
// modality); part rows have `stride` floats and the sums start at column
// `col_off`.  Groups without rows get zeros.  256 columns per workgroup: the
// four waves take every fourth block and their sums are added in wave order
// (a fixed order, so the result does not depend on timing).
__global__ __launch_bounds__(256) void group_sum_kernel(const float* __restrict__ part, long long stride,
                                                        int col_off, int ncol, const int* __restrict__ tstart,
                                                        int per, int part_rows, float* __restrict__ out) {
  __shared__ float4 red[4][64];
  const int g = blockIdx.x;
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int col = blockIdx.y * 256 + 4 * lane;
  const int s = g / 2, m = g % 2;
  const int p0 = s * per + m, p1 = m ? (s + 1) * per : s * per + 1;
  // blocks past the partial rows exist only for a malformed cu_pieces whose
  // overlapping pieces hold more tiles than the launch covered
  const int lo = min(4 * tstart[p0], part_rows), hi = min(4 * tstart[p1], part_rows);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (col < ncol) {
#pragma unroll 4
    for (int r = lo + q; r < hi; r += 4) {
      const float4 v = *reinterpret_cast<const float4*>(part + static_cast<size_t>(r) * stride + col_off + col);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
  }
  red[q][lane] = acc;
  __syncthreads();
  if (q == 0 && col < ncol) {
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float4 v = red[w][lane];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    *reinterpret_cast<float4*>(out + static_cast<size_t>(g) * ncol + col) = acc;
  }
}

// Modality m's gathered column range [lo, hi) (padded to 256), clamped to
// the cap columns the operands hold (a malformed cu_pieces with overlapping
// pieces can count more rows than the pack has).
__device__ __forceinline__ void modality_range(const int* __restrict__ kr, int m, int cap, int& lo, int& hi) {
  const int k0p = round256(kr[0]);
  lo = min(m ? k0p : 0, cap);
  hi = min(m ? k0p + round256(kr[1]) : k0p, cap);
}

// db_m[f] = sum of the 64-column block sums of modality m's columns.  64
// features per workgroup; the four waves take every fourth block, added in
// wave order.
__global__ __launch_bounds__(256) void bias_sum_kernel(const float* __restrict__ part, int n_feat,
                                                       const int* __restrict__ kr, int cap, float* __restrict__ db0,
                                                       float* __restrict__ db1) {
  __shared__ float red[4][64];
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int f = blockIdx.x * 64 + lane;
  const int m = blockIdx.y;
  float* out = m ? db1 : db0;
  if (out == nullptr) return;  // uniform over the workgroup
  int lo, hi;
  modality_range(kr, m, cap, lo, hi);
  float acc = 0.f;
  if (f < n_feat) {
#pragma unroll 8
    for (int b = lo / 64 + q; b < hi / 64; b += 4) acc += part[static_cast<size_t>(b) * n_feat + f];
  }
  red[q][lane] = acc;
  __syncthreads();
  if (q == 0 && f < n_feat) out[f] = ((acc + red[1][lane]) + red[2][lane]) + red[3][lane];
}

struct DgradArgs {
  const uint16_t* g[3];  // reduction columns [i kseg, (i + 1) kseg) come from g[i], rows [n_tokens][kseg]
  int kseg;
  const uint16_t* w0;    // transposed weights [n_out][k] per modality
  const uint16_t* w1;
  const int* cp;
  const int* tstart;
  int n_pieces, per, n_tokens, k, n_out, n_ntiles;
  uint16_t* out;  // [n_tokens][n_out]
};

// out = G W_m (G = [g0 | g1 | g2], W_m given transposed) over one 256-token x
// 256-feature tile of one piece; the forward's tile product and mapping.
__global__ __launch_bounds__(kPWaves * 64) void dgrad_kernel(DgradArgs a) {
  int mt, nt;
  window_tile(blockIdx.x, a.n_ntiles, mt, nt);
  if (mt >= a.tstart[a.n_pieces]) return;
  const int piece = piece_of_tile(a.tstart, a.n_pieces, mt);
  int pa, mend;
  piece_rows(a.cp, piece, a.n_tokens, pa, mend);
  const int m0 = pa + (mt - a.tstart[piece]) * kPT;
  if (m0 >= mend) return;
  const uint16_t* w = piece % a.per == 0 ? a.w0 : a.w1;
  const int n0 = nt * kFT;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const TileCopy256 copy_g(wave, lane, static_cast<unsigned>(a.kseg) * 2u);
  const TileCopy256 copy_w(wave, lane, static_cast<unsigned>(a.k) * 2u);
  auto load = [&](int ks, lds_char* tA, lds_char* tB) {
    const int kk = ks * kKS;  // a slice never straddles two sources (kseg is a multiple of 256)
    const uint16_t* src = kk < a.kseg ? a.g[0] + kk : kk < 2 * a.kseg ? a.g[1] + (kk - a.kseg)
                                                                     : a.g[2] + (kk - 2 * a.kseg);
    copy_g(src, m0, mend, tA);
    copy_w(w + kk, n0, a.n_out, tB);
  };
  f32x16 acc[kMB][4];
  zero_acc(acc);
  const int hh = lane >> 5, r32 = lane & 31;
  const int rbase = m0 + kWaveRows * wm;
  tile_gemm<2 * TileCopy256::kCopies>(a.k / kKS, wm, wn, lane, load, acc, [&](lds_char* sbuf) {
    const WaveStage st{sbuf};
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 v;
          v[0] = pack_bf16x2(acc[mb][nb][4 * g], acc[mb][nb][4 * g + 1]);
          v[1] = pack_bf16x2(acc[mb][nb][4 * g + 2], acc[mb][nb][4 * g + 3]);
          st.put(32 * mb + r32, 4 * nb + g, hh, v);
        }
    uint16_t* out = a.out + static_cast<size_t>(rbase) * a.n_out + n0 + 128 * wn;
    st.flush(lane, mend - rbase, [&](int row, int f, const u32x4& v) {
      *reinterpret_cast<u32x4*>(out + static_cast<size_t>(row) * a.n_out + f) = v;
    });
  });
}

// Token chunks of the weight gradient.  The `pairs` (chunk, modality) work
// items (at least 2) are shared between the modalities in proportion to their
// padded token counts, at least one each, and each modality's columns are cut
// into equal multiples of 256, so every chunk carries about the same work.  A
// modality with a single chunk has that chunk write dW itself (zeros when the
// modality has no tokens).  Item p's modality, chunk count and column range:
struct WgradChunk {
  int m, t, lo, hi;  // modality, chunks of that modality, columns [lo, hi)
  bool direct;       // the modality's only chunk: it writes dW itself
};

__device__ __forceinline__ WgradChunk wgrad_chunk(const int* __restrict__ kr, int cap, int pairs, int p) {
  const int k0 = min(round256(kr[0]), cap);
  const int k1 = min(round256(kr[1]), cap - k0);
  const int t0 = k0 + k1 == 0 ? 1
                 : min(max(static_cast<int>((static_cast<long long>(pairs) * k0 + (k0 + k1) / 2) / (k0 + k1)), 1),
                       pairs - 1);
  WgradChunk c;
  c.m = p < t0 ? 0 : 1;
  c.t = c.m ? pairs - t0 : t0;
  const int i = c.m ? p - t0 : p;
  const int s = c.m ? k0 : 0, k = c.m ? k1 : k0;
  const int len = round256((k + c.t - 1) / c.t);
  c.lo = min(s + i * len, s + k);
  c.hi = min(s + (i + 1) * len, s + k);
  c.direct = c.t == 1;
  return c;
}

struct WgradArgs {
  const uint16_t* a;  // [n_rows][pitch], gathered and transposed (the output gradient)
  const uint16_t* b;  // [n_cols][pitch] (the layer input)
  long long pitch;    // elements
  int n_rows, n_cols, n_ntiles, mtiles;
  const int* kr;
  int pairs;  // (chunk, modality) work items
  int group;  // consecutive (item, tile) pairs per XCD group: 32, or fewer when there are under 256
  float* out0;  // dW_text, dW_image [n_rows][n_cols]
  float* out1;
  float* part;  // [pairs][n_rows][n_cols]: chunk sums of modalities with several chunks
};

// Output tile t of a mtiles x n_ntiles grid in window-major order: windows of
// 8 row tiles x nw feature tiles (the last row of windows shorter when
// mtiles is not a multiple of 8), tiles column-major inside a window.
__device__ __forceinline__ void window_major_tile(int t, int mtiles, int n_ntiles, int& mt, int& nt) {
  const int nw = window_cols(n_ntiles), n_ntg = n_ntiles / nw;
  const int full = (mtiles / 8) * n_ntg;  // windows of 8 x nw tiles
  if (t < full * 8 * nw) {
    const int win = t / (8 * nw), pos = t % (8 * nw);
    mt = (win / n_ntg) * 8 + pos % 8;
    nt = (win % n_ntg) * nw + pos / 8;
  } else {
    const int rem = mtiles % 8, u = t - full * 8 * nw;
    const int win = u / (rem * nw), pos = u % (rem * nw);
    mt = (mtiles / 8) * 8 + pos % rem;
    nt = win * nw + pos / rem;
  }
}

// dW[j][i] = sum over one chunk of a modality's token columns k of
// A[j][k] B[i][k], one 256 x 256 output tile per workgroup.  The (item, tile)
// pairs are listed item by item, tiles window-major, and cut into groups of
// 32 (fewer when there are under 256, so all eight XCDs get work); group g
// runs on XCD g % 8 (blocks are dealt to the XCDs round-robin), so every XCD
// gets the same share of the work and each group's workgroups read about 12
// row slabs (one window) through that XCD's L2.
__global__ __launch_bounds__(kPWaves * 64) void wgrad_kernel(WgradArgs a) {
  const int b = blockIdx.x;
  const int x = b % kXcds, r = b / kXcds;
  const long long item = (static_cast<long long>(r / a.group) * kXcds + x) * a.group + r % a.group;
  const int tiles = a.mtiles * a.n_ntiles;
  if (item >= static_cast<long long>(tiles) * a.pairs) return;
  const int p = static_cast<int>(item / tiles);
  int mt, nt;
  window_major_tile(static_cast<int>(item % tiles), a.mtiles, a.n_ntiles, mt, nt);
  const WgradChunk ck = wgrad_chunk(a.kr, static_cast<int>(a.pitch), a.pairs, p);
  float* out = ck.direct ? (ck.m ? a.out1 : a.out0) : a.part + static_cast<size_t>(p) * a.n_rows * a.n_cols;
  const int m0 = mt * kPT, n0 = nt * kFT;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[kMB][4];
  zero_acc(acc);
  const int hh = lane >> 5, r32 = lane & 31;
  // An empty chunk writes zeros, so the reduction can add every chunk.  The
  // stores go through the wave's LDS buffer, half a block (32 rows) at a time.
  auto store_block = [&](lds_char* sbuf) {
    const WaveStageF32 st{sbuf};
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = {acc[mb][nb][4 * g], acc[mb][nb][4 * g + 1], acc[mb][nb][4 * g + 2], acc[mb][nb][4 * g + 3]};
          st.put(r32, 8 * nb + 2 * g + hh, v);
        }
      float* o = out + static_cast<size_t>(m0 + kWaveRows * wm + 32 * mb) * a.n_cols + n0 + 128 * wn;
      st.flush(lane, [&](int row, int f, const f32x4& v) {
        *reinterpret_cast<f32x4*>(o + static_cast<size_t>(row) * a.n_cols + f) = v;
      });
    }
  };
  if (ck.hi > ck.lo) {
    const TileCopy256 copy(wave, lane, static_cast<unsigned>(a.pitch) * 2u);
    const long long lo = ck.lo;
    auto load = [&](int ks, lds_char* tA, lds_char* tB) {
      const long long kk = lo + ks * kKS;
      copy(a.a + kk, m0, a.n_rows, tA);
      copy(a.b + kk, n0, a.n_cols, tB);
    };
    tile_gemm<2 * TileCopy256::kCopies>((ck.hi - ck.lo) / kKS, wm, wn, lane, load, acc, store_block);
  } else {
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int row = m0 + kWaveRows * wm + 32 * mb + r32;
          const int n = n0 + 128 * wn + 32 * nb + 8 * g + 4 * hh;
          store4<float>(out + static_cast<size_t>(row) * a.n_cols + n, 0.f, 0.f, 0.f, 0.f);
        }
  }
}

// dW_m = the sum of modality m's chunk sums in chunk order, for a modality
// with several chunks (one with a single chunk wrote dW_m itself).
__global__ __launch_bounds__(256) void split_sum_kernel(const float* __restrict__ part, long long n_elems,
                                                        const int* __restrict__ kr, int cap, int pairs,
                                                        float* __restrict__ out0, float* __restrict__ out1) {
  const long long e = (static_cast<long long>(blockIdx.x) * 256 + threadIdx.x) * 4;
  const int m = blockIdx.y;
  if (e >= n_elems) return;
  int first = -1, t = 0;
  for (int p = 0; p < pairs; ++p) {
    const WgradChunk ck = wgrad_chunk(kr, cap, pairs, p);
    if (ck.m == m) {
      if (first < 0) first = p;
      t = ck.t;
    }
  }
  if (t <= 1) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i = 0; i < t; ++i) {
    const float4 v = *reinterpret_cast<const float4*>(part + static_cast<size_t>(first + i) * n_elems + e);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  *reinterpret_cast<float4*>((m ? out1 : out0) + e) = acc;
}

}  // namespace

// ---------------------------------------------------------------------------
// Host launchers

int block_bwd_cols(int n_tokens) { return ((n_tokens + 255) / 256) * 256 + 256; }

// (chunk, modality) work items of a weight gradient [n_rows][n_cols].  In the
// usual pack one modality holds most tokens (image latents) and the other few
// (captions), so the items are taken as 1 + q: q equal chunks of the large
// modality plus one of the small.  q in [1, 7] minimises (rounds of
// one-workgroup-per-CU waves of tiles x q workgroups over the 256 CUs) / q,
// the time in units of one pass over the large modality's tokens, plus the
// extra traffic of the chunk sums written and read back when q > 1 (about 2 %
// of a pass per item at these tile sizes).  Tiny packs keep one chunk per
// modality.
int block_bwd_splits(int n_tokens, int n_rows, int n_cols) {
  const int tiles = (n_rows / kPT) * (n_cols / kFT);
  if (block_bwd_cols(n_tokens) < 4096) return 2;
  int best = 1;
  double best_cost = 1e30;
  for (int q = 1; q <= 7; ++q) {
    const long long rounds = (static_cast<long long>(tiles) * q + 255) / 256;
    const double cost = static_cast<double>(rounds) / q + (q > 1 ? 0.02 * (q + 1) : 0.0);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = q;
    }
  }
  return best + 1;
}

hipError_t launch_modality_cols(const int* cu_pieces, int n_samples, int frames, int n_tokens, int* col0, int* kr,
                                hipStream_t stream) {
  hipLaunchKernelGGL(modality_cols_kernel, dim3(1), dim3(1024), 0, stream, cu_pieces, n_samples, frames + 1,
                     n_tokens, col0, kr);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, int rows, int cols, void* dst, hipStream_t stream) {
  TrArgs a = {};
  a.src[0] = a.src[1] = a.src[2] = static_cast<const uint16_t*>(src);
  a.seg = cols;
  a.n_feat = cols;
  a.n_rows = rows;
  a.dst = static_cast<uint16_t*>(dst);
  a.pitch = rows;
  const dim3 grid(static_cast<unsigned>((rows + 63) / 64),
                  static_cast<unsigned>((cols / 64 + tr_feat_tiles<false>() - 1) / tr_feat_tiles<false>()));
  hipLaunchKernelGGL((transpose_kernel<false, 0>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gather_t(const void* const* src, int n_src, int seg, const int* cu_pieces, const int* col0,
                           const int* kr, int n_samples, int frames, int n_tokens, void* dst, long long pitch,
                           float* part, const GatherRotation* rot, hipStream_t stream) {
  TrArgs a = {};
  for (int i = 0; i < 3; ++i) a.src[i] = static_cast<const uint16_t*>(src[i < n_src ? i : 0]);
  a.seg = seg;
  a.n_feat = seg * n_src;
  a.dst = static_cast<uint16_t*>(dst);
  a.pitch = pitch;
  a.cp = cu_pieces;
  a.col0 = col0;
  a.kr = kr;
  a.n_samples = n_samples;
  a.per = frames + 1;
  a.n_tokens = n_tokens;
  a.part = part;
  const dim3 grid(static_cast<unsigned>(pitch / 64),
                  static_cast<unsigned>((a.n_feat / 64 + tr_feat_tiles<true>() - 1) / tr_feat_tiles<true>()));
  if (rot != nullptr) {
    a.pos = rot->pos;
    a.nax = rot->nax;
    a.max_pos = rot->max_pos;
    a.tab = rot->tab;
    a.rot_out[0] = static_cast<uint16_t*>(rot->out_q);
    a.rot_out[1] = static_cast<uint16_t*>(rot->out_k);
    if (rot->head_dim == 128)
      hipLaunchKernelGGL((transpose_kernel<true, 128>), grid, dim3(256), 0, stream, a);
    else if (rot->head_dim == 64)
      hipLaunchKernelGGL((transpose_kernel<true, 64>), grid, dim3(256), 0, stream, a);
    else
      return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL((transpose_kernel<true, 0>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_gate_bwd(const void* dy, const void* proj, const float* gate, const int* cu_pieces,
                           const int* tstart, int n_samples, int frames, int n_tokens, int channels, void* u,
                           float* part, hipStream_t stream) {
  const int n_pieces = (frames + 1) * n_samples;
  const dim3 grid(static_cast<unsigned>(4 * block_mtiles_bound(n_tokens, n_pieces)),
                  static_cast<unsigned>(channels / 256));
  hipLaunchKernelGGL(gate_bwd_kernel, grid, dim3(256), 0, stream, static_cast<const uint16_t*>(dy),
                     static_cast<const uint16_t*>(proj), gate, cu_pieces, tstart, n_pieces, frames + 1, n_tokens,
                     channels, static_cast<uint16_t*>(u), part);
  return hipGetLastError();
}

hipError_t launch_adaln_bwd(const void* dh, const void* x, const float* scale, const void* dres,
                            const int* cu_pieces, const int* tstart, int n_samples, int frames, int n_tokens,
                            int channels, float eps, void* dx, float2* stats, float* part, hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  if (channels > kAdaBwdMaxC) return hipErrorInvalidValue;
  const int per = frames + 1, n_pieces = per * n_samples;
  const dim3 grid(static_cast<unsigned>((n_tokens + 3) / 4));
  const size_t lds = static_cast<size_t>(channels) * sizeof(float);
  const uint16_t* dhs = static_cast<const uint16_t*>(dh);
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  const uint16_t* rs = static_cast<const uint16_t*>(dres);
  uint16_t* dxs = static_cast<uint16_t*>(dx);
  const int cpl = channels / 512;
  if (cpl <= 4)
    hipLaunchKernelGGL((adaln_bwd_rows_kernel<4>), grid, dim3(256), lds, stream, dhs, xs, scale, rs, cu_pieces,
                       n_pieces, per, n_tokens, channels, eps, dxs, stats);
  else if (cpl <= 6)
    hipLaunchKernelGGL((adaln_bwd_rows_kernel<6>), grid, dim3(256), lds, stream, dhs, xs, scale, rs, cu_pieces,
                       n_pieces, per, n_tokens, channels, eps, dxs, stats);
  else
    hipLaunchKernelGGL((adaln_bwd_rows_kernel<16>), grid, dim3(256), lds, stream, dhs, xs, scale, rs, cu_pieces,
                       n_pieces, per, n_tokens, channels, eps, dxs, stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 cgrid(static_cast<unsigned>(4 * block_mtiles_bound(n_tokens, n_pieces)),
                   static_cast<unsigned>(channels / 256));
  hipLaunchKernelGGL(adaln_bwd_cols_kernel, cgrid, dim3(256), 0, stream, dhs, xs, stats, cu_pieces, tstart, n_pieces,
                     n_tokens, channels, part);
  return hipGetLastError();
}

hipError_t launch_group_sum(const float* part, long long stride, int col_off, int ncol, const int* tstart,
                            int n_samples, int frames, int n_tokens, float* out, hipStream_t stream) {
  if (n_samples == 0) return hipSuccess;
  const int part_rows = 4 * block_mtiles_bound(n_tokens, (frames + 1) * n_samples);
  const dim3 grid(static_cast<unsigned>(2 * n_samples), static_cast<unsigned>((ncol + 255) / 256));
  hipLaunchKernelGGL(group_sum_kernel, grid, dim3(256), 0, stream, part, stride, col_off, ncol, tstart, frames + 1,
                     part_rows, out);
  return hipGetLastError();
}

hipError_t launch_bias_sum(const float* part, int n_feat, const int* kr, long long pitch, float* db0, float* db1,
                           hipStream_t stream) {
  if (db0 == nullptr && db1 == nullptr) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((n_feat + 63) / 64), 2);
  hipLaunchKernelGGL(bias_sum_kernel, grid, dim3(256), 0, stream, part, n_feat, kr, static_cast<int>(pitch), db0,
                     db1);
  return hipGetLastError();
}

hipError_t launch_dgrad(const void* const* g, int n_src, int kseg, const void* wt0, const void* wt1,
                        const int* cu_pieces, const int* tstart, int n_samples, int frames, int n_tokens, int n_out,
                        void* out, hipStream_t stream) {
  DgradArgs a = {};
  for (int i = 0; i < 3; ++i) a.g[i] = static_cast<const uint16_t*>(g[i < n_src ? i : 0]);
  a.kseg = kseg;
  a.w0 = static_cast<const uint16_t*>(wt0);
  a.w1 = static_cast<const uint16_t*>(wt1);
  a.cp = cu_pieces;
  a.tstart = tstart;
  a.per = frames + 1;
  a.n_pieces = a.per * n_samples;
  a.n_tokens = n_tokens;
  a.k = kseg * n_src;
  a.n_out = n_out;
  a.n_ntiles = n_out / kFT;
  a.out = static_cast<uint16_t*>(out);
  const long long blocks = window_blocks(block_mtiles_bound(n_tokens, a.n_pieces), a.n_ntiles);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(dgrad_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kPWaves * 64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_wgrad(const void* at, const void* bt, long long pitch, int n_rows, int n_cols, const int* kr,
                        int pairs, float* part, float* dw0, float* dw1, hipStream_t stream) {
  WgradArgs a = {};
  a.a = static_cast<const uint16_t*>(at);
  a.b = static_cast<const uint16_t*>(bt);
  a.pitch = pitch;
  a.n_rows = n_rows;
  a.n_cols = n_cols;
  a.n_ntiles = n_cols / kFT;
  a.mtiles = n_rows / kPT;
  a.kr = kr;
  a.pairs = pairs;
  a.out0 = dw0;
  a.out1 = dw1;
  a.part = part;
  const long long items = static_cast<long long>(a.mtiles) * a.n_ntiles * pairs;
  a.group = items >= 32 * kXcds ? 32 : static_cast<int>((items + kXcds - 1) / kXcds);
  const long long groups = (items + a.group - 1) / a.group;
  const long long blocks = (groups + kXcds - 1) / kXcds * kXcds * a.group;
  if (blocks > 0x7fffffffLL || pairs < 2) return hipErrorInvalidValue;
  hipLaunchKernelGGL(wgrad_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kPWaves * 64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_split_sum(const float* part, long long pitch, int n_rows, int n_cols, const int* kr, int pairs,
                            float* dw0, float* dw1, hipStream_t stream) {
  if (pairs <= 2) return hipSuccess;  // one chunk per modality
  const long long n_elems = static_cast<long long>(n_rows) * n_cols;
  const dim3 grid(static_cast<unsigned>((n_elems / 4 + 255) / 256), 2);
  hipLaunchKernelGGL(split_sum_kernel, grid, dim3(256), 0, stream, part, n_elems, kr, static_cast<int>(pitch), pairs,
                     dw0, dw1);
  return hipGetLastError();
}

}  // namespace mf

// The attention sub-block's fused chains around the packed joint attention:
// adaptive normalisation, the modality-specific QKV projection with the
// rotary embedding in its epilogue, and the output projection with the gated
// residual update in its epilogue.
//
// The backbone follows MMDiT -- joint self-attention over the concatenated
// text and image tokens with normalisation and projection layers specific to
// each modality (Mage-Flow paper section 3.2.1 "Model Architecture and Native
// Packing", paperlayer.ai summary; ai.thesatyajit.com explainer, Figure 5
// caption) -- and its training system fuses the transformer blocks' memory-
// bound chains of adaptive normalisation, rotary embeddings and gated
// residual updates (paper section 3.3 "Training Infrastructure").
//
// Rows are tokens in packed order, [N][C] with C = H D.  A token's sample and
// modality come from cu_pieces (frames + 1 pieces per sample; the first piece
// of a sample is its text, the others image grids).
//   adaln:  h = LN(x) (1 + scale[s][m]) + shift[s][m], LayerNorm without
//           affine, population variance, fp32 statistics.
//   qkv:    [q | k | v] = h W_m^T + b_m; q and k rotated by the token's
//           position, written [N][H][D] (the attention then needs no rotation).
//   out:    y = x + gate[s][m] (o W_o,m^T + b_o,m).
// The projections tile the token rows per piece, so a tile never mixes
// modalities and takes one weight matrix.
#include "block_gemm.h"
#include "mf_device.h"
#include "block_kernels.h"
#include "mf_kernels.h"

namespace mf {

namespace {

// tstart[p] = sum over pieces q < p of ceil(len_q / kPT); tstart[m] = total.
__global__ __launch_bounds__(1024) void piece_tiles_kernel(const int* __restrict__ cp, int m, int n_tokens,
                                                           int* __restrict__ tstart) {
  __shared__ int part[1024];
  const int t = threadIdx.x;
  const int per = (m + 1023) / 1024;
  const int a = min(t * per, m), b = min(a + per, m);
  int sum = 0;
  for (int i = a; i < b; ++i) {
    int r0, r1;
    piece_rows(cp, i, n_tokens, r0, r1);
    sum += (r1 - r0 + kPT - 1) / kPT;
  }
  part[t] = sum;
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int i = 0; i < 1024; ++i) {
      const int v = part[i];
      part[i] = run;
      run += v;
    }
    tstart[m] = run;
  }
  __syncthreads();
  int run = part[t];
  for (int i = a; i < b; ++i) {
    int r0, r1;
    piece_rows(cp, i, n_tokens, r0, r1);
    tstart[i] = run;
    run += (r1 - r0 + kPT - 1) / kPT;
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

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// One wave per token row, four rows per workgroup; lane l holds the 8-element
// chunks l, l + 64, ... of its row (coalesced 1 KB per load across the wave).
// The (1 + scale, shift) vectors of the first row's (sample, modality) are
// staged in LDS once per workgroup; a row of another piece (rows are in
// packed order, so rarely) reads its own from global memory.  C = 512 cpl,
// cpl <= kMaxCpl.
constexpr int kAdaMaxC = 8192;
template <int kMaxCpl>
__global__ __launch_bounds__(256) void adaln_kernel(const uint16_t* __restrict__ x, const float* __restrict__ shift,
                                                    const float* __restrict__ scale, const int* __restrict__ cp,
                                                    int m, int per, int n_tokens, int channels, float eps,
                                                    uint16_t* __restrict__ h) {
  extern __shared__ float mod_lds[];  // [2][channels]: 1 + scale, shift
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
    const float* sh = shift + static_cast<size_t>(g0) * channels;
    for (int e = threadIdx.x * 4; e < channels; e += 256 * 4) {
      const float4 s4 = *reinterpret_cast<const float4*>(sc + e);
      const float4 b4 = *reinterpret_cast<const float4*>(sh + e);
      *reinterpret_cast<float4*>(mod_lds + e) = make_float4(1.0f + s4.x, 1.0f + s4.y, 1.0f + s4.z, 1.0f + s4.w);
      *reinterpret_cast<float4*>(mod_lds + channels + e) = b4;
    }
  }
  __syncthreads();
  if (row >= n_tokens) return;
  const uint16_t* xr = x + static_cast<size_t>(row) * channels;
  float v[kMaxCpl][8];
  float sum = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxCpl; ++c)
    if (c < cpl) {
      load8<uint16_t>(xr + (c * 64 + lane) * 8, v[c]);
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
  uint16_t* hr = h + static_cast<size_t>(row) * channels;
#pragma unroll
  for (int c = 0; c < kMaxCpl; ++c)
    if (c < cpl) {
      const int e = (c * 64 + lane) * 8;
      float s1[8], b[8];
      if (g == g0 && g >= 0) {
        const float4* ls = reinterpret_cast<const float4*>(mod_lds + e);
        const float4* lb = reinterpret_cast<const float4*>(mod_lds + channels + e);
        const float4 s0 = ls[0], s4 = ls[1], b0 = lb[0], b4 = lb[1];
        const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s4.x, s4.y, s4.z, s4.w};
        const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          s1[j] = sv[j];
          b[j] = bv[j];
        }
      } else if (g >= 0) {
        const float* sc = scale + static_cast<size_t>(g) * channels + e;
        const float* sh = shift + static_cast<size_t>(g) * channels + e;
        const float4 s0 = *reinterpret_cast<const float4*>(sc), s4 = *reinterpret_cast<const float4*>(sc + 4);
        const float4 b0 = *reinterpret_cast<const float4*>(sh), b4 = *reinterpret_cast<const float4*>(sh + 4);
        const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s4.x, s4.y, s4.z, s4.w};
        const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          s1[j] = 1.0f + sv[j];
          b[j] = bv[j];
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          s1[j] = 1.0f;
          b[j] = 0.0f;
        }
      }
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = v[c][j] * rstd * s1[j] + b[j];
      store8<uint16_t>(hr + e, o);
    }
}

struct ProjArgs {
  const uint16_t* act;  // [n_tokens][k]
  const uint16_t* w0;   // text weights [n_out][k]
  const uint16_t* w1;   // image weights
  const float* b0;      // text bias [n_out] or nullptr
  const float* b1;      // image bias
  const int* cp;        // cu_pieces
  const int* tstart;    // first tile of each piece; tstart[n_pieces] = tiles
  int n_pieces, per, n_tokens, k, n_out, n_ntiles;
  // qkv epilogue
  uint16_t* q;
  uint16_t* kk;
  uint16_t* v;
  const int* pos;  // [n_tokens][nax] or nullptr
  int nax;
  const float2* tab;
  int max_pos;
  // gated-residual epilogue
  const uint16_t* x;
  const float* gate;  // [S][2][n_out]
  uint16_t* y;
  uint16_t* proj;  // o W^T + b before the gate, for the backward; or nullptr
};

enum { kEpiQkvRope = 0, kEpiGatedResidual = 1 };

// out = act W^T (+ b) over one 256-token x 256-feature tile.  MFMA A operand
// = weight rows (features), B operand = token rows, so the accumulator holds
// the transposed tile: lane element e of block (mb, nb) is feature
// 32 nb + 8 (e/4) + 4 (lane/32) + e%4 of token 32 mb + lane%32 -- four
// consecutive features per lane group, the rotary pairs inside one lane.
template <int D, int kEpi>
__global__ __launch_bounds__(kPWaves * 64) void proj_kernel(ProjArgs a) {
  const int b = blockIdx.x;
  int mt, nt;
  window_tile(b, a.n_ntiles, mt, nt);
  const int total = a.tstart[a.n_pieces];
  if (mt >= total) return;
  const int piece = piece_of_tile(a.tstart, a.n_pieces, mt);
  int pa, mend;
  piece_rows(a.cp, piece, a.n_tokens, pa, mend);
  const int m0 = pa + (mt - a.tstart[piece]) * kPT;
  if (m0 >= mend) return;
  const int modality = piece % a.per == 0 ? 0 : 1;
  const int sample = piece / a.per;
  const uint16_t* w = modality ? a.w1 : a.w0;
  const float* bias = modality ? a.b1 : a.b0;
  const int n0 = nt * kFT;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5;
  const int r32 = lane & 31;
  const int wm = wave >> 1;  // token rows kWaveRows wm .. + kWaveRows
  const int wn = wave & 1;   // features 128 wn .. + 128

  const TileCopy256 copy(wave, lane, static_cast<unsigned>(a.k) * 2u);
  auto load = [&](int ks, lds_char* tA, lds_char* tB) {
    copy(a.act + ks * kKS, m0, mend, tA);
    copy(w + ks * kKS, n0, a.n_out, tB);
  };
  f32x16 acc[kMB][4];
  zero_acc(acc);
  const int C = a.n_out / (kEpi == kEpiQkvRope ? 3 : 1);
  const int part = kEpi == kEpiQkvRope ? n0 / C : 0;  // q, k or v (a tile never straddles two)
  uint16_t* out = kEpi == kEpiQkvRope ? (part == 0 ? a.q : part == 1 ? a.kk : a.v) : a.y;
  const bool rotate = kEpi == kEpiQkvRope && part < 2 && a.pos != nullptr;
  const float* gate = nullptr;
  if constexpr (kEpi == kEpiGatedResidual) gate = a.gate + (static_cast<size_t>(sample) * 2 + modality) * C;
  const int rbase = m0 + kWaveRows * wm;
  const int cbase = n0 + 128 * wn - part * C;  // first output column of the wave's block
  // k is a multiple of 256, so the slice count a multiple of 8
  tile_gemm<2 * TileCopy256::kCopies>(a.k / kKS, wm, wn, lane, load, acc, [&](lds_char* sbuf) {
    const WaveStage st{sbuf};
    const int rows = mend - rbase;
    auto flush_to = [&](uint16_t* dst) {
      uint16_t* o = dst + static_cast<size_t>(rbase) * C + cbase;
      st.flush(lane, rows, [&](int row, int f, const u32x4& v) {
        *reinterpret_cast<u32x4*>(o + static_cast<size_t>(row) * C + f) = v;
      });
    };
    // the lane's 4 consecutive features of block (nb, g) plus the bias
    auto proj4 = [&](int mb, int nb, int g, float (&xv)[4]) {
      const int n = n0 + 128 * wn + 32 * nb + 8 * g + 4 * hh;
      float4 b4 = make_float4(0.f, 0.f, 0.f, 0.f);
      if (bias != nullptr) b4 = *reinterpret_cast<const float4*>(bias + n);
      xv[0] = acc[mb][nb][4 * g] + b4.x;
      xv[1] = acc[mb][nb][4 * g + 1] + b4.y;
      xv[2] = acc[mb][nb][4 * g + 2] + b4.z;
      xv[3] = acc[mb][nb][4 * g + 3] + b4.w;
    };
    auto put4 = [&](int mb, int nb, int g, const float (&xv)[4]) {
      u32x2 v;
      v[0] = pack_bf16x2(xv[0], xv[1]);
      v[1] = pack_bf16x2(xv[2], xv[3]);
      st.put(32 * mb + r32, 4 * nb + g, hh, v);
    };
    if constexpr (kEpi == kEpiQkvRope) {
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) {
        const int tok = rbase + 32 * mb + r32;
        Pos3 p = {0, 0, 0};
        if (rotate && tok < mend) p = load_pos(a.pos, tok, a.nax);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float xv[4];
            proj4(mb, nb, g, xv);
            if (rotate) rotate_n<D, 4>(xv, (n0 + 128 * wn + 32 * nb + 8 * g + 4 * hh - part * C) % D, p, a.tab,
                                       a.max_pos, 1.0f, a.nax);
            put4(mb, nb, g, xv);
          }
      }
      flush_to(out);
    } else {
      if (a.proj != nullptr) {  // the pre-gate projection, for the backward
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              float xv[4];
              proj4(mb, nb, g, xv);
              put4(mb, nb, g, xv);
            }
        flush_to(a.proj);
      }
      // y = x + gate (o W^T + b): the residual rows come in whole through the
      // staging buffer, and y goes back out the same way
      const uint16_t* xb = a.x + static_cast<size_t>(rbase) * C + cbase;
      st.fill(lane, rows, [&](int row) { return xb + static_cast<size_t>(row) * C; });
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float xv[4];
            proj4(mb, nb, g, xv);
            const float4 gv = *reinterpret_cast<const float4*>(gate + n0 + 128 * wn + 32 * nb + 8 * g + 4 * hh);
            const u32x2 raw = st.get(32 * mb + r32, 4 * nb + g, hh);
            xv[0] = bf16_bits_to_f32(static_cast<uint16_t>(raw[0] & 0xffffu)) + gv.x * xv[0];
            xv[1] = bf16_bits_to_f32(static_cast<uint16_t>(raw[0] >> 16)) + gv.y * xv[1];
            xv[2] = bf16_bits_to_f32(static_cast<uint16_t>(raw[1] & 0xffffu)) + gv.z * xv[2];
            xv[3] = bf16_bits_to_f32(static_cast<uint16_t>(raw[1] >> 16)) + gv.w * xv[3];
            put4(mb, nb, g, xv);
          }
      flush_to(out);
    }
  });
}

template <int D, int kEpi>
hipError_t launch_proj_t(const ProjArgs& a, int mtiles_max, hipStream_t stream) {
  const long long blocks = window_blocks(mtiles_max, a.n_ntiles);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((proj_kernel<D, kEpi>), dim3(static_cast<unsigned>(blocks)), dim3(kPWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int block_mtiles_bound(int n_tokens, int n_pieces) { return (n_tokens + kPT - 1) / kPT + n_pieces; }

int block_tile_rows() { return kPT; }

hipError_t launch_piece_tiles(const int* cu_pieces, int n_pieces, int n_tokens, int* tstart, hipStream_t stream) {
  hipLaunchKernelGGL(piece_tiles_kernel, dim3(1), dim3(1024), 0, stream, cu_pieces, n_pieces, n_tokens, tstart);
  return hipGetLastError();
}

hipError_t launch_adaln(const void* x, const float* shift, const float* scale, const int* cu_pieces, int n_samples,
                        int frames, int n_tokens, int channels, float eps, void* h, hipStream_t stream) {
  if (n_tokens == 0) return hipSuccess;
  if (channels > kAdaMaxC) return hipErrorInvalidValue;
  const int per = frames + 1;
  const dim3 grid(static_cast<unsigned>((n_tokens + 3) / 4));
  const size_t lds = 2 * static_cast<size_t>(channels) * sizeof(float);
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  uint16_t* hs = static_cast<uint16_t*>(h);
  const int cpl = channels / 512;
  if (cpl <= 4)
    hipLaunchKernelGGL((adaln_kernel<4>), grid, dim3(256), lds, stream, xs, shift, scale, cu_pieces,
                       per * n_samples, per, n_tokens, channels, eps, hs);
  else if (cpl <= 6)
    hipLaunchKernelGGL((adaln_kernel<6>), grid, dim3(256), lds, stream, xs, shift, scale, cu_pieces,
                       per * n_samples, per, n_tokens, channels, eps, hs);
  else
    hipLaunchKernelGGL((adaln_kernel<16>), grid, dim3(256), lds, stream, xs, shift, scale, cu_pieces,
                       per * n_samples, per, n_tokens, channels, eps, hs);
  return hipGetLastError();
}

hipError_t launch_qkv_rope(const void* h, const void* w_text, const void* w_image, const float* b_text,
                           const float* b_image, const int* cu_pieces, const int* tstart, int n_samples, int frames,
                           int n_tokens, int n_heads, int head_dim, const int* pos, int nax, const float2* tab,
                           int max_pos, void* q, void* k, void* v, hipStream_t stream) {
  ProjArgs a = {};
  const int c = n_heads * head_dim;
  a.act = static_cast<const uint16_t*>(h);
  a.w0 = static_cast<const uint16_t*>(w_text);
  a.w1 = static_cast<const uint16_t*>(w_image);
  a.b0 = b_text;
  a.b1 = b_image;
  a.cp = cu_pieces;
  a.tstart = tstart;
  a.per = frames + 1;
  a.n_pieces = a.per * n_samples;
  a.n_tokens = n_tokens;
  a.k = c;
  a.n_out = 3 * c;
  a.n_ntiles = 3 * c / kFT;
  a.q = static_cast<uint16_t*>(q);
  a.kk = static_cast<uint16_t*>(k);
  a.v = static_cast<uint16_t*>(v);
  a.pos = pos;
  a.nax = nax;
  a.tab = tab;
  a.max_pos = max_pos;
  const int mt = block_mtiles_bound(n_tokens, a.n_pieces);
  return head_dim == 128 ? launch_proj_t<128, kEpiQkvRope>(a, mt, stream)
                         : launch_proj_t<64, kEpiQkvRope>(a, mt, stream);
}

hipError_t launch_out_gated(const void* o, const void* x, const void* w_text, const void* w_image,
                            const float* b_text, const float* b_image, const float* gate, const int* cu_pieces,
                            const int* tstart, int n_samples, int frames, int n_tokens, int channels, void* y,
                            void* proj, hipStream_t stream) {
  ProjArgs a = {};
  a.act = static_cast<const uint16_t*>(o);
  a.w0 = static_cast<const uint16_t*>(w_text);
  a.w1 = static_cast<const uint16_t*>(w_image);
  a.b0 = b_text;
  a.b1 = b_image;
  a.cp = cu_pieces;
  a.tstart = tstart;
  a.per = frames + 1;
  a.n_pieces = a.per * n_samples;
  a.n_tokens = n_tokens;
  a.k = channels;
  a.n_out = channels;
  a.n_ntiles = channels / kFT;
  a.x = static_cast<const uint16_t*>(x);
  a.gate = gate;
  a.y = static_cast<uint16_t*>(y);
  a.proj = static_cast<uint16_t*>(proj);
  return launch_proj_t<128, kEpiGatedResidual>(a, block_mtiles_bound(n_tokens, a.n_pieces), stream);
}

}  // namespace mf

// Backward of packed block-diagonal attention with axial 2D RoPE.
//
// With P = softmax(scale * Qr Kr^T) recomputed from the forward's LSE:
//   Delta = rowsum(dO * O)                       delta kernel (HBM-bound)
//   dV = P^T dO,  dKr = scale * dS^T Qr          dkdv kernel, per 32 keys/wave
//   dQr = scale * dS Kr                          dq kernel,   per 32 queries/wave
// where dS = P * (dO V^T - Delta); dQ and dK are rotated back by the inverse
// rotation in the epilogues.  Each output element is written by exactly one
// lane and summed in a fixed order: results are deterministic (no atomics).
#include "mf_device.h"
#include "mf_kernels.h"

namespace mf {

namespace {

constexpr int kKB = kDkdvTile;  // keys per dkdv workgroup (32 per wave)
constexpr int kQB = 32;         // queries per dkdv LDS tile
constexpr int kQT = kDqTile;    // queries per dq workgroup (32 per wave)
constexpr int kKT = 64;         // keys per dq LDS tile
static_assert(kKB == kQT, "dkdv and dq share one schedule");

// Rotate 4 consecutive elements (two pairs) starting at d0 (multiple of 4).
template <int D>
__device__ __forceinline__ void rotate4(float (&x)[4], int d0, int prow, int pcol, const float2* __restrict__ tab,
                                        int max_pos, float sign) {
  const int half = d0 / (D / 2);
  int p = half ? pcol : prow;
  p = p < 0 ? 0 : (p >= max_pos ? max_pos - 1 : p);
  const int j0 = (d0 % (D / 2)) / 2;
  const float2* t = tab + static_cast<size_t>(p) * (D / 4) + j0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float2 cs = t[j];
    const float s = sign * cs.y;
    const float a = x[2 * j];
    const float b = x[2 * j + 1];
    x[2 * j] = a * cs.x - b * s;
    x[2 * j + 1] = a * s + b * cs.x;
  }
}

template <int D, typename T>
__global__ __launch_bounds__(256) void delta_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                    float* __restrict__ delta, int n_tokens, int heads) {
  constexpr int kLanesPerRow = D / 8;
  const long long rows = static_cast<long long>(n_tokens) * heads;
  const long long gid = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const long long row = gid / kLanesPerRow;
  const int sub = static_cast<int>(gid % kLanesPerRow);
  float acc = 0.f;
  if (row < rows) {
    float a[8], b[8];
    load8<T>(o + row * D + sub * 8, a);
    load8<T>(dout + row * D + sub * 8, b);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += a[j] * b[j];
  }
#pragma unroll
  for (int m = kLanesPerRow / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && sub == 0) {
    const long long t = row / heads;
    const int h = static_cast<int>(row % heads);
    delta[static_cast<size_t>(h) * n_tokens + t] = acc;
  }
}

template <int D, typename TOut>
__global__ __launch_bounds__(256, 2) void dkdv_kernel(
    const uint16_t* __restrict__ qr, const uint16_t* __restrict__ kr, const uint16_t* __restrict__ vb,
    const uint16_t* __restrict__ dob, const float* __restrict__ lse, const float* __restrict__ delta,
    TOut* __restrict__ dk, TOut* __restrict__ dv, const int* __restrict__ cu, const int* __restrict__ order,
    const int* __restrict__ pt, int n_seg, int n_tokens, int heads, const int2* __restrict__ pos,
    const float2* __restrict__ tab, int max_pos, float scale, float scale_log2) {
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CH = D / 8;
  constexpr int kTileBytes = kQB * D * 2;
  constexpr int kLoads = kQB * CH / 256;  // chunks per thread per tensor per tile
  __shared__ __attribute__((aligned(16))) char smem[4 * kTileBytes];  // [buf][Q, dO]
  __shared__ float sL[2][kQB];
  __shared__ float sD[2][kQB];

  WorkItem it;
  if (!decode_item(blockIdx.x, heads, n_seg, order, pt, it)) return;
  const int head = it.head;
  int s0, s1;
  seg_bounds(cu, it.seg, n_tokens, s0, s1);
  const int L = s1 - s0;
  const int kbase = it.tile * kKB;
  if (kbase >= L) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hh = lane >> 5;
  const int key = kbase + wave * 32 + (lane & 31);
  const bool kok = key < L;
  const long long krow = (static_cast<long long>(s0) + min(key, L - 1)) * heads + head;

  // K and V fragments (B operands of S = Q Kr^T and dP = dO V^T).
  bf16x8 kf[NKK], vf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int e0 = 16 * kk + 8 * hh;
    kf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kr + krow * D + e0));
    vf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vb + krow * D + e0));
  }

  u32x4 qreg[kLoads], oreg[kLoads];
  float lreg = 0.f, dreg = 0.f;
  auto gload = [&](int q0) {
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int ci = threadIdx.x + 256 * r;
      const int qq = min(q0 + ci / CH, L - 1);
      const size_t g = (static_cast<size_t>(s0 + qq) * heads + head) * D + (ci % CH) * 8;
      qreg[r] = *reinterpret_cast<const u32x4*>(qr + g);
      oreg[r] = *reinterpret_cast<const u32x4*>(dob + g);
    }
    if (threadIdx.x < kQB) {
      const int qq = q0 + threadIdx.x;
      const bool ok = qq < L;
      const size_t g = static_cast<size_t>(head) * n_tokens + s0 + min(qq, L - 1);
      lreg = ok ? lse[g] * kLog2e : INFINITY;  // rows past the end get P = 0
      dreg = ok ? delta[g] : 0.f;
    }
  };
  lds_char* const sbase = (lds_char*)(smem);
  auto lstore = [&](int buf) {
    lds_char* sQ = sbase + buf * 2 * kTileBytes;
    lds_char* sO = sQ + kTileBytes;
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int ci = threadIdx.x + 256 * r;
      const int off = Tile<D>::off(ci / CH, ci % CH);
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(sQ + off) = qreg[r];
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(sO + off) = oreg[r];
    }
    if (threadIdx.x < kQB) {
      sL[buf][threadIdx.x] = lreg;
      sD[buf][threadIdx.x] = dreg;
    }
  };

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dkacc[db][i] = 0.f;
      dvacc[db][i] = 0.f;
    }

  const int ntiles = (L + kQB - 1) / kQB;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    const bool more = j + 1 < ntiles;
    if (more) gload((j + 1) * kQB);
    const int buf = j & 1;
    const lds_char* sQ = sbase + buf * 2 * kTileBytes;
    const lds_char* sO = sQ + kTileBytes;

    f32x16 sacc, dpacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sacc[i] = 0.f;
      dpacc[i] = 0.f;
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      sacc = mfma32(lds_row_frag<D>(sQ, 0, kk, lane), kf[kk], sacc);
      dpacc = mfma32(lds_row_frag<D>(sO, 0, kk, lane), vf[kk], dpacc);
    }
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int qq = acc_row(i, hh);
      const float p = fast_exp2(__builtin_fmaf(sacc[i], scale_log2, -sL[buf][qq]));
      const float ds = p * (dpacc[i] - sD[buf][qq]);
      pb[i >> 3][i & 7] = static_cast<__bf16>(p);
      dsb[i >> 3][i & 7] = static_cast<__bf16>(ds);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dvacc[db] = mfma32(lds_col_frag<D>(sO, 16 * c, 32 * db, lane), pb[c], dvacc[db]);
        dkacc[db] = mfma32(lds_col_frag<D>(sQ, 16 * c, 32 * db, lane), dsb[c], dkacc[db]);
      }
    if (more) lstore(buf ^ 1);
    __syncthreads();
  }

  if (kok) {
    int2 kp = make_int2(0, 0);
    if (pos != nullptr) kp = pos[s0 + key];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * hh;
        float x[4] = {dkacc[db][4 * g4] * scale, dkacc[db][4 * g4 + 1] * scale, dkacc[db][4 * g4 + 2] * scale,
                      dkacc[db][4 * g4 + 3] * scale};
        if (pos != nullptr) rotate4<D>(x, d0, kp.x, kp.y, tab, max_pos, -1.0f);
        store4<TOut>(dk + krow * D + d0, x[0], x[1], x[2], x[3]);
        store4<TOut>(dv + krow * D + d0, dvacc[db][4 * g4], dvacc[db][4 * g4 + 1], dvacc[db][4 * g4 + 2],
                     dvacc[db][4 * g4 + 3]);
      }
  }
}

template <int D, typename TOut>
__global__ __launch_bounds__(256, 2) void dq_kernel(
    const uint16_t* __restrict__ qr, const uint16_t* __restrict__ kr, const uint16_t* __restrict__ vb,
    const uint16_t* __restrict__ dob, const float* __restrict__ lse, const float* __restrict__ delta,
    TOut* __restrict__ dq, const int* __restrict__ cu, const int* __restrict__ order, const int* __restrict__ pt,
    int n_seg, int n_tokens, int heads, const int2* __restrict__ pos, const float2* __restrict__ tab, int max_pos,
    float scale, float scale_log2) {
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CH = D / 8;
  constexpr int kTileBytes = kKT * D * 2;
  constexpr int kLoads = kKT * CH / 256;
  __shared__ __attribute__((aligned(16))) char smem[4 * kTileBytes];  // [buf][K, V]

  WorkItem it;
  if (!decode_item(blockIdx.x, heads, n_seg, order, pt, it)) return;
  const int head = it.head;
  int s0, s1;
  seg_bounds(cu, it.seg, n_tokens, s0, s1);
  const int L = s1 - s0;
  const int qbase = it.tile * kQT;
  if (qbase >= L) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hh = lane >> 5;
  const int qi = qbase + wave * 32 + (lane & 31);
  const bool qok = qi < L;
  const long long qrow = (static_cast<long long>(s0) + min(qi, L - 1)) * heads + head;

  bf16x8 qf[NKK], df[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int e0 = 16 * kk + 8 * hh;
    qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qr + qrow * D + e0));
    df[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(dob + qrow * D + e0));
  }
  const float lse2 = qok ? lse[static_cast<size_t>(head) * n_tokens + s0 + qi] * kLog2e : INFINITY;
  const float dl = qok ? delta[static_cast<size_t>(head) * n_tokens + s0 + qi] : 0.f;

  u32x4 kreg[kLoads], vreg[kLoads];
  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int ci = threadIdx.x + 256 * r;
      const int kq = min(k0 + ci / CH, L - 1);
      const size_t g = (static_cast<size_t>(s0 + kq) * heads + head) * D + (ci % CH) * 8;
      kreg[r] = *reinterpret_cast<const u32x4*>(kr + g);
      vreg[r] = *reinterpret_cast<const u32x4*>(vb + g);
    }
  };
  lds_char* const sbase = (lds_char*)(smem);
  auto lstore = [&](int buf) {
    lds_char* sK = sbase + buf * 2 * kTileBytes;
    lds_char* sV = sK + kTileBytes;
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int ci = threadIdx.x + 256 * r;
      const int off = Tile<D>::off(ci / CH, ci % CH);
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(sK + off) = kreg[r];
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(sV + off) = vreg[r];
    }
  };

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;

  const int ntiles = (L + kKT - 1) / kKT;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    const int k0 = j * kKT;
    const bool more = j + 1 < ntiles;
    if (more) gload(k0 + kKT);
    const lds_char* sK = sbase + (j & 1) * 2 * kTileBytes;
    const lds_char* sV = sK + kTileBytes;

    bf16x8 dsb[kKT / 16];
#pragma unroll
    for (int kb = 0; kb < kKT / 32; ++kb) {
      f32x16 sacc, dpacc;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sacc[i] = 0.f;
        dpacc[i] = 0.f;
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        sacc = mfma32(lds_row_frag<D>(sK, kb * 32, kk, lane), qf[kk], sacc);
        dpacc = mfma32(lds_row_frag<D>(sV, kb * 32, kk, lane), df[kk], dpacc);
      }
      const bool tail = k0 + kb * 32 + 32 > L;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(__builtin_fmaf(sacc[i], scale_log2, -lse2));
        if (tail && k0 + kb * 32 + acc_row(i, hh) >= L) p = 0.f;
        dsb[2 * kb + (i >> 3)][i & 7] = static_cast<__bf16>(p * (dpacc[i] - dl));
      }
    }
#pragma unroll
    for (int c = 0; c < kKT / 16; ++c)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        dqacc[db] = mfma32(lds_col_frag<D>(sK, 16 * c, 32 * db, lane), dsb[c], dqacc[db]);
    if (more) lstore((j + 1) & 1);
    __syncthreads();
  }

  if (qok) {
    int2 qp = make_int2(0, 0);
    if (pos != nullptr) qp = pos[s0 + qi];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * hh;
        float x[4] = {dqacc[db][4 * g4] * scale, dqacc[db][4 * g4 + 1] * scale, dqacc[db][4 * g4 + 2] * scale,
                      dqacc[db][4 * g4 + 3] * scale};
        if (pos != nullptr) rotate4<D>(x, d0, qp.x, qp.y, tab, max_pos, -1.0f);
        store4<TOut>(dq + qrow * D + d0, x[0], x[1], x[2], x[3]);
      }
  }
}

template <int D, typename T>
hipError_t launch_delta_t(const AttnArgs& a, const void* o, const void* dout, float* delta, hipStream_t stream) {
  const long long threads = static_cast<long long>(a.n_tokens) * a.n_heads * (D / 8);
  if (threads == 0) return hipSuccess;
  const long long blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((delta_kernel<D, T>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     static_cast<const T*>(o), static_cast<const T*>(dout), delta, a.n_tokens, a.n_heads);
  return hipGetLastError();
}

template <int D, typename TOut>
hipError_t launch_dkdv_t(const AttnArgs& a, const void* qr, const void* kr, const void* vb, const void* dob,
                         const float* lse, const float* delta, void* dk, void* dv, hipStream_t stream) {
  const long long blocks = sched_grid(a.n_tokens, a.n_segments, a.n_heads, kKB);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((dkdv_kernel<D, TOut>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(qr), static_cast<const uint16_t*>(kr),
                     static_cast<const uint16_t*>(vb), static_cast<const uint16_t*>(dob), lse, delta,
                     static_cast<TOut*>(dk), static_cast<TOut*>(dv), a.cu_seqlens, a.order, a.pt, a.n_segments,
                     a.n_tokens, a.n_heads, reinterpret_cast<const int2*>(a.pos), a.tab, a.max_pos, a.scale,
                     a.scale * kLog2e);
  return hipGetLastError();
}

template <int D, typename TOut>
hipError_t launch_dq_t(const AttnArgs& a, const void* qr, const void* kr, const void* vb, const void* dob,
                       const float* lse, const float* delta, void* dq, hipStream_t stream) {
  const long long blocks = sched_grid(a.n_tokens, a.n_segments, a.n_heads, kQT);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((dq_kernel<D, TOut>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(qr), static_cast<const uint16_t*>(kr),
                     static_cast<const uint16_t*>(vb), static_cast<const uint16_t*>(dob), lse, delta,
                     static_cast<TOut*>(dq), a.cu_seqlens, a.order, a.pt, a.n_segments, a.n_tokens, a.n_heads,
                     reinterpret_cast<const int2*>(a.pos), a.tab, a.max_pos, a.scale, a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_delta(const AttnArgs& a, const void* o, const void* dout, float* delta,
                                 hipStream_t stream) {
  if (a.head_dim == 128)
    return a.dtype == kDtypeBf16 ? launch_delta_t<128, uint16_t>(a, o, dout, delta, stream)
                                 : launch_delta_t<128, float>(a, o, dout, delta, stream);
  return a.dtype == kDtypeBf16 ? launch_delta_t<64, uint16_t>(a, o, dout, delta, stream)
                               : launch_delta_t<64, float>(a, o, dout, delta, stream);
}

hipError_t launch_attn_bwd_dkdv(const AttnArgs& a, const void* qr, const void* kr, const void* vb, const void* dob,
                                const float* lse, const float* delta, void* dk, void* dv, hipStream_t stream) {
  if (a.head_dim == 128)
    return a.dtype == kDtypeBf16 ? launch_dkdv_t<128, uint16_t>(a, qr, kr, vb, dob, lse, delta, dk, dv, stream)
                                 : launch_dkdv_t<128, float>(a, qr, kr, vb, dob, lse, delta, dk, dv, stream);
  return a.dtype == kDtypeBf16 ? launch_dkdv_t<64, uint16_t>(a, qr, kr, vb, dob, lse, delta, dk, dv, stream)
                               : launch_dkdv_t<64, float>(a, qr, kr, vb, dob, lse, delta, dk, dv, stream);
}

hipError_t launch_attn_bwd_dq(const AttnArgs& a, const void* qr, const void* kr, const void* vb, const void* dob,
                              const float* lse, const float* delta, void* dq, hipStream_t stream) {
  if (a.head_dim == 128)
    return a.dtype == kDtypeBf16 ? launch_dq_t<128, uint16_t>(a, qr, kr, vb, dob, lse, delta, dq, stream)
                                 : launch_dq_t<128, float>(a, qr, kr, vb, dob, lse, delta, dq, stream);
  return a.dtype == kDtypeBf16 ? launch_dq_t<64, uint16_t>(a, qr, kr, vb, dob, lse, delta, dq, stream)
                               : launch_dq_t<64, float>(a, qr, kr, vb, dob, lse, delta, dq, stream);
}

}  // namespace mf

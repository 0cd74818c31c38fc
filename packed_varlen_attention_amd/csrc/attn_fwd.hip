// Forward of block-diagonal multi-head attention over packed segments with
// axial 2D RoPE on Q and K (Mage-Flow paper section 3.2.1 "Model
// Architecture and Native Packing": joint self-attention over each sample's
// concatenated text and image tokens; samples packed into one stream never
// attend to each other).
//
// One workgroup = 4 waves = 128 query rows of one (segment, head); each wave
// owns 32 query rows.  The loop walks the segment's keys in tiles of 64:
//   K, V tile -> LDS (XOR-swizzled rows)
//   S^T = K Q^T      32x32x16 bf16 MFMA, Q held in registers (rotated at load)
//   online softmax   per query column, lane-local except one cross-half max/sum
//   O^T += V^T P^T   32x32x16 bf16 MFMA, V^T read from LDS by transpose reads
// Computing S^T rather than S puts each query's scores, running max/sum and
// output accumulator in the same lane, so the rescale needs no shuffles.
#include "mf_device.h"
#include "mf_kernels.h"

namespace mf {

namespace {

constexpr int kQT = 128;  // query rows per workgroup
constexpr int kKT = 64;   // keys per LDS tile

template <typename T>
__device__ __forceinline__ void load_q8(const T* p, bool ok, float (&x)[8]) {
  if (ok) {
    load8<T>(p, x);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = 0.f;
  }
}

template <int D, typename TIn>
__global__ __launch_bounds__(256) void attn_fwd_kernel(
    const TIn* __restrict__ q, const uint16_t* __restrict__ kr, const uint16_t* __restrict__ vb,
    TIn* __restrict__ o, float* __restrict__ lse, const int* __restrict__ cu, int n_tokens, int heads,
    const int2* __restrict__ pos, const float2* __restrict__ tab, int max_pos, float scale_log2) {
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int kTileBytes = kKT * D * 2;
  __shared__ __attribute__((aligned(16))) char smem[2 * kTileBytes];
  lds_char* sK = (lds_char*)(smem);
  lds_char* sV = sK + kTileBytes;

  const int seg = blockIdx.z;
  const int head = blockIdx.y;
  int s0 = cu[seg];
  int s1 = cu[seg + 1];
  s0 = min(max(s0, 0), n_tokens);
  s1 = min(max(s1, s0), n_tokens);
  const int L = s1 - s0;
  const int qbase = blockIdx.x * kQT;
  if (qbase >= L) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hh = lane >> 5;
  const int qi = qbase + wave * 32 + (lane & 31);
  const bool qok = qi < L;
  const long long qrow = (static_cast<long long>(s0) + qi) * heads + head;

  // Q fragments (B operand of S^T = K Q^T): Q[q][16kk + 8h .. +8], rotated.
  bf16x8 qf[NKK];
  {
    int2 qp = make_int2(0, 0);
    if (pos != nullptr && qok) qp = pos[s0 + qi];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int e0 = 16 * kk + 8 * hh;
      float x[8];
      load_q8<TIn>(q + qrow * D + e0, qok, x);
      if (pos != nullptr) rotate8<D>(x, e0, qp.x, qp.y, tab, max_pos, 1.0f);
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[kk][j] = static_cast<__bf16>(x[j]);
    }
  }

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

  for (int k0 = 0; k0 < L; k0 += kKT) {
    __syncthreads();
    for (int c = threadIdx.x; c < kKT * (D / 8); c += 256) {
      const int row = c / (D / 8);
      const int ch = c % (D / 8);
      const int key = k0 + row;
      u32x4 kv = {0u, 0u, 0u, 0u};
      u32x4 vv = {0u, 0u, 0u, 0u};
      if (key < L) {
        const size_t g = (static_cast<size_t>(s0 + key) * heads + head) * D + ch * 8;
        kv = *reinterpret_cast<const u32x4*>(kr + g);
        vv = *reinterpret_cast<const u32x4*>(vb + g);
      }
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(sK + Tile<D>::off(row, ch)) = kv;
      *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(sV + Tile<D>::off(row, ch)) = vv;
    }
    __syncthreads();

    f32x16 sacc[kKT / 32];
#pragma unroll
    for (int kb = 0; kb < kKT / 32; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) sacc[kb] = mfma32(lds_row_frag<D>(sK, kb * 32, kk, lane), qf[kk], sacc[kb]);
    }
    if (k0 + kKT > L) {
#pragma unroll
      for (int kb = 0; kb < kKT / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (k0 + kb * 32 + acc_row(i, hh) >= L) sacc[kb][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kKT / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = fast_exp2(m_run - m_new);
    float rsum = 0.f;
    bf16x8 pf[kKT / 16];
#pragma unroll
    for (int kb = 0; kb < kKT / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(sacc[kb][i] * scale_log2 - m_new);
        rsum += p;
        pf[2 * kb + (i >> 3)][i & 7] = static_cast<__bf16>(p);
      }
    rsum += __shfl_xor(rsum, 32, 64);
    l_run = l_run * alpha + rsum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
#pragma unroll
    for (int c = 0; c < kKT / 16; ++c)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        oacc[db] = mfma32(lds_col_frag<D>(sV, 16 * c, 32 * db, lane), pf[c], oacc[db]);
  }

  if (qok) {
    const float inv = 1.0f / l_run;
    TIn* orow = o + qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = 32 * db + 8 * g4 + 4 * hh;
        store4<TIn>(orow + d, oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv, oacc[db][4 * g4 + 2] * inv,
                    oacc[db][4 * g4 + 3] * inv);
      }
    if (lse != nullptr && hh == 0)
      lse[static_cast<size_t>(head) * n_tokens + s0 + qi] = (m_run + log2f(l_run)) * kLn2;
  }
}

template <int D, typename TIn>
hipError_t launch_fwd_t(const AttnArgs& a, const void* q, const void* kr, const void* vb, void* o, float* lse,
                        hipStream_t stream) {
  const dim3 grid((a.max_seqlen + kQT - 1) / kQT, a.n_heads, a.n_segments);
  hipLaunchKernelGGL((attn_fwd_kernel<D, TIn>), grid, dim3(256), 0, stream, static_cast<const TIn*>(q),
                     static_cast<const uint16_t*>(kr), static_cast<const uint16_t*>(vb), static_cast<TIn*>(o), lse,
                     a.cu_seqlens, a.n_tokens, a.n_heads, reinterpret_cast<const int2*>(a.pos), a.tab, a.max_pos,
                     a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a, const void* q, const void* kr, const void* vb, void* o, float* lse,
                           hipStream_t stream) {
  if (a.head_dim == 128) {
    return a.dtype == kDtypeBf16 ? launch_fwd_t<128, uint16_t>(a, q, kr, vb, o, lse, stream)
                                 : launch_fwd_t<128, float>(a, q, kr, vb, o, lse, stream);
  }
  return a.dtype == kDtypeBf16 ? launch_fwd_t<64, uint16_t>(a, q, kr, vb, o, lse, stream)
                               : launch_fwd_t<64, float>(a, q, kr, vb, o, lse, stream);
}

}  // namespace mf

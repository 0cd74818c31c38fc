// Forward of block-diagonal multi-head attention over packed segments with
// axial 2D RoPE on Q and K (Mage-Flow paper section 3.2.1 "Model
// Architecture and Native Packing": joint self-attention over each sample's
// concatenated text and image tokens; samples packed into one stream never
// attend to each other).
//
// One workgroup = 4 waves = 128 query rows of one (segment, head), taken from
// the longest-first, XCD-grouped schedule; each wave owns 32 query rows.  Two
// workgroups share a CU (<= 256 registers per lane, 64 KB LDS each), so each
// SIMD interleaves two waves' matrix and vector work.  The loop walks the
// segment's keys in tiles of 64:
//   the next K/V tile is loaded to registers while this one is computed, and
//   written to the other half of a double-buffered LDS (one barrier per tile);
//   S^T = K Q^T      32x32x16 bf16 MFMA, Q in registers (rotated at load);
//   online softmax   per query column, lane-local; the output is rescaled only
//                    when the running max grows by more than 2^8 (exact: the
//                    unnormalised weights then stay below 2^8);
//   O^T += V^T P^T   32x32x16 bf16 MFMA, V^T read by LDS transpose reads.
// Computing S^T rather than S puts each query's scores, running max and sum
// and output accumulator in the same lane, so no shuffles are needed except
// one max exchange between the two lane halves per tile.
#include "mf_device.h"
#include "mf_kernels.h"

namespace mf {

namespace {

constexpr int kQT = kFwdTile;  // query rows per workgroup
constexpr int kKT = 64;        // keys per LDS tile
constexpr float kRescaleSlack = 8.0f;  // log2 units the stale max may lag

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
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(
    const TIn* __restrict__ q, const uint16_t* __restrict__ kr, const uint16_t* __restrict__ vb,
    TIn* __restrict__ o, float* __restrict__ lse, const int* __restrict__ cu, const int* __restrict__ order,
    const int* __restrict__ pt, int n_seg, int n_tokens, int heads, const int2* __restrict__ pos,
    const float2* __restrict__ tab, int max_pos, float scale_log2) {
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int CH = D / 8;                   // 16-byte chunks per row
  constexpr int kTileBytes = kKT * D * 2;
  constexpr int kLoads = kKT * CH / 256;      // chunks per thread per tensor per tile
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

  // K/V staging: thread -> (row, chunk) pairs of a tile; rows past the end of
  // the segment re-read its last row (their scores are masked).
  u32x4 kreg[kLoads], vreg[kLoads];
  auto gload = [&](int k0) {
#pragma unroll
    for (int r = 0; r < kLoads; ++r) {
      const int ci = threadIdx.x + 256 * r;
      const int key = min(k0 + ci / CH, L - 1);
      const size_t g = (static_cast<size_t>(s0 + key) * heads + head) * D + (ci % CH) * 8;
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

  float m_run = -INFINITY;  // running max, log2 units, same in both lane halves
  float l_run = 0.f;        // this lane half's partial row sum
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

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
    const float mt = mx * scale_log2;
    if (__any(mt > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      m_run = m_new;
    }
    bf16x8 pf[kKT / 16];
#pragma unroll
    for (int kb = 0; kb < kKT / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(__builtin_fmaf(sacc[kb][i], scale_log2, -m_run));
        l_run += p;
        pf[2 * kb + (i >> 3)][i & 7] = static_cast<__bf16>(p);
      }
#pragma unroll
    for (int c = 0; c < kKT / 16; ++c)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        oacc[db] = mfma32(lds_col_frag<D>(sV, 16 * c, 32 * db, lane), pf[c], oacc[db]);

    if (more) lstore((j + 1) & 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (qok) {
    const float inv = 1.0f / l_tot;
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
      lse[static_cast<size_t>(head) * n_tokens + s0 + qi] = (m_run + log2f(l_tot)) * kLn2;
  }
}

template <int D, typename TIn>
hipError_t launch_fwd_t(const AttnArgs& a, const void* q, const void* kr, const void* vb, void* o, float* lse,
                        hipStream_t stream) {
  const long long blocks = sched_grid(a.n_tokens, a.n_segments, a.n_heads, kQT);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_fwd_kernel<D, TIn>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     static_cast<const TIn*>(q), static_cast<const uint16_t*>(kr), static_cast<const uint16_t*>(vb),
                     static_cast<TIn*>(o), lse, a.cu_seqlens, a.order, a.pt, a.n_segments, a.n_tokens, a.n_heads,
                     reinterpret_cast<const int2*>(a.pos), a.tab, a.max_pos, a.scale * kLog2e);
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

// Forward of block-diagonal multi-head attention over packed segments with
// axial 2D RoPE on Q and K (Mage-Flow paper section 3.2.1 "Model
// Architecture and Native Packing": joint self-attention over each sample's
// concatenated text and image tokens; samples packed into one stream never
// attend to each other).
//
// One workgroup = 4 waves = 128 query rows of one (segment, head), taken from
// the longest-first, XCD-grouped schedule; each wave owns 32 query rows and
// all four share each K/V tile.  With <= 168 registers per lane and 48 KB of
// LDS per workgroup, three workgroups share a CU, so each SIMD runs three
// waves and interleaves their matrix, vector and LDS work.  The loop walks
// the segment's keys in tiles of 32, software-pipelined.  Packs whose
// segments are all long (fwd_tile()) run the same kernel as 8 waves = 256 rows
// on 64-key tiles instead, one workgroup per CU at two waves per SIMD:
//   K and V tiles are copied global -> LDS directly (no registers) into
//   three buffers each, two tiles ahead, each copy a block-uniform tile base
//   plus a fixed 32-bit lane offset; K runs one tile ahead of V, so the
//   scores of tile j+1 are computed while the softmax and P V of tile j run;
//   one barrier per tile;
//   S^T = K Q^T      32x32x16 bf16 MFMA, Q in registers (rotated at load);
//   online softmax   per query column, lane-local; the output is rescaled only
//                    when the running max grows by more than 2^8 (exact: the
//                    unnormalised weights then stay below 2^8);
//   O^T += V^T P^T   32x32x16 bf16 MFMA, V^T read by LDS transpose reads.
// Computing S^T rather than S puts each query's scores, running max and sum
// and output accumulator in the same lane, so no shuffles are needed except
// one max exchange between the two lane halves per tile (v_permlane32_swap,
// a register-to-register swap, not a round trip through LDS).
#include <type_traits>

#include "mf_device.h"
#include "mf_kernels.h"

namespace mf {

namespace {

constexpr float kRescaleSlack = 8.0f;  // log2 units the stale max may lag

// v_permlane32_swap: each lane gets its own value and the one of the lane
// 32 away (in the same order in both halves).
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename T>
__device__ __forceinline__ void load_q8(const T* p, bool ok, float (&x)[8]) {
  if (ok) {
    load8<T>(p, x);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = 0.f;
  }
}

// QT query rows per workgroup (32 per wave), KT keys per LDS tile, WPS
// resident waves per SIMD (sets the register budget).
template <int D, typename TIn, bool kMulti, int QT, int KT, int WPS>
__global__ __launch_bounds__(QT / 32 * 64, WPS) void attn_fwd_kernel(
    const TIn* __restrict__ q, const uint16_t* __restrict__ kr, const uint16_t* __restrict__ vb,
    TIn* __restrict__ o, float* __restrict__ lse, const int* __restrict__ cu, const int* __restrict__ order,
    const int* __restrict__ pt, int n_seg, int n_tokens, int heads, const int* __restrict__ pos, int nax,
    const float2* __restrict__ tab, int max_pos, float scale_log2, const int* __restrict__ rcu,
    const int* __restrict__ vfirst, uint16_t* __restrict__ qr_out) {
  constexpr int kQT = QT;
  constexpr int kKT = KT;
  constexpr int kWaves = QT / 32;
  constexpr int kKB = KT / 32;  // 32-key blocks per tile
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int kRowBytes = D * 2;
  constexpr int kTileBytes = kKT * kRowBytes;
  // LDS: three K and three V tiles, as six separate objects so the compiler
  // can tell the tile being read from the tiles being filled by in-flight
  // copies (otherwise it waits for every copy before each transpose read).
  __shared__ __attribute__((aligned(16))) char smemK0[kTileBytes];
  __shared__ __attribute__((aligned(16))) char smemK1[kTileBytes];
  __shared__ __attribute__((aligned(16))) char smemK2[kTileBytes];
  __shared__ __attribute__((aligned(16))) char smemV0[kTileBytes];
  __shared__ __attribute__((aligned(16))) char smemV1[kTileBytes];
  __shared__ __attribute__((aligned(16))) char smemV2[kTileBytes];

  WorkItem it;
  if (!decode_item(blockIdx.x, heads, n_seg, order, pt, it)) return;
  const int head = it.head;
  int s0, s1;
  seg_bounds(cu, it.seg, n_tokens, s0, s1);
  const int L = s1 - s0;
  const int qbase = it.tile * kQT;
  if (qbase >= L) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5;
  const int qi = qbase + wave * 32 + (lane & 31);
  const bool qok = qi < L;
  // A multi-segment tile (several tiny segments, at most 255 tokens) is left
  // to the kMulti instance, where a query meets only the keys of its own
  // segment; the ordinary instance carries none of that code.
  const int f0 = vfirst != nullptr ? vfirst[it.seg] : it.seg;
  const int f1 = vfirst != nullptr ? vfirst[it.seg + 1] : it.seg + 1;
  if ((f1 - f0 > 1) != kMulti) return;
  const long long qrow = (static_cast<long long>(s0) + qi) * heads + head;

  // Q fragments (B operand of S^T = K Q^T): Q[q][16kk + 8h .. +8], rotated.
  bf16x8 qf[NKK];
  {
    Pos3 qp = {0, 0, 0};
    if (pos != nullptr && qok) qp = load_pos(pos, s0 + qi, nax);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int e0 = 16 * kk + 8 * hh;
      float x[8];
      load_q8<TIn>(q + qrow * D + e0, qok, x);
      if (pos != nullptr) rotate_n<D, 8>(x, e0, qp, tab, max_pos, 1.0f, nax);
#pragma unroll
      for (int j = 0; j < 8; ++j) qf[kk][j] = static_cast<__bf16>(x[j]);
      // The caller may keep the rotated bf16 Q for the backward.
      if (qr_out != nullptr && qok)
        *reinterpret_cast<u32x4*>(qr_out + qrow * D + e0) = __builtin_bit_cast(u32x4, qf[kk]);
    }
  }

  const size_t hD = static_cast<size_t>(heads) * D;
  const uint16_t* kseg = kr + static_cast<size_t>(s0) * hD + static_cast<size_t>(head) * D;
  const uint16_t* vseg = vb + static_cast<size_t>(s0) * hD + static_cast<size_t>(head) * D;
  const TileCopy<D, kKT, kWaves> copy(wave, lane, static_cast<unsigned>(hD * 2));
  lds_char* const sKb[3] = {(lds_char*)(smemK0), (lds_char*)(smemK1), (lds_char*)(smemK2)};
  lds_char* const sVb[3] = {(lds_char*)(smemV0), (lds_char*)(smemV1), (lds_char*)(smemV2)};
  auto load_rows = [&](const uint16_t* seg, int k0, lds_char* dst) { copy(seg, k0, L, dst); };

  // ---- LDS fragment offsets (bytes), fixed per lane; tile bases add on top.
  int roff[NKK];  // A-operand rows: row perm32(lane % 32), chunk 2kk + h
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) roff[kk] = Tile<D>::off(perm32(lane & 31), 2 * kk + hh);
  int coff[NDB][2];  // transpose reads: rows 8h + (lane/4)%4 (+4), columns of block db
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int g = lane >> 4;
    const int l16 = lane & 15;
    const int col = 32 * db + 16 * (g & 1) + 4 * (l16 & 3);
    const int row0 = 8 * hh + (l16 >> 2);
    coff[db][0] = Tile<D>::off(row0, col >> 3) + ((col >> 2) & 1) * 8;
    coff[db][1] = Tile<D>::off(row0 + 4, col >> 3) + ((col >> 2) & 1) * 8;
  }
  auto s_tile = [&](const lds_char* sK, f32x16 (&acc)[kKB]) {
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[kb][i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        const bf16x8 a = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            sK + roff[kk] + kb * 32 * kRowBytes);
        acc[kb] = mfma32(a, qf[kk], acc[kb]);
      }
  };
  auto col_frag = [&](const lds_char* sV, int c, int db) {
    const lds_char* p0 = sV + coff[db][0] + 16 * c * kRowBytes;
    const lds_char* p1 = sV + coff[db][1] + 16 * c * kRowBytes;
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) i16x4*>(const_cast<lds_char*>(p0)));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) i16x4*>(const_cast<lds_char*>(p1)));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, r);
  };

  // Running max, log2 units, same in both lane halves.  It starts finite, so
  // a key tile that a multi-segment tile masks entirely for this query leaves
  // it (and the sums) untouched instead of producing -inf - (-inf).
  float m_run = -1e30f;
  float l_run = 0.f;        // this lane half's partial row sum
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

  // Pipeline: K runs one tile ahead of V, so the scores of tile j+1 are
  // computed while the softmax of tile j runs, and the copies run two steps
  // ahead of their use.  Tile t of K lives in K buffer t % 3, tile t of V in
  // V buffer t % 3.  Step j issues the copies of K tile j+3 and V tile j+2
  // and, at its end, waits only for the copies issued before it (K tile j+2,
  // V tile j+1), leaving its own in flight across the next step.
  const int ntiles = (L + kKT - 1) / kKT;
  const int last_k0 = (ntiles - 1) * kKT;
  f32x16 scur[kKB], snext[kKB];
  load_rows(kseg, 0, sKb[0]);
  load_rows(vseg, 0, sVb[0]);
  if (ntiles > 1) load_rows(kseg, kKT, sKb[1]);
  wait_vmem();
  __syncthreads();
  s_tile(sKb[0], scur);
  if (ntiles > 2) load_rows(kseg, 2 * kKT, sKb[2]);
  if (ntiles > 1) load_rows(vseg, kKT, sVb[1]);
  __syncthreads();  // every wave is done with K tile 0 before tile 3 reuses its buffer

  // One pipeline step: softmax + P V of tile j, scores of tile j + 1.  Only
  // the last tile masks keys; that branch and the rescale branch are rare.
  // b (= j % 3) is compile-time, so every LDS address names its buffer
  // statically.  In a segment that fits one query tile, a wave whose 32
  // query rows all lie past the segment's end skips this work; it still
  // issues its copies and meets every barrier.  Longer segments keep their
  // idle waves busy: a last tile that finished early would start the next
  // (segment, head) sooner and break the XCD's shared sweep over K and V
  // (measured: 24% more HBM fetch on a pack of long segments, same time).
  const bool wave_q = qbase + wave * 32 < L || L > kQT;
  auto compute = [&](int j, auto buf_tag) {
    constexpr int b = decltype(buf_tag)::value;
    const int k0 = j * kKT;
    if (kMulti || k0 + kKT > L) {  // keys past the segment's end, or outside the query's segment
      if constexpr (kMulti) {
        int qlo, qhi;
        member_bounds(rcu, f0, f1, s0, s1, min(qi, L - 1), qlo, qhi);
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + kb * 32 + acc_row(i, hh);
            if (key < qlo || key >= qhi) scur[kb][i] = -INFINITY;
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (k0 + kb * 32 + acc_row(i, hh) >= L) scur[kb][i] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, scur[kb][i]);
    mx = half_max(mx);
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
    // Straight-line region: exp/sum/convert of tile j, S of tile j+1, P V of tile j.
    bf16x8 pf[kKT / 16];
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = fast_exp2(__builtin_fmaf(scur[kb][i], scale_log2, -m_run));
        const float p1 = fast_exp2(__builtin_fmaf(scur[kb][i + 1], scale_log2, -m_run));
        l_run += p0 + p1;
        pf[2 * kb + (i >> 3)][i & 7] = static_cast<__bf16>(p0);
        pf[2 * kb + (i >> 3)][(i & 7) + 1] = static_cast<__bf16>(p1);
      }
    // Scores of tile j + 1 (for the last tile they read a stale buffer and
    // are discarded).
    s_tile(sKb[(b + 1) % 3], snext);
    const lds_char* sV = sVb[b];
#pragma unroll
    for (int c = 0; c < kKT / 16; ++c)
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] = mfma32(col_frag(sV, c, db), pf[c], oacc[db]);
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) scur[kb] = snext[kb];
  };
  auto step = [&](int j, auto buf_tag) {
    constexpr int b = decltype(buf_tag)::value;
    const int k0 = j * kKT;
    // Every step issues both copies, so the wait below has a fixed count;
    // past the end they re-read the last tile into buffers no later step
    // reads.
    load_rows(kseg, min(k0 + 3 * kKT, last_k0), sKb[b]);
    load_rows(vseg, min(k0 + 2 * kKT, last_k0), sVb[(b + 2) % 3]);
    if (wave_q) compute(j, buf_tag);
    // Wait for everything but this step's own copies (they complete in order).
    wait_vmem_keep<2 * TileCopy<D, kKT, kWaves>::kCopies>();
    barrier_keep_loads();
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  int j = 0;
  for (; j + 3 <= ntiles; j += 3) {
    step(j, B0{});
    step(j + 1, B1{});
    step(j + 2, B2{});
  }
  if (j < ntiles) {
    step(j, B0{});
    if (j + 1 < ntiles) step(j + 1, B1{});
  }
  wait_vmem();  // the last step's copies land before the workgroup's LDS is released

  const float l_tot = half_sum(l_run);
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

template <int D, typename TIn, int QT, int KT, int WPS>
hipError_t launch_fwd_t(const AttnArgs& a, const void* q, const void* kr, const void* vb, void* o, float* lse,
                        hipStream_t stream) {
  const long long blocks = sched_grid(a.n_tokens, a.n_segments, a.n_heads, QT);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  // The ordinary tiles, then (with merged tiny segments) the multi-segment
  // ones; each launch's blocks exit at once on the other kind of item.
  hipLaunchKernelGGL((attn_fwd_kernel<D, TIn, false, QT, KT, WPS>), dim3(static_cast<unsigned>(blocks)),
                     dim3(QT / 32 * 64), 0, stream, static_cast<const TIn*>(q), static_cast<const uint16_t*>(kr),
                     static_cast<const uint16_t*>(vb), static_cast<TIn*>(o), lse, a.cu_seqlens, a.order, a.pt,
                     a.n_segments, a.n_tokens, a.n_heads, a.pos, a.nax, a.tab, a.max_pos, a.scale * kLog2e, a.rcu,
                     a.vfirst, static_cast<uint16_t*>(a.qr_out));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.vfirst == nullptr) return e;
  hipLaunchKernelGGL((attn_fwd_kernel<D, TIn, true, QT, KT, WPS>), dim3(static_cast<unsigned>(blocks)),
                     dim3(QT / 32 * 64), 0, stream, static_cast<const TIn*>(q), static_cast<const uint16_t*>(kr),
                     static_cast<const uint16_t*>(vb), static_cast<TIn*>(o), lse, a.cu_seqlens, a.order, a.pt,
                     a.n_segments, a.n_tokens, a.n_heads, a.pos, a.nax, a.tab, a.max_pos, a.scale * kLog2e, a.rcu,
                     a.vfirst, static_cast<uint16_t*>(a.qr_out));
  return hipGetLastError();
}

// The shape fwd_tile() picks for the call; the schedule was built with the
// same tile.
template <int D, typename TIn>
hipError_t launch_fwd_any(const AttnArgs& a, const void* q, const void* kr, const void* vb, void* o, float* lse,
                          hipStream_t stream) {
  if (fwd_tile(a.max_seqlen, a.n_tokens, a.n_segments) == kFwdTileLong)
    return launch_fwd_t<D, TIn, kFwdTileLong, 64, 2>(a, q, kr, vb, o, lse, stream);
  return launch_fwd_t<D, TIn, kFwdTile, 32, 3>(a, q, kr, vb, o, lse, stream);
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a, const void* q, const void* kr, const void* vb, void* o, float* lse,
                           hipStream_t stream) {
  if (a.head_dim == 128) {
    return a.dtype == kDtypeBf16 ? launch_fwd_any<128, uint16_t>(a, q, kr, vb, o, lse, stream)
                                 : launch_fwd_any<128, float>(a, q, kr, vb, o, lse, stream);
  }
  return a.dtype == kDtypeBf16 ? launch_fwd_any<64, uint16_t>(a, q, kr, vb, o, lse, stream)
                               : launch_fwd_any<64, float>(a, q, kr, vb, o, lse, stream);
}

}  // namespace mf

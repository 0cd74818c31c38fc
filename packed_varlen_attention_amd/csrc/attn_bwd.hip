// Backward of packed block-diagonal attention with axial 2D RoPE.
//
// With P = softmax(scale * Qr Kr^T) recomputed from the forward's LSE:
//   Delta = rowsum(dO * O)                       dq kernel prologue (written for dkdv)
//   dV = P^T dO,  dKr = scale * dS^T Qr          dkdv kernel, per 32 keys/wave
//                                                (K in registers, V rows in LDS)
//   dQr = scale * dS Kr                          dq kernel,   per 32 queries/wave
//                                                (8 waves and 64-key tiles, or 4
//                                                and 32 where tiny segments are
//                                                merged; K/V tiles three-buffered)
// where dS = P * (dO V^T - Delta); dQ and dK are rotated back by the inverse
// rotation in the epilogues.  Each output element is written by exactly one
// lane and summed in a fixed order: results are deterministic (no atomics).
#include <type_traits>

#include "mf_device.h"
#include "mf_kernels.h"

namespace mf {

namespace {

constexpr int kKB = kDkdvTile;  // keys per dkdv workgroup (32 per wave)
constexpr int kQB = 32;         // queries per dkdv LDS tile

template <int D, typename TOut>
__global__ __launch_bounds__(256, 2) void dkdv_kernel(
    const uint16_t* __restrict__ qr, const uint16_t* __restrict__ kr, const uint16_t* __restrict__ vb,
    const uint16_t* __restrict__ dob, const float* __restrict__ lse2, const float* __restrict__ delta,
    TOut* __restrict__ dk, TOut* __restrict__ dv, const int* __restrict__ cu, const int* __restrict__ order,
    const int* __restrict__ pt, int n_seg, int n_tokens, int heads, const int* __restrict__ pos, int nax,
    const float2* __restrict__ tab, int max_pos, float scale, float scale_log2) {
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int kRowBytes = D * 2;
  constexpr int kTileBytes = kQB * kRowBytes;
  // LDS: Q tiles [2], dO tiles [2], then per buffer 32 log2-LSE + 32 Delta
  __shared__ __attribute__((aligned(16))) char smem[4 * kTileBytes + 2 * 2 * kQB * 4 + kKB * kRowBytes];

  WorkItem it;
  if (!decode_item(blockIdx.x, heads, n_seg, order, pt, it)) return;
  const int head = it.head;
  int s0, s1;
  seg_bounds(cu, it.seg, n_tokens, s0, s1);
  const int L = s1 - s0;
  const int kbase = it.tile * kKB;
  if (kbase >= L) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hh = lane >> 5;
  const int key = kbase + wave * 32 + (lane & 31);
  const bool kok = key < L;
  const long long krow = (static_cast<long long>(s0) + min(key, L - 1)) * heads + head;

  // K fragments in registers (B operand of S = Q Kr^T); the workgroup's V
  // rows live in LDS and feed dP = dO V^T.
  bf16x8 kf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int e0 = 16 * kk + 8 * hh;
    kf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kr + krow * D + e0));
  }

  // ---- global -> LDS copies of the Q / dO tiles and their row statistics.
  const unsigned pitch = static_cast<unsigned>(heads) * D * 2;  // bytes per token row, < 2^24
  const uint16_t* qseg = qr + (static_cast<size_t>(s0) * heads + head) * D;
  const uint16_t* oseg = dob + (static_cast<size_t>(s0) * heads + head) * D;
  const float* stat_src = (lane < 32 ? lse2 : delta) + static_cast<size_t>(head) * n_tokens + s0;
  const TileCopy<D, kQB, 4> copy(wave, lane, pitch);
  lds_char* const sQ0 = (lds_char*)(smem);
  lds_char* const sO0 = sQ0 + 2 * kTileBytes;
  lds_char* const sS0 = sQ0 + 4 * kTileBytes;  // [buf][lse2 x 32, delta x 32]
  lds_char* const sVb = sS0 + 2 * 2 * kQB * 4;   // V rows of this workgroup's keys
  auto load_tile = [&](int q0, int buf) {
    copy(qseg, q0, L, sQ0 + buf * kTileBytes);
    copy(oseg, q0, L, sO0 + buf * kTileBytes);
    if (wave == 0) {
      const int row = min(q0 + (lane & 31), L - 1);
      __builtin_amdgcn_global_load_lds(stat_src + row, sS0 + buf * 2 * kQB * 4, 4, 0, 0);
    }
  };

  int roff[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) roff[kk] = Tile<D>::off(perm32(lane & 31), 2 * kk + hh);
  int coff[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int g = lane >> 4;
    const int l16 = lane & 15;
    const int col = 32 * db + 16 * (g & 1) + 4 * (l16 & 3);
    const int row0 = 8 * hh + (l16 >> 2);
    coff[db][0] = Tile<D>::off(row0, col >> 3) + ((col >> 2) & 1) * 8;
    coff[db][1] = Tile<D>::off(row0 + 4, col >> 3) + ((col >> 2) & 1) * 8;
  }
  auto row_frag = [&](const lds_char* t, int kk) {
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(t + roff[kk]);
  };
  auto col_frag = [&](const lds_char* t, int c, int db) {
    const lds_char* p0 = t + coff[db][0] + 16 * c * kRowBytes;
    const lds_char* p1 = t + coff[db][1] + 16 * c * kRowBytes;
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) i16x4*>(const_cast<lds_char*>(p0)));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) i16x4*>(const_cast<lds_char*>(p1)));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, r);
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
  // In a segment that fits one workgroup, a wave whose 32 keys all lie past
  // the segment's end skips the products; it still copies its share of each
  // tile and meets the barrier.
  const bool wave_keys = kbase + wave * 32 < L || L > kKB;
  auto compute = [&](int q0, int b) {
    const lds_char* sQ = sQ0 + b * kTileBytes;
    const lds_char* sO = sO0 + b * kTileBytes;
    const __attribute__((address_space(3))) float* st =
        reinterpret_cast<const __attribute__((address_space(3))) float*>(sS0 + b * 2 * kQB * 4);

    // S = Q Kr^T; P = exp2(S * scale * log2e - lse2) (rows past the end: 0)
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) acc = mfma32(row_frag(sQ, kk), kf[kk], acc);
    if (q0 + kQB > L) {  // only the segment's last tile holds rows past its end: exp2(-inf) = 0
#pragma unroll
      for (int g = 0; g < 2; ++g) mask_rows8(acc, g, L - (q0 + 16 * g + 8 * hh), -INFINITY);
    }
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) p[i] = fast_exp2(__builtin_fmaf(acc[i], scale_log2, -st[acc_row(i, hh)]));
    bf16x8 pb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) pb[i >> 3][i & 7] = static_cast<__bf16>(p[i]);
    // dP = dO V^T; dS = P (dP - Delta)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int vr = wave * 32 + (lane & 31);
      const bf16x8 vfr = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
          sVb + Tile<D>::off(vr, 2 * kk + hh));
      acc = mfma32(row_frag(sO, kk), vfr, acc);
    }
    bf16x8 dsb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) dsb[i >> 3][i & 7] = static_cast<__bf16>(p[i] * (acc[i] - st[kQB + acc_row(i, hh)]));
    // dV^T += dO^T P.  The transpose reads come last in the step: the compiler
    // waits for the next tile's copies before the first of them.
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < NDB; ++db) dvacc[db] = mfma32(col_frag(sO, c, db), pb[c], dvacc[db]);
    // dK^T += Q^T dS
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < NDB; ++db) dkacc[db] = mfma32(col_frag(sQ, c, db), dsb[c], dkacc[db]);
  };
  auto step = [&](int j) {
    const int q0 = j * kQB;
    const int b = j & 1;
    if (j + 1 < ntiles) load_tile(q0 + kQB, b ^ 1);
    if (wave_keys) compute(q0, b);
    wait_vmem();
    __syncthreads();
  };
  {
    const uint16_t* vseg = vb + (static_cast<size_t>(s0) * heads + head) * D;
    const TileCopy<D, kKB, 4> copy_v(wave, lane, pitch);
    copy_v(vseg, kbase, L, sVb);
  }
  load_tile(0, 0);
  wait_vmem();
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) step(j);

  if (kok) {
    Pos3 kp = {0, 0, 0};
    if (pos != nullptr) kp = load_pos(pos, s0 + key, nax);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * hh;
        float x[4] = {dkacc[db][4 * g4] * scale, dkacc[db][4 * g4 + 1] * scale, dkacc[db][4 * g4 + 2] * scale,
                      dkacc[db][4 * g4 + 3] * scale};
        if (pos != nullptr) rotate_n<D, 4>(x, d0, kp, tab, max_pos, -1.0f, nax);
        store4<TOut>(dk + krow * D + d0, x[0], x[1], x[2], x[3]);
        store4<TOut>(dv + krow * D + d0, dvacc[db][4 * g4], dvacc[db][4 * g4 + 1], dvacc[db][4 * g4 + 2],
                     dvacc[db][4 * g4 + 3]);
      }
  }
}

// dq in two shapes: QT queries per workgroup (32 per wave) and KT keys per
// LDS tile.  256 x 64 for ordinary packs; 128 x 32 where runs of tiny
// segments are merged, so that two short-lived workgroups share a CU.
template <int D, typename TOut, bool kMulti, int QT, int KT>
__global__ __launch_bounds__(QT / 32 * 64, 2) void dq_kernel(
    const uint16_t* __restrict__ qr, const uint16_t* __restrict__ kr, const uint16_t* __restrict__ vb,
    const uint16_t* __restrict__ dob, const TOut* __restrict__ o, const TOut* __restrict__ dout,
    const float* __restrict__ lse, float* __restrict__ lse2, float* __restrict__ delta,
    TOut* __restrict__ dq, const int* __restrict__ cu, const int* __restrict__ order, const int* __restrict__ pt,
    int n_seg, int n_tokens, int heads, const int* __restrict__ pos, int nax, const float2* __restrict__ tab,
    int max_pos, float scale, float scale_log2, const int* __restrict__ rcu, const int* __restrict__ vfirst) {
  constexpr int kQT = QT;
  constexpr int kKT = KT;
  constexpr int kDqWaves = QT / 32;
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int kRowBytes = D * 2;
  constexpr int kTileBytes = kKT * kRowBytes;
  constexpr int kInstPerWave = TileCopy<D, kKT, kDqWaves>::kCopies;  // copy instructions per wave and tile
  // LDS: three K and three V tiles, six separate objects so the compiler can
  // tell the tile being read from the tiles being filled by in-flight copies.
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
  // A multi-segment tile is left to the kMulti instance, where a query meets
  // only the keys of its own segment, [qlo, qhi) in tile rows.
  const int f0 = vfirst != nullptr ? vfirst[it.seg] : it.seg;
  const int f1 = vfirst != nullptr ? vfirst[it.seg + 1] : it.seg + 1;
  if ((f1 - f0 > 1) != kMulti) return;
  int qlo = 0, qhi = L;
  if constexpr (kMulti) member_bounds(rcu, f0, f1, s0, s1, min(qi, L - 1), qlo, qhi);
  const long long qrow = (static_cast<long long>(s0) + min(qi, L - 1)) * heads + head;
  // Keys this wave's queries can meet (in a multi-segment tile, the union of
  // their segments; wave-uniform).  Key tiles outside it give this wave
  // dS = 0 exactly, so it skips their work and only takes part in the copies
  // and barriers; so does, in a segment that fits one query tile, a wave
  // whose 32 query rows all lie past the segment's end (longer segments keep
  // such waves busy, as the forward does, to keep their tiles in step).
  int wklo = 0, wkhi = L;
  const bool wave_q = qbase + wave * 32 < L || L > kQT;
  if constexpr (kMulti) {
    int lo = qlo, hi = qhi;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      lo = min(lo, __shfl_xor(lo, off, 64));
      hi = max(hi, __shfl_xor(hi, off, 64));
    }
    wklo = __builtin_amdgcn_readfirstlane(lo);
    wkhi = __builtin_amdgcn_readfirstlane(hi);
  }

  bf16x8 qf[NKK], df[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int e0 = 16 * kk + 8 * hh;
    qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qr + qrow * D + e0));
    df[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(dob + qrow * D + e0));
  }
  // This query's row statistics, also written for dkdv (which runs after
  // dq): Delta = dot(dO, O) over the row -- each lane half holds half of it
  // -- and the LSE in log2 units.
  const size_t si = static_cast<size_t>(head) * n_tokens + s0 + min(qi, L - 1);
  float part = 0.f;
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int e0 = 16 * kk + 8 * hh;
    float a[8], g[8];
    load8<TOut>(o + qrow * D + e0, a);
    if constexpr (std::is_same<TOut, uint16_t>::value) {
#pragma unroll
      for (int j = 0; j < 8; ++j) g[j] = static_cast<float>(df[kk][j]);  // bf16 dO as given
    } else {
      load8<TOut>(dout + qrow * D + e0, g);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) part += a[j] * g[j];
  }
  const float dl = part + __shfl_xor(part, 32, 64);
  const float l2 = lse[si] * kLog2e;
  if (qok && hh == 0) {
    delta[si] = dl;
    lse2[si] = l2;
  }

  const unsigned pitch = static_cast<unsigned>(heads) * D * 2;  // bytes per token row, < 2^24
  const uint16_t* kseg = kr + (static_cast<size_t>(s0) * heads + head) * D;
  const uint16_t* vseg = vb + (static_cast<size_t>(s0) * heads + head) * D;
  const TileCopy<D, kKT, kDqWaves> copy(wave, lane, pitch);
  lds_char* const sKb[3] = {(lds_char*)(smemK0), (lds_char*)(smemK1), (lds_char*)(smemK2)};
  lds_char* const sVb[3] = {(lds_char*)(smemV0), (lds_char*)(smemV1), (lds_char*)(smemV2)};
  auto load_tile = [&](int k0, lds_char* dK, lds_char* dV) {
    copy(kseg, k0, L, dK);
    copy(vseg, k0, L, dV);
  };
  int roff[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) roff[kk] = Tile<D>::off(perm32(lane & 31), 2 * kk + hh);
  int coff[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int g = lane >> 4;
    const int l16 = lane & 15;
    const int col = 32 * db + 16 * (g & 1) + 4 * (l16 & 3);
    const int row0 = 8 * hh + (l16 >> 2);
    coff[db][0] = Tile<D>::off(row0, col >> 3) + ((col >> 2) & 1) * 8;
    coff[db][1] = Tile<D>::off(row0 + 4, col >> 3) + ((col >> 2) & 1) * 8;
  }
  auto col_frag = [&](const lds_char* t, int c, int db) {
    const lds_char* p0 = t + coff[db][0] + 16 * c * kRowBytes;
    const lds_char* p1 = t + coff[db][1] + 16 * c * kRowBytes;
    i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) i16x4*>(const_cast<lds_char*>(p0)));
    i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) i16x4*>(const_cast<lds_char*>(p1)));
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, r);
  };

  f32x16 dqacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;

  // Tile t lives in buffer t % 3.  Step j issues the copies of tile j + 2
  // (past the end: the last tile again, into a buffer no later step reads),
  // so every step issues the same number of copies, and at its end waits
  // only for those issued before it; b = j % 3 is compile-time.
  const int ntiles = (L + kKT - 1) / kKT;
  const int last_k0 = (ntiles - 1) * kKT;
  // The work of one key tile: S^T and dP^T, dS, dQ^T += Kr^T dS^T.
  auto compute = [&](int k0, auto buf_tag) {
    constexpr int b = decltype(buf_tag)::value;
    const lds_char* sK = sKb[b];
    const lds_char* sV = sVb[b];
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
        const bf16x8 ka = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            sK + roff[kk] + kb * 32 * kRowBytes);
        const bf16x8 va = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            sV + roff[kk] + kb * 32 * kRowBytes);
        sacc = mfma32(ka, qf[kk], sacc);
        dpacc = mfma32(va, df[kk], dpacc);
      }
      if (kMulti || k0 + kKT > L) {  // keys outside the query's segment (or past its end): exp2(-inf) = 0
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int r0 = k0 + 32 * kb + 16 * g + 8 * hh;
          mask_rows8_range(sacc, g, qlo - r0, qhi - r0, -INFINITY);
        }
      }
      float p[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = fast_exp2(__builtin_fmaf(sacc[i], scale_log2, -l2));
#pragma unroll
      for (int i = 0; i < 16; ++i) dsb[2 * kb + (i >> 3)][i & 7] = static_cast<__bf16>(p[i] * (dpacc[i] - dl));
    }
#pragma unroll
    for (int c = 0; c < kKT / 16; ++c)
#pragma unroll
      for (int db = 0; db < NDB; ++db) dqacc[db] = mfma32(col_frag(sK, c, db), dsb[c], dqacc[db]);
  };
  auto step = [&](int j, auto buf_tag) {
    constexpr int b = decltype(buf_tag)::value;
    const int k0 = j * kKT;
    load_tile(min(k0 + 2 * kKT, last_k0), sKb[(b + 2) % 3], sVb[(b + 2) % 3]);
    if (wave_q && (!kMulti || (k0 < wkhi && k0 + kKT > wklo))) compute(k0, buf_tag);
    wait_vmem_keep<2 * kInstPerWave>();
    barrier_keep_loads();
  };
  load_tile(0, sKb[0], sVb[0]);
  if (ntiles > 1) load_tile(kKT, sKb[1], sVb[1]);
  wait_vmem();
  __syncthreads();
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
  wait_vmem();  // the last steps' copies land before the workgroup's LDS is released

  if (qok) {
    Pos3 qp = {0, 0, 0};
    if (pos != nullptr) qp = load_pos(pos, s0 + qi, nax);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * db + 8 * g4 + 4 * hh;
        float x[4] = {dqacc[db][4 * g4] * scale, dqacc[db][4 * g4 + 1] * scale, dqacc[db][4 * g4 + 2] * scale,
                      dqacc[db][4 * g4 + 3] * scale};
        if (pos != nullptr) rotate_n<D, 4>(x, d0, qp, tab, max_pos, -1.0f, nax);
        store4<TOut>(dq + qrow * D + d0, x[0], x[1], x[2], x[3]);
      }
  }
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
                     a.n_tokens, a.n_heads, a.pos, a.nax, a.tab, a.max_pos, a.scale,
                     a.scale * kLog2e);
  return hipGetLastError();
}

template <int D, typename TOut, int QT, int KT, bool kMerged>
hipError_t launch_dq_t(const AttnArgs& a, const void* qr, const void* kr, const void* vb, const void* dob,
                       const void* o, const void* dout, const float* lse, float* lse2, float* delta, void* dq,
                       hipStream_t stream) {
  const long long blocks = sched_grid(a.n_tokens, a.n_segments, a.n_heads, QT);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((dq_kernel<D, TOut, false, QT, KT>), dim3(static_cast<unsigned>(blocks)), dim3(QT / 32 * 64), 0,
                     stream, static_cast<const uint16_t*>(qr), static_cast<const uint16_t*>(kr),
                     static_cast<const uint16_t*>(vb), static_cast<const uint16_t*>(dob),
                     static_cast<const TOut*>(o), static_cast<const TOut*>(dout), lse, lse2, delta,
                     static_cast<TOut*>(dq), a.cu_seqlens, a.order, a.pt, a.n_segments, a.n_tokens, a.n_heads,
                     a.pos, a.nax, a.tab, a.max_pos, a.scale, a.scale * kLog2e, a.rcu, a.vfirst);
  hipError_t e = hipGetLastError();
  if constexpr (kMerged) {
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dq_kernel<D, TOut, true, QT, KT>), dim3(static_cast<unsigned>(blocks)), dim3(QT / 32 * 64),
                       0, stream, static_cast<const uint16_t*>(qr), static_cast<const uint16_t*>(kr),
                       static_cast<const uint16_t*>(vb), static_cast<const uint16_t*>(dob),
                       static_cast<const TOut*>(o), static_cast<const TOut*>(dout), lse, lse2, delta,
                       static_cast<TOut*>(dq), a.cu_seqlens, a.order, a.pt, a.n_segments, a.n_tokens, a.n_heads,
                       a.pos, a.nax, a.tab, a.max_pos, a.scale, a.scale * kLog2e, a.rcu, a.vfirst);
    e = hipGetLastError();
  }
  return e;
}

// The merged shape runs exactly when the call merged tiny segments (vfirst
// set); its schedule was built with kDqTileMerged.
template <int D, typename TOut>
hipError_t launch_dq_any(const AttnArgs& a, const void* qr, const void* kr, const void* vb, const void* dob,
                         const void* o, const void* dout, const float* lse, float* lse2, float* delta, void* dq,
                         hipStream_t stream) {
  if (a.vfirst != nullptr)
    return launch_dq_t<D, TOut, kDqTileMerged, 32, true>(a, qr, kr, vb, dob, o, dout, lse, lse2, delta, dq, stream);
  return launch_dq_t<D, TOut, kDqTile, 64, false>(a, qr, kr, vb, dob, o, dout, lse, lse2, delta, dq, stream);
}

}  // namespace

hipError_t launch_attn_bwd_dkdv(const AttnArgs& a, const void* qr, const void* kr, const void* vb, const void* dob,
                                const float* lse, const float* delta, void* dk, void* dv, hipStream_t stream) {
  if (a.head_dim == 128)
    return a.dtype == kDtypeBf16 ? launch_dkdv_t<128, uint16_t>(a, qr, kr, vb, dob, lse, delta, dk, dv, stream)
                                 : launch_dkdv_t<128, float>(a, qr, kr, vb, dob, lse, delta, dk, dv, stream);
  return a.dtype == kDtypeBf16 ? launch_dkdv_t<64, uint16_t>(a, qr, kr, vb, dob, lse, delta, dk, dv, stream)
                               : launch_dkdv_t<64, float>(a, qr, kr, vb, dob, lse, delta, dk, dv, stream);
}

hipError_t launch_attn_bwd_dq(const AttnArgs& a, const void* qr, const void* kr, const void* vb, const void* dob,
                              const void* o, const void* dout, const float* lse, float* lse2, float* delta, void* dq,
                              hipStream_t stream) {
  if (a.head_dim == 128)
    return a.dtype == kDtypeBf16
               ? launch_dq_any<128, uint16_t>(a, qr, kr, vb, dob, o, dout, lse, lse2, delta, dq, stream)
               : launch_dq_any<128, float>(a, qr, kr, vb, dob, o, dout, lse, lse2, delta, dq, stream);
  return a.dtype == kDtypeBf16
             ? launch_dq_any<64, uint16_t>(a, qr, kr, vb, dob, o, dout, lse, lse2, delta, dq, stream)
             : launch_dq_any<64, float>(a, qr, kr, vb, dob, o, dout, lse, lse2, delta, dq, stream);
}

}  // namespace mf

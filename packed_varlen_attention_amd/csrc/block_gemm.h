// The 256 x 256 tile matrix product shared by the attention sub-block's
// projections (forward and backward), and the row tiling of the packed
// stream by pieces.
//
// Rows are tokens in packed order; cu_pieces splits them into pieces of
// frames + 1 per sample (the first piece of a sample is its text, the others
// image grids).  A projection tiles each piece's rows separately, so a tile
// never mixes modalities and takes one weight matrix.
#pragma once

#include "mf_device.h"

namespace mf {
namespace {

constexpr int kPT = 256;     // token rows per projection tile
constexpr int kFT = 256;     // output features per projection tile
constexpr int kKS = 32;      // reduction slice per pipeline step (one 64-byte LDS row)
constexpr int kStages = 4;   // LDS stages; copies run three steps ahead
constexpr int kPWaves = 8;   // (kPWaves / 2) x 2 waves, each kWaveRows tokens x 128 features
constexpr int kXcds = 8;     // workgroups are dealt round-robin to the XCDs
constexpr int kWaveRows = 256 / (kPWaves / 2);  // token rows per wave
constexpr int kMB = kWaveRows / 32;              // 32-row MFMA blocks per wave

using TileCopy256 = TileCopy<kKS, 256, kPWaves>;

// Wait until at most N (0..63) of this wave's global loads are outstanding:
// vmcnt's low four bits sit in bits 3:0 of the immediate, its high two in
// bits 15:14 (expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmem_keep_upto63() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 0..63");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Rows of piece i, clamped to [0, n_tokens] (cu_pieces is device data the
// host cannot check; a malformed one yields empty pieces, never a read past
// the tensors).
__device__ __forceinline__ void piece_rows(const int* __restrict__ cp, int i, int n_tokens, int& a, int& e) {
  a = min(max(cp[i], 0), n_tokens);
  e = min(max(cp[i + 1], a), n_tokens);
}

// Index p with tstart[p] <= t < tstart[p + 1] among the m pieces (tstart is
// non-decreasing and t < tstart[m]).
__device__ __forceinline__ int piece_of_tile(const int* __restrict__ tstart, int m, int t) {
  int lo = 0, hi = m;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (tstart[mid] <= t) lo = mid; else hi = mid;
  }
  return lo;
}

// Feature tiles per scheduling window: 4 when they divide the tile count.
__host__ __device__ __forceinline__ int window_cols(int n_ntiles) {
  return n_ntiles % 4 == 0 ? 4 : n_ntiles % 2 == 0 ? 2 : 1;
}

// Workgroups are dealt to the XCDs round-robin, so blocks b, b + 8, b + 16,
// ... run together on one XCD.  Each run of 32 such blocks is a window of
// (32 / nw) row tiles x nw feature tiles: the XCD's L2 then serves 12
// distinct operand tiles (8 + 4 with nw = 4) to 32 workgroups, not 33 with
// one row tile and 32 feature tiles.
__device__ __forceinline__ void window_tile(int b, int n_ntiles, int& mt, int& nt) {
  const int nw = window_cols(n_ntiles), mw = 32 / nw;
  const int x = b % kXcds, r = b / kXcds;
  const int win = (r / 32) * kXcds + x, p = r % 32;
  const int n_ntg = n_ntiles / nw;
  nt = (win % n_ntg) * nw + p / mw;
  mt = (win / n_ntg) * mw + p % mw;
}

// Blocks of a window grid covering mtiles x n_ntiles tiles (a multiple of
// 8 x 32, so the XCD of a block is the same in every such grid).
__host__ inline long long window_blocks(int mtiles, int n_ntiles) {
  const int nw = window_cols(n_ntiles), mw = 32 / nw;
  const long long wins = static_cast<long long>((mtiles + mw - 1) / mw) * (n_ntiles / nw);
  return (wins + kXcds - 1) / kXcds * kXcds * 32;
}

// acc += the product of one 256-row tile R (the MFMA B operand, "token"
// rows) and one 256-row tile W (the A operand, "feature" rows) over nsteps
// 32-wide reduction slices (nsteps a positive multiple of 4).
// load(ks, r_tile, w_tile) issues this wave's copies of slice ks of both
// tiles, kCopies in all.  The accumulator holds the transposed tile: lane
// element e of block (mb, nb) is feature 128 wn + 32 nb + 8 (e/4) + 4 (lane/32)
// + e%4 of row kWaveRows wm + 32 mb + lane%32 -- four consecutive features per
// lane.
template <int kCopies, class Load, class Epi>
__device__ __forceinline__ void tile_gemm(int nsteps, int wm, int wn, int lane, const Load& load,
                                          f32x16 (&acc)[kMB][4], const Epi& epi) {
  constexpr int kTileBytes = 256 * kKS * 2;  // 256 rows of 64 bytes
  // Four stages of a row tile and a feature tile, as separate objects so the
  // compiler can tell the stage being read from stages being filled.
  __shared__ __attribute__((aligned(16))) char smemA0[kTileBytes];
  __shared__ __attribute__((aligned(16))) char smemA1[kTileBytes];
  __shared__ __attribute__((aligned(16))) char smemA2[kTileBytes];
  __shared__ __attribute__((aligned(16))) char smemA3[kTileBytes];
  __shared__ __attribute__((aligned(16))) char smemB0[kTileBytes];
  __shared__ __attribute__((aligned(16))) char smemB1[kTileBytes];
  __shared__ __attribute__((aligned(16))) char smemB2[kTileBytes];
  __shared__ __attribute__((aligned(16))) char smemB3[kTileBytes];
  lds_char* const sA[kStages] = {(lds_char*)smemA0, (lds_char*)smemA1, (lds_char*)smemA2, (lds_char*)smemA3};
  lds_char* const sB[kStages] = {(lds_char*)smemB0, (lds_char*)smemB1, (lds_char*)smemB2, (lds_char*)smemB3};
  const int hh = lane >> 5;
  // Stage ks lives in buffer ks % 4.  Every step issues the copies of stage
  // ks + 3 (past the end: the last slice again, into a buffer no later step
  // reads), so the wait for stage ks + 1 keeps a fixed count in flight.
  auto load_stage = [&](int ks, int buf) { load(min(ks, nsteps - 1), sA[buf], sB[buf]); };

  // Row fragments: the chunk swizzle of Tile<32> depends on (row / 2) % 4,
  // the same for every 32-row block, so one offset per reduction step kk.
  const int r32 = lane & 31;
  int off[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) off[kk] = Tile<kKS>::off(r32, 2 * kk + hh);
  auto frag = [&](const lds_char* t, int row0, int kk) {
    return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(t + off[kk] + row0 * (kKS * 2));
  };

  auto step = [&](int ks, auto buf_tag) {
    constexpr int bf = decltype(buf_tag)::value;
    load_stage(ks + 3, (bf + 3) % kStages);
    const lds_char* A = sA[bf];
    const lds_char* B = sB[bf];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 tf[kMB], wf[4];
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) tf[mb] = frag(A, kWaveRows * wm + 32 * mb, kk);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) wf[nb] = frag(B, 128 * wn + 32 * nb, kk);
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = mfma32(wf[nb], tf[mb], acc[mb][nb]);
    }
    // Stage ks + 1 has landed once only the two newest stages' copies are
    // outstanding (copies complete in issue order).
    wait_vmem_keep_upto63<2 * kCopies>();
    barrier_keep_loads();
  };
  load_stage(0, 0);
  load_stage(1, 1);
  load_stage(2, 2);
  wait_vmem_keep_upto63<2 * kCopies>();
  barrier_keep_loads();
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  using B3 = std::integral_constant<int, 3>;
  for (int ks = 0; ks < nsteps; ks += 4) {
    step(ks, B0{});
    step(ks + 1, B1{});
    step(ks + 2, B2{});
    step(ks + 3, B3{});
  }
  // The trailing copies land, and every wave is done with every stage, before
  // the epilogue takes one 16 KB stage buffer per wave.
  wait_vmem();
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // constant indices only: a runtime index would put the pointer arrays in scratch
  lds_char* wbuf = sA[0];
#pragma unroll
  for (int i = 1; i < kStages; ++i)
    if (wave == i) wbuf = sA[i];
#pragma unroll
  for (int i = 0; i < kStages; ++i)
    if (wave == kStages + i) wbuf = sB[i];
  epi(wbuf);
}

// A wave's 64-row x 128-feature block of bf16 results, staged through the
// wave's own 16 KB LDS buffer so that the global stores are whole 256-byte
// row segments instead of 16 bytes in each of 32 rows.  put() takes the four
// consecutive features a lane holds (accumulator order); flush() stores each
// row with 16 lanes x 16 bytes.  The 16-byte units of a row are XOR-swizzled
// by the row, which spreads both access orders over the banks.
struct WaveStage {
  lds_char* buf;
  __device__ __forceinline__ void put(int row, int unit, int half, u32x2 v) const {
    *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(buf + row * 256 + ((unit ^ (row & 15)) * 16) +
                                                                   half * 8) = v;
  }
  __device__ __forceinline__ u32x2 get(int row, int unit, int half) const {
    return *reinterpret_cast<const __attribute__((address_space(3))) u32x2*>(buf + row * 256 +
                                                                             ((unit ^ (row & 15)) * 16) + half * 8);
  }
  // The block's rows < rows from global memory (src(row) = first of the row's
  // 128 bf16), 16 lanes x 16 bytes a row, into the staged layout.
  template <class Src>
  __device__ __forceinline__ void fill(int lane, int rows, const Src& src) const {
    const int unit = lane & 15;
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const int row = 4 * i + (lane >> 4);
      if (row < rows)
        *reinterpret_cast<__attribute__((address_space(3))) u32x4*>(buf + row * 256 + ((unit ^ (row & 15)) * 16)) =
            *reinterpret_cast<const u32x4*>(src(row) + unit * 8);
    }
  }
  // store(row, feature, u32x4 of 8 bf16) for every row < rows of the block
  template <class Store>
  __device__ __forceinline__ void flush(int lane, int rows, const Store& store) const {
    const int unit = lane & 15;
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const int row = 4 * i + (lane >> 4);
      if (row < rows) {
        const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
            buf + row * 256 + ((unit ^ (row & 15)) * 16));
        store(row, unit * 8, v);
      }
    }
  }
};

// The fp32 counterpart for half a wave's block (32 rows x 128 features, 512
// bytes a row, the lane's four features one 16-byte unit): flush() stores
// each row with 32 lanes x 16 bytes.
struct WaveStageF32 {
  lds_char* buf;
  __device__ __forceinline__ void put(int row, int unit, const f32x4& v) const {
    *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(buf + row * 512 + ((unit ^ (row & 31)) * 16)) = v;
  }
  template <class Store>
  __device__ __forceinline__ void flush(int lane, const Store& store) const {
    const int unit = lane & 31;
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const int row = 2 * i + (lane >> 5);
      const f32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
          buf + row * 512 + ((unit ^ (row & 31)) * 16));
      store(row, unit * 4, v);
    }
  }
};

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[kMB][4]) {
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mb][nb][i] = 0.f;
}

}  // namespace
}  // namespace mf

// Device-side building blocks shared by the gfx950 kernels of this library:
// vector types, bf16 conversion, the 32x32x16 bf16 MFMA, and LDS tile
// addressing with the fragment loads the attention kernels feed to it.
//
// MFMA v_mfma_f32_32x32x16_bf16 operand layout (wave64, h = lane / 32):
//   A (32 x 16, M x K): lane holds A[m = lane % 32][k = 8h .. 8h + 7]
//   B (16 x 32, K x N): lane holds B[k = 8h .. 8h + 7][n = lane % 32]
//   C (32 x 32):        lane element i holds C[m = 8(i/4) + 4h + i%4][n = lane % 32]
//
// ds_read_b64_tr_b16 (LDS transpose read): inside each group of 16 lanes,
// lane i receives, in slot t, element (i % 4) of the 8 bytes fetched by lane
// 4t + i/4 of the same group.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) char lds_char;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 bits (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16_bits(lo)) |
         (static_cast<uint32_t>(f32_to_bf16_bits(hi)) << 16);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row permutation applied to A operands loaded from LDS: swaps bits 2 and 3
// of the row index.  With it, accumulator element i of lane (h = lane / 32)
// belongs to tile row 16(i/8) + 8h + (i % 8): each lane then holds 8
// consecutive rows per 16-row chunk, exactly the K-operand fragment of the
// next product, so no cross-lane shuffle is needed between the two products.
__device__ __forceinline__ int perm32(int m) {
  return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Tile row of accumulator element i for lane half h (after perm32 rows).
__device__ __forceinline__ int acc_row(int i, int h) { return 16 * (i >> 3) + 8 * h + (i & 7); }

// Masks the 8 accumulator elements of group g (elements 8g .. 8g + 7, the
// rows acc_row(8g + c, h) = 16g + 8h + c of a 32-row block): element c is set
// to `fill` unless lo <= c < hi.  Built from bit tests instead of compares, so
// it holds no lane masks in scalar registers.
__device__ __forceinline__ void mask_rows8_range(f32x16& acc, int g, int lo, int hi, float fill) {
  const unsigned keep_bits = ((1u << min(max(hi, 0), 8)) - 1u) & ~((1u << min(max(lo, 0), 8)) - 1u);
  const int fill_bits = __float_as_int(fill);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int keep = static_cast<int>(keep_bits << (31 - c)) >> 31;  // 0 or -1
    acc[8 * g + c] = __int_as_float((__float_as_int(acc[8 * g + c]) & keep) | (fill_bits & ~keep));
  }
}

__device__ __forceinline__ void mask_rows8(f32x16& acc, int g, int valid, float fill) {
  mask_rows8_range(acc, g, 0, valid, fill);
}

// For a virtual segment [s0, s1) made of real segments f0 .. f1 - 1 (cu:
// their offsets), the bounds [lo, hi) relative to s0 of the real segment that
// holds token s0 + t: a row of a multi-segment tile meets only these rows.
__device__ __forceinline__ void member_bounds(const int* __restrict__ cu, int f0, int f1, int s0, int s1, int t,
                                              int& lo, int& hi) {
  const int tok = s0 + t;
  int a = f0, b = f1;
  while (b - a > 1) {
    const int mid = (a + b) >> 1;
    if (cu[mid] <= tok) a = mid; else b = mid;
  }
  lo = min(max(cu[a], s0), s1) - s0;
  hi = min(max(cu[a + 1], s0 + lo), s1) - s0;
}

// A [rows][D] bf16 tile in LDS, rows of D*2 bytes, 16-byte chunks XOR-swizzled
// per row so that both row-fragment and transpose reads spread over banks.
template <int D>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;
  __device__ static __forceinline__ int swz(int row) {
    if constexpr (D == 128) {
      return ((row & 3) << 2) | ((row >> 2) & 3);
    } else if constexpr (D == 64) {
      return (row >> 1) & 7;
    } else {
      static_assert(D == 32, "tiles of 32, 64 or 128 bf16 per row");
      return (row >> 1) & 3;  // 64-byte rows: 8 consecutive rows cover all banks
    }
  }
  __device__ static __forceinline__ int off(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ swz(row)) << 4);
  }
};

// A-operand fragment of rows [rbase, rbase + 32) (perm32 applied), columns
// 16*kk + 8h .. +8:  X[rbase + perm32(lane % 32)][16 kk + 8h + j].
template <int D>
__device__ __forceinline__ bf16x8 lds_row_frag(const lds_char* tile, int rbase, int kk, int lane) {
  const int row = rbase + perm32(lane & 31);
  const int chunk = 2 * kk + (lane >> 5);
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(tile + Tile<D>::off(row, chunk));
}

// Transposed fragment: X[rbase + 8h + j][dbase + lane % 32] for j = 0..7, as
// the A operand of a product that reduces over rows (or its B operand with
// the roles of m and n exchanged).  Two transpose reads of 4 rows each.
template <int D>
__device__ __forceinline__ bf16x8 lds_col_frag(const lds_char* tile, int rbase, int dbase, int lane) {
  const int g = lane >> 4;
  const int l16 = lane & 15;
  const int h = lane >> 5;
  const int col = dbase + 16 * (g & 1) + 4 * (l16 & 3);
  const int chunk = col >> 3;
  const int half = (col >> 2) & 1;
  const int row0 = rbase + 8 * h + (l16 >> 2);
  const lds_char* p0 = tile + Tile<D>::off(row0, chunk) + half * 8;
  const lds_char* p1 = tile + Tile<D>::off(row0 + 4, chunk) + half * 8;
  i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) i16x4*>(const_cast<lds_char*>(p0)));
  i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) i16x4*>(const_cast<lds_char*>(p1)));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Asynchronous copies of a [kRows][D] bf16 tile from a row-strided global
// matrix straight into a swizzled LDS tile (global_load_lds_dwordx4: lane i
// of a wave lands its 16 bytes at the wave's LDS base + 16 i, so a copy
// instruction fills 1 KB = kRowsPerInst whole rows; the swizzle is applied by
// choosing which global chunk each lane fetches).
//
// Copy r of wave w fills tile rows kStride r + kRowsPerInst w + lane / (D/8),
// kStride = kRowsPerInst * kWaves.  kStride is a multiple of the swizzle's
// 16-row period, so all copies of a lane fetch the same chunk.  The source
// is a block-uniform tile base (scalar registers) plus a 32-bit lane offset
// per copy; rows at or past `valid` re-read row valid - 1 (the caller masks
// what they feed), a clamp taken on the byte offset itself:
// min(row pitch + chunk, last pitch + chunk) = min(row, last) pitch + chunk,
// so each copy costs a lane one add and one min.  The caller waits on
// vmcnt, then a barrier, before the tile is read.
template <int D, int kRows, int kWaves>
struct TileCopy {
  static constexpr int kRowsPerInst = 1024 / (D * 2);
  static constexpr int kStride = kRowsPerInst * kWaves;
  static constexpr int kCopies = kRows / kStride;  // copy instructions per wave and tile
  static_assert(kCopies >= 1 && kRows % kStride == 0, "tile rows must split evenly over the waves");
  static_assert(kStride % 16 == 0, "the chunk swizzle repeats every 16 rows");

  unsigned off0;   // byte offset of this lane's chunk in copy 0, from the tile's first row
  unsigned chunk;  // byte offset of the lane's swizzled 16-byte chunk inside a row
  unsigned pitch;  // bytes per matrix row, below 2^24
  int wave;        // wave-uniform

  __device__ __forceinline__ TileCopy(int wave_, int lane, unsigned pitch_) : pitch(pitch_), wave(wave_) {
    const int row = wave * kRowsPerInst + lane / (D / 8);
    chunk = static_cast<unsigned>((lane % (D / 8)) ^ Tile<D>::swz(row)) * 16u;
    off0 = static_cast<unsigned>(row) * pitch + chunk;
  }
  // Copy matrix rows [r0, r0 + kRows) of `base` into `tile`; 0 <= r0 < valid.
  __device__ __forceinline__ void operator()(const void* base, int r0, int valid, lds_char* tile) const {
    const char* src = static_cast<const char*>(base) + static_cast<size_t>(r0) * pitch;  // block-uniform
    // Only this tile's rows are ever addressed, so the clamp row is bounded by
    // the tile height: (kRows - 1) * pitch + chunk stays below 2^32.
    const unsigned last = static_cast<unsigned>(min(valid - 1 - r0, kRows - 1)) * pitch + chunk;
#pragma unroll
    for (int r = 0; r < kCopies; ++r) {
      unsigned o = min(off0 + static_cast<unsigned>(r * kStride) * pitch, last);
      // Opaque to the optimiser, so the add stays a 32-bit lane offset on a
      // scalar base instead of being folded into a 64-bit per-lane select.
      asm("" : "+v"(o));
      __builtin_amdgcn_global_load_lds(src + o, tile + (r * kWaves + wave) * 1024, 16, 0, 0);
    }
  }
};

// Wait until this wave's outstanding global loads (including loads into LDS)
// have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wave's global loads are outstanding.  Loads
// complete in issue order, so this waits for all but the N most recent.
template <int N>
__device__ __forceinline__ void wait_vmem_keep() {
  static_assert(N >= 0 && N < 16, "vmcnt field holds 0..15 here");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Workgroup barrier that leaves this wave's newest loads into LDS in flight.
// __syncthreads() fences memory, and its fence waits for every outstanding
// copy into LDS; here the caller has already waited (wait_vmem_keep) for the
// copies other waves will read next.  This waits for the wave's own LDS
// accesses, then synchronises; the memory clobber keeps the compiler from
// moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_keep_loads() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
  asm volatile("s_barrier" ::: "memory");
}

// One unit of attention work: a tile of one (segment, head).
struct WorkItem {
  int seg, head, tile;
};

// Decodes block b of an attention launch against the schedule written by
// the scheduling kernel (order[r]: segment of rank r, longest first; pt[r]:
// exclusive prefix of tile counts in rank order).  XCD x = b % 8 owns heads
// x, x + 8, ...; its i-th block (i = b / 8) walks ranks, then its heads, then
// tiles.  Returns false for the blocks past the end of their XCD's list.
__device__ __forceinline__ bool decode_item(int b, int heads, int n_seg, const int* __restrict__ order,
                                            const int* __restrict__ pt, WorkItem& w) {
  const int x = b & 7;
  const int i = b >> 3;
  const int nx = (heads - x + 7) >> 3;
  if (nx <= 0) return false;
  const int total = pt[n_seg];
  if (static_cast<long long>(i) >= static_cast<long long>(nx) * total) return false;
  int lo = 0, hi = n_seg;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (static_cast<long long>(pt[mid]) * nx <= i) lo = mid; else hi = mid;
  }
  const int tiles = pt[lo + 1] - pt[lo];
  const int j = i - pt[lo] * nx;
  w.seg = order[lo];
  w.head = x + 8 * (j / tiles);
  w.tile = j % tiles;
  return true;
}

__device__ __forceinline__ void seg_bounds(const int* __restrict__ cu, int seg, int n_tokens, int& s0, int& s1) {
  s0 = cu[seg];
  s1 = cu[seg + 1];
  s0 = min(max(s0, 0), n_tokens);
  s1 = min(max(s1, s0), n_tokens);
}

// Load 8 consecutive elements of a bf16 or f32 row as float.
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&x)[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&x)[8]) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = __uint_as_float(v[j] << 16);
    x[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = a[j];
    x[4 + j] = b[j];
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&x)[8]);

template <>
__device__ __forceinline__ void store8<uint16_t>(uint16_t* p, const float (&x)[8]) {
  u32x4 v;
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = pack_bf16x2(x[2 * j], x[2 * j + 1]);
  *reinterpret_cast<u32x4*>(p) = v;
}

template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&x)[8]) {
  f32x4 a, b;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a[j] = x[j];
    b[j] = x[4 + j];
  }
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}

// Store 4 consecutive elements.
template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);

template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* p, float a, float b, float c, float d) {
  u32x2 v;
  v[0] = pack_bf16x2(a, b);
  v[1] = pack_bf16x2(c, d);
  *reinterpret_cast<u32x2*>(p) = v;
}

template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(p) = v;
}

// Position of one token on up to three axes: row, column, frame.
struct Pos3 {
  int r, c, f;
};

// Positions are [n][nax] int32: nax = 2 (row, col) for the axial 2D
// rotation, nax = 3 (row, col, frame) for the frame-aware 3D rotation.
__device__ __forceinline__ Pos3 load_pos(const int* __restrict__ pos, long long t, int nax) {
  Pos3 p;
  if (nax == 3) {
    p.r = pos[3 * t];
    p.c = pos[3 * t + 1];
    p.f = pos[3 * t + 2];
  } else {
    const int2 q = reinterpret_cast<const int2*>(pos)[t];
    p.r = q.x;
    p.c = q.y;
    p.f = 0;
  }
  return p;
}

// Rotary layout.  2D: dims [0, D/2) turn by the row and [D/2, D) by the
// column; the table row of a position holds D/4 (cos, sin) pairs, pair j of
// each half at p * theta^(-2j/(D/2)).  3D: blocks [0, 3D/8) row, [3D/8, 3D/4)
// column, [3D/4, D) frame; the table row holds the 3D/16 pairs of a row or
// column block (p * theta^(-2j/(3D/8))) followed by the D/8 pairs of the
// frame block (p * theta^(-2j/(D/4))).  Every block is a multiple of 8 dims,
// so one 8- or 4-element group never straddles two blocks.
template <int D>
__host__ __device__ constexpr int rope_tab_width(int nax) {
  return nax == 3 ? 3 * D / 16 + D / 8 : D / 4;
}

// Table entry of the first pair of the group starting at element e0, and the
// position along that group's axis.
template <int D>
__device__ __forceinline__ const float2* rope_entry(int e0, const Pos3& p, const float2* __restrict__ tab,
                                                   int max_pos, int nax) {
  int axis, j0;
  if (nax == 3) {
    constexpr int kB = 3 * D / 8;
    axis = e0 < kB ? 0 : (e0 < 2 * kB ? 1 : 2);
    j0 = axis == 2 ? kB / 2 + (e0 - 2 * kB) / 2 : (e0 - axis * kB) / 2;
  } else {
    axis = e0 / (D / 2);
    j0 = (e0 % (D / 2)) / 2;
  }
  int q = axis == 0 ? p.r : (axis == 1 ? p.c : p.f);
  q = q < 0 ? 0 : (q >= max_pos ? max_pos - 1 : q);
  return tab + static_cast<size_t>(q) * rope_tab_width<D>(nax) + j0;
}

// Rotate N consecutive elements x[0..N-1] (N = 4 or 8, two or four pairs) of
// one head row starting at element e0 (a multiple of N) by the rotation of
// position p.  sign = +1 forward, -1 inverse.
template <int D, int N>
__device__ __forceinline__ void rotate_n(float (&x)[N], int e0, const Pos3& p, const float2* __restrict__ tab,
                                         int max_pos, float sign, int nax) {
  const float2* t = rope_entry<D>(e0, p, tab, max_pos, nax);
#pragma unroll
  for (int j = 0; j < N / 2; ++j) {
    const float2 cs = t[j];
    const float c = cs.x;
    const float s = sign * cs.y;
    const float a = x[2 * j];
    const float b = x[2 * j + 1];
    x[2 * j] = a * c - b * s;
    x[2 * j + 1] = a * s + b * c;
  }
}

}  // namespace mf

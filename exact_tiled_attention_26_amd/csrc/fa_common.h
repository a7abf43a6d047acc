// Device helpers shared by the attention kernels (gfx950 / CDNA4 only).
//
// MFMA lane layouts used throughout (wave64, lane l, g = l / 16):
//   v_mfma_f32_16x16x32_bf16  A[m][k]: lane holds m = l % 16, k = 8g .. 8g+7
//                             B[k][n]: lane holds n = l % 16, k = 8g .. 8g+7
//                             C[m][n]: lane holds n = l % 16, m = 4g .. 4g+3
//   v_mfma_f32_16x16x4_f32    A: m = l % 16, k = g;  B: n = l % 16, k = g;
//                             C as above.
// A contraction only needs A and B to agree on which k each (lane group,
// slot) carries, so the kernels feed an accumulator tile of one product
// straight into the next product as an operand, with the k order that the
// accumulator layout gives (no register shuffles).
//
// ds_read_b64_tr_b16: inside each 16-lane group, lane i supplies the address
// of 4 consecutive 16-bit elements in row (i / 4) of a 4 x 16 block (column
// offset 4 * (i % 4)); lane n receives column n of that block (rows 0..3).
// That reads a column-major operand (k down the rows of a row-major tile)
// directly from LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) {  // v_exp_f32; exp2(-inf) = 0
  return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float wave_max_xor16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float wave_sum_xor16_32(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Pack two 4-float accumulator fragments into one bf16x8 operand
// (round to nearest even).
__device__ __forceinline__ bf16x8 pack_bf16(const f32x4& lo, const f32x4& hi) {
  bf16x8 r;
  r[0] = (__bf16)lo[0]; r[1] = (__bf16)lo[1]; r[2] = (__bf16)lo[2]; r[3] = (__bf16)lo[3];
  r[4] = (__bf16)hi[0]; r[5] = (__bf16)hi[1]; r[6] = (__bf16)hi[2]; r[7] = (__bf16)hi[3];
  return r;
}

__device__ __forceinline__ bf16x8 cat(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------------------
// bf16 tiles in LDS: [rows][D] elements stored in 16-byte chunks, chunk c of
// row r placed at chunk position c ^ sigma(r), with
//   sigma(r) = 2 * (r mod H) + ((r / H) mod 2),  H = D / 16.
// sigma is a permutation of the D/8 chunk positions over any D/8 consecutive
// rows (a 16-lane natural read of one chunk from 16 rows hits distinct
// positions when D = 128), and sigma / 2 is distinct over H consecutive rows
// (the 8 rows x 2 chunks of a transposed read spread over all positions).
// ---------------------------------------------------------------------------
template <int D>
struct SwzTile {
  static constexpr int NCH = D / 8;
  static constexpr int H = D / 16;
  __device__ __forceinline__ static int chunk_pos(int r, int c) {
    return c ^ (2 * (r % H) + ((r / H) & 1));
  }
  // element offset of (row, col)
  __device__ __forceinline__ static int off(int r, int col) {
    return r * D + (chunk_pos(r, col >> 3) << 3) + (col & 7);
  }
};

// 8 consecutive bf16 (one 16-byte chunk) at logical (row, 8 * chunk).
template <int D>
__device__ __forceinline__ bf16x8 lds_read_chunk(const __bf16* tile, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(tile + SwzTile<D>::off(row, chunk * 8));
}

// Transposed read of a 4 x 16 block of a row-major tile: every lane of a
// 16-lane group passes the same `row` and `col0`; lane `lane16` of the group
// receives the 4 elements of column col0 + lane16 in rows row .. row+3.
template <int D>
__device__ __forceinline__ bf16x4 lds_read_tr4(const __bf16* tile, int row, int col0, int lane16) {
  const __bf16* p = tile + SwzTile<D>::off(row + (lane16 >> 2), col0 + 4 * (lane16 & 3));
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)(p));
}

// Copy `rows` x D bf16 rows (global row-major, row stride D) into a swizzled
// LDS tile with the whole workgroup; rows at or past `valid` are zero-filled.
// Staging through registers: `load` fills regs, `store` writes them.
template <int D, int ROWS, int NTHREADS>
struct TileCopy {
  static constexpr int NCH = D / 8;
  static constexpr int CHUNKS = ROWS * NCH;
  static constexpr int PER_THREAD = (CHUNKS + NTHREADS - 1) / NTHREADS;
  static_assert(CHUNKS % NTHREADS == 0, "tile chunks must divide evenly over threads");
  u32x4 reg[PER_THREAD];

  __device__ __forceinline__ void load(const __bf16* g, int valid, int tid) {
#pragma unroll
    for (int it = 0; it < PER_THREAD; ++it) {
      const int u = tid + it * NTHREADS;
      const int r = u / NCH, c = u % NCH;
      if (r < valid) {
        reg[it] = *reinterpret_cast<const u32x4*>(g + (size_t)r * D + c * 8);
      } else {
        reg[it] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(__bf16* tile, int tid) const {
#pragma unroll
    for (int it = 0; it < PER_THREAD; ++it) {
      const int u = tid + it * NTHREADS;
      const int r = u / NCH, c = u % NCH;
      *reinterpret_cast<u32x4*>(tile + r * D + (SwzTile<D>::chunk_pos(r, c) << 3)) = reg[it];
    }
  }
};

}  // namespace fa

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

#include "fa_order.h"

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

// Max over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48) with
// the gfx950 row-swap instructions: permlane32_swap(x, x) returns x of the
// lower half in both halves of its first result and x of the upper half in
// both halves of its second, permlane16_swap likewise for adjacent rows.  No
// LDS traffic, so the LDS counter is left to the operand reads.
__device__ __forceinline__ float wave_max_rows(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float wave_sum_xor16_32(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// A zero that the compiler must treat as a per-lane value.  Added to the
// bounds that select between copies of a software-pipelined loop body, it
// makes those branches divergent in the compiler's eyes (they are uniform in
// fact): with provably uniform conditions the compiler moves work between
// the copies and runs out of registers.
__device__ __forceinline__ int divergent_zero() {
  int z;
  __asm__ volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// Lower edge of the visible keys: key j is hidden from query i when
// j <= i + lo.  Without a window no key is hidden from below.
__device__ __forceinline__ int window_lo(bool causal, int off, int window) {
  return (causal && window > 0) ? off - window : -(1 << 30);
}

// Pack two 4-float accumulator fragments into one bf16x8 operand
// (round to nearest even).
__device__ __forceinline__ bf16x8 pack_bf16(const f32x4& lo, const f32x4& hi) {
  bf16x8 r;
  r[0] = (__bf16)lo[0]; r[1] = (__bf16)lo[1]; r[2] = (__bf16)lo[2]; r[3] = (__bf16)lo[3];
  r[4] = (__bf16)hi[0]; r[5] = (__bf16)hi[1]; r[6] = (__bf16)hi[2]; r[7] = (__bf16)hi[3];
  return r;
}

// -x of eight bf16 values (sign bits flipped: exact)
__device__ __forceinline__ bf16x8 neg_bf16(const bf16x8& x) {
  const u32x4 u = __builtin_bit_cast(u32x4, x) ^ 0x80008000u;
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 cat(const bf16x4& lo, const bf16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------------------
// bf16 tiles in LDS: [rows][D] elements in 16-byte chunks (D/8 per row, no
// padding).  Chunk c of row r is stored at chunk position c ^ sigma(r).
//
// gfx950 LDS, as measured with SQ_LDS_BANK_CONFLICT on probe kernels: 64
// banks of 4 bytes (256 bytes per clock).  ds_read_b128 serves 16 lanes per
// clock, the lanes that agree on lane bit 5 and on the parity of lane bits
// 2..4; ds_read_b64_tr_b16 serves 32 consecutive lanes per clock.  The two
// reads every operand tile sees are
// * natural: lane (g = lane / 16, l16 = lane % 16) reads chunk 4 ds + g of
//   row R0 + l16 (R0 a multiple of 16);
// * transposed: lane (g, l16) reads half of chunk 2 db + (l16 / 2) % 2 of row
//   R0 + 4 g + l16 / 4.
// sigma below makes both conflict-free under that model for every ds, db
// and R0 (checked on the host, with the copy placement and the readers'
// offsets below, by tests/c_abi/swizzle_check.cpp): for D = 128, sigma(r) =
// (r mod 16) xor (12 (r mod 2)); for D = 64 (two rows per bank sweep),
// sigma(r) = r and 6.  The readers precompute one offset per ds / db step
// for each lane, so the unrolled loops read with immediate offsets only.
// ---------------------------------------------------------------------------
template <int D>
__host__ __device__ __forceinline__ int swz_sigma(int r) {
  static_assert(D == 64 || D == 128, "bf16 tiles are 64 or 128 wide");
  if constexpr (D == 128) return (r & 15) ^ (12 * (r & 1));
  else return r & 6;
}

// Element offset, in a swizzled tile, of the chunk that holds columns
// 8 c .. 8 c + 7 of row r.
template <int D>
__host__ __device__ __forceinline__ int swz_chunk(int r, int c) {
  return r * D + 8 * (c ^ swz_sigma<D>(r));
}

// Natural read of the operand "row R0 + l16, 8 elements at column 32 ds + 8 g"
// (R0 a multiple of 16).
template <int D>
struct NatReader {
  static constexpr int NDS = D / 32;
  // element offset that lane (g, l16) reads at step ds, for R0 = 0
  __host__ __device__ static int offset(int l16, int g, int ds) { return swz_chunk<D>(l16, 4 * ds + g); }
  int off[NDS];   // element offsets for R0 = 0
  __device__ __forceinline__ NatReader(int l16, int g) {
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) off[ds] = offset(l16, g, ds);
  }
  // r0 and ds must be compile-time constants after unrolling.
  __device__ __forceinline__ bf16x8 read(const __bf16* tile, int r0, int ds) const {
    return *reinterpret_cast<const bf16x8*>(tile + off[ds] + r0 * D);
  }
};

// Transposed read: lane (g, l16) receives the 4 elements of column
// 16 db + l16 in rows R0 + 4 g .. R0 + 4 g + 3 (R0 a multiple of 16).
// (The lanes of a 16-lane group give ds_read_b64_tr_b16 the rows of a 4 x 16
// block in order: lane j points at row j / 4, columns 4 (j mod 4) .. +3, and
// receives column j.)
template <int D>
struct TrReader {
  static constexpr int NDB = D / 16;
  // element offset that lane (g, l16) points at for column block db, R0 = 0
  __host__ __device__ static int offset(int l16, int g, int db) {
    const int row = 4 * g + (l16 >> 2);
    return swz_chunk<D>(row, 2 * db + ((l16 >> 1) & 1)) + 4 * (l16 & 1);
  }
  int off[NDB];
  __device__ __forceinline__ TrReader(int l16, int g) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) off[db] = offset(l16, g, db);
  }
  __device__ __forceinline__ bf16x4 read(const __bf16* tile, int r0, int db) const {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4*)(tile + off[db] + r0 * D));
  }
};

// HBM -> LDS copies without staging registers: global_load_lds_dwordx4
// writes the 16 bytes that lane i loads from gbase + byte_off to LDS address
// M0 + 16i; M0 holds the wave's LDS destination and must be
// written one wait state before the load.
//
// Two ways to issue them.  The compiler builtin lets the compiler see the
// copy; its wait-count analysis then treats the pending copy as an LDS
// access of unknown completion order and waits for every outstanding LDS
// read (lgkmcnt(0)) at each operand use.  The inline-assembly form below
// hides the copy: the compiler's own vmcnt waits only become stricter (the
// counter retires in issue order) and its lgkmcnt waits stay exact, and
// completion is the caller's job: async_copy_wait() and a barrier before any
// wave reads the data.  No other code here uses M0; the LDS address is the
// same in every lane and is read into a scalar register.  Which form is
// faster depends on the kernel's schedule (measured per kernel).
__device__ __forceinline__ unsigned lds_address(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
// lds_byte: the wave's LDS destination (byte address, uniform).  M0 is
// declared clobbered so that the compiler orders this copy against its own
// M0 writes (the builtin copies and other M0 readers) and never assumes M0
// survives it; clang warns that M0 is a reserved register, which is the
// point here, so that warning is silenced for this one statement.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* gbase, unsigned byte_off, unsigned lds_byte) {
  __asm__ volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                   :: "v"(byte_off), "s"(gbase), "s"(__builtin_amdgcn_readfirstlane(lds_byte)) : "memory", "m0");
}
#pragma clang diagnostic pop

// Asynchronous copy of a ROWS x D bf16 tile (global, row stride D) into a
// swizzled LDS tile with global_load_lds_dwordx4: lane i of a wave writes the
// 16 bytes at LDS chunk slot (base + i), so each lane fetches the global chunk
// that belongs at that slot.  The per-lane source offsets are fixed for a
// given tile shape, so they are computed once; a tile with fewer than ROWS
// valid rows re-reads its last valid row in place of the missing ones (finite
// values that the caller masks).  Every wave of the workgroup issues
// ROWS * D / 8 / 64 / NW instructions.
// HIDDEN selects the inline-assembly copy (see lds_dma16) over the builtin.
template <int D, int ROWS, int NW, bool HIDDEN = true>
struct AsyncTileCopy {
  static constexpr int NCH = D / 8;
  static constexpr int PER_WAVE = ROWS * NCH / 64 / NW;
  static_assert((ROWS * NCH / 64) % NW == 0, "tile must split evenly over the waves");
  int src_off[PER_WAVE];   // element offset of this lane's chunk in the global tile
  int lds_off[PER_WAVE];   // element offset of this wave's 64-chunk slot block (uniform)

  // element offset, in the global tile, of the chunk that LDS chunk slot p
  // receives (slot p sits at LDS element offset 8 p)
  __host__ __device__ static int source_offset(int p) {
    const int r = p / NCH;
    const int c = (p % NCH) ^ swz_sigma<D>(r);
    return r * D + c * 8;
  }
  __device__ __forceinline__ AsyncTileCopy(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int slot0 = (i * NW + wave) * 64;
      src_off[i] = source_offset(slot0 + lane);
      // uniform per wave: read into a scalar register once, so that no copy
      // needs a lane read to form its M0 value
      lds_off[i] = __builtin_amdgcn_readfirstlane(slot0 * 8);
    }
  }
  // Copy rows [0, ROWS) of the tile starting at g; `valid` >= 1 rows exist.
  // (the empty volatile statement in the partial-tile branch keeps the
  // compiler from merging the two branches into per-lane selects, which
  // would put the partial-tile arithmetic in front of every full-tile copy)
  __device__ __forceinline__ void issue(__bf16* tile, const __bf16* g, int valid) const {
    if (valid >= ROWS) {
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) issue_one(tile + lds_off[i], g, src_off[i]);
    } else {
      __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        const int row = src_off[i] / D;   // D is a power of two
        const int off = row < valid ? src_off[i] : src_off[i] - (row - valid + 1) * D;
        issue_one(tile + lds_off[i], g, off);
      }
    }
  }
  // Same as issue() with the tile given by its LDS byte address (uniform),
  // which spares the kernel a generic pointer per buffer.
  __device__ __forceinline__ void issue_at(unsigned tile_byte, const __bf16* g, int valid) const {
    if (valid >= ROWS) {
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) issue_one_at(tile_byte + 2u * lds_off[i], g, src_off[i]);
    } else {
      __asm__ volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) {
        const int row = src_off[i] / D;
        const int off = row < valid ? src_off[i] : src_off[i] - (row - valid + 1) * D;
        issue_one_at(tile_byte + 2u * lds_off[i], g, off);
      }
    }
  }
  __device__ __forceinline__ static void issue_one_at(unsigned lds_byte, const __bf16* g, int off) {
    if constexpr (HIDDEN) {
      lds_dma16(g, 2u * off, lds_byte);
    } else {
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)((const char*)g + 2u * (unsigned)off),
                                       (__attribute__((address_space(3))) void*)(uintptr_t)lds_byte, 16, 0, 0);
    }
  }
  __device__ __forceinline__ static void issue_one(__bf16* lds, const __bf16* g, int off) {
    if constexpr (HIDDEN) {
      lds_dma16(g, 2u * off, lds_address(lds));
    } else {
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)((const char*)g + 2u * (unsigned)off),
                                       (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
    }
  }
};

// Wait until this wave's asynchronous LDS copies have landed (the barrier
// that follows makes them visible to the workgroup).
__device__ __forceinline__ void async_copy_wait() { __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// ... all but the N most recently issued (the counter retires in issue order).
template <int N>
__device__ __forceinline__ void async_copy_wait_allbut() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  __asm__ volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

}  // namespace fa

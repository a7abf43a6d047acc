// Host-side check of the bf16 LDS tile layout (exact_tiled_attention_26_amd/
// csrc/fa_common.h): the placement of AsyncTileCopy, the offsets that
// NatReader and TrReader read, and the bank model stated there.
//  * copy: LDS chunk slot p receives global chunk source_offset(p); over a
//    tile this is a bijection onto the tile's chunks;
//  * natural read: lane (g, l16) at step ds finds row R0 + l16, columns
//    32 ds + 8 g .. +7 where the copy put them;
//  * transposed read: in each 16-lane group, lane j points at row R0 + 4 g +
//    j / 4, columns 16 db + 4 (j mod 4) .. +3 where the copy put them, so the
//    group's 4 x 16 block arrives transposed (lane j gets column 16 db + j);
//  * banks (64 banks of 4 bytes): the 16 lanes that a ds_read_b128 serves in
//    one clock (equal lane bit 5 and equal parity of lane bits 2..4) touch
//    64 different banks, and so do the 32 consecutive lanes that a
//    ds_read_b64_tr_b16 serves in one clock.
// Every tile height and row origin R0 (a multiple of 16) the kernels use is
// covered for D = 64 and 128.  Prints the number of lane accesses checked;
// exits nonzero on the first failure.
#include <cstdio>
#include <vector>

#include "../../exact_tiled_attention_26_amd/csrc/fa_common.h"

namespace {

long g_checked = 0;

int fail(const char* what, int d, int rows, int r0, int step, int lane) {
  std::printf("FAIL %s D=%d rows=%d R0=%d step=%d lane=%d\n", what, d, rows, r0, step, lane);
  return 1;
}

// LDS element offset of logical element (row, col) according to the copy:
// the slot whose source chunk holds it, plus the position in the chunk.
template <int D, int ROWS>
struct Placement {
  std::vector<int> slot_of_chunk;   // global chunk index (row * D / 8 + col / 8) -> slot
  bool ok = true;
  Placement() : slot_of_chunk(ROWS * D / 8, -1) {
    using Copy = fa::AsyncTileCopy<D, ROWS, 4>;
    for (int p = 0; p < ROWS * D / 8; ++p) {
      const int src = Copy::source_offset(p);
      if (src < 0 || src % 8 != 0 || src / 8 >= ROWS * D / 8 || slot_of_chunk[src / 8] != -1) ok = false;
      else slot_of_chunk[src / 8] = p;
    }
  }
  int lds(int row, int col) const { return 8 * slot_of_chunk[(row * D + col) / 8] + col % 8; }
};

// Banks touched by `bytes` bytes at LDS element offset `off` (bf16 elements).
void mark_banks(std::vector<int>& use, int off, int bytes) {
  for (int b = 0; b < bytes; b += 4) ++use[((2 * off + b) / 4) % 64];
}

template <int D, int ROWS>
int check() {
  const Placement<D, ROWS> pl;
  if (!pl.ok) return fail("copy placement is not a bijection", D, ROWS, 0, 0, 0);
  for (int r0 = 0; r0 + 16 <= ROWS; r0 += 16) {
    // natural reads
    for (int ds = 0; ds < D / 32; ++ds) {
      std::vector<int> banks[4];
      for (auto& b : banks) b.assign(64, 0);
      for (int lane = 0; lane < 64; ++lane) {
        const int g = lane >> 4, l16 = lane & 15;
        const int off = r0 * D + fa::NatReader<D>::offset(l16, g, ds);
        for (int e = 0; e < 8; ++e)
          if (off + e != pl.lds(r0 + l16, 32 * ds + 8 * g + e)) return fail("natural read offset", D, ROWS, r0, ds, lane);
        const int parity = ((lane >> 2) ^ (lane >> 3) ^ (lane >> 4)) & 1;
        mark_banks(banks[2 * (lane >> 5) + parity], off, 16);
        ++g_checked;
      }
      for (const auto& b : banks)
        for (int x : b)
          if (x > 1) return fail("natural read bank conflict", D, ROWS, r0, ds, -1);
    }
    // transposed reads
    for (int db = 0; db < D / 16; ++db) {
      std::vector<int> banks[2];
      for (auto& b : banks) b.assign(64, 0);
      for (int lane = 0; lane < 64; ++lane) {
        const int g = lane >> 4, l16 = lane & 15;
        const int off = r0 * D + fa::TrReader<D>::offset(l16, g, db);
        const int row = r0 + 4 * g + (l16 >> 2), col = 16 * db + 4 * (l16 & 3);
        for (int e = 0; e < 4; ++e)
          if (off + e != pl.lds(row, col + e)) return fail("transposed read offset", D, ROWS, r0, db, lane);
        mark_banks(banks[lane >> 5], off, 8);
        ++g_checked;
      }
      for (const auto& b : banks)
        for (int x : b)
          if (x > 1) return fail("transposed read bank conflict", D, ROWS, r0, db, -1);
    }
  }
  return 0;
}

}  // namespace

int main() {
  // tile heights of the bf16 kernels: K/V tiles of 32 and 64 keys, Q/dO
  // tiles of 64, 128 and 256 query rows
  const int bad = check<128, 32>() || check<128, 64>() || check<128, 128>() || check<128, 256>() ||
                  check<64, 32>() || check<64, 64>() || check<64, 128>() || check<64, 256>();
  if (bad) return 1;
  std::printf("swizzle ok: %ld lane reads\n", g_checked);
  return 0;
}

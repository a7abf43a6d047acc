// bf16 forward kernel: exact attention with an online softmax over key tiles.
//
// Method: "Assignment2: FlashAttention & Distributed Data Parallel notes"
// (CS336) section 1.2 -- per query tile keep a running max m, a running sum l
// and an unnormalised accumulator that is rescaled by exp(m - m_new) when the
// max grows; divide by l once at the end and save L = m + log l.  Section
// 1.3 -- one workgroup per (head, query tile); key tiles that start after the
// tile's last query are skipped in causal mode.  Only tiles crossing the
// diagonal are masked ("CS349E lecture 11, 03_flash_backward.py",
// demo4_causal).
//
// Mapping onto gfx950:
// * A workgroup owns BR = NW * QW query rows of one head; wave w owns QW rows.
//   The wave keeps its Q rows in registers for the whole kernel as the B
//   operand of S^T = K Q^T (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
// * Key/value tiles of BC rows go from HBM straight into swizzled,
//   double-buffered LDS tiles with global_load_lds (no staging registers);
//   the copy of tile j+1 runs while tile j is computed, one barrier per tile.
// * Scores are kept transposed (keys x queries) so that each lane owns one
//   query column: the row max is in-lane max operations plus two cross-lane
//   steps, and the accumulator layout of S^T is directly the B operand of
//   O^T += V^T P^T.  V^T comes from LDS with ds_read_b64_tr_b16.
// * The softmax runs in base 2 with scale * log2(e) folded into one FMA per
//   score before v_exp_f32; L is converted back to natural log on output.
// * The accumulator is rescaled only when some row's max has grown by more
//   than kRescaleSlack (base-2 units) since the last rescale; until then the
//   exponent base stays at the older, smaller max, so every probability is at
//   most 2^kRescaleSlack and the final O = acc / l and L = m + log2 l are
//   unchanged (the same stale m enters numerator, denominator and L).
// * Workgroup ids are mapped heaviest query tile first (causal work grows
//   with the tile index), and head = id mod bh keeps every tile of a head on
//   one XCD (ids are dealt to the 8 XCDs round robin) for L2 reuse of K/V.
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

constexpr float kRescaleSlack = 8.0f;

// RAGGED: n may not be a multiple of BC (the last key tile needs the mask).
template <int D, int QW, int NW, int BC, bool CAUSAL, bool RAGGED>
__global__ __launch_bounds__(NW * 64, (QW >= 64 ? 1 : 2))
void fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                     const __bf16* __restrict__ V, __bf16* __restrict__ O,
                     float* __restrict__ LSE, int bh, int n, float scale_log2) {
  constexpr int BR = QW * NW;
  constexpr int NQB = QW / 16;   // 16-query blocks per wave
  constexpr int NKB = BC / 16;   // 16-key blocks per tile
  constexpr int NDS = D / 32;    // 32-wide steps over the head dim (S)
  constexpr int NDB = D / 16;    // 16-wide blocks of the head dim (O)
  constexpr int NKS = BC / 32;   // 32-key steps (PV)

  // two distinct LDS buffers per operand, used in a fixed ping-pong order so
  // that the reads of one tile provably never alias the copy into the other
  __shared__ __bf16 k_lds0[BC * D], k_lds1[BC * D];
  __shared__ __bf16 v_lds0[BC * D], v_lds1[BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int ntq = (n + BR - 1) / BR;
  const int head = blockIdx.x % bh;
  const int qt = ntq - 1 - blockIdx.x / bh;
  const int q0 = qt * BR;
  const int q0w = q0 + wave * QW;
  const size_t hoff = (size_t)head * n * D;
  const __bf16* Qh = Q + hoff;
  const __bf16* Kh = K + hoff;
  const __bf16* Vh = V + hoff;

  const int kend = CAUSAL ? min(n, q0 + BR) : n;   // keys this workgroup can see
  const int ntk = (kend + BC - 1) / BC;
  const AsyncTileCopy<D, BC, NW> copier(wave, lane);
  copier.issue(k_lds0, Kh, min(BC, n));
  copier.issue(v_lds0, Vh, min(BC, n));

  // Q rows of this wave as B operands: lane holds Q[q0w + 16qb + l16][32ds + 8g .. +7]
  bf16x8 qf[NQB][NDS];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int row = q0w + 16 * qb + l16;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      if (row < n) {
        qf[qb][ds] = *reinterpret_cast<const bf16x8*>(Qh + (size_t)row * D + 32 * ds + 8 * g);
      } else {
        qf[qb][ds] = bf16x8{};
      }
    }
  }

  f32x4 acc[NDB][NQB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) acc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[NQB], lsum[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) { m[qb] = kNegInf; lsum[qb] = 0.f; }

  const NatReader<D> kread(l16, g);
  const TrReader<D> vread(l16, g);
  async_copy_wait();
  __syncthreads();

  // The work of one key tile; `masked` (a compile-time flag) selects the copy
  // with the in-tile mask, used only by tiles crossing the diagonal or the end
  // of the sequence, so that the other tiles carry no mask arithmetic.
  auto tile_compute = [&](const __bf16* kt, const __bf16* vt, int j0, auto masked) __attribute__((always_inline)) {
    {
      // S^T[key][query] = K Q^T: lane holds key 16kb + 4g + i, query 16qb + l16
      f32x4 s[NKB][NQB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
      // K operands are read PF steps ahead of the MFMAs that use them; the
      // scheduling fences keep each read where it was issued, so LDS latency
      // hides behind the matrix work instead of stalling it
      {
        constexpr int PF = 3, U = NDS * NKB;       // steps: (ds, kb)
        bf16x8 ka[PF];
#pragma unroll
        for (int u = 0; u < PF && u < U; ++u) ka[u] = kread.read(kt, 16 * (u % NKB), u / NKB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int ds = u / NKB, kb = u % NKB;
          const bf16x8 a = ka[u % PF];
          if (u + PF < U) ka[u % PF] = kread.read(kt, 16 * ((u + PF) % NKB), (u + PF) / NKB);
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) s[kb][qb] = mfma_bf16(a, qf[qb][ds], s[kb][qb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // in-tile mask: key j0 + 16kb + 4g + i is visible iff 16kb + i <= lim
      if constexpr (decltype(masked)::value) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const int last = CAUSAL ? min(q0w + 16 * qb + l16, n - 1) : n - 1;
          const int lim = last - j0 - 4 * g;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (16 * kb + i > lim) s[kb][qb][i] = kNegInf;
        }
      }
      // online softmax (base 2), per query column
      float mx[NQB];
      bool grow = false;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        float t = kNegInf;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) t = fmaxf(t, s[kb][qb][i]);
        mx[qb] = wave_max_xor16_32(t) * scale_log2;
        grow |= !(mx[qb] <= m[qb] + kRescaleSlack);   // also true while m = -inf
      }
      // uniform branch (the vote is read into a scalar register)
      if (__builtin_amdgcn_readfirstlane((int)__any(grow))) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const float m_new = fmaxf(m[qb], mx[qb]);
          const float corr = (m_new == kNegInf) ? 1.f : exp2_fast(m[qb] - m_new);
          m[qb] = m_new;
          lsum[qb] *= corr;
#pragma unroll
          for (int db = 0; db < NDB; ++db) acc[db][qb] *= corr;
        }
      }
      bf16x8 pb[NKS][NQB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const float m_use = (m[qb] == kNegInf) ? 0.f : m[qb];   // never (-inf) - (-inf)
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = exp2_fast(__builtin_fmaf(s[kb][qb][i], scale_log2, -m_use));
            s[kb][qb][i] = p;
            ps += p;
          }
        lsum[qb] += ps;
#pragma unroll
        for (int t = 0; t < NKS; ++t) pb[t][qb] = pack_bf16(s[2 * t][qb], s[2 * t + 1][qb]);
      }
      // O^T[d][query] += V^T P^T over the tile's keys (V^T read PF steps ahead)
      {
        constexpr int PF = 3, U = NKS * NDB;       // steps: (t, db)
        bf16x8 va[PF];
#pragma unroll
        for (int u = 0; u < PF && u < U; ++u)
          va[u] = cat(vread.read(vt, 32 * (u / NDB), u % NDB), vread.read(vt, 32 * (u / NDB) + 16, u % NDB));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int t = u / NDB, db = u % NDB;
          const bf16x8 a = va[u % PF];
          if (u + PF < U) {
            const int t2 = (u + PF) / NDB, db2 = (u + PF) % NDB;
            va[u % PF] = cat(vread.read(vt, 32 * t2, db2), vread.read(vt, 32 * t2 + 16, db2));
          }
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) acc[db][qb] = mfma_bf16(a, pb[t][qb], acc[db][qb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  // One key tile: prefetch tile j+1 into (kn, vn), compute tile j from (kt, vt).
  auto tile_step = [&](const __bf16* kt, const __bf16* vt, __bf16* kn, __bf16* vn, int j) __attribute__((always_inline)) {
    const int j0 = j * BC;
    if (j + 1 < ntk) {
      copier.issue(kn, Kh + (size_t)(j0 + BC) * D, n - j0 - BC);
      copier.issue(vn, Vh + (size_t)(j0 + BC) * D, n - j0 - BC);
    }
    // a wave whose rows all precede the tile has nothing to do in it
    if (!CAUSAL || (j0 <= q0w + QW - 1)) {
      if ((CAUSAL || RAGGED) && ((CAUSAL && j0 + BC - 1 > q0w) || (j0 + BC > n))) {
        tile_compute(kt, vt, j0, std::true_type{});
      } else {
        tile_compute(kt, vt, j0, std::false_type{});
      }
    }
    async_copy_wait();
    __syncthreads();
  };

#pragma unroll 1
  for (int j = 0; j < ntk; j += 2) {
    tile_step(k_lds0, v_lds0, k_lds1, v_lds1, j);
    if (j + 1 < ntk) tile_step(k_lds1, v_lds1, k_lds0, v_lds0, j + 1);
  }

  // epilogue: O = acc / l, L = (m + log2 l) * ln 2
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float lt = wave_sum_xor16_32(lsum[qb]);
    const float inv = 1.f / lt;
    const int qr = q0w + 16 * qb + l16;
    if (qr < n) {
      __bf16* orow = O + hoff + (size_t)qr * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        bf16x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = (__bf16)(acc[db][qb][i] * inv);
        *reinterpret_cast<bf16x4*>(orow + 16 * db + 4 * g) = o4;
      }
      if (g == 0) LSE[(size_t)head * n + qr] = (m[qb] + __builtin_amdgcn_logf(lt)) * kLn2;
    }
  }
}

template <int D, int QW, int NW, int BC>
static hipError_t launch_fwd_inst(const void* q, const void* k, const void* v, void* o, float* lse,
                                  int bh, int n, float scale, int causal, hipStream_t st) {
  constexpr int BR = QW * NW;
  const int ntq = (n + BR - 1) / BR;
  const dim3 grid((unsigned)(ntq * bh)), block(NW * 64);
  const float sl2 = scale * kLog2e;
  auto kern = causal ? fwd_bf16_kernel<D, QW, NW, BC, true, true>
            : (n % BC) ? fwd_bf16_kernel<D, QW, NW, BC, false, true>
                       : fwd_bf16_kernel<D, QW, NW, BC, false, false>;
  hipLaunchKernelGGL(kern, grid, block, 0, st, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                     (__bf16*)o, lse, bh, n, sl2);
  return hipGetLastError();
}

// Tuned tilings: (head dim, BR, BC) -> instance.
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int bh, int n, int d, float scale, int causal, int bm, int bn,
                           hipStream_t st) {
  if (d == 128 && bm == 128 && bn == 64) return launch_fwd_inst<128, 32, 4, 64>(q, k, v, o, lse, bh, n, scale, causal, st);
  if (d == 128 && bm == 256 && bn == 64) return launch_fwd_inst<128, 32, 8, 64>(q, k, v, o, lse, bh, n, scale, causal, st);
  if (d == 128 && bm == 128 && bn == 128) return launch_fwd_inst<128, 32, 4, 128>(q, k, v, o, lse, bh, n, scale, causal, st);
  if (d == 64 && bm == 128 && bn == 64) return launch_fwd_inst<64, 32, 4, 64>(q, k, v, o, lse, bh, n, scale, causal, st);
  if (d == 64 && bm == 256 && bn == 64) return launch_fwd_inst<64, 32, 8, 64>(q, k, v, o, lse, bh, n, scale, causal, st);
  return hipErrorInvalidValue;
}

}  // namespace fa

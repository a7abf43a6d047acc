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
// * Key/value tiles of BC rows are staged through registers into swizzled,
//   double-buffered LDS tiles shared by the workgroup (one barrier per tile).
// * Scores are kept transposed (keys x queries) so that each lane owns one
//   query column: the row max is 15 in-lane max operations plus two
//   cross-lane steps, and the accumulator layout of S^T is directly the B
//   operand of O^T += V^T P^T.  V^T comes from LDS with ds_read_b64_tr_b16.
// * The softmax runs in base 2 with scale * log2(e) folded into one FMA per
//   score before v_exp_f32; L is converted back to natural log on output.
// * Workgroup ids are mapped heaviest query tile first (causal work grows
//   with the tile index), and head = id mod bh keeps every tile of a head on
//   one XCD (ids are dealt to the 8 XCDs round robin) for L2 reuse of K/V.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

template <int D, int QW, int NW, int BC, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, (QW >= 64 ? 1 : 2))
void fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                     const __bf16* __restrict__ V, __bf16* __restrict__ O,
                     float* __restrict__ LSE, int bh, int n, float scale_log2) {
  constexpr int BR = QW * NW;
  constexpr int NT = NW * 64;
  constexpr int NQB = QW / 16;   // 16-query blocks per wave
  constexpr int NKB = BC / 16;   // 16-key blocks per tile
  constexpr int NDS = D / 32;    // 32-wide steps over the head dim (S)
  constexpr int NDB = D / 16;    // 16-wide blocks of the head dim (O)
  constexpr int NKS = BC / 32;   // 32-key steps (PV)

  __shared__ __bf16 k_lds[2][BC * D];
  __shared__ __bf16 v_lds[2][BC * D];

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

  const int kend = CAUSAL ? min(n, q0 + BR) : n;   // keys this workgroup can see
  const int ntk = (kend + BC - 1) / BC;

  TileCopy<D, BC, NT> kc, vc;
  kc.load(Kh, n, tid);
  vc.load(Vh, n, tid);
  kc.store(k_lds[0], tid);
  vc.store(v_lds[0], tid);
  __syncthreads();

  for (int j = 0; j < ntk; ++j) {
    const int j0 = j * BC;
    const int buf = j & 1;
    const bool more = j + 1 < ntk;
    if (more) {
      kc.load(Kh + (size_t)(j0 + BC) * D, n - j0 - BC, tid);
      vc.load(Vh + (size_t)(j0 + BC) * D, n - j0 - BC, tid);
    }
    // a wave whose rows all precede the tile has nothing to do in it
    const bool active = !CAUSAL || (j0 <= q0w + QW - 1);
    if (active) {
      const __bf16* kt = k_lds[buf];
      const __bf16* vt = v_lds[buf];
      // S^T[key][query] = K Q^T: lane holds key 16kb + 4g + i, query 16qb + l16
      f32x4 s[NKB][NQB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const bf16x8 a = lds_read_chunk<D>(kt, 16 * kb + l16, 4 * ds + g);
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) s[kb][qb] = mfma_bf16(a, qf[qb][ds], s[kb][qb]);
        }
      }
      // in-tile mask: only tiles crossing the diagonal or the end of the sequence
      const bool need_mask = (CAUSAL && j0 + BC - 1 > q0w) || (j0 + BC > n);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = j0 + 16 * kb + 4 * g + i;
              const int qr = q0w + 16 * qb + l16;
              if ((CAUSAL && key > qr) || key >= n) s[kb][qb][i] = kNegInf;
            }
      }
      // online softmax (base 2), per query column
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][qb][i]);
        mx = wave_max_xor16_32(mx);
        const float m_new = fmaxf(m[qb], mx * scale_log2);
        const float m_use = (m_new == kNegInf) ? 0.f : m_new;   // never (-inf) - (-inf)
        const float corr = exp2_fast(m[qb] - m_use);
        m[qb] = m_new;
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = exp2_fast(__builtin_fmaf(s[kb][qb][i], scale_log2, -m_use));
            s[kb][qb][i] = p;
            ps += p;
          }
        lsum[qb] = lsum[qb] * corr + ps;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db][qb] *= corr;
      }
      // O^T[d][query] += V^T P^T over the tile's keys
      bf16x8 pb[NKS][NQB];
#pragma unroll
      for (int t = 0; t < NKS; ++t)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) pb[t][qb] = pack_bf16(s[2 * t][qb], s[2 * t + 1][qb]);
#pragma unroll
      for (int t = 0; t < NKS; ++t) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 a = cat(lds_read_tr4<D>(vt, 32 * t + 4 * g, 16 * db, l16),
                               lds_read_tr4<D>(vt, 32 * t + 16 + 4 * g, 16 * db, l16));
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) acc[db][qb] = mfma_bf16(a, pb[t][qb], acc[db][qb]);
        }
      }
    }
    if (more) {
      kc.store(k_lds[buf ^ 1], tid);
      vc.store(v_lds[buf ^ 1], tid);
    }
    __syncthreads();
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
  if (causal) {
    hipLaunchKernelGGL((fwd_bf16_kernel<D, QW, NW, BC, true>), grid, block, 0, st,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, bh, n, sl2);
  } else {
    hipLaunchKernelGGL((fwd_bf16_kernel<D, QW, NW, BC, false>), grid, block, 0, st,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, bh, n, sl2);
  }
  return hipGetLastError();
}

// Tuned tilings: (head dim, BR, BC) -> instance.
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int bh, int n, int d, float scale, int causal, int bm, int bn,
                           hipStream_t st) {
  if (d == 128 && bm == 128 && bn == 64) return launch_fwd_inst<128, 32, 4, 64>(q, k, v, o, lse, bh, n, scale, causal, st);
  if (d == 128 && bm == 256 && bn == 64) return launch_fwd_inst<128, 64, 4, 64>(q, k, v, o, lse, bh, n, scale, causal, st);
  if (d == 64 && bm == 128 && bn == 64) return launch_fwd_inst<64, 32, 4, 64>(q, k, v, o, lse, bh, n, scale, causal, st);
  if (d == 64 && bm == 256 && bn == 64) return launch_fwd_inst<64, 64, 4, 64>(q, k, v, o, lse, bh, n, scale, causal, st);
  return hipErrorInvalidValue;
}

}  // namespace fa

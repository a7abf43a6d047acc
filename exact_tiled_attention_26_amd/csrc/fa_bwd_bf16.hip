// bf16 backward kernels: dK/dV (key/value-tile outer) and dQ (query-tile outer).
//
// Method: "Assignment2: FlashAttention & Distributed Data Parallel notes"
// (CS336) section 1.4.  P is not stored by the forward; each kernel rebuilds
// it on chip from the saved logsumexp (Eq 13 S = Q K^T / sqrt(d), Eq 14
// P = exp(S - L)), then forms Eq 15 dV = P^T dO, Eq 16 dP = dO V^T, Eq 17
// dS = P * (dP - D) with D = rowsum(O * dO) from fa_bwd_preprocess, Eq 18
// dQ = dS K / sqrt(d) and Eq 19 dK = dS^T Q / sqrt(d).  Two kernels with
// different outer loops mean every accumulator has one owner, so neither
// needs atomics; the price is that S and P are recomputed in both.
//
// gfx950 mapping (v_mfma_f32_16x16x32_bf16, fp32 accumulation):
// * dK/dV: a workgroup owns BC = NW * KW keys; wave w keeps its KW rows of K
//   and V in registers (B operands of S = Q K^T and dP = dO V^T) and fp32
//   accumulators for dK^T and dV^T.  Query tiles of BR rows of Q and dO are
//   staged through swizzled double-buffered LDS.  S and dP are kept
//   queries x keys, so their accumulator layout is directly the B operand of
//   dV^T += dO^T P and dK^T += Q^T dS; dO^T and Q^T come from LDS with
//   ds_read_b64_tr_b16.
// * dQ: a workgroup owns BR = NW * QW queries; wave w keeps its Q and dO rows
//   in registers.  Key tiles of K and V are staged through LDS.  S^T and dP^T
//   (keys x queries) feed dQ^T += K^T dS^T with K^T read transposed from LDS.
// * Causal mode visits only the tiles that hold a visible (query, key) pair
//   and masks only tiles crossing the diagonal.  Workgroups are ordered with
//   the heaviest tiles first.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

// Stage BR floats of L (converted to base 2) and D for rows [i0, i0 + BR).
// Rows past n get L = +inf (so P = 0) and D = 0.
template <int BR>
__device__ __forceinline__ void stage_rows(const float* lse, const float* delta, int i0, int n,
                                           float* l2_dst, float* d_dst, int tid) {
  if (tid < BR) {
    const int r = i0 + tid;
    l2_dst[tid] = (r < n) ? lse[r] * kLog2e : __builtin_inff();
    d_dst[tid] = (r < n) ? delta[r] : 0.f;
  }
}

template <int D, int KW, int NW, int BR, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, (KW >= 32 ? 1 : 2))
void dkdv_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                      const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                      const float* __restrict__ LSE, const float* __restrict__ DELTA,
                      __bf16* __restrict__ dK, __bf16* __restrict__ dV,
                      int bh, int n, float scale, float scale_log2) {
  constexpr int BC = KW * NW;
  constexpr int NT = NW * 64;
  constexpr int NKB = KW / 16;   // 16-key blocks per wave
  constexpr int NQB = BR / 16;   // 16-query blocks per query tile
  constexpr int NDS = D / 32;
  constexpr int NDB = D / 16;
  constexpr int NQS = BR / 32;   // 32-query steps (dV, dK contractions)
  static_assert(BR <= NT, "row staging needs one thread per row");

  __shared__ __bf16 q_lds[2][BR * D];
  __shared__ __bf16 do_lds[2][BR * D];
  __shared__ float l2_lds[2][BR];
  __shared__ float d_lds[2][BR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int head = blockIdx.x % bh;
  const int kt = blockIdx.x / bh;          // causal: tile 0 sees the most queries
  const int k0 = kt * BC;
  const int k0w = k0 + wave * KW;
  const size_t hoff = (size_t)head * n * D;
  const __bf16* Qh = Q + hoff;
  const __bf16* dOh = dO + hoff;
  const float* Lh = LSE + (size_t)head * n;
  const float* Dh = DELTA + (size_t)head * n;

  // K and V rows of this wave as B operands: lane holds row k0w + 16kb + l16,
  // columns 32ds + 8g .. +7.
  bf16x8 kf[NKB][NDS], vf[NKB][NDS];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const int key = k0w + 16 * kb + l16;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      if (key < n) {
        kf[kb][ds] = *reinterpret_cast<const bf16x8*>(K + hoff + (size_t)key * D + 32 * ds + 8 * g);
        vf[kb][ds] = *reinterpret_cast<const bf16x8*>(V + hoff + (size_t)key * D + 32 * ds + 8 * g);
      } else {
        kf[kb][ds] = bf16x8{};
        vf[kb][ds] = bf16x8{};
      }
    }
  }

  // dK^T, dV^T accumulators: lane holds d = 16db + 4g + i, key = 16kb + l16
  f32x4 dk[NDB][NKB], dv[NDB][NKB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      dk[db][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      dv[db][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  const int ntq = (n + BR - 1) / BR;
  const int it0 = CAUSAL ? (k0 / BR) : 0;   // earlier query rows see none of these keys

  TileCopy<D, BR, NT> qc, oc;
  {
    const int i0 = it0 * BR;
    qc.load(Qh + (size_t)i0 * D, n - i0, tid);
    oc.load(dOh + (size_t)i0 * D, n - i0, tid);
    qc.store(q_lds[0], tid);
    oc.store(do_lds[0], tid);
    stage_rows<BR>(Lh, Dh, i0, n, l2_lds[0], d_lds[0], tid);
  }
  __syncthreads();

  for (int it = it0; it < ntq; ++it) {
    const int i0 = it * BR;
    const int buf = (it - it0) & 1;
    const bool more = it + 1 < ntq;
    float l2_next = 0.f, d_next = 0.f;
    if (more) {
      qc.load(Qh + (size_t)(i0 + BR) * D, n - i0 - BR, tid);
      oc.load(dOh + (size_t)(i0 + BR) * D, n - i0 - BR, tid);
      if (tid < BR) {
        const int r = i0 + BR + tid;
        l2_next = (r < n) ? Lh[r] * kLog2e : __builtin_inff();
        d_next = (r < n) ? Dh[r] : 0.f;
      }
    }
    const bool active = !CAUSAL || (i0 + BR - 1 >= k0w);
    if (active) {
      const __bf16* qt = q_lds[buf];
      const __bf16* ot = do_lds[buf];
      const float* l2t = l2_lds[buf];
      const float* dt = d_lds[buf];
      // S = Q K^T and dP = dO V^T: lane holds query 16qb + 4g + i, key 16kb + l16
      f32x4 s[NQB][NKB], dp[NQB][NKB];
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          s[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[qb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const bf16x8 aq = lds_read_chunk<D>(qt, 16 * qb + l16, 4 * ds + g);
          const bf16x8 ao = lds_read_chunk<D>(ot, 16 * qb + l16, 4 * ds + g);
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            s[qb][kb] = mfma_bf16(aq, kf[kb][ds], s[qb][kb]);
            dp[qb][kb] = mfma_bf16(ao, vf[kb][ds], dp[qb][kb]);
          }
        }
      }
      // P = exp(S - L) (Eq 14) and dS = P (dP - D) (Eq 17)
      const bool need_mask = CAUSAL && (i0 < k0w + KW - 1);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rl = 16 * qb + 4 * g + i;
          const float l2 = l2t[rl];
          const float dd = dt[rl];
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            float p = exp2_fast(__builtin_fmaf(s[qb][kb][i], scale_log2, -l2));
            if (need_mask && (k0w + 16 * kb + l16 > i0 + rl)) p = 0.f;
            s[qb][kb][i] = p;
            dp[qb][kb][i] = p * (dp[qb][kb][i] - dd);
          }
        }
      // dV^T += dO^T P (Eq 15) and dK^T += Q^T dS (Eq 19, scale applied at the end)
#pragma unroll
      for (int t = 0; t < NQS; ++t) {
        bf16x8 pb[NKB], sb[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          pb[kb] = pack_bf16(s[2 * t][kb], s[2 * t + 1][kb]);
          sb[kb] = pack_bf16(dp[2 * t][kb], dp[2 * t + 1][kb]);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 ao = cat(lds_read_tr4<D>(ot, 32 * t + 4 * g, 16 * db, l16),
                                lds_read_tr4<D>(ot, 32 * t + 16 + 4 * g, 16 * db, l16));
          const bf16x8 aq = cat(lds_read_tr4<D>(qt, 32 * t + 4 * g, 16 * db, l16),
                                lds_read_tr4<D>(qt, 32 * t + 16 + 4 * g, 16 * db, l16));
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            dv[db][kb] = mfma_bf16(ao, pb[kb], dv[db][kb]);
            dk[db][kb] = mfma_bf16(aq, sb[kb], dk[db][kb]);
          }
        }
      }
    }
    if (more) {
      qc.store(q_lds[buf ^ 1], tid);
      oc.store(do_lds[buf ^ 1], tid);
      if (tid < BR) {
        l2_lds[buf ^ 1][tid] = l2_next;
        d_lds[buf ^ 1][tid] = d_next;
      }
    }
    __syncthreads();
  }

  // write dK = scale * dK_acc and dV
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const int key = k0w + 16 * kb + l16;
    if (key < n && key < k0 + BC) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        bf16x4 k4, v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          k4[i] = (__bf16)(dk[db][kb][i] * scale);
          v4[i] = (__bf16)dv[db][kb][i];
        }
        *reinterpret_cast<bf16x4*>(dK + hoff + (size_t)key * D + 16 * db + 4 * g) = k4;
        *reinterpret_cast<bf16x4*>(dV + hoff + (size_t)key * D + 16 * db + 4 * g) = v4;
      }
    }
  }
}

template <int D, int QW, int NW, int BC, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, (QW * D >= 4096 ? 1 : 2))
void dq_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                    const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                    const float* __restrict__ LSE, const float* __restrict__ DELTA,
                    __bf16* __restrict__ dQ, int bh, int n, float scale, float scale_log2) {
  constexpr int BR = QW * NW;
  constexpr int NT = NW * 64;
  constexpr int NQB = QW / 16;
  constexpr int NKB = BC / 16;
  constexpr int NDS = D / 32;
  constexpr int NDB = D / 16;
  constexpr int NKS = BC / 32;

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
  const __bf16* Kh = K + hoff;
  const __bf16* Vh = V + hoff;

  bf16x8 qf[NQB][NDS], of[NQB][NDS];
  float l2q[NQB], dq_d[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int row = q0w + 16 * qb + l16;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      if (row < n) {
        qf[qb][ds] = *reinterpret_cast<const bf16x8*>(Q + hoff + (size_t)row * D + 32 * ds + 8 * g);
        of[qb][ds] = *reinterpret_cast<const bf16x8*>(dO + hoff + (size_t)row * D + 32 * ds + 8 * g);
      } else {
        qf[qb][ds] = bf16x8{};
        of[qb][ds] = bf16x8{};
      }
    }
    l2q[qb] = (row < n) ? LSE[(size_t)head * n + row] * kLog2e : __builtin_inff();
    dq_d[qb] = (row < n) ? DELTA[(size_t)head * n + row] : 0.f;
  }

  // dQ^T accumulator: lane holds d = 16db + 4g + i, query 16qb + l16
  f32x4 acc[NDB][NQB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) acc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kend = CAUSAL ? min(n, q0 + BR) : n;
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
    const bool active = !CAUSAL || (j0 <= q0w + QW - 1);
    if (active) {
      const __bf16* kt = k_lds[buf];
      const __bf16* vt = v_lds[buf];
      // S^T = K Q^T, dP^T = V dO^T: lane holds key 16kb + 4g + i, query 16qb + l16
      f32x4 s[NKB][NQB], dp[NKB][NQB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const bf16x8 ak = lds_read_chunk<D>(kt, 16 * kb + l16, 4 * ds + g);
          const bf16x8 av = lds_read_chunk<D>(vt, 16 * kb + l16, 4 * ds + g);
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            s[kb][qb] = mfma_bf16(ak, qf[qb][ds], s[kb][qb]);
            dp[kb][qb] = mfma_bf16(av, of[qb][ds], dp[kb][qb]);
          }
        }
      }
      const bool need_mask = (CAUSAL && j0 + BC - 1 > q0w) || (j0 + BC > n);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float p = exp2_fast(__builtin_fmaf(s[kb][qb][i], scale_log2, -l2q[qb]));
            if (need_mask) {
              const int key = j0 + 16 * kb + 4 * g + i;
              if ((CAUSAL && key > q0w + 16 * qb + l16) || key >= n) p = 0.f;
            }
            dp[kb][qb][i] = p * (dp[kb][qb][i] - dq_d[qb]);
          }
      // dQ^T += K^T dS^T (Eq 18, scale applied at the end)
#pragma unroll
      for (int t = 0; t < NKS; ++t) {
        bf16x8 sb[NQB];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) sb[qb] = pack_bf16(dp[2 * t][qb], dp[2 * t + 1][qb]);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 a = cat(lds_read_tr4<D>(kt, 32 * t + 4 * g, 16 * db, l16),
                               lds_read_tr4<D>(kt, 32 * t + 16 + 4 * g, 16 * db, l16));
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) acc[db][qb] = mfma_bf16(a, sb[qb], acc[db][qb]);
        }
      }
    }
    if (more) {
      kc.store(k_lds[buf ^ 1], tid);
      vc.store(v_lds[buf ^ 1], tid);
    }
    __syncthreads();
  }

#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int row = q0w + 16 * qb + l16;
    if (row < n) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        bf16x4 q4;
#pragma unroll
        for (int i = 0; i < 4; ++i) q4[i] = (__bf16)(acc[db][qb][i] * scale);
        *reinterpret_cast<bf16x4*>(dQ + hoff + (size_t)row * D + 16 * db + 4 * g) = q4;
      }
    }
  }
}

template <int D, int KW, int NW, int BR>
static hipError_t launch_dkdv_inst(const void* q, const void* k, const void* v, const void* dO,
                                   const float* lse, const float* delta, void* dk, void* dv,
                                   int bh, int n, float scale, int causal, hipStream_t st) {
  constexpr int BC = KW * NW;
  const int ntk = (n + BC - 1) / BC;
  const dim3 grid((unsigned)(ntk * bh)), block(NW * 64);
  const float sl2 = scale * kLog2e;
  if (causal) {
    hipLaunchKernelGGL((dkdv_bf16_kernel<D, KW, NW, BR, true>), grid, block, 0, st,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dO,
                       lse, delta, (__bf16*)dk, (__bf16*)dv, bh, n, scale, sl2);
  } else {
    hipLaunchKernelGGL((dkdv_bf16_kernel<D, KW, NW, BR, false>), grid, block, 0, st,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dO,
                       lse, delta, (__bf16*)dk, (__bf16*)dv, bh, n, scale, sl2);
  }
  return hipGetLastError();
}

template <int D, int QW, int NW, int BC>
static hipError_t launch_dq_inst(const void* q, const void* k, const void* v, const void* dO,
                                 const float* lse, const float* delta, void* dq,
                                 int bh, int n, float scale, int causal, hipStream_t st) {
  constexpr int BR = QW * NW;
  const int ntq = (n + BR - 1) / BR;
  const dim3 grid((unsigned)(ntq * bh)), block(NW * 64);
  const float sl2 = scale * kLog2e;
  if (causal) {
    hipLaunchKernelGGL((dq_bf16_kernel<D, QW, NW, BC, true>), grid, block, 0, st,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dO,
                       lse, delta, (__bf16*)dq, bh, n, scale, sl2);
  } else {
    hipLaunchKernelGGL((dq_bf16_kernel<D, QW, NW, BC, false>), grid, block, 0, st,
                       (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dO,
                       lse, delta, (__bf16*)dq, bh, n, scale, sl2);
  }
  return hipGetLastError();
}

// dK/dV tilings: block_m = query rows per inner step, block_n = keys per workgroup.
hipError_t launch_dkdv_bf16(const void* q, const void* k, const void* v, const void* dO,
                            const float* lse, const float* delta, void* dk, void* dv,
                            int bh, int n, int d, float scale, int causal, int bm, int bn,
                            hipStream_t st) {
  if (d == 128 && bm == 64 && bn == 128)
    return launch_dkdv_inst<128, 32, 4, 64>(q, k, v, dO, lse, delta, dk, dv, bh, n, scale, causal, st);
  if (d == 64 && bm == 64 && bn == 128)
    return launch_dkdv_inst<64, 32, 4, 64>(q, k, v, dO, lse, delta, dk, dv, bh, n, scale, causal, st);
  return hipErrorInvalidValue;
}

// dQ tilings: block_m = queries per workgroup, block_n = keys per inner step.
hipError_t launch_dq_bf16(const void* q, const void* k, const void* v, const void* dO,
                          const float* lse, const float* delta, void* dq,
                          int bh, int n, int d, float scale, int causal, int bm, int bn,
                          hipStream_t st) {
  if (d == 128 && bm == 128 && bn == 64)
    return launch_dq_inst<128, 32, 4, 64>(q, k, v, dO, lse, delta, dq, bh, n, scale, causal, st);
  if (d == 64 && bm == 128 && bn == 64)
    return launch_dq_inst<64, 32, 4, 64>(q, k, v, dO, lse, delta, dq, bh, n, scale, causal, st);
  return hipErrorInvalidValue;
}

}  // namespace fa

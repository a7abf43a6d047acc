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
// * Eq 17's subtraction is folded into the products: each dP accumulator
//   starts at D of its rows and the operand that multiplies into dP (V in
//   dK/dV, dO in dQ) is negated once when loaded (exact in bf16), so the
//   products leave D - dP and one multiply gives -dS = P (D - dP).  The dK
//   and dQ accumulators therefore hold -dK / scale and -dQ / scale, and the
//   epilogues multiply by -scale.
// * Causal mode visits only the tiles that hold a visible (query, key) pair
//   and masks only tiles crossing the diagonal; a sliding window (BAND
//   instances) also bounds the loops from the band's other edge.  Workgroups
//   are ordered with the heaviest tiles first (within groups of heads when
//   there are many heads: head_and_tile).
// * The FUSED instance of the dK/dV kernel is the single-kernel alternative
//   (one pass, dQ gathered with fp32 atomic adds) that section 1.4 sets
//   aside; it is kept for comparison and measured slower on this device.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

// Asynchronous copy of BR consecutive fp32 row values (L or D) of one head
// into LDS with global_load_lds_dword (lane i -> LDS float i).  Rows at or past
// nrows re-read row nrows - 1; the kernels mask those rows.
template <int BR>
__device__ __forceinline__ void rows_load_async(float* lds, const float* src, int i0, int nrows,
                                                int lane) {
  static_assert(BR % 64 == 0, "one dword per lane");
#pragma unroll
  for (int k = 0; k < BR / 64; ++k) {
    const int r = min(i0 + 64 * k + lane, nrows - 1);
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + r),
                                     (__attribute__((address_space(3))) void*)(lds + 64 * k), 4, 0, 0);
  }
}

// nq query rows attend to nk key rows; causal masking is aligned to the end
// of the key sequence (query i sees keys 0 .. i + nk - nq), and a window > 0
// hides keys at or below i + nk - nq - window.
// RAGGED: nq may not be a multiple of BR (the last query tile needs the mask).
// BAND: causal with a window (0 < window < nk).
// FUSED: also accumulate dQ (unscaled, fp32) into dQacc with atomic adds,
// the single-kernel backward: after each 32-query step the waves put dS in
// LDS and wave w adds dS K for head-dim columns [w D/NW, (w+1) D/NW) over
// the workgroup's BC keys; K stays in LDS for the whole kernel.
template <int D, int KW, int NW, int BR, bool CAUSAL, bool RAGGED, bool BAND, bool FUSED = false>
__global__ __launch_bounds__(NW * 64, 1)
void dkdv_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                      const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                      const float* __restrict__ LSE, const float* __restrict__ DELTA,
                      __bf16* __restrict__ dK, __bf16* __restrict__ dV, float* __restrict__ dQacc,
                      int bh, int nq, int nk, int window, int hg, float scale, float scale_log2) {
  constexpr int BC = KW * NW;
  constexpr int NKB = KW / 16;   // 16-key blocks per wave
  constexpr int NDS = D / 32;
  constexpr int NDB = D / 16;
  constexpr int NQS = BR / 32;   // 32-query steps per query tile
  constexpr int DW = D / NW;     // fused dQ: head-dim columns per wave
  static_assert(NW >= 2, "two waves stage the row values");
  static_assert(!FUSED || (DW % 16 == 0 && BC % 32 == 0), "fused dQ split");

  __shared__ __bf16 q_lds0[BR * D], q_lds1[BR * D];
  __shared__ __bf16 o_lds0[BR * D], o_lds1[BR * D];
  __shared__ float l_lds0[BR], l_lds1[BR];
  __shared__ float d_lds0[BR], d_lds1[BR];
  // fused dQ: the workgroup's K rows (swizzled like the Q tiles) and dS of
  // the last two 32-query steps, stored [key][query]
  __shared__ __bf16 kt_lds[FUSED ? BC * D : 8];
  __shared__ __bf16 ds_lds[FUSED ? 2 * BC * 32 : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int nkt = (nk + KW * NW - 1) / (KW * NW);
  int head, kt;   // causal: key tile 0 sees the most queries, so it goes first
  head_and_tile(blockIdx.x, bh, nkt, hg, head, kt);
  const int k0 = kt * BC;
  const int k0w = k0 + wave * KW;
  const int off = CAUSAL ? nk - nq : 0;   // query i sees keys 0 .. i + off
  const int lo = BAND ? off - window : 0;   // with a window: only keys above i + lo
  const size_t hoffq = (size_t)head * nq * D, hoffk = (size_t)head * nk * D;
  const __bf16* Qh = Q + hoffq;
  const __bf16* dOh = dO + hoffq;
  const float* Lh = LSE + (size_t)head * nq;
  const float* Dh = DELTA + (size_t)head * nq;

  const int ntq = (nq + BR - 1) / BR;
  const int dz = divergent_zero();   // keeps the compiler from merging the masked and unmasked tiles
  const int it0 = CAUSAL ? max(0, k0 - off) / BR : 0;   // earlier query rows see none of these keys
  // later rows see none of them either once the window has moved past them
  const int it1 = BAND ? min(ntq, max(0, k0 + BC - 2 - lo) / BR + 1) : ntq;
  // compiler-visible copies: with them the compiler waits for all LDS reads
  // (lgkmcnt(0)) at each operand use, yet the hidden form (exact wait counts,
  // with the row loads below hidden as well) measured 4 % slower here
  const AsyncTileCopy<D, BR, NW, false> copier(wave, lane);
  auto issue_tile = [&](__bf16* qd, __bf16* od, float* ld, float* dd, int i0) __attribute__((always_inline)) {
    copier.issue(qd, Qh + (size_t)i0 * D, nq - i0);
    copier.issue(od, dOh + (size_t)i0 * D, nq - i0);
    if (wave == 0) rows_load_async<BR>(ld, Lh, i0, nq, lane);
    if (wave == 1) rows_load_async<BR>(dd, Dh, i0, nq, lane);
  };
  // L of the rows is turned to base 2 (times log2 e) in LDS once per row,
  // instead of once per lane and step: wave 0, whose copy it is, rescales
  // it in place once the copy has landed, before the barrier that publishes
  // the tile.  (Not with a window: there the compiler's register allocation
  // of the changed step spills; that variant keeps the per-step product.)
  constexpr bool L2_IN_LDS = !BAND;
  auto scale_l = [&](float* ld) __attribute__((always_inline)) {
    if (L2_IN_LDS && wave == 0) {
#pragma unroll
      for (int k = 0; k < BR / 64; ++k) ld[64 * k + lane] *= kLog2e;
    }
  };
  if constexpr (FUSED) {
    const AsyncTileCopy<D, BC, NW, false> kcopier(wave, lane);
    kcopier.issue(kt_lds, K + hoffk + (size_t)k0 * D, nk - k0);
  }
  issue_tile(q_lds0, o_lds0, l_lds0, d_lds0, it0 * BR);

  // K and V rows of this wave as B operands: lane holds row k0w + 16kb + l16,
  // columns 32ds + 8g .. +7.
  bf16x8 kf[NKB][NDS], vf[NKB][NDS];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const int key = k0w + 16 * kb + l16;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      if (key < nk) {
        kf[kb][ds] = *reinterpret_cast<const bf16x8*>(K + hoffk + (size_t)key * D + 32 * ds + 8 * g);
        vf[kb][ds] = *reinterpret_cast<const bf16x8*>(V + hoffk + (size_t)key * D + 32 * ds + 8 * g);
      } else {
        kf[kb][ds] = bf16x8{};
        vf[kb][ds] = bf16x8{};
      }
      vf[kb][ds] = neg_bf16(vf[kb][ds]);   // see the dP accumulators below
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

  const NatReader<D> nat(l16, g);
  const TrReader<D> tr(l16, g);
  async_copy_wait();
  scale_l(l_lds0);
  __syncthreads();
  if constexpr (FUSED) {
    // K rows past nk were copied from row nk - 1: clear them so that those
    // keys add nothing to dQ
    if (k0 + BC > nk) {
      for (int e = tid; e < (k0 + BC - nk) * (D / 8); e += NW * 64)
        *reinterpret_cast<bf16x8*>(kt_lds + (size_t)(nk - k0 + e / (D / 8)) * D + 8 * (e % (D / 8))) = bf16x8{};
      __syncthreads();
    }
  }

  // Fused dQ of one 32-query step (queries i0 + 32t ..): dS is stored
  // [key][query] with rows of 32 queries; the 16-query halves of a row swap
  // when bit 2 of the key is set, so the transposed reads below are free of
  // bank conflicts.  dQ[q][d] += sum over the BC keys of dS[q][key] K[key][d]
  // with A = dS (read transposed from ds_lds) and B = K (read transposed
  // from kt_lds); the lane then holds query 16qb + 4g + i, column
  // w DW + 16nb + l16, added to dQacc with one atomic per value.
  auto ds_off = [&](int row, int col) __attribute__((always_inline)) {
    return row * 32 + (col ^ (16 * ((row >> 2) & 1)));
  };
  auto dq_step = [&](const bf16x8 (&sb)[NKB], int i0, int t, __bf16* dsl) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int row = wave * KW + 16 * kb + l16;
      *reinterpret_cast<bf16x4*>(dsl + ds_off(row, 4 * g)) = __builtin_shufflevector(sb[kb], sb[kb], 0, 1, 2, 3);
      *reinterpret_cast<bf16x4*>(dsl + ds_off(row, 16 + 4 * g)) = __builtin_shufflevector(sb[kb], sb[kb], 4, 5, 6, 7);
    }
    __syncthreads();
    constexpr int NB = DW / 16;
    f32x4 acc[2][NB];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[qb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int trow = 4 * g + (l16 >> 2);          // transposed read: row in a 16-row block
#pragma unroll
    for (int kk = 0; kk < BC / 32; ++kk) {
      bf16x8 a[2], b[NB];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int c = 16 * qb + 4 * (l16 & 3);
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(dsl + ds_off(32 * kk + trow, c)));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(dsl + ds_off(32 * kk + 16 + trow, c)));
        a[qb] = cat(lo, hi);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int db = wave * NB + nb;
        b[nb] = cat(tr.read(kt_lds, 32 * kk, db), tr.read(kt_lds, 32 * kk + 16, db));
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[qb][nb] = mfma_bf16(a[qb], b[nb], acc[qb][nb]);
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = i0 + 32 * t + 16 * qb + 4 * g + i;
        if (!RAGGED || q < nq) {
          float* row = dQacc + hoffq + (size_t)q * D + wave * DW + l16;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            __hip_atomic_fetch_add(row + 16 * nb, acc[qb][nb][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
  };

  // One 32-query step t of a query tile has three stages:
  //   G1(t): S = Q K^T and dP = dO V^T          (2 D/32 MFMA groups of 2 NKB)
  //   EW(t): P = exp(S - L), dS = P (dP - D)    (16 elementwise items per lane)
  //   G2(t): dV^T += dO^T P, dK^T += Q^T dS      (D/16 MFMA groups of 2 NKB)
  // They run as a software pipeline, G2(t-1) | EW(t) | G1(t+1), with the
  // elementwise items of EW(t) spread over the MFMA groups of G2(t-1) and
  // G1(t+1): every fenced group holds a few MFMAs, the LDS reads for a later
  // group and one or two elementwise items, so the VALU work and the LDS
  // latency both hide behind the matrix cores within the one wave per SIMD.
  using Acc = f32x4[2][NKB];
  constexpr int NG1 = 2 * NDS;                   // MFMA groups of G1: (ds, h)
  constexpr int NG2 = NDB;                       // MFMA groups of G2: db
  constexpr int NE = 2 * 4 * NKB;                // elementwise items per lane per step
  constexpr int PF = 3;                          // operand prefetch distance (groups)

  struct EwState {
    float l2[2][4];
    f32x4 pv[2][NKB], dsv[2][NKB];
  };
  auto ew_begin = [&](const float* lt, int t, EwState& e) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rl = 32 * t + 16 * h + 4 * g;     // first of this lane's 4 rows
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(lt + rl);
#pragma unroll
      for (int i = 0; i < 4; ++i) e.l2[h][i] = L2_IN_LDS ? l4[i] : l4[i] * kLog2e;
    }
  };
  // item x = (h, i, kb) of step t
  auto ew_item = [&](int x, int i0, int t, bool need_mask, const Acc& s, const Acc& dp, EwState& e) __attribute__((always_inline)) {
    const int kb = x % NKB, i = (x / NKB) % 4, h = x / (4 * NKB);
    const float p = exp2_fast(__builtin_fmaf(s[h][kb][i], scale_log2, -e.l2[h][i]));
    e.pv[h][kb][i] = p;
    e.dsv[h][kb][i] = p * dp[h][kb][i];   // = -dS (dp holds D - dP)
  };
  // Masked entries (key after query + off, or query past nq) get P = dS = 0.  Only
  // tiles crossing the diagonal or the end of the sequence run this, behind
  // a uniform branch, so the other tiles carry no mask arithmetic.
  auto ew_mask = [&](int i0, int t, EwState& e) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = i0 + 32 * t + 16 * h + 4 * g + i;
        const int lim = (q < nq) ? (CAUSAL ? q + off - k0w - l16 : 0x7fffffff) : -1;
        const int llim = q + lo - k0w - l16;   // key 16kb + .. hidden from below iff 16kb <= llim
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          if (16 * kb > lim || (BAND && 16 * kb <= llim)) {
            e.pv[h][kb][i] = 0.f;
            e.dsv[h][kb][i] = 0.f;
          }
      }
  };
  auto ew_end = [&](const EwState& e, bf16x8 (&pb)[NKB], bf16x8 (&sb)[NKB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      pb[kb] = pack_bf16(e.pv[0][kb], e.pv[1][kb]);
      sb[kb] = pack_bf16(e.dsv[0][kb], e.dsv[1][kb]);
    }
  };

  // Operand reads for group u of G1 (natural Q, dO rows) and of G2 (transposed).
  auto g1_read = [&](const __bf16* qt, const __bf16* ot, int t, int u, bf16x8& aq, bf16x8& ao) __attribute__((always_inline)) {
    aq = nat.read(qt, 32 * t + 16 * (u & 1), u >> 1);
    ao = nat.read(ot, 32 * t + 16 * (u & 1), u >> 1);
  };
  auto g2_read = [&](const __bf16* qt, const __bf16* ot, int t, int u, bf16x8& aq, bf16x8& ao) __attribute__((always_inline)) {
    ao = cat(tr.read(ot, 32 * t, u), tr.read(ot, 32 * t + 16, u));
    aq = cat(tr.read(qt, 32 * t, u), tr.read(qt, 32 * t + 16, u));
  };
  auto g1_mfma = [&](int u, const bf16x8& aq, const bf16x8& ao, Acc& s, Acc& dp) __attribute__((always_inline)) {
    const int ds = u >> 1, h = u & 1;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[h][kb] = mfma_bf16(aq, kf[kb][ds], s[h][kb]);
      dp[h][kb] = mfma_bf16(ao, vf[kb][ds], dp[h][kb]);
    }
  };
  auto g2_mfma = [&](int u, const bf16x8& aq, const bf16x8& ao, const bf16x8 (&pb)[NKB], const bf16x8 (&sb)[NKB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      dv[u][kb] = mfma_bf16(ao, pb[kb], dv[u][kb]);
      dk[u][kb] = mfma_bf16(aq, sb[kb], dk[u][kb]);
    }
  };
  // S starts at zero; dP starts at D of its four rows, so that with V
  // negated the products leave D - dP and the elementwise pass needs no
  // subtraction (dS = P (dP - D) comes out negated; dK is scaled by -scale)
  auto init_acc = [&](Acc& s, Acc& dp, const float* dt, int t) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(dt + 32 * t + 16 * h + 4 * g);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[h][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[h][kb] = d4;
      }
    }
  };

  // One query tile: the pipeline over its NQS steps.  The operand stream of a
  // pipeline region is the concatenation [G2(t-1) groups] [G1(t+1) groups];
  // reads run PF groups ahead along that stream.
  auto run_tile = [&](const __bf16* qt, const __bf16* ot, const float* lt, const float* dt, int i0,
                      auto masked) __attribute__((always_inline)) {
    constexpr bool need_mask = decltype(masked)::value;
    Acc sa[2], pa[2];
    bf16x8 pbuf[2][NKB], sbuf[2][NKB];
    // prologue: G1(0) alone
    {
      init_acc(sa[0], pa[0], dt, 0);
      bf16x8 rq[PF], ro[PF];
#pragma unroll
      for (int u = 0; u < PF; ++u) g1_read(qt, ot, 0, u, rq[u], ro[u]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < NG1; ++u) {
        const bf16x8 aq = rq[u % PF], ao = ro[u % PF];
        if (u + PF < NG1) g1_read(qt, ot, 0, u + PF, rq[u % PF], ro[u % PF]);
        g1_mfma(u, aq, ao, sa[0], pa[0]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int t = 0; t < NQS; ++t) {
      const bool has_g2 = t >= 1, has_g1 = t + 1 < NQS;
      const int ngroups = (has_g2 ? NG2 : 0) + (has_g1 ? NG1 : 0);
      EwState e;
      ew_begin(lt, t, e);
      if (has_g1) init_acc(sa[(t + 1) & 1], pa[(t + 1) & 1], dt, t + 1);
      // read group v of the region's operand stream
      auto read_v = [&](int v, bf16x8& aq, bf16x8& ao) __attribute__((always_inline)) {
        if (has_g2 && v < NG2) g2_read(qt, ot, t - 1, v, aq, ao);
        else g1_read(qt, ot, t + 1, v - (has_g2 ? NG2 : 0), aq, ao);
      };
      bf16x8 rq[PF], ro[PF];
#pragma unroll
      for (int v = 0; v < PF; ++v) read_v(v, rq[v], ro[v]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int v = 0; v < NG1 + NG2; ++v) {
        if (v < ngroups) {
          const bf16x8 aq = rq[v % PF], ao = ro[v % PF];
          if (v + PF < ngroups) read_v(v + PF, rq[v % PF], ro[v % PF]);
          if (has_g2 && v < NG2) g2_mfma(v, aq, ao, pbuf[(t - 1) & 1], sbuf[(t - 1) & 1]);
          else g1_mfma(v - (has_g2 ? NG2 : 0), aq, ao, sa[(t + 1) & 1], pa[(t + 1) & 1]);
          // spread the NE elementwise items of step t over the region's groups
#pragma unroll
          for (int x = (v * NE) / ngroups; x < ((v + 1) * NE) / ngroups; ++x)
            ew_item(x, i0, t, need_mask, sa[t & 1], pa[t & 1], e);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (ngroups == 0) {
#pragma unroll
        for (int x = 0; x < NE; ++x) ew_item(x, i0, t, need_mask, sa[t & 1], pa[t & 1], e);
      }
      if constexpr (need_mask) ew_mask(i0, t, e);
      ew_end(e, pbuf[t & 1], sbuf[t & 1]);
      if constexpr (FUSED) dq_step(sbuf[t & 1], i0, t, ds_lds + (t & 1) * BC * 32);
    }
    // epilogue: G2 of the last step alone
    {
      bf16x8 rq[PF], ro[PF];
#pragma unroll
      for (int u = 0; u < PF; ++u) g2_read(qt, ot, NQS - 1, u, rq[u], ro[u]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < NG2; ++u) {
        const bf16x8 aq = rq[u % PF], ao = ro[u % PF];
        if (u + PF < NG2) g2_read(qt, ot, NQS - 1, u + PF, rq[u % PF], ro[u % PF]);
        g2_mfma(u, aq, ao, pbuf[(NQS - 1) & 1], sbuf[(NQS - 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  auto tile_step = [&](const __bf16* qt, const __bf16* ot, const float* lt, const float* dt,
                       __bf16* qn, __bf16* on, float* ln, float* dn, int it) __attribute__((always_inline)) {
    const int i0 = it * BR;
    if (it + 1 < it1) issue_tile(qn, on, ln, dn, i0 + BR);
    // (fused: every wave takes part in the dQ product of every step, so the
    // tests are made for the whole workgroup's keys)
    const int kl = FUSED ? k0 : k0w, kw = FUSED ? BC : KW;
    const bool active = !CAUSAL || (i0 + BR - 1 + off >= kl && (!BAND || i0 + lo < kl + kw - 1));
    if (active) {
      // only tiles crossing the diagonal, the window's edge or the end of the
      // sequence are masked; they run a separate copy so that the others carry
      // no mask arithmetic
      if ((CAUSAL || RAGGED) &&
          ((CAUSAL && i0 + off < kl + kw - 1) || (BAND && i0 + BR - 1 + lo >= kl) || (i0 + BR > nq + dz))) {
        run_tile(qt, ot, lt, dt, i0, std::true_type{});
      } else {
        run_tile(qt, ot, lt, dt, i0, std::false_type{});
      }
    }
    async_copy_wait();
    if (it + 1 < it1) scale_l(ln);
    __syncthreads();
  };

#pragma unroll 1
  for (int it = it0; it < it1; it += 2) {
    tile_step(q_lds0, o_lds0, l_lds0, d_lds0, q_lds1, o_lds1, l_lds1, d_lds1, it);
    if (it + 1 < it1) tile_step(q_lds1, o_lds1, l_lds1, d_lds1, q_lds0, o_lds0, l_lds0, d_lds0, it + 1);
  }

  // write dK = -scale * dK_acc (the accumulator holds -dK / scale) and dV
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const int key = k0w + 16 * kb + l16;
    if (key < nk && key < k0 + BC) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        bf16x4 k4, v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          k4[i] = (__bf16)(dk[db][kb][i] * -scale);
          v4[i] = (__bf16)dv[db][kb][i];
        }
        *reinterpret_cast<bf16x4*>(dK + hoffk + (size_t)key * D + 16 * db + 4 * g) = k4;
        *reinterpret_cast<bf16x4*>(dV + hoffk + (size_t)key * D + 16 * db + 4 * g) = v4;
      }
    }
  }
}

// Occupancy: with 32-key tiles the kernel fits two waves per SIMD (at most
// 256 registers each), so the matrix products of one wave overlap the
// element-wise work of the other; with 64-key tiles it holds one at d = 128
// and two at d = 64 (asked for: left free, the compiler takes up to 262
// registers there, and two waves measured 9 % faster causal).  Eight
// waves (256 query rows) share each K/V tile copy at d = 128: measured
// 1.5 % faster causal and 3 % non-causal than four at 32 x 8192 x 128.
template <int D, int QW, int NW, int BC, bool CAUSAL, bool BAND>
__global__ __launch_bounds__(NW * 64, (BC == 32 || D == 64) ? 2 : 1)
void dq_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                    const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                    const float* __restrict__ LSE, const float* __restrict__ DELTA,
                    __bf16* __restrict__ dQ, int bh, int nq, int nk, int window, int hg, float scale,
                    float scale_log2) {
  constexpr int BR = QW * NW;
  constexpr int NQB = QW / 16;
  constexpr int NKB = BC / 16;
  constexpr int NDS = D / 32;
  constexpr int NDB = D / 16;
  constexpr int NKS = BC / 32;

  __shared__ __bf16 k_lds0[BC * D], k_lds1[BC * D];
  __shared__ __bf16 v_lds0[BC * D], v_lds1[BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int ntq = (nq + BR - 1) / BR;
  int head, rank;
  head_and_tile(blockIdx.x, bh, ntq, hg, head, rank);
  const int qt = ntq - 1 - rank;   // heaviest (causal: last) query tile first
  const int q0 = qt * BR;
  const int q0w = q0 + wave * QW;
  const int off = CAUSAL ? nk - nq : 0;   // query i sees keys 0 .. i + off
  const int lo = BAND ? off - window : 0;   // with a window: only keys above i + lo
  const size_t hoffq = (size_t)head * nq * D;
  const __bf16* Kh = K + (size_t)head * nk * D;
  const __bf16* Vh = V + (size_t)head * nk * D;

  const int kend = CAUSAL ? min(nk, q0 + BR + off) : nk;
  const int jt0 = BAND ? max(0, q0 + lo + 1) / BC : 0;   // first key tile a row of the workgroup can see
  const int ntk = (kend + BC - 1) / BC;
  // hidden copies: the compiler keeps exact LDS wait counts for the operand
  // reads (measured 1-2 % faster than the compiler-visible form)
  const AsyncTileCopy<D, BC, NW, true> copier(wave, lane);
  copier.issue(k_lds0, Kh + (size_t)jt0 * BC * D, nk - jt0 * BC);
  copier.issue(v_lds0, Vh + (size_t)jt0 * BC * D, nk - jt0 * BC);

  bf16x8 qf[NQB][NDS], of[NQB][NDS];
  float l2q[NQB], dq_d[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int row = q0w + 16 * qb + l16;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      if (row < nq) {
        qf[qb][ds] = *reinterpret_cast<const bf16x8*>(Q + hoffq + (size_t)row * D + 32 * ds + 8 * g);
        of[qb][ds] = *reinterpret_cast<const bf16x8*>(dO + hoffq + (size_t)row * D + 32 * ds + 8 * g);
      } else {
        qf[qb][ds] = bf16x8{};
        of[qb][ds] = bf16x8{};
      }
      of[qb][ds] = neg_bf16(of[qb][ds]);   // see the dP^T accumulators below
    }
    l2q[qb] = (row < nq) ? LSE[(size_t)head * nq + row] * kLog2e : __builtin_inff();
    dq_d[qb] = (row < nq) ? DELTA[(size_t)head * nq + row] : 0.f;
  }

  // dQ^T accumulator: lane holds d = 16db + 4g + i, query 16qb + l16
  f32x4 acc[NDB][NQB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) acc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const NatReader<D> nat(l16, g);
  const TrReader<D> tr(l16, g);
  async_copy_wait();
  __syncthreads();

  auto tile_step = [&](const __bf16* kt, const __bf16* vt, __bf16* kn, __bf16* vn, int j) __attribute__((always_inline)) {
    const int j0 = j * BC;
    if (j + 1 < ntk) {
      copier.issue(kn, Kh + (size_t)(j0 + BC) * D, nk - j0 - BC);
      copier.issue(vn, Vh + (size_t)(j0 + BC) * D, nk - j0 - BC);
    }
    const bool active = !CAUSAL || (j0 <= q0w + QW - 1 + off && (!BAND || j0 + BC - 1 > q0w + lo));
    if (active) {
      // S^T = K Q^T, dP^T = V dO^T: lane holds key 16kb + 4g + i, query 16qb + l16.
      // dP^T starts at D of the lane's query and dO is negated, so the
      // products leave D - dP and the elementwise pass needs no subtraction
      // (dS = P (dP - D) comes out negated; dQ is scaled by -scale).
      f32x4 s[NKB][NQB], dp[NKB][NQB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
          dp[kb][qb] = f32x4{dq_d[qb], dq_d[qb], dq_d[qb], dq_d[qb]};
        }
      // operands are read PF steps ahead of the MFMAs that use them; the
      // scheduling fences keep each read where it was issued, so LDS latency
      // hides behind the matrix work instead of stalling it
      constexpr int PF = 3;
      constexpr int U1 = NDS * NKB;                // steps of S^T / dP^T: (ds, kb)
      bf16x8 ka[PF], va[PF];
#pragma unroll
      for (int u = 0; u < PF && u < U1; ++u) {
        ka[u] = nat.read(kt, 16 * (u % NKB), u / NKB);
        va[u] = nat.read(vt, 16 * (u % NKB), u / NKB);
      }
#pragma unroll
      for (int u = 0; u < U1; ++u) {
        const int ds = u / NKB, kb = u % NKB;
        const bf16x8 ak = ka[u % PF], av = va[u % PF];
        if (u + PF < U1) {
          ka[u % PF] = nat.read(kt, 16 * ((u + PF) % NKB), (u + PF) / NKB);
          va[u % PF] = nat.read(vt, 16 * ((u + PF) % NKB), (u + PF) / NKB);
        }
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          s[kb][qb] = mfma_bf16(ak, qf[qb][ds], s[kb][qb]);
          dp[kb][qb] = mfma_bf16(av, of[qb][ds], dp[kb][qb]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      const bool need_mask = (CAUSAL && j0 + BC - 1 > q0w + off) || (BAND && j0 <= q0w + QW - 1 + lo) ||
                             (j0 + BC > nk);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p = exp2_fast(__builtin_fmaf(s[kb][qb][i], scale_log2, -l2q[qb]));
            dp[kb][qb][i] = p * dp[kb][qb][i];   // = -dS
          }
      // masked entries get dS = 0; only tiles crossing the diagonal or the end
      // of the sequence run this, behind a uniform branch
      if (need_mask) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const int last = CAUSAL ? min(q0w + 16 * qb + l16 + off, nk - 1) : nk - 1;
          // key j0 + 16kb + 4g + i visible iff llim < 16kb + i <= lim
          const int lim = last - j0 - 4 * g;
          const int llim = q0w + 16 * qb + l16 + lo - j0 - 4 * g;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (16 * kb + i > lim || (BAND && 16 * kb + i <= llim)) dp[kb][qb][i] = 0.f;
        }
      }
      // dQ^T += K^T dS^T (Eq 18, scale applied at the end)
      bf16x8 sb[NKS][NQB];
#pragma unroll
      for (int t = 0; t < NKS; ++t)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) sb[t][qb] = pack_bf16(dp[2 * t][qb], dp[2 * t + 1][qb]);
      constexpr int PF3 = 4;
      constexpr int U3 = NKS * NDB;                // steps: (t, db)
      bf16x8 ta[PF3];
#pragma unroll
      for (int u = 0; u < PF3 && u < U3; ++u)
        ta[u] = cat(tr.read(kt, 32 * (u / NDB), u % NDB), tr.read(kt, 32 * (u / NDB) + 16, u % NDB));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U3; ++u) {
        const int t = u / NDB, db = u % NDB;
        const bf16x8 a = ta[u % PF3];
        if (u + PF3 < U3) {
          const int t2 = (u + PF3) / NDB, db2 = (u + PF3) % NDB;
          ta[u % PF3] = cat(tr.read(kt, 32 * t2, db2), tr.read(kt, 32 * t2 + 16, db2));
        }
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) acc[db][qb] = mfma_bf16(a, sb[t][qb], acc[db][qb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    async_copy_wait();
    __syncthreads();
  };

#pragma unroll 1
  for (int j = jt0; j < ntk; j += 2) {
    tile_step(k_lds0, v_lds0, k_lds1, v_lds1, j);
    if (j + 1 < ntk) tile_step(k_lds1, v_lds1, k_lds0, v_lds0, j + 1);
  }

#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int row = q0w + 16 * qb + l16;
    if (row < nq) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        bf16x4 q4;
#pragma unroll
        for (int i = 0; i < 4; ++i) q4[i] = (__bf16)(acc[db][qb][i] * -scale);   // acc holds -dQ / scale
        *reinterpret_cast<bf16x4*>(dQ + hoffq + (size_t)row * D + 16 * db + 4 * g) = q4;
      }
    }
  }
}

template <int D, int KW, int NW, int BR, bool FUSED = false>
static hipError_t launch_dkdv_inst(const void* q, const void* k, const void* v, const void* dO,
                                   const float* lse, const float* delta, void* dk, void* dv,
                                   int bh, int nq, int nk, float scale, int causal, int window,
                                   hipStream_t st, float* dqacc = nullptr) {
  constexpr int BC = KW * NW;
  const int ntk = (nk + BC - 1) / BC;
  const dim3 grid((unsigned)(ntk * bh)), block(NW * 64);
  const float sl2 = scale * kLog2e;
  // the non-causal kernel keeps its masked copy even when nq is a multiple of
  // BR: the uniform branch around it splits the tile into scheduling regions
  // small enough to stay within the register file
  auto kern = (causal && window > 0) ? dkdv_bf16_kernel<D, KW, NW, BR, true, true, true, FUSED>
             : causal ? dkdv_bf16_kernel<D, KW, NW, BR, true, true, false, FUSED>
                      : dkdv_bf16_kernel<D, KW, NW, BR, false, true, false, FUSED>;
  const int hg = head_group((const void*)kern, NW * 64, bh, ntk, st);
  hipLaunchKernelGGL(kern, grid, block, 0, st, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                     (const __bf16*)dO, lse, delta, (__bf16*)dk, (__bf16*)dv, dqacc, bh, nq, nk, window,
                     hg, scale, sl2);
  return hipGetLastError();
}

// dQ = bf16(scale * acc), four values per thread (n is a multiple of 4)
__global__ __launch_bounds__(256) void dq_from_acc_kernel(const float* __restrict__ acc,
                                                          __bf16* __restrict__ dq, size_t n4,
                                                          float scale) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const f32x4 a = reinterpret_cast<const f32x4*>(acc)[i];
    bf16x4 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = (__bf16)(a[j] * scale);
    reinterpret_cast<bf16x4*>(dq)[i] = r;
  }
}

// Single-kernel backward: zero the fp32 dQ accumulator, run the dK/dV kernel
// with the fused dQ product, then round scale * acc to bf16.
hipError_t launch_bwd_fused_bf16(const void* q, const void* k, const void* v, const void* dO,
                                 const float* lse, const float* delta, void* dq, void* dk, void* dv,
                                 float* dq_acc, int bh, int nq, int nk, int d, float scale, int causal,
                                 int window, int bm, int bn, hipStream_t st) {
  const size_t n = (size_t)bh * nq * d;
  hipError_t e = launch_zero_f32(dq_acc, n, st);
  if (e != hipSuccess) return e;
  if (d == 128 && bm == 64 && bn == 128)
    e = launch_dkdv_inst<128, 32, 4, 64, true>(q, k, v, dO, lse, delta, dk, dv, bh, nq, nk, scale, causal,
                                               window, st, dq_acc);
  else if (d == 64 && bm == 64 && bn == 128)
    e = launch_dkdv_inst<64, 32, 4, 64, true>(q, k, v, dO, lse, delta, dk, dv, bh, nq, nk, scale, causal,
                                              window, st, dq_acc);
  else
    return hipErrorInvalidValue;
  if (e != hipSuccess) return e;
  const size_t blocks = std::min<size_t>((n / 4 + 255) / 256, 8192);
  hipLaunchKernelGGL(dq_from_acc_kernel, dim3((unsigned)blocks), dim3(256), 0, st, dq_acc, (__bf16*)dq,
                     n / 4, -scale);   // the fused dK/dV kernel accumulates -dQ / scale
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Allocation-free single-kernel backward.  Its fp32 dQ accumulator lives in
// `scratch`, a fixed device array of this library (one copy on every GPU the
// library runs on, kept until the process ends), so the call needs no
// workspace argument and never allocates.  In host code `scratch` names a
// host-side stand-in, not device memory: the device address is looked up
// once per device with hipGetSymbolAddress and only that address is passed
// to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kScratchFloats = kNoAllocScratchBytes / sizeof(float);
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<float*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the device that runs `st` (looked up on the
// first call for that device, with the device current, then cached).
hipError_t scratch_for_stream(hipStream_t st, float** out) {
  hipDevice_t dev = 0;
  hipError_t e = hipStreamGetDevice(st, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  float* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      int cur = 0;
      if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (cur != dev) {
        const hipError_t e2 = hipSetDevice(cur);
        if (e == hipSuccess) e = e2;
      }
      if (e != hipSuccess) return e;
      if (addr == nullptr) return hipErrorInvalidSymbol;
      p = static_cast<float*>(addr);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}
}  // namespace

hipError_t launch_bwd_fused_bf16_noalloc(const void* q, const void* k, const void* v, const void* dO,
                                         const float* lse, const float* delta, void* dq, void* dk, void* dv,
                                         int bh, int nq, int nk, int d, float scale, int causal, int window,
                                         int bm, int bn, hipStream_t st) {
  if ((size_t)bh * nq * d > kScratchFloats) return hipErrorInvalidValue;   // the caller checks first
  float* acc = nullptr;
  const hipError_t e = scratch_for_stream(st, &acc);
  if (e != hipSuccess) return e;
  return launch_bwd_fused_bf16(q, k, v, dO, lse, delta, dq, dk, dv, acc, bh, nq, nk, d, scale, causal, window,
                               bm, bn, st);
}

template <int D, int QW, int NW, int BC>
static hipError_t launch_dq_inst(const void* q, const void* k, const void* v, const void* dO,
                                 const float* lse, const float* delta, void* dq,
                                 int bh, int nq, int nk, float scale, int causal, int window,
                                 hipStream_t st) {
  constexpr int BR = QW * NW;
  const int ntq = (nq + BR - 1) / BR;
  const dim3 grid((unsigned)(ntq * bh)), block(NW * 64);
  const float sl2 = scale * kLog2e;
  auto kern = (causal && window > 0) ? dq_bf16_kernel<D, QW, NW, BC, true, true>
             : causal ? dq_bf16_kernel<D, QW, NW, BC, true, false>
                      : dq_bf16_kernel<D, QW, NW, BC, false, false>;
  const int hg = head_group((const void*)kern, NW * 64, bh, ntq, st);
  hipLaunchKernelGGL(kern, grid, block, 0, st, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                     (const __bf16*)dO, lse, delta, (__bf16*)dq, bh, nq, nk, window, hg, scale, sl2);
  return hipGetLastError();
}

// dK/dV tilings: block_m = query rows per inner step, block_n = keys per workgroup.
hipError_t launch_dkdv_bf16(const void* q, const void* k, const void* v, const void* dO,
                            const float* lse, const float* delta, void* dk, void* dv,
                            int bh, int nq, int nk, int d, float scale, int causal, int window, int bm, int bn,
                            hipStream_t st) {
  if (d == 128 && bm == 64 && bn == 128)
    return launch_dkdv_inst<128, 32, 4, 64>(q, k, v, dO, lse, delta, dk, dv, bh, nq, nk, scale, causal, window, st);
  if (d == 128 && bm == 128 && bn == 128)
    return launch_dkdv_inst<128, 32, 4, 128>(q, k, v, dO, lse, delta, dk, dv, bh, nq, nk, scale, causal, window, st);
  if (d == 64 && bm == 64 && bn == 128)
    return launch_dkdv_inst<64, 32, 4, 64>(q, k, v, dO, lse, delta, dk, dv, bh, nq, nk, scale, causal, window, st);
  if (d == 64 && bm == 128 && bn == 128)
    return launch_dkdv_inst<64, 32, 4, 128>(q, k, v, dO, lse, delta, dk, dv, bh, nq, nk, scale, causal, window, st);
  return hipErrorInvalidValue;
}

// dQ tilings: block_m = queries per workgroup, block_n = keys per inner step.
hipError_t launch_dq_bf16(const void* q, const void* k, const void* v, const void* dO,
                          const float* lse, const float* delta, void* dq,
                          int bh, int nq, int nk, int d, float scale, int causal, int window, int bm, int bn,
                          hipStream_t st) {
  if (d == 128 && bm == 128 && bn == 32)
    return launch_dq_inst<128, 32, 4, 32>(q, k, v, dO, lse, delta, dq, bh, nq, nk, scale, causal, window, st);
  if (d == 128 && bm == 256 && bn == 32)
    return launch_dq_inst<128, 32, 8, 32>(q, k, v, dO, lse, delta, dq, bh, nq, nk, scale, causal, window, st);
  if (d == 128 && bm == 128 && bn == 64)
    return launch_dq_inst<128, 32, 4, 64>(q, k, v, dO, lse, delta, dq, bh, nq, nk, scale, causal, window, st);
  if (d == 64 && bm == 128 && bn == 32)
    return launch_dq_inst<64, 32, 4, 32>(q, k, v, dO, lse, delta, dq, bh, nq, nk, scale, causal, window, st);
  if (d == 64 && bm == 256 && bn == 64)
    return launch_dq_inst<64, 32, 8, 64>(q, k, v, dO, lse, delta, dq, bh, nq, nk, scale, causal, window, st);
  if (d == 64 && bm == 128 && bn == 64)
    return launch_dq_inst<64, 32, 4, 64>(q, k, v, dO, lse, delta, dq, bh, nq, nk, scale, causal, window, st);
  return hipErrorInvalidValue;
}

}  // namespace fa

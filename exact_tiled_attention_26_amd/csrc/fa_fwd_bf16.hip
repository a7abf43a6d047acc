// bf16 forward kernel: exact attention with an online softmax over key tiles.
//
// Method: "Assignment2: FlashAttention & Distributed Data Parallel notes"
// (CS336) section 1.2 -- per query tile keep a running max m, a running sum l
// and an unnormalised accumulator that is rescaled by exp(m - m_new) when the
// max grows; divide by l once at the end and save L = m + log l.  Section
// 1.3 -- one workgroup per (head, query tile); key tiles that start after the
// tile's last query are skipped in causal mode.  Only tiles crossing the
// diagonal are masked ("CS349E lecture 11, 03_flash_backward.py",
// demo4_causal).  With a sliding window ("CS324 lecture 8,
// 03_online_softmax_and_flash.py", window_attention_torch) tiles wholly
// before the band are skipped too and its lower edge is masked the same way.
//
// Mapping onto gfx950:
// * A workgroup owns BR = NW * QW query rows of one head; wave w owns QW rows.
//   The wave keeps its Q rows in registers for the whole kernel as the B
//   operand of S^T = K Q^T (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
// * Key/value tiles of BC rows go from HBM straight into swizzled,
//   double-buffered LDS tiles with global_load_lds (no staging registers);
//   the copy of tile j+1 runs while tile j is computed, one barrier per tile
//   -- or, with four buffers per operand, tiles go in pairs: the next pair
//   is copied while one pair is computed, one barrier per pair.
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
//   with the tile index) within groups of heads whose tiles are all in
//   flight together, every tile of a head on one XCD, for L2 reuse of K/V
//   (head_and_tile).
#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

constexpr float kRescaleSlack = 8.0f;
// LDS buffers per operand: 4 (steps in pairs, one barrier per pair) where
// the 4 x 2 tiles still leave room for the workgroups a CU can hold, else 2
// (d = 128 with four waves: 128 KB would allow one workgroup per CU)
template <int D, int NW>
constexpr int fwd_buffers() { return (D == 128 && NW == 4) ? 2 : 4; }

// nq query rows attend to nk key rows; causal masking is aligned to the end
// of the key sequence (query i sees keys 0 .. i + nk - nq), and a window > 0
// hides keys at or below i + nk - nq - window.
// RAGGED: nk may not be a multiple of BC (the last key tile needs the mask).
// BAND: causal with a window (0 < window < nk).
template <int D, int QW, int NW, int BC, bool CAUSAL, bool RAGGED, bool BAND, int NBUF>
__global__ __launch_bounds__(NW * 64, 2)
void fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                     const __bf16* __restrict__ V, __bf16* __restrict__ O,
                     float* __restrict__ LSE, int bh, int nq, int nk, int window, int hg,
                     float scale_log2) {
  constexpr int BR = QW * NW;
  constexpr int NQB = QW / 16;   // 16-query blocks per wave
  constexpr int NKB = BC / 16;   // 16-key blocks per tile
  constexpr int NDS = D / 32;    // 32-wide steps over the head dim (S)
  constexpr int NDB = D / 16;    // 16-wide blocks of the head dim (O)
  constexpr int NKS = BC / 32;   // 32-key steps (PV)
  constexpr int US = NDS * NKB;  // MFMA steps of S  (each NQB MFMAs)
  constexpr int UP = NKS * NDB;  // MFMA steps of PV (each NQB MFMAs)
  constexpr int NE = NKB * NQB * 4;   // probabilities per lane per tile
  static_assert(US == UP, "the two products of a tile are interleaved step by step");
  static_assert(NKS == 2, "probabilities are produced in two halves, one per PV half");
  static_assert(NBUF == 2 || NBUF == 3 || NBUF == 4, "double, triple or pairwise buffering");
  static_assert(!BAND || CAUSAL, "a window narrows causal attention");

  // NBUF LDS buffers per operand; K runs one tile ahead of V, and every copy
  // is issued NBUF - 1 steps before its data is used
  __shared__ __bf16 k_lds[NBUF][BC * D];
  __shared__ __bf16 v_lds[NBUF][BC * D];

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
  const __bf16* Qh = Q + (size_t)head * nq * D;
  const __bf16* Kh = K + (size_t)head * nk * D;
  const __bf16* Vh = V + (size_t)head * nk * D;

  const int kend = CAUSAL ? min(nk, q0 + BR + off) : nk;   // keys this workgroup can see
  const int ntk = (kend + BC - 1) / BC;
  // first key tile a row of the workgroup can see
  const int jt0 = BAND ? max(0, q0 + lo + 1) / BC : 0;
  // first and last key tiles with a key that one of this wave's rows can see
  // (dz: see divergent_zero)
  const int dz = divergent_zero();
  const int first = BAND ? max(jt0, (q0w + lo + 1) / BC) : 0;
  const int last = CAUSAL ? min(ntk - 1, (q0w + QW - 1 + off) / BC) : ntk - 1 + dz;
  const AsyncTileCopy<D, BC, NW> copier(wave, lane);
  // buffers are indexed by the tile's position t - jt0 in the loop
  // LDS byte addresses of the buffers: the copies take these, not pointers
  constexpr unsigned TB = BC * D * 2;
  const unsigned kbase = lds_address(&k_lds[0][0]), vbase = lds_address(&v_lds[0][0]);
  copier.issue_at(kbase, Kh + (size_t)jt0 * BC * D, nk - jt0 * BC);
  if (jt0 + 1 < ntk) copier.issue_at(kbase + TB, Kh + (size_t)(jt0 + 1) * BC * D, nk - (jt0 + 1) * BC);
  copier.issue_at(vbase, Vh + (size_t)jt0 * BC * D, nk - jt0 * BC);

  // Q rows of this wave as B operands: lane holds Q[q0w + 16qb + l16][32ds + 8g .. +7]
  bf16x8 qf[NQB][NDS];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int row = q0w + 16 * qb + l16;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      if (row < nq) {
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
  // running max (exponent base) and this lane's part of the running sum;
  // mb = m, or 0 while m = -inf (so that -inf - (-inf) never occurs), and
  // mraw = (m + slack) / (scale log2 e), the vote's threshold in raw score
  // units; both change only where m does
  float m[NQB], lsum[NQB], mb[NQB], mraw[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) { m[qb] = kNegInf; lsum[qb] = 0.f; mb[qb] = 0.f; mraw[qb] = kNegInf; }
  const float inv_sl2 = 1.f / scale_log2;

  const NatReader<D> kread(l16, g);
  const TrReader<D> vread(l16, g);

  // Scores are kept transposed, S^T[key][query]: lane holds key 16kb + 4g + i
  // of the tile and query 16qb + l16 of the wave.  Two register sets hold the
  // scores of consecutive tiles: the products of tile t+1 are issued while
  // the probabilities of tile t are formed (software pipelining across
  // tiles, so matrix and vector units work at the same time).
  f32x4 sa[NKB][NQB], sb[NKB][NQB];

  // does key tile j need the in-tile mask for this wave?
  auto tile_masked = [&](int j) __attribute__((always_inline)) {
    return (CAUSAL && j * BC + BC - 1 > q0w + off) || (BAND && j * BC <= q0w + QW - 1 + lo) ||
           (RAGGED && j * BC + BC > nk + dz);
  };
  // in-tile mask: key j0 + 16kb + 4g + i is visible iff llim < 16kb + i <= lim
  auto mask_item = [&](f32x4 (&s)[NKB][NQB], int j0, int qb, int kb) __attribute__((always_inline)) {
    const int lastq = CAUSAL ? min(q0w + 16 * qb + l16 + off, nk - 1) : nk - 1;
    const int lim = lastq - j0 - 4 * g;
    const int llim = q0w + 16 * qb + l16 + lo - j0 - 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (16 * kb + i > lim || (BAND && 16 * kb + i <= llim)) s[kb][qb][i] = kNegInf;
  };
  // raw (unscaled) max of one query block over this lane's 16 keys of the
  // tile; the other three lanes of the query hold the rest of the row
  auto row_max = [&](f32x4 (&s)[NKB][NQB], int qb) __attribute__((always_inline)) {
    float t = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) t = fmaxf(t, s[kb][qb][i]);
    return t;
  };
  // raise the exponent base when some score outgrew it by the slack.  The
  // test needs only each lane's partial max and a vote (a wave ballot, which
  // lands in scalar registers, so the branch is uniform); the full row max
  // is formed in the rare taken branch.
  // (the test compares raw maxima with mraw, which is equivalent because the
  // scale is positive; a rounding at the boundary only lets a probability
  // reach 2^8 by one ulp more)
  auto update_base = [&](const float (&mx)[NQB]) __attribute__((always_inline)) {
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) grow |= !(mx[qb] <= mraw[qb]);   // true while m = -inf
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const float m_new = fmaxf(m[qb], wave_max_rows(mx[qb]) * scale_log2);
        const float corr = (m_new == kNegInf) ? 1.f : exp2_fast(m[qb] - m_new);
        m[qb] = m_new;
        mb[qb] = (m_new == kNegInf) ? 0.f : m_new;
        mraw[qb] = (m_new + kRescaleSlack) * inv_sl2;
        lsum[qb] *= corr;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db][qb] *= corr;
      }
    }
  };
  // S^T = K Q^T of one tile, K operands read PF steps ahead (no interleaving)
  auto s_gemm_plain = [&](f32x4 (&s)[NKB][NQB], const __bf16* kt) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < US; ++u) {
      const int ds = u / NKB, kb = u % NKB;
      const bf16x8 a = kread.read(kt, 16 * kb, ds);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) s[kb][qb] = mfma_bf16(a, qf[qb][ds], s[kb][qb]);
    }
  };

  // scores of key tile j (keys in kt), masked when needed, and the exponent
  // base they call for
  auto scores_only = [&](f32x4 (&s)[NKB][NQB], const __bf16* kt, int j) __attribute__((always_inline)) {
    s_gemm_plain(s, kt);
    if (tile_masked(j)) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) mask_item(s, j * BC, qb, kb);
    }
    float mx[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) mx[qb] = row_max(s, qb);
    update_base(mx);
  };

  // prologue: scores of the first key tile and the first exponent base
  if constexpr (NBUF == 4) {
    // pairs of steps share one barrier: steps 0 and 1 also need K(2), V(1)
    if (jt0 + 2 < ntk) copier.issue_at(kbase + 2 * TB, Kh + (size_t)(jt0 + 2) * BC * D, nk - (jt0 + 2) * BC);
    if (jt0 + 1 < ntk) copier.issue_at(vbase + TB, Vh + (size_t)(jt0 + 1) * BC * D, nk - (jt0 + 1) * BC);
  }
  async_copy_wait();
  // copies that step 0 waits for when the distance is two steps
  if constexpr (NBUF == 3) {
    if (jt0 + 1 < ntk) copier.issue_at(vbase + TB, Vh + (size_t)(jt0 + 1) * BC * D, nk - (jt0 + 1) * BC);
    if (jt0 + 2 < ntk) copier.issue_at(kbase + 2 * TB, Kh + (size_t)(jt0 + 2) * BC * D, nk - (jt0 + 2) * BC);
  }
  __syncthreads();
  // (a wave whose band starts later computes its first scores in the step before)
  if (!BAND || first == jt0) scores_only(sa, k_lds[0], jt0);
  __syncthreads();   // every wave is done with K(0) before its buffer is refilled

  // One pipelined step: probabilities and PV of tile t (scores in sc, values
  // in vt) interleaved with the scores of tile t+1 (into sn, keys in kn).
  //   phase A: MFMA S(t+1)       | VALU: first 3/4 of P(t)
  //   phase B: MFMA O += V^T P^T | VALU: last 1/4 of P(t), then mask and
  //                                row max of S(t+1)
  auto body = [&](f32x4 (&sc)[NKB][NQB], f32x4 (&sn)[NKB][NQB], const __bf16* kn, const __bf16* vt,
                  int t, auto has_next, auto next_masked) __attribute__((always_inline)) {
    constexpr bool HN = decltype(has_next)::value;
    constexpr bool NM = decltype(next_masked)::value;
    bf16x8 pb[NKS][NQB];
    // probability item e: score (kb, qb, i) in the order of the PV halves
    auto p_item = [&](int e) __attribute__((always_inline)) {
      const int h = e / (NE / 2), r = e % (NE / 2);
      const int qb = r / 8, kb = 2 * h + (r / 4) % 2, i = r % 4;
      const float p = exp2_fast(__builtin_fmaf(sc[kb][qb][i], scale_log2, -mb[qb]));
      sc[kb][qb][i] = p;
      lsum[qb] += p;   // fp32: the row sum sets L, which bf16 terms would not resolve
      if (r % 8 == 7) pb[h][qb] = pack_bf16(sc[2 * h][qb], sc[2 * h + 1][qb]);
    };
    constexpr int EA = 3 * NE / 4;   // items done in phase A
    // The two waves of a SIMD run the same pipeline; issue priority is
    // raised for the score products and most of the probabilities (phase A)
    // and dropped for the PV products (phase B), so that a wave in phase A
    // gets the issue slots when the other is in phase B and the two drift
    // into complementary phases (measured 1.5 % faster than equal priority;
    // the opposite assignment measured no change).
    __builtin_amdgcn_s_setprio(1);
    // phase A
    {
      constexpr int PF = 3;
      bf16x8 ka[PF];
      // steps run key block by key block (u = kb * NDS + ds), so the
      // accumulators of S(t+1) come alive one key block at a time while the
      // scores of tile t die item by item
      if constexpr (HN) {
#pragma unroll
        for (int u = 0; u < PF; ++u) ka[u] = kread.read(kn, 16 * (u / NDS), u % NDS);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < US; ++u) {
        if constexpr (HN) {
          const int kb = u / NDS, ds = u % NDS;
          const bf16x8 a = ka[u % PF];
          if (u + PF < US) ka[u % PF] = kread.read(kn, 16 * ((u + PF) / NDS), (u + PF) % NDS);
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
            sn[kb][qb] = mfma_bf16(a, qf[qb][ds], ds == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sn[kb][qb]);
        }
#pragma unroll
        for (int e = u * EA / US; e < (u + 1) * EA / US; ++e) p_item(e);
        // order within the step: product, vector op, LDS read, product,
        // vector op, the rest after (measured about 1 % faster causal than
        // the compiler's own order; the same in phase B measured no gain)
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);   // VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // phase B
    {
      constexpr int PF = 3;
      constexpr int EB = NE - EA;           // probability items left
      constexpr int HB = UP / 2;            // steps in each PV half
      bf16x8 va[PF];
#pragma unroll
      for (int u = 0; u < PF; ++u)
        va[u] = cat(vread.read(vt, 32 * (u / NDB), u % NDB), vread.read(vt, 32 * (u / NDB) + 16, u % NDB));
      __builtin_amdgcn_sched_barrier(0);
      float mx[NQB];
#pragma unroll
      for (int u = 0; u < UP; ++u) {
        const int h = u / NDB, db = u % NDB;
        const bf16x8 a = va[u % PF];
        if (u + PF < UP) {
          const int h2 = (u + PF) / NDB, db2 = (u + PF) % NDB;
          va[u % PF] = cat(vread.read(vt, 32 * h2, db2), vread.read(vt, 32 * h2 + 16, db2));
        }
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) acc[db][qb] = mfma_bf16(a, pb[h][qb], acc[db][qb]);
        if (u < HB) {
#pragma unroll
          for (int e = EA + u * EB / HB; e < EA + (u + 1) * EB / HB; ++e) p_item(e);
        } else if constexpr (HN) {
          // second half: mask (when needed) and row max of the next tile
          const int v = u - HB;
          if constexpr (NM) {
            constexpr int MI = (NQB * NKB + HB - 1) / HB;   // mask items per step
#pragma unroll
            for (int w = v * MI; w < (v + 1) * MI && w < NQB * NKB; ++w) mask_item(sn, (t + 1) * BC, w / NKB, w % NKB);
          } else {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
              if (v == (2 * qb + 1) * HB / (2 * NQB)) mx[qb] = row_max(sn, qb);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (HN) {
        if constexpr (NM) {
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) mx[qb] = row_max(sn, qb);
        }
        update_base(mx);
      }
    }
  };

  // Step t: K(t+1) and V(t) are resident.  Copy K(t+NBUF) and V(t+NBUF-1)
  // into the buffers that step t-1 finished with, run the pipelined body when
  // this wave has rows that see tile t (with a window, only the scores of
  // tile t+1 in the step before the wave's first tile), then wait for the
  // copies that step t+1 needs and synchronise.
  // NBUF = 4: steps go in pairs (t, t+1) with one barrier after the pair.
  // K(t+1), K(t+2), V(t), V(t+1) are resident when the pair starts; its first
  // step copies the next pair's K(t+3), K(t+4), V(t+2), V(t+3) into the
  // buffers the previous pair finished with.  ph = (t - jt0) mod 4, a
  // compile-time constant, so every buffer address is one.
  constexpr int PER = AsyncTileCopy<D, BC, NW>::PER_WAVE;   // copy instructions per tile and wave
  auto step = [&](f32x4 (&sc)[NKB][NQB], f32x4 (&sn)[NKB][NQB], int t, auto ph) __attribute__((always_inline)) {
    const int r = NBUF == 4 ? decltype(ph)::value : t - jt0;
    const int b0 = r % NBUF, b1 = (r + 1) % NBUF, bl = (r + NBUF - 1) % NBUF;
    const bool ck = t + NBUF < ntk, cv = t + NBUF - 1 < ntk;
    if constexpr (NBUF == 4) {
      if (r % 2 == 0) {
        if (t + 2 < ntk) copier.issue_at(vbase + ((r + 2) % 4) * TB, Vh + (size_t)(t + 2) * BC * D, nk - (t + 2) * BC);
        if (t + 3 < ntk) {
          copier.issue_at(kbase + ((r + 3) % 4) * TB, Kh + (size_t)(t + 3) * BC * D, nk - (t + 3) * BC);
          copier.issue_at(vbase + ((r + 3) % 4) * TB, Vh + (size_t)(t + 3) * BC * D, nk - (t + 3) * BC);
        }
        if (t + 4 < ntk) copier.issue_at(kbase + b0 * TB, Kh + (size_t)(t + 4) * BC * D, nk - (t + 4) * BC);
      }
    } else {
      if (cv) copier.issue_at(vbase + bl * TB, Vh + (size_t)(t + NBUF - 1) * BC * D, nk - (t + NBUF - 1) * BC);
      if (ck) copier.issue_at(kbase + b0 * TB, Kh + (size_t)(t + NBUF) * BC * D, nk - (t + NBUF) * BC);
    }
    if (t <= last && (!BAND || t >= first)) {
      const __bf16* kn = k_lds[b1];
      const __bf16* vt = v_lds[b0];
      if (t + 1 <= last) {
        if ((CAUSAL || RAGGED) && tile_masked(t + 1)) {
          body(sc, sn, kn, vt, t, std::true_type{}, std::true_type{});
        } else {
          body(sc, sn, kn, vt, t, std::true_type{}, std::false_type{});
        }
      } else {
        body(sc, sn, kn, vt, t, std::false_type{}, std::false_type{});
      }
    } else if constexpr (BAND) {
      if (t + 1 == first && first <= last) scores_only(sn, k_lds[b1], t + 1);
    }
    if constexpr (NBUF == 4) {
      if (r % 2 == 1 || t + 1 >= ntk) {
        async_copy_wait();
        __syncthreads();
      }
    } else {
      if constexpr (NBUF == 3) {
        if (ck) async_copy_wait_allbut<2 * PER>();
        else if (cv) async_copy_wait_allbut<PER>();
        else async_copy_wait();
      } else {
        async_copy_wait();
      }
      __syncthreads();
    }
  };

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  if constexpr (NBUF == 4) {
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;
#pragma unroll 1
    for (int t = jt0; t < ntk; t += 4) {
      step(sa, sb, t, P0{});
      if (t + 1 < ntk) step(sb, sa, t + 1, P1{});
      if (t + 2 < ntk) step(sa, sb, t + 2, P2{});
      if (t + 3 < ntk) step(sb, sa, t + 3, P3{});
    }
  } else {
#pragma unroll 1
    for (int t = jt0; t < ntk; t += 2) {
      step(sa, sb, t, P0{});
      if (t + 1 < ntk) step(sb, sa, t + 1, P1{});
    }
  }

  // epilogue: O = acc / l, L = (m + log2 l) * ln 2
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float lt = wave_sum_xor16_32(lsum[qb]);
    const float inv = 1.f / lt;
    const int qr = q0w + 16 * qb + l16;
    if (qr < nq) {
      __bf16* orow = O + (size_t)head * nq * D + (size_t)qr * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        bf16x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = (__bf16)(acc[db][qb][i] * inv);
        *reinterpret_cast<bf16x4*>(orow + 16 * db + 4 * g) = o4;
      }
      if (g == 0) LSE[(size_t)head * nq + qr] = (m[qb] + __builtin_amdgcn_logf(lt)) * kLn2;
    }
  }
}

template <int D, int QW, int NW, int BC>
static hipError_t launch_fwd_inst(const void* q, const void* k, const void* v, void* o, float* lse,
                                  int bh, int nq, int nk, float scale, int causal, int window,
                                  hipStream_t st) {
  constexpr int BR = QW * NW;
  const int ntq = (nq + BR - 1) / BR;
  const dim3 grid((unsigned)(ntq * bh)), block(NW * 64);
  const float sl2 = scale * kLog2e;
  constexpr int NB = fwd_buffers<D, NW>();
  auto kern = (causal && window > 0) ? fwd_bf16_kernel<D, QW, NW, BC, true, true, true, NB>
            : causal ? fwd_bf16_kernel<D, QW, NW, BC, true, true, false, NB>
            : (nk % BC) ? fwd_bf16_kernel<D, QW, NW, BC, false, true, false, NB>
                       : fwd_bf16_kernel<D, QW, NW, BC, false, false, false, NB>;
  const int hg = head_group((const void*)kern, NW * 64, bh, ntq, st);
  hipLaunchKernelGGL(kern, grid, block, 0, st, (const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                     (__bf16*)o, lse, bh, nq, nk, window, hg, sl2);
  return hipGetLastError();
}

// Tuned tilings: (head dim, BR, BC) -> instance.
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int bh, int nq, int nk, int d, float scale, int causal, int window, int bm, int bn,
                           hipStream_t st) {
  if (d == 128 && bm == 128 && bn == 64) return launch_fwd_inst<128, 32, 4, 64>(q, k, v, o, lse, bh, nq, nk, scale, causal, window, st);
  if (d == 128 && bm == 256 && bn == 64) return launch_fwd_inst<128, 32, 8, 64>(q, k, v, o, lse, bh, nq, nk, scale, causal, window, st);
  if (d == 64 && bm == 128 && bn == 64) return launch_fwd_inst<64, 32, 4, 64>(q, k, v, o, lse, bh, nq, nk, scale, causal, window, st);
  if (d == 64 && bm == 256 && bn == 64) return launch_fwd_inst<64, 32, 8, 64>(q, k, v, o, lse, bh, nq, nk, scale, causal, window, st);
  return hipErrorInvalidValue;
}

}  // namespace fa

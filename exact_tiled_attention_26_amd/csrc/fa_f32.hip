// float32 kernels with run-time tile sizes: forward, dK/dV and dQ.
//
// Same method as the bf16 kernels ("Assignment2: FlashAttention & Distributed
// Data Parallel notes" (CS336) sections 1.2-1.4), computed entirely in fp32
// with v_mfma_f32_16x16x4_f32 (no reduced-precision operands).  These serve
// float32 I/O and any tiling the pages use: query tiles of 16-128 rows and
// key tiles of 4-128 columns (multiples of 4, e.g. the 16 x 12 tiling of the
// gradient check in "CS349E lecture 11, 03_flash_backward.py").  Every wave
// owns 16 query rows (forward, dQ) or 16 key rows (dK/dV); a key tile that
// is not a multiple of 16 occupies a 16-wide fragment whose extra columns are
// masked, the same mechanism as the ragged end of the sequence.
//
// Tiles sit in LDS as [rows][D + 1] floats (odd row stride: the 16 rows a
// fragment reads fall in distinct banks).
#include <algorithm>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

constexpr int kMaxBlk = 8;   // 128 / 16

template <int D>
__device__ __forceinline__ void stage_f32_rows(float* dst, const float* src, int rows_alloc,
                                               int valid, int tid, int nthr) {
  constexpr int LD = D + 1;
  for (int e = tid; e < rows_alloc * D; e += nthr) {
    const int r = e / D, c = e % D;
    dst[r * LD + c] = (r < valid) ? src[(size_t)r * D + c] : 0.f;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512)
void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                    const float* __restrict__ V, float* __restrict__ O, float* __restrict__ LSE,
                    int bh, int nq, int nk, int window, float scale_log2, int BR, int BC) {
  extern __shared__ float smem[];
  constexpr int LD = D + 1, NST = D / 4, NDB = D / 16;
  const int BCP = (BC + 15) & ~15, nkb = BCP / 16;
  float* ks = smem;
  float* vs = smem + BCP * LD;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int ntq = (nq + BR - 1) / BR;
  const int head = blockIdx.x % bh;
  const int q0 = (ntq - 1 - blockIdx.x / bh) * BR;
  const int q0w = q0 + 16 * wave;
  const int qr = q0w + l16;
  const int off = CAUSAL ? nk - nq : 0;   // query i sees keys 0 .. i + off
  const int lo = window_lo(CAUSAL, off, window);   // ... and only keys above i + lo
  const size_t hoffq = (size_t)head * nq * D, hoffk = (size_t)head * nk * D;

  // B operand of S^T = K Q^T: lane holds Q[qr][4st + g]
  float qf[NST];
#pragma unroll
  for (int st = 0; st < NST; ++st) qf[st] = (qr < nq) ? Q[hoffq + (size_t)qr * D + 4 * st + g] : 0.f;
  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, lsum = 0.f;

  const int kend = CAUSAL ? min(nk, q0 + BR + off) : nk;
  const int ntk = (kend + BC - 1) / BC;
  const int jt0 = max(0, q0 + lo + 1) / BC;   // first key tile any row can see
  for (int j = jt0; j < ntk; ++j) {
    const int j0 = j * BC;
    const int valid = min(BC, nk - j0);
    __syncthreads();
    stage_f32_rows<D>(ks, K + hoffk + (size_t)j0 * D, BCP, valid, tid, nthr);
    stage_f32_rows<D>(vs, V + hoffk + (size_t)j0 * D, BCP, valid, tid, nthr);
    __syncthreads();
    if (CAUSAL && (j0 > q0w + 15 + off || j0 + BC - 1 <= q0w + lo)) continue;
    // S^T: lane holds key j0 + 16kb + 4g + i, query qr
    f32x4 s[kMaxBlk];
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < kMaxBlk; ++kb) {
      if (kb < nkb) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < NST; ++st) c = mfma_f32(ks[(16 * kb + l16) * LD + 4 * st + g], qf[st], c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kl = 16 * kb + 4 * g + i;
          if (kl >= valid || (CAUSAL && (j0 + kl > qr + off || j0 + kl <= qr + lo))) c[i] = kNegInf;
          mx = fmaxf(mx, c[i]);
        }
        s[kb] = c;
      }
    }
    mx = wave_max_xor16_32(mx);
    const float m_new = fmaxf(m, mx * scale_log2);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float corr = exp2_fast(m - m_use);
    m = m_new;
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < kMaxBlk; ++kb) {
      if (kb < nkb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2_fast(__builtin_fmaf(s[kb][i], scale_log2, -m_use));
          s[kb][i] = p;
          ps += p;
        }
      }
    }
    lsum = lsum * corr + ps;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] *= corr;
    // O^T += V^T P^T: step t carries key 16kb + 4g + t for lane group g
#pragma unroll
    for (int kb = 0; kb < kMaxBlk; ++kb) {
      if (kb < nkb) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float* vrow = vs + (16 * kb + 4 * g + t) * LD;
#pragma unroll
          for (int db = 0; db < NDB; ++db) acc[db] = mfma_f32(vrow[16 * db + l16], s[kb][t], acc[db]);
        }
      }
    }
  }
  const float lt = wave_sum_xor16_32(lsum);
  if (qr < nq) {
    const float inv = 1.f / lt;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      f32x4 o4 = acc[db] * inv;
      *reinterpret_cast<f32x4*>(O + hoffq + (size_t)qr * D + 16 * db + 4 * g) = o4;
    }
    if (g == 0) LSE[(size_t)head * nq + qr] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
  }
}

// FUSED: also add scale * dS K into dQ (zeroed by the caller) with atomic
// adds, the single-kernel backward: each wave moves its 16 x 16 dS block
// through a private LDS tile so that dS is the A operand of dQ = dS K.
template <int D, bool CAUSAL, bool FUSED = false>
__global__ __launch_bounds__(512)
void dkdv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                     const float* __restrict__ V, const float* __restrict__ dO,
                     const float* __restrict__ LSE, const float* __restrict__ DELTA,
                     float* __restrict__ dK, float* __restrict__ dV, float* __restrict__ dQ,
                     int bh, int nq, int nk, int window, float scale, float scale_log2, int BR, int BC) {
  extern __shared__ float smem[];
  constexpr int LD = D + 1, NST = D / 4, NDB = D / 16;
  float* qs = smem;
  float* os = qs + BR * LD;
  float* l2s = os + BR * LD;
  float* dsm = l2s + BR;
  const int nqb = BR / 16;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int head = blockIdx.x % bh;
  const int k0 = (blockIdx.x / bh) * BC;
  const int k0w = k0 + 16 * wave;
  const int key = k0w + l16;
  const bool key_ok = key < nk && key < k0 + BC;
  const int off = CAUSAL ? nk - nq : 0;   // query i sees keys 0 .. i + off
  const int lo = window_lo(CAUSAL, off, window);   // ... and only keys above i + lo
  const size_t hoffq = (size_t)head * nq * D, hoffk = (size_t)head * nk * D;

  // B operands of S = Q K^T and dP = dO V^T: lane holds K[key][4st + g], V[key][4st + g]
  float kf[NST], vf[NST];
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    kf[st] = key_ok ? K[hoffk + (size_t)key * D + 4 * st + g] : 0.f;
    vf[st] = key_ok ? V[hoffk + (size_t)key * D + 4 * st + g] : 0.f;
  }
  f32x4 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const int ntq = (nq + BR - 1) / BR;
  const int it0 = CAUSAL ? max(0, k0 - off) / BR : 0;   // earlier queries see none of these keys
  // later queries see none of them either once the window has passed them
  const int it1 = min(ntq, max(0, k0 + BC - 2 - lo) / BR + 1);
  for (int it = it0; it < it1; ++it) {
    const int i0 = it * BR;
    const int valid = min(BR, nq - i0);
    __syncthreads();
    stage_f32_rows<D>(qs, Q + hoffq + (size_t)i0 * D, BR, valid, tid, nthr);
    stage_f32_rows<D>(os, dO + hoffq + (size_t)i0 * D, BR, valid, tid, nthr);
    for (int r = tid; r < BR; r += nthr) {
      l2s[r] = (r < valid) ? LSE[(size_t)head * nq + i0 + r] * kLog2e : __builtin_inff();
      dsm[r] = (r < valid) ? DELTA[(size_t)head * nq + i0 + r] : 0.f;
    }
    __syncthreads();
    if (CAUSAL && (i0 + BR - 1 + off < k0w || i0 + lo >= k0w + 15)) continue;
#pragma unroll
    for (int qb = 0; qb < kMaxBlk; ++qb) {
      if (qb < nqb) {
        // S and dP: lane holds query i0 + 16qb + 4g + i, key `key`
        f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
        const float* qrow = qs + (16 * qb + l16) * LD;
        const float* orow = os + (16 * qb + l16) * LD;
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          s = mfma_f32(qrow[4 * st + g], kf[st], s);
          dp = mfma_f32(orow[4 * st + g], vf[st], dp);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rl = 16 * qb + 4 * g + i;
          float p = exp2_fast(__builtin_fmaf(s[i], scale_log2, -l2s[rl]));
          if (CAUSAL && (key > i0 + rl + off || key <= i0 + rl + lo)) p = 0.f;
          s[i] = p;
          dp[i] = p * (dp[i] - dsm[rl]);
        }
        // dV^T += dO^T P, dK^T += Q^T dS: step t carries query 16qb + 4g + t
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float* qr2 = qs + (16 * qb + 4 * g + t) * LD;
          const float* or2 = os + (16 * qb + 4 * g + t) * LD;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            dv[db] = mfma_f32(or2[16 * db + l16], s[t], dv[db]);
            dk[db] = mfma_f32(qr2[16 * db + l16], dp[t], dk[db]);
          }
        }
        if constexpr (FUSED) {
          // dS block [query 4g + i][key l16] into the wave's tile, read back
          // as A = dS[query l16][key 4st + g]; B = K[key 4st + g][16db + l16]
          float* dsw = dsm + BR + wave * 16 * 17;
#pragma unroll
          for (int i = 0; i < 4; ++i) dsw[(4 * g + i) * 17 + l16] = dp[i];
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          float a[4];
#pragma unroll
          for (int st = 0; st < 4; ++st) a[st] = dsw[l16 * 17 + 4 * st + g];
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();   // reads done before the next block's writes
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < 4; ++st) {
              const int kr = k0w + 4 * st + g;
              const float b = (kr < nk && kr < k0 + BC) ? K[hoffk + (size_t)kr * D + 16 * db + l16] : 0.f;
              acc = mfma_f32(a[st], b, acc);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int qr = i0 + 16 * qb + 4 * g + i;
              if (qr < nq)
                __hip_atomic_fetch_add(dQ + hoffq + (size_t)qr * D + 16 * db + l16, acc[i] * scale,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      }
    }
  }
  if (key_ok) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      *reinterpret_cast<f32x4*>(dK + hoffk + (size_t)key * D + 16 * db + 4 * g) = dk[db] * scale;
      *reinterpret_cast<f32x4*>(dV + hoffk + (size_t)key * D + 16 * db + 4 * g) = dv[db];
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512)
void dq_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                   const float* __restrict__ V, const float* __restrict__ dO,
                   const float* __restrict__ LSE, const float* __restrict__ DELTA,
                   float* __restrict__ dQ, int bh, int nq, int nk, int window, float scale,
                   float scale_log2, int BR, int BC) {
  extern __shared__ float smem[];
  constexpr int LD = D + 1, NST = D / 4, NDB = D / 16;
  const int BCP = (BC + 15) & ~15, nkb = BCP / 16;
  float* ks = smem;
  float* vs = smem + BCP * LD;
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int ntq = (nq + BR - 1) / BR;
  const int head = blockIdx.x % bh;
  const int q0 = (ntq - 1 - blockIdx.x / bh) * BR;
  const int q0w = q0 + 16 * wave;
  const int qr = q0w + l16;
  const int off = CAUSAL ? nk - nq : 0;   // query i sees keys 0 .. i + off
  const int lo = window_lo(CAUSAL, off, window);   // ... and only keys above i + lo
  const size_t hoffq = (size_t)head * nq * D, hoffk = (size_t)head * nk * D;

  float qf[NST], of[NST];
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    qf[st] = (qr < nq) ? Q[hoffq + (size_t)qr * D + 4 * st + g] : 0.f;
    of[st] = (qr < nq) ? dO[hoffq + (size_t)qr * D + 4 * st + g] : 0.f;
  }
  const float l2q = (qr < nq) ? LSE[(size_t)head * nq + qr] * kLog2e : __builtin_inff();
  const float dd = (qr < nq) ? DELTA[(size_t)head * nq + qr] : 0.f;
  f32x4 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kend = CAUSAL ? min(nk, q0 + BR + off) : nk;
  const int ntk = (kend + BC - 1) / BC;
  const int jt0 = max(0, q0 + lo + 1) / BC;   // first key tile any row can see
  for (int j = jt0; j < ntk; ++j) {
    const int j0 = j * BC;
    const int valid = min(BC, nk - j0);
    __syncthreads();
    stage_f32_rows<D>(ks, K + hoffk + (size_t)j0 * D, BCP, valid, tid, nthr);
    stage_f32_rows<D>(vs, V + hoffk + (size_t)j0 * D, BCP, valid, tid, nthr);
    __syncthreads();
    if (CAUSAL && (j0 > q0w + 15 + off || j0 + BC - 1 <= q0w + lo)) continue;
#pragma unroll
    for (int kb = 0; kb < kMaxBlk; ++kb) {
      if (kb < nkb) {
        // S^T and dP^T: lane holds key j0 + 16kb + 4g + i, query qr
        f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
        const float* krow = ks + (16 * kb + l16) * LD;
        const float* vrow = vs + (16 * kb + l16) * LD;
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          s = mfma_f32(krow[4 * st + g], qf[st], s);
          dp = mfma_f32(vrow[4 * st + g], of[st], dp);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kl = 16 * kb + 4 * g + i;
          float p = exp2_fast(__builtin_fmaf(s[i], scale_log2, -l2q));
          if (kl >= valid || (CAUSAL && (j0 + kl > qr + off || j0 + kl <= qr + lo))) p = 0.f;
          dp[i] = p * (dp[i] - dd);
        }
        // dQ^T += K^T dS^T: step t carries key 16kb + 4g + t
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float* kr2 = ks + (16 * kb + 4 * g + t) * LD;
#pragma unroll
          for (int db = 0; db < NDB; ++db) acc[db] = mfma_f32(kr2[16 * db + l16], dp[t], acc[db]);
        }
      }
    }
  }
  if (qr < nq) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<f32x4*>(dQ + hoffq + (size_t)qr * D + 16 * db + 4 * g) = acc[db] * scale;
  }
}

size_t f32_lds_bytes(int kernel, int d, int bm, int bn) {
  const size_t ld = (size_t)d + 1;
  const size_t bcp = (size_t)((bn + 15) & ~15);
  if (kernel == 1) return (2 * (size_t)bm * ld + 2 * (size_t)bm) * sizeof(float);
  if (kernel == 3)   // dK/dV with the fused dQ: one 16 x 17 dS tile per wave
    return (2 * (size_t)bm * ld + 2 * (size_t)bm + (size_t)((bn + 15) / 16) * 16 * 17) * sizeof(float);
  return 2 * bcp * ld * sizeof(float);
}

template <typename KernelT>
static hipError_t set_lds(KernelT kern, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

#define FA_F32_DISPATCH_D(MACRO) \
  switch (d) {                   \
    case 16: MACRO(16); break;   \
    case 32: MACRO(32); break;   \
    case 64: MACRO(64); break;   \
    case 128: MACRO(128); break; \
    default: return hipErrorInvalidValue; \
  }

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int bh, int nq, int nk, int d, float scale, int causal, int window, int bm, int bn,
                          hipStream_t st) {
  const size_t lds = f32_lds_bytes(0, d, bm, bn);
  const dim3 grid((unsigned)(((nq + bm - 1) / bm) * bh)), block(bm * 4);
  const float sl2 = scale * kLog2e;
#define FA_FWD_F32(DD)                                                                      \
  {                                                                                         \
    auto kern = causal ? fwd_f32_kernel<DD, true> : fwd_f32_kernel<DD, false>;              \
    hipError_t e = set_lds(kern, lds);                                                      \
    if (e != hipSuccess) return e;                                                          \
    hipLaunchKernelGGL(kern, grid, block, lds, st, q, k, v, o, lse, bh, nq, nk, window, sl2,  \
                       bm, bn);                                                             \
  }
  FA_F32_DISPATCH_D(FA_FWD_F32)
#undef FA_FWD_F32
  return hipGetLastError();
}

hipError_t launch_dkdv_f32(const float* q, const float* k, const float* v, const float* dO,
                           const float* lse, const float* delta, float* dk, float* dv,
                           int bh, int nq, int nk, int d, float scale, int causal, int window, int bm, int bn,
                           hipStream_t st) {
  const size_t lds = f32_lds_bytes(1, d, bm, bn);
  const dim3 grid((unsigned)(((nk + bn - 1) / bn) * bh)), block(((bn + 15) / 16) * 64);
  const float sl2 = scale * kLog2e;
#define FA_DKDV_F32(DD)                                                                     \
  {                                                                                         \
    auto kern = causal ? dkdv_f32_kernel<DD, true> : dkdv_f32_kernel<DD, false>;            \
    hipError_t e = set_lds(kern, lds);                                                      \
    if (e != hipSuccess) return e;                                                          \
    hipLaunchKernelGGL(kern, grid, block, lds, st, q, k, v, dO, lse, delta, dk, dv,         \
                       (float*)nullptr, bh, nq,                                             \
                       nk, window,                                                          \
                       scale, sl2, bm, bn);                                                 \
  }
  FA_F32_DISPATCH_D(FA_DKDV_F32)
#undef FA_DKDV_F32
  return hipGetLastError();
}

// p[0 .. n) = 0 with a kernel (not hipMemsetAsync), so that a captured graph
// replays it like any other node.
__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ p, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.f;
}

hipError_t launch_zero_f32(float* p, size_t n, hipStream_t st) {
  const size_t blocks = std::min<size_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

hipError_t launch_bwd_fused_f32(const float* q, const float* k, const float* v, const float* dO,
                                const float* lse, const float* delta, float* dq, float* dk, float* dv,
                                int bh, int nq, int nk, int d, float scale, int causal, int window,
                                int bm, int bn, hipStream_t st) {
  hipError_t e = launch_zero_f32(dq, (size_t)bh * nq * d, st);
  if (e != hipSuccess) return e;
  const size_t lds = f32_lds_bytes(3, d, bm, bn);
  const dim3 grid((unsigned)(((nk + bn - 1) / bn) * bh)), block(((bn + 15) / 16) * 64);
  const float sl2 = scale * kLog2e;
#define FA_FUSED_F32(DD)                                                                    \
  {                                                                                         \
    auto kern = causal ? dkdv_f32_kernel<DD, true, true> : dkdv_f32_kernel<DD, false, true>; \
    e = set_lds(kern, lds);                                                                 \
    if (e != hipSuccess) return e;                                                          \
    hipLaunchKernelGGL(kern, grid, block, lds, st, q, k, v, dO, lse, delta, dk, dv, dq, bh, \
                       nq, nk, window, scale, sl2, bm, bn);                                 \
  }
  FA_F32_DISPATCH_D(FA_FUSED_F32)
#undef FA_FUSED_F32
  return hipGetLastError();
}

hipError_t launch_dq_f32(const float* q, const float* k, const float* v, const float* dO,
                         const float* lse, const float* delta, float* dq,
                         int bh, int nq, int nk, int d, float scale, int causal, int window, int bm, int bn,
                         hipStream_t st) {
  const size_t lds = f32_lds_bytes(2, d, bm, bn);
  const dim3 grid((unsigned)(((nq + bm - 1) / bm) * bh)), block(bm * 4);
  const float sl2 = scale * kLog2e;
#define FA_DQ_F32(DD)                                                                       \
  {                                                                                         \
    auto kern = causal ? dq_f32_kernel<DD, true> : dq_f32_kernel<DD, false>;                \
    hipError_t e = set_lds(kern, lds);                                                      \
    if (e != hipSuccess) return e;                                                          \
    hipLaunchKernelGGL(kern, grid, block, lds, st, q, k, v, dO, lse, delta, dq, bh, nq, nk,  \
                       window,                                                              \
                       scale, sl2, bm, bn);                                                 \
  }
  FA_F32_DISPATCH_D(FA_DQ_F32)
#undef FA_DQ_F32
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// D_i = sum_k O_ik dO_ik ("Assignment2 ... notes" section 1.4, Eq 17; the
// identity of "CS349E lecture 11" demo1_gradcheck that needs one row of O and
// dO only).  Each thread multiplies one 16-byte chunk of a row in fp32; the
// lanes of a row are reduced with cross-lane adds.  HBM-bound streaming pass.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256)
void preprocess_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                       float* __restrict__ delta, long long rows) {
  constexpr int EPT = 16 / (int)sizeof(T);   // elements per 16-byte chunk
  constexpr int LPR = D / EPT;                // lanes per row
  constexpr int RPB = 256 / LPR;              // rows per block
  static_assert(LPR >= 1 && LPR <= 64, "row must fit in a wave");
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = (threadIdx.x % LPR) * EPT;
  float acc = 0.f;
  if (row < rows) {
    typedef T vec_t __attribute__((ext_vector_type(EPT)));
    const vec_t o = *reinterpret_cast<const vec_t*>(O + row * D + c);
    const vec_t g = *reinterpret_cast<const vec_t*>(dO + row * D + c);
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc = __builtin_fmaf((float)o[e], (float)g[e], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && (threadIdx.x % LPR) == 0) delta[row] = acc;
}

template <typename T, int D>
static hipError_t launch_pre_inst(const void* o, const void* dO, float* delta, long long rows,
                                  hipStream_t st) {
  constexpr int LPR = D / (16 / (int)sizeof(T));
  constexpr int RPB = 256 / LPR;
  const dim3 grid((unsigned)((rows + RPB - 1) / RPB)), block(256);
  hipLaunchKernelGGL((preprocess_kernel<T, D>), grid, block, 0, st, (const T*)o, (const T*)dO,
                     delta, rows);
  return hipGetLastError();
}

hipError_t launch_preprocess(const void* o, const void* dO, float* delta, int bh, int nq, int d,
                             int dtype, hipStream_t st) {
  const long long rows = (long long)bh * nq;
  if (dtype == 0) {
    switch (d) {
      case 16: return launch_pre_inst<float, 16>(o, dO, delta, rows, st);
      case 32: return launch_pre_inst<float, 32>(o, dO, delta, rows, st);
      case 64: return launch_pre_inst<float, 64>(o, dO, delta, rows, st);
      case 128: return launch_pre_inst<float, 128>(o, dO, delta, rows, st);
    }
  } else {
    switch (d) {
      case 64: return launch_pre_inst<__bf16, 64>(o, dO, delta, rows, st);
      case 128: return launch_pre_inst<__bf16, 128>(o, dO, delta, rows, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace fa

// Host-side launchers behind the C ABI (include/fa.h).  Each returns the
// HIP error of its launch; arguments were validated by the caller.  A tiling
// that has no kernel instance returns hipErrorInvalidValue.
//
// nq query rows (Q, O, dO, dQ, L, D) attend to nk key rows (K, V, dK, dV).
// Causal masking is aligned to the end of the key sequence: query i sees key
// j iff j <= i + (nk - nq); the caller guarantees nk >= nq when causal and
// nq, nk >= 1.  window > 0 (causal only) also hides keys j <= i + (nk - nq)
// - window, so that each query sees its `window` most recent keys.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int bh, int nq, int nk, int d, float scale, int causal, int window, int bm, int bn,
                           hipStream_t st);
hipError_t launch_dkdv_bf16(const void* q, const void* k, const void* v, const void* dO,
                            const float* lse, const float* delta, void* dk, void* dv,
                            int bh, int nq, int nk, int d, float scale, int causal, int window, int bm, int bn,
                            hipStream_t st);
hipError_t launch_dq_bf16(const void* q, const void* k, const void* v, const void* dO,
                          const float* lse, const float* delta, void* dq,
                          int bh, int nq, int nk, int d, float scale, int causal, int window, int bm, int bn,
                          hipStream_t st);

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int bh, int nq, int nk, int d, float scale, int causal, int window, int bm, int bn,
                          hipStream_t st);
hipError_t launch_dkdv_f32(const float* q, const float* k, const float* v, const float* dO,
                           const float* lse, const float* delta, float* dk, float* dv,
                           int bh, int nq, int nk, int d, float scale, int causal, int window, int bm, int bn,
                           hipStream_t st);
hipError_t launch_dq_f32(const float* q, const float* k, const float* v, const float* dO,
                         const float* lse, const float* delta, float* dq,
                         int bh, int nq, int nk, int d, float scale, int causal, int window, int bm, int bn,
                         hipStream_t st);

// Single-kernel backward (dK, dV and dQ in one pass over the key tiles, dQ
// accumulated with fp32 atomic adds).  bf16: dq_acc is an fp32 workspace of
// bh * nq * d floats that the call clears and then rounds into dq; float32:
// dq itself is cleared and accumulated.  Tilings: the dK/dV ones whose query
// tile is 64 rows (bf16), any dK/dV tiling (float32).
hipError_t launch_bwd_fused_bf16(const void* q, const void* k, const void* v, const void* dO,
                                 const float* lse, const float* delta, void* dq, void* dk, void* dv,
                                 float* dq_acc, int bh, int nq, int nk, int d, float scale, int causal,
                                 int window, int bm, int bn, hipStream_t st);
hipError_t launch_bwd_fused_f32(const float* q, const float* k, const float* v, const float* dO,
                                const float* lse, const float* delta, float* dq, float* dk, float* dv,
                                int bh, int nq, int nk, int d, float scale, int causal, int window,
                                int bm, int bn, hipStream_t st);
// The same for bf16 with the fp32 dQ accumulator in the library's fixed
// device scratch array instead of a caller workspace (no allocation); the
// caller guarantees bh * nq * d * 4 <= kNoAllocScratchBytes.
constexpr size_t kNoAllocScratchBytes = size_t(1) << 27;
hipError_t launch_bwd_fused_bf16_noalloc(const void* q, const void* k, const void* v, const void* dO,
                                         const float* lse, const float* delta, void* dq, void* dk, void* dv,
                                         int bh, int nq, int nk, int d, float scale, int causal, int window,
                                         int bm, int bn, hipStream_t st);
// p[0 .. n) = 0 (a fill kernel, safe under graph capture)
hipError_t launch_zero_f32(float* p, size_t n, hipStream_t st);

// Heads per group for the workgroup order (fa_order.h), from how many
// workgroups of `kern` (`threads` each) the stream's device runs at once:
// the occupancy query's workgroups per CU times the device's CUs, cached
// per device and kernel.
int head_group(const void* kern, int threads, int bh, int ntiles, hipStream_t st);

// dtype: 0 = float32, 1 = bf16
hipError_t launch_preprocess(const void* o, const void* dO, float* delta, int bh, int nq, int d,
                             int dtype, hipStream_t st);

// LDS bytes the float32 kernels need for a tiling (host-side check).
size_t f32_lds_bytes(int kernel, int d, int bm, int bn);

}  // namespace fa

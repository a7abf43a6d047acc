// C ABI of libfa.so (declared in include/fa.h): argument validation and
// dispatch to the kernel launchers.  Validation runs entirely on the host and
// before any HIP call, so a rejected call launches nothing and needs no GPU.
#include <cmath>
#include <cstdint>
#include <initializer_list>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace {

constexpr int kMaxN = 1 << 24;          // keeps row * D offsets and grids in range
constexpr int kMaxBH = 1 << 20;
constexpr size_t kLdsBudget = 160 * 1024;

enum Kernel { kFwd = 0, kDkdv = 1, kDq = 2, kFused = 3 };

struct Tiles { int bm, bn; };

// Tuned bf16 tilings; the first entry per (kernel, d) is the default.
struct Bf16Tiling { int kernel, d, bm, bn; };
constexpr Bf16Tiling kBf16Tilings[] = {
    {kFwd, 128, 256, 64},  {kFwd, 128, 128, 64},
    {kFwd, 64, 128, 64},   {kFwd, 64, 256, 64},
    {kDkdv, 128, 128, 128}, {kDkdv, 128, 64, 128}, {kDkdv, 64, 128, 128}, {kDkdv, 64, 64, 128},
    {kDq, 128, 256, 32},   {kDq, 128, 128, 32},   {kDq, 128, 128, 64},   {kDq, 64, 128, 64},   {kDq, 64, 128, 32},   {kDq, 64, 256, 64},
    {kFused, 128, 64, 128}, {kFused, 64, 64, 128},
};

// bf16 forward default at d = 128 when a sliding window is set (measured at
// 32 x 8192 x 128: 16 % faster at a 256-key window, 8 % at 1024)
constexpr Tiles kFwdWindowTiles = {128, 64};
// the same holds for dQ: four-wave, 128-query tiles with a window (at a
// 256-key window 0.116 against 0.135 ms for the 256-query default)
constexpr Tiles kDqWindowTiles = {128, 32};

// float32 defaults per kernel (fwd, dkdv, dq, fused backward), measured at
// 16 x 4096 x 64: 128-query tiles suit the forward and dQ kernels, dK/dV
// keeps 64.
constexpr Tiles kF32Defaults[] = {{128, 64}, {64, 64}, {128, 64}, {64, 64}};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool f32_head_dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool bf16_head_dim_ok(int d) { return d == 64 || d == 128; }

fa_status resolve_tiles(fa_dtype dtype, int kernel, int d, int& bm, int& bn) {
  if (dtype == FA_BF16) {
    if (!bf16_head_dim_ok(d)) return FA_ERR_UNSUPPORTED;
    if (bm == 0 && bn == 0) {
      for (const auto& t : kBf16Tilings)
        if (t.kernel == kernel && t.d == d) { bm = t.bm; bn = t.bn; return FA_OK; }
      return FA_ERR_UNSUPPORTED;
    }
    for (const auto& t : kBf16Tilings)
      if (t.kernel == kernel && t.d == d && t.bm == bm && t.bn == bn) return FA_OK;
    return FA_ERR_UNSUPPORTED;
  }
  if (!f32_head_dim_ok(d)) return FA_ERR_UNSUPPORTED;
  if (bm == 0 && bn == 0) { bm = kF32Defaults[kernel].bm; bn = kF32Defaults[kernel].bn; }
  if (!(bm == 16 || bm == 32 || bm == 64 || bm == 128)) return FA_ERR_UNSUPPORTED;
  if (bn < 4 || bn > 128 || bn % 4 != 0) return FA_ERR_UNSUPPORTED;
  if (fa::f32_lds_bytes(kernel, d, bm, bn) > kLdsBudget) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

fa_status check_common(int bh, int nq, int nk, int d, fa_dtype dtype) {
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (bh < 0 || nq < 0 || nk < 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (nq > kMaxN || nk > kMaxN || bh > kMaxBH) return FA_ERR_UNSUPPORTED;
  if (dtype == FA_F32 ? !f32_head_dim_ok(d) : !bf16_head_dim_ok(d)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Query/key lengths and window of an attention call: sets `empty` for a
// no-op call; rejects rows without keys (one length zero, or causal with
// nq > nk) and a window without causal masking.  A window of nk keys or
// more hides nothing and is cleared, which also keeps the kernels' window
// bounds (row + nk - nq - window) far from overflow.
fa_status check_lengths(int bh, int nq, int nk, int causal, int& window, bool& empty) {
  if (window < 0 || (window > 0 && !causal)) return FA_ERR_INVALID_ARG;
  if (window >= nk) window = 0;
  empty = bh == 0 || (nq == 0 && nk == 0);
  if (empty) return FA_OK;
  if (nq == 0 || nk == 0) return FA_ERR_INVALID_ARG;
  if (causal && nq > nk) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Every launch grid must stay below 2^31 workgroups.
fa_status check_grid(int bh, int n, int tile) {
  const long long tiles = ((long long)n + tile - 1) / tile;
  return tiles * (long long)bh < (1LL << 31) ? FA_OK : FA_ERR_UNSUPPORTED;
}

fa_status check_scale(float scale) {
  return (std::isfinite(scale) && scale > 0.f) ? FA_OK : FA_ERR_INVALID_ARG;
}

template <typename... P>
fa_status check_ptrs(P... ptrs) {
  const void* list[] = {static_cast<const void*>(ptrs)...};
  for (const void* p : list)
    if (p == nullptr) return FA_ERR_INVALID_ARG;
  for (const void* p : list)
    if (!aligned16(p)) return FA_ERR_MISALIGNED;
  return FA_OK;
}

// Outputs must not coincide with inputs or with each other.
bool any_equal(std::initializer_list<const void*> outs, std::initializer_list<const void*> all) {
  for (const void* o : outs) {
    int hits = 0;
    for (const void* a : all) hits += (a == o);
    if (hits != 1) return true;
  }
  return false;
}

fa_status from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

}  // namespace

extern "C" {

int fa_abi_version(void) { return FA_ABI_VERSION; }

const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head dim, tiling or size";
    case FA_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_TOO_LARGE: return "problem exceeds the fixed scratch of the allocation-free call";
  }
  return "unknown status";
}

fa_status fa_default_tiles(fa_dtype dtype, int d, int kernel, int* block_m, int* block_n) {
  if (block_m == nullptr || block_n == nullptr) return FA_ERR_INVALID_ARG;
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (kernel < 0 || kernel > 3) return FA_ERR_INVALID_ARG;
  int bm = 0, bn = 0;
  const fa_status s = resolve_tiles(dtype, kernel, d, bm, bn);
  if (s != FA_OK) return s;
  *block_m = bm;
  *block_n = bn;
  return FA_OK;
}

fa_status fa_fwd_rect(const void* q, const void* k, const void* v, void* o, float* lse,
                      int bh, int nq, int nk, int d, fa_dtype dtype, float scale, int causal,
                      int window, int block_m, int block_n, void* stream) {
  fa_status s = check_common(bh, nq, nk, d, dtype);
  if (s != FA_OK) return s;
  if ((s = check_scale(scale)) != FA_OK) return s;
  if (block_m < 0 || block_n < 0) return FA_ERR_INVALID_ARG;
  const bool default_tiles = block_m == 0 && block_n == 0;
  if ((s = resolve_tiles(dtype, kFwd, d, block_m, block_n)) != FA_OK) return s;
  bool empty = false;
  if ((s = check_lengths(bh, nq, nk, causal, window, empty)) != FA_OK || empty) return s;
  // with a window each query tile spans only a band of keys: the 128-query
  // tiling (whose waves are less far apart along the band) is the default
  if (default_tiles && window > 0 && dtype == FA_BF16 && d == 128) {
    block_m = kFwdWindowTiles.bm;
    block_n = kFwdWindowTiles.bn;
  }
  if ((s = check_grid(bh, nq, block_m)) != FA_OK) return s;
  if ((s = check_ptrs(q, k, v, o, lse)) != FA_OK) return s;
  if (any_equal({o, lse}, {q, k, v, o, lse})) return FA_ERR_INVALID_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == FA_BF16)
    return from_hip(fa::launch_fwd_bf16(q, k, v, o, lse, bh, nq, nk, d, scale, causal != 0,
                                        window, block_m, block_n, st));
  return from_hip(fa::launch_fwd_f32((const float*)q, (const float*)k, (const float*)v,
                                     (float*)o, lse, bh, nq, nk, d, scale, causal != 0, window,
                                     block_m, block_n, st));
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int bh, int n, int d, fa_dtype dtype, float scale, int causal,
                 int block_m, int block_n, void* stream) {
  return fa_fwd_rect(q, k, v, o, lse, bh, n, n, d, dtype, scale, causal, 0, block_m, block_n,
                     stream);
}

fa_status fa_bwd_preprocess(const void* o, const void* dO, float* delta,
                            int bh, int n, int d, fa_dtype dtype, void* stream) {
  fa_status s = check_common(bh, n, n, d, dtype);
  if (s != FA_OK) return s;
  if (bh == 0 || n == 0) return FA_OK;
  if ((s = check_grid(bh, n, 8)) != FA_OK) return s;  // 8+ rows per block
  if ((s = check_ptrs(o, dO, delta)) != FA_OK) return s;
  if (any_equal({delta}, {o, dO, delta})) return FA_ERR_INVALID_ARG;
  return from_hip(fa::launch_preprocess(o, dO, delta, bh, n, d, dtype == FA_BF16 ? 1 : 0,
                                        static_cast<hipStream_t>(stream)));
}

fa_status fa_bwd_dkdv_rect(const void* q, const void* k, const void* v, const void* dO,
                           const float* lse, const float* delta, void* dk, void* dv,
                           int bh, int nq, int nk, int d, fa_dtype dtype, float scale,
                           int causal, int window, int block_m, int block_n, void* stream) {
  fa_status s = check_common(bh, nq, nk, d, dtype);
  if (s != FA_OK) return s;
  if ((s = check_scale(scale)) != FA_OK) return s;
  if (block_m < 0 || block_n < 0) return FA_ERR_INVALID_ARG;
  if ((s = resolve_tiles(dtype, kDkdv, d, block_m, block_n)) != FA_OK) return s;
  bool empty = false;
  if ((s = check_lengths(bh, nq, nk, causal, window, empty)) != FA_OK || empty) return s;
  if ((s = check_grid(bh, nk, block_n)) != FA_OK) return s;
  if ((s = check_ptrs(q, k, v, dO, lse, delta, dk, dv)) != FA_OK) return s;
  if (any_equal({dk, dv}, {q, k, v, dO, lse, delta, dk, dv})) return FA_ERR_INVALID_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == FA_BF16)
    return from_hip(fa::launch_dkdv_bf16(q, k, v, dO, lse, delta, dk, dv, bh, nq, nk, d, scale,
                                         causal != 0, window, block_m, block_n, st));
  return from_hip(fa::launch_dkdv_f32((const float*)q, (const float*)k, (const float*)v,
                                      (const float*)dO, lse, delta, (float*)dk, (float*)dv, bh,
                                      nq, nk, d, scale, causal != 0, window, block_m, block_n, st));
}

fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                      const float* lse, const float* delta, void* dk, void* dv,
                      int bh, int n, int d, fa_dtype dtype, float scale, int causal,
                      int block_m, int block_n, void* stream) {
  return fa_bwd_dkdv_rect(q, k, v, dO, lse, delta, dk, dv, bh, n, n, d, dtype, scale, causal, 0,
                          block_m, block_n, stream);
}

fa_status fa_bwd_dq_rect(const void* q, const void* k, const void* v, const void* dO,
                         const float* lse, const float* delta, void* dq,
                         int bh, int nq, int nk, int d, fa_dtype dtype, float scale,
                         int causal, int window, int block_m, int block_n, void* stream) {
  fa_status s = check_common(bh, nq, nk, d, dtype);
  if (s != FA_OK) return s;
  if ((s = check_scale(scale)) != FA_OK) return s;
  if (block_m < 0 || block_n < 0) return FA_ERR_INVALID_ARG;
  const bool default_tiles = block_m == 0 && block_n == 0;
  if ((s = resolve_tiles(dtype, kDq, d, block_m, block_n)) != FA_OK) return s;
  bool empty = false;
  if ((s = check_lengths(bh, nq, nk, causal, window, empty)) != FA_OK || empty) return s;
  if (default_tiles && window > 0 && dtype == FA_BF16 && d == 128) {
    block_m = kDqWindowTiles.bm;
    block_n = kDqWindowTiles.bn;
  }
  if ((s = check_grid(bh, nq, block_m)) != FA_OK) return s;
  if ((s = check_ptrs(q, k, v, dO, lse, delta, dq)) != FA_OK) return s;
  if (any_equal({dq}, {q, k, v, dO, lse, delta, dq})) return FA_ERR_INVALID_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == FA_BF16)
    return from_hip(fa::launch_dq_bf16(q, k, v, dO, lse, delta, dq, bh, nq, nk, d, scale,
                                       causal != 0, window, block_m, block_n, st));
  return from_hip(fa::launch_dq_f32((const float*)q, (const float*)k, (const float*)v,
                                    (const float*)dO, lse, delta, (float*)dq, bh, nq, nk, d,
                                    scale, causal != 0, window, block_m, block_n, st));
}

size_t fa_bwd_fused_workspace_bytes(int bh, int nq, int d, fa_dtype dtype) {
  if (dtype != FA_BF16 || bh <= 0 || nq <= 0 || d <= 0) return 0;
  return (size_t)bh * (size_t)nq * (size_t)d * sizeof(float);
}

fa_status fa_bwd_fused(const void* q, const void* k, const void* v, const void* dO,
                       const float* lse, const float* delta, void* dq, void* dk, void* dv,
                       float* workspace, int bh, int nq, int nk, int d, fa_dtype dtype,
                       float scale, int causal, int window, int block_m, int block_n,
                       void* stream) {
  fa_status s = check_common(bh, nq, nk, d, dtype);
  if (s != FA_OK) return s;
  if ((s = check_scale(scale)) != FA_OK) return s;
  if (block_m < 0 || block_n < 0) return FA_ERR_INVALID_ARG;
  if ((s = resolve_tiles(dtype, kFused, d, block_m, block_n)) != FA_OK) return s;
  bool empty = false;
  if ((s = check_lengths(bh, nq, nk, causal, window, empty)) != FA_OK || empty) return s;
  if ((s = check_grid(bh, nk, block_n)) != FA_OK) return s;
  if ((s = check_ptrs(q, k, v, dO, lse, delta, dq, dk, dv)) != FA_OK) return s;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == FA_BF16) {
    if ((s = check_ptrs(workspace)) != FA_OK) return s;
    if (any_equal({dq, dk, dv, workspace}, {q, k, v, dO, lse, delta, dq, dk, dv, workspace}))
      return FA_ERR_INVALID_ARG;
    return from_hip(fa::launch_bwd_fused_bf16(q, k, v, dO, lse, delta, dq, dk, dv, workspace, bh, nq,
                                              nk, d, scale, causal != 0, window, block_m, block_n,
                                              st));
  }
  if (any_equal({dq, dk, dv}, {q, k, v, dO, lse, delta, dq, dk, dv})) return FA_ERR_INVALID_ARG;
  return from_hip(fa::launch_bwd_fused_f32((const float*)q, (const float*)k, (const float*)v,
                                           (const float*)dO, lse, delta, (float*)dq, (float*)dk,
                                           (float*)dv, bh, nq, nk, d, scale, causal != 0, window,
                                           block_m, block_n, st));
}

fa_status fa_bwd_fused_noalloc(const void* q, const void* k, const void* v, const void* dO,
                               const float* lse, const float* delta, void* dq, void* dk, void* dv,
                               int bh, int nq, int nk, int d, fa_dtype dtype, float scale,
                               int causal, int window, int block_m, int block_n, void* stream) {
  static_assert(FA_NOALLOC_SCRATCH_BYTES == fa::kNoAllocScratchBytes, "one scratch size");
  fa_status s = check_common(bh, nq, nk, d, dtype);
  if (s != FA_OK) return s;
  if ((s = check_scale(scale)) != FA_OK) return s;
  if (block_m < 0 || block_n < 0) return FA_ERR_INVALID_ARG;
  if ((s = resolve_tiles(dtype, kFused, d, block_m, block_n)) != FA_OK) return s;
  bool empty = false;
  if ((s = check_lengths(bh, nq, nk, causal, window, empty)) != FA_OK || empty) return s;
  if ((s = check_grid(bh, nk, block_n)) != FA_OK) return s;
  if ((s = check_ptrs(q, k, v, dO, lse, delta, dq, dk, dv)) != FA_OK) return s;
  if (any_equal({dq, dk, dv}, {q, k, v, dO, lse, delta, dq, dk, dv})) return FA_ERR_INVALID_ARG;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == FA_BF16) {
    if ((size_t)bh * (size_t)nq * (size_t)d * sizeof(float) > FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_TOO_LARGE;
    return from_hip(fa::launch_bwd_fused_bf16_noalloc(q, k, v, dO, lse, delta, dq, dk, dv, bh, nq, nk, d, scale,
                                                      causal != 0, window, block_m, block_n, st));
  }
  return from_hip(fa::launch_bwd_fused_f32((const float*)q, (const float*)k, (const float*)v,
                                           (const float*)dO, lse, delta, (float*)dq, (float*)dk,
                                           (float*)dv, bh, nq, nk, d, scale, causal != 0, window,
                                           block_m, block_n, st));
}

fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
                    const float* lse, const float* delta, void* dq,
                    int bh, int n, int d, fa_dtype dtype, float scale, int causal,
                    int block_m, int block_n, void* stream) {
  return fa_bwd_dq_rect(q, k, v, dO, lse, delta, dq, bh, n, n, d, dtype, scale, causal, 0,
                        block_m, block_n, stream);
}

}  // extern "C"

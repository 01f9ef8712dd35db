// C ABI of libswattn (declared and documented in include/swattn.h).
// Validates arguments, sizes workspaces and enqueues the kernels on the caller's
// stream.  No allocation, no host synchronisation, no global state.
#include <limits.h>

#include <cmath>
#include <initializer_list>
#include <stdint.h>

#include "launch.h"
#include "swattn.h"

namespace {

constexpr int kVersion = 103;  // 0.1.3: QK-norm + rotary prologue (swattn_qk_norm_rope*)

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Whether the product of the (non-negative) factors is at most `limit`, decided without
// forming a product that could overflow.
bool product_at_most(long long limit, std::initializer_list<long long> factors) {
  long long p = 1;
  for (long long f : factors) {
    if (f < 0) return false;
    if (f != 0 && p > limit / f) return false;
    p *= f;
  }
  return true;
}

int check_common(int B, int H, int T, int D, int window) {
  if (B <= 0 || H <= 0 || T <= 0 || D <= 0 || window == 0) return SWATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return SWATTN_ERR_UNSUPPORTED;
  // kernels index rows of [B, T, H] and grid blocks with 32-bit ints
  if (!product_at_most(INT_MAX / 2, {B, T, H}) ||
      !product_at_most(INT_MAX / 2, {B, H, ((long long)T + 127) / 128}))
    return SWATTN_ERR_INVALID_ARG;
  // buffer loads address one sequence's [T, H, D] block with 32-bit byte offsets
  if (!product_at_most(INT_MAX, {(long long)T + 128, H, D, 2})) return SWATTN_ERR_UNSUPPORTED;
  return SWATTN_OK;
}

// Hkv K/V heads shared by H query heads in contiguous groups of H / Hkv
int check_group(int H, int Hkv) {
  if (Hkv <= 0 || H % Hkv != 0) return SWATTN_ERR_INVALID_ARG;
  return SWATTN_OK;
}

// bytes of the delta part of the backward workspace (float32 [B, H, T], 256-aligned)
size_t delta_bytes(int B, int H, int T) {
  const size_t bytes = (size_t)B * H * T * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

int all_aligned(std::initializer_list<const void *> ps) {
  for (const void *p : ps)
    if (p == nullptr || !aligned16(p)) return 0;
  return 1;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SWATTN_OK : SWATTN_ERR_HIP; }

// The softmax scale must be a positive finite number: the kernels fold it into the
// exponent and mask scores before scaling, which is only the masked softmax of
// scale * Q K^T for scale > 0 (scale 0 would turn masked scores into NaN, a negative
// one would give masked keys the largest weight).
int check_scale(float scale) {
  return (scale > 0.f && std::isfinite(scale)) ? SWATTN_OK : SWATTN_ERR_INVALID_ARG;
}

int check_decode(int B, int H, int D, int Tmax, int window) {
  if (B <= 0 || H <= 0 || D <= 0 || Tmax <= 0 || window == 0) return SWATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return SWATTN_ERR_UNSUPPORTED;
  if (!product_at_most(INT_MAX / 2, {B, Tmax, H}) || B > 65535 || H > 65535)
    return SWATTN_ERR_INVALID_ARG;
  return SWATTN_OK;
}

}  // namespace

namespace swattn {

hipError_t launch_bwd_pre(bool bf16, const void *o, const void *dO, float *delta, int B, int H,
                          int T, int D, hipStream_t st) {
  return bf16 ? launch_bwd_pre_bf16(o, dO, delta, B, H, T, D, st)
              : launch_bwd_pre_f32((const float *)o, (const float *)dO, delta, B, H, T, D, st);
}

hipError_t launch_bwd_dkdv(bool bf16, const void *q, const void *k, const void *v,
                           const void *dO, const float *lse, const float *delta, void *dk,
                           void *dv, float *part, int B, int H, int Hkv, int T, int D,
                           int window, float scale, hipStream_t st) {
  if (bf16)
    return launch_bwd_dkdv_bf16(q, k, v, dO, lse, delta, dk, dv, part, B, H, Hkv, T, D, window,
                                scale, st);
  if (Hkv != H) return hipErrorInvalidValue;  // the fp32 kernels take no K/V head groups
  return launch_bwd_dkdv_f32((const float *)q, (const float *)k, (const float *)v,
                             (const float *)dO, lse, delta, (float *)dk, (float *)dv, B, H, T, D,
                             window, scale, st);
}

hipError_t launch_bwd_dq(bool bf16, const void *q, const void *k, const void *v, const void *o,
                         const void *dO, const float *lse, float *delta, void *dq, int B, int H,
                         int Hkv, int T, int D, int window, float scale, hipStream_t st) {
  if (bf16)
    return launch_bwd_dq_bf16(q, k, v, o, dO, lse, delta, dq, B, H, Hkv, T, D, window, scale,
                              st);
  if (Hkv != H) return hipErrorInvalidValue;  // the fp32 kernels take no K/V head groups
  // fp32: delta by its own kernel, then the dQ pass
  hipError_t e = launch_bwd_pre_f32((const float *)o, (const float *)dO, delta, B, H, T, D, st);
  if (e != hipSuccess) return e;
  return launch_bwd_dq_f32((const float *)q, (const float *)k, (const float *)v,
                           (const float *)dO, lse, delta, (float *)dq, B, H, T, D, window, scale,
                           st);
}

}  // namespace swattn

namespace {

int bwd_all(bool bf16, const void *q, const void *k, const void *v, const void *o,
            const void *dO, const float *lse, void *dq, void *dk, void *dv, int B, int H,
            int Hkv, int T, int D, int window, float scale, void *workspace, hipStream_t st) {
  int s = check_common(B, H, T, D, window);
  if (s == SWATTN_OK) s = check_group(H, Hkv);
  if (s == SWATTN_OK) s = check_scale(scale);
  if (s != SWATTN_OK) return s;
  if (!all_aligned({q, k, v, o, dO, dq, dk, dv, workspace}) || lse == nullptr)
    return SWATTN_ERR_INVALID_ARG;
  // the dQ pass also writes delta, which the dK/dV pass then reads; with K/V head groups
  // the per-query-head dK / dV partials follow it
  float *delta = (float *)workspace;
  float *part = (float *)((char *)workspace + delta_bytes(B, H, T));
  hipError_t e = swattn::launch_bwd_dq(bf16, q, k, v, o, dO, lse, delta, dq, B, H, Hkv, T, D,
                                        window, scale, st);
  if (e == hipSuccess)
    e = swattn::launch_bwd_dkdv(bf16, q, k, v, dO, lse, delta, dk, dv, part, B, H, Hkv, T, D,
                                window, scale, st);
  return hip_status(e);
}

int bwd_pre(bool bf16, const void *o, const void *dO, void *workspace, int B, int H, int T, int D,
            hipStream_t st) {
  int s = check_common(B, H, T, D, -1);
  if (s != SWATTN_OK) return s;
  if (!all_aligned({o, dO, workspace})) return SWATTN_ERR_INVALID_ARG;
  return hip_status(swattn::launch_bwd_pre(bf16, o, dO, (float *)workspace, B, H, T, D, st));
}

int bwd_dkdv(bool bf16, const void *q, const void *k, const void *v, const void *dO,
             const float *lse, const void *workspace, void *dk, void *dv, int B, int H, int T,
             int D, int window, float scale, hipStream_t st) {
  int s = check_common(B, H, T, D, window);
  if (s == SWATTN_OK) s = check_scale(scale);
  if (s != SWATTN_OK) return s;
  if (!all_aligned({q, k, v, dO, workspace, dk, dv}) || lse == nullptr)
    return SWATTN_ERR_INVALID_ARG;
  return hip_status(swattn::launch_bwd_dkdv(bf16, q, k, v, dO, lse, (const float *)workspace, dk,
                                            dv, nullptr, B, H, H, T, D, window, scale, st));
}

int bwd_dq(bool bf16, const void *q, const void *k, const void *v, const void *o,
           const void *dO, const float *lse, void *workspace, void *dq, int B, int H, int T,
           int D, int window, float scale, hipStream_t st) {
  int s = check_common(B, H, T, D, window);
  if (s == SWATTN_OK) s = check_scale(scale);
  if (s != SWATTN_OK) return s;
  if (!all_aligned({q, k, v, o, dO, workspace, dq}) || lse == nullptr)
    return SWATTN_ERR_INVALID_ARG;
  return hip_status(swattn::launch_bwd_dq(bf16, q, k, v, o, dO, lse, (float *)workspace, dq, B,
                                          H, H, T, D, window, scale, st));
}

}  // namespace

extern "C" {

const char *swattn_status_string(int status) {
  switch (status) {
    case SWATTN_OK: return "SWATTN_OK";
    case SWATTN_ERR_INVALID_ARG: return "SWATTN_ERR_INVALID_ARG";
    case SWATTN_ERR_UNSUPPORTED: return "SWATTN_ERR_UNSUPPORTED";
    case SWATTN_ERR_HIP: return "SWATTN_ERR_HIP";
    case SWATTN_ERR_TOO_LARGE: return "SWATTN_ERR_TOO_LARGE";
    default: return "SWATTN_ERR_UNKNOWN";
  }
}

int swattn_version(void) { return kVersion; }

int swattn_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
               int T, int D, int window, float scale, swattn_stream_t stream) {
  int st = check_common(B, H, T, D, window);
  if (st == SWATTN_OK) st = check_scale(scale);
  if (st != SWATTN_OK) return st;
  if (!all_aligned({q, k, v, o}) || lse == nullptr) return SWATTN_ERR_INVALID_ARG;
  return hip_status(swattn::launch_fwd_bf16(q, k, v, o, lse, B, H, H, T, D, window, scale,
                                            (hipStream_t)stream));
}

int swattn_fwd_gqa(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                   int H, int Hkv, int T, int D, int window, float scale,
                   swattn_stream_t stream) {
  int st = check_common(B, H, T, D, window);
  if (st == SWATTN_OK) st = check_group(H, Hkv);
  if (st == SWATTN_OK) st = check_scale(scale);
  if (st != SWATTN_OK) return st;
  if (!all_aligned({q, k, v, o}) || lse == nullptr) return SWATTN_ERR_INVALID_ARG;
  return hip_status(swattn::launch_fwd_bf16(q, k, v, o, lse, B, H, Hkv, T, D, window, scale,
                                            (hipStream_t)stream));
}

int swattn_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse, int B,
                   int H, int T, int D, int window, float scale, swattn_stream_t stream) {
  int st = check_common(B, H, T, D, window);
  if (st == SWATTN_OK) st = check_scale(scale);
  if (st != SWATTN_OK) return st;
  if (!all_aligned({q, k, v, o}) || lse == nullptr) return SWATTN_ERR_INVALID_ARG;
  return hip_status(swattn::launch_fwd_f32(q, k, v, o, lse, B, H, T, D, window, scale,
                                           (hipStream_t)stream));
}

size_t swattn_bwd_workspace_size(int B, int H, int T, int D) {
  if (check_common(B, H, T, D, -1) != SWATTN_OK) return 0;
  return delta_bytes(B, H, T);
}

size_t swattn_bwd_gqa_workspace_size(int B, int H, int Hkv, int T, int D) {
  if (check_common(B, H, T, D, -1) != SWATTN_OK || check_group(H, Hkv) != SWATTN_OK) return 0;
  if (Hkv == H) return delta_bytes(B, H, T);
  return delta_bytes(B, H, T) + 2 * (size_t)B * T * H * D * sizeof(float);
}

int swattn_bwd(const void *q, const void *k, const void *v, const void *o, const void *dO,
               const float *lse, void *dq, void *dk, void *dv, int B, int H, int T, int D,
               int window, float scale, void *workspace, swattn_stream_t stream) {
  return bwd_all(true, q, k, v, o, dO, lse, dq, dk, dv, B, H, H, T, D, window, scale, workspace,
                 (hipStream_t)stream);
}

int swattn_bwd_gqa(const void *q, const void *k, const void *v, const void *o, const void *dO,
                   const float *lse, void *dq, void *dk, void *dv, int B, int H, int Hkv, int T,
                   int D, int window, float scale, void *workspace, swattn_stream_t stream) {
  return bwd_all(true, q, k, v, o, dO, lse, dq, dk, dv, B, H, Hkv, T, D, window, scale,
                 workspace, (hipStream_t)stream);
}

int swattn_bwd_f32(const float *q, const float *k, const float *v, const float *o,
                   const float *dO, const float *lse, float *dq, float *dk, float *dv, int B,
                   int H, int T, int D, int window, float scale, void *workspace,
                   swattn_stream_t stream) {
  return bwd_all(false, q, k, v, o, dO, lse, dq, dk, dv, B, H, H, T, D, window, scale,
                 workspace, (hipStream_t)stream);
}

int swattn_bwd_preprocess(const void *o, const void *dO, void *workspace, int B, int H, int T,
                          int D, swattn_stream_t stream) {
  return bwd_pre(true, o, dO, workspace, B, H, T, D, (hipStream_t)stream);
}

int swattn_bwd_preprocess_f32(const float *o, const float *dO, void *workspace, int B, int H,
                              int T, int D, swattn_stream_t stream) {
  return bwd_pre(false, o, dO, workspace, B, H, T, D, (hipStream_t)stream);
}

int swattn_bwd_dkdv(const void *q, const void *k, const void *v, const void *dO, const float *lse,
                    const void *workspace, void *dk, void *dv, int B, int H, int T, int D,
                    int window, float scale, swattn_stream_t stream) {
  return bwd_dkdv(true, q, k, v, dO, lse, workspace, dk, dv, B, H, T, D, window, scale,
                  (hipStream_t)stream);
}

int swattn_bwd_dkdv_f32(const float *q, const float *k, const float *v, const float *dO,
                        const float *lse, const void *workspace, float *dk, float *dv, int B,
                        int H, int T, int D, int window, float scale, swattn_stream_t stream) {
  return bwd_dkdv(false, q, k, v, dO, lse, workspace, dk, dv, B, H, T, D, window, scale,
                  (hipStream_t)stream);
}

int swattn_bwd_dq(const void *q, const void *k, const void *v, const void *o, const void *dO,
                  const float *lse, void *workspace, void *dq, int B, int H, int T, int D,
                  int window, float scale, swattn_stream_t stream) {
  return bwd_dq(true, q, k, v, o, dO, lse, workspace, dq, B, H, T, D, window, scale,
                (hipStream_t)stream);
}

int swattn_bwd_dq_f32(const float *q, const float *k, const float *v, const float *o,
                      const float *dO, const float *lse, void *workspace, float *dq, int B, int H,
                      int T, int D, int window, float scale, swattn_stream_t stream) {
  return bwd_dq(false, q, k, v, o, dO, lse, workspace, dq, B, H, T, D, window, scale,
                (hipStream_t)stream);
}

int swattn_prefill(const void *q, const void *k_new, const void *v_new, void *k_cache,
                   void *v_cache, const int *seqlens, void *o, float *lse, int B, int H,
                   int Hkv, int Tq, int D, int Tmax, int window, float scale,
                   swattn_stream_t stream) {
  int st = check_common(B, H, Tq, D, window);
  if (st == SWATTN_OK) st = check_group(H, Hkv);
  if (st == SWATTN_OK) st = check_scale(scale);
  if (st != SWATTN_OK) return st;
  if (Tmax <= 0 || Tq > Tmax) return SWATTN_ERR_INVALID_ARG;
  // the caches: 32-bit grid/row indices and 32-bit buffer offsets per sequence
  if (!product_at_most(INT_MAX / 2, {B, Tmax, Hkv})) return SWATTN_ERR_INVALID_ARG;
  if (!product_at_most(INT_MAX, {(long long)Tmax + 128, Hkv, D, 2}))
    return SWATTN_ERR_UNSUPPORTED;
  if (!all_aligned({q, k_new, v_new, k_cache, v_cache, o}) || seqlens == nullptr)
    return SWATTN_ERR_INVALID_ARG;
  return hip_status(swattn::launch_prefill_bf16(q, k_new, v_new, k_cache, v_cache, seqlens, o,
                                                lse, B, H, Hkv, Tq, D, Tmax, window, scale,
                                                (hipStream_t)stream));
}

size_t swattn_decode_workspace_size(int B, int H, int D, int Tmax, int window) {
  if (check_decode(B, H, D, Tmax, window) != SWATTN_OK) return 0;
  const size_t ns = (size_t)swattn::decode_num_splits(Tmax, window);
  const size_t bytes = (size_t)B * H * ns * (D + 1) * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

static int decode_common(bool bf16, const void *q, const void *k_cache, const void *v_cache,
                         const int *seqlens, void *o, float *lse, int B, int H, int Hkv, int D,
                         int Tmax, int window, float scale, void *workspace,
                         swattn_stream_t stream) {
  int st = check_decode(B, H, D, Tmax, window);
  if (st == SWATTN_OK) st = check_group(H, Hkv);
  if (st == SWATTN_OK) st = check_scale(scale);
  if (st != SWATTN_OK) return st;
  if (!all_aligned({q, k_cache, v_cache, o, workspace}) || seqlens == nullptr)
    return SWATTN_ERR_INVALID_ARG;
  return hip_status(swattn::launch_decode(bf16, q, k_cache, v_cache, seqlens, o, lse, B, H, Hkv,
                                          D, Tmax, window, scale, (float *)workspace,
                                          (hipStream_t)stream));
}

int swattn_decode(const void *q, const void *k_cache, const void *v_cache, const int *seqlens,
                  void *o, float *lse, int B, int H, int D, int Tmax, int window, float scale,
                  void *workspace, swattn_stream_t stream) {
  return decode_common(true, q, k_cache, v_cache, seqlens, o, lse, B, H, H, D, Tmax, window,
                       scale, workspace, stream);
}

int swattn_decode_gqa(const void *q, const void *k_cache, const void *v_cache, const int *seqlens,
                      void *o, float *lse, int B, int H, int Hkv, int D, int Tmax, int window,
                      float scale, void *workspace, swattn_stream_t stream) {
  return decode_common(true, q, k_cache, v_cache, seqlens, o, lse, B, H, Hkv, D, Tmax, window,
                       scale, workspace, stream);
}

int swattn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                          const int *seqlens, void *o, float *lse, int B, int H, int D, int Tmax,
                          int window, float scale, swattn_stream_t stream) {
  // every argument check of swattn_decode first, then the scratch bound: nothing here
  // touches the GPU before the arguments are known to be valid
  int st = check_decode(B, H, D, Tmax, window);
  if (st == SWATTN_OK) st = check_scale(scale);
  if (st != SWATTN_OK) return st;
  if (!all_aligned({q, k_cache, v_cache, o}) || seqlens == nullptr) return SWATTN_ERR_INVALID_ARG;
  if (swattn_decode_workspace_size(B, H, D, Tmax, window) > swattn::kNoAllocScratchBytes)
    return SWATTN_ERR_TOO_LARGE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SWATTN_ERR_HIP;
  if (stream != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return SWATTN_ERR_HIP;
    if (sdev != dev) return SWATTN_ERR_INVALID_ARG;  // the stream's device must be current
  }
  void *ws = swattn::noalloc_scratch(dev);
  if (ws == nullptr) return SWATTN_ERR_HIP;
  return decode_common(true, q, k_cache, v_cache, seqlens, o, lse, B, H, H, D, Tmax, window,
                       scale, ws, stream);
}

int swattn_decode_f32(const float *q, const float *k_cache, const float *v_cache,
                      const int *seqlens, float *o, float *lse, int B, int H, int D, int Tmax,
                      int window, float scale, void *workspace, swattn_stream_t stream) {
  return decode_common(false, q, k_cache, v_cache, seqlens, o, lse, B, H, H, D, Tmax, window,
                       scale, workspace, stream);
}

static int check_prologue(int B, int T, int H, int Hkv, int D, float base, float eps) {
  // H == 0 (keys only) or Hkv == 0 (queries only) is allowed, not both
  if (B <= 0 || T <= 0 || H < 0 || Hkv < 0 || (H == 0 && Hkv == 0) || D <= 0)
    return SWATTN_ERR_INVALID_ARG;
  // the kernel counts the row's q and k vectors, H + Hkv, in an int
  if ((long long)H + Hkv > INT_MAX / 2) return SWATTN_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return SWATTN_ERR_UNSUPPORTED;
  if (!(base > 0.f) || !std::isfinite(base) || !(eps >= 0.f) || !std::isfinite(eps))
    return SWATTN_ERR_INVALID_ARG;
  if (!product_at_most(INT_MAX / 2, {B, T})) return SWATTN_ERR_INVALID_ARG;  // 32-bit row indices
  return SWATTN_OK;
}

int swattn_qk_norm_rope(const void *q, const void *k, void *q_out, void *k_out,
                        const int *pos_offset, int B, int T, int H, int Hkv, int D, float base,
                        float eps, swattn_stream_t stream) {
  const int st = check_prologue(B, T, H, Hkv, D, base, eps);
  if (st != SWATTN_OK) return st;
  if ((H > 0 && !all_aligned({q, q_out})) || (Hkv > 0 && !all_aligned({k, k_out})))
    return SWATTN_ERR_INVALID_ARG;
  return hip_status(swattn::launch_qk_norm_rope(q, k, q_out, k_out, pos_offset, B, T, H, Hkv, D,
                                                base, eps, (hipStream_t)stream));
}

int swattn_qk_norm_rope_bwd(const void *q, const void *k, const void *dq_out,
                            const void *dk_out, void *dq, void *dk, const int *pos_offset, int B,
                            int T, int H, int Hkv, int D, float base, float eps,
                            swattn_stream_t stream) {
  const int st = check_prologue(B, T, H, Hkv, D, base, eps);
  if (st != SWATTN_OK) return st;
  if ((H > 0 && !all_aligned({q, dq_out, dq})) || (Hkv > 0 && !all_aligned({k, dk_out, dk})))
    return SWATTN_ERR_INVALID_ARG;
  return hip_status(swattn::launch_qk_norm_rope_bwd(q, k, dq_out, dk_out, dq, dk, pos_offset, B,
                                                    T, H, Hkv, D, base, eps,
                                                    (hipStream_t)stream));
}

static int check_rope_args(float base, float eps) {
  if (!(base > 0.f) || !std::isfinite(base) || !(eps >= 0.f) || !std::isfinite(eps))
    return SWATTN_ERR_INVALID_ARG;
  return SWATTN_OK;
}

static swattn::RopeArgs rope_args(const int *pos_offset, int D, float base, float eps) {
  swattn::RopeArgs ra;
  ra.pos_off = pos_offset;
  ra.ratio = std::pow((double)base, -2.0 / D);
  ra.eps = eps;
  return ra;
}

int swattn_fwd_rope_gqa(const void *q, const void *k_rope, const void *v, void *o, float *lse,
                        void *q_rope, const int *pos_offset, int B, int H, int Hkv, int T, int D,
                        int window, float scale, float base, float eps, swattn_stream_t stream) {
  int st = check_common(B, H, T, D, window);
  if (st == SWATTN_OK) st = check_group(H, Hkv);
  if (st == SWATTN_OK) st = check_scale(scale);
  if (st == SWATTN_OK) st = check_rope_args(base, eps);
  if (st != SWATTN_OK) return st;
  if (!all_aligned({q, k_rope, v, o}) || lse == nullptr) return SWATTN_ERR_INVALID_ARG;
  if (q_rope != nullptr && !all_aligned({q_rope})) return SWATTN_ERR_INVALID_ARG;
  const swattn::RopeArgs ra = rope_args(pos_offset, D, base, eps);
  return hip_status(swattn::launch_fwd_bf16_rope(q, k_rope, v, o, lse, q_rope, B, H, Hkv, T, D,
                                                 window, scale, ra, (hipStream_t)stream));
}

int swattn_fwd_rope(const void *q, const void *k_rope, const void *v, void *o, float *lse,
                    void *q_rope, const int *pos_offset, int B, int H, int T, int D, int window,
                    float scale, float base, float eps, swattn_stream_t stream) {
  return swattn_fwd_rope_gqa(q, k_rope, v, o, lse, q_rope, pos_offset, B, H, H, T, D, window,
                             scale, base, eps, stream);
}

int swattn_bwd_rope_gqa(const void *q, const void *k, const void *q_rope, const void *k_rope,
                        const void *v, const void *o, const void *dO, const float *lse, void *dq,
                        void *dk, void *dv, const int *pos_offset, int B, int H, int Hkv, int T,
                        int D, int window, float scale, float base, float eps, void *workspace,
                        swattn_stream_t stream) {
  int s = check_common(B, H, T, D, window);
  if (s == SWATTN_OK) s = check_group(H, Hkv);
  if (s == SWATTN_OK) s = check_scale(scale);
  if (s == SWATTN_OK) s = check_rope_args(base, eps);
  if (s != SWATTN_OK) return s;
  if (!all_aligned({q, k, q_rope, k_rope, v, o, dO, dq, dk, dv, workspace}) || lse == nullptr)
    return SWATTN_ERR_INVALID_ARG;
  const swattn::RopeArgs ra = rope_args(pos_offset, D, base, eps);
  float *delta = (float *)workspace;
  float *part = (float *)((char *)workspace + delta_bytes(B, H, T));
  // dQ pass: raw q held (and transformed) in registers, transformed k streamed; dK/dV pass:
  // raw k held, transformed q streamed (with K/V head groups: per-query-head partials
  // after delta in the workspace, then the group sum)
  hipError_t e = swattn::launch_bwd_dq_bf16(q, k_rope, v, o, dO, lse, delta, dq, B, H, Hkv, T, D,
                                             window, scale, (hipStream_t)stream, &ra);
  if (e == hipSuccess)
    e = swattn::launch_bwd_dkdv_bf16(q_rope, k, v, dO, lse, delta, dk, dv, part, B, H, Hkv, T, D,
                                     window, scale, (hipStream_t)stream, &ra);
  return hip_status(e);
}

int swattn_bwd_rope(const void *q, const void *k, const void *q_rope, const void *k_rope,
                    const void *v, const void *o, const void *dO, const float *lse, void *dq,
                    void *dk, void *dv, const int *pos_offset, int B, int H, int T, int D,
                    int window, float scale, float base, float eps, void *workspace,
                    swattn_stream_t stream) {
  return swattn_bwd_rope_gqa(q, k, q_rope, k_rope, v, o, dO, lse, dq, dk, dv, pos_offset, B, H,
                             H, T, D, window, scale, base, eps, workspace, stream);
}

}  // extern "C"

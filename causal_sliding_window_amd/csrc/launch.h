// Internal launchers shared by the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "rope.h"

namespace swattn {

// Number of KV rows one decode workgroup handles: grouped kernels (four waves of 32
// rows), and the ungrouped split kernel (eight waves of 32 rows).
constexpr int kDecodeChunk = 128;
constexpr int kDecodeChunkWide = 256;
// Query heads whose partials a grouped decode workgroup merges together (its LDS holds
// four wave partials of each).
constexpr int kDecodeHeadBatch = 16;

int decode_num_splits(int Tmax, int window);

// Allocation-free decode (noalloc.hip): the size of the per-device scratch array, and
// its device address on `device`, which must be the current device (looked up on the
// first call for that device, then cached; nullptr on a HIP error).
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
void *noalloc_scratch(int device);

// Hkv: K/V heads (H, or a divisor of H: query head h reads K/V head h / (H / Hkv)).
// The fp32 kernels take no Hkv (they serve H == Hkv only).
hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse,
                           int B, int H, int Hkv, int T, int D, int window, float scale,
                           hipStream_t st);
// Forward with the QK-norm + rotary prologue fused into the query load (q raw, k already
// transformed); q_rope (nullable) receives the transformed queries.
hipError_t launch_fwd_bf16_rope(const void *q, const void *k, const void *v, void *o, float *lse,
                                void *q_rope, int B, int H, int Hkv, int T, int D, int window,
                                float scale, const RopeArgs &ra, hipStream_t st);
// Chunked prefill: appends the chunk's K/V rows to the caches at seqlens[b] (clamped to
// [0, Tmax - Tq]), then runs the forward for its Tq queries against the caches.
hipError_t launch_prefill_bf16(const void *q, const void *k_new, const void *v_new,
                               void *k_cache, void *v_cache, const int *seqlens, void *o,
                               float *lse, int B, int H, int Hkv, int Tq, int D, int Tmax,
                               int window, float scale, hipStream_t st);
hipError_t launch_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                          int B, int H, int T, int D, int window, float scale, hipStream_t st);

// Backward passes; `bf16` selects the bf16 MFMA kernels, else the fp32 ones.
hipError_t launch_bwd_pre(bool bf16, const void *o, const void *dO, float *delta, int B, int H,
                          int T, int D, hipStream_t st);
// With Hkv < H, `part` holds 2 * B*T*H*D floats: per-query-head partials of dK, dV.
hipError_t launch_bwd_dkdv(bool bf16, const void *q, const void *k, const void *v,
                           const void *dO, const float *lse, const float *delta, void *dk,
                           void *dv, float *part, int B, int H, int Hkv, int T, int D,
                           int window, float scale, hipStream_t st);
// dQ pass; also computes delta = rowsum(dO * o) and writes it to `delta`.
hipError_t launch_bwd_dq(bool bf16, const void *q, const void *k, const void *v, const void *o,
                         const void *dO, const float *lse, float *delta, void *dq, int B, int H,
                         int Hkv, int T, int D, int window, float scale, hipStream_t st);

hipError_t launch_bwd_pre_bf16(const void *o, const void *dO, float *delta, int B, int H, int T,
                               int D, hipStream_t st);
// rope (non-null): k raw, q transformed; dk with respect to the raw k (with K/V head
// groups each query head's share is mapped back before the group sum)
hipError_t launch_bwd_dkdv_bf16(const void *q, const void *k, const void *v, const void *dO,
                                const float *lse, const float *delta, void *dk, void *dv,
                                float *part, int B, int H, int Hkv, int T, int D, int window,
                                float scale, hipStream_t st, const RopeArgs *rope = nullptr);
// rope (non-null): q raw, k transformed; dq with respect to the raw q (QK-norm + rotary
// prologue fused into the query load and the epilogue)
hipError_t launch_bwd_dq_bf16(const void *q, const void *k, const void *v, const void *o,
                              const void *dO, const float *lse, float *delta, void *dq, int B,
                              int H, int Hkv, int T, int D, int window, float scale,
                              hipStream_t st, const RopeArgs *rope = nullptr);
hipError_t launch_bwd_pre_f32(const float *o, const float *dO, float *delta, int B, int H, int T,
                              int D, hipStream_t st);
hipError_t launch_bwd_dkdv_f32(const float *q, const float *k, const float *v, const float *dO,
                               const float *lse, const float *delta, float *dk, float *dv, int B,
                               int H, int T, int D, int window, float scale, hipStream_t st);
hipError_t launch_bwd_dq_f32(const float *q, const float *k, const float *v, const float *dO,
                             const float *lse, const float *delta, float *dq, int B, int H, int T,
                             int D, int window, float scale, hipStream_t st);

hipError_t launch_decode(bool bf16, const void *q, const void *k_cache, const void *v_cache,
                         const int *seqlens, void *o, float *lse, int B, int H, int Hkv, int D,
                         int Tmax, int window, float scale, float *ws, hipStream_t st);

// QK-norm + rotary prologue (prologue.hip): q, k -> q_out, k_out; and its backward
// (dq_out, dk_out, with the raw q, k -> dq, dk).  pos_off: device int32[B] or null.
hipError_t launch_qk_norm_rope(const void *q, const void *k, void *q_out, void *k_out,
                               const int *pos_off, int B, int T, int H, int Hkv, int D,
                               float base, float eps, hipStream_t st);
hipError_t launch_qk_norm_rope_bwd(const void *q, const void *k, const void *dq_out,
                                   const void *dk_out, void *dq, void *dk, const int *pos_off,
                                   int B, int T, int H, int Hkv, int D, float base, float eps,
                                   hipStream_t st);

}  // namespace swattn

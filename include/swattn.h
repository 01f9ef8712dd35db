/*
 * libswattn — causal multi-head attention with an optional sliding window,
 * forward, backward and one-token KV-cache decode, for AMD Instinct MI355X (gfx950).
 *
 * What is computed (the nanochat pages):
 *   - nanochat guide ("Train your own ChatGPT", apidog), section 5 "Flash Attention
 *     unification": every attention layer makes one call with q, k, v, causal
 *     masking switched on and a window_size argument; off Hopper the same call is
 *     PyTorch's scaled-dot-product attention, i.e. plain masked softmax(scale*QK^T)V.
 *   - same guide, section 1 "GPT model", feature list: sliding-window attention
 *     whose window alternates between short and long across layers ("SSSL").
 *   - time-to-GPT-2 post (Jan-29 leaderboard), list of the biggest wins: the FA3
 *     kernels are faster and take the window_size argument.
 *   - same guide, section 6 "Inference engine": the engine keeps a KV cache that
 *     the kernels read (with-KV-cache entry) while decoding one token at a time.
 *   - same guide, section 1 feature list: grouped-query attention, fewer K/V heads
 *     than query heads (the *_gqa entry points; the one-K/V-head case is the
 *     multi-query attention of the release article's architecture list).
 *
 * Definitions used by every entry point (positions are 0-based):
 *   visible(i, j)  <=>  j <= i  and  (window < 0  or  i - j < window)
 *   s_ij = scale * q_i . k_j;  LSE_i = ln sum_{visible j} exp(s_ij)   (natural log)
 *   p_ij = exp(s_ij - LSE_i) on visible entries;  o_i = sum_j p_ij v_j
 *   window = W >= 1: a query sees its W most recent keys, itself included
 *   (FlashAttention's window_size = (W-1, 0)); window < 0: full causal;
 *   window == 0 is an error; W >= T equals full causal.
 *
 * Layout and types.
 *   - q, k, v, o, dO, dq, dk, dv: device memory, contiguous [B, T, H, D] (D fastest).
 *     Plain names take bf16 (raw 16-bit storage); the _f32 names take float32.
 *   - lse: device float32 [B, H, T].  Decode q/o: [B, H, D]; decode lse: [B, H].
 *   - k_cache, v_cache: device, contiguous [B, Tmax, H, D].
 *   - *_gqa entry points: k, v, dk, dv are [B, T, Hkv, D] and k_cache, v_cache
 *     [B, Tmax, Hkv, D], with Hkv >= 1 dividing H.  Query head h reads K/V head
 *     h / (H / Hkv) (contiguous groups; the pages do not say which heads share,
 *     this is the plain reading), and dk, dv of a K/V head sum over its group.
 *   - seqlens: device int32 [B].
 *   - D must be 64 or 128.  All arithmetic accumulates in float32; bf16 outputs
 *     are rounded to nearest even.
 *
 * Ownership and execution.
 *   - The caller allocates every buffer (including workspaces) and keeps it alive
 *     until the work on `stream` has finished.  The library allocates and frees
 *     nothing, keeps no global state and is safe to call from several threads.
 *   - Calls only enqueue kernels on `stream` (NULL = the default stream) and never
 *     synchronise the host.  Pass a hipStream_t; it is declared here as an opaque
 *     pointer so that this header needs no HIP include.
 *   - Outputs must not alias inputs.
 *
 * Errors: every entry point returns a swattn_status; nothing is thrown.
 *   SWATTN_ERR_INVALID_ARG  NULL required pointer, B/H/T/D/Tmax <= 0, window == 0,
 *                           scale not a positive finite number (every call that
 *                           takes a scale: the masked softmax of scale * QK^T is
 *                           computed with the mask applied before the scale, which
 *                           equals masking after it only for scale > 0),
 *                           Hkv <= 0 or not dividing H (*_gqa),
 *                           a size product that does not fit the kernels' 32-bit
 *                           grid/row indices, or a workspace pointer of NULL
 *   SWATTN_ERR_UNSUPPORTED  D not in {64, 128}, or (for the training calls) one
 *                           sequence's [T + 128, H, D] block of 2-byte elements
 *                           exceeding 2^31 - 1 bytes (32-bit buffer offsets)
 *   SWATTN_ERR_HIP          the HIP runtime reported an error at launch
 * On an error nothing has been enqueued (argument errors) or the state of the
 * outputs is unspecified (HIP errors).
 */
#ifndef SWATTN_H
#define SWATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *swattn_stream_t; /* == hipStream_t */

typedef enum {
  SWATTN_OK = 0,
  SWATTN_ERR_INVALID_ARG = 1,
  SWATTN_ERR_UNSUPPORTED = 2,
  SWATTN_ERR_HIP = 3,
  SWATTN_ERR_TOO_LARGE = 4 /* swattn_decode_noalloc: the sizes need more scratch than it has */
} swattn_status;

/* Human-readable name of a status code (static storage; never NULL). */
const char *swattn_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
int swattn_version(void);

/*
 * Forward: o = softmax(scale*QK^T, masked)V and lse (guide section 5; window from
 * section 1).  Inputs q, k, v; outputs o (same dtype as q) and lse (float32,
 * [B,H,T]).  Row i of o only depends on rows j <= i of k and v.
 */
int swattn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
               int B, int H, int T, int D, int window, float scale,
               swattn_stream_t stream);
int swattn_fwd_f32(const float *q, const float *k, const float *v, float *o,
                   float *lse, int B, int H, int T, int D, int window,
                   float scale, swattn_stream_t stream);
/* Grouped-query forward (bf16): k, v [B,T,Hkv,D]; otherwise as swattn_fwd, which it
 * equals for Hkv == H. */
int swattn_fwd_gqa(const void *q, const void *k, const void *v, void *o, float *lse,
                   int B, int H, int Hkv, int T, int D, int window, float scale,
                   swattn_stream_t stream);

/*
 * Backward workspace in bytes: delta_i = dO_i . o_i, float32 [B,H,T], rounded up
 * to 256 bytes.  Returns 0 for invalid sizes.
 */
size_t swattn_bwd_workspace_size(int B, int H, int T, int D);

/*
 * Backward: gradients of L = sum_i dO_i . o_i with respect to q, k, v, given the
 * forward's o and lse (the analytic gradient of the guide's section-5 attention;
 * training back-propagates through it).  P is recomputed from lse; dK/dV and dQ
 * are produced by separate passes with no atomics, so results are bitwise
 * reproducible.  dq, dk, dv have q's dtype.  `workspace` must hold
 * swattn_bwd_workspace_size() bytes; its contents on entry do not matter.
 */
int swattn_bwd(const void *q, const void *k, const void *v, const void *o,
               const void *dO, const float *lse, void *dq, void *dk, void *dv,
               int B, int H, int T, int D, int window, float scale,
               void *workspace, swattn_stream_t stream);
int swattn_bwd_f32(const float *q, const float *k, const float *v,
                   const float *o, const float *dO, const float *lse, float *dq,
                   float *dk, float *dv, int B, int H, int T, int D, int window,
                   float scale, void *workspace, swattn_stream_t stream);
/* Grouped-query backward workspace in bytes: delta (as swattn_bwd_workspace_size)
 * and, when Hkv < H, float32 partials of dk and dv per query head, 2*B*T*H*D*4
 * bytes.  Returns 0 for invalid sizes. */
size_t swattn_bwd_gqa_workspace_size(int B, int H, int Hkv, int T, int D);
/* Grouped-query backward (bf16): k, v, dk, dv [B,T,Hkv,D]; dk and dv of a K/V head
 * sum the gradients of its H / Hkv query heads.  The dK/dV pass writes each query
 * head's float32 contribution to the workspace and a second kernel adds the heads
 * of each group in head order: no atomics, bitwise reproducible.  `workspace` must
 * hold swattn_bwd_gqa_workspace_size() bytes; equals swattn_bwd for Hkv == H. */
int swattn_bwd_gqa(const void *q, const void *k, const void *v, const void *o,
                   const void *dO, const float *lse, void *dq, void *dk, void *dv,
                   int B, int H, int Hkv, int T, int D, int window, float scale,
                   void *workspace, swattn_stream_t stream);

/*
 * The passes of swattn_bwd, callable on their own (to time them, or to overlap
 * them with other work).  swattn_bwd is exactly swattn_bwd_dq followed by
 * swattn_bwd_dkdv on the same workspace:
 *   swattn_bwd_dq          dQ; it also computes delta = rowsum(dO * o) (fp32, per
 *                          query) and writes it to the workspace;
 *   swattn_bwd_dkdv        dK, dV; reads delta from the workspace, so it must run
 *                          after swattn_bwd_dq or swattn_bwd_preprocess;
 *   swattn_bwd_preprocess  delta alone (for running dK/dV before or beside dQ).
 */
int swattn_bwd_preprocess(const void *o, const void *dO, void *workspace, int B, int H,
                          int T, int D, swattn_stream_t stream);
int swattn_bwd_preprocess_f32(const float *o, const float *dO, void *workspace, int B,
                              int H, int T, int D, swattn_stream_t stream);
int swattn_bwd_dkdv(const void *q, const void *k, const void *v, const void *dO,
                    const float *lse, const void *workspace, void *dk, void *dv, int B,
                    int H, int T, int D, int window, float scale,
                    swattn_stream_t stream);
int swattn_bwd_dkdv_f32(const float *q, const float *k, const float *v,
                        const float *dO, const float *lse, const void *workspace,
                        float *dk, float *dv, int B, int H, int T, int D, int window,
                        float scale, swattn_stream_t stream);
int swattn_bwd_dq(const void *q, const void *k, const void *v, const void *o,
                  const void *dO, const float *lse, void *workspace, void *dq, int B, int H,
                  int T, int D, int window, float scale, swattn_stream_t stream);
int swattn_bwd_dq_f32(const float *q, const float *k, const float *v, const float *o,
                      const float *dO, const float *lse, void *workspace, float *dq, int B,
                      int H, int T, int D, int window, float scale, swattn_stream_t stream);

/*
 * Chunked prefill with cache append (bf16; guide section 6: the engine fills the KV
 * cache through the kernels' with-KV-cache entry).  q, o [B,Tq,H,D]; k_new, v_new
 * [B,Tq,Hkv,D]; k_cache, v_cache [B,Tmax,Hkv,D]; seqlens device int32 [B], the rows
 * already cached.  For sequence b, with L0 = seqlens[b] clamped to [0, Tmax - Tq],
 * rows L0 .. L0+Tq-1 of the caches are overwritten with k_new[b], v_new[b], then query
 * i attends as position L0 + i to cache rows j <= L0 + i inside the window (o and,
 * unless NULL, lse [B,H,Tq]).  seqlens is not updated (the caller adds Tq).  Hkv = H
 * without grouping.  INVALID_ARG also for Tmax <= 0 or Tq > Tmax.  No workspace.
 */
int swattn_prefill(const void *q, const void *k_new, const void *v_new, void *k_cache,
                   void *v_cache, const int *seqlens, void *o, float *lse, int B, int H,
                   int Hkv, int Tq, int D, int Tmax, int window, float scale,
                   swattn_stream_t stream);

/*
 * Decode workspace in bytes: per (sequence, head, KV split) one float32 partial
 * output [D] and one partial LSE.  Depends on Tmax and window because they bound
 * the number of splits.  Returns 0 for invalid sizes.  No initialisation needed;
 * calls that may run concurrently need separate workspaces.
 */
size_t swattn_decode_workspace_size(int B, int H, int D, int Tmax, int window);

/*
 * One-token decode against a KV cache (guide section 6).  Sequence b has
 * L = seqlens[b] valid cache rows, the new token's own K/V already written at row
 * L-1; its query sits at position L-1 and sees rows max(0, L-W) .. L-1 (all rows
 * 0 .. L-1 when window < 0).  Rows >= L are never read.  seqlens is read on the
 * device; values above Tmax are clamped to Tmax, and L <= 0 yields o = 0 and
 * lse = -inf.  lse may be NULL.  The visible range is split across workgroups
 * and the partial results are merged by their LSE in a fixed order (bitwise
 * reproducible).
 */
int swattn_decode(const void *q, const void *k_cache, const void *v_cache,
                  const int *seqlens, void *o, float *lse, int B, int H, int D,
                  int Tmax, int window, float scale, void *workspace,
                  swattn_stream_t stream);
int swattn_decode_f32(const float *q, const float *k_cache,
                      const float *v_cache, const int *seqlens, float *o,
                      float *lse, int B, int H, int D, int Tmax, int window,
                      float scale, void *workspace, swattn_stream_t stream);
/*
 * Allocation-free decode, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): exactly
 * swattn_decode (same kernels, same results, bitwise), with its partials kept in a
 * scratch array that the library holds in device memory instead of a workspace.
 * The array holds SWATTN_NOALLOC_SCRATCH_BYTES (16 MiB) on every GPU the library runs
 * on, from that GPU's first call until the process ends.  The call allocates nothing
 * and frees nothing; the first call on a device looks up the array's address there
 * (that device must be current; a non-NULL stream must belong to it).
 * Sizes whose swattn_decode_workspace_size() exceeds the array return
 * SWATTN_ERR_TOO_LARGE before anything is enqueued (e.g. B*H = 384 heads fit up to
 * Tmax = 8192 or any window <= 8192 at D = 128).  Every call on one GPU shares that
 * GPU's array: calls that may run at the same time on one GPU (other streams, other
 * threads) race on it and must be serialised by the caller.  Nothing in the array
 * needs to start at zero.  Other errors as swattn_decode.
 */
#define SWATTN_NOALLOC_SCRATCH_BYTES (16u << 20)
int swattn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                          const int *seqlens, void *o, float *lse, int B, int H, int D,
                          int Tmax, int window, float scale, swattn_stream_t stream);

/* Grouped-query decode (bf16): k_cache, v_cache [B,Tmax,Hkv,D]; each cache row is
 * read once for the H / Hkv query heads of its group.  The workspace is
 * swattn_decode_workspace_size(B, H, D, Tmax, window) bytes (partials per query
 * head); otherwise as swattn_decode.  With D = 128 and groups of 2 or more query
 * heads the scores and P V run on the matrix cores, with P rounded to bf16 before
 * P V as in the forward: results then differ from the ungrouped call on repeated
 * caches by rounding only (still deterministic). */
int swattn_decode_gqa(const void *q, const void *k_cache, const void *v_cache,
                      const int *seqlens, void *o, float *lse, int B, int H, int Hkv,
                      int D, int Tmax, int window, float scale, void *workspace,
                      swattn_stream_t stream);

/*
 * QK-norm + rotary prologue (bf16; nanochat release article, architecture list:
 * rotary embeddings as the only position encoding, QK norm, RMSNorm without
 * learnable parameters; guide section 1 "GPT model", feature list).  For every
 * head vector x [D] of q [B,T,H,D] and k [B,T,Hkv,D], token t of sequence b at
 * position p = max(pos_offset[b], 0) + t (p = t when pos_offset is NULL; device
 * int32 [B] otherwise):
 *   x_n = x / sqrt(mean(x^2) + eps), no weight;
 *   pair i = (x_n[i], x_n[i + D/2]), i < D/2, rotated by the angle p * base^(-2i/D):
 *   y[i] = a cos - b sin, y[i + D/2] = a sin + b cos   (a, b the pair).
 * Writes y into q_out [B,T,H,D] and k_out [B,T,Hkv,D] (bf16, rounded to nearest
 * even from fp32; angles in fp64).  Hkv is independent of H here.  One side may be
 * absent: H = 0 transforms k alone (q, q_out may be NULL), Hkv = 0 q alone (k, k_out
 * may be NULL); not both.  Outputs may be their own inputs (in place); other
 * overlaps are not allowed.
 * INVALID_ARG: a NULL or misaligned tensor of a present side, B, T <= 0, H or Hkv < 0,
 * H + Hkv == 0 or > INT_MAX / 2, base <= 0, eps < 0 or either not finite,
 * B * T > INT_MAX / 2.
 * UNSUPPORTED: D not 64 or 128.  Asynchronous on `stream`; no workspace.
 */
int swattn_qk_norm_rope(const void *q, const void *k, void *q_out, void *k_out,
                        const int *pos_offset, int B, int T, int H, int Hkv, int D, float base,
                        float eps, swattn_stream_t stream);

/*
 * Backward of swattn_qk_norm_rope: given the raw inputs q, k and the gradients of
 * its outputs dq_out [B,T,H,D], dk_out [B,T,Hkv,D], writes dq, dk (same shapes,
 * bf16): with g = dy rotated back by -angle and r = 1 / sqrt(mean(x^2) + eps),
 * dx = r g - r^3 x (x . g) / D.  Same positions, arguments and errors as the
 * forward; dq may be dq_out and dk may be dk_out (in place).
 */
int swattn_qk_norm_rope_bwd(const void *q, const void *k, const void *dq_out,
                            const void *dk_out, void *dq, void *dk, const int *pos_offset, int B,
                            int T, int H, int Hkv, int D, float base, float eps,
                            swattn_stream_t stream);

/*
 * Attention with the QK-norm + rotary prologue fused into the passes that hold q or k
 * in registers (bf16; k, v [B,T,H,D], or [B,T,Hkv,D] in the _gqa forms).  Same definitions as
 * swattn_qk_norm_rope (positions, base, eps, pos_offset) and swattn_fwd / swattn_bwd;
 * a training step through the prologue and attention becomes
 *   swattn_qk_norm_rope(NULL, k, NULL, k_rope, pos_offset, B, T, 0, H, ...)  (keys only)
 *   swattn_fwd_rope(q, k_rope, v, o, lse, q_rope, ...)
 *   swattn_bwd_rope(q, k, q_rope, k_rope, v, o, dO, lse, dq, dk, dv, ...)
 * where q and k are the raw projections and dq, dk the gradients with respect to them,
 * instead of the two-sided prologue, swattn_fwd, swattn_bwd and swattn_qk_norm_rope_bwd.
 * Each query (in the forward and the dQ pass) and each key (in the dK/dV pass) is
 * normalised and rotated as it is loaded into registers; the dQ and dK/dV passes map
 * their gradients back through the prologue in their epilogues (from fp32, with the
 * raw rows read again), so q' and k' gradients are never stored.  The streamed sides
 * (k_rope in the forward and the dQ pass, q_rope in the dK/dV pass) are the
 * transformed tensors.  Sines and cosines are taken on fp64-reduced angles by the
 * hardware's sine and cosine: q' and k' may differ from swattn_qk_norm_rope's in the
 * last bit of the bf16 rounding.
 *
 * swattn_fwd_rope: q raw [B,T,H,D]; k_rope = the prologue applied to k; o, lse as
 *   swattn_fwd.  q_rope (nullable) receives the transformed queries (bf16), which
 *   swattn_bwd_rope streams.
 * swattn_bwd_rope: q, k raw; q_rope, k_rope transformed; o, lse from swattn_fwd_rope;
 *   dq, dk with respect to the raw q and k, dv as swattn_bwd.  Workspace as
 *   swattn_bwd_workspace_size().
 * swattn_fwd_rope_gqa / swattn_bwd_rope_gqa: the same with Hkv K/V heads shared by
 *   groups of H / Hkv consecutive query heads (as swattn_fwd_gqa / swattn_bwd_gqa):
 *   k, k_rope, v, dk, dv are [B,T,Hkv,D].  The prologue is applied per head, so the
 *   keys-only prologue call takes Hkv heads.  In the dK/dV pass each query head's share
 *   of dk' is mapped back through the prologue (the mapping is linear in dk') into an
 *   fp32 partial before the group sum.  Workspace as swattn_bwd_gqa_workspace_size().
 *   With Hkv == H they equal swattn_fwd_rope / swattn_bwd_rope.
 * Errors: those of swattn_fwd / swattn_bwd (and of swattn_fwd_gqa / swattn_bwd_gqa for
 * the _gqa forms), and INVALID_ARG for base <= 0, eps < 0 or either not finite.
 */
int swattn_fwd_rope(const void *q, const void *k_rope, const void *v, void *o, float *lse,
                    void *q_rope, const int *pos_offset, int B, int H, int T, int D, int window,
                    float scale, float base, float eps, swattn_stream_t stream);
int swattn_bwd_rope(const void *q, const void *k, const void *q_rope, const void *k_rope,
                    const void *v, const void *o, const void *dO, const float *lse, void *dq,
                    void *dk, void *dv, const int *pos_offset, int B, int H, int T, int D,
                    int window, float scale, float base, float eps, void *workspace,
                    swattn_stream_t stream);
int swattn_fwd_rope_gqa(const void *q, const void *k_rope, const void *v, void *o, float *lse,
                        void *q_rope, const int *pos_offset, int B, int H, int Hkv, int T, int D,
                        int window, float scale, float base, float eps, swattn_stream_t stream);
int swattn_bwd_rope_gqa(const void *q, const void *k, const void *q_rope, const void *k_rope,
                        const void *v, const void *o, const void *dO, const float *lse, void *dq,
                        void *dk, void *dv, const int *pos_offset, int B, int H, int Hkv, int T,
                        int D, int window, float scale, float base, float eps, void *workspace,
                        swattn_stream_t stream);

/*
 * Measurement probes: what this GPU sustains, next to its published peaks (not part of
 * the attention method; used to report the kernels against measured ceilings).
 *
 * swattn_probe_mfma: `workgroups` workgroups of 256 threads (4 waves each); every wave
 *   issues iters x 4 bf16 matrix products of 32 x 32 x 16 (2 * 32 * 32 * 16 flops
 *   each), the instruction the attention passes use, back to back on four independent
 *   accumulator chains, with no memory traffic.  Total flops:
 *   workgroups * 4 * iters * 4 * 32768.  out: device float32 [workgroups * 256]; every
 *   element becomes iters / 64 (all operands 1/256: exact), which checks the products.
 *   INVALID_ARG for a NULL or misaligned out, workgroups outside [1, 2^20], iters
 *   outside [1, 2^24].
 * swattn_probe_read: reads nbytes of device memory at src once, 16 bytes per lane and
 *   load, non-temporal (as the decode kernels read the cache), eight loads in flight
 *   per lane, in a grid of `workgroups` workgroups of 256 threads, each streaming its
 *   own contiguous span (the buffer cut into `workgroups` equal spans, the last one
 *   shorter); out: device uint32 [workgroups * 256], each the XOR of the 32-bit words
 *   its thread read (the XOR of all of out is the XOR of the buffer).  INVALID_ARG for
 *   NULL pointers, src not 16-byte aligned, nbytes 0 or not a multiple of 16,
 *   workgroups outside [1, 2^20].
 * Both only enqueue work on `stream`; time them with events on that stream.
 */
int swattn_probe_mfma(float *out, int workgroups, int iters, swattn_stream_t stream);
int swattn_probe_read(const void *src, size_t nbytes, unsigned int *out, int workgroups,
                      swattn_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SWATTN_H */

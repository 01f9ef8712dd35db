// One-token KV-cache decode (nanochat guide, section 6 "Inference engine": the
// engine decodes one token per step against the cache its attention kernels
// read).  Bound by HBM: every visible K/V cache row is read exactly once.
//
// decode_split_kernel: workgroup (chunk c, head h, sequence b) reads seqlens[b] on
//   the device, takes its kDecodeChunk rows of the visible range
//   [max(0, L - W), L), and writes a partial (o_c normalised, lse_c) to the
//   workspace.  Each K/V row of one head is 256 contiguous bytes (bf16, D = 128)
//   read by D/8 lanes with 16-byte loads; all rows of a chunk are requested before
//   any is used.
// decode_merge_kernel: one workgroup per (b, h) combines the partials,
//   lse = ln sum_c exp(lse_c), o = sum_c exp(lse_c - lse) o_c.
#include "common.h"
#include "launch.h"

namespace swattn {

int decode_num_splits(int Tmax, int window) {
  const int vis = window > 0 ? (window < Tmax ? window : Tmax) : Tmax;
  return (vis + kDecodeChunk - 1) / kDecodeChunk;
}

template <typename TT> struct Elem;
template <> struct Elem<uint16_t> {
  static constexpr int PER16 = 8;
  __device__ static void unpack(const u32x4 &x, float *f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = bf16_lo(x[e]);
      f[2 * e + 1] = bf16_hi(x[e]);
    }
  }
  __device__ static uint16_t pack(float x) { return f32_to_bf16_bits(x); }
};
template <> struct Elem<float> {
  static constexpr int PER16 = 4;
  __device__ static void unpack(const u32x4 &x, float *f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(x[e]);
  }
  __device__ static float pack(float x) { return x; }
};

__device__ __forceinline__ int visible_lo(int L, int window) {
  return window > 0 ? max(0, L - window) : 0;
}

template <typename TT, int D>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const TT *__restrict__ q, const TT *__restrict__ kc, const TT *__restrict__ vc,
    const int *__restrict__ seqlens, float *__restrict__ ws_o, float *__restrict__ ws_lse,
    int H, int Tmax, int window, float scale, int nsplit) {
  constexpr int EPL = Elem<TT>::PER16;  // elements per 16-byte load
  constexpr int LPR = D / EPL;          // lanes per row
  constexpr int RPP = 256 / LPR;        // rows per pass
  constexpr int CH = kDecodeChunk;
  constexpr int PASSES = CH / RPP;
  constexpr int BATCH = PASSES < 8 ? PASSES : 8;  // rows in flight per thread
  __shared__ float sc[CH];
  __shared__ float part[RPP][D + 1];
  __shared__ float red[8];

  const int c = blockIdx.x, hh = blockIdx.y, b = blockIdx.z;
  const int L = min(seqlens[b], Tmax);
  if (L <= 0) return;
  const int lo = visible_lo(L, window);
  const int n = L - lo;
  if (c * CH >= n) return;
  const int t0 = lo + c * CH;
  const int cnt = min(CH, L - t0);

  const int tid = threadIdx.x, r = tid / LPR, sl = tid % LPR;
  float qf[EPL];
  Elem<TT>::unpack(ldg16(q + ((size_t)b * H + hh) * D + sl * EPL), qf);
  const size_t rs = (size_t)H * D;
  const TT *kb = kc + ((size_t)b * Tmax * H + hh) * D + sl * EPL;
  const TT *vb = vc + ((size_t)b * Tmax * H + hh) * D + sl * EPL;

  // scores
  for (int p0 = 0; p0 < PASSES; p0 += BATCH) {
    u32x4 kr[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int t = (p0 + j) * RPP + r;
      kr[j] = t < cnt ? ldg16(kb + (size_t)(t0 + t) * rs) : u32x4{};
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      float kf[EPL];
      Elem<TT>::unpack(kr[j], kf);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) dot = fmaf(qf[e], kf[e], dot);
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off, LPR);
      const int t = (p0 + j) * RPP + r;
      if (sl == 0 && t < cnt) sc[t] = dot * scale;
    }
  }
  __syncthreads();

  // chunk max and sum (CH == blockDim.x)
  const float x = tid < cnt ? sc[tid] : -INFINITY;
  float m = x;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float pw = tid < cnt ? expf(x - m) : 0.f;
  float s = pw;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  __syncthreads();  // everyone has read red[0..3]
  if ((tid & 63) == 0) red[4 + (tid >> 6)] = s;
  sc[tid] = pw;
  __syncthreads();
  const float lsum = (red[4] + red[5]) + (red[6] + red[7]);

  // o = sum_t p_t v_t
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  for (int p0 = 0; p0 < PASSES; p0 += BATCH) {
    u32x4 vr[BATCH];
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int t = (p0 + j) * RPP + r;
      vr[j] = t < cnt ? ldg16(vb + (size_t)(t0 + t) * rs) : u32x4{};
    }
#pragma unroll
    for (int j = 0; j < BATCH; ++j) {
      const int t = (p0 + j) * RPP + r;
      const float pj = t < cnt ? sc[t] : 0.f;
      float vf[EPL];
      Elem<TT>::unpack(vr[j], vf);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pj, vf[e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) part[r][sl * EPL + e] = acc[e];
  __syncthreads();
  const size_t slot = ((size_t)b * H + hh) * nsplit + c;
  if (tid < D) {
    float o = 0.f;
#pragma unroll
    for (int rr = 0; rr < RPP; ++rr) o += part[rr][tid];
    ws_o[slot * D + tid] = o / lsum;
  }
  if (tid == 0) ws_lse[slot] = m + logf(lsum);
}

template <typename TT, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(
    const float *__restrict__ ws_o, const float *__restrict__ ws_lse,
    const int *__restrict__ seqlens, TT *__restrict__ o, float *__restrict__ lse, int H,
    int Tmax, int window, int nsplit) {
  const int bh = blockIdx.x, b = bh / H;
  const int tid = threadIdx.x;
  const int L = min(seqlens[b], Tmax);
  if (L <= 0) {
    o[(size_t)bh * D + tid] = Elem<TT>::pack(0.f);
    if (lse && tid == 0) lse[bh] = -INFINITY;
    return;
  }
  const int n = L - visible_lo(L, window);
  const int nch = (n + kDecodeChunk - 1) / kDecodeChunk;
  const float *ls = ws_lse + (size_t)bh * nsplit;
  float m = -INFINITY;
  for (int c = 0; c < nch; ++c) m = fmaxf(m, ls[c]);
  float tot = 0.f;
  for (int c = 0; c < nch; ++c) tot += expf(ls[c] - m);
  const float lt = m + logf(tot);
  float acc = 0.f;
  for (int c = 0; c < nch; ++c) acc += expf(ls[c] - lt) * ws_o[((size_t)bh * nsplit + c) * D + tid];
  o[(size_t)bh * D + tid] = Elem<TT>::pack(acc);
  if (lse && tid == 0) lse[bh] = lt;
}

template <typename TT, int D>
static hipError_t launch_decode_t(const void *q, const void *k_cache, const void *v_cache,
                                  const int *seqlens, void *o, float *lse, int B, int H,
                                  int Tmax, int window, float scale, float *ws, hipStream_t st) {
  const int ns = decode_num_splits(Tmax, window);
  float *ws_o = ws;
  float *ws_lse = ws + (size_t)B * H * ns * D;
  decode_split_kernel<TT, D><<<dim3(ns, H, B), 256, 0, st>>>(
      (const TT *)q, (const TT *)k_cache, (const TT *)v_cache, seqlens, ws_o, ws_lse, H, Tmax,
      window, scale, ns);
  decode_merge_kernel<TT, D><<<B * H, D, 0, st>>>(ws_o, ws_lse, seqlens, (TT *)o, lse, H, Tmax,
                                                  window, ns);
  return hipGetLastError();
}

hipError_t launch_decode(bool bf16, const void *q, const void *k_cache, const void *v_cache,
                         const int *seqlens, void *o, float *lse, int B, int H, int D, int Tmax,
                         int window, float scale, float *ws, hipStream_t st) {
  if (bf16) {
    if (D == 128)
      return launch_decode_t<uint16_t, 128>(q, k_cache, v_cache, seqlens, o, lse, B, H, Tmax,
                                            window, scale, ws, st);
    return launch_decode_t<uint16_t, 64>(q, k_cache, v_cache, seqlens, o, lse, B, H, Tmax,
                                         window, scale, ws, st);
  }
  if (D == 128)
    return launch_decode_t<float, 128>(q, k_cache, v_cache, seqlens, o, lse, B, H, Tmax, window,
                                       scale, ws, st);
  return launch_decode_t<float, 64>(q, k_cache, v_cache, seqlens, o, lse, B, H, Tmax, window,
                                    scale, ws, st);
}

}  // namespace swattn

// float32 forward and backward of causal sliding-window attention.
//
// Same mathematics as the bf16 MFMA path (nanochat guide section 5 attention with
// the section 1 sliding window), computed on the vector ALUs in fp32 with
// libm-accurate exp/log so that results stay within 1e-5 of the fp64 definition.
// Layout: D/32 lanes own one query (forward, dQ) or one key (dK/dV) row, each
// lane holding 32 of its D elements; the other operand's rows stream through LDS
// in tiles of 32 rows; dot products are finished with lane shuffles.
#include "common.h"
#include "launch.h"

namespace swattn {

constexpr int kF32Tile = 32;

template <int D>
__device__ __forceinline__ float row_dot(const float *a, const float *lds_row) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) s = fmaf(a[e], lds_row[e], s);
#pragma unroll
  for (int off = D / 64; off > 0; off >>= 1) s += __shfl_xor(s, off, D / 32);
  return s;
}

// Cooperative load of `rows` rows of D floats (row stride rs) into LDS [rows][D].
template <int D>
__device__ __forceinline__ void load_rows(float *dst, const float *src, size_t rs, int row0,
                                          int T) {
  constexpr int CPR = D / 4;
  for (int idx = threadIdx.x; idx < kF32Tile * CPR; idx += blockDim.x) {
    const int r = idx / CPR, ch = idx % CPR;
    const int t = row0 + r;
    u32x4 x = t < T ? ldg16(src + t * rs + ch * 4) : u32x4{};
    *reinterpret_cast<u32x4 *>(dst + r * D + ch * 4) = x;
  }
}

__device__ __forceinline__ bool visible(int i, int j, int window) {
  return j <= i && (window < 0 || i - j < window);
}

// ---------------------------------------------------------------- forward
template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float *__restrict__ q,
                                                      const float *__restrict__ k,
                                                      const float *__restrict__ v,
                                                      float *__restrict__ o,
                                                      float *__restrict__ lse, int B, int H,
                                                      int T, int window, float scale, int nqt) {
  constexpr int LPR = D / 32, QPB = 256 / LPR;
  __shared__ __attribute__((aligned(16))) float Ks[kF32Tile * D];
  __shared__ __attribute__((aligned(16))) float Vs[kF32Tile * D];
  const int BH = B * H, bid = blockIdx.x;
  const int qt = nqt - 1 - bid / BH, bh = bid % BH, b = bh / H, hh = bh % H;
  const size_t rs = (size_t)H * D, base = ((size_t)b * T * H + hh) * D;
  const int q0 = qt * QPB;
  const int my_q = q0 + threadIdx.x / LPR, sl = threadIdx.x % LPR;
  float qf[32], of[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    qf[e] = my_q < T ? q[base + my_q * rs + sl * 32 + e] : 0.f;
    of[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int q_last = min(T, q0 + QPB) - 1;
  const int k_lo = window > 0 ? max(0, q0 - window + 1) : 0;
  for (int kbase = (k_lo / kF32Tile) * kF32Tile; kbase <= q_last; kbase += kF32Tile) {
    __syncthreads();
    load_rows<D>(Ks, k + base, rs, kbase, T);
    load_rows<D>(Vs, v + base, rs, kbase, T);
    __syncthreads();
    float sc[kF32Tile];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < kF32Tile; ++j) {
      const float s = row_dot<D>(qf, Ks + j * D + sl * 32) * scale;
      sc[j] = visible(my_q, kbase + j, window) ? s : -INFINITY;
      mt = fmaxf(mt, sc[j]);
    }
    const float m_new = fmaxf(m, mt);
    const float mu = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = expf(m - mu);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 32; ++e) of[e] *= alpha;
#pragma unroll
    for (int j = 0; j < kF32Tile; ++j) {
      const float p = expf(sc[j] - mu);
      l += p;
      const float *vr = Vs + j * D + sl * 32;
#pragma unroll
      for (int e = 0; e < 32; ++e) of[e] = fmaf(p, vr[e], of[e]);
    }
    m = m_new;
  }
  if (my_q < T) {
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < 32; ++e) o[base + my_q * rs + sl * 32 + e] = of[e] * inv;
    if (sl == 0) lse[(size_t)bh * T + my_q] = m + logf(l);
  }
}

// ---------------------------------------------------------------- delta
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_f32_kernel(const float *__restrict__ o,
                                                          const float *__restrict__ dO,
                                                          float *__restrict__ delta, int B,
                                                          int H, int T) {
  constexpr int LPR = D / 4;
  const int row = blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int sl = threadIdx.x % LPR;
  const int nrows = B * T * H;
  float acc = 0.f;
  if (row < nrows) {
    const u32x4 a = ldg16(o + (size_t)row * D + sl * 4);
    const u32x4 g = ldg16(dO + (size_t)row * D + sl * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf(__uint_as_float(a[e]), __uint_as_float(g[e]), acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (row < nrows && sl == 0) {
    const int hh = row % H, bt = row / H, t = bt % T, b = bt / T;
    delta[((size_t)b * H + hh) * T + t] = acc;
  }
}

// ---------------------------------------------------------------- dK, dV
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ dO, const float *__restrict__ lse, const float *__restrict__ delta,
    float *__restrict__ dk, float *__restrict__ dv, int B, int H, int T, int window,
    float scale, int nkt) {
  constexpr int LPR = D / 32, KPB = 256 / LPR;
  __shared__ __attribute__((aligned(16))) float Qs[kF32Tile * D];
  __shared__ __attribute__((aligned(16))) float Gs[kF32Tile * D];
  __shared__ float Ls[kF32Tile], Ds[kF32Tile];
  const int BH = B * H, bid = blockIdx.x;
  const int kt = bid / BH, bh = bid % BH, b = bh / H, hh = bh % H;
  const size_t rs = (size_t)H * D, base = ((size_t)b * T * H + hh) * D;
  const int k0 = kt * KPB;
  const int my_k = k0 + threadIdx.x / LPR, sl = threadIdx.x % LPR;
  float kf[32], vf[32], dkf[32], dvf[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    kf[e] = my_k < T ? k[base + my_k * rs + sl * 32 + e] : 0.f;
    vf[e] = my_k < T ? v[base + my_k * rs + sl * 32 + e] : 0.f;
    dkf[e] = 0.f;
    dvf[e] = 0.f;
  }
  const int k_last = min(T, k0 + KPB) - 1;
  const int q_hi = window > 0 ? min(T - 1, k_last + window - 1) : T - 1;
  for (int qbase = (k0 / kF32Tile) * kF32Tile; qbase <= q_hi; qbase += kF32Tile) {
    __syncthreads();
    load_rows<D>(Qs, q + base, rs, qbase, T);
    load_rows<D>(Gs, dO + base, rs, qbase, T);
    if (threadIdx.x < kF32Tile) {
      const int qq = qbase + threadIdx.x;
      Ls[threadIdx.x] = qq < T ? lse[(size_t)bh * T + qq] : INFINITY;
      Ds[threadIdx.x] = qq < T ? delta[(size_t)bh * T + qq] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int i = 0; i < kF32Tile; ++i) {
      const float *qr = Qs + i * D + sl * 32;
      const float *gr = Gs + i * D + sl * 32;
      const float s = row_dot<D>(kf, qr) * scale;
      const float dp = row_dot<D>(vf, gr);
      const float p = visible(qbase + i, my_k, window) ? expf(s - Ls[i]) : 0.f;
      const float ds = p * (dp - Ds[i]);
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        dvf[e] = fmaf(p, gr[e], dvf[e]);
        dkf[e] = fmaf(ds, qr[e], dkf[e]);
      }
    }
  }
  if (my_k < T) {
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      dk[base + my_k * rs + sl * 32 + e] = dkf[e] * scale;
      dv[base + my_k * rs + sl * 32 + e] = dvf[e];
    }
  }
}

// ---------------------------------------------------------------- dQ
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ dO, const float *__restrict__ lse, const float *__restrict__ delta,
    float *__restrict__ dq, int B, int H, int T, int window, float scale, int nqt) {
  constexpr int LPR = D / 32, QPB = 256 / LPR;
  __shared__ __attribute__((aligned(16))) float Ks[kF32Tile * D];
  __shared__ __attribute__((aligned(16))) float Vs[kF32Tile * D];
  const int BH = B * H, bid = blockIdx.x;
  const int qt = nqt - 1 - bid / BH, bh = bid % BH, b = bh / H, hh = bh % H;
  const size_t rs = (size_t)H * D, base = ((size_t)b * T * H + hh) * D;
  const int q0 = qt * QPB;
  const int my_q = q0 + threadIdx.x / LPR, sl = threadIdx.x % LPR;
  float qf[32], gf[32], dqf[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) {
    qf[e] = my_q < T ? q[base + my_q * rs + sl * 32 + e] : 0.f;
    gf[e] = my_q < T ? dO[base + my_q * rs + sl * 32 + e] : 0.f;
    dqf[e] = 0.f;
  }
  const float lq = my_q < T ? lse[(size_t)bh * T + my_q] : INFINITY;
  const float dl = my_q < T ? delta[(size_t)bh * T + my_q] : 0.f;
  const int q_last = min(T, q0 + QPB) - 1;
  const int k_lo = window > 0 ? max(0, q0 - window + 1) : 0;
  for (int kbase = (k_lo / kF32Tile) * kF32Tile; kbase <= q_last; kbase += kF32Tile) {
    __syncthreads();
    load_rows<D>(Ks, k + base, rs, kbase, T);
    load_rows<D>(Vs, v + base, rs, kbase, T);
    __syncthreads();
#pragma unroll 4
    for (int j = 0; j < kF32Tile; ++j) {
      const float *kr = Ks + j * D + sl * 32;
      const float s = row_dot<D>(qf, kr) * scale;
      const float dp = row_dot<D>(gf, Vs + j * D + sl * 32);
      const float p = visible(my_q, kbase + j, window) ? expf(s - lq) : 0.f;
      const float ds = p * (dp - dl);
#pragma unroll
      for (int e = 0; e < 32; ++e) dqf[e] = fmaf(ds, kr[e], dqf[e]);
    }
  }
  if (my_q < T) {
#pragma unroll
    for (int e = 0; e < 32; ++e) dq[base + my_q * rs + sl * 32 + e] = dqf[e] * scale;
  }
}

template <int D>
static hipError_t launch_fwd_f32_d(const float *q, const float *k, const float *v, float *o,
                                   float *lse, int B, int H, int T, int window, float scale,
                                   hipStream_t st) {
  constexpr int QPB = 256 / (D / 32);
  const int nqt = (T + QPB - 1) / QPB;
  fwd_f32_kernel<D><<<nqt * B * H, 256, 0, st>>>(q, k, v, o, lse, B, H, T, window, scale, nqt);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                          int B, int H, int T, int D, int window, float scale, hipStream_t st) {
  if (D == 128) return launch_fwd_f32_d<128>(q, k, v, o, lse, B, H, T, window, scale, st);
  return launch_fwd_f32_d<64>(q, k, v, o, lse, B, H, T, window, scale, st);
}

hipError_t launch_bwd_pre_f32(const float *o, const float *dO, float *delta, int B, int H, int T,
                              int D, hipStream_t st) {
  const int rows = B * T * H, rpb = 256 / (D / 4);
  const unsigned nb = (unsigned)((rows + rpb - 1) / rpb);
  if (D == 128) bwd_pre_f32_kernel<128><<<nb, 256, 0, st>>>(o, dO, delta, B, H, T);
  else bwd_pre_f32_kernel<64><<<nb, 256, 0, st>>>(o, dO, delta, B, H, T);
  return hipGetLastError();
}

template <int D>
static int f32_rows_per_block() { return 256 / (D / 32); }

hipError_t launch_bwd_dkdv_f32(const float *q, const float *k, const float *v, const float *dO,
                               const float *lse, const float *delta, float *dk, float *dv, int B,
                               int H, int T, int D, int window, float scale, hipStream_t st) {
  const int pb = D == 128 ? f32_rows_per_block<128>() : f32_rows_per_block<64>();
  const int nt = (T + pb - 1) / pb;
  const unsigned nb = (unsigned)(nt * B * H);
  if (D == 128)
    bwd_dkdv_f32_kernel<128><<<nb, 256, 0, st>>>(q, k, v, dO, lse, delta, dk, dv, B, H, T,
                                                  window, scale, nt);
  else
    bwd_dkdv_f32_kernel<64><<<nb, 256, 0, st>>>(q, k, v, dO, lse, delta, dk, dv, B, H, T, window,
                                                 scale, nt);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_f32(const float *q, const float *k, const float *v, const float *dO,
                             const float *lse, const float *delta, float *dq, int B, int H, int T,
                             int D, int window, float scale, hipStream_t st) {
  const int pb = D == 128 ? f32_rows_per_block<128>() : f32_rows_per_block<64>();
  const int nt = (T + pb - 1) / pb;
  const unsigned nb = (unsigned)(nt * B * H);
  if (D == 128)
    bwd_dq_f32_kernel<128><<<nb, 256, 0, st>>>(q, k, v, dO, lse, delta, dq, B, H, T, window,
                                                scale, nt);
  else
    bwd_dq_f32_kernel<64><<<nb, 256, 0, st>>>(q, k, v, dO, lse, delta, dq, B, H, T, window, scale,
                                               nt);
  return hipGetLastError();
}

}  // namespace swattn

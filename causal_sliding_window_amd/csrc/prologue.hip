// QK-norm + rotary prologue and its backward (nanochat release article,
// architecture list: rotary embeddings as the only position encoding, QK norm, a
// weightless RMSNorm; nanochat guide, section 1 "GPT model", feature list: rotary
// embeddings encode relative position, QK normalisation).
//
// Forward, per (b, t, head) D-vector x of q or k, token position p = max(off_b, 0) + t:
//   x_n = x / sqrt(mean(x^2) + eps);  pair i = (x_n[i], x_n[i + D/2]) rotated by
//   p * base^(-2i/D):  y_i = a cos - b sin,  y_{i+D/2} = a sin + b cos.
// Backward: g = the inverse rotation of dy, r = 1 / sqrt(mean(x^2) + eps),
//   dx = r g - r^3 x (x . g) / D.
// One pass over q and k (and dq', dk' in the backward) in one launch: bound by HBM.
//
// Each wave takes kPrologueRows consecutive token rows (b, t).  A D-vector is D/8
// lanes with one 16-byte load each; the two halves of every pair sit in lanes D/16
// apart and meet through one shuffle per dword.  The D/2 pair frequencies are computed
// once per wave in fp64; per row, lane i forms the angle of pair i as position times
// frequency in fp64, reduces it modulo 2 pi in fp64 and takes cos and sin in fp32
// (the error stays near fp32 rounding at any position), then shuffles hand each lane
// the values of its pairs.  Fp32 arithmetic, outputs rounded to bf16 (nearest even).
// Each lane writes only the elements it read, after reading them: outputs may alias
// their own inputs.
#include "common.h"
#include "launch.h"

namespace swattn {

constexpr int kPrologueRows = 4;  // token rows per wave

template <int D, bool BWD>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(
    // no __restrict__ on the tensors: q_out may be q, k_out k, and in the backward the
    // outputs may be dq_in, dk_in (in place)
    const uint16_t *q, const uint16_t *k, const uint16_t *dq_in,
    const uint16_t *dk_in, uint16_t *q_out, uint16_t *k_out, const int *__restrict__ pos_off,
    int T, int H, int Hkv, int nrows, float base, float eps) {
  constexpr int LPV = D / 8;     // lanes per vector
  constexpr int HALF = LPV / 2;  // lane distance between the halves of a pair
  constexpr int VPW = 64 / LPV;  // vectors per wave and pass
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int s = lane % LPV;  // position of this lane in its vector
  const int nvec = H + Hkv;
  const int i0 = 8 * (s % HALF);           // first pair index of this lane's 8 elements
  const float sg = s < HALF ? -1.f : 1.f;  // first half: a c - b s; second: b c + a s
  // lane i < D/2 holds the frequency of pair i (fp64), for all of the wave's rows
  const double inv = lane < D / 2 ? pow((double)base, -2.0 * lane / D) : 0.0;
  const int row0 = (blockIdx.x * 4 + w) * kPrologueRows;

  for (int rr = 0; rr < kPrologueRows; ++rr) {
    const int row = row0 + rr;  // b * T + t
    if (row >= nrows) break;
    const int b = row / T, t = row - b * T;
    // element offset of vector v's 16 bytes for this lane (q heads first, then k)
    auto elem = [&](int v) {
      return (v < H ? ((size_t)row * H + v) * D : ((size_t)row * Hkv + (v - H)) * D) + 8 * s;
    };
    auto load = [&](int v, u32x4 &raw, u32x4 &gr) {
      raw = u32x4{0, 0, 0, 0};
      gr = u32x4{0, 0, 0, 0};
      if (v < nvec) {
        raw = ldg16((v < H ? q : k) + elem(v));
        if constexpr (BWD) gr = ldg16((v < H ? dq_in : dk_in) + elem(v));
      }
    };
    // the row's first vectors are requested before its angles are computed
    int v = lane / LPV;
    u32x4 raw, gr;
    load(v, raw, gr);
    // angle of pair `lane`: position times frequency in fp64, reduced to [-pi, pi] in
    // fp64, then cos and sin in fp32
    const long long p = (long long)max(pos_off ? pos_off[b] : 0, 0) + t;
    double ang = (double)p * inv;
    ang -= rint(ang * 0.15915494309189535) * 6.283185307179586;
    float sv, cv;
    sincosf((float)ang, &sv, &cv);
    float c8[8], s8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      c8[e] = __shfl(cv, i0 + e);
      s8[e] = sg * __shfl(sv, i0 + e);
    }
    for (; v - lane / LPV < nvec; v += VPW) {
      const bool on = v < nvec;  // every lane of the wave takes part in the shuffles
      const size_t e0 = elem(v);
      uint16_t *dst = v < H ? q_out : k_out;
      float x[8], xp[8];
      float ss = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = bf16_lo(raw[j]);
        x[2 * j + 1] = bf16_hi(raw[j]);
        ss = fmaf(x[2 * j], x[2 * j], fmaf(x[2 * j + 1], x[2 * j + 1], ss));
      }
      u32x4 out;
      if constexpr (!BWD) {
        u32x4 pr;
#pragma unroll
        for (int j = 0; j < 4; ++j) pr[j] = __shfl_xor(raw[j], HALF);
#pragma unroll
        for (int m = 1; m < LPV; m <<= 1) ss += __shfl_xor(ss, m);
        const float r = 1.f / sqrtf(ss / D + eps);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xp[2 * j] = bf16_lo(pr[j]);
          xp[2 * j + 1] = bf16_hi(pr[j]);
        }
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = r * fmaf(x[e], c8[e], xp[e] * s8[e]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          out[j] = f32_to_bf16_bits(y[2 * j]) | ((uint32_t)f32_to_bf16_bits(y[2 * j + 1]) << 16);
      } else {
        // g = inverse rotation of dy: own c - sg * partner sin
        u32x4 pr;
#pragma unroll
        for (int j = 0; j < 4; ++j) pr[j] = __shfl_xor(gr[j], HALF);
        float g[8], xg = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float d0 = bf16_lo(gr[j]), d1 = bf16_hi(gr[j]);
          const float p0 = bf16_lo(pr[j]), p1 = bf16_hi(pr[j]);
          g[2 * j] = fmaf(d0, c8[2 * j], -p0 * s8[2 * j]);
          g[2 * j + 1] = fmaf(d1, c8[2 * j + 1], -p1 * s8[2 * j + 1]);
          xg = fmaf(x[2 * j], g[2 * j], fmaf(x[2 * j + 1], g[2 * j + 1], xg));
        }
#pragma unroll
        for (int m = 1; m < LPV; m <<= 1) {
          ss += __shfl_xor(ss, m);
          xg += __shfl_xor(xg, m);
        }
        const float r = 1.f / sqrtf(ss / D + eps);
        const float c = r * r * r * xg / D;
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = fmaf(r, g[e], -c * x[e]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          out[j] = f32_to_bf16_bits(y[2 * j]) | ((uint32_t)f32_to_bf16_bits(y[2 * j + 1]) << 16);
      }
      load(v + VPW, raw, gr);  // the next vectors, before this one is stored
      if (on) *reinterpret_cast<u32x4 *>(dst + e0) = out;
    }
  }
}

template <bool BWD>
static hipError_t launch_prologue_t(const void *q, const void *k, const void *dq_in,
                                    const void *dk_in, void *q_out, void *k_out,
                                    const int *pos_off, int B, int T, int H, int Hkv, int D,
                                    float base, float eps, hipStream_t st) {
  const int nrows = B * T;
  const dim3 grid((unsigned)((nrows + 4 * kPrologueRows - 1) / (4 * kPrologueRows))), block(256);
  if (D == 128)
    qk_norm_rope_kernel<128, BWD><<<grid, block, 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)dq_in,
        (const uint16_t *)dk_in, (uint16_t *)q_out, (uint16_t *)k_out, pos_off, T, H, Hkv, nrows,
        base, eps);
  else
    qk_norm_rope_kernel<64, BWD><<<grid, block, 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)dq_in,
        (const uint16_t *)dk_in, (uint16_t *)q_out, (uint16_t *)k_out, pos_off, T, H, Hkv, nrows,
        base, eps);
  return hipGetLastError();
}

hipError_t launch_qk_norm_rope(const void *q, const void *k, void *q_out, void *k_out,
                               const int *pos_off, int B, int T, int H, int Hkv, int D,
                               float base, float eps, hipStream_t st) {
  return launch_prologue_t<false>(q, k, nullptr, nullptr, q_out, k_out, pos_off, B, T, H, Hkv,
                                  D, base, eps, st);
}

hipError_t launch_qk_norm_rope_bwd(const void *q, const void *k, const void *dq_out,
                                   const void *dk_out, void *dq, void *dk, const int *pos_off,
                                   int B, int T, int H, int Hkv, int D, float base, float eps,
                                   hipStream_t st) {
  return launch_prologue_t<true>(q, k, dq_out, dk_out, dq, dk, pos_off, B, T, H, Hkv, D, base,
                                 eps, st);
}

}  // namespace swattn

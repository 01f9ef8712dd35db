// QK norm + rotary embedding inside the attention kernels (the prologue of the
// nanochat release article's architecture list and the guide's section 1 feature
// list, fused into the passes that hold q or k in registers).  Definitions as the
// standalone prologue (prologue.hip): per head vector x of D elements at token
// position p,
//   x_n = x / sqrt(mean(x^2) + eps);  pair i = (x_n[i], x_n[i + D/2]) rotated by
//   p * base^(-2i/D);  backward: g = the inverse rotation of dy, r = 1 / sqrt(mean(x^2)
//   + eps), dx = r g - r^3 x (x . g) / D.
// A vector is held by a lane pair (lane l and l ^ 32) in one of two orders:
//   operand order (Q or K rows as MFMA operands): element 16 st + 8 h + j in slot
//     [st][j] of the lane in half h (st < D/16, j < 8);
//   accumulator order (dQ^T or dK^T C registers): element 32 db + 8 g + 4 h + e in
//     register 4 g + e of block db (db < D/32, g, e < 4).
// In both orders the two elements of a pair sit in the same lane.  Angles: the pair
// frequencies base^(-2i/D) are powers of ratio = base^(-2/D) (fp64, computed on the
// host), formed by a few fp64 products per lane; the angle in revolutions p f / (2 pi)
// is reduced to [-1/2, 1/2] in fp64 and its sine and cosine taken by the hardware
// (v_sin_f32 / v_cos_f32 take revolutions).  The rounding of these steps stays far
// below the bf16 rounding of the rotated vector.
#pragma once

#include "common.h"

namespace swattn {

struct RopeArgs {
  const int *pos_off;  // device int32 [B] (offset of each sequence's token 0), or null
  double ratio;        // base^(-2/D)
  float eps;
};

constexpr double kInv2Pi = 0.15915494309189533577;

// cos and sin of the angle p * f (radians), via revolutions reduced in fp64
__device__ __forceinline__ void rope_cs(double pf, float &c, float &s) {
  double rev = pf * kInv2Pi;
  rev -= rint(rev);
  const float x = (float)rev;
  c = __builtin_amdgcn_cosf(x);
  s = __builtin_amdgcn_sinf(x);
}

// ratio^n for a small n >= 0 (repeated squaring, fp64)
__device__ __forceinline__ double rope_pow(double ratio, int n) {
  double r = 1.0, b = ratio;
  while (n > 0) {
    if (n & 1) r *= b;
    b *= b;
    n >>= 1;
  }
  return r;
}

// Token position of row t of sequence b.
__device__ __forceinline__ double rope_pos(const RopeArgs &ra, int b, int t) {
  return (double)(max(ra.pos_off ? ra.pos_off[b] : 0, 0)) + (double)t;
}

// Forward of the prologue on a vector in operand order (x: this lane's D/2 elements,
// bf16, replaced by the normalised, rotated vector rounded to bf16).  `valid` false:
// a padding row (past the sequence), returned as zeros.
template <int D>
__device__ __forceinline__ void rope_norm_operand(bf16x8 (&x)[D / 16], double p, bool valid,
                                                  const RopeArgs &ra, int h) {
  constexpr int KST = D / 16, HS = KST / 2;
  float f[KST][8];
  float ss = 0.f;
#pragma unroll
  for (int st = 0; st < KST; ++st)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      f[st][j] = (float)x[st][j];
      ss = fmaf(f[st][j], f[st][j], ss);
    }
  ss = xhalf_sum(ss);
  const float r = valid ? 1.f / sqrtf(ss / D + ra.eps) : 0.f;
  // frequency of pair 8 h + j, then of 16 st + 8 h + j
  double fr[8];
  fr[0] = h ? rope_pow(ra.ratio, 8) : 1.0;
#pragma unroll
  for (int j = 1; j < 8; ++j) fr[j] = fr[j - 1] * ra.ratio;
  const double r16 = rope_pow(ra.ratio, 16);
#pragma unroll
  for (int st = 0; st < HS; ++st) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float c, s;
      rope_cs(p * fr[j], c, s);
      const float a = f[st][j], b = f[st + HS][j];
      f[st][j] = r * fmaf(a, c, -b * s);
      f[st + HS][j] = r * fmaf(a, s, b * c);
      fr[j] *= r16;
    }
  }
#pragma unroll
  for (int st = 0; st < KST; ++st) x[st] = to_bf16x8_arr(f[st]);
}

// Backward of the prologue on a gradient in accumulator order: dy (this lane's D/2
// elements of dL/dx', fp32, D/32 blocks of 16) becomes dL/dx; xr is the raw vector's
// lane elements in the same order (fp32).  `valid` false: zeros.
template <int D>
__device__ __forceinline__ void rope_norm_grad_acc(f32x16 (&dy)[D / 32], const f32x16 (&xr)[D / 32],
                                                   double p, bool valid, const RopeArgs &ra,
                                                   int h) {
  constexpr int NDB = D / 32, HB = NDB / 2;
  // g = the inverse rotation of dy, pair by pair (blocks db and db + D/64 hold the two
  // halves); frequency of pair 32 db + 8 g + 4 h + e
  double fr[4];
  fr[0] = h ? rope_pow(ra.ratio, 4) : 1.0;
#pragma unroll
  for (int e = 1; e < 4; ++e) fr[e] = fr[e - 1] * ra.ratio;
  const double r8 = rope_pow(ra.ratio, 8), r32 = rope_pow(ra.ratio, 32);
#pragma unroll
  for (int db = 0; db < HB; ++db) {
    double fg[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) fg[e] = fr[e];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float c, s;
        rope_cs(p * fg[e], c, s);
        const int i = 4 * g + e;
        const float a = dy[db][i], b = dy[db + HB][i];
        dy[db][i] = fmaf(a, c, b * s);
        dy[db + HB][i] = fmaf(-a, s, b * c);
        fg[e] *= r8;
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) fr[e] *= r32;
  }
  float ss = 0.f, xg = 0.f;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ss = fmaf(xr[db][i], xr[db][i], ss);
      xg = fmaf(xr[db][i], dy[db][i], xg);
    }
  ss = xhalf_sum(ss);
  xg = xhalf_sum(xg);
  const float r = valid ? 1.f / sqrtf(ss / D + ra.eps) : 0.f;
  const float cc = r * r * r * xg / D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dy[db][i] = fmaf(r, dy[db][i], -cc * xr[db][i]);
}

// The raw vector's lane elements in accumulator order (bf16 row of D elements at `row`).
template <int D>
__device__ __forceinline__ void load_acc_order(const uint16_t *row, int h, f32x16 (&xr)[D / 32]) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2 w = *reinterpret_cast<const u32x2 *>(row + 32 * db + 8 * g + 4 * h);
      xr[db][4 * g + 0] = bf16_lo(w[0]);
      xr[db][4 * g + 1] = bf16_hi(w[0]);
      xr[db][4 * g + 2] = bf16_lo(w[1]);
      xr[db][4 * g + 3] = bf16_hi(w[1]);
    }
}

}  // namespace swattn

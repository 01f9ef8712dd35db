// Backward of causal sliding-window attention, bf16 in / bf16 out, fp32 accumulate.
//
// Gradients of L = sum_i dO_i . o_i for the attention of the nanochat guide's
// section 5 (the training step back-propagates through it).  With P recomputed
// from the stored LSE:
//   delta_i = dO_i . o_i                       (bwd_pre_kernel)
//   dV = P^T dO,  dK = scale * dS^T Q           (dkdv kernel, one pass per KV tile)
//   dQ = scale * dS K                           (dq kernel, one pass per Q tile)
//   with dP = dO V^T and dS = P * (dP - delta).
// The two passes each recompute S and dP, so no atomics are needed and the
// results are bitwise reproducible.
//
// Layouts inside the dK/dV pass: S = Q K^T is formed with one key per lane
// (A = Q rows from LDS, B = K^T from registers), so P and dS feed dV^T = dO^T P
// and dK^T = Q^T dS as B operands straight from registers; dO^T and Q^T come from
// transposed LDS reads.  Inside the dQ pass S^T = K Q^T is formed with one query
// per lane (as in the forward) and dS^T feeds dQ^T = K^T dS^T; K^T comes from
// transposed LDS reads.
#include "common.h"
#include "launch.h"

namespace swattn {

// ---------------------------------------------------------------- delta = rowsum(dO * O)
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_bf16_kernel(const uint16_t *__restrict__ o,
                                                           const uint16_t *__restrict__ dO,
                                                           float *__restrict__ delta, int B,
                                                           int H, int T) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  const int row = blockIdx.x * (256 / LPR) + threadIdx.x / LPR;  // row = (b*T + t)*H + h
  const int sl = threadIdx.x % LPR;
  const int nrows = B * T * H;
  float acc = 0.f;
  if (row < nrows) {
    const u32x4 a = ldg16(o + (size_t)row * D + sl * 8);
    const u32x4 g = ldg16(dO + (size_t)row * D + sl * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += bf16_lo(a[e]) * bf16_lo(g[e]) + bf16_hi(a[e]) * bf16_hi(g[e]);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (row < nrows && sl == 0) {
    const int hh = row % H;
    const int bt = row / H;
    const int t = bt % T, b = bt / T;
    delta[((size_t)b * H + hh) * T + t] = acc;
  }
}

// ---------------------------------------------------------------- dK, dV
template <int D>
struct DkdvCfg {
  static constexpr int BK = 128;          // keys per workgroup (4 waves x 32)
  static constexpr int BQ = 64;           // queries per LDS tile
  static constexpr int NT = 256;
  static constexpr int QLD = D + 8;       // Q / dO tile pitch (elements)
  static constexpr int QSZ = BQ * QLD;
  static constexpr int CPR = D / 8;
  static constexpr int RPP = NT / CPR;
  static constexpr int PASSES = BQ / RPP;
};

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ dO,
    const float *__restrict__ lse, const float *__restrict__ delta, uint16_t *__restrict__ dk,
    uint16_t *__restrict__ dv, int B, int H, int T, int window, float scale, int nkt) {
  using C = DkdvCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2 * C::QSZ];
  __shared__ __attribute__((aligned(16))) uint16_t Gs[2 * C::QSZ];  // dO
  __shared__ __attribute__((aligned(16))) float Ls[2 * C::BQ];        // lse * log2(e)
  __shared__ __attribute__((aligned(16))) float Ds[2 * C::BQ];        // delta

  const int BH = B * H;
  const int bid = blockIdx.x;
  const int kt = bid / BH;  // early key tiles see the most queries: first
  const int bh = bid % BH;
  const int b = bh / H, hh = bh % H;
  const int k0 = kt * C::BK;
  const size_t rs = (size_t)H * D;
  const size_t base = ((size_t)b * T * H + hh) * D;
  const uint16_t *qb = q + base, *kb = k + base, *vb = v + base, *gb = dO + base;
  const float *lseb = lse + (size_t)bh * T, *delb = delta + (size_t)bh * T;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, ln = lane & 31;
  const int kw0 = k0 + 32 * w;
  const int my_k = kw0 + ln;

  const int k_last = min(T, k0 + C::BK) - 1;
  const int q_hi = window > 0 ? min(T - 1, k_last + window - 1) : T - 1;
  const int qt0 = k0 / C::BQ, qt1 = q_hi / C::BQ;
  const int wk_hi = min(T - 1, kw0 + 31);
  const int wq_hi = window > 0 ? wk_hi + window - 1 : T - 1;

  bf16x8 kr[D / 16], vr[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    if (my_k < T) {
      kr[st] = *reinterpret_cast<const bf16x8 *>(kb + my_k * rs + 16 * st + 8 * h);
      vr[st] = *reinterpret_cast<const bf16x8 *>(vb + my_k * rs + 16 * st + 8 * h);
    } else {
      kr[st] = bf16x8{};
      vr[st] = bf16x8{};
    }
  }
  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) {
    dka[d] = f32x16{};
    dva[d] = f32x16{};
  }
  const float c = scale * kLog2e;

  u32x4 qreg[C::PASSES], greg[C::PASSES];
  float lreg = 0.f, dreg = 0.f;
  const int lrow = tid / C::CPR, lch = tid % C::CPR;

  auto gload = [&](int qt) {
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) {
      const int qq = qt * C::BQ + lrow + p * C::RPP;
      if (qq < T) {
        qreg[p] = ldg16(qb + qq * rs + lch * 8);
        greg[p] = ldg16(gb + qq * rs + lch * 8);
      } else {
        qreg[p] = u32x4{};
        greg[p] = u32x4{};
      }
    }
    if (tid < C::BQ) {
      const int qq = qt * C::BQ + tid;
      lreg = qq < T ? lseb[qq] * kLog2e : INFINITY;  // rows past T get p = 0
      dreg = qq < T ? delb[qq] : 0.f;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) {
      const int r = lrow + p * C::RPP;
      const int rp = (r & ~31) | swap23(r & 31);
      *reinterpret_cast<u32x4 *>(Qs + buf * C::QSZ + rp * C::QLD + lch * 8) = qreg[p];
      *reinterpret_cast<u32x4 *>(Gs + buf * C::QSZ + rp * C::QLD + lch * 8) = greg[p];
    }
    if (tid < C::BQ) {
      Ls[buf * C::BQ + tid] = lreg;
      Ds[buf * C::BQ + tid] = dreg;
    }
  };

  gload(qt0);
  sstore(0);
  __syncthreads();

  for (int qt = qt0; qt <= qt1; ++qt) {
    const int buf = (qt - qt0) & 1;
    if (qt < qt1) gload(qt + 1);
    const int qbase = qt * C::BQ;
    const bool active = kw0 <= wk_hi && qbase + C::BQ - 1 >= kw0 && qbase <= wq_hi;
    if (active) {
      const bool need_mask = (qbase < wk_hi) || (window > 0 && qbase + C::BQ - 1 - kw0 >= window);
      const uint16_t *Qt = Qs + buf * C::QSZ;
      const uint16_t *Gt = Gs + buf * C::QSZ;
      const float *Lt = Ls + buf * C::BQ;
      const float *Dt = Ds + buf * C::BQ;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        f32x16 s = f32x16{}, dp = f32x16{};
        const uint16_t *qp = Qt + (sb * 32 + ln) * C::QLD + 8 * h;
        const uint16_t *gp = Gt + (sb * 32 + ln) * C::QLD + 8 * h;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) s = mfma32(lds_read_b128(qp + 16 * st), kr[st], s);
#pragma unroll
        for (int st = 0; st < D / 16; ++st) dp = mfma32(lds_read_b128(gp + 16 * st), vr[st], dp);
        // register i holds query row sb*32 + c_row(i, h) = sb*32 + 16*(i/8) + 8h + i%8
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int r0 = sb * 32 + 16 * t + 8 * h;
          const f32x4 l0 = *reinterpret_cast<const f32x4 *>(Lt + r0);
          const f32x4 l1 = *reinterpret_cast<const f32x4 *>(Lt + r0 + 4);
          const f32x4 d0 = *reinterpret_cast<const f32x4 *>(Dt + r0);
          const f32x4 d1 = *reinterpret_cast<const f32x4 *>(Dt + r0 + 4);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int i = 8 * t + j;
            const float lj = j < 4 ? l0[j] : l1[j - 4];
            const float dj = j < 4 ? d0[j] : d1[j - 4];
            float p = fast_exp2(fmaf(s[i], c, -lj));
            if (need_mask) {
              const int qq = qbase + r0 + j;
              const bool vis = my_k <= qq && (window < 0 || qq - my_k < window);
              if (!vis) p = 0.f;
            }
            s[i] = p;
            dp[i] = p * (dp[i] - dj);
          }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          // P enters dV as bf16 hi + lo (P = hi + lo to ~16 bits): a single bf16 P
          // leaves |dV| >= 4 outside 2e-2 of the exact gradient.
          const bf16x8 pb = to_bf16x8(s, 8 * t);
          bf16x8 pl;
#pragma unroll
          for (int j = 0; j < 8; ++j) pl[j] = (__bf16)(s[8 * t + j] - (float)pb[j]);
          const bf16x8 sbv = to_bf16x8(dp, 8 * t);
          const uint16_t *gt = Gt + (sb * 32 + 16 * t) * C::QLD;
          const uint16_t *qt_ = Qt + (sb * 32 + 16 * t) * C::QLD;
#pragma unroll
          for (int d = 0; d < D / 32; ++d) {
            const bf16x8 ga = lds_read_tr_block_perm(gt + 32 * d, C::QLD, lane);
            dva[d] = mfma32(ga, pb, dva[d]);
            dva[d] = mfma32(ga, pl, dva[d]);
            dka[d] = mfma32(lds_read_tr_block_perm(qt_ + 32 * d, C::QLD, lane), sbv, dka[d]);
          }
        }
      }
    }
    if (qt < qt1) sstore(buf ^ 1);
    __syncthreads();
  }

  if (my_k < T) {
    uint16_t *dkb = dk + base, *dvb = dv + base;
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 pk, pv;
        pk[0] = (uint32_t)f32_to_bf16_bits(dka[d][4 * g] * scale) |
                ((uint32_t)f32_to_bf16_bits(dka[d][4 * g + 1] * scale) << 16);
        pk[1] = (uint32_t)f32_to_bf16_bits(dka[d][4 * g + 2] * scale) |
                ((uint32_t)f32_to_bf16_bits(dka[d][4 * g + 3] * scale) << 16);
        pv[0] = (uint32_t)f32_to_bf16_bits(dva[d][4 * g]) |
                ((uint32_t)f32_to_bf16_bits(dva[d][4 * g + 1]) << 16);
        pv[1] = (uint32_t)f32_to_bf16_bits(dva[d][4 * g + 2]) |
                ((uint32_t)f32_to_bf16_bits(dva[d][4 * g + 3]) << 16);
        const size_t off = my_k * rs + 32 * d + 8 * g + 4 * h;
        *reinterpret_cast<u32x2 *>(dkb + off) = pk;
        *reinterpret_cast<u32x2 *>(dvb + off) = pv;
      }
  }
}

// ---------------------------------------------------------------- dQ
template <int D>
struct DqCfg {
  static constexpr int BM = 128;          // queries per workgroup (4 waves x 32)
  static constexpr int BN = 64;           // keys per LDS tile
  static constexpr int NT = 256;
  static constexpr int KLD = D + 8;
  static constexpr int KSZ = BN * KLD;
  static constexpr int CPR = D / 8;
  static constexpr int RPP = NT / CPR;
  static constexpr int PASSES = BN / RPP;
};

template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ dO,
    const float *__restrict__ lse, const float *__restrict__ delta, uint16_t *__restrict__ dq,
    int B, int H, int T, int window, float scale, int nqt) {
  using C = DqCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2 * C::KSZ];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2 * C::KSZ];

  const int BH = B * H;
  const int bid = blockIdx.x;
  const int qt = nqt - 1 - bid / BH;
  const int bh = bid % BH;
  const int b = bh / H, hh = bh % H;
  const int q0 = qt * C::BM;
  const size_t rs = (size_t)H * D;
  const size_t base = ((size_t)b * T * H + hh) * D;
  const uint16_t *qb = q + base, *kb = k + base, *vb = v + base, *gb = dO + base;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, ln = lane & 31;
  const int qw0 = q0 + 32 * w;
  const int my_q = qw0 + ln;

  const int q_last = min(T, q0 + C::BM) - 1;
  const int k_lo = window > 0 ? max(0, q0 - window + 1) : 0;
  const int kt0 = k_lo / C::BN, kt1 = q_last / C::BN;
  const int wq_lo = qw0, wq_hi = min(T - 1, qw0 + 31);
  const int wk_lo = window > 0 ? wq_lo - window + 1 : 0;

  bf16x8 qr[D / 16], gr[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    if (my_q < T) {
      qr[st] = *reinterpret_cast<const bf16x8 *>(qb + my_q * rs + 16 * st + 8 * h);
      gr[st] = *reinterpret_cast<const bf16x8 *>(gb + my_q * rs + 16 * st + 8 * h);
    } else {
      qr[st] = bf16x8{};
      gr[st] = bf16x8{};
    }
  }
  const float l2 = my_q < T ? lse[(size_t)bh * T + my_q] * kLog2e : INFINITY;
  const float dl = my_q < T ? delta[(size_t)bh * T + my_q] : 0.f;
  const float c = scale * kLog2e;

  f32x16 acc[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) acc[d] = f32x16{};

  u32x4 kreg[C::PASSES], vreg[C::PASSES];
  const int lrow = tid / C::CPR, lch = tid % C::CPR;
  auto gload = [&](int kt) {
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) {
      const int key = kt * C::BN + lrow + p * C::RPP;
      if (key < T) {
        kreg[p] = ldg16(kb + key * rs + lch * 8);
        vreg[p] = ldg16(vb + key * rs + lch * 8);
      } else {
        kreg[p] = u32x4{};
        vreg[p] = u32x4{};
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < C::PASSES; ++p) {
      const int r = lrow + p * C::RPP;
      const int rp = (r & ~31) | swap23(r & 31);
      *reinterpret_cast<u32x4 *>(Ks + buf * C::KSZ + rp * C::KLD + lch * 8) = kreg[p];
      *reinterpret_cast<u32x4 *>(Vs + buf * C::KSZ + rp * C::KLD + lch * 8) = vreg[p];
    }
  };

  gload(kt0);
  sstore(0);
  __syncthreads();

  for (int kt = kt0; kt <= kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    if (kt < kt1) gload(kt + 1);
    const int kbase = kt * C::BN;
    const bool active = wq_hi >= wq_lo && kbase <= wq_hi && kbase + C::BN - 1 >= wk_lo;
    if (active) {
      const bool need_mask =
          (kbase + C::BN - 1 > wq_lo) || (window > 0 && wq_hi - kbase >= window);
      const uint16_t *Kt = Ks + buf * C::KSZ;
      const uint16_t *Vt = Vs + buf * C::KSZ;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        f32x16 s = f32x16{}, dp = f32x16{};
        const uint16_t *kp = Kt + (sb * 32 + ln) * C::KLD + 8 * h;
        const uint16_t *vp = Vt + (sb * 32 + ln) * C::KLD + 8 * h;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) s = mfma32(lds_read_b128(kp + 16 * st), qr[st], s);
#pragma unroll
        for (int st = 0; st < D / 16; ++st) dp = mfma32(lds_read_b128(vp + 16 * st), gr[st], dp);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = fast_exp2(fmaf(s[i], c, -l2));
          if (need_mask) {
            const int key = kbase + sb * 32 + c_row(i, h);
            const bool vis = key <= my_q && (window < 0 || my_q - key < window);
            if (!vis) p = 0.f;
          }
          s[i] = p * (dp[i] - dl);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 dsb = to_bf16x8(s, 8 * t);
          const uint16_t *kt_ = Kt + (sb * 32 + 16 * t) * C::KLD;
#pragma unroll
          for (int d = 0; d < D / 32; ++d)
            acc[d] = mfma32(lds_read_tr_block_perm(kt_ + 32 * d, C::KLD, lane), dsb, acc[d]);
        }
      }
    }
    if (kt < kt1) sstore(buf ^ 1);
    __syncthreads();
  }

  if (my_q < T) {
    uint16_t *dqb = dq + base;
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 pk;
        pk[0] = (uint32_t)f32_to_bf16_bits(acc[d][4 * g] * scale) |
                ((uint32_t)f32_to_bf16_bits(acc[d][4 * g + 1] * scale) << 16);
        pk[1] = (uint32_t)f32_to_bf16_bits(acc[d][4 * g + 2] * scale) |
                ((uint32_t)f32_to_bf16_bits(acc[d][4 * g + 3] * scale) << 16);
        *reinterpret_cast<u32x2 *>(dqb + my_q * rs + 32 * d + 8 * g + 4 * h) = pk;
      }
  }
}

hipError_t launch_bwd_pre_bf16(const void *o, const void *dO, float *delta, int B, int H, int T,
                               int D, hipStream_t st) {
  const int rows = B * T * H;
  const int rpb = 256 / (D / 8);
  const unsigned nb = (unsigned)((rows + rpb - 1) / rpb);
  if (D == 128)
    bwd_pre_bf16_kernel<128><<<nb, 256, 0, st>>>((const uint16_t *)o, (const uint16_t *)dO,
                                                 delta, B, H, T);
  else
    bwd_pre_bf16_kernel<64><<<nb, 256, 0, st>>>((const uint16_t *)o, (const uint16_t *)dO, delta,
                                                B, H, T);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(const void *q, const void *k, const void *v, const void *dO,
                                const float *lse, const float *delta, void *dk, void *dv, int B,
                                int H, int T, int D, int window, float scale, hipStream_t st) {
  const int nkt = (T + 127) / 128;
  const unsigned nb = (unsigned)(nkt * B * H);
  if (D == 128)
    bwd_dkdv_bf16_kernel<128><<<nb, 256, 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)dO, lse,
        delta, (uint16_t *)dk, (uint16_t *)dv, B, H, T, window, scale, nkt);
  else
    bwd_dkdv_bf16_kernel<64><<<nb, 256, 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)dO, lse,
        delta, (uint16_t *)dk, (uint16_t *)dv, B, H, T, window, scale, nkt);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16(const void *q, const void *k, const void *v, const void *dO,
                              const float *lse, const float *delta, void *dq, int B, int H,
                              int T, int D, int window, float scale, hipStream_t st) {
  const int nqt = (T + 127) / 128;
  const unsigned nb = (unsigned)(nqt * B * H);
  if (D == 128)
    bwd_dq_bf16_kernel<128><<<nb, 256, 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)dO, lse,
        delta, (uint16_t *)dq, B, H, T, window, scale, nqt);
  else
    bwd_dq_bf16_kernel<64><<<nb, 256, 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)dO, lse,
        delta, (uint16_t *)dq, B, H, T, window, scale, nqt);
  return hipGetLastError();
}

}  // namespace swattn

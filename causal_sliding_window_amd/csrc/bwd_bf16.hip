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
#include <type_traits>

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
  static constexpr int TSZ = BQ * D;      // elements of one Q (or dO) tile
  static constexpr int NDB = D / 32;
  static constexpr int KST = D / 16;
  static constexpr int CPW = (2 * TSZ * 2 / 1024) / 4;  // 1 KB copies per wave and tile
};

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ dO,
    const float *__restrict__ lse, const float *__restrict__ delta, uint16_t *__restrict__ dk,
    uint16_t *__restrict__ dv, int B, int H, int T, int window, float scale, int nkt) {
  using C = DkdvCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * 2 * C::TSZ];  // [buf][Q, dO]
  __shared__ __attribute__((aligned(16))) float Ls[2 * C::BQ];             // lse * log2(e)
  __shared__ __attribute__((aligned(16))) float Ds[2 * C::BQ];             // delta

  const int BH = B * H;
  const int bid = blockIdx.x;
  const int kt = bid / BH;  // early key tiles see the most queries: first
  const int bh = bid % BH;
  const int b = bh / H, hh = bh % H;
  const int k0 = kt * C::BK;
  const int rs = H * D;
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
  // query qq sees key my_k iff 0 <= qq - my_k <= wm1
  const unsigned wm1 = window > 0 ? (unsigned)(window - 1) : 0x7fffffffu;

  bf16x8 kr[C::KST], vr[C::KST];
  {
    const int row = min(my_k, T - 1);
#pragma unroll
    for (int st = 0; st < C::KST; ++st) {
      kr[st] = *reinterpret_cast<const bf16x8 *>(kb + (size_t)row * rs + 16 * st + 8 * h);
      vr[st] = *reinterpret_cast<const bf16x8 *>(vb + (size_t)row * rs + 16 * st + 8 * h);
    }
  }
  f32x16 dka[C::NDB], dva[C::NDB];
#pragma unroll
  for (int d = 0; d < C::NDB; ++d) {
    dka[d] = f32x16{};
    dva[d] = f32x16{};
  }
  const float c = scale * kLog2e;

  // Q and dO tiles: direct global -> LDS copies (rows in swap23 order).
  auto issue_tile = [&](int qt, int buf) {
#pragma unroll
    for (int cc = 0; cc < C::CPW; ++cc) {
      const int j = w * C::CPW + cc;
      const int tensor = j / (4 * C::NDB), jj = j % (4 * C::NDB);
      copy_rows16<C::BQ>(smem + (2 * buf + tensor) * C::TSZ, tensor ? gb : qb, rs, qt * C::BQ, T,
                         16 * (jj & 3), jj >> 2, true, lane);
    }
  };
  // lse / delta of the tile: staged through registers (rows past T: lse = +inf, so p = 0)
  float lreg = 0.f;
  auto load_vec = [&](int qt) {
    if (tid < 2 * C::BQ) {
      const int qq = qt * C::BQ + (tid & (C::BQ - 1));
      const bool ok = qq < T;
      const int qc = ok ? qq : T - 1;
      lreg = tid < C::BQ ? (ok ? lseb[qc] * kLog2e : INFINITY) : (ok ? delb[qc] : 0.f);
    }
  };
  auto store_vec = [&](int buf) {
    if (tid < C::BQ) Ls[buf * C::BQ + tid] = lreg;
    else if (tid < 2 * C::BQ) Ds[buf * C::BQ + tid - C::BQ] = lreg;
  };

  issue_tile(qt0, 0);
  load_vec(qt0);
  store_vec(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int qt = qt0; qt <= qt1; ++qt) {
    const int buf = (qt - qt0) & 1;
    if (qt < qt1) {
      issue_tile(qt + 1, buf ^ 1);
      load_vec(qt + 1);
    }
    const int qbase = qt * C::BQ;
    const bool active = kw0 <= wk_hi && qbase + C::BQ - 1 >= kw0 && qbase <= wq_hi;
    if (active) {
      const bool need_mask = (qbase < wk_hi) || (window > 0 && qbase + C::BQ - 1 - kw0 >= window);
      const uint16_t *Qt = smem + 2 * buf * C::TSZ;
      const uint16_t *Gt = Qt + C::TSZ;
      const float *Lt = Ls + buf * C::BQ;
      const float *Dt = Ds + buf * C::BQ;
      const int rel0 = qbase + 8 * h - my_k;
      // Two 32-query sub-blocks, software pipelined: the softmax-side VALU work of
      // one sub-block is placed between independent MFMAs of the other.
      auto body = [&](auto masked) {
        constexpr bool MASK = decltype(masked)::value;
        f32x16 s[2], dp[2];
        bf16x8 pb[2][2], pl[2][2], sbv[2][2];
        auto qk = [&](int sb) {  // S = Q K^T, dP = dO V^T, one key per lane
          s[sb] = f32x16{};
          dp[sb] = f32x16{};
          const int row = sb * 32 + ln;
          bf16x8 qa[C::KST], ga[C::KST];  // all operands requested before the first MFMA
#pragma unroll
          for (int st = 0; st < C::KST; ++st) {
            qa[st] = lds_read_b128(Qt + dt_off<C::BQ>(row, 2 * st + h));
            ga[st] = lds_read_b128(Gt + dt_off<C::BQ>(row, 2 * st + h));
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int st = 0; st < C::KST; ++st) {
            s[sb] = mfma32(qa[st], kr[st], s[sb]);
            dp[sb] = mfma32(ga[st], vr[st], dp[sb]);
          }
        };
        auto softmax = [&](int sb) {  // P = exp(S - LSE), dS = P (dP - delta)
          // register 8t + j holds query row sb*32 + 16t + 8h + j
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int r0 = sb * 32 + 16 * t + 8 * h;
            const f32x4 l0 = *reinterpret_cast<const f32x4 *>(Lt + r0);
            const f32x4 l1 = *reinterpret_cast<const f32x4 *>(Lt + r0 + 4);
            const f32x4 d0 = *reinterpret_cast<const f32x4 *>(Dt + r0);
            const f32x4 d1 = *reinterpret_cast<const f32x4 *>(Dt + r0 + 4);
            f32x16 &S = s[sb], &G = dp[sb];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const int i = 8 * t + j;
              const float lj = j < 4 ? l0[j] : l1[j - 4];
              const float dj = j < 4 ? d0[j] : d1[j - 4];
              float p = fast_exp2(fmaf(S[i], c, -lj));
              if (MASK) p = (unsigned)(rel0 + sb * 32 + 16 * t + j) <= wm1 ? p : 0.f;
              S[i] = p;
              G[i] = p * (G[i] - dj);
            }
            // P enters dV as bf16 hi + lo (P = hi + lo to ~16 bits): a single bf16 P
            // leaves |dV| >= 4 outside 2e-2 of the exact gradient.
            pb[sb][t] = to_bf16x8(S, 8 * t);
#pragma unroll
            for (int j = 0; j < 8; ++j) pl[sb][t][j] = (__bf16)(S[8 * t + j] - (float)pb[sb][t][j]);
            sbv[sb][t] = to_bf16x8(G, 8 * t);
          }
        };
        auto grads = [&](int sb) {  // dV^T += dO^T P, dK^T += Q^T dS
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            bf16x8 gt[C::NDB], qt_[C::NDB];
#pragma unroll
            for (int d = 0; d < C::NDB; ++d) {
              gt[d] = dt_read_tr_perm<C::BQ>(Gt, sb * 32 + 16 * t, d, lane);
              qt_[d] = dt_read_tr_perm<C::BQ>(Qt, sb * 32 + 16 * t, d, lane);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int d = 0; d < C::NDB; ++d) {
              dva[d] = mfma32(gt[d], pb[sb][t], dva[d]);
              dva[d] = mfma32(gt[d], pl[sb][t], dva[d]);
              dka[d] = mfma32(qt_[d], sbv[sb][t], dka[d]);
            }
          }
        };
        qk(0);
        qk(1);
        softmax(0);
        grads(0);
        softmax(1);
        grads(1);
      };
      if (need_mask) body(std::true_type{});
      else body(std::false_type{});
    }
    if (qt < qt1) store_vec(buf ^ 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (my_k < T) {
    uint16_t *dkb = dk + base, *dvb = dv + base;
#pragma unroll
    for (int d = 0; d < C::NDB; ++d)
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
        const size_t off = (size_t)my_k * rs + 32 * d + 8 * g + 4 * h;
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
  static constexpr int TSZ = BN * D;
  static constexpr int NDB = D / 32;
  static constexpr int KST = D / 16;
  static constexpr int CPW = (2 * TSZ * 2 / 1024) / 4;
};

template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ dO,
    const float *__restrict__ lse, const float *__restrict__ delta, uint16_t *__restrict__ dq,
    int B, int H, int T, int window, float scale, int nqt) {
  using C = DqCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * 2 * C::TSZ];  // [buf][K, V]

  const int BH = B * H;
  const int bid = blockIdx.x;
  const int qt = nqt - 1 - bid / BH;
  const int bh = bid % BH;
  const int b = bh / H, hh = bh % H;
  const int q0 = qt * C::BM;
  const int rs = H * D;
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
  // key kk is visible to my_q iff 0 <= my_q - kk <= wm1
  const unsigned wm1 = window > 0 ? (unsigned)(window - 1) : 0x7fffffffu;

  bf16x8 qr[C::KST], gr[C::KST];
  {
    const int row = min(my_q, T - 1);
#pragma unroll
    for (int st = 0; st < C::KST; ++st) {
      qr[st] = *reinterpret_cast<const bf16x8 *>(qb + (size_t)row * rs + 16 * st + 8 * h);
      gr[st] = *reinterpret_cast<const bf16x8 *>(gb + (size_t)row * rs + 16 * st + 8 * h);
    }
  }
  const float l2 = my_q < T ? lse[(size_t)bh * T + my_q] * kLog2e : INFINITY;
  const float dl = my_q < T ? delta[(size_t)bh * T + my_q] : 0.f;
  const float c = scale * kLog2e;

  f32x16 acc[C::NDB];
#pragma unroll
  for (int d = 0; d < C::NDB; ++d) acc[d] = f32x16{};

  auto issue_tile = [&](int kt, int buf) {
#pragma unroll
    for (int cc = 0; cc < C::CPW; ++cc) {
      const int j = w * C::CPW + cc;
      const int tensor = j / (4 * C::NDB), jj = j % (4 * C::NDB);
      copy_rows16<C::BN>(smem + (2 * buf + tensor) * C::TSZ, tensor ? vb : kb, rs, kt * C::BN, T,
                         16 * (jj & 3), jj >> 2, true, lane);
    }
  };

  issue_tile(kt0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int kt = kt0; kt <= kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    if (kt < kt1) issue_tile(kt + 1, buf ^ 1);
    const int kbase = kt * C::BN;
    const bool active = wq_hi >= wq_lo && kbase <= wq_hi && kbase + C::BN - 1 >= wk_lo;
    if (active) {
      const bool need_mask =
          (kbase + C::BN - 1 > wq_lo) || (window > 0 && wq_hi - kbase >= window);
      const uint16_t *Kt = smem + 2 * buf * C::TSZ;
      const uint16_t *Vt = Kt + C::TSZ;
      const int rel0 = my_q - kbase - 8 * h;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        f32x16 s = f32x16{}, dp = f32x16{};
        const int row = sb * 32 + ln;
        bf16x8 ka[C::KST], va[C::KST];
#pragma unroll
        for (int st = 0; st < C::KST; ++st) {
          ka[st] = lds_read_b128(Kt + dt_off<C::BN>(row, 2 * st + h));
          va[st] = lds_read_b128(Vt + dt_off<C::BN>(row, 2 * st + h));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < C::KST; ++st) {
          s = mfma32(ka[st], qr[st], s);
          dp = mfma32(va[st], gr[st], dp);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = fast_exp2(fmaf(s[i], c, -l2));
          // register i holds key kbase + sb*32 + c_row(i, h) = kbase + 8h + sb*32 + c_row(i, 0)
          if (need_mask) p = (unsigned)(rel0 - sb * 32 - c_row(i, 0)) <= wm1 ? p : 0.f;
          s[i] = p * (dp[i] - dl);
        }
        bf16x8 kt_op[2][C::NDB];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int d = 0; d < C::NDB; ++d) kt_op[t][d] = dt_read_tr_perm<C::BN>(Kt, sb * 32 + 16 * t, d, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 dsb = to_bf16x8(s, 8 * t);
#pragma unroll
          for (int d = 0; d < C::NDB; ++d) acc[d] = mfma32(kt_op[t][d], dsb, acc[d]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (my_q < T) {
    uint16_t *dqb = dq + base;
#pragma unroll
    for (int d = 0; d < C::NDB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 pk;
        pk[0] = (uint32_t)f32_to_bf16_bits(acc[d][4 * g] * scale) |
                ((uint32_t)f32_to_bf16_bits(acc[d][4 * g + 1] * scale) << 16);
        pk[1] = (uint32_t)f32_to_bf16_bits(acc[d][4 * g + 2] * scale) |
                ((uint32_t)f32_to_bf16_bits(acc[d][4 * g + 3] * scale) << 16);
        *reinterpret_cast<u32x2 *>(dqb + (size_t)my_q * rs + 32 * d + 8 * g + 4 * h) = pk;
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

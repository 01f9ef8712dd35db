// Backward of causal sliding-window attention, bf16 in / bf16 out, fp32 accumulate:
// the delta preprocess and the dQ pass (the dK/dV pass is in dkdv_bf16.hip).
//
// Gradients of L = sum_i dO_i . o_i for the attention of the nanochat guide's
// section 5 (the training step back-propagates through it).  With P recomputed
// from the stored LSE:
//   delta_i = dO_i . o_i                       (bwd_pre kernel, or the dq kernel itself)
//   dV = P^T dO,  dK = scale * dS^T Q           (dkdv kernel, one pass per key block)
//   dQ = scale * dS K                           (dq kernel, one pass per query block)
//   with dP = dO V^T and dS = P * (dP - delta).
// The two passes each recompute S and dP, so no atomics are needed and the
// results are bitwise reproducible.
//
// Inside the dQ pass S^T = K Q^T is formed with one query per lane (as in the
// forward) and dS^T feeds dQ^T = K^T dS^T; K^T comes from transposed LDS reads.
// The dQ pass computes delta for its own queries from o and dO (rows it reads
// anyway) and writes it to the workspace, so in the full backward it runs first
// and the dK/dV pass reads delta from there: no separate preprocess launch.
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
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ o,
    const uint16_t *__restrict__ dO, const float *__restrict__ lse, float *__restrict__ delta,
    uint16_t *__restrict__ dq, int B, int H, int T, int window, float scale, int nqt) {
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

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, held in an SGPR
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
  // delta = dO . o of the lane's query (each half of the wave holds half of the
  // row), also published in the workspace for the dK/dV pass
  float dl;
  {
    const int row = min(my_q, T - 1);
    float part = 0.f;
#pragma unroll
    for (int st = 0; st < C::KST; ++st) {
      const u32x4 ov = *reinterpret_cast<const u32x4 *>(o + base + (size_t)row * rs + 16 * st + 8 * h);
      const u32x4 gv = __builtin_bit_cast(u32x4, gr[st]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        part += bf16_lo(ov[e]) * bf16_lo(gv[e]) + bf16_hi(ov[e]) * bf16_hi(gv[e]);
    }
    dl = xhalf_sum(part);
    if (my_q < T && h == 0) delta[(size_t)bh * T + my_q] = dl;
  }
  const float c = scale * kLog2e;

  f32x16 acc[C::NDB];
#pragma unroll
  for (int d = 0; d < C::NDB; ++d) acc[d] = f32x16{};

  // K and V tiles (rows in swap23 order, d-block-major; rows past T read as zero
  // and are masked) by buffer -> LDS copies.  Piece j (1 KB): tensor j / (4 NDB),
  // LDS block db = (j % (4 NDB)) / 4, rows 16 (j % 4) .. + 15.
  const int rl = lane >> 2;
  const int lc = (lane & 3) ^ ((lane >> 4) & 3);  // logical chunk stored at this position
  const uint32_t lane_off = (swap23(rl) * rs + 8 * lc) * 2;
  auto issue_tile = [&](int kt, int buf) {
    const int row0 = kt * C::BN;
    const uint32_t nbytes = (uint32_t)(T - row0) * rs * 2;
#pragma unroll
    for (int cc = 0; cc < C::CPW; ++cc) {
      const int j = w * C::CPW + cc;
      const int tensor = j / (4 * C::NDB), jj = j % (4 * C::NDB);
      const int db = jj >> 2, row16 = 16 * (jj & 3);
      const __amdgpu_buffer_rsrc_t r = make_rsrc((tensor ? vb : kb) + (size_t)row0 * rs, nbytes);
      buf_copy16_to_lds(r, smem + (2 * buf + tensor) * C::TSZ + db * (C::BN * 32) + row16 * 32,
                        lane_off + (row16 * rs + 32 * db) * 2);
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
        // K^T operands: one asm block, so the copies of the next tile stay in flight
        bf16x8 kt_op[2][C::NDB];
        dt_read_tr_perm_block<C::BN, C::NDB>(Kt, sb * 32, lane, kt_op);
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

hipError_t launch_bwd_dq_bf16(const void *q, const void *k, const void *v, const void *o,
                              const void *dO, const float *lse, float *delta, void *dq, int B,
                              int H, int T, int D, int window, float scale, hipStream_t st) {
  const int nqt = (T + 127) / 128;
  const unsigned nb = (unsigned)(nqt * B * H);
  if (D == 128)
    bwd_dq_bf16_kernel<128><<<nb, 256, 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)o,
        (const uint16_t *)dO, lse, delta, (uint16_t *)dq, B, H, T, window, scale, nqt);
  else
    bwd_dq_bf16_kernel<64><<<nb, 256, 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)o,
        (const uint16_t *)dO, lse, delta, (uint16_t *)dq, B, H, T, window, scale, nqt);
  return hipGetLastError();
}

}  // namespace swattn

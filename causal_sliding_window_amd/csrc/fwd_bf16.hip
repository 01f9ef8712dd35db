// Forward of causal sliding-window attention, bf16 in / bf16 out, fp32 accumulate.
//
// Computes o = softmax(scale * Q K^T, causal + window mask) V and the natural-log
// LSE per query row: the attention call of the nanochat guide's section 5 ("Flash
// Attention unification") with the sliding window of its section 1 feature list.
//
// Work decomposition (one workgroup = 4 waves = 128 queries of one (b, h)):
//   * each wave owns 32 queries; its Q block stays in registers as the MFMA
//     B operand for S^T = K Q^T (32 keys x 32 queries per MFMA tile);
//   * K and V tiles of 64 keys are staged in LDS, double buffered, loaded with
//     16-byte coalesced global reads; only tiles that intersect the workgroup's
//     causal/window band are visited, and a wave skips tiles outside its own band;
//   * S^T lands with one query per lane, so the online-softmax row statistics are
//     per lane (plus one cross-half exchange), and P^T feeds O^T = V^T P^T as the
//     B operand straight from registers (the K rows are stored in swap23 order so
//     the C and B register orders coincide); V^T comes from transposed LDS reads;
//   * the element mask is applied only on tiles crossing the diagonal or the
//     window's lower edge.
#include "common.h"
#include "launch.h"

namespace swattn {

template <int D>
struct FwdCfg {
  static constexpr int BM = 128;          // queries per workgroup
  static constexpr int BN = 64;           // keys per LDS tile
  static constexpr int NT = 256;          // threads
  static constexpr int KLD = D + 8;       // K tile pitch (elements): b128 reads conflict free
  static constexpr int VLD = D + 32;      // V tile pitch: transposed reads conflict free
  static constexpr int KSZ = BN * KLD;
  static constexpr int VSZ = BN * VLD;
  static constexpr int CPR = D / 8;       // 16-byte chunks per row
  static constexpr int RPP = NT / CPR;    // rows per load pass
  static constexpr int PASSES = BN / RPP;
};

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, uint16_t *__restrict__ o, float *__restrict__ lse,
    int B, int H, int T, int window, float scale, int nqt) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2 * C::KSZ];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2 * C::VSZ];

  const int BH = B * H;
  const int bid = blockIdx.x;
  const int qt = nqt - 1 - bid / BH;  // longest (latest) query tiles first
  const int bh = bid % BH;            // consecutive blocks: different heads
  const int b = bh / H, hh = bh % H;
  const int q0 = qt * C::BM;
  const size_t rs = (size_t)H * D;
  const size_t base = ((size_t)b * T * H + hh) * D;
  const uint16_t *qb = q + base, *kb = k + base, *vb = v + base;
  uint16_t *ob = o + base;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int h = lane >> 5, ln = lane & 31;
  const int qw0 = q0 + 32 * w;
  const int my_q = qw0 + ln;

  const int q_last = min(T, q0 + C::BM) - 1;
  const int k_lo = window > 0 ? max(0, q0 - window + 1) : 0;
  const int kt0 = k_lo / C::BN, kt1 = q_last / C::BN;

  const int wq_lo = qw0, wq_hi = min(T - 1, qw0 + 31);
  const int wk_lo = window > 0 ? wq_lo - window + 1 : 0;

  bf16x8 qr[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    if (my_q < T) qr[st] = *reinterpret_cast<const bf16x8 *>(qb + my_q * rs + 16 * st + 8 * h);
    else qr[st] = bf16x8{};
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) acc[d] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = scale * kLog2e;

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
      const int rk = (r & ~31) | swap23(r & 31);
      *reinterpret_cast<u32x4 *>(Ks + buf * C::KSZ + rk * C::KLD + lch * 8) = kreg[p];
      *reinterpret_cast<u32x4 *>(Vs + buf * C::VSZ + r * C::VLD + lch * 8) = vreg[p];
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
      const uint16_t *Vt = Vs + buf * C::VSZ;
      f32x16 s[2];
      {
        bf16x8 ka[2][D / 16];  // all K operands requested before the first MFMA
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int st = 0; st < D / 16; ++st)
            ka[sb][st] = lds_read_b128(Kt + (sb * 32 + ln) * C::KLD + 8 * h + 16 * st);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int st = 0; st < D / 16; ++st)
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) {
            if (st == 0) s[sb] = f32x16{};
            s[sb] = mfma32(ka[sb][st], qr[st], s[sb]);
          }
      }
      if (need_mask) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kbase + sb * 32 + c_row(i, h);
            const bool vis = key <= my_q && (window < 0 || my_q - key < window);
            if (!vis) s[sb][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sb][i]);
      mx = xhalf_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float mc = (m_new == -INFINITY ? 0.f : m_new) * c;
      const float alpha = fast_exp2(m_run * c - mc);
      float psum = 0.f;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(s[sb][i], c, -mc));
          s[sb][i] = p;
          psum += p;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int d = 0; d < D / 32; ++d) acc[d] *= alpha;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        bf16x8 va[2][D / 32];  // V^T operands of this 32-key block, requested up front
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int d = 0; d < D / 32; ++d)
            va[t][d] = lds_read_tr_block(Vt + (sb * 32 + 16 * t) * C::VLD + 32 * d, C::VLD, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 pb = to_bf16x8(s[sb], 8 * t);
#pragma unroll
          for (int d = 0; d < D / 32; ++d) acc[d] = mfma32(va[t][d], pb, acc[d]);
        }
      }
    }
    if (kt < kt1) sstore(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = xhalf_sum(l_run);
  if (my_q < T) {
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 pk;
        pk[0] = (uint32_t)f32_to_bf16_bits(acc[d][4 * g] * inv) |
                ((uint32_t)f32_to_bf16_bits(acc[d][4 * g + 1] * inv) << 16);
        pk[1] = (uint32_t)f32_to_bf16_bits(acc[d][4 * g + 2] * inv) |
                ((uint32_t)f32_to_bf16_bits(acc[d][4 * g + 3] * inv) << 16);
        *reinterpret_cast<u32x2 *>(ob + my_q * rs + 32 * d + 8 * g + 4 * h) = pk;
      }
    if (h == 0) lse[(size_t)bh * T + my_q] = m_run * scale + logf(l_tot);
  }
}

hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse,
                           int B, int H, int T, int D, int window, float scale, hipStream_t st) {
  const int nqt = (T + 127) / 128;
  dim3 grid((unsigned)(nqt * B * H)), block(256);
  if (D == 128)
    fwd_bf16_kernel<128><<<grid, block, 0, st>>>((const uint16_t *)q, (const uint16_t *)k,
                                                 (const uint16_t *)v, (uint16_t *)o, lse, B, H,
                                                 T, window, scale, nqt);
  else
    fwd_bf16_kernel<64><<<grid, block, 0, st>>>((const uint16_t *)q, (const uint16_t *)k,
                                                (const uint16_t *)v, (uint16_t *)o, lse, B, H, T,
                                                window, scale, nqt);
  return hipGetLastError();
}

}  // namespace swattn

// dK, dV of causal sliding-window attention, bf16 in / bf16 out, fp32 accumulate
// (the dK/dV pass of the backward; see bwd_bf16.hip for the delta preprocess and
// the dQ pass).  Gradients of L = sum_i dO_i . o_i for the attention of the
// nanochat guide's section 5, with P recomputed from the stored LSE:
//   dV = P^T dO,  dK = scale * dS^T Q,  dS = P * (dP - delta),  dP = dO V^T.
//
// One workgroup = 4 waves x 32 keys of one (b, h).  Each wave keeps its K and V
// rows in registers as MFMA B operands; S = Q K^T and dP = dO V^T are formed with
// one key per lane, so P and dS feed dV^T = dO^T P and dK^T = Q^T dS as B
// operands straight from registers; dO^T and Q^T come from transposed LDS reads.
// Query tiles of 32 rows reach LDS by direct buffer -> LDS copies (four slots,
// issued three tiles ahead, each step waiting only for the tile it needs next);
// each step overlaps the S / dP MFMAs of the next tile with the gradient-side ALU
// work of the current one.
//
// Built without -amdgpu-mfma-vgpr-form: the dK / dV accumulators stay in AGPRs,
// which leaves the arch VGPRs to the operands.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace swattn {

// ---------------------------------------------------------------- dK, dV
template <int D>
struct DkdvCfg {
  static constexpr int BK = 128;          // keys per workgroup (4 waves x 32)
  static constexpr int BQ = 32;           // queries per tile
  static constexpr int NSLOT = 4;         // LDS tile slots (tile t in slot t % 4)
  static constexpr int AHEAD = NSLOT - 1; // tiles are copied this many steps ahead
  static constexpr int TSZ = BQ * D;      // elements of one Q (or dO) tile
  static constexpr int NDB = D / 32;
  static constexpr int KST = D / 16;
  static constexpr int HALF = TSZ * 2 / 1024;  // 1-KB pieces of one tensor's tile
  static constexpr int CPW = 2 * HALF / 4;     // pieces per wave and tile (Q and dO)
  static constexpr int RG = BQ / 16;           // 16-row groups per 32-column block
  static constexpr int NCOPY = CPW + 1;        // copies per wave and tile (+ lse/delta)
};

// s_waitcnt immediate: at most N vector-memory operations of the wave in flight,
// all LDS operations done, exports not waited for.
template <int N>
constexpr int kWaitVm = (N & 15) | ((N >> 4) << 14) | (7 << 4);

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ dO,
    const float *__restrict__ lse, const float *__restrict__ delta, uint16_t *__restrict__ dk,
    uint16_t *__restrict__ dv, int B, int H, int T, int window, float scale, int nkt) {
  using C = DkdvCfg<D>;
  // One LDS array (with a single __shared__ variable the compiler keeps the restrict
  // scopes below): [slot][Q, dO][TSZ] bf16, then [slot][lse, delta, spare, spare][64]
  // float.
  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::NSLOT * 2 * C::TSZ +
                                                          C::NSLOT * 4 * 64 * 2];
  float *const vec = reinterpret_cast<float *>(smem + C::NSLOT * 2 * C::TSZ);

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

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, held in an SGPR
  const int h = lane >> 5, ln = lane & 31;
  const int kw0 = k0 + 32 * w;
  const int my_k = kw0 + ln;

  // query tiles of the workgroup and of this wave (a wave's keys kw0 .. kw0 + 31 are
  // seen by queries kw0 .. kw0 + 31 + W - 1)
  const int k_last = min(T, k0 + C::BK) - 1;
  const int q_hi = window > 0 ? min(T - 1, k_last + window - 1) : T - 1;
  const int qt0 = k0 / C::BQ, qt1 = q_hi / C::BQ;
  int wqt0 = 1 << 30, wqt1 = -1;
  if (kw0 < T) {
    wqt0 = kw0 / C::BQ;
    wqt1 = (window > 0 ? min(T - 1, kw0 + 31 + window - 1) : T - 1) / C::BQ;
  }
  // tiles from mlo on hold a query past some key's window
  const int mlo = window > 0 ? (kw0 + window - 31 + C::BQ - 1) / C::BQ : (1 << 30);
  // query qq sees key my_k iff 0 <= qq - my_k <= wm1
  const unsigned wm1 = window > 0 ? (unsigned)(window - 1) : 0x7fffffffu;

  // K and V rows of the wave's keys (B operands), rows past T read as zero
  bf16x8 kr[C::KST], vr[C::KST];
  {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (uint32_t)T * rs * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (uint32_t)T * rs * 2);
#pragma unroll
    for (int st = 0; st < C::KST; ++st) {
      const uint32_t off = (my_k * rs + 16 * st + 8 * h) * 2;
      kr[st] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
      vr[st] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
    // landed before any tile copy is issued: later waits then only count copies
    __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
    __builtin_amdgcn_sched_barrier(0);
  }
  f32x16 dka[C::NDB], dva[C::NDB];
#pragma unroll
  for (int d = 0; d < C::NDB; ++d) {
    dka[d] = f32x16{};
    dva[d] = f32x16{};
  }
  const float c = scale * kLog2e;

  // Copies of a Q and dO tile (rows in swap23 order, d-block-major, rows past T read
  // as zero) and of its lse / delta (past T: zero; a zero Q and dO row adds nothing
  // to dK and dV whatever its p).  Piece j: tensor j / HALF, LDS block
  // db = (j % HALF) / RG, rows 16 ((j % HALF) % RG) .. + 15.
  const int rl = lane >> 2;
  const int lc = (lane & 3) ^ ((lane >> 4) & 3);  // logical chunk stored at this position
  const uint32_t lane_off = (swap23(rl) * rs + 8 * lc) * 2;
  auto issue_to = [&](int qt, uint16_t *tile, float *vdst) {
    const int row0 = qt * C::BQ;
    const uint32_t nbytes = (uint32_t)(T - row0) * rs * 2;
#pragma unroll
    for (int cc = 0; cc < C::CPW; ++cc) {
      const int j = w * C::CPW + cc;
      const int tensor = j / C::HALF, jj = j % C::HALF;
      const int db = jj / C::RG, row16 = 16 * (jj % C::RG);
      const __amdgpu_buffer_rsrc_t r = make_rsrc((tensor ? gb : qb) + (size_t)row0 * rs, nbytes);
      buf_copy16_to_lds(r, tile + tensor * C::TSZ + db * (C::BQ * 32) + row16 * 32,
                        lane_off + (row16 * rs + 32 * db) * 2);
    }
    // every wave issues exactly NCOPY copies per tile (waves 2 and 3 fill spare
    // rows), so the end-of-step wait can count them
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(((w & 1) ? delb : lseb) + row0, (uint32_t)(T - row0) * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void *)(vdst + w * 64), 4, lane * 4, 0, 0, 0);
  };
  auto q_tile = [&](int qt) { return smem + 2 * (qt % C::NSLOT) * C::TSZ; };
  auto vec_of = [&](int qt) { return vec + 4 * (qt % C::NSLOT) * 64; };
  auto issue = [&](int qt) { issue_to(qt, q_tile(qt), vec_of(qt)); };

  // S = Q K^T and dP = dO V^T of a tile, one key per lane: register 8t + j of half
  // h holds query 16t + 8h + j of the tile.
  auto sdp = [&](int qt, f32x16 &s, f32x16 &dp) {
    const uint16_t *Qt = q_tile(qt), *Gt = Qt + C::TSZ;
    bf16x8 qa[C::KST], ga[C::KST];
#pragma unroll
    for (int st = 0; st < C::KST; ++st) {
      qa[st] = lds_read_b128(Qt + dt_off<C::BQ>(ln, 2 * st + h));
      ga[st] = lds_read_b128(Gt + dt_off<C::BQ>(ln, 2 * st + h));
    }
#pragma unroll
    for (int st = 0; st < C::KST; ++st) {
      s = mfma32(qa[st], kr[st], st ? s : f32x16{});
      dp = mfma32(ga[st], vr[st], st ? dp : f32x16{});
    }
  };

  // Transposed operands of dV^T += dO^T P and dK^T += Q^T dS for a tile, by the
  // asm block that waits only for its own LDS reads (copies stay in flight).
  using TOps = bf16x8[2][C::NDB];
  auto tr_reads = [&](const uint16_t *Qt, TOps &gt, TOps &qtr) {
    const uint16_t *Gt = Qt + C::TSZ;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int d = 0; d < C::NDB; ++d) {
        gt[t][d] = dt_read_tr_perm<C::BQ>(Gt, 16 * t, d, lane);
        qtr[t][d] = dt_read_tr_perm<C::BQ>(Qt, 16 * t, d, lane);
      }
  };

  // P = exp(S - LSE) and dS = P (dP - delta) for elements [e0, e0 + n) of a tile.
  auto grad_elems = [&](auto mask_tag, f32x16 &s, f32x16 &dp, const f32x4 (&L)[4],
                        const f32x4 (&Dl)[4], int rel0, int e0, int n) {
    constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
    for (int i = e0; i < e0 + n; ++i) {
      const int t = i >> 3, j = i & 7;
      const float lj = L[2 * t + (j >> 2)][j & 3] * kLog2e;
      const float dj = Dl[2 * t + (j >> 2)][j & 3];
      float p = fast_exp2(fmaf(s[i], c, -lj));
      if (MASK) p = (unsigned)(rel0 + 16 * t + j) <= wm1 ? p : 0.f;
      s[i] = p;
      dp[i] = p * (dp[i] - dj);
    }
  };
  // P enters dV as bf16 hi + lo (P = hi + lo to ~16 bits): a single bf16 P leaves
  // |dV| >= 4 outside 2e-2 of the exact gradient.
  auto pack = [&](const f32x16 &s, const f32x16 &dp, int t, bf16x8 &ph, bf16x8 &pl,
                  bf16x8 &ds) {
    ph = to_bf16x8(s, 8 * t);
#pragma unroll
    for (int j = 0; j < 8; ++j) pl[j] = (__bf16)(s[8 * t + j] - (float)ph[j]);
    ds = to_bf16x8(dp, 8 * t);
  };
  auto grads = [&](const TOps &gt, const TOps &qtr, int t, const bf16x8 &ph, const bf16x8 &pl,
                   const bf16x8 &ds) {
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) {
      dva[d] = mfma32(gt[t][d], ph, dva[d]);
      dva[d] = mfma32(gt[t][d], pl, dva[d]);
      dka[d] = mfma32(qtr[t][d], ds, dka[d]);
    }
  };
  auto read_vecs = [&](const float *vl, f32x4 (&L)[4], f32x4 (&Dl)[4]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        L[2 * t + u] = *reinterpret_cast<const f32x4 *>(vl + 16 * t + 8 * h + 4 * u);
        Dl[2 * t + u] = *reinterpret_cast<const f32x4 *>(vl + 64 + 16 * t + 8 * h + 4 * u);
      }
  };

  auto pin = [](float x) {
    asm volatile("" ::"v"(x));
    __builtin_amdgcn_sched_barrier(0);
  };

  // One pipeline step for tile qt (S, dP in sc, dpc).  The copies of tile
  // qt + AHEAD start first; the operands of tile qt + 1's S / dP MFMAs and tile qt's
  // lse / delta are read; the S / dP MFMAs of tile qt + 1 (when NEXT) are issued
  // one pair at a time between the slices of the gradient-side ALU work of tile qt;
  // then tile qt's transposed operands are read and its dV / dK MFMAs close the
  // step.  The tiles come in as distinct restrict pointers: with that, the compiler
  // knows the reads do not touch the tiles being copied and does not make them wait
  // for the copies in flight (the copies a step reads were awaited at the barrier
  // before it).
  auto step_body = [&](auto mask_tag, auto next_tag, int qt, f32x16 &sc, f32x16 &dpc,
                       f32x16 &sn, f32x16 &dpn, const uint16_t *__restrict__ cur,
                       const uint16_t *__restrict__ nxt, const float *__restrict__ vcur,
                       uint16_t *__restrict__ dma, float *__restrict__ vdma) {
    constexpr bool NEXT = decltype(next_tag)::value;
    if (qt + C::AHEAD <= qt1) issue_to(qt + C::AHEAD, dma, vdma);
    const int rel0 = qt * C::BQ + 8 * h - my_k;
    bf16x8 qa[C::KST], ga[C::KST];
    if constexpr (NEXT) {
      const uint16_t *Gn = nxt + C::TSZ;
#pragma unroll
      for (int st = 0; st < C::KST; ++st) {
        qa[st] = lds_read_b128(nxt + dt_off<C::BQ>(ln, 2 * st + h));
        ga[st] = lds_read_b128(Gn + dt_off<C::BQ>(ln, 2 * st + h));
      }
    }
    f32x4 L[4], Dl[4];
    read_vecs(vcur, L, Dl);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NEXT) {
      constexpr int EPS = 16 / C::KST;  // elements per slice
#pragma unroll
      for (int st = 0; st < C::KST; ++st) {
        sn = mfma32(qa[st], kr[st], st ? sn : f32x16{});
        dpn = mfma32(ga[st], vr[st], st ? dpn : f32x16{});
        __builtin_amdgcn_sched_barrier(0);
        grad_elems(mask_tag, sc, dpc, L, Dl, rel0, EPS * st, EPS);
        pin(dpc[EPS * st + EPS - 1]);
      }
    } else {
      grad_elems(mask_tag, sc, dpc, L, Dl, rel0, 0, 16);
    }
    TOps gt, qtr;
    tr_reads(cur, gt, qtr);
    bf16x8 ph0, pl0, ds0, ph1, pl1, ds1;
    pack(sc, dpc, 0, ph0, pl0, ds0);
    __builtin_amdgcn_sched_barrier(0);
    grads(gt, qtr, 0, ph0, pl0, ds0);
    pack(sc, dpc, 1, ph1, pl1, ds1);
    grads(gt, qtr, 1, ph1, pl1, ds1);
  };
  auto step = [&](auto mask_tag, auto next_tag, int qt, f32x16 &sc, f32x16 &dpc, f32x16 &sn,
                  f32x16 &dpn) {
    step_body(mask_tag, next_tag, qt, sc, dpc, sn, dpn, q_tile(qt), q_tile(qt + 1), vec_of(qt),
              q_tile(qt + C::AHEAD), vec_of(qt + C::AHEAD));
  };
  // End of step qt: the tile needed next (copied a step earlier) must have landed;
  // the copies this step issued (tile qt + AHEAD) may stay in flight.
  auto sync = [&](int qt) {
    if (qt + C::AHEAD <= qt1) __builtin_amdgcn_s_waitcnt(kWaitVm<C::NCOPY>);
    else __builtin_amdgcn_s_waitcnt(kWaitVm<0>);
    lds_barrier();
  };

  // prologue: tiles qt0 .. qt0 + AHEAD - 1; all but the last must have landed
  for (int t = qt0; t < qt0 + C::AHEAD && t <= qt1; ++t) issue(t);
  sync(qt0 - 1);
  f32x16 sc, dpc, sn, dpn;
  if (wqt0 == qt0) sdp(qt0, sc, dpc);

  // Phases of the wave: idle tiles, S / dP of its first tile, the diagonal tile
  // (masked), unmasked tiles, tiles crossing the window's far edge (masked), the
  // last tile (no S / dP ahead), idle tiles.  One barrier per tile of the
  // workgroup in every phase.
  int qt = qt0;
  for (; qt < min(wqt0 - 1, qt1 + 1); ++qt) {
    if (qt + C::AHEAD <= qt1) issue(qt + C::AHEAD);
    sync(qt);
  }
  if (wqt0 > qt0 && qt == wqt0 - 1) {
    if (qt + C::AHEAD <= qt1) issue(qt + C::AHEAD);
    sdp(qt + 1, sc, dpc);
    sync(qt);
    ++qt;
  }
  auto advance = [&] {
    sc = sn;
    dpc = dpn;
  };
  if (qt == wqt0 && qt < wqt1) {  // diagonal tile
    step(std::true_type{}, std::true_type{}, qt, sc, dpc, sn, dpn);
    advance();
    sync(qt);
    ++qt;
  }
  for (; qt < min(wqt1, mlo); ++qt) {
    step(std::false_type{}, std::true_type{}, qt, sc, dpc, sn, dpn);
    advance();
    sync(qt);
  }
  for (; qt < wqt1; ++qt) {
    step(std::true_type{}, std::true_type{}, qt, sc, dpc, sn, dpn);
    advance();
    sync(qt);
  }
  if (qt == wqt1) {
    step(std::true_type{}, std::false_type{}, qt, sc, dpc, sn, dpn);
    sync(qt);
    ++qt;
  }
  for (; qt <= qt1; ++qt) {
    if (qt + C::AHEAD <= qt1) issue(qt + C::AHEAD);
    sync(qt);
  }

  if (my_k < T) {
    uint16_t *dkb = dk + base + (size_t)my_k * rs, *dvb = dv + base + (size_t)my_k * rs;
#pragma unroll
    for (int d = 0; d < C::NDB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 pk, pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pk[e] = (__bf16)(dka[d][4 * g + e] * scale);
          pv[e] = (__bf16)dva[d][4 * g + e];
        }
        *reinterpret_cast<bf16x4 *>(dkb + 32 * d + 8 * g + 4 * h) = pk;
        *reinterpret_cast<bf16x4 *>(dvb + 32 * d + 8 * g + 4 * h) = pv;
      }
  }
}

hipError_t launch_bwd_dkdv_bf16(const void *q, const void *k, const void *v, const void *dO,
                                const float *lse, const float *delta, void *dk, void *dv, int B,
                                int H, int T, int D, int window, float scale, hipStream_t st) {
  const int nkt = (T + DkdvCfg<128>::BK - 1) / DkdvCfg<128>::BK;
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

}  // namespace swattn

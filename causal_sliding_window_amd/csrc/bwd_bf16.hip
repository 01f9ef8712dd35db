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
#include "rope.h"

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
  static constexpr int BN = 32;           // keys per tile
  static constexpr int NSLOT = 4;         // LDS tile slots (tile t in slot t % 4)
  static constexpr int AHEAD = 3;         // tiles are copied this many steps ahead
  static constexpr int TSZ = BN * D;      // elements of one K (or V) tile
  static constexpr int NDB = D / 32;
  static constexpr int KST = D / 16;
  static constexpr int HALF = TSZ * 2 / 1024;  // 1-KB pieces of one tensor's tile
  static constexpr int CPW = 2 * HALF / 4;     // pieces per wave and tile (K and V)
  static constexpr int RG = BN / 16;           // 16-row groups per 32-column block
};

// Largest |dS| of a tile (any lane) from which dS enters dQ as bf16 hi + lo, and the
// head sizes that take that path.  At D = 128 the kernel holds 254 of its 256 VGPRs
// and every arrangement of the lo products tried spills, so there dS always enters as
// one bf16 (the D = 128 sweeps meet the bar with it).
constexpr float kLoDs = 1.0f;
template <int D>
constexpr bool kDsLo = D == 64;

// ROPE: q holds the raw queries (k the transformed keys); each query is normalised and
// rotated (QK norm + rotary embedding) as it is loaded, and dq is the gradient with
// respect to the raw query: the epilogue maps dL/dq' back through the prologue.
template <int D, bool ROPE = false>
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ o,
    const uint16_t *__restrict__ dO, const float *__restrict__ lse, float *__restrict__ delta,
    uint16_t *__restrict__ dq, int B, int H, int Hkv, int T, int window, float scale, int nqt,
    RopeArgs ra = RopeArgs{}) {
  using C = DqCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::NSLOT * 2 * C::TSZ];  // [slot][K, V]

  const int BH = B * H;
  const int bid = blockIdx.x;
  const int qt = nqt - 1 - bid / BH;  // longest (latest) query blocks first
  const int bh = bid % BH;
  const int b = bh / H, hh = bh % H;
  const int q0 = qt * C::BM;
  const int rs = H * D;                // row stride of q, o, dO and dq
  const int rsk = Hkv * D;             // row stride of k and v
  const int hk = hh / (H / Hkv);       // the K/V head of query head hh
  const size_t base = ((size_t)b * T * H + hh) * D;
  const size_t base_kv = ((size_t)b * T * Hkv + hk) * D;
  const uint16_t *qb = q + base, *kb = k + base_kv, *vb = v + base_kv, *gb = dO + base;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, held in an SGPR
  const int h = lane >> 5, ln = lane & 31;
  const int qw0 = q0 + 32 * w;
  const int my_q = qw0 + ln;

  // key tiles of the workgroup and of this wave
  const int q_last = min(T, q0 + C::BM) - 1;
  const int k_lo = window > 0 ? max(0, q0 - window + 1) : 0;
  const int kt0 = k_lo / C::BN, kt1 = q_last / C::BN;
  int wkt0 = 1 << 30, wkt1 = -1;
  if (qw0 < T) {
    wkt0 = (window > 0 ? max(0, qw0 - window + 1) : 0) / C::BN;
    wkt1 = min(T - 1, qw0 + 31) / C::BN;
  }
  const int wq_hi = min(T - 1, qw0 + 31);
  // key kk is visible to my_q iff 0 <= my_q - kk <= wm1
  const unsigned wm1 = window > 0 ? (unsigned)(window - 1) : 0x7fffffffu;

  // Q and dO rows of the lane's query (B operands), rows past T read as zero
  bf16x8 qr[C::KST], gr[C::KST];
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (uint32_t)T * rs * 2);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(gb, (uint32_t)T * rs * 2);
#pragma unroll
  for (int st = 0; st < C::KST; ++st) {
    const uint32_t off = (my_q * rs + 16 * st + 8 * h) * 2;
    qr[st] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
    gr[st] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0));
  }
  const float l2 = my_q < T ? lse[(size_t)bh * T + my_q] * kLog2e : INFINITY;
  // delta = dO . o of the lane's query (each half of the wave holds half of the
  // row), also published in the workspace for the dK/dV pass
  // (its o row is loaded here and used once the prologue's tile copies are issued, so
  // that the two waits overlap)
  u32x4 orow[C::KST];
  {
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(o + base, (uint32_t)T * rs * 2);
#pragma unroll
    for (int st = 0; st < C::KST; ++st)
      orow[st] =
          __builtin_amdgcn_raw_buffer_load_b128(ro, (my_q * rs + 16 * st + 8 * h) * 2, 0, 0);
  }
  float dl = 0.f;  // delta of the lane's query, set in the prologue below
  const float c = scale * kLog2e;

  f32x16 acc[C::NDB];
#pragma unroll
  for (int d = 0; d < C::NDB; ++d) acc[d] = f32x16{};

  // K and V tiles (rows in swap23 order, d-block-major; rows past T read as zero
  // and are masked) by buffer -> LDS copies.  Piece j (1 KB): tensor j / HALF, LDS
  // block db = (j % HALF) / RG, rows 16 ((j % HALF) % RG) .. + 15.
  const int rl = lane >> 2;
  const int lc = (lane & 3) ^ ((lane >> 4) & 3);  // logical chunk stored at this position
  const uint32_t lane_off = (swap23(rl) * rsk + 8 * lc) * 2;
  // One buffer resource per tensor over all T rows of this (b, K/V head): a tile's
  // row offset goes into the lane offsets, and offsets from row T on read as zero.
  const int my_tensor = (w * C::CPW) / C::HALF;  // every copy of a wave is K (0) or V (1)
  const __amdgpu_buffer_rsrc_t rsrc_t = make_rsrc(my_tensor ? vb : kb, (uint32_t)T * rsk * 2);
  // Tiles past the workgroup's last one (issued so that every step waits for the same
  // count) are copied from row T on: the buffer returns zeros and reads no memory.
  auto issue_to = [&](int kt, uint16_t *tile) {
    const uint32_t roff = (uint32_t)(kt <= kt1 ? kt * C::BN : T) * (uint32_t)rsk * 2;
#pragma unroll
    for (int cc = 0; cc < C::CPW; ++cc) {
      const int jj = (w * C::CPW + cc) % C::HALF;
      const int db = jj / C::RG, row16 = 16 * (jj % C::RG);
      buf_copy16_to_lds(rsrc_t, tile + my_tensor * C::TSZ + db * (C::BN * 32) + row16 * 32,
                        lane_off + (uint32_t)(row16 * rsk + 32 * db) * 2 + roff);
    }
  };
  auto k_tile = [&](int kt) { return smem + 2 * (kt & (C::NSLOT - 1)) * C::TSZ; };
  auto issue = [&](int kt) { issue_to(kt, k_tile(kt)); };

  // S^T = K Q^T and dP^T = V dO^T of a tile, one query per lane: register i of half
  // h holds key c_row(i, h) of the tile.
  auto sdp = [&](int kt, f32x16 &s, f32x16 &dp) {
    const uint16_t *Kt = k_tile(kt), *Vt = Kt + C::TSZ;
    bf16x8 ka[C::KST], va[C::KST];
#pragma unroll
    for (int st = 0; st < C::KST; ++st) {
      ka[st] = lds_read_b128(Kt + dt_off<C::BN>(ln, 2 * st + h));
      va[st] = lds_read_b128(Vt + dt_off<C::BN>(ln, 2 * st + h));
    }
#pragma unroll
    for (int st = 0; st < C::KST; ++st) {
      s = mfma32(ka[st], qr[st], st ? s : f32x16{});
      dp = mfma32(va[st], gr[st], st ? dp : f32x16{});
    }
  };

  // dS = P (dP - delta) for elements [e0, e0 + n) of a tile (into dp); dm keeps the
  // largest |dS| of the lane (only where the lo path exists).
  auto ds_elems = [&](auto mask_tag, f32x16 &s, f32x16 &dp, float &dm, int rel0, int e0, int n) {
    constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
    for (int i = e0; i < e0 + n; ++i) {
      float p = fast_exp2(fmaf(s[i], c, -l2));
      if (MASK) p = (unsigned)(rel0 - c_row(i, 0)) <= wm1 ? p : 0.f;
      dp[i] = p * (dp[i] - dl);
    }
    if constexpr (kDsLo<D>) {
#pragma unroll
      for (int i = e0; i < e0 + n; i += 2) dm = fmaxf(dm, fmaxf(fabsf(dp[i]), fabsf(dp[i + 1])));
    }
  };
  // dQ^T += K^T dS^T for a tile (K^T by one asm block of transposed reads, so the
  // copies in flight are not waited for).  dS enters as one bf16 (nearest even) unless
  // some |dS| of the wave's tile reaches kLoDs (D = 64); then as hi + lo, hi = dS
  // rounded and lo = the remainder rounded (dS = hi + lo to ~2^-17 relative).  With one
  // bf16 dS everywhere, large |dS| (peaked rows) move |dq| ~ 4..8 by up to 0.02 against
  // the exact gradient together with the bf16 output's own half ulp.
  auto dq_from = [&](const bf16x8 (&kt_op)[2][C::NDB], const f32x16 &ds, float dm, int kt) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x8 dsb = to_bf16x8(ds, 8 * t);
#pragma unroll
      for (int d = 0; d < C::NDB; ++d) acc[d] = mfma32(kt_op[t][d], dsb, acc[d]);
    }
    if (kDsLo<D> && __builtin_amdgcn_ballot_w64(dm >= kLoDs) != 0) {
      // the K^T operands are read again (tile kt stays in LDS until the next step)
      bf16x8 kt_op2[2][C::NDB];
      dt_read_tr_perm_block<C::BN, C::NDB>(k_tile(kt), 0, lane, kt_op2);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        bf16x8 lo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float hi = (float)(__bf16)ds[8 * t + j];
          lo[j] = (__bf16)(ds[8 * t + j] - hi);
        }
#pragma unroll
        for (int d = 0; d < C::NDB; ++d) acc[d] = mfma32(kt_op2[t][d], lo, acc[d]);
      }
    }
  };
  auto dq_mfma = [&](int kt, const f32x16 &ds, float dm) {
    bf16x8 kt_op[2][C::NDB];
    dt_read_tr_perm_block<C::BN, C::NDB>(k_tile(kt), 0, lane, kt_op);
    dq_from(kt_op, ds, dm, kt);
  };
  auto pin = [](float x) {
    asm volatile("" ::"v"(x));
    __builtin_amdgcn_sched_barrier(0);
  };

  // One pipeline step for tile kt (S^T, dP^T in sc, dpc): the copies of tile kt + 3
  // start first; the S / dP MFMAs of tile kt + 1 are issued one pair at a time
  // between the slices of tile kt's dS work, the last slices also read tile kt's
  // K^T operands, then dQ += dS K for tile kt.  The tiles come in as distinct
  // restrict pointers: the compiler then knows the reads do not touch the tile
  // being copied and does not make them wait for the copies in flight.
  auto step_body = [&](auto mask_tag, int kt, f32x16 &sc, f32x16 &dpc, f32x16 &sn,
                       f32x16 &dpn, const uint16_t *__restrict__ Kc,
                       const uint16_t *__restrict__ Kn, uint16_t *__restrict__ dma)
                       __attribute__((always_inline)) {
    issue_to(kt + C::AHEAD, dma);
    const uint16_t *Vn = Kn + C::TSZ;
    // operands are read AHEAD slices before their MFMAs
    constexpr int AHEAD = 2;
    bf16x8 ka[C::KST], va[C::KST];
    auto read_ops = [&](int st) {
      ka[st] = lds_read_b128(Kn + dt_off<C::BN>(ln, 2 * st + h));
      va[st] = lds_read_b128(Vn + dt_off<C::BN>(ln, 2 * st + h));
    };
#pragma unroll
    for (int st = 0; st < AHEAD; ++st) read_ops(st);
    __builtin_amdgcn_sched_barrier(0);
    const int rel0 = my_q - kt * C::BN - 8 * h;
    constexpr int EPS = 16 / C::KST;  // elements per slice
    float dm = 0.f;
    bf16x8 kt_op[2][C::NDB];
    constexpr int TR0 = C::KST / 2;  // first slice with K^T reads (two operands each)
#pragma unroll
    for (int st = 0; st < C::KST; ++st) {
      if (st + AHEAD < C::KST) read_ops(st + AHEAD);
      if (st >= TR0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int kk = 2 * (st - TR0) + u;
          kt_op[kk / C::NDB][kk % C::NDB] = dt_read_tr_perm<C::BN>(Kc, 16 * (kk / C::NDB),
                                                                   kk % C::NDB, lane);
        }
      }
      sn = mfma32(ka[st], qr[st], st ? sn : f32x16{});
      dpn = mfma32(va[st], gr[st], st ? dpn : f32x16{});
      __builtin_amdgcn_sched_barrier(0);
      ds_elems(mask_tag, sc, dpc, dm, rel0, EPS * st, EPS);
      pin(dpc[EPS * st + EPS - 1]);
    }
    dq_from(kt_op, dpc, dm, kt);
  };
  auto step = [&](auto mask_tag, int kt, f32x16 &sc, f32x16 &dpc, f32x16 &sn, f32x16 &dpn)
      __attribute__((always_inline)) {
    step_body(mask_tag, kt, sc, dpc, sn, dpn, k_tile(kt), k_tile(kt + 1), k_tile(kt + C::AHEAD));
  };
  auto last_step = [&](int kt, f32x16 &sc, f32x16 &dpc) {
    issue(kt + C::AHEAD);
    float dm = 0.f;
    ds_elems(std::true_type{}, sc, dpc, dm, my_q - kt * C::BN - 8 * h, 0, 16);
    dq_mfma(kt, dpc, dm);
  };
  // End of step kt: tile kt + 2 (copied a step earlier) must have landed; the copies
  // of this step (tile kt + AHEAD) may stay in flight.  Before every step kt, tiles
  // up to kt + 1 have landed and are visible to all waves.  Every step issues its
  // copies, also past the workgroup's last tile (rows from T on read as zero and
  // land in slots no step reads), so the wait count is always the same.
  auto sync = [&] {
    __builtin_amdgcn_s_waitcnt(kWaitVm<C::CPW>);
    lds_barrier();
  };

  // prologue: tiles kt0 .. kt0 + 2 in flight, the first two must land; delta (and with
  // ROPE the query transform) while they are in flight
  issue(kt0);
  issue(kt0 + 1);
  issue(kt0 + 2);
  if constexpr (ROPE) rope_norm_operand<D>(qr, rope_pos(ra, b, my_q), my_q < T, ra, h);
  {
    float part = 0.f;
#pragma unroll
    for (int st = 0; st < C::KST; ++st) {
      const u32x4 gv = __builtin_bit_cast(u32x4, gr[st]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        part += bf16_lo(orow[st][e]) * bf16_lo(gv[e]) + bf16_hi(orow[st][e]) * bf16_hi(gv[e]);
    }
    dl = xhalf_sum(part);
    if (my_q < T && h == 0) delta[(size_t)bh * T + my_q] = dl;
  }
  sync();
  f32x16 sc, dpc, sn, dpn;
  if (wkt0 == kt0) sdp(kt0, sc, dpc);

  // Phases of the wave (one barrier per tile of the workgroup in each): idle tiles,
  // S / dP of its first tile, tiles crossing the window's lower edge (masked),
  // unmasked tiles, its diagonal tile (masked, no S / dP ahead), idle tiles.
  const int mlim = (window > 0 && wq_hi - window >= 0) ? (wq_hi - window) / C::BN + 1 : 0;
  int kt = kt0;
  for (; kt < min(wkt0 - 1, kt1 + 1); ++kt) {
    issue(kt + C::AHEAD);
    sync();
  }
  if (wkt0 > kt0 && kt == wkt0 - 1) {
    issue(kt + C::AHEAD);
    sdp(kt + 1, sc, dpc);
    sync();
    ++kt;
  }
  for (; kt < min(wkt1, mlim); ++kt) {
    step(std::true_type{}, kt, sc, dpc, sn, dpn);
    sc = sn;
    dpc = dpn;
    sync();
  }
  // unmasked tiles, two per iteration: S / dP of the next tile alternate between the
  // two register sets, so nothing is copied
  for (; kt + 1 < wkt1; kt += 2) {
    step(std::false_type{}, kt, sc, dpc, sn, dpn);
    sync();
    step(std::false_type{}, kt + 1, sn, dpn, sc, dpc);
    sync();
  }
  if (kt < wkt1) {
    step(std::false_type{}, kt, sc, dpc, sn, dpn);
    sc = sn;
    dpc = dpn;
    sync();
    ++kt;
  }
  if (kt == wkt1) {
    last_step(kt, sc, dpc);
    sync();
    ++kt;
  }
  for (; kt <= kt1; ++kt) {
    issue(kt + C::AHEAD);
    sync();
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm<0>);  // no copy into LDS outlives the workgroup

#pragma unroll
  for (int d = 0; d < C::NDB; ++d) acc[d] *= scale;  // dL/dq (dL/dq' with ROPE)
  if constexpr (ROPE) {
    // back through the prologue, with the raw query row read again (every lane of the
    // wave takes part: the reductions pair lanes l and l ^ 32)
    // (the query index and the frequency ratio made opaque, so that nothing of the load's
    // prologue is held in registers through the loop for this)
    int qi = my_q;
    RopeArgs re = ra;
    asm volatile("" : "+v"(qi), "+s"(re.ratio));
    f32x16 xr[C::NDB];
    load_acc_order<D>(qb + (size_t)min(qi, T - 1) * rs, h, xr);
    rope_norm_grad_acc<D>(acc, xr, rope_pos(re, b, qi), qi < T, re, h);
  }
  // dq through LDS (stage_rows_bf16), in the tile slots once every wave's copies have
  // landed and every wave has finished its reads
  static_assert(4 * 32 * D <= C::NSLOT * 2 * C::TSZ, "the waves' rows fit the tile slots");
  __syncthreads();
  uint16_t *stage = smem + w * 32 * D;
  stage_rows_bf16<D>(stage, acc, 1.f, ln, h);
  __syncthreads();
  store_staged_rows<D>(stage, lane, T - qw0, dq + base + (size_t)qw0 * rs, rs);
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

template <int D, bool ROPE>
static void launch_dq_t(const void *q, const void *k, const void *v, const void *o, const void *dO,
                        const float *lse, float *delta, void *dq, int B, int H, int Hkv, int T,
                        int window, float scale, const RopeArgs &ra, hipStream_t st) {
  const int nqt = (T + 127) / 128;
  const unsigned nb = (unsigned)(nqt * B * H);
  bwd_dq_bf16_kernel<D, ROPE><<<nb, 256, 0, st>>>(
      (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)o,
      (const uint16_t *)dO, lse, delta, (uint16_t *)dq, B, H, Hkv, T, window, scale, nqt, ra);
}

hipError_t launch_bwd_dq_bf16(const void *q, const void *k, const void *v, const void *o,
                              const void *dO, const float *lse, float *delta, void *dq, int B,
                              int H, int Hkv, int T, int D, int window, float scale,
                              hipStream_t st, const RopeArgs *rope) {
  if (rope != nullptr) {
    if (D == 128)
      launch_dq_t<128, true>(q, k, v, o, dO, lse, delta, dq, B, H, Hkv, T, window, scale, *rope, st);
    else
      launch_dq_t<64, true>(q, k, v, o, dO, lse, delta, dq, B, H, Hkv, T, window, scale, *rope, st);
  } else if (D == 128) {
    launch_dq_t<128, false>(q, k, v, o, dO, lse, delta, dq, B, H, Hkv, T, window, scale,
                            RopeArgs{}, st);
  } else {
    launch_dq_t<64, false>(q, k, v, o, dO, lse, delta, dq, B, H, Hkv, T, window, scale,
                           RopeArgs{}, st);
  }
  return hipGetLastError();
}

}  // namespace swattn

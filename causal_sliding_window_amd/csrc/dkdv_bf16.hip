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
  static constexpr int NSLOT = 8;         // LDS tile slots (tile t in slot t % 8)
  static constexpr int AHEAD = 6;         // tiles are copied this many steps ahead
  static constexpr int TSZ = BQ * D;      // elements of one Q (or dO) tile
  static constexpr int NDB = D / 32;
  static constexpr int KST = D / 16;      // = 2 * NDB
  static constexpr int HALF = TSZ * 2 / 1024;  // 1-KB pieces of one tensor's tile
  static constexpr int CPW = 2 * HALF / 4;     // pieces per wave and tile (Q and dO)
  static constexpr int RG = BQ / 16;           // 16-row groups per 32-column block
  static constexpr int NCOPY = CPW + 1;        // copies per wave and tile (+ lse/delta)
  static constexpr int VSZ = 256;              // floats of lse / delta per slot
};

// Largest P of a tile (any lane) from which P enters dV as bf16 hi + lo.
constexpr float kLoP = 0.0625f;
// Largest |dS| of a tile (any lane) from which dS enters dK as bf16 hi + lo, and the head
// sizes that take that path (D = 128 has no registers to spare for it; its sweeps meet
// the bar with one bf16 dS).
constexpr float kLoDsK = 1.0f;
template <int D>
constexpr bool kDsLoK = D == 64;

// PARTIAL (grouped-query attention, H > Hkv): the workgroup's query head is one of
// the G = H / Hkv that read K/V head h / G; it writes its fp32 contributions to dK
// (already scaled) and dV to part_k / part_v, [B, T, H, D], and dkdv_group_sum_kernel
// adds the G of each K/V head.  Otherwise dk and dv are written directly.
template <int D, bool PARTIAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ dO,
    const float *__restrict__ lse, const float *__restrict__ delta, uint16_t *__restrict__ dk,
    uint16_t *__restrict__ dv, float *__restrict__ part_k, float *__restrict__ part_v, int B,
    int H, int Hkv, int T, int window, float scale, int nkt) {
  using C = DkdvCfg<D>;
  // One LDS array (with a single __shared__ variable the compiler keeps the restrict
  // scopes below): [slot][Q, dO][TSZ] bf16, then [slot][lse, delta, spare, spare][64]
  // float.
  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::NSLOT * 2 * C::TSZ +
                                                          C::NSLOT * C::VSZ * 2];
  float *const vec = reinterpret_cast<float *>(smem + C::NSLOT * 2 * C::TSZ);

  const int BH = B * H;
  const int bid = blockIdx.x;
  const int kt = bid / BH;  // early key tiles see the most queries: first
  const int bh = bid % BH;
  const int b = bh / H, hh = bh % H;
  const int k0 = kt * C::BK;
  const int rs = H * D;       // row stride of q and dO (and of the partials)
  const int rsk = Hkv * D;    // row stride of k, v, dk and dv
  const int hk = hh / (H / Hkv);  // the K/V head of query head hh
  const size_t base = ((size_t)b * T * H + hh) * D;
  const size_t base_kv = ((size_t)b * T * Hkv + hk) * D;
  const uint16_t *qb = q + base, *kb = k + base_kv, *vb = v + base_kv, *gb = dO + base;
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

  // K and V rows of the wave's keys (B operands), rows past T read as zero; loaded
  // in the prologue, between the tile copies
  bf16x8 kr[C::KST], vr[C::KST];
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
  // One buffer resource per tensor over all T rows of this (b, h): a tile's row
  // offset goes into the lane offsets, and offsets from row T on read as zero.
  const int my_tensor = (w * C::CPW) / C::HALF;  // every copy of a wave is Q (0) or dO (1)
  const __amdgpu_buffer_rsrc_t rsrc_t = make_rsrc(my_tensor ? gb : qb, (uint32_t)T * rs * 2);
  const __amdgpu_buffer_rsrc_t rsrc_v = make_rsrc((w & 1) ? delb : lseb, (uint32_t)T * 4);
  auto issue_to = [&](int qt, uint16_t *tile, float *vdst) {
    const uint32_t roff = (uint32_t)(qt * C::BQ) * (uint32_t)rs * 2;
#pragma unroll
    for (int cc = 0; cc < C::CPW; ++cc) {
      const int jj = (w * C::CPW + cc) % C::HALF;
      const int db = jj / C::RG, row16 = 16 * (jj % C::RG);
      buf_copy16_to_lds(rsrc_t, tile + my_tensor * C::TSZ + db * (C::BQ * 32) + row16 * 32,
                        lane_off + (uint32_t)(row16 * rs + 32 * db) * 2 + roff);
    }
    // every wave issues exactly NCOPY copies per tile (waves 2 and 3 fill spare
    // rows), so the end-of-step wait can count them
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc_v, (__attribute__((address_space(3))) void *)(vdst + w * 64), 4,
        (uint32_t)(lane + qt * C::BQ) * 4, 0, 0, 0);
  };
  auto q_tile = [&](int qt) { return smem + 2 * (qt & (C::NSLOT - 1)) * C::TSZ; };
  auto vec_of = [&](int qt) { return vec + (qt & (C::NSLOT - 1)) * C::VSZ; };
  auto issue = [&](int qt) { issue_to(qt, q_tile(qt), vec_of(qt)); };

  // lse and delta enter S and dP through one extra MFMA each.  MFMA row m of a tile
  // is query swap23(m); lane m of half 0 reads that query's lse, lane m of half 1
  // its delta, and splits -lse / scale (half 0) or -delta (half 1) into three bf16
  // terms (hi + mid + lo = the fp32 value to ~2^-24) in K slots 0..2 of its A
  // operand.  With B = ones in K slots 0..2 (for S) or 8..10 (for dP), the product
  // adds -lse / scale to every element of the query's S row, and -delta to its dP
  // row: S' = S - lse / scale gives P = exp2(c S') with c = scale log2(e), and dP'
  // = dP - delta gives dS = P dP'.
  const int vrow = 64 * h + swap23(ln);
  const float xmul = h ? -1.f : -1.f / scale;
  bf16x8 bsel_s, bsel_d;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    bsel_s[j] = (__bf16)((h == 0 && j < 3) ? 1.f : 0.f);
    bsel_d[j] = (__bf16)((h == 1 && j < 3) ? 1.f : 0.f);
  }
  auto bcast_op = [&](float xv) {
    const float x = xv * xmul;
    const __bf16 hi = (__bf16)x;
    const float r1 = x - (float)hi;
    const __bf16 mid = (__bf16)r1;
    const __bf16 lo = (__bf16)(r1 - (float)mid);
    bf16x8 a = {};
    a[0] = hi;
    a[1] = mid;
    a[2] = lo;
    return a;
  };

  // S' and dP' of a tile, one key per lane: register 8t + j of half h holds query
  // 16t + 8h + j of the tile.
  auto sdp_from = [&](const bf16x8 (&qa)[C::KST], const bf16x8 (&ga)[C::KST], float xv,
                      f32x16 &s, f32x16 &dp) {
    const bf16x8 av = bcast_op(xv);
    s = mfma32(av, bsel_s, f32x16{});
    dp = mfma32(av, bsel_d, f32x16{});
#pragma unroll
    for (int st = 0; st < C::KST; ++st) {
      s = mfma32(qa[st], kr[st], s);
      dp = mfma32(ga[st], vr[st], dp);
    }
  };
  // Operand reads of a tile for S' / dP' (b128 rows) and the lane's lse / delta.
  auto read_q = [&](const uint16_t *__restrict__ tile, int st) {
    return lds_read_b128(tile + dt_off<C::BQ>(ln, 2 * st + h));
  };
  // Transposed operand k (k < NDB: dO^T block k, else Q^T block k - NDB) of rows
  // 16 t .. 16 t + 15 of a tile.
  auto tr_op = [&](const uint16_t *__restrict__ tile, int t, int kk) {
    return dt_read_tr_perm<C::BQ>(kk < C::NDB ? tile + C::TSZ : tile, 16 * t, kk % C::NDB,
                                  lane);
  };

  // P = exp2(c S') and dS = P dP' for elements [e0, e0 + n) of a tile; pm keeps the
  // largest P of the lane.
  auto grad_elems = [&](auto mask_tag, f32x16 &s, f32x16 &dp, float &pm, float &dm, int rel0,
                        int e0, int n) {
    constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
    for (int i = e0; i < e0 + n; ++i) {
      const int t = i >> 3, j = i & 7;
      float p = fast_exp2(s[i] * c);
      if (MASK) p = (unsigned)(rel0 + 16 * t + j) <= wm1 ? p : 0.f;
      s[i] = p;
      dp[i] = p * dp[i];
    }
#pragma unroll
    for (int i = e0; i < e0 + n; i += 2) pm = fmaxf(pm, fmaxf(s[i], s[i + 1]));
    if constexpr (kDsLoK<D>) {
#pragma unroll
      for (int i = e0; i < e0 + n; i += 2) dm = fmaxf(dm, fmaxf(fabsf(dp[i]), fabsf(dp[i + 1])));
    }
  };
  // dS enters dK as one bf16 unless some |dS| of the wave's tile reaches kLoDsK (D = 64):
  // then also its remainder, lo = dS - bf16(dS) rounded to bf16.
  auto pack_ds_lo = [&](const f32x16 &dp, int t) {
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (__bf16)(dp[8 * t + j] - (float)(__bf16)dp[8 * t + j]);
    return r;
  };
  auto grads_ds_lo = [&](const bf16x8 (&ops)[2 * C::NDB], const bf16x8 &dl) {
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) dka[d] = mfma32(ops[C::NDB + d], dl, dka[d]);
  };
  // P enters dV as bf16.  Where some P of the wave's tile reaches kLoP, it enters as
  // hi + lo instead: hi = P truncated to bf16, lo = the exact remainder rounded to
  // bf16 (P = hi + lo to ~2^-16 relative).  A single bf16 P on those large values
  // leaves |dV| >= 4 outside 2e-2 of the exact gradient; below kLoP the rounding of
  // P (<= 2^-13 absolute) is far inside it.
  auto pack_rne = [&](const f32x16 &s, int t) { return to_bf16x8(s, 8 * t); };
  auto pack_hilo = [&](const f32x16 &s, int t, bf16x8 &ph, bf16x8 &pl) {
    u32x4 hp, lp;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = s[8 * t + 2 * j], b = s[8 * t + 2 * j + 1];
      const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
      hp[j] = __builtin_amdgcn_perm(ub, ua, 0x07060302u);
      const bf16x2 r = {(__bf16)(a - __uint_as_float(ua & 0xffff0000u)),
                        (__bf16)(b - __uint_as_float(ub & 0xffff0000u))};
      lp[j] = __builtin_bit_cast(uint32_t, r);
    }
    ph = __builtin_bit_cast(bf16x8, hp);
    pl = __builtin_bit_cast(bf16x8, lp);
  };
  auto grads = [&](const bf16x8 (&ops)[2 * C::NDB], int d, const bf16x8 &ph,
                   const bf16x8 &ds) {
    dva[d] = mfma32(ops[d], ph, dva[d]);
    dka[d] = mfma32(ops[C::NDB + d], ds, dka[d]);
  };
  auto grads_lo = [&](const bf16x8 (&ops)[2 * C::NDB], const bf16x8 &pl) {
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) dva[d] = mfma32(ops[d], pl, dva[d]);
  };

  auto pin = [](float x) {
    asm volatile("" ::"v"(x));
    __builtin_amdgcn_sched_barrier(0);
  };

  // One pipeline step for tile qt: S', dP' of tile qt in (sc, dpc); the S'/dP'
  // operands (qa, ga, xv) of tile qt + 1 in registers.  LDS reads are spread over
  // the MFMA phases so that every wave keeps its MFMAs busy while the LDS serves
  // the reads of all four:
  //   phase 1: S', dP' of tile qt + 1 (when NEXT) into (sn, dpn), one MFMA pair per
  //            slice, with a transposed operand read of tile qt rows 0..15 and the
  //            P / dS work of two (D = 128) elements per slice;
  //   phase 2a: dV^T, dK^T of rows 0..15, one 32-column block per slice, with the
  //            transposed operand reads of rows 16..31;
  //   phase 2b: dV^T, dK^T of rows 16..31, with the S'/dP' operand reads of tile
  //            qt + 2 (when LOAD) for the next step.
  // The tiles come in as distinct restrict pointers: the compiler then knows the
  // reads do not touch the tile being copied and does not make them wait for the
  // copies in flight (the tiles a step reads were awaited at an earlier barrier).
  auto step_body = [&](auto mask_tag, auto next_tag, auto load_tag, int qt, f32x16 &sc,
                       f32x16 &dpc, f32x16 &sn, f32x16 &dpn, bf16x8 (&qa)[C::KST],
                       bf16x8 (&ga)[C::KST], float &xv, const uint16_t *__restrict__ cur,
                       const uint16_t *__restrict__ nn, const float *__restrict__ vnn,
                       uint16_t *__restrict__ dma, float *__restrict__ vdma)
                       __attribute__((always_inline)) {
    constexpr bool NEXT = decltype(next_tag)::value;
    constexpr bool LOAD = decltype(load_tag)::value;
    issue_to(qt + C::AHEAD, dma, vdma);
    const int rel0 = qt * C::BQ + 8 * h - my_k;
    bf16x8 op0[2 * C::NDB], op1[2 * C::NDB];
    float pm = 0.f, dm = 0.f;
    if constexpr (NEXT) {
      const bf16x8 av = bcast_op(xv);
      sn = mfma32(av, bsel_s, f32x16{});
      dpn = mfma32(av, bsel_d, f32x16{});
    }
    __builtin_amdgcn_sched_barrier(0);
    constexpr int EPS = 16 / C::KST;  // elements per slice
#pragma unroll
    for (int st = 0; st < C::KST; ++st) {
      op0[st] = tr_op(cur, 0, st);
      if constexpr (NEXT) {
        sn = mfma32(qa[st], kr[st], sn);
        dpn = mfma32(ga[st], vr[st], dpn);
      }
      __builtin_amdgcn_sched_barrier(0);
      grad_elems(mask_tag, sc, dpc, pm, dm, rel0, EPS * st, EPS);
      pin(dpc[EPS * st + EPS - 1]);
    }
    // phases 2a and 2b; the lo part of P only where the tile holds a large P, its
    // MFMAs grouped after each phase (one branch per group)
    const bool lo = __builtin_amdgcn_ballot_w64(pm >= kLoP) != 0;
    const bool lods = kDsLoK<D> && __builtin_amdgcn_ballot_w64(dm >= kLoDsK) != 0;
    bf16x8 ph0, pl0, ph1, pl1;
    if (lo) {
      pack_hilo(sc, 0, ph0, pl0);
      pack_hilo(sc, 1, ph1, pl1);
    } else {
      ph0 = pack_rne(sc, 0);
      ph1 = pack_rne(sc, 1);
    }
    const bf16x8 ds0 = to_bf16x8(dpc, 0);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 ds1;
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) {
      op1[d] = tr_op(cur, 1, d);
      op1[C::NDB + d] = tr_op(cur, 1, C::NDB + d);
      grads(op0, d, ph0, ds0);
      __builtin_amdgcn_sched_barrier(0);
      if (d == C::NDB - 1) ds1 = to_bf16x8(dpc, 8);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (lo) grads_lo(op0, pl0);
    if (lods) grads_ds_lo(op0, pack_ds_lo(dpc, 0));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < C::NDB; ++d) {
      if constexpr (LOAD) {
#pragma unroll
        for (int u = 0; u < C::KST / C::NDB; ++u) {
          const int st = (C::KST / C::NDB) * d + u;
          qa[st] = read_q(nn, st);
          ga[st] = read_q(nn + C::TSZ, st);
        }
        if (d == 0) xv = vnn[vrow];
      }
      grads(op1, d, ph1, ds1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (lo) grads_lo(op1, pl1);
    if (lods) grads_ds_lo(op1, pack_ds_lo(dpc, 1));
  };
  auto step = [&](auto mask_tag, auto next_tag, auto load_tag, int qt, f32x16 &sc, f32x16 &dpc,
                  f32x16 &sn, f32x16 &dpn, bf16x8 (&qa)[C::KST], bf16x8 (&ga)[C::KST],
                  float &xv) __attribute__((always_inline)) {
    step_body(mask_tag, next_tag, load_tag, qt, sc, dpc, sn, dpn, qa, ga, xv, q_tile(qt),
              q_tile(qt + 2), vec_of(qt + 2), q_tile(qt + C::AHEAD), vec_of(qt + C::AHEAD));
  };
  // S', dP' of the wave's first tile t and the S'/dP' operands of tile t + 1.
  auto pre_body = [&](int t, f32x16 &sc, f32x16 &dpc, bf16x8 (&qa)[C::KST],
                      bf16x8 (&ga)[C::KST], float &xv, const uint16_t *__restrict__ t0p,
                      const float *__restrict__ v0p, const uint16_t *__restrict__ t1p,
                      const float *__restrict__ v1p) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 0; st < C::KST; ++st) {
      qa[st] = read_q(t0p, st);
      ga[st] = read_q(t0p + C::TSZ, st);
    }
    xv = v0p[vrow];
    sdp_from(qa, ga, xv, sc, dpc);
    if (t + 1 <= wqt1) {
#pragma unroll
      for (int st = 0; st < C::KST; ++st) {
        qa[st] = read_q(t1p, st);
        ga[st] = read_q(t1p + C::TSZ, st);
      }
      xv = v1p[vrow];
    }
  };
  // One barrier per two steps, after the steps qt with qt - qt0 odd: there, all
  // copies but those of the last two steps (tiles qt + AHEAD - 1, qt + AHEAD) must
  // have landed, so that the next two steps find tiles up to qt + 4 in LDS.  A step
  // reads tiles qt .. qt + 2 and copies into the slot of tile qt - 2, both of them
  // separated from the other uses of those slots by a barrier.  Every step issues
  // its copies, also past the workgroup's last tile (rows from T on read as zero
  // and land in slots no step reads), so the wait count is always the same.
  auto sync = [&](int qt) {
    if ((qt - qt0) & 1) {
      __builtin_amdgcn_s_waitcnt(kWaitVm<2 * C::NCOPY>);
      lds_barrier();
    }
  };

  // prologue: tiles qt0 .. qt0 + AHEAD - 1 in flight; those up to qt0 + 3 must land.
  // The K / V row loads go between the copies of tiles qt0 + 3 and qt0 + 4, so all
  // these memory latencies overlap and one wait covers the rows and the first four
  // tiles (vector-memory operations complete in order).
  for (int t = qt0; t < qt0 + 4; ++t) issue(t);
  {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (uint32_t)T * rsk * 2);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (uint32_t)T * rsk * 2);
#pragma unroll
    for (int st = 0; st < C::KST; ++st) {
      const uint32_t off = (my_k * rsk + 16 * st + 8 * h) * 2;
      kr[st] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
      vr[st] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
  }
  static_assert(C::AHEAD == 6, "the prologue issues tiles qt0 + 4 and qt0 + 5 last");
  issue(qt0 + 4);
  issue(qt0 + 5);
  __builtin_amdgcn_s_waitcnt(kWaitVm<2 * C::NCOPY>);
  lds_barrier();

  f32x16 sa, dpa, sb, dpb;
  bf16x8 qa[C::KST], ga[C::KST];
  float xv = 0.f;
  if (wqt0 == qt0)
    pre_body(qt0, sa, dpa, qa, ga, xv, q_tile(qt0), vec_of(qt0), q_tile(qt0 + 1),
             vec_of(qt0 + 1));

  // Phases of the wave: idle tiles, the step before its first tile (S', dP' of that
  // tile), its tiles (the first one and those from mlo on masked), idle tiles.  One
  // barrier per tile of the workgroup in every phase.
  using F = std::false_type;
  using Tr = std::true_type;
  int qt = qt0;
  for (; qt < min(wqt0 - 1, qt1 + 1); ++qt) {
    issue(qt + C::AHEAD);
    sync(qt);
  }
  if (wqt0 > qt0 && qt == wqt0 - 1) {
    issue(qt + C::AHEAD);
    pre_body(qt + 1, sa, dpa, qa, ga, xv, q_tile(qt + 1), vec_of(qt + 1), q_tile(qt + 2),
             vec_of(qt + 2));
    sync(qt);
    ++qt;
  }
  // The wave's tiles wqt0 .. wqt1; S' / dP' of tile qt in (sa, dpa) between steps.
  // Step qt computes S' / dP' of tile qt + 1 when qt < wqt1 (NEXT) and reads the
  // operands of tile qt + 2 when qt + 2 <= wqt1 (LOAD); tile wqt0, tiles from mlo on
  // and the last two tiles run the element mask.
  auto next = [&] {
    sa = sb;
    dpa = dpb;
  };
  if (qt == wqt0 && qt <= wqt1) {  // diagonal tile
    if (qt + 2 <= wqt1) {
      step(Tr{}, Tr{}, Tr{}, qt, sa, dpa, sb, dpb, qa, ga, xv);
      next();
    } else if (qt + 1 <= wqt1) {
      step(Tr{}, Tr{}, F{}, qt, sa, dpa, sb, dpb, qa, ga, xv);
      next();
    } else {
      step(Tr{}, F{}, F{}, qt, sa, dpa, sb, dpb, qa, ga, xv);
    }
    sync(qt);
    ++qt;
  }
  // unmasked steps with NEXT and LOAD, two per iteration (no register copies)
  const int ulim = min(wqt1 - 1, mlo);
  for (; qt + 1 < ulim; qt += 2) {
    step(F{}, Tr{}, Tr{}, qt, sa, dpa, sb, dpb, qa, ga, xv);
    sync(qt);
    step(F{}, Tr{}, Tr{}, qt + 1, sb, dpb, sa, dpa, qa, ga, xv);
    sync(qt + 1);
  }
  if (qt < ulim) {
    step(F{}, Tr{}, Tr{}, qt, sa, dpa, sb, dpb, qa, ga, xv);
    next();
    sync(qt);
    ++qt;
  }
  // masked steps with NEXT and LOAD
  for (; qt < wqt1 - 1; ++qt) {
    step(Tr{}, Tr{}, Tr{}, qt, sa, dpa, sb, dpb, qa, ga, xv);
    next();
    sync(qt);
  }
  // the last two steps always run the element mask (it keeps every element of an
  // unmasked tile): one code path each
  if (qt == wqt1 - 1) {
    step(Tr{}, Tr{}, F{}, qt, sa, dpa, sb, dpb, qa, ga, xv);
    next();
    sync(qt);
    ++qt;
  }
  if (qt == wqt1) {
    step(Tr{}, F{}, F{}, qt, sa, dpa, sb, dpb, qa, ga, xv);
    sync(qt);
    ++qt;
  }
  for (; qt <= qt1; ++qt) {
    issue(qt + C::AHEAD);
    sync(qt);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm<0>);  // no copy into LDS outlives the workgroup

  if (PARTIAL) {
    if (my_k < T) {
      float *pk = part_k + base + (size_t)my_k * rs, *pv = part_v + base + (size_t)my_k * rs;
#pragma unroll
      for (int d = 0; d < C::NDB; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 a, c4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = dka[d][4 * g + e] * scale;
            c4[e] = dva[d][4 * g + e];
          }
          *reinterpret_cast<f32x4 *>(pk + 32 * d + 8 * g + 4 * h) = a;
          *reinterpret_cast<f32x4 *>(pv + 32 * d + 8 * g + 4 * h) = c4;
        }
    }
  } else if (my_k < T) {
    uint16_t *dkb = dk + base_kv + (size_t)my_k * rsk, *dvb = dv + base_kv + (size_t)my_k * rsk;
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

// dk, dv [B, T, Hkv, D] (bf16) = sums of the G = H / Hkv partials [B, T, H, D] (fp32)
// of each K/V head, in head order; 8 elements per thread.
__global__ __launch_bounds__(256) void dkdv_group_sum_kernel(const float *__restrict__ part_k,
                                                             const float *__restrict__ part_v,
                                                             uint16_t *__restrict__ dk,
                                                             uint16_t *__restrict__ dv,
                                                             long long n8, int G, int D) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;  // group of 8 outputs
  if (i >= n8) return;
  const long long e = i * 8;               // output element: ((b T + t) Hkv + hk) D + d
  const long long row = e / D, d = e % D;  // row = (b T + t) Hkv + hk
  const float *pk = part_k + row * G * D + d, *pv = part_v + row * G * D + d;
  float sk[8], sv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) sk[j] = sv[j] = 0.f;
  for (int g = 0; g < G; ++g) {
    const f32x4 k0 = *reinterpret_cast<const f32x4 *>(pk + (size_t)g * D);
    const f32x4 k1 = *reinterpret_cast<const f32x4 *>(pk + (size_t)g * D + 4);
    const f32x4 v0 = *reinterpret_cast<const f32x4 *>(pv + (size_t)g * D);
    const f32x4 v1 = *reinterpret_cast<const f32x4 *>(pv + (size_t)g * D + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sk[j] += k0[j];
      sk[4 + j] += k1[j];
      sv[j] += v0[j];
      sv[4 + j] += v1[j];
    }
  }
  bf16x4 a0, a1, b0, b1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a0[j] = (__bf16)sk[j];
    a1[j] = (__bf16)sk[4 + j];
    b0[j] = (__bf16)sv[j];
    b1[j] = (__bf16)sv[4 + j];
  }
  *reinterpret_cast<bf16x4 *>(dk + e) = a0;
  *reinterpret_cast<bf16x4 *>(dk + e + 4) = a1;
  *reinterpret_cast<bf16x4 *>(dv + e) = b0;
  *reinterpret_cast<bf16x4 *>(dv + e + 4) = b1;
}

template <int D, bool PARTIAL>
static void launch_dkdv_t(const void *q, const void *k, const void *v, const void *dO,
                          const float *lse, const float *delta, void *dk, void *dv,
                          float *part_k, float *part_v, int B, int H, int Hkv, int T, int window,
                          float scale, hipStream_t st) {
  const int nkt = (T + DkdvCfg<D>::BK - 1) / DkdvCfg<D>::BK;
  const unsigned nb = (unsigned)(nkt * B * H);
  bwd_dkdv_bf16_kernel<D, PARTIAL><<<nb, 256, 0, st>>>(
      (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)dO, lse,
      delta, (uint16_t *)dk, (uint16_t *)dv, part_k, part_v, B, H, Hkv, T, window, scale, nkt);
}

hipError_t launch_bwd_dkdv_bf16(const void *q, const void *k, const void *v, const void *dO,
                                const float *lse, const float *delta, void *dk, void *dv,
                                float *part, int B, int H, int Hkv, int T, int D, int window,
                                float scale, hipStream_t st) {
  if (Hkv == H) {
    if (D == 128)
      launch_dkdv_t<128, false>(q, k, v, dO, lse, delta, dk, dv, nullptr, nullptr, B, H, Hkv, T,
                                window, scale, st);
    else
      launch_dkdv_t<64, false>(q, k, v, dO, lse, delta, dk, dv, nullptr, nullptr, B, H, Hkv, T,
                               window, scale, st);
    return hipGetLastError();
  }
  float *part_k = part, *part_v = part + (size_t)B * T * H * D;
  if (D == 128)
    launch_dkdv_t<128, true>(q, k, v, dO, lse, delta, dk, dv, part_k, part_v, B, H, Hkv, T,
                             window, scale, st);
  else
    launch_dkdv_t<64, true>(q, k, v, dO, lse, delta, dk, dv, part_k, part_v, B, H, Hkv, T,
                            window, scale, st);
  const long long n8 = (long long)B * T * Hkv * D / 8;
  dkdv_group_sum_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>(
      part_k, part_v, (uint16_t *)dk, (uint16_t *)dv, n8, H / Hkv, D);
  return hipGetLastError();
}

}  // namespace swattn

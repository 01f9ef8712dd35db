// dK, dV of causal sliding-window attention, bf16 in / bf16 out, fp32 accumulate
// (the dK/dV pass of the backward; see bwd_bf16.hip for the delta preprocess and
// the dQ pass).  Gradients of L = sum_i dO_i . o_i for the attention of the
// nanochat guide's section 5, with P recomputed from the stored LSE:
//   dV = P^T dO,  dK = scale * dS^T Q,  dS = P * (dP - delta),  dP = dO V^T.
//
// One workgroup = 32 keys x NG key groups of one (b, h), each group served by two
// waves in two roles (see bwd_dkdv_bf16_kernel): one keeps its K rows in registers
// and forms S = Q K^T, P and dV, the other keeps its V rows and forms dP = dO V^T, dS
// and dK.  S and dP are formed with one key per lane, so P and dS feed dV^T = dO^T P
// and dK^T = Q^T dS as B operands straight from registers; dO^T and Q^T come from
// transposed LDS reads.  Query tiles of 32 rows reach LDS by direct buffer -> LDS
// copies, two steps ahead; one workgroup barrier per step.
//
// Built with -amdgpu-mfma-vgpr-form like the other kernels: all MFMA results are in
// arch VGPRs (the build reports no AGPRs).
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "rope.h"

namespace swattn {

// ---------------------------------------------------------------- dK, dV
// NG key groups of 32 keys per workgroup: 4 (128 keys, eight waves, one workgroup per
// CU) or 2 (64 keys, four waves, two workgroups per CU; for short windows, where a
// workgroup's query range is mostly the window and a wide key block leaves each group
// idle through the others' tiles).
template <int D, int NG = 4>
struct DkdvCfg {
  static constexpr int BK = 32 * NG;      // keys per workgroup
  static constexpr int BQ = 32;           // queries per tile
  static constexpr int NW = 2 * NG;       // waves: NG P side + NG dS side
  static constexpr int NSLOT = 4;         // LDS slots of Q tiles (tile t in slot t % 4)
  static constexpr int NSLOT_O = NG == 4 ? 4 : 3;  // slots of dO tiles and lse / delta
  static constexpr int AHEAD = 2;         // tiles are copied this many steps ahead
  static constexpr int TSZ = BQ * D;      // elements of one Q (or dO) tile
  static constexpr int NDB = D / 32;
  static constexpr int KST = D / 16;      // = 2 * NDB
  static constexpr int HALF = TSZ * 2 / 1024;  // 1-KB pieces of one tensor's tile
  static constexpr int CPW = 2 * HALF / NW;    // pieces per wave and tile (Q and dO)
  static constexpr int RG = BQ / 16;           // 16-row groups per 32-column block
  static constexpr int NCOPY = CPW + 1;        // copies per wave and tile (+ lse/delta)
  static constexpr int VSZ = NW * 64;          // floats of lse / delta (and spares) per slot
  static constexpr int XSZ = 16 * 64;          // floats of one handed-over P tile
  static_assert(CPW >= 1 && (2 * HALF) % NW == 0, "whole 1-KB pieces per wave");
  static_assert(NG == 2 || NG == 4, "two or four key groups");
  // bytes of LDS; with NG = 2 two workgroups share a CU's 160 KB
  static constexpr int LDS_BYTES =
      (NSLOT + NSLOT_O) * TSZ * 2 + NSLOT_O * VSZ * 4 + NG * 2 * XSZ * 4;
  static_assert(NG == 4 || LDS_BYTES <= 80 * 1024, "two workgroups per CU");
};

// Largest P of a tile (any lane) from which P enters dV as bf16 hi + lo.
constexpr float kLoP = 0.0625f;
// Largest |dS| of a tile (any lane) from which dS enters dK as bf16 hi + lo, and the head
// sizes that take that path (at D = 128 the sweeps meet the bar with one bf16 dS).
constexpr float kLoDsK = 1.0f;
template <int D>
constexpr bool kDsLoK = D == 64;

// s_waitcnt immediate: at most N vector-memory operations in flight and every LDS
// operation of the wave complete.
template <int N>
constexpr int kWaitVmLgkm0 = (N & 15) | ((N >> 4) << 14) | (7 << 4);

// One workgroup = 2 NG waves = 32 NG keys of one (b, h), in NG groups of 32 keys; each
// group is served by two waves with the same keys (one per role); with NG = 4 the two
// run on the same SIMD (waves g and g + 4):
//   P side  (waves 0..NG-1):   S' = Q K^T - lse / scale, P = exp2(c S'), dV^T += dO^T P;
//                              hands P (fp32) to its partner through LDS;
//   dS side (waves NG..2NG-1): dP' = dO V^T - delta, and one step later, with the
//                              partner's P of that tile, dS = P dP' and dK^T += Q^T dS.
// Each wave holds one 32-key accumulator set (dV or dK, 64 registers) and one set of
// stationary operands (K or V rows), so two waves fit one SIMD and each covers the
// other's waits.  Query tiles of 32 rows reach LDS by direct buffer -> LDS copies,
// two steps ahead; one workgroup barrier per step.
//
// PARTIAL (grouped-query attention, H > Hkv): the workgroup's query head is one of
// the G = H / Hkv that read K/V head h / G; it writes its fp32 contributions to dK
// (already scaled) and dV to part_k / part_v, [B, T, H, D], and dkdv_group_sum_kernel
// adds the G of each K/V head.  Otherwise dk and dv are written directly.
// ROPE: k holds the raw keys (q the transformed queries); each key row is normalised and
// rotated (QK norm + rotary embedding) as the P side loads it, and dk is the gradient
// with respect to the raw key: the dS side's epilogue maps dL/dk' back through the
// prologue.  With PARTIAL it maps the query head's share (the map is linear in dL/dk')
// and writes it to part_k in fp32; the group sum then adds mapped shares.
template <int D, bool PARTIAL, bool ROPE = false, int NG = 4>
__global__ __launch_bounds__(128 * NG, 4 / NG) void bwd_dkdv_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const uint16_t *__restrict__ dO,
    const float *__restrict__ lse, const float *__restrict__ delta, uint16_t *__restrict__ dk,
    uint16_t *__restrict__ dv, float *__restrict__ part_k, float *__restrict__ part_v, int B,
    int H, int Hkv, int T, int window, float scale, int nkt, RopeArgs ra = RopeArgs{}) {
  using C = DkdvCfg<D, NG>;
  // One LDS array (with a single __shared__ variable the compiler keeps the restrict
  // scopes below): [NSLOT][TSZ] bf16 (Q tiles), [NSLOT_O][TSZ] bf16 (dO tiles), then
  // [NSLOT_O][VSZ] float (lse, delta, spares), then [key group][2][XSZ] float (the
  // handed-over P tiles).  Q of tile qt - 1 is read in step qt (dK); dO is not, so dO
  // and lse / delta need one slot fewer.
  __shared__ __attribute__((aligned(1024))) uint16_t smem[C::LDS_BYTES / 2];
  uint16_t *const osm = smem + C::NSLOT * C::TSZ;
  float *const vec = reinterpret_cast<float *>(osm + C::NSLOT_O * C::TSZ);
  float *const xp = vec + C::NSLOT_O * C::VSZ;

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
  const int grp = w & (NG - 1);                            // key group
  const bool pside = w < NG;                               // role
  const int h = lane >> 5, ln = lane & 31;
  const int kw0 = k0 + 32 * grp;
  const int my_k = kw0 + ln;

  // query tiles of the workgroup and of this key group (keys kw0 .. kw0 + 31 are seen by
  // queries kw0 .. kw0 + 31 + W - 1)
  const int k_last = min(T, k0 + C::BK) - 1;
  const int q_hi = window > 0 ? min(T - 1, k_last + window - 1) : T - 1;
  const int qt0 = k0 / C::BQ, qt1 = q_hi / C::BQ;
  int wqt0 = 1 << 30, wqt1 = -1;
  if (kw0 < T) {
    wqt0 = kw0 / C::BQ;
    wqt1 = (window > 0 ? min(T - 1, kw0 + 31 + window - 1) : T - 1) / C::BQ;
  }
  // tile wqt0 holds the diagonal; tiles from mlo on hold a query past some key's window
  const int mlo = window > 0 ? (kw0 + window - 31 + C::BQ - 1) / C::BQ : (1 << 30);
  // query qq sees key my_k iff 0 <= qq - my_k <= wm1
  const unsigned wm1 = window > 0 ? (unsigned)(window - 1) : 0x7fffffffu;

  // the stationary operand of the wave: K rows (P side) or V rows (dS side) of its keys
  // (B operands; rows past T read as zero), and its accumulators (dV or dK)
  bf16x8 kv[C::KST];
  f32x16 acc[C::NDB];
#pragma unroll
  for (int d = 0; d < C::NDB; ++d) acc[d] = f32x16{};
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
  // tile: this wave's destination (the Q or the dO tile of the slot, by my_tensor)
  // Tiles past the workgroup's last one (issued so that every step waits for the same
  // count) are copied from row T on: the buffer returns zeros and reads no memory.
  auto issue_to = [&](int qt, uint16_t *tile, float *vdst) {
    const int qr0 = qt <= qt1 ? qt * C::BQ : T;
    const uint32_t roff = (uint32_t)qr0 * (uint32_t)rs * 2;
#pragma unroll
    for (int cc = 0; cc < C::CPW; ++cc) {
      const int jj = (w * C::CPW + cc) % C::HALF;
      const int db = jj / C::RG, row16 = 16 * (jj % C::RG);
      buf_copy16_to_lds(rsrc_t, tile + db * (C::BQ * 32) + row16 * 32,
                        lane_off + (uint32_t)(row16 * rs + 32 * db) * 2 + roff);
    }
    // every wave issues exactly NCOPY copies per tile (lse by even waves, delta by odd
    // ones, each into its own 64 floats; waves 2 .. NW-1 fill spares), so the
    // end-of-step wait can count them
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsrc_v, (__attribute__((address_space(3))) void *)(vdst + w * 64), 4,
        (uint32_t)(lane + qr0) * 4, 0, 0, 0);
  };
  // qt >= 0 wherever a dO slot is taken (qt - 1 only indexes Q tiles)
  auto q_tile = [&](int qt) { return smem + (qt & (C::NSLOT - 1)) * C::TSZ; };
  auto o_tile = [&](int qt) { return osm + ((unsigned)qt % C::NSLOT_O) * C::TSZ; };
  auto vec_of = [&](int qt) { return vec + ((unsigned)qt % C::NSLOT_O) * C::VSZ; };
  auto xp_of = [&](int qt) { return xp + (2 * grp + (qt & 1)) * C::XSZ; };
  auto dst_of = [&](int qt) { return my_tensor ? o_tile(qt) : q_tile(qt); };
  auto issue = [&](int qt) { issue_to(qt, dst_of(qt), vec_of(qt)); };

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
  bf16x8 bsel;  // ones in K slots 0..2 (P side) or 8..10 (dS side)
#pragma unroll
  for (int j = 0; j < 8; ++j) bsel[j] = (__bf16)((h == (pside ? 0 : 1) && j < 3) ? 1.f : 0.f);
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
  // S' (P side: A = Q rows) or dP' (dS side: A = dO rows) of a tile, one key per lane:
  // register 8t + j of half h holds query 16t + 8h + j of the tile.
  auto sdp = [&](const uint16_t *__restrict__ rows, const float *__restrict__ vt, f32x16 &s) {
    bf16x8 a[C::KST];
#pragma unroll
    for (int st = 0; st < C::KST; ++st) a[st] = lds_read_b128(rows + dt_off<C::BQ>(ln, 2 * st + h));
    s = mfma32(bcast_op(vt[vrow]), bsel, f32x16{});
#pragma unroll
    for (int st = 0; st < C::KST; ++st) s = mfma32(a[st], kv[st], s);
  };
  // transposed operands (dO^T or Q^T) of rows 0..15 (t = 0) and 16..31 (t = 1)
  using TrOps = bf16x8[2][C::NDB];
  auto tr_ops = [&](const uint16_t *__restrict__ rows, TrOps &op) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int d = 0; d < C::NDB; ++d) op[t][d] = dt_read_tr_perm<C::BQ>(rows, 16 * t, d, lane);
  };
  auto grads = [&](const TrOps &op, const bf16x8 (&x)[2]) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int d = 0; d < C::NDB; ++d) acc[d] = mfma32(op[t][d], x[t], acc[d]);
  };

  // P side, tile qt: S', P (masked when MASK), P to the partner, dV^T += dO^T P.  P
  // enters dV as bf16; where some P of the wave's tile reaches kLoP, it enters as hi +
  // lo instead: hi = P truncated to bf16, lo = the exact remainder rounded to bf16
  // (P = hi + lo to ~2^-16 relative).  A single bf16 P on those large values leaves
  // |dV| >= 4 outside 2e-2 of the exact gradient; below kLoP the rounding of P
  // (<= 2^-13 absolute) is far inside it.
  auto p_side = [&](bool masked, int qt, const uint16_t *__restrict__ cur,
                    const uint16_t *__restrict__ curo, const float *__restrict__ vt,
                    float *__restrict__ xw) __attribute__((always_inline)) {
    f32x16 s;
    sdp(cur, vt, s);
    TrOps op;
    tr_ops(curo, op);  // dO^T, read while P is formed
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = fast_exp2(s[i] * c);
    // the element mask only changes P: the products below are the same code either way
    if (masked) {
      const int rel0 = qt * C::BQ + 8 * h - my_k;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        s[i] = (unsigned)(rel0 + 16 * (i >> 3) + (i & 7)) <= wm1 ? s[i] : 0.f;
    }
    float pm = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i += 2) pm = fmaxf(pm, fmaxf(s[i], s[i + 1]));
    // the partner lane (same lane of wave w + NG) reads these 16 values
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4)
      reinterpret_cast<f32x4 *>(xw)[64 * c4 + lane] =
          f32x4{s[4 * c4], s[4 * c4 + 1], s[4 * c4 + 2], s[4 * c4 + 3]};
    const bool lo = __builtin_amdgcn_ballot_w64(pm >= kLoP) != 0;
    bf16x8 ph[2];
    if (lo) {  // hi = P truncated
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 hp;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          hp[j] = __builtin_amdgcn_perm(__float_as_uint(s[8 * t + 2 * j + 1]),
                                        __float_as_uint(s[8 * t + 2 * j]), 0x07060302u);
        ph[t] = __builtin_bit_cast(bf16x8, hp);
      }
    } else {  // P rounded to nearest even
#pragma unroll
      for (int t = 0; t < 2; ++t) ph[t] = to_bf16x8(s, 8 * t);
    }
    grads(op, ph);
    if (lo) {  // lo = the exact remainder P - hi, rounded
      bf16x8 pl[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float a = s[8 * t + j];
          pl[t][j] = (__bf16)(a - __uint_as_float(__float_as_uint(a) & 0xffff0000u));
        }
      grads(op, pl);
    }
  };
  // dS side, tile qt - 1 (when DK): dS = P dP' with the partner's P, dK^T += Q^T dS; and
  // tile qt (when DP): dP' into dpn.  dS enters dK as one bf16 unless some |dS| of the
  // wave's tile reaches kLoDsK (D = 64): then also its remainder, rounded to bf16.
  auto ds_side = [&](bool do_dk, bool do_dp, const uint16_t *__restrict__ curo,
                     const float *__restrict__ vt, const uint16_t *__restrict__ prev,
                     const float *__restrict__ xr, f32x16 &dpp, f32x16 &dpn)
                     __attribute__((always_inline)) {
    if (do_dk) {
      TrOps op;
      tr_ops(prev, op);  // Q^T of tile qt - 1
      f32x16 p;
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const f32x4 x = reinterpret_cast<const f32x4 *>(xr)[64 * c4 + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[4 * c4 + e] = x[e];
      }
      float dm = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) dpp[i] = p[i] * dpp[i];
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kDsLoK<D>) {
#pragma unroll
        for (int i = 0; i < 16; i += 2) dm = fmaxf(dm, fmaxf(fabsf(dpp[i]), fabsf(dpp[i + 1])));
      }
      bf16x8 ds[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) ds[t] = to_bf16x8(dpp, 8 * t);
      grads(op, ds);
      if (kDsLoK<D> && __builtin_amdgcn_ballot_w64(dm >= kLoDsK) != 0) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            ds[t][j] = (__bf16)(dpp[8 * t + j] - (float)(__bf16)dpp[8 * t + j]);
        grads(op, ds);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (do_dp) sdp(curo, vt, dpn);
  };

  // Step qt: the copies of tile qt + AHEAD start (every step, also past the workgroup's
  // last tile: rows from T on read as zero and land in a slot no step reads, and the
  // wait count stays constant); the P side works on tile qt, the dS side on tiles
  // qt - 1 (dK) and qt (dP).  At the end, the wave's copies of tile qt + 1 and all its
  // LDS accesses are complete, then the barrier: tile qt + 1 and the P handed over in
  // this step are visible to every wave, and the slot of tile qt - 1 (read in this
  // step) is free for the copies of the next one.  The two roles run their own loops
  // (so neither holds the other's registers) over the same steps and barriers.  The
  // tiles and buffers come in as distinct restrict pointers, so the compiler does not
  // make the reads wait for the copies in flight.
  auto end_step = [&] {
    __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0<C::NCOPY>);
    lds_barrier();
  };
  auto p_step = [&](int qt, const uint16_t *__restrict__ cur, const uint16_t *__restrict__ curo,
                    const float *__restrict__ vt, float *__restrict__ xw,
                    uint16_t *__restrict__ dma, float *__restrict__ vdma)
                    __attribute__((always_inline)) {
    issue_to(qt + C::AHEAD, dma, vdma);
    if (qt >= wqt0 && qt <= wqt1) p_side(qt == wqt0 || qt >= mlo, qt, cur, curo, vt, xw);
    end_step();
  };
  auto ds_step = [&](int qt, const uint16_t *__restrict__ curo, const float *__restrict__ vt,
                     const uint16_t *__restrict__ prev, const float *__restrict__ xr,
                     uint16_t *__restrict__ dma, float *__restrict__ vdma, f32x16 &dpp,
                     f32x16 &dpn) __attribute__((always_inline)) {
    issue_to(qt + C::AHEAD, dma, vdma);
    ds_side(qt - 1 >= wqt0 && qt - 1 <= wqt1, qt >= wqt0 && qt <= wqt1, curo, vt, prev, xr,
            dpp, dpn);
    end_step();
  };

  // prologue: the stationary rows, then tiles qt0 and qt0 + 1, all awaited (with ROPE
  // the key transform runs while the copies are in flight: the rows were issued first)
  {
    const __amdgpu_buffer_rsrc_t rkv = make_rsrc(pside ? kb : vb, (uint32_t)T * rsk * 2);
#pragma unroll
    for (int st = 0; st < C::KST; ++st)
      kv[st] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                              rkv, (my_k * rsk + 16 * st + 8 * h) * 2, 0, 0));
  }
  issue(qt0);
  issue(qt0 + 1);
  if constexpr (ROPE) {
    if (pside) rope_norm_operand<D>(kv, rope_pos(ra, b, my_k), my_k < T, ra, h);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmLgkm0<0>);
  lds_barrier();

  // steps qt0 .. qt1 + 1 (the dS side's dK trails its dP by one step)
  if (pside) {
    for (int qt = qt0; qt <= qt1 + 1; ++qt)
      p_step(qt, q_tile(qt), o_tile(qt), vec_of(qt), xp_of(qt), dst_of(qt + C::AHEAD),
             vec_of(qt + C::AHEAD));
  } else {
    f32x16 dpa = f32x16{}, dpb = f32x16{};
    int qt = qt0;
    // two steps per iteration: dP' alternates between dpa and dpb
    for (; qt + 1 <= qt1 + 1; qt += 2) {
      ds_step(qt, o_tile(qt), vec_of(qt), q_tile(qt - 1), xp_of(qt - 1), dst_of(qt + C::AHEAD),
              vec_of(qt + C::AHEAD), dpa, dpb);
      ds_step(qt + 1, o_tile(qt + 1), vec_of(qt + 1), q_tile(qt), xp_of(qt),
              dst_of(qt + 1 + C::AHEAD), vec_of(qt + 1 + C::AHEAD), dpb, dpa);
    }
    if (qt == qt1 + 1)
      ds_step(qt, o_tile(qt), vec_of(qt), q_tile(qt - 1), xp_of(qt - 1), dst_of(qt + C::AHEAD),
              vec_of(qt + C::AHEAD), dpa, dpb);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm<0>);  // no copy into LDS outlives the workgroup

  // dk, dv through LDS, in the tile slots once every wave's copies have landed and
  // every wave has finished its reads: bf16 rows (stage_rows_bf16), or the fp32
  // partials half a row at a time (stage_rows_f32_half; the same bytes per wave).
  // Every wave of either role passes the same barriers.
  static_assert(C::NW * 32 * D <= (C::NSLOT + C::NSLOT_O) * C::TSZ,
                "the waves' rows fit the tile slots");
  __syncthreads();
  uint16_t *stage = smem + w * 32 * D;
  auto store_rows = [&](float mul, float *part, uint16_t *out) {
    if constexpr (PARTIAL) {
      float *fs = reinterpret_cast<float *>(stage);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        if (half) __syncthreads();  // the first half has been read back
        stage_rows_f32_half<D>(fs, acc, mul, ln, h, half);
        __syncthreads();
        store_staged_rows_f32_half<D>(fs, lane, T - kw0, part + base + (size_t)kw0 * rs, rs,
                                      half);
      }
    } else {
      stage_rows_bf16<D>(stage, acc, mul, ln, h);
      __syncthreads();
      store_staged_rows<D>(stage, lane, T - kw0, out + base_kv + (size_t)kw0 * rsk, rsk);
    }
  };

  if constexpr (ROPE) {
    if (!pside) {
      // dk: back through the prologue, with the raw key row read again (every lane of
      // the wave takes part: the reductions pair lanes l and l ^ 32); the key index and
      // the frequency ratio made opaque, so that nothing of the P side's prologue is
      // held in registers through the loop for this.  With K/V head groups this query
      // head's share of dk' is mapped (the map is linear in dk' for the fixed raw row,
      // so the group sum of the mapped shares is dk) and written as an fp32 partial.
      int ki = my_k;
      RopeArgs re = ra;
      asm volatile("" : "+v"(ki), "+s"(re.ratio));
#pragma unroll
      for (int d = 0; d < C::NDB; ++d) acc[d] *= scale;
      f32x16 xr[C::NDB];
      load_acc_order<D>(kb + (size_t)min(ki, T - 1) * rsk, h, xr);
      rope_norm_grad_acc<D>(acc, xr, rope_pos(re, b, ki), ki < T, re, h);
      store_rows(1.f, part_k, dk);
      return;
    }
  }
  store_rows(pside ? 1.f : scale, pside ? part_v : part_k, pside ? dv : dk);
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

// Windows up to this many keys (and shorter than the sequence) take two key groups per
// workgroup: a 128-key block under a window W walks (W + 127) / 32 query tiles while
// each of its groups works on (W + 31) / 32 of them, and the two waves of a group share
// a SIMD, so that SIMD idles through the rest; two 64-key workgroups per CU cover each
// other's idle steps and prologues.
constexpr int kDkdvShortWindow = 512;

template <int D, bool PARTIAL, bool ROPE, int NG>
static void launch_dkdv_ng(const void *q, const void *k, const void *v, const void *dO,
                           const float *lse, const float *delta, void *dk, void *dv,
                           float *part_k, float *part_v, int B, int H, int Hkv, int T,
                           int window, float scale, hipStream_t st, const RopeArgs &ra) {
  using C = DkdvCfg<D, NG>;
  const int nkt = (T + C::BK - 1) / C::BK;
  const unsigned nb = (unsigned)(nkt * B * H);
  bwd_dkdv_bf16_kernel<D, PARTIAL, ROPE, NG><<<nb, C::NW * 64, 0, st>>>(
      (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (const uint16_t *)dO, lse,
      delta, (uint16_t *)dk, (uint16_t *)dv, part_k, part_v, B, H, Hkv, T, window, scale, nkt, ra);
}

template <int D, bool PARTIAL, bool ROPE = false>
static void launch_dkdv_t(const void *q, const void *k, const void *v, const void *dO,
                          const float *lse, const float *delta, void *dk, void *dv,
                          float *part_k, float *part_v, int B, int H, int Hkv, int T, int window,
                          float scale, hipStream_t st, const RopeArgs &ra = RopeArgs{}) {
  if (window > 0 && window <= kDkdvShortWindow && window < T)
    launch_dkdv_ng<D, PARTIAL, ROPE, 2>(q, k, v, dO, lse, delta, dk, dv, part_k, part_v, B, H,
                                        Hkv, T, window, scale, st, ra);
  else
    launch_dkdv_ng<D, PARTIAL, ROPE, 4>(q, k, v, dO, lse, delta, dk, dv, part_k, part_v, B, H,
                                        Hkv, T, window, scale, st, ra);
}

hipError_t launch_bwd_dkdv_bf16(const void *q, const void *k, const void *v, const void *dO,
                                const float *lse, const float *delta, void *dk, void *dv,
                                float *part, int B, int H, int Hkv, int T, int D, int window,
                                float scale, hipStream_t st, const RopeArgs *rope) {
  if (rope != nullptr && Hkv == H) {
    if (D == 128)
      launch_dkdv_t<128, false, true>(q, k, v, dO, lse, delta, dk, dv, nullptr, nullptr, B, H, H,
                                      T, window, scale, st, *rope);
    else
      launch_dkdv_t<64, false, true>(q, k, v, dO, lse, delta, dk, dv, nullptr, nullptr, B, H, H,
                                     T, window, scale, st, *rope);
    return hipGetLastError();
  }
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
  if (rope != nullptr) {
    if (D == 128)
      launch_dkdv_t<128, true, true>(q, k, v, dO, lse, delta, dk, dv, part_k, part_v, B, H, Hkv,
                                     T, window, scale, st, *rope);
    else
      launch_dkdv_t<64, true, true>(q, k, v, dO, lse, delta, dk, dv, part_k, part_v, B, H, Hkv,
                                    T, window, scale, st, *rope);
  } else if (D == 128) {
    launch_dkdv_t<128, true>(q, k, v, dO, lse, delta, dk, dv, part_k, part_v, B, H, Hkv, T,
                             window, scale, st);
  } else {
    launch_dkdv_t<64, true>(q, k, v, dO, lse, delta, dk, dv, part_k, part_v, B, H, Hkv, T,
                            window, scale, st);
  }
  const long long n8 = (long long)B * T * Hkv * D / 8;
  dkdv_group_sum_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>(
      part_k, part_v, (uint16_t *)dk, (uint16_t *)dv, n8, H / Hkv, D);
  return hipGetLastError();
}

}  // namespace swattn

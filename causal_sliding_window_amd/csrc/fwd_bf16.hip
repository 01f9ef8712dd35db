// Forward of causal sliding-window attention, bf16 in / bf16 out, fp32 accumulate.
//
// Computes o = softmax(scale * Q K^T, causal + window mask) V and the natural-log
// LSE per query row: the attention call of the nanochat guide's section 5 ("Flash
// Attention unification") with the sliding window of its section 1 feature list.
//
// Work decomposition (one workgroup = NW waves = 32 NW queries of one (b, h); NW = 4,
// or 2 for short windows):
//   * each wave owns 32 queries; its Q block stays in registers as the MFMA B
//     operand of S^T = K Q^T (32 keys x 32 queries per MFMA tile), so a lane owns
//     one query and the row statistics are per lane plus one cross-half exchange;
//   * K and V tiles of 32 keys reach LDS by direct buffer -> LDS copies (no
//     register staging; rows past T read as zero), d-block-major with a chunk XOR
//     so that operand reads are free of bank conflicts; K rows in swap23 order so
//     the C registers of S^T are already the B operand of O^T = V^T P^T;
//   * K runs one tile ahead of V: while tile j's softmax runs on the vector ALU,
//     the MFMAs of S for tile j + 1 are issued between its instructions, then
//     P_j V_j follows.  Each wave only computes the tiles of its own band;
//   * the running max is only moved (and O rescaled) when a row max grows by
//     more than 2^8 in exp2 units, which keeps every P below 256;
//   * the element mask runs only on tiles crossing the diagonal or the window's
//     lower edge;
//   * the unmasked loop is aligned so that its two steps always use the same LDS
//     slots: every operand address is then a lane offset plus a constant.
//
// The same kernel serves chunked prefill (PREFILL): T query rows of a sequence sit at
// positions off .. off + T - 1 of a KV cache of Tkv rows, which already holds the
// chunk's own K/V rows (cache_append_kernel runs first), with off = seqlens[b] read
// on the device and clamped to [0, Tkv - T].  Work per (sequence, query tile) grows
// with off, so the prefill grid takes its items longest first (sequences ranked by
// off on the device).  Band, masks and tiles work in absolute
// positions; q, o and lse are indexed within the chunk.  With off not a multiple of
// 32 a wave's diagonal spans two key tiles, so every tile from the first one the
// diagonal touches runs the element mask.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "rope.h"

namespace swattn {

template <int D, int NW = 4>
struct FwdCfg {
  static constexpr int BM = 32 * NW;           // queries per workgroup (NW waves x 32)
  static constexpr int BN = 32;                // keys per tile
  static constexpr int KST = D / 16;           // k-steps of S over D
  static constexpr int NDB = D / 32;           // 32-column blocks of D
  static constexpr int TSZ = BN * D;           // elements of one K or V tile
  static constexpr int RG = BN / 16;           // 16-row groups per 32-column block
  static constexpr int CPW = TSZ * 2 / 1024 / NW;  // 1-KB copies per wave and tile
};

// Short windows: a workgroup steps through every key tile of its waves' bands, and each
// wave computes only those of its own band.  With windows up to this size the forward
// takes workgroups of 2 waves (64 queries), whose bands overlap more: at W = 256 a wave
// computes 9 of the 10 tiles its workgroup visits, against 9 of 12 with 4 waves.
constexpr int kShortWindow = 512;

// Prefill: up to this many sequences, workgroups take (sequence, query tile) items
// longest first, ranked on the device by cache offset.
constexpr int kPrefillOrderMaxB = 256;

// Row-max growth (exp2 units) tolerated before the running max is moved.
constexpr float kRescaleLog2 = 8.f;

// ROPE: q holds the raw queries; each is normalised and rotated (QK norm + rotary
// embedding) as it is loaded into registers, and written to q_rope when that is not null.
template <int D, bool PREFILL, bool ROPE = false, int NW = 4>
__global__ __launch_bounds__(64 * NW, 2) void fwd_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, uint16_t *__restrict__ o, float *__restrict__ lse,
    const int *__restrict__ seqlens, int B, int H, int Hkv, int T, int Tkv, int window,
    float scale, int nqt, RopeArgs ra = RopeArgs{}, uint16_t *__restrict__ q_rope = nullptr) {
  using C = FwdCfg<D, NW>;
  // [slot][K, V][TSZ]
  __shared__ __attribute__((aligned(1024))) uint16_t smem[2 * 2 * C::TSZ];

  const int BH = B * H;
  const int bid = blockIdx.x;
  int qt, bh, b, hh;
  if (PREFILL && B <= kPrefillOrderMaxB) {
    // longest work first: sequences by cache offset, largest first (ties by index),
    // then query tiles latest first, then heads.  Every workgroup ranks the B offsets
    // itself from LDS; the ranks are a permutation, so exactly one sequence matches.
    __shared__ int pick, offs[kPrefillOrderMaxB];
    const int per_seq = nqt * H;
    const int want = bid / per_seq;
    for (int bb = threadIdx.x; bb < B; bb += blockDim.x)
      offs[bb] = min(max(seqlens[bb], 0), Tkv - T);
    __syncthreads();
    for (int bb = threadIdx.x; bb < B; bb += blockDim.x) {
      const int ob = offs[bb];
      int r = 0;
      for (int j = 0; j < B; ++j) r += (offs[j] > ob) || (offs[j] == ob && j < bb);
      if (r == want) pick = bb;
    }
    __syncthreads();
    b = pick;
    const int rem = bid - want * per_seq;
    qt = nqt - 1 - rem / H;
    hh = rem % H;
    bh = b * H + hh;
  } else {
    qt = nqt - 1 - bid / BH;  // longest (latest) query tiles first
    bh = bid % BH;            // consecutive blocks: different heads
    b = bh / H;
    hh = bh % H;
  }
  // positions of the chunk's queries start at off; keys 0 .. Tk - 1 are in view
  const int off = PREFILL ? min(max(seqlens[b], 0), Tkv - T) : 0;
  const int Tk = off + T;
  const int q0 = off + qt * C::BM;
  const int rs = H * D;                // row stride of q and o (elements)
  const int rsk = Hkv * D;             // row stride of k and v
  const int hk = hh / (H / Hkv);       // the K/V head of query head hh
  const size_t base = ((size_t)b * T * H + hh) * D;
  const size_t base_kv = ((size_t)b * Tkv * Hkv + hk) * D;
  const uint16_t *qb = q + base, *kb = k + base_kv, *vb = v + base_kv;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, held in an SGPR
  const int h = lane >> 5, ln = lane & 31;
  const int qw0 = q0 + 32 * w;
  const int my_q = qw0 + ln;

  // key tiles of the workgroup and of this wave
  const int q_last = min(Tk, q0 + C::BM) - 1;
  const int k_lo = window > 0 ? max(0, q0 - window + 1) : 0;
  const int kt0 = k_lo / C::BN, kt1 = q_last / C::BN;
  int wkt0 = 1 << 30, wkt1 = -1;
  if (qw0 < Tk) {
    wkt0 = (window > 0 ? max(0, qw0 - window + 1) : 0) / C::BN;
    wkt1 = min(Tk - 1, qw0 + 31) / C::BN;
  }
  const int wq_lo = qw0, wq_hi = min(Tk - 1, qw0 + 31);
  // key kk is visible to my_q iff 0 <= my_q - kk <= wm1
  const unsigned wm1 = window > 0 ? (unsigned)(window - 1) : 0x7fffffffu;

  // Q block (B operand), rows past T read as zero
  bf16x8 qr[C::KST];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qb, (uint32_t)T * rs * 2);
#pragma unroll
    for (int st = 0; st < C::KST; ++st)
      qr[st] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, ((my_q - off) * rs + 16 * st + 8 * h) * 2,
                                                        0, 0));
  }

  // Copy j of a tile (1 KB): LDS block db = j / RG, rows 16 (j % RG) .. + 15.
  // Lane part of the source offset; this wave issues copies CPW w .. CPW w + CPW - 1.
  const int rl = lane >> 2;                          // LDS row within the 16-row group
  const int lc = (lane & 3) ^ ((lane >> 4) & 3);     // logical chunk stored at this position
  const uint32_t klane = (swap23(rl) * rsk + 8 * lc) * 2;
  const uint32_t vlane = (rl * rsk + 8 * lc) * 2;
  auto issue = [&](int tensor, int kt, int slot) {
    const uint16_t *src = tensor ? vb : kb;
    const int row0 = kt * C::BN;
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(src + (size_t)row0 * rsk, (uint32_t)(Tk - row0) * rsk * 2);
    uint16_t *tile = smem + (2 * slot + tensor) * C::TSZ;
#pragma unroll
    for (int cc = 0; cc < C::CPW; ++cc) {
      const int j = C::CPW * w + cc;
      const int db = j / C::RG, row16 = 16 * (j % C::RG);
      buf_copy16_to_lds(r, tile + db * (C::BN * 32) + row16 * 32,
                        (tensor ? vlane : klane) + (row16 * rsk + 32 * db) * 2);
    }
  };

  f32x16 acc[C::NDB];
#pragma unroll
  for (int d = 0; d < C::NDB; ++d) acc[d] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = scale * kLog2e;
  const float thr = kRescaleLog2 / c;

  // S^T of one tile: register i of a lane in half h holds key c_row(i, h),
  // query = lane % 32.
  auto qk = [&](const uint16_t *Kt, f32x16 &s) {
    bf16x8 ka[C::KST];
#pragma unroll
    for (int st = 0; st < C::KST; ++st) ka[st] = lds_read_b128(Kt + dt_off<C::BN>(ln, 2 * st + h));
#pragma unroll
    for (int st = 0; st < C::KST; ++st) s = mfma32(ka[st], qr[st], st ? s : f32x16{});
  };

  // Online softmax of one tile: masks (MASK), updates m_run / l_run, returns P as
  // bf16 B operands and whether O must be rescaled by alpha.
  auto softmax = [&](auto mask_tag, f32x16 &s, int kbase, bf16x8 (&p)[2], float &alpha) -> bool {
    constexpr bool MASK = decltype(mask_tag)::value;
    if constexpr (MASK) {
      const int rel0 = my_q - kbase - 8 * h;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((unsigned)(rel0 - c_row(i, 0)) > wm1) s[i] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = xhalf_max(mx);
    const bool need = __builtin_amdgcn_ballot_w64(mx > m_run + thr) != 0;
    const float m_new = need ? fmaxf(m_run, mx) : m_run;
    const float mc = (m_new == -INFINITY ? 0.f : m_new) * c;
    alpha = fast_exp2(m_run * c - mc);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = fast_exp2(fmaf(s[i], c, -mc));
      s[i] = e;
      psum += e;
    }
    l_run = fmaf(l_run, alpha, psum);
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < 2; ++t) p[t] = to_bf16x8(s, 8 * t);
    return need;
  };

  // V^T operands of a tile (transposed LDS reads), then O += P V.
  using VOps = bf16x8[2][C::NDB];
  auto v_reads = [&](const uint16_t *Vt, VOps &va) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int d = 0; d < C::NDB; ++d) va[t][d] = dt_read_tr<C::BN>(Vt, 16 * t, d, lane);
  };
  // O rescale (when some row max moved) and O += P V of a tile.  The PV MFMAs are
  // issued at raised wave priority: with two waves per SIMD, the one holding a
  // run of MFMAs then keeps the matrix unit busy while the other issues vector
  // work in between.
  auto finish = [&](bool need, float alpha, const VOps &va, const bf16x8 (&p)[2]) {
    if (need) {
#pragma unroll
      for (int d = 0; d < C::NDB; ++d) acc[d] *= alpha;
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int d = 0; d < C::NDB; ++d) acc[d] = mfma32(va[t][d], p[t], acc[d]);
    __builtin_amdgcn_s_setprio(0);
  };

  // Softmax of tile kt (S in sc) with the S MFMAs of tile kt + 1 (into sn) issued
  // between its instructions, then O += P V for tile kt.  The order is fixed by
  // hand: one MFMA, then a slice of the softmax that runs on the vector ALU while
  // the MFMA executes; sched_barrier keeps the compiler from regrouping them.
  // All LDS operand reads of the step are issued before the step's copies into
  // LDS start (`issue_loads`), so no read has to wait for those copies.
  auto step = [&](auto mask_tag, auto issue_loads, const uint16_t *Kn, const uint16_t *Vt,
                  int kbase, f32x16 &sc, f32x16 &sn) {
    constexpr bool MASK = decltype(mask_tag)::value;
    static_assert(C::KST == 8 || C::KST == 4, "");
    bf16x8 ka[C::KST];
#pragma unroll
    for (int st = 0; st < C::KST; ++st) ka[st] = lds_read_b128(Kn + dt_off<C::BN>(ln, 2 * st + h));
    VOps va;
    v_reads(Vt, va);
    __builtin_amdgcn_sched_barrier(0);
    issue_loads();
    __builtin_amdgcn_sched_barrier(0);
    int st = 0;
    // an empty asm use keeps a slice's result from drifting to its later uses
    auto pin = [](float x) {
      asm volatile("" ::"v"(x));
      __builtin_amdgcn_sched_barrier(0);
    };
    auto mfma_next = [&] {
      sn = mfma32(ka[st], qr[st], st ? sn : f32x16{});
      ++st;
      __builtin_amdgcn_sched_barrier(0);
    };
    // slice 1: mask, row max
    mfma_next();
    if constexpr (MASK) {
      const int rel0 = my_q - kbase - 8 * h;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((unsigned)(rel0 - c_row(i, 0)) > wm1) sc[i] = -INFINITY;
    }
    float mx = fmaxf(sc[0], sc[1]);
#pragma unroll
    for (int i = 2; i < 16; ++i) mx = fmaxf(mx, sc[i]);
    pin(mx);
    // slice 2: cross-half max, rescale decision
    mfma_next();
    mx = xhalf_max(mx);
    const bool need = __builtin_amdgcn_ballot_w64(mx > m_run + thr) != 0;
    const float m_new = need ? fmaxf(m_run, mx) : m_run;
    const float mc = (m_new == -INFINITY ? 0.f : m_new) * c;
    const float alpha = fast_exp2(m_run * c - mc);
    pin(mc);
    // slices 3..: exponentials and their sum, 16 / (KST - 3) per slice, then P
    float psum = 0.f;
    constexpr int NE = C::KST == 8 ? 4 : 8;   // exponentials per slice
#pragma unroll
    for (int e0 = 0; e0 < 16; e0 += NE) {
      mfma_next();
#pragma unroll
      for (int i = e0; i < e0 + NE; ++i) {
        const float e = fast_exp2(fmaf(sc[i], c, -mc));
        sc[i] = e;
        psum += e;
      }
      pin(psum);
    }
    bf16x8 p[2];
    while (st < C::KST) mfma_next();
#pragma unroll
    for (int t = 0; t < 2; ++t) p[t] = to_bf16x8(sc, 8 * t);
    l_run = fmaf(l_run, alpha, psum);
    m_run = m_new;
    __builtin_amdgcn_sched_barrier(0);
    finish(need, alpha, va, p);
  };

  // Tile pipeline.  K of tile t and V of tile t live in LDS slot (t - kt0) & 1; K
  // runs one tile ahead, so in step kt the copies of K[kt + 2] (over K[kt], read in
  // step kt - 1) and V[kt + 1] (over V[kt - 1]) are issued, and they are awaited
  // at the end of the step.  Every wave runs one barrier per
  // tile of the workgroup; the phases below only differ in what a wave computes.
  auto loads = [&](int kt) {
    const int slot = (kt - kt0) & 1;
    if (kt + 2 <= kt1) issue(0, kt + 2, slot);
    if (kt + 1 <= kt1) issue(1, kt + 1, slot ^ 1);
  };
  auto k_next = [&](int kt) { return smem + 2 * (((kt - kt0) & 1) ^ 1) * C::TSZ; };
  auto v_cur = [&](int kt) { return smem + (2 * ((kt - kt0) & 1) + 1) * C::TSZ; };
  auto sync = [&] {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  // prologue: K, V of tile kt0 and K of kt0 + 1 (and with ROPE the query transform
  // while those copies are in flight)
  issue(0, kt0, 0);
  issue(1, kt0, 0);
  if (kt0 < kt1) issue(0, kt0 + 1, 1);
  if constexpr (ROPE) {
    rope_norm_operand<D>(qr, rope_pos(ra, b, my_q - off), my_q < Tk, ra, h);
    if (q_rope != nullptr && my_q < Tk) {
      uint16_t *qo = q_rope + base + (size_t)(my_q - off) * rs + 8 * h;
#pragma unroll
      for (int st = 0; st < C::KST; ++st) *reinterpret_cast<bf16x8 *>(qo + 16 * st) = qr[st];
    }
  }
  sync();
  f32x16 sc, sn;
  if (wkt0 == kt0) qk(smem, sc);
  __syncthreads();

  // Tiles [wkt0, mlim) cross the window's lower edge and need the element mask;
  // the wave's last tile (wkt1) holds its diagonal.
  const int mlim = (window > 0 && wq_hi - window >= 0) ? (wq_hi - window) / C::BN + 1 : 0;
  int kt = kt0;
  for (; kt < min(wkt0 - 1, kt1 + 1); ++kt) {  // before the wave's band (or all tiles)
    loads(kt);
    sync();
  }
  if (wkt0 > kt0 && kt == wkt0 - 1) {  // S of the wave's first tile
    loads(kt);
    qk(k_next(kt), sc);
    sync();
    ++kt;
  }
  for (; kt < min(wkt1, mlim); ++kt) {
    step(std::true_type{}, [&] { loads(kt); }, k_next(kt), v_cur(kt), kt * C::BN, sc, sn);
    sc = sn;
    sync();
  }
  // Tiles from ulim on hold keys past some query of the wave (only the diagonal tile
  // wkt1 when the wave's queries start on a tile boundary).
  const int ulim = PREFILL ? min(wkt1, (qw0 + 1) / C::BN) : wkt1;
  // unmasked tiles, two per iteration: S of the next tile alternates between sc and
  // sn, so no registers are copied
  if (kt + 1 < ulim && ((kt - kt0) & 1)) {  // align the pair loop to slot 0
    step(std::false_type{}, [&] { loads(kt); }, k_next(kt), v_cur(kt), kt * C::BN, sc, sn);
    sc = sn;
    sync();
    ++kt;
  }
  // (kt - kt0) is even here: the slots of both steps are fixed, so every LDS address
  // is a loop-invariant lane offset plus a constant
  for (; kt + 1 < ulim; kt += 2) {
    step(std::false_type{}, [&] { loads(kt); }, smem + 2 * C::TSZ, smem + C::TSZ, kt * C::BN, sc,
         sn);
    sync();
    step(std::false_type{}, [&] { loads(kt + 1); }, smem, smem + 3 * C::TSZ, (kt + 1) * C::BN, sn,
         sc);
    sync();
  }
  if (kt < ulim) {
    step(std::false_type{}, [&] { loads(kt); }, k_next(kt), v_cur(kt), kt * C::BN, sc, sn);
    sc = sn;
    sync();
    ++kt;
  }
  if constexpr (PREFILL) {
    for (; kt < wkt1; ++kt) {  // tiles before the last one that the diagonal crosses
      step(std::true_type{}, [&] { loads(kt); }, k_next(kt), v_cur(kt), kt * C::BN, sc, sn);
      sc = sn;
      sync();
    }
  }
  if (kt == wkt1) {  // the diagonal tile: no S to compute ahead
    VOps va;
    v_reads(v_cur(kt), va);
    __builtin_amdgcn_sched_barrier(0);
    loads(kt);
    bf16x8 p[2];
    float alpha;
    const bool need = softmax(std::true_type{}, sc, kt * C::BN, p, alpha);
    finish(need, alpha, va, p);
    sync();
    ++kt;
  }
  for (; kt <= kt1; ++kt) {  // after the wave's band
    loads(kt);
    sync();
  }

  const float l_tot = xhalf_sum(l_run);
  // o through LDS (stage_rows_bf16): the tile slots are free here, since every copy
  // has landed and every wave has passed the last barrier of the loop
  static_assert(NW * 32 * D <= 2 * 2 * C::TSZ, "the waves' rows fit the tile slots");
  uint16_t *stage = smem + w * 32 * D;
  stage_rows_bf16<D>(stage, acc, my_q < Tk ? 1.f / l_tot : 0.f, ln, h);
  __syncthreads();
  store_staged_rows<D>(stage, lane, Tk - qw0, o + base + (size_t)(qw0 - off) * rs, rs);
  if (my_q < Tk && h == 0 && (!PREFILL || lse != nullptr))
    lse[(size_t)bh * T + (my_q - off)] = m_run * scale + logf(l_tot);
}

template <int D, int NW>
static void launch_fwd_t(const void *q, const void *k, const void *v, void *o, float *lse, int B,
                         int H, int Hkv, int T, int window, float scale, hipStream_t st) {
  const int nqt = (T + FwdCfg<D, NW>::BM - 1) / FwdCfg<D, NW>::BM;
  fwd_bf16_kernel<D, false, false, NW><<<dim3((unsigned)(nqt * B * H)), dim3(64 * NW), 0, st>>>(
      (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (uint16_t *)o, lse, nullptr,
      B, H, Hkv, T, T, window, scale, nqt);
}

hipError_t launch_fwd_bf16(const void *q, const void *k, const void *v, void *o, float *lse,
                           int B, int H, int Hkv, int T, int D, int window, float scale,
                           hipStream_t st) {
  const bool short_w = window > 0 && window <= kShortWindow && window < T;
  if (D == 128) {
    if (short_w)
      launch_fwd_t<128, 2>(q, k, v, o, lse, B, H, Hkv, T, window, scale, st);
    else
      launch_fwd_t<128, 4>(q, k, v, o, lse, B, H, Hkv, T, window, scale, st);
  } else {
    if (short_w)
      launch_fwd_t<64, 2>(q, k, v, o, lse, B, H, Hkv, T, window, scale, st);
    else
      launch_fwd_t<64, 4>(q, k, v, o, lse, B, H, Hkv, T, window, scale, st);
  }
  return hipGetLastError();
}

template <int D, int NW>
static void launch_fwd_rope_t(const void *q, const void *k, const void *v, void *o, float *lse,
                              void *q_rope, int B, int H, int Hkv, int T, int window,
                              float scale, const RopeArgs &ra, hipStream_t st) {
  const int nqt = (T + FwdCfg<D, NW>::BM - 1) / FwdCfg<D, NW>::BM;
  fwd_bf16_kernel<D, false, true, NW><<<dim3((unsigned)(nqt * B * H)), dim3(64 * NW), 0, st>>>(
      (const uint16_t *)q, (const uint16_t *)k, (const uint16_t *)v, (uint16_t *)o, lse, nullptr,
      B, H, Hkv, T, T, window, scale, nqt, ra, (uint16_t *)q_rope);
}

hipError_t launch_fwd_bf16_rope(const void *q, const void *k, const void *v, void *o, float *lse,
                                void *q_rope, int B, int H, int Hkv, int T, int D, int window,
                                float scale, const RopeArgs &ra, hipStream_t st) {
  const bool short_w = window > 0 && window <= kShortWindow && window < T;
  if (D == 128) {
    if (short_w)
      launch_fwd_rope_t<128, 2>(q, k, v, o, lse, q_rope, B, H, Hkv, T, window, scale, ra, st);
    else
      launch_fwd_rope_t<128, 4>(q, k, v, o, lse, q_rope, B, H, Hkv, T, window, scale, ra, st);
  } else {
    if (short_w)
      launch_fwd_rope_t<64, 2>(q, k, v, o, lse, q_rope, B, H, Hkv, T, window, scale, ra, st);
    else
      launch_fwd_rope_t<64, 4>(q, k, v, o, lse, q_rope, B, H, Hkv, T, window, scale, ra, st);
  }
  return hipGetLastError();
}

// Rows t of the chunk go to cache rows off_b + t, off_b = seqlens[b] clamped to
// [0, Tmax - Tq] (the same clamp as the prefill forward); 8 elements per thread.
__global__ __launch_bounds__(256) void cache_append_kernel(
    const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new,
    uint16_t *__restrict__ k_cache, uint16_t *__restrict__ v_cache,
    const int *__restrict__ seqlens, int Tq, int Hkv, int D, int Tmax, long long n8) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const long long e = i * 8;               // element of k_new: ((b Tq + t) Hkv + hk) D + d
  const long long row = e / D, d = e % D;  // row = (b Tq + t) Hkv + hk
  const long long hk = row % Hkv, bt = row / Hkv;
  const long long t = bt % Tq, b = bt / Tq;
  const int off = min(max(seqlens[b], 0), Tmax - Tq);
  const long long dst = ((b * Tmax + off + t) * Hkv + hk) * D + d;
  *reinterpret_cast<u32x4 *>(k_cache + dst) = *reinterpret_cast<const u32x4 *>(k_new + e);
  *reinterpret_cast<u32x4 *>(v_cache + dst) = *reinterpret_cast<const u32x4 *>(v_new + e);
}

hipError_t launch_prefill_bf16(const void *q, const void *k_new, const void *v_new,
                               void *k_cache, void *v_cache, const int *seqlens, void *o,
                               float *lse, int B, int H, int Hkv, int Tq, int D, int Tmax,
                               int window, float scale, hipStream_t st) {
  const long long n8 = (long long)B * Tq * Hkv * D / 8;
  cache_append_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>(
      (const uint16_t *)k_new, (const uint16_t *)v_new, (uint16_t *)k_cache,
      (uint16_t *)v_cache, seqlens, Tq, Hkv, D, Tmax, n8);
  const int nqt = (Tq + FwdCfg<128>::BM - 1) / FwdCfg<128>::BM;
  dim3 grid((unsigned)(nqt * B * H)), block(256);
  if (D == 128)
    fwd_bf16_kernel<128, true><<<grid, block, 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)k_cache, (const uint16_t *)v_cache, (uint16_t *)o,
        lse, seqlens, B, H, Hkv, Tq, Tmax, window, scale, nqt);
  else
    fwd_bf16_kernel<64, true><<<grid, block, 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)k_cache, (const uint16_t *)v_cache, (uint16_t *)o,
        lse, seqlens, B, H, Hkv, Tq, Tmax, window, scale, nqt);
  return hipGetLastError();
}

}  // namespace swattn

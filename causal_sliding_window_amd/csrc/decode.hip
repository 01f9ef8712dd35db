// One-token KV-cache decode (nanochat guide, section 6 "Inference engine": the
// engine decodes one token per step against the cache its attention kernels
// read).  Bound by HBM: every visible K/V cache row is read exactly once.
//
// decode_split_kernel: workgroup (K/V head hk, chunk c, sequence b) reads seqlens[b]
//   on the device, takes its chunk of the visible range [max(0, L - W), L) (32 rows per
//   wave: kDecodeChunkWide rows in 8 waves ungrouped, kDecodeChunk in 4 grouped), and
//   for each query head that reads K/V head hk (H / Hkv of them; one without
//   grouping) writes a partial (o_c normalised, lse_c) to the workspace (or o and lse
//   directly when the visible range is one chunk).  The cache rows are read once per
//   group, not once per query head.  Each
//   K/V row of one head is 256 contiguous bytes (bf16, D = 128) read by D/8 lanes
//   with non-temporal 16-byte loads; every wave requests all of its rows before
//   using any.
// decode_gqa_mfma_kernel: the same split for bf16, D = 128 and groups of at least
//   kGqaMfmaMinGroup query heads per K/V head, on the matrix cores (the group's heads
//   are the columns of S^T = K Q^T and of O^T = V^T P); same workspace and partials.
// decode_merge_kernel: lse = ln sum_c exp(lse_c), o = sum_c exp(lse_c - lse) o_c.
//   A separate launch: merging inside the split kernel needs agent-scope fences,
//   which on this chip write back and invalidate an XCD's whole L2 per workgroup.
#include "common.h"
#include "launch.h"

#include <type_traits>

namespace swattn {

int decode_num_splits(int Tmax, int window) {
  const int vis = window > 0 ? (window < Tmax ? window : Tmax) : Tmax;
  return (vis + kDecodeChunk - 1) / kDecodeChunk;
}

template <typename TT> struct Elem;
template <> struct Elem<uint16_t> {
  static constexpr int PER16 = 8;
  __device__ static void unpack(const u32x4 &x, float *f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = bf16_lo(x[e]);
      f[2 * e + 1] = bf16_hi(x[e]);
    }
  }
  __device__ static uint16_t pack(float x) { return f32_to_bf16_bits(x); }
};
template <> struct Elem<float> {
  static constexpr int PER16 = 4;
  __device__ static void unpack(const u32x4 &x, float *f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(x[e]);
  }
  __device__ static float pack(float x) { return x; }
};

__device__ __forceinline__ int visible_lo(int L, int window) {
  return window > 0 ? max(0, L - window) : 0;
}

// Reductions across the lanes of a wave without LDS: DPP within 16-lane rows
// (quad_perm, row_half_mirror, row_mirror, row_ror) and permlane16/32 swaps between
// rows.  group_sum<N>: sum over each aligned group of N lanes, in every lane of the
// group.  across_groups_*<N>: over the lanes 64 / N apart that share a position in
// their group (for max, a value constant within each group).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float swap16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16 || N == 32, "lanes per row");
  x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]: lane ^ 1
  x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]: lane ^ 2
  x += dpp<0x141>(x);  // row_half_mirror: the other quad of the 8 (values equal per quad)
  if constexpr (N >= 16) x += dpp<0x140>(x);  // row_mirror: the other 8 of the row
  if constexpr (N >= 32) x = swap16_sum(x);
  return x;
}
template <int N>
__device__ __forceinline__ float across_groups_max(float x) {
  if constexpr (N <= 8) x = fmaxf(x, dpp<0x140>(x));  // row_mirror: the other group of 8
  if constexpr (N <= 16) x = swap16_max(x);
  return xhalf_max(x);
}
template <int N>
__device__ __forceinline__ float across_groups_sum(float x) {
  if constexpr (N <= 8) x += dpp<0x128>(x);  // row_ror 8: lane ^ 8 within the row
  if constexpr (N <= 16) x = swap16_sum(x);
  return xhalf_sum(x);
}

// GROUPED: more than one query head per K/V head (H > Hkv).  Without it the head loop
// has one trip known at compile time, and the K/V rows need not stay in registers
// after their use.
template <typename TT, int D, bool GROUPED, int NW = 4>
__global__ __launch_bounds__(64 * NW) void decode_split_kernel(
    const TT *__restrict__ q, const TT *__restrict__ kc, const TT *__restrict__ vc,
    const int *__restrict__ seqlens, float *__restrict__ ws_o, float *__restrict__ ws_lse,
    TT *__restrict__ o, float *__restrict__ lse, int H, int Hkv, int Tmax, int window,
    float scale, int nsplit) {
  constexpr int EPL = Elem<TT>::PER16;  // elements per 16-byte load
  constexpr int LPR = D / EPL;          // lanes per cache row
  constexpr int GPW = 64 / LPR;         // rows per wave and round
  constexpr int CH = 32 * NW;          // rows per workgroup
  constexpr int TPW = 32;               // rows per wave
  constexpr int ROUNDS = TPW / GPW;
  // query heads merged per batch (the LDS partials hold NW x GB rows of D floats)
  constexpr int GB = GROUPED ? kDecodeHeadBatch * 4 / NW : 1;
  __shared__ float part_o[NW][GB][D];
  __shared__ float part_ml[NW][GB][2];

  // K/V heads vary fastest across workgroups: the workgroups reading the rows of one
  // token range (adjacent 256-byte pieces of the same cache lines' DRAM pages) run together
  const int hk = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
  const int G = GROUPED ? H / Hkv : 1;  // query heads hk * G .. hk * G + G - 1 read K/V head hk
  const int L = min(seqlens[b], Tmax);
  if (L <= 0) {  // empty sequence: o = 0, lse = -inf
    if (c == 0) {
      for (int g = 0; g < G; ++g) {
        const int bh = b * H + hk * G + g;
        for (int d = threadIdx.x; d < D; d += blockDim.x)
          o[(size_t)bh * D + d] = Elem<TT>::pack(0.f);
        if (lse && threadIdx.x == 0) lse[bh] = -INFINITY;
      }
    }
    return;
  }
  const int lo = visible_lo(L, window);
  const int n = L - lo;
  if (c * CH >= n) return;
  const int t0 = lo + c * CH;
  const int cnt = min(CH, L - t0);
  const int nch = (n + CH - 1) / CH;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int grp = lane / LPR, sl = lane % LPR;
  const size_t rs = (size_t)Hkv * D;
  const TT *kb = kc + ((size_t)b * Tmax * Hkv + hk) * D + sl * EPL;
  const TT *vb = vc + ((size_t)b * Tmax * Hkv + hk) * D + sl * EPL;

  // Every K and V row of this wave is requested before any is used.  Rows past the
  // chunk are read clamped to its last row and masked out below.
  u32x4 kr[ROUNDS], vr[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int t = min(w * TPW + r * GPW + grp, cnt - 1);
    kr[r] = ldg16_stream(kb + (size_t)(t0 + t) * rs);
  }
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int t = min(w * TPW + r * GPW + grp, cnt - 1);
    vr[r] = ldg16_stream(vb + (size_t)(t0 + t) * rs);
  }
  // scores in exp2 units: q is scaled by scale * log2(e)
  const float qs = scale * kLog2e;
  const TT *qg = q + ((size_t)b * H + hk * G) * D + sl * EPL;
  u32x4 qraw = ldg16(qg);  // each query head's q row is requested one head ahead

  for (int g0 = 0; g0 < G; g0 += GB) {
    const int gn = min(GB, G - g0);
    // each query head of the batch in turn: this wave's share of (m, l, o) into LDS
    for (int j = 0; j < gn; ++j) {
      const int g = g0 + j;
      const u32x4 qnext = g + 1 < G ? ldg16(qg + (size_t)(g + 1) * D) : qraw;
      float qf[EPL];
      Elem<TT>::unpack(qraw, qf);
      qraw = qnext;
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[e] *= qs;

      // scores of this wave's rows (each lane group holds one row per round)
      float sc[ROUNDS];
      float m = -INFINITY;
#pragma unroll
      for (int r = 0; r < ROUNDS; ++r) {
        float kf[EPL];
        Elem<TT>::unpack(kr[r], kf);
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot = fmaf(qf[e], kf[e], dot);
        dot = group_sum<LPR>(dot);
        const bool ok = w * TPW + r * GPW + grp < cnt;
        sc[r] = ok ? dot : -INFINITY;
        m = fmaxf(m, sc[r]);
      }
      m = across_groups_max<LPR>(m);
      const float mu = m == -INFINITY ? 0.f : m;
      float lsum = 0.f, acc[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll
      for (int r = 0; r < ROUNDS; ++r) {
        const float p = fast_exp2(sc[r] - mu);
        lsum += p;
        float vf[EPL];
        Elem<TT>::unpack(vr[r], vf);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(p, vf[e], acc[e]);
      }
      // sum over the lane groups of the wave (lanes with the same sl)
      lsum = across_groups_sum<LPR>(lsum);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = across_groups_sum<LPR>(acc[e]);
      if (grp == 0) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) part_o[w][j][sl * EPL + e] = acc[e];
        if (sl == 0) {
          part_ml[w][j][0] = m;
          part_ml[w][j][1] = lsum;
        }
      }
    }
    __syncthreads();
    // merge the NW wave partials of each head (a wave without visible rows has
    // m = -inf, l = 0); m is in exp2 units, lse in natural log
    for (int i = tid; i < gn * D; i += 64 * NW) {
      const int j = i / D, d = i % D;
      const int bh = b * H + hk * G + g0 + j;
      float M = part_ml[0][j][0];
#pragma unroll
      for (int u = 1; u < NW; ++u) M = fmaxf(M, part_ml[u][j][0]);
      float f[NW], Ltot = 0.f, ov = 0.f;
#pragma unroll
      for (int u = 0; u < NW; ++u) {
        f[u] = part_ml[u][j][0] == -INFINITY ? 0.f : fast_exp2(part_ml[u][j][0] - M);
        Ltot += f[u] * part_ml[u][j][1];
      }
#pragma unroll
      for (int u = 0; u < NW; ++u) ov += f[u] * part_o[u][j][d];
      ov /= Ltot;
      const size_t slot = (size_t)bh * nsplit + c;
      if (nch == 1) o[(size_t)bh * D + d] = Elem<TT>::pack(ov);  // nothing to merge
      else ws_o[slot * D + d] = ov;
      if (d == 0) {
        const float l = M * kLn2 + logf(Ltot);
        if (nch > 1) ws_lse[slot] = l;
        else if (lse) lse[bh] = l;
      }
    }
    __syncthreads();  // part_o / part_ml are written again for the next batch
  }
}

// One workgroup per (b, h) with more than one chunk.  Thread (g, d) (G = 256 / D
// groups) takes chunks g, g + G, ... of column d.  Each batch of up to MB of its
// chunks is loaded at once, partial o and lse together, before any is used, so a
// batch costs one memory latency; the maximum over all chunks' lse (thread tid
// loads chunks tid, tid + 256, ... with the first batch) is reduced in between.  The
// G column sums are added in a fixed order: the result does not depend on timing.
template <typename TT, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float *__restrict__ ws_o, const float *__restrict__ ws_lse,
    const int *__restrict__ seqlens, TT *__restrict__ o, float *__restrict__ lse, int H, int Tmax,
    int window, int nsplit, int chunk) {
  constexpr int G = 256 / D;
  constexpr int MB = 16;  // chunks per thread and batch
  __shared__ float red[4];
  __shared__ float part[G][D];
  const int bh = blockIdx.x, b = bh / H;
  const int L = min(seqlens[b], Tmax);
  if (L <= 0) return;
  const int n = L - visible_lo(L, window);
  const int nch = (n + chunk - 1) / chunk;
  if (nch <= 1) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = tid / D, d = tid % D;
  const float *ls = ws_lse + (size_t)bh * nsplit;
  const float *os = ws_o + (size_t)bh * nsplit * D + d;

  // first batch of this thread's chunks, and its share of the lse maximum
  float lv[MB], ov[MB];
#pragma unroll
  for (int u = 0; u < MB; ++u) {
    const int cc = g + u * G;
    lv[u] = cc < nch ? ls[cc] : -INFINITY;
    ov[u] = cc < nch ? os[(size_t)cc * D] : 0.f;
  }
  float m = -INFINITY;
  for (int cc = tid; cc < nch; cc += 256) m = fmaxf(m, ls[cc]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) red[w] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  // sum of exp(lse_c - M) over the chunks of column 0 of each group (every chunk
  // once), and this thread's o accumulation
  float acc = 0.f, s = 0.f;
#pragma unroll
  for (int u = 0; u < MB; ++u) {
    const float e = expf(lv[u] - M);  // 0 for chunks past nch
    acc = fmaf(e, ov[u], acc);
    s += e;
  }
  for (int c0 = G * MB; c0 < nch; c0 += G * MB) {  // later batches (more than G*MB chunks)
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const int cc = c0 + g + u * G;
      lv[u] = cc < nch ? ls[cc] : -INFINITY;
      ov[u] = cc < nch ? os[(size_t)cc * D] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < MB; ++u) {
      const float e = expf(lv[u] - M);
      acc = fmaf(e, ov[u], acc);
      s += e;
    }
  }
  part[g][d] = acc;
  __syncthreads();  // red[] is read above by every thread before it is reused below
  // total: the G groups of column 0 cover every chunk once
  if (d == 0) red[g] = s;
  __syncthreads();
  if (tid < D) {
    float tot = red[0];
#pragma unroll
    for (int i = 1; i < G; ++i) tot += red[i];
    float a = part[0][tid];
#pragma unroll
    for (int i = 1; i < G; ++i) a += part[i][tid];
    o[(size_t)bh * D + tid] = Elem<TT>::pack(a / tot);
    if (lse && tid == 0) lse[bh] = M + logf(tot);
  }
}

// Grouped decode on the matrix cores (bf16, D = 128): the G = H / Hkv query heads
// that read K/V head hk form the 32 columns of one MFMA operand, so each cache row
// costs a share of two 32 x 32 x 16 products instead of a vector-ALU dot product per
// query head.  Workgroup (hk, chunk c, b), four waves; wave w holds rows 32w ..
// 32w + 31 of the chunk's kDecodeChunk rows.
//   1. S^T (rows x heads) = K Q^T: q of up to 32 heads as B operands, K rows as A
//      operands.  K and V are read from HBM in whole 256-byte rows (16 lanes per
//      row, four rows per load): the 64-byte pieces an operand holds directly cost
//      about 30% more time per byte read.  The wave's K rows pass through its own
//      rows of the LDS V tile, where they are read back as operands; its V rows
//      are written over them afterwards.
//   2. Softmax in exp2 units against the chunk's maximum per head (wave maxima
//      exchanged through LDS), P rounded to bf16 and written to LDS per head.
//   3. O^T = V^T P: wave w forms the 32 columns 32w .. 32w + 31 of every head's
//      output over all the chunk's rows (V^T by transposed LDS reads), divides by
//      the row sum and writes the chunk's partial (o_c, lse_c) as the vector kernel.
// More than 32 heads per group: batches of 32 in turn; K stays in registers and V
// in LDS between batches.
constexpr int kGqaHeads = 32;
// Smallest group taken by the matrix-core kernel.  Measured on the 32-sequence
// decode workload (H = 12), cold: with 2 query heads per K/V head it takes 49.5 us
// causal against 55.9 for the vector-ALU kernel (26.0 against 28.3 at W = 1024), and
// the vector kernel serves the heads of a group one after another, so the gap grows
// with the group.
constexpr int kGqaMfmaMinGroup = 2;
constexpr int kGqaPitch = kDecodeChunk + 8;  // P tile row pitch (bf16): rows land on distinct banks

__global__ __launch_bounds__(256) void decode_gqa_mfma_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kc,
    const uint16_t *__restrict__ vc, const int *__restrict__ seqlens, float *__restrict__ ws_o,
    float *__restrict__ ws_lse, uint16_t *__restrict__ o, float *__restrict__ lse, int H, int Hkv,
    int Tmax, int window, float scale, int nsplit) {
  constexpr int D = 128, NDB = D / 32, CH = kDecodeChunk;
  static_assert(CH == 128 && NDB == 4, "one 32-row block per wave, one d block per wave");
  // V rows, d-block-major (dt_off layout) with blocks VP = CH + 1 rows apart: the
  // spare 64-byte row puts the four blocks of one cache row on different banks
  constexpr int VP = CH + 1;
  __shared__ __attribute__((aligned(16))) uint16_t vt[NDB * VP * 32];
  __shared__ __attribute__((aligned(16))) uint16_t pt[kGqaHeads * kGqaPitch];  // P^T, per head
  __shared__ float red_m[4][kGqaHeads], red_l[4][kGqaHeads];

  const int hk = blockIdx.x, c = blockIdx.y, b = blockIdx.z;
  const int G = H / Hkv;
  const int L = min(seqlens[b], Tmax);
  if (L <= 0) {  // empty sequence: o = 0, lse = -inf
    if (c == 0) {
      for (int i = threadIdx.x; i < G * D; i += blockDim.x)
        o[((size_t)b * H + hk * G) * D + i] = 0;
      if (lse)
        for (int g = threadIdx.x; g < G; g += blockDim.x) lse[b * H + hk * G + g] = -INFINITY;
    }
    return;
  }
  const int lo = visible_lo(L, window);
  const int n = L - lo;
  if (c * CH >= n) return;
  const int t0 = lo + c * CH;
  const int cnt = min(CH, L - t0);
  const int nch = (n + CH - 1) / CH;

  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, col = lane & 31;
  const size_t rs = (size_t)Hkv * D;
  const uint16_t *kb = kc + ((size_t)b * Tmax * Hkv + hk) * D;
  const uint16_t *vb = vc + ((size_t)b * Tmax * Hkv + hk) * D;

  // K and V rows 32w + 4j + l/16 (j = 0..7), 16-byte piece l % 16 of each, every load
  // issued before any is used; rows past the chunk are read clamped to its last row
  // (never used: their scores are masked, their P is 0)
  u32x4 kraw[8], vraw[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = min(32 * w + 4 * j + (lane >> 4), cnt - 1);
    kraw[j] = ldg16_stream(kb + (size_t)(t0 + r) * rs + 8 * (lane & 15));
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = min(32 * w + 4 * j + (lane >> 4), cnt - 1);
    vraw[j] = ldg16_stream(vb + (size_t)(t0 + r) * rs + 8 * (lane & 15));
  }
  // tile position of row r, 16-byte piece ch: block ch / 4, position ch % 4 ^ (r / 4) % 4
  auto tile_at = [&](int r, int ch) {
    return vt + (ch >> 2) * (VP * 32) + r * 32 + 8 * ((ch & 3) ^ ((r >> 2) & 3));
  };
  // K through the wave's own tile rows: A operand (u, s) of lane l is row 16u + l % 16,
  // piece 4s + l / 16 (8 k values of a 16 x 16 x 32 product)
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<u32x4 *>(tile_at(32 * w + 4 * j + (lane >> 4), lane & 15)) = kraw[j];
  bf16x8 ka[2][NDB];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int s = 0; s < NDB; ++s)
      ka[u][s] = lds_read_b128(tile_at(32 * w + 16 * u + (lane & 15), 4 * s + (lane >> 4)));
  // V over them (the reads above come first: one wave's LDS accesses complete in order)
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<u32x4 *>(tile_at(32 * w + 4 * j + (lane >> 4), lane & 15)) = vraw[j];

  const float qs = scale * kLog2e;  // scores in exp2 units
  const int l16 = lane & 15, q4 = lane >> 4;
  for (int g0 = 0; g0 < G; g0 += kGqaHeads) {
    const int gn = min(kGqaHeads, G - g0);
    const int ntile = (gn + 15) / 16;  // 16-head column tiles of S^T
    const bool hv = col < gn;  // this lane's P V column is a query head of the batch
    const size_t bh = (size_t)b * H + hk * G + g0 + col;
    // S^T (rows x heads) in 16 x 16 tiles: tile (u, nt) register i of lane l holds
    // row 32w + 16u + 4(l/16) + i of head 16nt + l % 16
    f32x4 sacc[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      if (nt < ntile) {
        const int hq = 16 * nt + l16;
        bf16x8 qb[NDB];
        const uint16_t *qr = q + ((size_t)b * H + hk * G + g0 + hq) * D + 8 * q4;
#pragma unroll
        for (int s = 0; s < NDB; ++s)
          qb[s] = hq < gn ? __builtin_bit_cast(bf16x8, ldg16(qr + 32 * s)) : bf16x8{};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          f32x4 a = {};
#pragma unroll
          for (int s = 0; s < NDB; ++s)
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[u][s], qb[s], a, 0, 0, 0);
          sacc[u][nt] = a;
        }
      }
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      if (nt < ntile) {
        float m = -INFINITY;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = 32 * w + 16 * u + 4 * q4 + i < cnt ? sacc[u][nt][i] * qs : -INFINITY;
            sacc[u][nt][i] = x;
            m = fmaxf(m, x);
          }
        m = xhalf_max(swap16_max(m));
        if (q4 == 0) red_m[w][16 * nt + l16] = m;
      }
    }
    __syncthreads();  // also completes every wave's V rows before the tile is read
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      if (nt < ntile) {
        const int hq = 16 * nt + l16;
        const float Mq =
            fmaxf(fmaxf(red_m[0][hq], red_m[1][hq]), fmaxf(red_m[2][hq], red_m[3][hq]));
        float l = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[i] = fast_exp2(sacc[u][nt][i] - Mq);  // rows past the chunk: exp2(-inf) = 0
            l += p[i];
          }
          // four consecutive rows of head hq: one 8-byte write into its P^T row
          u32x2 pk;
          pk[0] = f32_to_bf16_bits(p[0]) | ((uint32_t)f32_to_bf16_bits(p[1]) << 16);
          pk[1] = f32_to_bf16_bits(p[2]) | ((uint32_t)f32_to_bf16_bits(p[3]) << 16);
          *reinterpret_cast<u32x2 *>(pt + hq * kGqaPitch + 32 * w + 16 * u + 4 * q4) = pk;
        }
        l = xhalf_sum(swap16_sum(l));
        if (q4 == 0) red_l[w][hq] = l;
      }
    }
    __syncthreads();

    f32x16 oacc = {};
#pragma unroll
    for (int t = 0; t < CH / 16; ++t) {
      const bf16x8 va = dt_read_tr<VP>(vt, 16 * t, w, lane);
      const bf16x8 pb = lds_read_b128(pt + col * kGqaPitch + 16 * t + 8 * h);
      oacc = mfma32(va, pb, oacc);
    }
    const float M = fmaxf(fmaxf(red_m[0][col], red_m[1][col]), fmaxf(red_m[2][col], red_m[3][col]));
    const float Ltot = red_l[0][col] + red_l[1][col] + red_l[2][col] + red_l[3][col];
    if (hv) {
      const float inv = 1.f / Ltot;
      const size_t slot = bh * nsplit + c;
      // register i holds output column 32w + 8(i/4) + 4h + i%4 of head col
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = 32 * w + 8 * e + 4 * h;
        if (nch == 1) {
          u32x2 pk;
          pk[0] = f32_to_bf16_bits(oacc[4 * e] * inv) |
                  ((uint32_t)f32_to_bf16_bits(oacc[4 * e + 1] * inv) << 16);
          pk[1] = f32_to_bf16_bits(oacc[4 * e + 2] * inv) |
                  ((uint32_t)f32_to_bf16_bits(oacc[4 * e + 3] * inv) << 16);
          *reinterpret_cast<u32x2 *>(o + bh * D + d) = pk;
        } else {
          f32x4 v4 = {oacc[4 * e] * inv, oacc[4 * e + 1] * inv, oacc[4 * e + 2] * inv,
                      oacc[4 * e + 3] * inv};
          *reinterpret_cast<f32x4 *>(ws_o + slot * D + d) = v4;
        }
      }
      if (w == 0 && h == 0) {
        const float lv = M * kLn2 + logf(Ltot);
        if (nch > 1) ws_lse[slot] = lv;
        else if (lse) lse[bh] = lv;
      }
    }
    if (g0 + kGqaHeads < G) __syncthreads();  // red_m, red_l and pt are written again
  }
}

template <typename TT, int D>
static hipError_t launch_decode_t(const void *q, const void *k_cache, const void *v_cache,
                                  const int *seqlens, void *o, float *lse, int B, int H,
                                  int Hkv, int Tmax, int window, float scale, float *ws,
                                  hipStream_t st) {
  // the workspace holds decode_num_splits(Tmax, window) partials per (b, h): enough for
  // the kDecodeChunk-row chunks of the grouped kernels; the ungrouped split kernel takes
  // chunks of kDecodeChunkWide rows, half as many
  const int ns_ws = decode_num_splits(Tmax, window);
  float *ws_o = ws;
  float *ws_lse = ws + (size_t)B * H * ns_ws * D;
  int ns = ns_ws, chunk = kDecodeChunk;
  if (std::is_same<TT, uint16_t>::value && D == 128 && H >= kGqaMfmaMinGroup * Hkv) {
    decode_gqa_mfma_kernel<<<dim3(Hkv, ns, B), 256, 0, st>>>(
        (const uint16_t *)q, (const uint16_t *)k_cache, (const uint16_t *)v_cache, seqlens, ws_o,
        ws_lse, (uint16_t *)o, lse, H, Hkv, Tmax, window, scale, ns);
  } else if (Hkv != H) {
    // grouped, vector ALU: kDecodeChunk-row chunks of four waves.  The group's heads
    // are served in turn from K/V rows held in registers (172 VGPRs); with eight waves
    // per workgroup a CU would hold one workgroup instead of two (measured: groups of
    // two 54.0 against 70.7 us causal).
    decode_split_kernel<TT, D, true, 4><<<dim3(Hkv, ns, B), 256, 0, st>>>(
        (const TT *)q, (const TT *)k_cache, (const TT *)v_cache, seqlens, ws_o, ws_lse, (TT *)o,
        lse, H, Hkv, Tmax, window, scale, ns);
  } else {
    // ungrouped: kDecodeChunkWide-row chunks of eight waves
    constexpr int NWW = kDecodeChunkWide / 32;
    chunk = kDecodeChunkWide;
    const int vis = window > 0 ? (window < Tmax ? window : Tmax) : Tmax;
    ns = (vis + chunk - 1) / chunk;
    decode_split_kernel<TT, D, false, NWW><<<dim3(Hkv, ns, B), 64 * NWW, 0, st>>>(
        (const TT *)q, (const TT *)k_cache, (const TT *)v_cache, seqlens, ws_o, ws_lse, (TT *)o,
        lse, H, Hkv, Tmax, window, scale, ns);
  }
  // partials of (b, h) at slots b h ns .. + ns - 1 (ns <= ns_ws)
  if (ns > 1)
    decode_merge_kernel<TT, D><<<B * H, 256, 0, st>>>(ws_o, ws_lse, seqlens, (TT *)o, lse, H, Tmax,
                                                      window, ns, chunk);
  return hipGetLastError();
}

hipError_t launch_decode(bool bf16, const void *q, const void *k_cache, const void *v_cache,
                         const int *seqlens, void *o, float *lse, int B, int H, int Hkv, int D,
                         int Tmax, int window, float scale, float *ws, hipStream_t st) {
  if (bf16) {
    if (D == 128)
      return launch_decode_t<uint16_t, 128>(q, k_cache, v_cache, seqlens, o, lse, B, H, Hkv,
                                            Tmax, window, scale, ws, st);
    return launch_decode_t<uint16_t, 64>(q, k_cache, v_cache, seqlens, o, lse, B, H, Hkv, Tmax,
                                         window, scale, ws, st);
  }
  if (D == 128)
    return launch_decode_t<float, 128>(q, k_cache, v_cache, seqlens, o, lse, B, H, Hkv, Tmax,
                                       window, scale, ws, st);
  return launch_decode_t<float, 64>(q, k_cache, v_cache, seqlens, o, lse, B, H, Hkv, Tmax,
                                    window, scale, ws, st);
}

}  // namespace swattn

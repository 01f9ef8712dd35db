// Shared device helpers for the libswattn kernels (gfx950 only).
//
// MFMA conventions (v_mfma_f32_32x32x16_bf16, wave64), checked on the hardware:
//   A operand (32 x 16, M x K): lane l holds A[l % 32][8*(l/32) + j], j = 0..7
//   B operand (16 x 32, K x N): lane l holds B[8*(l/32) + j][l % 32]
//   C/D (32 x 32 fp32):         lane l, register i holds C[8*(i/4) + 4*(l/32) + i%4][l % 32]
// LDS transpose read ds_read_b64_tr_b16, per 16-lane group: lane i = 4c + e
// receives out[r] = (4 x b16 chunk addressed by lane 4r + c)[e], r = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// MFMA row m of a 32-row operand block maps to tile row swap23(m) (bits 2 and 3
// exchanged).  With this order, the C registers 8t..8t+7 of a lane in half h
// hold tile rows 16t + 8h + 0..7, which is exactly the B-operand (K = row) slot
// order of the next MFMA: a C tile feeds the next product without data movement.
__device__ __forceinline__ int swap23(int m) {
  return (m & ~12) | ((m & 8) >> 1) | ((m & 4) << 1);
}

// Tile row held by C register i of a lane in half h (for a 32-row block).
__device__ __forceinline__ int c_row(int i, int h) {
  return swap23(8 * (i >> 2) + 4 * h + (i & 3));
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Max / sum of a value and the same register in the other 32-lane half.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Eight fp32 -> bf16 (round to nearest even) as an MFMA operand.
__device__ __forceinline__ bf16x8 to_bf16x8(f32x16 s, int base) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)s[base + j];
  return r;
}

// Eight fp32 -> bf16 (round to nearest even) from an array.
__device__ __forceinline__ bf16x8 to_bf16x8_arr(const float (&f)[8]) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)f[j];
  return r;
}

__device__ __forceinline__ bf16x8 lds_read_b128(const uint16_t *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

// Transposed LDS read: 4 x bf16 (see the header comment for the lane mapping).
__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t *p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4 *)(reinterpret_cast<uintptr_t>(p)));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// A-operand (M = column of a row-major LDS tile, K = 8 consecutive tile rows) of a
// 32 x 16 block read with two transposed reads.  `base` points at tile element
// (row0, col0); rows row0 + 8h + 0..7 and columns col0 + (l % 32) are delivered
// to lane l in the A-operand order.  `ld` is the tile row pitch in elements.
// The same call also yields a B operand (K = rows, N = columns).
__device__ __forceinline__ bf16x8 lds_read_tr_block(const uint16_t *base, int ld, int lane) {
  const int h = lane >> 5;
  const int g = (lane >> 4) & 1;
  const int i = lane & 15;
  const uint16_t *p = base + (8 * h + (i >> 2)) * ld + 16 * g + 4 * (i & 3);
  return cat(lds_read_tr(p), lds_read_tr(p + 4 * ld));
}

// Same as lds_read_tr_block, for a tile whose 32-row blocks are stored in swap23
// order (LDS row swap23(r) holds tile row r): rows 8h + 0..3 sit at LDS rows
// 4h + 0..3 and rows 8h + 4..7 at LDS rows 8 + 4h + 0..3.
__device__ __forceinline__ bf16x8 lds_read_tr_block_perm(const uint16_t *base, int ld, int lane) {
  const int h = lane >> 5;
  const int g = (lane >> 4) & 1;
  const int i = lane & 15;
  const uint16_t *p = base + (4 * h + (i >> 2)) * ld + 16 * g + 4 * (i & 3);
  return cat(lds_read_tr(p), lds_read_tr(p + 8 * ld));
}

// LDS tiles of R rows x D bf16 are stored d-block-major, [D/32][R][32]: each
// 32-column block is a sub-tile of 64-byte rows, and inside a row the 16-byte
// chunk lc (0..3) sits at position lc ^ ((r >> 2) & 3).  Both access patterns
// used here are free of bank conflicts on the 64 x 4-byte banks: 16 consecutive
// rows read at one chunk (b128 operand reads) and 4 consecutive rows x one
// 32-column block (transposed reads by 32 lanes).  For a lane, the XOR term only
// depends on the lane when the row base is a multiple of 16, so every address is
// a per-lane base plus a compile-time offset.
template <int R>
__device__ __forceinline__ int dt_off(int r, int ch) {  // row r, 16-byte chunk ch (0..D/8-1)
  return (ch >> 2) * (R * 32) + r * 32 + 8 * ((ch & 3) ^ ((r >> 2) & 3));
}

// Transposed operand read from a d-block-major tile whose 32-row blocks are stored
// in swap23 order: delivers tile rows row0 + 8h + 0..7 (row0 % 16 == 0) and the
// columns 32*db + (lane % 32).
template <int R>
__device__ __forceinline__ bf16x8 dt_read_tr_perm(const uint16_t *tile, int row0, int db,
                                                  int lane) {
  const int h = lane >> 5, g = (lane >> 4) & 1, i = lane & 15;
  const int r1 = row0 + 4 * h + (i >> 2), r2 = r1 + 8;
  const int lc = 2 * g + ((i & 3) >> 1), w = 4 * (i & 1);
  const uint16_t *sub = tile + db * (R * 32);
  return cat(lds_read_tr(sub + r1 * 32 + 8 * (lc ^ ((r1 >> 2) & 3)) + w),
             lds_read_tr(sub + r2 * 32 + 8 * (lc ^ ((r2 >> 2) & 3)) + w));
}

// Same for a tile stored in natural row order: rows row0 + 8h + 0..3 and + 4..7.
template <int R>
__device__ __forceinline__ bf16x8 dt_read_tr(const uint16_t *tile, int row0, int db, int lane) {
  const int h = lane >> 5, g = (lane >> 4) & 1, i = lane & 15;
  const int r1 = row0 + 8 * h + (i >> 2), r2 = r1 + 4;
  const int lc = 2 * g + ((i & 3) >> 1), w = 4 * (i & 1);
  const uint16_t *sub = tile + db * (R * 32);
  return cat(lds_read_tr(sub + r1 * 32 + 8 * (lc ^ ((r1 >> 2) & 3)) + w),
             lds_read_tr(sub + r2 * 32 + 8 * (lc ^ ((r2 >> 2) & 3)) + w));
}

// s_waitcnt immediate: at most N vector-memory operations of the wave in flight;
// LDS operations and exports not waited for.
template <int N>
constexpr int kWaitVm = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);

// Workgroup barrier for handing LDS tiles between waves.  The caller first waits
// (s_waitcnt) for what must be complete: its own copies into the tiles about to be
// read (vmcnt) and its own LDS reads of the tiles about to be overwritten
// (lgkmcnt).  Unlike __syncthreads() there is no memory fence, whose
// s_waitcnt vmcnt(0) would also wait for the copies prefetching later tiles.  The
// empty asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// All 2 * NDB transposed operands ops[t][d] of one 32-row block of a d-block-major
// tile of R rows stored in swap23 order (what dt_read_tr_perm<R>(tile, row0 + 16 t,
// d, lane) returns; row0 % 32 == 0), read by one asm block that also waits for
// them (s_waitcnt lgkmcnt(0) inside).  Reason: the compiler makes every
// transposed-read builtin wait for all global -> LDS copies in flight, which would
// cut short the prefetch of the next tile; these reads do not touch the tiles being
// copied.  Outputs are early-clobber, so no address register is overwritten by a
// read still in flight.
template <int R, int NDB>
__device__ __forceinline__ void dt_read_tr_perm_block(const uint16_t *tile, int row0, int lane,
                                                      bf16x8 (&ops)[2][NDB]) {
  static_assert(NDB == 4 || NDB == 2, "D = 128 or 64");
  const int h = lane >> 5, g = (lane >> 4) & 1, i = lane & 15;
  const int lc = 2 * g + ((i & 3) >> 1), w = 4 * (i & 1);
  const int r1 = 4 * h + (i >> 2);  // rows of the first read (+ row0); second read: + 8
  const uint32_t base = lds_addr(tile) + (uint32_t)row0 * 64;
  const uint32_t a1 = base + 2 * (r1 * 32 + 8 * (lc ^ h) + w);
  const uint32_t a2 = base + 2 * ((r1 + 8) * 32 + 8 * (lc ^ (h + 2)) + w);
  constexpr int DS = 64 * R;  // bytes between 32-column blocks
  i16x4 r[4 * NDB];
  if constexpr (NDB == 4) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %16 offset:%18\n\t"
        "ds_read_b64_tr_b16 %1, %17 offset:%18\n\t"
        "ds_read_b64_tr_b16 %2, %16 offset:%19\n\t"
        "ds_read_b64_tr_b16 %3, %17 offset:%19\n\t"
        "ds_read_b64_tr_b16 %4, %16 offset:%20\n\t"
        "ds_read_b64_tr_b16 %5, %17 offset:%20\n\t"
        "ds_read_b64_tr_b16 %6, %16 offset:%21\n\t"
        "ds_read_b64_tr_b16 %7, %17 offset:%21\n\t"
        "ds_read_b64_tr_b16 %8, %16 offset:%22\n\t"
        "ds_read_b64_tr_b16 %9, %17 offset:%22\n\t"
        "ds_read_b64_tr_b16 %10, %16 offset:%23\n\t"
        "ds_read_b64_tr_b16 %11, %17 offset:%23\n\t"
        "ds_read_b64_tr_b16 %12, %16 offset:%24\n\t"
        "ds_read_b64_tr_b16 %13, %17 offset:%24\n\t"
        "ds_read_b64_tr_b16 %14, %16 offset:%25\n\t"
        "ds_read_b64_tr_b16 %15, %17 offset:%25\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
          "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
        : "v"(a1), "v"(a2), "i"(0), "i"(DS), "i"(2 * DS), "i"(3 * DS), "i"(1024),
          "i"(1024 + DS), "i"(1024 + 2 * DS), "i"(1024 + 3 * DS)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%10\n\t"
        "ds_read_b64_tr_b16 %1, %9 offset:%10\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:%11\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%11\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %5, %9 offset:%12\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:%13\n\t"
        "ds_read_b64_tr_b16 %7, %9 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7])
        : "v"(a1), "v"(a2), "i"(0), "i"(DS), "i"(1024), "i"(1024 + DS)
        : "memory");
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int d = 0; d < NDB; ++d) {
      const int k = 2 * (t * NDB + d);
      ops[t][d] = cat(__builtin_bit_cast(bf16x4, r[k]), __builtin_bit_cast(bf16x4, r[k + 1]));
    }
}

// Asynchronous 16-byte copy global -> LDS: lane l's 16 bytes land at lds + 16 l
// (lds must be the same for the whole wave).  Completion is awaited with
// s_waitcnt vmcnt before the barrier that publishes the tile.  CPOL: cache policy
// bits of the load (2 = non-temporal, for data read exactly once).
template <int CPOL = 0>
__device__ __forceinline__ void copy16_to_lds(const void *src, void *lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)lds, 16, 0,
                                   CPOL);
}

// Copy of 16 rows of one 32-column block of a row-major bf16 matrix (row stride
// rs elements, rows clamped to [0, nrows-1]) into a d-block-major LDS tile of R
// rows: tile rows row16 .. row16+15 of block db.  With perm, tile row r of each
// 32-row block is placed at LDS row swap23(r) (see dt_read_tr_perm).  One call per
// wave moves 1 KB.
template <int R, int CPOL = 0>
__device__ __forceinline__ void copy_rows16(uint16_t *tile, const uint16_t *src, int rs,
                                            int row_base, int nrows, int row16, int db,
                                            bool perm, int lane) {
  const int r = row16 + (lane >> 2);                 // LDS row
  const int lc = (lane & 3) ^ ((r >> 2) & 3);        // logical chunk stored at this position
  const int trow = perm ? ((r & ~31) | swap23(r & 31)) : r;
  const int grow = min(row_base + trow, nrows - 1);
  copy16_to_lds<CPOL>(src + (size_t)grow * rs + 32 * db + 8 * lc,
                      tile + db * (R * 32) + row16 * 32);
}

// Buffer resource over `nbytes` bytes from `base` (raw addressing, no stride):
// loads through it at byte offsets >= nbytes return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)nbytes,
                                           0x00020000);
}

// Asynchronous 16-byte copy through a buffer resource into LDS: lane l's bytes at
// byte offset voff land at lds + 16 l (lds uniform across the wave); offsets past
// the resource's size deliver zeros.  Completion: s_waitcnt vmcnt, then a barrier.
__device__ __forceinline__ void buf_copy16_to_lds(__amdgpu_buffer_rsrc_t r, void *lds,
                                                  uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                           voff, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ldg16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

// 16-byte load of data that is read exactly once (non-temporal: bypasses cache
// retention; measured ~25% more HBM read bandwidth than a plain load on gfx950).
__device__ __forceinline__ u32x4 ldg16_stream(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Output rows through LDS.  In MFMA accumulator order a lane (half h, lane ln of the
// half) holds 64 values of row ln: columns 32 d + 8 g + 4 h + e in acc[d][4 g + e].
// Stored directly that is 16 store instructions per lane, each writing 32 separate
// 16-byte pieces.  Instead a wave writes its 32 rows (times mul, as bf16) to its own
// 32 * D elements of LDS, piece c of row r at position c ^ (r mod D / 8)
// (stage_rows_bf16), and after a workgroup barrier reads them back 16 bytes per lane,
// D / 8 consecutive lanes per row, storing whole rows: rows 0 .. nrows - 1 to
// out + r * rs (store_staged_rows).
template <int D>
__device__ __forceinline__ void stage_rows_bf16(uint16_t *stage, const f32x16 (&acc)[D / 32],
                                                float mul, int ln, int h) {
  constexpr int CH = D / 8;
#pragma unroll
  for (int d = 0; d < D / 32; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = (__bf16)(acc[d][4 * g + e] * mul);
      const int pc = 4 * d + g;  // columns 8 pc .. 8 pc + 7; this lane's half is h
      *reinterpret_cast<bf16x4 *>(stage + ln * D + (pc ^ (ln & (CH - 1))) * 8 + 4 * h) = pk;
    }
}

template <int D>
__device__ __forceinline__ void store_staged_rows(const uint16_t *stage, int lane, int nrows,
                                                  uint16_t *out, size_t rs) {
  constexpr int CH = D / 8, RPI = 64 / CH;  // RPI rows per store instruction
  const int pc = lane % CH, pr = lane / CH;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = pr + RPI * i;
    const u32x4 val = *reinterpret_cast<const u32x4 *>(stage + r * D + (pc ^ (r & (CH - 1))) * 8);
    if (r < nrows) *reinterpret_cast<u32x4 *>(out + (size_t)r * rs + 8 * pc) = val;
  }
}

// The same for fp32 rows, half a row at a time (32 rows x D / 2 floats of LDS per
// wave): stage_rows_f32_half writes columns D / 2 * half .. + D / 2 - 1 (times mul),
// 16-byte piece c of row r at position c ^ (r mod D / 8); store_staged_rows_f32_half
// stores them to out + r * rs + D / 2 * half for rows 0 .. nrows - 1.
template <int D>
__device__ __forceinline__ void stage_rows_f32_half(float *stage, const f32x16 (&acc)[D / 32],
                                                    float mul, int ln, int h, int half) {
  constexpr int CH = D / 8;  // 16-byte pieces per half row
#pragma unroll
  for (int dd = 0; dd < D / 64; ++dd)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = D / 64 * half + dd;
      f32x4 a;
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = acc[d][4 * g + e] * mul;
      const int pc = 8 * dd + 2 * g + h;  // columns 4 pc .. 4 pc + 3 of the half row
      *reinterpret_cast<f32x4 *>(stage + ln * (D / 2) + (pc ^ (ln & (CH - 1))) * 4) = a;
    }
}

template <int D>
__device__ __forceinline__ void store_staged_rows_f32_half(const float *stage, int lane,
                                                           int nrows, float *out, size_t rs,
                                                           int half) {
  constexpr int CH = D / 8, RPI = 64 / CH;  // RPI rows per store instruction
  const int pc = lane % CH, pr = lane / CH;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = pr + RPI * i;
    const f32x4 val =
        *reinterpret_cast<const f32x4 *>(stage + r * (D / 2) + (pc ^ (r & (CH - 1))) * 4);
    if (r < nrows)
      *reinterpret_cast<f32x4 *>(out + (size_t)r * rs + D / 2 * half + 4 * pc) = val;
  }
}

}  // namespace swattn

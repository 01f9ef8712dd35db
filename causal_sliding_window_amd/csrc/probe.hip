// Measured ceilings of the GPU the library runs on, for reporting the attention
// kernels against what this chip sustains as well as against its published peaks:
//
// probe_mfma_kernel: each wave issues back to back the same bf16 matrix product the
//   attention passes use (v_mfma_f32_32x32x16_bf16), on four independent accumulator
//   chains and operands held in registers: no memory traffic and no other vector work.
// probe_read_kernel: streams a buffer once with the 16-byte non-temporal loads of the
//   decode kernels, eight loads in flight per lane, consecutive lanes on consecutive
//   16-byte pieces of their workgroup's contiguous span; folds what it reads into one
//   XOR word per thread, so the result can be checked and the loads are not removed.
#include "common.h"
#include "swattn.h"

namespace swattn {
namespace {

constexpr int kProbeThreads = 256;

__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(float *__restrict__ out,
                                                                   int iters) {
  // every operand element 1/256 (exact in bf16): one product adds 16 * 2^-16 = 2^-12
  // to each accumulator element, exactly, for up to 2^24 iterations
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(1.f / 256.f);
    b[j] = (__bf16)(1.f / 256.f);
  }
  f32x16 acc[4] = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = mfma32(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

// Workgroup g streams its own contiguous span of the buffer (spans of equal size, the
// last one shorter), 4 KB per load step of the workgroup, eight steps in flight.
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(
    const u32x4 *__restrict__ src, size_t n16, unsigned *__restrict__ out) {
  const size_t span = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t lo = (size_t)blockIdx.x * span;
  const size_t hi = lo + span < n16 ? lo + span : n16;
  size_t i = lo + threadIdx.x;
  unsigned x = 0;
  for (; i + 7 * kProbeThreads < hi; i += 8 * kProbeThreads) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = ldg16_stream(src + i + u * kProbeThreads);
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < hi; i += kProbeThreads) {
    const u32x4 v = ldg16_stream(src + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = x;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace
}  // namespace swattn

extern "C" {

int swattn_probe_mfma(float *out, int workgroups, int iters, swattn_stream_t stream) {
  if (out == nullptr || !swattn::aligned(out, 4) || workgroups < 1 || workgroups > (1 << 20) ||
      iters < 1 || iters > (1 << 24))
    return SWATTN_ERR_INVALID_ARG;
  swattn::probe_mfma_kernel<<<workgroups, swattn::kProbeThreads, 0, (hipStream_t)stream>>>(out,
                                                                                        iters);
  return hipGetLastError() == hipSuccess ? SWATTN_OK : SWATTN_ERR_HIP;
}

int swattn_probe_read(const void *src, size_t nbytes, unsigned int *out, int workgroups,
                      swattn_stream_t stream) {
  if (src == nullptr || out == nullptr || !swattn::aligned(src, 16) || !swattn::aligned(out, 4) ||
      nbytes == 0 || nbytes % 16 != 0 || workgroups < 1 || workgroups > (1 << 20))
    return SWATTN_ERR_INVALID_ARG;
  swattn::probe_read_kernel<<<workgroups, swattn::kProbeThreads, 0, (hipStream_t)stream>>>(
      reinterpret_cast<const swattn::u32x4 *>(src), nbytes / 16, out);
  return hipGetLastError() == hipSuccess ? SWATTN_OK : SWATTN_ERR_HIP;
}

}  // extern "C"

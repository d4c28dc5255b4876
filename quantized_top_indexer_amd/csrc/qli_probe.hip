// Ceiling probes for gfx950: a streaming HBM read and an INT8 MFMA loop, so
// that the benchmark can state achieved rates against measured ceilings as
// well as published peaks.  Neither kernel takes part in the indexer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qli.h"
#include "qli_probe.h"

namespace {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 256;
constexpr uint32_t kNever = 0x9E3779B9u;  // folded values equal to this are written (never in practice)

// Workgroup b reads its contiguous run [b*n/grid, (b+1)*n/grid) of 16-byte
// vectors, 4 vectors per thread in flight per step.
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const i32x4* buf, int64_t n, uint32_t* sink) {
  const int64_t b = blockIdx.x, g = gridDim.x;
  const int64_t lo = b * n / g, hi = (b + 1) * n / g;
  i32x4 acc = {0, 0, 0, 0};
  int64_t i = lo + threadIdx.x;
  for (; i + 3 * kProbeThreads < hi; i += 4 * kProbeThreads) {
    const i32x4 x0 = __builtin_nontemporal_load(buf + i);
    const i32x4 x1 = __builtin_nontemporal_load(buf + i + kProbeThreads);
    const i32x4 x2 = __builtin_nontemporal_load(buf + i + 2 * kProbeThreads);
    const i32x4 x3 = __builtin_nontemporal_load(buf + i + 3 * kProbeThreads);
    acc ^= x0 ^ x1 ^ x2 ^ x3;
  }
  for (; i < hi; i += kProbeThreads) acc ^= __builtin_nontemporal_load(buf + i);
  const uint32_t f = static_cast<uint32_t>(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
  if (f == kNever && threadIdx.x == 0) sink[b] = f;
}

// Four independent accumulation chains per wave keep the matrix core busy.
__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(int iterations, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const i32x4 a = {lane, lane + 1, lane + 2, lane + 3};
  const i32x4 bv = {3 * lane, lane ^ 5, lane + 7, 11};
  i32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iterations; ++it) {
    c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bv, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bv, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bv, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bv, c3, 0, 0, 0);
  }
  uint32_t f = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) f ^= static_cast<uint32_t>(c0[k] + c1[k] + c2[k] + c3[k]);
  if (f == kNever && lane == 0) sink[blockIdx.x] = f;
}

}  // namespace

extern "C" {

int qli_probe_hbm_read(const void* buf, size_t bytes, int grid, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15) ||
      grid < 1 || grid > 65536)
    return QLI_ERR_INVALID_ARG;
  (void)hipGetLastError();
  probe_read_kernel<<<grid, kProbeThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const i32x4*>(buf), static_cast<int64_t>(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? QLI_OK : QLI_ERR_HIP;
}

int qli_probe_int8_mfma(int grid, int iterations, uint32_t* sink, void* stream) {
  if (!sink || grid < 1 || grid > 65536 || iterations < 1 || iterations > (1 << 20))
    return QLI_ERR_INVALID_ARG;
  (void)hipGetLastError();
  probe_mfma_kernel<<<grid, kProbeThreads, 0, static_cast<hipStream_t>(stream)>>>(iterations, sink);
  return hipGetLastError() == hipSuccess ? QLI_OK : QLI_ERR_HIP;
}

double qli_probe_int8_mfma_ops(int grid, int iterations) {
  // per wave and iteration: 4 MFMAs of 32 x 32 x 32 multiply-adds
  return static_cast<double>(grid) * (kProbeThreads / 64) * iterations * 4.0 * 32 * 32 * 32 * 2;
}

}  // extern "C"

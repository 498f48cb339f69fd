// Measurement helper: a dense streaming read of device memory, the HBM read rate that the
// attention and resolver rates are compared with (the path itself never calls it).
//
// Every lane reads 16-byte chunks, eight loads in flight per pass, grid-strided so one pass
// of a workgroup covers 8 x 256 consecutive chunks (32 KiB); the loaded words are folded
// into one register, stored only if it equals a value no test buffer produces, so the loads
// stay but no write traffic is added.

#include "hs_internal.h"

namespace hs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int CT = 256;     // threads per workgroup
constexpr int CU = 8;       // loads in flight per thread
constexpr int CGRID = 8192; // workgroups: 32 per compute unit

__global__ __launch_bounds__(CT) void stream_read_kernel(const u32x4* __restrict__ src, uint64_t n16,
                                                         uint32_t* __restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * CT;
  uint64_t i = (uint64_t)blockIdx.x * CT + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (CU - 1) * stride < n16; i += CU * stride) {
    u32x4 v[CU];
#pragma unroll
    for (int u = 0; u < CU; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < CU; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(CGRID), dim3(CT), 0, s, (const u32x4*)src, (uint64_t)(bytes / 16),
                     sink);
  return hipGetLastError();
}

}  // namespace hs

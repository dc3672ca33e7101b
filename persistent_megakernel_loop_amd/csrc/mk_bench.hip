// HBM read-stream ceiling: the bandwidth a plain streaming read reaches on this
// device, the reference point for the decode kernel's achieved bytes per second.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_internal.h"
#include "mk_prefill.h"

namespace mk {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Every thread reads 16-byte chunks in a grid-stride loop, 8 loads in flight per
// iteration, and folds them into a value that is stored only if it matches a pattern
// it never matches on these inputs (so the loads cannot be dropped).
template <bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                          unsigned long long* sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = NT ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = NT ? __builtin_nontemporal_load(src + i) : src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace

int launch_stream_read(const void* src, size_t bytes, int nontemporal, unsigned long long* sink, int blocks,
                       void* stream) {
  const size_t n16 = bytes / 16;
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, n16,
                       sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src,
                       n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace mk

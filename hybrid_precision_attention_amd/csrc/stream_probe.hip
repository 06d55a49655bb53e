// Plain streaming read: the measured HBM ceiling the benchmark reports next to
// the nominal peak.  Grid-stride over 16-byte words, eight loads in flight per
// thread, every loaded word folded into a checksum; with ordinary loads or
// with the non-temporal policy the decode scan uses for its cache data.
#include <hip/hip_runtime.h>

#include "hq_probe.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <bool kNt>
__device__ __forceinline__ uint4 load(const uint4* p) {
  if constexpr (kNt) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *p;
  }
}

template <bool kNt>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src, size_t n,
                                                          uint32_t* sink, uint32_t never) {
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 7 * stride < n; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = load<kNt>(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n; i += stride) {
    const uint4 a = load<kNt>(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == never) sink[0] = acc;
}

}  // namespace

template <bool kNt>
static int launch(const void* src, size_t bytes, uint32_t* sink, uint32_t never, int grid,
                  hipStream_t stream) {
  if (!src || !sink || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) || grid < 1)
    return -1;
  hipLaunchKernelGGL(stream_read_kernel<kNt>, dim3(grid), dim3(256), 0, stream,
                     static_cast<const uint4*>(src), bytes / 16, sink, never);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

extern "C" int hq_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, uint32_t never,
                                    int grid, hipStream_t stream) {
  return launch<false>(src, bytes, sink, never, grid, stream);
}

extern "C" int hq_probe_stream_read_nt(const void* src, size_t bytes, uint32_t* sink, uint32_t never,
                                       int grid, hipStream_t stream) {
  return launch<true>(src, bytes, sink, never, grid, stream);
}

// Plain streaming read: the measured HBM ceiling the benchmark reports next to
// the nominal peak.  Also the matrix-core rate probe: chains of fp16 MFMAs of
// the two shapes the kernels could use, alone and with the column-mass
// exponential mix interleaved.  Grid-stride over 16-byte words, eight loads in flight per
// thread, every loaded word folded into a checksum; with ordinary loads or
// with the non-temporal policy the decode scan uses for its cache data.
#include <hip/hip_runtime.h>

#include <type_traits>

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

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// kShape 16: v_mfma_f32_16x16x32_f16 (16384 flop), 32: v_mfma_f32_32x32x16_f16
// (32768 flop); kChains independent accumulators per wave, `iters` rounds.
// kMix: after each MFMA, the column-mass work of the outputs it completes
// (an fma, an exp2 and an add per output element per lane: one element for
// 16x16x32 over d = 128, two for 32x32x16), independent of the MFMA chain.
template <int kShape, int kChains, bool kMix>
__global__ __launch_bounds__(256) void mfma_rate_kernel(float* sink, int iters, float seed) {
  half8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<_Float16>(seed * static_cast<float>(threadIdx.x + i));
    b[i] = static_cast<_Float16>(seed * static_cast<float>(i + 1));
  }
  using acc_t = std::conditional_t<kShape == 16, f32x4_t, f32x16_t>;
  constexpr int kN = kShape == 16 ? 4 : 16;
  acc_t c[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int e = 0; e < kN; ++e) c[k][e] = 0.0f;
  float v[8], acc = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = seed * static_cast<float>(e + threadIdx.x);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) {
      if constexpr (kShape == 16) c[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[k], 0, 0, 0);
      else c[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[k], 0, 0, 0);
      if constexpr (kMix) {
#pragma unroll
        for (int e = 0; e < (kShape == 16 ? 1 : 2); ++e) {
          const int i = (k * 2 + e) & 7;
          acc += __builtin_amdgcn_exp2f(fmaf(v[i], 0.999f, -0.5f));
          v[i] += 1e-7f;
        }
      }
    }
  }
  float s = acc;
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int e = 0; e < kN; ++e) s += c[k][e];
  if (s == 12345.678f) sink[threadIdx.x] = s;
}

}  // namespace

extern "C" int hq_probe_mfma_rate(int which, int grid, int iters, float* sink, hipStream_t stream) {
  if (!sink || grid < 1 || iters < 1) return -1;
  switch (which) {
    case 0: hipLaunchKernelGGL((mfma_rate_kernel<16, 8, false>), dim3(grid), dim3(256), 0, stream, sink, iters, 1e-3f); break;
    case 1: hipLaunchKernelGGL((mfma_rate_kernel<32, 4, false>), dim3(grid), dim3(256), 0, stream, sink, iters, 1e-3f); break;
    case 2: hipLaunchKernelGGL((mfma_rate_kernel<16, 8, true>), dim3(grid), dim3(256), 0, stream, sink, iters, 1e-3f); break;
    case 3: hipLaunchKernelGGL((mfma_rate_kernel<32, 4, true>), dim3(grid), dim3(256), 0, stream, sink, iters, 1e-3f); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

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
